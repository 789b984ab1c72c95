// Tied-embedding gather: rows of a quantised table, dequantised (gfx950).
//
// Model card "24B0978 - Week 02 - Track 2, 40% target", section "Recipe":
// the token embedding is tied to the output head and stored as RTN codes of
// 8 bits with group 128, so one table serves both the head's GEMV and this
// gather.  Output row i is (q[id_i][k] - z[id_i][g]) * s[id_i][g], g = k /
// 128, for every k: the grouped-affine dequantisation ("24B0978 - Week 01 -
// Track 2", paragraph on group-wise affine integer quantisation) of table
// row id_i, rounded once to fp16 or fp32.
//
// A thread makes 8 consecutive outputs.  Their codes are one field of 8 b
// bits at bit 8 b t of the row (a row's codes are contiguous along K, code
// j at bit b j of its little-endian words), read as a 64-bit window of at
// most two words, and they share one group.  The value is exact in fp64 (an
// integer below 256 minus an fp16 value needs at most 33 significant bits,
// times an fp16 value at most 44); fp32 outputs round it once; fp16 outputs
// round it to fp32 with round-to-odd first, which then rounds to fp16 as a
// single rounding would (fp32 carries 13 more significand bits than fp16,
// at least the 2 this needs).
//
// One 256-thread workgroup makes 2048 outputs of one token: grid (count,
// ceil(k / 2048)).  Ids outside [0, n) make rows of zeros without touching
// the table.
#include "wq_internal.h"

namespace wq {

namespace {

constexpr int kEmbedThreads = 256;
constexpr int kEmbedPer = 8;   // outputs per thread

// v rounded to fp32 toward zero, with the last significand bit set when the
// rounding was inexact (round to odd)
__device__ __forceinline__ float f32_round_odd(double v) {
  const float f = (float)v;
  const double back = (double)f;
  if (back == v) return f;
  uint32_t b = __float_as_uint(f);
  if (fabs(back) > fabs(v)) b -= 1u;   // one step toward zero, same sign
  return __uint_as_float(b | 1u);
}

template <int BITS, bool F32>
__global__ __launch_bounds__(kEmbedThreads) void embed_kernel(const uint32_t *codes, const uint16_t *scales,
                                                              const uint16_t *zeros, const int32_t *ids, int64_t n,
                                                              int32_t k, void *out, int64_t ldo) {
  const int64_t row = blockIdx.x;
  const int k0 = kEmbedPer * (int)(blockIdx.y * kEmbedThreads + threadIdx.x);
  if (k0 >= k) return;
  const int32_t id = ids[row];
  double v[kEmbedPer];
  if (id >= 0 && id < n) {
    const int64_t wpr = (int64_t)(k / 32) * BITS;   // words per row
    const uint32_t *rw = codes + (int64_t)id * wpr;
    const int64_t bit = (int64_t)k0 * BITS;
    const int64_t w0 = bit >> 5;
    const int sh = (int)(bit & 31);
    uint64_t win = rw[w0];
    // the second word only when the field reaches into it (the last field
    // of the last row may end with the table)
    if (sh + kEmbedPer * BITS > 32) win |= (uint64_t)rw[w0 + 1] << 32;
    const int64_t gi = (int64_t)id * (k / kGroup) + k0 / kGroup;
    const double s = (double)__builtin_bit_cast(_Float16, scales[gi]);
    const double z = (double)__builtin_bit_cast(_Float16, zeros[gi]);
#pragma unroll
    for (int e = 0; e < kEmbedPer; ++e) {
      const uint32_t q = (uint32_t)(win >> (sh + BITS * e)) & ((1u << BITS) - 1u);
      v[e] = ((double)q - z) * s;
    }
  } else {
#pragma unroll
    for (int e = 0; e < kEmbedPer; ++e) v[e] = 0.0;
  }
  if constexpr (F32) {
    float *o = static_cast<float *>(out) + row * ldo + k0;
    reinterpret_cast<float4 *>(o)[0] = make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
    reinterpret_cast<float4 *>(o)[1] = make_float4((float)v[4], (float)v[5], (float)v[6], (float)v[7]);
  } else {
    uint32_t h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const _Float16 lo = (_Float16)f32_round_odd(v[2 * e]), hi = (_Float16)f32_round_odd(v[2 * e + 1]);
      h[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    uint16_t *o = static_cast<uint16_t *>(out) + row * ldo + k0;
    *reinterpret_cast<uint4 *>(o) = make_uint4(h[0], h[1], h[2], h[3]);
  }
}

template <int BITS>
hipError_t launch_embed_bits(const wq_weight &w, const int32_t *ids, int64_t count, void *out, bool f32,
                             int64_t ldo, hipStream_t s) {
  const dim3 grid((unsigned)count, (unsigned)((w.k + kEmbedThreads * kEmbedPer - 1) / (kEmbedThreads * kEmbedPer)));
  const uint32_t *c = w.codes;
  const uint16_t *sc = w.scales, *z = w.zeros;
  if (f32)
    hipLaunchKernelGGL((embed_kernel<BITS, true>), grid, dim3(kEmbedThreads), 0, s, c, sc, z, ids, w.n,
                       (int32_t)w.k, out, ldo);
  else
    hipLaunchKernelGGL((embed_kernel<BITS, false>), grid, dim3(kEmbedThreads), 0, s, c, sc, z, ids, w.n,
                       (int32_t)w.k, out, ldo);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_embed(const wq_weight &w, const int32_t *ids, int64_t count, void *out, bool f32, int64_t ldo,
                        hipStream_t s) {
  if (count == 0) return hipSuccess;
  switch (w.bits) {
    case 3: return launch_embed_bits<3>(w, ids, count, out, f32, ldo, s);
    case 4: return launch_embed_bits<4>(w, ids, count, out, f32, ldo, s);
    case 6: return launch_embed_bits<6>(w, ids, count, out, f32, ldo, s);
    case 8: return launch_embed_bits<8>(w, ids, count, out, f32, ldo, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace wq

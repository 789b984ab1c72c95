// Offline weight preparation on the GPU: weight-side rotation and
// round-to-nearest group quantisation, bit-exact by construction.
//
// Model card "24B0978 - Week 02 - Track 2, 40% target": sections "Recipe"
// and "Recipe (exact)" (round-to-nearest, group 128; the random Hadamard
// transform is applied per weight block before quantisation); model card
// "24B0978 - Week 01 - Track 2", paragraph on the random Hadamard transform
// (the weight side of the rotation is folded in offline).
//
// Per (row, group of 128) one wave, two values per lane (l and l + 64):
//   1. v = w (fp32 -> fp64); with signs: v_k = d_k v_k, a Walsh-Hadamard
//      transform in fp64 (stride 64 inside the lane, strides 1..32 by lane
//      exchange), then v / sqrt(128) and a rounding to fp32.  For weights of
//      ordinary range the +-1 sums are exact in fp64, so the order of the
//      butterflies does not change the result.
//   2. lo = min(min v, 0), hi = max(max v, 0); s = fp16((hi - lo)/qmax),
//      nearest with ties to even, 1 if it rounds to 0;
//      z = clamp(rint(-lo/s), 0, qmax); q = clamp(rint(v/s + z), 0, qmax),
//      all in fp64, rint rounding half to even.  (The cards name
//      round-to-nearest without a formula; this is the library's reading.)
#include "wq_internal.h"

namespace wq {

namespace {

// fp64 -> fp16 bit pattern, round to nearest, ties to even (IEEE 754).
__device__ uint16_t f64_to_f16_rne(double d) {
  const uint64_t b = __builtin_bit_cast(uint64_t, d);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const uint64_t mag = b & 0x7FFFFFFFFFFFFFFFull;
  if (mag > 0x7FF0000000000000ull) return sign | 0x7E00;        // NaN
  const int e = (int)(mag >> 52) - 1023;                          // unbiased exponent
  if (e >= 16) return sign | 0x7C00;                              // >= 65536: infinity
  if (e < -25) return sign;                                       // < 2^-25: rounds to 0
  const uint64_t m = (mag & 0x000FFFFFFFFFFFFFull) | (1ull << 52);
  const int shift = (e >= -14) ? 42 : 42 + (-14 - e);             // keep 11 (or fewer) bits
  uint64_t q = m >> shift;
  const uint64_t rem = m & ((1ull << shift) - 1), half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  if (e >= -14) {
    int E = e + 15;
    if (q == 2048) { q = 1024; ++E; }
    if (E >= 31) return sign | 0x7C00;
    return sign | (uint16_t)(E << 10) | (uint16_t)(q - 1024);
  }
  return sign | (uint16_t)q;   // subnormal (q == 1024 is the smallest normal)
}

__device__ double f16_bits_to_f64(uint16_t h) {
  return (double)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ double shfl_xor_d(double v, int mask) {
  return __shfl_xor(v, mask, 64);
}

__global__ __launch_bounds__(256) void quantize_kernel(int bits, int64_t n, int64_t k,
                                                       const float *__restrict__ w,
                                                       const uint32_t *__restrict__ signs,
                                                       const uint8_t *__restrict__ block_bits,
                                                       uint8_t *__restrict__ codes,
                                                       uint16_t *__restrict__ scales,
                                                       uint16_t *__restrict__ zeros) {
  const int64_t G = k / 128;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (item >= n * G) return;   // whole waves leave together
  const int64_t row = item / G, g = item % G;
  const int b = bits ? bits : (int)block_bits[row / 64];
  const double qmax = (double)((1 << b) - 1);
  const float *src = w + row * k + g * 128;
  double v0 = (double)src[l], v1 = (double)src[l + 64];
  if (signs != nullptr) {
    const int64_t c0 = g * 128 + l, c1 = c0 + 64;
    if ((signs[c0 >> 5] >> (c0 & 31)) & 1u) v0 = -v0;
    if ((signs[c1 >> 5] >> (c1 & 31)) & 1u) v1 = -v1;
    double a = v0 + v1, c = v0 - v1;   // stride 64: elements l and l + 64
    v0 = a;
    v1 = c;
#pragma unroll
    for (int h = 1; h < 64; h <<= 1) {
      const double p0 = shfl_xor_d(v0, h), p1 = shfl_xor_d(v1, h);
      const bool upper = (l & h) != 0;
      v0 = upper ? p0 - v0 : v0 + p0;
      v1 = upper ? p1 - v1 : v1 + p1;
    }
    const double r = sqrt(128.0);
    v0 = (double)(float)(v0 / r);
    v1 = (double)(float)(v1 / r);
  }
  double lo = fmin(v0, v1), hi = fmax(v0, v1);
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
    lo = fmin(lo, shfl_xor_d(lo, h));
    hi = fmax(hi, shfl_xor_d(hi, h));
  }
  lo = fmin(lo, 0.0);
  hi = fmax(hi, 0.0);
  uint16_t s16 = f64_to_f16_rne((hi - lo) / qmax);
  if ((s16 & 0x7FFF) == 0) s16 = 0x3C00;   // 1.0
  const double s = f16_bits_to_f64(s16);
  const double z = fmin(fmax(rint(-lo / s), 0.0), qmax);
  const double q0 = fmin(fmax(rint(v0 / s + z), 0.0), qmax);
  const double q1 = fmin(fmax(rint(v1 / s + z), 0.0), qmax);
  uint8_t *dst = codes + row * k + g * 128;
  dst[l] = (uint8_t)q0;
  dst[l + 64] = (uint8_t)q1;
  if (l == 0) {
    scales[row * G + g] = s16;
    zeros[row * G + g] = f64_to_f16_rne(z);
  }
}

}  // namespace

hipError_t launch_quantize(int bits, int64_t n, int64_t k, const float *w, const uint32_t *signs,
                           const uint8_t *block_bits, uint8_t *codes, uint16_t *scales,
                           uint16_t *zeros, hipStream_t s) {
  const int64_t items = n * (k / 128);
  const int64_t blocks = (items + 3) / 4;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, s, bits, n, k, w, signs,
                     block_bits, codes, scales, zeros);
  return hipGetLastError();
}

}  // namespace wq

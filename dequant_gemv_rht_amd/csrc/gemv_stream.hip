// Persistent fused rotation + dequantising GEMV for batch sizes up to 16
// (gfx950).  Codes become fp16 (1024 + 2^s q) in registers, v_dot2_f32_f16
// accumulates against the rotated fp16 activations, the scale multiplies
// each 32-code partial once and the zero point (plus the 1024 offset) is
// removed with the partial's activation sums.  Source of the arithmetic:
// model card "24B0978 - Week 01 - Track 2, 20% target", section "How these
// techniques accelerate inference on CUDA" (group-wise affine codes
// dequantised inside the product, scale applied once per group; activations
// rotated by a fast Walsh-Hadamard transform at run time).
//
// Kernels in this file (one persistent workgroup per compute unit; the
// linears of a launch share the CUs in proportion to their estimated time,
// and each workgroup owns a contiguous range of whole output rows, so no
// output is shared between workgroups):
//   * gemv_ring_kernel: batch 1.  Rotates its linear's activations once into
//     LDS, streams the weights through an LDS ring by direct buffer-to-LDS
//     loads (section "Batch 1" below).
//   * gemv_ring_mixed_kernel: batch 1 over the mixed 6/8-bit layout: each
//     workgroup inside one 64-row block of uniform width, on that width's
//     ring, the blocks getting workgroups in proportion to their bytes.
//   * gemv_stream_kernel: batch 1 when the ring does not fit in LDS: codes
//     prefetched into registers.
//   * xprep_kernel + gemv_quad_kernel: batch tiles of 2, 4, 8 or 16 rows
//     (the host picks the tiles, within what fits in LDS): activations
//     rotated and arranged once, then row quads with register accumulation
//     (section "Batch tiles").
//
// Tasks.  A lane's unit of work is a 32-code slice of one or more rows in a
// 512-wide K segment (16 lanes of a DPP row cover the segment).  Every load
// is a raw buffer load: out-of-range lanes read zero without memory
// traffic, so loads are issued on straight-line paths.  Row partials are
// summed over the 16 lanes by DPP and added in a fixed order at the end
// (deterministic).
//
// Unpacking.  A code pair becomes two fp16 values with one v_and_or_b32
// against 1024.0's bit pattern; codes that sit at bit s of a 16-bit half are
// used in place, reading as 1024 + 2^s q, and the activations they meet are
// stored pre-multiplied by 2^-s.  int8 uses one v_perm_b32 per pair.  The
// offsets are removed with two per-slice activation sums: X (the sum of the
// values meant, for the zero point) and XS (1024 times the sum of the values
// stored, for the 1024 offsets).  The stored activations also carry a power
// of two 2^E that puts their largest magnitude (per 128-block at batch 1,
// per batch row in the batch tiles) in [2^14, 2^15), so no value becomes an
// fp16 subnormal through the 2^-s factors, whatever the activations' scale;
// the partials are multiplied by 2^-E before blocks of different E meet.
//
// LDS layout.  Each 32-code activation slice occupies 80 bytes (64 of pairs,
// the two sums, the factor 2^-E, 4 spare): with that stride the 16 lanes of
// a DPP row reading their slices with ds_read_b128 hit 16 distinct 4-bank
// groups.
#include <algorithm>

#include "wq_internal.h"

#include <climits>
#include <cstring>
#include <type_traits>

namespace wq {
using namespace dev;

namespace {

constexpr uint32_t kBias = 0x64006400u;
constexpr float kInvSqrt128 = 0.08838834764831845f;
constexpr int kRG = kStreamThreads / 16;    // DPP rows (row groups) per workgroup

template <int BITS>
__device__ __forceinline__ void load_slice(rsrc_t rs, uint32_t off, uint32_t (&w)[BITS]) {
  if constexpr (BITS == 4) {
    const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kNT));
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (BITS == 8) {
    const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kNT));
    const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16, 0, kNT));
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  } else if constexpr (BITS == 6) {
    const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kNT));
    const u32x2 b = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off + 16, 0, kNT));
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y;
  } else {
    const u32x3 v = __builtin_bit_cast(u32x3, __builtin_amdgcn_raw_buffer_load_b96(rs, off, 0, kNT));
    w[0] = v.x; w[1] = v.y; w[2] = v.z;
  }
}

template <int BIT, int WIDTH, int N>
__device__ __forceinline__ uint32_t field(const uint32_t (&w)[N]) {
  constexpr int wi = BIT / 32, off = BIT % 32;
  if constexpr (off + WIDTH <= 32) {
    return __builtin_amdgcn_ubfe(w[wi], off, WIDTH);
  } else {
    return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], off) & ((1u << WIDTH) - 1);
  }
}

struct UnpackConsts {
  uint32_t mask, mask2, bias;
};

// Constants kept in VGPRs so each code pair costs one v_and_or_b32 (gfx9
// VOP3 instructions cannot take literal constants).
//
// A code pair becomes two fp16 values with one v_and_or_b32: the masks keep
// one code in each 16-bit half of a 32-bit window of the packed bits, in
// place, and 1024.0's exponent is OR-ed in.  A code sitting at bit s of its
// half (s + bits <= 10) reads as 1024 + 2^s q, so the activation it meets is
// stored pre-multiplied by 2^-s (exact: the activation exponent keeps the
// stored values normal fp16 numbers).  Windows
// are the packed words themselves or funnel shifts of two of them.
//   int4: word i: (codes 8i+r, 8i+r+4) at s = 0 (r = 0, 2) or 4 (r = 1, 3),
//         r = 2, 3 from the word shifted right by 8.
//   int8: v_perm_b32 puts bytes r and r+2 of a word next to 0x64 bytes.
//   int3: octet o (codes 8o..8o+7, bits 24o..24o+23 of the 96-bit run):
//         window at bit 24o - 4 gives (8o, 8o+4) at s = (4, 0) and
//         (8o+1, 8o+5) at s = (7, 3); the window at bit 24o + 2 gives
//         (8o+2, 8o+6) and (8o+3, 8o+7) the same way.
//   int6: octet o (bits 48o'..48o'+47 of its 96-bit run of 16 codes,
//         o' = o mod 2): windows at 48o' - 4, +2, +20, +26 give the pairs
//         (0,2), (1,3), (4,6), (5,7) of the octet at s = (4, 0).
template <int BITS>
__device__ __forceinline__ UnpackConsts unpack_consts() {
  constexpr uint32_t m = BITS == 4 ? 0x000F000Fu : BITS == 8 ? 0x00FF00FFu : BITS == 3 ? 0x00070070u : 0x003F03F0u;
  constexpr uint32_t m2 = BITS == 3 ? 0x00380380u : 0u;
  constexpr uint32_t b = BITS == 8 ? 0x64646464u : kBias;
  UnpackConsts c;
  asm volatile("v_mov_b32 %0, %1" : "=v"(c.mask) : "i"(m));
  if constexpr (BITS == 3) asm volatile("v_mov_b32 %0, %1" : "=v"(c.mask2) : "i"(m2));
  else c.mask2 = 0u;
  asm volatile("v_mov_b32 %0, %1" : "=v"(c.bias) : "i"(b));
  return c;
}

// 32 bits of a run of N packed words starting at bit B (-32 < B < 32 N);
// bits outside the run read as zero.
template <int B, int N>
__device__ __forceinline__ uint32_t window(const uint32_t *w) {
  if constexpr (B < 0) {
    return w[0] << (-B);
  } else {
    constexpr int k = B / 32, sh = B % 32;
    if constexpr (sh == 0) return w[k];
    else if constexpr (k + 1 >= N) return w[k] >> sh;
    else return __builtin_amdgcn_alignbit(w[k + 1], w[k], sh);
  }
}

// Code pair P of a 32-code slice as two fp16 values.
template <int BITS, int P>
__device__ __forceinline__ uint32_t pair_at(const uint32_t (&w)[BITS], UnpackConsts c) {
  if constexpr (BITS == 4) {
    constexpr int wi = P / 4, r = P % 4;
    const uint32_t v = (r < 2) ? w[wi] : (w[wi] >> 8);
    return (r & 1) ? ((v & (c.mask << 4)) | c.bias) : ((v & c.mask) | c.bias);
  } else if constexpr (BITS == 8) {
    constexpr int wi = P / 2, r = P % 2;
    return __builtin_amdgcn_perm(c.bias, w[wi], r ? 0x04030401u : 0x04020400u);
  } else if constexpr (BITS == 3) {
    constexpr int o = P / 4, r = P % 4;
    const uint32_t v = window<(r < 2) ? 24 * o - 4 : 24 * o + 2, 3>(w);
    return (v & ((r & 1) ? c.mask2 : c.mask)) | c.bias;
  } else {
    constexpr int o = P / 4, r = P % 4;
    constexpr int off[4] = {-4, 2, 20, 26};
    const uint32_t v = window<48 * (o % 2) + off[r], 3>(w + 3 * (o / 2));
    return (v & c.mask) | c.bias;
  }
}

template <int BITS, int P = 0>
__device__ __forceinline__ void unpack_pairs(const uint32_t (&w)[BITS], UnpackConsts c, uint32_t (&p)[16]) {
  p[P] = pair_at<BITS, P>(w, c);
  if constexpr (P + 1 < 16) unpack_pairs<BITS, P + 1>(w, c, p);
}

// fp16 activation pairs in the order unpack_pairs produces code pairs (the
// lane's 8 values are codes 8o..8o+7 of its 32-code slice, octet o), each
// pre-multiplied by 2^-s of its code's position, and their contribution to
// the slice sums: x_eff (what multiplies q: the values as meant) and x_st
// (what multiplies the 1024 offset: the values as stored).
template <int BITS>
__device__ __forceinline__ void pairs_in_dot_order(const float (&v)[8], uint32_t (&o)[4], float &x_eff,
                                                   float &x_st) {
  if constexpr (BITS == 4) {
    constexpr float k16 = 0.0625f;
    o[0] = pack_half2(v[0], v[4]); o[1] = pack_half2(v[1] * k16, v[5] * k16);
    o[2] = pack_half2(v[2], v[6]); o[3] = pack_half2(v[3] * k16, v[7] * k16);
  } else if constexpr (BITS == 8) {
    o[0] = pack_half2(v[0], v[2]); o[1] = pack_half2(v[1], v[3]);
    o[2] = pack_half2(v[4], v[6]); o[3] = pack_half2(v[5], v[7]);
  } else if constexpr (BITS == 3) {
    o[0] = pack_half2(v[0] * 0.0625f, v[4]); o[1] = pack_half2(v[1] * 0.0078125f, v[5] * 0.125f);
    o[2] = pack_half2(v[2] * 0.0625f, v[6]); o[3] = pack_half2(v[3] * 0.0078125f, v[7] * 0.125f);
  } else {
    o[0] = pack_half2(v[0] * 0.0625f, v[2]); o[1] = pack_half2(v[1] * 0.0625f, v[3]);
    o[2] = pack_half2(v[4] * 0.0625f, v[6]); o[3] = pack_half2(v[5] * 0.0625f, v[7]);
  }
  // The sums of the stored values, as stored (XS) and times each one's 2^s
  // back to the values meant (X), by v_dot2 against fp16 pairs of those
  // powers of two: the products are exact, the sums fp32.
  // Factors (low half, high half) of the even pairs 0, 2 and the odd pairs 1, 3:
  constexpr uint32_t f_even = BITS == 3 || BITS == 6 ? 0x3C004C00u : 0x3C003C00u;   // (16, 1) or (1, 1)
  constexpr uint32_t f_odd = BITS == 4 ? 0x4C004C00u : BITS == 3 ? 0x48005800u : f_even;   // (16, 16), (128, 8)
  constexpr uint32_t one = 0x3C003C00u, fe = f_even, fo = f_odd;
  x_st = dot2(o[3], one, dot2(o[2], one, dot2(o[1], one, dot2(o[0], one, 0.0f))));
  x_eff = dot2(o[3], fo, dot2(o[2], fe, dot2(o[1], fo, dot2(o[0], fe, 0.0f))));
}

__device__ __forceinline__ void store_out(const LinDesc &L, int m, int row, float v) {
  if (L.out_f32) {
    reinterpret_cast<float *>(L.y)[(size_t)m * L.ldy + row] = v;
  } else {
    _Float16 h = (_Float16)v;
    reinterpret_cast<uint16_t *>(L.y)[(size_t)m * L.ldy + row] = __builtin_bit_cast(uint16_t, h);
  }
}

// Rotation item it = (batch row m, 128-block b): lane jj holds elements
// 8jj..8jj+7.  Offsets of its raw fp16 values and of its sign word; items
// past the end read nothing.
template <int MT>
__device__ __forceinline__ void item_mb(int it, int nb, int &m, int &b) {
  if constexpr (MT == 1) {
    m = 0;
    b = it;
  } else {
    m = it / nb;
    b = it - m * nb;
  }
}

template <int MT>
__device__ __forceinline__ void item_offsets(const LinDesc &L, int nb, int items, int it, int jj,
                                             uint32_t &xoff, uint32_t &soff) {
  int m, b;
  item_mb<MT>(it, nb, m, b);
  const int kk = 128 * b + 8 * jj;
  const bool ok = it < items;
  xoff = ok ? (uint32_t)(((size_t)m * L.ldx + kk) * 2) : kOOB;
  soff = ok ? (uint32_t)((kk >> 5) * 4) : kOOB;
}

constexpr int kSliceStride = 20;   // u32 per activation slice in LDS (80 bytes, 64 used)

// fp16 values e0 .. e0 + 7 of a resource holding n of them, zero from n on.
// A load that reaches past the end of its range returns zero as a whole, so
// the group of eight that holds the end is read one value at a time.
__device__ __forceinline__ u32x4 load8_h(rsrc_t rs, int e0, int n) {
  if (e0 + 8 <= n) return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)e0 * 2, 0, 0));
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    h[e] = e0 + e < n ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, (uint32_t)(e0 + e) * 2, 0, 0) : 0u;
  return u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

// Rotate one item into LDS.  Only DPP rows that hold an item do any work
// (the branch is uniform across the 16 lanes of a row).
//
// Activation scale.  The stored values are x' 2^E (and 2^-s on top where a
// code is read in place at bit s), with E chosen from the largest |x'| of
// the block (or of the batch row, in the batch-tile pre-pass) so that this
// maximum lands in [2^14, 2^15): whatever the activations' magnitude, the
// fp16 values are normal numbers well clear of overflow, and the
// in-place factors 2^-s (down to 2^-7) cost no precision.  The slice keeps
// 2^-E as an fp32 in word 18, and the consumer multiplies a partial by it
// once the partial no longer mixes blocks of different E (exact: a power
// of two).
//
// Slice words: 0..15 the fp16 pairs, 16 the sum X of the values meant (for
// the zero point), 17 1024 times the sum XS of the values stored (for the
// 1024 offsets), 18 the factor 2^-E, 19 spare.

// E for a largest magnitude mx: mx 2^E in [2^14, 2^15) (0 for mx = 0).
__device__ __forceinline__ int act_exponent(float mx) {
  return mx > 0.f ? 15 - __builtin_amdgcn_frexp_expf(mx) : 0;
}

__device__ __forceinline__ float absmax8(const float (&v)[8]) {
  float a = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fabsf(v[2]));
  float b = fmaxf(fmaxf(fabsf(v[3]), fabsf(v[4])), fabsf(v[5]));
  return fmaxf(fmaxf(a, b), fmaxf(fabsf(v[6]), fabsf(v[7])));
}

// Largest value over the 16 lanes of a DPP row; every lane gets it.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<kQuadXor1>(v));
  v = fmaxf(v, dpp<kQuadXor2>(v));
  v = fmaxf(v, dpp<kRowHalfMirror>(v));
  return fmaxf(v, dpp<kRowMirror>(v));
}

// Lane jj's eight activations of a 128-block (element kk = 128 b + 8 jj
// onwards) as fp32, with the signs and the butterflies applied when
// rotating (unscaled: each lane's values carry the sign (-1)^popcount(jj)
// and the factor sqrt(128), removed by rot_scale).
__device__ __forceinline__ void load_rotated8(bool rotate, u32x4 raw, uint32_t sword, int kk, int jj, float (&v)[8]) {
  v[0] = half_bits_to_float(raw.x & 0xFFFF); v[1] = half_bits_to_float(raw.x >> 16);
  v[2] = half_bits_to_float(raw.y & 0xFFFF); v[3] = half_bits_to_float(raw.y >> 16);
  v[4] = half_bits_to_float(raw.z & 0xFFFF); v[5] = half_bits_to_float(raw.z >> 16);
  v[6] = half_bits_to_float(raw.w & 0xFFFF); v[7] = half_bits_to_float(raw.w >> 16);
  if (rotate) {
    const uint32_t sb = sword >> (kk & 31);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = ((sb >> e) & 1u) ? -v[e] : v[e];
    fwht128_row16_signed(v, jj);
  }
}

// What turns load_rotated8's values into x' (magnitudes: 1/sqrt(128) or 1).
__device__ __forceinline__ float rot_scale(bool rotate) { return rotate ? kInvSqrt128 : 1.0f; }

// The values of load_rotated8 stored for the dot products with exponent E:
// fp16 pairs in dot order and the two slice sums (summed over the 4 lanes
// of the slice).
template <int BITS>
__device__ __forceinline__ void arrange8(bool rotate, float (&v)[8], int jj, int E, uint32_t (&o)[4], float &xe,
                                         float &xt) {
  const float sc = __builtin_amdgcn_ldexpf(rotate ? fwht_lane_sign(jj) * kInvSqrt128 : 1.0f, E);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] *= sc;
  pairs_in_dot_order<BITS>(v, o, xe, xt);
  xe += dpp<kQuadXor1>(xe);
  xe += dpp<kQuadXor2>(xe);
  xt += dpp<kQuadXor1>(xt);
  xt += dpp<kQuadXor2>(xt);
}

// One slice's four lanes: their pairs, and (lane 0 of the four) the sums
// and the factor 2^-E in words 16..18.
__device__ __forceinline__ void store_slice_part(uint32_t *slice, int jj, const uint32_t (&o)[4], float xe, float xt,
                                                 int E) {
  *reinterpret_cast<u32x4 *>(slice + 4 * (jj & 3)) = u32x4{o[0], o[1], o[2], o[3]};
  if ((jj & 3) == 0)
    *reinterpret_cast<u32x4 *>(slice + 16) =
        u32x4{__builtin_bit_cast(uint32_t, xe), __builtin_bit_cast(uint32_t, 1024.0f * xt),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_ldexpf(1.0f, -E)), 0u};
}

// Item it (batch row m, block b) of a batch-1 or stream workgroup into its
// LDS slices [m][S][20], with the block's own exponent.
template <int BITS, int MT>
__device__ __forceinline__ void rotate_item(bool rotate, u32x4 raw, uint32_t sword, int nb, int items, int it,
                                            int jj, uint32_t *xp, int S) {
  if (it >= items) return;
  int m, b;
  item_mb<MT>(it, nb, m, b);
  const int kk = 128 * b + 8 * jj;
  float v[8];
  load_rotated8(rotate, raw, sword, kk, jj, v);
  const int E = act_exponent(row16_max(absmax8(v)) * rot_scale(rotate));
  uint32_t o[4];
  float xe, xt;
  arrange8<BITS>(rotate, v, jj, E, o, xe, xt);
  store_slice_part(&xp[(m * S + 4 * b + (jj >> 2)) * kSliceStride], jj, o, xe, xt, E);
}

// Code loads of task (row pair p, segment s): rows 2p and 2p+1, this lane's
// 32-code slice.
template <int BITS>
__device__ __forceinline__ void issue_task(rsrc_t rc, bool ok, int p, int s, int S, int wpr, int j,
                                           uint32_t (&cw)[2][BITS]) {
  const int slice = s * 16 + j;
  const bool sv = ok && slice < S;
  const uint32_t co = (uint32_t)((2 * p * wpr + slice * BITS) * 4);
  load_slice<BITS>(rc, sv ? co : kOOB, cw[0]);
  load_slice<BITS>(rc, sv ? co + wpr * 4 : kOOB, cw[1]);
}

// LDS layout of a workgroup, in 4-byte words.
struct StreamLds {
  int xs, part, szl, total;
};

__host__ __device__ inline StreamLds stream_lds(int mt, int S, int KS, int G, int np) {
  StreamLds l;
  l.xs = mt * S * kSliceStride;                  // activations: [mt][S][20], sums and factor in words 16..18
  l.part = l.xs;
  l.szl = (l.part + 2 * np * KS * mt + 3) & ~3;  // partials: [2np][KS][mt]
  l.total = l.szl + ((2 * np * G + 7) & ~7) * 2; // scale, zero as fp32: [2np][G][2]
  return l;
}

template <int BITS, int MT, int D>
__device__ __forceinline__ void stream_rows(const LinDesc &L, const uint32_t *codes0, int m_valid, int r0, int rows,
                                            uint32_t *smem) {
  constexpr int XC = 2;                     // rotation passes whose loads precede the codes
  constexpr int ZL = 2;                     // 16-byte scale (zero) loads per thread before the codes
  const int t = threadIdx.x, rg = t >> 4, j = t & 15;
  const int K = L.k, KS = (K + kSeg - 1) / kSeg, G = K / kGroup, S = K / kSlice;
  const int wpr = S * BITS;
  const int NP = (rows + 1) >> 1, T = NP * KS;
  const bool full = (K % kSeg) == 0;        // every lane's slice exists in every segment
  const StreamLds lay = stream_lds(MT, S, KS, G, NP);
  uint32_t *xp = smem;
  float *part = reinterpret_cast<float *>(smem + lay.part);
  float *szl = reinterpret_cast<float *>(smem + lay.szl);

  const rsrc_t rc = make_rsrc(codes0, (uint32_t)rows * wpr * 4);
  const int nszv = rows * G;                 // scale (zero) values of the workgroup's rows
  const rsrc_t rsc = make_rsrc(L.scales + (size_t)r0 * G, (uint32_t)nszv * 2);
  const rsrc_t rz = make_rsrc(L.zeros + (size_t)r0 * G, (uint32_t)nszv * 2);
  const rsrc_t rx = make_rsrc(L.x, (uint32_t)(((size_t)(m_valid - 1) * L.ldx + K) * 2));
  const rsrc_t rsg = make_rsrc(L.signs, L.signs ? (uint32_t)(K / 8) : 0u);
  const bool rotate = L.signs != nullptr;

  for (int e = t; e < 2 * NP * KS * MT; e += kStreamThreads) part[e] = 0.f;

  // 1. activations, signs, scales and zeros, ahead of the weight stream
  const int nb = K / kGroup, items = MT * nb;
  u32x4 xr[XC];
  uint32_t sw[XC];
#pragma unroll
  for (int q = 0; q < XC; ++q) {
    uint32_t xo, so;
    item_offsets<MT>(L, nb, items, rg + kRG * q, j, xo, so);
    xr[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xo, 0, 0));
    sw[q] = rotate ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsg, so, 0, 0) : 0u;
  }
  const int nsz = 2 * NP * G;               // scale/zero entries, padded to whole row pairs
  u32x4 sr[ZL], zr[ZL];
#pragma unroll
  for (int q = 0; q < ZL; ++q) {
    const int e0 = 8 * (t + kStreamThreads * q);
    sr[q] = load8_h(rsc, e0, nszv);
    zr[q] = load8_h(rz, e0, nszv);
  }

  // 2. the first D steps of this DPP row's tasks: task = rg + 64 i
  const uint32_t seg_step = 16 * BITS * 4;                      // bytes per segment along a row
  const uint32_t pair_bytes = (uint32_t)(2 * wpr * 4);
  const int ds = kRG % KS, dp = kRG / KS;                       // task advance per step
  const uint32_t dco = (uint32_t)dp * pair_bytes + (uint32_t)ds * seg_step;
  const uint32_t wrap = pair_bytes - (uint32_t)KS * seg_step;   // extra bytes when the segment wraps
  int is = rg % KS;
  uint32_t co = __umul24((uint32_t)(rg / KS), pair_bytes) + (uint32_t)is * seg_step + (uint32_t)j * (BITS * 4);
  uint32_t cw[D][2][BITS];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const bool ok = rg + kRG * d < T && (full || is * 16 + j < S);
    load_slice<BITS>(rc, ok ? co : kOOB, cw[d][0]);
    load_slice<BITS>(rc, ok ? co + wpr * 4 : kOOB, cw[d][1]);
    co += dco;
    is += ds;
    if (is >= KS) { is -= KS; co += wrap; }
  }
  // 3. scales and zeros into LDS as fp32, then the rotation
#pragma unroll
  for (int q = 0; q < ZL; ++q) {
    const int e0 = 8 * (t + kStreamThreads * q);
    if (e0 < nsz) {
      const uint32_t av[4] = {sr[q].x, sr[q].y, sr[q].z, sr[q].w};
      const uint32_t bv[4] = {zr[q].x, zr[q].y, zr[q].z, zr[q].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        *reinterpret_cast<float4 *>(&szl[2 * (e0 + 2 * h)]) =
            make_float4(half_bits_to_float(av[h] & 0xFFFF), half_bits_to_float(bv[h] & 0xFFFF),
                        half_bits_to_float(av[h] >> 16), half_bits_to_float(bv[h] >> 16));
      }
    }
  }
  for (int e0 = 8 * (t + kStreamThreads * ZL); e0 < nsz; e0 += 8 * kStreamThreads) {
    const u32x4 a = load8_h(rsc, e0, nszv);
    const u32x4 b = load8_h(rz, e0, nszv);
    const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int h = 0; h < 4; ++h)
      *reinterpret_cast<float4 *>(&szl[2 * (e0 + 2 * h)]) =
          make_float4(half_bits_to_float(av[h] & 0xFFFF), half_bits_to_float(bv[h] & 0xFFFF),
                      half_bits_to_float(av[h] >> 16), half_bits_to_float(bv[h] >> 16));
  }
#pragma unroll
  for (int q = 0; q < XC; ++q) rotate_item<BITS, MT>(rotate, xr[q], sw[q], nb, items, rg + kRG * q, j, xp, S);
  for (int it0 = kRG * XC; it0 < items; it0 += kRG) {
    uint32_t xo, so;
    item_offsets<MT>(L, nb, items, it0 + rg, j, xo, so);
    const u32x4 raw = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xo, 0, 0));
    const uint32_t w1 = rotate ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsg, so, 0, 0) : 0u;
    rotate_item<BITS, MT>(rotate, raw, w1, nb, items, it0 + rg, j, xp, S);
  }
  __syncthreads();

  // 4. stream the tasks
  const UnpackConsts uc = unpack_consts<BITS>();
  int cp = rg / KS, cs = rg % KS;   // task being computed
  const int steps = (T + kRG - 1) / kRG;
  for (int i0 = 0; i0 < steps; i0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int tau = rg + kRG * (i0 + d);
      if (tau < T) {
        const int slice = cs * 16 + j;
        const bool sv = full || slice < S;
        const int sl = sv ? slice : 0;
        const uint32_t zi = __umul24((uint32_t)(2 * cp), (uint32_t)G) + (uint32_t)(sl >> 2);
        const float2 sz0 = *reinterpret_cast<const float2 *>(&szl[2 * zi]);
        const float2 sz1 = *reinterpret_cast<const float2 *>(&szl[2 * (zi + G)]);
        const float sf[2] = {sv ? sz0.x : 0.f, sv ? sz1.x : 0.f};
        const float zf[2] = {sz0.y, sz1.y};
        float acc[2][MT];
        // s * (sum (1024+q') x' - 1024 XS - z X) = s * sum (q - z) x
        if constexpr (MT <= 2) {
          // both rows' code pairs live, each activation slice read once
          uint32_t pr[2][16];
          unpack_pairs<BITS>(cw[d][0], uc, pr[0]);
          unpack_pairs<BITS>(cw[d][1], uc, pr[1]);
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            uint32_t xv[16];
            const u32x4 *src = reinterpret_cast<const u32x4 *>(&xp[(m * S + sl) * kSliceStride]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const u32x4 v = src[q];
              xv[4 * q + 0] = v.x; xv[4 * q + 1] = v.y; xv[4 * q + 2] = v.z; xv[4 * q + 3] = v.w;
            }
            // the slice's sums X and 1024 XS, and its factor 2^-E
            const float4 xq = *reinterpret_cast<const float4 *>(&xp[(m * S + sl) * kSliceStride + 16]);
#pragma unroll
            for (int r = 0; r < 2; ++r) {
              float dd = 0.f;
#pragma unroll
              for (int q = 0; q < 16; ++q) dd = dot2(pr[r][q], xv[q], dd);
              acc[r][m] = (sf[r] * xq.z) * fmaf(-zf[r], xq.x, dd - xq.y);
            }
          }
        } else {
          // one row's code pairs live at a time (register budget)
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            uint32_t pr[16];
            unpack_pairs<BITS>(cw[d][r], uc, pr);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              uint32_t xv[16];
              const u32x4 *src = reinterpret_cast<const u32x4 *>(&xp[(m * S + sl) * kSliceStride]);
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const u32x4 v = src[q];
                xv[4 * q + 0] = v.x; xv[4 * q + 1] = v.y; xv[4 * q + 2] = v.z; xv[4 * q + 3] = v.w;
              }
              const float4 xq = *reinterpret_cast<const float4 *>(&xp[(m * S + sl) * kSliceStride + 16]);
              float dd = 0.f;
#pragma unroll
              for (int q = 0; q < 16; ++q) dd = dot2(pr[q], xv[q], dd);
              acc[r][m] = (sf[r] * xq.z) * fmaf(-zf[r], xq.x, dd - xq.y);
            }
          }
        }
        // the task's two row partials, summed over the 16 lanes
        const uint32_t pb = __umul24((uint32_t)(2 * cp * KS + cs), (uint32_t)MT);
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const float v = row16_sum(acc[r][m]);
            if (j == 0) part[pb + r * KS * MT + m] = v;
          }
        cs += ds;
        cp += dp;
        if (cs >= KS) { cs -= KS; ++cp; }
      }
      // refill this buffer with the task D steps ahead
      const bool ok = tau + kRG * D < T && (full || is * 16 + j < S);
      load_slice<BITS>(rc, ok ? co : kOOB, cw[d][0]);
      load_slice<BITS>(rc, ok ? co + wpr * 4 : kOOB, cw[d][1]);
      co += dco;
      is += ds;
      if (is >= KS) { is -= KS; co += wrap; }
    }
  }
  __syncthreads();

  // 5. add each row's partials in segment order, store
  for (int e = t; e < rows * m_valid; e += kStreamThreads) {
    const int row = e / m_valid, m = e % m_valid;
    float sum = 0.f;
    for (int s = 0; s < KS; ++s) sum += part[(row * KS + s) * MT + m];
    store_out(L, m, r0 + row, sum);
  }
}

// ---------------------------------------------------------------------------
// Batch 1: the weight stream staged through an LDS ring.
//
// Codes travel from HBM to LDS by direct buffer-to-LDS loads, which hold no
// registers while in flight, so R steps of every wave's tasks are
// outstanding from the first instructions on: the workgroup's first steps
// of weights stream in while its activations are still being fetched and
// rotated.  Each wave owns its ring slots and reads back only what its own
// lanes loaded (lane L's bytes land at slot + L * chunk), so a slot is ready
// once the wave's own vector-load counter has drained past it; no barrier.
// Scales and zeros travel the same way (lanes 0..3 of a task's 16 fetch the
// task's 2 rows x 4 groups, two groups per 4-byte load).  The counter is
// waited on explicitly: every step issues the same number of loads on a
// straight-line path (out-of-range tasks read zero), so the count of loads
// younger than a slot is a constant, and no register is loaded inside the
// loop, so the compiler has no load of its own to wait for there.
// ---------------------------------------------------------------------------

// int4 and int8: a row's BITS words per lane travel as direct loads of 16
// bytes per lane (lane L's bytes land at chunk + 16 L), int4 one, int8 two;
// chunk c covers words [4c, 4c + 4) and sits at byte 64 * 16 c of the row's
// region.  The wave's four DPP rows hold consecutive tasks, so each load
// reads 1 KB of consecutive bytes unless the tasks wrap to the next row pair.
//
// int3 and int6 ("flat"): a lane's slice is 12 or 24 bytes, so the step's
// code bytes travel as 16-byte items in their order in LDS: row r of the
// pair, then DPP row g, then 16-byte piece c of g's run of 16 slices.  Item
// i = 64 k + L is lane L's piece in load k (int3: two loads, the second for
// lanes 0..31; int6: three), read from g's task.  Lane j of DPP row g finds
// row r of its slice at byte 256 BITS r + 64 BITS g + 4 BITS j of the
// region.
// Workgroup size of the rings: 8 waves, 16 for int3.  (16-wave rings for
// int6 and int8 measured slower: 7.57 against 6.81 us for an int6 9728 ->
// 2560 linear, and alike for the int6 block at one step in flight; an 8-bit
// 16-wave ring does not fit beside a long K's activations; a 16-wave int4
// ring took the int4 block from 11.17 to 12.35 us at two steps in flight and
// 11.4 us at one.  The int3 block: 12.1 -> 11.35-11.65 us with 16 waves
// and two steps in flight, 11.66 us with one.)
constexpr int kRingThreads = 512;

template <int BITS>
struct Ring {
  static constexpr bool flat = BITS == 3 || BITS == 6;
  static constexpr int nc = BITS == 4 ? 1 : 2;                      // loads per row (int4, int8)
  static constexpr int row = 64 * 4 * BITS;                         // bytes per row per wave per step
  static constexpr int codes = 2 * row;                             // code bytes per wave per step
  static constexpr int ni = (codes + 1023) / 1024;                  // loads per step (flat)
  // 8-bit rows: the workgroup's scales and zeros are staged in LDS once
  // (the 151936 x 2560 head 70.9 -> 69.0 us); the other widths fetch each
  // step's with its codes (staging measured even for int3 and int4 and
  // 1% slower for int6)
  static constexpr bool stage = BITS == 8;
  static constexpr int slot = codes + (stage ? 0 : 2 * 64 * 4);      // + scales, zeros
  // steps in flight: two (one for the wide int8 steps) keep a compute
  // unit's weight reads in flight and leave its queue of vector-memory
  // instructions room for the activation loads at the start.  Measured on
  // the seven-projection blocks at batch 1: int4 11.17 us at depth 2
  // against 11.85 us at 3 and 15.7 us at 1 (13.7, 14.2, 14.9 us at 4, 5, 6
  // in an earlier session); int3 with 8 waves 11.97 us at depth 3 against
  // 12.32 at 4, 12.36 at 2, 12.65 at 5, 13.09 at 6; int6 15.2 us at depth 2,
  // 18.0 at 1; int6 and int8 depth 3 8.56 and 9.66 us against 6.81 and 8.00
  // us at 2 for a 9728 -> 2560 linear; int8 depth 1: the 151936 x 2560 head
  // 69.2 -> 67.1 us, the mixed 6/8 down_proj 7.07 -> 7.11 us.
  static constexpr int depth = BITS == 8 ? 1 : 2;
  static constexpr int q = (flat ? ni : 2 * nc) + (stage ? 0 : 2);  // vector loads per wave per step
  static constexpr int threads = BITS == 3 ? 2 * kRingThreads : kRingThreads;
  static constexpr int waves = threads / 64;
};

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// One row's direct loads of a step: chunk c of every lane to its region.
// Tasks past the workgroup's rows have offsets past the buffer resource and
// read zero.  The whole offset is in the vector operand: the range check of
// a raw buffer load does not include the scalar offset.
template <int BITS, int C = 0>
__device__ __forceinline__ void ring_row_loads(rsrc_t rc, uint32_t row, uint32_t off) {
  using RS = Ring<BITS>;   // nc does not depend on the workgroup size
#if defined(__HIP_DEVICE_COMPILE__)   // 16-byte LDS loads exist only in the gfx950 pass
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (lds_ptr_t)(row + 1024 * C), 16, off + 16 * C, 0, 0, kNT);
#endif
  if constexpr (C + 1 < RS::nc) ring_row_loads<BITS, C + 1>(rc, row, off);
}

// Load-side position of a 16-lane task row in its workgroup's task list
// (task = (row pair, segment ls)), and the step issue into ring slot D.
// Every lane issues every load: out-of-range slices of a partial last
// segment read the next row's bytes (or zero), which only feed lanes whose
// scale is masked to 0.
template <int BITS>
struct RingCursor {
  using RS = Ring<BITS>;
  rsrc_t rc, rc1, rsc, rz;   // rc1: the codes from the workgroup's second row on
  uint32_t slot0;            // LDS address of the wave's slot in stage 0
  int KS, ds;
  uint32_t dco, wco, dso, wso;
  int ls;
  uint32_t lco;   // byte offset of this lane's code words, row 0 of the task
  uint32_t lso;   // byte offset of the scale/zero this lane fetches (lanes 0..7 of a task; not staged)
  // flat layouts: per load k, the segment and byte offset of this lane's item
  int fls[RS::flat ? RS::ni : 1];
  uint32_t flco[RS::flat ? RS::ni : 1];
  bool flast;     // int3: this lane carries an item in the last load

  template <int D>
  __device__ __forceinline__ void issue() {
    const uint32_t slot = slot0 + D * RS::waves * RS::slot;
    if constexpr (RS::flat) {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
      for (int k = 0; k < RS::ni; ++k) {
        // items past the pair's last row are out of range and read zero
        if (k + 1 < RS::ni || BITS == 6 || flast)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (lds_ptr_t)(slot + 1024 * k), 16, flco[k], 0, 0, kNT);
      }
#endif
#pragma unroll
      for (int k = 0; k < RS::ni; ++k) {
        fls[k] += ds;
        const bool w = fls[k] >= KS;
        fls[k] = w ? fls[k] - KS : fls[k];
        flco[k] += w ? wco : dco;
      }
    } else {
      // row 2p + 1 at the same offset from the second row: past the last
      // row (an odd row count) it is out of range and reads zero
      ring_row_loads<BITS>(rc, slot, lco);
      ring_row_loads<BITS>(rc1, slot + RS::row, lco);
    }
    if constexpr (!RS::stage) {
#if defined(__HIP_DEVICE_COMPILE__)
      // one fp16 per lane, zero-extended to 4 bytes at slot + 4 L: a 2-byte
      // load never reaches past the end of its range (a load that does
      // returns zero as a whole)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsc, (lds_ptr_t)(slot + RS::codes), 2, lso, 0, 0, kNT);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rz, (lds_ptr_t)(slot + RS::codes + 256), 2, lso, 0, 0, kNT);
#endif
    }
    ls += ds;
    const bool wrap = ls >= KS;
    ls = wrap ? ls - KS : ls;
    if constexpr (!RS::flat) lco += wrap ? wco : dco;
    if constexpr (!RS::stage) lso += wrap ? wso : dso;
  }
};

// Scales and zeros of an 8-bit ring workgroup's rows are staged in LDS once, each
// array as the bytes of its rows from the 16-byte boundary at or below the
// first row through one more row than the workgroup has (read, masked, by
// a missing odd row and by the groups past K of a partial last segment)
// and 16 bytes more.  Each wave issues kRingSzLoads direct 16-byte loads
// per array (64 items of 16 bytes each), whether needed or not, so that
// every wave issues the same loads; a wave's chunks past the rows land in a
// 1 KB dummy area.
constexpr int kRingSzLoads = 3;

// 16-byte items one staged array takes (at most the loads' reach)
__host__ __device__ inline int ring_sz_items(int np, int G) { return (15 + (2 * np + 1) * G * 2 + 16 + 15) / 16; }

// LDS layout of a ring workgroup, in bytes.
struct RingLds {
  int xs, part, ring, sc, zr, dummy, total;
};

__host__ __device__ inline RingLds ring_lds(int S, int KS, int np, int G, int slot, int depth, int waves,
                                            bool stage) {
  RingLds l;
  l.xs = S * kSliceStride * 4;                      // activations: [S][20] u32, sums in words 16, 17
  l.part = l.xs;                                    // partials: [2np][KS] f32
  l.ring = (l.part + 2 * np * KS * 4 + 15) & ~15;
  const int szb = stage ? (ring_sz_items(np, G) + 63) / 64 * 1024 : 0;   // whole 64-item chunks
  l.sc = l.ring + depth * waves * slot;             // staged scales
  l.zr = l.sc + szb;                                // staged zeros
  l.dummy = l.zr + szb;                             // chunks past the rows
  l.total = l.dummy + (stage ? 1024 : 0);
  return l;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most n * Q vector loads are outstanding (n < R, uniform).
template <int R, int Q, int J = R - 1>
__device__ __forceinline__ void wait_vmcnt_younger(int n) {
  if constexpr (J == 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= J) { wait_vmcnt<J * Q>(); return; }
    wait_vmcnt_younger<R, Q, J - 1>(n);
  }
}

__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(lds_ptr_t)p;
}

// A task's LDS operands, read in one asm statement that also waits for
// them: the activation slice (4 x 16 bytes) and its sums and factor (bytes
// 64..79 of the slice), the staged scales and zeros of the lane's group
// (rows 0, 1), and the lane's code words of both rows from the ring slot.  Keeping these reads out of the compiler's view
// keeps it from tying them to the ring's direct loads with waits of its own.
struct TaskOps {
  u32x4 x[4];
  uint64_t xq;   // the slice's sums X and 1024 XS, as one 64-bit scalar (a vector output whose
                 // elements were reinterpreted as floats came back from its first register only)
  uint32_t xf;   // the slice's factor 2^-E
  uint32_t s0, s1, z0, z1;
};

// sa, sb, za, zb: the scales of rows 0 and 1 and their zeros; staged, at
// any distances; else in the ring slot at fixed ones (sa only).
template <int BITS>
__device__ __forceinline__ void read_task(uint32_t xa, uint32_t sa, uint32_t sb, uint32_t za, uint32_t zb,
                                          uint32_t ca16, uint32_t ca4, TaskOps &o, uint32_t (&w)[2][BITS]) {
  static_assert(Ring<BITS>::stage == (BITS == 8), "the 8-bit reads take the staged addresses");
#define WQ_OPS_XREADS                   \
  "ds_read_b128 %[x0], %[xa]\n\t"       \
  "ds_read_b128 %[x1], %[xa] offset:16\n\t" \
  "ds_read_b128 %[x2], %[xa] offset:32\n\t" \
  "ds_read_b128 %[x3], %[xa] offset:48\n\t" \
  "ds_read_b64 %[xq], %[xa] offset:64\n\t" \
  "ds_read_b32 %[xf], %[xa] offset:72\n\t"
// ring slot: row r's scale at sa + 16 r, its zero 256 bytes on
#define WQ_OPS_READS                    \
  WQ_OPS_XREADS                         \
  "ds_read_u16 %[s0], %[sa]\n\t"       \
  "ds_read_u16 %[s1], %[sa] offset:16\n\t" \
  "ds_read_u16 %[z0], %[sa] offset:256\n\t" \
  "ds_read_u16 %[z1], %[sa] offset:272\n\t"
// staged: four addresses
#define WQ_OPS_READS_STAGED             \
  WQ_OPS_XREADS                         \
  "ds_read_u16 %[s0], %[sa]\n\t"        \
  "ds_read_u16 %[s1], %[sb]\n\t"        \
  "ds_read_u16 %[z0], %[za]\n\t"        \
  "ds_read_u16 %[z1], %[zb]\n\t"
#define WQ_OPS_OUT                                                                                      \
  [x0] "=&v"(o.x[0]), [x1] "=&v"(o.x[1]), [x2] "=&v"(o.x[2]), [x3] "=&v"(o.x[3]), [xq] "=&v"(o.xq), [xf] "=&v"(o.xf), \
      [s0] "=&v"(o.s0), [s1] "=&v"(o.s1), [z0] "=&v"(o.z0), [z1] "=&v"(o.z1)
#define WQ_OPS_IN [xa] "v"(xa), [sa] "v"(sa), [ca16] "v"(ca16), [ca4] "v"(ca4)
  if constexpr (BITS == 4) {
    // row r: 16 bytes at r * 1024 + 16 L
    u32x4 c0, c1;
    asm volatile(WQ_OPS_READS
                 "ds_read_b128 %[c0], %[ca16]\n\t"
                 "ds_read_b128 %[c1], %[ca16] offset:1024\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : WQ_OPS_OUT, [c0] "=&v"(c0), [c1] "=&v"(c1)
                 : WQ_OPS_IN
                 : "memory");
    w[0][0] = c0.x; w[0][1] = c0.y; w[0][2] = c0.z; w[0][3] = c0.w;
    w[1][0] = c1.x; w[1][1] = c1.y; w[1][2] = c1.z; w[1][3] = c1.w;
  } else if constexpr (BITS == 8) {
    // row r: words 0..3 at r * 2048 + 16 L, words 4..7 at r * 2048 + 1024 + 16 L
    u32x4 c0, c1, c2, c3;
    asm volatile(WQ_OPS_READS_STAGED
                 "ds_read_b128 %[c0], %[ca16]\n\t"
                 "ds_read_b128 %[c1], %[ca16] offset:1024\n\t"
                 "ds_read_b128 %[c2], %[ca16] offset:2048\n\t"
                 "ds_read_b128 %[c3], %[ca16] offset:3072\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : WQ_OPS_OUT, [c0] "=&v"(c0), [c1] "=&v"(c1), [c2] "=&v"(c2), [c3] "=&v"(c3)
                 : WQ_OPS_IN, [sb] "v"(sb), [za] "v"(za), [zb] "v"(zb)
                 : "memory");
    w[0][0] = c0.x; w[0][1] = c0.y; w[0][2] = c0.z; w[0][3] = c0.w;
    w[0][4] = c1.x; w[0][5] = c1.y; w[0][6] = c1.z; w[0][7] = c1.w;
    w[1][0] = c2.x; w[1][1] = c2.y; w[1][2] = c2.z; w[1][3] = c2.w;
    w[1][4] = c3.x; w[1][5] = c3.y; w[1][6] = c3.z; w[1][7] = c3.w;
  } else if constexpr (BITS == 3) {
    // row r: the lane's 12 bytes at r * 768 + 192 g + 12 j (ca4)
    uint32_t c[6];
    asm volatile(WQ_OPS_READS
                 "ds_read_b32 %[c0], %[ca4]\n\t"
                 "ds_read_b32 %[c1], %[ca4] offset:4\n\t"
                 "ds_read_b32 %[c2], %[ca4] offset:8\n\t"
                 "ds_read_b32 %[c3], %[ca4] offset:768\n\t"
                 "ds_read_b32 %[c4], %[ca4] offset:772\n\t"
                 "ds_read_b32 %[c5], %[ca4] offset:776\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : WQ_OPS_OUT, [c0] "=&v"(c[0]), [c1] "=&v"(c[1]), [c2] "=&v"(c[2]), [c3] "=&v"(c[3]),
                   [c4] "=&v"(c[4]), [c5] "=&v"(c[5])
                 : WQ_OPS_IN
                 : "memory");
#pragma unroll
    for (int e = 0; e < 3; ++e) {
      w[0][e] = c[e];
      w[1][e] = c[3 + e];
    }
  } else {
    // int6 row r: the lane's 24 bytes at r * 1536 + 384 g + 24 j (ca4)
    uint64_t c[6];
    asm volatile(WQ_OPS_READS
                 "ds_read_b64 %[c0], %[ca4]\n\t"
                 "ds_read_b64 %[c1], %[ca4] offset:8\n\t"
                 "ds_read_b64 %[c2], %[ca4] offset:16\n\t"
                 "ds_read_b64 %[c3], %[ca4] offset:1536\n\t"
                 "ds_read_b64 %[c4], %[ca4] offset:1544\n\t"
                 "ds_read_b64 %[c5], %[ca4] offset:1552\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : WQ_OPS_OUT, [c0] "=&v"(c[0]), [c1] "=&v"(c[1]), [c2] "=&v"(c[2]), [c3] "=&v"(c[3]),
                   [c4] "=&v"(c[4]), [c5] "=&v"(c[5])
                 : WQ_OPS_IN
                 : "memory");
#pragma unroll
    for (int e = 0; e < 3; ++e) {
      w[0][2 * e] = (uint32_t)c[e]; w[0][2 * e + 1] = (uint32_t)(c[e] >> 32);
      w[1][2 * e] = (uint32_t)c[3 + e]; w[1][2 * e + 1] = (uint32_t)(c[3 + e] >> 32);
    }
  }
#undef WQ_OPS_XREADS
#undef WQ_OPS_READS
#undef WQ_OPS_READS_STAGED
#undef WQ_OPS_OUT
#undef WQ_OPS_IN
}

__device__ __forceinline__ void lds_store(uint32_t addr, float v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}

// Marks loaded registers as consumed on every path, so that no load issued
// before the ring loop is still outstanding in the compiler's bookkeeping
// when the loop starts (it would otherwise drain all vector loads there).
__device__ __forceinline__ void consume(u32x4 a, uint32_t b) { asm volatile("" ::"v"(a), "v"(b)); }

// Workgroup barrier for LDS data only: waits for this wave's LDS accesses,
// not for its vector loads (the ring's loads stay in flight across it).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Activation items per DPP row whose loads precede the weight stream (the
// rest are loaded while rotating).  int4: 3, so that a K = 9728 linear's 76
// blocks on 32 DPP rows are all requested ahead of the ring (measured 6.76
// -> 6.36 us for down_proj).
template <int BITS>
constexpr int kActAhead = BITS == 3 ? 2 : 3;

// The activation loads a ring workgroup issues before anything else: loads
// complete in order, so activations requested after the weight stream would
// wait for it.  Item it = rg + RG q is rotation block it; lane j of DPP row
// rg holds its elements 8j .. 8j + 7 and the sign word that covers them.
// Without signs the sign range is empty and the loads read zero.
template <int XC>
struct ActAhead {
  u32x4 xr[XC];
  uint32_t sw[XC];
};

template <int XC, int TH = kRingThreads>
__device__ __forceinline__ void act_ahead_loads(const LinDesc &L, ActAhead<XC> &a) {
  constexpr int RG = TH / 16;
  const int t = threadIdx.x, rg = t >> 4, j = t & 15;
  const int items = L.k / kGroup;
  const rsrc_t rx = make_rsrc(L.x, (uint32_t)L.k * 2);
  const rsrc_t rsg = make_rsrc(L.signs, L.signs ? (uint32_t)(L.k / 8) : 0u);
#pragma unroll
  for (int q = 0; q < XC; ++q) {
    const int it = rg + RG * q;
    const bool ok = it < items;
    a.xr[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? (uint32_t)(256 * it + 16 * j) : kOOB, 0, 0));
    a.sw[q] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsg, ok ? (uint32_t)(16 * it + 4 * (j >> 2)) : kOOB, 0, 0);
  }
}

template <int BITS, bool FULL>
// r0: the workgroup's first row; codes0: that row's code words (the rows
// that follow are consecutive at BITS * k / 32 words each); ahead: the
// activation loads act_ahead_loads issued.
__device__ __forceinline__ void stream_ring(const LinDesc &L, const uint32_t *codes0, int r0, int rows,
                                            uint32_t *smem, const ActAhead<kActAhead<BITS>> &ahead) {
  using RS = Ring<BITS>;
  constexpr int R = RS::depth, Q = RS::q;
  constexpr int TH = RS::threads, RG = TH / 16;   // threads, DPP rows
  constexpr int XC = kActAhead<BITS>;
  const int t = threadIdx.x, rg = t >> 4, j = t & 15, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int K = L.k, KS = (K + kSeg - 1) / kSeg, G = K / kGroup, S = K / kSlice;
  const int wpr = S * BITS;
  const int NP = (rows + 1) >> 1, T = NP * KS;
  const RingLds lay = ring_lds(S, KS, NP, G, RS::slot, R, RS::waves, RS::stage);
  uint8_t *lds = reinterpret_cast<uint8_t *>(smem);
  uint32_t *xp = smem;
  float *part = reinterpret_cast<float *>(lds + lay.part);
  const int steps = (T + RG - 1) / RG;   // steps of this workgroup (uniform)
  const int nb = K / kGroup, items = nb;
  const rsrc_t rx = make_rsrc(L.x, (uint32_t)K * 2);
  const rsrc_t rsg = make_rsrc(L.signs, L.signs ? (uint32_t)(K / 8) : 0u);
  const bool rotate = L.signs != nullptr;

  // 2. the weight stream's cursor.  Task tau = rg + 64 i is (row pair
  //    tau / KS, segment tau % KS); quotients by KS of numbers up to 64 are
  //    (x * ks_inv) >> 16 exactly.  The first R steps are issued
  //    unconditionally (a slot past the workgroup's steps reads out of range:
  //    zeros, no traffic), which keeps the compiler's wait for the
  //    activations exact (it counts the stream's loads as younger).
  const int cp0 = (int)(__umul24((uint32_t)rg, (uint32_t)L.ks_inv) >> 16), cs0 = rg - cp0 * KS;
  const int dp = (RG * L.ks_inv) >> 16, ds = RG - dp * KS;
  RingCursor<BITS> cur;
  {
    const uint32_t row_bytes = (uint32_t)wpr * 4, pair_bytes = 2 * row_bytes;
    const uint32_t seg_step = 16 * BITS * 4;
    cur.rc = make_rsrc(codes0, (uint32_t)rows * row_bytes);
    cur.rc1 = make_rsrc(codes0 + wpr, (uint32_t)(rows - 1) * row_bytes);
    if constexpr (!RS::stage) {
      const uint32_t szb = (uint32_t)rows * G * 2;
      cur.rsc = make_rsrc(L.scales + (size_t)r0 * G, szb);
      cur.rz = make_rsrc(L.zeros + (size_t)r0 * G, szb);
      cur.dso = (uint32_t)(2 * (2 * dp * G + 4 * ds));
      cur.wso = cur.dso + (uint32_t)(2 * (2 * G - 4 * KS));
      // lanes j < 8 fetch the scale/zero of row 2p + (j >> 2), group 4s + (j & 3);
      // the other lanes start past any resource (bit 31 set) and stay there as the offset advances
      cur.lso = (__umul24((uint32_t)(2 * cp0 + (j >> 2)), (uint32_t)(2 * G)) + (uint32_t)(8 * cs0 + 2 * (j & 3))) |
                (j < 8 ? 0u : kOOB);
    }
    cur.slot0 = lds_addr(lds + lay.ring) + (uint32_t)(wave * RS::slot);
    cur.KS = KS;
    cur.ds = ds;
    cur.dco = (uint32_t)dp * pair_bytes + (uint32_t)ds * seg_step;
    cur.wco = cur.dco + pair_bytes - (uint32_t)KS * seg_step;
    cur.ls = cs0;
    cur.lco = __umul24((uint32_t)cp0, pair_bytes) + (uint32_t)cs0 * seg_step + (uint32_t)j * (BITS * 4);
    if constexpr (RS::flat) {
      constexpr int per_row = 16 * BITS, per_g = 4 * BITS;   // 16-byte items per row, per DPP row's run
#pragma unroll
      for (int k = 0; k < RS::ni; ++k) {
        const int i = 64 * k + lane;
        const int r = i / per_row, ir = i - r * per_row, g = ir / per_g, c = ir - g * per_g;
        const int rgk = 4 * wave + g;                   // the DPP row whose task this item belongs to
        const int pk = (int)(__umul24((uint32_t)rgk, (uint32_t)L.ks_inv) >> 16), sk = rgk - pk * KS;
        cur.fls[k] = sk;
        cur.flco[k] = __umul24((uint32_t)pk, pair_bytes) + (uint32_t)sk * seg_step + (uint32_t)r * row_bytes +
                      (uint32_t)(16 * c);
      }
      cur.flast = lane < 2 * per_row - 64 * (RS::ni - 1);
    }
  }
  // the scales and zeros of the workgroup's rows, staged once (before the
  // weight stream, so that waiting for them never waits for it)
  const uint32_t sz0 = (uint32_t)r0 * (uint32_t)G * 2, sz_al = sz0 & ~15u;   // first byte, its 16-byte boundary
  if constexpr (RS::stage) {
    const int n16 = ring_sz_items(NP, G);
    // the arrays' range rounded up to 16 bytes: a 16-byte load that reaches
    // past its range returns zero as a whole, which would drop the last
    // row's last scales; the array starts 16-byte aligned, so the rounded
    // end stays in its last page (the bytes past the array only reach
    // masked lanes and rows that are not stored)
    const uint32_t szn = ((uint32_t)L.n * (uint32_t)G * 2 + 15u) & ~15u;
    const rsrc_t rs = make_rsrc(L.scales, szn), rz = make_rsrc(L.zeros, szn);
#pragma unroll
    for (int q = 0; q < kRingSzLoads; ++q) {
      const int c = q * RS::waves + wave, it = 64 * c + lane;   // chunk, item
      const bool used = 64 * c < n16;
      const uint32_t dst_s = lds_addr(lds + (used ? lay.sc + 1024 * c : lay.dummy));
      const uint32_t dst_z = lds_addr(lds + (used ? lay.zr + 1024 * c : lay.dummy));
      const uint32_t src = it < n16 ? sz_al + 16u * (uint32_t)it : kOOB;
#if defined(__HIP_DEVICE_COMPILE__)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)dst_s, 16, src, 0, 0, kNT);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rz, (lds_ptr_t)dst_z, 16, src, 0, 0, kNT);
#endif
    }
  }
  cur.template issue<0>();
  if constexpr (R > 1) cur.template issue<1>();
  if constexpr (R > 2) cur.template issue<2>();
  if constexpr (R > 3) cur.template issue<3>();
  if constexpr (R > 4) cur.template issue<4>();
  if constexpr (R > 5) cur.template issue<5>();
  static_assert(R <= 6, "ring depth");

  // 3. the rotation into LDS.  (A compute unit holds a limited number of
  // outstanding vector memory instructions, so the second wave on each SIMD
  // meets the first waves' ring loads and starts rotating about a memory
  // latency later.  Letting those waves rotate before issuing their steps,
  // or a barrier between every wave's activation loads and the ring loads,
  // measured slower for the int3 and int4 blocks, and much slower for the
  // 16-wave int6 ring.)
#pragma unroll
  for (int q = 0; q < XC; ++q) {
    consume(ahead.xr[q], ahead.sw[q]);
    rotate_item<BITS, 1>(rotate, ahead.xr[q], ahead.sw[q], nb, items, rg + RG * q, j, xp, S);
  }
  for (int it0 = RG * XC; it0 < items; it0 += RG) {
    const int it = it0 + rg;
    const bool ok = it < items;
    const u32x4 raw = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? (uint32_t)(256 * it + 16 * j) : kOOB, 0, 0));
    const uint32_t w1 = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsg, ok ? (uint32_t)(16 * it + 4 * (j >> 2)) : kOOB, 0, 0);
    consume(raw, w1);
    rotate_item<BITS, 1>(rotate, raw, w1, nb, items, it0 + rg, j, xp, S);
  }
  if constexpr (RS::stage) wait_vmcnt<R * Q>();   // this wave's staged scales and zeros are in LDS
  lds_barrier();

  // 3. consume the ring
  const UnpackConsts uc = unpack_consts<BITS>();
  // Compute-side position of the task: its slice's LDS address xa (slice
  // 16 cs + j) and, for lanes 0 and 1, the address of row 2 cp + j's partial
  // for segment cs.  Both advance by a step's (dp pairs, ds segments), with
  // one compare for the segment wrap.
  constexpr uint32_t kSegBytes = 16 * kSliceStride * 4;
  uint32_t xa = lds_addr(xp) + (uint32_t)(j * kSliceStride * 4) + (uint32_t)cs0 * kSegBytes;
  const uint32_t xa_end = lds_addr(xp) + (uint32_t)(j * kSliceStride * 4) + (uint32_t)KS * kSegBytes;
  uint32_t pa = lds_addr(part) + (uint32_t)((((2 * cp0 + (j & 1)) * KS) + cs0) * 4);
  const uint32_t dxa = (uint32_t)ds * kSegBytes, wxa = (uint32_t)KS * kSegBytes;
  const uint32_t dpa = (uint32_t)((2 * dp * KS + ds) * 4), wpa = dpa + (uint32_t)(KS * 4);
  int cs = cs0;   // only needed to mask slices of a partial last segment
  // the staged scale of row 2 cp, group 4 cs + j / 4; the row below it and
  // the zeros at fixed distances; advancing like the activation slice
  // (unstaged: the lane's group in the ring slot, 4 bytes each at
  // task * 64 + 4 * (4 row + group), fetched by lanes 0..7 of its task)
  uint32_t sa = RS::stage ? lds_addr(lds + lay.sc) + (sz0 - sz_al) + (uint32_t)((2 * cp0 * G + 4 * cs0 + (j >> 2)) * 2)
                          : cur.slot0 + RS::codes + (lane & 48) * 4 + (j >> 2) * 4;
  const uint32_t srow = 2 * (uint32_t)G, zdist = (uint32_t)(lay.zr - lay.sc);
  const uint32_t dsa = (uint32_t)(2 * (2 * dp * G + 4 * ds)), wsa = dsa + (uint32_t)(2 * (2 * G - 4 * KS));
  const uint32_t ca16_l = cur.slot0 + lane * 16;
  const uint32_t ca4_l = cur.slot0 + (uint32_t)((lane >> 4) * (64 * BITS) + j * (4 * BITS));   // flat layouts
  constexpr uint32_t kStage = (TH / 64) * RS::slot;   // bytes between ring stages
  // one step i in ring slot D (a compile-time constant, so slot addresses fold)
  auto step = [&](auto dconst, int i) {
    constexpr int d = decltype(dconst)::value;
    {
      // wait for step i; the loads of steps i+1 .. min(i+R, steps)-1 may stay in flight
      wait_vmcnt_younger<R, Q>(min(R - 1, steps - 1 - i));
      if (rg + RG * i < T) {
        const bool sv = FULL || cs * 16 + j < S;
        TaskOps o;
        uint32_t cw[2][BITS];
        if constexpr (RS::stage)
          read_task<BITS>(sv ? xa : lds_addr(xp), sa, sa + srow, sa + zdist, sa + zdist + srow, ca16_l + d * kStage,
                          ca4_l + d * kStage, o, cw);
        else
          read_task<BITS>(sv ? xa : lds_addr(xp), sa + d * kStage, 0, 0, 0, ca16_l + d * kStage, ca4_l + d * kStage,
                          o, cw);
        uint32_t xv[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          xv[4 * q + 0] = o.x[q].x; xv[4 * q + 1] = o.x[q].y; xv[4 * q + 2] = o.x[q].z; xv[4 * q + 3] = o.x[q].w;
        }
        const float xsum = __builtin_bit_cast(float, (uint32_t)o.xq), xoff = __builtin_bit_cast(float, (uint32_t)(o.xq >> 32));
        const float xf = __builtin_bit_cast(float, o.xf);
        const float sc[2] = {half_bits_to_float(o.s0), half_bits_to_float(o.s1)};
        const float zc[2] = {half_bits_to_float(o.z0), half_bits_to_float(o.z1)};
        float a[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          uint32_t pr[16];
          unpack_pairs<BITS>(cw[r], uc, pr);
          // s * (sum (1024+q') x' - 1024 XS - z X) = s * sum (q - z) x
          float dd = fmaf(-zc[r], xsum, -xoff);
#pragma unroll
          for (int q = 0; q < 16; ++q) dd = dot2(pr[q], xv[q], dd);
          // one v_fma_mix with the fp16 scale; slices past K (partial last
          // segment) are dropped by a select, as their staged scale and
          // zero may be any bits
          a[r] = FULL ? fmaf(sc[r], dd, 0.0f) : sv ? fmaf(sc[r], dd, 0.0f) : 0.0f;
        }
        // both rows summed over the 16 lanes at once: after the first
        // exchange, even lanes carry row 0 and odd lanes row 1
        const bool odd = j & 1;
        float v = (odd ? a[1] : a[0]) + dpp<kQuadXor1>(odd ? a[0] : a[1]);
        v += dpp<kQuadXor2>(v);
        // the 4 lanes of a quad hold one 128-block, so one exponent: back to x' units
        v *= xf;
        v += dpp<kRowRor4>(v);
        v += dpp<kRowRor8>(v);
        if (j < 2) lds_store(pa, v);
        xa += dxa;
        const bool wrap = xa >= xa_end;
        xa = wrap ? xa - wxa : xa;
        pa += wrap ? wpa : dpa;
        if constexpr (RS::stage) sa += wrap ? wsa : dsa;
        if constexpr (!FULL) cs = wrap ? cs + ds - KS : cs + ds;
      }
      wait_lgkm0();   // this slot's bytes are in registers before it is refilled
      if (i + R < steps) cur.template issue<d>();
    }
  };
  for (int i0 = 0; i0 < steps; i0 += R) {
    step(std::integral_constant<int, 0>{}, i0);
    if constexpr (R > 1) if (i0 + 1 < steps) step(std::integral_constant<int, 1>{}, i0 + 1);
    if constexpr (R > 2) if (i0 + 2 < steps) step(std::integral_constant<int, 2>{}, i0 + 2);
    if constexpr (R > 3) if (i0 + 3 < steps) step(std::integral_constant<int, 3>{}, i0 + 3);
    if constexpr (R > 4) if (i0 + 4 < steps) step(std::integral_constant<int, 4>{}, i0 + 4);
    if constexpr (R > 5) if (i0 + 5 < steps) step(std::integral_constant<int, 5>{}, i0 + 5);
  }
  wait_vmcnt<0>();    // no load may still be writing LDS when the workgroup ends
  __syncthreads();

  // 4. add each row's partials in segment order, store
  for (int e = t; e < rows; e += TH) {
    float sum = 0.f;
    for (int s = 0; s < KS; ++s) sum += part[e * KS + s];
    store_out(L, 0, r0 + e, sum);
  }
}

// ---------------------------------------------------------------------------
// Batch tiles (2, 4, 8 or 16 rows): row quads, activations arranged once.
//
// With more than one batch row, rotating the activations in every
// workgroup would cost more than the workgroup's share of the product (each
// workgroup needs the whole K for every batch row), and a task of two rows
// would read every activation slice from LDS once per row.  So:
//   * one pre-pass (xprep_kernel) rotates each linear's activations once and
//     writes them in the LDS slice layout below (fp16 pairs in the order the
//     unpacker produces code pairs, the two slice sums in words 16 and 17);
//     each workgroup copies that block into LDS, its loads issued before the
//     first code loads so that waiting for them never waits for the weights;
//   * a 16-lane DPP row owns a "unit": one row quad and a contiguous range of
//     its 512-wide K segments (the whole K when the workgroup has at least
//     32 quads; otherwise p = 32 / quads DPP rows share a quad, one part of
//     K each).  It walks the unit's segments in order, keeping the 4 x MT
//     scaled partials of its lanes in registers;
//   * per segment a lane unpacks its 32-code slice of the four rows once,
//     then for each batch row reads the slice's activations once and feeds
//     all four rows (four v_dot2 chains per slice read); the chain starts
//     from the zero-point and offset correction, and the scale multiplies
//     the slice's sum into the accumulator;
//   * at the unit's end the partials are summed over the 16 lanes by a
//     reduce-scatter (each step halves the values a lane holds and pairs it
//     with a lane of the other half), leaving 4 MT / 16 values per lane
//     (one lane pair per value at MT 2), which go to LDS; the p parts of
//     each row are added in order at the end.
// 512-thread workgroups (two waves per SIMD) give each lane the registers
// for the four rows' unpacked codes and the 4 x MT partials.  At MT 8 and 16
// a lane reads one batch row's slice at a time (at 2 and 4 all of them ahead
// of the unpack).
// ---------------------------------------------------------------------------

constexpr int kQuadThreads = 512;
constexpr int kQRG = kQuadThreads / 16;   // DPP rows per workgroup

// One reduce-scatter step over V values: lanes whose `hi` bit is clear keep
// the lower half and receive their partner's lower half; the others the
// upper half.  CTRL pairs each lane with one in the other half.
template <int CTRL, int V, int N>
__device__ __forceinline__ void rs_step(float (&v)[N], bool hi) {
#pragma unroll
  for (int e = 0; e < V / 2; ++e) {
    const float keep = hi ? v[e + V / 2] : v[e];
    const float send = hi ? v[e] : v[e + V / 2];
    v[e] = keep + dpp<CTRL>(send);
  }
}

// Sum V (8, 16, 32 or 64) values over the 16 lanes of a DPP row.  Lane j
// ends with the sums of values (V / 16) j .. (V / 16) (j + 1) - 1 in v[0 ..]
// (V = 64: four values; 32: two; 16: one; V = 8: value j >> 1, lanes j and
// j ^ 1 alike).
template <int V, int N>
__device__ __forceinline__ void reduce_scatter16(float (&v)[N], int j) {
  static_assert(V == 8 || V == 16 || V == 32 || V == 64, "4 rows x 2, 4, 8 or 16 batch rows");
  rs_step<kRowRor8, V>(v, j & 8);
  rs_step<kRowHalfMirror, V / 2>(v, j & 4);
  rs_step<kQuadXor2, V / 4>(v, j & 2);
  if constexpr (V >= 16) {
    rs_step<kQuadXor1, V / 8>(v, j & 1);
  } else {
    v[0] += dpp<kQuadXor1>(v[0]);
  }
}

// DPP rows per quad: with fewer quads than DPP rows they share them, one
// contiguous part of the K segments each (at least one segment per part).
__host__ __device__ inline int quad_split(int nq, int ks) {
  const int p = nq >= kQRG ? 1 : kQRG / nq;
  return p < ks ? p : ks;
}

constexpr int kQuadMaxChunks = 4;
constexpr int kLdsWords = 160 * 1024 / 4;

// A workgroup's LDS: the arranged activations of one K chunk (kc segments
// of 16 slices, the last chunk shorter), the row parts of every unit and
// chunk, and the scales and zeros of the whole K.
struct QuadLds {
  int chunks, kc, p;      // K chunks of kc segments; DPP rows per quad
  int sc;                 // slices per batch row in the activation block
  int part, szl, total;   // 4-byte words
};

__host__ __device__ inline QuadLds quad_lds_at(int mt, int S, int KS, int G, int nq, int chunks) {
  QuadLds l;
  l.kc = (KS + chunks - 1) / chunks;
  l.chunks = (KS + l.kc - 1) / l.kc;
  l.p = quad_split(nq, KS - (l.chunks - 1) * l.kc);   // every chunk has a segment per part
  l.sc = S < 16 * l.kc ? S : 16 * l.kc;
  l.part = (mt * l.sc * kSliceStride + 3) & ~3;        // activations [mt][sc][20], sums in words 16, 17
  l.szl = (l.part + 4 * nq * l.p * l.chunks * mt + 1) & ~1;   // row parts [4 nq][chunks][p][mt]
  l.total = l.szl + ((4 * nq * G + 7) & ~7) * 2;      // scale, zero as fp32 [4 nq][G][2], whole groups of 8
  return l;
}

// The fewest K chunks (up to kQuadMaxChunks) whose layout fits in 160 KB.
__host__ __device__ inline QuadLds quad_lds(int mt, int S, int KS, int G, int nq) {
  QuadLds l = quad_lds_at(mt, S, KS, G, nq, 1);
  for (int c = 2; c <= kQuadMaxChunks && l.total > kLdsWords; ++c) l = quad_lds_at(mt, S, KS, G, nq, c);
  return l;
}

// Unit u (= quad q, part sub of p): its segments [s, e).  Quotients by p
// as (x * ceil(2^16 / p)) >> 16, exact for x < 2^16 / p (here x <= 32 KS
// or x = u with p = 1).
__device__ __forceinline__ void unit_range(int u, int p, uint32_t p_inv, int KS, int &q, int &s, int &e) {
  q = (int)(__umul24((uint32_t)u, p_inv) >> 16);
  const int sub = u - q * p;
  s = (int)(__umul24((uint32_t)(KS * sub), p_inv) >> 16);
  e = (int)(__umul24((uint32_t)(KS * (sub + 1)), p_inv) >> 16);
}

// A DPP row's walk over its tasks in one K chunk: the units rg, rg + 32,
// ... (quad q, part sub) over the chunk's segments, then idle steps (u at
// or past NU) up to the chunk's fixed step count T, so that every DPP row
// enters a chunk at the same step.
struct QuadWalk {
  int u, q, s, e;   // unit, quad, segment, the unit's end segment (absolute)
  int base, len;    // the chunk's first segment and segment count
};

struct QuadGeom {
  int rg, NU, p, KS, kc, T;   // T: steps per chunk, the same in every DPP row
  uint32_t p_inv;
};

__device__ __forceinline__ void walk_unit(const QuadGeom &g, QuadWalk &w) {
  unit_range(w.u, g.p, g.p_inv, w.len, w.q, w.s, w.e);
  w.s += w.base;
  w.e += w.base;
}

// the walk of chunk c (past the last chunk: idle throughout)
__device__ __forceinline__ void walk_start(const QuadGeom &g, QuadWalk &w, int c) {
  w.base = c * g.kc;
  w.len = min(g.kc, g.KS - w.base);
  w.u = w.len > 0 ? g.rg : g.NU;
  walk_unit(g, w);
}

__device__ __forceinline__ void walk_next(const QuadGeom &g, QuadWalk &w) {
  if (++w.s == w.e) {
    w.u += kQRG;
    walk_unit(g, w);
  }
}

template <int BITS, int MT, int D, bool CHUNKED, bool FULL>
__device__ __forceinline__ void stream_quads(const LinDesc &L, int m_valid, int r0, int rows, uint32_t *smem) {
  static_assert(MT == 2 || MT == 4 || MT == 8 || MT == 16, "batch tile");
  constexpr int ZL = 2;
  constexpr int XCH = MT <= 4 ? 3 * MT : MT == 8 ? 16 : 8;   // 8 KB copy passes held in registers
  const int t = threadIdx.x, rg = t >> 4, j = t & 15;
  const int K = L.k, KS = (K + kSeg - 1) / kSeg, G = K / kGroup, S = K / kSlice;
  const int wpr = S * BITS;
  const int NQ = (rows + 3) >> 2;
  const bool full = FULL || (K % kSeg) == 0;
  // the layout of a full workgroup (quad_lds, computed by the launcher): a
  // last workgroup with fewer quads keeps its split, as more DPP rows per
  // quad would need more room for row parts than the launch gave
  const int chunks = CHUNKED ? L.q_chunks : 1, p = L.q_p, NU = NQ * p, PC = p * chunks;
  QuadGeom geo;
  geo.rg = rg;
  geo.NU = NU;
  geo.p = p;
  geo.KS = KS;
  geo.kc = L.q_kc;
  geo.p_inv = L.q_pinv;
  geo.T = ((NU + kQRG - 1) / kQRG) * L.q_spu;
  geo.T = (geo.T + D - 1) / D * D;
  const int sc = L.q_sc;
  uint32_t *xp = smem;
  float *part = reinterpret_cast<float *>(smem + L.q_part);
  float *szl = reinterpret_cast<float *>(smem + L.q_szl);

  const rsrc_t rc = make_rsrc(L.codes + (size_t)r0 * wpr, (uint32_t)rows * wpr * 4);
  const int nszv = rows * G;
  const rsrc_t rsc = make_rsrc(L.scales + (size_t)r0 * G, (uint32_t)nszv * 2);
  const rsrc_t rz = make_rsrc(L.zeros + (size_t)r0 * G, (uint32_t)nszv * 2);

  // The activation block of chunk c: batch row m's slices [16 kc c, +sc) of
  // the arranged rows (S slices of 5 16-byte pieces each).  Piece x of the
  // block comes from piece (m S + 16 kc c) 5 + (x - 5 m sc), m = x / (5 sc)
  // by a 32-bit reciprocal (exact: x < 2^14).  With one chunk the block is
  // the arranged rows as they are.
  const uint32_t xrow = 5u * (uint32_t)sc;
  const uint32_t xrow_inv = L.q_xinv;
  const int xtotal = MT * sc * kSliceStride * 4;         // bytes of the LDS block
  const rsrc_t rxq = make_rsrc(L.xq, (uint32_t)(m_valid * S * kSliceStride * 4));
  auto x_src = [&](int off, int c) -> uint32_t {
    if (off >= xtotal) return kOOB;
    if constexpr (!CHUNKED) return (uint32_t)off;
    const uint32_t x = (uint32_t)off >> 4;
    const uint32_t m = __umulhi(x, xrow_inv);
    return ((m * (uint32_t)S + 16u * (uint32_t)(geo.kc * c)) * 5u + (x - m * xrow)) << 4;
  };
  auto x_load = [&](uint32_t src) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rxq, src, 0, 0));
  };

  // 1. scales and zeros, then the arranged activations of chunk 0 (batch
  //    rows past m_valid read zero), ahead of the weight stream
  const int nsz = 4 * NQ * G;               // scale/zero entries, padded to whole quads
  u32x4 sr[ZL], zr[ZL];
#pragma unroll
  for (int q = 0; q < ZL; ++q) {
    const int e0 = 8 * (t + kQuadThreads * q);
    sr[q] = load8_h(rsc, e0, nszv);
    zr[q] = load8_h(rz, e0, nszv);
  }
  // the first XCH 8 KB passes of the copy go to registers here and to LDS
  // once the code loads are out (their waits then cover these loads alone)
  u32x4 xr[XCH];
#pragma unroll
  for (int c = 0; c < XCH; ++c) xr[c] = x_load(x_src(16 * (t + kQuadThreads * c), 0));

  // 2. the first D steps of this DPP row's tasks
  const uint32_t seg_step = 16 * BITS * 4;
  const uint32_t row_bytes = (uint32_t)wpr * 4;
  const uint32_t quad_bytes = 4 * row_bytes;
  const uint32_t lane_off = (uint32_t)j * (BITS * 4);
  QuadWalk lw;                              // load side, D steps ahead
  walk_start(geo, lw, 0);
  uint32_t cw[D][4][BITS];
  auto issue = [&](uint32_t (&dst)[4][BITS]) {
    const bool ok = lw.u < NU && (full || lw.s * 16 + j < S);
    // past the range (kOOB + 3 rows stays above any buffer size): loads zero
    const uint32_t co =
        ok ? __umul24((uint32_t)lw.q, quad_bytes) + (uint32_t)lw.s * seg_step + lane_off : kOOB;
#pragma unroll
    for (int r = 0; r < 4; ++r) load_slice<BITS>(rc, co + r * row_bytes, dst[r]);
    walk_next(geo, lw);
  };
#pragma unroll
  for (int d = 0; d < D; ++d) issue(cw[d]);

  // 3. scales, zeros and activations into LDS
#pragma unroll
  for (int q = 0; q < ZL; ++q) {
    const int e0 = 8 * (t + kQuadThreads * q);
    if (e0 < nsz) {
      const uint32_t av[4] = {sr[q].x, sr[q].y, sr[q].z, sr[q].w};
      const uint32_t bv[4] = {zr[q].x, zr[q].y, zr[q].z, zr[q].w};
#pragma unroll
      for (int h = 0; h < 4; ++h)
        *reinterpret_cast<float4 *>(&szl[2 * (e0 + 2 * h)]) =
            make_float4(half_bits_to_float(av[h] & 0xFFFF), half_bits_to_float(bv[h] & 0xFFFF),
                        half_bits_to_float(av[h] >> 16), half_bits_to_float(bv[h] >> 16));
    }
  }
  for (int e0 = 8 * (t + kQuadThreads * ZL); e0 < nsz; e0 += 8 * kQuadThreads) {
    const u32x4 a = load8_h(rsc, e0, nszv);
    const u32x4 b = load8_h(rz, e0, nszv);
    const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int h = 0; h < 4; ++h)
      *reinterpret_cast<float4 *>(&szl[2 * (e0 + 2 * h)]) =
          make_float4(half_bits_to_float(av[h] & 0xFFFF), half_bits_to_float(bv[h] & 0xFFFF),
                      half_bits_to_float(av[h] >> 16), half_bits_to_float(bv[h] >> 16));
  }
#pragma unroll
  for (int c = 0; c < XCH; ++c) {
    const int off = 16 * (t + kQuadThreads * c);
    if (off < xtotal) *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(xp) + off) = xr[c];
  }
  for (int off = 16 * (t + kQuadThreads * XCH); off < xtotal; off += 16 * kQuadThreads)
    *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(xp) + off) = x_load(x_src(off, 0));
  __syncthreads();

  // 4. walk the units chunk by chunk: values r * MT + m accumulate
  //    s * sum (q - z) x over the unit's segments of the chunk
  const UnpackConsts uc = unpack_consts<BITS>();
  QuadWalk cw_;                             // compute side
  constexpr int NV = 4 * MT;   // partials of a unit: value r * MT + m
  float acc[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) acc[v] = 0.f;
  for (int c = 0; c < chunks; ++c) {
    if (CHUNKED && c > 0) {
      // every DPP row is done with chunk c - 1's activations: load chunk c's
      __syncthreads();
      for (int o0 = 16 * t; o0 < xtotal; o0 += 16 * kQuadThreads * XCH) {
#pragma unroll
        for (int h = 0; h < XCH; ++h) xr[h] = x_load(x_src(o0 + 16 * kQuadThreads * h, c));
#pragma unroll
        for (int h = 0; h < XCH; ++h) {
          const int off = o0 + 16 * kQuadThreads * h;
          if (off < xtotal) *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(xp) + off) = xr[h];
        }
      }
      __syncthreads();
    }
    const int xbase = 16 * geo.kc * c;      // the chunk's first slice
    walk_start(geo, cw_, c);
    for (int i0 = 0; i0 < geo.T; i0 += D) {
      // the refills of a chunk's last D steps issue the next chunk's first
      // (with one chunk the walk is idle past its units anyway)
      if (CHUNKED && i0 + D == geo.T) walk_start(geo, lw, c + 1);
#pragma unroll
      for (int d = 0; d < D; ++d) {
        if (cw_.u < NU) {
          const int slice = cw_.s * 16 + j;
          const bool sv = full || slice < S;
          const int sl = sv ? slice : xbase;
          const uint32_t zi = __umul24((uint32_t)(4 * cw_.q), (uint32_t)G) + (uint32_t)(sl >> 2);
          float sf[4], zf[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float2 sz = *reinterpret_cast<const float2 *>(&szl[2 * (zi + r * G)]);
            sf[r] = sv ? sz.x : 0.f;
            zf[r] = sz.y;
          }
          // the batch rows' activation slices (all of them up to 4 rows, read
          // before the unpack so their latency overlaps it; one at a time at 8)
          constexpr int XR = MT <= 4 ? MT : 1;
          uint32_t xv[XR][16];
          float2 xq[XR];
          auto read_x = [&](int m, int slot) {
            const uint32_t *src = &xp[(m * sc + sl - xbase) * kSliceStride];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const u32x4 v = reinterpret_cast<const u32x4 *>(src)[q];
              xv[slot][4 * q + 0] = v.x; xv[slot][4 * q + 1] = v.y; xv[slot][4 * q + 2] = v.z; xv[slot][4 * q + 3] = v.w;
            }
            xq[slot] = *reinterpret_cast<const float2 *>(src + 16);
          };
          if constexpr (MT <= 4) {
#pragma unroll
            for (int m = 0; m < MT; ++m) read_x(m, m);
          }
          uint32_t pr[4][16];
#pragma unroll
          for (int r = 0; r < 4; ++r) unpack_pairs<BITS>(cw[d][r], uc, pr[r]);
          // s * (sum (1024+q') x' - 1024 XS - z X) = s * sum (q - z) x
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const int xs = MT <= 4 ? m : 0;
            if constexpr (MT > 4) read_x(m, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float dd = fmaf(-zf[r], xq[xs].x, -xq[xs].y);
#pragma unroll
              for (int q = 0; q < 16; ++q) dd = dot2(pr[r][q], xv[xs][q], dd);
              acc[r * MT + m] = fmaf(sf[r], dd, acc[r * MT + m]);
            }
          }
          if (cw_.s + 1 == cw_.e) {
            // the unit's share of the chunk is done: its row parts over the
            // 16 lanes, NV / 16 per lane (one per lane pair at NV = 8)
            reduce_scatter16<NV>(acc, j);
            const int slot = c * p + (cw_.u - cw_.q * p);
            if constexpr (NV == 8) {
              const int vi = j >> 1;
              if ((j & 1) == 0) part[((4 * cw_.q + vi / MT) * PC + slot) * MT + vi % MT] = acc[0];
            } else {
#pragma unroll
              for (int e = 0; e < NV / 16; ++e) {
                const int vi = (NV / 16) * j + e;
                part[((4 * cw_.q + vi / MT) * PC + slot) * MT + vi % MT] = acc[e];
              }
            }
#pragma unroll
            for (int v2 = 0; v2 < NV; ++v2) acc[v2] = 0.f;
          }
        }
        walk_next(geo, cw_);
        // refill this buffer with the task D steps ahead
        issue(cw[d]);
      }
    }
  }
  __syncthreads();

  // 5. add each row's parts in order (chunk, then part), remove the batch
  //    row's activation exponent (the factor 2^-E in word 18 of each of its
  //    slices), store
  for (int e = t; e < rows * m_valid; e += kQuadThreads) {
    const int row = e / m_valid, m = e % m_valid;
    float sum = 0.f;
    for (int u = 0; u < PC; ++u) sum += part[(row * PC + u) * MT + m];
    store_out(L, m, r0 + row, sum * __builtin_bit_cast(float, L.xq[(size_t)m * S * kSliceStride + 18]));
  }
}

// The pre-pass of the batch-tile kernels: every linear's activations, all m
// rows, rotated (when the linear has signs) and arranged in the slice layout
// [m][K/32][20 words].  One exponent per batch row, so that the batch-tile
// kernel removes it from each output once (its partials add slices of many
// blocks in registers).  The exponent comes from a bound on the row's
// rotated values that needs no rotation: a rotated value is a sum of 128
// signed values over sqrt(128), so |x'| <= sqrt(128) max |x| (max |x| itself
// without rotation); E puts that bound in [2^14, 2^15), which keeps every
// stored value below 2^15 and the row's largest one at 2^7 or more.  So
// each workgroup of one wave can take its own 512-wide chunk of a row (one
// 128-block per DPP row) and still agree on E with the row's other chunks:
// it reads the whole row for the maximum (lane L's loads cover elements
// 512 i + 8 L .. + 7, and load i = its chunk holds its own elements), then
// rotates and stores its four blocks.  Workgroups per (linear, batch row):
// ceil(K / 512), dealt by a packed table of first workgroups.
constexpr int kXprepThreads = 64;
constexpr int kXprepAhead = 20;   // chunks of a row loaded at once (K up to 10240)

struct XprepMat {
  const uint16_t *x;
  uint32_t *out;
  const uint32_t *signs;
  int64_t ldx;
  int32_t k, m, chunks, wg_begin;
};

struct XprepBatch {
  int32_t first_wg[kMaxBatch];   // mat[i].wg_begin, packed; INT32_MAX past count
  XprepMat mat[kMaxBatch];
};

// Largest |value| of the eight fp16 values in v.
__device__ __forceinline__ float absmax8h(u32x4 v) {
  const uint32_t a = v.x & 0x7FFF7FFFu, b = v.y & 0x7FFF7FFFu, c = v.z & 0x7FFF7FFFu, d = v.w & 0x7FFF7FFFu;
  // magnitudes of finite fp16 values order as their bit patterns
  const uint32_t lo = max(max(a & 0xFFFFu, b & 0xFFFFu), max(c & 0xFFFFu, d & 0xFFFFu));
  const uint32_t hi = max(max(a >> 16, b >> 16), max(c >> 16, d >> 16));
  return half_bits_to_float(max(lo, hi));
}

template <int BITS>
__global__ __launch_bounds__(kXprepThreads) void xprep_kernel(XprepBatch a) {
  const int w = blockIdx.x;
  int l = 0;
#pragma unroll
  for (int i = 1; i < kMaxBatch; ++i)
    if (w >= a.first_wg[i]) l = i;
  const XprepMat M = a.mat[l];
  const int local = w - M.wg_begin, m = local / M.chunks, c = local - m * M.chunks;
  const int nb = M.k / kGroup, S = M.k / kSlice;
  const int lane = threadIdx.x, jj = lane & 15, b = 4 * c + (lane >> 4);
  const bool rotate = M.signs != nullptr;
  const rsrc_t rx = make_rsrc(M.x + (size_t)m * M.ldx, (uint32_t)M.k * 2u);   // elements past K read zero
  // the first kXprepAhead chunks' loads all go out before any is used (one
  // round of load latency for K up to 512 kXprepAhead); chunks past the row
  // read zero
  float mx = 0.f;
  u32x4 mine = u32x4{0u, 0u, 0u, 0u};
  u32x4 rowv[kXprepAhead];
#pragma unroll
  for (int i = 0; i < kXprepAhead; ++i)
    rowv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)(1024 * i + 16 * lane), 0, 0));
  __builtin_amdgcn_sched_barrier(0);   // every load out before the first use
#pragma unroll
  for (int i = 0; i < kXprepAhead; ++i) {
    mx = fmaxf(mx, absmax8h(rowv[i]));
    mine = i == c ? rowv[i] : mine;
  }
  for (int i = kXprepAhead; i < M.chunks; ++i) {
    const u32x4 u = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)(1024 * i + 16 * lane), 0, 0));
    mx = fmaxf(mx, absmax8h(u));
    if (i == c) mine = u;
  }
  mx = row16_max(mx);
  mx = fmaxf(fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx), 0)),
                   __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx), 16))),
             fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx), 32)),
                   __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx), 48))));
  const int E = act_exponent(rotate ? mx * 11.313708498984761f : mx);   // sqrt(128) max |x|
  if (b >= nb) return;   // uniform over the 16 lanes of a DPP row
  const int kk = 128 * b + 8 * jj;
  float v[8];
  load_rotated8(rotate, mine, rotate ? M.signs[kk >> 5] : 0u, kk, jj, v);
  uint32_t o[4];
  float xe, xt;
  arrange8<BITS>(rotate, v, jj, E, o, xe, xt);
  store_slice_part(M.out + ((size_t)m * S + (size_t)(4 * b + (jj >> 2))) * kSliceStride, jj, o, xe, xt, E);
}

template <int BITS, bool FULL>
__global__ __launch_bounds__(Ring<BITS>::threads) void gemv_ring_kernel(int t1, int t2, int t3, int t4, int t5, int t6, int t7, GemvArgs a) {
  extern __shared__ uint32_t smem[];
  const int w = blockIdx.x;
  const LinDesc L = fetch_desc(a, w, FirstTiles{t1, t2, t3, t4, t5, t6, t7});
  const int r0 = (w - L.tile_begin) * L.rows_per_wg;
  if (r0 >= L.n) return;
  ActAhead<kActAhead<BITS>> ahead;
  act_ahead_loads<kActAhead<BITS>, Ring<BITS>::threads>(L, ahead);
  stream_ring<BITS, FULL>(L, L.codes + (size_t)r0 * (L.k / kSlice) * BITS, r0, min(L.rows_per_wg, L.n - r0), smem,
                          ahead);
}


// Tasks (two code loads each) a lane keeps in flight.  A 1024-thread
// workgroup per CU with 4 tasks per lane has 128 KB of int4 codes in flight,
// twice what HBM latency times a CU's share of bandwidth needs; deeper
// rings would spill under the 128-VGPR limit of 1024-thread workgroups.
template <int BITS, int MT>
struct Depth {
  static constexpr int d = MT == 1 ? (BITS <= 4 ? 4 : 3) : (MT == 2 ? (BITS <= 4 ? 3 : 2) : 2);
};

template <int BITS, int MT>
__global__ __launch_bounds__(kStreamThreads) void gemv_stream_kernel(int t1, int t2, int t3, int t4, int t5, int t6, int t7, GemvArgs a) {
  extern __shared__ uint32_t smem[];
  const int w = blockIdx.x;
  const LinDesc L = fetch_desc(a, w, FirstTiles{t1, t2, t3, t4, t5, t6, t7});
  const int r0 = (w - L.tile_begin) * L.rows_per_wg;
  if (r0 >= L.n) return;
  const int rows = min(L.rows_per_wg, L.n - r0);
  stream_rows<BITS, MT, Depth<BITS, MT>::d>(L, L.codes + (size_t)r0 * (L.k / kSlice) * BITS, a.m, r0, rows, smem);
}

// The mixed 6/8-bit layout at batch 1: every workgroup streams rows of one
// width, on the LDS ring of that width.  Blocks of one width that follow
// each other form a run, whose rows lie one after another at one row
// stride: a run is one uniform-width matrix.  With mixed_wpb == 0 the
// grid's G workgroups are spread over the runs in proportion to their code
// words: run [bs, be) gets the workgroups w with F(off[bs]) <= w <
// F(off[be]), F(o) = floor(G o / off[nblk]), and its row pairs are split
// evenly among them, so every workgroup streams about the same bytes in
// about as many ring steps as the uniform kernel takes for that width.
// (Splitting each 64-row block on its own instead left 10- and 11-row
// workgroups beside each other; 11 rows are 6 row pairs, a ring step more
// than 5: the all-6-bit layout took 8.85 us against 6.70 us for the same
// matrix on the uniform kernel.)  The host takes this only when every
// block gets at least one workgroup (G >= 4/3 blocks), so every run does.
// With mixed_wpb == 1 each workgroup takes one whole block.  Without the
// caller's host copy of the widths the kernel finds its run in the block
// table; with it, the host places the workgroups
// (gemv_ring_mixed_table_kernel).
static_assert(kActAhead<6> == kActAhead<8>, "both widths take the same activation loads");

// One pass of the run search over blocks c .. c + 63, one lane per block:
// its width, its predecessor's width and its first word.
struct MixedPass {
  int bits, prev;
  uint64_t off;
};

__device__ __forceinline__ MixedPass mixed_pass_loads(const LinDesc &L, int nblk, int c) {
  const int b = c + (int)(threadIdx.x & 63);
  MixedPass p{0, 0, 0};
  if (b < nblk) {
    p.bits = L.block_bits[b];
    p.prev = b > 0 ? L.block_bits[b - 1] : 0;
    p.off = L.block_off[b];
  }
  return p;
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), l) << 32) |
         (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
}

template <bool FULL>
__global__ __launch_bounds__(kRingThreads) void gemv_ring_mixed_kernel(GemvArgs a) {
  extern __shared__ uint32_t smem[];
  const int g = blockIdx.x;   // one linear: its workgroups are the grid
  const LinDesc L = a.lin[0];
  asm volatile("" ::"s"(L.codes), "s"(L.scales), "s"(L.zeros), "s"(L.signs), "s"(L.x), "s"(L.y), "s"(L.n),
               "s"(L.k), "s"(L.block_bits), "s"(L.block_off), "s"(a.tiles), "s"(a.mixed_wpb));
  const int nblk = L.n / kMixedRows;
  const bool spread = a.mixed_wpb == 0;
  // The block table's loads (the search's first pass, or the block of a
  // one-block workgroup) go out before the activations: vector loads
  // return in order, and the two ways to the run meet before the ring
  // starts, where the compiler waits for every vector load either issued.
  // Every other value the search needs comes from the lanes holding it.
  // (Even so the search holds the ring back: the all-6-bit down_proj takes
  // 7.5 us here against 6.7 us for the same rows placed by the host in
  // gemv_ring_mixed_table_kernel.)
  MixedPass p0{0, 0, 0};
  uint64_t tot = 0, off1 = 0;
  int bits1 = 0;
  if (!spread) {
    bits1 = L.block_bits[g];
    off1 = L.block_off[g];
  } else {
    p0 = mixed_pass_loads(L, nblk, 0);
    tot = L.block_off[nblk];
  }
  asm volatile("" ::: "memory");
  ActAhead<kActAhead<6>> ahead;
  act_ahead_loads(L, ahead);
  int blk, r0, rows, bits;
  uint64_t off;
  if (!spread) {
    blk = g;
    r0 = 0;
    rows = kMixedRows;
    bits = bits1;
    off = off1;
  } else {
    // bs: the last run start with F(off[bs]) <= w; be: the first run start
    // after it (nblk, at word tot, if none)
    const int lane = threadIdx.x & 63;
    const double G = (double)a.tiles, T = (double)tot;
    int bs = -1, be = nblk;
    uint64_t off_e = tot;
    off = 0;
    bits = 0;
    for (int c = 0; c < nblk; c += 64) {
      const MixedPass p = c == 0 ? p0 : mixed_pass_loads(L, nblk, c);
      const bool start = c + lane < nblk && (c + lane == 0 || p.bits != p.prev);
      const int lo = (int)floor((double)p.off * G / T);
      const uint64_t before = __ballot(start && lo <= g), after = __ballot(start && lo > g);
      if (before) {
        const int l = 63 - __builtin_clzll(before);
        bs = c + l;
        off = readlane64(p.off, l);
        bits = __builtin_amdgcn_readlane(p.bits, l);
      }
      if (after) {
        const int l = __builtin_ctzll(after);
        be = c + l;
        off_e = readlane64(p.off, l);
        break;
      }
    }
    if (bs < 0) return;   // block 0 starts a run at F = 0 <= w: not reached
    // the run's workgroups and this one's index; every block of the run
    // brings at least one workgroup (wr >= be - bs), so a workgroup gets at
    // most 64 rows, what the host sized the LDS for
    const int lo = (int)floor((double)off * G / T), hi = (int)floor((double)off_e * G / T);
    const int wr = hi - lo, sub = g - lo;
    const int64_t pairs = (int64_t)(kMixedRows / 2) * (be - bs);
    const int q0 = (int)(pairs * sub / wr), q1 = (int)(pairs * (sub + 1) / wr);
    blk = bs;
    r0 = 2 * q0;
    rows = 2 * (q1 - q0);
  }
  // the same on every lane: say so, so that the ring's cursor, loop counts
  // and waits stay scalar as in the uniform kernel (as vector values they
  // cost 0.3 us on the down_proj)
  blk = __builtin_amdgcn_readfirstlane(blk);
  r0 = __builtin_amdgcn_readfirstlane(r0);
  rows = __builtin_amdgcn_readfirstlane(rows);
  bits = __builtin_amdgcn_readfirstlane(bits);
  off = readlane64(off, 0);
  if (rows <= 0) return;
  const uint32_t *codes0 = L.codes + off + (size_t)r0 * (L.k / kSlice) * bits;
  r0 += kMixedRows * blk;
  if (bits == 8)
    stream_ring<8, FULL>(L, codes0, r0, rows, smem, ahead);
  else
    stream_ring<6, FULL>(L, codes0, r0, rows, smem, ahead);
}

// The same with every workgroup placed by the host (from the caller's host
// copy of the widths): its record and the next one, read with the launch
// arguments, give its first code word, rows and width, so the ring starts
// right behind the activation loads, as in the uniform kernel.
template <bool FULL>
__global__ __launch_bounds__(kRingThreads) void gemv_ring_mixed_table_kernel(MixedArgs a) {
  extern __shared__ uint32_t smem[];
  const int g = blockIdx.x;
  const LinDesc L = a.lin;
  const uint64_t e0 = a.wg[g], e1 = a.wg[g + 1];
  asm volatile("" ::"s"(L.codes), "s"(L.scales), "s"(L.zeros), "s"(L.signs), "s"(L.x), "s"(L.y), "s"(L.n),
               "s"(L.k), "s"(e0), "s"(e1));
  ActAhead<kActAhead<6>> ahead;
  act_ahead_loads(L, ahead);
  const int r0 = (int)((uint32_t)(e0 >> 32) & 0x7FFFFFFFu);
  const int rows = (int)((uint32_t)(e1 >> 32) & 0x7FFFFFFFu) - r0;
  if (rows <= 0) return;
  const uint32_t *codes0 = L.codes + (uint32_t)e0;
  if (e0 >> 63)
    stream_ring<8, FULL>(L, codes0, r0, rows, smem, ahead);
  else
    stream_ring<6, FULL>(L, codes0, r0, rows, smem, ahead);
}

// Segments of code loads a lane keeps in flight (4 rows x BITS words each);
// deeper prefetch measured no faster, as most of a wave's segments are
// then requested at once at the start.
template <int BITS>
struct QDepth {
  static constexpr int d = 2;
};

template <int BITS, int MT, bool CHUNKED, bool FULL>
__global__ __launch_bounds__(kQuadThreads) void gemv_quad_kernel(int t1, int t2, int t3, int t4, int t5, int t6, int t7, GemvArgs a) {
  extern __shared__ uint32_t smem[];
  const int w = blockIdx.x;
  const LinDesc L = fetch_desc(a, w, FirstTiles{t1, t2, t3, t4, t5, t6, t7});
  asm volatile("" ::"s"(L.q_chunks), "s"(L.q_kc), "s"(L.q_p), "s"(L.q_spu), "s"(L.q_pinv), "s"(L.q_sc),
               "s"(L.q_xinv), "s"(L.q_part), "s"(L.q_szl));
  const int r0 = (w - L.tile_begin) * L.rows_per_wg;
  if (r0 >= L.n) return;
  stream_quads<BITS, MT, QDepth<BITS>::d, CHUNKED, FULL>(L, a.m, r0, min(L.rows_per_wg, L.n - r0), smem);
}

// the chunk-walking kernel only where some linear's activations need chunks;
// the partial-segment masks only where some linear's K is not a multiple of
// 512 (the int4 block at 4 rows: 22.56 -> 22.13 us without them)
template <int BITS, int MT>
hipError_t launch_quad(const GemvArgs &a, hipStream_t s) {
  bool chunked = false, full = true;
  for (int i = 0; i < a.count; ++i) {
    chunked = chunked || a.lin[i].q_chunks > 1;
    full = full && a.lin[i].k % kSeg == 0;
  }
#define WQ_QUAD(C, F) hipLaunchKernelGGL((gemv_quad_kernel<BITS, MT, C, F>), dim3(a.tiles), dim3(kQuadThreads), a.lds_bytes, s, a.first_tile[1], a.first_tile[2], a.first_tile[3], a.first_tile[4], a.first_tile[5], a.first_tile[6], a.first_tile[7], a)
  if (chunked && full) WQ_QUAD(true, true);
  else if (chunked) WQ_QUAD(true, false);
  else if (full) WQ_QUAD(false, true);
  else WQ_QUAD(false, false);
#undef WQ_QUAD
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(int mt, const GemvArgs &a, hipStream_t s) {
  if (a.ring) {
    if (mt != 1) return hipErrorInvalidValue;
    bool full = true;
    for (int i = 0; i < a.count; ++i) full = full && a.lin[i].k % kSeg == 0;
    if (full)
      hipLaunchKernelGGL((gemv_ring_kernel<BITS, true>), dim3(a.tiles), dim3(Ring<BITS>::threads), a.lds_bytes, s, a.first_tile[1], a.first_tile[2], a.first_tile[3], a.first_tile[4], a.first_tile[5], a.first_tile[6], a.first_tile[7], a);
    else
      hipLaunchKernelGGL((gemv_ring_kernel<BITS, false>), dim3(a.tiles), dim3(Ring<BITS>::threads), a.lds_bytes, s, a.first_tile[1], a.first_tile[2], a.first_tile[3], a.first_tile[4], a.first_tile[5], a.first_tile[6], a.first_tile[7], a);
    return hipGetLastError();
  }
  switch (mt) {
    case 1:
      hipLaunchKernelGGL((gemv_stream_kernel<BITS, 1>), dim3(a.tiles), dim3(kStreamThreads), a.lds_bytes, s, a.first_tile[1], a.first_tile[2], a.first_tile[3], a.first_tile[4], a.first_tile[5], a.first_tile[6], a.first_tile[7], a);
      break;
    case 2: return launch_quad<BITS, 2>(a, s);
    case 4: return launch_quad<BITS, 4>(a, s);
    case 8: return launch_quad<BITS, 8>(a, s);
    case 16: return launch_quad<BITS, 16>(a, s);
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int gemv_stream_lds_bytes(int bits, int mt, int64_t k, int rows_per_wg, bool ring) {
  const int64_t S = k / kSlice, KS = (k + kSeg - 1) / kSeg, G = k / kGroup;
  const int64_t np = (rows_per_wg + 1) / 2;
  if (S * kSliceStride * mt + np * (KS + G) * 4 * mt > (int64_t)1 << 26) return 1 << 30;
  if (!ring && mt >= 2) return quad_lds(mt, (int)S, (int)KS, (int)G, (rows_per_wg + 3) / 4).total * 4;
  if (!ring) return stream_lds(mt, (int)S, (int)KS, (int)G, (int)np).total * 4;
  if (mt != 1) return 1 << 30;
  // the staged scales and zeros (8-bit rows) must lie within the loads' reach
  if ((bits == 8 || bits == 0) && (int64_t)ring_sz_items((int)np, (int)G) > (int64_t)64 * kRingSzLoads * (kRingThreads / 64))
    return 1 << 30;
  const int s = (int)S, ks = (int)KS, n = (int)np, g = (int)G;
  auto need = [&](auto ring) {
    using RS = decltype(ring);
    return ring_lds(s, ks, n, g, RS::slot, RS::depth, RS::waves, RS::stage).total;
  };
  switch (bits) {
    case 0: return std::max(need(Ring<6>{}), need(Ring<8>{}));   // mixed 6/8: room for either ring
    case 3: return need(Ring<3>{});
    case 4: return need(Ring<4>{});
    case 6: return need(Ring<6>{});
    case 8: return need(Ring<8>{});
  }
  return 1 << 30;
}

hipError_t launch_xprep(int bits, int count, const uint16_t *const *x, const int64_t *ldx,
                        const uint32_t *const *signs, const int64_t *k, int64_t m, uint32_t *const *out,
                        hipStream_t s) {
  if (count <= 0 || count > kMaxBatch || m <= 0) return hipErrorInvalidValue;
  XprepBatch a;
  memset(&a, 0, sizeof a);
  for (int i = 0; i < kMaxBatch; ++i) a.first_wg[i] = INT32_MAX;
  int64_t wgs = 0;
  for (int i = 0; i < count; ++i) {
    XprepMat &M = a.mat[i];
    M.x = x[i];
    M.out = out[i];
    M.signs = signs[i];
    M.ldx = ldx[i];
    M.k = (int32_t)k[i];
    M.m = (int32_t)m;
    M.chunks = (int32_t)((k[i] + 511) / 512);
    M.wg_begin = (int32_t)wgs;
    a.first_wg[i] = (int32_t)wgs;
    wgs += m * M.chunks;   // one workgroup per batch row and 512-wide chunk
  }
  if (wgs > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)wgs), block(kXprepThreads);
  switch (bits) {
    case 3: hipLaunchKernelGGL(xprep_kernel<3>, grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL(xprep_kernel<4>, grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL(xprep_kernel<6>, grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL(xprep_kernel<8>, grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemv_mixed_table(const MixedArgs &a, hipStream_t s) {
  if (a.tiles < 1 || a.tiles > kMixedTableWgs) return hipErrorInvalidValue;
  if (a.lin.k % kSeg == 0)
    hipLaunchKernelGGL((gemv_ring_mixed_table_kernel<true>), dim3(a.tiles), dim3(kRingThreads), a.lds_bytes, s, a);
  else
    hipLaunchKernelGGL((gemv_ring_mixed_table_kernel<false>), dim3(a.tiles), dim3(kRingThreads), a.lds_bytes, s, a);
  return hipGetLastError();
}

hipError_t launch_gemv_stream(int bits, int mt, const GemvArgs &a, hipStream_t s) {
  if (bits == 0) {
    if (!a.ring || mt != 1 || a.count != 1 || a.mixed_wpb < 0 || a.mixed_wpb > 1) return hipErrorInvalidValue;
    if (a.lin[0].k % kSeg == 0)
      hipLaunchKernelGGL((gemv_ring_mixed_kernel<true>), dim3(a.tiles), dim3(kRingThreads), a.lds_bytes, s, a);
    else
      hipLaunchKernelGGL((gemv_ring_mixed_kernel<false>), dim3(a.tiles), dim3(kRingThreads), a.lds_bytes, s, a);
    return hipGetLastError();
  }
  if (a.ring || mt < 2) {
    switch (bits) {
      case 3: return launch_bits<3>(mt, a, s);
      case 4: return launch_bits<4>(mt, a, s);
      case 6: return launch_bits<6>(mt, a, s);
      case 8: return launch_bits<8>(mt, a, s);
    }
    return hipErrorInvalidValue;
  }
  // batch tiles: each linear's layout of a full workgroup, which must fit
  // in the LDS the launch gives
  GemvArgs b = a;
  for (int i = 0; i < a.count; ++i) {
    LinDesc &L = b.lin[i];
    const int S = L.k / kSlice, KS = (L.k + kSeg - 1) / kSeg, G = L.k / kGroup;
    const QuadLds l = quad_lds(mt, S, KS, G, (L.rows_per_wg + 3) / 4);
    if (l.total > kLdsWords || l.total * 4 > a.lds_bytes) return hipErrorInvalidValue;
    L.q_chunks = l.chunks;
    L.q_kc = l.kc;
    L.q_p = l.p;
    L.q_spu = (l.kc + l.p - 1) / l.p;
    L.q_pinv = (65536u + (uint32_t)l.p - 1u) / (uint32_t)l.p;
    L.q_sc = l.sc;
    L.q_xinv = 0xFFFFFFFFu / (5u * (uint32_t)l.sc) + 1u;
    L.q_part = l.part;
    L.q_szl = l.szl;
  }
  switch (bits) {
    case 3: return launch_bits<3>(mt, b, s);
    case 4: return launch_bits<4>(mt, b, s);
    case 6: return launch_bits<6>(mt, b, s);
    case 8: return launch_bits<8>(mt, b, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace wq

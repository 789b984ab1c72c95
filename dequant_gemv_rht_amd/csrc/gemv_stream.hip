// Persistent fused rotation + dequantising GEMV for batch tiles up to 4
// (gfx950).  Same arithmetic as the tiled kernel (gemv.hip): codes become
// fp16 (1024 + q) in registers, v_dot2_f32_f16 accumulates against the
// rotated fp16 activations, the scale multiplies each 32-code partial once
// and the zero point (plus the 1024 offset) is removed with the partial's
// activation sum.  Source of the arithmetic: model card "24B0978 - Week 01 -
// Track 2, 20% target", section "How these techniques accelerate inference
// on CUDA" (group-wise affine codes dequantised inside the product, scale
// applied once per group; activations rotated by a fast Walsh-Hadamard
// transform at run time).
//
// Work decomposition.  One 1024-thread workgroup per compute unit.  Each
// linear of a launch gets a number of workgroups proportional to its bytes,
// and each workgroup a contiguous range of rows.  A workgroup
//   1. rotates its linear's activations for the whole K once into LDS (the
//      rotation is paid once per workgroup, not once per tile);
//   2. splits its (row pair, 512-wide K segment) tasks into 64 contiguous,
//      equal runs, one per 16-lane DPP row;
//   3. streams each run with D tasks of code, scale and zero loads in flight
//      (raw buffer loads: out-of-range lanes read zero without memory
//      traffic, so every load is issued on a straight-line path);
//   4. accumulates consecutive segments of a row pair in registers, sums the
//      16 lanes by DPP when the pair (or the run) ends, and leaves the
//      partial in LDS at [row][first segment of the run piece];
//   5. adds each row's partials in segment order (deterministic) and stores.
//
// Unpacking.  A code pair becomes two fp16 values (1024 + q) with one
// v_and_or_b32 against 1024.0's bit pattern.  For int4, nibbles in bits 4..7
// of a 16-bit half are used in place: they read as (1024 + 16 q), so their
// activations are stored pre-divided by 16 (exact in fp16), which saves two
// of the three shifts per word.  int8 uses one v_perm_b32 per pair.  The
// offsets are removed with two per-slice activation sums: X (the sum of the
// effective activations, for the zero point) and XS (1024 times the sum of
// the stored values, the 1024 offsets).
//
// LDS layout.  Each 32-code activation slice occupies 80 bytes (64 used):
// with that stride the 16 lanes of a DPP row reading their slices with
// ds_read_b128 hit 16 distinct 4-bank groups.
#include "wq_internal.h"

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
  uint32_t mask, bias;
};

// Constants kept in VGPRs so each code pair costs one v_and_or_b32 (gfx9
// VOP3 instructions cannot take two literal constants).
template <int BITS>
__device__ __forceinline__ UnpackConsts unpack_consts() {
  constexpr uint32_t m = BITS == 4 ? 0x000F000Fu : BITS == 8 ? 0x00FF00FFu : BITS == 3 ? 0x00070007u : 0x003F003Fu;
  constexpr uint32_t b = BITS == 8 ? 0x64646464u : kBias;
  UnpackConsts c;
  asm volatile("v_mov_b32 %0, %1" : "=v"(c.mask) : "i"(m));
  asm volatile("v_mov_b32 %0, %1" : "=v"(c.bias) : "i"(b));
  return c;
}

// Code pair P of a 32-code slice as two fp16 values.
template <int BITS, int P>
__device__ __forceinline__ uint32_t pair_at(const uint32_t (&w)[BITS], UnpackConsts c) {
  if constexpr (BITS == 4) {
    // word P/4: r=0 codes (0,4), r=1 codes (1,5) read as 1024+16q, r=2
    // codes (2,6), r=3 codes (3,7) read as 1024+16q
    constexpr int wi = P / 4, r = P % 4;
    const uint32_t v = (r < 2) ? w[wi] : (w[wi] >> 8);
    return (r & 1) ? ((v & (c.mask << 4)) | c.bias) : ((v & c.mask) | c.bias);
  } else if constexpr (BITS == 8) {
    // word P/2: bytes (r, r+2) next to 0x64 bytes -> (1024 + q) each
    constexpr int wi = P / 2, r = P % 2;
    return __builtin_amdgcn_perm(c.bias, w[wi], r ? 0x04030401u : 0x04020400u);
  } else if constexpr (BITS == 3) {
    const uint32_t t = field<6 * P, 6>(w);       // codes 2P, 2P+1: bits [6P, 6P+6)
    return ((t | (t << 13)) & c.mask) | c.bias;
  } else {
    constexpr int run = P / 8, q = P % 8;         // two 96-bit runs of 16 codes
    const uint32_t t = (run == 0) ? field<12 * q, 12>(w) : field<96 + 12 * q, 12>(w);
    return ((t | (t << 10)) & c.mask) | c.bias;
  }
}

template <int BITS, int P = 0>
__device__ __forceinline__ void unpack_pairs(const uint32_t (&w)[BITS], UnpackConsts c, uint32_t (&p)[16]) {
  p[P] = pair_at<BITS, P>(w, c);
  if constexpr (P + 1 < 16) unpack_pairs<BITS, P + 1>(w, c, p);
}

// fp16 activation pairs in the order unpack_pairs produces code pairs (the
// lane's 8 values are codes 8w..8w+7 of its 32-code slice), and their
// contribution to the slice sums: x_eff (what multiplies q) and x_st (what
// multiplies the 1024 offset).
template <int BITS>
__device__ __forceinline__ void pairs_in_dot_order(const float (&v)[8], uint32_t (&o)[4], float &x_eff,
                                                   float &x_st) {
  if constexpr (BITS == 4) {
    constexpr float k16 = 0.0625f;
    o[0] = pack_half2(v[0], v[4]); o[1] = pack_half2(v[1] * k16, v[5] * k16);
    o[2] = pack_half2(v[2], v[6]); o[3] = pack_half2(v[3] * k16, v[7] * k16);
    const float a = half_bits_to_float(o[0] & 0xFFFF) + half_bits_to_float(o[0] >> 16) +
                    half_bits_to_float(o[2] & 0xFFFF) + half_bits_to_float(o[2] >> 16);
    const float b = half_bits_to_float(o[1] & 0xFFFF) + half_bits_to_float(o[1] >> 16) +
                    half_bits_to_float(o[3] & 0xFFFF) + half_bits_to_float(o[3] >> 16);
    x_eff = a + 16.0f * b;
    x_st = a + b;
  } else {
    if constexpr (BITS == 8) {
      o[0] = pack_half2(v[0], v[2]); o[1] = pack_half2(v[1], v[3]);
      o[2] = pack_half2(v[4], v[6]); o[3] = pack_half2(v[5], v[7]);
    } else {
      o[0] = pack_half2(v[0], v[1]); o[1] = pack_half2(v[2], v[3]);
      o[2] = pack_half2(v[4], v[5]); o[3] = pack_half2(v[6], v[7]);
    }
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) a += half_bits_to_float(o[e] & 0xFFFF) + half_bits_to_float(o[e] >> 16);
    x_eff = a;
    x_st = a;
  }
}

template <typename T>
__device__ __forceinline__ T select_desc(const GemvArgs &a, int l) {
  T L = a.lin[0];
#pragma unroll
  for (int i = 1; i < kMaxBatch; ++i)
    if (i == l) L = a.lin[i];
  return L;
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

// Rotate one item into LDS.  Only DPP rows that hold an item do any work
// (the branch is uniform across the 16 lanes of a row).
template <int BITS, int MT>
__device__ __forceinline__ void rotate_item(bool rotate, u32x4 raw, uint32_t sword, int nb, int items, int it,
                                            int jj, uint32_t *xp, float *xs, int S) {
  if (it >= items) return;
  int m, b;
  item_mb<MT>(it, nb, m, b);
  const int kk = 128 * b + 8 * jj;
  float v[8];
  v[0] = half_bits_to_float(raw.x & 0xFFFF); v[1] = half_bits_to_float(raw.x >> 16);
  v[2] = half_bits_to_float(raw.y & 0xFFFF); v[3] = half_bits_to_float(raw.y >> 16);
  v[4] = half_bits_to_float(raw.z & 0xFFFF); v[5] = half_bits_to_float(raw.z >> 16);
  v[6] = half_bits_to_float(raw.w & 0xFFFF); v[7] = half_bits_to_float(raw.w >> 16);
  if (rotate) {
    const uint32_t sb = sword >> (kk & 31);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = ((sb >> e) & 1u) ? -v[e] : v[e];
    fwht128_row16_signed(v, jj);
    const float sc = fwht_lane_sign(jj) * kInvSqrt128;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] *= sc;
  }
  uint32_t o[4];
  float xe, xt;
  pairs_in_dot_order<BITS>(v, o, xe, xt);
  xe += dpp<kQuadXor1>(xe);
  xe += dpp<kQuadXor2>(xe);
  xt += dpp<kQuadXor1>(xt);
  xt += dpp<kQuadXor2>(xt);
  const int slice = 4 * b + (jj >> 2);
  *reinterpret_cast<u32x4 *>(&xp[(m * S + slice) * kSliceStride + 4 * (jj & 3)]) = u32x4{o[0], o[1], o[2], o[3]};
  if ((jj & 3) == 0) {
    xs[2 * (m * S + slice)] = xe;
    xs[2 * (m * S + slice) + 1] = 1024.0f * xt;
  }
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
  l.xs = mt * S * kSliceStride;                  // activations: [mt][S][20]
  l.part = l.xs + mt * S * 2;                    // slice sums: [mt][S][2]
  l.szl = (l.part + 2 * np * KS * mt + 3) & ~3;  // partials: [2np][KS][mt]
  l.total = l.szl + ((2 * np * G + 7) & ~7) * 2; // scale, zero as fp32: [2np][G][2]
  return l;
}

template <int BITS, int MT, int D>
__device__ __forceinline__ void stream_rows(const LinDesc &L, int m_valid, int r0, int rows, uint32_t *smem) {
  constexpr int XC = 2;                     // rotation passes whose loads precede the codes
  constexpr int ZL = 2;                     // 16-byte scale (zero) loads per thread before the codes
  const int t = threadIdx.x, rg = t >> 4, j = t & 15;
  const int K = L.k, KS = (K + kSeg - 1) / kSeg, G = K / kGroup, S = K / kSlice;
  const int wpr = S * BITS;
  const int NP = (rows + 1) >> 1, T = NP * KS;
  const int Tr = (T + kRG - 1) / kRG;       // tasks per DPP row
  const int tb = min(T, rg * Tr), te = min(T, tb + Tr);
  const bool full = (K % kSeg) == 0;        // every lane's slice exists in every segment
  const StreamLds lay = stream_lds(MT, S, KS, G, NP);
  uint32_t *xp = smem;
  float *xs = reinterpret_cast<float *>(smem + lay.xs);
  float *part = reinterpret_cast<float *>(smem + lay.part);
  float *szl = reinterpret_cast<float *>(smem + lay.szl);

  const rsrc_t rc = make_rsrc(L.codes + (size_t)r0 * wpr, (uint32_t)rows * wpr * 4);
  // scale/zero ranges rounded up to the 16-byte loads: the extra bytes share
  // the last valid 16-byte granule and only feed rows past the matrix
  const uint32_t szb = ((uint32_t)rows * G * 2 + 15u) & ~15u;
  const rsrc_t rsc = make_rsrc(L.scales + (size_t)r0 * G, szb);
  const rsrc_t rz = make_rsrc(L.zeros + (size_t)r0 * G, szb);
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
    const uint32_t off = e0 < nsz ? (uint32_t)e0 * 2 : kOOB;
    sr[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsc, off, 0, 0));
    zr[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rz, off, 0, 0));
  }

  // 2. the first D tasks of this DPP row's run
  const uint32_t seg_step = 16 * BITS * 4;                      // bytes per segment along a row
  const uint32_t pair_step = (uint32_t)(2 * wpr * 4) - (uint32_t)KS * seg_step;
  uint32_t co = __umul24((uint32_t)(tb / KS), (uint32_t)(2 * wpr * 4)) + (uint32_t)(tb % KS) * seg_step +
                (uint32_t)j * (BITS * 4);
  int is = tb % KS;
  uint32_t cw[D][2][BITS];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const bool ok = tb + d < te && (full || is * 16 + j < S);
    load_slice<BITS>(rc, ok ? co : kOOB, cw[d][0]);
    load_slice<BITS>(rc, ok ? co + wpr * 4 : kOOB, cw[d][1]);
    co += seg_step;
    if (++is == KS) { is = 0; co += pair_step; }
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
    const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsc, (uint32_t)e0 * 2, 0, 0));
    const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rz, (uint32_t)e0 * 2, 0, 0));
    const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int h = 0; h < 4; ++h)
      *reinterpret_cast<float4 *>(&szl[2 * (e0 + 2 * h)]) =
          make_float4(half_bits_to_float(av[h] & 0xFFFF), half_bits_to_float(bv[h] & 0xFFFF),
                      half_bits_to_float(av[h] >> 16), half_bits_to_float(bv[h] >> 16));
  }
#pragma unroll
  for (int q = 0; q < XC; ++q) rotate_item<BITS, MT>(rotate, xr[q], sw[q], nb, items, rg + kRG * q, j, xp, xs, S);
  for (int it0 = kRG * XC; it0 < items; it0 += kRG) {
    uint32_t xo, so;
    item_offsets<MT>(L, nb, items, it0 + rg, j, xo, so);
    const u32x4 raw = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xo, 0, 0));
    const uint32_t w1 = rotate ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsg, so, 0, 0) : 0u;
    rotate_item<BITS, MT>(rotate, raw, w1, nb, items, it0 + rg, j, xp, xs, S);
  }
  __syncthreads();

  // 4. stream the run
  const UnpackConsts uc = unpack_consts<BITS>();
  float acc[2][MT];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;
  int cp = tb / KS, cs = tb % KS;   // task being computed
  int sfirst = cs;

  for (int i0 = 0; i0 < Tr; i0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int tau = tb + i0 + d;
      if (tau < te) {
        const int slice = cs * 16 + j;
        const bool sv = full || slice < S;
        const int sl = sv ? slice : 0;
        const uint32_t zi = __umul24((uint32_t)(2 * cp), (uint32_t)G) + (uint32_t)(sl >> 2);
        const float2 sz0 = *reinterpret_cast<const float2 *>(&szl[2 * zi]);
        const float2 sz1 = *reinterpret_cast<const float2 *>(&szl[2 * (zi + G)]);
        const float sf[2] = {sv ? sz0.x : 0.f, sv ? sz1.x : 0.f};
        const float zf[2] = {sz0.y, sz1.y};
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
            const float2 xq = *reinterpret_cast<const float2 *>(&xs[2 * (m * S + sl)]);
#pragma unroll
            for (int r = 0; r < 2; ++r) {
              float dd = 0.f;
#pragma unroll
              for (int q = 0; q < 16; ++q) dd = dot2(pr[r][q], xv[q], dd);
              acc[r][m] = fmaf(sf[r], fmaf(-zf[r], xq.x, dd - xq.y), acc[r][m]);
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
              const float2 xq = *reinterpret_cast<const float2 *>(&xs[2 * (m * S + sl)]);
              float dd = 0.f;
#pragma unroll
              for (int q = 0; q < 16; ++q) dd = dot2(pr[q], xv[q], dd);
              acc[r][m] = fmaf(sf[r], fmaf(-zf[r], xq.x, dd - xq.y), acc[r][m]);
            }
          }
        }
        // the pair's last segment or the run's last task: flush
        if (cs == KS - 1 || tau == te - 1) {
#pragma unroll
          for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              const float v = row16_sum(acc[r][m]);
              acc[r][m] = 0.f;
              if (j == 0) part[__umul24((uint32_t)((2 * cp + r) * KS + sfirst), MT) + m] = v;
            }
          sfirst = (cs == KS - 1) ? 0 : cs + 1;
        }
        if (++cs == KS) { cs = 0; ++cp; }
      }
      // refill this buffer with the task D ahead
      const bool ok = tau + D < te && (full || is * 16 + j < S);
      load_slice<BITS>(rc, ok ? co : kOOB, cw[d][0]);
      load_slice<BITS>(rc, ok ? co + wpr * 4 : kOOB, cw[d][1]);
      co += seg_step;
      if (++is == KS) { is = 0; co += pair_step; }
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

// Tasks (two code loads each) a lane keeps in flight.  A 1024-thread
// workgroup per CU with 4 tasks per lane has 128 KB of int4 codes in flight,
// twice what HBM latency times a CU's share of bandwidth needs; deeper
// rings would spill under the 128-VGPR limit of 1024-thread workgroups.
template <int BITS, int MT>
struct Depth {
  static constexpr int d = MT == 1 ? (BITS <= 4 ? 4 : 3) : (MT == 2 ? (BITS <= 4 ? 3 : 2) : 2);
};

template <int BITS, int MT>
__global__ __launch_bounds__(kStreamThreads) void gemv_stream_kernel(GemvArgs a) {
  extern __shared__ uint32_t smem[];
  const int w = blockIdx.x;
  int l = 0;
#pragma unroll
  for (int i = 1; i < kMaxBatch; ++i)
    if (i < a.count && w >= a.lin[i].tile_begin) l = i;
  const LinDesc L = select_desc<LinDesc>(a, l);
  const int r0 = (w - L.tile_begin) * L.rows_per_wg;
  if (r0 >= L.n) return;
  const int rows = min(L.rows_per_wg, L.n - r0);
  stream_rows<BITS, MT, Depth<BITS, MT>::d>(L, a.m, r0, rows, smem);
}

template <int BITS>
hipError_t launch_bits(int mt, const GemvArgs &a, hipStream_t s) {
  switch (mt) {
    case 1:
      hipLaunchKernelGGL((gemv_stream_kernel<BITS, 1>), dim3(a.tiles), dim3(kStreamThreads), a.lds_bytes, s, a);
      break;
    case 2:
      hipLaunchKernelGGL((gemv_stream_kernel<BITS, 2>), dim3(a.tiles), dim3(kStreamThreads), a.lds_bytes, s, a);
      break;
    case 4:
      hipLaunchKernelGGL((gemv_stream_kernel<BITS, 4>), dim3(a.tiles), dim3(kStreamThreads), a.lds_bytes, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int gemv_stream_lds_bytes(int mt, int64_t k, int rows_per_wg) {
  const int64_t S = k / kSlice, KS = (k + kSeg - 1) / kSeg, G = k / kGroup;
  const int64_t np = (rows_per_wg + 1) / 2;
  if (S * kSliceStride * mt + np * (KS + G) * 2 * mt > (int64_t)1 << 26) return 1 << 30;
  return stream_lds(mt, (int)S, (int)KS, (int)G, (int)np).total * 4;
}

hipError_t launch_gemv_stream(int bits, int mt, const GemvArgs &a, hipStream_t s) {
  switch (bits) {
    case 3: return launch_bits<3>(mt, a, s);
    case 4: return launch_bits<4>(mt, a, s);
    case 6: return launch_bits<6>(mt, a, s);
    case 8: return launch_bits<8>(mt, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace wq

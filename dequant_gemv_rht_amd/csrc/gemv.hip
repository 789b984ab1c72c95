// Tiled fused rotation + dequantising GEMV (gfx950): the mixed 6/8-bit
// layout above batch 1 (tiles of up to 16 batch rows), and any uniform
// width whose tile of up to 4 batch rows does not fit the stream kernels'
// LDS.
//
// What it computes (model card "24B0978 - Week 01 - Track 2, 20% target",
// section "How these techniques accelerate inference on CUDA"): for every
// output row n and batch row m,
//     y[m][n] = sum_g s[n][g] * ( sum_{k in g} q[n][k] x'[m][k] - z[n][g] sum_{k in g} x'[m][k] )
// i.e. w = (q - z) * s with the scale applied once per group partial sum,
// and x' = H D x / sqrt(128) per 128-block (paragraph on the random
// Hadamard transform) when the weight carries rotation signs.
//
// Work decomposition.  A 256-thread workgroup owns R = 16*RR whole output
// rows and walks K in 512-wide segments; no two workgroups share an output,
// so there is no cross-workgroup reduction and the result is deterministic.
//   * Thread t serves rows (t / 16) + 16 i, i < RR, and the 32-code slice
//     (t % 16) of every segment: the 16 lanes of a DPP row read one
//     contiguous run of packed codes per row and segment.
//   * The activations of the workgroup's K range are rotated once into LDS
//     (16 lanes x 8 elements per 128-block; butterflies of stride 1, 2, 4
//     inside a lane, 8..64 across lanes by DPP) as fp16 pairs in the order
//     the unpacker produces code pairs, with per-slice sums of the rounded
//     values.  Their loads are issued before the code loads so the rotation
//     overlaps the weight stream's latency (vmcnt retires in order).
//   * Code, scale and zero loads run D segments ahead of the products.
//   * Codes become fp16 (1024 + q) by OR-ing them into the mantissa of
//     1024.0, and v_dot2_f32_f16 accumulates (1024 + q) * x' in fp32; the
//     1024 offset is folded into the zero point, and the scale multiplies
//     each 32-code partial once.
//   * The 16 slice partials of a row are summed by DPP at the end.
//   * Large batches keep only a K chunk of the rotated activations in LDS
//     at a time.
#include "wq_internal.h"

namespace wq {
using namespace dev;

namespace {

constexpr uint32_t kBias = 0x64006400u;   // two fp16 1024.0
constexpr float kInvSqrt128 = 0.08838834764831845f;

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

// `width` bits of a little-endian word array starting at bit `bit`
// (compile-time position; may straddle two words).
template <int BIT, int WIDTH, int N>
__device__ __forceinline__ uint32_t field(const uint32_t (&w)[N]) {
  constexpr int wi = BIT / 32, off = BIT % 32;
  if constexpr (off + WIDTH <= 32) {
    return __builtin_amdgcn_ubfe(w[wi], off, WIDTH);
  } else {
    return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], off) & ((1u << WIDTH) - 1);
  }
}

// Unpacking constants kept in VGPRs: gfx9 VOP3 instructions cannot take two
// literal constants, and with both in registers every code pair costs one
// v_and_or_b32 (plus one shift or bit-field extract).
struct UnpackConsts {
  uint32_t mask, bias;
};

template <int BITS>
__device__ __forceinline__ UnpackConsts unpack_consts() {
  constexpr uint32_t m = BITS == 4 ? 0x000F000Fu : BITS == 8 ? 0x00FF00FFu : BITS == 3 ? 0x00070007u : 0x003F003Fu;
  UnpackConsts c;
  asm volatile("v_mov_b32 %0, %1" : "=v"(c.mask) : "i"(m));
  asm volatile("v_mov_b32 %0, %1" : "=v"(c.bias) : "i"(kBias));
  return c;
}

template <int BITS, int P>
__device__ __forceinline__ uint32_t pair_at(const uint32_t (&w)[BITS], UnpackConsts c) {
  if constexpr (BITS == 4) {
    // word P/4 holds codes 0..7; pair r = (code r, code r+4)
    constexpr int wi = P / 4, r = P % 4;
    return ((w[wi] >> (4 * r)) & c.mask) | c.bias;
  } else if constexpr (BITS == 8) {
    // word P/2 holds codes 0..3; pair r = (code r, code r+2)
    constexpr int wi = P / 2, r = P % 2;
    return ((w[wi] >> (8 * r)) & c.mask) | c.bias;
  } else if constexpr (BITS == 3) {
    // codes 2P and 2P+1 sit in bits [6P, 6P+6) of the 96-bit run
    const uint32_t t = field<6 * P, 6>(w);
    return ((t | (t << 13)) & c.mask) | c.bias;
  } else {
    // two 96-bit runs of 16 codes; codes 2q, 2q+1 of a run in bits [12q, 12q+12)
    constexpr int run = P / 8, q = P % 8;
    const uint32_t t = (run == 0) ? field<12 * q, 12>(w) : field<96 + 12 * q, 12>(w);
    return ((t | (t << 10)) & c.mask) | c.bias;
  }
}

template <int BITS, int P = 0>
__device__ __forceinline__ void unpack_pairs(const uint32_t (&w)[BITS], UnpackConsts c, uint32_t (&p)[16]) {
  p[P] = pair_at<BITS, P>(w, c);
  if constexpr (P + 1 < 16) unpack_pairs<BITS, P + 1>(w, c, p);
}

// Round the 8 values of a lane to fp16 pairs in the order unpack_pairs
// produces code pairs.  The lane's 8 values are codes 8w..8w+7 of its slice.
template <int BITS>
__device__ __forceinline__ void pairs_in_dot_order(const float (&v)[8], uint32_t (&o)[4]) {
  if constexpr (BITS == 4) {
    o[0] = pack_half2(v[0], v[4]); o[1] = pack_half2(v[1], v[5]);
    o[2] = pack_half2(v[2], v[6]); o[3] = pack_half2(v[3], v[7]);
  } else if constexpr (BITS == 8) {
    o[0] = pack_half2(v[0], v[2]); o[1] = pack_half2(v[1], v[3]);
    o[2] = pack_half2(v[4], v[6]); o[3] = pack_half2(v[5], v[7]);
  } else {
    o[0] = pack_half2(v[0], v[1]); o[1] = pack_half2(v[2], v[3]);
    o[2] = pack_half2(v[4], v[5]); o[3] = pack_half2(v[6], v[7]);
  }
}



__device__ __forceinline__ void store_out(const LinDesc &L, int m, int row, float v) {
  if (L.out_f32) {
    reinterpret_cast<float *>(L.y)[(size_t)m * L.ldy + row] = v;
  } else {
    _Float16 h = (_Float16)v;
    reinterpret_cast<uint16_t *>(L.y)[(size_t)m * L.ldy + row] = __builtin_bit_cast(uint16_t, h);
  }
}

// Byte offsets of the raw fp16 activations (16 bytes) and of the sign word
// of one rotation item (batch row m, 128-block b of the chunk) for lane jj,
// which holds elements 8jj..8jj+7 of the block.  Items past the chunk get
// out-of-range offsets (their loads return zero).
__device__ __forceinline__ void item_offsets(const LinDesc &L, int c0, int nb, int items, int it, int jj,
                                             uint32_t &xoff, uint32_t &soff) {
  const int m = it / nb, b = it % nb;
  const int kk = c0 + 128 * b + 8 * jj;
  const bool ok = it < items;
  xoff = ok ? (uint32_t)(((size_t)m * L.ldx + kk) * 2) : kOOB;
  soff = ok ? (uint32_t)((kk >> 5) * 4) : kOOB;
}

// Rotate one item and leave it in LDS: xp[m][slice][pair], xs[m][slice].
template <int BITS>
__device__ __forceinline__ void rotate_item(bool rotate, u32x4 raw, uint32_t sword, int c0, int nb, int items,
                                            int it, int jj, uint32_t *xp, float *xs, int sc) {
  const int m = it / nb, b = it % nb;
  const int kk = c0 + 128 * b + 8 * jj;
  float v[8];
  v[0] = half_bits_to_float(raw.x & 0xFFFF); v[1] = half_bits_to_float(raw.x >> 16);
  v[2] = half_bits_to_float(raw.y & 0xFFFF); v[3] = half_bits_to_float(raw.y >> 16);
  v[4] = half_bits_to_float(raw.z & 0xFFFF); v[5] = half_bits_to_float(raw.z >> 16);
  v[6] = half_bits_to_float(raw.w & 0xFFFF); v[7] = half_bits_to_float(raw.w >> 16);
  if (rotate) {
    const uint32_t sb = sword >> (kk & 31);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = ((sb >> e) & 1u) ? -v[e] : v[e];
    fwht128_row16(v, jj);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] *= kInvSqrt128;
  }
  uint32_t o[4];
  pairs_in_dot_order<BITS>(v, o);
  float rs = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) rs += half_bits_to_float(o[e] & 0xFFFF) + half_bits_to_float(o[e] >> 16);
  rs += dpp<kQuadXor1>(rs);
  rs += dpp<kQuadXor2>(rs);
  if (it < items) {
    const int slice = 4 * b + (jj >> 2);
    *reinterpret_cast<u32x4 *>(&xp[((size_t)m * sc + slice) * 16 + 4 * (jj & 3)]) = u32x4{o[0], o[1], o[2], o[3]};
    if ((jj & 3) == 0) xs[m * sc + slice] = rs;
  }
}

// Rotate a whole chunk [c0, c0 + ck) into LDS (loads, then butterflies).
template <int BITS, int MT>
__device__ __forceinline__ void stage_chunk(const LinDesc &L, rsrc_t rx, rsrc_t rsg, int c0, int ck, int grp, int jj,
                                            uint32_t *xp, float *xs, int sc) {
  const int nb = ck / kGroup, items = MT * nb;
  const bool rotate = L.signs != nullptr;
  for (int it0 = 0; it0 < items; it0 += 16) {
    uint32_t xo, so;
    item_offsets(L, c0, nb, items, it0 + grp, jj, xo, so);
    const u32x4 raw = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xo, 0, 0));
    const uint32_t sw = rotate ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsg, so, 0, 0) : 0u;
    rotate_item<BITS>(rotate, raw, sw, c0, nb, items, it0 + grp, jj, xp, xs, sc);
  }
}

// Code loads of segment s for this thread's RR rows.  Rows past the matrix
// fall outside the resource; slices past K get kOOB (no memory access).
template <int BITS, int RR>
__device__ __forceinline__ void issue_segment(rsrc_t rc, const uint32_t (&rowoff)[RR], int S, int j, int s,
                                              uint32_t (&cw)[RR][BITS]) {
  const int slice = s * 16 + j;
  const bool sv = slice < S;
  const uint32_t so = (uint32_t)slice * (BITS * 4);
#pragma unroll
  for (int i = 0; i < RR; ++i) load_slice<BITS>(rc, sv ? rowoff[i] + so : kOOB, cw[i]);
}

// Whole rows [rb*R, rb*R + R) over all of K, R = 16*RR.  Up to D segments of
// codes are in flight per lane; when K has at most D segments every code
// load of the workgroup is issued before the first product.
template <int BITS, int MT, int RR, int D>
__device__ __forceinline__ void gemv_rows(const LinDesc &L, int m_valid, int rb,
                                          const uint32_t *__restrict__ tile_codes, uint32_t *smem) {
  constexpr int R = 16 * RR;
  constexpr int MC = MT < 4 ? MT : 4;     // batch rows of activations held in registers at once
  constexpr int XC = 4;                   // rotation passes whose loads go out before the codes
  constexpr int ZL = 2;                   // 16-byte scale (and zero) loads per thread
  const int t = threadIdx.x, grp = t >> 4, rl = t >> 4, j = t & 15;
  const int K = L.k, KS = (K + kSeg - 1) / kSeg, G = K / kGroup, S = K / kSlice;
  const int wpr = S * BITS;
  const int r0 = rb * R;
  const int rows = min(R, L.n - r0);
  const int kc = L.kc, sc = kc / kSlice;
  // LDS: rotated activations [MT][sc][16] pairs, their slice sums [MT][sc],
  // then the tile's scale/zero pairs [R][G] as (s | z << 16)
  uint32_t *xp = smem;
  float *xs = reinterpret_cast<float *>(smem + (size_t)MT * sc * 16);
  uint32_t *szl = smem + (size_t)MT * sc * 17;

  const rsrc_t rc = make_rsrc(tile_codes, (uint32_t)rows * wpr * 4);
  // Scale/zero tiles are read with 16-byte loads, and a load that reaches
  // past the resource's end returns zero as a whole: round the range up to
  // 16 bytes.  The tile starts 32-byte aligned, so the extra bytes lie in the
  // last 16-byte granule that holds valid data (same page) and only feed
  // rows past the matrix, whose outputs are never stored.
  const uint32_t szb = ((uint32_t)rows * G * 2 + 15u) & ~15u;
  const rsrc_t rsc = make_rsrc(L.scales + (size_t)r0 * G, szb);
  const rsrc_t rz = make_rsrc(L.zeros + (size_t)r0 * G, szb);
  const rsrc_t rx = make_rsrc(L.x, (uint32_t)(((size_t)(m_valid - 1) * L.ldx + K) * 2));
  const rsrc_t rsg = make_rsrc(L.signs, L.signs ? (uint32_t)(K / 8) : 0u);
  const bool rotate = L.signs != nullptr;

  // 1. activations and signs of the first chunk, and the tile's scales and
  //    zeros, ahead of the weight stream
  int c0 = 0, ck = min(kc, K);
  int nb = ck / kGroup, items = MT * nb;
  u32x4 xr[XC];
  uint32_t sw[XC];
#pragma unroll
  for (int p = 0; p < XC; ++p) {
    uint32_t xo, so;
    item_offsets(L, c0, nb, items, grp + 16 * p, j, xo, so);
    xr[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xo, 0, 0));
    sw[p] = rotate ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsg, so, 0, 0) : 0u;
  }
  const int nsz = R * G;                  // scale (zero) values of the tile
  u32x4 sr[ZL], zr[ZL];
#pragma unroll
  for (int p = 0; p < ZL; ++p) {
    const int e0 = 8 * (t + kThreads * p);
    const uint32_t off = e0 < nsz ? (uint32_t)e0 * 2 : kOOB;
    sr[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsc, off, 0, 0));
    zr[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rz, off, 0, 0));
  }

  // 2. weight stream: D segments in flight
  uint32_t rowoff[RR];
#pragma unroll
  for (int i = 0; i < RR; ++i) rowoff[i] = (uint32_t)((rl + 16 * i) * wpr * 4);
  uint32_t cw[D][RR][BITS];
#pragma unroll
  for (int d = 0; d < D; ++d) issue_segment<BITS, RR>(rc, rowoff, S, j, d, cw[d]);

  // 3. scales and zeros into LDS, remaining ones (long K) by a plain loop;
  //    then the first chunk of rotated activations
#pragma unroll
  for (int p = 0; p < ZL; ++p) {
    const int e0 = 8 * (t + kThreads * p);
    if (e0 < nsz) {
      const u32x4 a = sr[p], b = zr[p];
      const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      u32x4 lo, hi;
      lo.x = (v[0] & 0xFFFF) | (v[4] << 16); lo.y = (v[0] >> 16) | (v[4] & 0xFFFF0000u);
      lo.z = (v[1] & 0xFFFF) | (v[5] << 16); lo.w = (v[1] >> 16) | (v[5] & 0xFFFF0000u);
      hi.x = (v[2] & 0xFFFF) | (v[6] << 16); hi.y = (v[2] >> 16) | (v[6] & 0xFFFF0000u);
      hi.z = (v[3] & 0xFFFF) | (v[7] << 16); hi.w = (v[3] >> 16) | (v[7] & 0xFFFF0000u);
      *reinterpret_cast<u32x4 *>(&szl[e0]) = lo;
      *reinterpret_cast<u32x4 *>(&szl[e0 + 4]) = hi;
    }
  }
  for (int e0 = 8 * (t + kThreads * ZL); e0 < nsz; e0 += 8 * kThreads) {
    const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsc, (uint32_t)e0 * 2, 0, 0));
    const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rz, (uint32_t)e0 * 2, 0, 0));
    const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      szl[e0 + 2 * q] = (v[q] & 0xFFFF) | (v[4 + q] << 16);
      szl[e0 + 2 * q + 1] = (v[q] >> 16) | (v[4 + q] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int p = 0; p < XC; ++p) rotate_item<BITS>(rotate, xr[p], sw[p], c0, nb, items, grp + 16 * p, j, xp, xs, sc);
  if (items > 16 * XC) {
    for (int it0 = 16 * XC; it0 < items; it0 += 16) {
      uint32_t xo, so;
      item_offsets(L, c0, nb, items, it0 + grp, j, xo, so);
      const u32x4 raw = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xo, 0, 0));
      const uint32_t w1 = rotate ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsg, so, 0, 0) : 0u;
      rotate_item<BITS>(rotate, raw, w1, c0, nb, items, it0 + grp, j, xp, xs, sc);
    }
  }
  __syncthreads();

  // 4. products, segment by segment; loads for segment s + D go out as
  //    soon as segment s's registers are free
  const UnpackConsts uc = unpack_consts<BITS>();
  float acc[RR][MT];
#pragma unroll
  for (int i = 0; i < RR; ++i)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[i][m] = 0.f;

  for (int s0 = 0; s0 < KS; s0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int s = s0 + d;
      if (s < KS) {
        if (s * kSeg >= c0 + ck) {         // next chunk of activations
          __syncthreads();
          c0 += ck;
          ck = min(kc, K - c0);
          stage_chunk<BITS, MT>(L, rx, rsg, c0, ck, grp, j, xp, xs, sc);
          __syncthreads();
        }
        const int slice = s * 16 + j;
        const bool sv = slice < S;
        const int sl = sv ? (s * kSeg - c0) / kSlice + j : 0;
        const int g = sv ? (slice >> 2) : 0;
        float sf[RR], zb[RR];
#pragma unroll
        for (int i = 0; i < RR; ++i) {
          const uint32_t szv = szl[(rl + 16 * i) * G + g];
          sf[i] = half_bits_to_float(szv & 0xFFFF);
          zb[i] = half_bits_to_float(szv >> 16) + 1024.0f;
        }
#pragma unroll
        for (int mc = 0; mc < MT; mc += MC) {
          uint32_t xv[MC][16];
          float xq[MC];
#pragma unroll
          for (int mm = 0; mm < MC; ++mm) {
            const u32x4 *src = reinterpret_cast<const u32x4 *>(&xp[((size_t)(mc + mm) * sc + sl) * 16]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const u32x4 v = src[q];
              xv[mm][4 * q + 0] = v.x; xv[mm][4 * q + 1] = v.y;
              xv[mm][4 * q + 2] = v.z; xv[mm][4 * q + 3] = v.w;
            }
            xq[mm] = xs[(mc + mm) * sc + sl];
          }
#pragma unroll
          for (int i = 0; i < RR; ++i) {
            uint32_t p[16];
            unpack_pairs<BITS>(cw[d][i], uc, p);
#pragma unroll
            for (int mm = 0; mm < MC; ++mm) {
              float dd = 0.f;
#pragma unroll
              for (int q = 0; q < 16; ++q) dd = dot2(p[q], xv[mm][q], dd);
              const float c = sf[i] * fmaf(-zb[i], xq[mm], dd);
              acc[i][mc + mm] += sv ? c : 0.f;
            }
          }
        }
      }
      issue_segment<BITS, RR>(rc, rowoff, S, j, s + D, cw[d]);
    }
  }

  // 5. sum the 16 slices of every row, store
#pragma unroll
  for (int i = 0; i < RR; ++i)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[i][m] = row16_sum(acc[i][m]);
#pragma unroll
  for (int i = 0; i < RR; ++i)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int row = r0 + rl + 16 * i;
      if (j == ((i * MT + m) & 15) && m < m_valid && row < L.n) store_out(L, m, row, acc[i][m]);
    }
}

// Per code width and batch tile: how many code loads a lane may hold in
// flight (about 64 VGPRs of payload), and the two tile shapes built from it:
// short K (whole K in flight, 2 rows per DPP row when it fits) and long K
// (1 row per DPP row, deepest prefetch).
template <int BITS, int MT>
struct Shape {
  static constexpr int budget = (BITS <= 4 ? 16 : (BITS == 6 ? 12 : 8)) / (MT >= 4 ? 2 : 1);
  static constexpr int short_rr = budget >= 16 ? 2 : 1;
  static constexpr int short_d = budget / short_rr;
  static constexpr int long_d = budget;
};

template <int BITS, int MT>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvArgs a) {
  extern __shared__ uint32_t smem[];
  const int tile = blockIdx.x;
  const LinDesc L = fetch_desc(a, tile);
  const int rb = tile - L.tile_begin;
  const size_t wpr = (size_t)(L.k / kSlice) * BITS;
  using Sh = Shape<BITS, MT>;
  if (L.mode == 0)
    gemv_rows<BITS, MT, Sh::short_rr, Sh::short_d>(L, a.m, rb, L.codes + (size_t)rb * (16 * Sh::short_rr) * wpr, smem);
  else
    gemv_rows<BITS, MT, 1, Sh::long_d>(L, a.m, rb, L.codes + (size_t)rb * 16 * wpr, smem);
}

// Mixed 6/8-bit: a workgroup owns 16 rows of one 64-row block, so the code
// width is uniform across it (block_bits of the block).
template <int MT>
__global__ __launch_bounds__(kThreads) void gemv_mixed_kernel(GemvArgs a) {
  extern __shared__ uint32_t smem[];
  const int tile = blockIdx.x;
  const LinDesc L = fetch_desc(a, tile);
  const int rb = tile - L.tile_begin;            // 16-row tile
  const int blk = rb >> 2;                        // 64-row block
  const int bits = L.block_bits[blk];
  const uint32_t *tc = L.codes + L.block_off[blk] + (size_t)(rb & 3) * 16 * (L.k / kSlice) * bits;
  if (bits == 8)
    gemv_rows<8, MT, 1, Shape<8, MT>::long_d>(L, a.m, rb, tc, smem);
  else
    gemv_rows<6, MT, 1, Shape<6, MT>::long_d>(L, a.m, rb, tc, smem);
}

template <int BITS, int MT>
hipError_t launch_t(const GemvArgs &a, hipStream_t s) {
  if constexpr (BITS == 0) {
    hipLaunchKernelGGL((gemv_mixed_kernel<MT>), dim3(a.tiles), dim3(kThreads), a.lds_bytes, s, a);
  } else {
    hipLaunchKernelGGL((gemv_kernel<BITS, MT>), dim3(a.tiles), dim3(kThreads), a.lds_bytes, s, a);
  }
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(int mt, const GemvArgs &a, hipStream_t s) {
  switch (mt) {
    case 1: return launch_t<BITS, 1>(a, s);
    case 2: return launch_t<BITS, 2>(a, s);
    case 4: return launch_t<BITS, 4>(a, s);
  }
  if constexpr (BITS == 0) {   // uniform widths reach this kernel in tiles of at most 4 rows
    switch (mt) {
      case 8: return launch_t<0, 8>(a, s);
      case 16: return launch_t<0, 16>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

namespace {
template <int BITS>
void shape_of(int mt, int &budget, int &short_rr) {
  switch (mt) {
    case 1: budget = Shape<BITS, 1>::budget; short_rr = Shape<BITS, 1>::short_rr; break;
    case 2: budget = Shape<BITS, 2>::budget; short_rr = Shape<BITS, 2>::short_rr; break;
    case 4: budget = Shape<BITS, 4>::budget; short_rr = Shape<BITS, 4>::short_rr; break;
    case 8: budget = Shape<BITS, 8>::budget; short_rr = Shape<BITS, 8>::short_rr; break;
    default: budget = Shape<BITS, 16>::budget; short_rr = Shape<BITS, 16>::short_rr; break;
  }
}
}  // namespace

// Tile shape for one linear: mode 0 (short K) keeps the whole K in flight
// with short_rr rows per DPP row; mode 1 (long K) one row per DPP row.
void gemv_shape(int bits, int mt, int64_t k, int &mode, int &rows) {
  if (bits == 0) {
    mode = 1;
    rows = 16;
    return;
  }
  int budget = 16, short_rr = 1;
  switch (bits) {
    case 3: shape_of<3>(mt, budget, short_rr); break;
    case 4: shape_of<4>(mt, budget, short_rr); break;
    case 6: shape_of<6>(mt, budget, short_rr); break;
    default: shape_of<8>(mt, budget, short_rr); break;
  }
  const int64_t ks = (k + kSeg - 1) / kSeg;
  if (ks <= budget / short_rr) {
    mode = 0;
    rows = 16 * short_rr;
  } else {
    mode = 1;
    rows = 16;
  }
}

// K per LDS chunk: the whole (512-padded) K when it fits the budget.
int gemv_chunk(int mt, int64_t k) {
  const int64_t budget = mt <= 2 ? 40 * 1024 : 64 * 1024;
  const int64_t per_elem_x16 = (int64_t)mt * 34;        // 2.125 bytes per element and batch row, x16
  int64_t kc = budget * 16 / per_elem_x16 / kSeg * kSeg;
  if (kc < kSeg) kc = kSeg;
  const int64_t kp = (k + kSeg - 1) / kSeg * kSeg;
  return (int)(kc < kp ? kc : kp);
}

// LDS bytes: rotated activations of a chunk, their slice sums, and the
// tile's scale/zero pairs.
int gemv_lds_bytes(int mt, int chunk, int rows, int64_t k) {
  return mt * (chunk / kSlice) * (16 * 4 + 4) + rows * (int)(k / kGroup) * 4;
}

hipError_t launch_gemv(int bits, int mt, const GemvArgs &a, hipStream_t s) {
  switch (bits) {
    case 0: return launch_bits<0>(mt, a, s);
    case 3: return launch_bits<3>(mt, a, s);
    case 4: return launch_bits<4>(mt, a, s);
    case 6: return launch_bits<6>(mt, a, s);
    case 8: return launch_bits<8>(mt, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace wq

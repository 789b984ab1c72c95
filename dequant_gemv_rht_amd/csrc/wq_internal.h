// Internal declarations shared by the libwq translation units (not part of
// the C ABI).  Kernels are written for gfx950 (CDNA4): wave64, DPP row
// operations within 16-lane rows, v_dot2_f32_f16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/wq.h"

namespace wq {

constexpr int kGroup = 128;        // quantisation group along K = rotation block
constexpr int kSeg = 512;          // K per GEMV tile segment: 16 lanes x 32 codes
constexpr int kSlice = 32;         // codes per lane per row
constexpr int kThreads = 256;      // GEMV workgroup
constexpr int kMaxBatch = WQ_MAX_BATCH;
constexpr int kMixedRows = WQ_MIXED_ROWS;   // rows per block of one width in the mixed layout

// ---------------------------------------------------------------------------
// GEMV launch description
// ---------------------------------------------------------------------------
struct LinDesc {
  const uint32_t *codes;
  const uint16_t *scales;
  const uint16_t *zeros;
  const uint8_t *block_bits;    // mixed width only
  const uint64_t *block_off;    // mixed width only
  const uint32_t *signs;        // nullptr: activations used as given
  union {
    const uint16_t *x;          // the fp16 activations [m][ldx]
    const uint32_t *xq;         // batch tiles 2 to 16: the tile's arranged activations [mt][k/32][20] (xprep)
  };
  void *y;
  int64_t ldx, ldy;
  int32_t n, k;
  int32_t kc;                   // K per LDS chunk of staged activations (multiple of 512)
  int32_t mode;                 // tiled kernel's tile shape: 0 short K, 1 long K
  int32_t rows_per_wg;          // stream kernel: output rows per workgroup (even)
  int32_t row_blocks;
  int32_t tile_begin;           // first workgroup of this linear in the grid
  int32_t out_f32;
  int32_t ks_inv;               // ceil(2^16 / KS), KS = ceil(k / 512): x / KS = (x * ks_inv) >> 16 for x <= 64
  // batch-tile (row-quad) kernel, set by its launcher: the LDS layout of a
  // full workgroup and its walk over K (no divisions left to the kernel)
  int32_t q_chunks, q_kc;       // K chunks of q_kc 512-wide segments (the last one shorter)
  int32_t q_p, q_spu;           // DPP rows per quad (K parts); segments per part, at most
  uint32_t q_pinv;              // ceil(2^16 / q_p)
  int32_t q_sc;                 // slices per batch row in the activation block
  uint32_t q_xinv;              // ceil(2^32 / (5 q_sc)): 16-byte pieces per batch row
  int32_t q_part, q_szl;        // word offsets of the row parts and of the scales and zeros
};

struct GemvArgs {
  int32_t first_tile[kMaxBatch];  // lin[i].tile_begin, packed; INT32_MAX past count
  LinDesc lin[kMaxBatch];
  int32_t count;
  int32_t m;                    // batch rows actually present (<= MT)
  int32_t tiles;                // total workgroups
  int32_t lds_bytes;            // dynamic LDS per workgroup
  int32_t ring;                 // stream kernel, batch 1: weights staged through an LDS ring
  int32_t mixed_wpb;            // batch-1 ring over the mixed 6/8-bit layout: 1 = one workgroup per
                                // 64-row block, 0 = workgroups spread over the blocks by code words
};

// The mixed 6/8-bit layout at batch 1 when the caller also gave the block
// widths on the host: the host places every workgroup (the same split as
// the kernel's own search: runs of same-width blocks, workgroups by code
// words, row pairs split evenly), and each workgroup reads its record and
// the next one.  Record w: low word the code word of its first row, high
// word that row | (1 << 31 if its rows are 8-bit); record G: n rows.
constexpr int kMixedTableWgs = WQ_MIXED_HOST_WORKGROUPS;
struct MixedArgs {
  LinDesc lin;
  int32_t tiles;                // workgroups G
  int32_t lds_bytes;
  uint64_t wg[kMixedTableWgs + 1];
};
static_assert(sizeof(MixedArgs) <= 4096, "mixed launch arguments within the 4 KB kernel-argument limit");
hipError_t launch_gemv_mixed_table(const MixedArgs &a, hipStream_t s);

// The calling thread's message for wq_last_error (api.cpp): set_error
// formats it and returns st; clear_error empties it.
wq_status set_error(wq_status st, const char *fmt, ...);
void clear_error();

// Host-side launchers (gemv*.hip).  `bits` 0 = mixed.  mt = 1,2,4,8,16.
hipError_t launch_gemv(int bits, int mt, const GemvArgs &a, hipStream_t s);
// Persistent stream kernels: one workgroup per CU, uniform code width (or
// the mixed layout at batch 1), batch tile 1, 2, 4, 8 or 16, the linear's
// rotated K range in LDS (in up to 4 chunks at batch tiles).
constexpr int kStreamThreads = 1024;
hipError_t launch_gemv_stream(int bits, int mt, const GemvArgs &a, hipStream_t s);
// Batch tiles 2 to 16: one pass arranging every linear's m activation rows
// (rotated when signs[i] is set) in the stream kernels' slice layout,
// out[i] = [m][k/32][20] u32 (80 bytes per 32-element slice).
hipError_t launch_xprep(int bits, int count, const uint16_t *const *x, const int64_t *ldx,
                        const uint32_t *const *signs, const int64_t *k, int64_t m, uint32_t *const *out,
                        hipStream_t s);
// LDS bytes of one stream workgroup; ring = batch-1 kernel with the LDS ring
int gemv_stream_lds_bytes(int bits, int mt, int64_t k, int rows_per_wg, bool ring);
void gemv_shape(int bits, int mt, int64_t k, int &mode, int &rows);
int gemv_chunk(int mt, int64_t k);              // K per LDS chunk
int gemv_lds_bytes(int mt, int chunk, int rows, int64_t k);

// Other launchers.
hipError_t launch_rht(const uint16_t *x, uint16_t *y, const uint32_t *signs, int64_t m,
                      int64_t k, int64_t ldx, int64_t ldy, hipStream_t s);
// One plain read of `bytes` (a multiple of 16) at `src`, nothing stored
// (the read ceiling of include/wq_measure.h).
hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t s);

// the same rotation for up to kMaxBatch matrices of m rows in one launch;
// with `pair_order` each 8 consecutive outputs are stored in the order
// 0, 4, 1, 5, 2, 6, 3, 7 (the order the int4 matrix-core kernel unpacks a
// code word in; gemm_pair_order)
hipError_t launch_rht_batch(int count, const uint16_t *const *x, uint16_t *const *y, const uint32_t *const *signs,
                            int64_t m, const int64_t *k, const int64_t *ldx, const int64_t *ldy, bool pair_order,
                            hipStream_t s);
hipError_t launch_quantize(int bits, int64_t n, int64_t k, const float *w,
                           const uint32_t *signs, const uint8_t *block_bits, uint8_t *codes,
                           uint16_t *scales, uint16_t *zeros, hipStream_t s);
hipError_t launch_pack(int bits, int64_t n, int64_t k, const uint8_t *codes,
                       const uint8_t *block_bits, uint32_t *packed, uint64_t *block_off,
                       hipStream_t s);
hipError_t launch_unpack(int bits, int64_t n, int64_t k, const uint32_t *packed,
                         const uint8_t *block_bits, const uint64_t *block_off, uint8_t *codes,
                         hipStream_t s);
// Rows ids[0..count) of a uniform-width table, dequantised to fp16 or fp32
// [count][ldo] (embed.hip); ids outside [0, n) give rows of zeros.
hipError_t launch_embed(const wq_weight &w, const int32_t *ids, int64_t count, void *out, bool f32, int64_t ldo,
                        hipStream_t s);

// MFMA GEMM for m >= 17 (gemm.hip), one launch for up to kMaxBatch linears
// of one code width.  xr[i]: fp16 activations already rotated (or used as
// given), [m][ldx[i]].  ksplit[i] > 1 cuts K over that many workgroups whose
// fp32 partials go to part[i] ([ksplit][m][n], gemm_partial_bytes) and are
// added by a second kernel.
bool gemm_available(int bits);
// whether the kernel for `bits` can take activations whose 8-element groups
// are in rht_batch's pair order (int4: a cheaper unpack)
bool gemm_pair_order(int bits);
void gemm_plan(int count, const wq_weight *w, int64_t m, int *ksplit);
size_t gemm_partial_bytes(const wq_weight &w, int64_t m, int ksplit);
// pair_order: every xr[i] is in rht_batch's pair order (only where
// gemm_pair_order(bits))
hipError_t launch_gemm_batch(int count, const wq_weight *w, const uint16_t *const *xr, const int64_t *ldx,
                             int64_t m, void *const *y, const int *out_f32, const int64_t *ldy,
                             const int *ksplit, float *const *part, bool pair_order, hipStream_t s);

}  // namespace wq

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
#if defined(__HIP__)
namespace wq {
namespace dev {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x3 __attribute__((ext_vector_type(3)));

// Raw buffer addressing: a load whose offset lies outside the resource's
// byte range returns zero without touching memory, which lets every load be
// issued unconditionally (straight-line code, exact vmcnt waits).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;          // an offset past any resource
constexpr int kRsrcWord3 = 0x00020000;           // gfx9 raw buffer descriptor word 3
constexpr int kNT = 2;                           // aux: non-temporal (streamed once)

__device__ __forceinline__ rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kRsrcWord3);
}

// DPP controls (GFX9 encoding).
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kQuadRev = 0x1B;       // quad_perm [3,2,1,0]  (lane ^ 3)
constexpr int kRowRor4 = 0x124;      // row_ror:4            (lane + 4 mod 16 in a row)
constexpr int kRowRor8 = 0x128;      // row_ror:8            (lane ^ 8 in a row)
constexpr int kRowMirror = 0x140;    // lane ^ 15 in a row
constexpr int kRowHalfMirror = 0x141; // lane ^ 7 within 8 lanes

// Lane permutation within 16-lane rows.  All source lanes of these
// permutations exist, so no "old" value is needed and the move can be folded
// into the instruction that consumes it (v_add_f32_dpp, v_fmac_f32_dpp).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// value of lane (this ^ 4) within a 16-lane row: (lane ^ 7) ^ 3
__device__ __forceinline__ float dpp_xor4(float v) {
  return dpp<kQuadRev>(dpp<kRowHalfMirror>(v));
}

// Sum over the 16 lanes of a DPP row; every lane gets the total.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<kQuadXor1>(v);
  v += dpp<kQuadXor2>(v);
  v += dpp<kRowHalfMirror>(v);
  v += dpp<kRowMirror>(v);
  return v;
}

// One butterfly stage across lanes: lanes whose `upper` bit is set hold the
// second element of each pair.  new = low + high (low lane), low - high
// (high lane), i.e. partner + (upper ? -mine : mine).
template <int CTRL>
__device__ __forceinline__ void xstage(float (&v)[8], bool upper) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float p = dpp<CTRL>(v[e]);
    v[e] = p + (upper ? -v[e] : v[e]);
  }
}

__device__ __forceinline__ void xstage_xor4(float (&v)[8], bool upper) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float p = dpp_xor4(v[e]);
    v[e] = p + (upper ? -v[e] : v[e]);
  }
}

// Walsh-Hadamard transform (Sylvester order, no scaling) of one 128-block
// spread over the 16 lanes of a DPP row: lane jj holds elements 8jj..8jj+7.
// Stages with strides 1, 2, 4 are inside a lane; strides 8, 16, 32, 64 pair
// lane jj with lane jj ^ 1, ^ 2, ^ 4, ^ 8.
__device__ __forceinline__ void fwht128_row16(float (&v)[8], int jj) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (!(e & h)) {
        float a = v[e], b = v[e + h];
        v[e] = a + b;
        v[e + h] = a - b;
      }
    }
  }
  xstage<kQuadXor1>(v, jj & 1);
  xstage<kQuadXor2>(v, jj & 2);
  xstage_xor4(v, jj & 4);
  xstage<kRowRor8>(v, jj & 8);
}

// The same transform with each cross-lane stage as one fused multiply-add
// fed by DPP: stored = mine + beta * partner, beta = -1 on the lane holding
// the pair's second element.  The high lane then holds the negated
// difference, so after the four cross-lane stages lane jj holds the
// transform times (-1)^popcount(jj); callers fold that sign into their
// scale (fwht_lane_sign).
template <int CTRL>
__device__ __forceinline__ void xstage_fma(float (&v)[8], float beta) {
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = fmaf(dpp<CTRL>(v[e]), beta, v[e]);
}

// The four cross-lane stages as fused DPP multiply-adds in one statement:
// v_fmac_f32_dpp takes the partner lane's value as its first source, so a
// stage is 8 instructions (the lane ^ 4 stage 16: two DPP moves make that
// partner).  Written with separate moves the compiler needs a move and a
// wait state per element and stage.  Hazards: a DPP source must be written
// at least two instructions before it is read; inside the statement every
// value is read 8 instructions after its write, the leading s_nop covers
// the writes just before it and the trailing one a DPP read of an output
// right after it.
__device__ __forceinline__ void fwht_xstages_dpp(float (&v)[8], float b1, float b2, float b4, float b8) {
#define WQ_X8(CTRL, B)                                                   \
  "v_fmac_f32_dpp %0, %0, " B " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
  "v_fmac_f32_dpp %1, %1, " B " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
  "v_fmac_f32_dpp %2, %2, " B " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
  "v_fmac_f32_dpp %3, %3, " B " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
  "v_fmac_f32_dpp %4, %4, " B " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
  "v_fmac_f32_dpp %5, %5, " B " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
  "v_fmac_f32_dpp %6, %6, " B " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
  "v_fmac_f32_dpp %7, %7, " B " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
  float t[8];
  asm volatile(
      "s_nop 1\n\t"
      WQ_X8("quad_perm:[1,0,3,2]", "%16")
      WQ_X8("quad_perm:[2,3,0,1]", "%17")
      "v_mov_b32_dpp %8, %0 row_half_mirror row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mov_b32_dpp %9, %1 row_half_mirror row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mov_b32_dpp %10, %2 row_half_mirror row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mov_b32_dpp %11, %3 row_half_mirror row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mov_b32_dpp %12, %4 row_half_mirror row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mov_b32_dpp %13, %5 row_half_mirror row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mov_b32_dpp %14, %6 row_half_mirror row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mov_b32_dpp %15, %7 row_half_mirror row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %0, %8, %18 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %1, %9, %18 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %2, %10, %18 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %3, %11, %18 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %4, %12, %18 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %5, %13, %18 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %6, %14, %18 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %7, %15, %18 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      WQ_X8("row_ror:8", "%19")
      "s_nop 1"
      : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]),
        "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]), "=&v"(t[6]), "=&v"(t[7])
      : "v"(b1), "v"(b2), "v"(b4), "v"(b8));
#undef WQ_X8
}

__device__ __forceinline__ void fwht128_row16_signed(float (&v)[8], int jj) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (!(e & h)) {
        float a = v[e], b = v[e + h];
        v[e] = a + b;
        v[e + h] = a - b;
      }
    }
  }
#if defined(__HIP_DEVICE_COMPILE__)
  fwht_xstages_dpp(v, (jj & 1) ? -1.0f : 1.0f, (jj & 2) ? -1.0f : 1.0f, (jj & 4) ? -1.0f : 1.0f,
                   (jj & 8) ? -1.0f : 1.0f);
#endif
}

__device__ __forceinline__ float fwht_lane_sign(int jj) {
  return (__builtin_popcount(jj & 15) & 1) ? -1.0f : 1.0f;
}

__device__ __forceinline__ uint32_t pack_half2(float lo, float hi) {
  _Float16 a = (_Float16)lo, b = (_Float16)hi;   // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// The descriptor of the linear that workgroup (or tile) w belongs to.  Its
// fields are all read in one round of scalar loads: read where first used,
// each would wait for its own round trip to the argument block, and the
// first weight load waits for the pointers.
// The first workgroups of linears 1 .. 7 (first_tile[1 .. 7]), passed as
// the kernel's first seven arguments: the build preloads them into scalar
// registers, so the descriptor's address is known without a round trip to
// the kernel arguments (0.1 us per launch of the seven-projection block).
struct FirstTiles {
  int t1, t2, t3, t4, t5, t6, t7;
};

__device__ __forceinline__ LinDesc fetch_desc(const GemvArgs &a, int w, FirstTiles f) {
  int l = 0;
  if (w >= f.t1) l = 1;
  if (w >= f.t2) l = 2;
  if (w >= f.t3) l = 3;
  if (w >= f.t4) l = 4;
  if (w >= f.t5) l = 5;
  if (w >= f.t6) l = 6;
  if (w >= f.t7) l = 7;
  const LinDesc L = a.lin[l];
  asm volatile("" ::"s"(L.codes), "s"(L.scales), "s"(L.zeros), "s"(L.signs), "s"(L.x), "s"(L.y), "s"(L.ldx),
               "s"(L.ldy), "s"(L.n), "s"(L.k), "s"(L.rows_per_wg), "s"(L.tile_begin), "s"(L.out_f32));
  return L;
}

// The same with the first workgroups read from the launch arguments.
__device__ __forceinline__ LinDesc fetch_desc(const GemvArgs &a, int w) {
  return fetch_desc(a, w, FirstTiles{a.first_tile[1], a.first_tile[2], a.first_tile[3], a.first_tile[4],
                                     a.first_tile[5], a.first_tile[6], a.first_tile[7]});
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

}  // namespace dev
}  // namespace wq
#endif

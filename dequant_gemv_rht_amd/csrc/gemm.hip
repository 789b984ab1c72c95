// Matrix-core path for batch sizes M >= 17 (gfx950): y = x' . W^T with the
// weight dequantised in registers and multiplied on MFMA
// (v_mfma_f32_32x32x16_f16, fp32 accumulate).  Same layer as the GEMV:
// w = (q - z) s per group of 128 along K (model card "24B0978 - Week 01 -
// Track 2, 20% target", section "How these techniques accelerate inference
// on CUDA", group-wise affine paragraph); x' is the activation already
// rotated by the block Hadamard transform (the caller runs rht_apply's
// kernel into the workspace first).
//
// One launch serves every linear of a batch: workgroups are dealt to the
// linears by a packed table of first tiles, like the GEMV.
//
// Tiling (Tile below).  A workgroup of 4 waves owns a tile of y and a range
// of K in steps of 64 (half a group, so a step never straddles two scales).
// From 65 batch rows the tile is 128 (batch rows) x 256 (outputs), each wave
// 128 x 64: 4 x 2 blocks of 32 x 32, 128 fp32 accumulators per lane.  From
// 17 to 64 rows, where the weights dominate the traffic, it is 32 or 64 x
// 128, each wave one or two blocks of one 32-wide column block, with more
// steps in flight.  A long K is split over several workgroups whose fp32
// partial tiles a second kernel adds.
//
// Activations (A operand) travel HBM -> LDS by direct buffer-to-LDS loads,
// kAhead steps in flight; every wave loads a quarter of the tile's rows and a
// barrier per step publishes them.  In LDS a row is 128 bytes (64 fp16) in
// eight 16-byte chunks, chunk c of row r stored at slot c ^ (r & 7): the 32
// lanes reading one chunk of 32 rows then spread over all banks.
//
// Weights (B operand) never pass through LDS.  The MFMA wants lane l to hold
// B[k = 8 (l / 32) .. +8][n = l % 32] of each 16-k block; the four blocks of
// a 64-k step are free to take any k of the step as long as the activations
// use the same ones, so lane l takes the step's k = 32 (l / 32) .. +32: the
// 32-code slice of row n the packing already keeps contiguous (int4: one
// 16-byte load).  Codes become fp16 in natural k order -- int4: v_perm_b32
// puts a code byte into both halves, one v_and_or_b32 masks the low nibble
// into the low half and the high nibble into bits 4..7 of the high half, each
// over 1024.0's bit pattern (1024 + q, 1024 + 16 q); int8: v_perm_b32 places
// two bytes next to 0x64 bytes; int3/int6: bit fields spread over the two
// halves -- then q exactly with one packed fma and q - z in fp16 (exact
// for an integer zero point, which round-to-nearest quantisation always
// gives).  int4 up to 64 batch rows takes activations that the rotation
// stored in pair order instead (b_operand4p): cheaper unpack, and one fma
// per pair where the wave's zero points are integers.
//
// Scales.  The products of a group of 128 are (q - z) x in fp32; the group's
// scale s multiplies their sum, not the weight, so the weight is never
// rounded to fp16 with its scale.  Instead of a second accumulator per group
// the accumulator is kept in units of the current group's scale: at the
// first step of a group it is multiplied by s_prev / s (one multiply per
// accumulator per group), and the epilogue multiplies it by the last scale.
// A group whose scale is 0 contributes nothing: its operand is masked to 0
// and the units stay those of the previous group.
//
// MFMA operand layout (checked on the device): lane l holds A[l % 32][8 (l /
// 32) .. +8] and B[8 (l / 32) .. +8][l % 32]; accumulator register v of lane
// l is C[8 (v / 4) + 4 (l / 32) + v % 4][l % 32].
#include "wq_internal.h"

#include <algorithm>
#include <climits>
#include <cstring>
#include <type_traits>

namespace wq {
using namespace dev;

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void *lds_ptr_t;

constexpr int kBK = 64;
constexpr int kWaves = 4, kGemmThreads = 64 * kWaves;
// Tile shapes: each wave owns MB x NB blocks of 32 x 32 outputs, the four
// waves side by side along N: a workgroup tile of 32 MB batch rows x 128 NB
// outputs.  MB = 4, NB = 2 (128 x 256) for long batches; MB = 1 or 2 with
// NB = 1 (32 or 64 x 128) from 17 to 64 rows, where the weights dominate
// the traffic and narrower tiles give enough workgroups without cutting K.
template <int MB, int NB>
struct Tile {
  static constexpr int TM = 32 * MB, TN = 32 * NB * kWaves;
  static constexpr int AStage = TM * kBK * 2;   // bytes of one step's activations in LDS
  // steps in flight + 1 (activation stages in LDS, weight register sets);
  // for the narrow tiles 3, 5 and 8 stages measured alike (3 marginally best)
  static constexpr int Stages = 3;
  // workgroups per CU: three narrow tiles fit (LDS: Stages x AStage of
  // activations plus the scale table; registers), two wide ones
  static constexpr int PerCU = MB == 4 ? 2 : 3;
};
constexpr int kMaxSteps = 48;                 // 64-k steps per workgroup at most (longer K is split)
constexpr int kMaxGroups = kMaxSteps / 2 + 1; // groups of 128 a workgroup's K range touches at most

// LDS slot of 16-byte chunk c of activation row r
__device__ __forceinline__ int a_slot(int c, int r) { return c ^ (r & 7); }
constexpr uint32_t kMagic = 0x64006400u;      // two fp16 1024.0

struct GemmLin {
  const uint32_t *codes;
  const uint16_t *scales, *zeros;
  const uint16_t *x;     // rotated activations [m][ldx]
  void *y;
  float *part;           // ksplit > 1: fp32 partial tiles [ksplit][m][n]
  int64_t ldx, ldy;
  int32_t m, n, k, out_f32;
  int32_t mtiles, ntiles, ksplit, ksteps;   // ksteps: 64-k steps per split
  int32_t tile_begin;
};

struct GemmBatch {
  int32_t first_tile[kMaxBatch];   // lin[i].tile_begin, packed; INT32_MAX past count
  GemmLin lin[kMaxBatch];
  int32_t count, tiles;
};

__device__ __forceinline__ half2v as_h2(uint32_t v) { return __builtin_bit_cast(half2v, v); }
__device__ __forceinline__ uint32_t as_u32(half2v v) { return __builtin_bit_cast(uint32_t, v); }

// A lane's 32-code slice (BITS words) of one weight row: vector offset
// `off` (the row, range checked), scalar offset `so` (the slice in the row).
template <int BITS>
__device__ __forceinline__ void load_slice(rsrc_t rs, uint32_t off, uint32_t so, uint32_t (&w)[BITS]) {
  if constexpr (BITS == 4) {
    const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, so, 0));
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (BITS == 8) {
    const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, so, 0));
    const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16, so, 0));
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  } else if constexpr (BITS == 6) {
    const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, so, 0));
    const u32x2 b = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off + 16, so, 0));
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y;
  } else {
    const u32x3 v = __builtin_bit_cast(u32x3, __builtin_amdgcn_raw_buffer_load_b96(rs, off, so, 0));
    w[0] = v.x; w[1] = v.y; w[2] = v.z;
  }
}

// Mask and bias of the unpack, held in VGPRs so that one v_and_or_b32 takes
// both (a VOP3 instruction encodes at most one literal).
struct PairConsts {
  uint32_t mask, bias;
};

template <int BITS>
__device__ __forceinline__ PairConsts pair_consts() {
  constexpr uint32_t m = BITS == 4 ? 0x00F0000Fu : BITS == 3 ? 0x00070007u : 0x003F003Fu;
  PairConsts c;
  asm volatile("v_mov_b32 %0, %1" : "=v"(c.mask) : "i"(m));
  asm volatile("v_mov_b32 %0, %1" : "=v"(c.bias) : "i"(kMagic));
  return c;
}

template <int BIT, int WIDTH, int N>
__device__ __forceinline__ uint32_t bits_at(const uint32_t (&w)[N]) {
  constexpr int wi = BIT / 32, off = BIT % 32;
  if constexpr (off + WIDTH <= 32) {
    return __builtin_amdgcn_ubfe(w[wi], off, WIDTH);
  } else {
    return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], off) & ((1u << WIDTH) - 1);
  }
}

// Codes 2P and 2P + 1 of the slice as two fp16 values over 1024: (1024 +
// q0, 1024 + q1), int4: (1024 + q0, 1024 + 16 q1).
template <int BITS, int P>
__device__ __forceinline__ uint32_t code_pair(const uint32_t (&w)[BITS], PairConsts k) {
  if constexpr (BITS == 4) {
    constexpr int wi = P / 4, b = P % 4;    // byte b of word wi holds codes 2P (low nibble), 2P + 1
    const uint32_t t = __builtin_amdgcn_perm(w[wi], w[wi], (uint32_t)(b | (b << 8) | (b << 16) | (b << 24)));
    return (t & k.mask) | k.bias;
  } else if constexpr (BITS == 8) {
    // bytes b, b + 1 of word wi next to byte 1 of the bias (0x64); selectors
    // 0..3 take bytes of the second operand, 4..7 of the first
    constexpr int wi = P / 2, b = 2 * (P % 2);
    return __builtin_amdgcn_perm(k.bias, w[wi], (uint32_t)(b | (5 << 8) | ((b + 1) << 16) | (5 << 24)));
  } else if constexpr (BITS == 3) {
    const uint32_t t = bits_at<6 * P, 6>(w);
    return ((t | (t << 13)) & k.mask) | k.bias;
  } else {
    constexpr int run = P / 8, q = P % 8;    // two 96-bit runs of 16 codes
    const uint32_t t = (run == 0) ? bits_at<12 * q, 12>(w) : bits_at<96 + 12 * q, 12>(w);
    return ((t | (t << 10)) & k.mask) | k.bias;
  }
}

// The lane's B operand of 16-k block kk: codes 8 kk .. 8 kk + 7 of its slice
// as q - z: q = h c + d exactly (c, d per half remove the 1024 offset and
// the int4 factor 16), then q - z, exact for an integer zero point and
// rounded once otherwise.  FAST (every zero point of the wave's rows an
// integer in [-1024, 1023]): the caller passes d - z as d and one fma gives
// q - z (h c and d - z are exact in fp16, and so is the integer q - z, of
// magnitude below 2048, that the fma rounds).  The scale is not applied
// here: the accumulator carries it (see the step below).  For a group whose
// scale is 0, c, d and z come in as 0 and the operand is 0.
template <int BITS, int KK, bool FAST = false>
__device__ __forceinline__ half8 b_operand(const uint32_t (&w)[BITS], PairConsts k, half2v c, half2v d, half2v z) {
  uint32_t p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t h;
    switch (i) {
      case 0: h = code_pair<BITS, 4 * KK + 0>(w, k); break;
      case 1: h = code_pair<BITS, 4 * KK + 1>(w, k); break;
      case 2: h = code_pair<BITS, 4 * KK + 2>(w, k); break;
      default: h = code_pair<BITS, 4 * KK + 3>(w, k); break;
    }
    const half2v q = __builtin_elementwise_fma(as_h2(h), c, d);
    p[i] = as_u32(FAST ? q : q - z);
  }
  return __builtin_bit_cast(half8, u32x4{p[0], p[1], p[2], p[3]});
}

// int4 with the activations in pair order (each 8-element group stored as
// 0, 4, 1, 5, 2, 6, 3, 7 by the rotation pre-pass): code word KK of the
// slice, nibbles 0..7, gives the pairs (0, 4) and (2, 6) as (1024 + q) from
// the word and the word shifted by 8 under mask 0x000F000F, and (1, 5),
// (3, 7) as (1024 + 16 q) under mask 0x00F000F0: one shift and four
// v_and_or_b32 for the eight codes (against a v_perm_b32 and a v_and_or_b32
// per pair in natural order).  Then q - z:
//  * FAST (every zero point of the step an integer in [-1024, 1023], as
//    round-to-nearest always gives): one fma per pair, h c + (d - z) with
//    (c, d) = (1, -1024) or (1/16, -64); the product and the addend are
//    exact in fp16, so the fma's one rounding of the exact q - z (an
//    integer below 2048) is exact;
//  * else h c + d (exactly q), then q - z, rounded once.
// c, d and z come in as 0 for a group whose scale is 0 (operand 0).
struct PairConsts4 {
  uint32_t lo, hi, bias;
};

__device__ __forceinline__ PairConsts4 pair_consts4() {
  PairConsts4 c;
  asm volatile("v_mov_b32 %0, %1" : "=v"(c.lo) : "i"(0x000F000Fu));
  asm volatile("v_mov_b32 %0, %1" : "=v"(c.hi) : "i"(0x00F000F0u));
  asm volatile("v_mov_b32 %0, %1" : "=v"(c.bias) : "i"(kMagic));
  return c;
}

template <int KK, bool FAST>
__device__ __forceinline__ half8 b_operand4p(const uint32_t (&w)[4], PairConsts4 k, half2v c1, half2v d1,
                                             half2v c16, half2v d16, half2v z) {
  const uint32_t x = w[KK], x8 = x >> 8;
  half2v q[4] = {__builtin_elementwise_fma(as_h2((x & k.lo) | k.bias), c1, d1),
                 __builtin_elementwise_fma(as_h2((x & k.hi) | k.bias), c16, d16),
                 __builtin_elementwise_fma(as_h2((x8 & k.lo) | k.bias), c1, d1),
                 __builtin_elementwise_fma(as_h2((x8 & k.hi) | k.bias), c16, d16)};
  if constexpr (!FAST) {
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = q[i] - z;
  }
  return __builtin_bit_cast(half8, u32x4{as_u32(q[0]), as_u32(q[1]), as_u32(q[2]), as_u32(q[3])});
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// The same wait, also taking a step's weight registers as operands, so that
// no arithmetic on them is scheduled above it.
template <int N, int BITS, int NB>
__device__ __forceinline__ void wait_vmcnt_regs(uint32_t (&w)[NB][BITS]) {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int e = 0; e < BITS; ++e) asm volatile("" : "+v"(w[j][e]));
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)(lds_ptr_t)p; }

// The A operands of one 16-k block for the MB m blocks (32 rows apart, 4096
// bytes) of a stage at byte offset OFF, read and waited for in one
// statement.  Reading the direct-loaded tile in asm keeps the compiler from
// tying these reads to the outstanding direct loads of other stages with
// waits of its own.
template <int OFF, int MB>
__device__ __forceinline__ void read_a(uint32_t addr, half8 (&a)[MB]) {
  if constexpr (MB == 4) {
    asm volatile(
        "ds_read_b128 %0, %4 offset:%5\n\t"
        "ds_read_b128 %1, %4 offset:%6\n\t"
        "ds_read_b128 %2, %4 offset:%7\n\t"
        "ds_read_b128 %3, %4 offset:%8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
        : "v"(addr), "i"(OFF), "i"(OFF + 4096), "i"(OFF + 8192), "i"(OFF + 12288)
        : "memory");
  } else if constexpr (MB == 2) {
    asm volatile(
        "ds_read_b128 %0, %2 offset:%3\n\t"
        "ds_read_b128 %1, %2 offset:%4\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a[0]), "=&v"(a[1])
        : "v"(addr), "i"(OFF), "i"(OFF + 4096)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %1 offset:%2\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a[0])
        : "v"(addr), "i"(OFF)
        : "memory");
  }
}

// The packed scale and zero (s | z << 16) of the lane's NB rows for one
// step, read from LDS and waited for in one statement (kept out of the
// compiler's view like read_a).
template <int NB>
__device__ __forceinline__ void read_sz(uint32_t a0, uint32_t a1, uint32_t (&v)[NB]) {
  if constexpr (NB == 2) {
    asm volatile(
        "ds_read_b32 %0, %2\n\t"
        "ds_read_b32 %1, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1])
        : "v"(a0), "v"(a1)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b32 %0, %1\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0])
        : "v"(a0)
        : "memory");
  }
}

// The step's LDS operands of a narrow tile (NB = 1, MB <= 2): the packed
// scale and zero of the lane's row and the A fragments of all four 16-k
// blocks, in one statement with one wait (with few products per step, LDS
// round trips waited on one by one would set the step's length).
template <int OFF, int MB>
__device__ __forceinline__ void read_step_narrow(uint32_t sza, const uint32_t (&ard)[4], uint32_t &sz,
                                                 half8 (&a)[4][MB]) {
  if constexpr (MB == 1) {
    asm volatile(
        "ds_read_b32 %0, %5\n\t"
        "ds_read_b128 %1, %6 offset:%10\n\t"
        "ds_read_b128 %2, %7 offset:%10\n\t"
        "ds_read_b128 %3, %8 offset:%10\n\t"
        "ds_read_b128 %4, %9 offset:%10\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(sz), "=&v"(a[0][0]), "=&v"(a[1][0]), "=&v"(a[2][0]), "=&v"(a[3][0])
        : "v"(sza), "v"(ard[0]), "v"(ard[1]), "v"(ard[2]), "v"(ard[3]), "i"(OFF)
        : "memory");
  } else {
    static_assert(MB == 2, "narrow tiles have one or two m blocks");
    asm volatile(
        "ds_read_b32 %0, %9\n\t"
        "ds_read_b128 %1, %10 offset:%14\n\t"
        "ds_read_b128 %2, %10 offset:%15\n\t"
        "ds_read_b128 %3, %11 offset:%14\n\t"
        "ds_read_b128 %4, %11 offset:%15\n\t"
        "ds_read_b128 %5, %12 offset:%14\n\t"
        "ds_read_b128 %6, %12 offset:%15\n\t"
        "ds_read_b128 %7, %13 offset:%14\n\t"
        "ds_read_b128 %8, %13 offset:%15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(sz), "=&v"(a[0][0]), "=&v"(a[0][1]), "=&v"(a[1][0]), "=&v"(a[1][1]), "=&v"(a[2][0]),
          "=&v"(a[2][1]), "=&v"(a[3][0]), "=&v"(a[3][1])
        : "v"(sza), "v"(ard[0]), "v"(ard[1]), "v"(ard[2]), "v"(ard[3]), "i"(OFF), "i"(OFF + 4096)
        : "memory");
  }
}

// Logical tile of workgroup b: runs of consecutive tiles (the m tiles of one
// n tile and K split, which read the same weights) on one XCD, so they share
// its L2; workgroups are dealt to the 8 XCDs round robin.
__device__ __forceinline__ int logical_tile(int b, int nb) {
  const int xcd = b % 8, slot = b / 8, q = nb / 8, rem = nb % 8;
  return (xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q) + slot;
}

// PAIR: int4 with the activations in pair order (b_operand4p)
template <int BITS, int MB, int NB, bool PAIR>
__global__ __launch_bounds__(kGemmThreads, (Tile<MB, NB>::PerCU)) void gemm_kernel(GemmBatch a) {
  static_assert(!PAIR || BITS == 4, "pair order is an int4 layout");
  using TL = Tile<MB, NB>;
  constexpr int kTM = TL::TM, kTN = TL::TN, kAStage = TL::AStage;
  constexpr int kStages = TL::Stages, kAhead = kStages - 1;   // kAhead: steps loaded ahead of the one computed
  constexpr int WR = 32 * NB;   // weight rows (outputs) per wave
  __shared__ __attribute__((aligned(16))) uint8_t As[kStages * kAStage];
  // scale and zero of each wave's WR rows over the workgroup's groups, (s | z << 16)
  __shared__ uint32_t SZ[kWaves * WR * kMaxGroups];
  const int tile = logical_tile(blockIdx.x, a.tiles);
  int l = 0;
#pragma unroll
  for (int i = 1; i < kMaxBatch; ++i)
    if (tile >= a.first_tile[i]) l = i;
  const GemmLin L = a.lin[l];
  int local = tile - L.tile_begin;
  const int mt = local % L.mtiles;
  local /= L.mtiles;
  const int nt = local % L.ntiles, ks = local / L.ntiles;
  const int m0 = mt * kTM, n0 = nt * kTN;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int S = L.k / kSlice, G = L.k / kGroup, wpr = S * BITS;
  const int kt0 = ks * L.ksteps, T = min(L.ksteps, L.k / kBK - kt0);

  // Each lane's offsets are fixed for the whole K range (the vector offset,
  // which the range check covers: rows past M or N read zero); a step's
  // position goes in the scalar offset, which never takes a load past its
  // row's end.  Steps past the range reload the range's last step, so every
  // step issues the same loads and the counts waited on are constants.
  //
  // activations: rows m0 .. m0 + kTM - 1; this wave loads rows 8 MB wave +
  // 8 i + lane / 8 (i < MB), chunk slot lane % 8
  const rsrc_t rx = make_rsrc(L.x + (size_t)m0 * L.ldx, (uint32_t)((size_t)min(kTM, L.m - m0) * L.ldx * 2));
  const int arow = 8 * MB * wave + (lane >> 3), aslot = lane & 7;
  uint32_t a_vo[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
    a_vo[i] = (uint32_t)((size_t)(arow + 8 * i) * L.ldx * 2) + (uint32_t)(a_slot(aslot, arow + 8 * i) * 16);
  const uint32_t as0 = lds_addr(As) + (uint32_t)(wave * MB * 1024);
  // weights: rows nw0 + 32 j + lane % 32, slice 2 kt + lane / 32 of the row
  const int nw0 = n0 + WR * wave;
  // (uniform: a clamp would otherwise become a vector med3 and the resources divergent)
  const int nrows = __builtin_amdgcn_readfirstlane(max(0, min(WR, L.n - nw0)));
  const rsrc_t rc = make_rsrc(L.codes + (size_t)nw0 * wpr, (uint32_t)nrows * wpr * 4);
  const rsrc_t rs = make_rsrc(L.scales + (size_t)nw0 * G, (uint32_t)nrows * G * 2);
  const rsrc_t rz = make_rsrc(L.zeros + (size_t)nw0 * G, (uint32_t)nrows * G * 2);
  const int bn = lane & 31, bh = lane >> 5;
  const uint32_t b_vo0 = (uint32_t)(bn * wpr * 4 + bh * BITS * 4), b_vo1 = b_vo0 + (uint32_t)(32 * wpr * 4);

  // scales and zeros of this wave's rows (lane = row, lanes < WR) over the
  // split's groups g0 .. g0 + ng - 1: loaded once here, written to LDS once
  // the first steps' loads are out; rows past N read zero
  const int g0 = kt0 >> 1, ng = ((kt0 + T - 1) >> 1) - g0 + 1;
  uint32_t szs[kMaxGroups], szz[kMaxGroups];
#pragma unroll
  for (int g = 0; g < kMaxGroups; ++g) {
    const uint32_t off = g < ng && lane < WR ? (uint32_t)((lane * G + g0 + g) * 2) : kOOB;
    szs[g] = __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0);
    szz[g] = __builtin_amdgcn_raw_buffer_load_b16(rz, off, 0, 0);
  }
  uint32_t *szw = SZ + wave * WR * kMaxGroups;
  const uint32_t sz_rd0 = lds_addr(szw) + (uint32_t)(bn * kMaxGroups * 4), sz_rd1 = sz_rd0 + 32 * kMaxGroups * 4;

  uint32_t cw[kStages][NB][BITS];
  auto issue = [&](auto sconst, int kt) {
    constexpr int st = decltype(sconst)::value;
    const int kc = min(kt, kt0 + T - 1);
    const uint32_t so_a = (uint32_t)kc * (kBK * 2), so_b = (uint32_t)kc * (2 * BITS * 4);
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
    for (int i = 0; i < MB; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)(as0 + st * kAStage + i * 1024), 16, a_vo[i], so_a, 0, 0);
#endif
    load_slice<BITS>(rc, b_vo0, so_b, cw[st][0]);
    if constexpr (NB == 2) load_slice<BITS>(rc, b_vo1, so_b, cw[st][1]);
  };
  // vector-memory operations of one issue, the count waited on
  constexpr int kLoadsB = BITS == 3 || BITS == 4 ? 1 : 2;
  constexpr int kIssue = MB + NB * kLoadsB;

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x16{};

  // A fragment of m block i, 16-k block kk: row 32 i + lane % 32, k 32 (lane / 32) + 8 kk,
  // i.e. chunk 4 (lane / 32) + kk of the row at slot chunk ^ (row & 7)
  const int ar = lane & 31;
  uint32_t a_rd[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) a_rd[kk] = lds_addr(As) + (uint32_t)(ar * 128 + (a_slot(4 * bh + kk, ar) << 4));
  constexpr _Float16 kHi = BITS == 4 ? (_Float16)0.0625f : (_Float16)1.0f;
  const PairConsts pk = pair_consts<BITS>();
  const PairConsts4 pk4 = pair_consts4();

  // One step: the waits, the barrier and the loads are unconditional (a
  // step past the range only skips the products), so every iteration of the
  // loop has the same loads in flight and the compiler's own waits for the
  // weight registers stay as loose as this step's explicit one.
  // unit[j]: the scale the accumulators of the lane's row j are counted in
  float unit[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) unit[j] = 1.0f;

  // FAST (narrow tiles): every zero point of the wave's rows over its K
  // range takes the one-fma path; chosen once per wave, before the loop, so
  // that the step stays one straight block the compiler can interleave
  auto step = [&](auto sconst, int kt, bool active, auto fconst) {
    constexpr int st = decltype(sconst)::value;
    constexpr bool fast = decltype(fconst)::value;
    constexpr int nx = (st + kAhead) % kStages;
    // this step's activations (this wave's rows) and weights: the younger
    // loads are those of the kAhead - 1 steps issued after it
    wait_vmcnt_regs<(kAhead - 1) * kIssue, BITS, NB>(cw[st]);
    __builtin_amdgcn_s_barrier();   // every wave's rows are in; step kt - 1's stage is free
    issue(std::integral_constant<int, nx>{}, kt + kAhead);
    if (!active) return;
    uint32_t szv[NB];
    const uint32_t gofs = (uint32_t)(((kt >> 1) - g0) * 4);
    constexpr bool kNarrow = NB == 1 && MB <= 2;
    half8 aall[4][kNarrow ? MB : 1];
    if constexpr (kNarrow)
      read_step_narrow<st * kAStage, MB>(sz_rd0 + gofs, a_rd, szv[0], aall);
    else
      read_sz<NB>(sz_rd0 + gofs, sz_rd1 + gofs, szv);
    // the first step of a group (or of the workgroup's K range): the
    // accumulators change units from the previous group's scale to this one's
    const bool gstart = (kt & 1) == 0 || kt == kt0;
    half8 bop[NB][4];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const float sf = half_bits_to_float(szv[j] & 0xFFFFu);
      const bool live = sf != 0.0f;
      if (gstart) {
        // the ratio need not be exact: its rounding (v_rcp_f32 is within
        // 1 ulp) changes the accumulated sum by a few parts in 2^24
        const float r = live ? unit[j] * __builtin_amdgcn_rcpf(sf) : 1.0f;
        unit[j] = live ? sf : unit[j];
#pragma unroll
        for (int i = 0; i < MB; ++i) acc[i][j] *= r;
      }
      const half2v z = live ? as_h2((szv[j] >> 16) * 0x10001u) : half2v{};
      if constexpr (PAIR) {
        const half2v c1 = live ? half2v{(_Float16)1.0f, (_Float16)1.0f} : half2v{};
        const half2v c16 = live ? half2v{(_Float16)0.0625f, (_Float16)0.0625f} : half2v{};
        half2v d1 = live ? half2v{(_Float16)-1024.0f, (_Float16)-1024.0f} : half2v{};
        half2v d16 = live ? half2v{(_Float16)-64.0f, (_Float16)-64.0f} : half2v{};
        if constexpr (fast) {
          d1 = d1 - z;
          d16 = d16 - z;
          bop[j][0] = b_operand4p<0, true>(cw[st][j], pk4, c1, d1, c16, d16, z);
          bop[j][1] = b_operand4p<1, true>(cw[st][j], pk4, c1, d1, c16, d16, z);
          bop[j][2] = b_operand4p<2, true>(cw[st][j], pk4, c1, d1, c16, d16, z);
          bop[j][3] = b_operand4p<3, true>(cw[st][j], pk4, c1, d1, c16, d16, z);
        } else {
          bop[j][0] = b_operand4p<0, false>(cw[st][j], pk4, c1, d1, c16, d16, z);
          bop[j][1] = b_operand4p<1, false>(cw[st][j], pk4, c1, d1, c16, d16, z);
          bop[j][2] = b_operand4p<2, false>(cw[st][j], pk4, c1, d1, c16, d16, z);
          bop[j][3] = b_operand4p<3, false>(cw[st][j], pk4, c1, d1, c16, d16, z);
        }
      } else {
        const half2v c = live ? half2v{(_Float16)1.0f, kHi} : half2v{};
        half2v d = live ? half2v{(_Float16)-1024.0f, (_Float16)(BITS == 4 ? -64.0f : -1024.0f)} : half2v{};
        if constexpr (fast) d = d - z;
        bop[j][0] = b_operand<BITS, 0, fast>(cw[st][j], pk, c, d, z);
        bop[j][1] = b_operand<BITS, 1, fast>(cw[st][j], pk, c, d, z);
        bop[j][2] = b_operand<BITS, 2, fast>(cw[st][j], pk, c, d, z);
        bop[j][3] = b_operand<BITS, 3, fast>(cw[st][j], pk, c, d, z);
      }
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      half8 aop[MB];
      if constexpr (kNarrow) {
#pragma unroll
        for (int i = 0; i < MB; ++i) aop[i] = aall[kk][i];
      } else {
        read_a<st * kAStage, MB>(a_rd[kk], aop);
      }
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
#if defined(__HIP_DEVICE_COMPILE__)   // the 32x32x16 f16 MFMA exists only in the gfx950 pass
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop[i], bop[j][kk], acc[i][j], 0, 0, 0);
#endif
        }
    }
  };

  // the waits count loads in issue order: keep step kt0's loads ahead of
  // step kt0 + 1's (inside the loop the steps' asm waits keep the order)
  issue(std::integral_constant<int, 0>{}, kt0);
  asm volatile("" ::: "memory");
  issue(std::integral_constant<int, 1>{}, kt0 + 1);
  if constexpr (kAhead > 2) {
    asm volatile("" ::: "memory");
    issue(std::integral_constant<int, 2>{}, kt0 + 2);
  }
  if constexpr (kAhead > 3) {
    asm volatile("" ::: "memory");
    issue(std::integral_constant<int, 3>{}, kt0 + 3);
  }
  if constexpr (kAhead > 4) {
    asm volatile("" ::: "memory");
    issue(std::integral_constant<int, 4>{}, kt0 + 4);
  }
  if constexpr (kAhead > 5) {
    asm volatile("" ::: "memory");
    issue(std::integral_constant<int, 5>{}, kt0 + 5);
  }
  if constexpr (kAhead > 6) {
    asm volatile("" ::: "memory");
    issue(std::integral_constant<int, 6>{}, kt0 + 6);
  }
  // the scales and zeros into LDS (each wave reads back only its own rows)
#pragma unroll
  for (int g = 0; g < kMaxGroups; ++g)
    if (g < ng && lane < WR) szw[lane * kMaxGroups + g] = (szs[g] & 0xFFFFu) | (szz[g] << 16);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  static_assert(kStages >= 3 && kStages <= 8, "the loop below unrolls up to 8 stages");
  auto loop = [&](auto fconst) {
    for (int i0 = 0; i0 < T; i0 += kStages) {
      step(std::integral_constant<int, 0>{}, kt0 + i0, true, fconst);
      step(std::integral_constant<int, 1>{}, kt0 + i0 + 1, i0 + 1 < T, fconst);
      step(std::integral_constant<int, 2>{}, kt0 + i0 + 2, i0 + 2 < T, fconst);
      if constexpr (kStages > 3) step(std::integral_constant<int, 3>{}, kt0 + i0 + 3, i0 + 3 < T, fconst);
      if constexpr (kStages > 4) step(std::integral_constant<int, 4>{}, kt0 + i0 + 4, i0 + 4 < T, fconst);
      if constexpr (kStages > 5) step(std::integral_constant<int, 5>{}, kt0 + i0 + 5, i0 + 5 < T, fconst);
      if constexpr (kStages > 6) step(std::integral_constant<int, 6>{}, kt0 + i0 + 6, i0 + 6 < T, fconst);
      if constexpr (kStages > 7) step(std::integral_constant<int, 7>{}, kt0 + i0 + 7, i0 + 7 < T, fconst);
    }
  };
  // narrow tiles: the wave's zero points (lane = row, its groups of the K
  // range; rows past N read 0) all integers in [-1024, 1023]?  The 128 x
  // 256 tile keeps the general path: there the one-fma operand measured
  // slower (the int4 block at M = 512: 160.8 -> 166.4 us; 204 -> 221 VGPRs)
  if constexpr (MB <= 2) {
    bool ok = true;
#pragma unroll
    for (int g = 0; g < kMaxGroups; ++g) {
      const float zf = half_bits_to_float(szz[g] & 0xFFFFu);
      ok = ok && (g >= ng || lane >= WR || (zf == __builtin_floorf(zf) && zf >= -1024.0f && zf <= 1023.0f));
    }
    if (__ballot(!ok) == 0)
      loop(std::true_type{});
    else
      loop(std::false_type{});
  } else {
    loop(std::false_type{});
  }
  wait_vmcnt<0>();   // the trailing out-of-range loads still write LDS

  // epilogue: accumulator register v of lane l is C[8 (v/4) + 4 (l/32) + v%4][l % 32]
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int col = nw0 + 32 * j + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < L.m && col < L.n) {
          const float r = acc[i][j][v] * unit[j];
          if (L.ksplit > 1) {
            L.part[((size_t)ks * L.m + row) * L.n + col] = r;
          } else if (L.out_f32) {
            reinterpret_cast<float *>(L.y)[(size_t)row * L.ldy + col] = r;
          } else {
            const _Float16 h = (_Float16)r;
            reinterpret_cast<uint16_t *>(L.y)[(size_t)row * L.ldy + col] = __builtin_bit_cast(uint16_t, h);
          }
        }
      }
    }
}

// The K splits of a linear, added in split order: y = sum_s part[s].  Four
// columns per thread when n % 4 == 0, else one.
__host__ __device__ inline int64_t finalize_items(const GemmLin &L) {
  const int64_t mn = (int64_t)L.m * L.n;
  return L.n % 4 ? mn : mn / 4;
}

constexpr int kFinAhead = 8;

__global__ __launch_bounds__(256) void gemm_finalize_kernel(GemmBatch a) {
  int l = -1, base = 0;
  for (int i = 0; i < a.count; ++i) {
    if (a.lin[i].ksplit <= 1) continue;
    const int nblk = (int)((finalize_items(a.lin[i]) + 255) / 256);
    if ((int)blockIdx.x < base + nblk) {
      l = i;
      break;
    }
    base += nblk;
  }
  if (l < 0) return;
  const GemmLin &L = a.lin[l];
  const int64_t mn = (int64_t)L.m * L.n;
  const int64_t item = (int64_t)(blockIdx.x - base) * 256 + threadIdx.x;
  if (item >= finalize_items(L)) return;
  if (L.n % 4) {
    float s = L.part[item];
    for (int q = 1; q < L.ksplit; ++q) s += L.part[(size_t)q * mn + item];
    const int64_t row = item / L.n, col = item - row * L.n;
    if (L.out_f32)
      reinterpret_cast<float *>(L.y)[row * L.ldy + col] = s;
    else
      reinterpret_cast<uint16_t *>(L.y)[row * L.ldy + col] = __builtin_bit_cast(uint16_t, (_Float16)s);
    return;
  }
  const int64_t e = item * 4;   // 4 columns of one row
  // the first kFinAhead splits' loads all go out before the first add (one
  // round of load latency instead of one per split), then the rest in turn
  float4 pv[kFinAhead];
#pragma unroll
  for (int q = 0; q < kFinAhead; ++q)
    pv[q] = q < L.ksplit ? *reinterpret_cast<const float4 *>(&L.part[(size_t)q * mn + e]) : float4{0.f, 0.f, 0.f, 0.f};
  float4 s = pv[0];
#pragma unroll
  for (int q = 1; q < kFinAhead; ++q)
    if (q < L.ksplit) {
      s.x += pv[q].x; s.y += pv[q].y; s.z += pv[q].z; s.w += pv[q].w;
    }
  for (int q = kFinAhead; q < L.ksplit; ++q) {
    const float4 p = *reinterpret_cast<const float4 *>(&L.part[(size_t)q * mn + e]);
    s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
  }
  const int64_t row = e / L.n, col = e - row * L.n;
  if (L.out_f32) {
    float *y = reinterpret_cast<float *>(L.y) + row * L.ldy + col;
    y[0] = s.x; y[1] = s.y; y[2] = s.z; y[3] = s.w;
  } else {
    uint16_t *y = reinterpret_cast<uint16_t *>(L.y) + row * L.ldy + col;
    y[0] = __builtin_bit_cast(uint16_t, (_Float16)s.x);
    y[1] = __builtin_bit_cast(uint16_t, (_Float16)s.y);
    y[2] = __builtin_bit_cast(uint16_t, (_Float16)s.z);
    y[3] = __builtin_bit_cast(uint16_t, (_Float16)s.w);
  }
}

}  // namespace

bool gemm_available(int bits) { return bits == 3 || bits == 4 || bits == 6 || bits == 8; }
bool gemm_pair_order(int bits) { return bits == 4; }

namespace {

// The tile shape for a batch of m rows: MB m blocks and NB n blocks of 32
// per wave (see Tile).
struct Shape {
  int mb, nb;
  int tm() const { return 32 * mb; }
  int tn() const { return 32 * nb * kWaves; }
};

// Up to 64 rows one n block per wave: two (tiles of 256 outputs, half as
// many workgroups) measured 8% slower for a decoder block's projections.
Shape shape_for(int64_t m) {
  if (m <= 32) return {1, 1};
  if (m <= 64) return {2, 1};
  return {4, 2};
}

}  // namespace

// K splits per linear: long K is cut so that the workgroups of a launch have
// similar lengths; a split costs 8 M N bytes of fp32 partial traffic, so
// short linears stay whole.  Up to 64 batch rows the narrow tiles already
// give a workgroup per CU or so for a decoder block's projections: only K
// longer than about 40 steps (2560) is cut there, as the weights, not the
// partials, must dominate the traffic.
void gemm_plan(int count, const wq_weight *w, int64_t m, int *ksplit) {
  const Shape sh = shape_for(m);
  int64_t units = 0;
  for (int i = 0; i < count; ++i) {
    const int64_t tiles = ((m + sh.tm() - 1) / sh.tm()) * ((w[i].n + sh.tn() - 1) / sh.tn());
    units += tiles * (w[i].k / kBK);
  }
  const int64_t slots = (sh.mb == 4 ? 2 : 3) * 256;   // workgroups resident per CU (Tile::PerCU)
  const int64_t floor_steps = sh.mb == 4 ? 24 : 40;   // narrow tiles: 24 measured 3% slower than 40
  const int64_t target = std::max<int64_t>(floor_steps, (units + slots - 1) / slots);
  for (int i = 0; i < count; ++i) {
    const int64_t kt = w[i].k / kBK;
    int64_t s = (kt + target - 1) / target;
    s = std::max<int64_t>(1, std::min<int64_t>(s, kt / 8));
    // a workgroup's scales and zeros sit in LDS: at most kMaxSteps steps each
    s = std::max<int64_t>(s, (kt + kMaxSteps - 1) / kMaxSteps);
    ksplit[i] = (int)s;
  }
}

namespace {
template <int BITS, bool PAIR>
hipError_t launch_shape(Shape sh, dim3 grid, dim3 block, const GemmBatch &a, hipStream_t s) {
  if (sh.mb == 1)
    hipLaunchKernelGGL((gemm_kernel<BITS, 1, 1, PAIR>), grid, block, 0, s, a);
  else if (sh.mb == 2)
    hipLaunchKernelGGL((gemm_kernel<BITS, 2, 1, PAIR>), grid, block, 0, s, a);
  else if constexpr (!PAIR)
    hipLaunchKernelGGL((gemm_kernel<BITS, 4, 2, false>), grid, block, 0, s, a);
  else
    return hipErrorInvalidValue;   // pair order is taken by the narrow tiles only
  return hipGetLastError();
}
}  // namespace

size_t gemm_partial_bytes(const wq_weight &w, int64_t m, int ksplit) {
  return ksplit > 1 ? (size_t)ksplit * (size_t)m * (size_t)w.n * sizeof(float) : 0;
}

hipError_t launch_gemm_batch(int count, const wq_weight *w, const uint16_t *const *xr, const int64_t *ldx,
                             int64_t m, void *const *y, const int *out_f32, const int64_t *ldy,
                             const int *ksplit, float *const *part, bool pair_order, hipStream_t s) {
  if (count <= 0 || count > kMaxBatch) return hipErrorInvalidValue;
  if (pair_order && (!gemm_pair_order(w[0].bits) || shape_for(m).mb > 2)) return hipErrorInvalidValue;
  GemmBatch a;
  memset(&a, 0, sizeof a);
  for (int i = 0; i < kMaxBatch; ++i) a.first_tile[i] = INT32_MAX;
  a.count = count;
  const Shape sh = shape_for(m);
  int64_t tiles = 0, fin_blocks = 0;
  for (int i = 0; i < count; ++i) {
    if (!gemm_available(w[i].bits) || w[i].bits != w[0].bits || w[i].k % kBK) return hipErrorInvalidValue;
    if ((uint64_t)m * (uint64_t)ldx[i] * 2 > 0x7FFFFFFFull || (uint64_t)w[i].n * (uint64_t)w[i].k > 0x7FFFFFFFull)
      return hipErrorInvalidValue;   // 32-bit buffer offsets
    GemmLin &L = a.lin[i];
    L.codes = w[i].codes;
    L.scales = w[i].scales;
    L.zeros = w[i].zeros;
    L.x = xr[i];
    L.y = y[i];
    L.part = ksplit[i] > 1 ? part[i] : nullptr;
    if (ksplit[i] > 1 && !part[i]) return hipErrorInvalidValue;
    L.ldx = ldx[i];
    L.ldy = ldy[i];
    L.m = (int32_t)m;
    L.n = (int32_t)w[i].n;
    L.k = (int32_t)w[i].k;
    L.out_f32 = out_f32[i];
    L.mtiles = (int32_t)((m + sh.tm() - 1) / sh.tm());
    L.ntiles = (int32_t)((w[i].n + sh.tn() - 1) / sh.tn());
    const int kt = (int)(w[i].k / kBK);
    L.ksplit = ksplit[i];
    L.ksteps = (kt + ksplit[i] - 1) / ksplit[i];
    L.ksplit = (kt + L.ksteps - 1) / L.ksteps;   // no empty split
    if (L.ksteps > kMaxSteps) return hipErrorInvalidValue;
    L.tile_begin = (int32_t)tiles;
    a.first_tile[i] = (int32_t)tiles;
    tiles += (int64_t)L.mtiles * L.ntiles * L.ksplit;
    if (L.ksplit > 1) fin_blocks += (finalize_items(L) + 255) / 256;
  }
  if (tiles > INT32_MAX) return hipErrorInvalidValue;
  a.tiles = (int32_t)tiles;
  const dim3 grid((unsigned)tiles), block(kGemmThreads);
  hipError_t e = hipSuccess;
  switch (w[0].bits) {
    case 3: e = launch_shape<3, false>(sh, grid, block, a, s); break;
    case 4:
      e = pair_order && sh.mb <= 2 ? launch_shape<4, true>(sh, grid, block, a, s) : launch_shape<4, false>(sh, grid, block, a, s);
      break;
    case 6: e = launch_shape<6, false>(sh, grid, block, a, s); break;
    case 8: e = launch_shape<8, false>(sh, grid, block, a, s); break;
  }
  if (e != hipSuccess || fin_blocks == 0) return e;
  hipLaunchKernelGGL(gemm_finalize_kernel, dim3((unsigned)fin_blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace wq

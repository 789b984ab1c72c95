// Matrix-core path for batch sizes M >= 64 (gfx950): y = x' . W^T with the
// weight dequantised tile by tile into LDS and multiplied on MFMA
// (v_mfma_f32_32x32x16_f16, fp32 accumulate).  Same layer as the GEMV:
// w = (q - z) s per group of 128 along K (model card "24B0978 - Week 01 -
// Track 2, 20% target", section "How these techniques accelerate inference
// on CUDA", group-wise affine paragraph); x' is the activation already
// rotated by the block Hadamard transform (the caller runs rht_apply's
// kernel into the workspace first).
//
// Tiling.  A workgroup of 256 threads owns a 128 x 128 tile of y (128 batch
// rows x 128 output columns) and walks K in steps of 64 (half a group, so a
// step never straddles two scales).  Per step every thread
//   - loads 32 activations of one batch row and the 32-code slice of one
//     weight row (plus that row's scale and zero), one step ahead, into
//     registers;
//   - writes them to LDS: the weight slice dequantised to fp16, the
//     activations permuted into the same k order (below);
// and each wave multiplies a 64 x 64 sub-tile: 2 x 2 MFMA blocks, 4 k-steps
// of 16.
//
// Dequantisation.  A code pair is unpacked to two fp16 values 1024 + q (the
// GEMV's magic-number unpack, one v_and_or_b32), then q = h - 1024 (or
// h / 16 - 64 for int4 nibbles read in place from bits 4..7), q - z (exact
// in fp16: |q - z| < 256 and z's ulp keeps the difference within 11
// significant bits), and (q - z) * s rounded once to fp16.  The pairs come
// out in the unpacker's order -- int4: codes (0,4) (1,5) (2,6) (3,7) of each
// word; int8: (0,2) (1,3) of each word; int3 and int6: natural -- so the
// activations are stored in LDS in the same k order; a dot product does not
// depend on the order of its terms.
//
// MFMA operand layout (checked on the device): lane l holds A[l % 32][8 (l /
// 32) .. +8] and B[8 (l / 32) .. +8][l % 32]; accumulator register v of lane
// l is C[8 (v / 4) + 4 (l / 32) + v % 4][l % 32].
#include "wq_internal.h"

namespace wq {
using namespace dev;

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLdk = kBK + 8;              // halfs per LDS row (144 bytes: spreads the 32 rows over the banks)
constexpr int kGemmThreads = 256;
constexpr uint32_t kMagic = 0x64006400u;   // two fp16 1024.0

template <int BITS>
__device__ __forceinline__ void load_codes(rsrc_t rs, uint32_t off, uint32_t (&w)[BITS]) {
  if constexpr (BITS == 4) {
    const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (BITS == 8) {
    const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16, 0, 0));
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  } else if constexpr (BITS == 6) {
    const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    const u32x2 b = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off + 16, 0, 0));
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y;
  } else {
    const u32x3 v = __builtin_bit_cast(u32x3, __builtin_amdgcn_raw_buffer_load_b96(rs, off, 0, 0));
    w[0] = v.x; w[1] = v.y; w[2] = v.z;
  }
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

// Code pair P of a 32-code slice as two fp16 values 1024 + q (int4 pairs
// with P % 4 odd: 1024 + 16 q).
template <int BITS, int P>
__device__ __forceinline__ uint32_t code_pair(const uint32_t (&w)[BITS]) {
  if constexpr (BITS == 4) {
    constexpr int wi = P / 4, r = P % 4;
    const uint32_t v = (r < 2) ? w[wi] : (w[wi] >> 8);
    return (r & 1) ? ((v & 0x00F000F0u) | kMagic) : ((v & 0x000F000Fu) | kMagic);
  } else if constexpr (BITS == 8) {
    constexpr int wi = P / 2, r = P % 2;
    return __builtin_amdgcn_perm(0x64646464u, w[wi], r ? 0x04030401u : 0x04020400u);
  } else if constexpr (BITS == 3) {
    const uint32_t t = bits_at<6 * P, 6>(w);
    return ((t | (t << 13)) & 0x00070007u) | kMagic;
  } else {
    constexpr int run = P / 8, q = P % 8;
    const uint32_t t = (run == 0) ? bits_at<12 * q, 12>(w) : bits_at<96 + 12 * q, 12>(w);
    return ((t | (t << 10)) & 0x003F003Fu) | kMagic;
  }
}

__device__ __forceinline__ half2v as_h2(uint32_t v) { return __builtin_bit_cast(half2v, v); }
__device__ __forceinline__ uint32_t as_u32(half2v v) { return __builtin_bit_cast(uint32_t, v); }

// Dequantise pair P: (q - z) * s, fp16.
template <int BITS, int P>
__device__ __forceinline__ uint32_t dequant_pair(const uint32_t (&w)[BITS], half2v z, half2v s) {
  const half2v h = as_h2(code_pair<BITS, P>(w));
  half2v q;
  if constexpr (BITS == 4 && (P % 2) == 1) {
    const half2v k16 = {(_Float16)0.0625f, (_Float16)0.0625f}, m64 = {(_Float16)-64.0f, (_Float16)-64.0f};
    q = __builtin_elementwise_fma(h, k16, m64);
  } else {
    const half2v m1024 = {(_Float16)-1024.0f, (_Float16)-1024.0f};
    q = h + m1024;
  }
  return as_u32((q - z) * s);
}

// Four u32 of natural-order activations (k, k+1), (k+2, k+3), ... permuted
// into the order the weight pairs of the same 8 codes come out in.
template <int BITS>
__device__ __forceinline__ u32x4 permute_acts(u32x4 a) {
  if constexpr (BITS == 4) {
    // halves 0..7 -> 0 4 1 5 2 6 3 7
    return u32x4{__builtin_amdgcn_perm(a.z, a.x, 0x05040100u), __builtin_amdgcn_perm(a.z, a.x, 0x07060302u),
                 __builtin_amdgcn_perm(a.w, a.y, 0x05040100u), __builtin_amdgcn_perm(a.w, a.y, 0x07060302u)};
  } else if constexpr (BITS == 8) {
    // halves 0..7 -> 0 2 1 3 4 6 5 7
    return u32x4{__builtin_amdgcn_perm(a.y, a.x, 0x05040100u), __builtin_amdgcn_perm(a.y, a.x, 0x07060302u),
                 __builtin_amdgcn_perm(a.w, a.z, 0x05040100u), __builtin_amdgcn_perm(a.w, a.z, 0x07060302u)};
  } else {
    return a;
  }
}

struct GemmArgs {
  const uint32_t *codes;
  const uint16_t *scales, *zeros;
  const uint16_t *x;   // rotated activations [m][ldx]
  void *y;
  int64_t ldx, ldy;
  int32_t m, n, k;
  int32_t mtiles, ntiles;
  int32_t out_f32;
};

// blockIdx -> (m tile, n tile).  Workgroups are dealt to the 8 XCDs round
// robin; the mapping puts runs of consecutive tiles (the m tiles of one n
// tile, which dequantise the same weights) on one XCD so they share its L2.
__device__ __forceinline__ void tile_of(const GemmArgs &a, int &mt, int &nt) {
  const int nb = a.mtiles * a.ntiles, b = blockIdx.x;
  const int xcd = b % 8, slot = b / 8, q = nb / 8, rem = nb % 8;
  const int logical = (xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q) + slot;
  nt = logical / a.mtiles;
  mt = logical - nt * a.mtiles;
}

template <int BITS>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kBM * kLdk];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kBN * kLdk];
  int mt, nt;
  tile_of(a, mt, nt);
  const int m0 = mt * kBM, n0 = nt * kBN;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int S = a.k / kSlice, G = a.k / kGroup, wpr = S * BITS;

  // per-thread load roles: row t / 2 of the tile, 32-wide k half t & 1
  const int lr = t >> 1, lh = t & 1;
  const rsrc_t rx = make_rsrc(a.x + (size_t)m0 * a.ldx, (uint32_t)((size_t)min(kBM, a.m - m0) * a.ldx * 2));
  const int nrows = min(kBN, a.n - n0);
  const rsrc_t rc = make_rsrc(a.codes + (size_t)n0 * wpr, (uint32_t)nrows * wpr * 4);
  const rsrc_t rs = make_rsrc(a.scales + (size_t)n0 * G, (uint32_t)nrows * G * 2);
  const rsrc_t rz = make_rsrc(a.zeros + (size_t)n0 * G, (uint32_t)nrows * G * 2);

  u32x4 xa[4];
  uint32_t cw[BITS];
  uint32_t sraw, zraw;
  auto load = [&](int kt) {
    const int k0 = kt * kBK + 32 * lh;
    const uint32_t xo = (uint32_t)(((size_t)lr * a.ldx + k0) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      xa[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xo + 16 * i, 0, 0));
    load_codes<BITS>(rc, (uint32_t)((lr * wpr + (k0 / kSlice) * BITS) * 4), cw);
    const uint32_t so = (uint32_t)((lr * G + k0 / kGroup) * 2);
    sraw = __builtin_amdgcn_raw_buffer_load_b16(rs, so, 0, 0);
    zraw = __builtin_amdgcn_raw_buffer_load_b16(rz, so, 0, 0);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int wm = (wave & 1) * 64, wn = (wave >> 1) * 64;
  const int KT = a.k / kBK;
  load(0);
  for (int kt = 0; kt < KT; ++kt) {
    // registers -> LDS: activations permuted, weights dequantised
    {
      u32x4 *dst = reinterpret_cast<u32x4 *>(&As[lr * kLdk + 32 * lh]);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = permute_acts<BITS>(xa[i]);
      const half2v s2 = as_h2((sraw & 0xFFFFu) * 0x10001u), z2 = as_h2((zraw & 0xFFFFu) * 0x10001u);
      uint32_t p[16];
      p[0] = dequant_pair<BITS, 0>(cw, z2, s2);   p[1] = dequant_pair<BITS, 1>(cw, z2, s2);
      p[2] = dequant_pair<BITS, 2>(cw, z2, s2);   p[3] = dequant_pair<BITS, 3>(cw, z2, s2);
      p[4] = dequant_pair<BITS, 4>(cw, z2, s2);   p[5] = dequant_pair<BITS, 5>(cw, z2, s2);
      p[6] = dequant_pair<BITS, 6>(cw, z2, s2);   p[7] = dequant_pair<BITS, 7>(cw, z2, s2);
      p[8] = dequant_pair<BITS, 8>(cw, z2, s2);   p[9] = dequant_pair<BITS, 9>(cw, z2, s2);
      p[10] = dequant_pair<BITS, 10>(cw, z2, s2); p[11] = dequant_pair<BITS, 11>(cw, z2, s2);
      p[12] = dequant_pair<BITS, 12>(cw, z2, s2); p[13] = dequant_pair<BITS, 13>(cw, z2, s2);
      p[14] = dequant_pair<BITS, 14>(cw, z2, s2); p[15] = dequant_pair<BITS, 15>(cw, z2, s2);
      u32x4 *bd = reinterpret_cast<u32x4 *>(&Bs[lr * kLdk + 32 * lh]);
#pragma unroll
      for (int i = 0; i < 4; ++i) bd[i] = u32x4{p[4 * i], p[4 * i + 1], p[4 * i + 2], p[4 * i + 3]};
    }
    __syncthreads();
    if (kt + 1 < KT) load(kt + 1);   // next step's loads overlap this step's products
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      half8 av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        av[i] = *reinterpret_cast<const half8 *>(&As[(wm + 32 * i + (lane & 31)) * kLdk + 16 * kk + 8 * (lane >> 5)]);
        bv[i] = *reinterpret_cast<const half8 *>(&Bs[(wn + 32 * i + (lane & 31)) * kLdk + 16 * kk + 8 * (lane >> 5)]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#if defined(__HIP_DEVICE_COMPILE__)   // the 32x32x16 f16 MFMA exists only in the gfx950 pass
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
#endif
        }
    }
    __syncthreads();
  }

  // epilogue: accumulator register v of lane l is C[8 (v/4) + 4 (l/32) + v%4][l % 32]
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn + 32 * j + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < a.m && col < a.n) {
          const float r = acc[i][j][v];
          if (a.out_f32) {
            reinterpret_cast<float *>(a.y)[(size_t)row * a.ldy + col] = r;
          } else {
            const _Float16 h = (_Float16)r;
            reinterpret_cast<uint16_t *>(a.y)[(size_t)row * a.ldy + col] = __builtin_bit_cast(uint16_t, h);
          }
        }
      }
    }
}

}  // namespace

bool gemm_available(int bits) { return bits == 3 || bits == 4 || bits == 6 || bits == 8; }

size_t gemm_workspace(const wq_weight &w, int64_t m) {
  (void)w;
  (void)m;
  return 0;
}

hipError_t launch_gemm(const wq_weight &w, const uint16_t *xr, int64_t m, int64_t ldx, void *y, int out_f32,
                       int64_t ldy, void *workspace, hipStream_t s) {
  (void)workspace;
  if (!gemm_available(w.bits) || w.k % kBK) return hipErrorInvalidValue;
  if ((uint64_t)m * (uint64_t)ldx * 2 > 0xFFFFFFFFull || (uint64_t)w.n * (uint64_t)w.k > 0xFFFFFFFFull)
    return hipErrorInvalidValue;   // 32-bit buffer offsets
  GemmArgs a;
  a.codes = w.codes;
  a.scales = w.scales;
  a.zeros = w.zeros;
  a.x = xr;
  a.y = y;
  a.ldx = ldx;
  a.ldy = ldy;
  a.m = (int32_t)m;
  a.n = (int32_t)w.n;
  a.k = (int32_t)w.k;
  a.mtiles = (int32_t)((m + kBM - 1) / kBM);
  a.ntiles = (int32_t)((w.n + kBN - 1) / kBN);
  a.out_f32 = out_f32;
  const unsigned grid = (unsigned)(a.mtiles * a.ntiles);
  switch (w.bits) {
    case 3: hipLaunchKernelGGL(gemm_kernel<3>, dim3(grid), dim3(kGemmThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL(gemm_kernel<4>, dim3(grid), dim3(kGemmThreads), 0, s, a); break;
    case 6: hipLaunchKernelGGL(gemm_kernel<6>, dim3(grid), dim3(kGemmThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL(gemm_kernel<8>, dim3(grid), dim3(kGemmThreads), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace wq

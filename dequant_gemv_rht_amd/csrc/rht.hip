// Standalone block random Hadamard rotation of fp16 activations (gfx950).
//
// y[m][128j : 128j+128] = H D_j x[m][128j : 128j+128] / sqrt(128)
// (model card "24B0978 - Week 01 - Track 2, 20% target", paragraph on the
// random Hadamard transform: a fast Walsh-Hadamard transform of log2(block)
// add/sub stages applied to the activations at run time).
//
// One 128-block per 16-lane DPP row: lane jj holds elements 8jj..8jj+7,
// butterflies of stride 1, 2, 4 run inside the lane and strides 8..64 across
// lanes by DPP.  fp32 inside, one rounding to fp16 at the end.
#include "wq_internal.h"

#include <climits>
#include <cstring>

namespace wq {
using namespace dev;

namespace {

// Block b of row `row`, lane jj's eight elements; with pair_order stored in
// the order 0, 4, 1, 5, 2, 6, 3, 7.
__device__ __forceinline__ void rotate_block(const uint16_t *__restrict__ x, uint16_t *y,
                                             const uint32_t *__restrict__ signs, int64_t row, int64_t b,
                                             int jj, int64_t ldx, int64_t ldy, bool pair_order = false) {
  const int64_t kk = b * 128 + 8 * jj;
  const uint4 raw = *reinterpret_cast<const uint4 *>(x + row * ldx + kk);
  float v[8];
  v[0] = half_bits_to_float(raw.x & 0xFFFF); v[1] = half_bits_to_float(raw.x >> 16);
  v[2] = half_bits_to_float(raw.y & 0xFFFF); v[3] = half_bits_to_float(raw.y >> 16);
  v[4] = half_bits_to_float(raw.z & 0xFFFF); v[5] = half_bits_to_float(raw.z >> 16);
  v[6] = half_bits_to_float(raw.w & 0xFFFF); v[7] = half_bits_to_float(raw.w >> 16);
  const uint32_t sb = signs[kk >> 5] >> (kk & 31);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = ((sb >> e) & 1u) ? -v[e] : v[e];
  fwht128_row16_signed(v, jj);
  const float sc = fwht_lane_sign(jj) * 0.08838834764831845f;
  uint4 out;
  if (pair_order) {
    out.x = pack_half2(v[0] * sc, v[4] * sc);
    out.y = pack_half2(v[1] * sc, v[5] * sc);
    out.z = pack_half2(v[2] * sc, v[6] * sc);
    out.w = pack_half2(v[3] * sc, v[7] * sc);
  } else {
    out.x = pack_half2(v[0] * sc, v[1] * sc);
    out.y = pack_half2(v[2] * sc, v[3] * sc);
    out.z = pack_half2(v[4] * sc, v[5] * sc);
    out.w = pack_half2(v[6] * sc, v[7] * sc);
  }
  *reinterpret_cast<uint4 *>(y + row * ldy + kk) = out;
}

__global__ __launch_bounds__(256) void rht_kernel(const uint16_t *__restrict__ x, uint16_t *y,
                                                  const uint32_t *__restrict__ signs, int64_t m,
                                                  int64_t k, int64_t ldx, int64_t ldy) {
  const int64_t nb = k / 128;
  const int64_t item = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (item >= m * nb) return;   // whole 16-lane rows leave together
  rotate_block(x, y, signs, item / nb, item % nb, threadIdx.x & 15, ldx, ldy);
}

// Several matrices in one launch: workgroups (16 blocks each) dealt to the
// matrices by a packed table of first workgroups.
struct RhtMat {
  const uint16_t *x;
  uint16_t *y;
  const uint32_t *signs;
  int64_t m, k, ldx, ldy;
  int32_t wg_begin;
};

struct RhtBatch {
  int32_t first_wg[kMaxBatch];   // mat[i].wg_begin, packed; INT32_MAX past count
  RhtMat mat[kMaxBatch];
  int32_t pair_order;
};

__global__ __launch_bounds__(256) void rht_batch_kernel(RhtBatch a) {
  const int w = blockIdx.x;
  int l = 0;
#pragma unroll
  for (int i = 1; i < kMaxBatch; ++i)
    if (w >= a.first_wg[i]) l = i;
  const RhtMat M = a.mat[l];
  const int64_t nb = M.k / 128;
  const int64_t item = (int64_t)(w - M.wg_begin) * 16 + (threadIdx.x >> 4);
  if (item >= M.m * nb) return;
  rotate_block(M.x, M.y, M.signs, item / nb, item % nb, threadIdx.x & 15, M.ldx, M.ldy, a.pair_order != 0);
}

}  // namespace

hipError_t launch_rht(const uint16_t *x, uint16_t *y, const uint32_t *signs, int64_t m, int64_t k,
                      int64_t ldx, int64_t ldy, hipStream_t s) {
  const int64_t items = m * (k / 128);
  const int64_t blocks = (items + 15) / 16;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(rht_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, y, signs, m, k, ldx, ldy);
  return hipGetLastError();
}

hipError_t launch_rht_batch(int count, const uint16_t *const *x, uint16_t *const *y, const uint32_t *const *signs,
                            int64_t m, const int64_t *k, const int64_t *ldx, const int64_t *ldy, bool pair_order,
                            hipStream_t s) {
  if (count <= 0 || count > kMaxBatch) return hipErrorInvalidValue;
  RhtBatch a;
  memset(&a, 0, sizeof a);
  a.pair_order = pair_order ? 1 : 0;
  for (int i = 0; i < kMaxBatch; ++i) a.first_wg[i] = INT32_MAX;
  int64_t wgs = 0;
  for (int i = 0; i < count; ++i) {
    RhtMat &M = a.mat[i];
    M.x = x[i];
    M.y = y[i];
    M.signs = signs[i];
    M.m = m;
    M.k = k[i];
    M.ldx = ldx[i];
    M.ldy = ldy[i];
    M.wg_begin = (int32_t)wgs;
    a.first_wg[i] = (int32_t)wgs;
    wgs += (m * (k[i] / 128) + 15) / 16;
  }
  if (wgs == 0) return hipSuccess;
  if (wgs > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rht_batch_kernel, dim3((unsigned)wgs), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace wq

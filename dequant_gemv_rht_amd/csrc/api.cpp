// C ABI of libwq: argument checks, workspace layout and kernel dispatch.
// Every check runs on the host before any HIP call, so a rejected call
// enqueues nothing.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>

#include "wq_internal.h"
#include "../../include/wq_measure.h"

namespace {

thread_local char g_err[512] = "";

wq_status fail(wq_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

void clear_err() { g_err[0] = 0; }

}  // namespace

// The thread's error message, for entry points in other translation units.
wq_status wq::set_error(wq_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

void wq::clear_error() { clear_err(); }

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool uniform_bits(int b) { return b == 3 || b == 4 || b == 6 || b == 8; }

int mtile(int64_t m) {
  if (m <= 1) return 1;
  if (m <= 2) return 2;
  if (m <= 4) return 4;
  if (m <= 8) return 8;
  return 16;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// validate a weight descriptor; `need_rht` true when the call rotates
wq_status check_weight(const wq_weight *w, const char *who) {
  if (!w) return fail(WQ_E_ARG, "%s: weight descriptor is NULL", who);
  if (!(uniform_bits(w->bits) || w->bits == 0))
    return fail(WQ_E_UNSUPPORTED, "%s: bits=%d (supported: 3, 4, 6, 8, 0 = mixed 6/8)", who, w->bits);
  if (w->group != WQ_GROUP) return fail(WQ_E_UNSUPPORTED, "%s: group=%d (only 128)", who, w->group);
  if (w->n <= 0 || w->k <= 0) return fail(WQ_E_ARG, "%s: n=%lld k=%lld must be positive", who,
                                          (long long)w->n, (long long)w->k);
  if (w->k % WQ_GROUP) return fail(WQ_E_ARG, "%s: k=%lld is not a multiple of 128", who, (long long)w->k);
  if (w->n > (int64_t)INT32_MAX || w->k > (int64_t)INT32_MAX)
    return fail(WQ_E_UNSUPPORTED, "%s: n or k above 2^31-1", who);
  if (!w->codes || !w->scales || !w->zeros)
    return fail(WQ_E_ARG, "%s: codes, scales and zeros must be non-NULL", who);
  if (!aligned16(w->codes) || !aligned16(w->scales) || !aligned16(w->zeros))
    return fail(WQ_E_ALIGN, "%s: codes/scales/zeros must be 16-byte aligned", who);
  if (w->bits == 0) {
    if (w->n % WQ_MIXED_ROWS) return fail(WQ_E_ARG, "%s: mixed width needs n %% 64 == 0 (n=%lld)", who,
                                          (long long)w->n);
    if (!w->block_bits || !w->block_off)
      return fail(WQ_E_ARG, "%s: mixed width needs block_bits and block_off", who);
    if (w->block_bits_host)
      for (int64_t b = 0; b < w->n / WQ_MIXED_ROWS; ++b)
        if (w->block_bits_host[b] != 6 && w->block_bits_host[b] != 8)
          return fail(WQ_E_ARG, "%s: block_bits_host[%lld]=%d (6 or 8)", who, (long long)b,
                      (int)w->block_bits_host[b]);
  }
  if (w->rht_signs) {
    if (w->rht_block != WQ_RHT_BLOCK)
      return fail(WQ_E_UNSUPPORTED, "%s: rht_block=%d (only 128)", who, w->rht_block);
    if (!aligned16(w->rht_signs)) return fail(WQ_E_ALIGN, "%s: rht_signs must be 16-byte aligned", who);
  }
  return WQ_OK;
}

wq_status hip_status(hipError_t e, const char *who) {
  if (e == hipSuccess) return WQ_OK;
  return fail(WQ_E_HIP, "%s: %s", who, hipGetErrorString(e));
}

// Workgroup layout of one linear in the GEMV path: whole rows per
// workgroup, K walked inside; the rotated activations of a K chunk sit in LDS.
struct GemvPlan {
  int mode, rows, row_blocks, kc, lds;
};

GemvPlan gemv_plan(const wq_weight &w, int64_t m) {
  GemvPlan p;
  const int mt = mtile(m);
  wq::gemv_shape(w.bits, mt, w.k, p.mode, p.rows);
  p.row_blocks = (int)((w.n + p.rows - 1) / p.rows);
  p.kc = wq::gemv_chunk(mt, w.k);
  p.lds = wq::gemv_lds_bytes(mt, p.kc, p.rows, w.k);
  return p;
}

int device_cus() {
  thread_local int cached_dev = -1, cached_cus = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev != cached_dev) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached_dev = dev;
    cached_cus = n;
  }
  return cached_cus;
}

constexpr int kMaxLds = 160 * 1024;

// Persistent stream kernel plan: workgroups (one per CU) split among the
// linears so that their estimated times match; each gets an even number of
// rows.  A workgroup's time is its weight bytes plus its activation
// preparation, which it does before any weight can be used: rounds of
// ceil(items / 16) over the linear's 128-blocks (times the batch tile), as
// for 16-lane rows of 4 waves per SIMD, about 0.25 us per round with the
// rotation (~185 vector instructions per block), which is what a CU streams
// of weights in that time (~32 KB/us): 8 KB per round; without the rotation
// ~70 instructions, 3 KB.  (The batch-1 rings of 3- and 4-bit codes run 2
// waves per SIMD; the estimate is kept, as the balance it gives was measured
// best for them too.)
bool plan_stream(int count, const wq_weight *w, int64_t m, bool rotate, int *wg, int *rows_per_wg, int *lds,
                 bool *ring) {
  const int mt = mtile(m);
  if (w[0].bits == 0 || mt > 16) return false;
  const int ncu = device_cus();
  if (count > ncu) return false;
  const double round_bytes = rotate ? 8192.0 : 3072.0;
  const int gran = mt >= 2 ? 4 : 2;   // rows per task: quads at batch tiles 2 to 16, pairs at 1
  double bytes[WQ_MAX_BATCH], prep[WQ_MAX_BATCH];
  int64_t maxwg[WQ_MAX_BATCH];
  for (int i = 0; i < count; ++i) {
    bytes[i] = (double)w[i].n * (double)w[i].k * (w[i].bits / 8.0 + 4.0 / 128.0);
    const int64_t items = mt * (w[i].k / wq::kGroup);
    // batch 1 rotates in the workgroup; batch tiles 2 to 16 copy the
    // arranged activations (80 bytes per 32 elements) from L2
    prep[i] = mt == 1 ? round_bytes * (double)((items + 15) / 16) : 0.625 * (double)(mt * w[i].k);
    // at batch 1 a workgroup takes at least 8 rows: a small linear then
    // launches fewer workgroups, which start sooner (1024 -> 512: 3.52 ->
    // 3.35 us), and a large one is unaffected
    const int minrows = mt == 1 ? 8 : gran;
    maxwg[i] = (w[i].n + minrows - 1) / minrows;
    wg[i] = 1;
  }
  // hand out the CUs one at a time to the linear with the longest estimate
  for (int sum = count; sum < ncu; ++sum) {
    int b = -1;
    double worst = 0;
    for (int i = 0; i < count; ++i) {
      const double est = bytes[i] / wg[i] + prep[i];
      if (wg[i] < maxwg[i] && est > worst) {
        worst = est;
        b = i;
      }
    }
    if (b < 0) break;
    ++wg[b];
  }
  *lds = 0;
  int ring_lds = 0;
  for (int i = 0; i < count; ++i) {
    int64_t r = (w[i].n + wg[i] - 1) / wg[i];
    r = (r + gran - 1) / gran * gran;
    rows_per_wg[i] = (int)r;
    wg[i] = (int)((w[i].n + r - 1) / r);
    const int need = wq::gemv_stream_lds_bytes(w[i].bits, mt, w[i].k, (int)r, false);
    if (need > *lds) *lds = need;
    const int rneed = wq::gemv_stream_lds_bytes(w[i].bits, mt, w[i].k, (int)r, true);
    if (rneed > ring_lds) ring_lds = rneed;
  }
  // batch 1: stage the weights through the LDS ring whenever it fits
  *ring = mt == 1 && ring_lds <= kMaxLds;
  if (*ring) *lds = ring_lds;
  return *lds <= kMaxLds;
}

// The first linear j <= i of a call whose input is linear i's: the same
// activations (pointer and row stride), the same K and the same rotation
// (sign vector pointer, or none).  Linears that share an input, such as the
// query, key and value projections quantised with one sign vector, then
// share its rotation ("24B0978 - Week 01 - Track 2", paragraph on the random
// Hadamard transform: one rotation of the activations per input).
int same_input(const wq_weight *w, const uint16_t *const *x, const int64_t *ldx, int i) {
  for (int j = 0; j < i; ++j)
    if (x[j] == x[i] && ldx[j] == ldx[i] && w[j].k == w[i].k && w[j].rht_signs == w[i].rht_signs) return j;
  return i;
}

// Bytes of the arranged activations of m rows of a linear with k columns
// (the batch-tile kernels' LDS slice layout: 80 bytes per 32 elements).
size_t xprep_bytes(int64_t k, int64_t m) { return align256((size_t)m * (size_t)(k / wq::kSlice) * 80); }

bool uses_xprep(const wq_weight &w, int64_t m) { return m >= 2 && w.bits != 0; }

wq_status launch_tile(int count, const wq_weight *w, const uint16_t *const *x, const int64_t *ldx, int64_t m,
                      void *const *y, const wq_dtype *ydt, const int64_t *ldy, bool rotate,
                      const uint32_t *const *xq, hipStream_t s);

// The linears in launch order: longest rows first, so that the longest
// workgroups start first.
void order_by_k(int count, const wq_weight *w, int *order, wq_weight *ws) {
  for (int i = 0; i < count; ++i) order[i] = i;
  for (int i = 1; i < count; ++i)
    for (int j = i; j > 0 && w[order[j]].k > w[order[j - 1]].k; --j) {
      int t = order[j];
      order[j] = order[j - 1];
      order[j - 1] = t;
    }
  for (int o = 0; o < count; ++o) ws[o] = w[order[o]];
}

// One GEMV over `count` linears with batch rows m (< 64; at most 16 for the
// mixed layout).  Above one row (uniform width) the activations are arranged
// once into the workspace, then each tile of batch rows is one pass of the
// row-quad kernel over the weights: 16 rows (from 13 rows left on) or 8
// (from 5 on) where that many rows' arranged activations (80 bytes per 32
// elements and row, in up to 4 chunks of K), the row parts and the scales
// fit in one workgroup's LDS for every linear of the call, else 4.  Below
// 13 rows a tile of 8 and one of up to 4 compute fewer rows than one of 16.
wq_status run_gemv(int count, const wq_weight *w, const uint16_t *const *x, const int64_t *ldx,
                   int64_t m, void *const *y, const wq_dtype *ydt, const int64_t *ldy,
                   bool rotate, void *workspace, hipStream_t s) {
  if (!uses_xprep(w[0], m)) return launch_tile(count, w, x, ldx, m, y, ydt, ldy, rotate, nullptr, s);
  bool fits16 = false, fits8 = false;
  if (m > 4) {
    int order[WQ_MAX_BATCH], wg[WQ_MAX_BATCH], rpw[WQ_MAX_BATCH], lds = 0;
    wq_weight ws[WQ_MAX_BATCH];
    bool ring = false;
    order_by_k(count, w, order, ws);
    fits16 = m > 12 && plan_stream(count, ws, 16, rotate, wg, rpw, &lds, &ring);
    fits8 = plan_stream(count, ws, 8, rotate, wg, rpw, &lds, &ring);
  }
  uint32_t *xq[WQ_MAX_BATCH];
  const uint16_t *px[WQ_MAX_BATCH];
  int64_t pld[WQ_MAX_BATCH], kk[WQ_MAX_BATCH];
  const uint32_t *sg[WQ_MAX_BATCH];
  uint32_t *pq[WQ_MAX_BATCH];
  int np = 0;
  size_t off = 0;
  for (int i = 0; i < count; ++i) {
    xq[i] = reinterpret_cast<uint32_t *>(static_cast<char *>(workspace) + off);
    off += xprep_bytes(w[i].k, m);
    const int j = same_input(w, x, ldx, i);
    if (j < i) {
      xq[i] = xq[j];
      continue;
    }
    px[np] = x[i];
    pld[np] = ldx[i];
    sg[np] = rotate ? w[i].rht_signs : nullptr;
    kk[np] = w[i].k;
    pq[np] = xq[i];
    ++np;
  }
  wq_status st = hip_status(wq::launch_xprep(w[0].bits, np, px, pld, sg, kk, m, pq, s), "wq_linear");
  if (st != WQ_OK) return st;
  const uint32_t *xt[WQ_MAX_BATCH];
  const uint16_t *xc[WQ_MAX_BATCH];
  void *yc[WQ_MAX_BATCH];
  for (int64_t m0 = 0, tile = 0; m0 < m; m0 += tile) {
    const int64_t rem = m - m0;
    tile = fits16 && rem > 12 ? 16 : fits8 && rem > 4 ? 8 : 4;
    for (int i = 0; i < count; ++i) {
      xt[i] = xq[i] + (size_t)m0 * (size_t)(w[i].k / wq::kSlice) * 20;
      xc[i] = x[i] + m0 * ldx[i];
      yc[i] = static_cast<char *>(y[i]) + (size_t)m0 * (size_t)ldy[i] * (ydt[i] == WQ_F32 ? 4 : 2);
    }
    st = launch_tile(count, w, xc, ldx, rem < tile ? rem : tile, yc, ydt, ldy, rotate, xt, s);
    if (st != WQ_OK) return st;
  }
  return WQ_OK;
}

// Every workgroup of a mixed 6/8 layout at batch 1, placed from the host
// copy of the widths as the kernel's own search would: runs of same-width
// blocks get the workgroups w with F(off[bs]) <= w < F(off[be]),
// F(o) = floor(G o / total words), and split their row pairs evenly.
// rec[w] = first code word | (first row | 8-bit << 31) << 32; rec[G] = n
// rows.  False where a workgroup would get more than the 64 rows the
// launch sizes the LDS for (not with one workgroup or more per block).
bool mixed_table(const wq_weight &w, int G, uint64_t *rec) {
  const int64_t nblk = w.n / WQ_MIXED_ROWS;
  const uint8_t *bits = w.block_bits_host;
  uint64_t tot = 0;
  for (int64_t b = 0; b < nblk; ++b) tot += 2 * (uint64_t)w.k * bits[b];
  uint64_t off = 0;
  for (int64_t bs = 0, be; bs < nblk; bs = be) {
    uint64_t words = 0;
    for (be = bs; be < nblk && bits[be] == bits[bs]; ++be) words += 2 * (uint64_t)w.k * bits[be];
    const int64_t lo = (int64_t)((unsigned __int128)off * (unsigned)G / tot);
    const int64_t hi = (int64_t)((unsigned __int128)(off + words) * (unsigned)G / tot);
    const int64_t pairs = (int64_t)(WQ_MIXED_ROWS / 2) * (be - bs), wr = hi - lo;
    const uint64_t row_words = (uint64_t)w.k * bits[bs] / 32;
    if (wr < 1) return false;
    for (int64_t sub = 0; sub < wr; ++sub) {
      const int64_t q0 = pairs * sub / wr, q1 = pairs * (sub + 1) / wr;
      if (2 * (q1 - q0) > WQ_MIXED_ROWS) return false;
      const uint64_t row = (uint64_t)(WQ_MIXED_ROWS * bs + 2 * q0), word = off + 2 * (uint64_t)q0 * row_words;
      rec[lo + sub] = word | ((row | (bits[bs] == 8 ? (uint64_t)1 << 31 : 0)) << 32);
    }
    off += words;
  }
  rec[G] = (uint64_t)w.n << 32;
  return true;
}

// One launch over `count` linears for a batch tile of m <= 16 rows.  xq:
// the tile's arranged activations per linear, or NULL where the kernel
// rotates for itself.
wq_status launch_tile(int count, const wq_weight *w, const uint16_t *const *x, const int64_t *ldx, int64_t m,
                      void *const *y, const wq_dtype *ydt, const int64_t *ldy, bool rotate,
                      const uint32_t *const *xq, hipStream_t s) {
  wq::GemvArgs a;
  memset(&a, 0, sizeof a);
  for (int i = 0; i < wq::kMaxBatch; ++i) a.first_tile[i] = INT32_MAX;
  a.count = count;
  a.m = (int32_t)m;
  int order[WQ_MAX_BATCH];
  wq_weight ws[WQ_MAX_BATCH];
  order_by_k(count, w, order, ws);
  int wg[WQ_MAX_BATCH], rpw[WQ_MAX_BATCH], slds = 0;
  bool ring = false;
  bool stream = plan_stream(count, ws, m, rotate, wg, rpw, &slds, &ring);
  bool table = false;   // mixed at batch 1, workgroups placed here from the host widths
  if (!stream && count == 1 && w[0].bits == 0 && m == 1) {
    // mixed 6/8 at batch 1: the rings, each workgroup on rows of one width
    // (within a run of same-width blocks).  One workgroup per CU spread over
    // the runs by their code words, where every block then gets one (an
    // 8-bit block has 4/3 the words of a 6-bit one: at most 3/4 as many
    // blocks as CUs), and at least 2 rows each, at most 64; else one
    // workgroup per block.
    const int64_t nblk = w[0].n / WQ_MIXED_ROWS, ncu = device_cus();
    const bool spread = 4 * nblk <= 3 * ncu;
    const int64_t wgs = spread ? (ncu < 32 * nblk ? ncu : 32 * nblk) : nblk;
    const int need = wq::gemv_stream_lds_bytes(0, 1, w[0].k, WQ_MIXED_ROWS, true);
    if (need <= kMaxLds && wgs <= INT32_MAX) {
      stream = ring = true;
      slds = need;
      rpw[0] = WQ_MIXED_ROWS;
      wg[0] = (int)wgs;
      a.mixed_wpb = spread ? 0 : 1;
      table = spread && w[0].block_bits_host && wgs <= wq::kMixedTableWgs;
    }
  }
  int64_t tiles = 0;
  int lds = 0;
  for (int o = 0; o < count; ++o) {
    const int i = order[o];
    GemvPlan p = gemv_plan(w[i], m);
    wq::LinDesc &L = a.lin[o];
    L.codes = w[i].codes;
    L.scales = w[i].scales;
    L.zeros = w[i].zeros;
    L.block_bits = w[i].block_bits;
    L.block_off = w[i].block_off;
    L.signs = rotate ? w[i].rht_signs : nullptr;
    if (xq && stream && m >= 2)
      L.xq = xq[i];   // the row-quad kernel reads the arranged activations
    else
      L.x = x[i];
    L.y = y[i];
    L.ldx = ldx[i];
    L.ldy = ldy[i];
    L.n = (int32_t)w[i].n;
    L.k = (int32_t)w[i].k;
    L.kc = p.kc;
    L.mode = p.mode;
    L.row_blocks = p.row_blocks;
    L.out_f32 = ydt[i] == WQ_F32;
    {
      const int64_t ks = (w[i].k + wq::kSeg - 1) / wq::kSeg;
      L.ks_inv = (int32_t)((65536 + ks - 1) / ks);
    }
    L.tile_begin = (int32_t)tiles;
    a.first_tile[o] = (int32_t)tiles;
    if (stream) {
      L.rows_per_wg = rpw[o];
      tiles += wg[o];
    } else {
      tiles += p.row_blocks;
      if (p.lds > lds) lds = p.lds;
    }
  }
  if (tiles > INT32_MAX) return fail(WQ_E_UNSUPPORTED, "wq_linear: too many workgroups");
  a.tiles = (int32_t)tiles;
  if (table) {
    wq::MixedArgs ma;
    memset(&ma, 0, sizeof ma);
    ma.lin = a.lin[0];
    ma.tiles = a.tiles;
    ma.lds_bytes = slds;
    if (mixed_table(w[0], a.tiles, ma.wg))
      return hip_status(wq::launch_gemv_mixed_table(ma, s), "wq_linear");
  }
  if (stream) {
    a.lds_bytes = slds;
    a.ring = ring ? 1 : 0;
    return hip_status(wq::launch_gemv_stream(w[0].bits, mtile(m), a, s), "wq_linear");
  }
  a.lds_bytes = lds;
  return hip_status(wq::launch_gemv(w[0].bits, mtile(m), a, s), "wq_linear");
}

wq_status check_io(const wq_weight &w, const uint16_t *x, int64_t m, int64_t ldx, const void *y,
                   wq_dtype ydt, int64_t ldy, const char *who) {
  if (m <= 0) return fail(WQ_E_ARG, "%s: m=%lld must be positive", who, (long long)m);
  if (!x || !y) return fail(WQ_E_ARG, "%s: x and y must be non-NULL", who);
  if (!aligned16(x) || !aligned16(y)) return fail(WQ_E_ALIGN, "%s: x and y must be 16-byte aligned", who);
  if (ldx < w.k) return fail(WQ_E_ARG, "%s: ldx=%lld < k=%lld", who, (long long)ldx, (long long)w.k);
  if (ldx % 8) return fail(WQ_E_ALIGN, "%s: ldx must be a multiple of 8 (16-byte rows)", who);
  if (ldy < w.n) return fail(WQ_E_ARG, "%s: ldy=%lld < n=%lld", who, (long long)ldy, (long long)w.n);
  if (ydt != WQ_F16 && ydt != WQ_F32) return fail(WQ_E_ARG, "%s: y_dtype must be WQ_F16 or WQ_F32", who);
  // every kernel addresses a linear's activations, codes, scales and zeros
  // with 32-bit buffer offsets: refuse here, before anything is launched,
  // what they could not reach
  if ((uint64_t)m * (uint64_t)ldx * 2 >= ((uint64_t)1 << 31))
    return fail(WQ_E_UNSUPPORTED, "%s: m * ldx * 2 = %llu bytes of activations (at most 2^31 - 1)", who,
                (unsigned long long)((uint64_t)m * (uint64_t)ldx * 2));
  if (w.k >= ((int64_t)1 << 27)) return fail(WQ_E_UNSUPPORTED, "%s: k=%lld (below 2^27)", who, (long long)w.k);
  if ((uint64_t)w.n * (uint64_t)w.k * (uint64_t)(w.bits ? w.bits : 8) / 8 >= ((uint64_t)1 << 32))
    return fail(WQ_E_UNSUPPORTED, "%s: n x k codes above 4 GiB", who);
  return WQ_OK;
}

// Matrix-core path: the rotated activations (fp16 [m][ldr]) live at the
// start of the workspace, followed by what the GEMM itself needs.
int64_t rotated_ld(const wq_weight &w) { return (w.k + 7) / 8 * 8; }

size_t rotated_bytes(const wq_weight &w, int64_t m) {
  return w.rht_signs ? align256((size_t)m * (size_t)rotated_ld(w) * sizeof(uint16_t)) : 0;
}

// Batch sizes above 16 run on the matrix cores (uniform code widths): from
// 17 rows on the product is a dense contraction that the GEMV, bound by its
// vector work per weight and batch row, runs slower (the int4 decoder block:
// 72 against 38 us at 17 rows, 226 against 47 us at 63).  The mixed-width
// layout stays on the GEMV, in chunks of 16 batch rows.
constexpr int64_t kGemmMinRows = 17;
bool use_gemm(const wq_weight &w, int64_t m) { return m >= kGemmMinRows && wq::gemm_available(w.bits); }

// Workspace of a matrix-core launch over `count` linears: each linear's
// rotated activations (when rotating), then each split linear's fp32
// partial sums, every part 256-byte aligned.
struct GemmLayout {
  size_t rot[WQ_MAX_BATCH], part[WQ_MAX_BATCH], total;
  int ksplit[WQ_MAX_BATCH];
};

GemmLayout gemm_layout(int count, const wq_weight *w, int64_t m, bool rotate) {
  GemmLayout g;
  wq::gemm_plan(count, w, m, g.ksplit);
  size_t off = 0;
  for (int i = 0; i < count; ++i) {
    g.rot[i] = off;
    if (rotate && w[i].rht_signs) off += rotated_bytes(w[i], m);
  }
  for (int i = 0; i < count; ++i) {
    g.part[i] = off;
    off += align256(wq::gemm_partial_bytes(w[i], m, g.ksplit[i]));
  }
  g.total = off;
  return g;
}

size_t gemm_path_workspace(const wq_weight &w, int64_t m) { return gemm_layout(1, &w, m, true).total; }

// Validated linears on the matrix cores: rotations into the workspace, then
// one GEMM launch for all of them (plus one launch adding K-split partials).
wq_status run_gemm(int count, const wq_weight *w, const uint16_t *const *x, const int64_t *ldx, int64_t m,
                   void *const *y, const wq_dtype *ydt, const int64_t *ldy, bool rotate, void *workspace,
                   hipStream_t s, const char *who) {
  const GemmLayout g = gemm_layout(count, w, m, rotate);
  char *ws = static_cast<char *>(workspace);
  const uint16_t *xr[WQ_MAX_BATCH];
  int64_t ldr[WQ_MAX_BATCH], ldo[WQ_MAX_BATCH];
  int f32[WQ_MAX_BATCH];
  float *part[WQ_MAX_BATCH];
  void *yo[WQ_MAX_BATCH];
  // the rotations of all linears in one launch
  int nr = 0;
  const uint16_t *rx[WQ_MAX_BATCH];
  uint16_t *ry[WQ_MAX_BATCH];
  const uint32_t *rs[WQ_MAX_BATCH];
  int64_t rk[WQ_MAX_BATCH], rlx[WQ_MAX_BATCH], rly[WQ_MAX_BATCH];
  for (int i = 0; i < count; ++i) {
    xr[i] = x[i];
    ldr[i] = ldx[i];
    const int j = rotate && w[i].rht_signs ? same_input(w, x, ldx, i) : i;
    if (j < i) {
      // an earlier linear of the call rotates this same input
      xr[i] = xr[j];
      ldr[i] = ldr[j];
    } else if (rotate && w[i].rht_signs) {
      uint16_t *xt = reinterpret_cast<uint16_t *>(ws + g.rot[i]);
      ldr[i] = rotated_ld(w[i]);
      rx[nr] = x[i];
      ry[nr] = xt;
      rs[nr] = w[i].rht_signs;
      rk[nr] = w[i].k;
      rlx[nr] = ldx[i];
      rly[nr] = ldr[i];
      ++nr;
      xr[i] = xt;
    }
    part[i] = g.ksplit[i] > 1 ? reinterpret_cast<float *>(ws + g.part[i]) : nullptr;
    f32[i] = ydt[i] == WQ_F32;
    ldo[i] = ldy[i];
    yo[i] = y[i];
  }
  // int4 up to 64 rows (the narrow tiles): when every linear's activations
  // pass through the rotation, it stores each 8-element group in the order
  // the kernel unpacks a code word in, cheaper than natural order (24 / 63
  // rows of the int4 block: 37.9 -> 37.3 / 46.8 -> 45.5 us).  The 128 x 256
  // tile keeps natural order: there the compiler interleaves the cheaper
  // unpack worse with the matrix products (M = 512: 141.7 -> 147.8 us).
  bool pair_order = wq::gemm_pair_order(w[0].bits) && m <= 64;
  for (int i = 0; i < count; ++i) pair_order = pair_order && rotate && w[i].rht_signs;
  if (nr) {
    const wq_status st = hip_status(wq::launch_rht_batch(nr, rx, ry, rs, m, rk, rlx, rly, pair_order, s), who);
    if (st != WQ_OK) return st;
  }
  return hip_status(wq::launch_gemm_batch(count, w, xr, ldr, m, yo, f32, ldo, g.ksplit, part, pair_order, s), who);
}

// One validated linear: the matrix-core path, the GEMV over all m rows
// (uniform width), or the GEMV in chunks of 16 batch rows (mixed width).
wq_status linear_one(const wq_weight &w, const uint16_t *x, int64_t m, int64_t ldx, void *y, wq_dtype y_dtype,
                     int64_t ldy, bool rotate, void *workspace, hipStream_t s) {
  if (use_gemm(w, m)) return run_gemm(1, &w, &x, &ldx, m, &y, &y_dtype, &ldy, rotate, workspace, s, "wq_linear");
  if (uses_xprep(w, m)) return run_gemv(1, &w, &x, &ldx, m, &y, &y_dtype, &ldy, rotate, workspace, s);
  const size_t esz = y_dtype == WQ_F32 ? 4 : 2;
  for (int64_t m0 = 0; m0 < m; m0 += 16) {
    const int64_t mc = (m - m0) < 16 ? (m - m0) : 16;
    const uint16_t *xc = x + m0 * ldx;
    void *yc = static_cast<char *>(y) + (size_t)m0 * (size_t)ldy * esz;
    wq_status st = run_gemv(1, &w, &xc, &ldx, mc, &yc, &y_dtype, &ldy, rotate, workspace, s);
    if (st != WQ_OK) return st;
  }
  return WQ_OK;
}

}  // namespace

extern "C" {

const char *wq_last_error(void) { return g_err; }

size_t wq_packed_words(int32_t bits, int64_t n, int64_t k, const uint8_t *block_bits_host) {
  clear_err();
  if (n <= 0 || k <= 0 || k % WQ_GROUP) {
    fail(WQ_E_ARG, "wq_packed_words: need n > 0 and k a positive multiple of 128");
    return 0;
  }
  if (uniform_bits(bits)) return (size_t)n * (size_t)(k / 32) * (size_t)bits;
  if (bits != 0) {
    fail(WQ_E_UNSUPPORTED, "wq_packed_words: bits=%d", bits);
    return 0;
  }
  if (n % WQ_MIXED_ROWS || !block_bits_host) {
    fail(WQ_E_ARG, "wq_packed_words: mixed width needs n %% 64 == 0 and host block_bits");
    return 0;
  }
  size_t total = 0;
  for (int64_t i = 0; i < n / WQ_MIXED_ROWS; ++i) {
    const int b = block_bits_host[i];
    if (b != 6 && b != 8) {
      fail(WQ_E_ARG, "wq_packed_words: block_bits[%lld]=%d (6 or 8)", (long long)i, b);
      return 0;
    }
    total += (size_t)WQ_MIXED_ROWS * (size_t)(k / 32) * (size_t)b;
  }
  return total;
}

wq_status wq_quantize(int32_t bits, int64_t n, int64_t k, const float *w, const uint32_t *rht_signs,
                      const uint8_t *block_bits, uint8_t *codes, uint16_t *scales, uint16_t *zeros,
                      void *stream) {
  clear_err();
  if (!(uniform_bits(bits) || bits == 0)) return fail(WQ_E_UNSUPPORTED, "wq_quantize: bits=%d", bits);
  if (n <= 0 || k <= 0 || k % WQ_GROUP) return fail(WQ_E_ARG, "wq_quantize: need n > 0, k %% 128 == 0");
  if (!w || !codes || !scales || !zeros) return fail(WQ_E_ARG, "wq_quantize: NULL buffer");
  if (bits == 0 && (n % WQ_MIXED_ROWS || !block_bits))
    return fail(WQ_E_ARG, "wq_quantize: mixed width needs n %% 64 == 0 and block_bits");
  if (!aligned16(w) || !aligned16(codes) || !aligned16(scales) || !aligned16(zeros) ||
      (rht_signs && !aligned16(rht_signs)))
    return fail(WQ_E_ALIGN, "wq_quantize: buffers must be 16-byte aligned");
  return hip_status(wq::launch_quantize(bits, n, k, w, rht_signs, block_bits, codes, scales, zeros,
                                        (hipStream_t)stream), "wq_quantize");
}

wq_status wq_pack(int32_t bits, int64_t n, int64_t k, const uint8_t *codes, const uint8_t *block_bits,
                  uint32_t *packed, uint64_t *block_off, void *stream) {
  clear_err();
  if (!(uniform_bits(bits) || bits == 0)) return fail(WQ_E_UNSUPPORTED, "wq_pack: bits=%d", bits);
  if (n <= 0 || k <= 0 || k % WQ_GROUP) return fail(WQ_E_ARG, "wq_pack: need n > 0, k %% 128 == 0");
  if (!codes || !packed) return fail(WQ_E_ARG, "wq_pack: NULL buffer");
  if (bits == 0 && (n % WQ_MIXED_ROWS || !block_bits || !block_off))
    return fail(WQ_E_ARG, "wq_pack: mixed width needs n %% 64 == 0, block_bits and block_off");
  if (!aligned16(codes) || !aligned16(packed) || (block_off && !aligned16(block_off)))
    return fail(WQ_E_ALIGN, "wq_pack: buffers must be 16-byte aligned");
  return hip_status(wq::launch_pack(bits, n, k, codes, block_bits, packed, block_off, (hipStream_t)stream),
                    "wq_pack");
}

wq_status wq_unpack(int32_t bits, int64_t n, int64_t k, const uint32_t *packed, const uint8_t *block_bits,
                    const uint64_t *block_off, uint8_t *codes, void *stream) {
  clear_err();
  if (!(uniform_bits(bits) || bits == 0)) return fail(WQ_E_UNSUPPORTED, "wq_unpack: bits=%d", bits);
  if (n <= 0 || k <= 0 || k % WQ_GROUP) return fail(WQ_E_ARG, "wq_unpack: need n > 0, k %% 128 == 0");
  if (!codes || !packed) return fail(WQ_E_ARG, "wq_unpack: NULL buffer");
  if (bits == 0 && (n % WQ_MIXED_ROWS || !block_bits || !block_off))
    return fail(WQ_E_ARG, "wq_unpack: mixed width needs n %% 64 == 0, block_bits and block_off");
  if (!aligned16(codes) || !aligned16(packed)) return fail(WQ_E_ALIGN, "wq_unpack: buffers must be 16-byte aligned");
  return hip_status(wq::launch_unpack(bits, n, k, packed, block_bits, block_off, codes, (hipStream_t)stream),
                    "wq_unpack");
}

wq_status wq_embed(const wq_weight *w, const int32_t *ids, int64_t count, void *out, wq_dtype out_dtype,
                   int64_t ldo, void *stream) {
  clear_err();
  wq_status st = check_weight(w, "wq_embed");
  if (st != WQ_OK) return st;
  if (w->bits == 0) return fail(WQ_E_UNSUPPORTED, "wq_embed: mixed width tables are not supported");
  if (w->rht_signs) return fail(WQ_E_UNSUPPORTED, "wq_embed: the table must not be rotated (rht_signs NULL)");
  if (out_dtype != WQ_F16 && out_dtype != WQ_F32) return fail(WQ_E_ARG, "wq_embed: out_dtype=%d", (int)out_dtype);
  if (count < 0) return fail(WQ_E_ARG, "wq_embed: count=%lld", (long long)count);
  if (count > (int64_t)INT32_MAX) return fail(WQ_E_UNSUPPORTED, "wq_embed: count above 2^31-1");
  if (count == 0) return WQ_OK;
  if (!ids || !out) return fail(WQ_E_ARG, "wq_embed: ids and out must be non-NULL");
  if (ldo < w->k) return fail(WQ_E_ARG, "wq_embed: ldo=%lld < k=%lld", (long long)ldo, (long long)w->k);
  if (ldo % (out_dtype == WQ_F32 ? 4 : 8))
    return fail(WQ_E_ALIGN, "wq_embed: ldo must be a multiple of %d", out_dtype == WQ_F32 ? 4 : 8);
  if (!aligned16(out) || ((uintptr_t)ids & 3u)) return fail(WQ_E_ALIGN, "wq_embed: out 16-byte, ids 4-byte aligned");
  return hip_status(wq::launch_embed(*w, ids, count, out, out_dtype == WQ_F32, ldo, (hipStream_t)stream),
                    "wq_embed");
}

wq_status rht_apply(const uint16_t *x, uint16_t *y, const uint32_t *signs, int64_t m, int64_t k, int64_t ldx,
                    int64_t ldy, int32_t block, void *stream) {
  clear_err();
  if (block != WQ_RHT_BLOCK) return fail(WQ_E_UNSUPPORTED, "rht_apply: block=%d (only 128)", block);
  if (m < 0 || k <= 0 || k % WQ_RHT_BLOCK) return fail(WQ_E_ARG, "rht_apply: need m >= 0, k %% 128 == 0");
  if (!x || !y || !signs) return fail(WQ_E_ARG, "rht_apply: NULL buffer");
  if (ldx < k || ldy < k) return fail(WQ_E_ARG, "rht_apply: ldx and ldy must be >= k");
  if (ldx % 8 || ldy % 8) return fail(WQ_E_ALIGN, "rht_apply: ldx and ldy must be multiples of 8");
  if (!aligned16(x) || !aligned16(y) || !aligned16(signs))
    return fail(WQ_E_ALIGN, "rht_apply: buffers must be 16-byte aligned");
  if (x == y && ldx != ldy) return fail(WQ_E_ARG, "rht_apply: in place needs ldx == ldy");
  return hip_status(wq::launch_rht(x, y, signs, m, k, ldx, ldy, (hipStream_t)stream), "rht_apply");
}

size_t wq_linear_workspace(const wq_weight *w, int64_t m) {
  clear_err();
  if (check_weight(w, "wq_linear_workspace") != WQ_OK) return (size_t)-1;
  if (m <= 0) {
    fail(WQ_E_ARG, "wq_linear_workspace: m must be positive");
    return (size_t)-1;
  }
  if (use_gemm(*w, m)) return gemm_path_workspace(*w, m);
  // the GEMV above one batch row: the arranged activations of all m rows
  return uses_xprep(*w, m) ? xprep_bytes(w->k, m) : 0;
}

wq_status wq_linear(const wq_weight *w, const uint16_t *x, int64_t m, int64_t ldx, void *y,
                    wq_dtype y_dtype, int64_t ldy, uint32_t flags, void *workspace, size_t workspace_bytes,
                    void *stream) {
  clear_err();
  wq_status st = check_weight(w, "wq_linear");
  if (st != WQ_OK) return st;
  st = check_io(*w, x, m, ldx, y, y_dtype, ldy, "wq_linear");
  if (st != WQ_OK) return st;
  if (flags & ~WQ_FUSE_RHT) return fail(WQ_E_ARG, "wq_linear: unknown flags 0x%x", flags);
  const size_t need = wq_linear_workspace(w, m);
  if (need > workspace_bytes || (need && !workspace))
    return fail(WQ_E_WORKSPACE, "wq_linear: workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (workspace && !aligned16(workspace)) return fail(WQ_E_ALIGN, "wq_linear: workspace must be 16-byte aligned");
  return linear_one(*w, x, m, ldx, y, y_dtype, ldy, (flags & WQ_FUSE_RHT) && w->rht_signs, workspace,
                    (hipStream_t)stream);
}

size_t wq_linear_batch_workspace(int32_t count, const wq_weight *w, int64_t m) {
  clear_err();
  if (count <= 0 || count > WQ_MAX_BATCH || !w) {
    fail(WQ_E_ARG, "wq_linear_batch_workspace: count must be 1..%d", WQ_MAX_BATCH);
    return (size_t)-1;
  }
  if (m <= 0) {
    fail(WQ_E_ARG, "wq_linear_batch_workspace: m must be positive");
    return (size_t)-1;
  }
  bool gemm = true;   // use_gemm alone decides which path, and so which workspace, the call takes
  size_t all = 0;
  for (int i = 0; i < count; ++i) {
    if (check_weight(&w[i], "wq_linear_batch_workspace") != WQ_OK) return (size_t)-1;
    gemm = gemm && use_gemm(w[i], m) && w[i].bits == w[0].bits;
    if (uses_xprep(w[i], m)) all += xprep_bytes(w[i].k, m);
  }
  // above 16 rows with one uniform width: one matrix-core launch over all of them;
  // below: every linear's arranged activations side by side (none for the
  // mixed layout, whose GEMV needs no workspace)
  if (gemm) return gemm_layout(count, w, m, true).total;
  return all;
}

wq_status wq_linear_batch(int32_t count, const wq_weight *w, const uint16_t *const *x, const int64_t *ldx,
                          int64_t m, void *const *y, const wq_dtype *y_dtype, const int64_t *ldy, uint32_t flags,
                          void *workspace, size_t workspace_bytes, void *stream) {
  clear_err();
  if (count <= 0 || count > WQ_MAX_BATCH) return fail(WQ_E_ARG, "wq_linear_batch: count must be 1..%d", WQ_MAX_BATCH);
  if (!w || !x || !ldx || !y || !y_dtype || !ldy) return fail(WQ_E_ARG, "wq_linear_batch: NULL argument array");
  if (m <= 0) return fail(WQ_E_ARG, "wq_linear_batch: m=%lld must be positive", (long long)m);
  if (flags & ~WQ_FUSE_RHT) return fail(WQ_E_ARG, "wq_linear_batch: unknown flags 0x%x", flags);
  for (int i = 0; i < count; ++i) {
    wq_status st = check_weight(&w[i], "wq_linear_batch");
    if (st != WQ_OK) return st;
    st = check_io(w[i], x[i], m, ldx[i], y[i], y_dtype[i], ldy[i], "wq_linear_batch");
    if (st != WQ_OK) return st;
    if (w[i].bits != w[0].bits)
      return fail(WQ_E_UNSUPPORTED, "wq_linear_batch: all weights must share one code width");
    if (((flags & WQ_FUSE_RHT) && w[i].rht_signs) != ((flags & WQ_FUSE_RHT) && w[0].rht_signs))
      return fail(WQ_E_UNSUPPORTED, "wq_linear_batch: rotate all linears or none");
  }
  const bool rotate = (flags & WQ_FUSE_RHT) && w[0].rht_signs;
  const size_t need = wq_linear_batch_workspace(count, w, m);
  if (need == (size_t)-1) return WQ_E_ARG;
  if (need > workspace_bytes || (need && !workspace))
    return fail(WQ_E_WORKSPACE, "wq_linear_batch: workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (workspace && !aligned16(workspace))
    return fail(WQ_E_ALIGN, "wq_linear_batch: workspace must be 16-byte aligned");
  if (use_gemm(w[0], m))   // one width (checked above): all on the matrix cores in one launch
    return run_gemm(count, w, x, ldx, m, y, y_dtype, ldy, rotate, workspace, (hipStream_t)stream,
                    "wq_linear_batch");
  if (m <= 16 || w[0].bits != 0)   // the GEMV: one launch per tile of batch rows over all the linears
    return run_gemv(count, w, x, ldx, m, y, y_dtype, ldy, rotate, workspace, (hipStream_t)stream);
  for (int i = 0; i < count; ++i) {   // mixed width above 16 rows: one linear after another
    const wq_status st = linear_one(w[i], x[i], m, ldx[i], y[i], y_dtype[i], ldy[i], rotate, workspace,
                                    (hipStream_t)stream);
    if (st != WQ_OK) return st;
  }
  return WQ_OK;
}

wq_status wq_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream) {
  clear_err();
  if (!src || !sink) return fail(WQ_E_ARG, "wq_stream_read: NULL pointer");
  if (bytes == 0 || bytes % 16)
    return fail(WQ_E_ARG, "wq_stream_read: bytes=%zu must be a positive multiple of 16", bytes);
  if (!aligned16(src) || !aligned16(sink)) return fail(WQ_E_ALIGN, "wq_stream_read: pointers must be 16-byte aligned");
  if ((bytes / 16 + 511) / 512 > 0x7FFFFFFFull) return fail(WQ_E_ARG, "wq_stream_read: %zu bytes is too large", bytes);
  const hipError_t e = wq::launch_stream_read(src, bytes, sink, (hipStream_t)stream);
  return e == hipSuccess ? WQ_OK : fail(WQ_E_HIP, "wq_stream_read: %s", hipGetErrorString(e));
}

}  // extern "C"

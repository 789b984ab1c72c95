/*
 * wq.h - C ABI of libwq: a rotated, grouped-affine low-bit linear layer for
 * AMD Instinct MI355X (gfx950).
 *
 * What the layer computes.  The weight of a linear layer with N output rows
 * and K input channels is stored as integer codes q (3, 4, 6 or 8 bits) with
 * one fp16 scale s and one fp16 zero point z per group of 128 consecutive
 * entries along K, and a weight is w = (q - z) * s.  The dequantised weight
 * is never written to memory: it is formed in registers inside the product.
 * Source: model card "24B0978 - Week 01 - Track 2, 20% target -
 * Submission 01", section "How these techniques accelerate inference on
 * CUDA", paragraph on group-wise affine integer quantisation.
 *
 * Before quantisation each weight row was rotated by a block random Hadamard
 * transform R = H . D / sqrt(128) per block of 128 channels (H: Sylvester
 * Hadamard matrix, D: random +-1 diagonal, one sign per input channel).  At
 * run time the same R is applied to the activations, so the layer computes
 *     y[m][n] = sum_k What[n][k] * (R x[m])[k].
 * Source: same card and section, paragraph on the random Hadamard transform;
 * model card "24B0978 - Week 02 - Track 2, 40% target - Submission 01",
 * section "Recipe" (rotation per weight block before quantisation).
 *
 * Conventions for every entry point:
 *  - Pointers are device pointers unless the argument says "host".
 *  - Every device pointer must be 16-byte aligned.
 *  - fp16 values travel as uint16_t bit patterns (IEEE binary16).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued asynchronously on it; nothing synchronises.
 *  - The library never allocates or frees device memory and never copies
 *    between host and device.  Buffers belong to the caller and must stay
 *    valid until the enqueued work has finished.
 *  - Arguments are checked on the host before anything is enqueued; a bad
 *    argument returns a negative wq_status and wq_last_error() says why.
 *    WQ_E_HIP reports a failed launch.  Faults inside a kernel surface as
 *    errors of the caller's next synchronising HIP call.
 *  - Calls are thread-safe.  Two calls that share a workspace must not run
 *    concurrently (order them on one stream).
 *
 * Data layout in device memory (the cards fix none of it; this is the
 * library's format):
 *  - codes: output rows one after another; the codes of one row are
 *    contiguous along K.  A row of K codes at b bits takes K*b/32 words.
 *      int4: 8 codes per uint32, code j of a word in bits [4j, 4j+4);
 *      int8: 4 codes per uint32, code j in byte j;
 *      int3: 32 codes per 3 uint32, int6: 16 codes per 3 uint32; the three
 *            words form the 96-bit little-endian integer w0|w1<<32|w2<<64
 *            and code j of the run sits in bits [b*j, b*j+b).
 *  - scales, zeros: fp16 [N][K/128], row-major.  (The batch-1 kernel for
 *    8-bit codes reads these arrays in 16-byte pieces, up to the 16-byte
 *    boundary after their last element: up to 15 bytes past their end,
 *    never past that boundary, so never into another page.  Those bytes do
 *    not affect any result.)
 *  - mixed width: rows are cut into blocks of 64; block i is coded at
 *    block_bits[i] bits (6 or 8) with the layout above; blocks follow each
 *    other with no padding; block i starts at word block_off[i], and
 *    block_off[N/64] is the total word count.  Source: model card
 *    "25M2111-Week02-Track2-40-Submission01", section "Method, selection,
 *    and reproduction" (dense mixed-width codes in 64-row blocks with byte
 *    selectors).
 *  - rotation signs: uint32 [K/32] bit vector; bit (k & 31) of word (k >> 5)
 *    set means d[k] = -1.
 *  - activations x: fp16 [M][ldx] row-major, ldx >= K; outputs y: fp16 or
 *    fp32 [M][ldy] row-major, ldy >= N.
 */
#ifndef WQ_H
#define WQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum wq_status {
  WQ_OK = 0,
  WQ_E_ARG = -1,          /* null pointer, bad size or value */
  WQ_E_UNSUPPORTED = -2,  /* valid request this library does not implement */
  WQ_E_ALIGN = -3,        /* a pointer is not 16-byte aligned */
  WQ_E_WORKSPACE = -4,    /* workspace missing or too small */
  WQ_E_HIP = -5           /* the HIP runtime reported an error */
} wq_status;

/* Output element types.  A plain 32-bit integer rather than an enum type,
 * so that any value a caller passes is a defined value for the library to
 * check (and refuse with WQ_E_ARG); the same size as an enum in the C ABI. */
typedef int32_t wq_dtype;
enum { WQ_F16 = 1, WQ_F32 = 2 };

/* wq_linear flag: rotate the activations (per 128-block, with the weight's
 * signs) inside the product.  Without it, x is used as given. */
#define WQ_FUSE_RHT 1u

#define WQ_GROUP 128
#define WQ_RHT_BLOCK 128
#define WQ_MIXED_ROWS 64
#define WQ_MAX_BATCH 8

/* A quantised weight.  The struct itself is a host object; the arrays it
 * points to are device arrays in the layout described above. */
typedef struct wq_weight {
  int32_t bits;                 /* 3, 4, 6 or 8; 0 = mixed 6/8 (block_bits) */
  int32_t group;                /* must be 128 */
  int64_t n;                    /* output rows */
  int64_t k;                    /* input channels, a multiple of 128 */
  const uint32_t *codes;        /* packed codes (wq_pack) */
  const uint16_t *scales;       /* fp16 [n][k/128] */
  const uint16_t *zeros;        /* fp16 [n][k/128]; any value, not only integers */
  const uint8_t *block_bits;    /* mixed only: [n/64], each 6 or 8; else NULL */
  const uint64_t *block_off;    /* mixed only: [n/64 + 1] word offsets; else NULL */
  const uint32_t *rht_signs;    /* [k/32] sign bits, or NULL for no rotation */
  int32_t rht_block;            /* 128 when rht_signs != NULL, else 0 */
  /* Mixed only, optional (else NULL): the widths of block_bits again, in
   * HOST memory, [n/64], each 6 or 8, read during the call only; they must
   * equal block_bits.  With them the batch-1 kernel gets every workgroup's
   * rows from the host (up to WQ_MIXED_HOST_WORKGROUPS workgroups) instead of
   * finding them in the block table before its first weight load: about
   * 0.9 us sooner on a 9728 -> 2560 layer.  Values other than 6 and 8 are
   * refused with WQ_E_ARG. */
  const uint8_t *block_bits_host;
} wq_weight;

/* Most batch-1 workgroups the host places for a mixed layout from a host
 * copy of its widths (a 256-CU MI355X launches one per CU). */
#define WQ_MIXED_HOST_WORKGROUPS 256

/* Number of uint32 words wq_pack writes for an n x k code matrix.  For
 * mixed width (bits == 0) pass the per-block widths in host memory; else
 * pass NULL.  Returns 0 for an invalid request (see wq_last_error). */
size_t wq_packed_words(int32_t bits, int64_t n, int64_t k, const uint8_t *block_bits_host);

/* Offline weight preparation: rotate every row of w by R (if rht_signs is
 * not NULL) in fp64, round the rotated weight to fp32, then quantise each
 * group of 128 by round-to-nearest:
 *   lo = min(min v, 0), hi = max(max v, 0),
 *   s  = fp16((hi - lo) / qmax) (nearest, ties to even; 1 if it is 0),
 *   z  = clamp(rint(-lo / s), 0, qmax), q = clamp(rint(v / s + z), 0, qmax),
 * in fp64, rint rounding half to even, qmax = 2^bits - 1.  The cards name
 * round-to-nearest for this format but give no formula; this is the
 * library's reading.  Sources: "24B0978 - Week 02 - Track 2, 40% target",
 * sections "Recipe" and "Recipe (exact)" (RTN, 8 bits, group 128; rotation
 * applied per weight block before quantisation).
 *   w          fp32 [n][k], read only
 *   rht_signs  [k/32] sign bits or NULL
 *   bits       3, 4, 6, 8, or 0 with block_bits (device, [n/64]) for mixed
 *   codes      out: uint8 [n][k], one code per byte
 *   scales     out: fp16 [n][k/128];  zeros: out fp16 [n][k/128] */
wq_status wq_quantize(int32_t bits, int64_t n, int64_t k, const float *w,
                      const uint32_t *rht_signs, const uint8_t *block_bits,
                      uint8_t *codes, uint16_t *scales, uint16_t *zeros, void *stream);

/* Pack one-code-per-byte codes (uint8 [n][k], each < 2^bits) into the code
 * layout above.  packed must hold wq_packed_words(...) words.  For mixed
 * width (bits == 0), block_bits is the device array [n/64] and block_off
 * (device, [n/64 + 1]) receives the block word offsets; otherwise both are
 * NULL.  Codes are not range-checked: bits above the width are dropped.
 * Sources: "24B0978 - Week 01 - Track 2", paragraph on the absence of
 * unstructured sparsity (dense packed codes with a regular stride);
 * "24B0908 ... Mixed-precision GPTQ", section "CUDA speedup potential"
 * (packed int3 read directly by the kernel). */
wq_status wq_pack(int32_t bits, int64_t n, int64_t k, const uint8_t *codes,
                  const uint8_t *block_bits, uint32_t *packed, uint64_t *block_off,
                  void *stream);

/* Inverse of wq_pack (a checking tool): packed words -> uint8 [n][k] codes.
 * For mixed width pass block_bits and the block_off written by wq_pack. */
wq_status wq_unpack(int32_t bits, int64_t n, int64_t k, const uint32_t *packed,
                    const uint8_t *block_bits, const uint64_t *block_off,
                    uint8_t *codes, void *stream);

/* Block random Hadamard rotation of activations:
 *   y[m][128j : 128j+128] = H . D_j . x[m][128j : 128j+128] / sqrt(128)
 * computed as log2(128) = 7 butterfly stages of adds and subtracts in fp32,
 * rounded once to fp16 (nearest even).  y may equal x (in place) when
 * ldy == ldx.  Source: "24B0978 - Week 01 - Track 2", paragraph on the
 * random Hadamard transform (fast Walsh-Hadamard transform on the
 * activations at run time).
 *   x  fp16 [m][ldx];  y  out fp16 [m][ldy];  signs  [k/32] sign bits
 *   block must be 128; k a multiple of 128. */
wq_status rht_apply(const uint16_t *x, uint16_t *y, const uint32_t *signs,
                    int64_t m, int64_t k, int64_t ldx, int64_t ldy, int32_t block,
                    void *stream);

/* Bytes of workspace wq_linear needs for this weight and batch size m.
 * 0 means none is needed: m = 1, or the mixed 6/8-bit layout (any m).
 * For 2 <= m <= 16 with one code width it is the arranged activations of
 * all m batch rows (80 bytes per 32 elements per row, rounded up to 256
 * bytes); for m >= 17 the matrix-core path's rotated activations and
 * split-K partials.  Returns (size_t)-1 for an invalid request. */
size_t wq_linear_workspace(const wq_weight *w, int64_t m);

/* The layer: y[m][n] = sum_k (q[n][k] - z[n][g]) * s[n][g] * x'[m][k],
 * g = k / 128, x' = R x[m] when flags has WQ_FUSE_RHT and w->rht_signs is
 * set, else x' = x[m].  The scale is applied once per group to the group's
 * partial sum and products accumulate in fp32 (source: "24B0978 - Week 01
 * - Track 2", paragraph on group-wise affine integer quantisation).
 * m <= 16 runs the dequantising GEMV; m >= 17 runs the matrix-core GEMM
 * (the codes become q - z in fp16 registers, exact for an integer zero
 * point and rounded once otherwise, and each group's scale multiplies the
 * fp32 accumulator; tiles of 32 batch rows up to m = 32, of 64 up to 64, of
 * 128 above).  The rotated activations are rounded to fp16 before the
 * product.  Above one
 * batch row the GEMV first rotates and arranges all m activation rows into
 * the workspace in one pass, then streams the weights once per tile of batch
 * rows: 16 while 13 or more rows are left, else 8 while 5 or more are, else
 * the rest, each where that many rows of arranged activations fit in a
 * workgroup's LDS in up to 4 chunks of K (else the next smaller).  The mixed
 * 6/8-bit layout runs its GEMV (any m, in chunks of 16 rows) without a
 * workspace.
 *   w          host struct describing the device weight
 *   x          fp16 [m][ldx]
 *   y          out: fp16 or fp32 [m][ldy] (y_dtype)
 *   workspace  device scratch of at least wq_linear_workspace(w, m) bytes
 *              (caller-owned, 16-byte aligned; NULL when that is 0).  The
 *              GEMV keeps the arranged activations there; the matrix-core
 *              path the rotated activations and the fp32 partial sums when
 *              it splits a long K over several workgroups.  Its contents
 *              need no initialisation and are not preserved.
 * Errors (all before anything is launched): WQ_E_ARG (NULL pointer, m <= 0,
 * ldx < k, ldy < n, bad y_dtype or flags, bad weight descriptor),
 * WQ_E_ALIGN (a pointer not 16-byte aligned, ldx not a multiple of 8),
 * WQ_E_UNSUPPORTED (bits, group or rht_block not supported; m * ldx * 2
 * of 2^31 bytes or more, k of 2^27 or more, or n x k codes above 4 GiB:
 * the kernels address them with 32-bit offsets), WQ_E_WORKSPACE (workspace
 * smaller than wq_linear_workspace); WQ_E_HIP if a launch fails.
 */
wq_status wq_linear(const wq_weight *w, const uint16_t *x, int64_t m, int64_t ldx,
                    void *y, wq_dtype y_dtype, int64_t ldy, uint32_t flags,
                    void *workspace, size_t workspace_bytes, void *stream);

/* Several independent linears (up to WQ_MAX_BATCH), each with its own
 * weight, activations and output, all at the same batch size m and code
 * width.  For m <= 16 they run as one GEMV launch per tile of batch rows
 * (tiles as for wq_linear, chosen so that every linear's tile fits in LDS;
 * after, for m > 1, one launch arranging every linear's activations in the
 * workspace).  For m >= 17 with a uniform code width they run as one
 * matrix-core launch (after one launch rotating every linear's
 * activations); the workspace of wq_linear_batch_workspace bytes then holds
 * every linear's rotated activations and split-K partial sums.  The mixed
 * 6/8-bit layout above m = 16 runs one linear after another on the stream
 * exactly as wq_linear would.  Same math and layout as wq_linear, applied to
 * each w[i], x[i], y[i].  In the grouped launches, linears with the same
 * input (x and ldx equal, the same k and the same rht_signs pointer, e.g.
 * query, key and value projections quantised with one sign vector) share
 * one rotation and arrangement of it ("24B0978 - Week 01 - Track 2",
 * paragraph on the random Hadamard transform).  Arrays of length `count`
 * are host arrays. */
size_t wq_linear_batch_workspace(int32_t count, const wq_weight *w, int64_t m);
wq_status wq_linear_batch(int32_t count, const wq_weight *w,
                          const uint16_t *const *x, const int64_t *ldx, int64_t m,
                          void *const *y, const wq_dtype *y_dtype, const int64_t *ldy,
                          uint32_t flags, void *workspace, size_t workspace_bytes,
                          void *stream);

/* wq_linear_batch for callers that cannot allocate device memory (code
 * under stream capture, tight serving loops, harnesses that forbid
 * allocation): the same call, arguments and results, with no workspace
 * argument.  Its workspace is a static scratch array inside the library,
 * WQ_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, which each GPU the library
 * runs on holds until the process ends.  The call itself allocates and
 * frees nothing.  The scratch needs no initialisation and keeps the last
 * call's contents; calls that overlap on one GPU (several streams or host
 * threads at once) share it and race: serialise them.  64 MiB covers, for
 * example, the seven projections of a 4B-class decoder block up to 512
 * batch rows (58.8 MB).
 * Errors: those of wq_linear_batch, and WQ_E_WORKSPACE (nothing launched)
 * when wq_linear_batch_workspace for the same arguments exceeds
 * WQ_NOALLOC_SCRATCH_BYTES; WQ_E_HIP if the scratch's address cannot be
 * looked up on the current device. */
#define WQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
wq_status wq_linear_batch_noalloc(int32_t count, const wq_weight *w,
                                  const uint16_t *const *x, const int64_t *ldx, int64_t m,
                                  void *const *y, const wq_dtype *y_dtype, const int64_t *ldy,
                                  uint32_t flags, void *stream);

/* Tied-embedding gather: rows ids[0..count) of a quantised table,
 * dequantised,
 *   out[i][k] = (q[ids[i]][k] - z[ids[i]][k/128]) * s[ids[i]][k/128],
 * computed exactly and rounded once (nearest even) to fp16 or fp32.  The
 * table of the output head serves as the token embedding (model card
 * "24B0978 - Week 02 - Track 2, 40% target", section "Recipe": embed_tokens
 * tied to lm_head, RTN 8-bit, group 128; the dequantisation is the
 * grouped-affine form of "24B0978 - Week 01 - Track 2").
 *   w          the table: uniform width (3, 4, 6 or 8), group 128, not
 *              rotated (rht_signs NULL; a rotated table would need its rows
 *              rotated back, which this call does not do)
 *   ids        device int32 [count]; an id outside [0, w->n) gives a row
 *              of zeros (the table is not read for it)
 *   out        device fp16 or fp32 (out_dtype) [count][ldo], 16-byte
 *              aligned; ldo >= k, a multiple of 8 (fp16) or 4 (fp32);
 *              columns past k are not written
 * count 0 does nothing.  Errors: WQ_E_ARG (NULL pointer, count < 0, ldo <
 * k), WQ_E_UNSUPPORTED (mixed width, a rotated table, count >= 2^31),
 * WQ_E_ALIGN, WQ_E_HIP (launch failure). */
wq_status wq_embed(const wq_weight *w, const int32_t *ids, int64_t count, void *out,
                   wq_dtype out_dtype, int64_t ldo, void *stream);

/* Message for the last failed call on this thread ("" if none). */
const char *wq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* WQ_H */

// wq_linear_batch_noalloc: wq_linear_batch with the library's own scratch
// memory as its workspace, for callers that cannot allocate device memory
// (code under stream capture, serving loops, harnesses that forbid it).
//
// The scratch is a file-scope device array of kScratchBytes; each GPU the
// library runs on holds its own copy until the process ends.  In host code
// the array's name is not a device address: its address on the current
// device is looked up once per device (hipGetSymbolAddress) and only that
// pointer is handed to the kernels.  Nothing in the workspace has to start
// at zero (the kernels write every byte they later read), so no clearing is
// needed between calls.  Every call on one GPU uses that GPU's one array:
// calls that overlap on one GPU (several streams, or threads) race on it.
#include <mutex>

#include "wq_internal.h"

namespace {

constexpr size_t kScratchBytes = WQ_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The scratch's device address on device `dev` (looked up on first use).
hipError_t scratch_on(int dev, void **ptr) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

wq_status wq_linear_batch_noalloc(int32_t count, const wq_weight *w, const uint16_t *const *x,
                                  const int64_t *ldx, int64_t m, void *const *y, const wq_dtype *y_dtype,
                                  const int64_t *ldy, uint32_t flags, void *stream) {
  wq::clear_error();
  const size_t need = wq_linear_batch_workspace(count, w, m);   // validates count, w and m
  if (need == (size_t)-1) return WQ_E_ARG;
  if (need > kScratchBytes)
    return wq::set_error(WQ_E_WORKSPACE,
                         "wq_linear_batch_noalloc: the call needs %zu bytes of workspace, more than the "
                         "%zu bytes of the library's static scratch (use wq_linear_batch with a workspace)",
                         need, kScratchBytes);
  void *ws = nullptr;
  if (need) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) e = hipErrorInvalidDevice;
    if (e == hipSuccess) e = scratch_on(dev, &ws);
    if (e != hipSuccess)
      return wq::set_error(WQ_E_HIP, "wq_linear_batch_noalloc: scratch address: %s", hipGetErrorString(e));
  }
  return wq_linear_batch(count, w, x, ldx, m, y, y_dtype, ldy, flags, ws, need ? kScratchBytes : 0, stream);
}

}  // extern "C"

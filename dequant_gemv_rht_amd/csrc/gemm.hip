// Matrix-core (MFMA) path for batch sizes >= 64: not built yet.
#include "wq_internal.h"

namespace wq {

bool gemm_available(int bits) {
  (void)bits;
  return false;
}

size_t gemm_workspace(const wq_weight &w, int64_t m) {
  (void)w;
  (void)m;
  return 0;
}

hipError_t launch_gemm(const wq_weight &w, const uint16_t *xr, int64_t m, int64_t ldx, void *y, int out_f32,
                       int64_t ldy, void *workspace, hipStream_t s) {
  (void)w; (void)xr; (void)m; (void)ldx; (void)y; (void)out_f32; (void)ldy; (void)workspace; (void)s;
  return hipErrorNotSupported;
}

}  // namespace wq

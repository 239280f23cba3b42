// W4A4G4 linear layer (placeholder entry points; kernels follow).
#include "common.hpp"

extern "C" size_t metis_linear_workspace_bytes(const metis_split_t *X, const metis_split_t *W,
                                               const metis_split_t *dY) {
  (void)X; (void)W; (void)dY;
  return 256;
}
extern "C" metis_status_t spectral_fp4_linear_fwd(const metis_split_t *X, const metis_split_t *W, float *Y,
                                                  int64_t ldy, void *ws, size_t ws_bytes, hipStream_t stream) {
  (void)X; (void)W; (void)Y; (void)ldy; (void)ws; (void)ws_bytes; (void)stream;
  return METIS_ERR_UNSUPPORTED;
}
extern "C" metis_status_t spectral_fp4_linear_bwd(const metis_split_t *dY, const metis_split_t *X,
                                                  const metis_split_t *W, float *dX, int64_t lddx, float *dW,
                                                  int64_t lddw, void *ws, size_t ws_bytes, hipStream_t stream) {
  (void)dY; (void)X; (void)W; (void)dX; (void)lddx; (void)dW; (void)lddw; (void)ws; (void)ws_bytes; (void)stream;
  return METIS_ERR_UNSUPPORTED;
}

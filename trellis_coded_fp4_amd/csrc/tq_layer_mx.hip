// tq_layer_mx.hip -- C ABI of the grouped MoE GEMV and layer on expanded
// MXFP4 weights (the kernels of tq_layer.h instantiated for FmtMx).
#include "tq_layer.h"

using namespace tq;

// Expanded MXFP4 weights: the same kernels with the weights' nibbles fed to
// the matrix cores as stored. MXFP4 steps never outnumber trellis steps for
// a width, so the trellis workspace sizes cover both.
static int check_mx_align(const trellis_mx_t *w) {
  if (!w) return TRELLIS_ENULL;
  if (((uintptr_t)w->codes & 15) || ((uintptr_t)w->scales & 15)) return TRELLIS_EINVAL;
  return TRELLIS_OK;
}

extern "C" int trellis_mxfp4_moe_gemv(hipStream_t stream, const trellis_mx_t *w, const void *x, int32_t x_dtype,
                                      int32_t x_per_slot, const int32_t *topk_ids, const float *topk_w,
                                      int32_t T, int32_t k, float *y, void *workspace, size_t workspace_bytes) {
  int rc = check_mx_align(w);
  if (rc) return rc;
  return gemv_impl<FmtMx>(stream, mx_mats(w), x, x_dtype, x_per_slot, topk_ids, topk_w, T, k, y, workspace,
                          workspace_bytes);
}

extern "C" int trellis_mxfp4_moe_ffn(hipStream_t stream, const trellis_mx_t *w_gate_up, const trellis_mx_t *w_down,
                                     const void *x, int32_t x_dtype, const int32_t *topk_ids, const float *topk_w,
                                     int32_t T, int32_t k, uint16_t *h, float *y, void *workspace,
                                     size_t workspace_bytes) {
  int rc;
  if ((rc = check_mx_align(w_gate_up)) || (rc = check_mx_align(w_down))) return rc;
  return ffn_impl<FmtMx>(stream, mx_mats(w_gate_up), mx_mats(w_down), x, x_dtype, topk_ids, topk_w, T, k, h, y,
                         workspace, workspace_bytes, nullptr);
}


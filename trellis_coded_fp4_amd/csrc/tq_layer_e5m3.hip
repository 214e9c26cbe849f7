// tq_layer_e5m3.hip -- C ABI of the fused trellis-decode MoE GEMV and layer
// for trellis-coded weights under E5M3 block scales (the kernels of
// tq_layer.h instantiated for FmtTrellisE5M3). The streams, shapes and
// workspaces are those of the UE8M0 calls; only the meaning of the scale
// bytes differs. The layer always runs the general persistent kernel (the
// single-token layer kernel takes UE8M0 scales only).
#include "tq_layer.h"

using namespace tq;

extern "C" int trellis_moe_gemv_e5m3(hipStream_t stream, const trellis_mat_t *w, const void *x, int32_t x_dtype,
                                     int32_t x_per_slot, const int32_t *topk_ids, const float *topk_w, int32_t T,
                                     int32_t k, float *y, void *workspace, size_t workspace_bytes) {
  if (!w) return TRELLIS_ENULL;
  return gemv_impl<FmtTrellisE5M3>(stream, trellis_mats(w), x, x_dtype, x_per_slot, topk_ids, topk_w, T, k, y,
                                   workspace, workspace_bytes);
}

extern "C" int trellis_moe_ffn_e5m3(hipStream_t stream, const trellis_mat_t *w_gate_up, const trellis_mat_t *w_down,
                                    const void *x, int32_t x_dtype, const int32_t *topk_ids, const float *topk_w,
                                    int32_t T, int32_t k, uint16_t *h, float *y, void *workspace,
                                    size_t workspace_bytes) {
  if (!w_gate_up || !w_down) return TRELLIS_ENULL;
  return ffn_impl<FmtTrellisE5M3>(stream, trellis_mats(w_gate_up), trellis_mats(w_down), x, x_dtype, topk_ids,
                                  topk_w, T, k, h, y, workspace, workspace_bytes, nullptr);
}

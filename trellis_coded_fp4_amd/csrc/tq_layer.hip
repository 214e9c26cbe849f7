// tq_layer.hip -- C ABI of the fused trellis-decode MoE GEMV and layer
// (the kernels and their host launch code are in tq_layer.h; this unit
// instantiates them for trellis-coded weights).
#include "tq_layer.h"

using namespace tq;

extern "C" size_t trellis_moe_gemv_workspace_size(int32_t n_mat, int32_t rows, int32_t cols, int32_t T,
                                                  int32_t k) {
  if (n_mat < 1 || cols < 32 || cols % 32 || rows < 1 || check_routing(T, k)) return 0;
  return make_layout<FmtTrellis>(0, (rows + 63) / 64, T * k, rows, 0, T, cols).total;
}

extern "C" int trellis_moe_gemv(hipStream_t stream, const trellis_mat_t *w, const void *x, int32_t x_dtype,
                                int32_t x_per_slot, const int32_t *topk_ids, const float *topk_w,
                                int32_t T, int32_t k, float *y, void *workspace, size_t workspace_bytes) {
  if (!w) return TRELLIS_ENULL;
  return gemv_impl<FmtTrellis>(stream, trellis_mats(w), x, x_dtype, x_per_slot, topk_ids, topk_w, T, k, y,
                               workspace, workspace_bytes);
}

extern "C" size_t trellis_moe_ffn_workspace_size(int32_t n_exp, int32_t hidden, int32_t inter, int32_t T,
                                                 int32_t k) {
  if (n_exp < 1 || hidden < 32 || hidden % 32 || inter < 32 || inter % 32 || check_routing(T, k)) return 0;
  return make_layout<FmtTrellis>(std::min(n_exp, T * k), 0, T * k, 0, inter, T, hidden).total;
}

extern "C" int trellis_moe_ffn_timed(hipStream_t stream, const trellis_mat_t *w_gate_up,
                                     const trellis_mat_t *w_down, const void *x, int32_t x_dtype,
                                     const int32_t *topk_ids, const float *topk_w, int32_t T, int32_t k,
                                     uint16_t *h, float *y, void *workspace, size_t workspace_bytes,
                                     hipEvent_t *events) {
  if (!w_gate_up || !w_down) return TRELLIS_ENULL;
  return ffn_impl<FmtTrellis>(stream, trellis_mats(w_gate_up), trellis_mats(w_down), x, x_dtype, topk_ids, topk_w,
                              T, k, h, y, workspace, workspace_bytes, events);
}

extern "C" int trellis_moe_ffn(hipStream_t stream, const trellis_mat_t *w_gate_up, const trellis_mat_t *w_down,
                               const void *x, int32_t x_dtype, const int32_t *topk_ids, const float *topk_w,
                               int32_t T, int32_t k, uint16_t *h, float *y, void *workspace,
                               size_t workspace_bytes) {
  return trellis_moe_ffn_timed(stream, w_gate_up, w_down, x, x_dtype, topk_ids, topk_w, T, k, h, y, workspace,
                               workspace_bytes, nullptr);
}

#ifdef TQ_TRACE
extern "C" void tq_set_trace(void *p) { tq::g_trace = p; }
#endif

// tq_layer.hip -- C ABI of the fused trellis-decode MoE GEMV and layer
// (the kernels and their host launch code are in tq_layer.h; this unit
// instantiates them for trellis-coded weights).
#include "tq_layer.h"

#include <mutex>

using namespace tq;

extern "C" size_t trellis_moe_gemv_workspace_size(int32_t n_mat, int32_t rows, int32_t cols, int32_t T,
                                                  int32_t k) {
  if (n_mat < 1 || cols < 32 || cols % 32 || rows < 1 || check_routing(T, k)) return 0;
  return make_layout<FmtTrellis>(0, (rows + 63) / 64, T * k, rows, 0, T, cols).total;
}

extern "C" size_t trellis_moe_gemv_workspace(const trellis_mat_t *w, int32_t T, int32_t k) {
  if (!w) return 0;
  return trellis_moe_gemv_workspace_size(w->n_mat, w->rows, w->cols, T, k);
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
  return make_layout<FmtTrellis>(std::min(n_exp, T * k), 0, T * k, 0, inter, T, hidden,
                                 tok_region(n_exp, hidden, inter).total).total;
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

extern "C" int trellis_moe_ffn_routed(hipStream_t stream, const trellis_mat_t *w_gate_up,
                                      const trellis_mat_t *w_down, const void *x, int32_t x_dtype,
                                      const uint16_t *w_router, int32_t k, int32_t *topk_ids_out,
                                      float *topk_w_out, uint16_t *h, float *y, void *workspace,
                                      size_t workspace_bytes, hipEvent_t *events) {
  if (!w_gate_up || !w_down) return TRELLIS_ENULL;
  const Mats gu = trellis_mats(w_gate_up), dn = trellis_mats(w_down);
  int rc;
  if ((rc = check_mats(gu)) || (rc = check_mats(dn))) return rc;
  if (!x || !w_router || !topk_ids_out || !topk_w_out || !h || !y || !workspace) return TRELLIS_ENULL;
  if (x_dtype != TRELLIS_F32 && x_dtype != TRELLIS_BF16) return TRELLIS_EINVAL;
  if ((rc = check_routing(1, k))) return rc;
  const int E = gu.n_mat, hidden = gu.cols, inter = gu.rows / 2;
  if (gu.rows % 64 || dn.n_mat != E || dn.rows != hidden || dn.cols != inter || k > E) return TRELLIS_EINVAL;
  const Layout L = make_layout<FmtTrellis>(std::min(E, k), 0, k, 0, inter, 1, hidden,
                                           tok_region(E, hidden, inter).total);
  if (((uintptr_t)workspace & 255) || workspace_bytes < L.total) return TRELLIS_EWORKSPACE;
  int cus = 0;
  if ((rc = device_check(&cus))) return rc;
  TokCall c{(const uint32_t *)gu.w, gu.scales, (const uint32_t *)dn.w, dn.scales, E, hidden, inter, k, nullptr,
            nullptr, x, x_dtype == TRELLIS_BF16, h, y, (char *)workspace, L.reserve};
  c.w_router = w_router;
  c.ids_out = topk_ids_out;
  c.gw_out = topk_w_out;
  if (!tok_supported(c, cus)) return TRELLIS_EINVAL;
  return tok_launch(c, cus, stream, events ? events[0] : nullptr, events ? events[1] : nullptr);
}

#ifdef TQ_TRACE
extern "C" void tq_set_trace(void *p) { tq::g_trace = p; }
#endif

// ---------------------------------------------------------------- layer with the library's own scratch
//
// trellis_moe_ffn_noalloc runs trellis_moe_ffn on a workspace that lives in
// the code object: `scratch` below, one copy per device, zero-filled when
// the code object is loaded (a device global without an initializer). Calls
// of every shape share it, so each call first zeroes the synchronisation
// state its layout uses (a fill kernel on the call's stream, not a memset,
// so that the call can be captured into a graph); the sticky error word is
// kept. Host code never uses the array's name as an address: the device
// address comes from hipGetSymbolAddress, once per device, with that device
// current.
namespace {
constexpr size_t kScratchBytes = TRELLIS_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];

int scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return TRELLIS_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return TRELLIS_EINVAL;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TRELLIS_EHIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return TRELLIS_OK;
}
}  // namespace

extern "C" int trellis_moe_ffn_noalloc(hipStream_t stream, const trellis_mat_t *w_gate_up,
                                       const trellis_mat_t *w_down, const void *x, int32_t x_dtype,
                                       const int32_t *topk_ids, const float *topk_w, int32_t T, int32_t k,
                                       uint16_t *h, float *y) {
  if (!w_gate_up || !w_down) return TRELLIS_ENULL;
  const size_t need = trellis_moe_ffn_workspace_size(w_gate_up->n_mat, w_gate_up->cols, w_gate_up->rows / 2, T, k);
  if (need == 0) return TRELLIS_EINVAL;
  if (need > kScratchBytes) return TRELLIS_EWORKSPACE;
  void *ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc != TRELLIS_OK) return rc;
  return ffn_impl<FmtTrellis>(stream, trellis_mats(w_gate_up), trellis_mats(w_down), x, x_dtype, topk_ids, topk_w,
                              T, k, h, y, ws, kScratchBytes, nullptr, true);
}

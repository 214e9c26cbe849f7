// tq_tok.h -- host interface of the single-token mixture-of-experts layer
// kernel (tq_tok.hip), which trellis_moe_ffn, trellis_moe_ffn_e5m3 and
// trellis_mxfp4_moe_ffn use for one token.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tq {

// Workspace region of the single-token kernel (inside the layer workspace,
// right after the status words): per-workspace call counter and arrival
// count, h of each active expert as tagged words, and one tag per 16-row
// tile of y recording that the tile was cleared in this call.
struct TokRegion {
  size_t sync, hx, yz, total;
};
TokRegion tok_region(int n_exp, int hidden, int inter);

struct TokCall {
  const uint32_t *w1; const uint8_t *s1;   // gate_up [E][2I][H]
  const uint32_t *w2; const uint8_t *s2;   // down    [E][H][I]
  // (trellis symbols, or with mx set expanded MXFP4 codes, cols / 2 bytes a row)
  int E, H, I, k;
  const int32_t *ids; const float *gate_w;
  const void *x; int x_bf16;
  uint16_t *h; float *y;
  char *ws;                                // layer workspace (status words at 0)
  size_t region_off;                       // offset of the TokRegion
  bool mx = false;                         // weights are expanded MXFP4
  bool e5m3 = false;                       // scale bytes are E5M3 (trellis streams)
  // routed calls: the kernel computes the routing from these router rows
  // (bf16 [E][H]) and writes it to ids_out / gw_out ([k] each); ids and
  // gate_w are then not read
  const uint16_t *w_router = nullptr;
  int32_t *ids_out = nullptr; float *gw_out = nullptr;
};

// True when the kernel takes this shape (otherwise the general layer kernel
// runs): one token, k <= 32, hidden and inter multiples of 64 and at most
// 4096, 16-byte aligned streams and activations, and per-workgroup work
// that fits the kernel's register arrays on this device.
bool tok_supported(const TokCall &c, int cus);

// Enqueue the kernel on `s` (argument checks already done by the caller);
// e0 / e1, when given, are stamped with the start and end of the kernel's
// execution by the dispatch itself.
int tok_launch(const TokCall &c, int cus, hipStream_t s, hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);

// One token through a routed matrix stack (trellis streams under UE8M0 or
// E5M3 scales, or expanded MXFP4 codes), every slot's output kept
// (trellis_moe_gemv and its variants with T = 1, shared x, no gate
// weights): y[k][rows], zeros for slots routed nowhere.
struct TokGemvCall {
  const uint32_t *w; const uint8_t *s;   // [E][rows][K / 16] (MXFP4: K / 2 bytes a row), [E][rows][K / 32]
  int E, rows, K, k;
  const int32_t *ids;
  const void *x; int x_bf16;
  float *y;
  int *status;                           // the workspace's status words
  bool mx = false, e5m3 = false;
};
// True when the kernel takes this shape: rows % 16 == 0, K % 64 == 0, K <=
// 4096, k <= 32, 16-byte aligned streams, scales and x, and at most eight
// tiles per workgroup for the worst-case routing.
bool tok_gemv_supported(const TokGemvCall &c, int cus);
int tok_gemv_launch(const TokGemvCall &c, int cus, hipStream_t s);

}  // namespace tq

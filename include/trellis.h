/*
 * trellis.h -- C ABI of libtrellis: trellis-coded FP4 weights on MI355X (gfx950).
 *
 * The weight format and its decoder follow two pages:
 *  - XOR-Trellis news article (aimodeling.com), bullet "XOR-Trellis FP4
 *    decoder": each weight comes from a 16-bit sliding state; four masked
 *    parities (0x1089, 0x2112, 0x0A24, 0x2441) give p0, p1, q0, q1; (p0, p1)
 *    picks one of the palettes P0=[-6,-1.5,0,2], P1=[-4,-1,0.5,3],
 *    P2=[-3,-0.5,1,4], P3=[-2,0,1.5,6]; (q0, q1) permutes branch -> entry.
 *  - HEPH abstract (ICLR 2027 submission page): the decoded value is scaled
 *    by the checkpoint block's UE8M0 exponent (one per 32 weights), so every
 *    decoded weight is an MXFP4 element; weights are either decoded inside
 *    the mixture-of-experts kernel on every forward pass ("fused") or
 *    expanded once into resident MXFP4 ("expand").
 *
 * Storage (what the pages leave open is fixed here):
 *  - A matrix is [rows = output features][cols = input features]; cols % 32 == 0.
 *  - Branch symbols: 2 bits each, 16 per uint32, little-endian (symbol j of a
 *    word in bits 2j..2j+1), rows contiguous: syms[n_mat][rows][cols/16].
 *  - The state is s = ((s << 2) | b) & 0xFFFF, reset to 0 at each row start;
 *    palette = p0 | p1 << 1, entry = b XOR (q0 | q1 << 1); P3's zero is -0.
 *  - UE8M0 bytes: scales[n_mat][rows][cols/32], value 2^(e-127).
 *  - E2M1 codes per the OCP MX v1.0 spec: sign bit 3, exponent bits 2..1,
 *    mantissa bit 0.
 *
 * Conventions for every call:
 *  - All array pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or synchronises. Work is enqueued on `stream`
 *    (NULL = the default stream) and runs asynchronously.
 *  - Return 0 on success or a negative TRELLIS_E* code. Argument checks run on
 *    the host before anything is enqueued; on error nothing is enqueued.
 *  - Outputs are overwritten, never accumulated into.
 *  - Calls that share a workspace must not overlap in time; otherwise calls
 *    are independent and reentrant.
 */
#ifndef TRELLIS_H_
#define TRELLIS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t;

enum {
  TRELLIS_OK = 0,
  TRELLIS_EINVAL = -1,      /* bad shape, dtype, flag or count */
  TRELLIS_ENULL = -2,       /* a required pointer is NULL */
  TRELLIS_EWORKSPACE = -3,  /* workspace too small or misaligned */
  TRELLIS_EHIP = -4,        /* a HIP runtime call failed (launch error) */
  TRELLIS_EDEVICE = -5      /* the current device is not gfx950 */
};

enum { TRELLIS_F32 = 0, TRELLIS_BF16 = 1 };

/* A stack of n_mat trellis-coded matrices of identical shape. */
typedef struct {
  const uint32_t *syms;    /* device, [n_mat][rows][cols/16] */
  const uint8_t *scales;   /* device, [n_mat][rows][cols/32] */
  int32_t n_mat;           /* >= 1 */
  int32_t rows;            /* >= 1; multiple of 16 for the GEMV calls */
  int32_t cols;            /* >= 32, multiple of 32 */
} trellis_mat_t;

/* Library version (major * 10000 + minor * 100 + patch). */
int trellis_version(void);

/* Static text for an error code. */
const char *trellis_strerror(int err);

/*
 * trellis_decode_expand -- HEPH's expand serving mode: decode every weight of
 * w into resident MXFP4.
 *   codes_out:  device, [n_mat][rows][cols/2] bytes; byte j of a row holds the
 *               E2M1 code of column 2j in its low nibble and of column 2j+1
 *               in its high nibble.
 *   scales_out: device, [n_mat][rows][cols/32]; a byte-for-byte copy of
 *               w->scales (the UE8M0 exponents are reused unchanged).
 * The output is bit-exact: it depends on nothing but the stored symbols.
 * Errors: ENULL for NULL pointers, EINVAL for n_mat/rows < 1 or cols not a
 * positive multiple of 32.
 */
int trellis_decode_expand(hipStream_t stream, const trellis_mat_t *w, uint8_t *codes_out,
                          uint8_t *scales_out);

/*
 * Workspace bytes needed by trellis_moe_gemv for this shape.
 *
 * Workspaces (for trellis_moe_gemv and trellis_moe_ffn) are device scratch
 * owned by the caller, 256-byte aligned, and must be ZERO-FILLED once before
 * their first use; afterwards the calls keep their own bookkeeping in it (the
 * synchronisation counters return to zero, a call counter advances), so a
 * workspace can be reused by later calls (of any shape that fits) without
 * clearing. Each call runs as one persistent kernel whose work items wait on
 * counters or tagged data in the workspace; the waits are bounded. After a
 * call completes:
 *   int32 at byte 0: routing slots skipped because their expert id >= n_mat;
 *   int32 at byte 4: nonzero once a wait has timed out (this happens only if
 *                    other work keeps the kernel's workgroups from being
 *                    resident at the same time). The word is sticky: the call
 *                    that timed out and every later call on the workspace
 *                    write NaN to y and compute nothing else, until the
 *                    workspace is zero-filled again.
 */
size_t trellis_moe_gemv_workspace_size(int32_t n_mat, int32_t rows, int32_t cols, int32_t T,
                                       int32_t k);

/*
 * trellis_moe_gemv_workspace -- the same size for the matrix stack w itself
 * (HEPH abstract, fused serving mode: one workspace per resident stack):
 * trellis_moe_gemv_workspace_size(w->n_mat, w->rows, w->cols, T, k); 0 when
 * w is NULL or describes no valid stack.
 */
size_t trellis_moe_gemv_workspace(const trellis_mat_t *w, int32_t T, int32_t k);

/*
 * trellis_moe_gemv -- routed ("mixture-of-experts") GEMV / small-batch GEMM
 * with the weights decoded inside the kernel on every call (HEPH's fused
 * serving mode). Expert e's matrix is w[e] (n_mat experts).
 *   x:          device activations, dtype x_dtype (TRELLIS_F32 or TRELLIS_BF16),
 *               [T][cols] when x_per_slot == 0, [T][k][cols] when x_per_slot == 1.
 *   topk_ids:   device int32 [T][k]; slot (t, j) uses expert topk_ids[t][j].
 *               A negative id is an empty slot; an id >= n_mat is skipped and
 *               counted (see the workspace note above). Neither is read from w.
 *   topk_w:     device float [T][k] gate weights, or NULL.
 *   y:          device float. With topk_w == NULL: y[T][k][rows],
 *               y[t][j] = W_e x_(t or t,j) (zero for empty/skipped slots).
 *               With topk_w: y[T][rows] = sum_j topk_w[t][j] * W_e x.
 * T in 1..128, k in 1..32, T*k <= 1024; rows % 16 == 0.
 * Accuracy: activations enter the block-scaled FP4 x FP8 matrix cores as a
 * two-term FP8 (E4M3) split with UE8M0 scales per 32; sums are fp32; each
 * output satisfies |y - y_exact| <= 2e-3 * sum |w| |x| (|topk_w| included).
 */
int trellis_moe_gemv(hipStream_t stream, const trellis_mat_t *w, const void *x, int32_t x_dtype,
                     int32_t x_per_slot, const int32_t *topk_ids, const float *topk_w, int32_t T,
                     int32_t k, float *y, void *workspace, size_t workspace_bytes);

/* Workspace bytes needed by trellis_moe_ffn for this layer shape. */
size_t trellis_moe_ffn_workspace_size(int32_t n_exp, int32_t hidden, int32_t inter, int32_t T,
                                      int32_t k);

/*
 * trellis_moe_ffn -- one whole mixture-of-experts layer in fused mode:
 * gate_up GEMV per routed slot, SwiGLU, down GEMV and the gate-weighted
 * combine over the k slots of each token.
 *   w_gate_up:  n_exp matrices [2*inter][hidden]; rows [0, inter) are the gate
 *               projection, rows [inter, 2*inter) the up projection.
 *   w_down:     n_exp matrices [hidden][inter].
 *   x:          device [T][hidden], dtype x_dtype.
 *   topk_ids, topk_w: as for trellis_moe_gemv; topk_w NULL means all ones.
 *   h:          device uint16 (bf16 bits) [T][k][inter], written: for each
 *               live slot, bf16(silu(gate) * up) with silu(z) = z / (1 + e^-z),
 *               rounded to nearest even; zero for empty/skipped slots.
 *   y:          device float [T][hidden], sum over slots of topk_w * W_down h.
 *               The slots' contributions are added into y with device-scope
 *               float atomics, so their order (and the last bits of y) can
 *               differ from call to call; the accuracy bound below holds for
 *               every order.
 * hidden and inter: multiples of 32; T, k limits as for trellis_moe_gemv.
 * Accuracy: as for trellis_moe_gemv, per GEMV; h is rounded to bf16 first.
 */
int trellis_moe_ffn(hipStream_t stream, const trellis_mat_t *w_gate_up, const trellis_mat_t *w_down,
                    const void *x, int32_t x_dtype, const int32_t *topk_ids, const float *topk_w,
                    int32_t T, int32_t k, uint16_t *h, float *y, void *workspace,
                    size_t workspace_bytes);

/*
 * trellis_moe_ffn_timed -- trellis_moe_ffn that also stamps HIP events with
 * the layer kernel's execution, for timing it in place:
 *   events[0] when the kernel starts,
 *   events[1] when it ends
 * (the events are attached to the kernel's dispatch, hipExtLaunchKernel,
 * rather than recorded as separate commands around it, so hipEventElapsedTime
 * between them is the kernel's duration). The whole layer -- routing,
 * activation split, gate_up + SwiGLU, down + combine -- is one persistent
 * kernel. `events` (caller-created hipEvent_t handles) may be NULL, as may
 * either entry. Same arguments, results and errors as trellis_moe_ffn
 * otherwise.
 */
typedef struct ihipEvent_t *hipEvent_t;
int trellis_moe_ffn_timed(hipStream_t stream, const trellis_mat_t *w_gate_up,
                          const trellis_mat_t *w_down, const void *x, int32_t x_dtype,
                          const int32_t *topk_ids, const float *topk_w, int32_t T, int32_t k,
                          uint16_t *h, float *y, void *workspace, size_t workspace_bytes,
                          hipEvent_t *events);

/*
 * trellis_moe_ffn_noalloc -- trellis_moe_ffn for callers that cannot allocate
 * device memory or hand over a workspace: code being captured into a HIP
 * graph, tight serving loops, harnesses that forbid allocation. The
 * workspace is the library's own device array of
 * TRELLIS_NOALLOC_SCRATCH_BYTES bytes, one per device (the current device
 * at the call; `stream` must belong to it), zero-filled when the library is
 * loaded and held until the process ends. Since calls of every shape share
 * it, each call first zeroes the counters and tagged words its shape uses,
 * with a small fill kernel enqueued on `stream` ahead of the layer kernel
 * (no memset node, so the pair can be captured into a graph). The call
 * allocates and frees nothing and synchronises nothing.
 *   Arguments, outputs (h, y), accuracy and the other errors: as for
 *   trellis_moe_ffn.
 *   TRELLIS_EWORKSPACE: the shape needs more than the array holds, i.e.
 *   trellis_moe_ffn_workspace_size(n_exp, hidden, inter, T, k) >
 *   TRELLIS_NOALLOC_SCRATCH_BYTES; nothing is enqueued.
 *   TRELLIS_EHIP: the array's device address could not be obtained.
 * Every call on a device uses that device's one array: calls that overlap in
 * time on one device (on different streams, or from different threads
 * without ordering) race and give wrong results. A wait that times out sets
 * the array's sticky error word (see the workspace note above), after which
 * every later call on that device writes NaN to y until the process ends.
 */
#define TRELLIS_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int trellis_moe_ffn_noalloc(hipStream_t stream, const trellis_mat_t *w_gate_up, const trellis_mat_t *w_down,
                            const void *x, int32_t x_dtype, const int32_t *topk_ids, const float *topk_w,
                            int32_t T, int32_t k, uint16_t *h, float *y);

/*
 * Expand serving mode, second half (HEPH abstract: the expanded MXFP4 weights
 * feed a grouped mixture-of-experts kernel): the same routed GEMV / layer as
 * above, on weights that trellis_decode_expand has already turned into
 * resident MXFP4.
 */
typedef struct {
  const uint8_t *codes;    /* device, [n_mat][rows][cols/2]: E2M1 codes, column 2j in the low
                              nibble of byte j, column 2j+1 in its high nibble (the
                              codes_out of trellis_decode_expand); 16-byte aligned */
  const uint8_t *scales;   /* device, [n_mat][rows][cols/32] UE8M0; 16-byte aligned */
  int32_t n_mat;           /* >= 1 */
  int32_t rows;            /* >= 1, multiple of 16 */
  int32_t cols;            /* >= 32, multiple of 32 */
} trellis_mx_t;

/*
 * trellis_mxfp4_moe_gemv -- trellis_moe_gemv with MXFP4 weights: same
 * arguments, outputs, accuracy bound, workspace (trellis_moe_gemv_workspace_size
 * covers it) and errors, plus EINVAL when codes or scales are not 16-byte
 * aligned.
 */
int trellis_mxfp4_moe_gemv(hipStream_t stream, const trellis_mx_t *w, const void *x, int32_t x_dtype,
                           int32_t x_per_slot, const int32_t *topk_ids, const float *topk_w, int32_t T,
                           int32_t k, float *y, void *workspace, size_t workspace_bytes);

/*
 * trellis_mxfp4_moe_ffn -- trellis_moe_ffn with MXFP4 weights (gate_up
 * [2*inter][hidden] and down [hidden][inter] per expert): same arguments,
 * outputs, workspace (trellis_moe_ffn_workspace_size) and errors, plus EINVAL
 * for misaligned codes or scales.
 */
int trellis_mxfp4_moe_ffn(hipStream_t stream, const trellis_mx_t *w_gate_up, const trellis_mx_t *w_down,
                          const void *x, int32_t x_dtype, const int32_t *topk_ids, const float *topk_w,
                          int32_t T, int32_t k, uint16_t *h, float *y, void *workspace,
                          size_t workspace_bytes);

/*
 * E5M3 block scales (XOR-Trellis article, the paragraph on the grouping
 * format: the paper puts E2M1 elements under E5M3 block scales; it gives no
 * encoding). Reading taken: each scale byte is an unsigned 8-bit float laid
 * out as the upper byte of an IEEE binary16 number without its sign,
 * exponent bits 7..3 with bias 15, mantissa bits 2..0, subnormal
 * (m/8 * 2^-14) at exponent 0, infinity (m = 0) or NaN at exponent 31.
 *
 * trellis_moe_gemv_e5m3 -- trellis_moe_gemv with w->scales read as E5M3
 * instead of UE8M0: same arguments, layout, outputs, workspace
 * (trellis_moe_gemv_workspace_size) and errors. Accuracy: the same bound as
 * trellis_moe_gemv (each scale enters the matrix cores as four exact
 * power-of-two terms). A block whose scale has exponent 31 makes its
 * outputs NaN (the oracle's infinity times a nonzero value is +-inf there).
 */
int trellis_moe_gemv_e5m3(hipStream_t stream, const trellis_mat_t *w, const void *x, int32_t x_dtype,
                          int32_t x_per_slot, const int32_t *topk_ids, const float *topk_w, int32_t T,
                          int32_t k, float *y, void *workspace, size_t workspace_bytes);

/*
 * trellis_moe_ffn_e5m3 -- trellis_moe_ffn with both matrix stacks' scales read
 * as E5M3 (the reading above): same arguments, outputs, workspace
 * (trellis_moe_ffn_workspace_size), accuracy and errors. It runs the general
 * layer kernel at every T.
 */
int trellis_moe_ffn_e5m3(hipStream_t stream, const trellis_mat_t *w_gate_up, const trellis_mat_t *w_down,
                         const void *x, int32_t x_dtype, const int32_t *topk_ids, const float *topk_w,
                         int32_t T, int32_t k, uint16_t *h, float *y, void *workspace,
                         size_t workspace_bytes);

/*
 * Workspace bytes needed by trellis_router_topk: T counters and T * E
 * float64 logits. 0 for E outside 1..1024 or T < 1. Like the layer's
 * workspaces it is zero-filled once before first use; every call leaves
 * the counters zero again.
 */
size_t trellis_router_workspace_size(int32_t E, int32_t T);

/*
 * trellis_router_topk -- the router in front of the layer, so that
 * trellis_moe_ffn can follow it on the same stream with no host round trip.
 * The pages leave routing unspecified; this is the usual mixture-of-experts
 * router: logits[t][e] = sum_h x[t][h] * w_router[e][h]; topk_ids[t] = the k
 * experts with the largest logits, in descending order, the lower id first
 * on equal logits; topk_w[t] = softmax over those k logits.
 *   x:        device, [T][H], fp32 or bf16 (x_dtype), 16-byte aligned.
 *   w_router: device, [E][H] bf16, 16-byte aligned.
 *   topk_ids: device, [T][k] int32 (written); topk_w: device, [T][k] fp32.
 *   workspace: device, 256-byte aligned, trellis_router_workspace_size bytes.
 * Products are exact and sums are float64, so a logit is within a few float64
 * roundings of the exact sum; the softmax is float64, rounded to fp32. Each
 * workgroup computes four experts' logits of one token; the last one of a
 * token to finish picks the top k. Limits: 1 <= E <= 1024,
 * 1 <= k <= min(E, 64), 8 <= H <= 8192 with H % 8 == 0, 1 <= T <= 65535.
 * Errors: ENULL for a NULL pointer; EINVAL for a shape outside the limits, a
 * bad x_dtype or misaligned pointers; EWORKSPACE for a small or misaligned
 * workspace.
 */
int trellis_router_topk(hipStream_t stream, const void *x, int32_t x_dtype, const uint16_t *w_router,
                        int32_t E, int32_t H, int32_t T, int32_t k, int32_t *topk_ids, float *topk_w,
                        void *workspace, size_t workspace_bytes);

/*
 * trellis_moe_ffn_routed -- trellis_router_topk and trellis_moe_ffn for one
 * token (T = 1) in one launch: every workgroup of the single-token layer
 * kernel computes the router itself (the same arithmetic as
 * trellis_router_topk, so the same ids and gate weights bit for bit), then
 * runs the layer (HEPH abstract, fused serving mode; the routing is the
 * usual router, which the pages leave unspecified).
 *   x:           device [1][hidden], fp32 or bf16 (x_dtype), 16-byte aligned.
 *   w_router:    device [E][hidden] bf16, 16-byte aligned (E = w_gate_up->n_mat).
 *   topk_ids_out, topk_w_out: device [1][k] (written): the routing used.
 *   h, y, workspace: as for trellis_moe_ffn (its workspace size for T = 1).
 *   events:      as for trellis_moe_ffn_timed (may be NULL).
 * Limits: the single-token kernel's shapes (hidden and inter multiples of
 * 64, at most 4096, 16-byte aligned streams), E <= 32, 1 <= k <= E,
 * trellis streams under UE8M0 scales. Other shapes get TRELLIS_EINVAL before
 * anything is enqueued: chain trellis_router_topk and trellis_moe_ffn there.
 * Errors otherwise as trellis_moe_ffn.
 */
int trellis_moe_ffn_routed(hipStream_t stream, const trellis_mat_t *w_gate_up, const trellis_mat_t *w_down,
                           const void *x, int32_t x_dtype, const uint16_t *w_router, int32_t k,
                           int32_t *topk_ids_out, float *topk_w_out, uint16_t *h, float *y, void *workspace,
                           size_t workspace_bytes, hipEvent_t *events);

/*
 * Workspace bytes needed by trellis_viterbi_encode for `rows` rows of n
 * positions on the current device: 1 KB per position for each row searched
 * at once (at most 2 per compute unit). 0 for rows < 1 or n < 1, or when
 * the device cannot be queried. The workspace needs no clearing.
 */
size_t trellis_viterbi_workspace_size(int32_t rows, int32_t n);

/*
 * trellis_viterbi_encode -- the encoder's symbol search (XOR-Trellis news
 * article, aimodeling.com, bullet "Curvature-aware Viterbi objective"): for
 * each row, the branch-symbol sequence that starts from state 0 and
 * minimises sum_k d[k] * (target[k] - value_k)^2, where value_k is the
 * palette value the decoder above gives position k (at scale 1, no block
 * scale).
 *   target:   device, [rows][n] float64, finite.
 *   d:        device, [rows][n] float64 per-position weights (the diagonal
 *             curvature factor), or NULL for all ones.
 *   syms_out: device, [rows][n] bytes, one symbol (0..3) per position.
 *   cost_out: device, [rows] float64, the minimum of the objective.
 * Arithmetic is float64 with every operation rounded (no fused multiply-add):
 * each step adds (d * err) * err, err = target - value, to the path cost, in
 * position order. Where several paths tie, the one kept at each position is
 * the one through the smaller predecessor, and the path ends in the smallest
 * final state. One workgroup searches one row over the 4096 histories of six
 * symbols (the value depends on the current symbol and the six before it).
 * Errors: ENULL for a NULL target, syms_out, cost_out or workspace; EINVAL for
 * rows or n < 1 or float64 arrays not 8-byte aligned; EWORKSPACE for a
 * workspace that is not 256-byte aligned or smaller than
 * trellis_viterbi_workspace_size(rows, n).
 */
int trellis_viterbi_encode(hipStream_t stream, const double *target, const double *d, int32_t rows,
                           int32_t n, uint8_t *syms_out, double *cost_out, void *workspace,
                           size_t workspace_bytes);

/*
 * trellis_read_bandwidth -- a measurement reference, not part of the method:
 * reads the `bytes` bytes at `buf` once (16-byte vector loads, every byte
 * read exactly once) and XORs all their 32-bit words, per workgroup, into
 * one of the 256 words of sink (atomically; the caller zero-fills sink to
 * check the result: the XOR of the 256 words is the XOR of every word of
 * buf). Timing it over the bytes one layer call reads gives the practical
 * streaming-read rate of HBM at that size, which the layer's
 * compressed-weight GB/s is compared with beside the 8 TB/s peak.
 *   buf:  device, 16-byte aligned; bytes: a multiple of 4.
 *   sink: device uint32[256].
 * Errors: ENULL for a NULL pointer, EINVAL for misalignment, EHIP for a
 * launch failure.
 */
int trellis_read_bandwidth(hipStream_t stream, const void *buf, size_t bytes, uint32_t *sink);

#ifdef __cplusplus
}
#endif

#endif /* TRELLIS_H_ */

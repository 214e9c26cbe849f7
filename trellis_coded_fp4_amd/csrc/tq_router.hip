// tq_router.hip -- the router in front of the mixture-of-experts layer on
// gfx950: logits = x . W_r^T per token, its k largest logits in descending
// order (ties to the lower expert id), and gate weights = softmax over those
// k logits. The pages leave routing unspecified; this is the usual router,
// and its outputs are exactly the topk_ids / topk_w the layer takes, so the
// two launches chain on one stream with no host round trip.
//
// One workgroup per token. The token's activations are staged in LDS as
// fp32; each wave takes experts e = wave, wave + 4, ..., its lanes 8
// consecutive hidden positions per 16-byte load of the bf16 router row.
// Products of an fp32 (or bf16) activation and a bf16 weight are exact in
// fp64, and the sums are fp64 (lane-sequential, then a fixed butterfly over
// the wave), so a logit is within a few units of the fp64 rounding of the
// exact sum. Top-k: wave 0, k rounds of a wave-wide argmax over the logits
// in LDS (largest value, lower id on ties). Softmax in fp64, rounded to fp32.
#include <hip/hip_runtime.h>

#include <math.h>

#include "tq_common.h"

namespace tq {

constexpr int kRThreads = 256;
constexpr int kRMaxE = 1024;
constexpr int kRMaxK = 64;
constexpr int kRMaxH = 8192;

struct RouterArgs {
  const void *x;        // [T][H] fp32 or bf16
  int x_bf16;
  const uint16_t *w;    // [E][H] bf16
  int E, H, T, k;
  int32_t *ids;         // [T][k]
  float *gw;            // [T][k]
};

__global__ void __launch_bounds__(kRThreads) k_router(RouterArgs a) {
  __shared__ float xs[kRMaxH];
  __shared__ double lg[kRMaxE];
  __shared__ int pick[kRMaxK];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  for (int h = tid; h < a.H; h += kRThreads)
    xs[h] = a.x_bf16 ? bf16_to_f32(((const uint16_t *)a.x)[(size_t)t * a.H + h])
                     : ((const float *)a.x)[(size_t)t * a.H + h];
  __syncthreads();

  for (int e = wave; e < a.E; e += kRThreads / 64) {
    const uint4 *row = (const uint4 *)(a.w + (size_t)e * a.H);
    double s = 0.0;
    for (int q = lane; q < a.H / 8; q += 64) {
      const uint4 u = row[q];
      const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s += (double)xs[8 * q + 2 * i] * (double)bf16_to_f32((uint16_t)(wv[i] & 0xFFFFu));
        s += (double)xs[8 * q + 2 * i + 1] * (double)bf16_to_f32((uint16_t)(wv[i] >> 16));
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) lg[e] = s;
  }
  __syncthreads();

  if (wave == 0) {
    // lane l owns experts l + 64 i; bit i of `mine` marks the picked ones
    uint32_t mine = 0u;
    for (int j = 0; j < a.k; ++j) {
      double bv = -INFINITY;
      int be = -1;
      for (int e = lane, i = 0; e < a.E; e += 64, ++i)
        if (!((mine >> i) & 1u) && (be < 0 || lg[e] > bv)) { bv = lg[e]; be = e; }
      // butterfly: every lane ends with the same (largest, lowest id) pair
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const double ov = __shfl_xor(bv, off);
        const int oe = __shfl_xor(be, off);
        if (oe >= 0 && (be < 0 || ov > bv || (ov == bv && oe < be))) { bv = ov; be = oe; }
      }
      if ((be & 63) == lane) mine |= 1u << (be >> 6);
      if (lane == 0) pick[j] = be;
    }
    if (lane == 0) {
      const double m = lg[pick[0]];
      double sum = 0.0;
      for (int j = 0; j < a.k; ++j) sum += exp(lg[pick[j]] - m);
      for (int j = 0; j < a.k; ++j) {
        a.ids[(size_t)t * a.k + j] = pick[j];
        a.gw[(size_t)t * a.k + j] = (float)(exp(lg[pick[j]] - m) / sum);
      }
    }
  }
}

}  // namespace tq

using namespace tq;

extern "C" int trellis_router_topk(hipStream_t stream, const void *x, int32_t x_dtype, const uint16_t *w_router,
                                   int32_t E, int32_t H, int32_t T, int32_t k, int32_t *topk_ids, float *topk_w) {
  if (!x || !w_router || !topk_ids || !topk_w) return TRELLIS_ENULL;
  if (x_dtype != TRELLIS_F32 && x_dtype != TRELLIS_BF16) return TRELLIS_EINVAL;
  if (E < 1 || E > kRMaxE || k < 1 || k > E || k > kRMaxK || T < 1 || H < 8 || H > kRMaxH || H % 8)
    return TRELLIS_EINVAL;
  if ((uintptr_t)w_router % 16 || (uintptr_t)x % (x_dtype == TRELLIS_BF16 ? 2 : 4) || (uintptr_t)topk_ids % 4 ||
      (uintptr_t)topk_w % 4)
    return TRELLIS_EINVAL;
  RouterArgs a{x, x_dtype == TRELLIS_BF16, w_router, E, H, T, k, topk_ids, topk_w};
  hipLaunchKernelGGL(k_router, dim3((unsigned)T), dim3(kRThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? TRELLIS_OK : TRELLIS_EHIP;
}

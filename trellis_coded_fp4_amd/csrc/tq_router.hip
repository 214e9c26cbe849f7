// tq_router.hip -- the router in front of the mixture-of-experts layer on
// gfx950: logits = x . W_r^T per token, its k largest logits in descending
// order (ties to the lower expert id), and gate weights = softmax over those
// k logits. The pages leave routing unspecified; this is the usual router,
// and its outputs are exactly the topk_ids / topk_w the layer takes, so the
// two launches chain on one stream with no host round trip.
//
// Each workgroup computes four experts' logits of one token (one per wave),
// so a token's router rows are read by ceil(E / 4) workgroups at once. A
// wave issues all its 16-byte loads of the bf16 router row before it
// multiplies (8 hidden positions per load, up to 16 loads per lane); the
// token's activations are staged in LDS as fp32. Products of an fp32 (or
// bf16) activation and a bf16 weight are exact in fp64, and the sums are
// fp64 (lane-sequential, then a fixed butterfly over the wave), so a logit
// is within a few units of the fp64 rounding of the exact sum. The logits
// go to the workspace with device-coherent stores; the last workgroup of a
// token to count (a per-token counter it clears again) reads them back and
// picks the top k in wave 0: k rounds of a wave-wide argmax (largest value,
// lower id on ties). Softmax in fp64 (one exp per lane, the sum a wave
// butterfly), rounded to fp32.
#include <hip/hip_runtime.h>

#include <math.h>

#include "tq_common.h"

namespace tq {

constexpr int kRThreads = 256;
constexpr int kRExpertsPerBlock = kRThreads / 64;
constexpr int kRMaxE = 1024;
constexpr int kRMaxK = 64;
constexpr int kRMaxH = 8192;
constexpr int kRLoads = kRMaxH / 8 / 64;   // 16-byte loads per lane, at most
constexpr int kRXLoads = kRMaxH * 4 / 16 / kRThreads;   // 16-byte loads of x per thread, at most
constexpr int kRPerLane = kRMaxE / 64;     // logits per lane in the top-k wave

struct RouterArgs {
  const void *x;        // [T][H] fp32 or bf16
  int x_bf16;
  const uint16_t *w;    // [E][H] bf16
  int E, H, T, k;
  int32_t *ids;         // [T][k]
  float *gw;            // [T][k]
  int *cnt;             // workspace: [T] counters
  double *lg;           // workspace: [T][E] logits
};

__global__ void __launch_bounds__(kRThreads) k_router(RouterArgs a) {
  __shared__ float xs[kRMaxH];
  __shared__ int last;
  const int t = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = blockIdx.x * kRExpertsPerBlock + wave;
  const int nq = a.H / 8;

  // this wave's router row, all loads in flight before anything waits
  uint4 r[kRLoads];
  const uint4 *row = (const uint4 *)(a.w + (size_t)min(e, a.E - 1) * a.H);
#pragma unroll
  for (int i = 0; i < kRLoads; ++i) r[i] = row[min(lane + 64 * i, nq - 1)];
  {
    // the token's activations, 16 bytes per load, all in flight at once
    const int nx = a.H * (a.x_bf16 ? 2 : 4) / 16;
    const uint4 *xr = (const uint4 *)((const uint8_t *)a.x + (size_t)t * a.H * (a.x_bf16 ? 2 : 4));
    uint4 xv[kRXLoads];
#pragma unroll
    for (int i = 0; i < kRXLoads; ++i) xv[i] = xr[min(tid + kRThreads * i, nx - 1)];
#pragma unroll
    for (int i = 0; i < kRXLoads; ++i) {
      const int c = tid + kRThreads * i;
      if (c < nx) {
        const uint32_t u[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
        if (a.x_bf16) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            xs[8 * c + 2 * j] = bf16_to_f32((uint16_t)(u[j] & 0xFFFFu));
            xs[8 * c + 2 * j + 1] = bf16_to_f32((uint16_t)(u[j] >> 16));
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) xs[4 * c + j] = __uint_as_float(u[j]);
        }
      }
    }
  }
  __syncthreads();

  if (e < a.E) {
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < kRLoads; ++i) {
      const int q = lane + 64 * i;
      if (q < nq) {
        const uint32_t wv[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s += (double)xs[8 * q + 2 * j] * (double)bf16_to_f32((uint16_t)(wv[j] & 0xFFFFu));
          s += (double)xs[8 * q + 2 * j + 1] * (double)bf16_to_f32((uint16_t)(wv[j] >> 16));
        }
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0)
      __hip_atomic_store((uint64_t *)(a.lg + (size_t)t * a.E + e), (uint64_t)__double_as_longlong(s),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // the stores are complete device-wide before the workgroup counts
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(a.cnt + t, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = old == (int)gridDim.x - 1;
  }
  __syncthreads();
  if (!last || wave != 0) return;

  // lane l owns experts l + 64 i: their logits, all loaded at once; bit i of
  // `mine` marks the picked ones
  const double *lt = a.lg + (size_t)t * a.E;
  double lv[kRPerLane];
#pragma unroll
  for (int i = 0; i < kRPerLane; ++i)
    lv[i] = __longlong_as_double((long long)__hip_atomic_load(
        (const uint64_t *)(lt + min(lane + 64 * i, a.E - 1)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  uint32_t mine = 0u;
  int my_pick = 0;
  double my_val = 0.0, top = 0.0;
  for (int j = 0; j < a.k; ++j) {
    double bv = -INFINITY;
    int be = -1;
#pragma unroll
    for (int i = 0; i < kRPerLane; ++i) {
      const int x = lane + 64 * i;
      if (x < a.E && !((mine >> i) & 1u) && (be < 0 || lv[i] > bv)) { bv = lv[i]; be = x; }
    }
    // butterfly: every lane ends with the same (largest, lowest id) pair
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const double ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      if (oe >= 0 && (be < 0 || ov > bv || (ov == bv && oe < be))) { bv = ov; be = oe; }
    }
    if ((be & 63) == lane) mine |= 1u << (be >> 6);
    // every lane holds the round's pick: lane j keeps pick j, all keep the first
    if (lane == j) {
      my_pick = be;
      my_val = bv;
    }
    if (j == 0) top = bv;
  }
  // softmax: lane j < k takes pick j (one exp each), the sum is a wave
  // butterfly (k <= 64)
  const double ex = lane < a.k ? exp(my_val - top) : 0.0;
  double sum = ex;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane < a.k) {
    a.ids[(size_t)t * a.k + lane] = my_pick;
    a.gw[(size_t)t * a.k + lane] = (float)(ex / sum);
  }
  // every workgroup of this token has counted: clear for the next call
  if (lane == 0) __hip_atomic_store(a.cnt + t, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

static size_t router_cnt_bytes(int T) { return ((size_t)T * sizeof(int) + 255) & ~(size_t)255; }

}  // namespace tq

using namespace tq;

extern "C" size_t trellis_router_workspace_size(int32_t E, int32_t T) {
  if (E < 1 || E > kRMaxE || T < 1) return 0;
  return router_cnt_bytes(T) + (size_t)T * E * sizeof(double);
}

extern "C" int trellis_router_topk(hipStream_t stream, const void *x, int32_t x_dtype, const uint16_t *w_router,
                                   int32_t E, int32_t H, int32_t T, int32_t k, int32_t *topk_ids, float *topk_w,
                                   void *workspace, size_t workspace_bytes) {
  if (!x || !w_router || !topk_ids || !topk_w || !workspace) return TRELLIS_ENULL;
  if (x_dtype != TRELLIS_F32 && x_dtype != TRELLIS_BF16) return TRELLIS_EINVAL;
  if (E < 1 || E > kRMaxE || k < 1 || k > E || k > kRMaxK || T < 1 || T > 65535 || H < 8 || H > kRMaxH || H % 8)
    return TRELLIS_EINVAL;
  if ((uintptr_t)w_router % 16 || (uintptr_t)x % 16 || (uintptr_t)topk_ids % 4 || (uintptr_t)topk_w % 4)
    return TRELLIS_EINVAL;
  if ((uintptr_t)workspace % 256) return TRELLIS_EWORKSPACE;
  if (workspace_bytes < trellis_router_workspace_size(E, T)) return TRELLIS_EWORKSPACE;
  RouterArgs a{x, x_dtype == TRELLIS_BF16, w_router, E, H, T, k, topk_ids, topk_w, (int *)workspace,
               (double *)((uint8_t *)workspace + router_cnt_bytes(T))};
  const dim3 grid((unsigned)((E + kRExpertsPerBlock - 1) / kRExpertsPerBlock), (unsigned)T);
  hipLaunchKernelGGL(k_router, grid, dim3(kRThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? TRELLIS_OK : TRELLIS_EHIP;
}

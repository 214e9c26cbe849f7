// tq_viterbi.hip -- the encoder's symbol search on gfx950: a curvature-aware
// Viterbi search (XOR-Trellis news article, aimodeling.com, bullet
// "Curvature-aware Viterbi objective") that picks, for each row, the symbol
// sequence from state 0 minimising sum_k d[k] * (target[k] - value_k)^2,
// values at scale 1.
//
// The value at a position depends on the state's bits 0..13 only (the
// decoder's masks 0x1089, 0x2112, 0x0A24, 0x2441 stop at bit 13): the current
// symbol and the six before it. The search therefore runs over the 4096
// histories of six symbols, four branches each: history h and symbol b lead
// to h' = ((h << 2) | b) & 0xFFF through the 14-bit state (h << 2 | b). The
// four predecessors of h' are (h' >> 2) | (t << 10), t = 0..3, and the four
// successors h' = (m << 2) | b of one m = h' >> 2 share them, so a thread
// owning m reads four costs and produces four.
//
// Arithmetic: fp64, each candidate cost formed as cost + (d * err) * err with
// err = target - value, rounded at every operation (no contraction), in
// position order. Ties keep the smaller predecessor (smaller t), and the
// final history with the smallest cost (smaller index on ties) ends the path.
//
// Layout: one workgroup per row (rows beyond the grid loop), 256 threads;
// thread i owns m = i + 256 j (j = 0..3), i.e. histories 4m .. 4m + 3. The
// costs of one position live in LDS (two 32 KB buffers). Each position's
// choices (2 bits per history) are one 32-bit word per thread, written to
// the workspace, 1 KB per position; the traceback stages them back through
// LDS 64 positions at a time.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <math.h>
#include <string.h>

#include "tq_common.h"

namespace tq {

constexpr int kVThreads = 256;
constexpr int kVHist = 4096;     // histories of six symbols
constexpr int kVChunk = 256;     // positions of target / d staged in LDS at a time
constexpr int kVTb = 64;         // positions of choices staged per traceback chunk
constexpr int kVBlocksPerCu = 2; // LDS: 68 KB per workgroup

struct VitArgs {
  const double *target;   // [rows][n]
  const double *d;        // [rows][n] or null (all ones)
  uint8_t *syms;          // [rows][n]
  double *cost;           // [rows]
  uint32_t *bp;           // [grid][n][kVThreads] choice words
  int rows, n;
};

// The palette value of a 14-bit state (current symbol in bits 0..1), times 2
// so that it is an integer.
__device__ __forceinline__ int vit_value2(uint32_t s) {
  const int p0 = __popc(s & 0x1089u) & 1, p1 = __popc(s & 0x2112u) & 1;
  const int q0 = __popc(s & 0x0A24u) & 1, q1 = __popc(s & 0x2441u) & 1;
  const int palette = p0 | (p1 << 1);
  const int entry = (int)(s & 3u) ^ (q0 | (q1 << 1));
  // P0..P3 times 2; P3's -0 becomes 0 (the sign of a zero value does not
  // change (target - value)^2)
  const int pal2[16] = {-12, -3, 0, 4, -8, -2, 1, 6, -6, -1, 2, 8, -4, 0, 3, 12};
  return pal2[palette * 4 + entry];
}

__global__ void __launch_bounds__(kVThreads) k_viterbi(VitArgs a) {
#pragma clang fp contract(off)
  __shared__ double cst[2][kVHist];
  __shared__ double tt[kVChunk], dd[kVChunk];
  __shared__ double best_c[kVThreads];
  __shared__ int best_h[kVThreads];
  const int tid = threadIdx.x;
  uint32_t *bpw = a.bp + (size_t)blockIdx.x * a.n * kVThreads;

  // the values this thread meets, fixed for the whole search
  double v[4][4][4];   // [j][t][b]
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        v[j][t][b] = 0.5 * (double)vit_value2(((uint32_t)t << 12) | ((uint32_t)(tid + 256 * j) << 2) | (uint32_t)b);

  for (int row = blockIdx.x; row < a.rows; row += gridDim.x) {
    const double *tr = a.target + (size_t)row * a.n;
    const double *dr = a.d ? a.d + (size_t)row * a.n : nullptr;
    for (int i = tid; i < kVHist; i += kVThreads) cst[0][i] = i == 0 ? 0.0 : INFINITY;
    int cur = 0;
    for (int k0 = 0; k0 < a.n; k0 += kVChunk) {
      __syncthreads();   // the previous chunk's reads of tt / dd are done
      if (k0 + tid < a.n) {
        tt[tid] = tr[k0 + tid];
        dd[tid] = dr ? dr[k0 + tid] : 1.0;
      }
      __syncthreads();
      const int kn = min(kVChunk, a.n - k0);
      for (int kk = 0; kk < kn; ++kk) {
        const double tk = tt[kk], dk = dd[kk];
        const double *ci = cst[cur];
        double *co = cst[cur ^ 1];
        uint32_t word = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int m = tid + 256 * j;
          double c[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) c[t] = ci[m | (t << 10)];
          double o[4];
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            double best = 0.0;
            uint32_t bt = 0u;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const double e = tk - v[j][t][b];
              const double q = c[t] + (dk * e) * e;
              if (t == 0 || q < best) {
                best = q;
                bt = (uint32_t)t;
              }
            }
            o[b] = best;
            word |= bt << (2 * (4 * j + b));
          }
          double2 *dst = (double2 *)(co + 4 * m);
          dst[0] = make_double2(o[0], o[1]);
          dst[1] = make_double2(o[2], o[3]);
        }
        bpw[(size_t)(k0 + kk) * kVThreads + tid] = word;
        cur ^= 1;
        __syncthreads();
      }
    }

    // the cheapest final history (smaller index on ties)
    {
      double bc = INFINITY;
      int bh = -1;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int h = 4 * (tid + 256 * j) + b;
          const double c = cst[cur][h];
          if (bh < 0 || c < bc) { bc = c; bh = h; }
        }
      best_c[tid] = bc;
      best_h[tid] = bh;
    }
    __syncthreads();
    int h = 0;
    if (tid == 0) {
      double bc = best_c[0];
      h = best_h[0];
      for (int i = 1; i < kVThreads; ++i) {
        const double c = best_c[i];
        if (c < bc || (c == bc && best_h[i] < h)) { bc = c; h = best_h[i]; }
      }
      a.cost[row] = bc;
    }

    // traceback, kVTb positions of choice words at a time through LDS
    uint32_t *stage = (uint32_t *)&cst[0][0];   // kVTb x kVThreads words (64 KB)
    uint8_t *so = a.syms + (size_t)row * a.n;
    for (int k1 = a.n; k1 > 0; k1 -= kVTb) {
      const int k0 = max(0, k1 - kVTb);
      __syncthreads();   // the last chunk's (or the argmin's) readers are done
      {
        // (k1 - k0) * 64 16-byte groups, all loads issued before the stores;
        // past the chunk a lane re-reads its last group and stores nothing
        constexpr int kPer = kVTb * kVThreads / 4 / kVThreads;
        const int ng = (k1 - k0) * (kVThreads / 4);
        const uint4 *src = (const uint4 *)(bpw + (size_t)k0 * kVThreads);
        uint4 r[kPer];
#pragma unroll
        for (int q = 0; q < kPer; ++q) r[q] = src[min(tid + kVThreads * q, ng - 1)];
#pragma unroll
        for (int q = 0; q < kPer; ++q)
          if (tid + kVThreads * q < ng) ((uint4 *)stage)[tid + kVThreads * q] = r[q];
      }
      __syncthreads();
      if (tid == 0) {
        for (int k = k1 - 1; k >= k0; --k) {
          const int m = h >> 2, b = h & 3;
          so[k] = (uint8_t)b;
          const uint32_t w = stage[(k - k0) * kVThreads + (m & 255)];
          const int t = (int)(w >> (2 * (4 * (m >> 8) + b))) & 3;
          h = m | (t << 10);
        }
      }
    }
    __syncthreads();   // before the next row overwrites the costs
  }
}

// Grid for `rows` rows on the current device (gfx950 only).
static int vit_grid(int rows, int *grid) {
  static int arch_ok[64], n_cu[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return TRELLIS_EHIP;
  if (arch_ok[dev] == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return TRELLIS_EHIP;
    n_cu[dev] = p.multiProcessorCount;
    arch_ok[dev] = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  }
  if (arch_ok[dev] < 0) return TRELLIS_EDEVICE;
  *grid = std::min(rows, std::max(1, n_cu[dev]) * kVBlocksPerCu);
  return TRELLIS_OK;
}

}  // namespace tq

using namespace tq;

extern "C" size_t trellis_viterbi_workspace_size(int32_t rows, int32_t n) {
  if (rows < 1 || n < 1) return 0;
  int grid = 0;
  if (vit_grid(rows, &grid) != TRELLIS_OK) return 0;
  return (size_t)grid * (size_t)n * kVThreads * sizeof(uint32_t);
}

extern "C" int trellis_viterbi_encode(hipStream_t stream, const double *target, const double *d, int32_t rows,
                                      int32_t n, uint8_t *syms_out, double *cost_out, void *workspace,
                                      size_t workspace_bytes) {
  if (!target || !syms_out || !cost_out || !workspace) return TRELLIS_ENULL;
  if (rows < 1 || n < 1) return TRELLIS_EINVAL;
  if ((uintptr_t)target % 8 || (d && (uintptr_t)d % 8) || (uintptr_t)cost_out % 8) return TRELLIS_EINVAL;
  if ((uintptr_t)workspace % 256) return TRELLIS_EWORKSPACE;
  int grid = 0;
  const int rc = vit_grid(rows, &grid);
  if (rc != TRELLIS_OK) return rc;
  if (workspace_bytes < (size_t)grid * (size_t)n * kVThreads * sizeof(uint32_t)) return TRELLIS_EWORKSPACE;
  VitArgs a{target, d, syms_out, cost_out, (uint32_t *)workspace, rows, n};
  hipLaunchKernelGGL(k_viterbi, dim3((unsigned)grid), dim3(kVThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? TRELLIS_OK : TRELLIS_EHIP;
}

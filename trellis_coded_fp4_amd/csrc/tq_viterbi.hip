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
// position order. Costs are never NaN, so the minimum of the four is exact;
// ties keep the smaller predecessor (the smallest t whose cost equals the
// minimum), and the final history with the smallest cost (smaller index on
// ties) ends the path.
//
// Work split: the palette and entry of the state (t << 12) | (m << 2) | b
// depend on m only through four parities of its bits (m1^m5, m2^m6,
// m0^m3^m7^m9, m4^m8: the m-part of the decoder's masks), the "class" of m.
// Each of the 16 classes holds 64 values of m. Wave w, slot j (j = 0..3)
// takes the 64 m of class 4w + j, one per lane, so in every candidate the
// palette entry is known when the code is compiled (one copy of the step per
// wave index). Per position a thread forms the 16 distortion terms
// (d * err) * err once, one per palette entry, and each candidate is then a
// single add to the predecessor's cost: the same operations and roundings as
// forming err per candidate.
//
// Layout: one workgroup per row (rows beyond the grid loop), 256 threads,
// 16 histories 4m .. 4m + 3 per thread. The costs of one position live in
// LDS (two 32 KB buffers). Each position's choices (2 bits per history) are
// one 32-bit word per thread, written to the workspace, 1 KB per position;
// the traceback stages them back through LDS 64 positions at a time.
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

// Palette values times 2 (integers), indexed palette * 4 + entry; P3's -0
// becomes 0 (the sign of a zero value does not change (target - value)^2).
__constant__ int kVPal2[16] = {-12, -3, 0, 4, -8, -2, 1, 6, -6, -1, 2, 8, -4, 0, 3, 12};

// Palette * 4 + entry of the state (t << 12) | (m << 2) | b for m of class c
// (bit 0: m1^m5, bit 1: m2^m6, bit 2: m0^m3^m7^m9, bit 3: m4^m8).
constexpr int vit_index(int c, int t, int b) {
  const int b0 = b & 1, b1 = b >> 1, t0 = t & 1, t1 = t >> 1;
  const int p0 = b0 ^ (c & 1) ^ t0, p1 = b1 ^ ((c >> 1) & 1) ^ t1;
  const int q0 = (c >> 2) & 1, q1 = b0 ^ ((c >> 3) & 1) ^ t1;
  return (p0 | (p1 << 1)) * 4 + (b ^ (q0 | (q1 << 1)));
}

// The m of class c at lane f: f's bits are m3, m5, m6, m7, m8, m9, and the
// class fixes m1, m2, m4 and m0.
__device__ __forceinline__ int vit_m(int c, int f) {
  const int m3 = f & 1, m5 = (f >> 1) & 1, m6 = (f >> 2) & 1, m7 = (f >> 3) & 1, m8 = (f >> 4) & 1,
            m9 = (f >> 5) & 1;
  const int m1 = (c & 1) ^ m5, m2 = ((c >> 1) & 1) ^ m6, m0 = ((c >> 2) & 1) ^ m3 ^ m7 ^ m9,
            m4 = ((c >> 3) & 1) ^ m8;
  return m0 | (m1 << 1) | (m2 << 2) | (m3 << 3) | (m4 << 4) | (m5 << 5) | (m6 << 6) | (m7 << 7) | (m8 << 8) |
         (m9 << 9);
}

// Thread and bit of history h's choice in a position's 256 words.
__device__ __forceinline__ void vit_owner(int h, int *thread, int *shift) {
  const int m = h >> 2, b = h & 3;
  const int c = (((m >> 1) ^ (m >> 5)) & 1) | ((((m >> 2) ^ (m >> 6)) & 1) << 1) |
                ((((m >> 0) ^ (m >> 3) ^ (m >> 7) ^ (m >> 9)) & 1) << 2) | ((((m >> 4) ^ (m >> 8)) & 1) << 3);
  const int f = ((m >> 3) & 1) | (((m >> 5) & 1) << 1) | (((m >> 6) & 1) << 2) | (((m >> 7) & 1) << 3) |
                (((m >> 8) & 1) << 4) | (((m >> 9) & 1) << 5);
  *thread = (c >> 2) * 64 + f;
  *shift = 2 * (4 * (c & 3) + b);
}

// One position for a thread of wave W: candidates from the costs ci, the
// cheapest of each history's four into co, the choices returned as a word.
template <int W>
__device__ __forceinline__ uint32_t vit_step(const double *ci, double *co, const int (&m)[4], const double (&D)[16]) {
  uint32_t word = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    constexpr int kC0 = 4 * W;
    double c[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) c[t] = ci[m[j] | (t << 10)];
    double o[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      double q[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) q[t] = c[t] + D[vit_index(kC0 + j, t, b)];
      // the cheapest of the four, and the smallest t that reaches it
      const double best = fmin(fmin(q[0], q[1]), fmin(q[2], q[3]));
      const int sh = 2 * (4 * j + b);
      uint32_t bits = q[2] == best ? 2u << sh : 3u << sh;
      bits = q[1] == best ? 1u << sh : bits;
      bits = q[0] == best ? 0u : bits;
      o[b] = best;
      word |= bits;
    }
    double2 *dst = (double2 *)(co + 4 * m[j]);
    dst[0] = make_double2(o[0], o[1]);
    dst[1] = make_double2(o[2], o[3]);
  }
  return word;
}

__global__ void __launch_bounds__(kVThreads) k_viterbi(VitArgs a) {
#pragma clang fp contract(off)
  __shared__ double cst[2][kVHist];
  __shared__ double tt[kVChunk], dd[kVChunk];
  __shared__ double best_c[kVThreads];
  __shared__ int best_h[kVThreads];
  const int tid = threadIdx.x;
  uint32_t *bpw = a.bp + (size_t)blockIdx.x * a.n * kVThreads;

  // this thread's four m (class 4 * wave + j, lane = free bits) and the
  // palette values, times 2
  const int wave = tid >> 6, lane = tid & 63;
  int m[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) m[j] = vit_m(4 * wave + j, lane);
  double pv[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) pv[e] = 0.5 * (double)kVPal2[e];

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
        // the distortion of each palette entry at this position
        double D[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const double er = tk - pv[e];
          D[e] = (dk * er) * er;
        }
        uint32_t word;
        switch (wave) {   // uniform over the wave
          case 0: word = vit_step<0>(ci, co, m, D); break;
          case 1: word = vit_step<1>(ci, co, m, D); break;
          case 2: word = vit_step<2>(ci, co, m, D); break;
          default: word = vit_step<3>(ci, co, m, D); break;
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
          const int h = 4 * m[j] + b;
          const double c = cst[cur][h];
          if (bh < 0 || c < bc || (c == bc && h < bh)) { bc = c; bh = h; }
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
          int owner, shift;
          vit_owner(h, &owner, &shift);
          so[k] = (uint8_t)(h & 3);
          const uint32_t w = stage[(k - k0) * kVThreads + owner];
          const int t = (int)(w >> shift) & 3;
          h = (h >> 2) | (t << 10);
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

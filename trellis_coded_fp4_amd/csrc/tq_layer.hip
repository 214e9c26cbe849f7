// tq_layer.hip -- fused trellis-decode mixture-of-experts layer on gfx950.
//
// HEPH abstract (ICLR 2027 submission page): in "fused" serving the
// compressed streams stay resident and every weight is decoded inside the
// grouped-MoE kernel on each forward pass. Here the decoded E2M1 nibbles go
// straight into the FP4 x FP8 block-scaled matrix cores, with the weights'
// UE8M0 exponents as the A scales, at every batch size: the vector ALUs do
// the decode, the matrix cores the multiply-accumulate.
//
// One persistent launch per call. Workgroups take work items round-robin:
//   prep items     one activation vector each: split into two FP8 E4M3 terms
//                  (hi + lo, UE8M0 scale per 32) in matrix-core B layout,
//                  optionally pre-multiplied by the slot's gate weight;
//                  bookkeeping for dead (empty / out-of-range) slots.
//   stage-1 items  one active expert x 64 output rows; columns = the slots
//                  routed to the expert. Epilogue: plain per-slot output, or
//                  SwiGLU over 32 gate rows and the matching 32 up rows,
//                  writing h (bf16) and its FP8 hi/lo copy (gate weight
//                  folded in) for stage 2.
//   stage-2 items  16 output rows summed over all active experts (one expert
//                  per wave at a time); columns = tokens. Deterministic, no
//                  atomics on outputs.
// Stage-1 items wait for all prep items, stage-2 items for all stage-1 items
// (or prep items when there is no stage 1). Every item issues all of its
// weight loads before it waits. Cross-workgroup data (activation splits, h)
// is written with device-coherent stores and read with device-coherent
// loads, so a dependency costs a store-completion wait and a counter, not a
// cache writeback or invalidate. The grid never exceeds the co-resident
// workgroup count, so every wait is for running work; waits are bounded and
// set an error word on timeout. A workgroup publishes its finished prep and
// stage-1 items in one count when it moves on; the last workgroup out
// publishes the status words and clears the counters.
//
// Weight streaming: a wave owns one 16-row tile over the full K. Lane
// (row i, lane-group g) loads "piece" j = 16 bytes = blocks 8j+2g, 8j+2g+1 of
// its row, and feeds them to matrix-core steps 2j and 2j+1 as K-block g (the
// activations are laid out to match). A wave instruction reads 16 rows x 64
// contiguous bytes; all pieces of a tile (up to 16, K <= 4096 per pass) are
// issued at once. The decoder history of a block is the word before it: from
// the neighbouring lane-group's piece via ds_bpermute, or the previous piece.
// Activation columns are staged in LDS before the matrix-core loop.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>

#include "tq_common.h"

namespace tq {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxT = 32;
constexpr int kMaxK = 32;
constexpr int kMaxSlots = 1024;
constexpr int kMaxExperts = 1024;
constexpr int kPieceMax = 16;               // pieces per pass: 16 x 256 weights
constexpr unsigned kSpinLimit = 1u << 20;   // polls (device-coherent load + sleep)
constexpr int kBBytes = 32 * 1024;          // LDS for staged activation columns (codes)
constexpr int kBScaleBytes = kBBytes / 32;  // and their UE8M0 scales

enum { MODE_FFN = 0, MODE_SLOTS = 1, MODE_COMBINE = 2 };

// int words at the start of the workspace
enum {
  ST_SKIPPED = 0,   // public: slots skipped (expert id >= n_exp) by the last call
  ST_ERROR = 1,     // public: nonzero if a wait timed out in the last call
  SY_PREP = 8,      // working counters, zero between calls
  SY_S1 = 9,
  SY_EXIT = 10,
  SY_SKIP = 11,
  SY_ERR = 12,
};

struct Layout {
  size_t sync, xq, xs, hq, hs, total;
};

static inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

static Layout make_layout(int x_vecs, int x_cols, int h_vecs, int h_cols) {
  Layout L;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align256(o + bytes); return r; };
  L.sync = take(256);
  const size_t xs = (size_t)steps_for_blocks(x_cols / 32);
  L.xq = take((size_t)x_vecs * 2 * xs * 128);
  L.xs = take((size_t)x_vecs * 2 * xs * 4);
  const size_t hs = h_cols ? (size_t)steps_for_blocks(h_cols / 32) : 0;
  L.hq = take((size_t)h_vecs * 2 * hs * 128);
  L.hs = take((size_t)h_vecs * 2 * hs * 4);
  L.total = o;
  return L;
}

struct LayerArgs {
  int mode;
  const uint32_t *w1; const uint8_t *s1; int rows1, cols1;   // stage-1 matrices
  const uint32_t *w2; const uint8_t *s2; int rows2, cols2;   // stage-2 matrices
  int E, T, k;
  const int32_t *ids;
  const float *gate_w;          // may be null (all ones)
  const void *x; int x_bf16; int x_per_slot;
  int n_prep, prep_per_slot, fold;
  int x_steps; uint8_t *xq; uint8_t *xs;
  int h_steps; uint8_t *hq; uint8_t *hs;
  int inter;                    // FFN intermediate width
  uint16_t *h;                  // FFN: [T][k][inter]
  float *y;                     // FFN / COMBINE: [T][rows2]; SLOTS: [T][k][rows1]
  int n_s1, n_rg1, n_s2;
  int *sync;
  int grid;
};

struct Shared {
  int ids[kMaxSlots];
  float gw[kMaxSlots];
  unsigned mask[kMaxExperts / 32];
  int wpre[kMaxExperts / 32 + 1];
  int active[kMaxExperts];
  int slots[kMaxSlots];
  int wcnt[kWaves];
  int n_active;
  // Staged activation columns (step-chunk layout: steps x 128 code bytes per
  // column) and their scales (steps x 4); after the matrix-core loop the code
  // area is reused for the per-wave accumulator dumps.
  uint8_t bq[kBBytes] __attribute__((aligned(16)));
  uint8_t bs[kBScaleBytes] __attribute__((aligned(16)));
};
static_assert(kWaves * 4 * 256 * sizeof(float) <= kBBytes, "accumulator dump must fit the column area");

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ float load_x(const void *x, int bf16, size_t i) {
  return bf16 ? bf16_to_f32(((const uint16_t *)x)[i]) : ((const float *)x)[i];
}

// Device-coherent accesses for data handed between workgroups.
__device__ __forceinline__ void st_dc(uint8_t *p, uint32_t v) {
  __hip_atomic_store(p, (uint8_t)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dc64(const uint8_t *p) {
  return __hip_atomic_load((uint64_t *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dc32(const uint8_t *p) {
  return __hip_atomic_load((uint32_t *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publish `n` finished items: every wave's device-coherent stores complete,
// then one thread bumps the counter.
__device__ __forceinline__ void signal_n(int *ctr, int n) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait (once per workgroup and counter: `seen` remembers) until the counter
// reaches `target`. Bounded: on timeout the error word is set.
__device__ __forceinline__ void wait_for(int *ctr, int target, int *err, bool &seen) {
  if (seen) return;
  if (threadIdx.x == 0) {
    unsigned spins = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(4);
      if (++spins > kSpinLimit) {
        __hip_atomic_fetch_or(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
  seen = true;
}

// Two-term FP8 split of one 32-value block held by the 32 lanes of a
// half-wave (lane = position in the block); device-coherent stores of the
// codes and scales of physical block `blk` into one column pair.
__device__ __forceinline__ void quantize_block(float v, int pos, int blk, uint8_t *q_hi, uint8_t *q_lo,
                                               uint8_t *s_hi, uint8_t *s_lo, bool store) {
  float amax = fabsf(v);
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 32));
  const int E = block_exponent(amax);
  const uint32_t hi = f32_to_e4m3(ldexpf(v, -E));
  const float r = v - ldexpf(e4m3_to_f32(hi), E);
  float rmax = fabsf(r);
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) rmax = fmaxf(rmax, __shfl_xor(rmax, m, 32));
  const int El = block_exponent(rmax);
  const uint32_t lo = f32_to_e4m3(ldexpf(r, -El));
  if (store) {
    const int off = act_offset(blk, pos);
    st_dc(q_hi + off, hi);
    st_dc(q_lo + off, lo);
    if (pos == 0) {
      st_dc(s_hi + act_scale_index(blk), (uint32_t)(E + 127));
      st_dc(s_lo + act_scale_index(blk), (uint32_t)(El + 127));
    }
  }
}

// Gate weight a slot's activation carries when gate weights are folded: the
// first slot of a (token, expert) pair gets the sum over the token's slots
// with that expert, later duplicates get 0.
__device__ __forceinline__ float folded_gate(const Shared &S, int slot, int k, int E) {
  const int e = S.ids[slot];
  if (e < 0 || e >= E) return 0.0f;
  const int t = slot / k, j = slot % k;
  for (int jj = 0; jj < j; ++jj)
    if (S.ids[t * k + jj] == e) return 0.0f;
  float g = 0.0f;
  for (int jj = 0; jj < k; ++jj)
    if (S.ids[t * k + jj] == e) g += S.gw[t * k + jj];
  return g;
}

// Copy activation columns into LDS: LDS column c <- global column src_col(c)
// (steps x 128 code bytes, steps x 4 scale bytes), device-coherent loads.
// `first`/`stride` split the work among the threads that call it.
template <typename ColMap>
__device__ __forceinline__ void copy_columns(uint8_t *lq, uint8_t *ls, const uint8_t *gq, const uint8_t *gs,
                                             int steps, int ncols, ColMap src_col, int first, int stride) {
  const int per_col = steps * 16;   // 8-byte pieces per column
  for (int idx = first; idx < ncols * per_col; idx += stride) {
    const int c = idx / per_col, p = idx - c * per_col;
    const size_t col = (size_t)src_col(c);
    *(uint64_t *)(lq + ((size_t)c * per_col + p) * 8) = ld_dc64(gq + (col * per_col + p) * 8);
  }
  for (int idx = first; idx < ncols * steps; idx += stride) {
    const int c = idx / steps, p = idx - c * steps;
    const size_t col = (size_t)src_col(c);
    *(uint32_t *)(ls + ((size_t)c * steps + p) * 4) = ld_dc32(gs + (col * steps + p) * 4);
  }
}

// ---------------------------------------------------------------- weight tiles

struct Tile {
  uint4 a[kPieceMax];       // piece j: words 16j+4g .. 16j+4g+3 of this lane's row
  uint32_t sc[kPieceMax];   // piece j: UE8M0 of blocks 8j+2g (byte 0) and 8j+2g+1 (byte 1)
};

// Issue the loads of pieces [p0, p0 + np) of one row into t (`row` null for
// an invalid tile: zeros). ALIGNED: words per row % 4 == 0, so a piece is one
// 16-byte load and one 2-byte scale load, whole or past the row end.
template <bool ALIGNED>
__device__ __forceinline__ void load_tile(Tile &t, const uint32_t *row, const uint8_t *srow, int wpr, int nb,
                                          int p0, int np, int g) {
#pragma unroll
  for (int q = 0; q < kPieceMax; ++q) {
    const int j = p0 + q;
    const int wi = 16 * j + 4 * g;
    const int b = 8 * j + 2 * g;
    const bool ok = q < np && row && wi < wpr;
    if (ALIGNED) {
      t.a[q] = ok ? *(const uint4 *)(row + wi) : make_uint4(0u, 0u, 0u, 0u);
      t.sc[q] = ok ? (uint32_t)*(const uint16_t *)(srow + b) : 0x7F7Fu;
    } else {
      t.a[q] = make_uint4(0u, 0u, 0u, 0u);
      t.sc[q] = 0x7F7Fu;
      if (ok) {
        const uint2 lo = *(const uint2 *)(row + wi);
        const uint2 hi = wi + 2 < wpr ? *(const uint2 *)(row + wi + 2) : make_uint2(0u, 0u);
        t.a[q] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        t.sc[q] = (uint32_t)srow[b] | ((b + 1 < nb ? (uint32_t)srow[b + 1] : 0x7Fu) << 8);
      }
    }
  }
}

// Decode pieces [p0, p0 + np) of the tile and accumulate them against NT
// N-tiles of LDS-staged columns. Lane (column jc = lane & 15, lane-group g):
// N-tile n reads LDS column col0[n] (or zeros when !on[n]).
template <int NT>
__device__ __forceinline__ void mma_tile(const Tile &t, int p0, int np, const uint8_t *lq, const uint8_t *ls,
                                         int steps, const int (&col)[NT], const bool (&on)[NT], v4f (&acc)[NT],
                                         uint32_t &carry, int lane) {
  const int g = lane >> 4;
  const int src = ((lane - 16) & 63) << 2;   // lane-group g-1 (mod 4), same row
#pragma unroll
  for (int q = 0; q < kPieceMax; ++q) {
    if (q < np) {
      const int j = p0 + q;
      const uint4 a = t.a[q];
      const uint32_t rot = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)a.w);
      const uint32_t hist = g == 0 ? carry : rot;
      carry = rot;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int step = 2 * j + hh;
        v8i B[NT];
        uint32_t sb[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          if (on[n]) {
            const uint4 *p = (const uint4 *)(lq + ((size_t)col[n] * steps + step) * 128 + g * 32);
            const uint4 u0 = p[0], u1 = p[1];
            B[n] = v8i{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
            sb[n] = ls[((size_t)col[n] * steps + step) * 4 + g];
          } else {
            B[n] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
            sb[n] = 127u;
          }
        }
        const uint32_t w0 = hh ? a.z : a.x, w1 = hh ? a.w : a.y, hw = hh ? a.y : hist;
        const nib2 d0 = decode_word(w0, hw);
        const nib2 d1 = decode_word(w1, w0);
        const v8i A = v8i{(int)d0.even, (int)d0.odd, (int)d1.even, (int)d1.odd, 0, 0, 0, 0};
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          if (hh == 0)
            acc[n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B[n], acc[n], 4, 0, 0, (int)t.sc[q], 0,
                                                                     (int)sb[n]);
          else
            acc[n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B[n], acc[n], 4, 0, 1, (int)t.sc[q], 0,
                                                                     (int)sb[n]);
        }
      }
    }
  }
}

template <int NT>
__device__ __forceinline__ int d_index(int wave, int nt, int row, int col) {
  const int lane = (row >> 2) * 16 + col;
  return ((wave * NT + nt) * 64 + lane) * 4 + (row & 3);
}

// Dump the wave accumulators into the (now free) column area; the caller
// synchronises before and after.
template <int NT>
__device__ __forceinline__ void dump_acc(Shared &S, const v4f (&acc)[NT], int wave, int lane) {
  float *red = (float *)S.bq;
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[((wave * NT + n) * 64 + lane) * 4 + r] = acc[n][r];
}

// ---------------------------------------------------------------- work items

__device__ __forceinline__ void prep_item(const LayerArgs &a, Shared &S, int v) {
  const int tid = threadIdx.x;
  int t, j0 = 0;
  if (a.prep_per_slot) { t = v / a.k; j0 = v % a.k; } else { t = v; }
  // bookkeeping for the slots this item covers
  const int s_lo = a.prep_per_slot ? v : t * a.k;
  const int s_hi = a.prep_per_slot ? v + 1 : t * a.k + a.k;
  if (tid == 0) {
    int skipped = 0;
    for (int s = s_lo; s < s_hi; ++s) skipped += S.ids[s] >= a.E;
    if (skipped) __hip_atomic_fetch_add(&a.sync[SY_SKIP], skipped, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  for (int s = s_lo; s < s_hi; ++s) {
    const int e = S.ids[s];
    const bool dead = e < 0 || e >= a.E;
    if (dead && a.mode == MODE_SLOTS)
      for (int r = tid; r < a.rows1; r += kThreads) a.y[(size_t)s * a.rows1 + r] = 0.0f;
    if (dead && a.mode == MODE_FFN)
      for (int c = tid; c < a.inter; c += kThreads) a.h[(size_t)s * a.inter + c] = 0;
    if (a.mode == MODE_FFN) {
      // K padding of the slot's down-projection activations: zero codes, finite scales
      const int nbh = a.inter / 32, npad = 4 * a.h_steps - nbh;
      for (int idx = tid; idx < 2 * npad * 32; idx += kThreads) {
        const int hl = idx / (npad * 32), rem = idx % (npad * 32);
        const int blk = nbh + rem / 32, pos = rem % 32;
        const size_t col = (size_t)s * 2 + hl;
        st_dc(a.hq + col * a.h_steps * 128 + act_offset(blk, pos), 0u);
        if (pos == 0) st_dc(a.hs + col * a.h_steps * 4 + act_scale_index(blk), 127u);
      }
    }
  }
  // the activation vector
  const int K = a.mode == MODE_COMBINE ? a.cols2 : a.cols1;
  const int nb = K / 32;
  const int nblk = 4 * a.x_steps;
  uint8_t *q_hi = a.xq + ((size_t)v * 2 + 0) * a.x_steps * 128;
  uint8_t *q_lo = a.xq + ((size_t)v * 2 + 1) * a.x_steps * 128;
  uint8_t *c_hi = a.xs + ((size_t)v * 2 + 0) * a.x_steps * 4;
  uint8_t *c_lo = a.xs + ((size_t)v * 2 + 1) * a.x_steps * 4;
  const int pos = tid & 31;
  for (int blk = tid >> 5; blk < nblk; blk += kThreads / 32) {
    float xv = 0.0f;
    if (blk < nb) {
      const size_t off = (size_t)blk * 32 + pos;
      if (!a.prep_per_slot) {
        xv = load_x(a.x, a.x_bf16, (size_t)t * K + off);
      } else if (!a.fold) {
        xv = load_x(a.x, a.x_bf16, (size_t)(a.x_per_slot ? v : t) * K + off);
      } else {
        // canonical slot of (token, expert): sum over the duplicates
        const int e = S.ids[v];
        bool canonical = e >= 0 && e < a.E;
        for (int jj = 0; jj < j0 && canonical; ++jj) canonical = S.ids[t * a.k + jj] != e;
        if (canonical)
          for (int jj = 0; jj < a.k; ++jj)
            if (S.ids[t * a.k + jj] == e)
              xv += S.gw[t * a.k + jj] * load_x(a.x, a.x_bf16, (size_t)(a.x_per_slot ? t * a.k + jj : t) * K + off);
      }
    }
    quantize_block(xv, pos, blk, q_hi, q_lo, c_hi, c_lo, true);
  }
}

// Slot list of expert e into S.slots (slot order); returns the count.
__device__ __forceinline__ int gather_slots(Shared &S, int e, int n) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int total = 0;
  for (int base = 0; base < n; base += kThreads) {
    const int i = base + threadIdx.x;
    const bool p = i < n && S.ids[i] == e;
    const unsigned long long bal = __ballot(p);
    if (lane == 0) S.wcnt[wave] = __popcll(bal);
    __syncthreads();
    int off = total;
    for (int w = 0; w < wave; ++w) off += S.wcnt[w];
    if (p) S.slots[off + __popcll(bal & ((1ull << lane) - 1ull))] = i;
    for (int w = 0; w < kWaves; ++w) total += S.wcnt[w];
    __syncthreads();
  }
  return total;
}

template <int NT, bool ALIGNED>
__device__ __forceinline__ void stage1_item(const LayerArgs &a, Shared &S, int item, bool &prep_seen) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int ai = item / a.n_rg1, rg = item % a.n_rg1;
  if (ai >= S.n_active) return;   // no such active expert: nothing to do
  const int e = S.active[ai];
  const bool ffn = a.mode == MODE_FFN;
  const int r0 = ffn ? (wave < 2 ? 0 : a.inter) + rg * 32 + 16 * (wave & 1) : rg * 64 + 16 * wave;
  const bool tile_ok = r0 < a.rows1;
  const int wpr = a.cols1 / 16, nb = a.cols1 / 32, J = (nb + 7) >> 3;
  const size_t row = (size_t)e * a.rows1 + (tile_ok ? r0 + i16 : 0);
  const uint32_t *rowp = tile_ok ? a.w1 + row * wpr : nullptr;
  const uint8_t *srow = a.s1 + row * nb;
  Tile tl;
  load_tile<ALIGNED>(tl, rowp, srow, wpr, nb, 0, min(J, kPieceMax), g);   // in flight while we wait
  const int ne = gather_slots(S, e, a.T * a.k);
  wait_for(&a.sync[SY_PREP], a.n_prep, &a.sync[SY_ERR], prep_seen);

  // slots per column group: whatever fits the LDS column area (<= NT * 8)
  const int steps = a.x_steps;
  const int gsz = min(NT * 8, kBBytes / (2 * steps * 128));
  for (int c0 = 0; c0 < ne; c0 += gsz) {
    const int ncol = min(ne - c0, gsz);
    // LDS column c = slot (c0 + c/2)'s hi (even c) or lo (odd c) term
    copy_columns(S.bq, S.bs, a.xq, a.xs, steps, 2 * ncol,
                 [&](int c) {
                   const int slot = S.slots[c0 + (c >> 1)];
                   return (a.prep_per_slot ? slot : slot / a.k) * 2 + (c & 1);
                 },
                 threadIdx.x, kThreads);
    __syncthreads();
    int col[NT];
    bool on[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      col[n] = n * 16 + i16;
      on[n] = n * 8 + (i16 >> 1) < ncol;
    }
    v4f acc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = v4f{0.f, 0.f, 0.f, 0.f};
    uint32_t carry = 0u;
    for (int p0 = 0; p0 < J; p0 += kPieceMax) {
      if (p0 > 0 || c0 > 0) load_tile<ALIGNED>(tl, rowp, srow, wpr, nb, p0, min(J - p0, kPieceMax), g);
      mma_tile<NT>(tl, p0, min(J - p0, kPieceMax), S.bq, S.bs, steps, col, on, acc, carry, lane);
    }
    __syncthreads();   // everyone is done with the staged columns
    dump_acc<NT>(S, acc, wave, lane);
    __syncthreads();
    const float *red = (const float *)S.bq;
    if (!ffn) {
      for (int idx = threadIdx.x; idx < ncol * 64; idx += kThreads) {
        const int c = idx >> 6, rr = idx & 63, w = rr >> 4, ri = rr & 15;
        if (rg * 64 + rr >= a.rows1) continue;
        const int n = c >> 3, cj = 2 * (c & 7);
        const float v = red[d_index<NT>(w, n, ri, cj)] + red[d_index<NT>(w, n, ri, cj + 1)];
        a.y[(size_t)S.slots[c0 + c] * a.rows1 + rg * 64 + rr] = v;
      }
    } else {
      for (int base = 0; base < ncol; base += kThreads / 32) {
        const int c = base + (threadIdx.x >> 5), i = threadIdx.x & 31;
        const bool live = c < ncol;
        float hv = 0.0f;
        int slot = 0;
        if (live) {
          const int n = c >> 3, cj = 2 * (c & 7), w = i >> 4, ri = i & 15;
          const float gate = red[d_index<NT>(w, n, ri, cj)] + red[d_index<NT>(w, n, ri, cj + 1)];
          const float up = red[d_index<NT>(w + 2, n, ri, cj)] + red[d_index<NT>(w + 2, n, ri, cj + 1)];
          const float silu = gate / (1.0f + expf(-gate));
          const uint16_t hb = f32_to_bf16_rne(silu * up);
          slot = S.slots[c0 + c];
          a.h[(size_t)slot * a.inter + rg * 32 + i] = hb;
          hv = bf16_to_f32(hb) * folded_gate(S, slot, a.k, a.E);
        }
        quantize_block(hv, i, rg, a.hq + ((size_t)slot * 2 + 0) * a.h_steps * 128,
                       a.hq + ((size_t)slot * 2 + 1) * a.h_steps * 128, a.hs + ((size_t)slot * 2 + 0) * a.h_steps * 4,
                       a.hs + ((size_t)slot * 2 + 1) * a.h_steps * 4, live);
      }
    }
    __syncthreads();
  }
}

// Stage 2: wave w handles experts w, w+4, ... of the active list. Each wave
// stages its own expert's columns (the tokens routed to it) in its quarter of
// the column area, in token groups that fit.
template <int NT, bool ALIGNED>
__device__ __forceinline__ void stage2_item(const LayerArgs &a, Shared &S, int rt, bool &dep_seen) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int wpr = a.cols2 / 16, nb = a.cols2 / 32, J = (nb + 7) >> 3;
  const int n_act = S.n_active;
  const bool ffn = a.mode == MODE_FFN;
  const uint8_t *gq = ffn ? a.hq : a.xq;
  const uint8_t *gs = ffn ? a.hs : a.xs;
  const int steps = ffn ? a.h_steps : a.x_steps;
  uint8_t *lq = S.bq + wave * (kBBytes / kWaves);
  uint8_t *ls = S.bs + wave * (kBScaleBytes / kWaves);
  const int tsz = max(1, min(NT * 8, kBBytes / kWaves / (2 * steps * 128)));   // tokens per group
  v4f acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = v4f{0.f, 0.f, 0.f, 0.f};
  Tile tl;
  for (int ai = wave; ai < n_act || !dep_seen; ai += kWaves) {
    const bool have = ai < n_act;
    const int e = have ? S.active[ai] : 0;
    const size_t row = (size_t)e * a.rows2 + rt * 16 + i16;
    const uint32_t *rowp = have ? a.w2 + row * wpr : nullptr;
    const uint8_t *srow = a.s2 + row * nb;
    if (have) load_tile<ALIGNED>(tl, rowp, srow, wpr, nb, 0, min(J, kPieceMax), g);
    if (!dep_seen) {
      // every wave reaches this once (block-wide barrier inside)
      if (ffn) wait_for(&a.sync[SY_S1], a.n_s1, &a.sync[SY_ERR], dep_seen);
      else wait_for(&a.sync[SY_PREP], a.n_prep, &a.sync[SY_ERR], dep_seen);
    }
    if (!have) break;
    // tokens [t0, t0 + tsz) per group, LDS column 2 * (t - t0) + hilo; the
    // group's matrix-core steps add into the batch-wide accumulators with
    // zero activations for tokens outside the group
    auto slot_of = [&](int t) {   // first slot of (token, e): duplicates were folded into it
      for (int jj = 0; jj < a.k; ++jj)
        if (S.ids[t * a.k + jj] == e) return t * a.k + jj;
      return -1;
    };
    for (int t0 = 0; t0 < a.T; t0 += tsz) {
      const int nt_tok = min(a.T - t0, tsz);
      copy_columns(lq, ls, gq, gs, steps, 2 * nt_tok,
                   [&](int c) {
                     const int s = slot_of(t0 + (c >> 1));
                     return (s < 0 ? 0 : s) * 2 + (c & 1);
                   },
                   lane, 64);
      int col[NT];
      bool on[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int tok = n * 8 + (i16 >> 1);
        const bool in = tok >= t0 && tok < t0 + nt_tok;
        on[n] = in && slot_of(tok) >= 0;
        col[n] = in ? 2 * (tok - t0) + (i16 & 1) : 0;
      }
      uint32_t carry = 0u;
      for (int p0 = 0; p0 < J; p0 += kPieceMax) {
        if (p0 > 0 || t0 > 0) load_tile<ALIGNED>(tl, rowp, srow, wpr, nb, p0, min(J - p0, kPieceMax), g);
        mma_tile<NT>(tl, p0, min(J - p0, kPieceMax), lq, ls, steps, col, on, acc, carry, lane);
      }
    }
  }
  __syncthreads();   // all waves done with their staged columns
  dump_acc<NT>(S, acc, wave, lane);
  __syncthreads();
  const float *red = (const float *)S.bq;
  for (int idx = threadIdx.x; idx < a.T * 16; idx += kThreads) {
    const int t = idx >> 4, ri = idx & 15;
    const int n = t >> 3, cj = 2 * (t & 7);
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += red[d_index<NT>(w, n, ri, cj)] + red[d_index<NT>(w, n, ri, cj + 1)];
    a.y[(size_t)t * a.rows2 + rt * 16 + ri] = v;
  }
  __syncthreads();
}

template <int NT, bool ALIGNED>
__global__ void __launch_bounds__(kThreads) k_layer(LayerArgs a) {
  __shared__ Shared S;
  const int tid = threadIdx.x;
  // routing, redundantly in every workgroup: active experts in id order
  const int n = a.T * a.k;
  const int nw = (a.E + 31) >> 5;
  for (int i = tid; i < n; i += kThreads) {
    S.ids[i] = a.ids[i];
    S.gw[i] = a.gate_w ? a.gate_w[i] : 1.0f;
  }
  for (int w = tid; w < nw; w += kThreads) S.mask[w] = 0u;
  __syncthreads();
  for (int i = tid; i < n; i += kThreads) {
    const int e = S.ids[i];
    if (e >= 0 && e < a.E) atomicOr(&S.mask[e >> 5], 1u << (e & 31));
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int w = 0; w < nw; ++w) { S.wpre[w] = acc; acc += __popc(S.mask[w]); }
    S.n_active = acc;
  }
  __syncthreads();
  for (int w = tid; w < nw; w += kThreads) {
    unsigned m = S.mask[w];
    int o = S.wpre[w];
    while (m) {
      const int b = __ffs(m) - 1;
      S.active[o++] = w * 32 + b;
      m &= m - 1u;
    }
  }
  __syncthreads();

  // Items come in index order, so a workgroup's prep items, then its stage-1
  // items, are contiguous: their completions are published in one signal
  // when the workgroup moves on (before it can wait on anyone), and each
  // dependency is waited for at most once per workgroup.
  const int n_items = a.n_prep + a.n_s1 + a.n_s2;
  int prep_done = 0, s1_done = 0;
  bool prep_seen = false, dep_seen = false;
  for (int item = blockIdx.x; item < n_items; item += a.grid) {
    if (item < a.n_prep) {
      prep_item(a, S, item);
      ++prep_done;
    } else if (item < a.n_prep + a.n_s1) {
      if (prep_done) { signal_n(&a.sync[SY_PREP], prep_done); prep_done = 0; }
      stage1_item<NT, ALIGNED>(a, S, item - a.n_prep, prep_seen);
      ++s1_done;
    } else {
      if (prep_done) { signal_n(&a.sync[SY_PREP], prep_done); prep_done = 0; }
      if (s1_done) { signal_n(&a.sync[SY_S1], s1_done); s1_done = 0; }
      stage2_item<NT, ALIGNED>(a, S, item - a.n_prep - a.n_s1, dep_seen);
    }
    __syncthreads();
  }
  if (prep_done) signal_n(&a.sync[SY_PREP], prep_done);
  if (s1_done) signal_n(&a.sync[SY_S1], s1_done);
  // the last workgroup out publishes the status and clears the counters
  __syncthreads();
  if (tid == 0) {
    if (__hip_atomic_fetch_add(&a.sync[SY_EXIT], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.grid - 1) {
      const int skipped = __hip_atomic_load(&a.sync[SY_SKIP], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int err = __hip_atomic_load(&a.sync[SY_ERR], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.sync[ST_SKIPPED], skipped, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.sync[ST_ERROR], err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int i = SY_PREP; i <= SY_ERR; ++i)
        __hip_atomic_store(&a.sync[i], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------- host side

static int device_check(int *cus) {
  static int cached[64];
  static int ncu[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return TRELLIS_EHIP;
  if (cached[dev] == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return TRELLIS_EHIP;
    cached[dev] = (strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    ncu[dev] = p.multiProcessorCount;
  }
  *cus = ncu[dev];
  return cached[dev] > 0 ? TRELLIS_OK : TRELLIS_EDEVICE;
}

template <int NT, bool ALIGNED>
static int resident_blocks() {
  static int cached[64];
  int dev = 0;
  hipGetDevice(&dev);
  if (dev < 0 || dev >= 64) return 1;
  if (cached[dev] == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_layer<NT, ALIGNED>, kThreads, 0) != hipSuccess ||
        nb < 1)
      nb = 1;
    cached[dev] = nb;
  }
  return cached[dev];
}

static int check_mat(const trellis_mat_t *w) {
  if (!w || !w->syms || !w->scales) return TRELLIS_ENULL;
  if (w->n_mat < 1 || w->rows < 1 || w->cols < 32 || w->cols % 32) return TRELLIS_EINVAL;
  if (w->rows % 16 || w->n_mat > kMaxExperts) return TRELLIS_EINVAL;
  return TRELLIS_OK;
}

static int check_routing(int T, int k) {
  if (T < 1 || T > kMaxT || k < 1 || k > kMaxK || T * k > kMaxSlots) return TRELLIS_EINVAL;
  return TRELLIS_OK;
}

template <int NT, bool ALIGNED>
static int launch_nt(LayerArgs &a, int cus, hipStream_t s) {
  const int n_items = a.n_prep + a.n_s1 + a.n_s2;
  a.grid = std::max(1, std::min(n_items, cus * resident_blocks<NT, ALIGNED>()));
  hipLaunchKernelGGL((k_layer<NT, ALIGNED>), dim3(a.grid), dim3(kThreads), 0, s, a);
  return hipGetLastError() == hipSuccess ? TRELLIS_OK : TRELLIS_EHIP;
}

template <bool ALIGNED>
static int launch_al(LayerArgs &a, int cus, hipStream_t s) {
  switch ((a.T + 7) / 8) {
    case 1: return launch_nt<1, ALIGNED>(a, cus, s);
    case 2: return launch_nt<2, ALIGNED>(a, cus, s);
    case 3: return launch_nt<3, ALIGNED>(a, cus, s);
    default: return launch_nt<4, ALIGNED>(a, cus, s);
  }
}

// The aligned instances need every streamed matrix to have cols % 64 == 0
// (words per row % 4 == 0) and 16-byte aligned symbol / 2-byte aligned
// scale bases.
static int launch(LayerArgs &a, int cus, hipStream_t s) {
  const bool aligned = a.cols1 % 64 == 0 && a.cols2 % 64 == 0 && ((uintptr_t)a.w1 & 15) == 0 &&
                       ((uintptr_t)a.w2 & 15) == 0 && ((uintptr_t)a.s1 & 1) == 0 && ((uintptr_t)a.s2 & 1) == 0;
  return aligned ? launch_al<true>(a, cus, s) : launch_al<false>(a, cus, s);
}

}  // namespace tq

using namespace tq;

extern "C" size_t trellis_moe_gemv_workspace_size(int32_t n_mat, int32_t rows, int32_t cols, int32_t T,
                                                  int32_t k) {
  if (n_mat < 1 || cols < 32 || cols % 32 || rows < 1 || check_routing(T, k)) return 0;
  return make_layout(T * k, cols, 0, 0).total;
}

extern "C" int trellis_moe_gemv(hipStream_t stream, const trellis_mat_t *w, const void *x, int32_t x_dtype,
                                int32_t x_per_slot, const int32_t *topk_ids, const float *topk_w,
                                int32_t T, int32_t k, float *y, void *workspace, size_t workspace_bytes) {
  int rc = check_mat(w);
  if (rc) return rc;
  if (!x || !topk_ids || !y || !workspace) return TRELLIS_ENULL;
  if ((x_dtype != TRELLIS_F32 && x_dtype != TRELLIS_BF16) || (x_per_slot != 0 && x_per_slot != 1))
    return TRELLIS_EINVAL;
  if ((rc = check_routing(T, k))) return rc;
  const bool combine = topk_w != nullptr;
  const bool per_slot = combine || x_per_slot;
  const Layout L = make_layout(per_slot ? T * k : T, w->cols, 0, 0);
  if (((uintptr_t)workspace & 255) || workspace_bytes < L.total) return TRELLIS_EWORKSPACE;
  int cus = 0;
  if ((rc = device_check(&cus))) return rc;
  char *ws = (char *)workspace;
  LayerArgs a{};
  a.mode = combine ? MODE_COMBINE : MODE_SLOTS;
  a.w1 = w->syms; a.s1 = w->scales; a.rows1 = w->rows; a.cols1 = w->cols;
  a.w2 = w->syms; a.s2 = w->scales; a.rows2 = w->rows; a.cols2 = w->cols;
  a.E = w->n_mat; a.T = T; a.k = k; a.ids = topk_ids; a.gate_w = topk_w;
  a.x = x; a.x_bf16 = x_dtype == TRELLIS_BF16; a.x_per_slot = x_per_slot;
  a.n_prep = per_slot ? T * k : T; a.prep_per_slot = per_slot; a.fold = combine;
  a.x_steps = steps_for_blocks(w->cols / 32);
  a.xq = (uint8_t *)(ws + L.xq); a.xs = (uint8_t *)(ws + L.xs);
  a.y = y;
  a.sync = (int *)(ws + L.sync);
  const int max_active = std::min(w->n_mat, T * k);
  if (combine) {
    a.n_s1 = 0; a.n_rg1 = 1; a.n_s2 = w->rows / 16;
  } else {
    a.n_rg1 = (w->rows + 63) / 64; a.n_s1 = max_active * a.n_rg1; a.n_s2 = 0;
  }
  return launch(a, cus, stream);
}

extern "C" size_t trellis_moe_ffn_workspace_size(int32_t n_exp, int32_t hidden, int32_t inter, int32_t T,
                                                 int32_t k) {
  if (n_exp < 1 || hidden < 32 || hidden % 32 || inter < 32 || inter % 32 || check_routing(T, k)) return 0;
  return make_layout(T, hidden, T * k, inter).total;
}

extern "C" int trellis_moe_ffn_timed(hipStream_t stream, const trellis_mat_t *w_gate_up,
                                     const trellis_mat_t *w_down, const void *x, int32_t x_dtype,
                                     const int32_t *topk_ids, const float *topk_w, int32_t T, int32_t k,
                                     uint16_t *h, float *y, void *workspace, size_t workspace_bytes,
                                     hipEvent_t *events) {
  int rc;
  if ((rc = check_mat(w_gate_up)) || (rc = check_mat(w_down))) return rc;
  if (!x || !topk_ids || !h || !y || !workspace) return TRELLIS_ENULL;
  if (x_dtype != TRELLIS_F32 && x_dtype != TRELLIS_BF16) return TRELLIS_EINVAL;
  if ((rc = check_routing(T, k))) return rc;
  const int E = w_gate_up->n_mat, hidden = w_gate_up->cols, inter = w_gate_up->rows / 2;
  if (w_gate_up->rows % 64 || w_down->n_mat != E || w_down->rows != hidden || w_down->cols != inter)
    return TRELLIS_EINVAL;
  const Layout L = make_layout(T, hidden, T * k, inter);
  if (((uintptr_t)workspace & 255) || workspace_bytes < L.total) return TRELLIS_EWORKSPACE;
  int cus = 0;
  if ((rc = device_check(&cus))) return rc;
  char *ws = (char *)workspace;
  LayerArgs a{};
  a.mode = MODE_FFN;
  a.w1 = w_gate_up->syms; a.s1 = w_gate_up->scales; a.rows1 = w_gate_up->rows; a.cols1 = hidden;
  a.w2 = w_down->syms; a.s2 = w_down->scales; a.rows2 = hidden; a.cols2 = inter;
  a.E = E; a.T = T; a.k = k; a.ids = topk_ids; a.gate_w = topk_w;
  a.x = x; a.x_bf16 = x_dtype == TRELLIS_BF16; a.x_per_slot = 0;
  a.n_prep = T; a.prep_per_slot = 0; a.fold = 0;
  a.x_steps = steps_for_blocks(hidden / 32);
  a.xq = (uint8_t *)(ws + L.xq); a.xs = (uint8_t *)(ws + L.xs);
  a.h_steps = steps_for_blocks(inter / 32);
  a.hq = (uint8_t *)(ws + L.hq); a.hs = (uint8_t *)(ws + L.hs);
  a.inter = inter; a.h = h; a.y = y;
  a.sync = (int *)(ws + L.sync);
  a.n_rg1 = inter / 32;
  a.n_s1 = std::min(E, T * k) * a.n_rg1;
  a.n_s2 = hidden / 16;
  if (events && events[0]) hipEventRecord(events[0], stream);
  rc = launch(a, cus, stream);
  if (events && events[1]) hipEventRecord(events[1], stream);
  return rc;
}

extern "C" int trellis_moe_ffn(hipStream_t stream, const trellis_mat_t *w_gate_up, const trellis_mat_t *w_down,
                               const void *x, int32_t x_dtype, const int32_t *topk_ids, const float *topk_w,
                               int32_t T, int32_t k, uint16_t *h, float *y, void *workspace,
                               size_t workspace_bytes) {
  return trellis_moe_ffn_timed(stream, w_gate_up, w_down, x, x_dtype, topk_ids, topk_w, T, k, h, y, workspace,
                               workspace_bytes, nullptr);
}

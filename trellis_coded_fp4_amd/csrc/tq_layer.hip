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
//   stage-2 items  16 output rows summed over all active experts; columns =
//                  tokens. Deterministic, no atomics on outputs.
// Stage-1 items wait (spin on a device counter) for all prep items, stage-2
// items for all stage-1 items (or prep items when there is no stage 1); each
// item issues its weight loads before waiting. The grid never exceeds the
// number of co-resident workgroups, so every wait is for a running
// workgroup; waits are bounded and set an error flag on timeout. The last
// workgroup to finish publishes the status words and clears the counters.
//
// Weight streaming: a wave owns one 16-row tile over the full K. Lane
// (row i, lane-group g) loads "piece" j = 16 bytes = blocks 8j+2g, 8j+2g+1 of
// its row, and feeds them to matrix-core steps 2j and 2j+1 as K-block g (the
// activations are laid out to match). A wave instruction therefore reads 16
// rows x 64 contiguous bytes; all of a tile's pieces (up to 16, K <= 4096 per
// pass) are in flight before the first decode. The decoder history of a
// block is the word before it: from the neighbouring lane-group's piece via
// ds_bpermute, or from the previous piece.
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
constexpr unsigned kSpinLimit = 1u << 20;   // polls (each a device-coherent load + short sleep)

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
  int n_slots;
  float red[kWaves * 4 * 256];  // per-wave accumulator dumps (NT <= 4)
};

// ---------------------------------------------------------------- small helpers

__device__ __forceinline__ float load_x(const void *x, int bf16, size_t i) {
  return bf16 ? bf16_to_f32(((const uint16_t *)x)[i]) : ((const float *)x)[i];
}

__device__ __forceinline__ void signal(int *ctr) {
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    atomicAdd(ctr, 1);
  }
}

__device__ __forceinline__ void wait_for(int *ctr, int target, int *err) {
  if (threadIdx.x == 0) {
    unsigned spins = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit) {
        atomicOr(err, 1);
        break;
      }
    }
    __threadfence();
  }
  __syncthreads();
}

// Two-term FP8 split of one 32-value block held by the 32 lanes of a
// half-wave (lane = position in the block); stores codes and scales of
// physical block `blk` into one column pair.
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
    q_hi[off] = (uint8_t)hi;
    q_lo[off] = (uint8_t)lo;
    if (pos == 0) {
      s_hi[act_scale_index(blk)] = (uint8_t)(E + 127);
      s_lo[act_scale_index(blk)] = (uint8_t)(El + 127);
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

// ---------------------------------------------------------------- weight tiles

constexpr int kRing = 8;   // pieces in flight per wave (8 x 1 KiB per wave instruction stream)

struct Piece {
  uint4 a;       // words 16j+4g .. 16j+4g+3 of this lane's row
  uint32_t sc;   // UE8M0 of blocks 8j+2g (byte 0) and 8j+2g+1 (byte 1)
};

// Load piece j of one row (`row` null: an invalid tile, all zeros).
// ALIGNED: words per row % 4 == 0 (so blocks per row are even): one 16-byte
// load and one 2-byte scale load per lane, a piece is either whole or past
// the row end. Otherwise pieces may be half-filled and rows 8-byte aligned.
template <bool ALIGNED>
__device__ __forceinline__ void load_piece(Piece &p, const uint32_t *row, const uint8_t *srow, int wpr, int nb,
                                           int j, int g) {
  const int wi = 16 * j + 4 * g;
  const int b = 8 * j + 2 * g;
  if (ALIGNED) {
    const bool ok = row && wi < wpr;
    p.a = ok ? *(const uint4 *)(row + wi) : make_uint4(0u, 0u, 0u, 0u);
    p.sc = ok ? (uint32_t)*(const uint16_t *)(srow + b) : 0x7F7Fu;
  } else {
    p.a = make_uint4(0u, 0u, 0u, 0u);
    p.sc = 0x7F7Fu;
    if (row && wi < wpr) {
      const uint2 lo = *(const uint2 *)(row + wi);
      const uint2 hi = wi + 2 < wpr ? *(const uint2 *)(row + wi + 2) : make_uint2(0u, 0u);
      p.a = make_uint4(lo.x, lo.y, hi.x, hi.y);
      p.sc = (uint32_t)srow[b] | ((b + 1 < nb ? (uint32_t)srow[b + 1] : 0x7Fu) << 8);
    }
  }
}

struct BCol {
  const uint8_t *q;     // this lane's 32-byte operand of step 0 (advance 128 B per step)
  const uint8_t *s;     // this lane's scale byte of step 0 (advance 4 B per step)
  bool on;
};

__device__ __forceinline__ void load_b(v8i &b, uint32_t &s, const BCol &c, int step) {
  if (c.on) {
    const uint4 *p = (const uint4 *)(c.q + step * 128);
    const uint4 u0 = p[0], u1 = p[1];
    b = v8i{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
    s = c.s[step * 4];
  } else {
    b = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    s = 127u;
  }
}

// A wave's 16-row tile streamed through a ring of kRing pieces: the first
// kRing pieces are issued by start_tile (before any wait), and each piece
// consumed refills its slot kRing pieces ahead.
struct TileStream {
  const uint32_t *row;
  const uint8_t *srow;
  int wpr, nb, J;
  Piece ring[kRing];
};

template <bool ALIGNED>
__device__ __forceinline__ void start_tile(TileStream &ts, const uint32_t *row, const uint8_t *srow, int wpr,
                                           int nb, int g) {
  ts.row = row;
  ts.srow = srow;
  ts.wpr = wpr;
  ts.nb = nb;
  ts.J = (nb + 7) >> 3;
#pragma unroll
  for (int r = 0; r < kRing; ++r) {
    if (r < ts.J) load_piece<ALIGNED>(ts.ring[r], row, srow, wpr, nb, r, g);
  }
}

// Decode the tile and accumulate it against the B columns (all of K).
template <int NT, bool ALIGNED>
__device__ __forceinline__ void mma_tile(TileStream &ts, const BCol (&bc)[NT], v4f (&acc)[NT], int lane) {
  const int g = lane >> 4;
  const int src = ((lane - 16) & 63) << 2;   // lane-group g-1 (mod 4), same row
  v8i bq[NT], bn[NT];
  uint32_t bs[NT], bsn[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) load_b(bq[n], bs[n], bc[n], 0);
  uint32_t carry = 0u;
  for (int base = 0; base < ts.J; base += kRing) {
#pragma unroll
    for (int r = 0; r < kRing; ++r) {
      const int j = base + r;
      if (j < ts.J) {
        const uint4 a = ts.ring[r].a;
        const uint32_t sc = ts.ring[r].sc;
        if (j + kRing < ts.J) load_piece<ALIGNED>(ts.ring[r], ts.row, ts.srow, ts.wpr, ts.nb, j + kRing, g);
        const uint32_t rot = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)a.w);
        const uint32_t hist = g == 0 ? carry : rot;
        carry = rot;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int step = 2 * j + hh;
          const bool more = hh == 0 || j + 1 < ts.J;
          if (more) {
#pragma unroll
            for (int n = 0; n < NT; ++n) load_b(bn[n], bsn[n], bc[n], step + 1);
          }
          const uint32_t w0 = hh ? a.z : a.x, w1 = hh ? a.w : a.y, hw = hh ? a.y : hist;
          const nib2 d0 = decode_word(w0, hw);
          const nib2 d1 = decode_word(w1, w0);
          const v8i A = v8i{(int)d0.even, (int)d0.odd, (int)d1.even, (int)d1.odd, 0, 0, 0, 0};
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            if (hh == 0)
              acc[n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, bq[n], acc[n], 4, 0, 0, (int)sc, 0,
                                                                       (int)bs[n]);
            else
              acc[n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, bq[n], acc[n], 4, 0, 1, (int)sc, 0,
                                                                       (int)bs[n]);
          }
          if (more) {
#pragma unroll
            for (int n = 0; n < NT; ++n) {
              bq[n] = bn[n];
              bs[n] = bsn[n];
            }
          }
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

template <int NT>
__device__ __forceinline__ void dump_acc(Shared &S, const v4f (&acc)[NT], int wave, int lane) {
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) S.red[((wave * NT + n) * 64 + lane) * 4 + r] = acc[n][r];
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
    if (skipped) atomicAdd(&a.sync[SY_SKIP], skipped);
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
      const int nbh = a.inter / 32;
      for (int idx = tid; idx < 2 * (4 * a.h_steps - nbh) * 32; idx += kThreads) {
        const int hl = idx / ((4 * a.h_steps - nbh) * 32), rem = idx % ((4 * a.h_steps - nbh) * 32);
        const int blk = nbh + rem / 32, pos = rem % 32;
        const size_t col = (size_t)s * 2 + hl;
        a.hq[col * a.h_steps * 128 + act_offset(blk, pos)] = 0;
        if (pos == 0) a.hs[col * a.h_steps * 4 + act_scale_index(blk)] = 127;
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
__device__ __forceinline__ void stage1_item(const LayerArgs &a, Shared &S, int item) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int ai = item / a.n_rg1, rg = item % a.n_rg1;
  if (ai >= S.n_active) {
    signal(&a.sync[SY_S1]);
    return;
  }
  const int e = S.active[ai];
  const bool ffn = a.mode == MODE_FFN;
  const int r0 = ffn ? (wave < 2 ? 0 : a.inter) + rg * 32 + 16 * (wave & 1) : rg * 64 + 16 * wave;
  const bool tile_ok = r0 < a.rows1;
  const int wpr = a.cols1 / 16, nb = a.cols1 / 32;
  const size_t row = (size_t)e * a.rows1 + (tile_ok ? r0 + i16 : 0);
  const uint32_t *rowp = tile_ok ? a.w1 + row * wpr : nullptr;
  const uint8_t *srow = a.s1 + row * nb;
  TileStream ts;
  start_tile<ALIGNED>(ts, rowp, srow, wpr, nb, g);   // in flight while we gather slots and wait
  const int ne = gather_slots(S, e, a.T * a.k);
  wait_for(&a.sync[SY_PREP], a.n_prep, &a.sync[SY_ERR]);

  for (int cg = 0; cg * NT * 8 < ne; ++cg) {
    BCol bc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int c = cg * NT * 8 + n * 8 + (i16 >> 1);
      bc[n].on = c < ne;
      const int slot = bc[n].on ? S.slots[c] : 0;
      const int vec = a.prep_per_slot ? slot : slot / a.k;
      const size_t col = (size_t)vec * 2 + (i16 & 1);
      bc[n].q = a.xq + col * a.x_steps * 128 + g * 32;
      bc[n].s = a.xs + col * a.x_steps * 4 + g;
    }
    v4f acc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = v4f{0.f, 0.f, 0.f, 0.f};
    if (cg > 0) start_tile<ALIGNED>(ts, rowp, srow, wpr, nb, g);
    mma_tile<NT, ALIGNED>(ts, bc, acc, lane);
    dump_acc<NT>(S, acc, wave, lane);
    __syncthreads();
    const int ncol = min(ne - cg * NT * 8, NT * 8);
    if (!ffn) {
      for (int idx = threadIdx.x; idx < ncol * 64; idx += kThreads) {
        const int c = idx >> 6, rr = idx & 63, w = rr >> 4, ri = rr & 15;
        if (rg * 64 + rr >= a.rows1) continue;
        const int n = c >> 3, cj = 2 * (c & 7);
        const float v = S.red[d_index<NT>(w, n, ri, cj)] + S.red[d_index<NT>(w, n, ri, cj + 1)];
        a.y[(size_t)S.slots[cg * NT * 8 + c] * a.rows1 + rg * 64 + rr] = v;
      }
    } else {
      for (int base = 0; base < ncol; base += kThreads / 32) {
        const int c = base + (threadIdx.x >> 5), i = threadIdx.x & 31;
        const bool live = c < ncol;
        float hv = 0.0f;
        int slot = 0;
        if (live) {
          const int n = c >> 3, cj = 2 * (c & 7), w = i >> 4, ri = i & 15;
          const float gate = S.red[d_index<NT>(w, n, ri, cj)] + S.red[d_index<NT>(w, n, ri, cj + 1)];
          const float up = S.red[d_index<NT>(w + 2, n, ri, cj)] + S.red[d_index<NT>(w + 2, n, ri, cj + 1)];
          const float silu = gate / (1.0f + expf(-gate));
          const uint16_t hb = f32_to_bf16_rne(silu * up);
          slot = S.slots[cg * NT * 8 + c];
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
  signal(&a.sync[SY_S1]);
}

template <int NT, bool ALIGNED>
__device__ __forceinline__ void stage2_item(const LayerArgs &a, Shared &S, int rt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int wpr = a.cols2 / 16, nb = a.cols2 / 32;
  const int n_act = S.n_active;
  const bool ffn = a.mode == MODE_FFN;
  const uint8_t *bq = ffn ? a.hq : a.xq;
  const uint8_t *bsc = ffn ? a.hs : a.xs;
  const int bsteps = ffn ? a.h_steps : a.x_steps;
  v4f acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = v4f{0.f, 0.f, 0.f, 0.f};
  TileStream ts;
  bool waited = false;
  for (int ai = wave; ai < n_act || !waited; ai += kWaves) {
    const bool have = ai < n_act;
    const int e = have ? S.active[ai] : 0;
    const size_t row = (size_t)e * a.rows2 + rt * 16 + i16;
    const uint32_t *rowp = have ? a.w2 + row * wpr : nullptr;
    const uint8_t *srow = a.s2 + row * nb;
    if (have) start_tile<ALIGNED>(ts, rowp, srow, wpr, nb, g);
    if (!waited) {
      // every wave reaches this once (block-wide barrier inside)
      if (ffn) wait_for(&a.sync[SY_S1], a.n_s1, &a.sync[SY_ERR]);
      else wait_for(&a.sync[SY_PREP], a.n_prep, &a.sync[SY_ERR]);
      waited = true;
    }
    if (!have) break;
    BCol bc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int t = n * 8 + (i16 >> 1);
      int slot = -1;
      if (t < a.T)
        for (int jj = 0; jj < a.k; ++jj)
          if (S.ids[t * a.k + jj] == e) { slot = t * a.k + jj; break; }
      bc[n].on = slot >= 0;
      const size_t col = (size_t)(slot < 0 ? 0 : slot) * 2 + (i16 & 1);
      bc[n].q = bq + col * bsteps * 128 + g * 32;
      bc[n].s = bsc + col * bsteps * 4 + g;
    }
    mma_tile<NT, ALIGNED>(ts, bc, acc, lane);
  }
  dump_acc<NT>(S, acc, wave, lane);
  __syncthreads();
  for (int idx = threadIdx.x; idx < a.T * 16; idx += kThreads) {
    const int t = idx >> 4, ri = idx & 15;
    const int n = t >> 3, cj = 2 * (t & 7);
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += S.red[d_index<NT>(w, n, ri, cj)] + S.red[d_index<NT>(w, n, ri, cj + 1)];
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

  const int n_items = a.n_prep + a.n_s1 + a.n_s2;
  for (int item = blockIdx.x; item < n_items; item += a.grid) {
    if (item < a.n_prep) {
      prep_item(a, S, item);
      signal(&a.sync[SY_PREP]);
    } else if (item < a.n_prep + a.n_s1) {
      stage1_item<NT, ALIGNED>(a, S, item - a.n_prep);
    } else {
      stage2_item<NT, ALIGNED>(a, S, item - a.n_prep - a.n_s1);
    }
    __syncthreads();
  }
  // the last workgroup out publishes the status and clears the counters
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    if (atomicAdd(&a.sync[SY_EXIT], 1) == a.grid - 1) {
      __threadfence();
      const int skipped = __hip_atomic_load(&a.sync[SY_SKIP], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int err = __hip_atomic_load(&a.sync[SY_ERR], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.sync[ST_SKIPPED], skipped, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.sync[ST_ERROR], err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int i = SY_PREP; i <= SY_ERR; ++i)
        __hip_atomic_store(&a.sync[i], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __threadfence();
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

// tq_moe.hip -- fused trellis-decode mixture-of-experts GEMV on gfx950.
//
// HEPH abstract (ICLR 2027 submission page): in "fused" serving the
// compressed streams stay resident and each weight is decoded inside the
// grouped-MoE kernel on every forward pass. Here the decoded E2M1 nibbles go
// straight into the FP4 x FP8 block-scaled matrix cores (the UE8M0 exponents
// of the weights are the A scales), at every batch size: the decoder keeps
// the vector ALUs busy and the matrix cores take the multiply-accumulate.
//
// Per call:
//   k_prep      routing tables (per-expert slot lists, active experts, a
//               (expert, token) -> slot map) and the activations in MFMA-B
//               layout: each vector split into two FP8 E4M3 terms (hi + lo)
//               with a UE8M0 scale per 32, optionally pre-multiplied by the
//               slot's gate weight.
//   k_slots     one unit = one active expert x 64 output rows, columns = the
//               slots routed to that expert. Epilogue: plain per-slot output,
//               or SwiGLU (32 gate rows + the matching 32 up rows) writing h
//               in bf16 and its FP8 hi/lo copy for the down projection.
//   k_combine   one unit = 16 output rows, looping over all active experts;
//               columns = tokens; the gate weights are already folded into
//               the activations, so the weighted sum over a token's experts
//               happens in the accumulator (deterministic, no atomics).
// Inside a unit the waves of a workgroup split the (expert, K-chunk)
// iteration space and reduce their accumulators through LDS.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>

#include "tq_common.h"

namespace tq {

constexpr int kWaves = 4;            // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxT = 32;
constexpr int kMaxK = 32;
constexpr int kMaxSlots = 1024;

// ---------------------------------------------------------------- workspace

struct Layout {
  size_t status, counts, active, n_active, slot_off, slot_list, tok_slot, gsum;
  size_t xq, xs, hq, hs;  // activation buffers (x for the first GEMV, h for the down GEMV)
  size_t total;
};

static inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// x_vecs / x_cols: vectors and width of the first GEMV's activations;
// h_vecs / h_cols: same for the second (down) GEMV, 0 if none.
static Layout make_layout(int E, int T, int k, int x_vecs, int x_cols, int h_vecs, int h_cols) {
  Layout L;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align256(o + bytes); return r; };
  L.status = take(64);
  L.counts = take(sizeof(int) * (size_t)E);
  L.active = take(sizeof(int) * (size_t)E);
  L.n_active = take(sizeof(int));
  L.slot_off = take(sizeof(int) * (size_t)(E + 1));
  L.slot_list = take(sizeof(int) * (size_t)T * k);
  L.tok_slot = take(sizeof(int) * (size_t)E * T);
  L.gsum = take(sizeof(float) * (size_t)T * k);
  const size_t xch = (size_t)(x_cols / 32 + 3) / 4;
  L.xq = take((size_t)x_vecs * 2 * xch * 128);
  L.xs = take((size_t)x_vecs * 2 * xch * 4);
  const size_t hch = h_cols ? (size_t)(h_cols / 32 + 3) / 4 : 0;
  L.hq = take((size_t)h_vecs * 2 * hch * 128);
  L.hs = take((size_t)h_vecs * 2 * hch * 4);
  L.total = o;
  return L;
}

struct Tables {
  int *status, *counts, *active, *n_active, *slot_off, *slot_list, *tok_slot;
  float *gsum;
};

static Tables tables_at(void *ws, const Layout &L) {
  char *b = (char *)ws;
  Tables t;
  t.status = (int *)(b + L.status);
  t.counts = (int *)(b + L.counts);
  t.active = (int *)(b + L.active);
  t.n_active = (int *)(b + L.n_active);
  t.slot_off = (int *)(b + L.slot_off);
  t.slot_list = (int *)(b + L.slot_list);
  t.tok_slot = (int *)(b + L.tok_slot);
  t.gsum = (float *)(b + L.gsum);
  return t;
}

// ---------------------------------------------------------------- prep

struct PrepArgs {
  Tables tb;
  const int32_t *ids;
  const float *gate_w;  // may be null (all ones)
  int T, k, E;
  // activation quantization
  const void *x;
  int x_bf16;
  int x_per_slot;       // x is [T][k][K] (else [T][K])
  int per_slot_out;     // one output vector per slot (else per token)
  int fold;             // multiply by the combined gate weight of the slot
  int K, nchunk;
  uint8_t *xq, *xs;
  // zeroing of outputs that belong to dead (empty or skipped) slots
  float *y_slots;       // [T][k][rows] or null
  int y_rows;
  uint16_t *h;          // [T][k][h_cols] or null
  int h_cols;
  // padded K blocks (past h_cols/32, up to 4*h_nchunk) of the down activations
  uint8_t *hq, *hs;
  int h_nchunk;
};

__device__ __forceinline__ float load_x(const void *x, int bf16, size_t i) {
  return bf16 ? bf16_to_f32(((const uint16_t *)x)[i]) : ((const float *)x)[i];
}

// Quantize one 32-element block v[0..31] (held by the 32 lanes of a half-wave,
// lane = position within the block) to the two-term FP8 split and store it in
// B layout. `col` is the vector's column base (already includes hi/lo * 0).
__device__ __forceinline__ void quantize_block_halfwave(float v, int pos, int blk, uint8_t *q_hi,
                                                        uint8_t *q_lo, uint8_t *s_hi,
                                                        uint8_t *s_lo) {
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
  const int chunk = blk >> 2, beta = blk & 3;
  const int off = chunk * 128 + bchunk_offset(canonical_k(beta, pos));
  q_hi[off] = (uint8_t)hi;
  q_lo[off] = (uint8_t)lo;
  if (pos == 0) {
    s_hi[blk] = (uint8_t)(E + 127);
    s_lo[blk] = (uint8_t)(El + 127);
  }
}

// Block 0 builds the routing tables; blocks 1.. quantize activation vectors.
__global__ void __launch_bounds__(kThreads) k_prep(PrepArgs a) {
  const int tid = threadIdx.x;
  if (blockIdx.x == 0) {
    __shared__ int s_ids[kMaxSlots];
    __shared__ int s_cnt[1024];
    const int n = a.T * a.k;
    for (int i = tid; i < n; i += kThreads) s_ids[i] = a.ids[i];
    if (tid == 0) a.tb.status[0] = 0;
    __syncthreads();
    // each thread owns experts e = tid, tid + 256, ...: count, and list slots in slot order
    for (int e = tid; e < a.E; e += kThreads) {
      int c = 0;
      for (int i = 0; i < n; ++i) c += (s_ids[i] == e);
      s_cnt[e] = c;
      a.tb.counts[e] = c;
    }
    int skipped = 0;
    for (int i = tid; i < n; i += kThreads) skipped += (s_ids[i] >= a.E);
    if (skipped) atomicAdd(&a.tb.status[0], skipped);
    __syncthreads();
    if (tid == 0) {
      int na = 0, off = 0;
      for (int e = 0; e < a.E; ++e) {
        if (s_cnt[e] > 0) {
          a.tb.active[na] = e;
          a.tb.slot_off[na] = off;
          s_cnt[e] = off;  // reuse as this expert's list offset
          off += a.tb.counts[e];
          ++na;
        } else {
          s_cnt[e] = -1;
        }
      }
      a.tb.slot_off[na] = off;
      a.tb.n_active[0] = na;
    }
    __syncthreads();
    for (int e = tid; e < a.E; e += kThreads) {
      for (int t = 0; t < a.T; ++t) a.tb.tok_slot[e * a.T + t] = -1;
      int o = s_cnt[e];
      if (o < 0) continue;
      for (int i = 0; i < n; ++i) {
        if (s_ids[i] != e) continue;
        a.tb.slot_list[o++] = i;
        const int t = i / a.k;
        // the first slot of (token, expert) is canonical; duplicates fold into it
        if (a.tb.tok_slot[e * a.T + t] < 0) a.tb.tok_slot[e * a.T + t] = i;
      }
    }
    __syncthreads();
    // combined gate weight per slot: canonical slots carry the sum over duplicates
    for (int i = tid; i < n; i += kThreads) {
      const int e = s_ids[i];
      float g = 0.0f;
      if (e >= 0 && e < a.E) {
        const int t = i / a.k;
        if (a.tb.tok_slot[e * a.T + t] == i)
          for (int j = 0; j < a.k; ++j)
            if (s_ids[t * a.k + j] == e) g += a.gate_w ? a.gate_w[t * a.k + j] : 1.0f;
      }
      a.tb.gsum[i] = g;
      const bool dead = e < 0 || e >= a.E;
      if (dead && a.y_slots)
        for (int r = 0; r < a.y_rows; ++r) a.y_slots[(size_t)i * a.y_rows + r] = 0.0f;
      if (dead && a.h)
        for (int c = 0; c < a.h_cols; ++c) a.h[(size_t)i * a.h_cols + c] = 0;
      if (a.hq) {
        // zero B data and give a finite scale to the K padding of both terms
        for (int hl = 0; hl < 2; ++hl) {
          const size_t col = (size_t)i * 2 + hl;
          for (int blk = a.h_cols / 32; blk < 4 * a.h_nchunk; ++blk) {
            a.hs[col * a.h_nchunk * 4 + blk] = 127;
            for (int p = 0; p < 32; ++p)
              a.hq[(col * a.h_nchunk + (blk >> 2)) * 128 + bchunk_offset(canonical_k(blk & 3, p))] = 0;
          }
          if (dead) {
            // a dead slot's vector is never read, but keep it finite
            for (int blk = 0; blk < a.h_cols / 32; ++blk) a.hs[col * a.h_nchunk * 4 + blk] = 127;
            for (int b = 0; b < a.h_nchunk * 128; ++b) a.hq[col * a.h_nchunk * 128 + b] = 0;
          }
        }
      }
    }
    return;
  }
  // ---- activation vectors: blockIdx.x - 1 = output vector index
  const int v = blockIdx.x - 1;
  const int nb = a.K / 32;
  uint8_t *q_hi = a.xq + ((size_t)v * 2 + 0) * a.nchunk * 128;
  uint8_t *q_lo = a.xq + ((size_t)v * 2 + 1) * a.nchunk * 128;
  uint8_t *s_hi = a.xs + ((size_t)v * 2 + 0) * a.nchunk * 4;
  uint8_t *s_lo = a.xs + ((size_t)v * 2 + 1) * a.nchunk * 4;
  // Which source rows feed this vector, with which weight. Per token: x[t].
  // Per slot without folding: the slot's own input. Per slot with folding:
  // the canonical slot of a (token, expert) pair carries
  // sum_j gate_w[t][j] * x_(t or t,j) over the token's slots with that
  // expert; other slots of the pair (and dead slots) get a zero vector.
  int t = v, j0 = 0, n_src = 1;
  if (a.per_slot_out) {
    t = v / a.k;
    j0 = v % a.k;
    if (a.fold) {
      const int e = a.ids[v];
      bool canonical = e >= 0 && e < a.E;
      for (int jj = 0; jj < j0 && canonical; ++jj) canonical = a.ids[t * a.k + jj] != e;
      n_src = canonical ? a.k : 0;
    }
  }
  const int pos = tid & 31;
  for (int blk = tid >> 5; blk < a.nchunk * 4; blk += kThreads / 32) {
    float x = 0.0f;
    if (blk < nb) {
      const size_t off = (size_t)blk * 32 + pos;
      if (!a.per_slot_out) {
        x = load_x(a.x, a.x_bf16, (size_t)t * a.K + off);
      } else if (!a.fold) {
        x = load_x(a.x, a.x_bf16, (size_t)(a.x_per_slot ? v : t) * a.K + off);
      } else {
        const int e = a.ids[v];
        for (int jj = 0; jj < n_src; ++jj) {
          if (a.ids[t * a.k + jj] != e) continue;
          const float gw = a.gate_w ? a.gate_w[t * a.k + jj] : 1.0f;
          x += gw * load_x(a.x, a.x_bf16, (size_t)(a.x_per_slot ? t * a.k + jj : t) * a.K + off);
        }
      }
    }
    quantize_block_halfwave(x, pos, blk, q_hi, q_lo, s_hi, s_lo);
  }
}

// ---------------------------------------------------------------- fused GEMV

// One lane's share of a 16-row tile for one 128-K chunk: the two symbol words
// of its 32-weight block, the word before them (decoder history; 0 at a row
// start) and the block's UE8M0 byte.
struct ALoad {
  uint2 w;
  uint32_t hist;
  uint32_t scale;
};

__device__ __forceinline__ ALoad load_a(const uint32_t *row_words, const uint8_t *row_scales,
                                        int blk, bool ok) {
  ALoad r;
  r.w = make_uint2(0u, 0u);
  r.hist = 0u;
  r.scale = 127u;
  if (ok) {
    r.w = *(const uint2 *)(row_words + 2 * blk);
    if (blk > 0) r.hist = row_words[2 * blk - 1];
    r.scale = row_scales[blk];
  }
  return r;
}

__device__ __forceinline__ v8i decode_a(const ALoad &l) {
  const nib2 n0 = decode_word(l.w.x, l.hist);
  const nib2 n1 = decode_word(l.w.y, l.w.x);
  v8i a;
  a[0] = (int)n0.even;
  a[1] = (int)n0.odd;
  a[2] = (int)n1.even;
  a[3] = (int)n1.odd;
  a[4] = a[5] = a[6] = a[7] = 0;
  return a;
}

struct BLoad {
  v8i q;
  uint32_t scale;
};

__device__ __forceinline__ BLoad load_b(const uint8_t *q, const uint8_t *sc, bool on) {
  BLoad r;
  if (on) {
    const uint4 *p = (const uint4 *)q;
    const uint4 u0 = p[0], u1 = p[1];
    r.q[0] = (int)u0.x; r.q[1] = (int)u0.y; r.q[2] = (int)u0.z; r.q[3] = (int)u0.w;
    r.q[4] = (int)u1.x; r.q[5] = (int)u1.y; r.q[6] = (int)u1.z; r.q[7] = (int)u1.w;
    r.scale = *sc;
  } else {
    r.q = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    r.scale = 127u;
  }
  return r;
}

// Index of D(tile, ntile, row, col) in the [tile][ntile][lane][reg] accumulator dump.
template <int NT>
__device__ __forceinline__ int d_index(int tile, int nt, int row, int col) {
  const int lane = (row >> 2) * 16 + col;
  return ((tile * NT + nt) * 64 + lane) * 4 + (row & 3);
}

// Cross-wave sum of the accumulators: every wave dumps its [NTILE][NT] tiles
// to LDS; the result replaces wave 0's copy.
template <int NTILE, int NT>
__device__ __forceinline__ void reduce_waves(v4f (&acc)[NTILE][NT], float *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int N = NTILE * NT * 256;
#pragma unroll
  for (int t = 0; t < NTILE; ++t)
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave * N + ((t * NT + n) * 64 + lane) * 4 + r] = acc[t][n][r];
  __syncthreads();
  for (int i = threadIdx.x; i < N; i += kThreads) {
    float s = red[i];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) s += red[w * N + i];
    red[i] = s;
  }
  __syncthreads();
}

struct MatArgs {
  const uint32_t *syms;
  const uint8_t *scales;
  int rows, cols;
};

struct SlotArgs {
  MatArgs w;
  Tables tb;
  int k, nchunk;
  int vec_per_slot;           // activation vector = slot (else token = slot / k)
  const uint8_t *xq, *xs;
  // MODE 0: per-slot output y[slot][rows]
  float *y;
  // MODE 1 (SwiGLU; rows = 2 * inter): h[slot][inter] in bf16 and its FP8 copy
  int inter;
  uint16_t *h;
  uint8_t *hq, *hs;
  int h_nchunk;
};

// MODE 0: unit = 64 consecutive rows. MODE 1: unit = 32 gate rows and the
// matching 32 up rows.
template <int NT, int MODE>
__global__ void __launch_bounds__(kThreads) k_slots(SlotArgs a) {
  constexpr int NTILE = 4;
  __shared__ float red[kWaves * NTILE * NT * 256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int rows = a.w.rows, wpr = a.w.cols / 16, spr = a.w.cols / 32, nb = a.w.cols / 32;
  const int n_rg = MODE == 0 ? (rows + 63) / 64 : a.inter / 32;
  const int ai = blockIdx.x / n_rg, rg = blockIdx.x % n_rg;
  if (ai >= *a.tb.n_active) return;
  const int e = a.tb.active[ai];
  const int s0 = a.tb.slot_off[ai], ne = a.tb.slot_off[ai + 1] - s0;

  const uint32_t *wrow[NTILE];
  const uint8_t *srow[NTILE];
  bool tok[NTILE];
#pragma unroll
  for (int t = 0; t < NTILE; ++t) {
    const int r0 = MODE == 0 ? rg * 64 + 16 * t : (t < 2 ? 0 : a.inter) + rg * 32 + 16 * (t & 1);
    tok[t] = r0 < rows;
    const size_t row = (size_t)e * rows + (tok[t] ? r0 + i16 : 0);
    wrow[t] = a.w.syms + row * wpr;
    srow[t] = a.w.scales + row * spr;
  }
  const int nsteps = a.nchunk;
  const int per = (nsteps + kWaves - 1) / kWaves;
  const int S0 = wave * per, S1 = min(nsteps, S0 + per);

  for (int cg = 0; cg * NT * 8 < ne; ++cg) {
    const uint8_t *bq[NT];
    const uint8_t *bs[NT];
    bool bon[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int c = cg * NT * 8 + n * 8 + (i16 >> 1);
      bon[n] = c < ne;
      const int slot = bon[n] ? a.tb.slot_list[s0 + c] : 0;
      const int vec = a.vec_per_slot ? slot : slot / a.k;
      const size_t col = (size_t)vec * 2 + (i16 & 1);
      bq[n] = a.xq + col * a.nchunk * 128 + g * 32;
      bs[n] = a.xs + col * a.nchunk * 4 + g;
    }
    v4f acc[NTILE][NT];
#pragma unroll
    for (int t = 0; t < NTILE; ++t)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[t][n] = v4f{0.f, 0.f, 0.f, 0.f};

    ALoad la[NTILE];
    BLoad lb[NT];
    if (S0 < S1) {
      const int blk = 4 * S0 + g;
#pragma unroll
      for (int t = 0; t < NTILE; ++t) la[t] = load_a(wrow[t], srow[t], blk, tok[t] && blk < nb);
#pragma unroll
      for (int n = 0; n < NT; ++n) lb[n] = load_b(bq[n] + S0 * 128, bs[n] + S0 * 4, bon[n]);
    }
    for (int S = S0; S < S1; ++S) {
      ALoad na[NTILE];
      BLoad nbl[NT];
      if (S + 1 < S1) {
        const int blk = 4 * (S + 1) + g;
#pragma unroll
        for (int t = 0; t < NTILE; ++t) na[t] = load_a(wrow[t], srow[t], blk, tok[t] && blk < nb);
#pragma unroll
        for (int n = 0; n < NT; ++n) nbl[n] = load_b(bq[n] + (S + 1) * 128, bs[n] + (S + 1) * 4, bon[n]);
      }
#pragma unroll
      for (int t = 0; t < NTILE; ++t) {
        const v8i A = decode_a(la[t]);
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[t][n] = mfma_fp4_fp8(A, lb[n].q, acc[t][n], (int)la[t].scale, (int)lb[n].scale);
      }
      if (S + 1 < S1) {
#pragma unroll
        for (int t = 0; t < NTILE; ++t) la[t] = na[t];
#pragma unroll
        for (int n = 0; n < NT; ++n) lb[n] = nbl[n];
      }
    }
    reduce_waves<NTILE, NT>(acc, red);

    const int ncol = min(ne - cg * NT * 8, NT * 8);
    if (MODE == 0) {
      for (int idx = threadIdx.x; idx < ncol * 64; idx += kThreads) {
        const int c = idx >> 6, rr = idx & 63, t = rr >> 4, ri = rr & 15;
        if (rg * 64 + rr >= rows) continue;
        const int n = c >> 3, cj = 2 * (c & 7);
        const float v = red[d_index<NT>(t, n, ri, cj)] + red[d_index<NT>(t, n, ri, cj + 1)];
        const int slot = a.tb.slot_list[s0 + cg * NT * 8 + c];
        a.y[(size_t)slot * rows + rg * 64 + rr] = v;
      }
    } else {
      // half-wave per slot: lane = position i in this 32-row block of h
      for (int base = 0; base < ncol; base += kThreads / 32) {
        const int c = base + (threadIdx.x >> 5), i = threadIdx.x & 31;
        const bool live = c < ncol;
        float hv = 0.0f;
        int slot = 0;
        if (live) {
          const int n = c >> 3, cj = 2 * (c & 7), t = i >> 4, ri = i & 15;
          const float gate = red[d_index<NT>(t, n, ri, cj)] + red[d_index<NT>(t, n, ri, cj + 1)];
          const float up = red[d_index<NT>(t + 2, n, ri, cj)] + red[d_index<NT>(t + 2, n, ri, cj + 1)];
          const float silu = gate / (1.0f + expf(-gate));
          const uint16_t hb = f32_to_bf16_rne(silu * up);
          slot = a.tb.slot_list[s0 + cg * NT * 8 + c];
          a.h[(size_t)slot * a.inter + rg * 32 + i] = hb;
          hv = bf16_to_f32(hb) * a.tb.gsum[slot];
        }
        // all 32 lanes of the half-wave take part in the block reductions;
        // only live ones store
        float amax = fabsf(hv);
#pragma unroll
        for (int m = 16; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 32));
        const int E = block_exponent(amax);
        const uint32_t hi = f32_to_e4m3(ldexpf(hv, -E));
        const float r = hv - ldexpf(e4m3_to_f32(hi), E);
        float rmax = fabsf(r);
#pragma unroll
        for (int m = 16; m >= 1; m >>= 1) rmax = fmaxf(rmax, __shfl_xor(rmax, m, 32));
        const int El = block_exponent(rmax);
        const uint32_t lo = f32_to_e4m3(ldexpf(r, -El));
        if (live) {
          const int off = (rg >> 2) * 128 + bchunk_offset(canonical_k(rg & 3, i));
          uint8_t *qh = a.hq + ((size_t)slot * 2 + 0) * a.h_nchunk * 128;
          uint8_t *ql = a.hq + ((size_t)slot * 2 + 1) * a.h_nchunk * 128;
          qh[off] = (uint8_t)hi;
          ql[off] = (uint8_t)lo;
          if (i == 0) {
            a.hs[((size_t)slot * 2 + 0) * a.h_nchunk * 4 + rg] = (uint8_t)(E + 127);
            a.hs[((size_t)slot * 2 + 1) * a.h_nchunk * 4 + rg] = (uint8_t)(El + 127);
          }
        }
      }
    }
    __syncthreads();
  }
}

struct CombArgs {
  MatArgs w;
  Tables tb;
  int T, nchunk;
  const uint8_t *xq, *xs;   // per-slot activation vectors, gate weight folded in
  float *y;                 // [T][rows]
};

// Unit = 16 output rows; the waves split the (active expert, K-chunk) space;
// column pair (2t, 2t+1) = token t's hi/lo terms.
template <int NT>
__global__ void __launch_bounds__(kThreads) k_combine(CombArgs a) {
  __shared__ float red[kWaves * NT * 256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int rows = a.w.rows, wpr = a.w.cols / 16, spr = a.w.cols / 32, nb = a.w.cols / 32;
  const int r0 = blockIdx.x * 16;
  const int n_active = *a.tb.n_active;
  const int nsteps = a.nchunk;
  const int total = n_active * nsteps;
  const int per = (total + kWaves - 1) / kWaves;
  const int I0 = wave * per, I1 = min(total, I0 + per);

  v4f acc[1][NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[0][n] = v4f{0.f, 0.f, 0.f, 0.f};

  auto fetch = [&](int it, ALoad &la, BLoad (&lb)[NT]) {
    const int ai = it / nsteps, S = it - ai * nsteps;
    const int e = a.tb.active[ai];
    const size_t row = (size_t)e * rows + r0 + i16;
    const int blk = 4 * S + g;
    la = load_a(a.w.syms + row * wpr, a.w.scales + row * spr, blk, blk < nb);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int t = n * 8 + (i16 >> 1);
      const int slot = t < a.T ? a.tb.tok_slot[e * a.T + t] : -1;
      const size_t col = (size_t)(slot < 0 ? 0 : slot) * 2 + (i16 & 1);
      lb[n] = load_b(a.xq + (col * a.nchunk + S) * 128 + g * 32, a.xs + col * a.nchunk * 4 + 4 * S + g,
                     slot >= 0);
    }
  };

  ALoad la;
  BLoad lb[NT];
  if (I0 < I1) fetch(I0, la, lb);
  for (int it = I0; it < I1; ++it) {
    ALoad na;
    BLoad nbl[NT];
    if (it + 1 < I1) fetch(it + 1, na, nbl);
    const v8i A = decode_a(la);
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[0][n] = mfma_fp4_fp8(A, lb[n].q, acc[0][n], (int)la.scale, (int)lb[n].scale);
    if (it + 1 < I1) {
      la = na;
#pragma unroll
      for (int n = 0; n < NT; ++n) lb[n] = nbl[n];
    }
  }
  reduce_waves<1, NT>(acc, red);
  for (int idx = threadIdx.x; idx < a.T * 16; idx += kThreads) {
    const int t = idx >> 4, ri = idx & 15;
    const int n = t >> 3, cj = 2 * (t & 7);
    a.y[(size_t)t * rows + r0 + ri] = red[d_index<NT>(0, n, ri, cj)] + red[d_index<NT>(0, n, ri, cj + 1)];
  }
}

// ---------------------------------------------------------------- host side

static int device_check() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return TRELLIS_EHIP;
  if (cached[dev] == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return TRELLIS_EHIP;
    cached[dev] = (strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
  }
  return cached[dev] > 0 ? TRELLIS_OK : TRELLIS_EDEVICE;
}

static int check_mat(const trellis_mat_t *w, bool gemv) {
  if (!w || !w->syms || !w->scales) return TRELLIS_ENULL;
  if (w->n_mat < 1 || w->rows < 1 || w->cols < 32 || w->cols % 32) return TRELLIS_EINVAL;
  if (gemv && (w->rows % 16 || w->n_mat > 1024)) return TRELLIS_EINVAL;
  return TRELLIS_OK;
}

static int check_routing(int T, int k) {
  if (T < 1 || T > kMaxT || k < 1 || k > kMaxK || T * k > kMaxSlots) return TRELLIS_EINVAL;
  return TRELLIS_OK;
}

static int launch_status() { return hipGetLastError() == hipSuccess ? TRELLIS_OK : TRELLIS_EHIP; }

static int nt_for(int T) { return (T + 7) / 8; }

template <int MODE>
static void launch_slots(int NT, dim3 grid, hipStream_t s, const SlotArgs &a) {
  switch (NT) {
    case 1: hipLaunchKernelGGL((k_slots<1, MODE>), grid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_slots<2, MODE>), grid, dim3(kThreads), 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_slots<3, MODE>), grid, dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL((k_slots<4, MODE>), grid, dim3(kThreads), 0, s, a); break;
  }
}

static void launch_combine(int NT, dim3 grid, hipStream_t s, const CombArgs &a) {
  switch (NT) {
    case 1: hipLaunchKernelGGL((k_combine<1>), grid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_combine<2>), grid, dim3(kThreads), 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_combine<3>), grid, dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL((k_combine<4>), grid, dim3(kThreads), 0, s, a); break;
  }
}

static Layout gemv_layout(const trellis_mat_t *w, int T, int k, bool per_slot) {
  const int vecs = per_slot ? T * k : T;
  return make_layout(w->n_mat, T, k, vecs, w->cols, 0, 0);
}

}  // namespace tq

using namespace tq;

extern "C" size_t trellis_moe_gemv_workspace_size(int32_t n_mat, int32_t rows, int32_t cols, int32_t T,
                                                  int32_t k) {
  if (n_mat < 1 || cols < 32 || cols % 32 || rows < 1 || check_routing(T, k)) return 0;
  // per-slot vectors cover every variant of the call
  return make_layout(n_mat, T, k, T * k, cols, 0, 0).total;
}

extern "C" int trellis_moe_gemv(hipStream_t stream, const trellis_mat_t *w, const void *x, int32_t x_dtype,
                                int32_t x_per_slot, const int32_t *topk_ids, const float *topk_w,
                                int32_t T, int32_t k, float *y, void *workspace, size_t workspace_bytes) {
  int rc = check_mat(w, true);
  if (rc) return rc;
  if (!x || !topk_ids || !y || !workspace) return TRELLIS_ENULL;
  if ((x_dtype != TRELLIS_F32 && x_dtype != TRELLIS_BF16) || (x_per_slot != 0 && x_per_slot != 1))
    return TRELLIS_EINVAL;
  if ((rc = check_routing(T, k))) return rc;
  const bool combine = topk_w != nullptr;
  const bool per_slot = combine || x_per_slot;
  const Layout L = gemv_layout(w, T, k, per_slot);
  if (((uintptr_t)workspace & 255) || workspace_bytes < L.total) return TRELLIS_EWORKSPACE;
  if ((rc = device_check())) return rc;

  Tables tb = tables_at(workspace, L);
  char *ws = (char *)workspace;
  const int nchunk = (w->cols / 32 + 3) / 4;
  PrepArgs p{};
  p.tb = tb; p.ids = topk_ids; p.gate_w = topk_w; p.T = T; p.k = k; p.E = w->n_mat;
  p.x = x; p.x_bf16 = x_dtype == TRELLIS_BF16; p.x_per_slot = x_per_slot;
  p.per_slot_out = per_slot; p.fold = combine; p.K = w->cols; p.nchunk = nchunk;
  p.xq = (uint8_t *)(ws + L.xq); p.xs = (uint8_t *)(ws + L.xs);
  p.y_slots = combine ? nullptr : y; p.y_rows = w->rows;
  p.h = nullptr; p.h_cols = 0; p.hq = nullptr; p.hs = nullptr; p.h_nchunk = 0;
  const int vecs = per_slot ? T * k : T;
  hipLaunchKernelGGL(k_prep, dim3(1 + vecs), dim3(kThreads), 0, stream, p);
  if ((rc = launch_status())) return rc;

  const MatArgs m{w->syms, w->scales, w->rows, w->cols};
  const int NT = nt_for(T);
  if (!combine) {
    SlotArgs a{};
    a.w = m; a.tb = tb; a.k = k; a.nchunk = nchunk; a.vec_per_slot = per_slot;
    a.xq = p.xq; a.xs = p.xs; a.y = y;
    const int max_active = std::min(w->n_mat, T * k);
    const int n_rg = (w->rows + 63) / 64;
    launch_slots<0>(NT, dim3(max_active * n_rg), stream, a);
  } else {
    CombArgs a{};
    a.w = m; a.tb = tb; a.T = T; a.nchunk = nchunk; a.xq = p.xq; a.xs = p.xs; a.y = y;
    launch_combine(NT, dim3(w->rows / 16), stream, a);
  }
  return launch_status();
}

extern "C" size_t trellis_moe_ffn_workspace_size(int32_t n_exp, int32_t hidden, int32_t inter, int32_t T,
                                                 int32_t k) {
  if (n_exp < 1 || hidden < 32 || hidden % 32 || inter < 32 || inter % 32 || check_routing(T, k)) return 0;
  return make_layout(n_exp, T, k, T, hidden, T * k, inter).total;
}

extern "C" int trellis_moe_ffn_timed(hipStream_t stream, const trellis_mat_t *w_gate_up,
                                     const trellis_mat_t *w_down, const void *x, int32_t x_dtype,
                                     const int32_t *topk_ids, const float *topk_w, int32_t T, int32_t k,
                                     uint16_t *h, float *y, void *workspace, size_t workspace_bytes,
                                     hipEvent_t *events) {
  auto mark = [&](int i) {
    if (events && events[i]) hipEventRecord(events[i], stream);
  };
  int rc;
  if ((rc = check_mat(w_gate_up, true)) || (rc = check_mat(w_down, true))) return rc;
  if (!x || !topk_ids || !h || !y || !workspace) return TRELLIS_ENULL;
  if (x_dtype != TRELLIS_F32 && x_dtype != TRELLIS_BF16) return TRELLIS_EINVAL;
  if ((rc = check_routing(T, k))) return rc;
  const int E = w_gate_up->n_mat, hidden = w_gate_up->cols, inter = w_gate_up->rows / 2;
  if (w_gate_up->rows % 64 || w_down->n_mat != E || w_down->rows != hidden || w_down->cols != inter)
    return TRELLIS_EINVAL;
  const Layout L = make_layout(E, T, k, T, hidden, T * k, inter);
  if (((uintptr_t)workspace & 255) || workspace_bytes < L.total) return TRELLIS_EWORKSPACE;
  if ((rc = device_check())) return rc;

  Tables tb = tables_at(workspace, L);
  char *ws = (char *)workspace;
  const int xch = (hidden / 32 + 3) / 4, hch = (inter / 32 + 3) / 4;
  PrepArgs p{};
  p.tb = tb; p.ids = topk_ids; p.gate_w = topk_w; p.T = T; p.k = k; p.E = E;
  p.x = x; p.x_bf16 = x_dtype == TRELLIS_BF16; p.x_per_slot = 0; p.per_slot_out = 0; p.fold = 0;
  p.K = hidden; p.nchunk = xch; p.xq = (uint8_t *)(ws + L.xq); p.xs = (uint8_t *)(ws + L.xs);
  p.y_slots = nullptr; p.h = h; p.h_cols = inter;
  p.hq = (uint8_t *)(ws + L.hq); p.hs = (uint8_t *)(ws + L.hs); p.h_nchunk = hch;
  mark(0);
  hipLaunchKernelGGL(k_prep, dim3(1 + T), dim3(kThreads), 0, stream, p);
  if ((rc = launch_status())) return rc;

  const int NT = nt_for(T);
  SlotArgs a{};
  a.w = MatArgs{w_gate_up->syms, w_gate_up->scales, w_gate_up->rows, hidden};
  a.tb = tb; a.k = k; a.nchunk = xch; a.vec_per_slot = 0; a.xq = p.xq; a.xs = p.xs;
  a.inter = inter; a.h = h; a.hq = (uint8_t *)(ws + L.hq); a.hs = (uint8_t *)(ws + L.hs); a.h_nchunk = hch;
  const int max_active = std::min(E, T * k);
  mark(1);
  launch_slots<1>(NT, dim3(max_active * (inter / 32)), stream, a);
  if ((rc = launch_status())) return rc;

  CombArgs c{};
  c.w = MatArgs{w_down->syms, w_down->scales, hidden, inter};
  c.tb = tb; c.T = T; c.nchunk = hch; c.xq = a.hq; c.xs = a.hs; c.y = y;
  mark(2);
  launch_combine(NT, dim3(hidden / 16), stream, c);
  mark(3);
  return launch_status();
}

extern "C" int trellis_moe_ffn(hipStream_t stream, const trellis_mat_t *w_gate_up, const trellis_mat_t *w_down,
                               const void *x, int32_t x_dtype, const int32_t *topk_ids, const float *topk_w,
                               int32_t T, int32_t k, uint16_t *h, float *y, void *workspace,
                               size_t workspace_bytes) {
  return trellis_moe_ffn_timed(stream, w_gate_up, w_down, x, x_dtype, topk_ids, topk_w, T, k, h, y, workspace,
                               workspace_bytes, nullptr);
}

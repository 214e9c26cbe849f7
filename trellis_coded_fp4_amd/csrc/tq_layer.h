// tq_layer.h -- fused trellis-decode mixture-of-experts GEMV / small-batch GEMM on gfx950.
//
// HEPH abstract (ICLR 2027 submission page): in "fused" serving the
// compressed streams stay resident and every weight is decoded inside the
// grouped-MoE kernel on each forward pass. Here the decoded E2M1 nibbles go
// straight into the FP4 x FP8 block-scaled matrix cores, with the weights'
// UE8M0 exponents as the A scales, at every batch size: the vector ALUs do
// the decode, the matrix cores the multiply-accumulate.
//
// One persistent launch per call; its workgroups take work items
// round-robin. An item is one active expert x 64 output rows (a 16-row tile
// per wave) of a grouped GEMM whose columns are the routing slots sent to
// that expert:
//   stage-1 items  the first (or only) matrix; the activations are split on
//                  the spot into two FP8 E4M3 terms (hi + lo, UE8M0 scale per
//                  32) in matrix-core B layout in LDS. Epilogue: per-slot
//                  output; or per-slot partial output + combine (below); or,
//                  in a layer, SwiGLU over 32 gate rows and the matching 32
//                  up rows, writing h (bf16) and its FP8 hi/lo split, which
//                  is exactly one K-block of the down projection.
//   stage-2 items  a layer's down projection; its columns are the h splits
//                  of the expert's slots, copied into LDS once every
//                  stage-1 item of that expert has finished.
// Combine: in the routed GEMV with gate weights, per-slot partial outputs
// go to the workspace and the item that arrives last at a 64-row output
// tile (a counter per tile) sums them with the gate weights, in slot order,
// into y (deterministic). In a layer, the down-projection items add their
// gate-weighted rows into y with device-scope float atomics, so the order
// of a token's k terms, and the last bits of y, can vary between calls.
//
// Synchronisation costs no grid-wide barrier: counters live one per
// 128-byte line (device-scope atomics on one address serialise), each is
// cleared by the last work item that reads it, so a workspace returns to
// zero at the end of every call. Cross-workgroup data (h splits, partial
// outputs) moves through device-coherent stores and loads; a producer waits
// for its stores to complete before it counts. The grid never exceeds the
// co-resident workgroup count and items run in index order, so every wait
// is for running work; waits are bounded and set an error word on timeout.
//
// Weight streaming: a wave owns one 16-row tile. Lane (row i, lane-group g)
// loads "piece" j = 16 bytes = blocks 8j+2g, 8j+2g+1 of its row and feeds
// them to matrix-core steps 2j and 2j+1 as K-block g (the activations are
// laid out to match). A wave instruction reads 16 rows x 64 contiguous bytes;
// up to 16 pieces (K <= 4096) are in flight at once. The tile's UE8M0 bytes
// are one contiguous run (rows are contiguous): they are fetched with a few
// 16-byte loads into the wave's LDS slot instead of one 2-byte load per
// piece. Activation loads are issued before the weight loads, because loads
// complete in issue order. The decoder history of a block is the word before
// it: from the neighbouring lane-group's piece via ds_bpermute, or the
// previous piece.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>

#include "tq_common.h"
#include "tq_tok.h"

namespace tq {

// threadIdx.x behind an empty asm: the compiler cannot see that it is the
// same value on every read, so it recomputes the lane-derived indexes where
// they are used instead of hoisting them out of the item loop. Hoisted, they
// outlive everything else in the kernel and are spilled to scratch (several
// MB of HBM writes per launch, written back at the kernel's end).
__device__ __forceinline__ int tix() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}
// Only the one-N-tile kernel spills without it; the others run faster with
// the plain index (so do the several-token activation split's loops).
template <int NT>
__device__ __forceinline__ int tidx() {
  if constexpr (NT == 1) return tix();
  else return threadIdx.x;
}

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
static_assert(kThreads == 256, "one E5M3 term-table entry per thread");
constexpr int kMaxT = 128;
constexpr int kMaxK = 32;
constexpr int kMaxSlots = 1024;
constexpr int kMaxExperts = 1024;
constexpr int kPieceMax = 16;               // pieces per register window: 16 x 256 weights
constexpr unsigned kSpinLimit = 1u << 20;   // polls (device-coherent load + sleep)
constexpr int kBBytes = 32 * 1024;          // LDS for one pass of activation columns (codes)
constexpr int kBScaleBytes = 1024;          // and their UE8M0 scales
constexpr int kAScaleBytes = 2048;          // per wave: its tile's UE8M0 bytes (16 rows x <= 128)
constexpr int kXPre = 16;                   // activation values per lane fetched ahead of the weights
constexpr int kLineInts = 32;               // one counter per 128-byte line

enum { MODE_FFN = 0, MODE_SLOTS = 1, MODE_COMBINE = 2 };

// Weight formats. A "piece" is what a lane loads with one 16-byte load from
// its row: for trellis-coded weights 8 blocks of 32 (256 two-bit symbols)
// feeding two matrix-core steps; for expanded MXFP4 weights one step's 4
// blocks (128 E2M1 nibbles, natural order). Each format has its own
// activation layout: block b of a column goes to byte offset(b, pos) of the
// step-chunk layout, its UE8M0 byte to scale_index(b).
struct FmtTrellis {
  static constexpr bool kE5M3 = false;   // UE8M0 block scales
  static constexpr int kSteps = 2;    // matrix-core steps per piece
  static constexpr int kBlocks = 8;   // 32-weight blocks per piece
  static constexpr int kWords = 2;    // 32-bit words per block
  __device__ __host__ static int offset(int b, int pos) { return act_offset(b, pos); }
  __device__ __host__ static int scale_index(int b) { return act_scale_index(b); }
  // block of step st (within a pass) whose data is K-block beta of the step
  __device__ __host__ static int block_of(int st, int beta) { return 8 * (st >> 1) + 2 * beta + (st & 1); }
};
struct FmtMx {
  static constexpr bool kE5M3 = false;
  static constexpr int kSteps = 1;
  static constexpr int kBlocks = 4;
  static constexpr int kWords = 4;
  __device__ __host__ static int offset(int b, int pos) { return (b >> 2) * 128 + bchunk_offset(32 * (b & 3) + pos); }
  __device__ __host__ static int scale_index(int b) { return b; }
  __device__ __host__ static int block_of(int st, int beta) { return 4 * st + beta; }
};
// Trellis-coded weights under E5M3 block scales: the same streams and
// layout; each matrix-core step is issued once per UE8M0 term of its A
// scale (e5m3_terms, four terms) against one accumulator.
struct FmtTrellisE5M3 : FmtTrellis {
  static constexpr bool kE5M3 = true;
};
template <typename F>
__host__ __device__ inline int fmt_steps(int nb) { return F::kSteps * ((nb + F::kBlocks - 1) / F::kBlocks); }

// int words at the start of the workspace (public)
enum { ST_SKIPPED = 0, ST_ERROR = 1 };

// Every device lambda is inlined: a real call would force the argument
// block and the live registers through scratch memory.
#define TQ_INLINE __attribute__((always_inline))

// Timeline instrumentation, compiled in only with -DTQ_TRACE: per workgroup
// 512 u64 slots of s_memrealtime stamps (entry, routing done, then ten per
// item for its first 51 items: id, start, marks 2..8, end).
#ifdef TQ_TRACE
#define TQ_MARK(S, k) do { if (tix() == 0 && (S).trp) (S).trp[k] = __builtin_amdgcn_s_memrealtime(); } while (0)
static void *g_trace = nullptr;
#else
#define TQ_MARK(S, k) do { } while (0)
#endif

struct Layout {
  size_t status, reserve, cnt1, obs1, cnt2, cntp, obsp, yslot, hq, hs, xq, xs, total;
};

static inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// n_act: first-stage completion counters (layer only); n_rt: 64-row output
// tiles that combine partial outputs and n_slots x y_rows partial outputs
// (the routed GEMV's combine; zero for the layer, which adds into y);
// h_cols: width of the h splits (layer only); n_tok x x_cols: the tokens'
// activations, split once per call for every stage-1 item.
// reserve: bytes kept right after the status words (the single-token layer
// kernel's region; zero for the routed GEMV).
template <typename F>
static Layout make_layout(int n_act, int n_rt, int n_slots, int y_rows, int h_cols, int n_tok, int x_cols,
                          size_t reserve = 0) {
  Layout L;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align256(o + bytes); return r; };
  L.status = take(256);
  L.reserve = take(reserve);
  L.cnt1 = take((size_t)n_act * kLineInts * 4);
  L.obs1 = take((size_t)n_act * kLineInts * 4);
  L.cnt2 = take((size_t)n_rt * kLineInts * 4);
  L.yslot = take((size_t)n_slots * y_rows * 4);
  const size_t hs = h_cols ? (size_t)fmt_steps<F>(h_cols / 32) : 0;
  L.hq = take((size_t)n_slots * 2 * hs * 128);
  L.hs = take((size_t)n_slots * 2 * hs * 4);
  L.cntp = take(kLineInts * 4);
  L.obsp = take(kLineInts * 4);
  const size_t xs = (size_t)fmt_steps<F>(x_cols / 32);
  L.xq = take((size_t)n_tok * 2 * xs * 128);
  L.xs = take((size_t)n_tok * 2 * xs * 4);
  L.total = o;
  return L;
}

struct LayerArgs {
  int mode;
  const uint32_t *w1; const uint8_t *s1; int rows1, cols1, fast1;   // stage-1 matrices
  const uint32_t *w2; const uint8_t *s2; int rows2, cols2, fast2;   // stage-2 matrices (layer)
  int E, T, k;
  const int32_t *ids;
  const float *gate_w;          // may be null (all ones)
  const void *x; int x_bf16; int x_per_slot;
  int inter;                    // layer: intermediate width
  uint16_t *h;                  // layer: [T][k][inter]
  int h_steps; uint8_t *hq; uint8_t *hs;
  float *yslot;                 // partial outputs [T*k][y_rows]
  float *y;                     // SLOTS: [T][k][rows1]; COMBINE / layer: [T][y_rows]
  int y_rows;
  int *status, *cnt1, *obs1, *cnt2;
  int n_rg1, n_s1;              // stage-1 row groups per expert, items
  int n_rt2, n_s2;              // stage-2 row tiles per expert, items
  int x_resident;               // one token, K <= 4096, 16-byte aligned: split by each workgroup once, kept in LDS
  int n_prep;                   // otherwise (x shared by a token's slots): tokens split once per call, by the first items
  int x_steps; uint8_t *xq; uint8_t *xs;   // ... into these columns (hi, lo per token)
  int *cntp, *obsp;             // split tokens; stage-1 items that have seen them all
  int grid;
  int s1_ilv;                   // stage-1 items take the active experts in turn (see launch_nt)
#ifdef TQ_TRACE
  unsigned long long *trace;
#endif
};

struct Shared {
  int16_t ids[kMaxSlots];       // expert per slot: -1 empty, >= E skipped (clamped)
  int16_t slots[kMaxSlots];     // slots of the current expert, in slot order
  int16_t active[kMaxExperts];  // active experts in id order
  float gw[kMaxSlots];
  unsigned mask[kMaxExperts / 32];
  int wpre[kMaxExperts / 32 + 1];
  int wcnt[kWaves];
  int n_active;
  int last;
  int x_done;                   // the resident token's columns are in place
#ifdef TQ_TRACE
  unsigned long long *trp;
#endif
  // One pass of activation columns (step-chunk layout: 128 code bytes and 4
  // scale bytes per column and step); after the matrix-core loop its upper
  // half is reused for the per-wave accumulator dumps (a resident single
  // token's columns, in the lower half, stay).
  uint8_t bq[kBBytes] __attribute__((aligned(16)));
  uint8_t bs[kBScaleBytes] __attribute__((aligned(16)));
  uint8_t as[kWaves][kAScaleBytes] __attribute__((aligned(16)));
};
static_assert(kWaves * 4 * 256 * sizeof(float) <= kBBytes / 2, "accumulator dump must fit the column area");

// ---------------------------------------------------------------- A scales

// e5m3_terms of every byte, filled by each E5M3 workgroup at entry (LDS;
// allocated only in the kernels that use it).
__shared__ uint32_t g_e5m3_terms[256];

// A-scale operand of K-block HH of a step: `sa` holds the raw scale bytes of
// the piece's two steps (byte HH is this step's). UE8M0: sa as it is (the
// matrix-core op selects byte HH). E5M3: the byte's four terms; a zero
// scale zeroes A (no UE8M0 sum is zero).
template <typename F, int HH>
__device__ __forceinline__ uint32_t a_scale(uint32_t sa, v8i &A) {
  if constexpr (!F::kE5M3) {
    return sa;
  } else {
    const uint32_t t = g_e5m3_terms[(sa >> (8 * HH)) & 0xFFu];
#pragma unroll
    for (int i = 0; i < 4; ++i) A[i] = t ? A[i] : 0;
    return t;
  }
}

// One matrix-core step, with the A scale from a_scale<F, HH>.
template <typename F, int HH>
__device__ __forceinline__ v4f mma_a(const v8i &A, const v8i &B, v4f c, uint32_t sx, uint32_t sb) {
  if constexpr (!F::kE5M3) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 0, HH, (int)sx, 0, (int)sb);
  } else {
    c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 0, 0, (int)sx, 0, (int)sb);
    c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 0, 1, (int)sx, 0, (int)sb);
    c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 0, 2, (int)sx, 0, (int)sb);
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 0, 3, (int)sx, 0, (int)sb);
  }
}

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ float load_x(const void *x, int bf16, size_t i) {
  return bf16 ? bf16_to_f32(((const uint16_t *)x)[i]) : ((const float *)x)[i];
}

// Device-coherent accesses for data handed between workgroups.
__device__ __forceinline__ void st_dc8(uint8_t *p, uint32_t v) {
  __hip_atomic_store(p, (uint8_t)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dcf(float *p, float v) {
  __hip_atomic_store((uint32_t *)p, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dc64(const uint8_t *p) {
  return __hip_atomic_load((const uint64_t *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dc32(const void *p) {
  return __hip_atomic_load((const uint32_t *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_ctr(const int *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_ctr(int *p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// y += v at the device's coherence point (no value returned).
__device__ __forceinline__ void add_dcf(float *p, float v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every thread's device-coherent stores have completed (the workgroup's
// results are visible device-wide); then one thread may count.
__device__ __forceinline__ void stores_done() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for LDS hand-offs only: this wave's LDS writes are
// complete (its LDS direct loads must have been waited for with vm_wait),
// then s_barrier. Unlike __syncthreads it does not wait for this wave's
// outstanding global loads, so weight loads stay in flight across it. The
// memory clobber keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Thread 0 waits until the counter reaches `target`; bounded: on timeout
// the error word is set. The caller synchronises the workgroup after.
__device__ __forceinline__ void spin_until(const int *ctr, int target, int *status) {
  unsigned spins = 0;
  while (ld_ctr(ctr) < target) {
    __builtin_amdgcn_s_sleep(2);
    if (++spins > kSpinLimit) {
      __hip_atomic_fetch_or(&status[ST_ERROR], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
  }
}

// Maximum of a non-negative float over the 32 lanes of a half-wave. On
// non-negative IEEE floats the bit patterns order like the values, so this
// is an integer max: four DPP steps (quad xor 1, quad xor 2, half-row
// mirror, row mirror) give the maximum over each 16-lane row, a swizzle
// (xor 16) combines the two rows.
__device__ __forceinline__ float halfwave_max(float v) {
  int m = __float_as_int(v);
  m = max(m, __builtin_amdgcn_update_dpp(0, m, 0xB1, 0xF, 0xF, false));
  m = max(m, __builtin_amdgcn_update_dpp(0, m, 0x4E, 0xF, 0xF, false));
  m = max(m, __builtin_amdgcn_update_dpp(0, m, 0x141, 0xF, 0xF, false));
  m = max(m, __builtin_amdgcn_update_dpp(0, m, 0x140, 0xF, 0xF, false));
  m = max(m, __builtin_amdgcn_ds_swizzle(m, 0x401F));
  return __int_as_float(m);
}

// Two-term FP8 split of one 32-value block held by the 32 lanes of a
// half-wave (lane = position in the block).
struct Split {
  uint32_t hi, lo;
  int E, El;
};
__device__ __forceinline__ Split split_block(float v) {
  Split s;
  s.E = block_exponent(halfwave_max(fabsf(v)));
  s.hi = f32_to_e4m3(ldexpf(v, -s.E));
  const float r = v - ldexpf(e4m3_to_f32(s.hi), s.E);
  s.El = block_exponent(halfwave_max(fabsf(r)));
  s.lo = f32_to_e4m3(ldexpf(r, -s.El));
  return s;
}

// Slot list of expert e into S.slots (slot order); returns the count.
template <int NT>
__device__ __forceinline__ int gather_slots(Shared &S, int e, int n) {
  const int lane = tidx<NT>() & 63, wave = tidx<NT>() >> 6;
  int total = 0;
  for (int base = 0; base < n; base += kThreads) {
    const int i = base + tidx<NT>();
    const bool p = i < n && S.ids[i] == e;
    const unsigned long long bal = __ballot(p);
    if (lane == 0) S.wcnt[wave] = __popcll(bal);
    __syncthreads();
    int off = total;
    for (int w = 0; w < wave; ++w) off += S.wcnt[w];
    if (p) S.slots[off + __popcll(bal & ((1ull << lane) - 1ull))] = (int16_t)i;
    for (int w = 0; w < kWaves; ++w) total += S.wcnt[w];
    __syncthreads();
  }
  return total;
}

// ---------------------------------------------------------------- activation columns in LDS
//
// A pass covers pieces [kp, kp + np) of K: column c holds 2*np step chunks
// (128 code bytes each, then 4 scale bytes per step in the scale area).
// Column 2c / 2c+1 is the hi / lo term of column pair c.

// Activation values of the pass, one unit = (column pair, block) per
// half-wave; the first kXPre units of every half-wave can be fetched ahead.
typedef uint32_t u32xp __attribute__((ext_vector_type(kXPre)));
struct XPre {
  u32xp v;                  // raw 32-bit words holding the values (a vector: stays in registers)
};

// Register hygiene for the loads below: a load's destination is never
// written before the load (no "zero, then load if in range"), because that
// makes the compiler wait for every load in flight. Out-of-range lanes load
// from a clamped, valid address and the value is discarded at its use.

// Element index of activation unit u (column pair, block) of the pass for
// this lane's position; ok false past the pass or the row.
template <typename F, typename RowMap>
__device__ __forceinline__ size_t x_elem(const LayerArgs &a, int K, int nb, int kp, int np, int npairs, int u,
                                         RowMap row_of, bool &ok) {
  const int nbp = F::kBlocks * np, c = u / nbp, blk = F::kBlocks * kp + u - c * nbp;
  ok = u < npairs * nbp && blk < nb;
  return ok ? (size_t)row_of(c) * K + (size_t)blk * 32 + (threadIdx.x & 31) : 0;
}

// One dword load per value for either dtype: the aligned word holding it
// (a bf16 row has an even length, so the word stays inside the buffer).
__device__ __forceinline__ uint32_t x_word(const LayerArgs &a, size_t elem) {
  const size_t byte = elem << (a.x_bf16 ? 1 : 2);
  return *(const uint32_t *)((const uint8_t *)a.x + (byte & ~(size_t)3));
}

__device__ __forceinline__ float x_value(const LayerArgs &a, size_t elem, uint32_t word) {
  if (!a.x_bf16) return __uint_as_float(word);
  return __uint_as_float((elem & 1 ? word >> 16 : word & 0xFFFFu) << 16);
}

// Raw words of units first, first + 8, ... (kXPre of them) of the pass.
template <typename F, typename RowMap>
__device__ __forceinline__ void x_load(u32xp &v, const LayerArgs &a, int K, int nb, int kp, int np,
                                       int npairs, int first, RowMap row_of) {
  constexpr int kStride = kThreads / 32;
  const int nbp = F::kBlocks * np, total = npairs * nbp;
  int c = first / nbp, b = first - c * nbp;   // unit (c, b); nbp >= 4, so b wraps at most twice a step
  size_t rbase = (size_t)row_of(min(c, npairs - 1)) * K + (threadIdx.x & 31);
#pragma unroll
  for (int m = 0; m < kXPre; ++m) {
    const int u = first + m * kStride, blk = F::kBlocks * kp + b;
    const bool ok = u < total && blk < nb;
    v[m] = x_word(a, ok ? rbase + (size_t)blk * 32 : 0);
    b += kStride;
    if (b >= nbp) {
      b -= nbp;
      ++c;
      if (b >= nbp) {
        b -= nbp;
        ++c;
      }
      rbase = (size_t)row_of(min(c, npairs - 1)) * K + (threadIdx.x & 31);
    }
  }
}

template <typename F, typename RowMap>
__device__ __forceinline__ void x_prefetch(XPre &xp, const LayerArgs &a, int K, int nb, int kp, int np, int npairs,
                                           RowMap row_of) {
  x_load<F>(xp.v, a, K, nb, kp, np, npairs, threadIdx.x >> 5, row_of);
}

template <typename F>
__device__ __forceinline__ void x_store_unit(uint8_t *lq, uint8_t *ls, int np, int u, float v, bool store) {
  const int nbp = F::kBlocks * np, psteps = F::kSteps * np;
  const int c = u / nbp, b = u % nbp, pos = threadIdx.x & 31;
  const Split s = split_block(v);
  if (!store) return;
  const int off = F::offset(b, pos);
  lq[(size_t)(2 * c) * psteps * 128 + off] = (uint8_t)s.hi;
  lq[(size_t)(2 * c + 1) * psteps * 128 + off] = (uint8_t)s.lo;
  if (pos == 0) {
    ls[(size_t)(2 * c) * psteps * 4 + F::scale_index(b)] = (uint8_t)(s.E + 127);
    ls[(size_t)(2 * c + 1) * psteps * 4 + F::scale_index(b)] = (uint8_t)(s.El + 127);
  }
}

// Split the prefetched units, then load and split the rest of the pass.
template <typename F, typename RowMap>
__device__ __forceinline__ void x_finish(const XPre &xp, uint8_t *lq, uint8_t *ls, const LayerArgs &a, int K, int nb,
                                         int kp, int np, int npairs, RowMap row_of) {
  const int hw = threadIdx.x >> 5, total = npairs * F::kBlocks * np;
  constexpr int kStride = kThreads / 32;
  // Every half-wave splits all its prefetched units without branches (the
  // cross-lane steps need the whole half-wave) and stores the real ones.
#pragma unroll
  for (int m = 0; m < kXPre; ++m) {
    const int u = hw + m * kStride;
    bool ok;
    const size_t el = x_elem<F>(a, K, nb, kp, np, npairs, u, row_of, ok);
    x_store_unit<F>(lq, ls, np, u, ok ? x_value(a, el, xp.v[m]) : 0.0f, u < total);
  }
  for (int base = hw + kXPre * kStride; base < total; base += kXPre * kStride) {
    u32xp v;
    x_load<F>(v, a, K, nb, kp, np, npairs, base, row_of);
#pragma unroll
    for (int m = 0; m < kXPre; ++m) {
      const int u = base + m * kStride;
      bool ok;
      const size_t el = x_elem<F>(a, K, nb, kp, np, npairs, u, row_of, ok);
      x_store_unit<F>(lq, ls, np, u, ok ? x_value(a, el, v[m]) : 0.0f, u < total);
    }
  }
}

// A single token's activations, split by each workgroup that needs them
// (once, on its first stage-1 item) into LDS columns 0 (hi) and 1 (lo): four
// lanes per 32-value block, eight values per lane, the block's maxima over
// the four lanes of a quad. Blocks past K (up to the window's end) get zero
// codes. 64 blocks per round, two rounds: K <= 4096. The raw values are
// loaded first (tok_load), ahead of the weight loads, so that only they
// are waited for when the split runs (tok_split).
constexpr int kTokRounds = 2;
struct TokRaw {
  uint4 v[kTokRounds][2];   // bf16: v[r][0]; fp32: v[r][0..1]
};

// One token's raw values (x: its first element, 16-byte aligned).
__device__ __forceinline__ void tok_load_at(TokRaw &t, const void *x, bool bf16, int nb) {
  const int j = tix() & 3;
#pragma unroll
  for (int r = 0; r < kTokRounds; ++r) {
    const int b = 64 * r + (tix() >> 2);
    const size_t el = b < nb ? (size_t)b * 32 + 8 * j : 0;   // (past K: a valid address, value unused)
    if (bf16) {
      t.v[r][0] = *(const uint4 *)((const uint16_t *)x + el);
      t.v[r][1] = t.v[r][0];
    } else {
      t.v[r][0] = *(const uint4 *)((const float *)x + el);
      t.v[r][1] = *(const uint4 *)((const float *)x + el + 4);
    }
  }
}

template <typename F>
__device__ __forceinline__ void tok_load(TokRaw &t, const LayerArgs &a, int nb, int np) {
  tok_load_at(t, a.x, a.x_bf16, nb);
}

__device__ __forceinline__ float quad_max(float v) {
  int m = __float_as_int(v);   // non-negative: integer order is float order
  m = max(m, __builtin_amdgcn_update_dpp(0, m, 0xB1, 0xF, 0xF, false));
  m = max(m, __builtin_amdgcn_update_dpp(0, m, 0x4E, 0xF, 0xF, false));
  return __int_as_float(m);
}

template <typename F>
__device__ __forceinline__ void tok_split(const TokRaw &t, uint8_t *lq, uint8_t *ls, int psteps, int nb,
                                          bool bf16) {
  const int j = tix() & 3, nblk = F::kBlocks * (psteps / F::kSteps);
#pragma unroll
  for (int r = 0; r < kTokRounds; ++r) {
    const int b = 64 * r + (tix() >> 2);
    float f[8];
    const uint32_t w[8] = {t.v[r][0].x, t.v[r][0].y, t.v[r][0].z, t.v[r][0].w,
                           t.v[r][1].x, t.v[r][1].y, t.v[r][1].z, t.v[r][1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t bits = bf16 ? (w[i >> 1] >> (16 * (i & 1))) << 16 : w[i];
      f[i] = b < nb ? __uint_as_float(bits) : 0.0f;
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
    const int E = block_exponent(quad_max(m));
    uint32_t hi[4], lo[4];
    float res[8], m2 = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      hi[i / 2] = f32x2_to_e4m3(ldexpf(f[i], -E), ldexpf(f[i + 1], -E));
      res[i] = f[i] - ldexpf(e4m3_to_f32(hi[i / 2]), E);
      res[i + 1] = f[i + 1] - ldexpf(e4m3_to_f32(hi[i / 2] >> 8), E);
      m2 = fmaxf(m2, fmaxf(fabsf(res[i]), fabsf(res[i + 1])));
    }
    const int El = block_exponent(quad_max(m2));
#pragma unroll
    for (int i = 0; i < 8; i += 2) lo[i / 2] = f32x2_to_e4m3(ldexpf(res[i], -El), ldexpf(res[i + 1], -El));
    if (b < nblk) {   // uniform over the quad
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int off = F::offset(b, 8 * j + i);
        lq[off] = (uint8_t)(hi[i / 2] >> (8 * (i & 1)));
        lq[(size_t)psteps * 128 + off] = (uint8_t)(lo[i / 2] >> (8 * (i & 1)));
      }
      if (j == 0) {
        ls[F::scale_index(b)] = (uint8_t)(E + 127);
        ls[(size_t)psteps * 4 + F::scale_index(b)] = (uint8_t)(El + 127);
      }
    }
  }
}

// Block (0-based in the pass) held at byte `o` of pass step `st`'s chunk:
// the chunk's 16-byte halves belong to K-blocks 0, 2, 0, 2, 1, 3, 1, 3.
template <typename F>
__device__ __forceinline__ int chunk_block(int st, int o) {
  return F::block_of(st, 2 * ((o >> 4) & 1) + (o >> 6));
}

// Copy the pass's slice of stored activation columns (global step-chunk
// layout, gsteps steps per column; LDS column c <- global column src_col(c))
// with device-coherent loads, issued 8 per thread before any LDS write.
// Blocks >= nb (the K padding, never written in global memory) become zero
// codes with scale 127.
template <typename F, int NT, typename ColMap>
__device__ __forceinline__ void copy_pass(uint8_t *lq, uint8_t *ls, const uint8_t *gq, const uint8_t *gs,
                                          int gsteps, int kp, int np, int nb, int ncols, ColMap src_col) {
  constexpr int kBatch = 8;
  if (F::kSteps == 2 && ncols <= 128 && np <= kPieceMax) {
    // Trellis windows (32 eight-byte units per column and piece): the same
    // copy with multiply-shift quotients (exact: every dividend times the
    // divisor stays below 2^20) in place of the general case's divisions.
    // (tix: the per-unit addresses are recomputed per window, not hoisted
    // out of the caller's window loop into registers)
    const uint32_t m_np = ((1u << 20) + np - 1) / np, m_ps = ((1u << 20) + 2 * np - 1) / (2 * np);
    const int per_col = 32 * np, total = ncols * per_col;
    for (int base = tix(); base < total; base += kBatch * kThreads) {
      uint64_t v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int idx = min(base + u * kThreads, total - 1);
        const int c = (int)(((uint32_t)(idx >> 5) * m_np) >> 20), p = idx - c * per_col;
        v[u] = ld_dc64(gq + ((size_t)src_col(c) * gsteps + 2 * kp + (p >> 4)) * 128 + (p & 15) * 8);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int idx = base + u * kThreads;
        if (idx < total) {
          const int c = (int)(((uint32_t)(idx >> 5) * m_np) >> 20), p = idx - c * per_col;
          const bool pad = F::kBlocks * kp + chunk_block<F>(p >> 4, (p & 15) * 8) >= nb;
          *(uint64_t *)(lq + (size_t)idx * 8) = pad ? 0ull : v[u];
        }
      }
    }
    const int stotal = ncols * 2 * np;
    for (int idx = tix(); idx < stotal; idx += kThreads) {
      const int c = (int)(((uint32_t)idx * m_ps) >> 20), st = idx - c * 2 * np;
      uint32_t w = ld_dc32(gs + ((size_t)src_col(c) * gsteps + 2 * kp + st) * 4);
#pragma unroll
      for (int beta = 0; beta < 4; ++beta)
        if (F::kBlocks * kp + F::block_of(st, beta) >= nb) w = (w & ~(0xFFu << (8 * beta))) | (127u << (8 * beta));
      *(uint32_t *)(ls + (size_t)idx * 4) = w;
    }
    return;
  }
  const int psteps = F::kSteps * np, per_col = psteps * 16;   // 8-byte pieces per column
  const int total = ncols * per_col;
  for (int base = tidx<NT>(); base < total; base += kBatch * kThreads) {
    uint64_t v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int idx = min(base + u * kThreads, total - 1);
      const int c = idx / per_col, p = idx - c * per_col;
      v[u] = ld_dc64(gq + ((size_t)src_col(c) * gsteps + F::kSteps * kp + (p >> 4)) * 128 + (p & 15) * 8);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int idx = base + u * kThreads;
      if (idx < total) {
        const int p = idx % per_col;
        const bool pad = F::kBlocks * kp + chunk_block<F>(p >> 4, (p & 15) * 8) >= nb;   // never written: zero it
        *(uint64_t *)(lq + (size_t)idx * 8) = pad ? 0ull : v[u];
      }
    }
  }
  const int stotal = ncols * psteps;
  for (int idx = tidx<NT>(); idx < stotal; idx += kThreads) {
    const int c = idx / psteps, st = idx - c * psteps;
    uint32_t w = ld_dc32(gs + ((size_t)src_col(c) * gsteps + F::kSteps * kp + st) * 4);
#pragma unroll
    for (int beta = 0; beta < 4; ++beta)
      if (F::kBlocks * kp + F::block_of(st, beta) >= nb) w = (w & ~(0xFFu << (8 * beta))) | (127u << (8 * beta));
    *(uint32_t *)(ls + (size_t)idx * 4) = w;
  }
}

// ---------------------------------------------------------------- weight tiles

struct Tile {
  uint4 a[kPieceMax];       // piece q: words 16(p0+q)+4g .. +3 of this lane's row
};

// Issue the loads of pieces [p0, p0 + np) of one row (`row` is always a
// valid row; the caller masks tiles past the matrix). Lanes past the row end
// load a clamped address; mma_tile zeroes those words. ALIGNED: words per
// row % 4 == 0, so a piece is one 16-byte load.
template <bool ALIGNED>
__device__ __forceinline__ void load_tile(Tile &t, const uint32_t *row, int wpr, int p0, int np, int g) {
  // Every piece but the last lies inside the row: one base address plus
  // immediate offsets. Only the last piece's address is clamped.
  const uint32_t *base = row + 16 * p0 + 4 * g;
  const int wl = 16 * (p0 + np - 1) + 4 * g;   // the last piece's first word
#pragma unroll
  for (int q = 0; q < kPieceMax; ++q) {
    if (q < np - 1) {   // uniform
      if (ALIGNED) {
        t.a[q] = *(const uint4 *)(base + 16 * q);
      } else {
        const uint2 lo = *(const uint2 *)(base + 16 * q);
        const uint2 hi = *(const uint2 *)(base + 16 * q + 2);
        t.a[q] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    } else if (q == np - 1) {
      if (ALIGNED) {
        t.a[q] = *(const uint4 *)(row + min(wl, wpr - 4));
      } else {
        const uint2 lo = *(const uint2 *)(row + min(wl, wpr - 2));
        const uint2 hi = *(const uint2 *)(row + min(wl + 2, wpr - 2));
        t.a[q] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    }
  }
}

// load_tile for the single-window case with a fixed instruction count:
// exactly NLOAD loads (2 NLOAD unaligned), pieces past np re-reading the
// last one. With a count that does not depend on np, the compiler's
// wait before piece q's first use lets the later pieces stay in flight, so
// the decode of the first pieces overlaps the arrival of the rest.
template <bool ALIGNED, int NLOAD>
__device__ __forceinline__ void load_tile_full(Tile &t, const uint32_t *row, int wpr, int np, int g) {
  const uint32_t *base = row + 4 * g;
  const int wl = 16 * (np - 1) + 4 * g;
#pragma unroll
  for (int q = 0; q < NLOAD; ++q) {
    if (q < np - 1) {   // uniform; one load (pair) on either side
      if (ALIGNED) {
        t.a[q] = *(const uint4 *)(base + 16 * q);
      } else {
        const uint2 lo = *(const uint2 *)(base + 16 * q);
        const uint2 hi = *(const uint2 *)(base + 16 * q + 2);
        t.a[q] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    } else {
      if (ALIGNED) {
        t.a[q] = *(const uint4 *)(row + min(wl, wpr - 4));
      } else {
        const uint2 lo = *(const uint2 *)(row + min(wl, wpr - 2));
        const uint2 hi = *(const uint2 *)(row + min(wl + 2, wpr - 2));
        t.a[q] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    }
  }
}

// The tile's UE8M0 bytes in the wave's LDS slot, row i at i * stride:
//  fast   (16-byte aligned base, whole row in one window): the tile's 16 x nb
//         bytes are contiguous; two 16-byte loads per lane, stride nb.
//  generic: per window, each lane fetches its two bytes per piece, stride 128.
struct AScalePre {
  uint4 v0, v1;
};

__device__ __forceinline__ void ascale_prefetch(AScalePre &sp, const uint8_t *sblk, int nb) {
  const int lane = tix() & 63;
  sp.v0 = ((const uint4 *)sblk)[min(lane, nb - 1)];
  sp.v1 = ((const uint4 *)sblk)[min(lane + 64, nb - 1)];
}

__device__ __forceinline__ void ascale_store(uint8_t *as_w, const AScalePre &sp, int nb) {
  const int lane = tix() & 63;
  if (lane < nb) ((uint4 *)as_w)[lane] = sp.v0;
  if (lane + 64 < nb) ((uint4 *)as_w)[lane + 64] = sp.v1;
}

// (A lane's blocks of piece j: trellis 8j+2g and 8j+2g+1, MXFP4 4j+g.)
template <typename F>
__device__ __forceinline__ void ascale_generic(uint8_t *as_w, const uint8_t *srow, int nb, int p0, int np, bool ok) {
  const int lane = tix() & 63, i16 = lane & 15, g = lane >> 4;
  constexpr int kPer = F::kBlocks / 4;   // blocks per lane and piece
#pragma unroll
  for (int q = 0; q < kPieceMax; ++q) {
    if (q < np) {
      const int b = F::kBlocks * (p0 + q) + kPer * g;
#pragma unroll
      for (int h = 0; h < kPer; ++h)
        as_w[i16 * 128 + F::kBlocks * q + kPer * g + h] = ok && b + h < nb ? srow[b + h] : (uint8_t)127;
    }
  }
}

// A whole trellis window (K <= 3072) decoded ahead of the matrix-core loop:
// a down-projection item decodes it while it waits for its h, so only the
// matrix-core steps are left once h arrives; the tile's registers are free
// again once it is decoded. (Longer windows are not pre-decoded: their
// decoded pieces would not fit the register file.)
constexpr int kPre = 12;
struct PreDec {
  uint4 s[kPre][2];   // A operands of steps 2q and 2q+1
};

__device__ __forceinline__ void predecode(PreDec &d, const Tile &t, int np, uint32_t &carry, int lane) {
  const int g = lane >> 4;
  const int src = ((lane - 16) & 63) << 2;
#pragma unroll
  for (int q = 0; q < kPre; ++q) {
    if (q < np) {
      const uint4 a = t.a[q];
      const uint32_t rot = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)a.w);
      const uint32_t hist = g == 0 ? carry : rot;
      carry = rot;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint32_t w0 = hh ? a.z : a.x, w1 = hh ? a.w : a.y, hw = hh ? a.y : hist;
        const nib2 d0 = decode_word(w0, hw);
        const nib2 d1 = decode_word(w1, w0);
        d.s[q][hh] = make_uint4(d0.even, d0.odd, d1.even, d1.odd);
      }
    }
  }
}

// Decode window pieces [0, np) (global piece p0 + q) and accumulate them
// against NT N-tiles of the window's LDS columns. Lane
// (column jc = lane & 15, lane-group g): N-tile n reads LDS column col[n]
// (zeros when !on[n]).
template <typename F, int NT>
__device__ __forceinline__ void mma_tile(const Tile &t, int p0, int np, bool tile_ok,
                                         int wpr, const uint8_t *as_w, int astride, int a_p0, int nb,
                                         const uint8_t *lq, const uint8_t *ls, int psteps,
                                         const int (&col)[NT], const bool (&on)[NT], v4f (&acc)[NT],
                                         uint32_t &carry, int lane) {
  const int g = lane >> 4, i16 = lane & 15;
  const int src = ((lane - 16) & 63) << 2;   // lane-group g-1 (mod 4), same row
  if (F::kSteps == 1) {
    // Expanded MXFP4: a piece is one step's A operand as stored, scaled by
    // the UE8M0 byte of block 4j + g.
#pragma unroll
    for (int q = 0; q < kPieceMax; ++q) {
      if (q < np) {
        const int j = p0 + q;
        const uint4 a = t.a[q];
        const uint32_t sa = tile_ok && 4 * j + g < nb ? (uint32_t)as_w[i16 * astride + 4 * (a_p0 + q) + g] : 0x7Fu;
        v8i B[NT];
        uint32_t sb[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const int c = on[n] ? col[n] : (col[n] & 1);
          const uint4 *p = (const uint4 *)(lq + ((size_t)c * psteps + q) * 128 + g * 32);
          const uint4 u0 = p[0], u1 = p[1];
          B[n] = v8i{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
          sb[n] = ls[((size_t)c * psteps + q) * 4 + g];
        }
        const v8i A = v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
#pragma unroll
        for (int n = 0; n < NT; ++n)
          acc[n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B[n], acc[n], 4, 0, 0, (int)sa, 0, (int)sb[n]);
      }
    }
    return;
  }
#pragma unroll
  for (int q = 0; q < kPieceMax; ++q) {
    if (q < np) {
      const int j = p0 + q;
      // Words past the row end (clamped loads) decode to finite E2M1 values
      // that meet the zero codes of the activations' K padding, and rows past
      // the matrix give outputs that are never stored: no masking needed.
      const uint4 a = t.a[q];
      const uint32_t rot = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)a.w);
      const uint32_t hist = g == 0 ? carry : rot;
      carry = rot;
      const int sb_a = 8 * j + 2 * g;
      const uint32_t sa =
          tile_ok && sb_a < nb ? (uint32_t)*(const uint16_t *)(as_w + i16 * astride + 8 * (a_p0 + q) + 2 * g) : 0x7F7Fu;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int step = 2 * q + hh;
        v8i B[NT];
        uint32_t sb[NT];
        // Output column c of D depends only on B column c, and the columns
        // of unused N-tile lanes are never read: those lanes load column 0
        // or 1 instead of zeros, so the loads need no lane masking.
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const int c = on[n] ? col[n] : (col[n] & 1);
          const uint4 *p = (const uint4 *)(lq + ((size_t)c * psteps + step) * 128 + g * 32);
          const uint4 u0 = p[0], u1 = p[1];
          B[n] = v8i{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
          sb[n] = ls[((size_t)c * psteps + step) * 4 + g];
        }
        const uint32_t w0 = hh ? a.z : a.x, w1 = hh ? a.w : a.y, hw = hh ? a.y : hist;
        const nib2 d0 = decode_word(w0, hw);
        const nib2 d1 = decode_word(w1, w0);
        v8i A = v8i{(int)d0.even, (int)d0.odd, (int)d1.even, (int)d1.odd, 0, 0, 0, 0};
        if (hh == 0) {
          const uint32_t sx = a_scale<F, 0>(sa, A);
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[n] = mma_a<F, 0>(A, B[n], acc[n], sx, sb[n]);
        } else {
          const uint32_t sx = a_scale<F, 1>(sa, A);
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[n] = mma_a<F, 1>(A, B[n], acc[n], sx, sb[n]);
        }
      }
    }
  }
}

// One matrix-core step's B operands (LDS) for the NT N-tiles.
template <int NT>
struct BStep {
  v8i b[NT];
  uint32_t s[NT];
};

template <int NT>
__device__ __forceinline__ void read_bstep(BStep<NT> &o, const uint8_t *lq, const uint8_t *ls, int psteps, int step,
                                           const int (&c)[NT], int g) {
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const uint4 *p = (const uint4 *)(lq + ((size_t)c[n] * psteps + step) * 128 + g * 32);
    const uint4 u0 = p[0], u1 = p[1];
    o.b[n] = v8i{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
    o.s[n] = ls[((size_t)c[n] * psteps + step) * 4 + g];
  }
}

// Matrix-core pass over a window whose np (<= kPre) pieces were all decoded
// ahead. Nothing waits for memory here, so the pass is latency-bound unless
// it is pipelined: each step's LDS operands are read kD steps ahead, and the
// even and odd steps of a piece accumulate in separate registers (summed at
// the end), so consecutive matrix-core ops do not depend on each other. The
// steps are a compile-time recursion that returns past the last one: a loop
// of guarded steps would rejoin after each, and at every join the compiler
// waits for all outstanding LDS reads, which undoes the reading ahead.
template <int NT>
struct PreCtx {
  const uint8_t *as_row;   // this lane's A-scale bytes of piece 0 (LDS)
  const uint8_t *lq, *ls;
  int c[NT];
  int psteps, ns, nb, g;
  bool tile_ok;
};

template <int NT>
__device__ __forceinline__ uint32_t pre_sa(const PreCtx<NT> &x, int q) {
  return x.tile_ok && 8 * q + 2 * x.g < x.nb ? (uint32_t)*(const uint16_t *)(x.as_row + 8 * q) : 0x7F7Fu;
}

template <typename F, int NT, int S>
__device__ __forceinline__ void pre_step(const PreCtx<NT> &x, const PreDec &pd, BStep<NT> (&ring)[NT == 1 ? 3 : 1],
                                         uint32_t (&sa)[2], v4f (&acc)[NT], v4f (&acc2)[NT]) {
  constexpr int kD = NT == 1 ? 2 : 0;
  if constexpr (S < 2 * kPre) {
    if (S >= x.ns) return;
    constexpr int q = S >> 1, hh = S & 1;
    if (S + kD < x.ns) read_bstep<NT>(ring[(S + kD) % (kD + 1)], x.lq, x.ls, x.psteps, S + kD, x.c, x.g);
    if (hh == 0 && S + 2 < x.ns) sa[(q + 1) & 1] = pre_sa(x, q + 1);
    const uint4 w = pd.s[q][hh];
    v8i A = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
    const BStep<NT> &cur = ring[S % (kD + 1)];
    const uint32_t sx = a_scale<F, hh>(sa[q & 1], A);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      if (hh == 0)
        acc[n] = mma_a<F, 0>(A, cur.b[n], acc[n], sx, cur.s[n]);
      else
        acc2[n] = mma_a<F, 1>(A, cur.b[n], acc2[n], sx, cur.s[n]);
    }
    pre_step<F, NT, S + 1>(x, pd, ring, sa, acc, acc2);
  }
}

template <typename F, int NT>
__device__ __forceinline__ void mma_pre(const PreDec &pd, int np, bool tile_ok, const uint8_t *as_w, int astride,
                                        int nb, const uint8_t *lq, const uint8_t *ls, int psteps,
                                        const int (&col)[NT], const bool (&on)[NT], v4f (&acc)[NT], int lane) {
  constexpr int kD = NT == 1 ? 2 : 0;   // steps read ahead (registers: only with one N-tile)
  PreCtx<NT> x;
  x.g = lane >> 4;
  x.as_row = as_w + (lane & 15) * astride + 2 * x.g;
  x.lq = lq;
  x.ls = ls;
  x.psteps = psteps;
  x.ns = 2 * np;
  x.nb = nb;
  x.tile_ok = tile_ok;
  v4f acc2[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    // unused N-tile lanes read column 0 or 1 (see mma_tile)
    x.c[n] = on[n] ? col[n] : (col[n] & 1);
    acc2[n] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  BStep<NT> ring[kD + 1];
  uint32_t sa[2];
#pragma unroll
  for (int d = 0; d < kD; ++d) read_bstep<NT>(ring[d], lq, ls, psteps, d < x.ns ? d : 0, x.c, x.g);
  sa[0] = pre_sa(x, 0);
  sa[1] = 0x7F7Fu;
  pre_step<F, NT, 0>(x, pd, ring, sa, acc, acc2);
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] += acc2[n];
}

// ---------------------------------------------------------------- streamed window
//
// The single-window case without pre-decoding streams its pieces through a
// ring of kRing registers with kAhead loads in flight per wave: piece q is
// decoded and multiplied while pieces q+1 .. q+kAhead are on their way, and
// each step issues the load of piece q+kAhead. Issuing a whole tile up front
// instead would stall the wave at the issue (the memory pipeline accepts a
// limited number of requests per compute unit) until most of the tile had
// arrived, and the decode would start only then. Every step issues exactly
// one load (past the window's end, a re-read of its last piece), so the
// compiler's wait before piece q always leaves the kAhead younger loads in
// flight.
constexpr int kRing = 8;
constexpr int kAhead = 6;   // < kRing; ring slots kAhead.. carry the tile's scales at first
struct Ring {
  uint4 r[kRing];
};

// Piece p of a window of np pieces; p >= np - 1 reads the (clamped) last one.
template <bool ALIGNED>
__device__ __forceinline__ uint4 load_piece(const uint32_t *row, int wpr, int p, int np, int g) {
  if (p < np - 1) {   // uniform; one load (pair) on either side
    if (ALIGNED) return *(const uint4 *)(row + 16 * p + 4 * g);
    const uint2 lo = *(const uint2 *)(row + 16 * p + 4 * g);
    const uint2 hi = *(const uint2 *)(row + 16 * p + 4 * g + 2);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
  const int wl = 16 * (np - 1) + 4 * g;
  if (ALIGNED) return *(const uint4 *)(row + min(wl, wpr - 4));
  const uint2 lo = *(const uint2 *)(row + min(wl, wpr - 2));
  const uint2 hi = *(const uint2 *)(row + min(wl + 2, wpr - 2));
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

template <int NT>
struct StreamCtx {
  const uint32_t *row;
  int wpr, np, nb, astride, psteps, lane, g, i16, src;
  const uint32_t *rowg;   // this lane's first word of piece 0 (row + 4g)
  int lastw;              // piece p starts at rowg + min(16p, lastw) (aligned rows)
  const uint8_t *sa;      // this lane's A scales of piece 0 in the wave's LDS slot
  const uint8_t *bq[NT];  // N-tile n's B bytes of step 0 for this lane
  const uint8_t *bs[NT];  // and its B scale
  uint32_t carry;
  uint32_t rot;   // the current piece's last word from lane-group g-1 (fetched a piece ahead)
};

// One piece of the stream; the pieces are chained by template recursion so
// that a window that ends early leaves straight away (no join after each
// piece, which would make the compiler's count of loads in flight drop by
// one per piece).
template <typename F, int NT, bool ALIGNED, int Q>
__device__ __forceinline__ void stream_piece(StreamCtx<NT> &c, Ring &R, v4f (&acc)[NT]) {
  if constexpr (Q < kPieceMax) {
    if (Q >= c.np) return;
    if (ALIGNED)
      R.r[(Q + kAhead) % kRing] = *(const uint4 *)(c.rowg + min(16 * (Q + kAhead), c.lastw));
    else
      R.r[(Q + kAhead) % kRing] = load_piece<ALIGNED>(c.row, c.wpr, Q + kAhead, c.np, c.g);
    __builtin_amdgcn_sched_barrier(0);
    const uint4 a = R.r[Q % kRing];
    if constexpr (F::kSteps == 1) {
      // (A scales past the row's blocks: finite bytes that meet zero codes)
      const uint32_t sa = c.sa[4 * Q];
      v8i B[NT];
      uint32_t sb[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const uint4 *p = (const uint4 *)(c.bq[n] + Q * 128);
        const uint4 u0 = p[0], u1 = p[1];
        B[n] = v8i{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
        sb[n] = c.bs[n][Q * 4];
      }
      const v8i A = v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
#pragma unroll
      for (int n = 0; n < NT; ++n)
        acc[n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B[n], acc[n], 4, 0, 0, (int)sa, 0, (int)sb[n]);
    } else {
      // All of the piece's LDS reads go out before its decode, so that
      // their latency hides behind it; the next piece's history word is
      // fetched here too (its slot always holds a loaded piece).
      const uint32_t rot = c.rot;
      // (A scales past the row's blocks: finite bytes that meet zero codes)
      const uint32_t sa = *(const uint16_t *)(c.sa + 8 * Q);
      v8i B[2][NT];
      uint32_t sb[2][NT];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const uint4 *p = (const uint4 *)(c.bq[n] + (2 * Q + hh) * 128);
          const uint4 u0 = p[0], u1 = p[1];
          B[hh][n] = v8i{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
          sb[hh][n] = c.bs[n][(2 * Q + hh) * 4];
        }
      }
      c.rot = (uint32_t)__builtin_amdgcn_ds_bpermute(c.src, (int)R.r[(Q + 1) % kRing].w);
      __builtin_amdgcn_sched_barrier(0);
      const uint32_t hist = c.g == 0 ? c.carry : rot;
      c.carry = rot;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint32_t w0 = hh ? a.z : a.x, w1 = hh ? a.w : a.y, hw = hh ? a.y : hist;
        const nib2 d0 = decode_word(w0, hw);
        const nib2 d1 = decode_word(w1, w0);
        v8i A = v8i{(int)d0.even, (int)d0.odd, (int)d1.even, (int)d1.odd, 0, 0, 0, 0};
        if (hh == 0) {
          const uint32_t sx = a_scale<F, 0>(sa, A);
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[n] = mma_a<F, 0>(A, B[0][n], acc[n], sx, sb[0][n]);
        } else {
          const uint32_t sx = a_scale<F, 1>(sa, A);
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[n] = mma_a<F, 1>(A, B[1][n], acc[n], sx, sb[1][n]);
        }
      }
    }
    stream_piece<F, NT, ALIGNED, Q + 1>(c, R, acc);
  }
}

// Decode and multiply the window's np pieces, the first kAhead of which
// the caller has issued into the ring (later ones are issued here).
template <typename F, int NT, bool ALIGNED>
__device__ __forceinline__ void mma_stream(Ring &R, const uint32_t *row, int wpr, int np, bool tile_ok,
                                           const uint8_t *as_w, int astride, int nb, const uint8_t *lq,
                                           const uint8_t *ls, int psteps, const int (&col)[NT],
                                           const bool (&on)[NT], v4f (&acc)[NT], int lane) {
  StreamCtx<NT> c;
  c.row = row; c.wpr = wpr; c.np = np; c.nb = nb; c.astride = astride; c.psteps = psteps;
  c.lane = lane; c.g = lane >> 4; c.i16 = lane & 15; c.src = ((lane - 16) & 63) << 2;
  c.rowg = row + 4 * c.g;
  c.lastw = min(16 * (np - 1), wpr - 4 - 4 * c.g);
  c.sa = as_w + c.i16 * astride + (F::kSteps == 2 ? 2 : 1) * c.g;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int cc = on[n] ? col[n] : (col[n] & 1);
    c.bq[n] = lq + (size_t)cc * psteps * 128 + c.g * 32;
    c.bs[n] = ls + (size_t)cc * psteps * 4 + c.g;
  }
  c.carry = 0u;
  if (F::kSteps == 2) c.rot = (uint32_t)__builtin_amdgcn_ds_bpermute(c.src, (int)R.r[0].w);
  stream_piece<F, NT, ALIGNED, 0>(c, R, acc);
  // Every ring slot is read once more here (never-true store): without a
  // use on the early-exit paths the compiler would sink each load down to
  // its piece, and nothing would be in flight ahead of the decode.
  uint32_t keep = 0u;
#pragma unroll
  for (int i = 0; i < kRing; ++i) keep ^= R.r[i].x;
  if (np < 0 && keep == 0x9E3779B9u) *(volatile uint32_t *)as_w = keep;
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
  float *red = (float *)(S.bq + kBBytes / 2);
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[((wave * NT + n) * 64 + lane) * 4 + r] = acc[n][r];
}

// hi + lo of column pair (n*8 + i16/2), row 4g + r, summed in the even lane.
template <int NT, typename Out>
__device__ __forceinline__ void per_slot_out(const v4f (&acc)[NT], int ncol, int lane, Out out) {
  const int i16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = acc[n][r] + __shfl_xor(acc[n][r], 1);
      const int c = n * 8 + (i16 >> 1);
      if ((i16 & 1) == 0 && c < ncol) out(c, 4 * g + r, v);
    }
}

// Sum the partial outputs of rows [rt*64, rt*64 + 64) over each token's live
// slots, in slot order, weighted by the gate weights.
__device__ __forceinline__ void combine_rows(const LayerArgs &a, const Shared &S, int rt) {
  for (int idx = tix(); idx < a.T * 64; idx += kThreads) {
    const int t = idx >> 6, r = rt * 64 + (idx & 63);
    if (r >= a.y_rows) continue;
    float v = 0.0f;
    for (int j = 0; j < a.k; ++j) {
      const int s = t * a.k + j, e = S.ids[s];
      if (e >= 0 && e < a.E) v += S.gw[s] * __uint_as_float(ld_dc32(a.yslot + (size_t)s * a.y_rows + r));
    }
    a.y[(size_t)t * a.y_rows + r] = v;
  }
}

// The item's partial outputs are stored; count it at its output tile and,
// if it is the last of the n_active experts there, combine the tile.
__device__ __forceinline__ void arrive_and_combine(const LayerArgs &a, Shared &S, int rt) {
  stores_done();
  if (tix() == 0) {
    int *ctr = a.cnt2 + (size_t)rt * kLineInts;
    const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    S.last = old == S.n_active - 1;
    if (S.last) st_ctr(ctr, 0);   // every arrival is in: clear for the next call
  }
  __syncthreads();
  if (S.last) combine_rows(a, S, rt);
}

// ---------------------------------------------------------------- many slots per expert

// One piece of a many-slot pass: decode piece Q of the tile (history from
// lane-group g-1 of the same piece, or the previous piece's last word) and
// multiply it into the accumulators of the pass's up to 64 slots: N-tiles
// 0..3 (LDS columns 0..63) in acc0, 4..7 (columns 64..127) in acc1. The LDS
// holds the slots' activation columns of the window's pieces (psteps steps
// per column); the piece's steps are st0 and st0 + 1 there.
template <typename F, int Q>
__device__ __forceinline__ void pf_piece(const Tile &tl, int psteps, int st0, const uint8_t *as_w, int astride,
                                         int nb, bool tile_ok, uint32_t &carry, const uint8_t *lq, const uint8_t *ls,
                                         int ncol, v4f (&acc0)[4], v4f (&acc1)[4]) {
  // (tix: the lane-derived LDS addresses are recomputed here, per piece;
  // hoisted out of the window loop they would outlive it in registers)
  const int lane = tix() & 63, g = lane >> 4, i16 = lane & 15;
  const uint4 a = tl.a[Q];
  const uint32_t rot = (uint32_t)__builtin_amdgcn_ds_bpermute(((lane - 16) & 63) << 2, (int)a.w);
  const uint32_t hist = g == 0 ? carry : rot;
  carry = rot;
  // (A scales past the row's blocks, and of tiles past the matrix: finite
  // bytes that meet zero codes or unused rows)
  const uint32_t sa = tile_ok && 8 * Q + 2 * g < nb
                          ? (uint32_t)*(const uint16_t *)(as_w + i16 * astride + 2 * g + 8 * Q) : 0x7F7Fu;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const uint32_t w0 = hh ? a.z : a.x, w1 = hh ? a.w : a.y, hw = hh ? a.y : hist;
    const nib2 d0 = decode_word(w0, hw);
    const nib2 d1 = decode_word(w1, w0);
    v8i A = v8i{(int)d0.even, (int)d0.odd, (int)d1.even, (int)d1.odd, 0, 0, 0, 0};
    const uint32_t sx = hh ? a_scale<F, 1>(sa, A) : a_scale<F, 0>(sa, A);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      if (n >= 4 && ncol <= 32) break;   // uniform
      // unused N-tile lanes read column 0 or 1 (their outputs are never stored)
      const int c = n * 8 + (i16 >> 1) < ncol ? n * 16 + i16 : (i16 & 1);
      const int cs = c * psteps + st0 + hh;
      const uint4 *p = (const uint4 *)(lq + cs * 128 + g * 32);
      const uint4 u0 = p[0], u1 = p[1];
      const v8i B = v8i{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
      const uint32_t sb = ls[cs * 4 + g];
      v4f &d = n < 4 ? acc0[n & 3] : acc1[n & 3];
      d = hh ? mma_a<F, 1>(A, B, d, sx, sb) : mma_a<F, 0>(A, B, d, sx, sb);
    }
  }
}

// The window's pieces [p0, p0 + np), by compile-time recursion over the
// tile's piece index (the tile stays in registers).
template <typename F, int Q>
__device__ __forceinline__ void pf_window(int p0, int np, const Tile &tl, const uint8_t *as_w, int astride, int nb,
                                          bool tile_ok, uint32_t &carry, const uint8_t *lq, const uint8_t *ls,
                                          int ncol, v4f (&acc0)[4], v4f (&acc1)[4]) {
  if constexpr (Q < kPieceMax) {
    if (Q >= p0 + np) return;
    if (Q >= p0) pf_piece<F, Q>(tl, 2 * np, 2 * (Q - p0), as_w, astride, nb, tile_ok, carry, lq, ls, ncol, acc0, acc1);
    pf_window<F, Q + 1>(p0, np, tl, as_w, astride, nb, tile_ok, carry, lq, ls, ncol, acc0, acc1);
  }
}

// An item whose expert has more slots than one window pass of the general
// loop holds (at K = 4096 that is 4): each pass of up to 64 slots loads the
// tile (<= 16 pieces) once, all of it in flight at once, and decodes it
// once. The pass's activation columns come into LDS a window of pieces at a
// time, as many pieces as the 32 KB column area holds for its slots (one
// piece for 64 slots, eight for 8). The pass's two halves of 32 slots go to
// the epilogue one after the other.
template <typename F, bool ALIGNED, typename Stage, typename Epi>
__device__ __forceinline__ void pf_item(Shared &S, Tile &tl, const uint32_t *rowp, const uint8_t *srow,
                                        const uint8_t *stile, int wpr, int nb, int J, int fast, bool tile_ok, int ne,
                                        Stage &stage, Epi &epilogue) {
  const int lane = tix() & 63, wave = tix() >> 6, g = lane >> 4;
  uint8_t *as_w = S.as[wave];
  if (fast) {
    AScalePre sp;
    ascale_prefetch(sp, stile, nb);
    ascale_store(as_w, sp, nb);
    // the last row's last piece may read a byte past the tile's scales: a finite one
    if (lane == 0 && 16 * nb + 8 <= kAScaleBytes) *(uint64_t *)(as_w + 16 * nb) = 0x7F7F7F7F7F7F7F7Full;
  } else {
    ascale_generic<F>(as_w, srow, nb, 0, J, tile_ok);
  }
  const int astride = fast ? nb : 128;
  for (int c0 = 0; c0 < ne; c0 += 64) {
    const int ncol = min(ne - c0, 64);
    const int W = max(1, min(J, kBBytes / (ncol * 2 * F::kSteps * 128)));   // pieces per window
    v4f acc0[4], acc1[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) acc0[n] = acc1[n] = v4f{0.f, 0.f, 0.f, 0.f};
    uint32_t carry = 0u;
    load_tile_full<ALIGNED, kPieceMax>(tl, rowp, wpr, J, g);
    TQ_MARK(S, 3);
    for (int p0 = 0; p0 < J; p0 += W) {
      const int np = min(W, J - p0);
      stage(c0, ncol, p0, np);   // the window's activation columns of the pass's slots
      __syncthreads();
      if (p0 == 0) TQ_MARK(S, 4);
      pf_window<F, 0>(p0, np, tl, as_w, astride, nb, tile_ok, carry, S.bq, S.bs, ncol, acc0, acc1);
      __syncthreads();   // everyone is done with the window's columns
      if (p0 == 0) TQ_MARK(S, 5);
    }
    TQ_MARK(S, 6);
    epilogue(c0, min(ncol, 32), acc0);
    if (ncol > 32) {
      __syncthreads();
      epilogue(c0 + 32, ncol - 32, acc1);
    }
    __syncthreads();
    TQ_MARK(S, 7);
  }
}

// ---------------------------------------------------------------- work items

// The grouped GEMM of one item: expert e, 16 rows per wave starting at r0
// (past the matrix: zeros, no output), columns = the expert's ne slots. K
// is covered in register windows of up to 16 pieces; the LDS holds one
// window of activation columns for a group of slots (as many as fit, at
// most 8*NT). fetch_ahead(c0, ncol, p0, np) runs before the window's weight
// loads are issued; stage(c0, ncol, p0, np) then fills the LDS;
// epilogue(c0, ncol, acc) runs per slot group with the LDS free. With one
// window the weight tile stays in registers across slot groups.
// shared_cols: every slot reads LDS columns 0 (hi) and 1 (lo). predec:
// decode the first pieces before stage runs (stage may wait).
template <typename F, int NT, bool ALIGNED, typename Ahead, typename Stage, typename Epi>
__device__ __forceinline__ void gemm_item(Shared &S, const uint32_t *w, const uint8_t *sc, int rows, int K,
                                          int fast, int e, int r0, int ne, bool shared_cols, bool predec,
                                          Ahead fetch_ahead, Stage stage, Epi epilogue) {
  const int lane = tidx<NT>() & 63, wave = tidx<NT>() >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const bool tile_ok = r0 < rows;
  const int wpr = K / 32 * F::kWords, nb = K / 32, J = (nb + F::kBlocks - 1) / F::kBlocks;
  const size_t row0 = (size_t)e * rows + (tile_ok ? r0 : 0);
  const uint32_t *rowp = w + (row0 + i16) * wpr;
  const uint8_t *srow = sc + (row0 + i16) * nb;
  uint8_t *as_w = S.as[wave];
  const int astride = fast ? nb : 128;
  const int gsz = min(NT * 8, kBBytes / (min(J, kPieceMax) * F::kSteps * 256));
  Tile tl;
  if constexpr (NT == 4 && F::kSteps == 2) {
    if (J <= kPieceMax && ne > gsz) {
      pf_item<F, ALIGNED>(S, tl, rowp, srow, sc + row0 * nb, wpr, nb, J, fast, tile_ok, ne, stage, epilogue);
      return;
    }
  }
  if (J <= kPieceMax && ne <= gsz) {
    // The common case, one window and one slot group, as straight-line code.
    // Load order: activations, the tile's pieces, whatever the stage loads,
    // then the tile's scales (loads complete in issue order; the scales are
    // needed only once the pieces are, and issuing them late keeps them from
    // occupying registers across the stage).
    int col[NT];
    bool on[NT];
    v4f acc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      col[n] = shared_cols ? (i16 & 1) : n * 16 + i16;
      on[n] = n * 8 + (i16 >> 1) < ne;
      acc[n] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    // (not with 3-4 N-tiles: their accumulators leave no registers for it)
    const int npre = predec && F::kSteps == 2 && NT <= 2 && J <= kPre ? J : 0;
    if (npre) {
      // A down-projection item: the whole tile is loaded (it has time until
      // its h is complete) and its first pieces decoded while it waits.
      // Loads go out in the order they are needed, and they complete in
      // that order: the tile's scales, then a fixed number of pieces. The
      // scales ride in the two last piece registers when the tile leaves
      // them free; otherwise they are loaded after the pieces.
      uint32_t carry = 0u;
      fetch_ahead(0, ne, 0, J);
      const bool sp_in_tile = fast && J <= kPieceMax - 2;
      __builtin_amdgcn_sched_barrier(0);
      if (sp_in_tile) {
        const uint4 *sblk = (const uint4 *)(sc + row0 * nb);
        tl.a[kPieceMax - 2] = sblk[min(lane, nb - 1)];
        tl.a[kPieceMax - 1] = sblk[min(lane + 64, nb - 1)];
        __builtin_amdgcn_sched_barrier(0);
        load_tile_full<ALIGNED, kPieceMax - 2>(tl, rowp, wpr, J, g);
      } else {
        load_tile_full<ALIGNED, kPieceMax>(tl, rowp, wpr, J, g);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (sp_in_tile) {
        AScalePre sp;
        sp.v0 = tl.a[kPieceMax - 2];
        sp.v1 = tl.a[kPieceMax - 1];
        ascale_store(as_w, sp, nb);
      }
      TQ_MARK(S, 3);
      PreDec pd;
      predecode(pd, tl, npre, carry, lane);
      stage(0, ne, 0, J);
      TQ_MARK(S, 4);
      if (!sp_in_tile && fast) {
        AScalePre sp;
        ascale_prefetch(sp, sc + row0 * nb, nb);
        ascale_store(as_w, sp, nb);
      } else if (!fast) {
        ascale_generic<F>(as_w, srow, nb, 0, J, tile_ok);
      }
      vm_wait<0>();
      TQ_MARK(S, 5);
      lds_barrier();
      TQ_MARK(S, 6);
      mma_pre<F, NT>(pd, J, tile_ok, as_w, astride, nb, S.bq, S.bs, F::kSteps * J, col, on, acc, lane);
    } else {
      // Streamed (see mma_stream). fetch_ahead first (a resident token's
      // split, on a workgroup's first stage-1 item: it waits for the split
      // to be complete and copies it; loads complete in issue order, so
      // behind weight loads it would wait for them too), then the tile's
      // scales (in the ring slots the first kAhead pieces leave free) and
      // the first kAhead pieces.
      Ring R;
      fetch_ahead(0, ne, 0, J);
      __builtin_amdgcn_sched_barrier(0);
      if (fast) {
        const uint4 *sblk = (const uint4 *)(sc + row0 * nb);
        R.r[kAhead] = sblk[min(lane, nb - 1)];
        R.r[kAhead + 1] = sblk[min(lane + 64, nb - 1)];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int p = 0; p < kAhead; ++p) R.r[p] = load_piece<ALIGNED>(rowp, wpr, p, J, g);
      __builtin_amdgcn_sched_barrier(0);
      TQ_MARK(S, 3);
      TQ_MARK(S, 4);
      if (fast) {
        AScalePre sp;
        sp.v0 = R.r[kAhead];
        sp.v1 = R.r[kAhead + 1];
        ascale_store(as_w, sp, nb);
        // the last row's last piece may read up to 7 bytes past the tile's
        // scales: finite ones (2^0)
        if (lane == 0 && 16 * nb + 8 <= kAScaleBytes) *(uint64_t *)(as_w + 16 * nb) = 0x7F7F7F7F7F7F7F7Full;
      }
      stage(0, ne, 0, J);
      if (!fast) {
        ascale_generic<F>(as_w, srow, nb, 0, J, tile_ok);
        vm_wait<kAhead * (ALIGNED ? 1 : 2)>();
      }
      TQ_MARK(S, 5);
      lds_barrier();
      TQ_MARK(S, 6);
      mma_stream<F, NT, ALIGNED>(R, rowp, wpr, J, tile_ok, as_w, astride, nb, S.bq, S.bs, F::kSteps * J, col, on,
                                 acc, lane);
    }
    TQ_MARK(S, 7);
    __syncthreads();
    epilogue(0, ne, acc);
    TQ_MARK(S, 8);
    return;
  }
  for (int c0 = 0; c0 < ne; c0 += gsz) {
    const int ncol = min(ne - c0, gsz);
    int col[NT];
    bool on[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      col[n] = shared_cols ? (i16 & 1) : n * 16 + i16;
      on[n] = n * 8 + (i16 >> 1) < ncol;
    }
    v4f acc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = v4f{0.f, 0.f, 0.f, 0.f};
    uint32_t carry = 0u;
    for (int p0 = 0; p0 < J; p0 += kPieceMax) {
      const int np = min(J - p0, kPieceMax);
      const bool reload = c0 == 0 || J > kPieceMax;
      fetch_ahead(c0, ncol, p0, np);
      if (reload) load_tile<ALIGNED>(tl, rowp, wpr, p0, np, g);
      stage(c0, ncol, p0, np);
      if (reload && fast) {
        // (straight copy: through an AScalePre here the pair lands in scratch)
        const uint4 *sblk = (const uint4 *)(sc + row0 * nb);
        const uint4 v0 = sblk[min(lane, nb - 1)], v1 = sblk[min(lane + 64, nb - 1)];
        if (lane < nb) ((uint4 *)as_w)[lane] = v0;
        if (lane + 64 < nb) ((uint4 *)as_w)[lane + 64] = v1;
      } else if (reload) {
        ascale_generic<F>(as_w, srow, nb, p0, np, tile_ok);
      }
      vm_wait<0>();   // LDS copies of the stage
      __syncthreads();
      mma_tile<F, NT>(tl, p0, np, tile_ok, wpr, as_w, astride, fast ? p0 : 0, nb, S.bq, S.bs, F::kSteps * np, col, on,
                      acc, carry, lane);
      __syncthreads();   // everyone is done with the window's columns
    }
    epilogue(c0, ncol, acc);
  }
}

// One work item. Stage-1 items (item < n_s1): expert active[item / n_rg1],
// row group item % n_rg1 of the first matrix; columns from the activations.
// Stage-2 items: expert active[i / n_rt2], row tile i % n_rt2 of the down
// projection (i = item - n_s1); columns from the h splits. A single call
// site of the grouped GEMM serves every kind, so the kernel holds one copy
// of the matrix-core loop.
template <typename F, int NT, bool ALIGNED>
__device__ __forceinline__ void run_item(const LayerArgs &a, Shared &S, int item) {
  const int lane = tidx<NT>() & 63, wave = tidx<NT>() >> 6;
  const bool s1 = item < a.n_s1;
  const int i2 = item - a.n_s1;
  // Stage-1 items in expert order, or (s1_ilv) the experts in turn: item i
  // is row group i / n_active of expert i % n_active.
  if (s1 && a.s1_ilv && item >= S.n_active * a.n_rg1) return;   // no such item: nothing to do
  const int ai = s1 ? (a.s1_ilv ? item % S.n_active : item / a.n_rg1) : i2 / a.n_rt2;
  const int tile = s1 ? (a.s1_ilv ? item / S.n_active : item % a.n_rg1) : i2 % a.n_rt2;   // row group / row tile
  if (ai >= S.n_active) return;   // no such active expert: nothing to do
  const int e = S.active[ai];
  const bool ffn = a.mode == MODE_FFN;
  const int r0 = s1 && ffn ? (wave < 2 ? 0 : a.inter) + tile * 32 + 16 * (wave & 1) : tile * 64 + 16 * wave;
  const uint32_t *w = s1 ? a.w1 : a.w2;
  const uint8_t *sc = s1 ? a.s1 : a.s2;
  const int rows = s1 ? a.rows1 : a.rows2, K = s1 ? a.cols1 : a.cols2, fast = s1 ? a.fast1 : a.fast2;
  const int nb = K / 32;
  // (read before gather_slots' barriers: a thread may set it in this item)
  // (one token means one N-tile: compiled for NT == 1 only)
  const bool tok_first = NT == 1 && s1 && a.x_resident && !S.x_done;
  const int ne = gather_slots<NT>(S, e, a.T * a.k);
  TQ_MARK(S, 2);
  auto row_of = [&](int c) TQ_INLINE {
    const int slot = S.slots[c];
    return a.x_per_slot ? slot : slot / a.k;
  };
  const bool resident = NT == 1 && s1 && a.x_resident;
  int obs_old = 0, obs0_old = 0;
  bool waited = false;
  TokRaw tok;
  auto ahead = [&](int c0, int ncol, int kp, int np) TQ_INLINE {
    // this workgroup's first stage-1 item: the token's raw values, ahead of
    // the weight loads (split once those are out)
    if (tok_first) tok_load<F>(tok, a, nb, np);
  };
  auto stage = [&](int c0, int ncol, int kp, int np) TQ_INLINE {
    if (tok_first) {
      tok_split<F>(tok, S.bq, S.bs, F::kSteps * np, nb, a.x_bf16);
      if (tidx<NT>() == 0) S.x_done = 1;
    }
    if (resident) return;
    if (s1 && a.n_prep) {
      // The tokens were split once for the call (run_prep): wait until all
      // of them are, then copy this group's columns.
      if (!waited) {
        if (tidx<NT>() == 0) {
          spin_until(a.cntp, a.n_prep, a.status);
          obs_old = __hip_atomic_fetch_add(a.obsp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        waited = true;
      }
      copy_pass<F, NT>(S.bq, S.bs, a.xq, a.xs, a.x_steps, kp, np, nb, 2 * ncol, [&](int c) TQ_INLINE {
        return row_of(c0 + (c >> 1)) * 2 + (c & 1);
      });
      vm_wait<0>();
      return;
    }
    if (s1) {
      // Each slot its own activations: split them here. All of this
      // branch's loads are consumed within it, so none stays pending where
      // the item kinds' paths meet (the compiler's waits are not
      // path-sensitive).
      XPre xp;
      x_prefetch<F>(xp, a, K, nb, kp, np, ncol, [&](int c) TQ_INLINE { return row_of(c0 + c); });
      x_finish<F>(xp, S.bq, S.bs, a, K, nb, kp, np, ncol, [&](int c) TQ_INLINE { return row_of(c0 + c); });
      vm_wait<0>();
      return;
    }
    if (!waited) {
      // the expert's h is complete once all its stage-1 items have counted;
      // the first window's weight loads are already in flight
      if (tidx<NT>() == 0) {
        spin_until(a.cnt1 + (size_t)ai * kLineInts, a.n_rg1, a.status);
        obs_old = __hip_atomic_fetch_add(a.obs1 + (size_t)ai * kLineInts, 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
        if (ai != 0) {
          // y is cleared by the first active expert's stage-1 items: their
          // count must be complete before this item adds into y
          spin_until(a.cnt1, a.n_rg1, a.status);
          obs0_old = __hip_atomic_fetch_add(a.obs1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      __syncthreads();
      waited = true;
    }
    copy_pass<F, NT>(S.bq, S.bs, a.hq, a.hs, a.h_steps, kp, np, nb, 2 * ncol, [&](int c) TQ_INLINE {
      return S.slots[c0 + (c >> 1)] * 2 + (c & 1);
    });
    vm_wait<0>();   // (loads whose store a lane skipped count as pending for the compiler)
  };
  auto epilogue = [&](int c0, int ncol, const v4f (&acc)[NT]) TQ_INLINE {
    if (s1 && ffn) {
      // SwiGLU: gate rows in waves 0, 1, the matching up rows in waves 2, 3
      dump_acc<NT>(S, acc, wave, lane);
      __syncthreads();
      const float *red = (const float *)(S.bq + kBBytes / 2);
      for (int base = 0; base < ncol; base += kThreads / 32) {
        const int c = base + (tidx<NT>() >> 5), i = tidx<NT>() & 31;
        if (c < ncol) {   // uniform over the half-wave
          const int n = c >> 3, cj = 2 * (c & 7), wv = i >> 4, ri = i & 15;
          const float gate = red[d_index<NT>(wv, n, ri, cj)] + red[d_index<NT>(wv, n, ri, cj + 1)];
          const float up = red[d_index<NT>(wv + 2, n, ri, cj)] + red[d_index<NT>(wv + 2, n, ri, cj + 1)];
          const float silu = gate / (1.0f + expf(-gate));
          const uint16_t hb = f32_to_bf16_rne(silu * up);
          const int slot = S.slots[c0 + c];
          a.h[(size_t)slot * a.inter + tile * 32 + i] = hb;
          const Split s = split_block(bf16_to_f32(hb));
          uint8_t *q_hi = a.hq + (size_t)(slot * 2) * a.h_steps * 128;
          uint8_t *q_lo = a.hq + (size_t)(slot * 2 + 1) * a.h_steps * 128;
          st_dc8(q_hi + F::offset(tile, i), s.hi);
          st_dc8(q_lo + F::offset(tile, i), s.lo);
          if (i == 0) {
            st_dc8(a.hs + (size_t)(slot * 2) * a.h_steps * 4 + F::scale_index(tile), (uint32_t)(s.E + 127));
            st_dc8(a.hs + (size_t)(slot * 2 + 1) * a.h_steps * 4 + F::scale_index(tile), (uint32_t)(s.El + 127));
          }
        }
      }
      __syncthreads();
      return;
    }
    if (r0 >= rows) return;
    if (!s1) {
      // down projection: the gate-weighted rows go straight into y
      per_slot_out<NT>(acc, ncol, lane, [&](int c, int rr, float v) TQ_INLINE {
        const int slot = S.slots[c0 + c];
        add_dcf(a.y + (size_t)(slot / a.k) * a.y_rows + r0 + rr, S.gw[slot] * v);
      });
      return;
    }
    const bool partial = a.mode == MODE_COMBINE;
    per_slot_out<NT>(acc, ncol, lane, [&](int c, int rr, float v) TQ_INLINE {
      const int slot = S.slots[c0 + c];
      if (partial) st_dcf(a.yslot + (size_t)slot * a.y_rows + r0 + rr, v);
      else a.y[(size_t)slot * a.rows1 + r0 + rr] = v;
    });
  };
  gemm_item<F, NT, ALIGNED>(S, w, sc, rows, K, fast, e, r0, ne, resident, !s1, ahead, stage, epilogue);
  if (s1 && a.n_prep && tidx<NT>() == 0 && obs_old == S.n_active * a.n_rg1 - 1) {
    // the last stage-1 item to see the split tokens clears their counts
    st_ctr(a.cntp, 0);
    st_ctr(a.obsp, 0);
  }
  if (s1 && ffn) {
    if (ai == 0) {
      // y starts at zero: the first active expert's stage-1 items clear it,
      // a slice of rows each, before they count (every down-projection item
      // waits for that count before adding into y)
      const int z = (a.y_rows + a.n_rg1 - 1) / a.n_rg1, lo = tile * z, nz = min(a.y_rows - lo, z);
      for (int i = tidx<NT>(); i < a.T * z; i += kThreads)
        if (i % z < nz) st_dcf(a.y + (size_t)(i / z) * a.y_rows + lo + i % z, 0.0f);
    }
    stores_done();
    if (tidx<NT>() == 0)
      __hip_atomic_fetch_add(a.cnt1 + (size_t)ai * kLineInts, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  if (!s1) {
    // The last reader of a stage-1 count clears it (and its readers' count)
    // for the next call. Expert 0's count is read by every down-projection
    // item (see stage), the others' by their own expert's items.
    if (tidx<NT>() == 0) {
      const int n0 = S.n_active * a.n_rt2;
      if (obs_old == (ai == 0 ? n0 : a.n_rt2) - 1) {
        st_ctr(a.cnt1 + (size_t)ai * kLineInts, 0);
        st_ctr(a.obs1 + (size_t)ai * kLineInts, 0);
      }
      if (ai != 0 && obs0_old == n0 - 1) {
        st_ctr(a.cnt1, 0);
        st_ctr(a.obs1, 0);
      }
    }
    return;
  }
  if (a.mode == MODE_COMBINE) arrive_and_combine(a, S, tile);
}

// Work done once per call by workgroup 0: status words and the outputs of
// dead (empty / out-of-range) slots.
__device__ __forceinline__ void bookkeeping(const LayerArgs &a, Shared &S) {
  const int tid = tix(), n = a.T * a.k;
  if (tid == 0) {
    int skipped = 0;
    for (int s = 0; s < n; ++s) skipped += S.ids[s] >= a.E;
    st_ctr(&a.status[ST_SKIPPED], skipped);
  }
  for (int s = 0; s < n; ++s) {
    const int e = S.ids[s];
    if (e >= 0 && e < a.E) continue;
    if (a.mode == MODE_SLOTS)
      for (int r = tid; r < a.rows1; r += kThreads) a.y[(size_t)s * a.rows1 + r] = 0.0f;
    if (a.mode == MODE_FFN)
      for (int c = tid; c < a.inter; c += kThreads) a.h[(size_t)s * a.inter + c] = 0;
  }
  if (S.n_active == 0 && a.mode != MODE_SLOTS)
    for (int i = tid; i < a.T * a.y_rows; i += kThreads) a.y[i] = 0.0f;
}

// Split token t's activations (the stage-1 input width) once for the whole
// call: hi and lo E4M3 columns with their UE8M0 scales, in the step-chunk
// layout the stage-1 items copy into LDS. Splitting per item instead redid
// the same work for every item of every expert the token is routed to.
// The split goes to LDS first and leaves in 16-byte stores (the split's own
// byte-scattered stores, straight to global memory, took ~30 us per token).
template <typename F, int NT>
__device__ __forceinline__ void run_prep(const LayerArgs &a, Shared &S, int t) {
  const int K = a.cols1, nb = K / 32;
  const size_t el = (size_t)t * K;
  const void *xt = a.x_bf16 ? (const void *)((const uint16_t *)a.x + el) : (const void *)((const float *)a.x + el);
  TokRaw tok;
  tok_load_at(tok, xt, a.x_bf16, nb);
  tok_split<F>(tok, S.bq, S.bs, a.x_steps, nb, a.x_bf16);   // every byte of both columns (K padding: zeros)
  __syncthreads();
  {
    uint4 *dq = (uint4 *)(a.xq + (size_t)t * 2 * a.x_steps * 128);
    for (int i = tidx<NT>(); i < a.x_steps * 16; i += kThreads) dq[i] = ((const uint4 *)S.bq)[i];
    uint32_t *ds = (uint32_t *)(a.xs + (size_t)t * 2 * a.x_steps * 4);
    for (int i = tidx<NT>(); i < a.x_steps * 2; i += kThreads) ds[i] = ((const uint32_t *)S.bs)[i];
  }
  // visible device-wide before it is counted
  __threadfence();
  __syncthreads();
  if (tidx<NT>() == 0) __hip_atomic_fetch_add(a.cntp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename F, int NT, bool ALIGNED>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) k_layer(LayerArgs a) {
  __shared__ Shared S;
  const int tid = tidx<NT>();
#ifdef TQ_TRACE
  unsigned long long *TR = a.trace ? a.trace + (size_t)blockIdx.x * 512 : nullptr;
  if (TR && tid == 0) TR[0] = __builtin_amdgcn_s_memrealtime();
  if (tid == 0) S.trp = nullptr;
#endif
  if constexpr (F::kE5M3) g_e5m3_terms[tid] = e5m3_terms((uint32_t)tid);   // kThreads == 256
  if (tid == 0) {
    S.x_done = 0;
    // a wait of an earlier call on this workspace timed out: its counters
    // may be off, so the call only marks its output invalid
    S.last = __hip_atomic_load(&a.status[ST_ERROR], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (S.last) {
    if (blockIdx.x == 0) {
      const size_t ny = a.mode == MODE_SLOTS ? (size_t)a.T * a.k * a.rows1 : (size_t)a.T * a.y_rows;
      for (size_t i = tid; i < ny; i += kThreads) a.y[i] = __builtin_nanf("");
    }
    return;
  }
  // routing, redundantly in every workgroup: active experts in id order
  const int n = a.T * a.k;
  const int nw = (a.E + 31) >> 5;
  for (int i = tid; i < n; i += kThreads) {
    const int e = a.ids[i];
    S.ids[i] = (int16_t)(e < 0 ? -1 : (e >= a.E ? kMaxExperts : e));
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
      S.active[o++] = (int16_t)(w * 32 + b);
      m &= m - 1u;
    }
  }
  __syncthreads();
  if (blockIdx.x == 0) bookkeeping(a, S);

#ifdef TQ_TRACE
  if (TR && tid == 0) TR[1] = __builtin_amdgcn_s_memrealtime();
  int it_no = 0;
#endif
  const int n_items = a.n_prep + a.n_s1 + a.n_s2;
  for (int item = blockIdx.x; item < n_items; item += a.grid) {
#ifdef TQ_TRACE
    if (tid == 0) {
      S.trp = (TR && it_no < 51) ? TR + 2 + 10 * it_no : nullptr;
      if (S.trp) S.trp[0] = (unsigned long long)item;
    }
    __syncthreads();
    TQ_MARK(S, 1);
    ++it_no;
#endif
    if (item < a.n_prep) run_prep<F, NT>(a, S, item);
    else run_item<F, NT, ALIGNED>(a, S, item - a.n_prep);
    // nothing of this item stays in flight into the next one (the
    // compiler's waits in the next item then count only its own loads)
    vm_wait<0>();
    __syncthreads();
    TQ_MARK(S, 9);
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

template <typename F, int NT, bool ALIGNED>
static int resident_blocks() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  if (cached[dev] == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_layer<F, NT, ALIGNED>, kThreads, 0) != hipSuccess ||
        nb < 1)
      nb = 1;
    cached[dev] = nb;
  }
  return cached[dev];
}

// A stack of n_mat matrices of either format: base pointers as given.
struct Mats {
  const void *w;
  const uint8_t *scales;
  int n_mat, rows, cols;
};

static int check_mats(const Mats &m) {
  if (!m.w || !m.scales) return TRELLIS_ENULL;
  if (m.n_mat < 1 || m.rows < 1 || m.cols < 32 || m.cols % 32) return TRELLIS_EINVAL;
  if (m.rows % 16 || m.n_mat > kMaxExperts) return TRELLIS_EINVAL;
  return TRELLIS_OK;
}

static int check_routing(int T, int k) {
  if (T < 1 || T > kMaxT || k < 1 || k > kMaxK || T * k > kMaxSlots) return TRELLIS_EINVAL;
  return TRELLIS_OK;
}

template <typename F, int NT, bool ALIGNED>
static int launch_nt(LayerArgs &a, int cus, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int n_items = a.n_prep + a.n_s1 + a.n_s2;
  a.grid = std::max(1, std::min(n_items, cus * resident_blocks<F, NT, ALIGNED>()));
  // A single resident token whose items about fit one round of workgroups:
  // the stage-1 items take the experts in turn, so that every expert's h is
  // complete at about the same time instead of the last expert's well after
  // the first's (items dispatched later are served later by the memory
  // system). With many rounds of items (several tokens, or many experts'
  // down projections) expert order is faster.
  a.s1_ilv = a.mode == MODE_FFN && a.x_resident && 4 * n_items <= 5 * a.grid;
  if (e0 || e1)   // events stamped by the dispatch itself (start and end of the kernel's execution)
    hipExtLaunchKernelGGL((k_layer<F, NT, ALIGNED>), dim3(a.grid), dim3(kThreads), 0, s, e0, e1, 0, a);
  else
    hipLaunchKernelGGL((k_layer<F, NT, ALIGNED>), dim3(a.grid), dim3(kThreads), 0, s, a);
  return hipGetLastError() == hipSuccess ? TRELLIS_OK : TRELLIS_EHIP;
}

template <typename F, bool ALIGNED>
static int launch_al(LayerArgs &a, int cus, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  switch ((a.T + 7) / 8) {
    case 1: return launch_nt<F, 1, ALIGNED>(a, cus, s, e0, e1);
    case 2: return launch_nt<F, 2, ALIGNED>(a, cus, s, e0, e1);
    case 3: return launch_nt<F, 3, ALIGNED>(a, cus, s, e0, e1);
    default: return launch_nt<F, 4, ALIGNED>(a, cus, s, e0, e1);
  }
}

// The aligned instances need every streamed matrix to have whole 16-byte
// pieces per row (words per row % 4 == 0) and a 16-byte aligned base. The
// fast scale path needs a 16-byte aligned scale base and cols <= 4096.
template <typename F>
static int launch(LayerArgs &a, int cus, hipStream_t s, hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr) {
  const bool aligned = (a.cols1 / 32 * F::kWords) % 4 == 0 && (a.cols2 / 32 * F::kWords) % 4 == 0 &&
                       ((uintptr_t)a.w1 & 15) == 0 && ((uintptr_t)a.w2 & 15) == 0;
  a.fast1 = aligned && ((uintptr_t)a.s1 & 15) == 0 && a.cols1 / 32 <= kAScaleBytes / 16;
  a.fast2 = aligned && ((uintptr_t)a.s2 & 15) == 0 && a.cols2 / 32 <= kAScaleBytes / 16;
  return aligned ? launch_al<F, true>(a, cus, s, e0, e1) : launch_al<F, false>(a, cus, s, e0, e1);
}

// Tokens split once per call (see run_prep) when the token is not resident,
// the slots share their token's activations, K <= 4096 and x is 16-byte
// aligned (the single-token split's loads); otherwise each item splits them.
template <typename F>
static void set_prep(LayerArgs &a, const Layout &L, char *ws, bool on) {
  a.n_prep = on ? a.T : 0;
  a.x_steps = fmt_steps<F>(a.cols1 / 32);
  a.xq = (uint8_t *)(ws + L.xq); a.xs = (uint8_t *)(ws + L.xs);
  a.cntp = (int *)(ws + L.cntp); a.obsp = (int *)(ws + L.obsp);
}

template <typename F>
static int gemv_impl(hipStream_t stream, const Mats &w, const void *x, int32_t x_dtype, int32_t x_per_slot,
                     const int32_t *topk_ids, const float *topk_w, int32_t T, int32_t k, float *y,
                     void *workspace, size_t workspace_bytes) {
  int rc = check_mats(w);
  if (rc) return rc;
  if (!x || !topk_ids || !y || !workspace) return TRELLIS_ENULL;
  if ((x_dtype != TRELLIS_F32 && x_dtype != TRELLIS_BF16) || (x_per_slot != 0 && x_per_slot != 1))
    return TRELLIS_EINVAL;
  if ((rc = check_routing(T, k))) return rc;
  const bool combine = topk_w != nullptr;
  const int n_rt = (w.rows + 63) / 64;
  const Layout L = make_layout<F>(0, n_rt, T * k, w.rows, 0, T, w.cols);
  if (((uintptr_t)workspace & 255) || workspace_bytes < L.total) return TRELLIS_EWORKSPACE;
  int cus = 0;
  if ((rc = device_check(&cus))) return rc;
  char *ws = (char *)workspace;
  {
    // one token, shared x, every slot's output: the single-token GEMV kernel
    TokGemvCall c{(const uint32_t *)w.w, w.scales, w.n_mat, w.rows, w.cols, k, topk_ids, x,
                  x_dtype == TRELLIS_BF16, y, (int *)(ws + L.status), F::kSteps == 1, F::kE5M3};
    if (T == 1 && !combine && !x_per_slot && tok_gemv_supported(c, cus)) return tok_gemv_launch(c, cus, stream);
  }
  LayerArgs a{};
  a.mode = combine ? MODE_COMBINE : MODE_SLOTS;
  a.w1 = (const uint32_t *)w.w; a.s1 = w.scales; a.rows1 = w.rows; a.cols1 = w.cols;
  a.w2 = (const uint32_t *)w.w; a.s2 = w.scales; a.rows2 = w.rows; a.cols2 = w.cols;
  a.E = w.n_mat; a.T = T; a.k = k; a.ids = topk_ids; a.gate_w = topk_w;
  a.x = x; a.x_bf16 = x_dtype == TRELLIS_BF16; a.x_per_slot = x_per_slot;
  a.y = y; a.y_rows = w.rows;
  a.status = (int *)(ws + L.status);
  a.cnt2 = (int *)(ws + L.cnt2);
  a.yslot = (float *)(ws + L.yslot);
  a.n_rg1 = n_rt;
  a.n_s1 = std::min(w.n_mat, T * k) * a.n_rg1;
  a.n_rt2 = 1; a.n_s2 = 0;
  const int J = (w.cols / 32 + F::kBlocks - 1) / F::kBlocks;
  a.x_resident = T == 1 && !x_per_slot && J <= kPieceMax && ((uintptr_t)x & 15) == 0;
  set_prep<F>(a, L, ws, !a.x_resident && !x_per_slot && w.cols / 32 <= 64 * kTokRounds && ((uintptr_t)x & 15) == 0);
  return launch<F>(a, cus, stream);
}

// Zero the 16-byte words [0, n0) of p0 and [0, n1) of p1 (vector stores).
static __global__ void __launch_bounds__(256) k_clear2(uint4 *p0, size_t n0, uint4 *p1, size_t n1) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n0 + n1; i += stride)
    (i < n0 ? p0[i] : p1[i - n0]) = make_uint4(0u, 0u, 0u, 0u);
}

// clear_state: first zero the workspace's synchronisation state on the
// stream (every counter and tagged word; the status words stay), so that a
// workspace last used by a call of another shape serves this one.
template <typename F>
static int ffn_impl(hipStream_t stream, const Mats &gu, const Mats &dn, const void *x, int32_t x_dtype,
                    const int32_t *topk_ids, const float *topk_w, int32_t T, int32_t k, uint16_t *h, float *y,
                    void *workspace, size_t workspace_bytes, hipEvent_t *events, bool clear_state = false) {
  int rc;
  if ((rc = check_mats(gu)) || (rc = check_mats(dn))) return rc;
  if (!x || !topk_ids || !h || !y || !workspace) return TRELLIS_ENULL;
  if (x_dtype != TRELLIS_F32 && x_dtype != TRELLIS_BF16) return TRELLIS_EINVAL;
  if ((rc = check_routing(T, k))) return rc;
  const int E = gu.n_mat, hidden = gu.cols, inter = gu.rows / 2;
  if (gu.rows % 64 || dn.n_mat != E || dn.rows != hidden || dn.cols != inter) return TRELLIS_EINVAL;
  const int max_act = std::min(E, T * k);
  // (no partial outputs or combine counters: the down projection adds into y)
  const Layout L = make_layout<F>(max_act, 0, T * k, 0, inter, T, hidden, tok_region(E, hidden, inter).total);
  if (((uintptr_t)workspace & 255) || workspace_bytes < L.total) return TRELLIS_EWORKSPACE;
  int cus = 0;
  if ((rc = device_check(&cus))) return rc;
  char *ws = (char *)workspace;
  if (clear_state) {
    // [end of the status words, first data region) and [cntp, xq): the
    // single-token region, the stage counters and the prep counters
    const size_t n0 = (L.yslot - (L.status + 256)) / 16, n1 = (L.xq - L.cntp) / 16;
    const int blocks = (int)std::min<size_t>((n0 + n1 + 255) / 256, 1024);
    hipLaunchKernelGGL(k_clear2, dim3(blocks), dim3(256), 0, stream, (uint4 *)(ws + L.status + 256), n0,
                       (uint4 *)(ws + L.cntp), n1);
    if (hipGetLastError() != hipSuccess) return TRELLIS_EHIP;
  }
  {
    // one token (trellis-coded under either scale format, or expanded
    // MXFP4): the single-token layer kernel
    TokCall c{(const uint32_t *)gu.w, gu.scales, (const uint32_t *)dn.w, dn.scales, E, hidden, inter, k,
              topk_ids, topk_w, x, x_dtype == TRELLIS_BF16, h, y, ws, L.reserve, F::kSteps == 1, F::kE5M3};
    if (T == 1 && tok_supported(c, cus))
      return tok_launch(c, cus, stream, events ? events[0] : nullptr, events ? events[1] : nullptr);
  }
  LayerArgs a{};
  a.mode = MODE_FFN;
  a.w1 = (const uint32_t *)gu.w; a.s1 = gu.scales; a.rows1 = gu.rows; a.cols1 = hidden;
  a.w2 = (const uint32_t *)dn.w; a.s2 = dn.scales; a.rows2 = hidden; a.cols2 = inter;
  a.E = E; a.T = T; a.k = k; a.ids = topk_ids; a.gate_w = topk_w;
  a.x = x; a.x_bf16 = x_dtype == TRELLIS_BF16; a.x_per_slot = 0;
  a.inter = inter; a.h = h;
  a.h_steps = fmt_steps<F>(inter / 32);
  a.hq = (uint8_t *)(ws + L.hq); a.hs = (uint8_t *)(ws + L.hs);
  a.y = y; a.y_rows = hidden;
  a.status = (int *)(ws + L.status);
  a.cnt1 = (int *)(ws + L.cnt1); a.obs1 = (int *)(ws + L.obs1);
#ifdef TQ_TRACE
  a.trace = (unsigned long long *)g_trace;
#endif
  a.n_rg1 = inter / 32;
  a.n_s1 = max_act * a.n_rg1;
  a.n_rt2 = (hidden + 63) / 64;
  a.n_s2 = max_act * a.n_rt2;
  const int J = (hidden / 32 + F::kBlocks - 1) / F::kBlocks;
  a.x_resident = T == 1 && J <= kPieceMax && ((uintptr_t)x & 15) == 0;
  set_prep<F>(a, L, ws, !a.x_resident && hidden / 32 <= 64 * kTokRounds && ((uintptr_t)x & 15) == 0);
  return launch<F>(a, cus, stream, events ? events[0] : nullptr, events ? events[1] : nullptr);
}

static Mats trellis_mats(const trellis_mat_t *w) {
  return w ? Mats{w->syms, w->scales, w->n_mat, w->rows, w->cols} : Mats{nullptr, nullptr, 0, 0, 0};
}
static Mats mx_mats(const trellis_mx_t *w) {
  return w ? Mats{w->codes, w->scales, w->n_mat, w->rows, w->cols} : Mats{nullptr, nullptr, 0, 0, 0};
}

}  // namespace tq

// tq_tok.hip -- one mixture-of-experts layer for a single token, weights
// decoded inside the kernel, on gfx950.
//
// HEPH abstract (ICLR 2027 submission page), fused serving mode: the trellis
// streams stay resident and are decoded in the grouped-MoE kernel on every
// forward pass. The decoder is the XOR-Trellis one (news article, bullet
// "XOR-Trellis FP4 decoder"), bit-sliced in tq_decode.h; the decoded E2M1
// nibbles and the weights' UE8M0 bytes feed the block-scaled FP4 x FP8
// matrix cores, the token's activations entering as a two-term FP8 split.
// The same kernel serves expand mode (HEPH abstract): weights already
// expanded to MXFP4 go to the matrix cores as loaded, with no decode; and
// trellis streams under E5M3 block scales (each matrix-core step issued
// once per power-of-two term of its scale).
//
// Why a kernel of its own for one token: the layer moves ~28 MB at the
// 32-expert shape and every weight costs ~1.5 VALU operations to decode, so
// the decode work alone keeps all 1024 SIMDs busy for about as long as HBM
// needs to deliver the bytes. Both must overlap on every compute unit, and
// every compute unit must carry the same share. So:
//  - one workgroup per compute unit (the grid is the compute-unit count; a
//    large dynamic LDS request keeps a second one off each unit);
//  - work comes in units of equal decode cost: a "pair" (16 gate rows and
//    the 16 matching up rows of one active expert, giving 16 values of h)
//    and a "down tile" (16 rows of one active expert's down projection).
//    Workgroup w takes pairs [w NP / G, (w+1) NP / G) and down tiles
//    [w' ND / G, (w'+1) ND / G) with w' = G-1-w, so no unit carries more
//    than one pair or one down tile above the average;
//  - inside a workgroup the waves split every tile along K: wave v owns
//    piece v (16 rows x 64 bytes, 256 weights per row) of each of the
//    workgroup's tiles, so the four SIMDs share the decode evenly and a
//    wave's activation operand (its piece of x) is read from LDS once and
//    used for all its tiles. Partial sums meet in LDS and are added in
//    piece order (h is deterministic);
//  - every weight load of a wave is issued at the start, in the order it is
//    consumed (loads complete in issue order): pairs first, then the down
//    tiles, which are decoded ahead while the workgroup waits for h;
//  - h crosses workgroups as tagged 64-bit words (call tag in the high
//    half, two bf16 values in the low half) stored device-coherently: a
//    consumer polls the words themselves, so no counter round trip and no
//    fence lies between the last pair and the down projection;
//  - y is cleared tile by tile (each 16-row tile by one workgroup, which
//    then tags it) and the down tiles add their gate-weighted rows into it
//    with device-scope float atomics.
// The call tag comes from a counter in the workspace: every workgroup reads
// it at entry and then counts itself in; the last to count advances it.
// Every wait is bounded; a timeout sets a sticky error word, and a call
// that finds it set writes NaN to y and does nothing else.
#include "tq_tok.h"

#include <hip/hip_ext.h>

#include <math.h>

#include <algorithm>

#include "tq_common.h"

namespace tq {
namespace {

constexpr int kMaxJ = 16;            // 256-weight pieces per row: K <= 4096
constexpr int kMaxSlots = 32;        // k
constexpr int kMaxEx = 2;            // experts spanned by one workgroup's down tiles
constexpr int kMaxPairs = 3;         // pairs per workgroup
constexpr int kMaxDown = 8;          // down tiles per workgroup
constexpr size_t kCuLds = 160 * 1024;   // LDS of a compute unit
constexpr unsigned kPolls = 1u << 20;

struct Args {
  const uint32_t *w1; const uint8_t *s1;
  const uint32_t *w2; const uint8_t *s2;
  int E, H, I, k;
  const int32_t *ids; const float *gate_w;
  const void *x; int x_bf16;
  uint16_t *h; float *y;
  int *status;          // [0] skipped slots, [1] sticky error
  uint32_t *sync;       // [0] call counter, [32] arrivals (own 128-byte line)
  uint64_t *hx;         // [n_exp <= 32][I / 2]: tag << 32 | bf16 pair
  uint32_t *yz;         // [H / 16]: tag of the call that cleared the tile
  int G;
  // routed instances: the router rows, and where workgroup 0 writes the
  // routing it computed (ids and gate_w above are then unused)
  const uint16_t *w_router;   // [E][H] bf16
  int32_t *ids_out; float *gw_out;
#ifdef TQ_TRACE
  unsigned long long *trace;   // [G][16] s_memrealtime stamps
#endif
};

// Timeline instrumentation, compiled in only with -DTQ_TRACE: thread 0 of
// each workgroup stamps s_memrealtime at the phase boundaries.
#ifdef TQ_TRACE
#define TOK_MARK_T(k, t) do { if (threadIdx.x == (t)) S.trace[k] = __builtin_amdgcn_s_memrealtime(); } while (0)
#define TOK_MARK(k) TOK_MARK_T(k, 0)
static unsigned long long *g_tok_trace = nullptr;
#else
#define TOK_MARK(k) do { } while (0)
#define TOK_MARK_T(k, t) do { } while (0)
#endif

struct Smem {
  // activation splits in the matrix-core step-chunk layout: column c holds
  // 2J steps of 128 code bytes, its scales 2J x 4 bytes
  uint8_t xq[2 * 2 * kMaxJ * 128];                 // x: hi, lo
  uint8_t xs[2 * 2 * kMaxJ * 4];
  uint8_t hq[2 * kMaxEx * 2 * kMaxJ * 128];        // h of up to two experts: hi, lo each
  uint8_t hs[2 * kMaxEx * 2 * kMaxJ * 4];
  float red1[2 * kMaxPairs][4][16];                // [tile][wave][row] partial sums
  float red2[kMaxDown][4][16];
  uint32_t tag;
  int poisoned;
  int x_ready;      // the call tag is in LDS
  int up_issued;    // gate/up waves that have issued all their loads
  int up_done;      // gate/up waves that have stored their partial sums
  int down_done;    // down waves that have stored theirs
  uint32_t e5t[256];   // E5M3 instances: e5m3_terms of every scale byte
#ifdef TQ_TRACE
  unsigned long long trace[16];   // phase stamps, copied out at the end
#endif
};

__device__ __forceinline__ uint64_t ld_dc64(const uint64_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dc32(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dc64(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dc32(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void set_error(int *status) {
  __hip_atomic_fetch_or(&status[1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Maximum of non-negative floats over the four lanes of a quad (integer
// order equals float order for them).
__device__ __forceinline__ float quad_max4(float v) {
  int m = __float_as_int(v);
  m = max(m, __builtin_amdgcn_update_dpp(0, m, 0xB1, 0xF, 0xF, false));
  m = max(m, __builtin_amdgcn_update_dpp(0, m, 0x4E, 0xF, 0xF, false));
  return __int_as_float(m);
}

// Two-term FP8 split of one 32-value block held by a quad (lane j of the
// quad: values 8j .. 8j+7): hi = E4M3(v / 2^E), lo = E4M3((v - hi 2^E) / 2^El),
// each with its UE8M0 exponent, written into column pair (lq, lq + psteps*128)
// at block b's place in the step-chunk layout of the weight format (MX:
// expanded MXFP4, natural order, block b in step b / 4 as K-block b % 4;
// otherwise the trellis decoder's order). `store` is uniform per quad.
template <bool MX>
__device__ __forceinline__ void split_block8(const float (&f)[8], int b, int j, uint8_t *lq, uint8_t *ls,
                                             int psteps, bool store) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
  const int E = block_exponent(quad_max4(m));
  uint32_t hi[4], lo[4];
  float res[8], m2 = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    hi[i / 2] = f32x2_to_e4m3(ldexpf(f[i], -E), ldexpf(f[i + 1], -E));
    res[i] = f[i] - ldexpf(e4m3_to_f32(hi[i / 2]), E);
    res[i + 1] = f[i + 1] - ldexpf(e4m3_to_f32(hi[i / 2] >> 8), E);
    m2 = fmaxf(m2, fmaxf(fabsf(res[i]), fabsf(res[i + 1])));
  }
  const int El = block_exponent(quad_max4(m2));
#pragma unroll
  for (int i = 0; i < 8; i += 2) lo[i / 2] = f32x2_to_e4m3(ldexpf(res[i], -El), ldexpf(res[i + 1], -El));
  if (!store) return;
  const uint32_t h01 = hi[0] | hi[1] << 16, h23 = hi[2] | hi[3] << 16;
  const uint32_t l01 = lo[0] | lo[1] << 16, l23 = lo[2] | lo[3] << 16;
  if (MX) {
    // values 8j .. 8j+7 are eight consecutive bytes of the chunk
    const int off = (b >> 2) * 128 + bchunk_offset(32 * (b & 3) + 8 * j);
    *(uint2 *)(lq + off) = make_uint2(h01, h23);
    *(uint2 *)(lq + (size_t)psteps * 128 + off) = make_uint2(l01, l23);
    if (j == 0) {
      ls[b] = (uint8_t)(E + 127);
      ls[(size_t)psteps * 4 + b] = (uint8_t)(El + 127);
    }
    return;
  }
  // values 8j + 2m (m = 0..3) sit at four consecutive bytes of the chunk,
  // values 8j + 2m + 1 eight bytes further on (the decoder's even/odd order)
  const int off = act_offset(b, 8 * j);
  *(uint32_t *)(lq + off) = __builtin_amdgcn_perm(h23, h01, 0x06040200u);
  *(uint32_t *)(lq + off + 8) = __builtin_amdgcn_perm(h23, h01, 0x07050301u);
  *(uint32_t *)(lq + (size_t)psteps * 128 + off) = __builtin_amdgcn_perm(l23, l01, 0x06040200u);
  *(uint32_t *)(lq + (size_t)psteps * 128 + off + 8) = __builtin_amdgcn_perm(l23, l01, 0x07050301u);
  if (j == 0) {
    ls[act_scale_index(b)] = (uint8_t)(E + 127);
    ls[(size_t)psteps * 4 + act_scale_index(b)] = (uint8_t)(El + 127);
  }
}

// The 32 bytes of B operand (column c, step st) for this lane's K-block g,
// and the column's UE8M0 byte of that block.
struct BOp {
  v8i b;
  uint32_t s;
};
__device__ __forceinline__ BOp read_b(const uint8_t *lq, const uint8_t *ls, int psteps, int c, int st, int g) {
  const uint4 *p = (const uint4 *)(lq + ((size_t)c * psteps + st) * 128 + g * 32);
  const uint4 u0 = p[0], u1 = p[1];
  BOp o;
  o.b = v8i{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
  o.s = ls[((size_t)c * psteps + st) * 4 + g];
  return o;
}

// Matrix-core steps 2p and 2p+1 of a decoded piece (A), x or h operands (B);
// byte 0 / 1 of `sa` is the A scale of step 2p / 2p+1.
struct DecA {
  uint4 s0, s1;
};
__device__ __forceinline__ v4f mma2(const DecA &d, const BOp &b0, const BOp &b1, uint32_t sa, v4f acc) {
  const v8i A0 = v8i{(int)d.s0.x, (int)d.s0.y, (int)d.s0.z, (int)d.s0.w, 0, 0, 0, 0};
  const v8i A1 = v8i{(int)d.s1.x, (int)d.s1.y, (int)d.s1.z, (int)d.s1.w, 0, 0, 0, 0};
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A0, b0.b, acc, 4, 0, 0, (int)sa, 0, (int)b0.s);
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A1, b1.b, acc, 4, 0, 1, (int)sa, 0, (int)b1.s);
  return acc;
}

// The same two steps under E5M3 block scales (XOR-Trellis article, the
// paragraph on the grouping format; reading: unsigned binary16 upper byte).
// The matrix cores take power-of-two A scales only, so each scale byte is
// looked up in `terms` (e5m3_terms of every byte: four UE8M0 terms that sum
// to it exactly) and the step is issued once per term, byte select i, on
// one accumulator; a zero scale has no such sum and zeroes A instead.
__device__ __forceinline__ v4f mma2_e5m3(const DecA &d, const BOp &b0, const BOp &b1, uint32_t sa, v4f acc,
                                         const uint32_t *terms) {
  const uint32_t t0 = terms[sa & 0xFFu], t1 = terms[(sa >> 8) & 0xFFu];
  const v8i A0 = t0 ? v8i{(int)d.s0.x, (int)d.s0.y, (int)d.s0.z, (int)d.s0.w, 0, 0, 0, 0} : v8i{0, 0, 0, 0, 0, 0, 0, 0};
  const v8i A1 = t1 ? v8i{(int)d.s1.x, (int)d.s1.y, (int)d.s1.z, (int)d.s1.w, 0, 0, 0, 0} : v8i{0, 0, 0, 0, 0, 0, 0, 0};
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A0, b0.b, acc, 4, 0, 0, (int)t0, 0, (int)b0.s);
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A0, b0.b, acc, 4, 0, 1, (int)t0, 0, (int)b0.s);
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A0, b0.b, acc, 4, 0, 2, (int)t0, 0, (int)b0.s);
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A0, b0.b, acc, 4, 0, 3, (int)t0, 0, (int)b0.s);
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A1, b1.b, acc, 4, 0, 0, (int)t1, 0, (int)b1.s);
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A1, b1.b, acc, 4, 0, 1, (int)t1, 0, (int)b1.s);
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A1, b1.b, acc, 4, 0, 2, (int)t1, 0, (int)b1.s);
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A1, b1.b, acc, 4, 0, 3, (int)t1, 0, (int)b1.s);
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for LDS hand-offs: this wave's LDS accesses are done,
// then s_barrier. Unlike __syncthreads it does not wait for the wave's
// outstanding global loads, so weight loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Row i of the 16-row tile as fp32: D column 0 (hi term) + column 1 (lo
// term). Lane (i16 = 0, g) returns rows 4g .. 4g+3.
__device__ __forceinline__ float pair_sum(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}

// Keep a decoded operand in registers here: the compiler would otherwise
// sink the decode of the down pieces to their use, after the wait for h.
__device__ __forceinline__ void pin(DecA &d) {
  asm volatile("" : "+v"(d.s0.x), "+v"(d.s0.y), "+v"(d.s0.z), "+v"(d.s0.w), "+v"(d.s1.x), "+v"(d.s1.y),
               "+v"(d.s1.z), "+v"(d.s1.w));
}

// One wave's loads of one tile: its PPW pieces and, for trellis streams,
// the word before its first piece (decoder history of lane-group 0). A
// piece is 8 blocks of 32 weights of each of the 16 rows, two matrix-core
// steps. Trellis: 16 bytes of symbols per lane (blocks 8p+2g, 8p+2g+1),
// decoded into the two steps' A operands. Expanded MXFP4 (MX): the two A
// operands as stored, 16 bytes each (blocks 8p+g and 8p+4+g).
template <int PPW, bool MX>
struct TileLd {
  uint4 w[MX ? 2 * PPW : PPW];
  uint32_t hist;
  uint32_t sc[PPW];   // the UE8M0 bytes of the piece's two blocks (byte 0: first step)
};

// Decode piece words `a` whose history is `hist` (lane-group 0: the word
// before the piece; others: the neighbour's last word).
__device__ __forceinline__ DecA decode_words(const uint4 &a, uint32_t hist) {
  const nib2 d0 = decode_word(a.x, hist), d1 = decode_word(a.y, a.x);
  const nib2 d2 = decode_word(a.z, a.y), d3 = decode_word(a.w, a.z);
  DecA d;
  d.s0 = make_uint4(d0.even, d0.odd, d1.even, d1.odd);
  d.s1 = make_uint4(d2.even, d2.odd, d3.even, d3.odd);
  return d;
}

// One token's routing, in every lane of a wave: lane s (< k; lanes 32-63
// mirror 0-31) holds slot s's expert id `idv` and gate weight `gwr`. The
// active experts are taken in order of first occurrence; a duplicate slot
// adds its gate weight to its expert's, in slot order. Lane r < n_act
// receives active expert r (act_e) and its summed gate weight (act_g) by a
// forward permutation: first occurrences to their rank, the other low lanes
// after them, the high lanes to themselves.
struct TokRoute {
  bool valid;      // this lane's slot routes to an expert of the stack
  int rank;        // active index of this slot's expert
  int n_act, n_skipped;
  int act_e;
  float act_g;
};
__device__ __forceinline__ TokRoute tok_route(int lane, int k, int E, int idv, float gwr, bool weighted) {
  TokRoute R;
  const int sl = lane & 31;
  R.valid = sl < k && idv >= 0 && idv < E;
  const int e_me = R.valid ? idv : -1;
  const float gw_me = weighted ? gwr : 1.0f;
  bool first = R.valid;
  int dup_of = sl;
  float gsum = 0.0f;
  for (int s2 = 0; s2 < k; ++s2) {
    const int e2 = __builtin_amdgcn_readlane(e_me, s2);
    const float w2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gw_me), s2));
    if (R.valid && e2 == e_me) {
      gsum += w2;
      if (s2 < sl && first) {
        first = false;
        dup_of = s2;
      }
    }
  }
  const uint32_t fm = (uint32_t)__ballot(first);
  R.n_skipped = __popc((uint32_t)__ballot(sl < k && idv >= E));
  R.n_act = __popc(fm);
  R.rank = __popc(fm & ((1u << dup_of) - 1u));
  const int dst = lane >= 32 ? lane : first ? R.rank : R.n_act + __popc(~fm & ((1u << sl) - 1u));
  R.act_e = __builtin_amdgcn_ds_permute(dst << 2, e_me);
  R.act_g = __int_as_float(__builtin_amdgcn_ds_permute(dst << 2, __float_as_int(gsum)));
  return R;
}

// A operands of piece q of a tile (trellis: decoded, history `hist`).
template <int PPW, bool MX>
__device__ __forceinline__ DecA piece_a(const TileLd<PPW, MX> &L, int q, uint32_t hist) {
  if constexpr (MX) {
    DecA d;
    d.s0 = L.w[2 * q];
    d.s1 = L.w[2 * q + 1];
    return d;
  } else {
    return decode_words(L.w[q], hist);
  }
}

// The router in front of the layer, computed by every workgroup for the one
// token (routed instances): logits[e] = sum_h x[h] w_router[e][h], the k
// largest in descending order (ties to the lower id), gate weights = softmax
// over them. The arithmetic is the standalone router's (trellis_router_topk)
// step for step -- fp64 sums of exact products, lane-sequential over 16-byte
// chunks and then an xor butterfly; k rounds of a wave-wide argmax; an fp64
// softmax rounded to fp32 -- so both give the same bits. Wave v takes the
// experts v, v + 8, v + 16, v + 24, issuing every load of their router rows
// before anything waits, and sums them as independent chains; x goes
// through LDS as fp32. Lane j < k returns pick j (id, gate weight); lanes
// 32..63 mirror 0..31. E <= 32, H <= 4096.
constexpr int kRtMaxE = 32, kRtMaxH = 4096;
__device__ __forceinline__ void tok_router(const Args &a, int tid, int *idv, float *gwr) {
  __shared__ float rx[kRtMaxH];
  __shared__ double rlg[kRtMaxE];
  const int lane = tid & 63, wave = tid >> 6;
  const int H = a.H, nq = H / 8;
  constexpr int kLd = kRtMaxH / 8 / 64;   // 16-byte loads per lane and expert, at most
  constexpr int kPer = kRtMaxE / 8;       // experts per wave, at most
  uint4 r[kPer][kLd];
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    const uint4 *row = (const uint4 *)(a.w_router + (size_t)min(wave + 8 * m, a.E - 1) * H);
#pragma unroll
    for (int i = 0; i < kLd; ++i) r[m][i] = row[min(lane + 64 * i, nq - 1)];
  }
  {
    const int nx = H * (a.x_bf16 ? 2 : 4) / 16;   // 16-byte loads of x
    for (int c = tid; c < nx; c += 512) {
      const uint4 v = ((const uint4 *)a.x)[c];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
      if (a.x_bf16) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          rx[8 * c + 2 * j] = bf16_to_f32((uint16_t)(u[j] & 0xFFFFu));
          rx[8 * c + 2 * j + 1] = bf16_to_f32((uint16_t)(u[j] >> 16));
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) rx[4 * c + j] = __uint_as_float(u[j]);
      }
    }
  }
  __syncthreads();
  double sum[kPer];
#pragma unroll
  for (int m = 0; m < kPer; ++m) sum[m] = 0.0;
#pragma unroll
  for (int i = 0; i < kLd; ++i) {
    const int q = lane + 64 * i;
    if (q < nq) {
#pragma unroll
      for (int m = 0; m < kPer; ++m) {
        const uint32_t wv[4] = {r[m][i].x, r[m][i].y, r[m][i].z, r[m][i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sum[m] += (double)rx[8 * q + 2 * j] * (double)bf16_to_f32((uint16_t)(wv[j] & 0xFFFFu));
          sum[m] += (double)rx[8 * q + 2 * j + 1] * (double)bf16_to_f32((uint16_t)(wv[j] >> 16));
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum[m] += __shfl_xor(sum[m], off);
    if (lane == 0 && wave + 8 * m < a.E) rlg[wave + 8 * m] = sum[m];
  }
  __syncthreads();
  // every wave picks the top k itself (lane l owns expert l)
  const double lv = rlg[min(lane, a.E - 1)];
  bool taken = false;
  int my_pick = 0;
  double my_val = 0.0, top = 0.0;
  for (int j = 0; j < a.k; ++j) {
    double bv = -INFINITY;
    int be = -1;
    if (lane < a.E && !taken) {
      bv = lv;
      be = lane;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const double ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      if (oe >= 0 && (be < 0 || ov > bv || (ov == bv && oe < be))) {
        bv = ov;
        be = oe;
      }
    }
    if (be == lane) taken = true;
    if (lane == j) {
      my_pick = be;
      my_val = bv;
    }
    if (j == 0) top = bv;
  }
  const double ex = lane < a.k ? exp(my_val - top) : 0.0;
  double den = ex;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off);
  const float g = (float)(ex / den);
  if (blockIdx.x == 0 && wave == 0 && lane < a.k) {
    a.ids_out[lane] = my_pick;
    a.gw_out[lane] = g;
  }
  *idv = __shfl(my_pick, lane & 31);
  *gwr = __shfl(g, lane & 31);
}

// Eight waves, two per SIMD, in two roles. Waves 0-3 ("gate/up waves")
// each own PPW consecutive pieces of every gate/up tile of the workgroup
// (T1 tiles at most), streamed through a register ring AT tiles deep (a
// wave that issued all its loads at once would sit at the issue, which
// stalls until the memory pipeline has room, instead of decoding what has
// arrived); they run at raised priority. Waves 4-7 ("down waves") split x
// and clear the workgroup's tiles of y, then, once every gate/up load of
// the workgroup is issued, load PPW pieces of each down tile (T2 at most)
// and decode them while the gate/up waves work and h is on its way; after
// h arrives they run the down projection's matrix-core steps. The roles
// meet through LDS flags until the gate/up work is done, so neither waits
// at a barrier for the other's loads. MX: the weights are expanded MXFP4
// (codes [rows][cols / 2], even column in the low nibble, same scales),
// fed to the matrix cores as loaded; the activations take that format's
// layout. E5: the scale bytes are E5M3 (trellis streams only). RT: the
// kernel computes the routing itself (tok_router) instead of reading it.
template <int PPW, int T1, int T2, int AT, bool MX, bool E5, bool RT = false>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) k_tok(Args a) {
  static_assert(!(MX && E5), "E5M3 scales are served on trellis streams");
  constexpr int NW = 8, NR = 4;   // waves, waves per role
  __shared__ Smem S;
#ifdef TQ_TRACE
  const unsigned long long t_entry = __builtin_amdgcn_s_memrealtime();
#endif
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool up_role = wave < NR;           // gate/up wave
  const int rw = wave & (NR - 1);           // index within the role
  const int i16 = lane & 15, g = lane >> 4;
  const int w = blockIdx.x, G = a.G;
  const int H = a.H, I = a.I;
  const int nb1 = H >> 5, J1 = (nb1 + 7) >> 3, wpr1 = H >> 4, ps1 = 2 * J1;
  const int nb2 = I >> 5, J2 = (nb2 + 7) >> 3, wpr2 = I >> 4, ps2 = 2 * J2;
  const int rt_per = H >> 4, pr_per = I >> 4;   // down tiles / pairs per expert
  const int src = ((lane - 16) & 63) << 2;       // lane-group g-1, same row (ds_bpermute address)
  const int rtid = tid & (64 * NR - 1);          // thread index within the role
  if (E5 && tid < 256) S.e5t[tid] = e5m3_terms((uint32_t)tid);
  if (tid == 0) {
    S.x_ready = 0;
    S.up_issued = 0;
    S.up_done = 0;
    S.down_done = 0;
  }
  __syncthreads();   // (nothing is in flight yet)
#ifdef TQ_TRACE
  if (tid == 0) S.trace[0] = t_entry;
#endif

  // ---- routing inputs (every wave), x and the call counter (down waves).
  // Every global load up to the wait for h is unconditional within its
  // role (clamped addresses), so the compiler's waits count exactly the
  // loads issued after each one.
  const int sl = lane & 31, slc = sl < a.k ? sl : 0;
  int idv;
  float gwr;
  if constexpr (RT) {
    tok_router(a, tid, &idv, &gwr);
  } else {
    idv = a.ids[slc];
    gwr = *(a.gate_w ? a.gate_w + slc : (const float *)(a.ids + slc));
  }
  // x: a gate/up wave splits the 32-value blocks of its own pieces
  // (8 PPW of them, four lanes each, 16 per pass), loaded ahead of its tiles
  constexpr int kXPass = (8 * PPW + 15) / 16;
  uint4 xr[kXPass][2];
  uint32_t epoch = 0;
  int err0 = 0;
  if (up_role) {
    const int pa1 = min(rw * PPW, J1);
#pragma unroll
    for (int ps = 0; ps < kXPass; ++ps) {
      const int xb = 8 * pa1 + 16 * ps + (lane >> 2), xj = lane & 3;
      const int xbc = xb < nb1 ? xb : 0;
      const char *xp = (const char *)a.x + (size_t)(32 * xbc + 8 * xj) * (a.x_bf16 ? 2 : 4);
      xr[ps][0] = *(const uint4 *)xp;
      xr[ps][1] = *(const uint4 *)(a.x_bf16 ? xp : xp + 16);
    }
  } else {
    epoch = ld_dc32(a.sync);
    err0 = __hip_atomic_load(&a.status[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- routing, in every wave's registers (tok_route)
  const TokRoute route = tok_route(lane, a.k, a.E, idv, gwr, RT || a.gate_w != nullptr);
  const bool valid = route.valid;
  const int n_skipped = route.n_skipped, n_act = route.n_act, rank = route.rank;
  const int act_e = route.act_e;
  const float act_g = route.act_g;
  TOK_MARK(1);

  // ---- this workgroup's units: pairs [p0, p0 + np), down tiles [d0, d0 + nd)
  const uint32_t NP = (uint32_t)n_act * pr_per, ND = (uint32_t)n_act * rt_per;
  const int wd = G - 1 - w;
  const int p0 = (int)((uint32_t)w * NP / (uint32_t)G), np = (int)((uint32_t)(w + 1) * NP / (uint32_t)G) - p0;
  const int d0 = (int)((uint32_t)wd * ND / (uint32_t)G), nd = (int)((uint32_t)(wd + 1) * ND / (uint32_t)G) - d0;
  const int n1 = 2 * np;
  // this wave's pieces [pa, pa + c) of each of its role's tiles
  const int J = up_role ? J1 : J2;
  const int pa = min(rw * PPW, J), c = min(J - pa, PPW);
  // loads of the tile whose first row is `r0` (gate/up matrix if s1)
  auto load_tile = [&](size_t r0, bool s1) -> TileLd<PPW, MX> {
    TileLd<PPW, MX> L;
    const size_t r = r0 + i16;
    const uint8_t *sp = s1 ? a.s1 + r * nb1 : a.s2 + r * nb2;
    const int nb = s1 ? nb1 : nb2;
    if constexpr (MX) {
      // 16 bytes per block; the row's last block stands in for blocks past it
      const uint8_t *rp = (const uint8_t *)(s1 ? a.w1 : a.w2) + r * (size_t)nb * 16;
#pragma unroll
      for (int q = 0; q < PPW; ++q)
        L.sc[q] = (uint32_t)sp[min(8 * (pa + q) + g, nb - 1)] | (uint32_t)sp[min(8 * (pa + q) + 4 + g, nb - 1)] << 8;
#pragma unroll
      for (int q = 0; q < PPW; ++q) {
        L.w[2 * q] = *(const uint4 *)(rp + 16 * min(8 * (pa + q) + g, nb - 1));
        L.w[2 * q + 1] = *(const uint4 *)(rp + 16 * min(8 * (pa + q) + 4 + g, nb - 1));
      }
      L.hist = 0;
    } else {
      const uint32_t *rp = s1 ? a.w1 + r * wpr1 : a.w2 + r * wpr2;
      const int wpr = s1 ? wpr1 : wpr2;
#pragma unroll
      for (int q = 0; q < PPW; ++q) L.sc[q] = *(const uint16_t *)(sp + min(8 * (pa + q) + 2 * g, nb - 2));
#pragma unroll
      for (int q = 0; q < PPW; ++q) L.w[q] = *(const uint4 *)(rp + min(16 * (pa + q) + 4 * g, wpr - 4));
      L.hist = rp[min(max(16 * pa - 1, 0), wpr - 1)];
    }
    return L;
  };
  // A-scale pair of piece p (blocks past the row: 2^0, meeting zero
  // activations; the codes there are the row's own, finite)
  auto a_scale = [&](uint32_t sc, int nb, int p) -> uint32_t {
    if constexpr (MX)
      return (8 * p + g < nb ? sc & 0xFFu : 0x7Fu) | (8 * p + 4 + g < nb ? sc & 0xFF00u : 0x7F00u);
    else
      return 8 * p + 2 * g < nb ? sc : 0x7F7Fu;
  };

  DecA D2[T2][PPW];
  uint32_t sc2[T2][PPW];
  uint32_t tag;
  bool poisoned;
  if (up_role) {
    // ---- gate/up tiles, AT loads ahead. Tile t: gate rows (t even) or up
    // rows (t odd) of pair p0 + t/2 = (active expert ai0, 16-row group j0)
    // advanced by t/2; positions past the workgroup's tiles repeat its last.
    __builtin_amdgcn_s_setprio(2);
    const int ai0 = p0 / pr_per, j0 = p0 - ai0 * pr_per;
    size_t row[T1];
#pragma unroll
    for (int t = 0; t < T1; ++t) {
      const int tc = n1 > 0 ? min(t, n1 - 1) : 0;
      int j = j0 + (tc >> 1), ai = ai0;
      if (j >= pr_per) {   // t/2 < kMaxPairs <= pr_per: one wrap at most
        j -= pr_per;
        ++ai;
      }
      row[t] = n1 > 0 ? (size_t)__builtin_amdgcn_readlane(act_e, ai) * 2 * I + (tc & 1 ? I : 0) + 16 * j : 0;
    }
    TileLd<PPW, MX> R[AT];
#pragma unroll
    for (int t = 0; t < AT; ++t) R[t] = load_tile(row[t], true);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (AT >= T1 && lane == 0) __hip_atomic_fetch_add(&S.up_issued, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    TOK_MARK(3);
    // split this wave's blocks of x into LDS (blocks past K, up to the last
    // piece, get zero codes); the wave reads them back itself
#pragma unroll
    for (int ps = 0; ps < kXPass; ++ps) {
      const int xb = 8 * pa + 16 * ps + (lane >> 2), xj = lane & 3;
      float f[8];
      const uint32_t wv[8] = {xr[ps][0].x, xr[ps][0].y, xr[ps][0].z, xr[ps][0].w,
                              xr[ps][1].x, xr[ps][1].y, xr[ps][1].z, xr[ps][1].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t bits = a.x_bf16 ? (wv[i >> 1] >> (16 * (i & 1))) << 16 : wv[i];
        f[i] = xb < nb1 ? __uint_as_float(bits) : 0.0f;
      }
      split_block8<MX>(f, xb, xj, S.xq, S.xs, ps1, xb < 8 * (pa + c));
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    TOK_MARK(2);
    // this wave's x operands (B), read once
    BOp bx[PPW][2];
#pragma unroll
    for (int q = 0; q < PPW; ++q)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        bx[q][hh] = read_b(S.xq, S.xs, ps1, i16 & 1, min(2 * (pa + q) + hh, ps1 - 1), g);
#pragma unroll
    for (int t = 0; t < T1; ++t) {
      const TileLd<PPW, MX> cur = R[t % AT];
      if (t + AT < T1) {
        R[t % AT] = load_tile(row[t + AT], true);
        if (t + AT == T1 - 1 && lane == 0)
          __hip_atomic_fetch_add(&S.up_issued, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      if (t < n1 && c > 0) {
        uint32_t carry = pa == 0 ? 0u : cur.hist;
        v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < PPW; ++q) {
          if (q < c) {
            const uint32_t rot = MX ? 0u : (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)cur.w[q].w);
            const DecA d = piece_a<PPW, MX>(cur, q, g == 0 ? carry : rot);
            carry = rot;
            if constexpr (E5)
              acc = mma2_e5m3(d, bx[q][0], bx[q][1], a_scale(cur.sc[q], nb1, pa + q), acc, S.e5t);
            else
              acc = mma2(d, bx[q][0], bx[q][1], a_scale(cur.sc[q], nb1, pa + q), acc);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = pair_sum(acc[r]);
          if (i16 == 0) S.red1[t][rw][4 * g + r] = v;
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
    TOK_MARK(4);
    // the call tag (set by the down waves at entry)
    while (__hip_atomic_load(&S.x_ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < 1)
      __builtin_amdgcn_s_sleep(1);
    asm volatile("" ::: "memory");
    tag = S.tag;
    poisoned = S.poisoned != 0;
    // the last gate/up wave to finish computes SwiGLU for the workgroup:
    // thread q < 16 np, row q % 16 of pair q / 16 (its partial sums are
    // stored before it counts: LDS accesses of a wave complete in order)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    int arrived = 0;
    if (lane == 0) arrived = __hip_atomic_fetch_add(&S.up_done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    arrived = __builtin_amdgcn_readfirstlane(arrived);
    if (arrived == NR - 1 && !poisoned) {
      asm volatile("" ::: "memory");
      for (int qq = lane; qq < 16 * np; qq += 64) {
        const int uo = qq >> 4, r = qq & 15;
        float gs = 0.0f, us = 0.0f;
#pragma unroll
        for (int v = 0; v < NR; ++v) {
          if (v * PPW < J1) {
            gs += S.red1[2 * uo][v][r];
            us += S.red1[2 * uo + 1][v][r];
          }
        }
        const float silu = gs / (1.0f + expf(-gs));
        const uint32_t hb = f32_to_bf16_rne(silu * us);
        const int jj = j0 + uo, ai = jj >= pr_per ? ai0 + 1 : ai0, j = jj >= pr_per ? jj - pr_per : jj;
        const int col = 16 * j + r;
        // two values per tagged word: the even row's lane stores
        const uint32_t hb_next = __shfl_down(hb, 1, 64);
        if ((r & 1) == 0)
          st_dc64(a.hx + ((size_t)ai * I + col) / 2, ((uint64_t)tag << 32) | (hb | (hb_next << 16)));
        for (int s = 0; s < a.k; ++s)
          if (__builtin_amdgcn_readlane((int)valid, s) && __builtin_amdgcn_readlane(rank, s) == ai)
            a.h[(size_t)s * I + col] = (uint16_t)hb;
      }
    }
    TOK_MARK(5);
  } else {
    tag = epoch + 1u;   // 1 .. 2^32 - 1 (the counter skips 2^32 - 1)
    poisoned = err0 != 0;
    if (rtid == 0) {
      S.tag = tag;
      S.poisoned = err0;
    }
    // the tag is in LDS before the flag goes up
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (rtid == 0) __hip_atomic_store(&S.x_ready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    // clear this workgroup's tiles of y, tag them once the zeros are at the
    // coherence point, and count the workgroup in; the last workgroup to
    // count in advances the call counter (every workgroup read it first)
    if (rw == 0) {
      for (int rt = w; rt < rt_per; rt += G)
        if (lane < 16) __hip_atomic_store(&a.y[16 * rt + lane], err0 ? __builtin_nanf("") : 0.0f,
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
      uint32_t seen_old = 0;
      if (lane == 0) {
        for (int rt = w; rt < rt_per; rt += G) st_dc32(a.yz + rt, tag);
        seen_old = __hip_atomic_fetch_add(&a.sync[32], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (seen_old == (uint32_t)(G - 1)) {
          st_dc32(&a.sync[32], 0u);
          st_dc32(&a.sync[0], epoch + 1u == 0xFFFFFFFFu ? 0u : epoch + 1u);
        }
      }
    }
    TOK_MARK_T(7, 256);
    // down tile t: 16-row group rt[t] of active expert dai[t] (from d0,
    // advanced by t; positions past the workgroup's tiles repeat its last)
    int dai[T2], drt[T2];
    {
      const int ai0 = d0 / rt_per;
      int ai = ai0, rt = d0 - ai0 * rt_per;
#pragma unroll
      for (int t = 0; t < T2; ++t) {
        if (t > 0 && t < nd) {
          if (++rt == rt_per) {
            rt = 0;
            ++ai;
          }
        }
        dai[t] = ai;
        drt[t] = rt;
      }
    }
    // ---- down tiles: loads once every gate/up load is issued, then the decode
    while (__hip_atomic_load(&S.up_issued, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < NR)
      __builtin_amdgcn_s_sleep(2);
    asm volatile("" ::: "memory");
    TileLd<PPW, MX> L2[T2];
#pragma unroll
    for (int t = 0; t < T2; ++t)
      L2[t] = load_tile(nd > 0 ? (size_t)__builtin_amdgcn_readlane(act_e, dai[t]) * H + 16 * drt[t] : 0, false);
#pragma unroll
    for (int t = 0; t < T2; ++t) {
      if (!poisoned && t < nd && c > 0) {
        uint32_t carry = pa == 0 ? 0u : L2[t].hist;
#pragma unroll
        for (int q = 0; q < PPW; ++q) {
          if (q < c) {
            const uint32_t rot = MX ? 0u : (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)L2[t].w[q].w);
            D2[t][q] = piece_a<PPW, MX>(L2[t], q, g == 0 ? carry : rot);
            carry = rot;
            sc2[t][q] = a_scale(L2[t].sc[q], nb2, pa + q);
            pin(D2[t][q]);
          }
        }
      }
    }
    TOK_MARK_T(6, 256);
    // ---- this wave's part of h (the K range of its pieces) for each expert
    // of the workgroup's down tiles, polled as tagged words and split into
    // LDS columns (2 ex, 2 ex + 1): blocks 8 pa .. 8 (pa + c) - 1, four lanes
    // each, 16 per pass. No other wave reads them, so no barrier.
    const int a_lo = dai[0];
    const int n_ex = nd > 0 ? dai[T2 - 1] - a_lo + 1 : 0;
    constexpr int kHPass = (8 * PPW + 15) / 16;
    // the tags of this workgroup's tiles of y (stored at entry by the
    // workgroups that cleared them): loaded here, checked once h is in
    int rt_l = drt[0];
#pragma unroll
    for (int t = 1; t < T2; ++t)
      if (lane == t) rt_l = drt[t];
    uint32_t yzv = lane < nd ? ld_dc32(a.yz + rt_l) : tag;
    for (int ex = 0; ex < n_ex && !poisoned && c > 0; ++ex) {
      const int ai = a_lo + ex;
      uint64_t v[kHPass][4];
      for (unsigned it = 0;; ++it) {
        bool ok = true;
#pragma unroll
        for (int ps = 0; ps < kHPass; ++ps) {
          const int hb = 8 * pa + 16 * ps + (lane >> 2), hj = lane & 3;
          const bool live = hb < min(nb2, 8 * (pa + c));
          const uint64_t *hsrc = a.hx + ((size_t)ai * I + 32 * (live ? hb : 8 * pa) + 8 * hj) / 2;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v[ps][q] = ld_dc64(hsrc + q);
            ok = ok && (!live || (uint32_t)(v[ps][q] >> 32) == tag);
          }
        }
        if (__ballot(!ok) == 0ull) break;
        if (it >= kPolls) {
          if (lane == 0) set_error(a.status);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
#pragma unroll
      for (int ps = 0; ps < kHPass; ++ps) {
        const int hb = 8 * pa + 16 * ps + (lane >> 2), hj = lane & 3;
        float f[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          f[i] = hb < nb2 ? __uint_as_float(((uint32_t)(v[ps][i >> 1] >> (16 * (i & 1))) & 0xFFFFu) << 16) : 0.0f;
        split_block8<MX>(f, hb, hj, S.hq + (size_t)(2 * ex) * ps2 * 128, S.hs + (size_t)(2 * ex) * ps2 * 4, ps2,
                         hb < 8 * (pa + c));
      }
    }
    for (unsigned it = 0; __ballot(yzv != tag) != 0ull; ++it) {
      if (it >= kPolls) {
        if (lane == 0) set_error(a.status);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
      if (lane < nd) yzv = ld_dc32(a.yz + rt_l);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    TOK_MARK_T(8, 256);
    // ---- down projection: matrix-core steps on the pre-decoded pieces, one
    // accumulator chain per tile, a piece's h operands read once per expert
    if (!poisoned && nd > 0 && c > 0) {
      v4f acc[T2];
#pragma unroll
      for (int t = 0; t < T2; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < PPW; ++q) {
        if (q < c) {
          const int st = 2 * (pa + q);
          const BOp b00 = read_b(S.hq, S.hs, ps2, i16 & 1, st, g);
          const BOp b01 = read_b(S.hq, S.hs, ps2, i16 & 1, st + 1, g);
          BOp b10 = b00, b11 = b01;
          if (n_ex > 1) {
            b10 = read_b(S.hq, S.hs, ps2, 2 + (i16 & 1), st, g);
            b11 = read_b(S.hq, S.hs, ps2, 2 + (i16 & 1), st + 1, g);
          }
#pragma unroll
          for (int t = 0; t < T2; ++t) {
            if (t < nd) {
              if constexpr (E5) {
                if (dai[t] == a_lo)
                  acc[t] = mma2_e5m3(D2[t][q], b00, b01, sc2[t][q], acc[t], S.e5t);
                else
                  acc[t] = mma2_e5m3(D2[t][q], b10, b11, sc2[t][q], acc[t], S.e5t);
              } else {
                if (dai[t] == a_lo)
                  acc[t] = mma2(D2[t][q], b00, b01, sc2[t][q], acc[t]);
                else
                  acc[t] = mma2(D2[t][q], b10, b11, sc2[t][q], acc[t]);
              }
            }
          }
        }
      }
#pragma unroll
      for (int t = 0; t < T2; ++t) {
        if (t < nd) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float v = pair_sum(acc[t][r]);
            if (i16 == 0) S.red2[t][rw][4 * g + r] = v;
          }
        }
      }
    }
    TOK_MARK_T(9, 256);
    // ---- the last down wave to finish adds the gate-weighted rows into y
    // (every down wave saw the tiles cleared in this call; the partial sums
    // of the other waves are in LDS: they were stored before those waves
    // counted)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    int arrived = 0;
    if (lane == 0) arrived = __hip_atomic_fetch_add(&S.down_done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    arrived = __builtin_amdgcn_readfirstlane(arrived);
    if (arrived == NR - 1 && !poisoned) {
      asm volatile("" ::: "memory");
      for (int q = lane; q < 16 * nd; q += 64) {
        const int t = q >> 4, r = q & 15;
        float v = 0.0f;
#pragma unroll
        for (int wv = 0; wv < NR; ++wv)
          if (wv * PPW < J2) v += S.red2[t][wv][r];
        int rt = drt[0];
        float gw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(act_g), dai[0]));
#pragma unroll
        for (int tt = 1; tt < T2; ++tt)
          if (t == tt) {
            rt = drt[tt];
            gw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(act_g), dai[tt]));
          }
        __hip_atomic_fetch_add(a.y + 16 * rt + r, gw * v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    TOK_MARK_T(10, 256);
  }

  // ---- once per call: skipped-slot count, h rows of dead slots
  if (w == 0) {
    if (tid == 0) __hip_atomic_store(&a.status[0], n_skipped, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int s = 0; s < a.k; ++s)
      if (!__builtin_amdgcn_readlane((int)valid, s))
        for (int cc = tid; cc < I; cc += 64 * NW) a.h[(size_t)s * I + cc] = 0;
  }
  TOK_MARK_T(11, 256);
#ifdef TQ_TRACE
  __syncthreads();
  if (tid < 12 && a.trace) a.trace[blockIdx.x * 16 + tid] = S.trace[tid];
#endif
}

// Kernel instances: (pieces per wave, gate/up tiles, down tiles, format).
struct Inst {
  int ppw, t1, t2;
  bool mx, e5m3, routed;
  const void *fn;
};
#ifndef TQ_TOK_AT
#define TQ_TOK_AT 2
#endif
#ifndef TQ_TOK_AT_MX
#define TQ_TOK_AT_MX 2
#endif
#define TQ_TOK_INST(PPW, T1, T2) \
  {PPW, T1, T2, false, false, false, (const void *)k_tok<PPW, T1, T2, TQ_TOK_AT, false, false>}
#define TQ_TOK_INST_MX(PPW, T1, T2) \
  {PPW, T1, T2, true, false, false, (const void *)k_tok<PPW, T1, T2, TQ_TOK_AT_MX, true, false>}
#define TQ_TOK_INST_E5(PPW, T1, T2) \
  {PPW, T1, T2, false, true, false, (const void *)k_tok<PPW, T1, T2, TQ_TOK_AT, false, true>}
#define TQ_TOK_INST_RT(PPW, T1, T2) \
  {PPW, T1, T2, false, false, true, (const void *)k_tok<PPW, T1, T2, TQ_TOK_AT, false, false, true>}
const Inst kInsts[] = {
    TQ_TOK_INST(3, 6, 3), TQ_TOK_INST(4, 6, 3), TQ_TOK_INST(3, 6, 4), TQ_TOK_INST(4, 6, 4),
    TQ_TOK_INST_RT(3, 6, 3), TQ_TOK_INST_RT(4, 6, 3), TQ_TOK_INST_RT(3, 6, 4), TQ_TOK_INST_RT(4, 6, 4),
    TQ_TOK_INST_MX(3, 6, 3), TQ_TOK_INST_MX(4, 6, 3), TQ_TOK_INST_MX(3, 6, 4), TQ_TOK_INST_MX(4, 6, 4),
    TQ_TOK_INST_E5(3, 6, 3), TQ_TOK_INST_E5(4, 6, 3), TQ_TOK_INST_E5(3, 6, 4), TQ_TOK_INST_E5(4, 6, 4),
};

// ---------------------------------------------------------------- single-token routed GEMV
//
// One token through one routed matrix stack, each slot's output kept
// (trellis_moe_gemv with T = 1, shared x and no gate weights; HEPH abstract,
// fused serving mode). A unit is one 16-row tile of one active expert;
// workgroup w takes units [w NU / G, (w + 1) NU / G), at most T1 of them,
// streamed through a register ring two tiles deep. Its four waves split
// every tile along K (wave v: pieces [v PPW, (v+1) PPW), x split by the wave
// for its own range, as in the layer kernel), meet in LDS, and the tile's 16
// rows go to every slot routed to its expert. A tile's rows are final in one
// workgroup, so nothing waits on another workgroup. Slots that route to no
// expert get zeros from the tiles of active expert 0, which cover every row
// once (or from workgroup 0 when no slot is active). A set sticky error word
// makes the call write NaN to y and nothing else. MX: expanded MXFP4 codes;
// E5: trellis streams under E5M3 scales (each matrix-core step once per
// power-of-two term of its scale), as in the layer kernel.
struct GemvArgs {
  const uint32_t *w; const uint8_t *s;   // [E][rows][K / 16] symbols, [E][rows][K / 32] scales
  int E, rows, K, k;
  const int32_t *ids;
  const void *x; int x_bf16;
  float *y;                              // [k][rows]
  int *status;
  int G;
};

template <int PPW, int T1, bool MX, bool E5>
__global__ void __launch_bounds__(256) k_tok_gemv(GemvArgs a) {
  static_assert(!(MX && E5), "E5M3 scales are served on trellis streams");
  constexpr int NR = 4, AT = T1 < 2 ? T1 : 2;
  __shared__ uint8_t xq[2 * 2 * kMaxJ * 128], xs[2 * 2 * kMaxJ * 4];
  __shared__ float red[T1][NR][16];
  __shared__ uint32_t e5t[E5 ? 256 : 1];
  const int tid = threadIdx.x, lane = tid & 63, rw = tid >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int w = blockIdx.x, G = a.G;
  const int nb = a.K >> 5, J = (nb + 7) >> 3, wpr = a.K >> 4, ps = 2 * J;
  const int rpe = a.rows >> 4;                 // tiles per expert
  const int src = ((lane - 16) & 63) << 2;     // lane-group g-1, same row (ds_bpermute address)
  const int pa = min(rw * PPW, J), c = min(J - pa, PPW);

  if constexpr (E5) e5t[tid] = e5m3_terms((uint32_t)tid);   // 256 threads
  const int sl = lane & 31, slc = sl < a.k ? sl : 0;
  const int idv = a.ids[slc];
  const int err = __hip_atomic_load(&a.status[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  constexpr int kXPass = (8 * PPW + 15) / 16;
  uint4 xr[kXPass][2];
#pragma unroll
  for (int p = 0; p < kXPass; ++p) {
    const int xb = 8 * pa + 16 * p + (lane >> 2), xj = lane & 3;
    const char *xp = (const char *)a.x + (size_t)(32 * (xb < nb ? xb : 0) + 8 * xj) * (a.x_bf16 ? 2 : 4);
    xr[p][0] = *(const uint4 *)xp;
    xr[p][1] = *(const uint4 *)(a.x_bf16 ? xp : xp + 16);
  }
  const TokRoute route = tok_route(lane, a.k, a.E, idv, 0.0f, false);
  if (err) {
    const size_t n = (size_t)a.k * a.rows;
    for (size_t i = (size_t)w * 256 + tid; i < n; i += (size_t)G * 256) a.y[i] = __builtin_nanf("");
    return;
  }
  const uint32_t NU = (uint32_t)route.n_act * rpe;
  const int u0 = (int)((uint32_t)w * NU / (uint32_t)G), nu = (int)((uint32_t)(w + 1) * NU / (uint32_t)G) - u0;
  // tile t: unit u0 + t (positions past the workgroup's units repeat its last)
  int tai[T1], trt[T1];
  {
    int ai = u0 / max(rpe, 1), rt = u0 - ai * rpe;
#pragma unroll
    for (int t = 0; t < T1; ++t) {
      if (t > 0 && t < nu && ++rt == rpe) {
        rt = 0;
        ++ai;
      }
      tai[t] = ai;
      trt[t] = rt;
    }
  }
  auto load_tile = [&](int t) -> TileLd<PPW, MX> {
    TileLd<PPW, MX> L;
    const size_t r = (nu > 0 ? (size_t)__builtin_amdgcn_readlane(route.act_e, tai[t]) * a.rows + 16 * trt[t] : 0) + i16;
    const uint8_t *sp = a.s + r * nb;
    if constexpr (MX) {
      // 16 bytes per block; the row's last block stands in for blocks past it
      const uint8_t *rp = (const uint8_t *)a.w + r * (size_t)nb * 16;
#pragma unroll
      for (int q = 0; q < PPW; ++q)
        L.sc[q] = (uint32_t)sp[min(8 * (pa + q) + g, nb - 1)] | (uint32_t)sp[min(8 * (pa + q) + 4 + g, nb - 1)] << 8;
#pragma unroll
      for (int q = 0; q < PPW; ++q) {
        L.w[2 * q] = *(const uint4 *)(rp + 16 * min(8 * (pa + q) + g, nb - 1));
        L.w[2 * q + 1] = *(const uint4 *)(rp + 16 * min(8 * (pa + q) + 4 + g, nb - 1));
      }
      L.hist = 0;
    } else {
      const uint32_t *rp = a.w + r * wpr;
#pragma unroll
      for (int q = 0; q < PPW; ++q) L.sc[q] = *(const uint16_t *)(sp + min(8 * (pa + q) + 2 * g, nb - 2));
#pragma unroll
      for (int q = 0; q < PPW; ++q) L.w[q] = *(const uint4 *)(rp + min(16 * (pa + q) + 4 * g, wpr - 4));
      L.hist = rp[min(max(16 * pa - 1, 0), wpr - 1)];
    }
    return L;
  };
  // A-scale pair of piece p (blocks past the row: 2^0 or E5M3 1.875,
  // meeting zero activations; the codes there are the row's own, finite)
  auto a_scale = [&](uint32_t sc, int p) -> uint32_t {
    if constexpr (MX)
      return (8 * p + g < nb ? sc & 0xFFu : 0x7Fu) | (8 * p + 4 + g < nb ? sc & 0xFF00u : 0x7F00u);
    else
      return 8 * p + 2 * g < nb ? sc : 0x7F7Fu;
  };
  TileLd<PPW, MX> R[AT > 0 ? AT : 1];
#pragma unroll
  for (int t = 0; t < AT; ++t) R[t] = load_tile(t);
  // this wave's blocks of x, split into LDS (blocks past K, up to the last
  // piece, get zero codes); the wave reads them back itself
#pragma unroll
  for (int p = 0; p < kXPass; ++p) {
    const int xb = 8 * pa + 16 * p + (lane >> 2), xj = lane & 3;
    float f[8];
    const uint32_t wv[8] = {xr[p][0].x, xr[p][0].y, xr[p][0].z, xr[p][0].w,
                            xr[p][1].x, xr[p][1].y, xr[p][1].z, xr[p][1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t bits = a.x_bf16 ? (wv[i >> 1] >> (16 * (i & 1))) << 16 : wv[i];
      f[i] = xb < nb ? __uint_as_float(bits) : 0.0f;
    }
    split_block8<MX>(f, xb, xj, xq, xs, ps, xb < 8 * (pa + c));
  }
  if constexpr (E5) __syncthreads();   // the term table is complete
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  BOp bx[PPW][2];
#pragma unroll
  for (int q = 0; q < PPW; ++q)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) bx[q][hh] = read_b(xq, xs, ps, i16 & 1, min(2 * (pa + q) + hh, ps - 1), g);
#pragma unroll
  for (int t = 0; t < T1; ++t) {
    const TileLd<PPW, MX> cur = R[t % AT];
    if (t + AT < T1) R[t % AT] = load_tile(t + AT);
    if (t < nu && c > 0) {
      uint32_t carry = pa == 0 ? 0u : cur.hist;
      v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < PPW; ++q) {
        if (q < c) {
          const uint32_t rot = MX ? 0u : (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)cur.w[q].w);
          const DecA d = piece_a<PPW, MX>(cur, q, g == 0 ? carry : rot);
          carry = rot;
          if constexpr (E5)
            acc = mma2_e5m3(d, bx[q][0], bx[q][1], a_scale(cur.sc[q], pa + q), acc, e5t);
          else
            acc = mma2(d, bx[q][0], bx[q][1], a_scale(cur.sc[q], pa + q), acc);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = pair_sum(acc[r]);
        if (i16 == 0) red[t][rw][4 * g + r] = v;
      }
    }
  }
  __syncthreads();
  // row r of tile t to every slot of its expert (zeros to the slots that
  // route nowhere, from active expert 0's tiles)
  for (int q = tid; q < 16 * nu; q += 256) {
    const int t = q >> 4, r = q & 15;
    float v = 0.0f;
#pragma unroll
    for (int v4 = 0; v4 < NR; ++v4)
      if (v4 * PPW < J) v += red[t][v4][r];
    int ai = tai[0], rt = trt[0];
#pragma unroll
    for (int tt = 1; tt < T1; ++tt)
      if (t == tt) {
        ai = tai[tt];
        rt = trt[tt];
      }
    for (int sidx = 0; sidx < a.k; ++sidx) {
      const bool vs = __builtin_amdgcn_readlane((int)route.valid, sidx) != 0;
      if (vs ? __builtin_amdgcn_readlane(route.rank, sidx) == ai : ai == 0)
        a.y[(size_t)sidx * a.rows + 16 * rt + r] = vs ? v : 0.0f;
    }
  }
  if (w == 0) {
    if (tid == 0) __hip_atomic_store(&a.status[0], route.n_skipped, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (route.n_act == 0)
      for (int i = tid; i < a.k * a.rows; i += 256) a.y[i] = 0.0f;
  }
}

// Worst-case work of a workgroup (every slot a distinct expert).
struct Plan {
  int nw, ppw, t1, t2;
  bool ok;
};
Plan plan(const TokCall &c, int cus) {
  Plan p{4, 0, 0, 0, false};   // four waves per role
  const int J1 = (c.H / 32 + 7) / 8, J2 = (c.I / 32 + 7) / 8;
  if (J1 > kMaxJ || J2 > kMaxJ) return p;
  p.ppw = std::max((J1 + p.nw - 1) / p.nw, (J2 + p.nw - 1) / p.nw);
  const int n_act = std::min(c.E, c.k);
  const int NP = n_act * (c.I / 16), ND = n_act * (c.H / 16);
  p.t1 = 2 * ((NP + cus - 1) / cus);
  p.t2 = (ND + cus - 1) / cus;
  // a workgroup's down tiles span at most two experts
  const bool span_ok = p.t2 <= c.H / 16 + 1;
  p.ok = p.t1 <= 2 * kMaxPairs && p.t2 <= kMaxDown && span_ok;
  return p;
}

const Inst *pick(const Plan &p, bool mx, bool e5m3, bool routed) {
  const Inst *best = nullptr;
  for (const Inst &i : kInsts)
    if (i.mx == mx && i.e5m3 == e5m3 && i.routed == routed && i.ppw >= p.ppw && i.t1 >= p.t1 && i.t2 >= p.t2 &&
        (!best || i.ppw * (i.t1 + i.t2) < best->ppw * (best->t1 + best->t2)))
      best = &i;
  return best;
}

}  // namespace

TokRegion tok_region(int n_exp, int hidden, int inter) {
  auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
  TokRegion r;
  r.sync = 0;
  r.hx = 256;
  r.yz = al(r.hx + (size_t)std::min(n_exp, kMaxSlots) * inter * 4);
  r.total = al(r.yz + (size_t)(hidden / 16) * 4);
  return r;
}

bool tok_supported(const TokCall &c, int cus) {
  if (c.k < 1 || c.k > kMaxSlots || c.H % 64 || c.I % 64 || c.H < 64 || c.I < 64) return false;
  if (((uintptr_t)c.w1 & 15) || ((uintptr_t)c.w2 & 15) || ((uintptr_t)c.x & 15)) return false;
  if (((uintptr_t)c.s1 & 15) || ((uintptr_t)c.s2 & 15)) return false;
  const Plan p = plan(c, cus);
  if (c.w_router && (c.mx || c.e5m3 || c.E > kRtMaxE || c.H > kRtMaxH || c.k > c.E || !c.ids_out || !c.gw_out ||
                    ((uintptr_t)c.w_router & 15)))
    return false;
  return p.ok && !(c.mx && c.e5m3) && pick(p, c.mx, c.e5m3, c.w_router != nullptr) != nullptr;
}

int tok_launch(const TokCall &c, int cus, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const Plan p = plan(c, cus);
  const Inst *inst = p.ok ? pick(p, c.mx, c.e5m3, c.w_router != nullptr) : nullptr;
  if (!inst) return TRELLIS_EINVAL;
  const TokRegion R = tok_region(c.E, c.H, c.I);
  char *base = c.ws + c.region_off;
  Args a;
  a.w1 = c.w1; a.s1 = c.s1; a.w2 = c.w2; a.s2 = c.s2;
  a.E = c.E; a.H = c.H; a.I = c.I; a.k = c.k;
  a.ids = c.ids; a.gate_w = c.gate_w;
  a.x = c.x; a.x_bf16 = c.x_bf16;
  a.h = c.h; a.y = c.y;
  a.status = (int *)c.ws;
  a.sync = (uint32_t *)(base + R.sync);
  a.hx = (uint64_t *)(base + R.hx);
  a.yz = (uint32_t *)(base + R.yz);
  a.G = cus;
  a.w_router = c.w_router; a.ids_out = c.ids_out; a.gw_out = c.gw_out;
#ifdef TQ_TRACE
  a.trace = g_tok_trace;
#endif
  // dynamic LDS (unused) bringing the workgroup above half a compute
  // unit's LDS, so that no unit holds two of them
  static size_t pad[sizeof(kInsts) / sizeof(kInsts[0])];
  const size_t ii = (size_t)(inst - kInsts);
  if (!pad[ii]) {
    hipFuncAttributes fa;
    if (hipFuncGetAttributes(&fa, inst->fn) != hipSuccess) return TRELLIS_EHIP;
    pad[ii] = std::max<size_t>(kCuLds / 2 + 1024 - std::min<size_t>(fa.sharedSizeBytes, kCuLds / 2), 1);
  }
  void *args[] = {&a};
  const hipError_t e = e0 || e1 ? hipExtLaunchKernel(inst->fn, dim3(cus), dim3(512), args, pad[ii], s, e0, e1, 0)
                               : hipLaunchKernel(inst->fn, dim3(cus), dim3(512), args, pad[ii], s);
  if (e != hipSuccess) return TRELLIS_EHIP;
  return hipGetLastError() == hipSuccess ? TRELLIS_OK : TRELLIS_EHIP;
}

// ---------------------------------------------------------------- single-token routed GEMV (host)

namespace {
struct GemvInst {
  int ppw, t1;
  bool mx, e5m3;
  const void *fn;
};
#define TQ_TOKV_INST(PPW, T1, MX, E5) {PPW, T1, MX, E5, (const void *)k_tok_gemv<PPW, T1, MX, E5>}
#define TQ_TOKV_FMT(MX, E5)                                                                             \
  TQ_TOKV_INST(1, 1, MX, E5), TQ_TOKV_INST(2, 1, MX, E5), TQ_TOKV_INST(3, 1, MX, E5), TQ_TOKV_INST(4, 1, MX, E5), \
      TQ_TOKV_INST(1, 8, MX, E5), TQ_TOKV_INST(2, 8, MX, E5), TQ_TOKV_INST(3, 8, MX, E5), TQ_TOKV_INST(4, 8, MX, E5)
const GemvInst kGemvInsts[] = {TQ_TOKV_FMT(false, false), TQ_TOKV_FMT(true, false), TQ_TOKV_FMT(false, true)};

// The instance and grid for the worst case (every slot a distinct expert).
const GemvInst *gemv_pick(const TokGemvCall &c, int cus, int *grid) {
  if (c.k < 1 || c.k > kMaxSlots || c.rows < 16 || c.rows % 16 || c.K < 64 || c.K % 64 || c.K > 32 * 8 * kMaxJ ||
      (c.mx && c.e5m3))
    return nullptr;
  if (((uintptr_t)c.w & 15) || ((uintptr_t)c.s & 15) || ((uintptr_t)c.x & 15)) return nullptr;
  const int J = (c.K / 32 + 7) / 8, ppw = (J + 3) / 4;
  const long nu = (long)std::min(c.E, c.k) * (c.rows / 16);
  const int G = (int)std::min<long>(nu, cus);
  const long t1 = (nu + G - 1) / G;
  for (const GemvInst &i : kGemvInsts)
    if (i.mx == c.mx && i.e5m3 == c.e5m3 && i.ppw == ppw && i.t1 >= t1) {
      *grid = G;
      return &i;
    }
  return nullptr;
}
}  // namespace

bool tok_gemv_supported(const TokGemvCall &c, int cus) {
  int grid = 0;
  return gemv_pick(c, cus, &grid) != nullptr;
}

int tok_gemv_launch(const TokGemvCall &c, int cus, hipStream_t s) {
  int grid = 0;
  const GemvInst *inst = gemv_pick(c, cus, &grid);
  if (!inst) return TRELLIS_EINVAL;
  GemvArgs a;
  a.w = c.w; a.s = c.s; a.E = c.E; a.rows = c.rows; a.K = c.K; a.k = c.k;
  a.ids = c.ids; a.x = c.x; a.x_bf16 = c.x_bf16; a.y = c.y; a.status = c.status; a.G = grid;
  void *args[] = {&a};
  if (hipLaunchKernel(inst->fn, dim3(grid), dim3(256), args, 0, s) != hipSuccess) return TRELLIS_EHIP;
  return hipGetLastError() == hipSuccess ? TRELLIS_OK : TRELLIS_EHIP;
}

}  // namespace tq

#ifdef TQ_TRACE
extern "C" void tq_tok_set_trace(void *p) { tq::g_tok_trace = (unsigned long long *)p; }
#endif

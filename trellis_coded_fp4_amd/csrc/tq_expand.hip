// tq_expand.hip -- HEPH's expand serving mode on gfx950: trellis streams ->
// resident MXFP4 (packed E2M1 nibbles, even column in the low nibble, plus a
// byte copy of the UE8M0 exponents, which the HEPH abstract reuses as the
// exact block scales).
//
// Bandwidth-bound: 0.28125 B/weight read, 0.53125 B/weight written. Each
// thread streams 4 consecutive symbol words (64 weights) of one row: one
// 16-byte load, the preceding word for history (0 at a row start; from the
// neighbouring lane), 32 bytes of codes stored as two 16-byte non-temporal
// stores. A wave covers 1 KiB of symbols.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "tq_common.h"

namespace tq {

constexpr int kExpandThreads = 256;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct ExpandArgs {
  const uint32_t *syms;
  const uint8_t *scales;
  uint8_t *codes;
  uint8_t *scales_out;
  int64_t n_quads;       // groups of 4 words (rows * wpr / 4 when wpr % 4 == 0)
  int64_t n_words;
  int wpr;               // words per row
  int64_t n_scale_u4;    // scale bytes / 16
  int64_t n_scale_bytes;
};

// wpr % 4 == 0: every group of four words lies inside one row.
__global__ void __launch_bounds__(kExpandThreads) k_expand_quads(ExpandArgs a) {
  const int64_t q = (int64_t)blockIdx.x * kExpandThreads + threadIdx.x;
  if (q < a.n_quads) {
    const int64_t w0 = 4 * q;
    const uint4 g = *(const uint4 *)(a.syms + w0);
    // The preceding word is the last one of the lane below (DPP wave shift
    // right by one); lane 0 of a wave loads it.
    uint32_t prev = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)g.w, 0x138, 0xF, 0xF, false);
    if ((threadIdx.x & 63) == 0) prev = w0 ? a.syms[w0 - 1] : 0u;
    if (w0 % a.wpr == 0) prev = 0u;
    uint32_t o[8];
    natural_order(decode_word(g.x, prev), &o[0], &o[1]);
    natural_order(decode_word(g.y, g.x), &o[2], &o[3]);
    natural_order(decode_word(g.z, g.y), &o[4], &o[5]);
    natural_order(decode_word(g.w, g.z), &o[6], &o[7]);
    // written once and not read back here: non-temporal stores
    u32x4 *dst = (u32x4 *)(a.codes + 8 * w0);
    __builtin_nontemporal_store((u32x4){o[0], o[1], o[2], o[3]}, dst);
    __builtin_nontemporal_store((u32x4){o[4], o[5], o[6], o[7]}, dst + 1);
  }
  // scale copy: 16 bytes per thread over the same grid
  if (q < a.n_scale_u4) ((uint4 *)a.scales_out)[q] = ((const uint4 *)a.scales)[q];
  if (q == 0)
    for (int64_t b = a.n_scale_u4 * 16; b < a.n_scale_bytes; ++b) a.scales_out[b] = a.scales[b];
}

// General rows (wpr even, any multiple of 2): one thread per word.
__global__ void __launch_bounds__(kExpandThreads) k_expand_words(ExpandArgs a) {
  const int64_t w = (int64_t)blockIdx.x * kExpandThreads + threadIdx.x;
  if (w < a.n_words) {
    const uint32_t prev = (w % a.wpr) ? a.syms[w - 1] : 0u;
    uint32_t lo, hi;
    natural_order(decode_word(a.syms[w], prev), &lo, &hi);
    *(uint2 *)(a.codes + 8 * w) = make_uint2(lo, hi);
  }
  if (w < a.n_scale_u4) ((uint4 *)a.scales_out)[w] = ((const uint4 *)a.scales)[w];
  if (w == 0)
    for (int64_t b = a.n_scale_u4 * 16; b < a.n_scale_bytes; ++b) a.scales_out[b] = a.scales[b];
}

}  // namespace tq

using namespace tq;

extern "C" int trellis_decode_expand(hipStream_t stream, const trellis_mat_t *w, uint8_t *codes_out,
                                     uint8_t *scales_out) {
  if (!w || !w->syms || !w->scales || !codes_out || !scales_out) return TRELLIS_ENULL;
  if (w->n_mat < 1 || w->rows < 1 || w->cols < 32 || w->cols % 32) return TRELLIS_EINVAL;
  ExpandArgs a{};
  a.syms = w->syms;
  a.scales = w->scales;
  a.codes = codes_out;
  a.scales_out = scales_out;
  a.wpr = w->cols / 16;
  a.n_words = (int64_t)w->n_mat * w->rows * a.wpr;
  a.n_scale_bytes = (int64_t)w->n_mat * w->rows * (w->cols / 32);
  const bool aligned16 = ((uintptr_t)w->scales % 16 == 0) && ((uintptr_t)scales_out % 16 == 0);
  a.n_scale_u4 = aligned16 ? a.n_scale_bytes / 16 : 0;
  const bool quads = (a.wpr % 4 == 0) && ((uintptr_t)w->syms % 16 == 0) && ((uintptr_t)codes_out % 16 == 0);
  if (quads) {
    a.n_quads = a.n_words / 4;
    const int64_t n = std::max(a.n_quads, a.n_scale_u4);
    const int64_t blocks = (n + kExpandThreads - 1) / kExpandThreads;
    hipLaunchKernelGGL(k_expand_quads, dim3((unsigned)blocks), dim3(kExpandThreads), 0, stream, a);
  } else {
    if (((uintptr_t)codes_out % 8) || ((uintptr_t)w->syms % 4)) return TRELLIS_EINVAL;
    const int64_t n = std::max(a.n_words, a.n_scale_u4);
    const int64_t blocks = (n + kExpandThreads - 1) / kExpandThreads;
    hipLaunchKernelGGL(k_expand_words, dim3((unsigned)blocks), dim3(kExpandThreads), 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? TRELLIS_OK : TRELLIS_EHIP;
}

extern "C" int trellis_version(void) { return 100; }

extern "C" const char *trellis_strerror(int err) {
  switch (err) {
    case TRELLIS_OK: return "ok";
    case TRELLIS_EINVAL: return "invalid argument (shape, dtype, flag or count)";
    case TRELLIS_ENULL: return "a required pointer is NULL";
    case TRELLIS_EWORKSPACE: return "workspace too small or not 256-byte aligned";
    case TRELLIS_EHIP: return "HIP runtime error while enqueueing work";
    case TRELLIS_EDEVICE: return "current device is not gfx950 (MI355X)";
    default: return "unknown error";
  }
}

// tq_decode.h -- bit-sliced decoder for trellis-coded FP4 symbol words.
//
// Decoder being implemented (XOR-Trellis news article, aimodeling.com, bullet
// "XOR-Trellis FP4 decoder"): after shifting symbol b into the 16-bit state s,
// p0, p1, q0, q1 are the parities of s & 0x1089, 0x2112, 0x0A24, 0x2441;
// (p0, p1) select the palette and (q0, q1) permute branch -> entry:
//   P0=[-6,-1.5,0,2] P1=[-4,-1,0.5,3] P2=[-3,-0.5,1,4] P3=[-2,0,1.5,6]
// with palette = p0 | p1<<1, entry = b ^ (q0 | q1<<1), P3's zero = -0, and
// the result written as an OCP E2M1 code (sign bit 3, exponent bits 2..1,
// mantissa bit 0).
//
// Why it is a few word-wide XORs: written as E2M1 bits, the 16 palette
// entries are a bijection onto the 16 codes, and every code bit is affine
// over GF(2) in the state bits. With e0 = b_lo ^ q0 and e1 = b_hi ^ q1:
//   mantissa = ~(p0 ^ e1), exp_lo = ~(p1 ^ e1), exp_hi = ~(e0 ^ e1), sign = ~e1.
// So a whole 32-bit symbol word (16 weights) decodes with funnel shifts of
// the (current:previous) word pair and XORs, no per-weight work.
//
// Lane algebra.  In a symbol word each weight owns a 2-bit slot (bits 2i,
// 2i+1: "lo" and "hi" lane). Bit 2t+c of weight i's state is bit c of the
// symbol t places earlier. Shifting the stream left by a bits puts, in slot
// i, state bit a (even a) or a+2 (odd a) into the lo lane and state bit a+1
// (even a) or a-1 (odd a) into the hi lane. Reading the masks through that
// table:
//   e0 (lo lane): s0 s2 s5 s9 s11  -> shifts {0,2,3,7,9}
//   e1 (hi lane): s1 s0 s6 s10 s13 -> shifts {0,1,7,11,12}
//   p0 (lo lane): s0 s3 s7 s12     -> shifts {0,1,5,12}
//   p1 (hi lane): s1 s4 s8 s13     -> shifts {0,5,9,12}
// i.e. 8 distinct funnel shifts {1,2,3,5,7,9,11,12} per word. The previous
// word supplies the 12 history bits (6 symbols); it is 0 at a row start,
// which is the state reset.
//
// Output layout: the 16 codes of a word go into two nibble words, "even"
// (weights 0,2,..,14 in nibbles 0..7) and "odd" (weights 1,3,..,15). Both
// consumers handle that order: the matrix-core GEMV permutes activations to
// match; the expand kernel interleaves to natural order.
#pragma once
#include <stdint.h>

#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)
#define TQ_HD __host__ __device__ __forceinline__
#else
#define TQ_HD inline
#endif

namespace tq {

// Low word of ((cur:prev) << n), n in 1..31.
TQ_HD uint32_t shl_hist(uint32_t cur, uint32_t prev, int n) {
  return (cur << n) | (prev >> (32 - n));
}

struct nib2 {
  uint32_t even;  // nibble m = E2M1 code of weight 2m of the word
  uint32_t odd;   // nibble m = E2M1 code of weight 2m+1
};

// Three-input bitwise function with truth table IMM: output bit =
// IMM bit ((a << 2) | (b << 1) | c), the v_bitop3_b32 form (IMM for f is
// f(0xF0, 0xCC, 0xAA)). The host version serves the CPU check of this file.
template <uint32_t IMM>
TQ_HD uint32_t bop3(uint32_t a, uint32_t b, uint32_t c) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_bitop3_b32(a, b, c, IMM);
#else
  uint32_t r = 0;
  for (int i = 0; i < 8; ++i)
    if ((IMM >> i) & 1u) r |= ((i & 4) ? a : ~a) & ((i & 2) ? b : ~b) & ((i & 1) ? c : ~c);
  return r;
#endif
}
constexpr uint32_t kXor3 = 0x96;   // a ^ b ^ c
constexpr uint32_t kSel = 0xCA;    // (a & b) | (~a & c): bits of b where a is set, else c
constexpr uint32_t kXnorAnd = 0x87;   // ~(a ^ (b & c))

// Decode one symbol word `g` whose predecessor in the row is `prev`
// (0 at the row start). 8 funnel shifts and 15 three-input operations.
TQ_HD nib2 decode_word(uint32_t g, uint32_t prev) {
  const uint32_t LO = 0x55555555u, M33 = 0x33333333u;
  const uint32_t x1 = shl_hist(g, prev, 1), x2 = shl_hist(g, prev, 2), x3 = shl_hist(g, prev, 3);
  const uint32_t x5 = shl_hist(g, prev, 5), x7 = shl_hist(g, prev, 7), x9 = shl_hist(g, prev, 9);
  const uint32_t x11 = shl_hist(g, prev, 11), x12 = shl_hist(g, prev, 12);
  // E: (e0, e1) in (lo, hi) lanes.  P: (p0, p1).
  const uint32_t e_lo = bop3<kXor3>(x2, x3, x9);
  const uint32_t e_hi = bop3<kXor3>(x1, x11, x12);
  const uint32_t E = bop3<kXor3>(g, x7, bop3<kSel>(LO, e_lo, e_hi));
  const uint32_t P = bop3<kXor3>(bop3<kXor3>(g, x5, x12), bop3<kSel>(LO, x1, x9), 0u);
  const uint32_t N = E >> 1;                    // e1 moved into the lo lane
  const uint32_t A = ~(P ^ bop3<kSel>(LO, N, E));   // (mantissa, exp_lo) = ~(P ^ (e1, e1))
  const uint32_t B = bop3<kXnorAnd>(E, N, LO);      // (exp_hi, sign) = ~(E ^ (e1, 0))
  nib2 r;
  r.even = bop3<kSel>(M33, A, B << 2);
  r.odd = bop3<kSel>(M33, A >> 2, B);
  return r;
}

// Nibbles 0..3 of v spread to the low nibble of bytes 0..3.
TQ_HD uint32_t spread_nibbles(uint32_t v) {
  v &= 0xFFFFu;
  v = (v | (v << 8)) & 0x00FF00FFu;
  return (v | (v << 4)) & 0x0F0F0F0Fu;
}

// Natural-order packed codes of a word: byte j = code(2j) | code(2j+1) << 4.
// lo covers weights 0..7, hi weights 8..15.
TQ_HD void natural_order(nib2 n, uint32_t *lo, uint32_t *hi) {
  *lo = spread_nibbles(n.even) | (spread_nibbles(n.odd) << 4);
  *hi = spread_nibbles(n.even >> 16) | (spread_nibbles(n.odd >> 16) << 4);
}

// Position inside a 32-weight block of the code held in nibble n (0..31) of
// the four decoded registers {even(word0), odd(word0), even(word1), odd(word1)}.
TQ_HD int nibble_position(int n) {
  const int r = n >> 3, m = n & 7;
  return 16 * (r >> 1) + 2 * m + (r & 1);
}

// ---- E5M3 block scales
//
// The XOR-Trellis article's paragraph on the grouping format puts E2M1
// elements under E5M3 block scales without giving the encoding. Reading
// taken: an unsigned 8-bit float laid out as the upper byte of an IEEE
// binary16 number without its sign: exponent E in bits 7..3 (bias 15),
// mantissa m in bits 2..0, subnormal at E = 0, infinity / NaN at E = 31.
//
// The matrix cores take UE8M0 (power-of-two) A scales only. A finite,
// nonzero E5M3 value is n units of 2^(max(E,1) - 18) with significand
// n = 8 + m (or m when subnormal), which has at most four binary digits;
// halving the largest term until there are four writes it as a sum of
// exactly four powers of two. e5m3_terms returns those four as UE8M0
// bytes (byte i of the result); a step issued once per term with that
// term as its A scale sums to the E5M3-scaled product exactly (each term's
// products are exact). Returns 0 for the zero scale (no UE8M0 sum is zero:
// the caller zeroes the A operand) and 0xFFFFFFFF (four NaN bytes) for
// E = 31.
TQ_HD uint32_t e5m3_terms(uint32_t s) {
  const int E = (int)((s >> 3) & 31u), m = (int)(s & 7u);
  if (E == 31) return 0xFFFFFFFFu;
  const int n = E ? 8 + m : m;
  if (n == 0) return 0u;
  const int unit = (E ? E : 1) - 18 + 127;   // UE8M0 byte of one unit
  int t[4], cnt = 0;
  for (int j = 3; j >= 0; --j)
    if ((n >> j) & 1) t[cnt++] = unit + j;
  while (cnt < 4) {   // halve the largest term into two
    int big = 0;
    for (int i = 1; i < cnt; ++i)
      if (t[i] > t[big]) big = i;
    t[big] -= 1;
    t[cnt++] = t[big];
  }
  return (uint32_t)t[0] | (uint32_t)t[1] << 8 | (uint32_t)t[2] << 16 | (uint32_t)t[3] << 24;
}

// ---- activation layout for the matrix cores (see tq_common.h for the operand layout)

// Byte offset, inside one 128-K chunk of a B column (128 bytes laid out as the
// four lanes' 32-byte operands), of canonical K index k (0..127).
TQ_HD int bchunk_offset(int k) {
  return k < 64 ? (k >> 4) * 32 + (k & 15) : ((k - 64) >> 4) * 32 + 16 + (k & 15);
}

// Canonical K (0..127) of weight `pos` (0..31) of block `beta` (0..3) of a
// chunk, given the decoder's nibble order (see nibble_position).
TQ_HD int canonical_k(int beta, int pos) {
  const int w = pos >> 4, q = pos & 15;
  const int n = 8 * (2 * w + (q & 1)) + (q >> 1);
  return 32 * beta + n;
}

// Which matrix-core step consumes a 32-weight block of a row, and as which of
// its four K-blocks. A lane of lane-group g loads 16 bytes = physical blocks
// 8j+2g and 8j+2g+1 of its row ("piece" j) and feeds them to steps 2j and
// 2j+1; so physical block b goes to step 2*(b/8) + b%2 as K-block (b%8)/2.
TQ_HD int block_step(int b) { return 2 * (b >> 3) + (b & 1); }
TQ_HD int block_beta(int b) { return (b & 7) >> 1; }

// Byte offset of weight `pos` of physical block `b` inside one activation
// column laid out as consecutive 128-byte step chunks.
TQ_HD int act_offset(int b, int pos) {
  return block_step(b) * 128 + bchunk_offset(canonical_k(block_beta(b), pos));
}

// Index of the UE8M0 byte of physical block `b` in a column's scale array.
TQ_HD int act_scale_index(int b) { return block_step(b) * 4 + block_beta(b); }

// Matrix-core steps for a row of nb blocks (pieces of 8 blocks, two steps each).
TQ_HD int steps_for_blocks(int nb) { return 2 * ((nb + 7) >> 3); }

}  // namespace tq

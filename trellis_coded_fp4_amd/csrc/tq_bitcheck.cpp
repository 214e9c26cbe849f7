// tq_bitcheck.cpp -- host build of the device decoder's integer arithmetic
// (tq_decode.h), exported for the CPU test suite so the bit-sliced decode and
// the activation layout can be checked against the oracle without a GPU.
// Not part of libtrellis; nothing in the product path calls it.
#include <stdint.h>

#include "tq_decode.h"

extern "C" void tq_bitcheck_decode_word(uint32_t g, uint32_t prev, uint32_t *even, uint32_t *odd) {
  const tq::nib2 n = tq::decode_word(g, prev);
  *even = n.even;
  *odd = n.odd;
}

extern "C" void tq_bitcheck_natural(uint32_t g, uint32_t prev, uint32_t *lo, uint32_t *hi) {
  tq::natural_order(tq::decode_word(g, prev), lo, hi);
}

extern "C" int tq_bitcheck_nibble_position(int n) { return tq::nibble_position(n); }
extern "C" int tq_bitcheck_canonical_k(int beta, int pos) { return tq::canonical_k(beta, pos); }
extern "C" int tq_bitcheck_bchunk_offset(int k) { return tq::bchunk_offset(k); }
extern "C" int tq_bitcheck_act_offset(int b, int pos) { return tq::act_offset(b, pos); }
extern "C" int tq_bitcheck_act_scale_index(int b) { return tq::act_scale_index(b); }
extern "C" uint32_t tq_bitcheck_e5m3_terms(uint32_t s) { return tq::e5m3_terms(s); }

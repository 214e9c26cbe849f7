/*
 * trellis_oracle.c -- CPU oracle for trellis-coded FP4 weights.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, plain, sequential
 * reference that the HIP library is checked against. Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it. It
 * shares no code, tables or headers with trellis_coded_fp4_amd/.
 *
 * What it computes, and where each step comes from:
 *
 *  - XOR-Trellis news article (aimodeling.com, English and Chinese pages),
 *    bullet "XOR-Trellis FP4 decoder": the four palettes P0..P3, the 16-bit
 *    sliding state, and the four masked parities 0x1089, 0x2112, 0x0A24,
 *    0x2441 giving p0, p1, q0, q1; (p0, p1) picks the palette and (q0, q1)
 *    permutes which branch maps to which palette entry.
 *  - HEPH abstract (ICLR 2027 submission page): every decoded weight is an
 *    E2M1 value scaled by the checkpoint block's UE8M0 exponent, i.e. a
 *    valid MXFP4 element; "expand" turns the streams into resident MXFP4.
 *  - "Tied Trit-Planes" paper (arXiv 2608.08910), section 2.1: MXFP4 is
 *    fp4-e2m1 codes with one e8m0 scale per 32 elements; its reference list
 *    names the OCP Microscaling Formats v1.0 spec for both encodings.
 *
 * Readings where the pages leave a step open (each one is listed, with its
 * reason, in the design notes that ship with the repository):
 *
 *  R1  2-bit branch symbols are packed 16 per uint32, little-endian (symbol
 *      j of a word sits in bits 2j..2j+1), rows contiguous, K-major.
 *  R2  State update s = ((s << 2) | b) & 0xFFFF, s = 0 at each row start;
 *      the parities are taken on the state after the new symbol is in.
 *  R3  Palette index = p0 | (p1 << 1); palette entry = b XOR (q0 | q1 << 1).
 *  R4  P3's "0" is negative zero (E2M1 code 0x8) and P0's "0" is +0
 *      (code 0x0): the only reading under which the four palettes are
 *      disjoint, as the article says they are.
 *  R5  E2M1 bit layout per OCP MX: sign bit 3, exponent bits 2..1 (bias 1),
 *      mantissa bit 0.  UE8M0 byte e scales by 2^(e-127); e = 255 is NaN.
 *  R6  Expand output: two codes per byte, the even column in the low nibble.
 *  R7  SwiGLU between gate_up and down: gate = the first I rows of the
 *      gate_up output, up = the last I rows, h = silu(gate) * up rounded to
 *      bf16 (round to nearest even).
 *  R14 E5M3 block scales (the XOR-Trellis article's grouping-format
 *      paragraph names them, nothing more): an unsigned 8-bit float, the
 *      upper byte of an IEEE binary16 number without its sign (bias 15,
 *      subnormals at E = 0, E = 31 infinite or NaN). See oracle_e5m3_scale.
 *
 * Numbers: GEMV sums are accumulated in fp64, in column order. Inputs
 * (bf16 or fp32) are passed in as doubles, which holds them exactly.
 *
 * Parity pins (tests/, not this file): palette table equality, E2M1 set
 * membership and uniform use over all states, closed forms for constant
 * streams, hand-derived golden vectors, GF(2)-affinity of the code map,
 * windowed == sequential decoding, exact rational GEMV, numpy float64
 * matmul on the dense decoded weights, and brute force for the Viterbi
 * search. R1, R3, R4, R6 and R7 have no pin outside the readings above.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- constants from the XOR-Trellis article, "XOR-Trellis FP4 decoder" ---- */

static const double PALETTE[4][4] = {
    {-6.0, -1.5, 0.0, 2.0},  /* P0 */
    {-4.0, -1.0, 0.5, 3.0},  /* P1 */
    {-3.0, -0.5, 1.0, 4.0},  /* P2 */
    {-2.0, -0.0, 1.5, 6.0},  /* P3; its zero is negative zero (reading R4) */
};

static const uint32_t MASK_P0 = 0x1089u;
static const uint32_t MASK_P1 = 0x2112u;
static const uint32_t MASK_Q0 = 0x0A24u;
static const uint32_t MASK_Q1 = 0x2441u;

/* Palette entry as stored (exposed so tests can compare it with the article). */
double oracle_palette_entry(int palette, int entry) {
    return PALETTE[palette & 3][entry & 3];
}

/* ---- E2M1 and UE8M0 per the OCP MX v1.0 spec (reading R5) ---- */

/* Value of a 4-bit E2M1 code from its fields. */
double oracle_e2m1_value(int code) {
    int sign = (code >> 3) & 1;
    int exponent = (code >> 1) & 3;
    int mantissa = code & 1;
    double mag;
    if (exponent == 0)
        mag = 0.5 * mantissa;                                  /* subnormal: 2^(1-bias) * m/2 */
    else
        mag = ldexp(1.0 + 0.5 * mantissa, exponent - 1);       /* 2^(e-bias) * (1 + m/2) */
    return sign ? -mag : mag;
}

/* E2M1 code of a value, matching sign bit and magnitude; -1 if none. */
int oracle_e2m1_code(double v) {
    for (int code = 0; code < 16; ++code) {
        double c = oracle_e2m1_value(code);
        if (c == v && signbit(c) == signbit(v)) return code;
    }
    return -1;
}

/* Scale factor of a UE8M0 byte. */
double oracle_ue8m0_scale(int e) {
    if (e == 255) return NAN;
    return ldexp(1.0, e - 127);
}

/* ---- E5M3 block scales (XOR-Trellis article, "So what", the paragraph on
 * the grouping format: E2M1 elements with E5M3 block scales) ----
 *
 * The article names the format only. Reading R14: an unsigned 8-bit float,
 * 5 exponent bits (bias 15) above 3 mantissa bits, laid out and valued like
 * the upper byte of an IEEE binary16 number without its sign: E = byte >> 3,
 * m = byte & 7; E = 0 is subnormal, m/8 * 2^-14; E in 1..30 is normal,
 * (1 + m/8) * 2^(E - 15); E = 31 is +infinity (m = 0) or NaN. */
double oracle_e5m3_scale(int byte) {
    const int E = (byte >> 3) & 31, m = byte & 7;
    if (E == 31) return m == 0 ? INFINITY : NAN;
    if (E == 0) return ldexp((double)m / 8.0, -14);
    return ldexp(1.0 + (double)m / 8.0, E - 15);
}

enum { SCALE_UE8M0 = 0, SCALE_E5M3 = 1 };

static double block_scale(int fmt, int byte) {
    return fmt == SCALE_E5M3 ? oracle_e5m3_scale(byte) : oracle_ue8m0_scale(byte);
}

/* ---- the decoder ---- */

static int masked_parity(uint32_t state, uint32_t mask) {
    uint32_t v = state & mask;
    int p = 0;
    while (v) {
        p ^= (int)(v & 1u);
        v >>= 1;
    }
    return p;
}

/* Symbol k of a row (reading R1). */
static int row_symbol(const uint32_t *row_words, int64_t k) {
    return (int)((row_words[k / 16] >> (2 * (k % 16))) & 3u);
}

/* Palette value for a state that already holds the current symbol in its
 * low two bits (reading R2).  Steps in the article's order: four masked
 * parities; (p0, p1) select the palette; (q0, q1) permute branch -> entry. */
double oracle_state_value(uint32_t state) {
    int b = (int)(state & 3u);
    int p0 = masked_parity(state, MASK_P0);
    int p1 = masked_parity(state, MASK_P1);
    int q0 = masked_parity(state, MASK_Q0);
    int q1 = masked_parity(state, MASK_Q1);
    int palette = p0 | (p1 << 1);          /* reading R3 */
    int entry = b ^ (q0 | (q1 << 1));      /* reading R3 */
    return PALETTE[palette][entry];
}

int oracle_state_code(uint32_t state) {
    return oracle_e2m1_code(oracle_state_value(state));
}

/* Sequential decode of `rows` rows of `cols` weights into one E2M1 code per
 * weight. Row r's symbols start at syms + r * words_per_row. */
void oracle_decode_codes(const uint32_t *syms, int64_t rows, int64_t cols,
                         int64_t words_per_row, uint8_t *codes) {
    for (int64_t r = 0; r < rows; ++r) {
        const uint32_t *w = syms + r * words_per_row;
        uint32_t s = 0;                                   /* reset per row (R2) */
        for (int64_t k = 0; k < cols; ++k) {
            s = ((s << 2) | (uint32_t)row_symbol(w, k)) & 0xFFFFu;
            codes[r * cols + k] = (uint8_t)oracle_state_code(s);
        }
    }
}

/* Windowed decode of one weight: rebuild the state from s = 0 over the last
 * (at most) eight symbols of the row, which fill all 16 state bits. */
int oracle_decode_window(const uint32_t *row_words, int64_t k) {
    int64_t first = k - 7 < 0 ? 0 : k - 7;
    uint32_t s = 0;
    for (int64_t j = first; j <= k; ++j)
        s = ((s << 2) | (uint32_t)row_symbol(row_words, j)) & 0xFFFFu;
    return oracle_state_code(s);
}

/* Dense decoded weights: w[r][k] = palette value * block scale (UE8M0:
 * 2^(e - 127); E5M3: reading R14). */
void oracle_decode_values_fmt(const uint32_t *syms, const uint8_t *scales,
                              int64_t rows, int64_t cols, int scale_fmt, double *w) {
    const int64_t wpr = cols / 16, spr = cols / 32;
    for (int64_t r = 0; r < rows; ++r) {
        const uint32_t *words = syms + r * wpr;
        uint32_t s = 0;
        for (int64_t k = 0; k < cols; ++k) {
            s = ((s << 2) | (uint32_t)row_symbol(words, k)) & 0xFFFFu;
            w[r * cols + k] = oracle_state_value(s) * block_scale(scale_fmt, scales[r * spr + k / 32]);
        }
    }
}

void oracle_decode_values(const uint32_t *syms, const uint8_t *scales,
                          int64_t rows, int64_t cols, double *w) {
    oracle_decode_values_fmt(syms, scales, rows, cols, SCALE_UE8M0, w);
}

/* Expand to resident MXFP4 (HEPH's second serving mode): packed E2M1 codes,
 * two per byte with the even column in the low nibble (R6), and the UE8M0
 * bytes copied unchanged.  n_mat matrices of rows x cols each. */
void oracle_expand(const uint32_t *syms, const uint8_t *scales, int64_t n_mat,
                   int64_t rows, int64_t cols, uint8_t *packed, uint8_t *scales_out) {
    const int64_t wpr = cols / 16;
    uint8_t *codes = (uint8_t *)malloc((size_t)cols);
    for (int64_t r = 0; r < n_mat * rows; ++r) {
        oracle_decode_codes(syms + r * wpr, 1, cols, wpr, codes);
        for (int64_t j = 0; j < cols / 2; ++j)
            packed[r * (cols / 2) + j] = (uint8_t)(codes[2 * j] | (codes[2 * j + 1] << 4));
    }
    free(codes);
    memcpy(scales_out, scales, (size_t)(n_mat * rows * (cols / 32)));
}

/* One row's dot product with x, decoding as it goes, in fp64:
 * y = sum_k w[k] x[k] and bound = sum_k |w[k]| |x[k]|. */
static void row_dot(const uint32_t *words, const uint8_t *row_scales, int64_t cols,
                    const double *x, double *y, double *bound, int scale_fmt) {
    uint32_t s = 0;
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < cols; ++k) {
        s = ((s << 2) | (uint32_t)row_symbol(words, k)) & 0xFFFFu;
        double w = oracle_state_value(s) * block_scale(scale_fmt, row_scales[k / 32]);
        acc += w * x[k];
        mag += fabs(w) * fabs(x[k]);
    }
    *y = acc;
    *bound = mag;
}

/* Plain GEMV of one matrix [rows][cols] with nx input vectors x[nx][cols]:
 * y[t][r], bound[t][r]. */
void oracle_gemv(const uint32_t *syms, const uint8_t *scales, int64_t rows, int64_t cols,
                 const double *x, int64_t nx, double *y, double *bound) {
    const int64_t wpr = cols / 16, spr = cols / 32;
    for (int64_t t = 0; t < nx; ++t)
        for (int64_t r = 0; r < rows; ++r)
            row_dot(syms + r * wpr, scales + r * spr, cols, x + t * cols,
                    &y[t * rows + r], &bound[t * rows + r], SCALE_UE8M0);
}

/* Routed (mixture-of-experts) GEMV over n_exp matrices [rows][cols].
 *
 * Slot (t, j) uses expert ids[t*k + j]; x is [T][cols] (x_per_slot = 0) or
 * [T][k][cols] (x_per_slot = 1).  Without gate weights (gate_w == NULL) the
 * output is per slot, y[T][k][rows]; with them it is combined per token,
 * y[T][rows] = sum_j gate_w[t][j] * (W_e x).  A negative id is an empty
 * slot (contributes zero); an id >= n_exp is skipped and counted. Returns the
 * number of skipped slots.  bound has the shape of y and holds
 * sum |gate_w| * sum_k |w| |x|. */
int64_t oracle_moe_gemv_fmt(const uint32_t *syms, const uint8_t *scales, int64_t n_exp,
                            int64_t rows, int64_t cols, int scale_fmt, const double *x, int x_per_slot,
                            const int32_t *ids, const double *gate_w, int64_t T, int64_t k,
                            double *y, double *bound) {
    const int64_t wpr = cols / 16, spr = cols / 32;
    int64_t skipped = 0;
    int64_t n_out = gate_w ? T * rows : T * k * rows;
    for (int64_t i = 0; i < n_out; ++i) y[i] = bound[i] = 0.0;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t j = 0; j < k; ++j) {
            int32_t e = ids[t * k + j];
            if (e < 0) continue;
            if (e >= n_exp) { ++skipped; continue; }
            const double *xv = x + (x_per_slot ? (t * k + j) : t) * cols;
            double *yo = gate_w ? y + t * rows : y + (t * k + j) * rows;
            double *bo = gate_w ? bound + t * rows : bound + (t * k + j) * rows;
            double g = gate_w ? gate_w[t * k + j] : 1.0;
            for (int64_t r = 0; r < rows; ++r) {
                double d, b;
                row_dot(syms + (e * rows + r) * wpr, scales + (e * rows + r) * spr, cols, xv, &d, &b,
                        scale_fmt);
                yo[r] += g * d;
                bo[r] += fabs(g) * b;
            }
        }
    }
    return skipped;
}

int64_t oracle_moe_gemv(const uint32_t *syms, const uint8_t *scales, int64_t n_exp,
                        int64_t rows, int64_t cols, const double *x, int x_per_slot,
                        const int32_t *ids, const double *gate_w, int64_t T, int64_t k,
                        double *y, double *bound) {
    return oracle_moe_gemv_fmt(syms, scales, n_exp, rows, cols, SCALE_UE8M0, x, x_per_slot, ids, gate_w, T, k,
                               y, bound);
}

/* Round a double to the nearest bf16 value (ties to even), as a double. */
double oracle_round_bf16(double v) {
    if (v == 0.0 || isnan(v) || isinf(v)) return v;
    int e;
    double m = frexp(v, &e);                  /* v = m * 2^e, 0.5 <= |m| < 1 */
    int shift = 8;                            /* bf16 keeps 8 significant bits */
    if (e - 1 < -126) shift = 8 - (-126 - (e - 1));  /* below the normal range */
    double q = nearbyint(ldexp(m, shift));    /* default rounding: nearest, ties to even */
    double r = ldexp(q, e - shift);
    if (fabs(r) > 3.3895313892515355e38) r = copysign(INFINITY, v);
    return r;
}

/* SwiGLU between gate_up and down (reading R7), per slot:
 * y_gu[n][2I] -> h[n][I] = bf16(silu(gate) * up), silu(z) = z / (1 + e^-z). */
void oracle_swiglu_bf16(const double *y_gu, int64_t n, int64_t inter, double *h) {
    for (int64_t s = 0; s < n; ++s)
        for (int64_t i = 0; i < inter; ++i) {
            double g = y_gu[s * 2 * inter + i];
            double u = y_gu[s * 2 * inter + inter + i];
            double silu = g / (1.0 + exp(-g));
            h[s * inter + i] = oracle_round_bf16(silu * u);
        }
}

/* Whole MoE layer: gate_up GEMV per slot, SwiGLU, down GEMV per slot and the
 * gate-weighted combine.  gate_up is [n_exp][2I][H], down is [n_exp][H][I].
 * h[T][k][I] receives the bf16 activations between the two GEMVs (slots that
 * are empty or skipped hold zero); y[T][H] and bound[T][H] as in
 * oracle_moe_gemv.  Returns the number of skipped slots.  scale_fmt: both
 * stacks' scale bytes as UE8M0 or E5M3 (reading R14). */
int64_t oracle_moe_ffn_fmt(const uint32_t *gu_syms, const uint8_t *gu_scales,
                           const uint32_t *dn_syms, const uint8_t *dn_scales,
                           int64_t n_exp, int64_t hidden, int64_t inter, int scale_fmt,
                           const double *x, const int32_t *ids, const double *gate_w,
                           int64_t T, int64_t k, double *h, double *y, double *bound) {
    double *ygu = (double *)malloc(sizeof(double) * (size_t)(T * k * 2 * inter));
    double *bgu = (double *)malloc(sizeof(double) * (size_t)(T * k * 2 * inter));
    int64_t skipped = oracle_moe_gemv_fmt(gu_syms, gu_scales, n_exp, 2 * inter, hidden, scale_fmt,
                                          x, 0, ids, NULL, T, k, ygu, bgu);
    oracle_swiglu_bf16(ygu, T * k, inter, h);
    oracle_moe_gemv_fmt(dn_syms, dn_scales, n_exp, hidden, inter, scale_fmt, h, 1, ids, gate_w,
                        T, k, y, bound);
    free(ygu);
    free(bgu);
    return skipped;
}

int64_t oracle_moe_ffn(const uint32_t *gu_syms, const uint8_t *gu_scales,
                       const uint32_t *dn_syms, const uint8_t *dn_scales,
                       int64_t n_exp, int64_t hidden, int64_t inter,
                       const double *x, const int32_t *ids, const double *gate_w,
                       int64_t T, int64_t k, double *h, double *y, double *bound) {
    return oracle_moe_ffn_fmt(gu_syms, gu_scales, dn_syms, dn_scales, n_exp, hidden, inter,
                              SCALE_UE8M0, x, ids, gate_w, T, k, h, y, bound);
}

/* ---- test-only encoder: Viterbi search over the trellis ----
 *
 * XOR-Trellis article, bullet "Curvature-aware Viterbi objective": the
 * symbols are found by a Viterbi search whose additive distortion weighs
 * each position by a diagonal factor d (from H = L D L^T).  Here: minimise
 * sum_k d[k] * (target[k] - value_k)^2 over the symbol sequences of one row
 * starting from s = 0, values at scale 1.  The cost adds position by
 * position in index order.  Ties go to the smaller predecessor state, then
 * the smaller symbol; the final state with the lowest cost (smallest state
 * on ties) ends the path.  Writes n symbols (one per byte) and returns the
 * minimum cost. */
double oracle_viterbi(const double *target, const double *d, int n, uint8_t *symbols_out) {
    const int NS = 1 << 16;
    double *cost = (double *)malloc(sizeof(double) * NS);
    double *next = (double *)malloc(sizeof(double) * NS);
    int32_t *back = (int32_t *)malloc(sizeof(int32_t) * (size_t)NS * (size_t)n);
    for (int s = 0; s < NS; ++s) cost[s] = INFINITY;
    cost[0] = 0.0;
    for (int k = 0; k < n; ++k) {
        for (int s = 0; s < NS; ++s) { next[s] = INFINITY; back[(size_t)k * NS + s] = -1; }
        for (int prev = 0; prev < NS; ++prev) {          /* ascending: ties keep the smaller prev */
            if (isinf(cost[prev])) continue;
            for (int b = 0; b < 4; ++b) {                 /* ascending: then the smaller symbol */
                uint32_t s = (((uint32_t)prev << 2) | (uint32_t)b) & 0xFFFFu;
                double err = target[k] - oracle_state_value(s);
                double c = cost[prev] + d[k] * err * err;
                if (c < next[s]) {
                    next[s] = c;
                    back[(size_t)k * NS + s] = prev;
                }
            }
        }
        double *tmp = cost; cost = next; next = tmp;
    }
    int best = -1;
    for (int s = 0; s < NS; ++s)
        if (!isinf(cost[s]) && (best < 0 || cost[s] < cost[best])) best = s;
    double best_cost = cost[best];
    int s = best;
    for (int k = n - 1; k >= 0; --k) {
        symbols_out[k] = (uint8_t)(s & 3);
        s = back[(size_t)k * NS + s];
    }
    free(cost);
    free(next);
    free(back);
    return best_cost;
}

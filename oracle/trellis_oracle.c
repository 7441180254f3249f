/*
 * CPU oracle for the packed Trellis-quantized linear layer.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code,
 * header, table or constant generator with the HIP library: it is a second,
 * independent and deliberately slow statement of what the layer computes.
 *
 * Source of the method: the web page "mlx-bun 0.2.0 -> 0.4.0" (npm diff,
 * page 57), section "src/model/trellis-wide-prefill.ts", Metal kernel body:
 * bit-window extraction, 1MAD hash, byte sum, reciprocal-refinement
 * normalisation, per-row scale and bf16 rounding, then the narrow-M dot
 * product out = x . W^T. Every step below restates one of those facts in
 * plain C; none of it is translated from the printed kernel.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC.
 * The float steps rely on IEEE binary32 with round-to-nearest-even, one
 * rounding per operation (no contraction), and C99 fmaf (single rounding).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_T 256      /* weights per block */
#define ORACLE_L 12       /* window width in bits */

/* Bit j of a block's cyclic stream of 256*bits bits. Words are read LSB
 * first: stream bit j is bit (j mod 32) of word (j / 32). Indices wrap
 * inside the block ("tail-biting"): the window that runs past the last
 * word continues at word 0 of the same block (page 57, kernel body: the
 * word after the last one of a block is the block's first word). */
static uint32_t stream_bit(const uint32_t *block, int bits, uint32_t j) {
    uint32_t nbits = (uint32_t)ORACLE_T * (uint32_t)bits;
    j %= nbits;
    return (block[j >> 5] >> (j & 31u)) & 1u;
}

/* The 12-bit window of weight t (0 <= t < 256) inside a block: bits
 * [(255 - t)*bits, (255 - t)*bits + 12) of the cyclic stream, bit i of the
 * window being stream bit pos + i (page 57, kernel body: pos = (BT-1-t)*BITS,
 * L = 12). Built one bit at a time. */
uint32_t oracle_window(const uint32_t *block, int bits, int t) {
    uint32_t pos = (uint32_t)(ORACLE_T - 1 - t) * (uint32_t)bits;
    uint32_t w = 0;
    for (uint32_t i = 0; i < ORACLE_L; ++i)
        w |= stream_bit(block, bits, pos + i) << i;
    return w;
}

/* Integer code of a window (page 57, kernel body, 1MAD hash): z is the
 * window times 34038481 plus 76625530, modulo 2^32; the code is the sum of
 * the four bytes of z minus 510, so it lies in [-510, 510]. */
int32_t oracle_code(uint32_t win) {
    uint32_t z = win * 34038481u + 76625530u;   /* unsigned wrap = mod 2^32 */
    int32_t sum = 0;
    for (int i = 0; i < 4; ++i)
        sum += (int32_t)((z >> (8 * i)) & 0xFFu);
    return sum - 510;
}

/* float32 value of a code (page 57, kernel body, normalisation): with
 * C = 147.800537109375 and r = 1/C rounded to float32, take a = c*r, then
 * the residual c - a*C in one fused step, then a + residual*r in one fused
 * step. */
float oracle_value(int32_t code) {
    const float C = 147.800537109375f;
    const float r = 1.0f / C;
    const float c = (float)code;
    const float a = c * r;
    const float residual = fmaf(-a, C, c);
    return fmaf(residual, r, a);
}

/* The reciprocal constant used above, exported so the tests can pin it to
 * the exact rational 1/147.800537109375. */
float oracle_reciprocal(void) {
    const float C = 147.800537109375f;
    return 1.0f / C;
}

float oracle_bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* float32 -> bf16, round to nearest, ties to even (NaN kept quiet). */
uint16_t oracle_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep_lsb = (u >> 16) & 1u;
    u += 0x7FFFu + keep_lsb;
    return (uint16_t)(u >> 16);
}

/* Decoded bf16 weight (page 57, kernel body): the float32 value times the
 * row's scale (scale widened from bf16 exactly), product rounded to
 * float32, then rounded to the activation dtype bf16. */
uint16_t oracle_weight(uint32_t win, uint16_t scale_bf16) {
    float value = oracle_value(oracle_code(win));
    float product = value * oracle_bf16_to_f32(scale_bf16);
    return oracle_f32_to_bf16(product);
}

/* Decode rows [row0, row0 + nrows) of W[N, K] into w (nrows x K, bf16 bits).
 * codes is the full row-major stream [N, K*bits/32]; row n's block b starts
 * at word n*(K*bits/32) + b*(256*bits/32) (page 57: row_words, wpb). */
void oracle_decode_rows(const uint32_t *codes, const uint16_t *scales,
                        int k, int bits, int row0, int nrows, uint16_t *w) {
    const long row_words = (long)k * bits / 32;
    const long wpb = (long)ORACLE_T * bits / 32;
    for (int r = 0; r < nrows; ++r) {
        const int n = row0 + r;
        for (int kk = 0; kk < k; ++kk) {
            const int block = kk / ORACLE_T;
            const int t = kk % ORACLE_T;
            const uint32_t *bw = codes + (long)n * row_words + (long)block * wpb;
            w[(long)r * k + kk] = oracle_weight(oracle_window(bw, bits, t), scales[n]);
        }
    }
}

/* y[m, r] = sum_kk W[row0 + r, kk] * x[m, kk] for r < nrows, m < M, summed in
 * float64 in natural kk order (every bf16 x bf16 product is exact in
 * binary64). a[m, r] = sum_kk |W * x| for the error bound. Both outputs are
 * laid out [M, nrows]. The decoded rows are recomputed here one at a time;
 * nothing is cached. */
void oracle_prefill_rows(const uint16_t *x, int m, const uint32_t *codes,
                         const uint16_t *scales, int k, int bits, int row0,
                         int nrows, double *y, double *a) {
    const long row_words = (long)k * bits / 32;
    const long wpb = (long)ORACLE_T * bits / 32;
    for (int r = 0; r < nrows; ++r) {
        const int n = row0 + r;
        for (int i = 0; i < m; ++i) {
            y[(long)i * nrows + r] = 0.0;
            a[(long)i * nrows + r] = 0.0;
        }
        for (int kk = 0; kk < k; ++kk) {
            const uint32_t *bw = codes + (long)n * row_words + (long)(kk / ORACLE_T) * wpb;
            const double wv = (double)oracle_bf16_to_f32(
                oracle_weight(oracle_window(bw, bits, kk % ORACLE_T), scales[n]));
            for (int i = 0; i < m; ++i) {
                const double p = wv * (double)oracle_bf16_to_f32(x[(long)i * k + kk]);
                y[(long)i * nrows + r] += p;
                a[(long)i * nrows + r] += fabs(p);
            }
        }
    }
}

/* y[m, n] from an already decoded W (nrows x K bf16); same summation. */
void oracle_contract(const uint16_t *x, int m, const uint16_t *w, int k,
                     int nrows, double *y, double *a) {
    for (int r = 0; r < nrows; ++r)
        for (int i = 0; i < m; ++i) {
            double s = 0.0, sa = 0.0;
            for (int kk = 0; kk < k; ++kk) {
                const double p = (double)oracle_bf16_to_f32(w[(long)r * k + kk]) *
                                 (double)oracle_bf16_to_f32(x[(long)i * k + kk]);
                s += p;
                sa += fabs(p);
            }
            y[(long)i * nrows + r] = s;
            a[(long)i * nrows + r] = sa;
        }
}

/* ---- gate/up tail of an MLP ---------------------------------------------
 * Page "mlx-bun 0.0.4" (npm, page 62), section src/model/minicpm5.ts, MLP
 * forward: the gate and up projections are bf16 arrays, and sigmoid(gate),
 * gate * sigmoid(gate) and that product times up each yield a bf16 array.
 * Here every step is taken exactly (float64 stands in for the exact real
 * result: the products of two bf16 values are exact in it, and the sigmoid is
 * accurate to about 1e-16 relative) and rounded once to bf16. */

/* Round a double to bf16, to nearest, ties to even, in one step (no float32
 * intermediate, so no double rounding). NaN maps to the quiet NaN 0x7FC0;
 * values whose rounded magnitude reaches 2^128 become infinities. */
uint16_t oracle_f64_to_bf16(double v) {
    if (isnan(v))
        return 0x7FC0u;
    const uint16_t sign = signbit(v) ? 0x8000u : 0u;
    const double a = fabs(v);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);
    int e;
    (void)frexp(a, &e);             /* a = f * 2^e, 0.5 <= f < 1 */
    int qexp = e - 8;               /* 8 significant bits: quantum 2^(e-8) */
    if (qexp < -133)
        qexp = -133;                /* bf16 subnormal quantum */
    const double r = rint(ldexp(a, -qexp));   /* default mode: nearest, ties even */
    const double res = ldexp(r, qexp);        /* a bf16 value, or >= 2^128 */
    if (res >= 0x1p128)
        return (uint16_t)(sign | 0x7F80u);
    const float f = (float)res;                /* exact */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

/* 1 if the exact sigmoid of gate lies within 2^-21 (relative) of a point
 * halfway between two bf16 values: there a float32 evaluation of the sigmoid,
 * accurate to a few float32 ulps, may round to either neighbour. */
static int near_bf16_midpoint(double s) {
    const double a = fabs(s);
    if (a == 0.0)
        return 0;
    int e;
    (void)frexp(a, &e);
    int qexp = e - 8;
    if (qexp < -133)
        qexp = -133;
    const double scaled = ldexp(a, -qexp);
    const double mid = floor(scaled) + 0.5;
    return fabs(scaled - mid) * ldexp(1.0, qexp) <= a * 0x1p-21;
}

/* h = bf16(bf16(gate * bf16(sigmoid(gate))) * up) for bf16 gate and up.
 * *ambiguous (if not NULL) is set when the sigmoid sits so close to a bf16
 * rounding boundary that a float32 sigmoid may round the other way. */
uint16_t oracle_gate_up_chain(uint16_t gate_bf16, uint16_t up_bf16, int *ambiguous) {
    const double g = (double)oracle_bf16_to_f32(gate_bf16);
    const double u = (double)oracle_bf16_to_f32(up_bf16);
    const double sig_exact = 1.0 / (1.0 + exp(-g));
    if (ambiguous)
        *ambiguous = near_bf16_midpoint(sig_exact);
    const double sig = (double)oracle_bf16_to_f32(oracle_f64_to_bf16(sig_exact));
    const double silu = (double)oracle_bf16_to_f32(oracle_f64_to_bf16(g * sig));
    return oracle_f64_to_bf16(silu * u);
}

/* Elementwise over n pairs. */
void oracle_gate_up_chain_n(const uint16_t *gate, const uint16_t *up, long n, uint16_t *h, uint8_t *ambiguous) {
    for (long i = 0; i < n; ++i) {
        int amb = 0;
        h[i] = oracle_gate_up_chain(gate[i], up[i], &amb);
        if (ambiguous)
            ambiguous[i] = (uint8_t)amb;
    }
}

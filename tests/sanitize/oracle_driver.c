/* Drives every oracle entry point on small inputs, for an AddressSanitizer /
 * UndefinedBehaviorSanitizer build (tests/test_sanitizers.py). Exits 0 when
 * every call ran; the sanitizers abort on the first fault they find. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

uint32_t oracle_window(const uint32_t *block, int bits, int t);
int32_t oracle_code(uint32_t win);
float oracle_value(int32_t code);
float oracle_reciprocal(void);
float oracle_bf16_to_f32(uint16_t h);
uint16_t oracle_f32_to_bf16(float f);
uint16_t oracle_weight(uint32_t win, uint16_t scale_bf16);
void oracle_decode_rows(const uint32_t *codes, const uint16_t *scales, int k, int bits, int row0, int nrows,
                        uint16_t *w);
void oracle_prefill_rows(const uint16_t *x, int m, const uint32_t *codes, const uint16_t *scales, int k, int bits,
                         int row0, int nrows, double *y, double *a);
void oracle_contract(const uint16_t *x, int m, const uint16_t *w, int k, int nrows, double *y, double *a);
uint16_t oracle_f64_to_bf16(double v);
void oracle_gate_up_chain_n(const uint16_t *gate, const uint16_t *up, long n, uint16_t *h, uint8_t *ambiguous);

static uint32_t rng_state = 12345u;
static uint32_t next_u32(void) {   /* xorshift32 */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 17;
    rng_state ^= rng_state << 5;
    return rng_state;
}

int main(void) {
    /* windows of every weight of a random block, each k */
    for (int bits = 2; bits <= 4; ++bits) {
        uint32_t *block = malloc(sizeof(uint32_t) * 8 * bits);
        for (int i = 0; i < 8 * bits; ++i) block[i] = next_u32();
        for (int t = 0; t < 256; ++t) (void)oracle_code(oracle_window(block, bits, t));
        free(block);
    }
    double acc = oracle_reciprocal();
    for (int c = -510; c <= 510; ++c) acc += oracle_value(c);
    for (uint32_t w = 0; w < 4096; ++w) acc += oracle_bf16_to_f32(oracle_weight(w, (uint16_t)(0x3BA4 + (w & 255))));
    for (uint32_t b = 0; b < 65536; b += 7) acc += oracle_f32_to_bf16(oracle_bf16_to_f32((uint16_t)b));
    acc += oracle_f64_to_bf16(1e300) + oracle_f64_to_bf16(-1e-300) + oracle_f64_to_bf16(0.0 / 0.0);
    /* decode, prefill and contraction on M = 5, K = 512, N = 12, each k */
    const int m = 5, k = 512, n = 12;
    for (int bits = 2; bits <= 4; ++bits) {
        const int words = k * bits / 32;
        uint32_t *codes = malloc(sizeof(uint32_t) * n * words);
        uint16_t *scales = malloc(sizeof(uint16_t) * n);
        uint16_t *x = malloc(sizeof(uint16_t) * m * k);
        uint16_t *w = malloc(sizeof(uint16_t) * n * k);
        double *y = malloc(sizeof(double) * m * n), *a = malloc(sizeof(double) * m * n);
        for (int i = 0; i < n * words; ++i) codes[i] = next_u32();
        for (int i = 0; i < n; ++i) scales[i] = (uint16_t)(0x3BA4 + next_u32() % 257);
        for (int i = 0; i < m * k; ++i) x[i] = (uint16_t)(0x3E00 + next_u32() % 512);
        oracle_decode_rows(codes, scales, k, bits, 0, n, w);
        oracle_prefill_rows(x, m, codes, scales, k, bits, 2, n - 2, y, a);
        oracle_contract(x, m, w, k, n, y, a);
        acc += y[0] + a[m * n - 1];
        free(codes); free(scales); free(x); free(w); free(y); free(a);
    }
    /* the gate/up chain over every bf16 gate */
    uint16_t *g = malloc(sizeof(uint16_t) * 65536), *u = malloc(sizeof(uint16_t) * 65536);
    uint16_t *h = malloc(sizeof(uint16_t) * 65536);
    uint8_t *amb = malloc(65536);
    for (int i = 0; i < 65536; ++i) { g[i] = (uint16_t)i; u[i] = (uint16_t)(0x3F80 + (i & 127)); }
    oracle_gate_up_chain_n(g, u, 65536, h, amb);
    acc += h[1000] + amb[3];
    free(g); free(u); free(h); free(amb);
    printf("oracle driver ok %g\n", acc);
    return 0;
}

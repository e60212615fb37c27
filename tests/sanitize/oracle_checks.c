/*
 * Host-sanitizer run of the CPU oracle (built with gcc -fsanitize=address,
 * undefined by tests/test_sanitizers.py; test infrastructure only).
 *
 * The oracle source is compiled into this program as it is. Every exported
 * routine runs on small seeded layers that cover the three packings, every
 * block size, the optional biases and zero-point tensors, interleaved FC1
 * rows, both routing modes, the emulation flags and non-finite inputs, with
 * one and several threads. Besides the sanitizers' own checks, the program
 * checks that the thread count does not change a single output bit and that
 * the routing weights of every token sum to one.
 */
#include "../../oracle/qmoe_oracle.c"

#include <stdio.h>

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static uint64_t next_u64(void)
{
    /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static double uniform(void) { return (double)(next_u64() >> 11) * 0x1.0p-53; }

static double normalish(void) { return uniform() + uniform() + uniform() - 1.5; }

static int failures = 0;

#define CHECK(cond, ...)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                 \
            fprintf(stderr, "\n");                        \
            ++failures;                                   \
        }                                                 \
    } while (0)

static uint16_t scale_bits(void)
{
    /* fp16 of a small positive scale: exponent 2^-10..2^-5, random mantissa */
    return (uint16_t)(((5 + next_u64() % 6) << 10) | (next_u64() & 0x3FF));
}

static void run_layer(int bits, int bs, int E, int k, int64_t H, int64_t I, int64_t T, int extras,
                      int normalize, int interleaved, int emulate)
{
    oracle_layer L = {H, I, E, k, bits, bs, -1, emulate, normalize, interleaved, 0};
    L.zero_point = 1 << (bits - 1);
    const int64_t rb1 = H * bits / 8, rb2 = I * bits / 8;
    uint8_t *c1 = malloc((size_t)(E * 2 * I * rb1)), *c2 = malloc((size_t)(E * H * rb2));
    uint16_t *s1 = malloc(sizeof(uint16_t) * (size_t)(E * 2 * I * (H / bs)));
    uint16_t *s2 = malloc(sizeof(uint16_t) * (size_t)(E * H * (I / bs)));
    uint8_t *z1 = malloc((size_t)(E * 2 * I * (H / bs))), *z2 = malloc((size_t)(E * H * (I / bs)));
    double *b1 = malloc(sizeof(double) * (size_t)(E * 2 * I)), *b2 = malloc(sizeof(double) * (size_t)(E * H));
    double *x = malloc(sizeof(double) * (size_t)(T * H)), *lg = malloc(sizeof(double) * (size_t)(T * E));
    double *o1 = malloc(sizeof(double) * (size_t)(T * H)), *o3 = malloc(sizeof(double) * (size_t)(T * H));
    for (int64_t i = 0; i < E * 2 * I * rb1; ++i) c1[i] = (uint8_t)next_u64();
    for (int64_t i = 0; i < E * H * rb2; ++i) c2[i] = (uint8_t)next_u64();
    for (int64_t i = 0; i < E * 2 * I * (H / bs); ++i) { s1[i] = scale_bits(); z1[i] = (uint8_t)(next_u64() % (1u << bits)); }
    for (int64_t i = 0; i < E * H * (I / bs); ++i) { s2[i] = scale_bits(); z2[i] = (uint8_t)(next_u64() % (1u << bits)); }
    for (int64_t i = 0; i < E * 2 * I; ++i) b1[i] = 0.1 * normalish();
    for (int64_t i = 0; i < E * H; ++i) b2[i] = 0.1 * normalish();
    for (int64_t i = 0; i < T * H; ++i) x[i] = 2.0 * normalish();
    for (int64_t i = 0; i < T * E; ++i) lg[i] = normalish();
    /* a token with equal logits and a token with a huge activation */
    if (T > 2) {
        for (int e = 0; e < E; ++e) lg[1 * E + e] = 0.25;
        x[2 * H] = 1.0e6;
    }
    int st1 = oracle_forward_ext(&L, x, lg, c1, s1, c2, s2, extras ? b1 : NULL, extras ? b2 : NULL,
                                 extras ? z1 : NULL, extras ? z2 : NULL, T, o1, 1);
    int st3 = oracle_forward_ext(&L, x, lg, c1, s1, c2, s2, extras ? b1 : NULL, extras ? b2 : NULL,
                                 extras ? z1 : NULL, extras ? z2 : NULL, T, o3, 3);
    CHECK(st1 == ORACLE_OK && st3 == ORACLE_OK, "forward status %d %d", st1, st3);
    CHECK(memcmp(o1, o3, sizeof(double) * (size_t)(T * H)) == 0,
          "thread count changed the output (bits %d bs %d emulate %d)", bits, bs, emulate);

    int32_t *ids = malloc(sizeof(int32_t) * (size_t)(T * k));
    double *w = malloc(sizeof(double) * (size_t)(T * k));
    CHECK(oracle_route(lg, T, E, k, normalize, ids, w) == ORACLE_OK, "route status");
    for (int64_t t = 0; t < T && normalize; ++t) {
        double s = 0.0;
        for (int j = 0; j < k; ++j) s += w[t * k + j];
        CHECK(fabs(s - 1.0) < 1e-12, "weights of token %ld sum to %.17g", (long)t, s);
    }
    int32_t *cnt = malloc(sizeof(int32_t) * (size_t)E), *off = malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *sorted = malloc(sizeof(int32_t) * (size_t)(T * k)), *inv = malloc(sizeof(int32_t) * (size_t)(T * k));
    CHECK(oracle_permute(ids, T * k, E, cnt, off, sorted, inv) == ORACLE_OK, "permute status");
    for (int64_t r = 0; r < T * k; ++r) CHECK(sorted[inv[r]] == r, "inverse of route %ld", (long)r);

    double *dq = malloc(sizeof(double) * (size_t)(2 * I * H));
    uint16_t *dh = malloc(sizeof(uint16_t) * (size_t)(2 * I * H));
    CHECK(oracle_dequant_zp(c1, s1, extras ? z1 : NULL, 2 * I, H, bits, bs, L.zero_point, dq) == ORACLE_OK,
          "dequant status");
    CHECK(oracle_dequant_f16(c1, s1, extras ? z1 : NULL, 2 * I, H, bits, bs, L.zero_point, dh) == ORACLE_OK,
          "dequant f16 status");
    for (int64_t i = 0; i < 2 * I * H; ++i)
        CHECK(fabs(oracle_half_to_double(dh[i]) - dq[i]) <= fabs(dq[i]) * 0x1.0p-11, "f16 dequant %ld", (long)i);

    float *f = malloc(sizeof(float) * (size_t)(T * H));
    uint16_t *b = malloc(sizeof(uint16_t) * (size_t)(T * H));
    oracle_round_output(o1, T * H, f, b);
    free(f); free(b); free(dq); free(dh); free(cnt); free(off); free(sorted); free(inv); free(ids); free(w);
    free(c1); free(c2); free(s1); free(s2); free(z1); free(z2); free(b1); free(b2); free(x); free(lg);
    free(o1); free(o3);
}

static void conversions(void)
{
    /* every fp16 pattern round-trips; specials and out-of-range values convert without UB */
    for (uint32_t h = 0; h < 65536; ++h) {
        double v = oracle_half_to_double((uint16_t)h);
        uint16_t back = oracle_double_to_half(v);
        if (v == v) CHECK(back == h || (v == 0.0 && (back & 0x7FFF) == 0), "fp16 %04x -> %04x", h, back);
    }
    const double specials[] = {0.0, -0.0, 1e-300, -1e-300, 65504.0, 65520.0, 1e300, -1e300,
                               INFINITY, -INFINITY, NAN, 0x1.0p-24, 0x1.0p-25, 0x1.8p-25};
    for (size_t i = 0; i < sizeof(specials) / sizeof(specials[0]); ++i) {
        (void)oracle_double_to_half(specials[i]);
        (void)oracle_f32_to_bf16((float)specials[i]);
    }
    double rows[3 * 64];
    for (int i = 0; i < 3 * 64; ++i) rows[i] = normalish() * (i < 64 ? 1e-9 : i < 128 ? 1e9 : 1.0);
    rows[130] = INFINITY;
    rows[131] = NAN;
    double tmp[64];
    oracle_emulate_x_rows(rows, 3, 64, tmp);
    for (int i = 0; i < 3 * 64; ++i) rows[i] = normalish() * (i < 64 ? 1e-12 : 1e12);
    oracle_emulate_h_rows(rows, 3, 64);
    uint16_t hb[3 * 64];
    oracle_double_to_half_n(rows, 3 * 64, hb);
}

int main(void)
{
    conversions();
    const int fmts[][2] = {{4, 32}, {4, 64}, {4, 128}, {3, 32}, {3, 64}, {3, 128}, {2, 32}, {2, 64}, {2, 128}};
    for (size_t f = 0; f < sizeof(fmts) / sizeof(fmts[0]); ++f) {
        const int bits = fmts[f][0], bs = fmts[f][1];
        run_layer(bits, bs, 6, 3, 256, 128, 7, (int)(f & 1), 1, 0, 0);
        run_layer(bits, bs, 5, 2, 128, 128, 5, 1, (int)(f & 1), 1, EMU_X_F16 | EMU_W_F16 | EMU_H_F16);
    }
    run_layer(4, 32, 4, 4, 64, 32, 9, 1, 0, 0, EMU_W_BF16 | EMU_H_BF16);
    run_layer(2, 32, 1, 1, 64, 32, 3, 0, 1, 0, EMU_X_F16);
    /* invalid arguments are rejected, not read */
    oracle_layer bad = {64, 32, 4, 5, 4, 32, 8, 0, 1, 0, 0};
    double one = 1.0, out = 0.0;
    uint8_t byte = 0;
    uint16_t half = 0;
    CHECK(oracle_forward_ext(&bad, &one, &one, &byte, &half, &byte, &half, NULL, NULL, NULL, NULL, 1, &out, 1)
              == ORACLE_BAD_ARG, "top_k > E accepted");
    bad.top_k = 2;
    bad.bits = 5;
    CHECK(oracle_forward_ext(&bad, &one, &one, &byte, &half, &byte, &half, NULL, NULL, NULL, NULL, 1, &out, 1)
              == ORACLE_BAD_ARG, "bits 5 accepted");
    CHECK(oracle_route(&one, 1, 1, 2, 1, NULL, NULL) == ORACLE_BAD_ARG, "route NULL accepted");
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer checks passed\n");
    return 0;
}

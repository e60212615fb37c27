/*
 * Plain, slow CPU oracle for the quantized MoE layer (com.microsoft::QMoE
 * semantics with SwiGLU experts).
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. It shares no code,
 * header, table or helper with the GPU library, and the GPU library never
 * calls it.
 *
 * Every quantity is computed in double precision from the stored inputs read
 * as exact values. Sources (web pages on onnxruntime pull requests):
 *
 *  - "Document and test packed token inputs for MoE and QMoE" (Description):
 *    input [total_tokens, hidden], router [total_tokens, num_experts], output
 *    [total_tokens, hidden]; routing is token-local, so packed sequences need
 *    no boundaries. QMoE takes raw router logits; the reference block applies
 *    a softmax over the top-k logits (review comments on the test harness).
 *  - "[CUDA/CPU] Add AVX2 INT4 cold-expert kernel and zero-cold doorbell
 *    short-circuit" (Motivation & Summary, item 3): SwiGLU contract, fc1 rows
 *    = 2 * inter_size, unsigned codes with a zero-point code.
 *  - "[CUDA] Add INT4 and INT3 QMoE CPU/GPU offload support" (Description):
 *    integer quantization with expert_weight_bits 4/3 and block sizes
 *    {32, 64, 128}; scales stored [N, K/block] (not block-major).
 *  - "[CUDA] Add MoEPacked CPU/GPU hybrid offload ..." (Key Changes, item 4
 *    and the review-fix commit): the partial sums stay in fp32 and the
 *    combine rounds once; NaN stays NaN when rounding to bf16; dot products
 *    get K-sized heap scratch, not stack arrays.
 *
 * Readings taken where the pages leave a step open:
 *  - top-k on raw logits, ties to the lower expert index, slots ordered by
 *    descending logit then ascending index;
 *  - routing weights: with normalized routing, the softmax over the k
 *    selected logits; without it, each selected expert's softmax probability
 *    over all num_experts logits (the selection is the same top-k either
 *    way, since the softmax is monotonic);
 *  - fc1 rows [0, I) are the gate, rows [I, 2I) the up projection, and
 *    h = silu(gate) * up with silu(g) = g / (1 + exp(-g)) and no clamp;
 *    with interleaved FC1 rows (the exporter layout named in the review of
 *    "[CUDA] Add INT4 and INT3 QMoE CPU/GPU offload support", producer/
 *    consumer contract) row 2n is gate n and row 2n+1 is up n, and the scale
 *    rows follow the same order;
 *  - optional biases ("[CUDA] Add INT4 and INT3 QMoE CPU/GPU offload
 *    support", commit notes: FC1/FC2 biases [E, 2I] and [E, H] in the
 *    activation dtype; the FC2 bias, indexed by the original expert, is added
 *    before rounding): the FC1 bias of a row is added to that row's dot
 *    product (gate and up, in the rows' storage order) before SwiGLU, and the
 *    FC2 bias of output m to y[m] before the routing-weighted sum;
 *  - W[n][k] = (q[n][k] - zp) * s[n][k / block], where zp is the layer's
 *    scalar zero-point code or, when a zero-point tensor is given, its code
 *    zp[n][k / block] (one unsigned byte per row and quant block, laid out
 *    like the scales); INT4 two codes per byte low
 *    nibble first, INT2 four per byte low bits first, INT3 eight codes per
 *    three bytes with code i at bits [3i, 3i+3) of the little-endian 24-bit
 *    word;
 *  - the permutation is the stable counting sort of route ids r = t*k + j by
 *    expert;
 *  - the output is the double accumulator rounded once to fp32 and, for bf16
 *    outputs, that fp32 rounded to bf16 (round to nearest even).
 *
 * An optional emulation mode (EMU_* flags, off by default) applies the
 * rounding points of the GPU's fp16 matrix-core datapath to the activations,
 * the dequantized weights and the SwiGLU output (described where the flags
 * are defined). It is pinned, like the plain definition, by the tests:
 * against numpy's float16 conversion (every fp16 value, every tie, the
 * range edges) and against an independent vectorized twin of each rounding
 * point and of the whole layer.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_NO_MEM 2

/* IEEE binary16 bit pattern -> double (exact). */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int exponent = (h >> 10) & 31;
    int mantissa = h & 1023;
    double v;
    if (exponent == 0)
        v = ldexp((double)mantissa, -24);                 /* subnormal or zero */
    else if (exponent == 31)
        v = mantissa ? NAN : INFINITY;
    else
        v = ldexp((double)(mantissa | 1024), exponent - 25);
    return sign ? -v : v;
}

/* fp32 -> bf16 bit pattern, round to nearest even; NaN stays NaN. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);           /* quiet NaN, sign kept */
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

/* IEEE binary16 nearest to a double (round to nearest, ties to even, with
 * gradual underflow), as a bit pattern. NaN keeps its sign and becomes the
 * quiet NaN 0x7E00; magnitudes from 65520 up round to infinity (65520 lies
 * half way between 65504 and 2^16, and the tie goes to the even pattern).
 * Every finite value is rounded on the grid of its binade: steps of 2^-24
 * below 2^-14, else 2^(E-10) for values in [2^E, 2^(E+1)). */
uint16_t oracle_double_to_half(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v)) return (uint16_t)(sign | 0x7E00u);
    double a = fabs(v);
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);
    if (a == 0.0) return sign;
    int ex;
    (void)frexp(a, &ex);                 /* a = f * 2^ex, f in [0.5, 1) */
    int E = ex - 1;                      /* a in [2^E, 2^(E+1)) */
    if (E < -14) E = -14;
    double step = ldexp(1.0, E - 10);
    double r = nearbyint(a / step) * step;   /* exact scaling; ties to even */
    if (r == 0.0) return sign;
    if (r < ldexp(1.0, -14))                 /* subnormal: r = m * 2^-24 */
        return (uint16_t)(sign | (uint16_t)ldexp(r, 24));
    (void)frexp(r, &ex);                     /* the rounding may reach the next binade */
    E = ex - 1;
    int mant = (int)(ldexp(r, 10 - E)) - 1024;
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)mant);
}

static double round_half(double v) { return oracle_half_to_double(oracle_double_to_half(v)); }

/* Unsigned code number kk of one packed row. */
static int code_at(const uint8_t *row, int64_t kk, int bits)
{
    if (bits == 4) {
        uint8_t b = row[kk >> 1];
        return (kk & 1) ? (b >> 4) : (b & 15);
    }
    if (bits == 2) {
        uint8_t b = row[kk >> 2];
        return (b >> (2 * (kk & 3))) & 3;
    }
    /* bits == 3 */
    int64_t g = kk >> 3;
    int i = (int)(kk & 7);
    uint32_t w = (uint32_t)row[3 * g] | ((uint32_t)row[3 * g + 1] << 8) |
                 ((uint32_t)row[3 * g + 2] << 16);
    return (int)((w >> (3 * i)) & 7u);
}

static int64_t row_bytes(int64_t K, int bits) { return K * bits / 8; }

static int valid_format(int64_t K, int bits, int bs)
{
    if (bits != 2 && bits != 3 && bits != 4) return 0;
    if (bs <= 0 || K <= 0 || K % bs != 0) return 0;
    if (K % 8 != 0) return 0;
    return 1;
}

/* (q - zp) * s for one [N, K] matrix; zps [N, K/bs] or NULL for the scalar zp. */
int oracle_dequant_zp(const uint8_t *codes, const uint16_t *scales, const uint8_t *zps, int64_t N,
                      int64_t K, int bits, int bs, int zp, double *out)
{
    if (!codes || !scales || !out || N < 0 || !valid_format(K, bits, bs)) return ORACLE_BAD_ARG;
    int64_t rb = row_bytes(K, bits), nblk = K / bs;
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t *row = codes + n * rb;
        for (int64_t kk = 0; kk < K; ++kk) {
            double s = oracle_half_to_double(scales[n * nblk + kk / bs]);
            int z = zps ? (int)zps[n * nblk + kk / bs] : zp;
            out[n * K + kk] = (double)(code_at(row, kk, bits) - z) * s;
        }
    }
    return ORACLE_OK;
}

/* The fp16 operand of the emulated datapath: fp16((q - zp) * s) bit patterns. */
int oracle_dequant_f16(const uint8_t *codes, const uint16_t *scales, const uint8_t *zps, int64_t N,
                       int64_t K, int bits, int bs, int zp, uint16_t *out)
{
    if (!codes || !scales || !out || N < 0 || !valid_format(K, bits, bs)) return ORACLE_BAD_ARG;
    int64_t rb = row_bytes(K, bits), nblk = K / bs;
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t *row = codes + n * rb;
        for (int64_t kk = 0; kk < K; ++kk) {
            double s = oracle_half_to_double(scales[n * nblk + kk / bs]);
            int z = zps ? (int)zps[n * nblk + kk / bs] : zp;
            out[n * K + kk] = oracle_double_to_half((double)(code_at(row, kk, bits) - z) * s);
        }
    }
    return ORACLE_OK;
}

int oracle_dequant(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                   int bits, int bs, int zp, double *out)
{
    return oracle_dequant_zp(codes, scales, NULL, N, K, bits, bs, zp, out);
}

/* Top-k selection and the routing weights, per token: the softmax over the
 * selected logits (normalize != 0) or over all E logits (normalize == 0). */
int oracle_route(const double *logits, int64_t T, int64_t E, int k, int normalize,
                 int32_t *topk_id, double *topk_w)
{
    if (!logits || !topk_id || !topk_w || T < 0 || E < 1 || k < 1 || k > E) return ORACLE_BAD_ARG;
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
    if (!taken) return ORACLE_NO_MEM;
    for (int64_t t = 0; t < T; ++t) {
        const double *l = logits + t * E;
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                if (taken[e]) continue;
                /* strict '>' keeps the lowest index among equal logits */
                if (best < 0 || l[e] > l[best]) best = e;
            }
            taken[best] = 1;
            topk_id[t * k + j] = (int32_t)best;
        }
        double lmax = l[topk_id[t * k]];
        double denom = 0.0;
        if (normalize)
            for (int j = 0; j < k; ++j) denom += exp(l[topk_id[t * k + j]] - lmax);
        else
            for (int64_t e = 0; e < E; ++e) denom += exp(l[e] - lmax);
        for (int j = 0; j < k; ++j) topk_w[t * k + j] = exp(l[topk_id[t * k + j]] - lmax) / denom;
    }
    free(taken);
    return ORACLE_OK;
}

/* Stable counting sort of the routes r = t*k + j by expert. */
int oracle_permute(const int32_t *topk_id, int64_t R, int64_t E, int32_t *counts,
                   int32_t *offsets, int32_t *sorted_routes, int32_t *inv_pos)
{
    if (!topk_id || !counts || !offsets || !sorted_routes || !inv_pos || R < 0 || E < 1)
        return ORACLE_BAD_ARG;
    for (int64_t e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t r = 0; r < R; ++r) {
        if (topk_id[r] < 0 || topk_id[r] >= E) return ORACLE_BAD_ARG;
        counts[topk_id[r]]++;
    }
    offsets[0] = 0;
    for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *cursor = (int32_t *)malloc((size_t)E * sizeof(int32_t));
    if (!cursor) return ORACLE_NO_MEM;
    for (int64_t e = 0; e < E; ++e) cursor[e] = offsets[e];
    for (int64_t r = 0; r < R; ++r) {
        int32_t pos = cursor[topk_id[r]]++;
        sorted_routes[pos] = (int32_t)r;
        inv_pos[r] = pos;
    }
    free(cursor);
    return ORACLE_OK;
}

/* Rounding-point emulation of the fp16 matrix-core datapath of the grouped
 * (prefill) path (off by default; each flag rounds one operand):
 * A range exponent e of a set of values with largest magnitude M, for a
 * lower bound lo, is 0 while M lies in [lo, 2^15] (or M is 0 or the set holds
 * a non-finite value), else (exponent of M) - 15, which puts M * 2^-e in
 * [2^14, 2^15), clamped to [-120, 120]; values v are then stored as
 * fp16(v * 2^-e).
 *  EMU_X_F16: token t's activations enter as fp16(x * 2^-e_t) * 2^e_t, e_t
 *    the range exponent (lo = 2^-3) of the token's row;
 *  EMU_W_F16: each dequantized weight is fp16((q - zp) * s);
 *  EMU_H_F16: each route's SwiGLU output h enters FC2 as fp16 in chunks of
 *    32 consecutive values n: chunk c is stored as fp16(h * 2^-e_c), e_c its
 *    range exponent (lo = 2^-14); the route's exponent is E = max_c e_c and
 *    FC2 reads fp16(stored * 2^(e_c - E)) * 2^E.
 * fp16() is oracle_double_to_half: nearest, ties to even, gradual underflow. */
#define EMU_X_F16 1
#define EMU_W_F16 2
#define EMU_H_F16 4
#define EMU_H_CHUNK 32
/* The earlier bf16 datapath's rounding points (x is rounded by the caller):
 * weights and h rounded to bf16, nearest even. */
#define EMU_W_BF16 8
#define EMU_H_BF16 16

static double to_bf16(double v)
{
    uint32_t u = (uint32_t)oracle_f32_to_bf16((float)v) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* The range exponent of a set of values with largest magnitude M (finite),
 * for the lower bound lo. */
static int range_exponent(double M, double lo)
{
    if (M == 0.0 || (M >= lo && M <= 32768.0)) return 0;
    int ex;
    (void)frexp(M, &ex);       /* M = f * 2^ex, f in [0.5, 1): M * 2^-(ex-15) in [2^14, 2^15) */
    int e = ex - 15;
    return e < -120 ? -120 : e > 120 ? 120 : e;
}

static void emulate_x(const double *x, int64_t H, double *out)
{
    double M = 0.0;
    int finite = 1;
    for (int64_t i = 0; i < H; ++i) {
        if (!isfinite(x[i])) finite = 0;
        else if (fabs(x[i]) > M) M = fabs(x[i]);
    }
    int e = finite ? range_exponent(M, 0.125) : 0;
    for (int64_t i = 0; i < H; ++i) out[i] = ldexp(round_half(ldexp(x[i], -e)), e);
}

static void emulate_h(double *h, int64_t I)
{
    int64_t nc = I / EMU_H_CHUNK;
    int E = INT32_MIN;
    /* first pass: chunk exponents and the stored fp16 values */
    int *ec = (int *)malloc((size_t)nc * sizeof(int));
    if (!ec) return;   /* unreachable in practice; leaves h unrounded */
    for (int64_t c = 0; c < nc; ++c) {
        double M = 0.0;
        int finite = 1;
        for (int64_t n = c * EMU_H_CHUNK; n < (c + 1) * EMU_H_CHUNK; ++n) {
            if (!isfinite(h[n])) finite = 0;
            else if (fabs(h[n]) > M) M = fabs(h[n]);
        }
        int e = finite ? range_exponent(M, ldexp(1.0, -14)) : 0;
        ec[c] = e;
        if (e > E) E = e;
        for (int64_t n = c * EMU_H_CHUNK; n < (c + 1) * EMU_H_CHUNK; ++n) h[n] = round_half(ldexp(h[n], -e));
    }
    /* second pass: every chunk brought to the route's exponent */
    for (int64_t c = 0; c < nc; ++c)
        for (int64_t n = c * EMU_H_CHUNK; n < (c + 1) * EMU_H_CHUNK; ++n)
            h[n] = ldexp(round_half(ldexp(h[n], ec[c] - E)), E);
    free(ec);
}

typedef struct {
    int64_t hidden, inter, num_experts;
    int32_t top_k, bits, block_size, zero_point;
    int32_t emulate;     /* EMU_* bitmask, 0 for the plain definition */
    int32_t normalize;   /* routing weights: 1 over the selected k, 0 over all experts */
    int32_t fc1_interleaved;  /* FC1 rows: 0 gate block then up block, 1 interleaved */
    int32_t pad;
} oracle_layer;

typedef struct {
    const oracle_layer *L;
    const double *x, *logits;
    const uint8_t *fc1_codes, *fc2_codes;
    const uint16_t *fc1_scales, *fc2_scales;
    const double *fc1_bias, *fc2_bias;   /* [E, 2I] and [E, H], or NULL */
    const uint8_t *fc1_zp, *fc2_zp;      /* [E, 2I, H/bs] and [E, H, I/bs], or NULL */
    double *out;
    int64_t t0, t1;
    int status;
} job;

/* dot of one dequantized weight row with a double vector */
static double row_dot(const uint8_t *row, const uint16_t *srow, const uint8_t *zrow,
                      const double *v, int64_t K, int bits, int bs, int zp, int emu_w, int emu_wb)
{
    double acc = 0.0;
    for (int64_t kk = 0; kk < K; ++kk) {
        int z = zrow ? (int)zrow[kk / bs] : zp;
        double w = (double)(code_at(row, kk, bits) - z) * oracle_half_to_double(srow[kk / bs]);
        if (emu_w) w = round_half(w);
        if (emu_wb) w = to_bf16(w);
        acc += w * v[kk];
    }
    return acc;
}

static void *run_tokens(void *arg)
{
    job *jb = (job *)arg;
    const oracle_layer *L = jb->L;
    int64_t H = L->hidden, I = L->inter, E = L->num_experts;
    int k = L->top_k, bits = L->bits, bs = L->block_size, zp = L->zero_point;
    int64_t rb1 = row_bytes(H, bits), rb2 = row_bytes(I, bits);
    int64_t nb1 = H / bs, nb2 = I / bs;
    int emu_x = (L->emulate & EMU_X_F16) != 0;
    int emu_w = (L->emulate & EMU_W_F16) != 0;
    int emu_h = (L->emulate & EMU_H_F16) != 0;
    int emu_wb = (L->emulate & EMU_W_BF16) != 0;
    int emu_hb = (L->emulate & EMU_H_BF16) != 0;

    double *h = (double *)malloc((size_t)I * sizeof(double));
    double *acc = (double *)malloc((size_t)H * sizeof(double));
    double *xe = (double *)malloc((size_t)H * sizeof(double));
    int32_t *ids = (int32_t *)malloc((size_t)k * sizeof(int32_t));
    double *w = (double *)malloc((size_t)k * sizeof(double));
    if (!h || !acc || !xe || !ids || !w) {
        jb->status = ORACLE_NO_MEM;
        free(h); free(acc); free(xe); free(ids); free(w);
        return NULL;
    }
    for (int64_t t = jb->t0; t < jb->t1; ++t) {
        const double *xt = jb->x + t * H;
        if (emu_x) {
            emulate_x(xt, H, xe);
            xt = xe;
        }
        int st = oracle_route(jb->logits + t * E, 1, E, k, jb->L->normalize, ids, w);
        if (st != ORACLE_OK) { jb->status = st; break; }
        for (int64_t m = 0; m < H; ++m) acc[m] = 0.0;
        for (int j = 0; j < k; ++j) {
            int64_t e = ids[j];
            const uint8_t *c1 = jb->fc1_codes + e * (2 * I) * rb1;
            const uint16_t *s1 = jb->fc1_scales + e * (2 * I) * nb1;
            const uint8_t *c2 = jb->fc2_codes + e * H * rb2;
            const uint16_t *s2 = jb->fc2_scales + e * H * nb2;
            for (int64_t n = 0; n < I; ++n) {
                const int64_t gr = jb->L->fc1_interleaved ? 2 * n : n;
                const int64_t ur = jb->L->fc1_interleaved ? 2 * n + 1 : I + n;
                const uint8_t *z1 = jb->fc1_zp ? jb->fc1_zp + e * (2 * I) * nb1 : NULL;
                double g = row_dot(c1 + gr * rb1, s1 + gr * nb1, z1 ? z1 + gr * nb1 : NULL, xt, H,
                                   bits, bs, zp, emu_w, emu_wb);
                double u = row_dot(c1 + ur * rb1, s1 + ur * nb1, z1 ? z1 + ur * nb1 : NULL, xt, H,
                                   bits, bs, zp, emu_w, emu_wb);
                if (jb->fc1_bias) {
                    g += jb->fc1_bias[e * 2 * I + gr];
                    u += jb->fc1_bias[e * 2 * I + ur];
                }
                h[n] = g / (1.0 + exp(-g)) * u;
                if (emu_hb) h[n] = to_bf16(h[n]);
            }
            if (emu_h) emulate_h(h, I);
            for (int64_t m = 0; m < H; ++m) {
                const uint8_t *z2 = jb->fc2_zp ? jb->fc2_zp + (e * H + m) * nb2 : NULL;
                double y = row_dot(c2 + m * rb2, s2 + m * nb2, z2, h, I, bits, bs, zp, emu_w, emu_wb);
                if (jb->fc2_bias) y += jb->fc2_bias[e * H + m];
                acc[m] += w[j] * y;
            }
        }
        for (int64_t m = 0; m < H; ++m) jb->out[t * H + m] = acc[m];
    }
    free(h); free(acc); free(xe); free(ids); free(w);
    return NULL;
}

/*
 * Whole layer: out[t][m] = sum_j w[t][j] * (W2[e] silu(W1g[e] x_t) * (W1u[e] x_t))[m]
 * for the k experts e = topk_id[t][j], accumulated in double.
 * x: [T, H] double, logits: [T, E] double, out: [T, H] double.
 * Tokens are split into contiguous ranges over nthreads POSIX threads.
 */
int oracle_forward_ext(const oracle_layer *L, const double *x, const double *logits,
                       const uint8_t *fc1_codes, const uint16_t *fc1_scales,
                       const uint8_t *fc2_codes, const uint16_t *fc2_scales,
                       const double *fc1_bias, const double *fc2_bias,
                       const uint8_t *fc1_zp, const uint8_t *fc2_zp,
                       int64_t T, double *out, int nthreads)
{
    if (!L || T < 0) return ORACLE_BAD_ARG;
    if (T == 0) return ORACLE_OK;
    if (!x || !logits || !fc1_codes || !fc1_scales || !fc2_codes || !fc2_scales || !out)
        return ORACLE_BAD_ARG;
    if (L->num_experts < 1 || L->top_k < 1 || L->top_k > L->num_experts) return ORACLE_BAD_ARG;
    if (!valid_format(L->hidden, L->bits, L->block_size) ||
        !valid_format(L->inter, L->bits, L->block_size))
        return ORACLE_BAD_ARG;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > T) nthreads = (int)T;
    job *jobs = (job *)calloc((size_t)nthreads, sizeof(job));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return ORACLE_NO_MEM; }
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = (job){L, x, logits, fc1_codes, fc2_codes, fc1_scales, fc2_scales, fc1_bias,
                        fc2_bias, fc1_zp, fc2_zp, out, T * i / nthreads, T * (i + 1) / nthreads,
                        ORACLE_OK};
    }
    int started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, run_tokens, &jobs[i]) != 0) break;
        started = i;
    }
    run_tokens(&jobs[0]);
    for (int i = 1; i <= started; ++i) pthread_join(th[i], NULL);
    for (int i = started + 1; i < nthreads; ++i) run_tokens(&jobs[i]);  /* not started */
    int st = ORACLE_OK;
    for (int i = 0; i < nthreads; ++i)
        if (jobs[i].status != ORACLE_OK) st = jobs[i].status;
    free(jobs); free(th);
    return st;
}

int oracle_forward(const oracle_layer *L, const double *x, const double *logits,
                   const uint8_t *fc1_codes, const uint16_t *fc1_scales,
                   const uint8_t *fc2_codes, const uint16_t *fc2_scales,
                   int64_t T, double *out, int nthreads)
{
    return oracle_forward_ext(L, x, logits, fc1_codes, fc1_scales, fc2_codes, fc2_scales, NULL,
                              NULL, NULL, NULL, T, out, nthreads);
}

/* Final rounding: double accumulator -> fp32 (one rounding) and -> bf16 of that fp32. */
void oracle_round_output(const double *acc, int64_t n, float *out_f32, uint16_t *out_bf16)
{
    for (int64_t i = 0; i < n; ++i) {
        float f = (float)acc[i];
        if (out_f32) out_f32[i] = f;
        if (out_bf16) out_bf16[i] = oracle_f32_to_bf16(f);
    }
}

/* Batch helpers for exhaustive checks. */
void oracle_half_to_double_n(const uint16_t *h, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_half_to_double(h[i]);
}

void oracle_f32_to_bf16_n(const float *f, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(f[i]);
}

/* The datapath emulation's activation and SwiGLU-output rounding points,
 * applied in place to `rows` rows (for the pin tests). */
void oracle_emulate_x_rows(double *x, int64_t rows, int64_t H, double *tmp)
{
    for (int64_t r = 0; r < rows; ++r) {
        emulate_x(x + r * H, H, tmp);
        memcpy(x + r * H, tmp, (size_t)H * sizeof(double));
    }
}

void oracle_emulate_h_rows(double *h, int64_t rows, int64_t I)
{
    for (int64_t r = 0; r < rows; ++r) emulate_h(h + r * I, I);
}

void oracle_double_to_half_n(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_double_to_half(v[i]);
}

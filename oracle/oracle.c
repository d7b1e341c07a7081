/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU implementation of what the quantized
 * GEMV / MoE path computes, in IEEE double precision.  Only the test suite,
 * the smoke check and the bench's CPU-baseline leg load this library; the HIP
 * library never links, includes or calls it, and the two share no code,
 * headers, tables or constants.
 *
 * Method: every GGUF block is dequantized to exact f64 values by the block
 * formulas, then the dot product is taken in f64 (the pages state that their
 * in-shader products equal llama.cpp's "up to summation order", so the plain
 * definition dequantize-then-dot is the result to reproduce).  No factorisation
 * used by the kernels (block-scale-once, x-sums for the K-quant mins) appears
 * here.
 *
 * Sources (the five diskformer package-diff pages; each function names its own):
 *   [bonsai]  diskformer 0.5.4 -> 0.6.6, engines/ternary_bonsai_2_dflash.js
 *   [gemma4]  diskformer 0.0.1 -> 0.2.0, engines/gemma4_moe_ssd.js
 *   [qwen3]   diskformer 0.0.1 -> 0.3.0, engines/qwen3_moe_ssd.js
 *   [qwen35]  diskformer 0.0.1 -> 0.3.0, engines/qwen35_moe_ssd.js
 *   [dense]   diskformer 0.5.4 -> 0.6.6, engines/qwen35_dense.js
 *
 * Parity status: every function here is pinned by tests/test_oracle_*.py
 * against closed forms, second decoders written from the pages' other
 * renderings, brute force and library routines.
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* GGML type ids (the GGUF on-disk enum; [bonsai] header section prints
 * Q4_K = 12 and Q6_K = 14; Q4_0 = 2 and Q8_0 = 8 complete the same enum, where
 * plain f32 is 0: the router and shared-gate weights stay f32 on the pages,
 * [qwen3] WGSL matmulF32). */
#define OR_F32 0
#define OR_Q4_0 2
#define OR_Q8_0 8
#define OR_Q4_K 12
#define OR_Q6_K 14

#define OR_ACT_SILU 0
#define OR_ACT_GELU_TANH 1

/* ---------------------------------------------------------------- f16 ---- */
/* IEEE binary16 -> double, exact for every pattern (subnormals, inf, NaN).
 * [bonsai] "f16 codecs" section, f16ToF32: sign bit 15, 5-bit exponent
 * (bias 15), 10-bit fraction; exponent 0 is subnormal, 31 is inf/NaN. */
double or_f16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* ------------------------------------------------------- block formats ---- */
int or_block_values(int type)  /* values per block */
{
    switch (type) {
    case OR_F32: return 1;
    case OR_Q8_0: case OR_Q4_0: return 32;
    case OR_Q4_K: case OR_Q6_K: return 256;
    default: return 0;
    }
}

int or_block_bytes(int type)
{
    switch (type) {
    case OR_F32: return 4;                         /* one IEEE binary32, little-endian */
    case OR_Q8_0: return 2 + 32;                   /* f16 d, int8 q[32] */
    case OR_Q4_0: return 2 + 16;                   /* f16 d, 16 bytes of nibbles */
    case OR_Q4_K: return 2 + 2 + 12 + 128;         /* d, dmin, scales[12], qs[128] */
    case OR_Q6_K: return 128 + 64 + 16 + 2;        /* ql, qh, scales[16], d */
    default: return 0;
    }
}

/* Q8_0: value i = d * int8(q[i]).
 * [qwen3] header comment (a block is an f16 scale and 32 int8 values, copied
 * bit-exact) and the WGSL i8at / matmulQ8 kernels (int8 times the f16 scale of
 * its 32-value group). Reading: d occupies bytes 0-1, codes bytes 2..33. */
static void deq_q8_0(const uint8_t *b, double *out)
{
    double d = or_f16(rd16(b));
    for (int i = 0; i < 32; i++)
        out[i] = d * (double)(int8_t)b[2 + i];
}

/* Q4_0: byte j of the 16 nibble bytes holds value j in its low nibble and value
 * j+16 in its high nibble; value = (nibble - 8) * d.
 * [gemma4] WGSL section, the Q4_0 plane comment and q4dot. Reading: d first. */
static void deq_q4_0(const uint8_t *b, double *out)
{
    double d = or_f16(rd16(b));
    for (int j = 0; j < 16; j++) {
        out[j] = d * (double)((b[2 + j] & 15) - 8);
        out[j + 16] = d * (double)((b[2 + j] >> 4) - 8);
    }
}

/* The 12 scale bytes of a Q4_K block hold eight 6-bit scales and eight 6-bit
 * mins.  Sub-blocks 0..3 use the low 6 bits of bytes s and s+4; sub-blocks
 * 4..7 take their low 4 bits from byte s+4 (low / high nibble) and their top 2
 * bits from the top 2 bits of bytes s-4 (scale) and s (min).
 * [bonsai] "dequantizers" section, scaleMinK4. */
static void q4k_scale_min(const uint8_t *S, int s, int *sc, int *mn)
{
    if (s < 4) {
        *sc = S[s] & 63;
        *mn = S[s + 4] & 63;
    } else {
        *sc = (S[s + 4] & 15) | ((S[s - 4] >> 6) << 4);
        *mn = (S[s + 4] >> 4) | ((S[s] >> 6) << 4);
    }
}

/* Q4_K (144 B, 256 values): d, dmin (f16), scales[12], qs[128].  Chunk c of 32
 * qs bytes feeds sub-block 2c with its low nibbles and sub-block 2c+1 with its
 * high nibbles; value = d*sc*q - dmin*m.
 * [bonsai] "dequantizers" section, dequantQ4K. */
static void deq_q4_k(const uint8_t *b, double *out)
{
    double d = or_f16(rd16(b)), dmin = or_f16(rd16(b + 2));
    const uint8_t *S = b + 4, *Q = b + 16;
    for (int c = 0; c < 4; c++) {
        int sc0, m0, sc1, m1;
        q4k_scale_min(S, 2 * c, &sc0, &m0);
        q4k_scale_min(S, 2 * c + 1, &sc1, &m1);
        for (int l = 0; l < 32; l++) {
            out[64 * c + l] = d * sc0 * (double)(Q[32 * c + l] & 15) - dmin * m0;
            out[64 * c + 32 + l] = d * sc1 * (double)(Q[32 * c + l] >> 4) - dmin * m1;
        }
    }
}

/* Q6_K (210 B, 256 values): ql[128], qh[64], int8 scales[16], f16 d at byte
 * 208.  Each half n of 128 values uses ql[64n..], qh[32n..], scales[8n..]; for
 * l in 0..31 the four values at offsets l, l+32, l+64, l+96 take the low nibble
 * of ql[l], low nibble of ql[l+32], high nibble of ql[l], high nibble of
 * ql[l+32] as their low 4 bits and bit pairs 0-1, 2-3, 4-5, 6-7 of qh[l] as
 * their top 2 bits; value = d * scale[l/16 + 2p] * (q - 32) for p = 0..3.
 * [bonsai] "dequantizers" section, dequantQ6K. */
static void deq_q6_k(const uint8_t *b, double *out)
{
    double d = or_f16(rd16(b + 208));
    for (int n = 0; n < 2; n++) {
        const uint8_t *ql = b + 64 * n, *qh = b + 128 + 32 * n;
        const int8_t *sc = (const int8_t *)(b + 192 + 8 * n);
        double *o = out + 128 * n;
        for (int l = 0; l < 32; l++) {
            int i = l / 16;
            int q1 = ((ql[l] & 15) | (((qh[l] >> 0) & 3) << 4)) - 32;
            int q2 = ((ql[l + 32] & 15) | (((qh[l] >> 2) & 3) << 4)) - 32;
            int q3 = ((ql[l] >> 4) | (((qh[l] >> 4) & 3) << 4)) - 32;
            int q4 = ((ql[l + 32] >> 4) | (((qh[l] >> 6) & 3) << 4)) - 32;
            o[l] = d * sc[i + 0] * (double)q1;
            o[l + 32] = d * sc[i + 2] * (double)q2;
            o[l + 64] = d * sc[i + 4] * (double)q3;
            o[l + 96] = d * sc[i + 6] * (double)q4;
        }
    }
}

/* F32: the 4 bytes are the value's IEEE binary32 pattern, low byte first. */
static void deq_f32(const uint8_t *b, double *out)
{
    float f;
    memcpy(&f, b, 4);
    out[0] = (double)f;
}

static int deq_block(int type, const uint8_t *b, double *out)
{
    switch (type) {
    case OR_F32: deq_f32(b, out); return 0;
    case OR_Q8_0: deq_q8_0(b, out); return 0;
    case OR_Q4_0: deq_q4_0(b, out); return 0;
    case OR_Q4_K: deq_q4_k(b, out); return 0;
    case OR_Q6_K: deq_q6_k(b, out); return 0;
    default: return -1;
    }
}

/* Dequantize n consecutive values (n a multiple of the block size). */
int or_dequant(int type, const uint8_t *blocks, int64_t n, double *out)
{
    int qk = or_block_values(type), bb = or_block_bytes(type);
    if (!qk || n % qk) return -1;
    for (int64_t b = 0; b < n / qk; b++)
        if (deq_block(type, blocks + b * bb, out + b * qk)) return -1;
    return 0;
}

/* ----------------------------------------------------- Q6_K planes ---- */
/* The aligned device layout of Q6_K ([gemma4] q6kPlanes: at load the
 * 210-byte blocks, which sit at 2-byte alignment, are split into planes of
 * ql, qh, scales and d).  Here n blocks become four planes, one after another
 * in one buffer of 210 n bytes:
 *   ql [n][128] at 0, qh [n][64] at 128 n, scales [n][16] at 192 n,
 *   d [n] at 208 n as the block's own two f16 bytes
 * (the page widens d to f32; kept in f16 here, the planes hold the blocks'
 * bytes and nothing more).  A permutation of the bytes; or_q6k_unplanes is
 * its inverse. */
int or_q6k_planes(const uint8_t *blocks, int64_t n, uint8_t *planes)
{
    if (n < 0) return -1;
    for (int64_t b = 0; b < n; b++) {
        const uint8_t *s = blocks + 210 * b;
        memcpy(planes + 128 * b, s, 128);
        memcpy(planes + 128 * n + 64 * b, s + 128, 64);
        memcpy(planes + 192 * n + 16 * b, s + 192, 16);
        memcpy(planes + 208 * n + 2 * b, s + 208, 2);
    }
    return 0;
}

int or_q6k_unplanes(const uint8_t *planes, int64_t n, uint8_t *blocks)
{
    if (n < 0) return -1;
    for (int64_t b = 0; b < n; b++) {
        uint8_t *d = blocks + 210 * b;
        memcpy(d, planes + 128 * b, 128);
        memcpy(d + 128, planes + 128 * n + 64 * b, 64);
        memcpy(d + 192, planes + 192 * n + 16 * b, 16);
        memcpy(d + 208, planes + 208 * n + 2 * b, 2);
    }
    return 0;
}

/* ----------------------------------------------------- Q8_0 planes ---- */
/* The Q8_0 device layout the pages' engines use: the codes in a plane of
 * their own and the scales in another ([qwen3] WGSL i8at reads value e as
 * byte e & 3 of word e >> 2 of the code plane, scaled by the f16 of group
 * e >> 5).  n blocks become one buffer of 34 n bytes: the codes [n][32]
 * (int8) at 0, then the scales d [n] (f16 bytes) at 32 n.  A permutation of
 * the bytes; or_q8_0_unplanes is its inverse. */
int or_q8_0_planes(const uint8_t *blocks, int64_t n, uint8_t *planes)
{
    if (n < 0) return -1;
    for (int64_t b = 0; b < n; b++) {
        const uint8_t *s = blocks + 34 * b;
        memcpy(planes + 32 * n + 2 * b, s, 2);
        memcpy(planes + 32 * b, s + 2, 32);
    }
    return 0;
}

int or_q8_0_unplanes(const uint8_t *planes, int64_t n, uint8_t *blocks)
{
    if (n < 0) return -1;
    for (int64_t b = 0; b < n; b++) {
        uint8_t *d = blocks + 34 * b;
        memcpy(d, planes + 32 * n + 2 * b, 2);
        memcpy(d + 2, planes + 32 * b, 32);
    }
    return 0;
}

/* ------------------------------------------------------------ GEMV ---- */
/* y[t][r] = sum_c W[r][c] * x[t][c] and A[t][r] = sum_c |W[r][c] * x[t][c]|,
 * for the rows listed in row_idx (all rows when row_idx is NULL).  W is
 * row-major in whole blocks: row r starts at byte r * (cols/QK) * block_bytes.
 * The pages' GEMV kernels ([qwen3] WGSL matmulQ8, [gemma4] matmulQ4 and
 * matmulQ6K, [bonsai] packed-weight GEMMs) all compute this sum. */
static int gemv_impl(int type, const uint8_t *W, const float *x, int64_t rows,
                     int64_t cols, int ntok, const int64_t *row_idx, int64_t n_idx,
                     double *y, double *A)
{
    int qk = or_block_values(type), bb = or_block_bytes(type);
    if (!qk || cols <= 0 || cols % qk || ntok <= 0) return -1;
    int64_t row_bytes = (cols / qk) * bb;
    int64_t nout = row_idx ? n_idx : rows;
    int bad = 0;
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)cols);
        if (!w) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(static)
        for (int64_t i = 0; i < nout; i++) {
            if (!w) continue;
            int64_t r = row_idx ? row_idx[i] : i;
            if (r < 0 || r >= rows) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            or_dequant(type, W + r * row_bytes, cols, w);
            for (int t = 0; t < ntok; t++) {
                const float *xt = x + (int64_t)t * cols;
                double s = 0.0, a = 0.0;
                for (int64_t c = 0; c < cols; c++) {
                    double p = w[c] * (double)xt[c];
                    s += p;
                    a += fabs(p);
                }
                y[(int64_t)t * nout + i] = s;
                if (A) A[(int64_t)t * nout + i] = a;
            }
        }
        free(w);
    }
    return bad ? -1 : 0;
}

int or_gemv(int type, const uint8_t *W, const float *x, int64_t rows, int64_t cols,
            int ntok, double *y, double *A)
{
    return gemv_impl(type, W, x, rows, cols, ntok, NULL, 0, y, A);
}

/* Same sum for a sample of rows; y and A are [ntok][n_idx]. */
int or_gemv_rows(int type, const uint8_t *W, const float *x, int64_t rows, int64_t cols,
                 int ntok, const int64_t *row_idx, int64_t n_idx, double *y, double *A)
{
    if (!row_idx) return -1;
    return gemv_impl(type, W, x, rows, cols, ntok, row_idx, n_idx, y, A);
}

/* Same sum with an f64 input vector (used for chained stages fed from the
 * oracle's own f64 intermediates). */
int or_gemv_f64(int type, const uint8_t *W, const double *x, int64_t rows, int64_t cols,
                double *y, double *A)
{
    int qk = or_block_values(type), bb = or_block_bytes(type);
    if (!qk || cols <= 0 || cols % qk) return -1;
    int64_t row_bytes = (cols / qk) * bb;
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)cols);
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; r++) {
            if (!w) continue;
            or_dequant(type, W + r * row_bytes, cols, w);
            double s = 0.0, a = 0.0;
            for (int64_t c = 0; c < cols; c++) {
                double p = w[c] * x[c];
                s += p;
                a += fabs(p);
            }
            y[r] = s;
            if (A) A[r] = a;
        }
        free(w);
    }
    return 0;
}

/* ------------------------------------------------------ activations ---- */
/* SiLU(g) = g / (1 + e^-g).  [qwen3] WGSL siluMulMoe; [dense] siluMul. */
double or_silu(double g) { return g / (1.0 + exp(-g)); }

/* GELU, tanh form, with the tanh argument clamped to [-10, 10]:
 * 0.5 g (1 + tanh(clamp(0.7978845608 g (1 + 0.044715 g^2), -10, 10))).
 * [gemma4] WGSL section, the GELU / tanhc helpers and geglu. */
double or_gelu_tanh(double g)
{
    double u = 0.7978845608 * g * (1.0 + 0.044715 * g * g);
    if (u < -10.0) u = -10.0;
    if (u > 10.0) u = 10.0;
    return 0.5 * g * (1.0 + tanh(u));
}

static double act_fn(int act, double g)
{
    return act == OR_ACT_GELU_TANH ? or_gelu_tanh(g) : or_silu(g);
}

/* act[f] = act_fn(gu[f]) * gu[F + f] for one [gate F | up F] vector.
 * [dense] siluMul, [qwen3] siluMulMoe, [gemma4] geglu. */
void or_glu(int act, const double *gu, int64_t F, double *out)
{
    for (int64_t f = 0; f < F; f++) out[f] = act_fn(act, gu[f]) * gu[F + f];
}

/* Same from f32 inputs (a stage fed with a GPU intermediate). */
void or_glu_f32(int act, const float *gu, int64_t F, double *out)
{
    for (int64_t f = 0; f < F; f++)
        out[f] = act_fn(act, (double)gu[f]) * (double)gu[F + f];
}

/* ------------------------------------------------------------ router ---- */
/* Per token: the k experts with the largest logits, ties to the lower index,
 * in pick order; weights renormalised over the picks:
 * w_j = exp(l_j - lmax) / sum_{i in picks} exp(l_i - lmax).
 * [qwen3] WGSL topk (softmax over the logits, k rounds of argmax with ties to
 * the lowest index, division by the sum of the picked probabilities).  Ranking
 * the logits is the same order as ranking exact probabilities, and the full
 * softmax denominator cancels in the renormalised weights. */
/* Logit a ranks above logit b in the pick order: the larger number; a NaN
 * ranks below every number and two NaNs (or equal numbers, -0 and +0
 * included) leave the order to the index.  The pages' kernel softmaxes
 * finite logits only and says nothing about NaN; this reading never prefers
 * a NaN to a number. */
static int ranks_above(float a, float b)
{
    if (isnan(a)) return 0;
    if (isnan(b)) return 1;
    return a > b;
}

int or_router_topk(const float *logits, int E, int k, int ntok, int32_t *ids, double *w)
{
    if (E <= 0 || k <= 0 || k > E || ntok <= 0) return -1;
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
    if (!taken) return -1;
    for (int t = 0; t < ntok; t++) {
        const float *l = logits + (int64_t)t * E;
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; j++) {
            int best = -1;
            for (int e = 0; e < E; e++) {
                if (taken[e]) continue;
                if (best < 0 || ranks_above(l[e], l[best])) best = e;   /* strict: ties keep lower index */
            }
            taken[best] = 1;
            ids[t * k + j] = best;
        }
        double lmax = (double)l[ids[t * k]];
        double s = 0.0;
        for (int j = 0; j < k; j++) s += exp((double)l[ids[t * k + j]] - lmax);
        for (int j = 0; j < k; j++) w[t * k + j] = exp((double)l[ids[t * k + j]] - lmax) / s;
    }
    free(taken);
    return 0;
}

/* --------------------------------------------------------------- MoE ---- */
/* One routed-expert FFN over ntok tokens.
 *   ids, c  = router(logits[t])                          (or_router_topk)
 *   slot_j  = slots[ids_j]; a token with an absent pick (slot < 0) is skipped
 *   gu_j    = W_gu[slot_j] . x[t]          (2F rows, gate rows first)
 *   a_j     = act(gu_j[0:F]) * gu_j[F:2F]
 *   dn_j    = W_d[slot_j] . a_j            (H rows)
 *   y[t]    = sum_j (dn_j * s[ids_j]) * c_j   (s = 1 when down_scale is NULL)
 * [qwen3] WGSL expertQ8 / siluMulMoe / moeAccum and engine encodeExperts;
 * [gemma4] expertQ4 / geglu / moeSum (the per-expert down scale).
 * Outputs: y and its bound A_y[t][h] = sum_j |c_j s_j| sum_f |W_d[h,f] a_j[f]|
 * ([ntok][H] each), gu ([ntok][k][2F], may be NULL), ids/c ([ntok][k]).
 * Returns the number of tokens skipped for an absent expert, or -1. */
int or_moe_ffn(int type, int act, int64_t H, int64_t F, int E,
               const uint8_t *gate_up, int64_t gu_stride,
               const uint8_t *down, int64_t d_stride, const float *down_scale,
               const float *logits, int k, const int32_t *slots,
               const float *x, int ntok,
               double *y, double *Ay, double *gu_out, int32_t *ids, double *c)
{
    if (or_router_topk(logits, E, k, ntok, ids, c)) return -1;
    double *gu = (double *)malloc(sizeof(double) * (size_t)(2 * F));
    double *a = (double *)malloc(sizeof(double) * (size_t)F);
    double *dn = (double *)malloc(sizeof(double) * (size_t)H);
    double *dA = (double *)malloc(sizeof(double) * (size_t)H);
    double *xd = (double *)malloc(sizeof(double) * (size_t)H);
    if (!gu || !a || !dn || !dA || !xd) return -1;
    int skipped = 0;
    for (int t = 0; t < ntok; t++) {
        int absent = 0;
        for (int j = 0; j < k; j++)
            if (slots[ids[t * k + j]] < 0) absent = 1;
        if (absent) { skipped++; continue; }
        double *yt = y + (int64_t)t * H, *At = Ay + (int64_t)t * H;
        for (int64_t h = 0; h < H; h++) { yt[h] = 0.0; At[h] = 0.0; }
        for (int64_t h = 0; h < H; h++) xd[h] = (double)x[(int64_t)t * H + h];
        for (int j = 0; j < k; j++) {
            int e = ids[t * k + j];
            int64_t slot = slots[e];
            double s = down_scale ? (double)down_scale[e] : 1.0;
            or_gemv_f64(type, gate_up + slot * gu_stride, xd, 2 * F, H, gu, NULL);
            if (gu_out)
                memcpy(gu_out + ((int64_t)t * k + j) * 2 * F, gu, sizeof(double) * (size_t)(2 * F));
            or_glu(act, gu, F, a);
            or_gemv_f64(type, down + slot * d_stride, a, H, F, dn, dA);
            double cj = c[t * k + j];
            for (int64_t h = 0; h < H; h++) {
                yt[h] += (dn[h] * s) * cj;
                At[h] += fabs(cj * s) * dA[h];
            }
        }
    }
    free(gu); free(a); free(dn); free(dA); free(xd);
    return skipped;
}

/* The down half of the same FFN fed with a given gate||up stage (an f32
 * intermediate read back from another implementation): per token and pick,
 * a = act(gu[0:F]) * gu[F:2F], dn = W_d[slot] . a, y = sum_j (dn * s) * c_j.
 * gu is [ntok][k][2F]; ids and c come from the caller.  Writes y, A_y and the
 * weighted absolute row sums R[t][h] = sum_j |c_j s_j| sum_f |W_d[h,f]| * eps_f
 * where eps_f = |g_f| * |u_f| (the scale of the activation's rounding error). */
int or_moe_down(int type, int act, int64_t H, int64_t F,
                const uint8_t *down, int64_t d_stride, const float *down_scale,
                const int32_t *slots, const int32_t *ids, const double *c, int k,
                const float *gu, int ntok, double *y, double *Ay, double *R)
{
    double *a = (double *)malloc(sizeof(double) * (size_t)F);
    double *ga = (double *)malloc(sizeof(double) * (size_t)F);
    double *dn = (double *)malloc(sizeof(double) * (size_t)H);
    double *dA = (double *)malloc(sizeof(double) * (size_t)H);
    double *dR = (double *)malloc(sizeof(double) * (size_t)H);
    double *wrow = (double *)malloc(sizeof(double) * (size_t)F);
    if (!a || !ga || !dn || !dA || !dR || !wrow) return -1;
    int qk = or_block_values(type), bb = or_block_bytes(type);
    int64_t row_bytes = (F / qk) * bb;
    for (int t = 0; t < ntok; t++) {
        double *yt = y + (int64_t)t * H, *At = Ay + (int64_t)t * H, *Rt = R + (int64_t)t * H;
        for (int64_t h = 0; h < H; h++) { yt[h] = 0.0; At[h] = 0.0; Rt[h] = 0.0; }
        for (int j = 0; j < k; j++) {
            int e = ids[t * k + j];
            int64_t slot = slots[e];
            double s = down_scale ? (double)down_scale[e] : 1.0;
            const float *g = gu + ((int64_t)t * k + j) * 2 * F;
            or_glu_f32(act, g, F, a);
            for (int64_t f = 0; f < F; f++) ga[f] = fabs((double)g[f] * (double)g[F + f]);
            or_gemv_f64(type, down + slot * d_stride, a, H, F, dn, dA);
            for (int64_t h = 0; h < H; h++) {
                or_dequant(type, down + slot * d_stride + h * row_bytes, F, wrow);
                double r = 0.0;
                for (int64_t f = 0; f < F; f++) r += fabs(wrow[f]) * ga[f];
                dR[h] = r;
            }
            double cj = c[t * k + j];
            for (int64_t h = 0; h < H; h++) {
                yt[h] += (dn[h] * s) * cj;
                At[h] += fabs(cj * s) * dA[h];
                Rt[h] += fabs(cj * s) * dR[h];
            }
        }
    }
    free(a); free(ga); free(dn); free(dA); free(dR); free(wrow);
    return 0;
}

/* ------------------------------------------------ around the MoE step ---- */
/* RMS norm with a scalar factor, per token of n values:
 *   r = 1 / sqrt(sum_i x_i^2 / n + eps),   y_i = ((x_i * r) * k) * w_i.
 * [qwen3] WGSL rmsnorm (k = 1) and [gemma4] rmsnormK (k = 1/sqrt(H) and the
 * router's scale vector as w: the router's input).  In f64 from f32 inputs. */
int or_rmsnorm(const float *x, const float *w, int64_t n, int ntok, double eps, double k, double *y)
{
    if (n <= 0 || ntok <= 0) return -1;
    for (int t = 0; t < ntok; t++) {
        const float *xt = x + (int64_t)t * n;
        double ss = 0.0;
        for (int64_t i = 0; i < n; i++) ss += (double)xt[i] * (double)xt[i];
        double r = 1.0 / sqrt(ss / (double)n + eps);
        for (int64_t i = 0; i < n; i++) y[(int64_t)t * n + i] = (((double)xt[i] * r) * k) * (double)w[i];
    }
    return 0;
}

/* The logistic function 1 / (1 + e^-g).  [qwen35] SIGMOID helper, used on the
 * shared expert's scalar gate logit. */
double or_sigmoid(double g) { return 1.0 / (1.0 + exp(-g)); }

/* The last step of a MoE block with a shared expert, per token:
 *   sg    = sum_c gate_inp[c] * x[c]                 (the scalar gate logit)
 *   y[h]  = (sum_j terms_j[h] + sh[h] * sigmoid(sg)) + resid[h]
 * where terms_j = (dn_j * s_j) * c_j are the routed picks' weighted down
 * outputs, added in pick order, and resid is the residual stream.
 * [qwen35] WGSL moeAccumShared / moeAccumSharedB (routed experts, then the
 * gated shared expert, then the residual) and the engine's shgate binding (an
 * f32 GEMV of one row on the normed input).
 * Inputs f32: terms [ntok][k][H], sh [ntok][H], gate_inp [H], x [ntok][H],
 * resid [ntok][H].  Outputs f64 [ntok][H]: y, and the error scale
 *   A[h] = sum_j |terms_j[h]| + |sh[h]| sigmoid(sg) + |resid[h]|
 *          + |sh[h]| / 4 * sum_c |gate_inp[c] x[c]|
 * (the last term: the logistic slope is at most 1/4, times the scale of the
 * gate logit's own rounding).  sg_out [ntok] may be NULL. */
int or_moe_shared_combine(const float *terms, int k, const float *sh, const float *gate_inp,
                          const float *x, const float *resid, int64_t H, int ntok,
                          double *y, double *A, double *sg_out)
{
    if (H <= 0 || ntok <= 0 || k <= 0) return -1;
    for (int t = 0; t < ntok; t++) {
        const float *xt = x + (int64_t)t * H;
        double sg = 0.0, sa = 0.0;
        for (int64_t c = 0; c < H; c++) {
            double p = (double)gate_inp[c] * (double)xt[c];
            sg += p;
            sa += fabs(p);
        }
        if (sg_out) sg_out[t] = sg;
        double gs = or_sigmoid(sg);
        for (int64_t h = 0; h < H; h++) {
            double acc = 0.0, aa = 0.0;
            for (int j = 0; j < k; j++) {
                double v = (double)terms[((int64_t)t * k + j) * H + h];
                acc += v;
                aa += fabs(v);
            }
            double s = (double)sh[(int64_t)t * H + h], r = (double)resid[(int64_t)t * H + h];
            y[(int64_t)t * H + h] = (acc + s * gs) + r;
            A[(int64_t)t * H + h] = aa + fabs(s) * gs + fabs(r) + fabs(s) * 0.25 * sa;
        }
    }
    return 0;
}

/* Gemma's FFN tail, per token of n values:
 *   m  = rmsnorm(mlp, w1)   (the dense MLP's output, post_ffw_norm_1)
 *   e  = rmsnorm(moe, w2)   (the MoE sum, post_ffw_norm_2)
 *   v  = m + e
 *   x  = ((v * r_v) * w + x) * os          r_v = 1 / sqrt(sum v^2 / n + eps)
 * [gemma4] engine encodeExperts (mpost, mpost2) and WGSL postFfn (the last
 * norm, the residual add and the layer's output scalar os).  x is updated in
 * place (f32 in, f64 out as y).  A[i] = |os| ((|m_i| + |e_i|) r_v |w_i| + |x_i|)
 * is the scale of the rounding error of an f32 evaluation. */
int or_post_ffn(const float *mlp, const float *moe, const float *w1, const float *w2,
                const float *w, double os, const float *x, int64_t n, int ntok, double eps,
                double *y, double *A)
{
    if (n <= 0 || ntok <= 0) return -1;
    double *m = (double *)malloc(sizeof(double) * (size_t)n);
    double *e = (double *)malloc(sizeof(double) * (size_t)n);
    if (!m || !e) { free(m); free(e); return -1; }
    for (int t = 0; t < ntok; t++) {
        int64_t o = (int64_t)t * n;
        or_rmsnorm(mlp + o, w1, n, 1, eps, 1.0, m);
        or_rmsnorm(moe + o, w2, n, 1, eps, 1.0, e);
        double ss = 0.0;
        for (int64_t i = 0; i < n; i++) ss += (m[i] + e[i]) * (m[i] + e[i]);
        double r = 1.0 / sqrt(ss / (double)n + eps);
        for (int64_t i = 0; i < n; i++) {
            y[o + i] = (((m[i] + e[i]) * r) * (double)w[i] + (double)x[o + i]) * os;
            A[o + i] = fabs(os) * ((fabs(m[i]) + fabs(e[i])) * r * fabs((double)w[i]) + fabs((double)x[o + i]));
        }
    }
    free(m); free(e);
    return 0;
}

/* --------------------------------------------------- embedding and head ---- */
/* Embedding rows of a quantized table, scaled:
 *   out[t][c] = f32(f32(W[tok_t][c]) * scale)
 * each value first rounded to the f32 nearest its exact value (exact for
 * Q8_0, Q4_0, Q6_K and F32), then multiplied by scale in f32.
 * [qwen3] WGSL embedQ8 (scale 1) and [gemma4] embedQ6K (its scale uniform).
 * Returns -1 for a token outside [0, rows). */
int or_embed(int type, const uint8_t *W, int64_t rows, int64_t cols, const int32_t *tok, int ntok,
             float scale, float *out)
{
    int qk = or_block_values(type), bb = or_block_bytes(type);
    if (!qk || cols <= 0 || cols % qk || ntok <= 0) return -1;
    int64_t row_bytes = (cols / qk) * bb;
    double *w = (double *)malloc(sizeof(double) * (size_t)cols);
    if (!w) return -1;
    for (int t = 0; t < ntok; t++) {
        if (tok[t] < 0 || tok[t] >= rows) { free(w); return -1; }
        or_dequant(type, W + (int64_t)tok[t] * row_bytes, cols, w);
        for (int64_t c = 0; c < cols; c++) {
            float v = (float)w[c];
            out[(int64_t)t * cols + c] = (float)((double)v * (double)scale);
        }
    }
    free(w);
    return 0;
}

/* Final logit soft cap: l = tanh(clamp(l * inv, -10, 10)) * cap, inv the f32
 * nearest 1/cap.  [gemma4] WGSL softcap with the tanhc clamp.  f64 out. */
int or_softcap(const float *l, int64_t n, float cap, double *out)
{
    if (n < 0 || !(cap > 0.0f)) return -1;
    float inv = (float)(1.0 / (double)cap);
    for (int64_t i = 0; i < n; i++) {
        double a = (double)l[i] * (double)inv;
        if (a < -10.0) a = -10.0;
        if (a > 10.0) a = 10.0;
        out[i] = tanh(a) * (double)cap;
    }
    return 0;
}

/* Greedy pick per token: the index of the largest value, ties to the lowest
 * index; NaN entries never win; a row with no number gives 0.
 * [qwen3] WGSL argmax (strict greater-than while scanning, the lower index on
 * equal values while reducing). */
int or_argmax(const float *l, int64_t n, int ntok, int32_t *idx)
{
    if (n <= 0 || ntok <= 0) return -1;
    for (int t = 0; t < ntok; t++) {
        const float *lt = l + (int64_t)t * n;
        int64_t best = -1;
        for (int64_t i = 0; i < n; i++) {
            if (lt[i] != lt[i]) continue;   /* NaN */
            if (best < 0 || lt[i] > lt[best]) best = i;
        }
        idx[t] = (int32_t)(best < 0 ? 0 : best);
    }
    return 0;
}

/* Host threads the parallel loops above use (n > 0 sets them); returns the
 * count in force.  Timing only: no result depends on it. */
int or_set_threads(int n)
{
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
}

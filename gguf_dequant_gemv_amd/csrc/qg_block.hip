// qg_block.hip -- the steps on either side of the routed experts (gfx950):
// RMS norm, the f32 GEMV of the router and shared-expert gate weights, the
// shared-expert combine with the residual, Gemma's FFN tail, embedding rows,
// and the logit soft cap with the greedy pick.
#include "../../include/qgemv.h"
#include "qg_kernels.h"
#include "qg_block.h"

namespace qg {

// Sum over a workgroup of NW waves, returned to every thread.  The additions
// run in a fixed order (DPP inside each wave, then the wave sums in wave
// order), so every workgroup that reduces the same data gets the same bits.
template <int NW>
QG_DEV float block_sum(float v, float *s_red) {
    v = wave_sum(v);
    __syncthreads();   // s_red may still be read by an earlier call
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
    __syncthreads();
    float s = s_red[0];
#pragma unroll
    for (int i = 1; i < NW; i++) s += s_red[i];
    return s;
}

QG_DEV float rms_factor(float ss, int64_t n, float eps) { return 1.0f / sqrtf(ss / (float)n + eps); }

// Loads go out in batches of LB per thread before any of them is used, so a
// short vector costs one memory round trip per pass instead of one per element.
constexpr int LB = 16;

// ------------------------------------------------------------- RMS norm ----
// One workgroup per token: r = 1/sqrt(mean x^2 + eps), y = ((x r) k) w.  The
// qwen3_moe_ssd.js rmsnorm kernel (k = 1) and gemma4_moe_ssd.js rmsnormK (the
// router input: k = 1/sqrt(H), w the router's scale vector).  Every x is read
// for the sum before any y is written, so y may be x.
QG_DEV void k_rmsnorm_row(const float *xt, const float *w, float *yt, int64_t n, float eps, float k) {
    __shared__ float s_red[4];
    if (n <= 256 * LB) {
        // one batch per thread: x and w loaded once, the row's factor and the
        // outputs from registers (same operations, same order)
        const int i0 = threadIdx.x;
        float v[LB], g[LB];
#pragma unroll
        for (int b = 0; b < LB; b++) {
            const bool in = i0 + b * 256 < n;
            v[b] = in ? xt[i0 + b * 256] : 0.0f;
            g[b] = in ? w[i0 + b * 256] : 0.0f;
        }
        float ss = 0.0f;
#pragma unroll
        for (int b = 0; b < LB; b++) ss = fmaf(v[b], v[b], ss);
        const float r = rms_factor(block_sum<4>(ss, s_red), n, eps);
#pragma unroll
        for (int b = 0; b < LB; b++)
            if (i0 + b * 256 < n) yt[i0 + b * 256] = ((v[b] * r) * k) * g[b];
        return;
    }
    float ss = 0.0f;
    for (int64_t i0 = threadIdx.x; i0 < n; i0 += 256 * LB) {
        float v[LB];
#pragma unroll
        for (int b = 0; b < LB; b++) v[b] = i0 + b * 256 < n ? xt[i0 + b * 256] : 0.0f;
#pragma unroll
        for (int b = 0; b < LB; b++) ss = fmaf(v[b], v[b], ss);
    }
    const float r = rms_factor(block_sum<4>(ss, s_red), n, eps);
    for (int64_t i0 = threadIdx.x; i0 < n; i0 += 256 * LB) {
        float v[LB], g[LB];
#pragma unroll
        for (int b = 0; b < LB; b++) {
            const bool in = i0 + b * 256 < n;
            v[b] = in ? xt[i0 + b * 256] : 0.0f;
            g[b] = in ? w[i0 + b * 256] : 0.0f;
        }
#pragma unroll
        for (int b = 0; b < LB; b++)
            if (i0 + b * 256 < n) yt[i0 + b * 256] = ((v[b] * r) * k) * g[b];
    }
}

__global__ __launch_bounds__(256) void k_rmsnorm(const float *x, const float *w, float *y, int64_t n, float eps,
                                                 float k) {
    k_rmsnorm_row(x + (int64_t)blockIdx.x * n, w, y + (int64_t)blockIdx.x * n, n, eps, k);
}

// The same norms of one row into several outputs: workgroup (token, o)
// computes the row's factor as k_rmsnorm does and writes output o.
struct NormOuts {
    const float *w[QG_MAX_NORMS];
    float *y[QG_MAX_NORMS];
    float k[QG_MAX_NORMS];
};

__global__ __launch_bounds__(256) void k_rmsnorm_multi(const float *x, int64_t n, float eps, NormOuts o) {
    const int j = blockIdx.y;
    k_rmsnorm_row(x + (int64_t)blockIdx.x * n, o.w[j], o.y[j] + (int64_t)blockIdx.x * n, n, eps, o.k[j]);
}

// --------------------------------------------- norms + the router GEMV ----
// One launch for a block's input norms and its f32 router: every workgroup
// finds the tokens' RMS factors r_t (the sums of squares taken as k_rmsnorm
// takes them), writes its slice of each output norm y_o = ((x r_t) k_o) w_o,
// and its waves compute router rows e against the router's input norm
// ((x r_t) rk) rw, formed on the fly, with k_gemv_f32's loads and order
// (WPR waves to a row as there): the logits and norms equal the separate
// launches' bit for bit.
template <int NT, bool V4, int WPR>
__global__ __launch_bounds__(256) void k_norm_gemv_f32(const float *x, int64_t n, int ntok, float eps,
                                                       const float *rw, float rk, const float *W, int64_t rows,
                                                       float *y, NormOuts o, int nout) {
    static_assert(WPR == 1 || (WPR == 4 && V4 && NT > 1), "rows shared by the 4 waves only on the float4 path");
    __shared__ float s_red[4][NT];
    __shared__ float s_r[NT];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    constexpr int B = NT == 1 ? 8 : (NT <= 4 ? 4 : 2);
    // this wave's router row, and its share of the row's column passes
    const int64_t r = WPR == 1 ? (int64_t)blockIdx.x * 4 + wave : (int64_t)blockIdx.x;
    const int part = WPR == 1 ? 0 : wave;
    const float *wr = W + (r < rows ? r : 0) * n;
    // One token whose x is one batch: x's loads, then the first batch of the
    // router row and its norm gains, then the sums, which wait for x alone
    // (loads return in order), so the row's round trip overlaps the norm.
    // Every load here is unconditional (clamped addresses, values selected
    // after), so the count of loads in flight is exact.
    const bool early = NT == 1 && V4 && n <= 256 * LB;
    [[maybe_unused]] float4 wv0[B], gv0[B];
    if (early) {
        float v[LB];
#pragma unroll
        for (int b = 0; b < LB; b++) {
            const int64_t i = (int64_t)threadIdx.x + b * 256;
            const float xv = x[i < n ? i : n - 1];
            v[b] = i < n ? xv : 0.0f;
        }
        if constexpr (V4) {
#pragma unroll
            for (int b = 0; b < B; b++) {
                const int64_t c = min((int64_t)(4 * lane + 256 * b), n - 4);
                wv0[b] = *(const float4 *)(wr + c);
                gv0[b] = *(const float4 *)(rw + c);
            }
        }
        float ss = 0.0f;
#pragma unroll
        for (int b = 0; b < LB; b++) ss = fmaf(v[b], v[b], ss);
        ss = wave_sum(ss);
        if (lane == 0) s_red[wave][0] = ss;
    } else {
        // the tokens' sums of squares: thread i's values i, i + 256, ... in
        // order, TB tokens' loads out together (clamped token and index,
        // values selected after)
        constexpr int TB = NT < 8 ? NT : 8;
        for (int t0 = 0; t0 < ntok; t0 += TB) {
            float ss[TB];
#pragma unroll
            for (int u = 0; u < TB; u++) ss[u] = 0.0f;
            for (int64_t i0 = threadIdx.x; i0 < n; i0 += 256 * LB) {
                float v[TB][LB];
#pragma unroll
                for (int u = 0; u < TB; u++) {
                    const int64_t tt = t0 + u < ntok ? t0 + u : ntok - 1;
#pragma unroll
                    for (int b = 0; b < LB; b++) {
                        const int64_t i = i0 + b * 256;
                        const float xv = x[tt * n + (i < n ? i : n - 1)];
                        v[u][b] = i < n ? xv : 0.0f;
                    }
                }
#pragma unroll
                for (int u = 0; u < TB; u++)
#pragma unroll
                    for (int b = 0; b < LB; b++) ss[u] = fmaf(v[u][b], v[u][b], ss[u]);
            }
#pragma unroll
            for (int u = 0; u < TB; u++) {
                const float s = wave_sum(ss[u]);
                if (lane == 0 && t0 + u < ntok) s_red[wave][t0 + u] = s;
            }
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < ntok) {
        const int t = threadIdx.x;
        float sum = s_red[0][t];
#pragma unroll
        for (int w2 = 1; w2 < 4; w2++) sum += s_red[w2][t];
        s_r[t] = rms_factor(sum, n, eps);
    }
    __syncthreads();
    // this workgroup's slice of the output norms
    const int64_t chunk = (n + gridDim.x - 1) / gridDim.x;
    const int64_t c_lo = (int64_t)blockIdx.x * chunk, c_hi = min(n, c_lo + chunk);
    if constexpr (NT == 1) {
        for (int j = 0; j < nout; j++)
            for (int64_t c = c_lo + threadIdx.x; c < c_hi; c += 256)
                o.y[j][c] = ((x[c] * s_r[0]) * o.k[j]) * o.w[j][c];
    } else if (nout > 0) {   // a column's loads (every token's x, every output's gain) before its stores
        for (int64_t c = c_lo + threadIdx.x; c < c_hi; c += 256) {
            float xc[NT], wc[QG_MAX_NORMS];
#pragma unroll
            for (int t = 0; t < NT; t++) xc[t] = x[(int64_t)(t < ntok ? t : ntok - 1) * n + c];
#pragma unroll
            for (int j = 0; j < QG_MAX_NORMS; j++) wc[j] = o.w[j < nout ? j : 0][c];
#pragma unroll
            for (int j = 0; j < QG_MAX_NORMS; j++)
#pragma unroll
                for (int t = 0; t < NT; t++)
                    if (j < nout && t < ntok) o.y[j][(int64_t)t * n + c] = ((xc[t] * s_r[t]) * o.k[j]) * wc[j];
        }
    }
    // router row r of wave w
    if (r >= rows) return;
    float rt[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) rt[t] = t < ntok ? s_r[t] : 0.0f;
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t] = 0.0f;
    auto xin = [&](float xv, int t, float g) { return ((xv * rt[t]) * rk) * g; };
    if constexpr (V4 && NT == 1) {
        for (int64_t c0 = 4 * lane; c0 < n; c0 += 256 * B) {
            float4 wv[B], gv[B];
            if (early && c0 == 4 * lane) {   // the first batch, loaded before the norm
#pragma unroll
                for (int b = 0; b < B; b++) {
                    const bool in = c0 + 256 * b < n;
                    wv[b] = in ? wv0[b] : make_float4(0, 0, 0, 0);
                    gv[b] = in ? gv0[b] : make_float4(0, 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int b = 0; b < B; b++) {
                    const bool in = c0 + 256 * b < n;
                    wv[b] = in ? *(const float4 *)(wr + c0 + 256 * b) : make_float4(0, 0, 0, 0);
                    gv[b] = in ? *(const float4 *)(rw + c0 + 256 * b) : make_float4(0, 0, 0, 0);
                }
            }
            float4 xv[B];
#pragma unroll
            for (int b = 0; b < B; b++)
                xv[b] = c0 + 256 * b < n ? *(const float4 *)(x + c0 + 256 * b) : make_float4(0, 0, 0, 0);
#pragma unroll
            for (int b = 0; b < B; b++) {
                acc[0] = fmaf(wv[b].x, xin(xv[b].x, 0, gv[b].x), acc[0]);
                acc[0] = fmaf(wv[b].y, xin(xv[b].y, 0, gv[b].y), acc[0]);
                acc[0] = fmaf(wv[b].z, xin(xv[b].z, 0, gv[b].z), acc[0]);
                acc[0] = fmaf(wv[b].w, xin(xv[b].w, 0, gv[b].w), acc[0]);
            }
        }
    } else if constexpr (V4) {
        // several tokens: loads unconditional as in k_gemv_f32 (clamped token
        // and column, values selected after), so a pass's x loads go out together
        const float4 z4 = make_float4(0, 0, 0, 0);
        for (int64_t c0 = 4 * lane + (int64_t)part * 256 * B; c0 < n; c0 += 256 * B * WPR) {
            float4 wv[B], gv[B];
            {
#pragma unroll
                for (int b = 0; b < B; b++) {
                    const int64_t c = c0 + 256 * b;
                    const float4 w4 = *(const float4 *)(wr + (c < n ? c : n - 4));
                    const float4 g4 = *(const float4 *)(rw + (c < n ? c : n - 4));
                    wv[b] = c < n ? w4 : z4;
                    gv[b] = c < n ? g4 : z4;
                }
            }
            float4 xv[NT][B];
#pragma unroll
            for (int t = 0; t < NT; t++) {
                const int64_t tt = t < ntok ? t : ntok - 1;
#pragma unroll
                for (int b = 0; b < B; b++) {
                    const int64_t c = c0 + 256 * b;
                    const float4 v = *(const float4 *)(x + tt * n + (c < n ? c : n - 4));
                    xv[t][b] = c < n ? v : z4;
                }
            }
#pragma unroll
            for (int t = 0; t < NT; t++) {
#pragma unroll
                for (int b = 0; b < B; b++) {
                    acc[t] = fmaf(wv[b].x, xin(xv[t][b].x, t, gv[b].x), acc[t]);
                    acc[t] = fmaf(wv[b].y, xin(xv[t][b].y, t, gv[b].y), acc[t]);
                    acc[t] = fmaf(wv[b].z, xin(xv[t][b].z, t, gv[b].z), acc[t]);
                    acc[t] = fmaf(wv[b].w, xin(xv[t][b].w, t, gv[b].w), acc[t]);
                }
            }
        }
    } else {
        for (int64_t c0 = lane; c0 < n; c0 += 64 * B) {
            float wv[B], gv[B];
#pragma unroll
            for (int b = 0; b < B; b++) {
                const bool in = c0 + 64 * b < n;
                wv[b] = in ? wr[c0 + 64 * b] : 0.0f;
                gv[b] = in ? rw[c0 + 64 * b] : 0.0f;
            }
#pragma unroll
            for (int t = 0; t < NT; t++) {
                if (t < ntok) {
#pragma unroll
                    for (int b = 0; b < B; b++)
                        if (c0 + 64 * b < n) acc[t] = fmaf(wv[b], xin(x[t * n + c0 + 64 * b], t, gv[b]), acc[t]);
                }
            }
        }
    }
    if constexpr (WPR == 1) {
#pragma unroll
        for (int t = 0; t < NT; t++) {
            if (t < ntok) {
                const float sum = wave_sum(acc[t]);
                if (lane == 0) y[t * rows + r] = sum;
            }
        }
    } else {   // the waves' sums in wave order, as k_gemv_f32 adds them (s_red is free again)
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const float s = wave_sum(acc[t]);
            if (lane == 0) s_red[wave][t] = s;
        }
        __syncthreads();
        if ((int)threadIdx.x < ntok) {
            const int t = threadIdx.x;
            float s = s_red[0][t];
#pragma unroll
            for (int w = 1; w < WPR; w++) s += s_red[w][t];
            y[t * rows + r] = s;
        }
    }
}

// ------------------------------------------------------------ f32 GEMV ----
// y[t][r] = sum_c W[r][c] x[t][c] for f32 weights (the router's logits and the
// shared expert's gate: qwen3_moe_ssd.js matmulF32).  One wave per row; each
// lane takes 4 consecutive columns per step (V4: 16-byte loads), the row's
// values are loaded once and used for all NT tokens, and the lane partials are
// summed across the wave.  With WPR = 4 the four waves of a workgroup share
// one row (wave w takes the column passes w, w + 4, ...), which puts four
// times the workgroups on the chip when the rows are few and each pass is
// long (16 tokens' x loads); their sums are added in wave order through LDS.
template <int NT, bool V4, int WPR>
__global__ __launch_bounds__(256) void k_gemv_f32(const float *W, const float *x, float *y, int64_t rows,
                                                  int64_t cols, int ntok) {
    static_assert(WPR == 1 || (WPR == 4 && V4), "rows shared by the 4 waves only on the float4 path");
    // weight loads in flight per lane: all of a 2048-wide row for one token,
    // fewer as the token count (and the x loads per weight) grows
    constexpr int B = NT == 1 ? 8 : (NT <= 4 ? 4 : 2);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t r = WPR == 1 ? (int64_t)blockIdx.x * 4 + wave : (int64_t)blockIdx.x;
    const int part = WPR == 1 ? 0 : wave;
    if (r >= rows) return;   // the whole wave (WPR 4: workgroup) leaves; nothing below waits on it
    const float *wr = W + r * cols;
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t] = 0.0f;
    if constexpr (V4) {
        // every load unconditional (token slots past ntok read the last
        // token, columns past the row its last float4; their values are
        // replaced by zeros or dropped), so the tokens' x loads of a pass go
        // out together instead of one token's round trip after another
        const float4 z4 = make_float4(0, 0, 0, 0);
        for (int64_t c0 = 4 * lane + (int64_t)part * 256 * B; c0 < cols; c0 += 256 * B * WPR) {
            float4 wv[B];
#pragma unroll
            for (int b = 0; b < B; b++) {
                const int64_t c = c0 + 256 * b;
                const float4 v = *(const float4 *)(wr + (c < cols ? c : cols - 4));
                wv[b] = c < cols ? v : z4;
            }
            float4 xv[NT][B];
#pragma unroll
            for (int t = 0; t < NT; t++) {
                const int64_t tt = t < ntok ? t : ntok - 1;
#pragma unroll
                for (int b = 0; b < B; b++) {
                    const int64_t c = c0 + 256 * b;
                    const float4 v = *(const float4 *)(x + tt * cols + (c < cols ? c : cols - 4));
                    xv[t][b] = c < cols ? v : z4;
                }
            }
#pragma unroll
            for (int t = 0; t < NT; t++) {
#pragma unroll
                for (int b = 0; b < B; b++) {
                    acc[t] = fmaf(wv[b].x, xv[t][b].x, acc[t]);
                    acc[t] = fmaf(wv[b].y, xv[t][b].y, acc[t]);
                    acc[t] = fmaf(wv[b].z, xv[t][b].z, acc[t]);
                    acc[t] = fmaf(wv[b].w, xv[t][b].w, acc[t]);
                }
            }
        }
    } else {
        for (int64_t c0 = lane; c0 < cols; c0 += 64 * B) {
            float wv[B];
#pragma unroll
            for (int b = 0; b < B; b++) wv[b] = c0 + 64 * b < cols ? wr[c0 + 64 * b] : 0.0f;
#pragma unroll
            for (int t = 0; t < NT; t++) {
                if (t < ntok) {
#pragma unroll
                    for (int b = 0; b < B; b++)
                        if (c0 + 64 * b < cols) acc[t] = fmaf(wv[b], x[t * cols + c0 + 64 * b], acc[t]);
                }
            }
        }
    }
    if constexpr (WPR == 1) {
#pragma unroll
        for (int t = 0; t < NT; t++) {
            if (t < ntok) {
                const float s = wave_sum(acc[t]);
                if (lane == 0) y[t * rows + r] = s;
            }
        }
    } else {
        __shared__ float s_part[WPR][NT];
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const float s = wave_sum(acc[t]);
            if (lane == 0) s_part[wave][t] = s;
        }
        __syncthreads();
        if ((int)threadIdx.x < ntok) {
            const int t = threadIdx.x;
            float s = s_part[0][t];
#pragma unroll
            for (int w = 1; w < WPR; w++) s += s_part[w][t];
            y[t * rows + r] = s;
        }
    }
}

// ----------------------------------------------- shared-expert combine ----
// Per token t and hidden index h:
//   sg   = gate_inp . x[t]                    (the shared expert's gate logit)
//   y[h] = (sum_j terms_j[h] + sh[h] sigmoid(sg)) + resid[h]      -> resid[h]
// terms_j = (dn_j s_j) c_j come from the expert down launch; added in pick
// order.  qwen35_moe_ssd.js moeAccumShared: routed experts, the gated shared
// expert, then the residual.  Each workgroup of token t reduces the same gate
// products in the same order, so all of them use the same sg.
__global__ __launch_bounds__(256) void k_combine_shared(const float *dn, const int32_t *rt_valid, const float *sh,
                                                        const float *gate_inp, const float *x, float *resid,
                                                        int64_t H, int k) {
    __shared__ float s_red[4];
    const int t = blockIdx.y;
    const int64_t h = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool mine = h < H;
    const int64_t o = (int64_t)t * H + (mine ? h : 0);
    // this thread's operands first, so their loads overlap the gate's
    const float *q = dn + (int64_t)t * k * H + (mine ? h : 0);
    float v[QG_MAX_TOPK];
#pragma unroll
    for (int j = 0; j < QG_MAX_TOPK; j++) v[j] = j < k ? q[(int64_t)j * H] : 0.0f;
    const float s_o = sh[o], r_o = resid[o];
    const int ok = rt_valid[t];
    const float *xt = x + (int64_t)t * H;
    float p = 0.0f;
    for (int64_t c0 = threadIdx.x; c0 < H; c0 += 256 * LB) {
        float gv[LB], xv[LB];
#pragma unroll
        for (int b = 0; b < LB; b++) {
            const bool in = c0 + b * 256 < H;
            gv[b] = in ? gate_inp[c0 + b * 256] : 0.0f;
            xv[b] = in ? xt[c0 + b * 256] : 0.0f;
        }
#pragma unroll
        for (int b = 0; b < LB; b++) p = fmaf(gv[b], xv[b], p);
    }
    const float sg = block_sum<4>(p, s_red);
    const float gs = 1.0f / (1.0f + expf(-sg));
    if (!mine) return;
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < QG_MAX_TOPK; j++)
        if (j < k) acc += v[j];
    if (ok) resid[o] = (acc + s_o * gs) + r_o;
}

// ----------------------------------------------------- Gemma's FFN tail ----
// One workgroup per token:
//   m = rmsnorm(mlp) w1,  e = rmsnorm(moe) w2,  v = m + e,
//   x = ((v r_v) w + x) os
// gemma4_moe_ssd.js encodeExperts (post_ffw_norm_1 / _2) and postFfn, in one
// launch: the sums of squares of mlp and moe first, then that of v, then the
// update (v recomputed from the same f32 operations each time).
__global__ __launch_bounds__(256) void k_post_ffn(const float *mlp, const float *moe, const float *w1,
                                                  const float *w2, const float *w, const float *os, float *x,
                                                  int64_t n, float eps) {
    __shared__ float s_red[4];
    const int64_t o = (int64_t)blockIdx.x * n;
    const float *a = mlp + o, *b = moe + o;
    float *xt = x + o;
    if (n <= 256 * LB) {
        // one batch per thread: every operand is loaded once, up front, and
        // the three passes below run on registers (same operations, same order)
        const int i0 = threadIdx.x;
        float va[LB], vb[LB], g1[LB], g2[LB], g[LB], xv[LB];
#pragma unroll
        for (int u = 0; u < LB; u++) {
            const bool in = i0 + u * 256 < n;
            va[u] = in ? a[i0 + u * 256] : 0.0f;
            vb[u] = in ? b[i0 + u * 256] : 0.0f;
            g1[u] = in ? w1[i0 + u * 256] : 0.0f;
            g2[u] = in ? w2[i0 + u * 256] : 0.0f;
            g[u] = in ? w[i0 + u * 256] : 0.0f;
            xv[u] = in ? xt[i0 + u * 256] : 0.0f;
        }
        const float ko = os[0];
        float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
        for (int u = 0; u < LB; u++) {
            s1 = fmaf(va[u], va[u], s1);
            s2 = fmaf(vb[u], vb[u], s2);
        }
        const float r1 = rms_factor(block_sum<4>(s1, s_red), n, eps);
        const float r2 = rms_factor(block_sum<4>(s2, s_red), n, eps);
        float v[LB], s3 = 0.0f;
#pragma unroll
        for (int u = 0; u < LB; u++) {
            v[u] = (va[u] * r1) * g1[u] + (vb[u] * r2) * g2[u];
            s3 = fmaf(v[u], v[u], s3);
        }
        const float r3 = rms_factor(block_sum<4>(s3, s_red), n, eps);
#pragma unroll
        for (int u = 0; u < LB; u++)
            if (i0 + u * 256 < n) xt[i0 + u * 256] = ((v[u] * r3) * g[u] + xv[u]) * ko;
        return;
    }
    float s1 = 0.0f, s2 = 0.0f;
    for (int64_t i0 = threadIdx.x; i0 < n; i0 += 256 * LB) {
        float va[LB], vb[LB];
#pragma unroll
        for (int u = 0; u < LB; u++) {
            const bool in = i0 + u * 256 < n;
            va[u] = in ? a[i0 + u * 256] : 0.0f;
            vb[u] = in ? b[i0 + u * 256] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < LB; u++) {
            s1 = fmaf(va[u], va[u], s1);
            s2 = fmaf(vb[u], vb[u], s2);
        }
    }
    const float r1 = rms_factor(block_sum<4>(s1, s_red), n, eps);
    const float r2 = rms_factor(block_sum<4>(s2, s_red), n, eps);
    // v = m + e, recomputed from the same f32 operations in both passes below
    auto vsum = [&](int64_t i0, float (&v)[LB]) {
        float va[LB], vb[LB], g1[LB], g2[LB];
#pragma unroll
        for (int u = 0; u < LB; u++) {
            const bool in = i0 + u * 256 < n;
            va[u] = in ? a[i0 + u * 256] : 0.0f;
            vb[u] = in ? b[i0 + u * 256] : 0.0f;
            g1[u] = in ? w1[i0 + u * 256] : 0.0f;
            g2[u] = in ? w2[i0 + u * 256] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < LB; u++) v[u] = (va[u] * r1) * g1[u] + (vb[u] * r2) * g2[u];
    };
    float s3 = 0.0f;
    for (int64_t i0 = threadIdx.x; i0 < n; i0 += 256 * LB) {
        float v[LB];
        vsum(i0, v);
#pragma unroll
        for (int u = 0; u < LB; u++) s3 = fmaf(v[u], v[u], s3);
    }
    const float r3 = rms_factor(block_sum<4>(s3, s_red), n, eps);
    const float ko = os[0];
    for (int64_t i0 = threadIdx.x; i0 < n; i0 += 256 * LB) {
        float v[LB], g[LB], xv[LB];
        vsum(i0, v);
#pragma unroll
        for (int u = 0; u < LB; u++) {
            const bool in = i0 + u * 256 < n;
            g[u] = in ? w[i0 + u * 256] : 0.0f;
            xv[u] = in ? xt[i0 + u * 256] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < LB; u++)
            if (i0 + u * 256 < n) xt[i0 + u * 256] = ((v[u] * r3) * g[u] + xv[u]) * ko;
    }
}

// ------------------------------------------------------ embedding rows ----
// out[t][c] = value(W[tokens[t]][c]) * scale, decoded by the same block units
// as the GEMV (qwen3_moe_ssd.js embedQ8, gemma4_moe_ssd.js embedQ6K with its
// scale).  A lane writes 8 values of one block: wave w of the grid takes part
// w % P (values 8p .. 8p+7, P = VALUES / 8 parts a block) of 64 consecutive
// blocks, so the part -- and with it every register index of the decode -- is
// the same across the wave.  A token outside [0, rows) reads nothing and gets
// a row of NaN.
constexpr int EMBED_VALUES = 8;   // values per lane

template <class U, int P>
QG_DEV void embed8(const u32 (&w)[U::ND], float scale, float *o) {
#pragma unroll
    for (int i = 0; i < EMBED_VALUES; i++) o[i] = U::value(w, EMBED_VALUES * P + i) * scale;
}

// the part p (wave-uniform) as a chain of uniform branches to unrolled code
template <class U, int P = 0>
QG_DEV void embed_part(int p, const u32 (&w)[U::ND], float scale, float *o) {
    if constexpr (P < U::VALUES / EMBED_VALUES) {
        if (p == P)
            embed8<U, P>(w, scale, o);
        else
            embed_part<U, P + 1>(p, w, scale, o);
    }
}

// this workgroup's share of row id of token blockIdx.y (the grid as k_embed's)
template <class U>
QG_DEV void embed_row(const uint8_t *W, int64_t rows, int cols, int64_t row_bytes, int32_t id, float scale,
                      float *out) {
    constexpr int NP = U::VALUES / EMBED_VALUES;
    const int nbr = cols / U::VALUES;
    const int gw = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    const int p = gw % NP;
    const int b = (gw / NP) * 64 + (threadIdx.x & 63);
    if (b >= nbr) return;
    float *o = out + (int64_t)blockIdx.y * cols + (int64_t)b * U::VALUES + EMBED_VALUES * p;
    if (id < 0 || id >= rows) {
#pragma unroll
        for (int i = 0; i < EMBED_VALUES; i++) o[i] = __builtin_nanf("");
        return;
    }
    const uint8_t *q = W + (int64_t)id * row_bytes + (int64_t)b * U::BYTES;
    const u32 ph = (u32)((uintptr_t)q & 3u);
    const rsrc_t rs = make_rsrc(q - ph, (u32)(ph + U::BYTES + 3) & ~3u);
    u32 w[U::ND];
    U::load(rs, ph, w);
    embed_part<U>(p, w, scale, o);
}

// ---- rows of the plane layouts: one thread per value ----------------------
// value c of row id of a rows x cols tensor held in planes, as qg_dequant
// gives it: Q8_0 d * code ([qwen3] i8at's code plane), Q6_K (d * scale) *
// (q - 32) ([bonsai] dequantQ6K's fields in their planes); exact in f32
template <int TY>
QG_DEV float plane_value(const uint8_t *W, int64_t rows, int cols, int64_t id, int c) {
    if constexpr (TY == T_Q8_0P) {
        const int64_t nb = cols / 32;
        const uint8_t *D = W + rows * (int64_t)cols;
        return h2f(*(const uint16_t *)(D + 2 * (id * nb + c / 32))) * (float)(int8_t)W[id * (int64_t)cols + c];
    } else {
        const int64_t n = rows * (int64_t)(cols / 256), b = id * (cols / 256) + c / 256;
        const int t = c & 255, half = t >> 7, r = t & 127, p = r >> 5, l = r & 31;
        const int lo = W[128 * b + 64 * half + l + 32 * (p & 1)];
        const int q4 = p >= 2 ? lo >> 4 : lo & 15;
        const int hb = (W[128 * n + 64 * b + 32 * half + l] >> (2 * p)) & 3;
        const int sc = (int8_t)W[192 * n + 16 * b + 8 * half + (l >> 4) + 2 * p];
        const float d = h2f(*(const uint16_t *)(W + 208 * n + 2 * b));
        return (d * (float)sc) * (float)((q4 | (hb << 4)) - 32);
    }
}

// this workgroup's 256 values of row id of token blockIdx.y (an id outside
// the table gives NaN, as embed_row)
template <int TY>
QG_DEV void embed_row_planes(const uint8_t *W, int64_t rows, int cols, int32_t id, float scale, float *out) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= cols) return;
    float *o = out + (int64_t)blockIdx.y * cols + c;
    *o = id < 0 || id >= rows ? __builtin_nanf("") : plane_value<TY>(W, rows, cols, id, c) * scale;
}

template <int TY>
__global__ __launch_bounds__(256) void k_embed_planes(const uint8_t *W, int64_t rows, int cols, const int32_t *tok,
                                                      float scale, float *out) {
    embed_row_planes<TY>(W, rows, cols, tok[blockIdx.y], scale, out);
}

template <class U>
__global__ __launch_bounds__(256) void k_embed(const uint8_t *W, int64_t rows, int cols, int64_t row_bytes,
                                               const int32_t *tok, float scale, float *out) {
    embed_row<U>(W, rows, cols, row_bytes, tok[blockIdx.y], scale, out);
}

template <class U>
static int launch_embed_t(const uint8_t *W, int64_t rows, int cols, int64_t row_bytes, const int32_t *tok,
                          int ntok, float scale, float *out, hipStream_t st) {
    const int nbr = cols / U::VALUES;
    const int64_t waves = (int64_t)((nbr + 63) / 64) * (U::VALUES / EMBED_VALUES);
    const dim3 grid((unsigned)((waves + 3) / 4), ntok);
    hipLaunchKernelGGL(k_embed<U>, grid, dim3(256), 0, st, W, rows, cols, row_bytes, tok, scale, out);
    return hipGetLastError() == hipSuccess ? 0 : QG_EHIP;
}

int launch_embed(int type, const uint8_t *W, int64_t rows, int cols, int64_t row_bytes, const int32_t *tok,
                 int ntok, float scale, float *out, hipStream_t st) {
    if (type == T_Q8_0P || type == T_Q6_KP) {
        const dim3 grid((unsigned)((cols + 255) / 256), ntok);
        if (type == T_Q8_0P)
            hipLaunchKernelGGL(k_embed_planes<T_Q8_0P>, grid, dim3(256), 0, st, W, rows, cols, tok, scale, out);
        else
            hipLaunchKernelGGL(k_embed_planes<T_Q6_KP>, grid, dim3(256), 0, st, W, rows, cols, tok, scale, out);
        return hipGetLastError() == hipSuccess ? 0 : QG_EHIP;
    }
    switch (type) {
    case T_Q8_0: return launch_embed_t<UQ8_0B>(W, rows, cols, row_bytes, tok, ntok, scale, out, st);
    case T_Q4_0: return launch_embed_t<UQ4_0B>(W, rows, cols, row_bytes, tok, ntok, scale, out, st);
    case T_Q4_K: return launch_embed_t<UQ4_K>(W, rows, cols, row_bytes, tok, ntok, scale, out, st);
    default: return launch_embed_t<UQ6_K>(W, rows, cols, row_bytes, tok, ntok, scale, out, st);
    }
}

// ---------------------------------------------------- soft cap, argmax ----
// (value, index) candidates: the larger value wins, equal values go to the
// lower index, an empty candidate (index < 0) always loses.  The winner over
// any set is unique, so the order of the merges does not matter.
QG_DEV void am_merge(float &bv, int &bi, float ov, int oi) {
    if (oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi))) {
        bv = ov;
        bi = oi;
    }
}

QG_DEV void am_wave(float &bv, int &bi) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const float ov = __shfl_xor(bv, m);
        const int oi = __shfl_xor(bi, m);
        am_merge(bv, bi, ov, oi);
    }
}

// Phase 1, workgroup (g, t): the span [g span, (g+1) span) of token t's
// logits.  With cap > 0 each logit is first capped in place,
// l = tanh(clamp(l inv, -10, 10)) cap (gemma4_moe_ssd.js softcap); NaN stays
// NaN.  Then the first index of the largest value, NaN skipped
// (qwen3_moe_ssd.js argmax: strict greater-than, lower index on ties).
constexpr int AB = 8;   // logits per thread per batch of loads

__global__ __launch_bounds__(256) void k_argmax_part(float *l, int64_t n, int64_t span, float cap, float inv,
                                                     float *pv, int32_t *pi) {
    __shared__ float s_v[4];
    __shared__ int s_i[4];
    float *lt = l + (int64_t)blockIdx.y * n;
    const int64_t lo = (int64_t)blockIdx.x * span;
    const int64_t hi = min(n, lo + span);
    float bv = 0.0f;
    int bi = -1;
    for (int64_t i0 = lo + threadIdx.x; i0 < hi; i0 += 256 * AB) {
        float v[AB];
#pragma unroll
        for (int u = 0; u < AB; u++) v[u] = i0 + u * 256 < hi ? lt[i0 + u * 256] : 0.0f;
#pragma unroll
        for (int u = 0; u < AB; u++) {
            const int64_t i = i0 + u * 256;
            if (i >= hi) continue;
            float e = v[u];
            if (cap > 0.0f) {
                float z = e * inv;
                z = z < -10.0f ? -10.0f : (z > 10.0f ? 10.0f : z);
                e = tanhf(z) * cap;
                lt[i] = e;
            }
            // indices rise within a thread, so strict > keeps the first of equal values
            if (e == e && (bi < 0 || e > bv)) {
                bv = e;
                bi = (int)i;
            }
        }
    }
    am_wave(bv, bi);
    if ((threadIdx.x & 63) == 0) {
        s_v[threadIdx.x >> 6] = bv;
        s_i[threadIdx.x >> 6] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < 4; w++) am_merge(bv, bi, s_v[w], s_i[w]);
        pv[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = bv;
        pi[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = bi;
    }
}

// Phase 2, one wave per token: the winner over the G partials; 0 when the
// token's logits hold no number at all.
QG_DEV int argmax_final_wave(const float *pv, const int32_t *pi, int G, int t, int lane) {
    float bv = 0.0f;
    int bi = -1;
    float v[ARGMAX_MAX_PARTS / 64];
    int ix[ARGMAX_MAX_PARTS / 64];
#pragma unroll
    for (int u = 0; u < ARGMAX_MAX_PARTS / 64; u++) {
        const int g = lane + 64 * u;
        v[u] = g < G ? pv[(int64_t)t * G + g] : 0.0f;
        ix[u] = g < G ? pi[(int64_t)t * G + g] : -1;
    }
#pragma unroll
    for (int u = 0; u < ARGMAX_MAX_PARTS / 64; u++) am_merge(bv, bi, v[u], ix[u]);
    am_wave(bv, bi);
    return bi < 0 ? 0 : bi;
}

// Phase 2 and the picked token's embedding row in one launch: wave 0 of
// every workgroup of token t takes the winner as k_argmax_final does (the
// same merges, so the same index), workgroup (0, t) stores it, and the
// workgroup then gathers its share of row idx as k_embed does.
template <class U>
__global__ __launch_bounds__(256) void k_argmax_embed(const float *pv, const int32_t *pi, int G, int32_t *idx,
                                                      const uint8_t *W, int64_t rows, int cols, int64_t row_bytes,
                                                      float scale, float *out) {
    __shared__ int s_id;
    if (threadIdx.x < 64) {
        const int id = argmax_final_wave(pv, pi, G, blockIdx.y, threadIdx.x);
        if (threadIdx.x == 0) {
            s_id = id;
            if (blockIdx.x == 0) idx[blockIdx.y] = id;
        }
    }
    __syncthreads();
    embed_row<U>(W, rows, cols, row_bytes, s_id, scale, out);
}

// the same with the row gathered from a plane layout
template <int TY>
__global__ __launch_bounds__(256) void k_argmax_embed_planes(const float *pv, const int32_t *pi, int G, int32_t *idx,
                                                             const uint8_t *W, int64_t rows, int cols, float scale,
                                                             float *out) {
    __shared__ int s_id;
    if (threadIdx.x < 64) {
        const int id = argmax_final_wave(pv, pi, G, blockIdx.y, threadIdx.x);
        if (threadIdx.x == 0) {
            s_id = id;
            if (blockIdx.x == 0) idx[blockIdx.y] = id;
        }
    }
    __syncthreads();
    embed_row_planes<TY>(W, rows, cols, s_id, scale, out);
}

__global__ __launch_bounds__(64) void k_argmax_final(const float *pv, const int32_t *pi, int G, int32_t *idx) {
    const int t = blockIdx.x, lane = threadIdx.x;
    float bv = 0.0f;
    int bi = -1;
    float v[ARGMAX_MAX_PARTS / 64];
    int ix[ARGMAX_MAX_PARTS / 64];
#pragma unroll
    for (int u = 0; u < ARGMAX_MAX_PARTS / 64; u++) {
        const int g = lane + 64 * u;
        v[u] = g < G ? pv[(int64_t)t * G + g] : 0.0f;
        ix[u] = g < G ? pi[(int64_t)t * G + g] : -1;
    }
#pragma unroll
    for (int u = 0; u < ARGMAX_MAX_PARTS / 64; u++) am_merge(bv, bi, v[u], ix[u]);
    am_wave(bv, bi);
    if (lane == 0) idx[t] = bi < 0 ? 0 : bi;
}

// ------------------------------------------------------------ launches ----
int launch_rmsnorm(const float *x, const float *w, float *y, int64_t n, int ntok, float eps, float k,
                   hipStream_t st) {
    hipLaunchKernelGGL(k_rmsnorm, dim3(ntok), dim3(256), 0, st, x, w, y, n, eps, k);
    return hipGetLastError() == hipSuccess ? 0 : QG_EHIP;
}

int launch_rmsnorm_multi(const float *x, int64_t n, int ntok, float eps, int nout, const float *const *w,
                         const float *k, float *const *y, hipStream_t st) {
    NormOuts o = {};
    for (int j = 0; j < nout; j++) {
        o.w[j] = w[j];
        o.y[j] = y[j];
        o.k[j] = k[j];
    }
    hipLaunchKernelGGL(k_rmsnorm_multi, dim3(ntok, nout), dim3(256), 0, st, x, n, eps, o);
    return hipGetLastError() == hipSuccess ? 0 : QG_EHIP;
}

int launch_norm_gemv_f32(const float *x, int64_t n, int ntok, float eps, const float *rw, float rk, const float *W,
                         int64_t rows, float *y, int nout, const float *const *w, const float *k, float *const *yo,
                         hipStream_t st) {
    NormOuts o = {};
    for (int j = 0; j < nout; j++) {
        o.w[j] = w[j];
        o.y[j] = yo[j];
        o.k[j] = k[j];
    }
    const bool v4 = (n % 4) == 0 && ((uintptr_t)W % 16) == 0 && ((uintptr_t)x % 16) == 0 && ((uintptr_t)rw % 16) == 0;
    // the same row split as launch_gemv_f32 takes for these sizes, so the
    // logits keep its summation order
    const bool split = v4 && ntok > 4 && rows <= 65536;
    const dim3 grid((unsigned)(split ? rows : (rows + 3) / 4));
    void (*f)(const float *, int64_t, int, float, const float *, float, const float *, int64_t, float *, NormOuts, int);
    if (ntok == 1) f = v4 ? k_norm_gemv_f32<1, true, 1> : k_norm_gemv_f32<1, false, 1>;
    else if (ntok <= 4) f = v4 ? k_norm_gemv_f32<4, true, 1> : k_norm_gemv_f32<4, false, 1>;
    else f = split ? k_norm_gemv_f32<16, true, 4> : v4 ? k_norm_gemv_f32<16, true, 1> : k_norm_gemv_f32<16, false, 1>;
    hipLaunchKernelGGL(f, grid, dim3(256), 0, st, x, n, ntok, eps, rw, rk, W, rows, y, o, nout);
    return hipGetLastError() == hipSuccess ? 0 : QG_EHIP;
}

int launch_gemv_f32(const float *W, const float *x, float *y, int64_t rows, int64_t cols, int ntok,
                    hipStream_t st) {
    const bool v4 = (cols % 4) == 0 && ((uintptr_t)W % 16) == 0 && ((uintptr_t)x % 16) == 0;
    // 5 to 16 tokens over at most 64K rows (the routers and gates): one row a
    // workgroup, its column passes spread over the 4 waves
    const bool split = v4 && ntok > 4 && rows <= 65536;
    const dim3 grid((unsigned)(split ? rows : (rows + 3) / 4));
    void (*f)(const float *, const float *, float *, int64_t, int64_t, int);
    if (ntok == 1) f = v4 ? k_gemv_f32<1, true, 1> : k_gemv_f32<1, false, 1>;
    else if (ntok <= 4) f = v4 ? k_gemv_f32<4, true, 1> : k_gemv_f32<4, false, 1>;
    else f = split ? k_gemv_f32<16, true, 4> : v4 ? k_gemv_f32<16, true, 1> : k_gemv_f32<16, false, 1>;
    hipLaunchKernelGGL(f, grid, dim3(256), 0, st, W, x, y, rows, cols, ntok);
    return hipGetLastError() == hipSuccess ? 0 : QG_EHIP;
}

int launch_combine_shared(const float *dn, const int32_t *rt_valid, const float *sh, const float *gate_inp,
                          const float *x, float *resid, int64_t H, int k, int ntok, hipStream_t st) {
    hipLaunchKernelGGL(k_combine_shared, dim3((unsigned)((H + 255) / 256), ntok), dim3(256), 0, st, dn, rt_valid,
                       sh, gate_inp, x, resid, H, k);
    return hipGetLastError() == hipSuccess ? 0 : QG_EHIP;
}

int launch_post_ffn(const float *mlp, const float *moe, const float *w1, const float *w2, const float *w,
                    const float *os, float *x, int64_t n, int ntok, float eps, hipStream_t st) {
    hipLaunchKernelGGL(k_post_ffn, dim3(ntok), dim3(256), 0, st, mlp, moe, w1, w2, w, os, x, n, eps);
    return hipGetLastError() == hipSuccess ? 0 : QG_EHIP;
}

int argmax_parts(int64_t n) {
    int64_t g = (n + ARGMAX_SPAN - 1) / ARGMAX_SPAN;
    return (int)(g < ARGMAX_MAX_PARTS ? g : ARGMAX_MAX_PARTS);
}

template <class U>
static int launch_argmax_embed_t(int G, const float *pv, const int32_t *pi, int32_t *idx, const uint8_t *W,
                                 int64_t rows, int cols, int64_t row_bytes, int ntok, float scale, float *out,
                                 hipStream_t st) {
    const int nbr = cols / U::VALUES;
    const int64_t waves = (int64_t)((nbr + 63) / 64) * (U::VALUES / EMBED_VALUES);
    const dim3 grid((unsigned)((waves + 3) / 4), ntok);
    hipLaunchKernelGGL(k_argmax_embed<U>, grid, dim3(256), 0, st, pv, pi, G, idx, W, rows, cols, row_bytes, scale,
                       out);
    return hipGetLastError() == hipSuccess ? 0 : QG_EHIP;
}

int launch_argmax_embed(float *l, int64_t n, int ntok, float cap, float *pv, int32_t *pi, int32_t *idx, int type,
                        const uint8_t *W, int64_t rows, int cols, int64_t row_bytes, float scale, float *out,
                        hipStream_t st) {
    const int G = argmax_parts(n);
    const int64_t span = (n + G - 1) / G;
    const float inv = cap > 0.0f ? (float)(1.0 / (double)cap) : 0.0f;
    hipLaunchKernelGGL(k_argmax_part, dim3(G, ntok), dim3(256), 0, st, l, n, span, cap, inv, pv, pi);
    if (hipGetLastError() != hipSuccess) return QG_EHIP;
    if (type == T_Q8_0P || type == T_Q6_KP) {
        const dim3 grid((unsigned)((cols + 255) / 256), ntok);
        if (type == T_Q8_0P)
            hipLaunchKernelGGL(k_argmax_embed_planes<T_Q8_0P>, grid, dim3(256), 0, st, pv, pi, G, idx, W, rows, cols,
                               scale, out);
        else
            hipLaunchKernelGGL(k_argmax_embed_planes<T_Q6_KP>, grid, dim3(256), 0, st, pv, pi, G, idx, W, rows, cols,
                               scale, out);
        return hipGetLastError() == hipSuccess ? 0 : QG_EHIP;
    }
    switch (type) {
    case T_Q8_0: return launch_argmax_embed_t<UQ8_0B>(G, pv, pi, idx, W, rows, cols, row_bytes, ntok, scale, out, st);
    case T_Q4_0: return launch_argmax_embed_t<UQ4_0B>(G, pv, pi, idx, W, rows, cols, row_bytes, ntok, scale, out, st);
    case T_Q4_K: return launch_argmax_embed_t<UQ4_K>(G, pv, pi, idx, W, rows, cols, row_bytes, ntok, scale, out, st);
    default: return launch_argmax_embed_t<UQ6_K>(G, pv, pi, idx, W, rows, cols, row_bytes, ntok, scale, out, st);
    }
}

int launch_argmax(float *l, int64_t n, int ntok, float cap, float *pv, int32_t *pi, int32_t *idx,
                  hipStream_t st) {
    const int G = argmax_parts(n);
    const int64_t span = (n + G - 1) / G;
    // the f32 nearest 1/cap, as the soft cap's uniform holds it
    const float inv = cap > 0.0f ? (float)(1.0 / (double)cap) : 0.0f;
    hipLaunchKernelGGL(k_argmax_part, dim3(G, ntok), dim3(256), 0, st, l, n, span, cap, inv, pv, pi);
    if (hipGetLastError() != hipSuccess) return QG_EHIP;
    hipLaunchKernelGGL(k_argmax_final, dim3(ntok), dim3(64), 0, st, pv, pi, G, idx);
    return hipGetLastError() == hipSuccess ? 0 : QG_EHIP;
}

}  // namespace qg

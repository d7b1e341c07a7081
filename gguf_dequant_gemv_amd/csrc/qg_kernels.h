// qg_kernels.h -- the GEMV kernel family (dense and expert-grouped), the
// dequantization kernel, the router and the MoE combine, for gfx950.
//
// GEMV geometry (one kernel for every block type; T = 1..16 tokens):
//   - a workgroup is 4 wave64s; a wave owns RPW = 64/LPR consecutive rows and
//     LPR lanes share a row; lane `sub` of a row takes units sub, sub+LPR, ...
//   - each lane loads whole units (GGUF bytes as they sit in HBM, 16-byte
//     buffer loads, dword aligned) and decodes them in registers; the block
//     scale is applied once per scale group;
//   - x (one vector per token of the workgroup's token chunk) is staged in LDS
//     once per workgroup, with the per-group x-sums some formats fold with;
//   - row results are reduced across the LPR lanes with DPP / swizzles.
// The pages' GEMVs (qwen3_moe_ssd.js matmulQ8 / expertQ8, gemma4_moe_ssd.js
// matmulQ4 / matmulQ6K / expertQ4, their subgroup variants, and the
// qwen35_moe_ssd.js matmulQ8T / expertQ8B batch kernels) compute the same
// sums; the mapping here is designed for wave64 and 16-byte HBM loads.
#pragma once
#include "qg_device.h"

namespace qg {

// ------------------------------------------------------------ activations --
// act(gate) * up.  SiLU: the qwen3_moe_ssd.js siluMulMoe kernel; GELU (tanh
// form, argument clamped to [-10, 10]): the gemma4_moe_ssd.js GELU helper.
enum { XM_PLAIN = 0, XM_SILU = 1, XM_GELU = 2 };

QG_DEV float silu_f(float g) { return g / (1.0f + expf(-g)); }
QG_DEV float gelu_f(float g) {
    float u = 0.7978845608f * g * (1.0f + 0.044715f * g * g);
    u = fminf(fmaxf(u, -10.0f), 10.0f);
    return 0.5f * g * (1.0f + tanhf(u));
}
QG_DEV float glu(int xmode, float g, float u) { return (xmode == XM_GELU ? gelu_f(g) : silu_f(g)) * u; }

// ------------------------------------------------------------ arguments ----
// Routing / grouping table written by k_route into the workspace (int32):
//   [0]                     number of groups G (distinct picked experts)
//   [1 + g*GREC + 0]        expert id of group g (groups in ascending id)
//   [1 + g*GREC + 1]        pool slot of that expert
//   [1 + g*GREC + 2]        n = number of (token, pick) pairs in the group
//   [1 + g*GREC + 3 + i]    token of pair i (ascending), i < n
//   [1 + g*GREC + 19 + i]   pair index z = t*k + j of pair i
constexpr int GREC = 35;
constexpr int MAXT = 16;

struct GemvArgs {
    // weights: dense rows [0, rows0) come from W0, rows [rows0, rows) from W1;
    // grouped: W0 + slot * slot_stride for the group's slot.
    const uint8_t *W0, *W1;
    int64_t rows0, rows, row_bytes, slot_stride;
    int cols, upr, nb;
    // inputs: vector i of the chunk is x + idx_i * x_stride (+ GLU transform)
    const float *x;
    int64_t x_stride;
    int xmode;
    int x_vec;         // x rows are 16-byte aligned (x and x_stride * 4)
    // outputs: vector i goes to y + idx_i * y_stride
    float *y;
    int64_t y_stride;
    int ntok;          // dense: tokens 0..ntok-1
    const int *grp;    // grouped: the routing table, or nullptr for dense
    int in_by_pair;    // grouped input index: 0 = token, 1 = pair
    int ntiles;        // row tiles of 4*RPW rows
};

// -------------------------------------------------------- unit dot product --
// acc[t] += sum over the unit of value(i) * x_t[i], for all NT token slots
// (slots past the chunk's last token hold a copy of it; their sums are dropped).
// Per scale group: s = sum(code * x) with f32 FMAs, then fold(s, sum(x)); the
// unit's groups are summed before joining the lane accumulator.
template <class U, int NT>
QG_DEV void unit_dot(const u32 (&w)[U::ND], const float *__restrict__ xs, int xstride,
                     const float *__restrict__ ss, int sstride, float (&acc)[NT]) {
    float us[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) us[t] = 0.0f;
#pragma unroll
    for (int g = 0; g < U::GROUPS; g++) {
        float s0[NT], s1[NT];
#pragma unroll
        for (int t = 0; t < NT; t++) { s0[t] = 0.0f; s1[t] = 0.0f; }
#pragma unroll
        for (int k = 0; k < U::GSIZE / 4; k++) {
            const int i = g * U::GSIZE + 4 * k;
            const float q0 = U::code(w, i), q1 = U::code(w, i + 1);
            const float q2 = U::code(w, i + 2), q3 = U::code(w, i + 3);
#pragma unroll
            for (int t = 0; t < NT; t++) {
                const f32x4 xv = *(const f32x4 *)(xs + t * xstride + i + ((i >> 6) << 2));
                float &s = (k & 1) ? s1[t] : s0[t];
                s = fmaf(q0, xv.x, s);
                s = fmaf(q1, xv.y, s);
                s = fmaf(q2, xv.z, s);
                s = fmaf(q3, xv.w, s);
            }
        }
#pragma unroll
        for (int t = 0; t < NT; t++)
            us[t] += U::fold(w, g, s0[t] + s1[t], U::SUMS ? ss[t * sstride + g] : 0.0f);
    }
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t] += us[t];
}

// One wave's pass over its rows: lane (grp, sub) accumulates row grp's units
// sub, sub+LPR, ...; UNR units are loaded before any is decoded.  Pair units
// are whole pairs in the main loop; with an odd number of blocks per row the
// last, single block is a separate step taken by one lane per row.
template <class U, int LPR, int NT, int UNR>
QG_DEV void lane_rows(rsrc_t rs, u32 row_off, int upr, int nb, int sub, const float *xs, int xstride,
                      const float *ss, int sstride, float (&acc)[NT]) {
    constexpr int UV = U::VALUES;
    constexpr int SPU = UV / (U::SUMS ? U::SUMS : UV) * (U::SUMS ? 1 : 0);  // x-sums per unit
    const int nfull = (UV == 64) ? (nb >> 1) : upr;
    for (int u0 = sub; u0 < nfull; u0 += LPR * UNR) {
        // every lane loads UNR units (a lane past the row's end re-loads the
        // row's last unit, a cache hit) so the loads are straight-line code
        u32 w[UNR][U::ND];
#pragma unroll
        for (int i = 0; i < UNR; i++) {
            const int u = min(u0 + i * LPR, nfull - 1);
            U::load(rs, row_off + (u32)u * U::BYTES, w[i], true);
        }
#pragma unroll
        for (int i = 0; i < UNR; i++) {
            const int u = u0 + i * LPR;
            if (u < nfull) unit_dot<U, NT>(w[i], xs + xpad(u * UV), xstride, ss + u * SPU, sstride, acc);
        }
    }
    if (UV == 64 && (nb & 1) && sub == nfull % LPR) {
        u32 w[U::ND];
        U::load(rs, row_off + (u32)nfull * U::BYTES, w, false);
        unit_dot<U, NT>(w, xs + xpad(nfull * UV), xstride, ss + nfull * SPU, sstride, acc);
    }
}

// Pairs of Q8_0/Q4_0 blocks are templated on the pair's phase (start mod 4).
template <int TYPE, int PH> struct UnitOf;
template <int PH> struct UnitOf<T_Q8_0, PH> { typedef UQ8_0<PH> U; };
template <int PH> struct UnitOf<T_Q4_0, PH> { typedef UQ4_0<PH> U; };
template <int PH> struct UnitOf<T_Q4_K, PH> { typedef UQ4_K<PH> U; };
template <int PH> struct UnitOf<T_Q6_K, PH> { typedef UQ6_K U; };

// x[t] (or act(gate) * up from a [gate | up] row) into LDS, zero-padded from
// cols to cpad.  a.x_vec: every source row is 16-byte aligned, so whole
// float4s are loaded (cols is a multiple of 32).
template <int NT>
QG_DEV void stage_x(const GemvArgs &a, const int (&in_idx)[NT], int cols, int cpad, float *xs, int xstride) {
    constexpr int B = 8;  // float4 loads in flight per thread
    const int tid = threadIdx.x;
    if (a.x_vec) {
        const int n4 = cpad >> 2, c4 = cols >> 2;
        for (int t = 0; t < NT; t++) {
            const f32x4 *src = (const f32x4 *)(a.x + (int64_t)in_idx[t] * a.x_stride);
            for (int base = tid; base < n4; base += 256 * B) {
                f32x4 v[B], u[B];
#pragma unroll
                for (int b = 0; b < B; b++) {
                    const int i = min(base + 256 * b, c4 - 1);
                    v[b] = src[i];
                    if (a.xmode != XM_PLAIN) u[b] = src[c4 + i];
                }
#pragma unroll
                for (int b = 0; b < B; b++) {
                    const int i = base + 256 * b;
                    if (i < n4) {
                        f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
                        if (i < c4) {
                            if (a.xmode == XM_PLAIN) {
                                o = v[b];
                            } else {
                                o.x = glu(a.xmode, v[b].x, u[b].x);
                                o.y = glu(a.xmode, v[b].y, u[b].y);
                                o.z = glu(a.xmode, v[b].z, u[b].z);
                                o.w = glu(a.xmode, v[b].w, u[b].w);
                            }
                        }
                        *(f32x4 *)(xs + t * xstride + xpad(4 * i)) = o;
                    }
                }
            }
        }
    } else {
        for (int t = 0; t < NT; t++) {
            const float *src = a.x + (int64_t)in_idx[t] * a.x_stride;
            for (int c = tid; c < cpad; c += 256) {
                float v = 0.0f;
                if (c < cols) v = a.xmode == XM_PLAIN ? src[c] : glu(a.xmode, src[c], src[cols + c]);
                xs[t * xstride + xpad(c)] = v;
            }
        }
    }
}

// ------------------------------------------------------------ GEMV kernel --
// grid.x: row tiles (grid-stride); grid.y: dense token chunk, or group;
// grid.z: grouped token chunk.  LDS: x for NT vectors + their x-sums.
template <int TYPE, int LPR, int NT, int UNR>
__global__ __launch_bounds__(256) void k_gemv(GemvArgs a) {
    extern __shared__ float lds[];
    typedef typename UnitOf<TYPE, 0>::U U0;
    constexpr int RPW = 64 / LPR;
    constexpr int SUMS = U0::SUMS;

    // ---- which vectors this workgroup serves, and which weights ----
    const uint8_t *Wg0 = a.W0, *Wg1 = a.W1;
    int nt;
    int in_idx[NT], out_idx[NT];
    if (a.grp) {
        const int G = a.grp[0];
        const int g = blockIdx.y;
        if (g >= G) return;
        const int *rec = a.grp + 1 + g * GREC;
        const int n = rec[2];
        const int c0 = blockIdx.z * NT;
        if (c0 >= n) return;
        nt = min(NT, n - c0);
        Wg0 = Wg1 = a.W0 + (int64_t)rec[1] * a.slot_stride;
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const int i = c0 + min(t, nt - 1);
            in_idx[t] = a.in_by_pair ? rec[19 + i] : rec[3 + i];
            out_idx[t] = rec[19 + i];
        }
    } else {
        const int c0 = blockIdx.y * NT;
        nt = min(NT, a.ntok - c0);
#pragma unroll
        for (int t = 0; t < NT; t++) in_idx[t] = out_idx[t] = c0 + min(t, nt - 1);
    }

    // ---- stage x (and the GLU transform) into LDS ----
    // x is zero-padded to whole units (cpad values), so a row's last, half
    // pair reads zeros rather than whatever follows the vector.  Loads are
    // 16-byte vectors, all issued before any is stored, so staging costs about
    // one L2 round trip rather than one per element.
    const int cols = a.cols;
    const int cpad = a.upr * U0::VALUES;
    const int xstride = xstride_of(cpad);
    const int nsum = SUMS ? cpad / SUMS : 0;
    float *xs = lds;
    float *ss = lds + NT * xstride;
    stage_x<NT>(a, in_idx, cols, cpad, xs, xstride);
    __syncthreads();
    if constexpr (SUMS != 0) {
        for (int i = threadIdx.x; i < NT * nsum; i += 256) {
            const int t = i / nsum, gi = i - t * nsum;
            const float *p = xs + t * xstride + xpad(gi * SUMS);  // SUMS divides 64: no pad inside
            float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
            for (int j = 0; j < SUMS; j += 2) { s0 += p[j]; s1 += p[j + 1]; }
            ss[t * nsum + gi] = s0 + s1;
        }
        __syncthreads();
    }

    // ---- rows ----
    // the wave index is uniform; saying so keeps the buffer descriptors in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int grp = lane / LPR, sub = lane % LPR;
    for (int tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
        const int64_t r0 = ((int64_t)tile * 4 + wave) * RPW;
        if (r0 >= a.rows) break;
        const bool lo = r0 < a.rows0;
        const int64_t end = lo ? a.rows0 : a.rows;
        const int nrows = (int)min((int64_t)RPW, end - r0);
        const uint8_t *rowp = lo ? Wg0 + r0 * a.row_bytes : Wg1 + (r0 - a.rows0) * a.row_bytes;
        const u32 ph = (u32)((uintptr_t)rowp & 3u);
        const u32 span = (u32)(ph + (u32)nrows * (u32)a.row_bytes + 3u) & ~3u;
        const rsrc_t rs = make_rsrc(rowp - ph, span);
        float acc[NT];
#pragma unroll
        for (int t = 0; t < NT; t++) acc[t] = 0.0f;
        if (grp < nrows) {
            const u32 roff = (u32)grp * (u32)a.row_bytes;
            if constexpr (TYPE == T_Q6_K) {
                lane_rows<UQ6_K, LPR, NT, UNR>(rs, roff + ph, a.upr, a.nb, sub, xs, xstride, ss, nsum, acc);
            } else {
                // rows of one wave share a phase (host guarantees row_bytes % 4 == 0 or RPW == 1)
                if (ph == 0)
                    lane_rows<typename UnitOf<TYPE, 0>::U, LPR, NT, UNR>(rs, roff, a.upr, a.nb, sub, xs, xstride, ss, nsum, acc);
                else
                    lane_rows<typename UnitOf<TYPE, 2>::U, LPR, NT, UNR>(rs, roff, a.upr, a.nb, sub, xs, xstride, ss, nsum, acc);
            }
        }
#pragma unroll
        for (int t = 0; t < NT; t++) acc[t] = group_sum<LPR>(acc[t]);
        if (sub == 0 && grp < nrows) {
            const int64_t r = r0 + grp;
#pragma unroll
            for (int t = 0; t < NT; t++)
                if (t < nt) a.y[(int64_t)out_idx[t] * a.y_stride + r] = acc[t];
        }
    }
}

// ------------------------------------------------------- dequantization ---
// One thread per unit: out[r][c] = value of W[r][c] as f32, through the same
// loads and decoders as the GEMV.
template <int TYPE>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t *W, float *out, int64_t rows, int cols,
                                                 int64_t row_bytes, int upr, int nb) {
    typedef typename UnitOf<TYPE, 0>::U U0;
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= rows * upr) return;
    const int64_t r = id / upr;
    const int u = (int)(id - r * upr);
    const uint8_t *p = W + r * row_bytes + (int64_t)u * U0::BYTES;
    const u32 ph = (u32)((uintptr_t)p & 3u);
    const int vals = min(U0::VALUES, cols - u * U0::VALUES);
    const rsrc_t rs = make_rsrc(p - ph, (u32)(ph + U0::BYTES + 3) & ~3u);
    float *o = out + r * cols + (int64_t)u * U0::VALUES;
    auto emit = [&](auto unit) {
        typedef decltype(unit) U;
        u32 w[U::ND];
        U::load(rs, TYPE == T_Q6_K ? ph : 0u, w, vals > 32);
#pragma unroll
        for (int i = 0; i < U::VALUES; i++)
            if (i < vals) o[i] = U::value(w, i);
    };
    if (TYPE == T_Q6_K || ph == 0)
        emit(typename UnitOf<TYPE, 0>::U());
    else
        emit(typename UnitOf<TYPE, 2>::U());
}

// ------------------------------------------------------ instance tables ---
typedef void (*gemv_fn)(GemvArgs);
typedef void (*dequant_fn)(const uint8_t *, float *, int64_t, int, int64_t, int, int);
// One per (block type, tokens per workgroup), each in its own translation
// unit (qg_inst_<type>_t<NT>.hip); qg_inst_dequant.hip holds the dequantizers.
#define QG_DECL_GEMV(NAME) \
    gemv_fn gemv_kernel_##NAME##_t1(int lpr, int unr); \
    gemv_fn gemv_kernel_##NAME##_t2(int lpr, int unr); \
    gemv_fn gemv_kernel_##NAME##_t4(int lpr, int unr); \
    gemv_fn gemv_kernel_##NAME##_t8(int lpr, int unr);
QG_DECL_GEMV(q8_0)
QG_DECL_GEMV(q4_0)
QG_DECL_GEMV(q4_k)
QG_DECL_GEMV(q6_k)
#undef QG_DECL_GEMV
dequant_fn dequant_kernel(int type);

// Router / grouping and combine kernels (qg_route.hip).
__global__ void k_route(const float *logits, int E, int k, int T, const int32_t *slots, int n_slots, int32_t *ids_out,
                        float *w_out, int32_t *status, int32_t *rt_ids, float *rt_w, int32_t *rt_valid,
                        int32_t *grp);
__global__ void k_combine(const float *dn, const int32_t *rt_ids, const float *rt_w, const int32_t *rt_valid,
                          const float *dscale, float *y, int64_t H, int k);

}  // namespace qg

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
    // grouped: W0 + slot * slot_stride for the group's slot.  Gated pairs:
    // gate rows [0, rows) from W0, up rows [0, rows) from W1 (grouped: the up
    // rows follow the gate rows in the slot).
    const uint8_t *W0, *W1;
    int64_t rows0, rows, row_bytes, slot_stride;
    int64_t bytes0, bytes1;   // bytes of the W0 / W1 ranges
    int cols, nunits;         // values per row; units per row
    // inputs: vector i of the chunk is x + idx_i * x_stride
    const float *x;
    int64_t x_stride;
    int x_vec;         // x rows are 16-byte aligned (x and x_stride * 4)
    // outputs: vector i goes to y + idx_i * y_stride
    float *y;
    int64_t y_stride;
    // gated pairs (XM_SILU / XM_GELU): row r of the output is act(g_r) * u_r
    // where g_r is row r of W0 and u_r row r of W1 (rows = the gate rows);
    // the raw g_r, u_r also go to y2 + idx_i * y2_stride + r (+ rows), if set
    int glu;
    float *y2;
    int64_t y2_stride;
    int ntok;          // dense: tokens 0..ntok-1
    const int *grp;    // grouped: the routing table, or nullptr for dense
    int in_by_pair;    // grouped input index: 0 = token, 1 = pair
    // grouped outputs scaled as (y * escale[expert]) * pscale[pair] when set
    // (the MoE combine's per-expert down scale and routing weight)
    const float *escale;
    const float *pscale;
    // LDS-staged variant (k_gemv_lds): stages in flight per wave and the byte
    // offset of the stage rings in LDS
    int depth;
    int ring_off;
    int ntiles;        // row tiles of 4*RPW rows
};

// -------------------------------------------------------- unit dot product --
// acc[t] += sum over the unit of value(i) * x_t[i], for all NT token slots
// (slots past the chunk's last token hold a copy of it; their sums are dropped).
// Per scale group: s = sum(code * x) with f32 FMAs, then fold(s, sum(x)); the
// unit's groups are summed before joining the lane accumulator.
template <class U, int NT>
QG_DEV void unit_dot(const u32 (&w)[U::ND], const float *xs, int xstride,
                     const float *ss, int sstride, float (&acc)[NT]) {
    float us[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) us[t] = 0.0f;
#pragma unroll
    for (int g = 0; g < U::GROUPS; g++) {
        float s0[NT], s1[NT];
#pragma unroll
        for (int t = 0; t < NT; t++) { s0[t] = 0.0f; s1[t] = 0.0f; }
        // s0 sums the group's first half, s1 its second (dcode scale dfix)
#pragma unroll
        for (int k = 0; k < U::GSIZE / 4; k++) {
            const int i = g * U::GSIZE + 4 * k;
            const float q0 = U::dcode(w, i), q1 = U::dcode(w, i + 1);
            const float q2 = U::dcode(w, i + 2), q3 = U::dcode(w, i + 3);
#pragma unroll
            for (int t = 0; t < NT; t++) {
                const f32x4 xv = *(const f32x4 *)(xs + t * xstride + i + ((i >> 6) << 2));
                float &s = (k >= U::GSIZE / 8) ? s1[t] : s0[t];
                s = fmaf(q0, xv.x, s);
                s = fmaf(q1, xv.y, s);
                s = fmaf(q2, xv.z, s);
                s = fmaf(q3, xv.w, s);
            }
        }
#pragma unroll
        for (int t = 0; t < NT; t++)
            us[t] += U::fold(w, g, fmaf(s1[t], U::dfix(g, 1), s0[t] * U::dfix(g, 0)),
                             U::SUMS ? ss[t * sstride + g] : 0.0f);
        // decode group by group: keeps a block's codes from all being live at once
        if constexpr (U::GROUPS > 2) {
            // finish this group's sums before the next group's x reads start
#pragma unroll
            for (int t = 0; t < NT; t++) asm volatile("" : "+v"(us[t])::"memory");
        }
    }
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t] += us[t];
}

// The same sums for one token with the unit's x values already in registers
// (xr[k] = x[4k .. 4k+3] of the unit), so all of a unit's LDS reads can be in
// flight together before the arithmetic starts.
template <class U>
QG_DEV void unit_dot_x(const u32 (&w)[U::ND], const f32x4 (&xr)[U::VALUES / 4], const float *ss, float &acc) {
    float us = 0.0f;
#pragma unroll
    for (int g = 0; g < U::GROUPS; g++) {
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int k = 0; k < U::GSIZE / 4; k++) {
            const int i = g * U::GSIZE + 4 * k;
            const f32x4 xv = xr[i >> 2];
            float &s = (k >= U::GSIZE / 8) ? s1 : s0;
            s = fmaf(U::dcode(w, i), xv.x, s);
            s = fmaf(U::dcode(w, i + 1), xv.y, s);
            s = fmaf(U::dcode(w, i + 2), xv.z, s);
            s = fmaf(U::dcode(w, i + 3), xv.w, s);
        }
        us += U::fold(w, g, fmaf(s1, U::dfix(g, 1), s0 * U::dfix(g, 0)), U::SUMS ? ss[g] : 0.0f);
    }
    acc += us;
}

// ---- staging x[t] into LDS, zero-padded from cols to cpad ----
// Vector path (a.x_vec: every source row 16-byte aligned, cols a multiple of
// 32): batches of XB float4 per thread; the group sums the folding formats
// need (SUMS consecutive values) are reduced across the SUMS/4 lanes holding
// them while the batch is in registers.
constexpr int XB = 8;

QG_DEV void x_load(const float *src, int base0, int c4, f32x4 (&v)[XB]) {
#pragma unroll
    for (int b = 0; b < XB; b++) v[b] = ((const f32x4 *)src)[min(base0 + (int)threadIdx.x + 256 * b, c4 - 1)];
}

template <int SUMS>
QG_DEV void x_put(const f32x4 (&v)[XB], int base0, int n4, int c4, float *xt, float *st) {
#pragma unroll
    for (int b = 0; b < XB; b++) {
        const int i = base0 + (int)threadIdx.x + 256 * b;
        const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
        const f32x4 val = i < c4 ? v[b] : z;
        if constexpr (SUMS != 0) {
            // every lane takes part; n4 is a multiple of SUMS/4, so a lane
            // group is wholly inside or wholly past the row
            const float g = group_sum<SUMS / 4>((val.x + val.y) + (val.z + val.w));
            if (i < n4 && (i & (SUMS / 4 - 1)) == 0) st[(4 * i) / SUMS] = g;
        }
        if (i < n4) *(f32x4 *)(xt + xpad(4 * i)) = val;
    }
}

// Scalar path (unaligned x): element by element, then the sums from LDS.
template <int NT, int SUMS>
QG_DEV void stage_x_scalar(const GemvArgs &a, const int (&in_idx)[NT], int cols, int cpad, float *xs, int xstride,
                           float *ss, int nsum) {
    for (int t = 0; t < NT; t++) {
        const float *src = a.x + (int64_t)in_idx[t] * a.x_stride;
        for (int c = threadIdx.x; c < cpad; c += 256) xs[t * xstride + xpad(c)] = c < cols ? src[c] : 0.0f;
    }
    if constexpr (SUMS != 0) {
        __syncthreads();
        for (int i = threadIdx.x; i < NT * nsum; i += 256) {
            const int t = i / nsum, gi = i - t * nsum;
            const float *p = xs + t * xstride + xpad(gi * SUMS);  // SUMS divides 64: no pad inside
            float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
            for (int j = 0; j < SUMS; j += 2) { s0 += p[j]; s1 += p[j + 1]; }
            ss[t * nsum + gi] = s0 + s1;
        }
    }
}

// Units in flight per lane: about 72 dwords of loads (the decode and the
// accumulators need the rest of the register file).
template <class U, int NT>
constexpr int pipe_depth() {
    return (U::NR >= 36) ? 2 : (72 / U::NR > 8 ? 8 : 72 / U::NR) / (NT >= 4 ? 2 : 1);
}

// ------------------------------------------------------------ GEMV kernel --
// One kernel for every block type, dense or expert-grouped, T = 1..16 tokens.
//   grid.x: row tiles, grid-stride (tile = 4 waves x RPW rows, RPW = 64/L);
//   grid.y: dense token chunk, or expert group;  grid.z: grouped token chunk.
// Each lane runs one stream of elements (row tile p, unit slot j): unit
// u = sub + j*L of row (tile's rows) + grp, across all the wave's tiles, with
// D elements' loads always in flight.  Lanes past the row's last unit, and
// rows past the matrix's last row, re-load a valid unit (a cache hit) and do
// not compute, so every load is unconditional and in bounds.  The first D
// elements' loads are issued before x is staged, so weight latency overlaps
// the staging.  In gated mode a tile's slots run over its gate rows' units
// and then over the same rows of the up matrix, and the row outputs are
// act(gate) * up.
template <class U, int L, int NT>
__global__ __launch_bounds__(256) void k_gemv(GemvArgs a) {
    extern __shared__ float lds[];
    constexpr int RPW = 64 / L;
    constexpr int UV = U::VALUES;
    constexpr int SUMS = U::SUMS;
    constexpr int SPU = SUMS ? UV / SUMS : 0;
    constexpr int D = pipe_depth<U, NT>();

    // ---- which vectors this workgroup serves, and which weights ----
    const uint8_t *Wg0 = a.W0, *Wg1 = a.W1;
    int nt;
    int in_idx[NT], out_idx[NT];
    float osc_e[NT], osc_p[NT];   // output scales (1 unless a grouped launch sets them)
    if (a.grp) {
        const int G = a.grp[0];
        const int g = blockIdx.y;
        if (g >= G) return;
        const int *rec = a.grp + 1 + g * GREC;
        const int n = rec[2];
        const int c0 = blockIdx.z * NT;
        if (c0 >= n) return;
        nt = min(NT, n - c0);
        Wg0 = a.W0 + (int64_t)rec[1] * a.slot_stride;
        Wg1 = a.glu ? Wg0 + a.rows * a.row_bytes : Wg0;   // up rows follow the gate rows
        const float es = a.escale ? a.escale[rec[0]] : 1.0f;
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const int i = c0 + min(t, nt - 1);
            in_idx[t] = a.in_by_pair ? rec[19 + i] : rec[3 + i];
            out_idx[t] = rec[19 + i];
            osc_e[t] = es;
            osc_p[t] = a.pscale ? a.pscale[out_idx[t]] : 1.0f;
        }
    } else {
        const int c0 = blockIdx.y * NT;
        nt = min(NT, a.ntok - c0);
#pragma unroll
        for (int t = 0; t < NT; t++) {
            in_idx[t] = out_idx[t] = c0 + min(t, nt - 1);
            osc_e[t] = osc_p[t] = 1.0f;
        }
    }

    // ---- descriptors over the two weight ranges (tensor start aligned down) ----
    const u32 ph0 = (u32)((uintptr_t)Wg0 & 3u), ph1 = (u32)((uintptr_t)Wg1 & 3u);
    const rsrc_t rs0 = make_rsrc(Wg0 - ph0, (u32)((ph0 + a.bytes0 + 3) & ~(int64_t)3));
    const rsrc_t rs1 = make_rsrc(Wg1 - ph1, (u32)((ph1 + a.bytes1 + 3) & ~(int64_t)3));

    // ---- the lane's element stream ----
    // the wave index is uniform; saying so keeps the descriptors in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int grp = lane / L, sub = lane % L;
    const int K = (a.nunits + L - 1) / L;     // unit slots per lane per row and matrix
    const int KT = a.glu ? 2 * K : K;         // slots per row tile
    const int P = ((int)a.ntiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    const int S = P * KT;
    const int64_t rows = a.rows, rows0 = a.rows0;
    const int64_t rb = a.row_bytes;

    // element (p, j) -> descriptor + byte offset of the unit to load
    auto locate = [&](int p, int j, u32 &off) -> bool {  // returns: from range 1
        const int64_t tile = (int64_t)blockIdx.x + (int64_t)p * gridDim.x;
        const int64_t r0 = (tile * 4 + wave) * RPW;
        const int64_t r = min(r0 + grp, rows - 1);
        bool hi;
        int64_t rl;
        int jj = j;
        if (a.glu) {             // slots [0, K): gate row r; [K, 2K): up row r
            hi = j >= K;
            jj = hi ? j - K : j;
            rl = r;
        } else {                 // waves never straddle rows0
            hi = rows0 < rows && r0 >= rows0;
            rl = hi ? r - rows0 : r;
        }
        const int u = min(sub + jj * L, a.nunits - 1);
        off = (hi ? ph1 : ph0) + (u32)(rl * rb) + (u32)u * U::BYTES;
        return hi;
    };

    // ---- x: the first batch of the first vector goes out before the
    //      weights, so that waiting for it does not wait for them ----
    const int cols = a.cols;
    const int cpad = a.nunits * UV;
    const int xstride = xstride_of(cpad);
    const int nsum = SUMS ? cpad / SUMS : 0;
    const int n4 = cpad >> 2, c4 = cols >> 2;
    float *xs = lds;
    float *ss = lds + NT * xstride;
    f32x4 xv[XB];
    if (a.x_vec) x_load(a.x + (int64_t)in_idx[0] * a.x_stride, 0, c4, xv);
    __builtin_amdgcn_sched_barrier(0);

    u32 w[D][U::NR];     // raw dwords of the units in flight
    u32 woff[D];         // and their byte offsets (the re-alignment shift)
    // issue pointer (element s + D), compute pointer (element s)
    int ip = 0, ij = 0, cp = 0, cj = 0;
#pragma unroll
    for (int d = 0; d < D; d++) {
        u32 off;
        const int sp = min(ip, P - 1), sj = ip < P ? ij : KT - 1;   // past the end: re-load the last element
        const bool hi = locate(sp, sj, off);
        U::issue(hi ? rs1 : rs0, off, w[d]);
        woff[d] = off;
        if (++ij == KT) { ij = 0; ++ip; }
        // keep the issue order: slot d's loads go out before slot d+1's
        __builtin_amdgcn_sched_barrier(0);
    }

    // ---- the rest of x, and the group sums ----
    if (a.x_vec) {
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const float *src = a.x + (int64_t)in_idx[t] * a.x_stride;
            for (int base0 = 0; base0 < n4; base0 += 256 * XB) {
                if (t != 0 || base0 != 0) x_load(src, base0, c4, xv);
                x_put<SUMS>(xv, base0, n4, c4, xs + t * xstride, ss + t * nsum);
            }
        }
    } else {
        stage_x_scalar<NT, SUMS>(a, in_idx, cols, cpad, xs, xstride, ss, nsum);
    }
    __syncthreads();

    float acc[NT], gate[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) { acc[t] = 0.0f; gate[t] = 0.0f; }
    // one element: consume slot d, refill it with element s + D, and close the
    // row (or its gate half) when its last unit slot has been consumed
    auto element = [&](u32 (&ws)[U::NR], u32 &wo) {
        const int64_t tile = (int64_t)blockIdx.x + (int64_t)cp * gridDim.x;
        const int64_t r0 = (tile * 4 + wave) * RPW;
        const int u = sub + (cj >= K ? cj - K : cj) * L;
        if (u < a.nunits) {
            u32 wd[U::ND];
            U::prep(ws, wo, wd);
            unit_dot<U, NT>(wd, xs + xpad(u * UV), xstride, ss + u * SPU, nsum, acc);
        }
        // this element's arithmetic is done before the next element's decode
#pragma unroll
        for (int t = 0; t < NT; t++) asm volatile("" : "+v"(acc[t])::"memory");
        // the slot is consumed before it is refilled, and the refill is issued
        // before the next slot is consumed
        __builtin_amdgcn_sched_barrier(0);
        {
            u32 off;
            const int sp = min(ip, P - 1), sj = ip < P ? ij : KT - 1;  // past the end: re-load the last element
            const bool hi = locate(sp, sj, off);
            U::issue(hi ? rs1 : rs0, off, ws);
            wo = off;
            if (++ij == KT) { ij = 0; ++ip; }
        }
        __builtin_amdgcn_sched_barrier(0);
        ++cj;
        if (a.glu && cj == K) {   // gate half done: keep its row sums
#pragma unroll
            for (int t = 0; t < NT; t++) {
                gate[t] = group_sum<L>(acc[t]);
                acc[t] = 0.0f;
            }
        }
        if (cj == KT) {  // end of this tile's row: reduce over the row's L lanes and store
            cj = 0;
            ++cp;
#pragma unroll
            for (int t = 0; t < NT; t++) acc[t] = group_sum<L>(acc[t]);
            const int64_t r = r0 + grp;
            if (sub == 0 && r < rows) {
#pragma unroll
                for (int t = 0; t < NT; t++) {
                    if (t < nt) {
                        if (a.glu) {
                            a.y[(int64_t)out_idx[t] * a.y_stride + r] = glu(a.glu, gate[t], acc[t]);
                            if (a.y2) {
                                a.y2[(int64_t)out_idx[t] * a.y2_stride + r] = gate[t];
                                a.y2[(int64_t)out_idx[t] * a.y2_stride + rows + r] = acc[t];
                            }
                        } else {
                            a.y[(int64_t)out_idx[t] * a.y_stride + r] = (acc[t] * osc_e[t]) * osc_p[t];
                        }
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < NT; t++) acc[t] = 0.0f;
        }
    };
    // full rounds of D elements (no per-slot conditions), then the tail
    int s0 = 0;
    for (; s0 + D <= S; s0 += D) {
#pragma unroll
        for (int d = 0; d < D; d++) element(w[d], woff[d]);
    }
#pragma unroll
    for (int d = 0; d < D; d++)
        if (s0 + d < S) element(w[d], woff[d]);
}

// ------------------------------------------- GEMV, weights staged in LDS ---
// The same element stream as k_gemv, but a wave's weights reach it through
// LDS: for element (tile p, slot j) the wave needs, for each of its RPW rows,
// the L consecutive units [jL, jL+L) -- one contiguous segment of L*BYTES
// bytes per row, 16-byte aligned when rows and the tensor are.  Those
// segments are copied HBM -> LDS with 16-byte buffer-to-LDS loads whose lanes
// take consecutive 16-byte pieces of each segment, so every load instruction
// reads whole cache lines; lane (grp, sub) then finds its unit at byte
// lane*BYTES of the stage.  Each wave owns a ring of `depth` stages; a stage
// is refilled as soon as its unit has been read into registers, so `depth`
// stages stay in flight while the unit is decoded.  The waits on the
// buffer-to-LDS loads are explicit vmcnt waits (the compiler does not track
// them); y stores in between only make those waits stricter.
template <class U, bool ALN>
QG_DEV void lds_unit(const uint8_t *stage, u32 off, u32 (&wd)[U::ND]) {
    if constexpr (!ALN) {   // any 2-byte phase: aligned dwords, shifted into place
        const u32 *p = (const u32 *)(stage + (off & ~3u));
        u32 t[U::ND + 1];
#pragma unroll
        for (int i = 0; i <= U::ND; i++) t[i] = p[i];
        realign<U::ND>(t, off, wd);
    } else if constexpr (U::BYTES % 16 == 0) {
        const u32x4 *p = (const u32x4 *)(stage + off);
#pragma unroll
        for (int i = 0; i < U::ND / 4; i++) {
            const u32x4 v = p[i];
            wd[4 * i] = v.x; wd[4 * i + 1] = v.y; wd[4 * i + 2] = v.z; wd[4 * i + 3] = v.w;
        }
    } else if constexpr (U::BYTES % 4 == 0) {
        const u32 *p = (const u32 *)(stage + off);
#pragma unroll
        for (int i = 0; i < U::ND; i++) wd[i] = p[i];
    } else {
        const u32 *p = (const u32 *)(stage + (off & ~3u));
        u32 t[U::NR];
#pragma unroll
        for (int i = 0; i < U::NR; i++) t[i] = p[i];
        U::prep(t, off, wd);
    }
}

// s_waitcnt vmcnt(n) (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and
// lgkmcnt left at their maxima, i.e. not waited on)
#define QG_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
#define QG_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)

template <int NI>
QG_DEV void wait_stages(int k) {   // at most k stages (NI loads each) still in flight
    switch (k) {
    case 0: QG_WAIT_VM(0); break;
    case 1: QG_WAIT_VM(NI); break;
    case 2: QG_WAIT_VM(2 * NI); break;
    default: QG_WAIT_VM(3 * NI); break;
    }
}

// A stage: for each of the wave's RPW rows, SEGP 16-byte pieces from the
// segment's 16-byte-aligned start (one more than the segment's own when the
// segment may start mid-piece).
template <class U, int L, bool ALN>
struct StageGeom {
    static constexpr int RPW = 64 / L;
    static constexpr int SEG = L * U::BYTES / 16;         // pieces per row segment
    static constexpr int SEGP = SEG + (ALN ? 0 : 1);      // pieces fetched per row
    static constexpr int PIECES = RPW * SEGP;
    static constexpr int NI = (PIECES + 63) / 64;         // load instructions per stage
    static constexpr int LAST = PIECES - 64 * (NI - 1);   // lanes active in the last one
    static constexpr int STAGE = NI * 1024;               // stage bytes in LDS
};

template <class U, int L, int NT, bool ALN>
__global__ __launch_bounds__(256) void k_gemv_lds(GemvArgs a) {
    extern __shared__ float lds[];
    constexpr int RPW = 64 / L;
    constexpr int UV = U::VALUES;
    constexpr int SUMS = U::SUMS;
    constexpr int SPU = SUMS ? UV / SUMS : 0;
    typedef StageGeom<U, L, ALN> G;
    constexpr int SEGP = G::SEGP;
    static_assert((L * U::BYTES) % 16 == 0, "row segments must be whole 16-byte pieces");
    static_assert(3 * G::NI <= 63, "vmcnt range");

    // ---- which vectors this workgroup serves, and which weights ----
    const uint8_t *Wg0 = a.W0, *Wg1 = a.W1;
    int nt;
    int in_idx[NT], out_idx[NT];
    float osc_e[NT], osc_p[NT];   // output scales (1 unless a grouped launch sets them)
    if (a.grp) {
        const int Gn = a.grp[0];
        const int g = blockIdx.y;
        if (g >= Gn) return;
        const int *rec = a.grp + 1 + g * GREC;
        const int n = rec[2];
        const int c0 = blockIdx.z * NT;
        if (c0 >= n) return;
        nt = min(NT, n - c0);
        Wg0 = a.W0 + (int64_t)rec[1] * a.slot_stride;
        Wg1 = a.glu ? Wg0 + a.rows * a.row_bytes : Wg0;   // up rows follow the gate rows
        const float es = a.escale ? a.escale[rec[0]] : 1.0f;
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const int i = c0 + min(t, nt - 1);
            in_idx[t] = a.in_by_pair ? rec[19 + i] : rec[3 + i];
            out_idx[t] = rec[19 + i];
            osc_e[t] = es;
            osc_p[t] = a.pscale ? a.pscale[out_idx[t]] : 1.0f;
        }
    } else {
        const int c0 = blockIdx.y * NT;
        nt = min(NT, a.ntok - c0);
#pragma unroll
        for (int t = 0; t < NT; t++) {
            in_idx[t] = out_idx[t] = c0 + min(t, nt - 1);
            osc_e[t] = osc_p[t] = 1.0f;
        }
    }
    // descriptors from the ranges' 16-byte-aligned starts (ALN: the ranges,
    // their rows and segments all start 16-byte aligned; the host checks).
    // The range check works on whole loads, so each range is rounded up to
    // the 16-byte piece holding its last byte (that piece lies in the same
    // page as the byte, so reading it is safe; the bytes past the end are
    // never decoded).
    const u32 ph0 = ALN ? 0u : (u32)((uintptr_t)Wg0 & 15u), ph1 = ALN ? 0u : (u32)((uintptr_t)Wg1 & 15u);
    const rsrc_t rs0 = make_rsrc(Wg0 - ph0, (u32)((ph0 + a.bytes0 + 15) & ~(int64_t)15));
    const rsrc_t rs1 = make_rsrc(Wg1 - ph1, (u32)((ph1 + a.bytes1 + 15) & ~(int64_t)15));

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int grp = lane / L, sub = lane % L;
    const int K = (a.nunits + L - 1) / L;
    const int KT = a.glu ? 2 * K : K;
    const int P = ((int)a.ntiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    const int S = P * KT;
    const int D = a.depth;
    const int64_t rows = a.rows, rows0 = a.rows0;
    const u32 rb = (u32)a.row_bytes;
    uint8_t *ring = (uint8_t *)lds + a.ring_off + wave * D * G::STAGE;

    // this lane's pieces: row within the wave's rows, byte within the segment
    int prow[G::NI];
    u32 poff[G::NI];
#pragma unroll
    for (int c = 0; c < G::NI; c++) {
        const int pc = min(c * 64 + lane, G::PIECES - 1);
        prow[c] = pc / SEGP;
        poff[c] = (u32)(pc % SEGP) * 16u;
    }
    // copy element (p, j)'s segments into stage `slot`
    auto issue = [&](int p, int j, int slot) {
        const int64_t tile = (int64_t)blockIdx.x + (int64_t)p * gridDim.x;
        const int64_t r0 = (tile * 4 + wave) * RPW;
        bool hi;
        int jj = j;
        int64_t shift = 0;
        if (a.glu) {
            hi = j >= K;
            jj = hi ? j - K : j;
        } else {                 // waves never straddle rows0
            hi = rows0 < rows && r0 >= rows0;
            shift = hi ? rows0 : 0;
        }
        const rsrc_t rs = hi ? rs1 : rs0;
        const u32 seg = (u32)jj * (u32)(L * U::BYTES) + (hi ? ph1 : ph0);
        __attribute__((address_space(3))) void *dst =
            (__attribute__((address_space(3))) void *)(ring + slot * G::STAGE);
#pragma unroll
        for (int c = 0; c < G::NI; c++) {
            const int64_t r = min(r0 + prow[c], rows - 1) - shift;
            const u32 off = (((u32)r * rb + seg) & ~15u) + poff[c];
            if (c < G::NI - 1 || lane < G::LAST)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)
                                                         ((__attribute__((address_space(3))) uint8_t *)dst + c * 1024),
                                                         16, off, 0, 0, 0);
        }
    };

    // ---- x: the first batch goes out before the weights ----
    const int cols = a.cols;
    const int cpad = a.nunits * UV;
    const int xstride = xstride_of(cpad);
    const int nsum = SUMS ? cpad / SUMS : 0;
    const int n4 = cpad >> 2, c4 = cols >> 2;
    float *xs = lds;
    float *ss = lds + NT * xstride;
    f32x4 xv[XB];
    if (a.x_vec) x_load(a.x + (int64_t)in_idx[0] * a.x_stride, 0, c4, xv);
    __builtin_amdgcn_sched_barrier(0);

    // ---- the first `depth` stages ----
    int ip = 0, ij = 0;          // next element to issue
    for (int d = 0; d < D; d++) {
        if (ip < P) {
            issue(ip, ij, d);
            if (++ij == KT) { ij = 0; ++ip; }
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- the rest of x, and the group sums ----
    if (a.x_vec) {
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const float *src = a.x + (int64_t)in_idx[t] * a.x_stride;
            for (int base0 = 0; base0 < n4; base0 += 256 * XB) {
                if (t != 0 || base0 != 0) x_load(src, base0, c4, xv);
                x_put<SUMS>(xv, base0, n4, c4, xs + t * xstride, ss + t * nsum);
            }
        }
    } else {
        stage_x_scalar<NT, SUMS>(a, in_idx, cols, cpad, xs, xstride, ss, nsum);
    }
    __syncthreads();

    float acc[NT], gate[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) { acc[t] = 0.0f; gate[t] = 0.0f; }
    int cp = 0, cj = 0;          // element being consumed
    for (int s = 0; s < S; s++) {
        const int slot = s % D;
        // stage s has landed once no more than the later issued ones are in flight
        wait_stages<G::NI>(min(D - 1, S - 1 - s));
        u32 wd[U::ND];
        u32 uoff = (u32)lane * U::BYTES;   // where this lane's unit sits in the stage
        if constexpr (!ALN) {
            const int64_t tl = (int64_t)blockIdx.x + (int64_t)cp * gridDim.x;
            const int64_t rw0 = (tl * 4 + wave) * RPW;
            const bool hi = a.glu ? cj >= K : (rows0 < rows && rw0 >= rows0);
            const int64_t rr = min(rw0 + grp, rows - 1) - (!a.glu && hi ? rows0 : 0);
            const u32 jj = (u32)(a.glu && hi ? cj - K : cj);
            const u32 phase = ((u32)rr * rb + jj * (u32)(L * U::BYTES) + (hi ? ph1 : ph0)) & 15u;
            uoff = (u32)grp * (SEGP * 16) + phase + (u32)sub * U::BYTES;
        }
        lds_unit<U, ALN>(ring + slot * G::STAGE, uoff, wd);
        QG_WAIT_LGKM0();   // the unit is in registers: the stage can be refilled
        __builtin_amdgcn_sched_barrier(0);
        if (ip < P) {
            issue(ip, ij, slot);
            if (++ij == KT) { ij = 0; ++ip; }
        }
        __builtin_amdgcn_sched_barrier(0);
        const int64_t tile = (int64_t)blockIdx.x + (int64_t)cp * gridDim.x;
        const int64_t r0 = (tile * 4 + wave) * RPW;
        const int u = sub + (cj >= K ? cj - K : cj) * L;
        if constexpr (NT == 1 && UV <= 64) {
            // one token, 64-value units: all the unit's x reads go out at once
            const float *xp = xs + xpad(min(u, a.nunits - 1) * UV);
            f32x4 xr[UV / 4];
#pragma unroll
            for (int q = 0; q < UV / 4; q++) xr[q] = *(const f32x4 *)(xp + 4 * q);
            if (u < a.nunits) unit_dot_x<U>(wd, xr, ss + u * SPU, acc[0]);
        } else {
            if (u < a.nunits) unit_dot<U, NT>(wd, xs + xpad(u * UV), xstride, ss + u * SPU, nsum, acc);
        }
        ++cj;
        if (a.glu && cj == K) {   // gate half done: keep its row sums
#pragma unroll
            for (int t = 0; t < NT; t++) {
                gate[t] = group_sum<L>(acc[t]);
                acc[t] = 0.0f;
            }
        }
        if (cj == KT) {  // end of this tile's row: reduce over the row's L lanes and store
            cj = 0;
            ++cp;
#pragma unroll
            for (int t = 0; t < NT; t++) acc[t] = group_sum<L>(acc[t]);
            const int64_t r = r0 + grp;
            if (sub == 0 && r < rows) {
#pragma unroll
                for (int t = 0; t < NT; t++) {
                    if (t < nt) {
                        if (a.glu) {
                            a.y[(int64_t)out_idx[t] * a.y_stride + r] = glu(a.glu, gate[t], acc[t]);
                            if (a.y2) {
                                a.y2[(int64_t)out_idx[t] * a.y2_stride + r] = gate[t];
                                a.y2[(int64_t)out_idx[t] * a.y2_stride + rows + r] = acc[t];
                            }
                        } else {
                            a.y[(int64_t)out_idx[t] * a.y_stride + r] = (acc[t] * osc_e[t]) * osc_p[t];
                        }
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < NT; t++) acc[t] = 0.0f;
        }
    }
    // no buffer-to-LDS load may still be in flight when the wave ends
    QG_WAIT_VM(0);
}

// ------------------------------------------------------- dequantization ---
// One thread per block: out[r][c] = value of W[r][c] as f32, through the same
// loads and decoders as the GEMV (block units: any 2-byte phase).
template <class U>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t *W, float *out, int64_t rows, int cols,
                                                 int64_t row_bytes) {
    const int nbr = cols / U::VALUES;
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= rows * nbr) return;
    const int64_t r = id / nbr;
    const int b = (int)(id - r * nbr);
    const uint8_t *p = W + r * row_bytes + (int64_t)b * U::BYTES;
    const u32 ph = (u32)((uintptr_t)p & 3u);
    // descriptor over this block's dwords only
    const rsrc_t rs = make_rsrc(p - ph, (u32)(ph + U::BYTES + 3) & ~3u);
    u32 w[U::ND];
    U::load(rs, ph, w);
    float *o = out + r * cols + (int64_t)b * U::VALUES;
#pragma unroll
    for (int i = 0; i < U::VALUES; i++) o[i] = U::value(w, i);
}

// ------------------------------------------------------ instance tables ---
typedef void (*gemv_fn)(GemvArgs);
typedef void (*dequant_fn)(const uint8_t *, float *, int64_t, int, int64_t);
// Unit kinds: block units for every type; pair units for Q8_0 / Q4_0.
// UK_LDS: k_gemv_lds over pair units (Q8_0 / Q4_0) or the K-quant blocks,
// 16-byte aligned ranges and rows; UK_LDS2: the same for 2-byte alignment.
enum { UK_BLOCK = 0, UK_PAIR = 1, UK_LDS = 2, UK_LDS2 = 3 };
// One function per (block type, tokens per workgroup), each instantiated in
// its own translation unit (qg_inst_<type>_t<NT>.hip); returns the kernel for
// (unit kind, lanes per row).  qg_inst_dequant.hip holds the dequantizers.
#define QG_DECL_GEMV(NAME) \
    gemv_fn gemv_kernel_##NAME##_t1(int kind, int lpr); \
    gemv_fn gemv_kernel_##NAME##_t2(int kind, int lpr); \
    gemv_fn gemv_kernel_##NAME##_t4(int kind, int lpr); \
    gemv_fn gemv_kernel_##NAME##_t8(int kind, int lpr);
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
__global__ void k_combine(const float *dn, const int32_t *rt_valid, float *y, int64_t H, int k);

}  // namespace qg

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
// followed, when the host asked for them, by two set lists (one per chunk
// size c, for the gate-up and the down launch), each
//   [0]                     number of sets S
//   [1 + s]                 (g << 16) | c0: group g, its pairs c0 .. c0+c-1
// holding every (group, chunk) that carries pairs, groups ascending, so a
// launch over the list has no empty workgroups before the last set.
constexpr int GREC = 35;
constexpr int MAXT = 16;
// ints of a set list for `pairs` (token, pick) pairs
constexpr int set_list_ints(int pairs) { return 1 + pairs; }

struct GemvArgs {
    // weights: rows [0, rows) of W0 (grouped: W0 + slot * slot_stride for the
    // group's slot).  Gated pairs: gate rows from W0, the same up rows from W1
    // (grouped: the up rows follow the gate rows in the slot).
    const uint8_t *W0, *W1;
    int64_t rows, row_bytes, slot_stride;
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
    const int *sets;   // grouped: the set list of this launch's chunk size
                       // (blockIdx.y = set), or nullptr (blockIdx.y = group,
                       // blockIdx.z = chunk)
    // a routing launch (RT) may carry xg_n extra groups after its r_k routed
    // ones (a shared expert, or the row slices of a dense MLP beside the
    // experts): group r_k + i takes its gate rows from xg_W0 + i * xg_step and
    // the same up rows from xg_W1 + i * xg_step (a routed expert's shape), its
    // input from xg_x, and writes act(g) * u to xg_y + i * rows and the raw
    // g, u to xg_y2 + i * rows and xg_y2 + xg_up + i * rows
    const uint8_t *xg_W0, *xg_W1;
    int64_t xg_step, xg_up;
    const float *xg_x;
    float *xg_y, *xg_y2;
    int xg_n;
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
    // k_gemv_lds: x is staged in chunks of this many row elements (units of
    // L lanes), restaged as each tile row reaches the next chunk; 0 = all of x
    int xchunk;
    // prefill chunks split along the row (k_gemm_mfma): workgroup z of grid.z
    // sums k-chunks [z * kchunks, (z + 1) * kchunks) and writes its raw sums
    // to part + (z * ptok + t) * prow + r (gated: up sums at prow / 2 + r);
    // part == nullptr: one split, results written to y as usual
    float *part;
    int kchunks;
    int64_t ptok, prow;
    // prefill chunks: x split into bf16 parts by k_split_x (device scratch)
    const uint8_t *xs;
    // caller scratch for prefill chunks: split x, then partial sums
    uint8_t *ws;
    size_t ws_bytes;
    // prefill chunks: the logical grid (row tiles x token tiles x splits)
    // behind the 1-D launch
    int wg_x, wg_y, wg_z;
    // grouped launch routing its one token itself (r_logits set): router
    // logits [r_E], top r_k, expert -> slot; workgroup (0, 0, 0) writes the
    // routing outputs (ids, weights, validity, status, the group table)
    const float *r_logits;
    int r_E, r_k, r_nslots;
    const int32_t *r_slots;
    int32_t *r_ids_out, *r_status, *r_ids, *r_valid, *r_grp;
    float *r_w_out, *r_w;
    // and, for the one-token down launch, each pick's pool slot and down
    // scale (r_escale[id], 1 without one) in pick order, when r_pslot is set
    const float *r_escale;
    int32_t *r_pslot;
    float *r_pes;
    // and, with a shared expert riding in the launch, its gate logit
    // r_gate_inp . x (cols values), written to r_gate_out[0] when set
    const float *r_gate_inp;
    float *r_gate_out;
};

// ------------------------------------------- one token's routing in-launch --
// Every wave selects the top k of the router logits itself (the keys, the
// lowest index among equal keys and the weights of k_route), so no routing
// launch precedes the expert launches.  Group g is the pick with the g-th
// smallest expert id, the order k_route's group table lists them in.  The
// lead workgroup writes what k_route writes for one token.
constexpr int ROUTE1_MAXK = 8;

struct Route1 {        // this lane's share of the router inputs (E <= 256)
    float lv[4];       // logit of expert lane + 64 i (0 past E)
    int sl[4];         // its pool slot (-1 past E)
    float es[4];       // its down scale (1 past E, without one, or unasked)
};

// Issued as early as possible: nothing else in the launch depends on less.
QG_DEV void route1_load(const GemvArgs &a, Route1 &r) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int e = lane + 64 * i;
        r.lv[i] = e < a.r_E ? a.r_logits[e] : 0.0f;
        r.sl[i] = e < a.r_E ? a.r_slots[e] : -1;
        r.es[i] = (a.r_pslot && a.r_escale && e < a.r_E) ? a.r_escale[e] : 1.0f;
    }
}

// Value of lane `e & 63` of register set (e >> 6), e wave-uniform: each set
// is read at that lane and the scalar results selected (a select over the
// sets themselves would become a dynamically indexed register array, which
// the compiler keeps in scratch memory).
QG_DEV int pick_lane_i(const int (&v)[4], int e) {
    const int ln = e & 63, hi = e >> 6;
    const int r0 = __builtin_amdgcn_readlane(v[0], ln), r1 = __builtin_amdgcn_readlane(v[1], ln);
    const int r2 = __builtin_amdgcn_readlane(v[2], ln), r3 = __builtin_amdgcn_readlane(v[3], ln);
    return hi == 0 ? r0 : hi == 1 ? r1 : hi == 2 ? r2 : r3;
}
QG_DEV float pick_lane_f(const float (&v)[4], int e) {
    const int (&vi)[4] = reinterpret_cast<const int (&)[4]>(v);
    return __builtin_bit_cast(float, pick_lane_i(vi, e));
}

// The k picks in pick order, held across lanes: lane j < k gets pick j's
// expert id and pool slot (other lanes keep 0).  One rolled round per pick
// (the code runs once per wave, so its size, not its count of operations,
// sets its time: every instruction line it spans is fetched from memory
// while the weight streams fill the caches).  Returns false when a pick has
// no pool slot.
struct Picked {
    int id, slot;   // this lane's pick (lane < k)
    bool ok;        // every pick has a slot
};
QG_DEV Picked route1_pick(const GemvArgs &a, const Route1 &r) {
    const int lane = threadIdx.x & 63;
    const int E = a.r_E, k = a.r_k;
    u32 key[4];
    u32 taken = 0u;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        key[i] = order_key(r.lv[i]);
        if (lane + 64 * i >= E) taken |= 1u << i;
    }
    Picked p = {0, 0, true};
#pragma unroll 1
    for (int j = 0; j < k; j++) {
        u32 lm = 0u;
#pragma unroll
        for (int i = 0; i < 4; i++)
            if (!((taken >> i) & 1u)) lm = max(lm, key[i]);
        const u32 M = wave_max_u32(lm);
        int e = -1;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const unsigned long long b = __ballot(!((taken >> i) & 1u) && key[i] == M);
            if (e < 0 && b) e = 64 * i + (int)__builtin_ctzll(b);
        }
        e = __builtin_amdgcn_readfirstlane(e);
        if ((e & 63) == lane) taken |= 1u << (e >> 6);
        const int sl = pick_lane_i(r.sl, e);
        if (lane == j) { p.id = e; p.slot = sl; }
        p.ok = p.ok && sl >= 0 && sl < a.r_nslots;
    }
    return p;
}

// Pick j's expert id and slot (j wave-uniform)
QG_DEV int pick_id(const Picked &p, int j) { return __builtin_amdgcn_readlane(p.id, j); }
QG_DEV int pick_slot(const Picked &p, int j) { return __builtin_amdgcn_readlane(p.slot, j); }

// Value of expert `e` (per lane) from a per-expert vector held as register
// sets v[i] = entry lane + 64 i: every set read at lane e & 63, then set
// e >> 6 selected
QG_DEV float expert_value(const float (&v)[4], int e) {
    const int src = (e & 63) << 2, hi = e >> 6;
    const int c0 = __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, v[0]));
    const int c1 = __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, v[1]));
    const int c2 = __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, v[2]));
    const int c3 = __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, v[3]));
    return __builtin_bit_cast(float, hi == 0 ? c0 : hi == 1 ? c1 : hi == 2 ? c2 : c3);
}

// Lane j < k gets w_j = exp(l_j - l_0) / sum over the picks (the same
// operations in every wave, so every wave holds the same bits).
QG_DEV float route1_weight(const Route1 &r, const Picked &p, int k) {
    const int lane = threadIdx.x & 63;
    const float l0 = pick_lane_f(r.lv, pick_id(p, 0));
    const float lj = expert_value(r.lv, p.id);
    const float ex = lane < k ? expf(lj - l0) : 0.0f;
    return ex / wave_sum(ex);
}

// Lane j < k gets the rank of pick j among the picks' expert ids (distinct)
QG_DEV int route1_rank(const Picked &p, int k) {
    int rank = 0;
#pragma unroll 1
    for (int i = 0; i < k; i++) rank += pick_id(p, i) < p.id ? 1 : 0;
    return rank;
}

// The routing outputs of one token (ids, weights, validity, status, the
// group table), written by the lead workgroup's first wave.
QG_DEV void route1_write(const GemvArgs &a, const Route1 &r, const Picked &p, int rank) {
    const int lane = threadIdx.x & 63;
    const int k = a.r_k;
    const float wj = route1_weight(r, p, k);
    const float es = expert_value(r.es, p.id);
    if (lane < k) {
        if (a.r_pslot) {
            a.r_pslot[lane] = p.slot;
            a.r_pes[lane] = es;
        }
        a.r_ids[lane] = p.id;
        a.r_w[lane] = wj;
        if (a.r_ids_out) a.r_ids_out[lane] = p.id;
        if (a.r_w_out) a.r_w_out[lane] = wj;
        if (p.ok) {
            int *rec = a.r_grp + 1 + rank * GREC;
            rec[0] = p.id;
            rec[1] = p.slot;
            rec[2] = 1;
            rec[3] = 0;
            rec[19] = lane;
        }
    }
    if (lane == 0) {
        a.r_valid[0] = p.ok ? 1 : 0;
        if (a.r_status) a.r_status[0] = p.ok ? 0 : -2;   // QG_OK / QG_EABSENT
        a.r_grp[0] = p.ok ? k : 0;
    }
}

// Group g of a routing launch: its expert, slot and pick index.  Returns
// false when a pick has no pool slot (the token's groups are then empty).
QG_DEV bool route1_group(const GemvArgs &a, const Route1 &r, int g, bool lead, int &e_out, int &slot_out,
                         int &z_out) {
    const Picked p = route1_pick(a, r);
    const int lane = threadIdx.x & 63;
    const int rank = route1_rank(p, a.r_k);
    // the lane holding the pick of rank g
    const unsigned long long b = __ballot(lane < a.r_k && rank == g);
    const int z = b ? (int)__builtin_ctzll(b) : 0;
    z_out = z;
    e_out = pick_id(p, z);
    slot_out = pick_slot(p, z);
    if (lead && threadIdx.x < 64) route1_write(a, r, p, rank);
    return p.ok;
}

// The same for a whole workgroup: its first wave loads the router inputs and
// selects, the others take the result from LDS (selection is serial work,
// and every wave of a launch doing it at once would fill the vector units
// for microseconds).  In the lead workgroup the other three waves meanwhile
// reduce the shared expert's gate logit (when asked), in three parts added
// in a fixed order, so the down launch reads one value.  Call from every
// thread of a 256-thread workgroup, before any early return.
QG_DEV bool route1_group_wg(const GemvArgs &a, int g, bool lead, int &e_out, int &slot_out, int &z_out) {
    __shared__ int s_r[4];
    __shared__ float s_g[4];
    if (threadIdx.x >= 64 && lead && a.r_gate_out) {
        const int w = (int)(threadIdx.x >> 6) - 1, l = (int)threadIdx.x & 63;
        float gp = 0.0f;
        for (int c0 = 64 * w + l; c0 < a.cols; c0 += 192 * 8) {
            float gv[8], xv[8];
#pragma unroll
            for (int b = 0; b < 8; b++) {
                const bool in = c0 + 192 * b < a.cols;
                gv[b] = in ? a.r_gate_inp[c0 + 192 * b] : 0.0f;
                xv[b] = in ? a.x[c0 + 192 * b] : 0.0f;
            }
#pragma unroll
            for (int b = 0; b < 8; b++) gp = fmaf(gv[b], xv[b], gp);
        }
        gp = wave_sum(gp);
        if (l == 0) s_g[w] = gp;
    }
    if (threadIdx.x < 64) {
        Route1 r;
        route1_load(a, r);
        int e, sl, z;
        const bool ok = route1_group(a, r, g, lead, e, sl, z);
        if (threadIdx.x == 0) {
            s_r[0] = e;
            s_r[1] = sl;
            s_r[2] = z;
            s_r[3] = ok ? 1 : 0;
        }
    }
    __syncthreads();
    if (lead && a.r_gate_out && threadIdx.x == 0) a.r_gate_out[0] = (s_g[0] + s_g[1]) + s_g[2];
    e_out = __builtin_amdgcn_readfirstlane(s_r[0]);
    slot_out = __builtin_amdgcn_readfirstlane(s_r[1]);
    z_out = __builtin_amdgcn_readfirstlane(s_r[2]);
    return __builtin_amdgcn_readfirstlane(s_r[3]) != 0;
}

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

// One token, many scale groups (the K-quant blocks): the next group's x reads
// are issued before this group's arithmetic, so LDS latency hides behind it.
template <class U>
QG_DEV void unit_dot_pf(const u32 (&w)[U::ND], const float *xs, const float *ss, float &acc) {
    constexpr int Q = U::GSIZE / 4;          // float4 reads per group
    float us = 0.0f;
    f32x4 xn[Q];
#pragma unroll
    for (int k = 0; k < Q; k++) xn[k] = *(const f32x4 *)(xs + 4 * k);
#pragma unroll
    for (int g = 0; g < U::GROUPS; g++) {
        f32x4 xc[Q];
#pragma unroll
        for (int k = 0; k < Q; k++) xc[k] = xn[k];
        if (g + 1 < U::GROUPS) {
#pragma unroll
            for (int k = 0; k < Q; k++) {
                const int i = (g + 1) * U::GSIZE + 4 * k;
                xn[k] = *(const f32x4 *)(xs + i + ((i >> 6) << 2));
            }
        }
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int k = 0; k < Q; k++) {
            const int i = g * U::GSIZE + 4 * k;
            float &s = (k >= Q / 2) ? s1 : s0;
            s = fmaf(U::dcode(w, i), xc[k].x, s);
            s = fmaf(U::dcode(w, i + 1), xc[k].y, s);
            s = fmaf(U::dcode(w, i + 2), xc[k].z, s);
            s = fmaf(U::dcode(w, i + 3), xc[k].w, s);
        }
        us += U::fold(w, g, fmaf(s1, U::dfix(g, 1), s0 * U::dfix(g, 0)), U::SUMS ? ss[g] : 0.0f);
        // this group's sums close before the group after next is read
        asm volatile("" : "+v"(us)::"memory");
    }
    acc += us;
}

// The same sums for one token with the unit's x values already in registers
// (xr[k] = x[4k .. 4k+3] of the unit), so all of a unit's LDS reads can be in
// flight together before the arithmetic starts.
template <class U, int NS>
QG_DEV void unit_dot_x(const u32 (&w)[U::ND], const f32x4 (&xr)[U::VALUES / 4], const float (&ss)[NS], float &acc) {
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
// Columns [c0, c0 + cpad) of x land at xs[xpad(0..cpad)], zero past cols.
template <int NT, int SUMS>
QG_DEV void stage_x_scalar(const float *x, int64_t x_stride, const int (&in_idx)[NT], int cols, int cpad, float *xs,
                           int xstride, float *ss, int nsum, int c0 = 0) {
    for (int t = 0; t < NT; t++) {
        const float *src = x + (int64_t)in_idx[t] * x_stride;
        for (int c = threadIdx.x; c < cpad; c += 256)
            xs[t * xstride + xpad(c)] = c0 + c < cols ? src[c0 + c] : 0.0f;
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
    float *yo = a.y, *y2o = a.y2;  // where the rows go
    if (a.grp) {
        int g = blockIdx.y, c0 = blockIdx.z * NT;
        if (a.sets) {
            if ((int)blockIdx.y >= a.sets[0]) return;
            const int e = a.sets[1 + blockIdx.y];
            g = e >> 16;
            c0 = e & 0xffff;
        } else if (g >= a.grp[0]) {
            return;
        }
        const int *rec = a.grp + 1 + g * GREC;
        const int n = rec[2];
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
    const int64_t rows = a.rows;
    const int64_t rb = a.row_bytes;

    // element (p, j) -> descriptor + byte offset of the unit to load
    auto locate = [&](int p, int j, u32 &off) -> bool {  // returns: from W1
        const int64_t tile = (int64_t)blockIdx.x + (int64_t)p * gridDim.x;
        const int64_t r0 = (tile * 4 + wave) * RPW;
        const int64_t r = min(r0 + grp, rows - 1);
        // gated: slots [0, K) are gate row r, [K, 2K) up row r (uniform)
        const bool hi = __builtin_amdgcn_readfirstlane((int)(a.glu && j >= K)) != 0;
        const int jj = hi ? j - K : j;
        const int u = min(sub + jj * L, a.nunits - 1);
        off = (hi ? ph1 : ph0) + (u32)(r * rb) + (u32)u * U::BYTES;
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
        stage_x_scalar<NT, SUMS>(a.x, a.x_stride, in_idx, cols, cpad, xs, xstride, ss, nsum);
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
                            yo[(int64_t)out_idx[t] * a.y_stride + r] = glu(a.glu, gate[t], acc[t]);
                            if (y2o) {
                                y2o[(int64_t)out_idx[t] * a.y2_stride + r] = gate[t];
                                y2o[(int64_t)out_idx[t] * a.y2_stride + rows + r] = acc[t];
                            }
                        } else {
                            yo[(int64_t)out_idx[t] * a.y_stride + r] = (acc[t] * osc_e[t]) * osc_p[t];
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

// Q float4 of x from LDS byte address a, by asm (see lds_ldn)
template <int Q, int I = 0>
QG_DEV void load_x16(u32 a, f32x4 (&x)[Q]) {
    if constexpr (I < Q) {
        x[I] = lds_ld128f<16 * I>(a);
        load_x16<Q, I + 1>(a, x);
    }
}

// XC: x staged in chunks (restaged inside the element loop).  Kept apart from
// the whole-x variant: global loads inside the loop make the compiler wait for
// every load in flight, the stage copies included, at the unit reads.
// The body runs for workgroup (bx, by, bz) of a grid gdx wide along the
// rows, so a launch that also holds other work can run it under virtual
// coordinates; `lead` marks the workgroup that writes a routing launch's
// outputs (RT).
template <class U, int L, int NT, bool ALN, bool XC, bool RT>
QG_DEV void gemv_lds_body(const GemvArgs &a, int bx, int by, int bz, int gdx, bool lead) {
    static_assert(!RT || (NT == 1 && !XC), "a launch that routes its token serves one token, x unchunked");
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
    float *yo = a.y, *y2o = a.y2;  // where the rows go
    int64_t y2_up = a.rows;        // the raw up sums' offset after the gate sums
    const float *xsrc = a.x;       // the input vectors
    bool routed = false;
    if constexpr (RT) {
        if (a.xg_n > 0 && by >= a.r_k) {   // an extra group: a shared expert, or a dense MLP's row slice
            const int i = by - a.r_k;
            if (i >= a.xg_n || bz > 0) return;
            nt = 1;
            Wg0 = a.xg_W0 + (int64_t)i * a.xg_step;
            Wg1 = a.xg_W1 + (int64_t)i * a.xg_step;
            in_idx[0] = out_idx[0] = 0;
            osc_e[0] = osc_p[0] = 1.0f;
            xsrc = a.xg_x;
            yo = a.xg_y + (int64_t)i * a.rows;
            y2o = a.xg_y2 ? a.xg_y2 + (int64_t)i * a.rows : nullptr;
            y2_up = a.xg_up;
            routed = true;
        } else {   // this launch routes its one token itself
            int e, sl, z;
            const bool ok = route1_group_wg(a, by, lead, e, sl, z);
            if (!ok || by >= a.r_k || bz > 0) return;
            nt = 1;
            Wg0 = a.W0 + (int64_t)sl * a.slot_stride;
            Wg1 = a.glu ? Wg0 + a.rows * a.row_bytes : Wg0;   // up rows follow the gate rows
            in_idx[0] = a.in_by_pair ? z : 0;
            out_idx[0] = z;
            osc_e[0] = a.escale ? a.escale[e] : 1.0f;
            osc_p[0] = a.pscale ? a.pscale[z] : 1.0f;
            routed = true;
        }
    }
    if (routed) {
    } else if (a.grp) {
        int g = by, c0 = bz * NT;
        if (a.sets) {
            if (by >= a.sets[0]) return;
            const int e = a.sets[1 + by];
            g = e >> 16;
            c0 = e & 0xffff;
        } else if (g >= a.grp[0]) {
            return;
        }
        const int *rec = a.grp + 1 + g * GREC;
        const int n = rec[2];
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
        const int c0 = by * NT;
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
    Wg0 = uniform_ptr(Wg0);
    Wg1 = uniform_ptr(Wg1);
    const u32 ph0 = ALN ? 0u : (u32)((uintptr_t)Wg0 & 15u), ph1 = ALN ? 0u : (u32)((uintptr_t)Wg1 & 15u);
    const rsrc_t rs0 = make_rsrc(Wg0 - ph0, (u32)((ph0 + a.bytes0 + 15) & ~(int64_t)15));
    const rsrc_t rs1 = make_rsrc(Wg1 - ph1, (u32)((ph1 + a.bytes1 + 15) & ~(int64_t)15));

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int grp = lane / L, sub = lane % L;
    const int K = (a.nunits + L - 1) / L;
    const int KT = a.glu ? 2 * K : K;
    const int P = ((int)a.ntiles - bx + gdx - 1) / gdx;
    const int S = P * KT;
    const int D = a.depth;
    const int64_t rows = a.rows;
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
        const int64_t tile = (int64_t)bx + (int64_t)p * gdx;
        const int64_t r0 = (tile * 4 + wave) * RPW;
        // gated: [K, 2K) are the up rows (uniform; saying so keeps the
        // descriptor choice in scalar registers)
        const bool hi = __builtin_amdgcn_readfirstlane((int)(a.glu && j >= K)) != 0;
        const int jj = hi ? j - K : j;
        const rsrc_t rs = hi ? rs1 : rs0;
        const u32 seg = (u32)jj * (u32)(L * U::BYTES) + (hi ? ph1 : ph0);
        __attribute__((address_space(3))) void *dst =
            (__attribute__((address_space(3))) void *)(ring + slot * G::STAGE);
#pragma unroll
        for (int c = 0; c < G::NI; c++) {
            const int64_t r = min(r0 + prow[c], rows - 1);
            const u32 off = (((u32)r * rb + seg) & ~15u) + poff[c];
            if (c < G::NI - 1 || lane < G::LAST)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)
                                                         ((__attribute__((address_space(3))) uint8_t *)dst + c * 1024),
                                                         16, off, 0, 0, 0);
        }
    };

    // ---- x, staged whole or in chunks of JC row elements (JC*L units) ----
    const int cols = a.cols;
    const int JC = XC && a.xchunk > 0 ? a.xchunk : K;
    const int NCH = (K + JC - 1) / JC;
    const int ccols = JC * L * UV;                      // columns per chunk
    const int cpad = min(a.nunits, JC * L) * UV;        // staged span (the widest chunk)
    const int xstride = xstride_of(cpad);
    const int nsum = SUMS ? cpad / SUMS : 0;
    float *xs = lds;
    float *ss = lds + NT * xstride;
    const u32 xs_l = lds_off(xs), ss_l = lds_off(ss), ring_l = lds_off(ring);
    f32x4 xv[XB];
    // chunk ch: columns [ch*ccols, +cw) of the padded row, valid below cols
    // (the LDS kinds' padded width equals cols, so every chunk has valid x)
    auto chunk_w = [&](int ch) { return min(ccols, a.nunits * UV - ch * ccols); };
    auto stage = [&](int ch, bool first_loaded) {
        const int c0 = ch * ccols, cw = chunk_w(ch);
        const int n4 = cw >> 2, c4 = min(cols - c0, cw) >> 2;
        if (a.x_vec) {
#pragma unroll
            for (int t = 0; t < NT; t++) {
                const float *src = xsrc + (int64_t)in_idx[t] * a.x_stride + c0;
                for (int base0 = 0; base0 < n4; base0 += 256 * XB) {
                    if (!first_loaded || t != 0 || base0 != 0) x_load(src, base0, c4, xv);
                    x_put<SUMS>(xv, base0, n4, c4, xs + t * xstride, ss + t * nsum);
                }
            }
        } else {
            stage_x_scalar<NT, SUMS>(xsrc, a.x_stride, in_idx, cols, cw, xs, xstride, ss, nsum, c0);
        }
    };
    // the first batch of x goes out before the weights
    if (a.x_vec) x_load(xsrc + (int64_t)in_idx[0] * a.x_stride, 0, min(cols, chunk_w(0)) >> 2, xv);
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

    // ---- the rest of the first chunk, and its group sums ----
    stage(0, true);
    __syncthreads();

    float acc[NT], gate[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) { acc[t] = 0.0f; gate[t] = 0.0f; }
    int cp = 0, cj = 0;          // element being consumed
    for (int s = 0; s < S; s++) {
        const int slot = s % D;
        const int jm = cj >= K ? cj - K : cj;      // the element's place in its row
        if (XC && NCH > 1 && s > 0 && jm % JC == 0) {
            // every wave has finished with the previous chunk (all waves walk
            // the same element sequence, so they all meet here)
            __syncthreads();
            stage(jm / JC, false);
            __syncthreads();
        }
        const int ub = (jm / JC) * JC * L;         // first unit of the staged chunk
        // stage s has landed once no more than the later issued ones are in flight
        wait_stages<G::NI>(min(D - 1, S - 1 - s));
        u32 wd[U::ND];
        u32 uoff = (u32)lane * U::BYTES;   // where this lane's unit sits in the stage
        if constexpr (!ALN) {
            const int64_t tl = (int64_t)bx + (int64_t)cp * gdx;
            const int64_t rw0 = (tl * 4 + wave) * RPW;
            const bool hi = a.glu && cj >= K;
            const int64_t rr = min(rw0 + grp, rows - 1);
            const u32 jj = (u32)(hi ? cj - K : cj);
            const u32 phase = ((u32)rr * rb + jj * (u32)(L * U::BYTES) + (hi ? ph1 : ph0)) & 15u;
            uoff = (u32)grp * (SEGP * 16) + phase + (u32)sub * U::BYTES;
        }
        const int u = sub + jm * L;
        const int ul = u - ub;                     // its place in the staged chunk
        // one token, 64-value units: the unit's words, its x and its x-sums
        // are read by asm, so the copies of the later stages stay in flight
        // (the compiler would wait for every copy before any LDS read)
        constexpr bool XPF = NT == 1 && UV <= 64 && U::BYTES % 4 == 0;
        constexpr int NW = U::ND + (ALN ? 0 : 1);   // dwords read for the unit
        f32x4 xr[XPF ? UV / 4 : 1];
        float sv[U::GROUPS] = {};                 // x-sums of the unit's groups (SUMS formats)
        if constexpr (XPF) {
            u32 t[NW];
            lds_ldn<NW>(ring_l + slot * G::STAGE + (uoff & ~3u), t);
            load_x16<UV / 4>(xs_l + 4u * (u32)xpad((min(u, a.nunits - 1) - ub) * UV), xr);
            u32 sw[SUMS ? U::GROUPS : 1];
            if constexpr (SUMS != 0) lds_ldn<U::GROUPS>(ss_l + 4u * (u32)((min(u, a.nunits - 1) - ub) * SPU), sw);
            lds_wait();
#pragma unroll
            for (int i = 0; i < NW; i++) lds_ready(t[i]);
#pragma unroll
            for (int q = 0; q < UV / 4; q++) lds_ready(xr[q]);
            if constexpr (SUMS != 0) {
#pragma unroll
                for (int g = 0; g < U::GROUPS; g++) {
                    lds_ready(sw[g]);
                    sv[g] = __builtin_bit_cast(float, sw[g]);
                }
            }
            if constexpr (ALN) {
#pragma unroll
                for (int i = 0; i < U::ND; i++) wd[i] = t[i];
            } else {
                realign<U::ND>(t, uoff, wd);
            }
        } else {
            lds_unit<U, ALN>(ring + slot * G::STAGE, uoff, wd);
            QG_WAIT_LGKM0();   // the unit is in registers: the stage can be refilled
        }
        __builtin_amdgcn_sched_barrier(0);
        if (ip < P) {
            issue(ip, ij, slot);
            if (++ij == KT) { ij = 0; ++ip; }
        }
        __builtin_amdgcn_sched_barrier(0);
        const int64_t tile = (int64_t)bx + (int64_t)cp * gdx;
        const int64_t r0 = (tile * 4 + wave) * RPW;
        if constexpr (XPF) {
            if (u < a.nunits) unit_dot_x<U>(wd, xr, sv, acc[0]);
        } else if constexpr (NT == 1 && U::GROUPS > 2) {
            if (u < a.nunits) unit_dot_pf<U>(wd, xs + xpad(ul * UV), ss + ul * SPU, acc[0]);
        } else {
            if (u < a.nunits) unit_dot<U, NT>(wd, xs + xpad(ul * UV), xstride, ss + ul * SPU, nsum, acc);
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
                            float *py = yo + (int64_t)out_idx[t] * a.y_stride + r;
                            *py = glu(a.glu, gate[t], acc[t]);
                            if (y2o) {
                                y2o[(int64_t)out_idx[t] * a.y2_stride + r] = gate[t];
                                y2o[(int64_t)out_idx[t] * a.y2_stride + y2_up + r] = acc[t];
                            }
                        } else {
                            yo[(int64_t)out_idx[t] * a.y_stride + r] = (acc[t] * osc_e[t]) * osc_p[t];
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

template <class U, int L, int NT, bool ALN, bool XC, bool RT>
__global__ __launch_bounds__(256) void k_gemv_lds(GemvArgs a) {
    gemv_lds_body<U, L, NT, ALN, XC, RT>(a, (int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z, (int)gridDim.x,
                                         blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0);
}

// ------------------------------------------- small batch on the MFMA units ---
// T tokens (up to 16) against Q8_0 / Q4_0 rows with v_mfma_f32_16x16x32_bf16:
// per 32-value block, A (16 x 32) holds the tokens' x, B (32 x 16) sixteen
// rows' codes, and D[token][row] is accumulated as d_row * D into f32.  The
// products are exact: codes (int8, or nibble - 8) are small integers in bf16,
// and x enters as three bf16 parts whose sum is x exactly (truncation splits
// leave at most 16, then 8 significant bits), each part taking one MFMA.
// Lane l holds token l%16 / row l%16 of its fragments for k = 8(l/16)..+7
// (values 8q..8q+7 of the block: Q8_0 code bytes 2+8q.., Q4_0 low nibbles of
// code bytes 8(q&1).. for q < 2, high nibbles for q >= 2), and D rows (tokens)
// 4(l/16)..+3 of column (row) l%16.  A wave owns RG groups of 16 rows (gated:
// RG/2 gate groups and the same up groups); a workgroup is 4 waves.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// x = h + m + l exactly, each part a bf16 (truncation splits)
QG_DEV void split3(const f32x4 &x0, const f32x4 &x1, u32 (&h)[4], u32 (&m)[4], u32 (&l)[4]) {
    float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    u32 hb[8], mb[8], lb[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        hb[j] = __builtin_bit_cast(u32, x[j]) & 0xFFFF0000u;
        const float r = x[j] - __builtin_bit_cast(float, hb[j]);
        mb[j] = __builtin_bit_cast(u32, r) & 0xFFFF0000u;
        lb[j] = __builtin_bit_cast(u32, r - __builtin_bit_cast(float, mb[j]));
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {   // element 2j in the low half, 2j+1 in the high half
        h[j] = __builtin_amdgcn_perm(hb[2 * j + 1], hb[2 * j], 0x07060302u);
        m[j] = __builtin_amdgcn_perm(mb[2 * j + 1], mb[2 * j], 0x07060302u);
        l[j] = __builtin_amdgcn_perm(lb[2 * j + 1], lb[2 * j], 0x07060302u);
    }
}

QG_DEV bf16x8 as_bf16x8(const u32 (&v)[4]) {
    u32x4 t = {v[0], v[1], v[2], v[3]};
    return __builtin_bit_cast(bf16x8, t);
}

// 8 codes (as f32-exact integers) -> packed bf16 pairs
template <int TY>
QG_DEV void codes_bf16(u32 c0, u32 c1, int q, u32 (&o)[4]) {
    float f[8];
    if constexpr (TY == T_Q8_0) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            f[j] = (float)(int8_t)(c0 >> (8 * j));
            f[4 + j] = (float)(int8_t)(c1 >> (8 * j));
        }
    } else {
        const u32 m0 = opaque(q >= 2 ? (c0 >> 4) & 0x0F0F0F0Fu : c0 & 0x0F0F0F0Fu);
        const u32 m1 = opaque(q >= 2 ? (c1 >> 4) & 0x0F0F0F0Fu : c1 & 0x0F0F0F0Fu);
#pragma unroll
        for (int j = 0; j < 4; j++) {
            f[j] = u8_of(m0, j) - 8.0f;
            f[4 + j] = u8_of(m1, j) - 8.0f;
        }
    }
#pragma unroll
    for (int j = 0; j < 4; j++)
        o[j] = __builtin_amdgcn_perm(__builtin_bit_cast(u32, f[2 * j + 1]), __builtin_bit_cast(u32, f[2 * j]), 0x07060302u);
}

template <int TY, int RG>
__global__ __launch_bounds__(256) void k_gemv_mfma(GemvArgs a) {
    constexpr int BYTES = TY == T_Q8_0 ? 34 : 18;
    constexpr int GR = RG;                 // row groups of 16 rows per tile
    constexpr int PF = 2;                  // blocks in flight ahead of the one in use
    __shared__ int s_in[16], s_out[16];
    __shared__ float s_osc[16];
    __shared__ float s_red[4][GR * 4][64];   // per-wave partial sums

    // ---- which vectors this workgroup serves, and which weights ----
    const uint8_t *Wg0 = a.W0, *Wg1 = a.W1;
    int nt;
    float es = 1.0f;
    const int *rec = nullptr;
    int c0 = 0;
    if (a.grp) {
        int g = blockIdx.y;
        c0 = blockIdx.z * 16;
        if (a.sets) {
            if ((int)blockIdx.y >= a.sets[0]) return;
            const int e = a.sets[1 + blockIdx.y];
            g = e >> 16;
            c0 = e & 0xffff;
        } else if (g >= a.grp[0]) {
            return;
        }
        rec = a.grp + 1 + g * GREC;
        const int n = rec[2];
        if (c0 >= n) return;
        nt = min(16, n - c0);
        Wg0 = a.W0 + (int64_t)rec[1] * a.slot_stride;
        Wg1 = a.glu ? Wg0 + a.rows * a.row_bytes : Wg0;
        es = a.escale ? a.escale[rec[0]] : 1.0f;
    } else {
        c0 = blockIdx.y * 16;
        nt = min(16, a.ntok - c0);
    }
    if (threadIdx.x < 16) {
        const int t = threadIdx.x, i = c0 + min(t, nt - 1);
        if (rec) {
            s_in[t] = a.in_by_pair ? rec[19 + i] : rec[3 + i];
            s_out[t] = rec[19 + i];
            s_osc[t] = a.pscale ? a.pscale[rec[19 + i]] : 1.0f;
        } else {
            s_in[t] = s_out[t] = i;
            s_osc[t] = 1.0f;
        }
    }
    __syncthreads();

    // descriptors from the ranges' 4-byte-aligned starts, up to the dword that
    // holds the last byte (no load below reads past that dword)
    const u32 ph0 = (u32)((uintptr_t)Wg0 & 3u), ph1 = (u32)((uintptr_t)Wg1 & 3u);
    const rsrc_t rs0 = make_rsrc(Wg0 - ph0, (u32)((ph0 + a.bytes0 + 3) & ~(int64_t)3));
    const rsrc_t rs1 = make_rsrc(Wg1 - ph1, (u32)((ph1 + a.bytes1 + 3) & ~(int64_t)3));

    // the four waves split each row's blocks (wave w takes blocks w, w+4, ...)
    // and their partial sums are added in wave order at the tile's end.  A
    // split launch (dense, a.part set) gives workgroup z the blocks
    // [z kchunks, (z+1) kchunks) and stores the raw sums for the reduce.
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int n16 = lane & 15, q = lane >> 4;
    const int nb = a.cols / 32;
    const bool split = a.part != nullptr && !a.grp;
    const int b_lo = split ? (int)blockIdx.z * a.kchunks : 0;
    const int b_hi = split ? min(nb, b_lo + a.kchunks) : nb;
    const int64_t rows = a.rows;
    const u32 rb = (u32)a.row_bytes;
    const u32 cpos = 2u + 8u * (u32)(TY == T_Q8_0 ? q : (q & 1));
    const float *xrow = a.x + (int64_t)s_in[n16] * a.x_stride + 8 * q;
    const int tile_rows = a.glu ? 16 * (GR / 2) : 16 * GR;

    for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
        u32 rbase[GR];
        bool hi[GR];
#pragma unroll
        for (int gi = 0; gi < GR; gi++) {
            // gated: groups [0, GR/2) gate rows, [GR/2, GR) the same up rows
            hi[gi] = a.glu && gi >= GR / 2;
            const int64_t r0 = tile * tile_rows + 16 * (a.glu ? gi % (GR / 2) : gi);
            const int64_t r = min(r0 + n16, rows - 1);
            rbase[gi] = (u32)r * rb + (hi[gi] ? ph1 : ph0);
        }
        float acc[GR][4];
#pragma unroll
        for (int gi = 0; gi < GR; gi++)
#pragma unroll
            for (int i = 0; i < 4; i++) acc[gi][i] = 0.0f;

        // block b's raw data: the dwords holding the lane's 8 code bytes (two
        // when they start on a dword, else three), the dword holding its row's
        // scale, and its token's 8 x values
        u32 win[PF + 1][GR][3], sd[PF + 1][GR];
        f32x4 xa[PF + 1], xb[PF + 1];
        auto fetch = [&](int b, int k) {
            b = min(b, b_hi - 1);   // past this range's end: re-load its last block
#pragma unroll
            for (int gi = 0; gi < GR; gi++) {
                const u32 o = rbase[gi] + (u32)b * BYTES + cpos;
                const rsrc_t rs = hi[gi] ? rs1 : rs0;
                const u32 oa = o & ~3u;
                const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, oa, 0, 0);
                // a third dword only when the codes straddle three; else the
                // second again (the shift below then never takes its bytes), so
                // no load reaches past the dword holding the block's last byte
                win[k][gi][2] = __builtin_amdgcn_raw_buffer_load_b32(rs, oa + ((o & 3u) ? 8u : 4u), 0, 0);
                win[k][gi][0] = v.x; win[k][gi][1] = v.y;
                sd[k][gi] = __builtin_amdgcn_raw_buffer_load_b32(rs, (rbase[gi] + (u32)b * BYTES) & ~3u, 0, 0);
            }
            if (a.x_vec) {
                xa[k] = *(const f32x4 *)(xrow + 32 * b);
                xb[k] = *(const f32x4 *)(xrow + 32 * b + 4);
            } else {
                const float *p = xrow + 32 * b;
                xa[k] = f32x4{p[0], p[1], p[2], p[3]};
                xb[k] = f32x4{p[4], p[5], p[6], p[7]};
            }
        };
        auto consume = [&](int b, int k) {
            u32 ph[4], pm[4], pl[4];
            split3(xa[k], xb[k], ph, pm, pl);
            const bf16x8 xh = as_bf16x8(ph), xm = as_bf16x8(pm), xl = as_bf16x8(pl);
#pragma unroll
            for (int gi = 0; gi < GR; gi++) {
                const u32 o = rbase[gi] + (u32)b * BYTES + cpos;
                const u32 sh = o & 3u;
                const u32 cw0 = __builtin_amdgcn_alignbyte(win[k][gi][1], win[k][gi][0], sh);
                const u32 cw1 = __builtin_amdgcn_alignbyte(win[k][gi][2], win[k][gi][1], sh);
                u32 cb[4];
                codes_bf16<TY>(cw0, cw1, q, cb);
                const u32 so = rbase[gi] + (u32)b * BYTES;
                const float d = h2f(sd[k][gi] >> (8 * (so & 3u)));
                const bf16x8 wv = as_bf16x8(cb);
                f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, wv, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xm, wv, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xl, wv, c, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; i++) acc[gi][i] = fmaf(d, c[i], acc[gi][i]);
            }
        };
        // blocks b_lo + wave, + 4, ...: PF of them in flight ahead of the one in use
        const int bw = b_lo + wave;
        const int nmine = b_hi > bw ? (b_hi - bw + 3) / 4 : 0;
#pragma unroll
        for (int k = 0; k < PF; k++) fetch(bw + 4 * k, k);
        int j = 0;
        for (; j + PF + 1 <= nmine; j += PF + 1) {
#pragma unroll
            for (int k = 0; k <= PF; k++) {
                fetch(bw + 4 * (j + k + PF), (k + PF) % (PF + 1));
                consume(bw + 4 * (j + k), k);
            }
        }
#pragma unroll
        for (int k = 0; k <= PF; k++) {
            if (j + k < nmine) {
                fetch(bw + 4 * (j + k + PF), (k + PF) % (PF + 1));
                consume(bw + 4 * (j + k), k);
            }
        }
        // the four waves' partial sums, added in wave order
#pragma unroll
        for (int gi = 0; gi < GR; gi++)
#pragma unroll
            for (int i = 0; i < 4; i++) s_red[wave][gi * 4 + i][lane] = acc[gi][i];
        __syncthreads();
        // every wave finishes one quarter of the (group, token) outputs
#pragma unroll
        for (int gi = 0; gi < GR; gi++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int e = gi * 4 + i;
                acc[gi][i] = ((s_red[0][e][lane] + s_red[1][e][lane]) + s_red[2][e][lane]) + s_red[3][e][lane];
            }
        __syncthreads();   // s_red is free for the next tile
        // lane holds tokens 4q..4q+3 of row n16 of each group; wave w stores token 4q+w
        {
            const int i = wave;
            const int t = 4 * q + i;
            if (t < nt && split) {
                // raw sums of this split: [z][token][rows] (gated: gate rows, then up rows)
                float *pp = a.part + ((int64_t)blockIdx.z * a.ptok + s_out[t]) * a.prow;
                if (a.glu) {
#pragma unroll
                    for (int gi = 0; gi < GR / 2; gi++) {
                        const int64_t r = tile * tile_rows + 16 * gi + n16;
                        if (r < rows) {
                            pp[r] = acc[gi][i];
                            pp[rows + r] = acc[gi + GR / 2][i];
                        }
                    }
                } else {
#pragma unroll
                    for (int gi = 0; gi < GR; gi++) {
                        const int64_t r = tile * tile_rows + 16 * gi + n16;
                        if (r < rows) pp[r] = acc[gi][i];
                    }
                }
            } else if (t < nt) {
                const int64_t oi = s_out[t];
                const float osc = s_osc[t];
                if (a.glu) {
#pragma unroll
                    for (int gi = 0; gi < GR / 2; gi++) {
                        const int64_t r = tile * tile_rows + 16 * gi + n16;
                        if (r < rows) {
                            const float gv = acc[gi][i], uv = acc[gi + GR / 2][i];
                            a.y[oi * a.y_stride + r] = glu(a.glu, gv, uv);
                            if (a.y2) {
                                a.y2[oi * a.y2_stride + r] = gv;
                                a.y2[oi * a.y2_stride + rows + r] = uv;
                            }
                        }
                    }
                } else {
#pragma unroll
                    for (int gi = 0; gi < GR; gi++) {
                        const int64_t r = tile * tile_rows + 16 * gi + n16;
                        if (r < rows) a.y[oi * a.y_stride + r] = (acc[gi][i] * es) * osc;
                    }
                }
            }
        }
    }
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
// Kernel kinds.  UK_BLOCK: k_gemv over single Q8_0 / Q4_0 blocks (rows with
// an odd block count).  UK_LDS: k_gemv_lds over pair units (Q8_0 / Q4_0) or
// the K-quant blocks, 16-byte aligned ranges and rows; UK_LDS2: the same for
// any 2-byte phase.
// UK_MFMA: k_gemv_mfma (Q8_0 / Q4_0, 4..16 tokens).
enum { UK_BLOCK = 0, UK_LDS = 1, UK_LDS2 = 2, UK_MFMA = 3 };
// One function per (block type, tokens per workgroup), each instantiated in
// its own translation unit (qg_inst_<type>_t<NT>.hip); returns the kernel for
// (kernel kind, lanes per row, x staged in chunks).  qg_inst_dequant.hip
// holds the dequantizers.
#define QG_DECL_GEMV(NAME) \
    gemv_fn gemv_kernel_##NAME##_t1(int kind, int lpr, bool xc, bool rt); \
    gemv_fn gemv_kernel_##NAME##_t2(int kind, int lpr, bool xc, bool rt); \
    gemv_fn gemv_kernel_##NAME##_t4(int kind, int lpr, bool xc, bool rt); \
    gemv_fn gemv_kernel_##NAME##_t8(int kind, int lpr, bool xc, bool rt);
QG_DECL_GEMV(q8_0)
QG_DECL_GEMV(q4_0)
QG_DECL_GEMV(q4_k)
QG_DECL_GEMV(q6_k)
#undef QG_DECL_GEMV
dequant_fn dequant_kernel(int type);
// MFMA small-batch kernels (Q8_0 / Q4_0), qg_inst_mfma.hip
gemv_fn gemv_kernel_mfma(int type, int groups);
// prefill chunks (qg_gemm.hip): Q8_0 / Q4_0; a workgroup of gemm_threads()
// threads owns gemm_tile_rows(glu) rows (gated: that many gate rows and the
// same up rows) by gemm_token_tile() tokens, one workgroup per CU
gemv_fn gemm_kernel_mfma(int type);
int gemm_tile_rows(int glu);
int gemm_threads();
int gemm_token_tile();
int gemm_chunk_values();   // row values per k-chunk
// bytes of x [ntok][cols] split for the prefill kernel, and the launch that
// splits it (x rows x_stride floats apart)
size_t gemm_xs_bytes(int64_t cols, int ntok);
int gemm_split_x(const float *x, int64_t x_stride, int ntok, int64_t cols, uint8_t *xs, hipStream_t st);
// adds the raw sums of a.kchunks-long splits (grid.z = nsplit of them) in
// split order and writes y (gated: act(g) * u, and g, u to y2 when set)
int gemm_reduce(const GemvArgs &a, int nsplit, hipStream_t st);

// Router / grouping and combine kernels (qg_route.hip).
typedef void (*route_fn)(const float *logits, int E, int k, int T, const int32_t *slots, int n_slots,
                         int32_t *ids_out, float *w_out, int32_t *status, int32_t *rt_ids, float *rt_w,
                         int32_t *rt_valid, int32_t *grp, int ca, int32_t *sets_a, int cb, int32_t *sets_b,
                         const float *escale, int32_t *rt_pslot, float *rt_pes);
// k_route for E experts (E <= 256): the instance with the fewest register sets
route_fn route_kernel(int E);
__global__ void k_combine(const float *dn, const int32_t *rt_valid, float *y, int64_t H, int k);

}  // namespace qg

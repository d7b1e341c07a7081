// qg_down1.h -- one token's down projections and combine, for one workgroup
// of 8 output rows: every routed pick's expert row and an optional extra pick
// (a shared expert's down row, or a dense MLP's down row beside the experts).
//
// Each lane requests its units of every pick's row at once (one memory round
// trip for the whole workgroup), the activation rows go to LDS as one batch,
// and the pick terms (dn_j * s[e_j]) * w_j are added in pick order: the same
// terms in the same order as a grouped down launch followed by the combine
// ([qwen3] encodeExperts: expertQ8 on down, moeAccum; [gemma4]
// encodeExpertsB: expertQ4B on down, moeSumB; [qwen35] moeAccumShared for the
// shared expert).
#pragma once
#include "qg_moe1.h"

namespace qg {

// The shared expert's gate logit (gate_inp . x over the H values), one
// thread's part: its products in the order the shared-expert combine takes
// them (16 columns 256 apart per batch), for a workgroup of 256 threads.
QG_DEV float gate_part(const Moe1Args &a, int tid) {
    float gp = 0.0f;
    for (int64_t c0 = tid; c0 < a.rows; c0 += 256 * 16) {
        float gv[16], xv[16];
#pragma unroll
        for (int b = 0; b < 16; b++) {
            const bool in = c0 + b * 256 < a.rows;
            gv[b] = in ? a.gate_inp[c0 + b * 256] : 0.0f;
            xv[b] = in ? a.x[c0 + b * 256] : 0.0f;
        }
#pragma unroll
        for (int b = 0; b < 16; b++) gp = fmaf(gv[b], xv[b], gp);
    }
    return gp;
}
// the workgroup's sum of the parts (wave sums, then the 4 waves in order),
// through the sigmoid; every workgroup takes the same steps, so all get the
// same value
QG_DEV float gate_finish(float gp, int wave, int lane, float *s_red) {
    gp = wave_sum(gp);
    if (lane == 0) s_red[wave] = gp;
    __syncthreads();
    const float sg = ((s_red[0] + s_red[1]) + s_red[2]) + s_red[3];
    return 1.0f / (1.0f + expf(-sg));
}

// Workgroup bx: rows bx*8 .. +7 (lane (grp, sub) of wave w: row (bx*4 + w)*2
// + grp, units sub, sub + 32, ... of that row).  KMAX routed picks at most
// (k of them), UPL units per lane of a routed row; XP the extra pick (its
// units per lane: UPL for the shared expert, up to MOE1_MAXX for a dense
// row).
template <class U, int KMAX, int UPL, int XP>
QG_DEV void down1_body(const Moe1Args &a, int bx, const Picks &pk) {
    extern __shared__ float lds[];
    __shared__ float s_red[4];
    constexpr int L = MOE1_L, RPW = 64 / L;
    constexpr int UV = U::VALUES, SUMS = U::SUMS, SPU = SUMS ? UV / (SUMS ? SUMS : 1) : 0;
    constexpr int UPLX = XP == XP_SHARED ? UPL : XP == XP_DENSE ? MOE1_MAXX : 1;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int grp = lane / L, sub = lane % L;
    const int64_t r = ((int64_t)bx * 4 + wave) * RPW + grp;
    const int64_t rl = r < a.rows ? r : a.rows - 1;   // past the last row: load a valid row, store nothing
    const int k = KMAX ? a.k : 0, nb = a.nb;

    // every routed pick's units in flight at once (pk repeats the last pick
    // past k: those loads are issued, never used; an absent expert loads
    // slot 0 or the last one and leaves y as it is)
    [[maybe_unused]] u32 t[KMAX ? KMAX : 1][UPL][U::NR];
    [[maybe_unused]] u32 off[KMAX ? KMAX : 1][UPL];
#pragma unroll
    for (int j = 0; j < KMAX; j++) {
        const int s0 = pk.slot[j];
        const int sl = s0 < 0 ? 0 : (s0 >= a.n_slots ? a.n_slots - 1 : s0);
        const uint8_t *base = uniform_ptr(a.W + (int64_t)sl * a.stride);
        const u32 ph = (u32)((uintptr_t)base & 3u);
        const rsrc_t rs = make_rsrc(base - ph, (u32)((ph + a.rows * a.row_bytes + 3) & ~(int64_t)3));
#pragma unroll
        for (int i = 0; i < UPL; i++) {
            const int u = min(sub + i * L, nb - 1);
            off[j][i] = ph + (u32)(rl * a.row_bytes) + (u32)u * U::BYTES;
            U::issue(rs, off[j][i], t[j][i]);
        }
    }
    // the extra pick's units after them
    [[maybe_unused]] u32 tx[UPLX][U::NR];
    [[maybe_unused]] u32 offx[UPLX];
    const int nbx = XP == XP_DENSE ? a.d_nb : nb;
    if constexpr (XP != XP_NONE) {
        const uint8_t *base = XP == XP_SHARED ? a.shW : a.dW;
        const int64_t rb = XP == XP_SHARED ? a.row_bytes : a.d_row_bytes;
        const u32 ph = (u32)((uintptr_t)base & 3u);
        const rsrc_t rs = make_rsrc(base - ph, (u32)((ph + a.rows * rb + 3) & ~(int64_t)3));
#pragma unroll
        for (int i = 0; i < UPLX; i++) {
            const int u = min(sub + i * L, nbx - 1);
            offx[i] = ph + (u32)(rl * rb) + (u32)u * U::BYTES;
            if (XP == XP_SHARED || sub + i * L < nbx) U::issue(rs, offx[i], tx[i]);
        }
    }
    [[maybe_unused]] float gp = 0.0f;
    if constexpr (XP == XP_SHARED) {
        if (!a.gate_logit) gp = gate_part(a, tid);
    }

    // the activation rows (and their 32-value sums) into LDS, as one flat
    // batch over (row, float4): every thread's loads are issued before any
    // is used; a 32-value group is 8 consecutive float4 in 8 consecutive
    // lanes (n4 is a multiple of 8), summed across them.  Rows 0..k-1: the
    // picks; row KMAX (XP_SHARED: the shared expert's, F wide; XP_DENSE: the
    // dense MLP's, its own width) after the routed rows' room.
    const int cpad = nb * UV;
    const int xstride = xstride_of(cpad);
    const int nsum = SUMS ? cpad / (SUMS ? SUMS : 1) : 0;
    const int n4 = cpad >> 2;
    const int cpadx = nbx * UV, xstridex = xstride_of(cpadx), nsumx = SUMS ? cpadx / (SUMS ? SUMS : 1) : 0;
    const int n4x = XP == XP_NONE ? 0 : cpadx >> 2;
    float *xs = lds;
    float *xsx = lds + KMAX * xstride;                      // the extra row
    float *ss = xsx + (XP == XP_NONE ? 0 : xstridex);       // sums: the picks' rows, then the extra row's
    float *ssx = ss + KMAX * nsum;
    const int total4 = k * n4 + n4x;
    for (int b0 = 0; b0 < total4; b0 += 256 * XB) {
        f32x4 v[XB];
#pragma unroll
        for (int b = 0; b < XB; b++) {
            const int idx = min(b0 + tid + 256 * b, total4 - 1);
            const bool ext = idx >= k * n4;
            const int j = ext ? 0 : idx / n4, i = ext ? idx - k * n4 : idx - j * n4;
            const float *src = ext ? (XP == XP_SHARED ? a.sh_act : a.d_act) : a.act + (int64_t)j * a.act_stride;
            v[b] = ((const f32x4 *)src)[i];
        }
#pragma unroll
        for (int b = 0; b < XB; b++) {
            const int idx = b0 + tid + 256 * b;
            const bool ext = idx >= k * n4;
            const int j = ext ? 0 : idx / n4, i = ext ? idx - k * n4 : idx - j * n4;
            if constexpr (SUMS != 0) {
                const float g = group_sum<SUMS / 4>((v[b].x + v[b].y) + (v[b].z + v[b].w));
                if (idx < total4 && (i & (SUMS / 4 - 1)) == 0) {
                    if (ext) ssx[(4 * i) / SUMS] = g;
                    else ss[j * nsum + (4 * i) / SUMS] = g;
                }
            }
            if (idx < total4) *(f32x4 *)(ext ? xsx + xpad(4 * i) : xs + j * xstride + xpad(4 * i)) = v[b];
        }
    }
    __syncthreads();
    [[maybe_unused]] float gs = 0.0f;
    if constexpr (XP == XP_SHARED)
        gs = a.gate_logit ? 1.0f / (1.0f + expf(-a.gate_logit[0])) : gate_finish(gp, wave, lane, s_red);

    float yacc = 0.0f;
#pragma unroll
    for (int j = 0; j < KMAX; j++) {
        if (j < k) {
            float acc[1] = {0.0f};
#pragma unroll
            for (int i = 0; i < UPL; i++) {
                const int u = sub + i * L;
                if (u < nb) {
                    u32 wd[U::ND];
                    U::prep(t[j][i], off[j][i], wd);
                    unit_dot<U, 1>(wd, xs + j * xstride + xpad(u * UV), xstride, ss + j * nsum + u * SPU, nsum, acc);
                }
            }
            const float term = (group_sum<L>(acc[0]) * pk.es[j]) * pk.wj[j];
            if (sub == 0 && r < a.rows) a.dn[(int64_t)j * a.rows + r] = term;
            yacc += term;
        }
    }
    [[maybe_unused]] float xv = 0.0f;
    if constexpr (XP != XP_NONE) {
        float acc[1] = {0.0f};
#pragma unroll
        for (int i = 0; i < UPLX; i++) {
            const int u = sub + i * L;
            if (u < nbx) {
                u32 wd[U::ND];
                U::prep(tx[i], offx[i], wd);
                unit_dot<U, 1>(wd, xsx + xpad(u * UV), xstridex, ssx + u * SPU, nsumx, acc);
            }
        }
        xv = group_sum<L>(acc[0]);
    }
    if (sub == 0 && r < a.rows) {
        if constexpr (XP == XP_SHARED) {
            a.sh_out[r] = xv;
            if (pk.ok) a.resid[r] = (yacc + xv * gs) + a.resid[r];
        }
        if constexpr (XP == XP_DENSE) a.y_mlp[r] = xv;
        if (KMAX && a.y && pk.ok) a.y[r] = yacc;
    }
}

// ---- column layout -------------------------------------------------------
// The (pick, block) columns of one output row: routed pick j's block b is
// column j*nb + b, the extra pick's blocks follow (k*nb + nbx columns, at
// most D1C_NT).  Thread c of the workgroup takes column c for the
// workgroup's R consecutive rows: it loads the column's 32 activation values
// into registers once (their sum too, for the folding formats), then that
// block of each of the R rows, and leaves each block's dot in LDS.  Every
// lane has work whatever nb is, and a workgroup stages nothing.  Then one
// thread per (row, pick) adds the pick's block dots in block order and forms
// the term (dn_j * s[e_j]) * w_j, and one thread per row adds the terms in
// pick order.  The routed blocks are read through one descriptor over the
// whole expert pool (the launcher checks that its bytes fit 32 bits).
constexpr int D1C_NT = 256, D1C_RMAX = 12;

// one block against 32 activation values held in registers: the two halves'
// sums as unit_dot forms them, folded with the block's scale
template <class U>
QG_DEV float reg_dot(const u32 (&w)[U::ND], const f32x4 (&x)[8], float xs) {
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; q++) {
        float &s = q >= 4 ? s1 : s0;
        s = fmaf(U::dcode(w, 4 * q), x[q].x, s);
        s = fmaf(U::dcode(w, 4 * q + 1), x[q].y, s);
        s = fmaf(U::dcode(w, 4 * q + 2), x[q].z, s);
        s = fmaf(U::dcode(w, 4 * q + 3), x[q].w, s);
    }
    return U::fold(w, 0, fmaf(s1, U::dfix(0, 1), s0 * U::dfix(0, 0)), xs);
}

// the routed pool's descriptor range: through the last slot's last row
__host__ __device__ inline int64_t down1c_pool_bytes(int64_t ph, int64_t n_slots, int64_t stride, int64_t rows,
                                                     int64_t row_bytes) {
    return (ph + (n_slots - 1) * stride + rows * row_bytes + 3) & ~(int64_t)3;
}

// Workgroup bx: rows bx*R .. bx*R + R - 1 (R <= D1C_RMAX)
template <class U, int XP>
QG_DEV void down1c_body(const Moe1Args &a, int bx, int R) {
    static_assert(U::VALUES == 32 && U::GROUPS == 1, "down1c_body: one 32-value block per unit");
    __shared__ float s_dot[D1C_RMAX][D1C_NT];
    __shared__ float s_term[D1C_RMAX][MOE1_MAXK + 1];
    __shared__ float s_red[4];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int k = a.k, nb = a.nb, kn = k * nb;
    const int nbx = XP == XP_DENSE ? a.d_nb : XP == XP_SHARED ? nb : 0;
    const int C = kn + nbx;
    const int c = min(tid, C - 1);   // threads past the columns repeat the last one and store nothing
    const bool routed = c < kn;
    const int j = routed ? c / nb : 0;
    const int b = routed ? c - j * nb : c - kn;
    const int64_t r0 = (int64_t)bx * R;
    // the phase-two role of this thread: (row i2, pick s2) while tid < R * S
    const int S = k + (XP != XP_NONE ? 1 : 0);
    const int i2 = tid / S, s2 = tid - i2 * S;
    const bool ok = a.valid[0] != 0;

    // the column's activation values first: they depend on the column only,
    // so their loads go out while the picks' slots are still on their way
    const float *xsrc = routed ? a.act + (int64_t)j * a.act_stride : (XP == XP_SHARED ? a.sh_act : a.d_act);
    f32x4 xr[8];
#pragma unroll
    for (int q = 0; q < 8; q++) xr[q] = ((const f32x4 *)(xsrc + 32 * b))[q];

    // the column's block of each row: the routed pool or the extra matrix
    const uint8_t *pool = uniform_ptr(a.W);
    const u32 ph = (u32)((uintptr_t)pool & 3u);
    const rsrc_t rp = make_rsrc(pool - ph, (u32)down1c_pool_bytes(ph, a.n_slots, a.stride, a.rows, a.row_bytes));
    [[maybe_unused]] rsrc_t rx = rp;
    u32 coff = 0, rb = 0;
    if constexpr (XP != XP_NONE) {
        const uint8_t *xb = uniform_ptr(XP == XP_SHARED ? a.shW : a.dW);
        const int64_t rbx = XP == XP_SHARED ? a.row_bytes : a.d_row_bytes;
        const u32 phx = (u32)((uintptr_t)xb & 3u);
        rx = make_rsrc(xb - phx, (u32)((phx + a.rows * rbx + 3) & ~(int64_t)3));
        coff = phx + (u32)b * U::BYTES;
        rb = (u32)rbx;
    }
    // this lane's pick: its slot (read per lane, so no per-pick array is
    // indexed by lane), and for phase two the down scale and weight of s2
    const int s0 = a.pslot[j];
    const int s2c = min(s2, k - 1);
    const float es2 = a.pes[s2c], w2 = a.w[s2c];
    if (routed) {
        const int sl = s0 < 0 ? 0 : (s0 >= a.n_slots ? a.n_slots - 1 : s0);
        coff = ph + (u32)sl * (u32)a.stride + (u32)b * U::BYTES;
        rb = (u32)a.row_bytes;
    }
    u32 t[D1C_RMAX][U::NR], off[D1C_RMAX];
#pragma unroll
    for (int i = 0; i < D1C_RMAX; i++) {
        const int64_t r = r0 + i < a.rows ? r0 + i : a.rows - 1;   // past the last row: a valid row, unused
        off[i] = coff + (u32)r * rb;
    }
    // the routed lanes' loads, then the extra lanes' (two one-sided blocks
    // apart, so that each load keeps its own uniform descriptor rather than
    // one chosen per lane)
    if (XP == XP_NONE || routed) {
#pragma unroll
        for (int i = 0; i < D1C_RMAX; i++)
            if (i < R) U::issue(rp, off[i], t[i]);
    }
    if constexpr (XP != XP_NONE) {
        asm volatile("" ::: "memory");
        if (!routed) {
#pragma unroll
            for (int i = 0; i < D1C_RMAX; i++)
                if (i < R) U::issue(rx, off[i], t[i]);
        }
    }
    [[maybe_unused]] float gp = 0.0f;
    if constexpr (XP == XP_SHARED) {
        if (!a.gate_logit) gp = gate_part(a, tid);
    }
    float xs = 0.0f;
    if constexpr (U::SUMS != 0) {
        float h[8];
#pragma unroll
        for (int q = 0; q < 8; q++) h[q] = (xr[q].x + xr[q].y) + (xr[q].z + xr[q].w);
        xs = ((h[0] + h[1]) + (h[2] + h[3])) + ((h[4] + h[5]) + (h[6] + h[7]));
    }
#pragma unroll
    for (int i = 0; i < D1C_RMAX; i++) {
        if (i < R) {
            u32 wd[U::ND];
            U::prep(t[i], off[i], wd);
            s_dot[i][tid] = reg_dot<U>(wd, xr, xs);
        }
    }
    [[maybe_unused]] float gs = 0.0f;
    if constexpr (XP == XP_SHARED)   // (gate_finish holds a barrier; gate_logit is the same for all threads)
        gs = a.gate_logit ? 1.0f / (1.0f + expf(-a.gate_logit[0])) : gate_finish(gp, wave, lane, s_red);
    __syncthreads();

    // one thread per (row, pick): the pick's block dots in block order
    if (tid < R * S) {
        const int i = i2, s = s2;
        const bool ex = s >= k;
        const int c0 = ex ? kn : s * nb, n = ex ? nbx : nb;
        float sum = 0.0f;
        for (int q = 0; q < n; q++) sum += s_dot[i][c0 + q];
        if (!ex) {
            sum = (sum * es2) * w2;
            if (r0 + i < a.rows) a.dn[(int64_t)s * a.rows + r0 + i] = sum;
        }
        s_term[i][s] = sum;
    }
    __syncthreads();
    // one thread per row: the terms in pick order
    if (tid < R && r0 + tid < a.rows) {
        const int64_t r = r0 + tid;
        float yacc = 0.0f;
        for (int s = 0; s < k; s++) yacc += s_term[tid][s];
        [[maybe_unused]] const float xv = s_term[tid][k];
        if constexpr (XP == XP_SHARED) {
            a.sh_out[r] = xv;
            if (ok) a.resid[r] = (yacc + xv * gs) + a.resid[r];
        }
        if constexpr (XP == XP_DENSE) a.y_mlp[r] = xv;
        if (a.y && ok) a.y[r] = yacc;
    }
}

// LDS of down1_body: the routed picks' rows (room for MOE1_MAXK) and the
// extra pick's row, each padded, then their 32-value sums
inline size_t down1_lds_bytes(int nb, int sums, int xp, int nbx) {
    const int cpad = nb * 32, cpadx = nbx * 32;
    size_t n = (size_t)MOE1_MAXK * xstride_of(cpad) + (sums ? (size_t)MOE1_MAXK * cpad / sums : 0);
    if (xp != XP_NONE) n += (size_t)xstride_of(cpadx) + (sums ? (size_t)cpadx / sums : 0);
    return n * 4;
}

}  // namespace qg

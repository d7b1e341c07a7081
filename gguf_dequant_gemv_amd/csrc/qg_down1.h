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
    // the shared expert's gate logit: this thread's products in the order
    // the shared-expert combine takes them (16 columns 256 apart per batch)
    [[maybe_unused]] float gp = 0.0f;
    if constexpr (XP == XP_SHARED) {
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
    if constexpr (XP == XP_SHARED) {   // the block's sum: wave sums, then the waves in order
        gp = wave_sum(gp);
        if (lane == 0) s_red[wave] = gp;
        __syncthreads();
        const float sg = ((s_red[0] + s_red[1]) + s_red[2]) + s_red[3];
        gs = 1.0f / (1.0f + expf(-sg));
    }

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

// LDS of down1_body: the routed picks' rows (room for MOE1_MAXK) and the
// extra pick's row, each padded, then their 32-value sums
inline size_t down1_lds_bytes(int nb, int sums, int xp, int nbx) {
    const int cpad = nb * 32, cpadx = nbx * 32;
    size_t n = (size_t)MOE1_MAXK * xstride_of(cpad) + (sums ? (size_t)MOE1_MAXK * cpad / sums : 0);
    if (xp != XP_NONE) n += (size_t)xstride_of(cpadx) + (sums ? (size_t)cpadx / sums : 0);
    return n * 4;
}

}  // namespace qg

// qg_moe1.hip -- one token's routed experts: the down projection of every
// pick and the weighted combine in a single launch.
//
// The grouped path runs the down projection as one launch over (expert group,
// row tile) and the combine as another; for a decode step (one token, top-k of
// a few picks) each of those launches moves only a few MB and is dominated by
// its fill and drain.  Here a workgroup takes 8 rows of H and every pick: each
// lane's block of each pick's expert row is requested at once (one memory
// round trip for the whole workgroup), the k activation rows are staged in
// LDS, and the pick terms (dn_j * s[e_j]) * w_j are added in pick order -- the
// same terms and the same order as the grouped down launch followed by the
// combine.  [qwen3] encodeExperts (expertQ8 on down, moeAccum) and [gemma4]
// encodeExpertsB (expertQ4B on down, moeSumB).  With a shared expert (SH) its
// down row is one more pick and the launch ends with the shared-expert
// combine into the residual ([qwen35] moeAccumShared): the gate logit is
// reduced in every workgroup in the same order, so all use the same value.
#include "../../include/qgemv.h"
#include "qg_kernels.h"
#include "qg_moe1.h"

namespace qg {

constexpr int MOE1_L = 32;     // lanes per row: 8 rows per workgroup
constexpr int MOE1_MAXK = 8;   // picks one launch serves

// Lane (row grp, sub) of wave w: row (blockIdx.x * 4 + w) * 2 + grp, blocks
// sub, sub + 32, ... (UPL of them) of that row in each pick's expert matrix.
template <class U, int UPL, bool SH>
__global__ __launch_bounds__(256) void k_moe_down1(Moe1Args a) {
    extern __shared__ float lds[];
    __shared__ float s_red[4];
    constexpr int L = MOE1_L, RPW = 64 / L;
    constexpr int UV = U::VALUES, SUMS = U::SUMS, SPU = SUMS ? UV / (SUMS ? SUMS : 1) : 0;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int grp = lane / L, sub = lane % L;
    const int64_t r = ((int64_t)blockIdx.x * 4 + wave) * RPW + grp;
    const int64_t rl = r < a.rows ? r : a.rows - 1;   // past the last row: load a valid row, store nothing
    const int k = a.k, nb = a.nb;

    // the picks' experts, slots and scales: each a batch of independent
    // uniform loads (picks past k repeat the last one, results unused), so
    // the weight loads wait for two round trips, not two per pick
    int e[MOE1_MAXK], slot[MOE1_MAXK];
    float es[MOE1_MAXK], wj[MOE1_MAXK];
#pragma unroll
    for (int j = 0; j < MOE1_MAXK; j++) {
        e[j] = a.ids[min(j, k - 1)];
        wj[j] = a.w[min(j, k - 1)];
    }
#pragma unroll
    for (int j = 0; j < MOE1_MAXK; j++) {
        slot[j] = a.slots[e[j]];
        es[j] = a.escale ? a.escale[e[j]] : 1.0f;
    }
    // every pick's units in flight at once (the shared expert's after them)
    u32 t[MOE1_MAXK][UPL][U::NR];
    u32 off[MOE1_MAXK][UPL];
    [[maybe_unused]] u32 ts[SH ? UPL : 1][U::NR];
    [[maybe_unused]] u32 offs[SH ? UPL : 1];
#pragma unroll
    for (int j = 0; j < MOE1_MAXK; j++) {
        // an absent expert (no slot) loads slot 0 or the last one; y is then left as it is
        const int sl = slot[j] < 0 ? 0 : (slot[j] >= a.n_slots ? a.n_slots - 1 : slot[j]);
        const uint8_t *base = a.W + (int64_t)sl * a.stride;
        const u32 ph = (u32)((uintptr_t)base & 3u);
        const rsrc_t rs = make_rsrc(base - ph, (u32)((ph + a.rows * a.row_bytes + 3) & ~(int64_t)3));
#pragma unroll
        for (int i = 0; i < UPL; i++) {
            const int u = min(sub + i * L, nb - 1);
            off[j][i] = ph + (u32)(rl * a.row_bytes) + (u32)u * U::BYTES;
            U::issue(rs, off[j][i], t[j][i]);
        }
    }
    if constexpr (SH) {
        const u32 ph = (u32)((uintptr_t)a.shW & 3u);
        const rsrc_t rs = make_rsrc(a.shW - ph, (u32)((ph + a.rows * a.row_bytes + 3) & ~(int64_t)3));
#pragma unroll
        for (int i = 0; i < UPL; i++) {
            const int u = min(sub + i * L, nb - 1);
            offs[i] = ph + (u32)(rl * a.row_bytes) + (u32)u * U::BYTES;
            U::issue(rs, offs[i], ts[i]);
        }
    }
    // the shared expert's gate logit: this thread's products in the order
    // the shared-expert combine takes them (16 columns 256 apart per batch)
    [[maybe_unused]] float gp = 0.0f;
    if constexpr (SH) {
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

    // the k activation rows (and their 32-value sums) into LDS
    const int cpad = nb * UV;
    const int xstride = xstride_of(cpad);
    const int nsum = SUMS ? cpad / (SUMS ? SUMS : 1) : 0;
    const int n4 = cpad >> 2;
    float *xs = lds;
    float *ss = lds + (MOE1_MAXK + 1) * xstride;   // after the rows (and the shared expert's)
    // as one flat batch over (pick, float4): every thread's loads are issued
    // before any is used; a 32-value group is 8 consecutive float4 in 8
    // consecutive lanes (n4 is a multiple of 8), summed across them
    const int nrows_x = k + (SH ? 1 : 0);   // the shared expert's activation row last
    const int total4 = nrows_x * n4;
    for (int b0 = 0; b0 < total4; b0 += 256 * XB) {
        f32x4 v[XB];
#pragma unroll
        for (int b = 0; b < XB; b++) {
            const int idx = min(b0 + tid + 256 * b, total4 - 1);
            const int j = idx / n4, i = idx - j * n4;
            const float *src = (SH && j == k) ? a.sh_act : a.act + (int64_t)j * a.act_stride;
            v[b] = ((const f32x4 *)src)[i];
        }
#pragma unroll
        for (int b = 0; b < XB; b++) {
            const int idx = b0 + tid + 256 * b;
            const int j = idx / n4, i = idx - j * n4;
            if constexpr (SUMS != 0) {
                const float g = group_sum<SUMS / 4>((v[b].x + v[b].y) + (v[b].z + v[b].w));
                if (idx < total4 && (i & (SUMS / 4 - 1)) == 0) ss[j * nsum + (4 * i) / SUMS] = g;
            }
            if (idx < total4) *(f32x4 *)(xs + j * xstride + xpad(4 * i)) = v[b];
        }
    }
    __syncthreads();
    [[maybe_unused]] float gs = 0.0f;
    if constexpr (SH) {   // the block's sum: wave sums, then the waves in order
        gp = wave_sum(gp);
        if (lane == 0) s_red[wave] = gp;
        __syncthreads();
        const float sg = ((s_red[0] + s_red[1]) + s_red[2]) + s_red[3];
        gs = 1.0f / (1.0f + expf(-sg));
    }

    float yacc = 0.0f;
#pragma unroll
    for (int j = 0; j < MOE1_MAXK; j++) {
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
            const float term = (group_sum<L>(acc[0]) * es[j]) * wj[j];
            if (sub == 0 && r < a.rows) a.dn[(int64_t)j * a.rows + r] = term;
            yacc += term;
        }
    }
    if constexpr (SH) {
        float acc[1] = {0.0f};
#pragma unroll
        for (int i = 0; i < UPL; i++) {
            const int u = sub + i * L;
            if (u < nb) {
                u32 wd[U::ND];
                U::prep(ts[i], offs[i], wd);
                unit_dot<U, 1>(wd, xs + k * xstride + xpad(u * UV), xstride, ss + k * nsum + u * SPU, nsum, acc);
            }
        }
        const float shv = group_sum<L>(acc[0]);
        if (sub == 0 && r < a.rows) {
            a.sh_out[r] = shv;
            if (a.valid[0]) a.resid[r] = (yacc + shv * gs) + a.resid[r];
        }
    }
    if (a.y && sub == 0 && r < a.rows && a.valid[0]) a.y[r] = yacc;
}

bool moe_down1_fits(int type, int64_t cols, int k) {
    return (type == T_Q8_0 || type == T_Q4_0) && k >= 1 && k <= MOE1_MAXK && cols / 32 <= 2 * MOE1_L;
}

typedef void (*moe1_fn)(Moe1Args);

template <bool SH>
moe1_fn moe1_kernel(int type, bool two) {
    if (type == T_Q8_0) return two ? k_moe_down1<UQ8_0B, 2, SH> : k_moe_down1<UQ8_0B, 1, SH>;
    return two ? k_moe_down1<UQ4_0B, 2, SH> : k_moe_down1<UQ4_0B, 1, SH>;
}

int launch_moe_down1(int type, const Moe1Args &a, hipStream_t st) {
    const int cpad = a.nb * 32;
    const int nrows_x = MOE1_MAXK + 1;   // (room for the shared expert's row)
    const size_t lds = (size_t)nrows_x * xstride_of(cpad) * 4 + (size_t)nrows_x * (cpad / 32) * 4;
    const bool two = a.nb > MOE1_L;
    const dim3 grid((unsigned)((a.rows + 7) / 8));
    const moe1_fn f = a.shW ? moe1_kernel<true>(type, two) : moe1_kernel<false>(type, two);
    if (lds > 64 * 1024 &&
        hipFuncSetAttribute((const void *)f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return QG_EHIP;
    hipLaunchKernelGGL(f, grid, dim3(256), lds, st, a);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_EHIP;
}

}  // namespace qg

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
// encodeExpertsB (expertQ4B on down, moeSumB).
#include "../../include/qgemv.h"
#include "qg_kernels.h"
#include "qg_moe1.h"

namespace qg {

constexpr int MOE1_L = 32;     // lanes per row: 8 rows per workgroup
constexpr int MOE1_MAXK = 8;   // picks one launch serves

// Lane (row grp, sub) of wave w: row (blockIdx.x * 4 + w) * 2 + grp, blocks
// sub, sub + 32, ... (UPL of them) of that row in each pick's expert matrix.
template <class U, int UPL>
__global__ __launch_bounds__(256) void k_moe_down1(Moe1Args a) {
    extern __shared__ float lds[];
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
    // every pick's units in flight at once
    u32 t[MOE1_MAXK][UPL][U::NR];
    u32 off[MOE1_MAXK][UPL];
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

    // the k activation rows (and their 32-value sums) into LDS
    const int cpad = nb * UV;
    const int xstride = xstride_of(cpad);
    const int nsum = SUMS ? cpad / (SUMS ? SUMS : 1) : 0;
    const int n4 = cpad >> 2;
    float *xs = lds;
    float *ss = lds + MOE1_MAXK * xstride;
    // as one flat batch over (pick, float4): every thread's loads are issued
    // before any is used; a 32-value group is 8 consecutive float4 in 8
    // consecutive lanes (n4 is a multiple of 8), summed across them
    const int total4 = k * n4;
    for (int b0 = 0; b0 < total4; b0 += 256 * XB) {
        f32x4 v[XB];
#pragma unroll
        for (int b = 0; b < XB; b++) {
            const int idx = min(b0 + tid + 256 * b, total4 - 1);
            const int j = idx / n4, i = idx - j * n4;
            v[b] = ((const f32x4 *)(a.act + (int64_t)j * a.act_stride))[i];
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
    if (sub == 0 && r < a.rows && a.valid[0]) a.y[r] = yacc;
}

bool moe_down1_fits(int type, int64_t cols, int k) {
    return (type == T_Q8_0 || type == T_Q4_0) && k >= 1 && k <= MOE1_MAXK && cols / 32 <= 2 * MOE1_L;
}

int launch_moe_down1(int type, const Moe1Args &a, hipStream_t st) {
    const int cpad = a.nb * 32;
    const size_t lds = (size_t)MOE1_MAXK * xstride_of(cpad) * 4 + (size_t)MOE1_MAXK * (cpad / 32) * 4;
    const bool two = a.nb > MOE1_L;
    const dim3 grid((unsigned)((a.rows + 7) / 8));
    if (lds > 64 * 1024) {
        const void *f = type == T_Q8_0 ? (two ? (const void *)k_moe_down1<UQ8_0B, 2> : (const void *)k_moe_down1<UQ8_0B, 1>)
                                       : (two ? (const void *)k_moe_down1<UQ4_0B, 2> : (const void *)k_moe_down1<UQ4_0B, 1>);
        if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) return QG_EHIP;
    }
    if (type == T_Q8_0) {
        if (two)
            hipLaunchKernelGGL((k_moe_down1<UQ8_0B, 2>), grid, dim3(256), lds, st, a);
        else
            hipLaunchKernelGGL((k_moe_down1<UQ8_0B, 1>), grid, dim3(256), lds, st, a);
    } else {
        if (two)
            hipLaunchKernelGGL((k_moe_down1<UQ4_0B, 2>), grid, dim3(256), lds, st, a);
        else
            hipLaunchKernelGGL((k_moe_down1<UQ4_0B, 1>), grid, dim3(256), lds, st, a);
    }
    return hipGetLastError() == hipSuccess ? QG_OK : QG_EHIP;
}

}  // namespace qg

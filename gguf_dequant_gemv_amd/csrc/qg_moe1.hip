// qg_moe1.hip -- one token's routed experts: the down projection of every
// pick and the weighted combine in a single launch that follows the gated
// expert launch (the picks read from the routing outputs in the workspace).
//
// The grouped path runs the down projection as one launch over (expert group,
// row tile) and the combine as another; for a decode step (one token, top-k of
// a few picks) each of those launches moves only a few MB and is dominated by
// its fill and drain.  Here a workgroup takes 8 rows of H and every pick
// (down1_body in qg_down1.h).  [qwen3] encodeExperts (expertQ8 on down,
// moeAccum), [gemma4] encodeExpertsB (expertQ4B on down, moeSumB); with a
// shared expert its down row is one more pick and the launch ends with the
// shared-expert combine into the residual ([qwen35] moeAccumShared): the
// gate logit is reduced in every workgroup in the same order, so all use the
// same value.  A dense MLP beside the experts ([gemma4] encodeLayer) gives
// its down row as the extra pick instead, its output kept apart.
#include "../../include/qgemv.h"
#include <algorithm>

#include "qg_down1.h"

namespace qg {

// the picks' slots, down scales and weights from the routing outputs (the
// routing launch wrote them per pick): one batch of independent uniform
// loads (picks past k repeat the last one, unused), so the weight loads wait
// for one round trip
QG_DEV void picks_from_ws(const Moe1Args &a, Picks &pk) {
#pragma unroll
    for (int j = 0; j < MOE1_MAXK; j++) {
        const int jj = min(j, a.k - 1);
        pk.slot[j] = a.pslot[jj];
        pk.es[j] = a.pes[jj];
        pk.wj[j] = a.w[jj];
    }
    pk.ok = a.valid[0] != 0;
}

template <class U, int UPL, int XP>
__global__ __launch_bounds__(256) void k_moe_down1(Moe1Args a) {
    Picks pk;
    picks_from_ws(a, pk);
    down1_body<U, MOE1_MAXK, UPL, XP>(a, (int)blockIdx.x, pk);
}

template <class U, int XP>
__global__ __launch_bounds__(D1C_NT) void k_moe_down1c(Moe1Args a, int R) {
    down1c_body<U, XP>(a, (int)blockIdx.x, R);
}

bool moe_down1_fits(int type, int64_t cols, int k) {
    return (type == T_Q8_0 || type == T_Q4_0) && k >= 1 && k <= MOE1_MAXK && cols / 32 <= 2 * MOE1_L;
}

bool moe_down1_fits_dense(int type, int64_t cols, int64_t dense_cols, int k) {
    return moe_down1_fits(type, cols, k) && cols / 32 <= MOE1_L && dense_cols % 32 == 0 &&
           dense_cols / 32 <= MOE1_L * MOE1_MAXX;
}

typedef void (*moe1_fn)(Moe1Args);

template <int XP>
moe1_fn moe1_kernel(int type, bool two) {
    if (type == T_Q8_0) return two ? k_moe_down1<UQ8_0B, 2, XP> : k_moe_down1<UQ8_0B, 1, XP>;
    return two ? k_moe_down1<UQ4_0B, 2, XP> : k_moe_down1<UQ4_0B, 1, XP>;
}
// a dense row beside routed rows of one unit per lane (moe_down1_fits_dense)
moe1_fn moe1_kernel_dense(int type) {
    return type == T_Q8_0 ? k_moe_down1<UQ8_0B, 1, XP_DENSE> : k_moe_down1<UQ4_0B, 1, XP_DENSE>;
}

typedef void (*moe1c_fn)(Moe1Args, int);

template <int XP>
moe1c_fn moe1c_kernel(int type) {
    return type == T_Q8_0 ? k_moe_down1c<UQ8_0B, XP> : k_moe_down1c<UQ4_0B, XP>;
}

// The column layout (down1c_body) where the (pick, block) columns fit one
// workgroup and the pool's bytes fit a 32-bit descriptor.  R rows a
// workgroup: about two workgroups a CU (a SIMD then holds two waves, one
// computing while the other waits; measured 7.9 us against 8.5 at one a CU
// and 9.1 at three for the 2816-row Q4_0 layer with its dense row), but one
// a CU with a shared expert whose gate logit every workgroup reduces again
// (7.7 us against 10.4 at two a CU, 2048 rows of Q8_0); two when the
// routing launch has reduced it.
bool down1c_plan(const Moe1Args &a, int xp, int *rows_per_wg, int *wgs) {
    const int nbx = xp == XP_DENSE ? a.d_nb : xp == XP_SHARED ? a.nb : 0;
    if ((int64_t)a.k * a.nb + nbx > D1C_NT || a.n_slots < 1) return false;
    const int64_t ph = (int64_t)((uintptr_t)a.W & 3u);
    if (down1c_pool_bytes(ph, a.n_slots, a.stride, a.rows, a.row_bytes) > (int64_t)0xFFFFFFF0) return false;
    const int64_t per = xp == XP_SHARED && !a.gate_logit ? 256 : 512;
    const int64_t R = std::min<int64_t>(D1C_RMAX, (a.rows + per - 1) / per);
    *rows_per_wg = (int)R;
    *wgs = (int)((a.rows + R - 1) / R);
    return true;
}

int launch_moe_down1(int type, const Moe1Args &a, hipStream_t st) {
    const int xp = a.dW ? XP_DENSE : a.shW ? XP_SHARED : XP_NONE;
    int R = 0, g = 0;
    if (down1c_plan(a, xp, &R, &g)) {
        const moe1c_fn f = xp == XP_DENSE    ? moe1c_kernel<XP_DENSE>(type)
                           : xp == XP_SHARED ? moe1c_kernel<XP_SHARED>(type)
                                             : moe1c_kernel<XP_NONE>(type);
        hipLaunchKernelGGL(f, dim3((unsigned)g), dim3(D1C_NT), 0, st, a, R);
        return hipGetLastError() == hipSuccess ? QG_OK : QG_EHIP;
    }
    const size_t lds = down1_lds_bytes(a.nb, type == T_Q8_0 ? 0 : 32, xp, xp == XP_DENSE ? a.d_nb : a.nb);
    const bool two = a.nb > MOE1_L;
    if (xp == XP_DENSE && (two || a.d_nb > MOE1_L * MOE1_MAXX)) return QG_EINVAL;
    const dim3 grid((unsigned)((a.rows + 7) / 8));
    const moe1_fn f = xp == XP_DENSE    ? moe1_kernel_dense(type)
                      : xp == XP_SHARED ? moe1_kernel<XP_SHARED>(type, two)
                                        : moe1_kernel<XP_NONE>(type, two);
    if (lds > 64 * 1024 &&
        hipFuncSetAttribute((const void *)f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return QG_EHIP;
    hipLaunchKernelGGL(f, grid, dim3(256), lds, st, a);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_EHIP;
}

}  // namespace qg

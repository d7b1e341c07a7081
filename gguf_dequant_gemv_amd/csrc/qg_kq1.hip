// qg_kq1.hip -- instances, plan and launch of the one-token K-quant GEMV
// (k_kq1 in qg_kq1.h).
#include <mutex>

#include "../../include/qgemv.h"
#include "qg_kq1.h"

namespace qg {

namespace {
typedef void (*kq1_fn)(Kq1Args);
constexpr int KQ1_CU = 256;
constexpr size_t KQ1_MAX_LDS = 150 * 1024;

template <class U, int NW, int XN>
kq1_fn by_lanes(int L) {
    return L == 16 ? k_kq1<U, 16, NW, XN> : L == 32 ? k_kq1<U, 32, NW, XN> : k_kq1<U, 64, NW, XN>;
}

// x's float4 per thread, XN = 4, 9 or 12: the least that holds cols /
// (4 * 64 NW) (each float4 of the bound is a register set held while the
// first weight loads go out; other bounds measured to upset the register
// allocation of the unit ring)
template <class U, int NW>
kq1_fn by_x(int L, int cols) {
    const int n = (cols / 4 + 64 * NW - 1) / (64 * NW);
    return n <= 4 ? by_lanes<U, NW, 4>(L) : n <= 9 ? by_lanes<U, NW, 9>(L) : by_lanes<U, NW, 12>(L);
}

// waves per workgroup: 4, 8, 10 or 16
template <class U>
kq1_fn by_waves(int L, int nw, int cols) {
    return nw == 16 ? by_x<U, 16>(L, cols) : nw == 10 ? by_x<U, 10>(L, cols)
         : nw == 8 ? by_x<U, 8>(L, cols) : by_x<U, 4>(L, cols);
}

kq1_fn kq1_kernel(int type, bool aln, int L, int nw, int cols) {
    if (type == T_Q6_K) return by_waves<KQ6>(L, nw, cols);
    if (type == T_Q6_KP) return by_waves<KQ6P>(L, nw, cols);
    return aln ? by_waves<KQ4<true>>(L, nw, cols) : by_waves<KQ4<false>>(L, nw, cols);
}

// workgroups resident at once (all CUs): measured for the instance when a
// device is there to ask, else estimated from LDS and the waves per SIMD
// its register budget leaves room for
int kq1_resident(kq1_fn f, int type, int nw, size_t lds, bool query) {
    int per_cu = 0;
    if (query) {
        struct Entry { kq1_fn f; size_t lds; int n; };
        static std::mutex mu;
        static Entry cache[64];
        static int used = 0;
        std::lock_guard<std::mutex> lock(mu);
        for (int i = 0; i < used; i++)
            if (cache[i].f == f && cache[i].lds == lds) return cache[i].n;
        // (the limit is set to the largest LDS any plan takes, so a launch
        // never finds it lowered by a smaller shape's plan)
        if (hipFuncSetAttribute((const void *)f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)KQ1_MAX_LDS) !=
            hipSuccess)
            return -1;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)f, 64 * nw, lds) != hipSuccess)
            return -1;
        if (per_cu < 1) per_cu = 1;
        if (used < 64) cache[used++] = {f, lds, per_cu * KQ1_CU};
        return per_cu * KQ1_CU;
    }
    const int by_lds = (int)((160 * 1024) / (lds ? lds : 1));
    const int by_waves = 4 * (type == T_Q4_K ? KQ4<true>::WAVES : type == T_Q6_KP ? KQ6P::WAVES : KQ6::WAVES) / nw;
    per_cu = by_lds < by_waves ? by_lds : by_waves;
    return (per_cu < 1 ? 1 : per_cu) * KQ1_CU;
}
}  // namespace

// Whether the one-token K-quant kernel serves (type, rows, cols) with W and
// x where they are, and its geometry: lanes per row, waves per workgroup,
// workgroups, LDS bytes.  0: it serves; QG_EINVAL: the caller takes the
// block-unit kernels; QG_EHIP: a device query failed.
//
// The choice of lanes per row and waves per workgroup weighs the unit slots
// a lane runs (more lanes, fewer slots) against the waves the busiest SIMD
// then holds (the decode keeps the vector units busy, so a SIMD's time grows
// with its waves once it holds two or more; with fewer, latency sets it):
// the estimate is slots times the sum over the launch's rounds of max(2,
// waves on the busiest SIMD), a round's workgroups spread evenly over the
// CUs and a workgroup's waves over the 4 SIMDs of its CU.  (At Q6_K 5120 x
// 17408 the busiest CUs held 2 of 320 workgroups of 8 waves: 4 waves per
// SIMD against 2.5 on average.)
int kq1_plan(int type, int64_t rows, int64_t cols, const void *W, const float *x, bool query, int *lpr, int *nw,
             int *wgs, size_t *lds) {
    if ((type != T_Q4_K && type != T_Q6_K && type != T_Q6_KP) || rows < 1 || cols < 256 || cols % 256)
        return QG_EINVAL;
    if (((uintptr_t)x & 15u) || ((uintptr_t)W & (type == T_Q6_KP ? 15u : 1u))) return QG_EINVAL;
    const size_t l = kq1_lds_bytes(type, (int)cols);
    if (cols > (1 << 20) || l > KQ1_MAX_LDS) return QG_EINVAL;
    const int bb = type == T_Q4_K ? 144 : 210;
    if (rows * (cols / 256) * bb >= ((int64_t)1 << 32) - 8) return QG_EINVAL;
    const bool aln = ((uintptr_t)W & 3u) == 0;
    // (4-wave workgroups only for an x of up to 4096 values; wider ones
    // take 8 or more waves: fewer copies of x, and a thread's share of its
    // loads within the register bound)
    const bool wide = l > 40 * 1024 || cols > 4 * 4 * 64 * 4;
    static const int small_w[1] = {4}, wide_w[3] = {8, 10, 16};
    const int *ws = wide ? wide_w : small_w;
    const int nws = wide ? 3 : 1;
    const int nu = (int)(cols / 64);
    double best = 0.0;
    int bl = 0, bw = 0;
    int64_t bwg = 0;
    for (int wi = 0; wi < nws; wi++) {
        const int w = ws[wi];
        if (cols > 12 * 4 * 64 * w) continue;
        // the busiest SIMD's waves in a round of n workgroups, and what the
        // busiest CU's x staging costs in the same unit (each workgroup
        // stages all of x: 0.2 slots per 1024 values, measured at Q6_K
        // 5120 x 17408, where 256 workgroups of 10 waves at 32 lanes per row
        // ran 19.5 us against 21.6 us for 512 at 64 lanes per row)
        auto busiest = [w](int64_t n) {
            const int64_t v = ((n + KQ1_CU - 1) / KQ1_CU * w + 3) / 4;
            return (double)(v > 2 ? v : 2);
        };
        auto staging = [cols](int64_t n) { return 0.2 * (double)cols / 1024.0 * (double)((n + KQ1_CU - 1) / KQ1_CU); };
        for (int L = 16; L <= 64; L *= 2) {
            const int K = (nu + L - 1) / L;
            const int64_t waves = (rows + 64 / L - 1) / (64 / L);
            const int64_t g = (waves + w - 1) / w;
            const int cap = kq1_resident(kq1_kernel(type, aln, L, w, (int)cols), type, w, l, query);
            if (cap < 0) return QG_EHIP;
            const int64_t full = g / cap, rest = g % cap;
            const double est = K * ((double)full * busiest(cap) + (rest ? busiest(rest) : 0.0)) +
                               (double)full * staging(cap) + (rest ? staging(rest) : 0.0);
            if (bl == 0 || est < best - 1e-9) { best = est; bl = L; bw = w; bwg = g; }
        }
    }
    if (bl == 0) return QG_EINVAL;
    if (bwg > 0x7fffffff) return QG_EINVAL;
    *lpr = bl;
    *nw = bw;
    *wgs = (int)bwg;
    *lds = l;
    return QG_OK;
}

int launch_kq1(int type, const Kq1Args &a, hipStream_t st) {
    int L = 0, nw = 0, g = 0;
    size_t lds = 0;
    const int rc = kq1_plan(type, a.rows, a.cols, a.W, a.x, true, &L, &nw, &g, &lds);
    if (rc) return rc;
    const kq1_fn f = kq1_kernel(type, ((uintptr_t)a.W & 3u) == 0, L, nw, a.cols);
    hipLaunchKernelGGL(f, dim3((unsigned)g), dim3(64 * nw), lds, st, a);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_EHIP;
}

}  // namespace qg

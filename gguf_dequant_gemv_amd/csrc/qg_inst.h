// qg_inst.h -- instance table of the GEMV kernel for one (block type, tokens
// per workgroup) pair.  Each qg_inst_<type>_t<NT>.hip includes it once, so the
// instances compile in parallel translation units.
#pragma once
#include "qg_kernels.h"

namespace qg {
namespace inst {

template <int TY, int LPR, int NT>
gemv_fn pick_unr(int unr) {
    constexpr int MAXU = TY == T_Q6_K ? 1 : TY == T_Q4_K ? 2 : 4;
    if constexpr (MAXU >= 4)
        if (unr >= 4) return k_gemv<TY, LPR, NT, 4>;
    if constexpr (MAXU >= 2)
        if (unr >= 2) return k_gemv<TY, LPR, NT, 2>;
    return k_gemv<TY, LPR, NT, 1>;
}

template <int TY, int NT>
gemv_fn pick_lpr(int lpr, int unr) {
    switch (lpr) {
    case 4: return pick_unr<TY, 4, NT>(unr);
    case 8: return pick_unr<TY, 8, NT>(unr);
    case 16: return pick_unr<TY, 16, NT>(unr);
    case 32: return pick_unr<TY, 32, NT>(unr);
    default: return pick_unr<TY, 64, NT>(unr);
    }
}

}  // namespace inst
}  // namespace qg

#define QG_GEMV_INSTANCES(NAME, TY, NT) \
    namespace qg { \
    gemv_fn gemv_kernel_##NAME##_t##NT(int lpr, int unr) { return inst::pick_lpr<TY, NT>(lpr, unr); } \
    }

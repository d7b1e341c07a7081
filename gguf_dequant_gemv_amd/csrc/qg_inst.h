// qg_inst.h -- instance table of the GEMV kernel for one (block type, tokens
// per workgroup) pair.  Each qg_inst_<type>_t<NT>.hip includes it once, so the
// instances compile in parallel translation units.
#pragma once
#include "qg_kernels.h"

namespace qg {
namespace inst {

template <class U, int NT>
gemv_fn pick_lpr(int lpr) {
    switch (lpr) {
    case 4: return k_gemv<U, 4, NT>;
    case 8: return k_gemv<U, 8, NT>;
    case 16: return k_gemv<U, 16, NT>;
    case 32: return k_gemv<U, 32, NT>;
    default: return k_gemv<U, 64, NT>;
    }
}

template <class U, int NT, bool ALN, bool XC, bool RT = false>
gemv_fn pick_lpr_lds(int lpr) {
    if constexpr (U::BYTES % 4 != 0) {   // 8 lanes or more make whole 16-byte segments
        switch (lpr) {
        case 16: return k_gemv_lds<U, 16, NT, ALN, XC, RT>;
        case 32: return k_gemv_lds<U, 32, NT, ALN, XC, RT>;
        case 64: return k_gemv_lds<U, 64, NT, ALN, XC, RT>;
        default: return k_gemv_lds<U, 8, NT, ALN, XC, RT>;
        }
    } else {
        switch (lpr) {
        case 4: return k_gemv_lds<U, 4, NT, ALN, XC, RT>;
        case 8: return k_gemv_lds<U, 8, NT, ALN, XC, RT>;
        case 16: return k_gemv_lds<U, 16, NT, ALN, XC, RT>;
        case 32: return k_gemv_lds<U, 32, NT, ALN, XC, RT>;
        default: return k_gemv_lds<U, 64, NT, ALN, XC, RT>;
        }
    }
}

// rt: the launch routes its one token itself (a separate instance, so the
// routing code costs the other launches nothing)
template <class U, int NT, bool ALN>
gemv_fn pick_lds(int lpr, bool xc, bool rt) {
    if constexpr (NT == 1) {
        if (rt && !xc) return pick_lpr_lds<U, NT, ALN, false, true>(lpr);
    }
    return xc ? pick_lpr_lds<U, NT, ALN, true>(lpr) : pick_lpr_lds<U, NT, ALN, false>(lpr);
}

template <int TY> struct Units;
template <> struct Units<T_Q8_0> { typedef UQ8_0B B; typedef UQ8_0P P; };
template <> struct Units<T_Q4_0> { typedef UQ4_0B B; typedef UQ4_0P P; };
template <> struct Units<T_Q4_K> { typedef UQ4_K B; typedef UQ4_K P; };
template <> struct Units<T_Q6_K> { typedef UQ6_K B; typedef UQ6_K P; };

// UK_BLOCK exists for Q8_0 / Q4_0, and for Q6_K at one token per workgroup
// (Q4_K always stages in LDS)
template <int TY, int NT>
gemv_fn pick(int kind, int lpr, bool xc, bool rt) {
    if constexpr (TY == T_Q8_0 || TY == T_Q4_0 || (TY == T_Q6_K && NT == 1)) {
        if (kind == UK_BLOCK) return pick_lpr<typename Units<TY>::B, NT>(lpr);
    }
    if (kind == UK_LDS) return pick_lds<typename Units<TY>::P, NT, true>(lpr, xc, rt);
    return pick_lds<typename Units<TY>::P, NT, false>(lpr, xc, rt);
}

}  // namespace inst
}  // namespace qg

#define QG_GEMV_INSTANCES(NAME, TY, NT) \
    namespace qg { \
    gemv_fn gemv_kernel_##NAME##_t##NT(int kind, int lpr, bool xc, bool rt) { \
        return inst::pick<TY, NT>(kind, lpr, xc, rt); \
    } \
    }

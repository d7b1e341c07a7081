// Dequantization kernel instances (one per block type).
#include "qg_kernels.h"

namespace qg {
dequant_fn dequant_kernel(int type) {
    switch (type) {
    case T_Q8_0: return k_dequant<T_Q8_0>;
    case T_Q4_0: return k_dequant<T_Q4_0>;
    case T_Q4_K: return k_dequant<T_Q4_K>;
    default: return k_dequant<T_Q6_K>;
    }
}
}  // namespace qg

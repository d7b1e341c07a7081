// Dequantization kernel instances (one per block type, on the block units).
#include "qg_kernels.h"

namespace qg {
dequant_fn dequant_kernel(int type) {
    switch (type) {
    case T_Q8_0: return k_dequant<UQ8_0B>;
    case T_Q4_0: return k_dequant<UQ4_0B>;
    case T_Q4_K: return k_dequant<UQ4_K>;
    default: return k_dequant<UQ6_K>;
    }
}
}  // namespace qg

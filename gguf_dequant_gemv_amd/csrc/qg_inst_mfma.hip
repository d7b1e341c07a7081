// MFMA small-batch GEMV instances (Q8_0 / Q4_0): 4 or 2 groups of 16 rows
// per tile (gated tiles split their groups between gate and up rows).
#include "qg_kernels.h"

namespace qg {

gemv_fn gemv_kernel_mfma(int type, int groups) {
    if (type == T_Q8_0) return groups == 4 ? k_gemv_mfma<T_Q8_0, 4> : k_gemv_mfma<T_Q8_0, 2>;
    return groups == 4 ? k_gemv_mfma<T_Q4_0, 4> : k_gemv_mfma<T_Q4_0, 2>;
}

}  // namespace qg

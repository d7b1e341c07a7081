// Q6_K GEMV instances with 4 token(s) per workgroup.
#include "qg_inst.h"
QG_GEMV_INSTANCES(q6_k, qg::T_Q6_K, 4)

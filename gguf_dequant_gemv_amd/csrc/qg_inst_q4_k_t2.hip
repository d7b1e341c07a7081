// Q4_K GEMV instances with 2 token(s) per workgroup.
#include "qg_inst.h"
QG_GEMV_INSTANCES(q4_k, qg::T_Q4_K, 2)

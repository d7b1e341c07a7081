// Q4_0 GEMV instances with 2 token(s) per workgroup.
#include "qg_inst.h"
QG_GEMV_INSTANCES(q4_0, qg::T_Q4_0, 2)

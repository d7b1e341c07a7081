// Q8_0 GEMV instances with 1 token(s) per workgroup.
#include "qg_inst.h"
QG_GEMV_INSTANCES(q8_0, qg::T_Q8_0, 1)

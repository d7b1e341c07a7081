// qg_moe1.h -- the one-token down projection + combine of the routed experts
// (qg_moe1.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

struct Moe1Args {
    const uint8_t *W;        // pool of expert down matrices, slot s at W + s * stride
    int64_t stride;
    int64_t rows, row_bytes; // H rows of row_bytes each
    int nb;                  // blocks per row (F / 32)
    const float *act;        // [k][act_stride] activations of the picks, pick order
    int64_t act_stride;
    const int32_t *ids;      // [k] picked experts, pick order
    const float *w;          // [k] routing weights
    const int32_t *slots;    // expert -> pool slot
    int n_slots;
    const float *escale;     // per-expert down scale, or nullptr
    const int32_t *valid;    // [1] 0: a pick has no slot, y is left as it is
    float *dn;               // [k][rows] the terms (dn_j * s) * w_j
    float *y;                // [rows] the sum of the terms, or nullptr
    int k;
    // the shared expert, when shW is set: its down matrix (rows x the same
    // row_bytes), its activation row, and the scalar gate (gate_inp . x);
    // then resid[r] = (sum of the terms + sh[r] * sigmoid(gate)) + resid[r]
    // and sh[r] (the raw shared output) goes to sh_out
    const uint8_t *shW;
    const float *sh_act;
    const float *gate_inp;
    const float *x;
    float *resid;
    float *sh_out;
};

// whether a (block type, F, top-k) the one-token launch serves
bool moe_down1_fits(int type, int64_t cols, int k);
int launch_moe_down1(int type, const Moe1Args &a, hipStream_t st);

}  // namespace qg

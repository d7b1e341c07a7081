// qg_moe1.h -- one token's down projections and combine (qg_moe1.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qg_kernels.h"

namespace qg {

constexpr int MOE1_L = 32;      // lanes per row: 8 rows per workgroup
constexpr int MOE1_MAXK = 8;    // routed picks one launch serves
constexpr int MOE1_MAXX = 4;    // units per lane of a dense MLP's down row (F up to 4096)

// Extra pick beside the routed ones
enum { XP_NONE = 0, XP_SHARED = 1, XP_DENSE = 2 };

struct Moe1Args {
    const uint8_t *W;        // pool of expert down matrices, slot s at W + s * stride
    int64_t stride;
    int64_t rows, row_bytes; // H rows of row_bytes each
    int nb;                  // blocks per row (F / 32)
    const float *act;        // [k][act_stride] activations of the picks, pick order
    int64_t act_stride;
    const float *w;          // [k] routing weights, pick order
    const int32_t *pslot;    // [k] the picks' pool slots, pick order
    const float *pes;        // [k] their down scales (1 without one)
    int n_slots;
    const int32_t *valid;    // [1] 0: a pick has no slot, y is left as it is
    float *dn;               // [k][rows] the terms (dn_j * s) * w_j
    float *y;                // [rows] the sum of the terms, or nullptr
    int k;
    // XP_SHARED (shW set): the shared expert's down matrix (rows x the same
    // row_bytes), its activation row, and the scalar gate (gate_inp . x);
    // then resid[r] = (sum of the terms + sh[r] * sigmoid(gate)) + resid[r]
    // and sh[r] (the raw shared output) goes to sh_out
    const uint8_t *shW;
    const float *sh_act;
    const float *gate_inp;
    const float *x;
    float *resid;
    float *sh_out;
    const float *gate_logit;   // when set: the gate logit, already reduced (the routing launch's)
    // XP_DENSE (dW set): a dense MLP's down matrix beside the experts (rows x
    // d_row_bytes, d_nb blocks a row), its activation row [d_nb * 32] and its
    // output y_mlp [rows], kept apart from the experts' sum
    const uint8_t *dW;
    int64_t d_row_bytes;
    int d_nb;
    const float *d_act;
    float *y_mlp;
};

// What a down workgroup takes from the routing, per pick j < k: the pool
// slot, the per-expert scale, the routing weight; and the token's validity.
struct Picks {
    int slot[MOE1_MAXK];
    float es[MOE1_MAXK], wj[MOE1_MAXK];
    bool ok;
};

// whether a (block type, F, top-k) the one-token launch serves
bool moe_down1_fits(int type, int64_t cols, int k);
// the same with a dense MLP's down row (dense_cols wide) as the extra pick
bool moe_down1_fits_dense(int type, int64_t cols, int64_t dense_cols, int k);
int launch_moe_down1(int type, const Moe1Args &a, hipStream_t st);

}  // namespace qg

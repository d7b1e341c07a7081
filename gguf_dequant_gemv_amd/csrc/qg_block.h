// qg_block.h -- host-side launchers of the kernels around the routed experts
// (qg_block.hip), used by the C ABI in qg_abi.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

int launch_embed(int type, const uint8_t *W, int64_t rows, int cols, int64_t row_bytes, const int32_t *tok,
                 int ntok, float scale, float *out, hipStream_t st);

// argmax: logits per workgroup in the first phase, and at most this many
// partial results per token
constexpr int64_t ARGMAX_SPAN = 2048;
constexpr int ARGMAX_MAX_PARTS = 256;
int argmax_parts(int64_t n);

int launch_rmsnorm(const float *x, const float *w, float *y, int64_t n, int ntok, float eps, float k,
                   hipStream_t st);
int launch_norm_gemv_f32(const float *x, int64_t n, int ntok, float eps, const float *rw, float rk, const float *W,
                         int64_t rows, float *y, int nout, const float *const *w, const float *k, float *const *yo,
                         hipStream_t st);
int launch_rmsnorm_multi(const float *x, int64_t n, int ntok, float eps, int nout, const float *const *w,
                         const float *k, float *const *y, hipStream_t st);
int launch_gemv_f32(const float *W, const float *x, float *y, int64_t rows, int64_t cols, int ntok,
                    hipStream_t st);
int launch_combine_shared(const float *dn, const int32_t *rt_valid, const float *sh, const float *gate_inp,
                          const float *x, float *resid, int64_t H, int k, int ntok, hipStream_t st);
int launch_post_ffn(const float *mlp, const float *moe, const float *w1, const float *w2, const float *w,
                    const float *os, float *x, int64_t n, int ntok, float eps, hipStream_t st);
int launch_argmax(float *l, int64_t n, int ntok, float cap, float *pv, int32_t *pi, int32_t *idx,
                  hipStream_t st);
int launch_argmax_embed(float *l, int64_t n, int ntok, float cap, float *pv, int32_t *pi, int32_t *idx, int type,
                        const uint8_t *W, int64_t rows, int cols, int64_t row_bytes, float scale, float *out,
                        hipStream_t st);

}  // namespace qg

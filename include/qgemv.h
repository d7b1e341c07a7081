/*
 * qgemv.h -- C ABI of libqgemv: decode-time matrix-vector products over GGUF
 * block-quantized weights, dequantized inside HIP kernels for gfx950 (MI355X)
 * with f32 accumulation, and the routed mixture-of-experts step built on them.
 *
 * Sources (the diskformer package-diff pages this library follows):
 *   [bonsai]  diskformer 0.5.4 -> 0.6.6, engines/ternary_bonsai_2_dflash.js
 *   [gemma4]  diskformer 0.0.1 -> 0.2.0, engines/gemma4_moe_ssd.js
 *   [qwen3]   diskformer 0.0.1 -> 0.3.0, engines/qwen3_moe_ssd.js
 *   [qwen35]  diskformer 0.0.1 -> 0.3.0, engines/qwen35_moe_ssd.js
 *   [dense]   diskformer 0.5.4 -> 0.6.6, engines/qwen35_dense.js
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a DEVICE pointer unless stated otherwise; the
 *     caller owns all memory (the library allocates nothing on any call).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *     work on it and return without synchronising; results are valid once the
 *     stream has reached that point.
 *   - Return value: QG_OK, or a negative qg_err code from synchronous argument
 *     validation (nothing is enqueued then), or QG_EHIP when a launch fails.
 *     No C++ exception crosses the ABI.
 *   - Weights are GGUF block streams: row-major, rows contiguous, row r at byte
 *     r * (cols / QK) * block_bytes, blocks exactly as GGUF stores them (no
 *     padding, no plane split).  W needs only 2-byte alignment.  The GGUF dims
 *     order is (cols, rows): dims[0] is the contiguous, quantized axis.
 *   - Activations are f32, token-major: x is [ntok][cols], y is [ntok][rows].
 *     Outputs are overwritten, except where an entry point states that it
 *     updates the residual stream in place.
 *   - 1 <= ntok <= QG_MAX_TOKENS unless an entry point states its own limit;
 *     cols must be a multiple of the block's QK.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Block types, numbered as GGML/GGUF number them ([bonsai] GGUF reader prints
 * Q4_K = 12 and Q6_K = 14; Q4_0 = 2 and Q8_0 = 8 are the same enum).
 *   Q8_0  34 B / 32 values : f16 d | int8 q[32]            value = d*q
 *         ([qwen3] header comment and WGSL i8at / matmulQ8)
 *   Q4_0  18 B / 32 values : f16 d | 16 B nibbles           value = (nib-8)*d,
 *         byte j holds value j (low nibble) and j+16 (high) ([gemma4] q4dot)
 *   Q4_K 144 B / 256 values: f16 d | f16 dmin | scales[12] | qs[128]
 *         value = d*sc*q - dmin*m per 32-value sub-block ([bonsai] dequantQ4K)
 *   Q6_K 210 B / 256 values: ql[128] | qh[64] | int8 scales[16] | f16 d
 *         value = d*sc*(q-32) per 16 values ([bonsai] dequantQ6K)
 *   F32     4 B / 1 value  : IEEE binary32 (GGML's 0), accepted by qg_gemv only:
 *         the router and shared-expert gate weights ([qwen3] matmulF32)     */
enum qg_type {
    QG_F32 = 0, QG_Q4_0 = 2, QG_Q8_0 = 8, QG_Q4_K = 12, QG_Q6_K = 14,
    QG_Q8_0_PLANES = 264, QG_Q6_K_PLANES = 270
};

/* QG_Q6_K_PLANES: a Q6_K tensor in the device layout qg_prepare writes
 * ([gemma4] q6kPlanes: the 210-byte blocks, which sit at 2-byte alignment,
 * split into aligned planes at load).  A tensor of n = rows * cols / 256
 * blocks is one buffer of 210 n bytes, 16-byte aligned, holding
 *   ql [n][128] at byte 0, qh [n][64] at 128 n, int8 scales [n][16] at
 *   192 n, f16 d [n] at 208 n
 * in the blocks' row-major order: the blocks' bytes, reordered (the page
 * widens d to f32; here it keeps its two bytes).  Not a GGUF type (GGML's
 * Q6_K id with bit 8 set).  Accepted by qg_gemv at ntok = 1 with x 16-byte
 * aligned and 210 n <= 2 GiB, by qg_dequant, qg_embed, qg_argmax_embed,
 * qg_gemv_plan, qg_block_values (256) and qg_block_bytes (210); every other
 * entry point rejects it.
 *
 * QG_Q8_0_PLANES: a Q8_0 tensor in the layout qg_prepare writes ([qwen3]
 * WGSL i8at reads Q8_0 from a code plane and per-group scales): for rows x
 * cols values, one buffer of 34 rows cols / 32 bytes, 16-byte aligned:
 *   the int8 codes [rows][cols] at byte 0, then the f16 scales
 *   [rows][cols / 32] at byte rows * cols
 * (the blocks' bytes, reordered: a row of codes is cols contiguous bytes,
 * whole 128-byte lines when cols is a multiple of 128).  Accepted by qg_gemv
 * at ntok = 1 with x 16-byte aligned, rows * cols < 2^31 and cols <= 12288,
 * by qg_mlp at ntok = 1 (all three tensors in the layout), by qg_dequant,
 * qg_embed, qg_argmax_embed, qg_gemv_plan (kind 5), qg_block_values (32)
 * and qg_block_bytes (34); every other entry point rejects it. */

/* Gated activations: act(gate) * up.
 *   QG_ACT_SILU       gate / (1 + exp(-gate))           ([qwen3] siluMulMoe)
 *   QG_ACT_GELU_TANH  0.5 g (1 + tanh(clamp(0.7978845608 g (1 + 0.044715 g^2),
 *                     -10, 10)))                         ([gemma4] GELU, geglu) */
enum qg_act { QG_ACT_SILU = 0, QG_ACT_GELU_TANH = 1 };

enum qg_err {
    QG_OK = 0,
    QG_EINVAL = -1,   /* bad type, size, pointer or alignment                  */
    QG_EABSENT = -2,  /* (status word only) a picked expert has no slot        */
    QG_EHIP = -3,     /* a HIP launch or query failed                           */
    QG_ELIMIT = -4    /* a size limit below is exceeded                         */
};

#define QG_MAX_TOKENS 16    /* small-batch (speculative verify) limit          */
#define QG_MAX_PREFILL 4096 /* prefill chunk limit of qg_gemm and qg_mlp       */
#define QG_MAX_EXPERTS 256  /* router width limit ([qwen3] engine: n <= 256)    */
#define QG_MAX_TOPK 32      /* picks per token limit ([qwen3] engine: k <= 32)  */

/* Values and bytes per block of `type` (1 and 4 for QG_F32); 0 for an unknown
 * type.  Host only. */
int qg_block_values(int type);
int qg_block_bytes(int type);

/* Human-readable name of a qg_err code (static string).  Host only. */
const char *qg_strerror(int code);

/* Quantized GEMV / small-batch GEMV.
 *   y[t][r] = sum_c W[r][c] * x[t][c]   for t < ntok, r < rows
 * with W dequantized in registers and f32 accumulation.  Each weight byte is
 * read once per call for ntok <= 8 (twice at most for ntok <= 16 when the
 * tokens do not fit in local memory together).
 * The sum the pages' GEMV kernels compute: [qwen3] WGSL matmulQ8, [gemma4]
 * matmulQ4 / matmulQ6K, [bonsai] packed-weight GEMMs, [qwen35] matmulQ8T.
 * W: rows x cols GGUF blocks; x: [ntok][cols] f32; y: [ntok][rows] f32.
 * type QG_F32: W is a plain row-major f32 matrix (4-byte aligned), the
 * router's logits and the shared expert's gate logit ([qwen3] matmulF32,
 * [qwen35] shgate binding).
 * type QG_Q6_K_PLANES: W is a Q6_K tensor in the plane layout (16-byte
 * aligned, 210 * rows * cols / 256 <= 2^31 bytes), one token, x 16-byte
 * aligned; the same sum as on the blocks.  QG_Q8_0_PLANES likewise (rows *
 * cols < 2^31, cols <= 12288).
 * Errors: QG_EINVAL (type, rows<=0, cols<=0 or cols % QK, null pointer, W not
 * 2-byte aligned, x/y not 4-byte aligned; for the plane layouts W or x not
 * 16-byte aligned, ntok != 1, or Q8_0 planes with cols > 12288), QG_ELIMIT
 * (ntok outside 1..16; a plane tensor over 2 GiB). */
int qg_gemv(int type, const void *W, const float *x, float *y,
            int64_t rows, int64_t cols, int ntok, void *stream);

/* Prefill-size product: the same sum as qg_gemv for a chunk of up to
 * QG_MAX_PREFILL tokens ([qwen35] / [gemma4] WGSL matmulQ8T / matmulQ4T, the
 * tiled prompt-chunk GEMMs).  Q8_0 / Q4_0 run on the matrix cores with every
 * product exact (codes and three bf16 parts of x); the K-quants and f32 run
 * on the vector kernels in chunks of tokens.
 * workspace: device scratch of at least qg_gemm_workspace_size(type, rows,
 * cols, ntok) bytes, 256-byte aligned (may be NULL when that size is 0).  It
 * holds partial sums when a launch with few row tiles is split along the row
 * (prefill chunks, and Q8_0 / Q4_0 batches of 4..16 tokens over rows of 192
 * or more blocks; qg_gemv runs those batches unsplit); its contents after the
 * call are unspecified.
 * Arguments and errors as qg_gemv, with QG_ELIMIT for ntok outside
 * 1..QG_MAX_PREFILL and QG_EINVAL for a short or misaligned workspace. */
size_t qg_gemm_workspace_size(int type, int64_t rows, int64_t cols, int ntok);
int qg_gemm(int type, const void *W, const float *x, float *y,
            int64_t rows, int64_t cols, int ntok, void *workspace,
            size_t workspace_bytes, void *stream);

/* The launch plan qg_gemv takes for a shape (host only; for tests and tuning).
 * out[8] (a HOST array) receives: [0] kernel kind (0 per-lane unit loads, 1
 * weights staged through LDS from 16-byte-aligned rows, 2 the same for any
 * 2-byte phase, 3 matrix-core small batch, 4 one token against Q4_K / Q6_K
 * rows in quarter-block units, taken when x is 16-byte aligned), [1] lanes per
 * row (0 for kind 3), [2] tokens per workgroup, [3] row tiles, [4] workgroups
 * along the rows (grid-stride: each walks row tiles wg, wg + [4], ...; needs a
 * device query, 0 when query_device is 0; kind 4: one tile each), [5] dynamic
 * LDS bytes, [6] weight stages in flight per wave (kind 4: units in flight per
 * lane), [7] x chunk (row elements staged at a time, 0 = all of x; kind 4:
 * waves per workgroup).  Kind 5: one token against Q8_0 planes, a wave
 * walking rows in 16-byte code pieces ([1] 64 lanes a row, [3] workgroups
 * for one row a wave, [4] workgroups launched (every one that fits, each
 * wave walking rows w, w + W, ...), [6] pieces in flight per lane, [7]
 * waves per workgroup).
 * The plan of the first launch of the call (launches cover at most 2 GiB of
 * weights each).  w_aligned16: W would start 16-byte aligned.
 * Errors: as qg_gemv, QG_EINVAL for a null out, QG_EHIP when the device query
 * fails. */
int qg_gemv_plan(int type, int64_t rows, int64_t cols, int ntok, int w_aligned16, int query_device,
                 int32_t *out);

/* Dequantize a whole tensor: out[r][c] = W[r][c] as f32, bit-exact (each
 * value is the f32 nearest to its exact value; for Q8_0, Q4_0 and Q6_K the
 * exact value is always an f32).  The block-unpack layer's test hook.
 * Formulas: [bonsai] dequantQ4K / dequantQ6K, [gemma4] q4dot, [qwen3] i8at.
 * Errors: as qg_gemv (no ntok). */
int qg_dequant(int type, const void *W, float *out, int64_t rows, int64_t cols, void *stream);

/* The aligned device layouts of Q6_K and Q8_0 tensors, and back ([gemma4]
 * q6kPlanes, [qwen3] i8at's code plane).
 * qg_prepare:   src = the GGUF blocks of a rows x cols Q6_K or Q8_0 tensor
 *               (2-byte aligned), dst = as many bytes (16-byte aligned),
 *               written in the QG_Q6_K_PLANES / QG_Q8_0_PLANES layout.
 * qg_unprepare: the inverse (src the planes, 16-byte aligned; dst the
 *               blocks, 2-byte aligned).
 * A byte permutation: unprepare(prepare(W)) is W byte for byte, and qg_gemv /
 * qg_dequant give the same sums / values on either layout (up to summation
 * order for the GEMV).  A load-time step: one launch of one thread per 2
 * bytes.  type: QG_Q6_K or QG_Q8_0, the types with a prepared layout.
 * Errors: QG_EINVAL (another type, rows or cols out of range, cols not a
 * multiple of 256, a null or misaligned pointer, src and dst overlapping),
 * QG_ELIMIT (more than 2^31 workgroups). */
int qg_prepare(int type, const void *src, void *dst, int64_t rows, int64_t cols, void *stream);
int qg_unprepare(int type, const void *src, void *dst, int64_t rows, int64_t cols, void *stream);

/* Router: per token, the k experts with the largest logits (ties go to the
 * lower expert index), in pick order, and their weights renormalised over the
 * picks: w_j = exp(l_j - l_max) / sum_{i picked} exp(l_i - l_max).  This is the
 * [qwen3] WGSL topk kernel (softmax, k argmax rounds with ties to the lowest
 * index, renormalisation); the selection ranks logits, which orders exactly as
 * the probabilities do.
 * logits: [ntok][n_experts] f32; ids: [ntok][k] int32; weights: [ntok][k] f32.
 * Errors: QG_EINVAL (null pointer), QG_ELIMIT (n_experts outside 1..256, k
 * outside 1..min(32, n_experts), ntok outside 1..16). */
int qg_router_topk(const float *logits, int n_experts, int k, int ntok,
                   int32_t *ids, float *weights, void *stream);

/* Dense gated MLP (one FFN without norms or residual):
 *   gu   = [W_gate x | W_up x]
 *   a    = act(gu[0:ff]) * gu[ff:2ff]          (same launch as gu: each row
 *                                              tile reads its gate rows, then
 *                                              the same rows of W_up)
 *   y    = W_down a
 * [dense] encodeLayer (gate and up into the two halves of one buffer, siluMul,
 * down); [gemma4] dense GELU MLP (geglu).
 * W_gate, W_up: ff x hidden; W_down: hidden x ff (same block type).
 * x: [ntok][hidden], y: [ntok][hidden]; 1 <= ntok <= QG_MAX_PREFILL (a
 * decode step, a verify batch or a prefill chunk).
 * workspace: device scratch of at least qg_mlp_workspace_size(type, hidden,
 * ff, ntok) bytes, 256-byte aligned.  After the call it holds gu as
 * [ntok][2*ff] f32 at offset 0 and a as [ntok][ff] f32 after it (at the next
 * 256-byte boundary): documented intermediates, useful for staged checking.
 * Prefill chunks and split small batches (as qg_gemm) may use more scratch
 * after a (unspecified contents).
 * type QG_Q8_0_PLANES (all three tensors in that layout, 16-byte aligned, x
 * too): one token, the gated plane launch and the plane GEMV of down; the
 * workspace and its gu / a parts as for QG_Q8_0.
 * Errors: as qg_gemv for both shapes, QG_EINVAL for a short workspace or an
 * unknown act (for QG_Q8_0_PLANES also ntok != 1, or hidden or ff over
 * 12288). */
size_t qg_mlp_workspace_size(int type, int64_t hidden, int64_t ff, int ntok);
int qg_mlp(int type, int act, const void *W_gate, const void *W_up, const void *W_down,
           int64_t hidden, int64_t ff, const float *x, float *y, int ntok,
           void *workspace, size_t workspace_bytes, void *stream);

/* A pool of routed experts (a HOST struct; its pointers are device pointers).
 * Expert e lives in pool slot expert_slots[e] (0 <= slot < n_slots); the
 * weights of slot s are
 *   gate_up + s * gate_up_stride : (2 ff) x hidden blocks, gate rows first
 *   down    + s * down_stride    : hidden x ff blocks
 * (strides in bytes; [qwen3] expert record guQ then dQ, [gemma4] fused
 * ffn_gate_up_exps).  down_scale: [n_experts] f32 per-expert factor applied to
 * the down output ([gemma4] moeSum), or NULL for 1. */
typedef struct qg_moe {
    int type;            /* qg_type of both projections                        */
    int act;             /* qg_act                                             */
    int64_t hidden;      /* H: x and y width                                   */
    int64_t ff;          /* F: expert feed-forward width                       */
    int n_experts;       /* E: router width                                    */
    const void *gate_up; int64_t gate_up_stride;
    const void *down;    int64_t down_stride;
    const float *down_scale;
    int n_slots;         /* slots in the pool; a slot outside [0, n_slots) is
                            treated as absent.  0 means n_experts.          */
} qg_moe;

/* Routed-expert FFN for ntok tokens ([qwen3] encodeExperts: topk, expertQ8 on
 * gate||up, siluMulMoe, expertQ8 on down, moeAccum; [gemma4] encodeExpertsB:
 * topkB, expertQ4B, geglu, expertQ4B, moeSumB):
 *   ids, c = router(router_logits[t])       (as qg_router_topk)
 *   gu_j   = W_gate_up[slot(ids_j)] x[t]
 *   a_j    = act(gu_j[0:F]) * gu_j[F:2F]
 *   dn_j   = W_down[slot(ids_j)] a_j
 *   y[t]   = sum_j (dn_j * s[ids_j]) * c_j   (pick order)
 * Pairs that pick the same expert are grouped so each picked expert's weights
 * are read once per call for all the tokens that picked it.
 * m: host pointer to the pool description.
 * router_logits: [ntok][E]; expert_slots: [E] int32 (-1 = not resident);
 * x, y: [ntok][H]; ids_out: [ntok][topk] int32; w_out: [ntok][topk] f32
 * (both may be NULL); status: one device int32, set to QG_OK or QG_EABSENT.
 * A token with an absent pick gets no output (its y row is left as it was)
 * and the status word reads QG_EABSENT.
 * workspace: at least qg_moe_workspace_size(m, topk, ntok) bytes, 256-byte
 * aligned.  After the call it holds, at offset 0, gu as [ntok][topk][2F] f32,
 * and a as [ntok][topk][F] f32 after it (at the next 256-byte boundary).
 * Errors: as qg_gemv for both shapes; QG_ELIMIT (n_experts > 256, topk > 32 or
 * > n_experts, ntok > 16); QG_EINVAL (short workspace, null pointer, bad act). */
size_t qg_moe_workspace_size(const qg_moe *m, int topk, int ntok);
int qg_moe_ffn(const qg_moe *m, const float *router_logits, int topk,
               const int32_t *expert_slots, const float *x, float *y, int ntok,
               int32_t *ids_out, float *w_out, int32_t *status,
               void *workspace, size_t workspace_bytes, void *stream);

/* qg_moe_ffn without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc).  Its scratch is a static device array of
 * QG_NOALLOC_SCRATCH_BYTES inside the library: one copy per GPU, created with
 * the library's code object on that GPU and held until the process ends; the
 * call itself allocates nothing.  The current device must be the stream's.
 * Every call on a GPU uses that GPU's one copy, so calls that overlap on one
 * GPU (on different streams, or from different host threads) race and must
 * not be issued.  After a call the scratch holds what qg_moe_ffn's workspace
 * would (gu, act, ...); the next call overwrites it.
 * Arguments, results and errors as qg_moe_ffn, and QG_ELIMIT when
 * qg_moe_workspace_size(m, topk, ntok) exceeds QG_NOALLOC_SCRATCH_BYTES. */
#define QG_NOALLOC_SCRATCH_BYTES (8u << 20)
int qg_moe_ffn_noalloc(const qg_moe *m, const float *router_logits, int topk, const int32_t *expert_slots,
                       const float *x, float *y, int ntok, int32_t *ids_out, float *w_out, int32_t *status,
                       void *stream);

/* ------------------------------------------------ around the routed experts */

/* RMS norm with a scalar factor, per token of n values:
 *   r = 1 / sqrt(sum_i x_i^2 / n + eps),   y_i = ((x_i * r) * k) * w_i
 * [qwen3] WGSL rmsnorm (k = 1: the FFN input xn) and [gemma4] rmsnormK (the
 * router's input: k = 1/sqrt(H), w = ffn_gate_inp.scale).
 * x, y: [ntok][n] f32 (y may equal x); w: [n] f32.  One workgroup per token.
 * Errors: QG_EINVAL (n <= 0, ntok < 1, eps < 0 or NaN, null or misaligned
 * pointer). */
int qg_rmsnorm(const float *x, const float *w, float *y, int64_t n, int ntok, float eps, float k,
               void *stream);

/* Several RMS norms of the same vectors in one launch: output o is
 *   y_o[t][i] = ((x[t][i] * r_t) * k[o]) * w_o[i]
 * with r_t as in qg_rmsnorm, bit for bit what nout qg_rmsnorm calls give.
 * Gemma's FFN block takes three of them from one residual row: ffn_norm (the
 * dense MLP's input), pre_ffw_norm_2 (the experts' input) and the router's
 * rmsnormK ([gemma4] encodeLayer's norms before the FFN).
 * w, y, k: HOST arrays of nout entries (device pointers w[o], y[o]; factors
 * k[o]); no y[o] may overlap x or another y.  1 <= nout <= QG_MAX_NORMS.
 * Errors: as qg_rmsnorm, and QG_ELIMIT for nout outside 1..QG_MAX_NORMS. */
#define QG_MAX_NORMS 4
int qg_rmsnorm_multi(const float *x, int64_t n, int ntok, float eps, int nout, const float *const *w,
                     const float *k, float *const *y, void *stream);

/* A block's input norms and its f32 router in one launch, per token t:
 *   logits[t][e] = sum_i W[e][i] * (((x[t][i] * r_t) * rk) * rw[i])
 *   y_o[t][i]    = ((x[t][i] * r_t) * k[o]) * w_o[i]      (o < nout)
 * r_t as in qg_rmsnorm: the router's logits of its normed input ([qwen35]
 * rmsnorm then the router matmulF32; [gemma4] rmsnormK then the router) and
 * up to QG_MAX_NORMS other norms of the same rows (the experts' and the
 * dense MLP's inputs), bit for bit what qg_rmsnorm / qg_rmsnorm_multi and
 * qg_gemv(QG_F32, ...) on the router's norm give when x, rw and W are
 * 16-byte aligned and n % 4 == 0.  Meant for decode steps: every workgroup
 * takes every token's sums of squares, so at many tokens the separate
 * launches are faster.
 * x: [ntok][n]; rw: [n]; W: [rows][n] f32 (row-major); logits: [ntok][rows];
 * w, k, y: HOST arrays of nout entries as in qg_rmsnorm_multi (nout may be 0);
 * no y[o] may overlap x, W or logits.
 * Errors: QG_EINVAL (n <= 0, rows <= 0, eps < 0 or NaN, null or misaligned
 * pointer), QG_ELIMIT (ntok outside 1..16, nout outside 0..QG_MAX_NORMS). */
int qg_rmsnorm_router(const float *x, int64_t n, int ntok, float eps, const float *rw, float rk, const float *W,
                      int64_t rows, float *logits, int nout, const float *const *w, const float *k,
                      float *const *y, void *stream);

/* The shared expert of a MoE block (a HOST struct; its pointers are device
 * pointers): a dense gated MLP with ff SF beside the routed experts, scaled
 * by the logistic of a scalar gate logit ([qwen35] ffn_gate_shexp,
 * ffn_up_shexp, ffn_down_shexp, ffn_gate_inp_shexp). */
typedef struct qg_shared_expert {
    int type;               /* qg_type of gate, up and down (not QG_F32)       */
    int64_t ff;             /* SF                                              */
    const void *gate;       /* SF x H blocks                                   */
    const void *up;         /* SF x H blocks                                   */
    const void *down;       /* H x SF blocks                                   */
    const float *gate_inp;  /* [H] f32: the scalar gate's weight row           */
} qg_shared_expert;

/* MoE block with a shared expert and the residual ([qwen35] encodeAttention's
 * shared-expert dispatches and encodeExperts; WGSL moeAccumShared /
 * moeAccumSharedB), per token t:
 *   terms_j = (dn_j * s[ids_j]) * c_j          (the routed part, as qg_moe_ffn)
 *   sh      = W_sd (act(W_sg x) * (W_su x))    (act = m->act)
 *   sg      = gate_inp . x
 *   resid   = (sum_j terms_j + sh * sigmoid(sg)) + resid      (in place)
 * x is the block's (normed) input, resid the residual stream [ntok][H],
 * updated in place.  A token with an absent pick keeps its resid row and the
 * status word reads QG_EABSENT.
 * workspace: at least qg_moe_shared_workspace_size(m, sh, topk, ntok) bytes,
 * 256-byte aligned: qg_moe_ffn's workspace (same layout), then the shared
 * expert's gu [ntok][2 SF] and act [ntok][SF] (qg_mlp's layout, with its
 * scratch after act when it needs one), 256 bytes for the gate logit
 * gate_inp . x (one token: reduced by the routing launch) and its output
 * sh [ntok][H] last, each at a 256-byte boundary.
 * Errors: as qg_moe_ffn, and as qg_mlp for the shared expert's shapes (all
 * checked before anything is enqueued). */
size_t qg_moe_shared_workspace_size(const qg_moe *m, const qg_shared_expert *sh, int topk, int ntok);
int qg_moe_ffn_shared(const qg_moe *m, const qg_shared_expert *sh, const float *router_logits, int topk,
                      const int32_t *expert_slots, const float *x, float *resid, int ntok, int32_t *ids_out,
                      float *w_out, int32_t *status, void *workspace, size_t workspace_bytes, void *stream);

/* A dense gated MLP that runs beside the routed experts on an input of its
 * own (a HOST struct; its pointers are device pointers): [gemma4]
 * encodeLayer's dense GELU MLP (ffn_gate, ffn_up, ffn_down) next to the
 * experts, on ffn_norm's output while the experts take pre_ffw_norm_2's. */
typedef struct qg_dense_mlp {
    int type;               /* qg_type of gate, up and down (not QG_F32)       */
    int64_t ff;             /* FD                                              */
    const void *gate;       /* FD x H blocks                                   */
    const void *up;         /* FD x H blocks                                   */
    const void *down;       /* H x FD blocks                                   */
} qg_dense_mlp;

/* The routed experts and the dense MLP beside them, per token t:
 *   y[t]     = the routed-expert FFN of x[t]            (as qg_moe_ffn)
 *   y_mlp[t] = W_down (act(W_gate x_mlp[t]) * (W_up x_mlp[t]))
 *                                                       (as qg_mlp, act = m->act)
 * One token, d->type == m->type and FD a multiple of F: two launches in all
 * instead of four, the MLP's gate / up rows riding in the experts' gated
 * launch as FD / F more row groups and its down rows in their one-token
 * down launch (values within the same bound as the separate calls; only the
 * order of a row's sums may differ).  Otherwise the two calls in turn.
 * y and y_mlp are separate outputs ([ntok][H] each; Gemma's FFN tail
 * normalises them apart); neither may overlap x, x_mlp or the other.
 * workspace: at least qg_moe_dense_workspace_size(m, d, topk, ntok) bytes,
 * 256-byte aligned: qg_moe_ffn's workspace (same layout), then the MLP's
 * (qg_mlp's layout: gu [ntok][2 FD], act [ntok][FD], ...) at
 * qg_moe_workspace_size(m, topk, ntok).
 * Errors: as qg_moe_ffn, and as qg_mlp for the MLP's shapes and pointers
 * (all checked before anything is enqueued). */
size_t qg_moe_dense_workspace_size(const qg_moe *m, const qg_dense_mlp *d, int topk, int ntok);
int qg_moe_ffn_dense(const qg_moe *m, const qg_dense_mlp *d, const float *router_logits, int topk,
                     const int32_t *expert_slots, const float *x, float *y, const float *x_mlp, float *y_mlp,
                     int ntok, int32_t *ids_out, float *w_out, int32_t *status, void *workspace,
                     size_t workspace_bytes, void *stream);

/* Gemma's FFN tail, per token of n values ([gemma4] encodeExperts: the
 * post_ffw_norm_1 / post_ffw_norm_2 rmsnorms, then WGSL postFfn):
 *   m = rmsnorm(mlp) * w1,  e = rmsnorm(moe) * w2,  v = m + e
 *   x = ((v * r_v) * w + x) * out_scale[0],   r_v = 1/sqrt(sum v^2 / n + eps)
 * mlp: the dense MLP's output, moe: the MoE sum, x: the residual stream
 * (updated in place), all [ntok][n]; w1, w2, w: [n]; out_scale: one f32 (the
 * layer's output scalar).  One launch, one workgroup per token.
 * Errors: QG_EINVAL (n <= 0, ntok < 1, eps < 0, null or misaligned pointer). */
int qg_post_ffn(const float *mlp, const float *moe, const float *w1, const float *w2, const float *w,
                const float *out_scale, float *x, int64_t n, int ntok, float eps, void *stream);

/* Embedding rows of a quantized table: out[t][c] = W[tokens[t]][c] * scale,
 * each value the f32 nearest its exact value (as qg_dequant), multiplied by
 * scale in f32 ([qwen3] WGSL embedQ8 with scale 1, [gemma4] embedQ6K with its
 * scale).  tokens: [ntok] int32 on the device; a token outside [0, rows) reads
 * nothing and gets a row of NaN.  out: [ntok][cols].  A table in a plane
 * layout (QG_Q8_0_PLANES, QG_Q6_K_PLANES; 16-byte aligned) gives the same
 * values, gathered one thread a value.
 * Errors: as qg_dequant; QG_ELIMIT for ntok outside 1..65535. */
int qg_embed(int type, const void *W, int64_t rows, int64_t cols, const int32_t *tokens, int ntok, float scale,
             float *out, void *stream);

/* Greedy pick over logits, per token: with softcap > 0 each logit is first
 * replaced in place by tanh(clamp(l * inv, -10, 10)) * softcap, inv the f32
 * nearest 1/softcap ([gemma4] WGSL softcap); then idx[t] = the index of the
 * largest value, ties to the lowest index, NaN never picked, 0 for a row with
 * no number ([qwen3] WGSL argmax).  Two launches: partial winners of spans of
 * the row, then the winner of those.
 * logits: [ntok][n] f32; idx: [ntok] int32.  workspace: at least
 * qg_argmax_workspace_size(n, ntok) bytes, 256-byte aligned.
 * Errors: QG_EINVAL (n <= 0, ntok < 1, softcap < 0 or NaN, null or misaligned
 * pointer, short workspace), QG_ELIMIT (n > 2^31 - 1, ntok > 65535). */
size_t qg_argmax_workspace_size(int64_t n, int ntok);
int qg_argmax(float *logits, int64_t n, int ntok, float softcap, int32_t *idx, void *workspace,
              size_t workspace_bytes, void *stream);

/* The decode loop's tail in two launches: qg_argmax, then the picked
 * tokens' rows of the (tied) embedding table as qg_embed gathers them,
 * out[t] = W[idx[t]] * scale ([qwen3] argmax then embedQ8, [gemma4] argmax
 * then embedQ6K).  The winner over the partial spans is taken inside the
 * gathering launch; idx and out equal what qg_argmax followed by qg_embed
 * give, bit for bit.  Arguments as those two calls (logits, idx, workspace
 * as qg_argmax; type, W, rows, cols, scale, out as qg_embed).
 * Errors: as qg_argmax and qg_embed (ntok up to 65535). */
int qg_argmax_embed(float *logits, int64_t n, int ntok, float softcap, int32_t *idx, void *workspace,
                    size_t workspace_bytes, int type, const void *W, int64_t rows, int64_t cols, float scale,
                    float *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* QGEMV_H */

// qg_planes.hip -- the plane layout of Q6_K ([gemma4] q6kPlanes: at load the
// 2-byte-aligned 210-byte blocks are split into aligned planes), its inverse,
// and the dequantization of a tensor held in it.
//
// Layout (QG_Q6_K_PLANES) of a tensor of n blocks, one buffer of 210 n bytes:
//   ql [n][128] at 0, qh [n][64] at 128 n, int8 scales [n][16] at 192 n,
//   f16 d [n] at 208 n
// in the blocks' row-major order.  The page widens d to f32; here it keeps
// its two bytes, so the planes are the blocks' bytes reordered.  Every
// copy moves 2 bytes, the blocks' own alignment.
#include "../../include/qgemv.h"
#include "qg_kq1.h"

namespace qg {

namespace {
constexpr int HW = 105;   // 2-byte words per block

// where byte j (even) of block b lands in the planes
__device__ __forceinline__ int64_t plane_pos(int64_t n, int64_t b, int j) {
    return j < 128 ? 128 * b + j
         : j < 192 ? 128 * n + 64 * b + (j - 128)
         : j < 208 ? 192 * n + 16 * b + (j - 192)
                   : 208 * n + 2 * b;
}

// one thread per 2-byte word of the blocks
__global__ __launch_bounds__(256) void k_q6k_planes(const uint16_t *src, uint8_t *dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n * HW) return;
    const int64_t b = i / HW;
    const int j = 2 * (int)(i - b * HW);
    *(uint16_t *)(dst + plane_pos(n, b, j)) = src[i];
}

__global__ __launch_bounds__(256) void k_q6k_unplanes(const uint8_t *src, uint16_t *dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n * HW) return;
    const int64_t b = i / HW;
    const int j = 2 * (int)(i - b * HW);
    dst[i] = *(const uint16_t *)(src + plane_pos(n, b, j));
}

// one thread per value: value t of block b ([bonsai] dequantQ6K's fields,
// read from their planes), (d * scale) * (q - 32) in f32 with one rounding
// (d * scale is exact: 11 by 8 significant bits)
__global__ __launch_bounds__(256) void k_q6k_planes_dequant(const uint8_t *P, float *out, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n * 256) return;
    const int64_t b = i >> 8;
    const int t = (int)(i & 255), half = t >> 7, r = t & 127, p = r >> 5, l = r & 31;
    const int lo = P[128 * b + 64 * half + l + 32 * (p & 1)];
    const int q4 = p >= 2 ? lo >> 4 : lo & 15;
    const int hb = (P[128 * n + 64 * b + 32 * half + l] >> (2 * p)) & 3;
    const int sc = (int8_t)P[192 * n + 16 * b + 8 * half + (l >> 4) + 2 * p];
    const float d = h2f(*(const uint16_t *)(P + 208 * n + 2 * b));
    out[i] = (d * (float)sc) * (float)((q4 | (hb << 4)) - 32);
}

bool ptr_ok(const void *p, uintptr_t a) { return p && ((uintptr_t)p & (a - 1)) == 0; }

// the blocks of a rows x cols Q6_K tensor, or -1
int64_t q6k_blocks(int type, int64_t rows, int64_t cols) {
    if (type != QG_Q6_K || rows <= 0 || cols <= 0 || cols % 256 || cols > (1 << 20)) return -1;
    const int64_t nb = cols / 256;
    if (rows > ((int64_t)1 << 40) / nb) return -1;
    return rows * nb;
}

bool overlap(const void *a, const void *b, int64_t bytes) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + (uintptr_t)bytes && y < x + (uintptr_t)bytes;
}

int planes_call(bool forward, int type, const void *src, void *dst, int64_t rows, int64_t cols, void *stream) {
    const int64_t n = q6k_blocks(type, rows, cols);
    if (n < 0) return QG_EINVAL;
    // the blocks side 2-byte aligned (GGUF), the planes side 16-byte aligned
    const void *blk = forward ? src : dst, *pl = forward ? dst : src;
    if (!ptr_ok(blk, 2) || !ptr_ok(pl, 16) || overlap(src, dst, 210 * n)) return QG_EINVAL;
    const int64_t wg = (n * HW + 255) / 256;
    if (wg > 0x7fffffff) return QG_ELIMIT;
    if (forward)
        hipLaunchKernelGGL(k_q6k_planes, dim3((unsigned)wg), dim3(256), 0, (hipStream_t)stream, (const uint16_t *)src,
                           (uint8_t *)dst, n);
    else
        hipLaunchKernelGGL(k_q6k_unplanes, dim3((unsigned)wg), dim3(256), 0, (hipStream_t)stream, (const uint8_t *)src,
                           (uint16_t *)dst, n);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_EHIP;
}
}  // namespace

int launch_q6k_planes_dequant(const uint8_t *P, float *out, int64_t nblk, hipStream_t st) {
    const int64_t wg = nblk;   // 256 values a workgroup
    if (wg > 0x7fffffff) return QG_ELIMIT;
    hipLaunchKernelGGL(k_q6k_planes_dequant, dim3((unsigned)wg), dim3(256), 0, st, P, out, nblk);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_EHIP;
}

}  // namespace qg

extern "C" {

int qg_prepare(int type, const void *src, void *dst, int64_t rows, int64_t cols, void *stream) {
    return qg::planes_call(true, type, src, dst, rows, cols, stream);
}

int qg_unprepare(int type, const void *src, void *dst, int64_t rows, int64_t cols, void *stream) {
    return qg::planes_call(false, type, src, dst, rows, cols, stream);
}

}  // extern "C"

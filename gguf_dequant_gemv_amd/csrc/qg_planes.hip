// qg_planes.hip -- the plane layouts: Q6_K ([gemma4] q6kPlanes: at load the
// 2-byte-aligned 210-byte blocks are split into aligned planes) and Q8_0
// (a code plane and a scale plane, as [qwen3] i8at reads them), their
// inverses, the dequantization of a tensor held in them, and the launch of
// the one-token Q8_0 plane GEMV (k_q8p1 in qg_planes.h).
//
// Layout QG_Q6_K_PLANES of a tensor of n blocks, one buffer of 210 n bytes:
//   ql [n][128] at 0, qh [n][64] at 128 n, int8 scales [n][16] at 192 n,
//   f16 d [n] at 208 n
// Layout QG_Q8_0_PLANES, 34 n bytes: codes [n][32] at 0, f16 d [n] at 32 n.
// Both in the blocks' row-major order.  The Q6_K page widens d to f32; here
// it keeps its two bytes, so the planes are the blocks' bytes reordered.
// Every copy moves 2 bytes, the blocks' own alignment.
#include <mutex>

#include "../../include/qgemv.h"
#include "qg_planes.h"

namespace qg {

namespace {
// 2-byte words per block: Q6_K 105, Q8_0 17
template <int TY> struct PlaneMap;
template <> struct PlaneMap<T_Q6_K> {
    static constexpr int HW = 105;
    // where byte j (even) of block b lands in the planes
    __device__ static int64_t pos(int64_t n, int64_t b, int j) {
        return j < 128 ? 128 * b + j
             : j < 192 ? 128 * n + 64 * b + (j - 128)
             : j < 208 ? 192 * n + 16 * b + (j - 192)
                       : 208 * n + 2 * b;
    }
};
template <> struct PlaneMap<T_Q8_0> {
    static constexpr int HW = 17;
    __device__ static int64_t pos(int64_t n, int64_t b, int j) { return j < 2 ? 32 * n + 2 * b : 32 * b + (j - 2); }
};

// one thread per 2-byte word of the blocks
template <int TY>
__global__ __launch_bounds__(256) void k_planes(const uint16_t *src, uint8_t *dst, int64_t n) {
    constexpr int HW = PlaneMap<TY>::HW;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n * HW) return;
    const int64_t b = i / HW;
    const int j = 2 * (int)(i - b * HW);
    *(uint16_t *)(dst + PlaneMap<TY>::pos(n, b, j)) = src[i];
}

template <int TY>
__global__ __launch_bounds__(256) void k_unplanes(const uint8_t *src, uint16_t *dst, int64_t n) {
    constexpr int HW = PlaneMap<TY>::HW;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n * HW) return;
    const int64_t b = i / HW;
    const int j = 2 * (int)(i - b * HW);
    dst[i] = *(const uint16_t *)(src + PlaneMap<TY>::pos(n, b, j));
}

// one thread per value: d * code, exact
__global__ __launch_bounds__(256) void k_q8_planes_dequant(const uint8_t *P, float *out, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n * 32) return;
    out[i] = h2f(*(const uint16_t *)(P + 32 * n + 2 * (i >> 5))) * (float)(int8_t)P[i];
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

// the blocks of a rows x cols Q6_K / Q8_0 tensor, or -1
int64_t plane_blocks(int type, int64_t rows, int64_t cols) {
    const int qk = type == QG_Q6_K ? 256 : type == QG_Q8_0 ? 32 : 0;
    if (!qk || rows <= 0 || cols <= 0 || cols % qk || cols > (1 << 20)) return -1;
    const int64_t nb = cols / qk;
    if (rows > ((int64_t)1 << 40) / nb) return -1;
    return rows * nb;
}

bool overlap(const void *a, const void *b, int64_t bytes) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + (uintptr_t)bytes && y < x + (uintptr_t)bytes;
}

int planes_call(bool forward, int type, const void *src, void *dst, int64_t rows, int64_t cols, void *stream) {
    const int64_t n = plane_blocks(type, rows, cols);
    if (n < 0) return QG_EINVAL;
    const bool q6 = type == QG_Q6_K;
    const int64_t bb = q6 ? 210 : 34, hw = bb / 2;
    // the blocks side 2-byte aligned (GGUF), the planes side 16-byte aligned
    const void *blk = forward ? src : dst, *pl = forward ? dst : src;
    if (!ptr_ok(blk, 2) || !ptr_ok(pl, 16) || overlap(src, dst, bb * n)) return QG_EINVAL;
    const int64_t wg = (n * hw + 255) / 256;
    if (wg > 0x7fffffff) return QG_ELIMIT;
    const hipStream_t st = (hipStream_t)stream;
    if (forward) {
        if (q6) hipLaunchKernelGGL(k_planes<T_Q6_K>, dim3((unsigned)wg), dim3(256), 0, st, (const uint16_t *)src, (uint8_t *)dst, n);
        else hipLaunchKernelGGL(k_planes<T_Q8_0>, dim3((unsigned)wg), dim3(256), 0, st, (const uint16_t *)src, (uint8_t *)dst, n);
    } else {
        if (q6) hipLaunchKernelGGL(k_unplanes<T_Q6_K>, dim3((unsigned)wg), dim3(256), 0, st, (const uint8_t *)src, (uint16_t *)dst, n);
        else hipLaunchKernelGGL(k_unplanes<T_Q8_0>, dim3((unsigned)wg), dim3(256), 0, st, (const uint8_t *)src, (uint16_t *)dst, n);
    }
    return hipGetLastError() == hipSuccess ? QG_OK : QG_EHIP;
}
}  // namespace

int launch_q8_planes_dequant(const uint8_t *P, float *out, int64_t nblk, hipStream_t st) {
    const int64_t wg = (nblk * 32 + 255) / 256;
    if (wg > 0x7fffffff) return QG_ELIMIT;
    hipLaunchKernelGGL(k_q8_planes_dequant, dim3((unsigned)wg), dim3(256), 0, st, P, out, nblk);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_EHIP;
}

namespace {
typedef void (*q8p_fn)(Q8pArgs);


// x's float4 per thread: 4 up to 1024 NW values, 12 up to 3072 NW
template <int NW>
q8p_fn q8p_plain(int cols) {
    return cols <= 4 * 4 * 64 * NW ? k_q8p1<NW, Q8P_NF, 4, false> : k_q8p1<NW, Q8P_NF, 12, false>;
}
q8p_fn q8p_kernel(int cols, bool gated, int nw) {
    if (gated)
        return cols <= 4 * 4 * 64 * Q8P_NW ? k_q8p1<Q8P_NW, Q8P_NF, 4, true> : k_q8p1<Q8P_NW, Q8P_NF, 12, true>;
    switch (nw) {
    case 4: return q8p_plain<4>(cols);
    case 10: return q8p_plain<10>(cols);
    case 12: return q8p_plain<12>(cols);
    case 14: return q8p_plain<14>(cols);
    case 16: return q8p_plain<16>(cols);
    default: return q8p_plain<8>(cols);
    }
}

// workgroups resident at once on all CUs (measured when a device is there to
// ask, else 8 a CU)
int q8p_resident(q8p_fn f, int nw, size_t lds, bool query) {
    if (!query) return 8 * 256;
    static std::mutex mu;
    static q8p_fn cf[8];
    static size_t cl[8];
    static int cn[8], used = 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; i++)
        if (cf[i] == f && cl[i] == lds) return cn[i];
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)f, 64 * nw, lds) != hipSuccess)
        return -1;
    if (per_cu < 1) per_cu = 1;
    if (used < 8) { cf[used] = f; cl[used] = lds; cn[used] = per_cu * 256; used++; }
    return per_cu * 256;
}
}  // namespace

// One token against a Q8_0 tensor in the plane layout: nw waves a workgroup
// (q8p_waves), every workgroup that fits at once (each wave walks rows w,
// w + W, ...), at most one per nw rows.
int q8p_plan(int64_t rows, int64_t cols, bool gated, bool query, int *wgs, size_t *lds, int *nw) {
    if (rows < 1 || cols < 32 || cols % 32 || cols > Q8P_MAX_COLS) return QG_EINVAL;
    if (rows * cols >= ((int64_t)1 << 31)) return QG_ELIMIT;
    const size_t l = q8p_lds_bytes((int)cols);
    const int w = q8p_waves(rows, gated);
    const int cap = q8p_resident(q8p_kernel((int)cols, gated, w), w, l, query);
    if (cap < 0) return QG_EHIP;
    const int64_t need = (rows + w - 1) / w;
    *wgs = (int)(need < cap ? need : cap);
    *lds = l;
    *nw = w;
    return QG_OK;
}

int launch_q8p1(const Q8pArgs &a, bool gated, hipStream_t st) {
    int g = 0, w = 0;
    size_t l = 0;
    const int rc = q8p_plan(a.rows, a.cols, gated, true, &g, &l, &w);
    if (rc) return rc;
    hipLaunchKernelGGL(q8p_kernel(a.cols, gated, w), dim3((unsigned)g), dim3(64 * w), l, st, a);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_EHIP;
}

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

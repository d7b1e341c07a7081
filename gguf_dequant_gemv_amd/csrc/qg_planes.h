// qg_planes.h -- kernels over the plane layouts (qg_planes.hip): one token
// against Q8_0 rows held as a code plane and a scale plane.
//
// Layout (QG_Q8_0_PLANES) of rows x cols values: the int8 codes [rows][cols]
// at byte 0, then the f16 scales [rows][cols / 32] ([qwen3] WGSL i8at's code
// plane and scales by group).  A row of codes is cols contiguous bytes, so
// where cols is a multiple of 128 every row is whole 128-byte lines.
//
// k_q8p1: a wave walks its rows (row w, w + W, ... for wave w of W) as a
// stream of 16-byte code pieces: lane j takes pieces j, j + 64, ... of each
// row, so each load instruction reads 1 KB of one row and consumes every
// line it touches (the loads carry the non-temporal hint, measured worth
// ~10% on whole-line streams).  NF pieces are in flight per lane; x is
// staged once per workgroup in LDS; a row's 64 lane sums meet in a DPP
// reduction and lane 0 stores y.  The gated form (a gated MLP's gate and up
// projections) walks row r of the gate tensor, then row r of the up tensor,
// and stores act(g) * u, with g and u themselves in y2.
#pragma once
#include "qg_kernels.h"
#include "qg_kq1.h"

namespace qg {

struct Q8pArgs {
    const uint8_t *C;   // codes [rows][cols] int8, 16-byte aligned
    const uint8_t *D;   // scales [rows][cols / 32] f16, 2-byte aligned
    int64_t rows;
    int cols;           // a multiple of 32; rows * cols < 2^31
    const float *x;     // [cols], 16-byte aligned
    float *y;           // [rows]
    // gated form only: the up tensor's planes, g and u ([2][rows]: g at
    // y2[r], u at y2[rows + r]), the activation (XM_SILU / XM_GELU)
    const uint8_t *C2, *D2;
    float *y2;
    int glu;
};

// x in LDS: 4 floats of padding after every 32 values, so the 16-byte reads
// of 8 neighbouring lanes (64-byte pieces 64 bytes apart) land on distinct
// banks
QG_DEV int q8p_xpos(int v) { return v + 4 * (v >> 5); }
constexpr int Q8P_MAX_COLS = 12288;   // x within the LDS of the largest instance (55 KB)
// waves per workgroup and pieces in flight per lane (measured best of NW 4 /
// 8 / 16 and NF 1..8 on the 151936 x 2560 head)
constexpr int Q8P_NW = 8, Q8P_NF = 2;
// Waves per workgroup of the plain (not gated) launch: up to 4096 rows, the
// fewest of 4, 8, 10, 12, 14, 16 that put every row on its own wave within
// 256 workgroups (one a CU: a CU holding two workgroups of a launch ends its
// waves last, measured 8.6 against 6.3 us on 2560 rows); beyond that Q8P_NW,
// every wave walking several rows.
__host__ __device__ inline int q8p_waves(int64_t rows, bool gated) {
    if (gated || rows > 16 * 256) return Q8P_NW;
    const int per = (int)((rows + 255) / 256);
    return per <= 4 ? 4 : per <= 8 ? 8 : per <= 10 ? 10 : per <= 12 ? 12 : per <= 14 ? 14 : 16;
}
__host__ __device__ inline size_t q8p_lds_bytes(int cols) { return (size_t)(cols + cols / 8) * 4; }

template <int NW, int NF, int XN, bool GATED>
__global__ __launch_bounds__(64 * NW) void k_q8p1(Q8pArgs a) {
    extern __shared__ float lds[];
    constexpr int NT = 64 * NW;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t w0 = (int64_t)blockIdx.x * NW + wave, W = (int64_t)gridDim.x * NW;
    const int cols = a.cols, nb = cols / 32, P = cols / 16, S = (P + 63) / 64;
    const int SR = GATED ? 2 * S : S;   // slots a row: the gate's, then the up's
    const u32 crange = (u32)(a.rows * cols), drange = (u32)(a.rows * nb * 2);
    const rsrc_t rc = make_rsrc(a.C, crange), rd = make_rsrc(a.D, drange);
    const rsrc_t rc2 = GATED ? make_rsrc(a.C2, crange) : rc, rd2 = GATED ? make_rsrc(a.D2, drange) : rd;
    const int64_t nrows = w0 < a.rows ? (a.rows - w0 + W - 1) / W : 0;
    const int64_t Q = nrows * (int64_t)SR;   // pieces this wave computes

    // x's loads, then the first NF pieces' loads (x's wait then excludes the
    // weights'), then x into LDS
    f32x4 xv[XN];
    kq1_x_load<NT, XN>(a.x, cols, xv);
    kq1_fence();
    // the issue pointer: row irow, slot isl; pieces past the wave's last row
    // load at offsets out of every range (nothing read, zeros returned)
    int64_t irow = w0;
    int isl = 0;
    auto issue = [&](u32 (&t)[5]) {
        const u32 kill = irow < a.rows ? 0u : 0x80000000u;
        const u32 rr = (u32)(irow < a.rows ? irow : a.rows - 1);
        const bool up = GATED && isl >= S;
        const int pc = min(lane + 64 * (up ? isl - S : isl), P - 1);
        const u32x4 v =
            __builtin_amdgcn_raw_buffer_load_b128(up ? rc2 : rc, rr * (u32)cols + 16u * (u32)pc + kill, 0, 2);
        t[0] = v.x; t[1] = v.y; t[2] = v.z; t[3] = v.w;
        t[4] = __builtin_amdgcn_raw_buffer_load_b16(up ? rd2 : rd, 2u * (rr * (u32)nb + (u32)(pc >> 1)) + kill, 0, 0);
        if (++isl == SR) { isl = 0; irow += W; }
    };
    u32 t[NF][5];
#pragma unroll
    for (int f = 0; f < NF; f++) issue(t[f]);
    {
        const int n4 = cols >> 2;
#pragma unroll
        for (int b = 0; b < XN; b++) {
            const int i = tid + b * NT;
            if (i < n4) *(f32x4 *)(lds + q8p_xpos(4 * i)) = xv[b];
        }
    }
    __syncthreads();

    // the compute pointer: row crow, slot csl
    int64_t crow = w0;
    int csl = 0;
    float acc = 0.0f, gsum = 0.0f;
    auto step = [&](const u32 (&tc)[5]) {
        const int piece = lane + 64 * (GATED && csl >= S ? csl - S : csl);
        const int pc = min(piece, P - 1);
        const float *xp = lds + q8p_xpos(16 * pc);
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; w++) {
            const f32x4 xw = *(const f32x4 *)(xp + 4 * w);
            s = fmaf((float)(int8_t)(tc[w]), xw.x, s);
            s = fmaf((float)(int8_t)(tc[w] >> 8), xw.y, s);
            s = fmaf((float)(int8_t)(tc[w] >> 16), xw.z, s);
            s = fmaf((float)(int8_t)(tc[w] >> 24), xw.w, s);
        }
        acc += piece < P ? h2f(tc[4]) * s : 0.0f;
        ++csl;
        if (GATED && csl == S) {   // the gate row's sum
            gsum = group_sum<64>(acc);
            acc = 0.0f;
        }
        if (csl == SR) {
            const float tot = group_sum<64>(acc);
            if (lane == 0) {
                if constexpr (GATED) {
                    a.y2[crow] = gsum;
                    a.y2[a.rows + crow] = tot;
                    a.y[crow] = glu(a.glu, gsum, tot);
                } else {
                    a.y[crow] = tot;
                }
            }
            acc = 0.0f;
            csl = 0;
            crow += W;
        }
    };
#pragma unroll 1
    for (int64_t q0 = 0; q0 < Q; q0 += NF) {
#pragma unroll
        for (int f = 0; f < NF; f++) {
            if (q0 + f < Q) {
                kq1_fence();
                step(t[f]);
                issue(t[f]);
            }
        }
    }
}

int q8p_plan(int64_t rows, int64_t cols, bool gated, bool query, int *wgs, size_t *lds, int *nw);
int launch_q8p1(const Q8pArgs &a, bool gated, hipStream_t st);
// f32 values of nblk Q6_K / Q8_0 blocks held in their plane layouts
int launch_q6k_planes_dequant(const uint8_t *P, float *out, int64_t nblk, hipStream_t st);
int launch_q8_planes_dequant(const uint8_t *P, float *out, int64_t nblk, hipStream_t st);

}  // namespace qg

// qg_gemm.hip -- prefill-size chunks (tens to thousands of tokens) of Q8_0 /
// Q4_0 products on the matrix cores (gfx950 v_mfma_f32_16x16x32_bf16).
//
// y[t][r] = sum_c W[r][c] x[t][c] with every product exact, as in the small
// batch kernel: codes are small integers (exact in bf16) and x enters as three
// bf16 parts whose sum is x exactly, so only the f32 accumulation order
// differs from an f32 FMA chain.  What changes at prefill size is reuse: a
// workgroup owns 64 tokens (TG = 4 groups of 16) and 8 waves x RG groups of
// 16 rows, and every weight block it loads feeds 3 * TG MFMAs per row group.
// Every x chunk it loads feeds all 256 rows (x, in three parts, is as many
// bytes per chunk as the rows' weights).
//
// x is split into its three bf16 parts once per launch (k_split_x), laid out
// k-chunk by k-chunk: one 64-token tile's KC values of one chunk are a single
// contiguous block of 3 x 64 x KC bf16.  The GEMM then copies, per k-chunk,
// that block and the tile's weight row segments HBM -> LDS with 16-byte
// buffer-to-LDS loads two chunks ahead of use, so its loop holds no x
// arithmetic, no LDS stores and one barrier per chunk.  The pages' prompt-chunk
// GEMMs ([qwen35] / [gemma4] WGSL matmulQ8T / matmulQ4T) tile 16 rows x 16
// tokens through workgroup memory in f32; this keeps their "each weight byte
// serves many tokens" and moves the contraction to the matrix cores.
#include "../../include/qgemv.h"
#include "qg_kernels.h"
#include "qg_block.h"

namespace qg {

constexpr int GEMM_KC = 64;                     // x values per k-chunk (2 blocks)
constexpr int GEMM_TG = 4;                      // token groups of 16 per workgroup
constexpr int GEMM_TT = 16 * GEMM_TG;
constexpr int GEMM_WAVES = 8;                   // waves per workgroup (two per SIMD)
constexpr int GEMM_THREADS = 64 * GEMM_WAVES;
constexpr int NUM_XCD = 8;                      // accelerator dies, each with its own L2
constexpr int GEMM_XROW = GEMM_KC * 2;          // bytes of one (part, token) row of a chunk
constexpr int GEMM_XBLK = 3 * GEMM_TT * GEMM_XROW;   // bytes of one (token tile, chunk) block

// Position of 16-byte piece p (8 values) of token row t inside its row.  The
// MFMA operand reads take one piece from each of 16 consecutive token rows
// (128 bytes apart); permuting the pieces by t spreads those reads over all
// banks whether the LDS serves 8 lanes from 32 banks or 16 lanes from 64.
QG_DEV int xs_pos(int p, int t) { return p ^ (t & 7) ^ ((t >> 3) & 1); }

// four values x = h + m + l exactly, each part a bf16 (truncation splits),
// packed two to a dword, element 2j in the low half
QG_DEV void split3x4(const f32x4 &x, u32 (&h)[2], u32 (&m)[2], u32 (&l)[2]) {
    const float v[4] = {x.x, x.y, x.z, x.w};
    u32 hb[4], mb[4], lb[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        hb[j] = __builtin_bit_cast(u32, v[j]) & 0xFFFF0000u;
        const float r = v[j] - __builtin_bit_cast(float, hb[j]);
        mb[j] = __builtin_bit_cast(u32, r) & 0xFFFF0000u;
        lb[j] = __builtin_bit_cast(u32, r - __builtin_bit_cast(float, mb[j]));
    }
#pragma unroll
    for (int j = 0; j < 2; j++) {
        h[j] = __builtin_amdgcn_perm(hb[2 * j + 1], hb[2 * j], 0x07060302u);
        m[j] = __builtin_amdgcn_perm(mb[2 * j + 1], mb[2 * j], 0x07060302u);
        l[j] = __builtin_amdgcn_perm(lb[2 * j + 1], lb[2 * j], 0x07060302u);
    }
}

// x [ntok][x_stride] f32 -> xs [token tile][chunk][part][64 tokens][KC values]
// bf16 (pieces permuted by xs_pos).  One thread per 8 values; tokens past
// ntok and values past cols are zeros.
__global__ __launch_bounds__(256) void k_split_x(const float *x, int64_t x_stride, int ntok, int cols, int nch,
                                                 int64_t total, uint8_t *xs) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int p = (int)(i & 7), t = (int)((i >> 3) & (GEMM_TT - 1));
    const int64_t rest = i >> 9;                       // token tile * nch + chunk
    const int c = (int)(rest % nch);
    const int tok = (int)(rest / nch) * GEMM_TT + t;
    const int k0 = c * GEMM_KC + 8 * p;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; j++)
        v[j] = tok < ntok && k0 + j < cols ? x[(int64_t)tok * x_stride + k0 + j] : 0.0f;
    u32 h0[2], m0[2], l0[2], h1[2], m1[2], l1[2];
    split3x4(f32x4{v[0], v[1], v[2], v[3]}, h0, m0, l0);
    split3x4(f32x4{v[4], v[5], v[6], v[7]}, h1, m1, l1);
    uint8_t *d = xs + rest * GEMM_XBLK + (int64_t)t * GEMM_XROW + 16 * xs_pos(p, t);
    *(u32x4 *)d = u32x4{h0[0], h0[1], h1[0], h1[1]};
    *(u32x4 *)(d + GEMM_TT * GEMM_XROW) = u32x4{m0[0], m0[1], m1[0], m1[1]};
    *(u32x4 *)(d + 2 * GEMM_TT * GEMM_XROW) = u32x4{l0[0], l0[1], l1[0], l1[1]};
}

template <int TY>
struct GemmGeom {
    static constexpr int BYTES = TY == T_Q8_0 ? 34 : 18;
    static constexpr int RG = 2;                                  // row groups per wave
    static constexpr int NS = GEMM_WAVES * RG * 16;               // row slots per tile
    static constexpr int SEGP = (15 + (GEMM_KC / 32) * BYTES + 15) / 16;   // pieces per slot
    static constexpr int PIECES = NS * SEGP;
    static constexpr int NI = PIECES / GEMM_THREADS;              // weight loads per thread per chunk
    static constexpr int XI = GEMM_XBLK / 16 / GEMM_THREADS;      // x loads per thread per chunk
    static constexpr int AHEAD = 2;                               // chunks requested ahead of use
    static constexpr int RING = AHEAD + 1;
    static constexpr int SLOT = PIECES * 16;                      // weight bytes per ring slot
    static_assert(PIECES % GEMM_THREADS == 0 && XI * GEMM_THREADS * 16 == GEMM_XBLK, "whole loads per thread");
    static_assert((NS / 2) * SEGP % 64 == 0, "a load instruction reads one matrix");
};

// Workgroup tile: 8 waves x RG groups of 16 rows (gated: RG/2 gate groups and
// the same up groups per wave) x 64 tokens; a 1-D launch of wg_x row-tile
// slots (grid-stride over the row tiles) x wg_y 64-token tiles x wg_z splits
// of the row.  Lane l: row / token l%16,
// k-group l/16 of each 32-value block; D[4(l/16)+i][l%16] = token 4(l/16)+i,
// row l%16.
//
// Per k-chunk, the tile's row segments (each from the 16-byte-aligned start
// below it, one more piece than it needs; row slots numbered gate rows first,
// so every load instruction reads one matrix) and the chunk's split-x block go
// HBM -> LDS into ring slot (chunk mod RING), AHEAD chunks before use.  Every
// chunk issues the same loads (chunks past the split's end clamped to its last
// one, results unused), so a fixed wait count retires exactly one chunk's.
template <int TY>
__global__ __launch_bounds__(GEMM_THREADS) void k_gemm_mfma(GemvArgs a) {
    typedef GemmGeom<TY> G;
    constexpr int BYTES = G::BYTES, RG = G::RG, SEGP = G::SEGP;
    constexpr int BPC = GEMM_KC / 32;           // blocks per k-chunk
    __shared__ __attribute__((aligned(16))) uint8_t s_x[G::RING * GEMM_XBLK];
    __shared__ __attribute__((aligned(16))) uint8_t s_w[G::RING * G::SLOT];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int n16 = lane & 15, q = lane >> 4;
    const int nb = a.cols / 32;
    // Workgroups go to the XCDs round-robin by launch index; renumbered so
    // that each XCD runs one contiguous range of (split, row tile, token
    // tile), the row tiles of a split (which read the same x chunks) and the
    // token tiles of a row tile (the same weights) share that XCD's L2.
    const int nwg = a.wg_x * a.wg_y * a.wg_z;
    const int xcd = (int)blockIdx.x % NUM_XCD, per = nwg / NUM_XCD;
    const int lid = xcd * per + min(xcd, nwg % NUM_XCD) + (int)blockIdx.x / NUM_XCD;
    const int gy = lid % a.wg_y, gx = (lid / a.wg_y) % a.wg_x, gz = lid / (a.wg_y * a.wg_x);
    // this workgroup's k-chunks [c_lo, nch): the whole row, or one split of it
    const int nch_all = (nb + BPC - 1) / BPC;
    const int c_lo = a.part ? gz * a.kchunks : 0;
    const int nch = a.part ? min(nch_all, c_lo + a.kchunks) : nch_all;
    const int64_t rows = a.rows;
    const u32 rb = (u32)a.row_bytes;
    const int t0 = gy * GEMM_TT;
    const int nt = min(GEMM_TT, a.ntok - t0);
    const int gpw = a.glu ? RG / 2 : RG;        // distinct row groups per wave
    const int tile_rows = GEMM_WAVES * 16 * gpw;

    const u32 ph0 = (u32)((uintptr_t)a.W0 & 15u), ph1 = (u32)((uintptr_t)a.W1 & 15u);
    const rsrc_t rs0 = make_rsrc(a.W0 - ph0, (u32)((ph0 + a.bytes0 + 15) & ~(int64_t)15));
    const rsrc_t rs1 = make_rsrc(a.W1 - ph1, (u32)((ph1 + a.bytes1 + 15) & ~(int64_t)15));
    // this token tile's split-x blocks, chunk after chunk
    const rsrc_t rsx = make_rsrc(a.xs + (int64_t)gy * nch_all * GEMM_XBLK, (u32)(nch_all * GEMM_XBLK));
    const u32 cpos = 2u + 8u * (u32)(TY == T_Q8_0 ? q : (q & 1));
    const u32 sx0 = lds_off(s_x), sw0 = lds_off(s_w);
    // this lane's x piece offset within a (part, token group) row block, per block of the chunk
    u32 xoff[BPC];
#pragma unroll
    for (int bl = 0; bl < BPC; bl++) xoff[bl] = (u32)n16 * GEMM_XROW + 16u * (u32)xs_pos(4 * bl + q, n16);

    // row slot -> (matrix, row): gated launches number their gate rows first
    auto slot_row = [&](int64_t tile, int slot, bool &hi) {
        const int half = G::NS / 2;
        hi = a.glu && slot >= half;
        const int sl = a.glu ? slot % half : slot;       // wave * gpw * 16 + g * 16 + n
        return min(tile * tile_rows + sl, rows - 1);
    };
    auto dma = [&](int64_t tile, int chunk) {
        const int cc = min(chunk, nch - 1);
        const int slot = (chunk - c_lo) % G::RING;
        uint8_t *dst = s_w + slot * G::SLOT;
        const u32 cbyte = (u32)cc * (u32)(BPC * BYTES);
#pragma unroll
        for (int i = 0; i < G::NI; i++) {
            // pieces [i*THREADS + 64*wave, +64) lie in one matrix
            const bool hiw = __builtin_amdgcn_readfirstlane(
                                 (int)(a.glu && (i * GEMM_THREADS + 64 * wave) >= (G::NS / 2) * SEGP)) != 0;
            // this thread's piece: a row slot and a piece of its segment
            const int p = i * GEMM_THREADS + tid;
            bool hi;
            const int64_t r = slot_row(tile, p / SEGP, hi);
            const u32 off = (((u32)r * rb + cbyte + (hiw ? ph1 : ph0)) & ~15u) + 16u * (u32)(p % SEGP);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(hiw ? rs1 : rs0,
                                                     (__attribute__((address_space(3))) void *)(
                                                         (__attribute__((address_space(3))) uint8_t *)dst +
                                                         (i * GEMM_THREADS + 64 * wave) * 16),
                                                     16, off, 0, 0, 0);
        }
        uint8_t *xdst = s_x + slot * GEMM_XBLK;
        const u32 xbyte = (u32)cc * (u32)GEMM_XBLK;
#pragma unroll
        for (int i = 0; i < G::XI; i++)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsx,
                                                     (__attribute__((address_space(3))) void *)(
                                                         (__attribute__((address_space(3))) uint8_t *)xdst +
                                                         (i * GEMM_THREADS + 64 * wave) * 16),
                                                     16, xbyte + 16u * (u32)(i * GEMM_THREADS + tid), 0, 0, 0);
    };

    for (int64_t tile = gx; tile < a.ntiles; tile += a.wg_x) {
        // this lane's row slots and rows, one per row group
        int myslot[RG];
        u32 rstart[RG];
#pragma unroll
        for (int gi = 0; gi < RG; gi++) {
            const bool hi = a.glu && gi >= RG / 2;
            const int g = a.glu ? gi % (RG / 2) : gi;
            const int sl = (wave * gpw + g) * 16 + n16;
            myslot[gi] = (hi ? G::NS / 2 : 0) + sl;
            bool h2;
            const int64_t r = slot_row(tile, myslot[gi], h2);
            rstart[gi] = (u32)r * rb + (hi ? ph1 : ph0);
        }
        float acc[RG][GEMM_TG][4];
#pragma unroll
        for (int gi = 0; gi < RG; gi++)
#pragma unroll
            for (int tg = 0; tg < GEMM_TG; tg++)
#pragma unroll
                for (int i = 0; i < 4; i++) acc[gi][tg][i] = 0.0f;

        // a chunk's operands (every block's code words, scales and x parts)
        // are read from LDS before any of its MFMAs, so the reads of later
        // blocks overlap the arithmetic of earlier ones
        auto consume = [&](int chunk) {
            const u32 sw = sw0 + (u32)((chunk - c_lo) % G::RING) * G::SLOT;
            const u32 sx = sx0 + (u32)((chunk - c_lo) % G::RING) * GEMM_XBLK;
            const u32 cbyte = (u32)chunk * (u32)(BPC * BYTES);
            const int nbl = min(BPC, nb - chunk * BPC);
            u32 w[BPC][RG][4];
            u32 sh[BPC][RG], so[BPC][RG];
            u32x4 xq[BPC][3][GEMM_TG];
#pragma unroll
            for (int bl = 0; bl < BPC; bl++) {
                const int blc = bl < nbl ? bl : 0;   // past the row's end: any valid block
#pragma unroll
                for (int gi = 0; gi < RG; gi++) {
                    // the block's bytes sit at the segment's phase past the slot's start
                    const u32 phase = (rstart[gi] + cbyte) & 15u;
                    const u32 base = (u32)myslot[gi] * (SEGP * 16) + phase + (u32)blc * BYTES;
                    const u32 co = base + cpos;
                    const u32 cw = sw + (co & ~3u);
                    w[bl][gi][0] = lds_ld32(cw);
                    w[bl][gi][1] = lds_ld32(cw + 4);
                    w[bl][gi][2] = lds_ld32(cw + 8);
                    w[bl][gi][3] = lds_ld32(sw + (base & ~3u));
                    sh[bl][gi] = co & 3u;
                    so[bl][gi] = base & 3u;
                }
#pragma unroll
                for (int tg = 0; tg < GEMM_TG; tg++) {
                    const u32 off = sx + (u32)(16 * tg) * GEMM_XROW + xoff[blc];
#pragma unroll
                    for (int pt = 0; pt < 3; pt++) xq[bl][pt][tg] = lds_ld128(off + pt * GEMM_TT * GEMM_XROW);
                }
            }
            lds_wait();
#pragma unroll
            for (int bl = 0; bl < BPC; bl++) {
#pragma unroll
                for (int gi = 0; gi < RG; gi++)
#pragma unroll
                    for (int k = 0; k < 4; k++) lds_ready(w[bl][gi][k]);
#pragma unroll
                for (int pt = 0; pt < 3; pt++)
#pragma unroll
                    for (int tg = 0; tg < GEMM_TG; tg++) lds_ready(xq[bl][pt][tg]);
            }
#pragma unroll
            for (int bl = 0; bl < BPC; bl++) {
                if (bl >= nbl) break;
                bf16x8 wv[RG];
                float d[RG];
#pragma unroll
                for (int gi = 0; gi < RG; gi++) {
                    const u32 cw0 = __builtin_amdgcn_alignbyte(w[bl][gi][1], w[bl][gi][0], sh[bl][gi]);
                    const u32 cw1 = __builtin_amdgcn_alignbyte(w[bl][gi][2], w[bl][gi][1], sh[bl][gi]);
                    u32 cb[4];
                    codes_bf16<TY>(cw0, cw1, q, cb);
                    wv[gi] = as_bf16x8(cb);
                    d[gi] = h2f(w[bl][gi][3] >> (8 * so[bl][gi]));
                }
                // the MFMAs part by part across all (row group, token group)
                // pairs, so each dependent chain of three has others between
                // its links
                f32x4 cc[RG][GEMM_TG];
#pragma unroll
                for (int gi = 0; gi < RG; gi++)
#pragma unroll
                    for (int tg = 0; tg < GEMM_TG; tg++) cc[gi][tg] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int pt = 0; pt < 3; pt++)
#pragma unroll
                    for (int gi = 0; gi < RG; gi++)
#pragma unroll
                        for (int tg = 0; tg < GEMM_TG; tg++)
                            cc[gi][tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8, xq[bl][pt][tg]), wv[gi], cc[gi][tg], 0, 0, 0);
#pragma unroll
                for (int gi = 0; gi < RG; gi++)
#pragma unroll
                    for (int tg = 0; tg < GEMM_TG; tg++)
#pragma unroll
                        for (int i = 0; i < 4; i++) acc[gi][tg][i] = fmaf(d[gi], cc[gi][tg][i], acc[gi][tg][i]);
            }
        };

        // chunk c: its copies waited for (this wave's: issued later than
        // them are at most AHEAD - 1 chunks' loads), then the barrier (every
        // wave's pieces are in, and every wave is done with chunk c - 1, whose
        // ring slot chunk c + AHEAD takes), then that request, then c's blocks
#pragma unroll
        for (int j = 0; j < G::AHEAD; j++) dma(tile, c_lo + j);
        for (int c = c_lo; c < nch; c++) {
            QG_WAIT_VM((G::AHEAD - 1) * (G::NI + G::XI));
            lds_barrier();
            dma(tile, c + G::AHEAD);
            consume(c);
        }
        QG_WAIT_VM(0);     // the chunks past the end were requested too

        // lane holds tokens 16 tg + 4q + i of row n16 of each group (the
        // token base is re-derived per tile: kept live across the whole
        // kernel, its store addresses would not fit the registers)
        int q4 = 4 * q;
        asm volatile("" : "+v"(q4));
#pragma unroll
        for (int tg = 0; tg < GEMM_TG; tg++) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int t = 16 * tg + q4 + i;
                if (t >= nt) continue;
                const int64_t oi = t0 + t;
                if (a.part) {   // raw sums of this split, gate and up apart
                    float *pp = a.part + ((int64_t)gz * a.ptok + oi) * a.prow;
#pragma unroll
                    for (int gi = 0; gi < RG; gi++) {
                        const bool hi = a.glu && gi >= RG / 2;
                        const int g = a.glu ? gi % (RG / 2) : gi;
                        const int64_t r = tile * tile_rows + 16 * (wave * gpw + g) + n16;
                        if (r < rows) pp[(hi ? rows : 0) + r] = acc[gi][tg][i];
                    }
                } else if (a.glu) {
#pragma unroll
                    for (int gi = 0; gi < RG / 2; gi++) {
                        const int64_t r = tile * tile_rows + 16 * (wave * gpw + gi) + n16;
                        if (r < rows) {
                            const float gv = acc[gi][tg][i], uv = acc[gi + RG / 2][tg][i];
                            a.y[oi * a.y_stride + r] = glu(a.glu, gv, uv);
                            if (a.y2) {
                                a.y2[oi * a.y2_stride + r] = gv;
                                a.y2[oi * a.y2_stride + rows + r] = uv;
                            }
                        }
                    }
                } else {
#pragma unroll
                    for (int gi = 0; gi < RG; gi++) {
                        const int64_t r = tile * tile_rows + 16 * (wave * gpw + gi) + n16;
                        if (r < rows) a.y[oi * a.y_stride + r] = acc[gi][tg][i];
                    }
                }
            }
        }
        lds_barrier();   // the next tile's first loads reuse the ring and x
    }
    // no buffer-to-LDS load may still be in flight when the wave ends
    QG_WAIT_VM(0);
}

gemv_fn gemm_kernel_mfma(int type) { return type == T_Q8_0 ? k_gemm_mfma<T_Q8_0> : k_gemm_mfma<T_Q4_0>; }

int gemm_tile_rows(int glu) { return GEMM_WAVES * 16 * (glu ? GemmGeom<T_Q8_0>::RG / 2 : GemmGeom<T_Q8_0>::RG); }

int gemm_threads() { return GEMM_THREADS; }

int gemm_token_tile() { return GEMM_TT; }

int gemm_chunk_values() { return GEMM_KC; }

size_t gemm_xs_bytes(int64_t cols, int ntok) {
    const int64_t nch = (cols + GEMM_KC - 1) / GEMM_KC, tiles = (ntok + GEMM_TT - 1) / GEMM_TT;
    return (size_t)(tiles * nch * GEMM_XBLK);
}

int gemm_split_x(const float *x, int64_t x_stride, int ntok, int64_t cols, uint8_t *xs, hipStream_t st) {
    const int64_t nch = (cols + GEMM_KC - 1) / GEMM_KC, tiles = (ntok + GEMM_TT - 1) / GEMM_TT;
    const int64_t total = tiles * nch * GEMM_TT * 8;      // threads: 8 values each
    hipLaunchKernelGGL(k_split_x, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, x, x_stride, ntok,
                       (int)cols, (int)nch, total, xs);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_EHIP;
}

// One thread per V consecutive outputs (token blockIdx.y, rows r..r+V-1): the
// splits' raw sums added in split order, so the result does not depend on
// which split finished first.  V = 4 when every row offset is a multiple of 4
// floats (16-byte loads and stores).
template <int V>
__global__ __launch_bounds__(256) void k_gemm_reduce(const float *part, int nsplit, int64_t ptok, int64_t prow,
                                                     int64_t rows, int glu, float *y, int64_t y_stride, float *y2,
                                                     int64_t y2_stride) {
    typedef float vec __attribute__((ext_vector_type(V)));
    const int64_t r = ((int64_t)blockIdx.x * 256 + threadIdx.x) * V;
    const int64_t t = blockIdx.y;
    if (r >= rows) return;
    const float *p = part + t * prow + r;
    const int64_t zs = ptok * prow;
    vec g = (vec)0.0f, u = (vec)0.0f;
#pragma unroll 8
    for (int z = 0; z < nsplit; z++) {
        g += *(const vec *)(p + z * zs);
        if (glu) u += *(const vec *)(p + z * zs + rows);
    }
    if (glu) {
        vec o;
#pragma unroll
        for (int i = 0; i < V; i++) o[i] = qg::glu(glu, g[i], u[i]);
        *(vec *)(y + t * y_stride + r) = o;
        if (y2) {
            *(vec *)(y2 + t * y2_stride + r) = g;
            *(vec *)(y2 + t * y2_stride + rows + r) = u;
        }
    } else {
        *(vec *)(y + t * y_stride + r) = g;
    }
}

int gemm_reduce(const GemvArgs &a, int nsplit, hipStream_t st) {
    const bool v4 = a.rows % 4 == 0 && a.prow % 4 == 0 && a.y_stride % 4 == 0 && ((uintptr_t)a.part & 15) == 0 &&
                    ((uintptr_t)a.y & 15) == 0 && (!a.y2 || (a.y2_stride % 4 == 0 && ((uintptr_t)a.y2 & 15) == 0));
    const int V = v4 ? 4 : 1;
    const dim3 grid((unsigned)((a.rows / V + 255) / 256), (unsigned)a.ntok);
    if (v4)
        hipLaunchKernelGGL(k_gemm_reduce<4>, grid, dim3(256), 0, st, a.part, nsplit, a.ptok, a.prow, a.rows, a.glu,
                           a.y, a.y_stride, a.y2, a.y2_stride);
    else
        hipLaunchKernelGGL(k_gemm_reduce<1>, grid, dim3(256), 0, st, a.part, nsplit, a.ptok, a.prow, a.rows, a.glu,
                           a.y, a.y_stride, a.y2, a.y2_stride);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_EHIP;
}

}  // namespace qg

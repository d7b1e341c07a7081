// qg_gemm.hip -- prefill-size chunks (tens to thousands of tokens) of Q8_0 /
// Q4_0 products on the matrix cores (gfx950 v_mfma_f32_16x16x32_bf16).
//
// y[t][r] = sum_c W[r][c] x[t][c] with every product exact, as in the small
// batch kernel: codes are small integers (exact in bf16) and x enters as three
// bf16 parts whose sum is x exactly, so only the f32 accumulation order
// differs from an f32 FMA chain.  What changes at prefill size is reuse: a
// workgroup owns 64 tokens (TG = 4 groups of 16) and 4 waves x RG groups of
// 16 rows, and every weight block it loads feeds 3 * TG MFMAs per row group.
// The tokens' x is staged in LDS a k-chunk (KC values) at a time, already
// split into its three bf16 parts, so the split is paid once per workgroup
// rather than once per MFMA, and the weights' row segments go HBM -> LDS by
// asynchronous 16-byte copies two k-chunks ahead.  The pages' prompt-chunk GEMMs (qwen35_moe_ssd.js
// matmulQ8T, gemma4_moe_ssd.js matmulQ4T) tile 16 rows x 16 tokens through
// workgroup memory in f32; this keeps their "each weight byte serves many
// tokens" and moves the contraction to the matrix cores.
#include "../../include/qgemv.h"
#include "qg_kernels.h"
#include "qg_block.h"

namespace qg {

constexpr int GEMM_KC = 64;                     // x values per staged k-chunk (2 blocks)
constexpr int GEMM_XROW = GEMM_KC * 2 + 16;     // LDS bytes per (part, token) row, padded
constexpr int GEMM_TG = 4;                      // token groups of 16 per workgroup
constexpr int GEMM_TT = 16 * GEMM_TG;

// Workgroup tile: 4 waves x RG groups of 16 rows (gated: RG/2 gate groups and
// the same up groups per wave) x 64 tokens; grid.x row tiles (grid-stride),
// grid.y 64-token chunks.  Lane l: row / token l%16, k-group l/16 of each
// 32-value block; D[4(l/16)+i][l%16] = token 4(l/16)+i, row l%16.
//
// Per k-chunk (2 blocks) the tile's row segments are copied HBM -> LDS by
// 16-byte buffer-to-LDS loads, three chunks ahead of use in a ring of four,
// each from the 16-byte-aligned start below the segment (one more piece than
// the segment needs); row slots are numbered gate rows first, so every load
// instruction reads one matrix.  x is loaded into registers two chunks ahead
// of its split, neighbouring lanes reading neighbouring 16-byte pieces.  Every chunk issues the same loads (indices clamped to valid
// memory past the end, results unused), so a fixed wait count retires
// exactly the loads a chunk needs.
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

template <int TY>
struct GemmGeom {
    static constexpr int BYTES = TY == T_Q8_0 ? 34 : 18;
    static constexpr int RG = 2;                                  // row groups per wave
    static constexpr int NS = 4 * RG * 16;                        // row slots per tile
    static constexpr int SEGP = (15 + (GEMM_KC / 32) * BYTES + 15) / 16;   // pieces per slot
    static constexpr int PIECES = NS * SEGP;
    static constexpr int NI = PIECES / 256;                       // loads per thread per chunk
    static constexpr int RING = 4;
    static constexpr int SLOT = PIECES * 16;                      // bytes per ring slot
    static_assert(PIECES % 256 == 0, "whole loads per thread");
    static_assert((NS / 2) * SEGP % 64 == 0, "a load instruction reads one matrix");
};

template <int TY>
__global__ __launch_bounds__(256) void k_gemm_mfma(GemvArgs a) {
    typedef GemmGeom<TY> G;
    constexpr int BYTES = G::BYTES, RG = G::RG, SEGP = G::SEGP;
    constexpr int BPC = GEMM_KC / 32;           // blocks per k-chunk
    __shared__ __attribute__((aligned(16))) uint8_t s_x[3 * GEMM_TT * GEMM_XROW];
    __shared__ __attribute__((aligned(16))) uint8_t s_w[G::RING * G::SLOT];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int n16 = lane & 15, q = lane >> 4;
    const int nb = a.cols / 32;
    // this workgroup's k-chunks [c_lo, nch): the whole row, or one split of it
    const int nch_all = (nb + BPC - 1) / BPC;
    const int c_lo = a.part ? (int)blockIdx.z * a.kchunks : 0;
    const int nch = a.part ? min(nch_all, c_lo + a.kchunks) : nch_all;
    const int64_t rows = a.rows;
    const u32 rb = (u32)a.row_bytes;
    const int t0 = blockIdx.y * GEMM_TT;
    const int nt = min(GEMM_TT, a.ntok - t0);
    const int gpw = a.glu ? RG / 2 : RG;        // distinct row groups per wave
    const int tile_rows = 4 * 16 * gpw;

    const u32 ph0 = (u32)((uintptr_t)a.W0 & 15u), ph1 = (u32)((uintptr_t)a.W1 & 15u);
    const rsrc_t rs0 = make_rsrc(a.W0 - ph0, (u32)((ph0 + a.bytes0 + 15) & ~(int64_t)15));
    const rsrc_t rs1 = make_rsrc(a.W1 - ph1, (u32)((ph1 + a.bytes1 + 15) & ~(int64_t)15));
    const u32 cpos = 2u + 8u * (u32)(TY == T_Q8_0 ? q : (q & 1));
    const u32 sx0 = lds_off(s_x), sw0 = lds_off(s_w);

    // row slot -> (matrix, row): gated launches number their gate rows first
    auto slot_row = [&](int64_t tile, int slot, bool &hi) {
        const int half = G::NS / 2;
        hi = a.glu && slot >= half;
        const int sl = a.glu ? slot % half : slot;       // wave * gpw * 16 + g * 16 + n
        return min(tile * tile_rows + sl, rows - 1);
    };
    auto dma = [&](int64_t tile, int chunk) {
        uint8_t *dst = s_w + ((chunk - c_lo) % G::RING) * G::SLOT;
        const u32 cbyte = (u32)min(chunk, nch - 1) * (u32)(BPC * BYTES);
#pragma unroll
        for (int i = 0; i < G::NI; i++) {
            // pieces [i*256 + 64*wave, +64) lie in one matrix
            const bool hiw = __builtin_amdgcn_readfirstlane(
                                 (int)(a.glu && (i * 256 + 64 * wave) >= (G::NS / 2) * SEGP)) != 0;
            // this thread's piece: a row slot and a piece of its segment
            const int p = i * 256 + tid;
            bool hi;
            const int64_t r = slot_row(tile, p / SEGP, hi);
            const u32 off = (((u32)r * rb + cbyte + (hiw ? ph1 : ph0)) & ~15u) + 16u * (u32)(p % SEGP);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(hiw ? rs1 : rs0,
                                                     (__attribute__((address_space(3))) void *)(
                                                         (__attribute__((address_space(3))) uint8_t *)dst +
                                                         (i * 256 + 64 * wave) * 16),
                                                     16, off, 0, 0, 0);
        }
    };

    // x staging: a chunk is 64 tokens x KC values = TT * KC/4 pieces of 16
    // bytes; piece j of thread tid is piece (tid % P4) of token tid / P4 +
    // j * (256 / P4), so the 16-byte loads of neighbouring lanes are
    // neighbours in memory
    constexpr int P4 = GEMM_KC / 4;                    // pieces per token row
    constexpr int XL = GEMM_TT * P4 / 256;             // pieces (loads) per thread
    static_assert(256 % P4 == 0 && XL * 256 == GEMM_TT * P4, "x staging map");
    const int st_p = tid % P4, st_t0 = tid / P4;
    f32x4 xv[2][XL];
    auto x_fetch = [&](int chunk, int xb) {
        const int k = min(chunk, nch - 1) * GEMM_KC + 4 * st_p;
#pragma unroll
        for (int j = 0; j < XL; j++) {
            const int tok = st_t0 + j * (256 / P4);
            const bool in = tok < nt && chunk < nch && k < a.cols;
            const f32x4 v = *(const f32x4 *)(a.x + (int64_t)(t0 + (tok < nt ? tok : 0)) * a.x_stride +
                                             min(k, a.cols - 4));
            xv[xb][j] = in ? v : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    };
    auto x_put3 = [&](int xb) {
#pragma unroll
        for (int j = 0; j < XL; j++) {
            const int tok = st_t0 + j * (256 / P4);
            u32 h[2], m[2], l[2];
            split3x4(xv[xb][j], h, m, l);
            const u32 off = sx0 + (u32)tok * GEMM_XROW + (u32)st_p * 8u;
            lds_st64(off, h[0], h[1]);
            lds_st64(off + GEMM_TT * GEMM_XROW, m[0], m[1]);
            lds_st64(off + 2 * GEMM_TT * GEMM_XROW, l[0], l[1]);
        }
    };

    for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
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
                    const u32 off = sx0 + (u32)(16 * tg + n16) * GEMM_XROW + (u32)(32 * blc + 8 * q) * 2u;
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

        // chunk c: its x (in registers) split into LDS, its segments waited
        // for, then x two chunks on and segments three chunks on requested,
        // then c's blocks computed
        auto step = [&](int c, int xb) {
            lds_barrier();   // every wave is done with the previous chunk's x and ring slot
            x_put3(xb);
            // chunk c's segments have landed: issued before them, or later
            // than them, are at most 2 * NI + XL loads still outstanding
            QG_WAIT_VM(2 * G::NI + XL);
            lds_barrier();
            x_fetch(c + 2, xb);
            dma(tile, c + 3);
            consume(c);
        };
        x_fetch(c_lo, 0);
        dma(tile, c_lo);
        x_fetch(c_lo + 1, 1);
        dma(tile, c_lo + 1);
        dma(tile, c_lo + 2);
        int c = c_lo;
        for (; c + 2 <= nch; c += 2) {
            step(c, 0);
            step(c + 1, 1);
        }
        if (c < nch) step(c, 0);
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
                    float *pp = a.part + ((int64_t)blockIdx.z * a.ptok + oi) * a.prow;
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

int gemm_rows_per_wave(int glu) { return 16 * (glu ? GemmGeom<T_Q8_0>::RG / 2 : GemmGeom<T_Q8_0>::RG); }

int gemm_token_tile() { return GEMM_TT; }

int gemm_chunk_values() { return GEMM_KC; }

// One thread per output (token blockIdx.y, row r): the splits' raw sums added
// in split order, so the result does not depend on which split finished first.
__global__ __launch_bounds__(256) void k_gemm_reduce(const float *part, int nsplit, int64_t ptok, int64_t prow,
                                                     int64_t rows, int glu, float *y, int64_t y_stride, float *y2,
                                                     int64_t y2_stride) {
    const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t t = blockIdx.y;
    if (r >= rows) return;
    const float *p = part + t * prow + r;
    const int64_t zs = ptok * prow;
    float g = 0.0f, u = 0.0f;
    for (int z = 0; z < nsplit; z++) {
        g += p[z * zs];
        if (glu) u += p[z * zs + rows];
    }
    if (glu) {
        y[t * y_stride + r] = qg::glu(glu, g, u);
        if (y2) {
            y2[t * y2_stride + r] = g;
            y2[t * y2_stride + rows + r] = u;
        }
    } else {
        y[t * y_stride + r] = g;
    }
}

int gemm_reduce(const GemvArgs &a, int nsplit, hipStream_t st) {
    hipLaunchKernelGGL(k_gemm_reduce, dim3((unsigned)((a.rows + 255) / 256), (unsigned)a.ntok), dim3(256), 0, st,
                       a.part, nsplit, a.ptok, a.prow, a.rows, a.glu, a.y, a.y_stride, a.y2, a.y2_stride);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_EHIP;
}

}  // namespace qg

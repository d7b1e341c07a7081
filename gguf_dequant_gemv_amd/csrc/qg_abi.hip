// qg_abi.hip -- the extern "C" entry points of libqgemv (see include/qgemv.h):
// synchronous argument validation, launch planning and kernel dispatch.
// Nothing here allocates memory or synchronises a stream.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/qgemv.h"
#include "qg_moe1.h"
#include "qg_kernels.h"
#include "qg_block.h"
#include "qg_kq1.h"
#include "qg_planes.h"

using namespace qg;

namespace {

struct TypeInfo {
    int qk, bytes;        // values / bytes per GGUF block
    int block_vals;       // values per block unit
    int pairs;            // 1: Q8_0 / Q4_0 can use pair units
};

bool type_info(int t, TypeInfo &ti) {
    switch (t) {
    case QG_Q8_0: ti = {32, 34, 32, 1}; return true;
    case QG_Q4_0: ti = {32, 18, 32, 1}; return true;
    case QG_Q4_K: ti = {256, 144, 256, 0}; return true;
    case QG_Q6_K: ti = {256, 210, 256, 0}; return true;
    default: return false;
    }
}

constexpr int NUM_CU = 256;
constexpr int64_t MAX_RANGE = (int64_t)1 << 31;   // bytes one buffer descriptor addresses per launch

struct Shape {
    int type;
    TypeInfo ti;
    int64_t rows, row_bytes;
    int cols, nb;
};

int make_shape(int type, int64_t rows, int64_t cols, Shape &s) {
    if (!type_info(type, s.ti)) return QG_EINVAL;
    if (rows <= 0 || cols <= 0 || cols % s.ti.qk) return QG_EINVAL;
    if (cols > (1 << 20) || rows > ((int64_t)1 << 40)) return QG_ELIMIT;
    s.type = type;
    s.rows = rows;
    s.cols = (int)cols;
    s.nb = (int)(cols / s.ti.qk);
    s.row_bytes = (int64_t)s.nb * s.ti.bytes;
    return QG_OK;
}

int sums_of(int type) { return type == QG_Q6_K ? 16 : (type == QG_Q8_0 ? 0 : 32); }

size_t lds_bytes(int type, int cpad, int nt) {
    const int sums = sums_of(type);
    const size_t per = (size_t)xstride_of(cpad) + (sums ? cpad / sums : 0);
    return (size_t)nt * per * sizeof(float);
}

struct Plan {
    int kind, lpr, nt;
    int nunits;          // units per row
    int ntiles;          // row tiles of 4 * 64/lpr rows
    int64_t copies;      // independent problems sharing the GPU in one launch
    int depth;           // UK_LDS: stages in flight per wave
    bool valu_heavy;     // K-quant units: decode-bound rather than HBM-bound
    bool fill_all;       // grid-stride launches take every resident slot
    int ring_off;        // UK_LDS: byte offset of the stage rings in LDS
    int xchunk;          // UK_LDS: row elements per staged x chunk (0: all of x)
    size_t lds;
};

bool lds_kind(int kind) { return kind == UK_LDS || kind == UK_LDS2; }

// Bytes of one LDS stage in whole KiB: 64/lpr rows of lpr units in 16-byte
// pieces (UK_LDS2 fetches one more piece per row), 64 pieces per load.
int stage_bytes(const TypeInfo &ti, int lpr, int kind) {
    const int ub = ti.pairs ? 2 * ti.bytes : ti.bytes;
    const int pieces = (64 / lpr) * (lpr * ub / 16 + (kind == UK_LDS2 ? 1 : 0));
    return (pieces + 63) / 64 * 1024;
}

int unit_count(const Shape &s, int kind) {
    if (lds_kind(kind) && s.ti.pairs) return s.nb / 2;
    return s.cols / s.ti.block_vals;
}

// Kernel kind and lanes per row: best lane utilisation (units per row spread
// evenly over the row's lanes), then segment length and wave fill.
//   ntok_max:   most tokens one workgroup must serve
//   copies:     independent problems sharing the GPU in one launch
//   lds_ok:     every weight range starts 16-byte aligned (with rows a whole
//               number of 16-byte pieces, the aligned LDS variant applies)
//   mfma_ntok:  tokens a workgroup's chunk may hold (MFMA from 4 on)
// T = 4..16 tokens of Q8_0 / Q4_0 go to the MFMA kernel (one 16-token chunk).
constexpr int MFMA_MIN_TOK = 4;

Plan make_plan(const Shape &s, int ntok_max, int64_t copies, bool lds_ok, int mfma_ntok = -1) {
    Plan p;
    if (mfma_ntok < 0) mfma_ntok = ntok_max;
    if ((s.type == QG_Q8_0 || s.type == QG_Q4_0) && mfma_ntok >= MFMA_MIN_TOK) {
        p.kind = UK_MFMA;
        p.lpr = 0;
        p.nt = 16;
        p.nunits = s.nb;
        p.copies = copies > 0 ? copies : 1;
        p.depth = 0;
        p.ring_off = 0;
        p.valu_heavy = false;
        p.fill_all = false;
        p.lds = 0;
        p.ntiles = 0;     // set at launch (gated tiles hold half the rows)
        p.xchunk = 0;
        return p;
    }
    int nt = 1;
    while (nt < ntok_max && nt < 8) nt <<= 1;
    p.copies = copies > 0 ? copies : 1;
    // staged through LDS (16-byte aligned, or any 2-byte phase) unless a
    // Q8_0 / Q4_0 row has an odd block count (pair units need whole pairs)
    const bool units_ok = !s.ti.pairs || (s.nb % 2) == 0;
    p.kind = !units_ok ? UK_BLOCK : (lds_ok && (s.row_bytes % 16) == 0) ? UK_LDS : UK_LDS2;
    p.lpr = 64;
    double best = -1.0;
    {
        const int kind = p.kind;
        const int nunits = unit_count(s, kind);
        const int cands[5] = {4, 8, 16, 32, 64};   // ties go to fewer lanes per row
        for (int ci = 0; ci < 5; ci++) {
            const int lpr = cands[ci], rpw = 64 / lpr;
            if (lds_kind(kind) && s.type == QG_Q6_K && lpr < 8) continue;   // 210-byte units: 16-byte segments need 8
            const int per_lane = (nunits + lpr - 1) / lpr;
            const double util = (double)nunits / ((double)lpr * per_lane);
            const double waves = (double)((s.rows + rpw - 1) / rpw) * (double)p.copies;
            const double fill = waves >= 8.0 * NUM_CU ? 1.0 : waves / (8.0 * NUM_CU);
            // Staged through LDS, each wave streams 64/lpr row segments of lpr
            // units: segments of 1 KiB or more keep HBM reads in long runs
            // (measured worth more than the idle lanes of a ragged last slot).
            // The K-quant decode is VALU-bound: there idle lanes cost most and
            // fewer lanes per row (more units each) measured fastest.  Grouped
            // expert launches of several tokens read a few short rows per
            // expert whatever the lanes, so there the idle lanes alone count
            // (128 experts, Q4_0 704 x 2816 gate-up and down, 16 tokens: down
            // 16 -> 4 lanes per row, 126.5 -> 119 us for the layer).
            const bool heavy = s.type == QG_Q4_K || s.type == QG_Q6_K;
            const bool grouped_tok = p.copies > 1 && ntok_max > 1;
            double seg = 1.0;
            if (lds_kind(kind) && !heavy && !grouped_tok) {
                const double sb = (double)lpr * (s.ti.pairs ? 2 * s.ti.bytes : s.ti.bytes);
                seg = 0.5 + 0.5 * (sb >= 1024.0 ? 1.0 : sb / 1024.0);
            }
            const double fw = heavy ? 0.1 : 0.35;
            const double score = util * seg * (1.0 - fw + fw * fill);
            if (score > best + 1e-9) { best = score; p.lpr = lpr; }
        }
    }
    // Q6_K at one token: per-lane loads (k_gemv) with 8 lanes per row beat the
    // LDS-staged stream, whose rings of 210-byte units cost the residency the
    // VALU-heavy decode needs (measured 31.9 vs 33.6 us at 5120 x 17408 and
    // 134 vs 168 us at 262144 x 2816); x must fit the LDS whole
    if (s.type == QG_Q6_K && nt == 1 && lds_bytes(s.type, s.nb * s.ti.block_vals, 1) <= 96 * 1024) {
        p.kind = UK_BLOCK;
        p.lpr = 8;
    }
    p.nunits = unit_count(s, p.kind);
    const int uv = (lds_kind(p.kind) && s.ti.pairs) ? 2 * s.ti.qk : s.ti.block_vals;
    const int cpad = p.nunits * uv;
    const size_t xcap = lds_kind(p.kind) ? 96 * 1024 : 64 * 1024;
    while (nt > 1 && lds_bytes(s.type, cpad, nt) > xcap) nt >>= 1;
    p.nt = nt;
    p.lds = lds_bytes(s.type, cpad, nt);
    p.depth = 0;
    p.ring_off = 0;
    p.xchunk = 0;
    p.valu_heavy = s.type == QG_Q4_K || s.type == QG_Q6_K;
    // Every resident slot also pays for the grouped expert launches of Q4_0
    // (twice the values per byte of Q8_0, and one decode shared by at most a
    // chunk of a few tokens): at 128 experts 704 x 2816, top-8, measured
    // 91.5 -> 67.6 us at 8 tokens and 150.8 -> 115.8 us at 16 (gate-up plus
    // down).  Grouped Q8_0 stays on the long streams (256 experts 512 x 2048,
    // 16 tokens: 89.1 us on them, 98.7 us on every slot).
    p.fill_all = p.valu_heavy || (s.type == QG_Q4_0 && p.copies > 1);
    if (lds_kind(p.kind)) {
        // stage rings after x: two stages per wave when two workgroups still
        // fit a CU's 160 KiB, else one (a stage is refilled as soon as it has
        // been read, so even one keeps a stage per wave in flight)
        // A launch whose workgroups take a tile or two each runs best with one
        // stage per wave (smaller rings, more workgroups resident); long
        // streams keep two in flight.
        p.ring_off = (int)((p.lds + 255) & ~(size_t)255);
        const size_t per_depth = 4 * (size_t)stage_bytes(s.ti, p.lpr, p.kind);
        const int64_t tiles_all = (s.rows + 4LL * (64 / p.lpr) - 1) / (4LL * (64 / p.lpr)) * p.copies;
        p.depth = 1;
        // (the grouped Q4_0 launches spread a few tiles over every resident
        // slot: one stage, more slots; 128 experts 704 x 2816 at 16 tokens,
        // gate-up 73.4 -> 65.9 us)
        const bool short_streams = p.fill_all && p.copies > 1 && !p.valu_heavy;
        if (tiles_all > 4 * NUM_CU && !short_streams && p.ring_off + 2 * per_depth <= 80 * 1024) p.depth = 2;
        p.lds = p.ring_off + p.depth * per_depth;
        // x too wide for two workgroups per CU while the tiles need more than
        // one round at one per CU: stage x in chunks of whole row elements,
        // the widest that still lets two fit (each chunk is restaged per tile
        // row from the L2, which costs more than it gains when one round
        // holds every tile anyway)
        const int K = (p.nunits + p.lpr - 1) / p.lpr;
        if (p.lds > 80 * 1024 && K >= 2 && tiles_all > NUM_CU) {
            for (int jc = K - 1; jc >= 1; jc--) {
                const int cp = (p.nunits < jc * p.lpr ? p.nunits : jc * p.lpr) * uv;
                const size_t xl = lds_bytes(s.type, cp, nt);
                const int roff = (int)((xl + 255) & ~(size_t)255);
                if (roff + p.depth * per_depth <= 80 * 1024) {
                    p.xchunk = jc;
                    p.ring_off = roff;
                    p.lds = roff + p.depth * per_depth;
                    break;
                }
            }
        }
    }
    const int64_t tile_rows = 4LL * (64 / p.lpr);
    p.ntiles = (int)((s.rows + tile_rows - 1) / tile_rows);
    return p;
}

// Workgroups that stay resident at once (all CUs), from the kernel's actual
// register and LDS use; cached per kernel and LDS size.
int resident_wgs_of(const void *f, size_t lds) {
    struct Entry { const void *f; size_t lds; int n; };
    static std::mutex mu;
    static Entry cache[512];
    static int used = 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; i++)
        if (cache[i].f == f && cache[i].lds == lds) return cache[i].n;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, 256, lds) != hipSuccess || per_cu < 1)
        per_cu = 1;
    const int n = per_cu * NUM_CU;
    if (used < 512) cache[used++] = {f, lds, n};
    return n;
}
int resident_wgs(gemv_fn f, size_t lds) { return resident_wgs_of((const void *)f, lds); }

// Grid-stride width.  Workgroups that cannot be resident at once run in
// later rounds, and fewer workgroups than resident slots leave memory
// parallelism unused; pick the tiles per workgroup that minimises
//   rounds * tiles per workgroup * (slots / workgroups, if fewer) + a start
// cost per round (staging x and filling the pipeline).
int grid_for(const Plan &p, gemv_fn f) {
    int64_t cap = resident_wgs(f, p.lds) / p.copies;
    if (cap < 1) cap = 1;
    if (lds_kind(p.kind)) {
        // every tile its own workgroup while they all fit at once; past that,
        // about two workgroups per CU, each streaming many tiles (fewer,
        // longer HBM streams measured faster than filling every slot)
        if (p.ntiles <= cap) return p.ntiles;
        // the K-quant decode is VALU-heavy: there every resident slot helps
        int64_t target = p.fill_all ? cap : 2 * NUM_CU / p.copies;
        if (target < 1) target = 1;
        if (target > cap) target = cap;
        const int64_t tpw = (p.ntiles + target - 1) / target;
        return (int)((p.ntiles + tpw - 1) / tpw);
    }
    double best = 1e300;
    int64_t best_gx = p.ntiles;
    for (int64_t tpw = 1; tpw <= 16; tpw++) {
        const int64_t gx = (p.ntiles + tpw - 1) / tpw;
        const int64_t rounds = (gx + cap - 1) / cap;
        const double under = gx < cap ? (double)cap / (double)gx : 1.0;
        const double cost = (double)rounds * (double)tpw * under + 0.3 * (double)rounds;
        if (cost < best - 1e-9) { best = cost; best_gx = gx; }
        if (gx == 1) break;
    }
    return (int)best_gx;
}

#define QG_PICK_NT(NAME) \
    (p.nt == 1 ? gemv_kernel_##NAME##_t1(p.kind, p.lpr, p.xchunk > 0, rt) \
     : p.nt == 2 ? gemv_kernel_##NAME##_t2(p.kind, p.lpr, p.xchunk > 0, false) \
     : p.nt == 4 ? gemv_kernel_##NAME##_t4(p.kind, p.lpr, p.xchunk > 0, false) \
     : gemv_kernel_##NAME##_t8(p.kind, p.lpr, p.xchunk > 0, false))

gemv_fn pick(int type, const Plan &p, bool rt) {
    switch (type) {
    case QG_Q8_0: return QG_PICK_NT(q8_0);
    case QG_Q4_0: return QG_PICK_NT(q4_0);
    case QG_Q4_K: return QG_PICK_NT(q4_k);
    default: return QG_PICK_NT(q6_k);
    }
}
#undef QG_PICK_NT

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Prefill launches split along the row when their row and token tiles alone
// leave CUs idle (the 2560-row down projection of a 64-token chunk is 10
// tiles): each split sums a run of whole k-chunks into a partial buffer, and
// a second launch adds the splits in order.  The split count minimises the
// estimated time: rounds of resident workgroups (one per CU) x (chunks per
// split + pipeline fill) at ~2 us a chunk, plus the adding launch (a few us
// and its bytes at ~2.5 TB/s).  Launches that fill the CUs already are not
// split.  The same rule sizes the workspace.
struct GemmSplit {
    int n, kchunks;
};
GemmSplit gemm_split(int type, int64_t rows, int64_t cols, int ntok, int glu) {
    const int64_t kv = gemm_chunk_values();
    const int64_t nch = (cols + kv - 1) / kv;
    GemmSplit best = {1, (int)nch};
    if ((type != QG_Q8_0 && type != QG_Q4_0) || ntok <= QG_MAX_TOKENS || ntok > QG_MAX_PREFILL) return best;
    const int64_t tt = gemm_token_tile();
    const int64_t tile_rows = gemm_tile_rows(glu);
    const int64_t wgs = ((rows + tile_rows - 1) / tile_rows) * ((ntok + tt - 1) / tt);
    if (wgs >= NUM_CU) return best;
    const double step_us = 2.0, fill = 2.0;
    // partial sums read, plus the outputs written (gated: y, gate and up)
    const double out_bytes = (double)ntok * (double)rows * (glu ? 2.0 : 1.0) * 4.0;
    const double out_written = glu ? 1.5 : 1.0;
    double best_us = ((double)nch + fill) * step_us;
    for (int n = 2; n <= 32; n++) {
        const int64_t kc = (nch + n - 1) / n;
        if (kc < 4) break;
        const int64_t ns = (nch + kc - 1) / kc;
        const int64_t rounds = (wgs * ns + NUM_CU - 1) / NUM_CU;
        const double us =
            (double)rounds * ((double)kc + fill) * step_us + 4.0 + ((double)ns + out_written) * out_bytes / 2.5e6;
        if (us < best_us) {
            best_us = us;
            best = {(int)ns, (int)kc};
        }
    }
    return best;
}

// Small-batch MFMA launches (4..16 tokens, dense): row groups of 16 per tile
// (four, or two when four leave fewer tiles than twice the CUs), and, when
// the tiles still leave most CUs idle (a few thousand rows of a long row),
// the blocks of each row split over `n` workgroups of at least 32 blocks
// (eight per wave) whose raw sums the reduce launch adds in split order.
// Rows under 192 blocks stay whole: there the reduce launch costs more than
// the shorter walk saves (2816 x 2112 Q4_0 MLP at 16 tokens: 22.1 us whole,
// 26.8 us split) -- unless the tiles fill under a quarter of the CUs, when
// rows of 64+ blocks split into splits of 16+.  2560 x 9728 Q8_0 at 16
// tokens is 80 tiles: 7 splits (the MLP at 4 tokens 69 -> 34 us).
int small_groups(int64_t rows, int glu, int64_t copies) {
    return (rows + 16 * (glu ? 2 : 4) - 1) / (16 * (glu ? 2 : 4)) * copies < 2 * NUM_CU ? 2 : 4;
}
GemmSplit small_split(int type, int64_t rows, int64_t cols, int ntok, int glu) {
    const int64_t nb = cols / 32;
    GemmSplit none = {1, (int)nb};
    if ((type != QG_Q8_0 && type != QG_Q4_0) || ntok < MFMA_MIN_TOK || ntok > QG_MAX_TOKENS) return none;
    const int groups = small_groups(rows, glu, 1);
    const int64_t tile_rows = 16 * (glu ? groups / 2 : groups);
    const int64_t wgs = (rows + tile_rows - 1) / tile_rows;
    // a launch of under a quarter of the CUs' worth of tiles splits rows of
    // 64+ blocks into splits of 16+ (the shared expert's 512 x 2048 gate and
    // up at 16 tokens: 32 tiles)
    const bool sparse = wgs < NUM_CU / 4;
    if (wgs >= NUM_CU || nb < (sparse ? 64 : 192)) return none;
    const int64_t want = (2 * NUM_CU + wgs - 1) / wgs;
    int64_t kb = (nb + want - 1) / want;
    if (kb < (sparse ? 16 : 32)) kb = sparse ? 16 : 32;
    const int64_t n = (nb + kb - 1) / kb;
    if (n < 2) return none;
    return {(int)n, (int)kb};
}
size_t small_part_bytes(int type, int64_t rows, int64_t cols, int ntok, int glu) {
    const GemmSplit sp = small_split(type, rows, cols, ntok, glu);
    if (sp.n < 2) return 0;
    return ((size_t)sp.n * (size_t)ntok * (size_t)(glu ? 2 : 1) * (size_t)rows * 4 + 255) & ~(size_t)255;
}

bool prefill_kernel(int type, int ntok) {
    return (type == QG_Q8_0 || type == QG_Q4_0) && ntok > QG_MAX_TOKENS && ntok <= QG_MAX_PREFILL;
}

// bytes of the partial sums of a split prefill launch (0: no split)
size_t gemm_part_bytes(int type, int64_t rows, int64_t cols, int ntok, int glu) {
    const GemmSplit sp = gemm_split(type, rows, cols, ntok, glu);
    if (sp.n < 2) return 0;
    return ((size_t)sp.n * (size_t)ntok * (size_t)(glu ? 2 : 1) * (size_t)rows * 4 + 255) & ~(size_t)255;
}

// scratch of one prefill launch: the split x, then the partial sums (or of a
// split small-batch launch: its partial sums)
size_t gemm_scratch_bytes(int type, int64_t rows, int64_t cols, int ntok, int glu) {
    if (ntok <= QG_MAX_TOKENS) return small_part_bytes(type, rows, cols, ntok, glu);
    if (!prefill_kernel(type, ntok)) return 0;
    return ((gemm_xs_bytes(cols, ntok) + 255) & ~(size_t)255) + gemm_part_bytes(type, rows, cols, ntok, glu);
}

// the same for a qg_gemm call, whose rows go out in launches of at most
// MAX_RANGE weight bytes: the largest any of those launches needs (a short
// last launch may split its rows where the full-size ones do not)
size_t gemm_call_scratch_bytes(int type, int64_t rows, int64_t cols, int ntok) {
    Shape s;
    if (make_shape(type, rows, cols, s)) return 0;
    const int64_t chunk = MAX_RANGE / s.row_bytes;
    size_t need = gemm_scratch_bytes(type, rows < chunk ? rows : chunk, cols, ntok, 0);
    if (rows > chunk && rows % chunk) {
        const size_t last = gemm_scratch_bytes(type, rows % chunk, cols, ntok, 0);
        if (last > need) need = last;
    }
    return need;
}

// a: weights, x/y, tokens or groups and rows set by the caller.
int launch_mfma(const Shape &s, const Plan &p, GemvArgs a, dim3 grid, hipStream_t st) {
    a.x_vec = aligned(a.x, 16) && (a.x_stride % 4) == 0;
    a.cols = s.cols;
    a.nunits = p.nunits;
    if (!a.grp && a.ntok > QG_MAX_TOKENS) {
        // prefill chunk: x split once into the scratch, then 64-token tiles,
        // each weight block feeding every token group of the tile
        if (!a.ws || a.ws_bytes < gemm_scratch_bytes(s.type, a.rows, s.cols, a.ntok, a.glu)) return QG_EINVAL;
        int rc = gemm_split_x(a.x, a.x_stride, a.ntok, s.cols, a.ws, st);
        if (rc) return rc;
        a.xs = a.ws;
        const int tt = gemm_token_tile();
        const int64_t tchunks = (a.ntok + tt - 1) / tt;
        const int64_t tile_rows = gemm_tile_rows(a.glu);
        a.ntiles = (int)((a.rows + tile_rows - 1) / tile_rows);
        gemv_fn f = gemm_kernel_mfma(s.type);
        int64_t cap = NUM_CU / tchunks;   // its LDS ring holds one workgroup per CU
        if (cap < 1) cap = 1;
        const GemmSplit sp = gemm_split(s.type, a.rows, s.cols, a.ntok, a.glu);
        const bool split = sp.n > 1;
        a.part = split ? (float *)(a.ws + ((gemm_xs_bytes(s.cols, a.ntok) + 255) & ~(size_t)255)) : nullptr;
        a.kchunks = sp.kchunks;
        a.ptok = a.ntok;
        a.prow = (a.glu ? 2 : 1) * a.rows;
        a.wg_x = (int)(a.ntiles < cap ? a.ntiles : cap);
        a.wg_y = (int)tchunks;
        a.wg_z = split ? sp.n : 1;
        grid = dim3((unsigned)a.wg_x * (unsigned)a.wg_y * (unsigned)a.wg_z);
        hipLaunchKernelGGL(f, grid, dim3(gemm_threads()), 0, st, a);
        if (hipGetLastError() != hipSuccess) return QG_EHIP;
        return split ? gemm_reduce(a, sp.n, st) : QG_OK;
    }
    // four groups of 16 rows per tile, or two when that leaves too few tiles
    // to spread over the CUs
    const int groups = small_groups(a.rows, a.glu, p.copies);
    const int tile_rows = 16 * (a.glu ? groups / 2 : groups);
    a.ntiles = (int)((a.rows + tile_rows - 1) / tile_rows);
    gemv_fn f = gemv_kernel_mfma(s.type, groups);
    int64_t cap = resident_wgs(f, 0) / p.copies;
    if (cap < 1) cap = 1;
    grid.x = (unsigned)(a.ntiles < cap ? a.ntiles : cap);
    // dense, with a workspace: split long rows when the tiles leave CUs idle
    const GemmSplit sp = a.grp ? GemmSplit{1, 0} : small_split(s.type, a.rows, s.cols, a.ntok, a.glu);
    const bool split = sp.n > 1 && a.ws && a.ws_bytes >= small_part_bytes(s.type, a.rows, s.cols, a.ntok, a.glu);
    if (split) {
        a.part = (float *)a.ws;
        a.kchunks = sp.kchunks;
        a.ptok = a.ntok;
        a.prow = (a.glu ? 2 : 1) * a.rows;
        grid.x = (unsigned)a.ntiles;
        grid.z = (unsigned)sp.n;
    }
    hipLaunchKernelGGL(f, grid, dim3(256), 0, st, a);
    if (hipGetLastError() != hipSuccess) return QG_EHIP;
    return split ? gemm_reduce(a, sp.n, st) : QG_OK;
}

// The plan's fields in the kernel arguments of a vector-kernel launch.
int prep_gemv(const Shape &s, const Plan &p, GemvArgs &a) {
    a.row_bytes = s.row_bytes;
    // gated: gate rows in W0, the same rows of the up matrix in W1
    a.bytes0 = a.bytes1 = a.rows * s.row_bytes;
    if (!a.glu) a.W1 = a.W0;
    if (a.bytes0 > MAX_RANGE || a.bytes1 > MAX_RANGE) return QG_ELIMIT;
    a.x_vec = aligned(a.x, 16) && (a.x_stride % 4) == 0 && (!a.xg_x || aligned(a.xg_x, 16));
    a.cols = s.cols;
    a.nunits = p.nunits;
    a.ntiles = p.ntiles;
    a.depth = p.depth;
    a.ring_off = p.ring_off;
    a.xchunk = p.xchunk;
    return QG_OK;
}

int launch_gemv(const Shape &s, const Plan &p, GemvArgs a, dim3 grid, hipStream_t st) {
    if (p.kind == UK_MFMA) {
        a.row_bytes = s.row_bytes;
        a.bytes0 = a.bytes1 = a.rows * s.row_bytes;
        if (!a.glu) a.W1 = a.W0;
        if (a.bytes0 > MAX_RANGE || a.bytes1 > MAX_RANGE) return QG_ELIMIT;
        return a.r_logits ? QG_EINVAL : launch_mfma(s, p, a, grid, st);
    }
    const int rc = prep_gemv(s, p, a);
    if (rc) return rc;
    // a launch that routes its token needs the routing instance (one token,
    // LDS-staged, x whole); anything else would read a group table that no
    // routing launch wrote
    if (a.r_logits && !(p.nt == 1 && p.xchunk == 0)) return QG_EINVAL;
    gemv_fn f = pick(s.type, p, a.r_logits != nullptr);
    if (p.lds > 64 * 1024 && hipFuncSetAttribute((const void *)f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds) != hipSuccess)
        return QG_EHIP;
    grid.x = grid_for(p, f);
    hipLaunchKernelGGL(f, grid, dim3(256), p.lds, st, a);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_EHIP;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

int qg_block_values(int type) {
    if (type == QG_F32) return 1;
    if (type == QG_Q6_K_PLANES) type = QG_Q6_K;
    if (type == QG_Q8_0_PLANES) type = QG_Q8_0;
    TypeInfo ti;
    return type_info(type, ti) ? ti.qk : 0;
}

int qg_block_bytes(int type) {
    if (type == QG_F32) return 4;
    if (type == QG_Q6_K_PLANES) type = QG_Q6_K;
    if (type == QG_Q8_0_PLANES) type = QG_Q8_0;
    TypeInfo ti;
    return type_info(type, ti) ? ti.bytes : 0;
}

const char *qg_strerror(int code) {
    switch (code) {
    case QG_OK: return "ok";
    case QG_EINVAL: return "invalid argument (type, size, pointer or alignment)";
    case QG_EABSENT: return "a picked expert has no pool slot";
    case QG_EHIP: return "HIP launch or query failed";
    case QG_ELIMIT: return "size limit exceeded (ntok <= 16, experts <= 256, topk <= 32)";
    default: return "unknown error";
    }
}

}  // extern "C"

namespace {
// One token against a Q6_K tensor in the plane layout: the quarter-block
// kernel on its planes (one launch: the planes' offsets span the tensor)
int planes_gemv(const void *W, const float *x, float *y, int64_t rows, int64_t cols, int ntok, int max_tok,
                void *stream) {
    Shape s;
    int rc = make_shape(QG_Q6_K, rows, cols, s);
    if (rc) return rc;
    if (ntok < 1 || ntok > max_tok) return QG_ELIMIT;
    if (ntok != 1 || !W || !x || !y || !aligned(W, 16) || !aligned(x, 16) || !aligned(y, 4)) return QG_EINVAL;
    const int64_t n = rows * s.nb;
    if (n * s.ti.bytes > MAX_RANGE) return QG_ELIMIT;
    const uint8_t *P = (const uint8_t *)W;
    Kq1Args ka = {};
    ka.W = P;
    ka.Ph = P + 128 * n;
    ka.Ps = P + 192 * n;
    ka.Pd = P + 208 * n;
    ka.rows = rows;
    ka.row_bytes = (u32)s.row_bytes;
    ka.range = (u32)(128 * n);
    ka.nu = (int)(cols / 64);
    ka.cols = (int)cols;
    ka.x = x;
    ka.y = y;
    return launch_kq1(T_Q6_KP, ka, (hipStream_t)stream);
}

// One token against a Q8_0 tensor in the plane layout (qg_planes.h)
int q8_planes_gemv(const void *W, const float *x, float *y, int64_t rows, int64_t cols, int ntok, int max_tok,
                   void *stream) {
    Shape s;
    int rc = make_shape(QG_Q8_0, rows, cols, s);
    if (rc) return rc;
    if (ntok < 1 || ntok > max_tok) return QG_ELIMIT;
    if (ntok != 1 || !W || !x || !y || !aligned(W, 16) || !aligned(x, 16) || !aligned(y, 4)) return QG_EINVAL;
    if (rows * cols >= MAX_RANGE) return QG_ELIMIT;
    Q8pArgs qa = {};
    qa.C = (const uint8_t *)W;
    qa.D = (const uint8_t *)W + rows * cols;
    qa.rows = rows;
    qa.cols = (int)cols;
    qa.x = x;
    qa.y = y;
    return launch_q8p1(qa, false, (hipStream_t)stream);
}

// qg_gemv / qg_gemm: the same sum for up to max_tok tokens
int gemv_entry(int type, const void *W, const float *x, float *y, int64_t rows, int64_t cols, int ntok, int max_tok,
               void *ws, size_t ws_bytes, void *stream) {
    if (type == QG_F32) {   // plain f32 weights (router, shared-expert gate)
        if (rows <= 0 || cols <= 0) return QG_EINVAL;
        if (ntok < 1 || ntok > max_tok) return QG_ELIMIT;
        if (!W || !x || !y || !aligned(W, 4) || !aligned(x, 4) || !aligned(y, 4)) return QG_EINVAL;
        for (int t0 = 0; t0 < ntok; t0 += QG_MAX_TOKENS) {   // the f32 kernel serves 16 tokens a launch
            const int nt = ntok - t0 < QG_MAX_TOKENS ? ntok - t0 : QG_MAX_TOKENS;
            const int rc = launch_gemv_f32((const float *)W, x + (int64_t)t0 * cols, y + (int64_t)t0 * rows, rows,
                                           cols, nt, (hipStream_t)stream);
            if (rc) return rc;
        }
        return QG_OK;
    }
    if (type == QG_Q6_K_PLANES) return planes_gemv(W, x, y, rows, cols, ntok, max_tok, stream);
    if (type == QG_Q8_0_PLANES) return q8_planes_gemv(W, x, y, rows, cols, ntok, max_tok, stream);
    Shape s;
    int rc = make_shape(type, rows, cols, s);
    if (rc) return rc;
    if (ntok < 1 || ntok > max_tok) return QG_ELIMIT;
    if (!W || !x || !y || !aligned(W, 2) || !aligned(x, 4) || !aligned(y, 4)) return QG_EINVAL;
    // (qg_gemv brings no workspace: its small batches run unsplit)
    const bool takes_ws = max_tok > QG_MAX_TOKENS;
    if ((takes_ws && ws_bytes < gemm_call_scratch_bytes(type, rows, cols, ntok)) ||
        (ws_bytes && (!ws || !aligned(ws, 256))))
        return QG_EINVAL;
    // rows in launches of at most MAX_RANGE weight bytes each
    const int64_t chunk = MAX_RANGE / s.row_bytes;
    for (int64_t r0 = 0; r0 < rows; r0 += chunk) {
        Shape sc = s;
        sc.rows = rows - r0 < chunk ? rows - r0 : chunk;
        const uint8_t *Wc = (const uint8_t *)W + r0 * s.row_bytes;
        if (ntok == 1 && (type == QG_Q4_K || type == QG_Q6_K)) {   // quarter-block units (qg_kq1.h)
            Kq1Args ka = {};
            ka.W = Wc;
            ka.rows = sc.rows;
            ka.row_bytes = (u32)s.row_bytes;
            ka.range = (u32)(sc.rows * s.row_bytes);
            ka.nu = (int)(cols / 64);
            ka.cols = (int)cols;
            ka.x = x;
            ka.y = y + r0;
            rc = launch_kq1(type, ka, (hipStream_t)stream);
            if (rc == QG_OK) continue;
            if (rc != QG_EINVAL) return rc;   // else: the block-unit kernels below
        }
        Plan p = make_plan(sc, ntok, 1, aligned(Wc, 16));
        GemvArgs a = {};
        a.W0 = a.W1 = Wc;
        a.rows = sc.rows;
        a.x = x;
        a.x_stride = cols;
        a.y = y + r0;
        a.y_stride = rows;
        a.ntok = ntok;
        a.ws = (uint8_t *)ws;
        a.ws_bytes = ws_bytes;
        rc = launch_gemv(sc, p, a, dim3(1, (ntok + p.nt - 1) / p.nt, 1), (hipStream_t)stream);
        if (rc) return rc;
    }
    return QG_OK;
}
}  // namespace

extern "C" {

int qg_gemv(int type, const void *W, const float *x, float *y, int64_t rows, int64_t cols, int ntok, void *stream) {
    return gemv_entry(type, W, x, y, rows, cols, ntok, QG_MAX_TOKENS, nullptr, 0, stream);
}

size_t qg_gemm_workspace_size(int type, int64_t rows, int64_t cols, int ntok) {
    if (rows <= 0 || cols <= 0 || ntok < 1 || ntok > QG_MAX_PREFILL) return 0;
    return gemm_call_scratch_bytes(type, rows, cols, ntok);
}

int qg_gemm(int type, const void *W, const float *x, float *y, int64_t rows, int64_t cols, int ntok, void *workspace,
            size_t workspace_bytes, void *stream) {
    return gemv_entry(type, W, x, y, rows, cols, ntok, QG_MAX_PREFILL, workspace, workspace_bytes, stream);
}

int qg_gemv_plan(int type, int64_t rows, int64_t cols, int ntok, int w_aligned16, int query_device, int32_t *out) {
    if (!out) return QG_EINVAL;
    const bool planes = type == QG_Q6_K_PLANES;
    Shape s;
    int rc = make_shape(planes ? QG_Q6_K : type == QG_Q8_0_PLANES ? QG_Q8_0 : type, rows, cols, s);
    if (rc) return rc;
    if (type == QG_Q8_0_PLANES) {
        if (ntok < 1 || ntok > QG_MAX_TOKENS) return QG_ELIMIT;
        if (ntok != 1 || !w_aligned16) return QG_EINVAL;
        int g = 0, nw = 0;
        size_t lds = 0;
        rc = q8p_plan(rows, cols, false, query_device != 0, &g, &lds, &nw);
        if (rc) return rc;
        for (int i = 0; i < 8; i++) out[i] = 0;
        out[0] = 5;
        out[1] = 64;
        out[2] = 1;
        out[3] = (int32_t)((rows + nw - 1) / nw);
        out[4] = query_device ? g : 0;
        out[5] = (int32_t)lds;
        out[6] = Q8P_NF;
        out[7] = nw;
        return QG_OK;
    }
    if (planes) {
        if (ntok < 1 || ntok > QG_MAX_TOKENS) return QG_ELIMIT;
        if (ntok != 1 || !w_aligned16) return QG_EINVAL;
        if (rows * s.nb * s.ti.bytes > MAX_RANGE) return QG_ELIMIT;
    }
    if (ntok < 1 || ntok > QG_MAX_TOKENS) return QG_ELIMIT;
    // the first launch of the call (rows in launches of at most MAX_RANGE bytes)
    const int64_t chunk = MAX_RANGE / s.row_bytes;
    if (s.rows > chunk) s.rows = chunk;
    for (int i = 0; i < 8; i++) out[i] = 0;
    if (ntok == 1 && (type == QG_Q4_K || type == QG_Q6_K || planes)) {
        int L = 0, nw = 0, g = 0;
        size_t lds = 0;
        // (a W at the given alignment and an aligned x stand in for the call's)
        const void *Wq = (const void *)(uintptr_t)(w_aligned16 ? 0x10000 : 0x10002);
        rc = kq1_plan(type, s.rows, s.cols, Wq, (const float *)(uintptr_t)0x10000, query_device != 0, &L, &nw, &g,
                      &lds);
        if (rc == QG_OK) {
            out[0] = 4;
            out[1] = L;
            out[2] = 1;
            out[3] = g;
            out[4] = query_device ? g : 0;
            out[5] = (int32_t)lds;
            out[6] = type == QG_Q4_K ? KQ4<true>::NF : planes ? KQ6P::NF : KQ6::NF;
            out[7] = nw;
            return QG_OK;
        }
        if (rc != QG_EINVAL || planes) return rc;
    }
    const Plan p = make_plan(s, ntok, 1, w_aligned16 != 0);
    out[0] = p.kind;
    out[2] = p.nt;
    if (p.kind == UK_MFMA) {
        const int groups = small_groups(s.rows, 0, 1);
        out[3] = (int32_t)((s.rows + 16 * groups - 1) / (16 * groups));
        if (query_device) {
            const int64_t cap = resident_wgs(gemv_kernel_mfma(type, groups), 0);
            out[4] = (int32_t)(out[3] < cap ? out[3] : cap);
        }
        return QG_OK;
    }
    out[1] = p.lpr;
    out[3] = p.ntiles;
    if (query_device) {
        gemv_fn f = pick(type, p, false);
        if (p.lds > 64 * 1024 &&
            hipFuncSetAttribute((const void *)f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds) != hipSuccess)
            return QG_EHIP;
        out[4] = grid_for(p, f);
    }
    out[5] = (int32_t)p.lds;
    out[6] = p.depth;
    out[7] = p.xchunk;
    return QG_OK;
}

int qg_dequant(int type, const void *W, float *out, int64_t rows, int64_t cols, void *stream) {
    Shape s;
    if (type == QG_Q6_K_PLANES) {
        const int rc = make_shape(QG_Q6_K, rows, cols, s);
        if (rc) return rc;
        if (!W || !out || !aligned(W, 16) || !aligned(out, 4)) return QG_EINVAL;
        return launch_q6k_planes_dequant((const uint8_t *)W, out, rows * s.nb, (hipStream_t)stream);
    }
    if (type == QG_Q8_0_PLANES) {
        const int rc = make_shape(QG_Q8_0, rows, cols, s);
        if (rc) return rc;
        if (!W || !out || !aligned(W, 16) || !aligned(out, 4)) return QG_EINVAL;
        return launch_q8_planes_dequant((const uint8_t *)W, out, rows * s.nb, (hipStream_t)stream);
    }
    int rc = make_shape(type, rows, cols, s);
    if (rc) return rc;
    if (!W || !out || !aligned(W, 2) || !aligned(out, 4)) return QG_EINVAL;
    const int64_t blocks = rows * s.nb;
    dim3 grid((unsigned)((blocks + 255) / 256));
    hipLaunchKernelGGL(dequant_kernel(type), grid, dim3(256), 0, (hipStream_t)stream, (const uint8_t *)W, out, rows,
                       s.cols, s.row_bytes);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_EHIP;
}

int qg_router_topk(const float *logits, int n_experts, int k, int ntok, int32_t *ids, float *weights, void *stream) {
    if (n_experts < 1 || n_experts > QG_MAX_EXPERTS || k < 1 || k > QG_MAX_TOPK || k > n_experts ||
        ntok < 1 || ntok > QG_MAX_TOKENS)
        return QG_ELIMIT;
    if (!logits || !ids || !weights || !aligned(logits, 4) || !aligned(ids, 4) || !aligned(weights, 4))
        return QG_EINVAL;
    hipLaunchKernelGGL(route_kernel(n_experts), dim3(1), dim3(64 * ntok), 0, (hipStream_t)stream, logits, n_experts, k, ntok,
                       (const int32_t *)nullptr, 1, ids, weights, (int32_t *)nullptr, ids, weights,
                       (int32_t *)nullptr, (int32_t *)nullptr, 0, (int32_t *)nullptr, 0, (int32_t *)nullptr,
                       (const float *)nullptr, (int32_t *)nullptr, (float *)nullptr);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_EHIP;
}

// Workspace of qg_mlp: gu [ntok][2ff] f32 at offset 0, then act [ntok][ff],
// then the partial sums of split prefill launches (gate||up, then down).
namespace {
size_t mlp_scratch_bytes(int type, int64_t hidden, int64_t ff, int ntok) {
    const size_t a = gemm_scratch_bytes(type, ff, hidden, ntok, 1), b = gemm_scratch_bytes(type, hidden, ff, ntok, 0);
    return a > b ? a : b;
}
}  // namespace

size_t qg_mlp_workspace_size(int type, int64_t hidden, int64_t ff, int ntok) {
    if (hidden <= 0 || ff <= 0 || ntok < 1 || ntok > QG_MAX_PREFILL) return 0;
    if (type == QG_Q8_0_PLANES) type = QG_Q8_0;   // (one token: gu and act only)
    return align256((size_t)ntok * 2 * (size_t)ff * sizeof(float)) + align256((size_t)ntok * (size_t)ff * sizeof(float)) +
           mlp_scratch_bytes(type, hidden, ff, ntok);
}

}  // extern "C"

namespace {
// qg_mlp's argument checks (nothing enqueued)
int mlp_check(int type, int act, const void *W_gate, const void *W_up, const void *W_down, int64_t hidden,
              int64_t ff, const float *x, const float *y, int ntok, const void *workspace, size_t workspace_bytes) {
    Shape s_g, s_dn;
    int rc = make_shape(type, ff, hidden, s_g);
    if (rc) return rc;
    rc = make_shape(type, hidden, ff, s_dn);
    if (rc) return rc;
    if (ntok < 1 || ntok > QG_MAX_PREFILL) return QG_ELIMIT;
    if (act != QG_ACT_SILU && act != QG_ACT_GELU_TANH) return QG_EINVAL;
    if (!W_gate || !W_up || !W_down || !x || !y || !workspace) return QG_EINVAL;
    if (!aligned(W_gate, 2) || !aligned(W_up, 2) || !aligned(W_down, 2) || !aligned(x, 4) || !aligned(y, 4) ||
        !aligned(workspace, 256))
        return QG_EINVAL;
    if (workspace_bytes < qg_mlp_workspace_size(type, hidden, ff, ntok)) return QG_EINVAL;
    return QG_OK;
}
// One token through a gated MLP whose three tensors are Q8_0 planes: the
// gated plane launch (gate and up rows, act(g) * u, g and u in gu), then the
// plane GEMV of down on the activations
int q8_planes_mlp(int act, const void *W_gate, const void *W_up, const void *W_down, int64_t hidden, int64_t ff,
                  const float *x, float *y, int ntok, void *workspace, size_t workspace_bytes, void *stream) {
    Shape s_g, s_dn;
    int rc = make_shape(QG_Q8_0, ff, hidden, s_g);
    if (rc) return rc;
    rc = make_shape(QG_Q8_0, hidden, ff, s_dn);
    if (rc) return rc;
    if (ntok < 1 || ntok > QG_MAX_PREFILL) return QG_ELIMIT;
    if (ntok != 1 || (act != QG_ACT_SILU && act != QG_ACT_GELU_TANH)) return QG_EINVAL;
    if (hidden > Q8P_MAX_COLS || ff > Q8P_MAX_COLS) return QG_EINVAL;
    if (ff * hidden >= MAX_RANGE) return QG_ELIMIT;
    if (!W_gate || !W_up || !W_down || !x || !y || !workspace || !aligned(W_gate, 16) || !aligned(W_up, 16) ||
        !aligned(W_down, 16) || !aligned(x, 16) || !aligned(y, 4) || !aligned(workspace, 256))
        return QG_EINVAL;
    if (workspace_bytes < qg_mlp_workspace_size(QG_Q8_0_PLANES, hidden, ff, 1)) return QG_EINVAL;
    hipStream_t st = (hipStream_t)stream;
    float *gu = (float *)workspace;
    float *av = (float *)((uint8_t *)workspace + align256((size_t)2 * (size_t)ff * sizeof(float)));
    Q8pArgs g = {};
    g.C = (const uint8_t *)W_gate;
    g.D = (const uint8_t *)W_gate + ff * hidden;
    g.C2 = (const uint8_t *)W_up;
    g.D2 = (const uint8_t *)W_up + ff * hidden;
    g.rows = ff;
    g.cols = (int)hidden;
    g.x = x;
    g.y = av;
    g.y2 = gu;
    g.glu = act == QG_ACT_GELU_TANH ? XM_GELU : XM_SILU;
    rc = launch_q8p1(g, true, st);
    if (rc) return rc;
    Q8pArgs d = {};
    d.C = (const uint8_t *)W_down;
    d.D = (const uint8_t *)W_down + hidden * ff;
    d.rows = hidden;
    d.cols = (int)ff;
    d.x = av;
    d.y = y;
    return launch_q8p1(d, false, st);
}
}  // namespace

extern "C" {

int qg_mlp(int type, int act, const void *W_gate, const void *W_up, const void *W_down, int64_t hidden, int64_t ff,
           const float *x, float *y, int ntok, void *workspace, size_t workspace_bytes, void *stream) {
    if (type == QG_Q8_0_PLANES)
        return q8_planes_mlp(act, W_gate, W_up, W_down, hidden, ff, x, y, ntok, workspace, workspace_bytes, stream);
    int rc = mlp_check(type, act, W_gate, W_up, W_down, hidden, ff, x, y, ntok, workspace, workspace_bytes);
    if (rc) return rc;
    Shape s_g, s_dn;
    make_shape(type, ff, hidden, s_g);
    make_shape(type, hidden, ff, s_dn);
    hipStream_t st = (hipStream_t)stream;
    float *gu = (float *)workspace;
    float *av = (float *)((uint8_t *)workspace + align256((size_t)ntok * 2 * (size_t)ff * sizeof(float)));
    uint8_t *scratch = (uint8_t *)av + align256((size_t)ntok * (size_t)ff * sizeof(float));
    const size_t scratch_bytes = mlp_scratch_bytes(type, hidden, ff, ntok);
    // gate and up rows together: act(gate) * up per row, raw gate / up kept in gu
    Plan p1 = make_plan(s_g, ntok, 1, aligned(W_gate, 16) && aligned(W_up, 16));
    GemvArgs a = {};
    a.W0 = (const uint8_t *)W_gate;
    a.W1 = (const uint8_t *)W_up;
    a.rows = ff;
    a.x = x;
    a.x_stride = hidden;
    a.y = av;
    a.y_stride = ff;
    a.glu = act == QG_ACT_GELU_TANH ? XM_GELU : XM_SILU;
    a.y2 = gu;
    a.y2_stride = 2 * ff;
    a.ntok = ntok;
    a.ws = scratch;
    a.ws_bytes = scratch_bytes;
    rc = launch_gemv(s_g, p1, a, dim3(1, (ntok + p1.nt - 1) / p1.nt, 1), st);
    if (rc) return rc;
    // down on the activations
    Plan p2 = make_plan(s_dn, ntok, 1, aligned(W_down, 16));
    GemvArgs b = {};
    b.W0 = b.W1 = (const uint8_t *)W_down;
    b.rows = hidden;
    b.x = av;
    b.x_stride = ff;
    b.y = y;
    b.y_stride = hidden;
    b.ntok = ntok;
    b.ws = scratch;
    b.ws_bytes = scratch_bytes;
    return launch_gemv(s_dn, p2, b, dim3(1, (ntok + p2.nt - 1) / p2.nt, 1), st);
}

// Workspace layout for qg_moe_ffn (each part 256-byte aligned, in order):
//   gu [T*k][2F] f32 | act [T*k][F] f32 | dn [T*k][H] f32 | ids [T*k] i32 |
//   w [T*k] f32 | valid [T] i32 | group table (1 + min(E, T*k) * GREC) i32 |
//   set lists | each pair's pool slot [T*k] i32 and down scale [T*k] f32
namespace {
struct MoeWs {
    size_t gu, act, dn, ids, w, valid, grp, sets, pslot, pes, total;
};
MoeWs moe_ws(int64_t H, int64_t F, int E, int k, int T) {
    MoeWs o;
    size_t off = 0;
    const size_t pairs = (size_t)T * k;
    const size_t groups = pairs < (size_t)E ? pairs : (size_t)E;
    o.gu = off; off += align256(pairs * 2 * (size_t)F * 4);
    o.act = off; off += align256(pairs * (size_t)F * 4);
    o.dn = off; off += align256(pairs * (size_t)H * 4);
    o.ids = off; off += align256(pairs * 4);
    o.w = off; off += align256(pairs * 4);
    o.valid = off; off += align256((size_t)T * 4);
    o.grp = off; off += align256((1 + groups * GREC) * 4);
    o.sets = off; off += align256(2 * (size_t)set_list_ints((int)pairs) * 4);   // gate-up and down lists
    o.pslot = off; off += align256(pairs * 4);
    o.pes = off; off += align256(pairs * 4);
    o.total = off;
    return o;
}
}  // namespace

size_t qg_moe_workspace_size(const qg_moe *m, int topk, int ntok) {
    if (!m || m->hidden <= 0 || m->ff <= 0 || m->n_experts < 1 || topk < 1 || ntok < 1 || ntok > QG_MAX_TOKENS)
        return 0;
    return moe_ws(m->hidden, m->ff, m->n_experts, topk, ntok).total;
}

}  // extern "C"

namespace {
// Validation, routing, and the two grouped expert launches of a MoE step.  On
// success dn holds the weighted terms (dn_j s_j) c_j as [ntok][topk][H] and
// valid the per-token validity, both inside the workspace.
// Row groups that ride after the routed ones in a one-token gated launch,
// each of a routed expert's shape (F gate rows and the same up rows): a
// shared expert (one group), or the F-row slices of a dense MLP's gate / up
// matrices (n groups, slice i at byte i * step).  Their input x, their
// act(g) * u rows into act (slice i at act + i F) and raw sums into gu
// (gate slice i at gu + i F, up slice i at gu + up_off + i F).
struct ExtraGroups {
    const void *gate, *up;
    int64_t step, up_off;
    int n;
    const float *x;
    float *act, *gu;
    // a shared expert's gate logit (gate_inp . x), reduced in the routing
    // launch into gate_out[0] when both are set
    const float *gate_inp;
    float *gate_out;
};

int moe_routed(const qg_moe *m, const float *router_logits, int topk, const int32_t *expert_slots, const float *x,
               const float *y, int ntok, int32_t *ids_out, float *w_out, int32_t *status, void *workspace,
               size_t workspace_bytes, size_t ws_extra, hipStream_t st, float **dn_out, int32_t **valid_out,
               bool down = true, const ExtraGroups *xg = nullptr, bool *xg_done = nullptr) {
    if (!m) return QG_EINVAL;
    const int E = m->n_experts;
    if (E < 1 || E > QG_MAX_EXPERTS || topk < 1 || topk > QG_MAX_TOPK || topk > E || ntok < 1 ||
        ntok > QG_MAX_TOKENS)
        return QG_ELIMIT;
    if (m->act != QG_ACT_SILU && m->act != QG_ACT_GELU_TANH) return QG_EINVAL;
    Shape s_g, s_dn;
    int rc = make_shape(m->type, m->ff, m->hidden, s_g);
    if (rc) return rc;
    rc = make_shape(m->type, m->hidden, m->ff, s_dn);
    if (rc) return rc;
    if (!m->gate_up || !m->down || !router_logits || !expert_slots || !x || !y || !status || !workspace)
        return QG_EINVAL;
    if (m->gate_up_stride < 2 * s_g.rows * s_g.row_bytes || m->down_stride < s_dn.rows * s_dn.row_bytes)
        return QG_EINVAL;
    if (!aligned(m->gate_up, 2) || !aligned(m->down, 2) || (m->gate_up_stride & 1) || (m->down_stride & 1) ||
        !aligned(router_logits, 4) || !aligned(expert_slots, 4) || !aligned(x, 4) || !aligned(y, 4) ||
        !aligned(status, 4) || !aligned(workspace, 256) || (m->down_scale && !aligned(m->down_scale, 4)))
        return QG_EINVAL;
    const int64_t H = m->hidden, F = m->ff;
    const MoeWs L = moe_ws(H, F, E, topk, ntok);
    if (workspace_bytes < L.total + ws_extra) return QG_EINVAL;
    uint8_t *ws = (uint8_t *)workspace;
    float *gu = (float *)(ws + L.gu);
    float *av = (float *)(ws + L.act);
    float *dn = (float *)(ws + L.dn);
    int32_t *rt_ids = (int32_t *)(ws + L.ids);
    float *rt_w = (float *)(ws + L.w);
    int32_t *rt_valid = (int32_t *)(ws + L.valid);
    int32_t *grp = (int32_t *)(ws + L.grp);

    const int n_slots = m->n_slots > 0 ? m->n_slots : E;
    const int pairs = ntok * topk;
    const int gmax = pairs < E ? pairs : E;
    // tokens per workgroup for a group: a group holds the pairs that picked one
    // expert, on average about ntok*topk/E of them, so chunks sized for the
    // typical group (a few tokens) keep workgroups from computing copies
    int gtok = (2 * ntok * topk + E - 1) / E;
    gtok = gtok < 1 ? 1 : (gtok > ntok ? ntok : gtok);
    const int busy = (pairs + gtok - 1) / gtok;   // about this many (group, chunk) sets carry work
    // (a group takes the MFMA kernel only when groups typically hold 4+ tokens:
    // smaller groups would leave most of its 16 token columns empty)
    // The gated launch on the vector kernels takes chunks of one token: its
    // sets then read an expert's rows once per token, close together in time
    // (the set list keeps a group's chunks adjacent), and each chunk's decode
    // serves one token with no idle token slot.  Measured at 128 experts,
    // top-8 (gate-up): Gemma-shaped 704 x 2816 Q4_0, 16 tokens 63.4 -> 59.5
    // us, 12 tokens 58.2 -> 49.9 us; Qwen3-shaped 768 x 2048 Q8_0, 16 tokens
    // 74.1 -> 65.0 us.  The down launch keeps the two-token chunks.
    const int gtok1 = gtok >= MFMA_MIN_TOK ? gtok : 1;
    const int busy1 = (pairs + gtok1 - 1) / gtok1;
    Plan p1 = make_plan(s_g, gtok1, busy1, aligned(m->gate_up, 16) && (m->gate_up_stride % 16) == 0, gtok1);
    Plan p2 = make_plan(s_dn, gtok, busy, aligned(m->down, 16) && (m->down_stride % 16) == 0, gtok);
    // one token on the LDS-staged kernel: the gated launch routes the token
    // itself
    const bool route_in = ntok == 1 && topk <= ROUTE1_MAXK && lds_kind(p1.kind) && p1.nt == 1 && p1.xchunk == 0;
    // the (group, chunk) sets of each launch, listed by the routing launch:
    // workgroup y takes set y, so only the last few (past the count) are empty
    const int ca = p1.kind == UK_MFMA ? 16 : p1.nt, cb = p2.kind == UK_MFMA ? 16 : p2.nt;
    int32_t *sets_a = route_in ? nullptr : (int32_t *)(ws + L.sets);
    int32_t *sets_b = route_in ? nullptr : sets_a + set_list_ints(pairs);
    auto set_grid = [&](int c, const int32_t *sets) {
        if (!sets) return dim3(1, gmax, (ntok + c - 1) / c);
        const int64_t most = (int64_t)gmax * ((ntok + c - 1) / c);
        return dim3(1, (unsigned)(most < pairs ? most : pairs), 1);
    };

    // 1. route: top-k, weights, slot lookup, grouping by expert
    if (!route_in) {
        const int nthreads = 64 * ntok < 256 ? 256 : 64 * ntok;
        hipLaunchKernelGGL(route_kernel(E), dim3(1), dim3(nthreads), 0, st, router_logits, E, topk, ntok, expert_slots,
                           n_slots, ids_out, w_out, status, rt_ids, rt_w, rt_valid, grp, ca, sets_a, cb, sets_b,
                           m->down_scale, (int32_t *)(ws + L.pslot), (float *)(ws + L.pes));
        if (hipGetLastError() != hipSuccess) return QG_EHIP;
    }

    // 2. gate and up rows of every group's expert together: act(gate) * up per
    //    pair into act, raw gate / up into gu
    GemvArgs a = {};
    if (route_in) {
        a.r_logits = router_logits;
        a.r_E = E;
        a.r_k = topk;
        a.r_nslots = n_slots;
        a.r_slots = expert_slots;
        a.r_ids_out = ids_out;
        a.r_w_out = w_out;
        a.r_status = status;
        a.r_ids = rt_ids;
        a.r_w = rt_w;
        a.r_valid = rt_valid;
        a.r_grp = grp;
        a.r_escale = m->down_scale;
        a.r_pslot = (int32_t *)(ws + L.pslot);
        a.r_pes = (float *)(ws + L.pes);
    }
    a.W0 = a.W1 = (const uint8_t *)m->gate_up;
    a.rows = F;
    a.slot_stride = m->gate_up_stride;
    a.x = x;
    a.x_stride = H;
    a.y = av;
    a.y_stride = F;
    a.glu = m->act == QG_ACT_GELU_TANH ? XM_GELU : XM_SILU;
    a.y2 = gu;
    a.y2_stride = 2 * F;
    a.grp = grp;
    a.sets = sets_a;
    a.in_by_pair = 0;
    dim3 grid_a = set_grid(ca, sets_a);
    // extra groups of the routed experts' shape ride along as groups k, k+1,
    // ... of the routing launch (the aligned-copy variant needs their ranges
    // aligned too)
    if (xg_done) *xg_done = false;
    if (route_in && xg && xg->n >= 1 &&
        (p1.kind != UK_LDS || (aligned(xg->gate, 16) && aligned(xg->up, 16) && xg->step % 16 == 0))) {
        a.xg_W0 = (const uint8_t *)xg->gate;
        a.xg_W1 = (const uint8_t *)xg->up;
        a.xg_step = xg->step;
        a.xg_up = xg->up_off;
        a.xg_x = xg->x;
        a.xg_y = xg->act;
        a.xg_y2 = xg->gu;
        a.xg_n = xg->n;
        a.r_gate_inp = xg->gate_inp;
        a.r_gate_out = xg->gate_inp ? xg->gate_out : nullptr;
        grid_a.y += xg->n;
        if (xg_done) *xg_done = true;
    }
    rc = launch_gemv(s_g, p1, a, grid_a, st);
    if (rc) return rc;
    *dn_out = dn;
    *valid_out = rt_valid;
    if (!down) return QG_OK;   // the caller runs the down projection itself

    // 3. down on each pair's activations
    GemvArgs b = {};
    b.W0 = b.W1 = (const uint8_t *)m->down;
    b.rows = s_dn.rows;
    b.slot_stride = m->down_stride;
    b.x = av;
    b.x_stride = F;
    b.y = dn;
    b.y_stride = H;
    b.grp = grp;
    b.sets = sets_b;
    b.in_by_pair = 1;
    b.escale = m->down_scale;   // (dn * s[e]) * c_z, the combine's terms
    b.pscale = rt_w;
    rc = launch_gemv(s_dn, p2, b, set_grid(cb, sets_b), st);
    if (rc) return rc;
    *dn_out = dn;
    *valid_out = rt_valid;
    return QG_OK;
}

// Workspace of a shared expert after the routed part's: gu [ntok][2 SF],
// act [ntok][SF] and the scratch of its qg_mlp call (qg_mlp's layout), then
// sh [ntok][H], each 256-byte aligned.
struct SharedWs {
    size_t gu, act, sh, glog, total;
};
// the one-token down launch's arguments for a pool, its workspace and output
Moe1Args down1_args(const qg_moe *m, int topk, void *workspace, float *y) {
    const MoeWs L = moe_ws(m->hidden, m->ff, m->n_experts, topk, 1);
    uint8_t *ws = (uint8_t *)workspace;
    Moe1Args b = {};
    b.W = (const uint8_t *)m->down;
    b.stride = m->down_stride;
    b.rows = m->hidden;
    b.row_bytes = m->ff / 32 * qg_block_bytes(m->type);
    b.nb = (int)(m->ff / 32);
    b.act = (const float *)(ws + L.act);
    b.act_stride = m->ff;
    b.w = (const float *)(ws + L.w);
    b.pslot = (const int32_t *)(ws + L.pslot);
    b.pes = (const float *)(ws + L.pes);
    b.n_slots = m->n_slots > 0 ? m->n_slots : m->n_experts;
    b.valid = (const int32_t *)(ws + L.valid);
    b.dn = (float *)(ws + L.dn);
    b.y = y;
    b.k = topk;
    return b;
}

SharedWs shared_ws(int type, int64_t H, int64_t SF, int ntok) {
    SharedWs o;
    o.gu = 0;
    o.act = align256((size_t)ntok * 2 * (size_t)SF * 4);
    o.glog = o.act + align256((size_t)ntok * (size_t)SF * 4) + mlp_scratch_bytes(type, H, SF, ntok);
    o.sh = o.glog + 256;   // after the gate logit (one token), the output sh last
    o.total = o.sh + align256((size_t)ntok * (size_t)H * 4);
    return o;
}
}  // namespace

extern "C" {

int qg_moe_ffn(const qg_moe *m, const float *router_logits, int topk, const int32_t *expert_slots, const float *x,
               float *y, int ntok, int32_t *ids_out, float *w_out, int32_t *status, void *workspace,
               size_t workspace_bytes, void *stream) {
    hipStream_t st = (hipStream_t)stream;
    float *dn = nullptr;
    int32_t *valid = nullptr;
    // one token: the down projection of every pick and the combine in one
    // launch
    const bool one = m && ntok == 1 && moe_down1_fits(m->type, m->ff, topk);
    int rc = moe_routed(m, router_logits, topk, expert_slots, x, y, ntok, ids_out, w_out, status, workspace,
                        workspace_bytes, 0, st, &dn, &valid, !one);
    if (rc) return rc;
    if (one) return launch_moe_down1(m->type, down1_args(m, topk, workspace, y), st);
    // weighted combine in pick order
    hipLaunchKernelGGL(k_combine, dim3((unsigned)((m->hidden + 255) / 256), ntok), dim3(256), 0, st, dn, valid, y,
                       m->hidden, topk);
    return hipGetLastError() == hipSuccess ? QG_OK : QG_EHIP;
}

}  // extern "C"

// ------------------------------------------------ allocation-free variant --
// qg_moe_ffn_noalloc's scratch: a file-scope device array, one copy per GPU
// the library runs on, held until the process ends.  Host code never passes
// the array's name to a kernel (on the host it is only a stand-in): the
// device address comes from hipGetSymbolAddress, taken once per device with
// that device current, and kept below.
static __device__ __align__(256) uint8_t scratch[QG_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex noalloc_mu;
void *noalloc_ptr[NOALLOC_MAX_DEVICES];

// the current device's copy of `scratch` (looked up on its first use)
int noalloc_scratch(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEVICES) return QG_EHIP;
    std::lock_guard<std::mutex> lock(noalloc_mu);
    if (!noalloc_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QG_EHIP;
        noalloc_ptr[dev] = p;
    }
    *out = noalloc_ptr[dev];
    return QG_OK;
}
}  // namespace

extern "C" {

int qg_moe_ffn_noalloc(const qg_moe *m, const float *router_logits, int topk, const int32_t *expert_slots,
                       const float *x, float *y, int ntok, int32_t *ids_out, float *w_out, int32_t *status,
                       void *stream) {
    if (!m) return QG_EINVAL;
    if (ntok < 1 || ntok > QG_MAX_TOKENS || topk < 1 || topk > QG_MAX_TOPK || m->n_experts > QG_MAX_EXPERTS)
        return QG_ELIMIT;
    const size_t need = qg_moe_workspace_size(m, topk, ntok);
    if (!need) return QG_EINVAL;
    if (need > QG_NOALLOC_SCRATCH_BYTES) return QG_ELIMIT;
    void *ws = nullptr;
    const int rc = noalloc_scratch(&ws);
    if (rc) return rc;
    return qg_moe_ffn(m, router_logits, topk, expert_slots, x, y, ntok, ids_out, w_out, status, ws,
                      QG_NOALLOC_SCRATCH_BYTES, stream);
}

size_t qg_moe_shared_workspace_size(const qg_moe *m, const qg_shared_expert *sh, int topk, int ntok) {
    const size_t a = qg_moe_workspace_size(m, topk, ntok);
    if (!a || !sh || sh->ff <= 0) return 0;
    return a + shared_ws(sh->type, m->hidden, sh->ff, ntok).total;
}

int qg_moe_ffn_shared(const qg_moe *m, const qg_shared_expert *sh, const float *router_logits, int topk,
                      const int32_t *expert_slots, const float *x, float *resid, int ntok, int32_t *ids_out,
                      float *w_out, int32_t *status, void *workspace, size_t workspace_bytes, void *stream) {
    if (!m || !sh) return QG_EINVAL;
    if (!sh->gate || !sh->up || !sh->down || !sh->gate_inp || !aligned(sh->gate_inp, 4) || sh->ff <= 0)
        return QG_EINVAL;
    {   // the shared expert's shapes, checked before anything is enqueued
        Shape a, b;
        int rc = make_shape(sh->type, sh->ff, m->hidden, a);
        if (!rc) rc = make_shape(sh->type, m->hidden, sh->ff, b);
        if (rc) return rc;
        if (!aligned(sh->gate, 2) || !aligned(sh->up, 2) || !aligned(sh->down, 2)) return QG_EINVAL;
    }
    hipStream_t st = (hipStream_t)stream;
    const size_t base = qg_moe_workspace_size(m, topk, ntok);
    if (!base) return ntok < 1 || ntok > QG_MAX_TOKENS ? QG_ELIMIT : QG_EINVAL;
    const SharedWs S = shared_ws(sh->type, m->hidden, sh->ff, ntok);
    float *dn = nullptr;
    int32_t *valid = nullptr;
    uint8_t *ws = (uint8_t *)workspace + base;
    // One token with a shared expert of the routed experts' shape: its gate
    // and up rows ride in the routing launch, its down row and the whole
    // combine in the one-token down launch (two launches in all).
    const bool one = ntok == 1 && sh->type == m->type && sh->ff == m->ff && moe_down1_fits(m->type, m->ff, topk);
    const ExtraGroups shg = {sh->gate, sh->up, 0, m->ff, 1, x, (float *)(ws + S.act), (float *)(ws + S.gu),
                             sh->gate_inp, (float *)(ws + S.glog)};
    bool fused = false;
    int rc = moe_routed(m, router_logits, topk, expert_slots, x, resid, ntok, ids_out, w_out, status, workspace,
                        workspace_bytes, S.total, st, &dn, &valid, !one, one ? &shg : nullptr, &fused);
    if (rc) return rc;
    if (one) {
        Moe1Args b = down1_args(m, topk, workspace, nullptr);
        b.shW = (const uint8_t *)sh->down;
        b.sh_act = (const float *)(ws + S.act);
        b.gate_inp = sh->gate_inp;
        b.x = x;
        b.resid = resid;
        b.sh_out = (float *)(ws + S.sh);
        b.gate_logit = (const float *)(ws + S.glog);   // reduced by the routing launch
        if (fused) return launch_moe_down1(m->type, b, st);
        b.shW = nullptr;   // the routed terms only (no y); the shared expert below
        rc = launch_moe_down1(m->type, b, st);
        if (rc) return rc;
    }
    // the shared expert: a dense gated MLP on the same input, into the workspace
    rc = qg_mlp(sh->type, m->act, sh->gate, sh->up, sh->down, m->hidden, sh->ff, x, (float *)(ws + S.sh), ntok,
                ws + S.gu, S.glog - S.gu, stream);
    if (rc) return rc;
    // routed terms + gated shared output + residual
    return launch_combine_shared(dn, valid, (const float *)(ws + S.sh), sh->gate_inp, x, resid, m->hidden, topk,
                                 ntok, st);
}

size_t qg_moe_dense_workspace_size(const qg_moe *m, const qg_dense_mlp *d, int topk, int ntok) {
    const size_t a = qg_moe_workspace_size(m, topk, ntok);
    if (!a || !d || d->ff <= 0) return 0;
    const size_t b = qg_mlp_workspace_size(d->type, m->hidden, d->ff, ntok);
    return b ? a + b : 0;
}

int qg_moe_ffn_dense(const qg_moe *m, const qg_dense_mlp *d, const float *router_logits, int topk,
                     const int32_t *expert_slots, const float *x, float *y, const float *x_mlp, float *y_mlp,
                     int ntok, int32_t *ids_out, float *w_out, int32_t *status, void *workspace,
                     size_t workspace_bytes, void *stream) {
    if (!m || !d) return QG_EINVAL;
    hipStream_t st = (hipStream_t)stream;
    const size_t base = qg_moe_workspace_size(m, topk, ntok);
    if (!base) return ntok < 1 || ntok > QG_MAX_TOKENS || topk < 1 || topk > QG_MAX_TOPK ||
                          m->n_experts > QG_MAX_EXPERTS ? QG_ELIMIT : QG_EINVAL;
    if (!workspace || workspace_bytes < base) return QG_EINVAL;
    uint8_t *wsd = (uint8_t *)workspace + base;   // the MLP's part: qg_mlp's layout
    const size_t wsd_bytes = workspace_bytes - base;
    // the dense MLP's arguments, checked before anything is enqueued
    int rc = mlp_check(d->type, m->act, d->gate, d->up, d->down, m->hidden, d->ff, x_mlp, y_mlp, ntok, wsd,
                       wsd_bytes);
    if (rc) return rc;
    const int64_t H = m->hidden, F = m->ff, FD = d->ff;
    float *gu = (float *)wsd;
    float *av = (float *)(wsd + align256((size_t)ntok * 2 * (size_t)FD * 4));
    // One token, the MLP of the experts' block type and FD a multiple of F:
    // its gate / up rows as FD / F more groups of the experts' gated launch
    // and its down row as the extra pick of their down launch (two launches
    // in all).  Otherwise (or when the gated launch cannot take the groups)
    // the experts' launches, then qg_mlp's.
    const bool one = ntok == 1 && d->type == m->type && FD % F == 0 &&
                     moe_down1_fits_dense(m->type, F, FD, topk);
    if (!one) {
        rc = qg_moe_ffn(m, router_logits, topk, expert_slots, x, y, ntok, ids_out, w_out, status, workspace, base,
                        stream);
        if (rc) return rc;
        return qg_mlp(d->type, m->act, d->gate, d->up, d->down, H, FD, x_mlp, y_mlp, ntok, wsd, wsd_bytes, stream);
    }
    const int64_t rb = H / 32 * qg_block_bytes(m->type);   // a gate / up row's bytes
    const ExtraGroups xg = {d->gate, d->up, F * rb, FD, (int)(FD / F), x_mlp, av, gu, nullptr, nullptr};
    float *dn = nullptr;
    int32_t *valid = nullptr;
    bool taken = false;
    rc = moe_routed(m, router_logits, topk, expert_slots, x, y, ntok, ids_out, w_out, status, workspace, base, 0, st,
                    &dn, &valid, false, &xg, &taken);
    if (rc) return rc;
    Moe1Args b = down1_args(m, topk, workspace, y);
    if (!taken) {   // the experts' down launch, then the MLP on its own
        rc = launch_moe_down1(m->type, b, st);
        if (rc) return rc;
        return qg_mlp(d->type, m->act, d->gate, d->up, d->down, H, FD, x_mlp, y_mlp, ntok, wsd, wsd_bytes, stream);
    }
    b.dW = (const uint8_t *)d->down;
    b.d_row_bytes = FD / 32 * qg_block_bytes(d->type);
    b.d_nb = (int)(FD / 32);
    b.d_act = av;
    b.y_mlp = y_mlp;
    return launch_moe_down1(m->type, b, st);
}

int qg_rmsnorm(const float *x, const float *w, float *y, int64_t n, int ntok, float eps, float k, void *stream) {
    if (n <= 0 || ntok < 1 || !x || !w || !y || !aligned(x, 4) || !aligned(w, 4) || !aligned(y, 4))
        return QG_EINVAL;
    if (!(eps >= 0.0f)) return QG_EINVAL;
    return launch_rmsnorm(x, w, y, n, ntok, eps, k, (hipStream_t)stream);
}

int qg_rmsnorm_multi(const float *x, int64_t n, int ntok, float eps, int nout, const float *const *w,
                     const float *k, float *const *y, void *stream) {
    if (n <= 0 || ntok < 1 || !x || !aligned(x, 4) || !(eps >= 0.0f)) return QG_EINVAL;
    if (nout < 1 || nout > QG_MAX_NORMS) return QG_ELIMIT;
    if (!w || !k || !y) return QG_EINVAL;
    for (int j = 0; j < nout; j++)
        if (!w[j] || !y[j] || !aligned(w[j], 4) || !aligned(y[j], 4)) return QG_EINVAL;
    return launch_rmsnorm_multi(x, n, ntok, eps, nout, w, k, y, (hipStream_t)stream);
}

int qg_rmsnorm_router(const float *x, int64_t n, int ntok, float eps, const float *rw, float rk, const float *W,
                      int64_t rows, float *logits, int nout, const float *const *w, const float *k, float *const *y,
                      void *stream) {
    if (n <= 0 || rows <= 0 || !(eps >= 0.0f)) return QG_EINVAL;
    if (ntok < 1 || ntok > QG_MAX_TOKENS || nout < 0 || nout > QG_MAX_NORMS) return QG_ELIMIT;
    if (!x || !rw || !W || !logits || !aligned(x, 4) || !aligned(rw, 4) || !aligned(W, 4) || !aligned(logits, 4))
        return QG_EINVAL;
    if (nout > 0 && (!w || !k || !y)) return QG_EINVAL;
    for (int j = 0; j < nout; j++)
        if (!w[j] || !y[j] || !aligned(w[j], 4) || !aligned(y[j], 4)) return QG_EINVAL;
    return launch_norm_gemv_f32(x, n, ntok, eps, rw, rk, W, rows, logits, nout, w, k, y, (hipStream_t)stream);
}

int qg_post_ffn(const float *mlp, const float *moe, const float *w1, const float *w2, const float *w,
                const float *out_scale, float *x, int64_t n, int ntok, float eps, void *stream) {
    if (n <= 0 || ntok < 1 || !(eps >= 0.0f)) return QG_EINVAL;
    const float *ps[] = {mlp, moe, w1, w2, w, out_scale, x};
    for (const float *p : ps)
        if (!p || !aligned(p, 4)) return QG_EINVAL;
    return launch_post_ffn(mlp, moe, w1, w2, w, out_scale, x, n, ntok, eps, (hipStream_t)stream);
}

int qg_embed(int type, const void *W, int64_t rows, int64_t cols, const int32_t *tokens, int ntok, float scale,
             float *out, void *stream) {
    Shape s;
    const bool planes = type == QG_Q8_0_PLANES || type == QG_Q6_K_PLANES;
    int rc = make_shape(type == QG_Q8_0_PLANES ? QG_Q8_0 : type == QG_Q6_K_PLANES ? QG_Q6_K : type, rows, cols, s);
    if (rc) return rc;
    if (ntok < 1 || ntok > 65535) return QG_ELIMIT;
    if (!W || !tokens || !out || !aligned(W, planes ? 16 : 2) || !aligned(tokens, 4) || !aligned(out, 4))
        return QG_EINVAL;
    return launch_embed(type, (const uint8_t *)W, rows, (int)s.cols, s.row_bytes, tokens, ntok, scale, out,
                        (hipStream_t)stream);
}

size_t qg_argmax_workspace_size(int64_t n, int ntok) {
    if (n <= 0 || ntok < 1) return 0;
    const size_t parts = (size_t)ntok * argmax_parts(n);
    return align256(parts * 4) * 2;
}

int qg_argmax(float *logits, int64_t n, int ntok, float softcap, int32_t *idx, void *workspace,
              size_t workspace_bytes, void *stream) {
    if (n <= 0 || ntok < 1 || !(softcap >= 0.0f)) return QG_EINVAL;
    if (n > INT32_MAX || ntok > 65535) return QG_ELIMIT;
    if (!logits || !idx || !workspace || !aligned(logits, 4) || !aligned(idx, 4) || !aligned(workspace, 256))
        return QG_EINVAL;
    const size_t need = qg_argmax_workspace_size(n, ntok);
    if (workspace_bytes < need) return QG_EINVAL;
    float *pv = (float *)workspace;
    int32_t *pi = (int32_t *)((uint8_t *)workspace + need / 2);
    return launch_argmax(logits, n, ntok, softcap, pv, pi, idx, (hipStream_t)stream);
}

int qg_argmax_embed(float *logits, int64_t n, int ntok, float softcap, int32_t *idx, void *workspace,
                    size_t workspace_bytes, int type, const void *W, int64_t rows, int64_t cols, float scale,
                    float *out, void *stream) {
    if (n <= 0 || ntok < 1 || !(softcap >= 0.0f)) return QG_EINVAL;
    if (n > INT32_MAX || ntok > 65535) return QG_ELIMIT;
    if (!logits || !idx || !workspace || !aligned(logits, 4) || !aligned(idx, 4) || !aligned(workspace, 256))
        return QG_EINVAL;
    const size_t need = qg_argmax_workspace_size(n, ntok);
    if (workspace_bytes < need) return QG_EINVAL;
    Shape s;
    const bool planes = type == QG_Q8_0_PLANES || type == QG_Q6_K_PLANES;
    int rc = make_shape(type == QG_Q8_0_PLANES ? QG_Q8_0 : type == QG_Q6_K_PLANES ? QG_Q6_K : type, rows, cols, s);
    if (rc) return rc;
    if (!W || !out || !aligned(W, planes ? 16 : 2) || !aligned(out, 4)) return QG_EINVAL;
    float *pv = (float *)workspace;
    int32_t *pi = (int32_t *)((uint8_t *)workspace + need / 2);
    return launch_argmax_embed(logits, n, ntok, softcap, pv, pi, idx, type, (const uint8_t *)W, rows, (int)s.cols,
                               s.row_bytes, scale, out, (hipStream_t)stream);
}

}  // extern "C"

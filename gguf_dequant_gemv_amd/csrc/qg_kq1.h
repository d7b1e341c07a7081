// qg_kq1.h -- one token against Q4_K / Q6_K rows in 64-value units.
//
// The K-quant decode costs several vector instructions per weight, so a
// one-token GEMV over these rows is as much a matter of keeping every SIMD
// busy as of streaming HBM.  Whole 256-value blocks as the lanes' units leave
// too few waves (a row of 20 or 68 blocks spread over 4 or 8 lanes), so here
// a lane's unit is a quarter block: 64 values whose codes, scales and super
// scales it loads straight into registers:
//   Q4_K  quarter c of a block: the 16-byte head (d, dmin, the 12 bytes of
//         6-bit scales and mins) and qs bytes 32c .. 32c+31, whose low
//         nibbles are sub-block 2c and high nibbles sub-block 2c+1
//         ([ternary-bonsai] dequantQ4K / scaleMinK4 layout);
//   Q6_K  half n, lane half h of a block: ql bytes 64n+16h .. +15 and
//         64n+32+16h .. +15, qh bytes 32n+16h .. +15, scales 8n .. 8n+7 and
//         d: the 64 values 128n + 32p + 16h + i (p = 0..3, i < 16), one scale
//         group of 16 for each p ([ternary-bonsai] dequantQ6K layout).
// L lanes share a row (lane `sub` takes units sub, sub + L, ...), a wave
// holds 64/L rows, a workgroup NW waves.  x is staged once per workgroup in
// LDS (4 floats of padding after every 64 values, so the b128 reads of 8
// neighbouring lanes spread over the banks) with its sums over each scale
// group, which fold the Q4_K mins and the Q6_K offset of 32.  (Padding Q6_K's
// x per 128 values spreads its lanes wider but measured slower, as did a
// third Q6_K unit in flight.)
// NF units per lane are in flight: 1 for Q4_K and Q6_K planes, 2 for Q6_K
// blocks.  Each wave holds only a few units a lane, so with more in flight
// most of the matrix is requested at once and a wave's decode waits on
// whichever of its units the memory delivers last: one in flight measured
// 15.2 -> 13.0 us at Q4_K 17408 x 5120 and 19.3 -> 18.3 us on Q6_K planes
// 5120 x 17408 (3 to 5 in flight: 15.2 to 17.3 us); Q6_K blocks measured
// alike at 1 and 2.
#pragma once
#include "qg_device.h"

namespace qg {

struct Kq1Args {
    const uint8_t *W;   // row 0: 4-byte aligned (Q4_K) / 2-byte aligned (Q6_K)
    int64_t rows;
    u32 row_bytes;      // blocks per row * block bytes
    u32 range;          // bytes the descriptor covers (rows * row_bytes)
    int nu;             // 64-value units per row (cols / 64)
    int cols;
    const float *x;     // [cols], 16-byte aligned
    float *y;           // [rows]
    // Q6_K plane layout only (W: the ql plane, range: its bytes): the qh,
    // scales and d planes, each 16-byte aligned
    const uint8_t *Ph, *Ps, *Pd;
};

// a ? x : y for a per-lane condition, as bit masks (a conditional there
// would become a branch over the lanes, which the x reads are then hoisted
// above)
QG_DEV u32 kq1_sel(bool a, u32 x, u32 y) {
    const u32 m = 0u - (u32)a;
    return (x & m) | (y & ~m);
}

// A fence for the compiler only: no load moves across it and the sums
// passed through it are complete on its far side, at the IR level (an empty
// asm with a memory clobber that reads and writes them) and in the machine
// schedule; it emits nothing.  Placed between the steps of a unit's dot
// product, it keeps one step's x reads in flight at a time (with several
// waves per SIMD hiding LDS latency, reading further ahead only costs
// registers).
QG_DEV void kq1_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}
QG_DEV void kq1_fence(float (&s)[4]) {
    asm volatile("" : "+v"(s[0]), "+v"(s[1]), "+v"(s[2]), "+v"(s[3]) : : "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// x in LDS: 4 floats of padding after every PG values (PG = 64 or 128, the
// span whose offsets spread the lanes of a row over the banks)
template <int PG>
QG_DEV int kq1_xpos(int c) { return c + 4 * (c / PG); }
template <int PG>
__host__ __device__ inline int kq1_xstride(int cols) { return cols + 4 * (cols / PG) + 4; }

// x into LDS at kq1_xpos positions, with the sums of its groups of G
// values, in two steps: kq1_x_load puts this thread's share (XN float4, a
// compile-time bound on cols / 4 / NT) in registers, kq1_x_put stores it.
// The loads go out before the weight loads, so their wait does not include
// the weights' (loads retire in order).
// (every load is issued, past the end at the last float4: a load under a
// condition would be waited for inside its branch)
template <int NT, int XN>
QG_DEV void kq1_x_load(const float *x, int cols, f32x4 (&v)[XN]) {
    const int n4 = cols >> 2;   // a multiple of 64: a wave's lanes are all in range or all out
#pragma unroll
    for (int b = 0; b < XN; b++) v[b] = ((const f32x4 *)x)[min((int)threadIdx.x + b * NT, n4 - 1)];
}
template <int NT, int XN, int G, int PG>
QG_DEV void kq1_x_put(const f32x4 (&v)[XN], int cols, float *xs, float *ss) {
    const int n4 = cols >> 2;
#pragma unroll
    for (int b = 0; b < XN; b++) {
        const int i = (int)threadIdx.x + b * NT;
        if (i < n4) {
            *(f32x4 *)(xs + kq1_xpos<PG>(4 * i)) = v[b];
            const float g = group_sum<G / 4>((v[b].x + v[b].y) + (v[b].z + v[b].w));
            if ((i & (G / 4 - 1)) == 0) ss[(4 * i) / G] = g;
        }
    }
}

// The descriptor over a block stream W at byte phase ph0: the range rounded
// up to whole dwords (a realigned field's last dword may hold the tensor's
// last bytes, and a dword load reads 0 unless all of it is in range)
QG_DEV rsrc_t kq1_rsrc(const Kq1Args &a, u32 ph0) { return make_rsrc(a.W - ph0, (a.range + ph0 + 3u) & ~3u); }

// ---- Q4_K: quarter c (= unit & 3) of block unit >> 2 ----------------------
template <bool ALN>
struct KQ4 {
    // WAVES: waves per SIMD its registers leave room for (an estimate for
    // plans made without a device to ask)
    static constexpr int TYPE = T_Q4_K, BB = 144, G = 32, PG = 64, NF = 1, WAVES = 6;
    static constexpr int RAW = ALN ? 12 : 14;   // head, codes (+1 dword each when realigned)
    typedef rsrc_t R;
    QG_DEV static R rsrc(const Kq1Args &a, u32 ph0) { return kq1_rsrc(a, ph0); }
    QG_DEV static u32 row_base(const Kq1Args &a, int64_t rl, u32 ph0) { return ph0 + (u32)rl * a.row_bytes; }
    QG_DEV static void issue(rsrc_t r, u32 rowoff, int u, u32 (&t)[RAW]) {
        const u32 b = rowoff + (u32)(u >> 2) * BB;
        const u32 q = b + 16 + 32 * (u32)(u & 3);
        if constexpr (ALN) {
            ldn<4, 0>(r, b, t);
            ldn<8, 4>(r, q, t);
        } else {
            u32 h[5], c[9];
            raw_load<4>(r, b, h);
            raw_load<8>(r, q, c);
#pragma unroll
            for (int i = 0; i < 5; i++) t[i] = h[i];
#pragma unroll
            for (int i = 0; i < 9; i++) t[5 + i] = c[i];
        }
    }
    // sum over the unit's 64 values of value * x; xu: the unit's x (68u in
    // LDS), su: its two sub-block sums of x
    QG_DEV static float dot(const u32 (&t)[RAW], u32 ph, int c, const float *xu, const float *su) {
        u32 h[4], q[8];
        if constexpr (ALN) {
#pragma unroll
            for (int i = 0; i < 4; i++) h[i] = t[i];
#pragma unroll
            for (int i = 0; i < 8; i++) q[i] = t[4 + i];
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++) h[i] = __builtin_amdgcn_alignbyte(t[i + 1], t[i], ph);
#pragma unroll
            for (int i = 0; i < 8; i++) q[i] = __builtin_amdgcn_alignbyte(t[6 + i], t[5 + i], ph);
        }
        // sub-blocks 2c, 2c+1: 6-bit scale and min ([ternary-bonsai] scaleMinK4)
        const bool lo4 = c < 2;
        const u32 sc4 = kq1_sel(lo4, h[1] & 0x3F3F3F3Fu, (h[3] & 0x0F0F0F0Fu) | ((h[1] >> 2) & 0x30303030u));
        const u32 mn4 = kq1_sel(lo4, h[2] & 0x3F3F3F3Fu, ((h[3] >> 4) & 0x0F0F0F0Fu) | ((h[2] >> 2) & 0x30303030u));
        const u32 sh = 16u * (u32)(c & 1);
        const u32 sc = sc4 >> sh, mn = mn4 >> sh;
        const float d = h2f(h[0]), dm = h2f(h[0] >> 16);
        // (the high nibbles are summed in place: 16 times their codes)
        const float a0 = d * u8_of(sc, 0), a1 = (d * u8_of(sc, 1)) * 0.0625f;
        const float m0 = dm * u8_of(mn, 0), m1 = dm * u8_of(mn, 1);
        float sa[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // sub-block 2c (two chains), 2c+1 (two chains)
#pragma unroll
        for (int k = 0; k < 8; k++) {
            kq1_fence(sa);
            const u32 lo = opaque(q[k] & 0x0F0F0F0Fu), hi = opaque(q[k] & 0xF0F0F0F0u);
            const f32x4 xa = *(const f32x4 *)(xu + 4 * k);
            const f32x4 xb = *(const f32x4 *)(xu + 32 + 4 * k);
            float &s0 = sa[k & 1];
            float &s1 = sa[2 + (k & 1)];
            s0 = fmaf(u8_of(lo, 0), xa.x, s0);
            s0 = fmaf(u8_of(lo, 1), xa.y, s0);
            s0 = fmaf(u8_of(lo, 2), xa.z, s0);
            s0 = fmaf(u8_of(lo, 3), xa.w, s0);
            s1 = fmaf(u8_of(hi, 0), xb.x, s1);
            s1 = fmaf(u8_of(hi, 1), xb.y, s1);
            s1 = fmaf(u8_of(hi, 2), xb.z, s1);
            s1 = fmaf(u8_of(hi, 3), xb.w, s1);
        }
        kq1_fence(sa);
        const float s0 = sa[0] + sa[1], s1 = sa[2] + sa[3];
        return fmaf(a0, s0, -(m0 * su[0])) + fmaf(a1, s1, -(m1 * su[1]));
    }
};

// ---- Q6_K: half n = (unit >> 1) & 1, lane half h = unit & 1 of block unit >> 2
// The dot product of one unit from its fields in registers: A, B the two ql
// pieces (bytes 64n + 16h and 64n + 32 + 16h), H the qh piece (32n + 16h),
// S the 8 int8 scales of half n, d the super scale.  xs: x in LDS, v0: the
// row index of value 128n + 16h of the block (piece p: values v0 + 32p ..);
// sb: the block's 16 group sums of x.
// (v0 is 16h past a multiple of 128, so piece p's x sits a constant
// kq6_xoff<PG>(p) floats past v0's: one address per unit, the rest in the
// LDS reads' offsets)
template <int PG>
QG_DEV constexpr int kq6_xoff(int p) { return 32 * p + (PG == 64 ? 4 * (p >> 1) : 0); }
template <int PG>
QG_DEV float kq6_dot(const u32 (&A)[4], const u32 (&B)[4], const u32 (&H)[4], const u32 (&S)[2], float d, int h,
                     int n, const float *xs, int v0, const float *sb) {
    static_assert(PG == 64 || PG == 128, "kq6_dot: x padded per 64 or 128 values");
    const float *xb = xs + kq1_xpos<PG>(v0);
    // group 8n + 2p + h: int8 scale byte 2p + h of the half's scales, times d
    float dsc[4];
#pragma unroll
    for (int p = 0; p < 4; p++) dsc[p] = d * (float)(int8_t)(S[p >> 1] >> (8 * (2 * (p & 1) + h)));
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        kq1_fence(s);
        // codes of values 32p + 16h + 4i .. +3 of the half, p = 0..3: the
        // low / high nibbles of the two ql pieces, bit pairs p of qh
        u32 cd[4];
        cd[0] = opaque((A[i] & 0x0F0F0F0Fu) | ((H[i] << 4) & 0x30303030u));
        cd[1] = opaque((B[i] & 0x0F0F0F0Fu) | ((H[i] << 2) & 0x30303030u));
        cd[2] = opaque(((A[i] >> 4) & 0x0F0F0F0Fu) | (H[i] & 0x30303030u));
        cd[3] = opaque(((B[i] >> 4) & 0x0F0F0F0Fu) | ((H[i] >> 2) & 0x30303030u));
#pragma unroll
        for (int p = 0; p < 4; p++) {
            const f32x4 xv = *(const f32x4 *)(xb + kq6_xoff<PG>(p) + 4 * i);
            s[p] = fmaf(u8_of(cd[p], 0), xv.x, s[p]);
            s[p] = fmaf(u8_of(cd[p], 1), xv.y, s[p]);
            s[p] = fmaf(u8_of(cd[p], 2), xv.z, s[p]);
            s[p] = fmaf(u8_of(cd[p], 3), xv.w, s[p]);
        }
    }
    kq1_fence(s);
    // (q - 32) folded as sum(q x) - 32 sum(x)
    float acc = 0.0f;
#pragma unroll
    for (int p = 0; p < 4; p++) acc = fmaf(dsc[p], fmaf(-32.0f, sb[8 * n + 2 * p + h], s[p]), acc);
    return acc;
}

// GGUF blocks: every field of a block sits at the block's own 2-byte phase
// (the fields start at multiples of 4 within it), so one shift realigns
// them all.
struct KQ6 {
    static constexpr int TYPE = T_Q6_K, BB = 210, G = 16, PG = 64, NF = 2, WAVES = 5;
    static constexpr int RAW = 5 + 5 + 5 + 6;   // ql (two pieces), qh, scales + d: each +1 dword
    typedef rsrc_t R;
    QG_DEV static R rsrc(const Kq1Args &a, u32 ph0) { return kq1_rsrc(a, ph0); }
    QG_DEV static u32 row_base(const Kq1Args &a, int64_t rl, u32 ph0) { return ph0 + (u32)rl * a.row_bytes; }
    // the shift that realigns unit uc's fields
    QG_DEV static u32 phase(u32 rowoff, int uc) { return (rowoff + (u32)(uc >> 2) * BB) & 3u; }
    QG_DEV static void issue(const R &r, u32 rowoff, int u, u32 (&t)[RAW]) {
        const u32 b = rowoff + (u32)(u >> 2) * BB;
        const u32 n = (u32)(u >> 1) & 1u, h = (u32)u & 1u;
        u32 a[5], c[5], e[5], s[6];
        raw_load<4>(r, b + 64 * n + 16 * h, a);
        raw_load<4>(r, b + 64 * n + 32 + 16 * h, c);
        raw_load<4>(r, b + 128 + 32 * n + 16 * h, e);
        raw_load<5>(r, b + 192, s);   // scales[0..15], d
#pragma unroll
        for (int i = 0; i < 5; i++) { t[i] = a[i]; t[5 + i] = c[i]; t[10 + i] = e[i]; }
#pragma unroll
        for (int i = 0; i < 6; i++) t[15 + i] = s[i];
    }
    QG_DEV static float dot(const u32 (&t)[RAW], u32 ph, int n, int h, const float *xs, int v0, const float *sb) {
        u32 A[4], B[4], H[4], S[5];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            A[i] = __builtin_amdgcn_alignbyte(t[i + 1], t[i], ph);
            B[i] = __builtin_amdgcn_alignbyte(t[6 + i], t[5 + i], ph);
            H[i] = __builtin_amdgcn_alignbyte(t[11 + i], t[10 + i], ph);
        }
#pragma unroll
        for (int i = 0; i < 5; i++) S[i] = __builtin_amdgcn_alignbyte(t[16 + i], t[15 + i], ph);
        const u32 Sn[2] = {kq1_sel(n != 0, S[2], S[0]), kq1_sel(n != 0, S[3], S[1])};
        return kq6_dot<PG>(A, B, H, Sn, h2f(S[4]), h, n, xs, v0, sb);
    }
};

// The plane layout ([gemma4] q6kPlanes, d kept as f16): ql [nb][128], qh
// [nb][64], scales [nb][16] and d [nb] in planes of their own, each 16-byte
// aligned, so every field loads whole: the two ql pieces and the qh piece as
// 16 bytes, the half's scales as 8, d as its 2 bytes (a dword would reach
// past the last plane's end for an odd block count).  The 4 lanes of a
// block's units read 128 contiguous bytes of ql, 64 of qh.
struct KQ6P {
    static constexpr int TYPE = T_Q6_KP, BB = 210, G = 16, PG = 64, NF = 1, WAVES = 5;
    static constexpr int RAW = 4 + 4 + 4 + 2 + 1;
    struct R { rsrc_t q, h, s, d; };
    QG_DEV static R rsrc(const Kq1Args &a, u32) {
        const u32 nblk = a.range / 128u;
        return {make_rsrc(a.W, a.range), make_rsrc(a.Ph, 64u * nblk), make_rsrc(a.Ps, 16u * nblk),
                make_rsrc(a.Pd, 2u * nblk)};
    }
    // the index of the row's first block
    QG_DEV static u32 row_base(const Kq1Args &a, int64_t rl, u32) { return (u32)rl * (a.row_bytes / BB); }
    QG_DEV static u32 phase(u32, int) { return 0; }
    QG_DEV static void issue(const R &r, u32 rowoff, int u, u32 (&t)[RAW]) {
        const u32 bi = rowoff + (u32)(u >> 2);
        const u32 n = (u32)(u >> 1) & 1u, h = (u32)u & 1u;
        ldn<4, 0>(r.q, 128 * bi + 64 * n + 16 * h, t);
        ldn<4, 4>(r.q, 128 * bi + 64 * n + 32 + 16 * h, t);
        ldn<4, 8>(r.h, 64 * bi + 32 * n + 16 * h, t);
        ldn<2, 12>(r.s, 16 * bi + 8 * n, t);
        t[14] = __builtin_amdgcn_raw_buffer_load_b16(r.d, 2 * bi, 0, 0);
    }
    QG_DEV static float dot(const u32 (&t)[RAW], u32, int n, int h, const float *xs, int v0, const float *sb) {
        u32 A[4], B[4], H[4];
#pragma unroll
        for (int i = 0; i < 4; i++) { A[i] = t[i]; B[i] = t[4 + i]; H[i] = t[8 + i]; }
        const u32 Sn[2] = {t[12], t[13]};
        return kq6_dot<PG>(A, B, H, Sn, h2f(t[14]), h, n, xs, v0, sb);
    }
};

// ---- the kernel ------------------------------------------------------------
// Workgroup bx: rows (bx * NW + wave) * RPW + grp, RPW = 64 / L.  Lanes past
// the last row load the last row and store nothing; unit slots past the
// row's last unit load its last unit and add nothing.  XN: float4 of x per
// thread (cols <= XN * 4 * 64 * NW).
template <class U, int L, int NW, int XN>
__global__ __launch_bounds__(64 * NW) void k_kq1(Kq1Args a) {
    extern __shared__ float lds[];
    constexpr int RPW = 64 / L, NT = 64 * NW;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane / L, sub = lane % L;
    const int64_t r = ((int64_t)blockIdx.x * NW + wave) * RPW + grp;
    const int64_t rl = r < a.rows ? r : a.rows - 1;
    const int nu = a.nu;
    const int K = (nu + L - 1) / L;   // unit slots per lane
    const u32 ph0 = (u32)((uintptr_t)a.W & 3u);
    const typename U::R rs = U::rsrc(a, ph0);
    const u32 rowoff = U::row_base(a, rl, ph0);

    // x's loads, then U::NF units' loads in flight per lane (ring entry f
    // holds slots f, f + NF, ...), then x into LDS
    constexpr int NF = U::NF;
    f32x4 xv[XN];
    kq1_x_load<NT, XN>(a.x, a.cols, xv);
    kq1_fence();   // (kept ahead of the weight loads)
    u32 t[NF][U::RAW];
#pragma unroll
    for (int f = 0; f < NF; f++) U::issue(rs, rowoff, min(sub + f * L, nu - 1), t[f]);
    float *xs = lds;
    float *ss = lds + kq1_xstride<U::PG>(a.cols);
    kq1_x_put<NT, XN, U::G, U::PG>(xv, a.cols, xs, ss);
    __syncthreads();

    // slot k's unit: sub + k L (past the row's end: the last unit, not added)
    auto unit = [&](const u32 (&tu)[U::RAW], int k) {
        const int u = sub + k * L;
        const int uc = min(u, nu - 1);
        float v;
        kq1_fence();
        if constexpr (U::TYPE == T_Q4_K) {
            v = U::dot(tu, ph0, uc & 3, xs + kq1_xpos<U::PG>(64 * uc), ss + 2 * uc);
        } else {
            const u32 ph = U::phase(rowoff, uc);
            v = U::dot(tu, ph, (uc >> 1) & 1, uc & 1, xs, 64 * (uc & ~1) + 16 * (uc & 1), ss + 16 * (uc >> 2));
        }
        kq1_fence();
        return u < nu ? v : 0.0f;
    };
    float acc = 0.0f;
    kq1_fence();
#pragma unroll 1
    for (int k0 = 0; k0 < K; k0 += NF) {
#pragma unroll
        for (int f = 0; f < NF; f++) {
            const int k = k0 + f;
            if (k < K) {
                acc += unit(t[f], k);
                if (k + NF < K) U::issue(rs, rowoff, min(sub + (k + NF) * L, nu - 1), t[f]);
            }
        }
    }
    acc = group_sum<L>(acc);
    if (sub == 0 && r < a.rows) a.y[r] = acc;
}

// LDS bytes of k_kq1 for a row of `cols` values (x and its group sums)
// (from the same constants the kernel lays LDS out with)
template <class U>
inline size_t kq1_lds_bytes_of(int cols) {
    return ((size_t)kq1_xstride<U::PG>(cols) + (size_t)cols / U::G) * 4;
}
inline size_t kq1_lds_bytes(int type, int cols) {
    return type == T_Q4_K ? kq1_lds_bytes_of<KQ4<true>>(cols)
                          : type == T_Q6_KP ? kq1_lds_bytes_of<KQ6P>(cols) : kq1_lds_bytes_of<KQ6>(cols);
}

int kq1_plan(int type, int64_t rows, int64_t cols, const void *W, const float *x, bool query, int *lpr, int *nw,
             int *wgs, size_t *lds);
int launch_kq1(int type, const Kq1Args &a, hipStream_t st);

}  // namespace qg

// qg_device.h -- device helpers and the per-type block-unpack layer (gfx950).
//
// A "unit" is the piece of a weight row one lane loads and decodes at a time:
//   Q8_0  a pair of blocks  (64 values,  68 B)
//   Q4_0  a pair of blocks  (64 values,  36 B)
//   Q4_K  one block         (256 values, 144 B)
//   Q6_K  one block         (256 values, 210 B)
// Pairs make every unit start on a 4-byte boundary when the row does (34*2 and
// 18*2 are multiples of 4), so the lane's loads are plain dword-aligned buffer
// loads and every byte position inside the unit is a compile-time constant.
// Q6_K blocks alternate between 0 and 2 mod 4; they are loaded from the
// aligned-down address and re-aligned in registers with v_alignbyte.
//
// Each unit type exposes
//   code(w, i)   the integer code of value i as f32 (exact)
//   GROUPS/GSIZE the scale groups (values sharing one scale) in value order
//   fold(...)    a group's contribution from  sum(code * x)  and  sum(x)
//   value(w, i)  the dequantized f32 value (one rounding of the exact value)
// so the GEMV dot products and the dequantization kernel share one decoder.
// Block formulas: the ternary_bonsai_2_dflash.js page (dequantQ4K,
// dequantQ6K, scaleMinK4), the gemma4_moe_ssd.js page (Q4_0 plane comment,
// q4dot) and the qwen3_moe_ssd.js page (i8at, matmulQ8).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define QG_DEV __device__ __forceinline__

namespace qg {

typedef uint32_t u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x3 __attribute__((ext_vector_type(3)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

enum { T_Q4_0 = 2, T_Q8_0 = 8, T_Q4_K = 12, T_Q6_K = 14 };

// ---------------------------------------------------------------- scalars --
QG_DEV float h2f(u32 bits) {  // low 16 bits: IEEE binary16 -> f32 (exact)
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
}

// 16-bit field at byte `pos` (even) of a dword array.
QG_DEV u32 half_at(const u32 *w, int pos) { return (w[pos >> 2] >> (8 * (pos & 3))) & 0xFFFFu; }

// Signed / unsigned byte `pos` of a dword array as f32 (one v_cvt with a byte select).
QG_DEV float s8_at(const u32 *w, int pos) { return (float)(int8_t)(w[pos >> 2] >> (8 * (pos & 3))); }
QG_DEV float u8_of(u32 word, int b) { return (float)((word >> (8 * b)) & 0xFFu); }

// ------------------------------------------------------- buffer loads -----
// Raw buffer descriptor over [base, base + bytes): loads past the end read 0.
QG_DEV rsrc_t make_rsrc(const void *base, u32 bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// N consecutive dwords at byte offset `off` (4-aligned) into w[O .. O+N).
template <int N, int O = 0, int M>
QG_DEV void ldn(rsrc_t r, u32 off, u32 (&w)[M]) {
    static_assert(O + N <= M, "ldn: out of range");
#pragma unroll
    for (int i = 0; i + 4 <= N; i += 4) {
        u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 4 * i, 0, 0);
        w[O + i] = v.x; w[O + i + 1] = v.y; w[O + i + 2] = v.z; w[O + i + 3] = v.w;
    }
    constexpr int B = N & ~3, R = N & 3;
    if constexpr (R == 3) {
        u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, off + 4 * B, 0, 0);
        w[O + B] = v.x; w[O + B + 1] = v.y; w[O + B + 2] = v.z;
    } else if constexpr (R == 2) {
        u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off + 4 * B, 0, 0);
        w[O + B] = v.x; w[O + B + 1] = v.y;
    } else if constexpr (R == 1) {
        w[O + B] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * B, 0, 0);
    }
}

// ---------------------------------------------------------- cross-lane ----
template <int CTRL>
QG_DEV float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// All-reduce (sum) over aligned groups of G lanes; every lane of a group ends
// with the same value (each step adds a pair in both orders, and IEEE addition
// is commutative).
template <int G>
QG_DEV float group_sum(float v) {
    if constexpr (G >= 2) v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (G >= 4) v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (G >= 8) v += dpp_f<0x141>(v);   // row_half_mirror: quads of a half-row
    if constexpr (G >= 16) v += dpp_f<0x140>(v);  // row_mirror: halves of a row
    if constexpr (G >= 32) v += __shfl_xor(v, 16);
    if constexpr (G >= 64) v += __shfl_xor(v, 32);
    return v;
}

// ------------------------------------------------ x staging layout (LDS) ----
// x values are stored with 4 floats of padding after every 64, so that lanes
// reading the 64- or 256-value spans of different units hit different banks.
QG_DEV int xpad(int c) { return c + ((c >> 6) << 2); }
__host__ __device__ inline int xstride_of(int cols) { return cols + ((cols >> 6) << 2) + 4; }

// ================================================================ units ====

// ---- Q8_0: pair of blocks; block A at byte PH, block B at byte PH+34 ------
template <int PH>
struct UQ8_0 {
    static constexpr int TYPE = T_Q8_0, VALUES = 64, BYTES = 68, ND = PH ? 18 : 17;
    static constexpr int GROUPS = 2, GSIZE = 32, SUMS = 0;  // no x-sums needed
    // has_b == false: the row ends after block A (odd blocks per row).
    QG_DEV static void load(rsrc_t r, u32 off, u32 (&w)[ND], bool has_b) {
        ldn<9>(r, off, w);
        if (has_b) {
            ldn<ND - 9, 9>(r, off + 36, w);
        } else {
#pragma unroll
            for (int i = 9; i < ND; i++) w[i] = 0;
        }
    }
    QG_DEV static float scale(const u32 (&w)[ND], int g) { return h2f(half_at(w, PH + 34 * g)); }
    QG_DEV static float code(const u32 (&w)[ND], int i) { return s8_at(w, PH + 34 * (i >> 5) + 2 + (i & 31)); }
    QG_DEV static float fold(const u32 (&w)[ND], int g, float s, float) { return scale(w, g) * s; }
    QG_DEV static float value(const u32 (&w)[ND], int i) { return scale(w, i >> 5) * code(w, i); }
};

// ---- Q4_0: pair of blocks; block A at byte PH, block B at byte PH+18 ------
// Byte j of a block's 16 nibble bytes: low nibble = value j, high = value j+16.
template <int PH>
struct UQ4_0 {
    static constexpr int TYPE = T_Q4_0, VALUES = 64, BYTES = 36, ND = PH ? 10 : 9;
    static constexpr int GROUPS = 2, GSIZE = 32, SUMS = 32;  // x-sums over 32 values
    QG_DEV static void load(rsrc_t r, u32 off, u32 (&w)[ND], bool has_b) {
        ldn<5>(r, off, w);
        if (has_b) {
            ldn<ND - 5, 5>(r, off + 20, w);
        } else {
#pragma unroll
            for (int i = 5; i < ND; i++) w[i] = 0;
        }
    }
    QG_DEV static float scale(const u32 (&w)[ND], int g) { return h2f(half_at(w, PH + 18 * g)); }
    QG_DEV static float code(const u32 (&w)[ND], int i) {  // nibble 0..15
        const int pos = PH + 18 * (i >> 5) + 2 + (i & 15);
        const u32 word = w[pos >> 2];
        const u32 m = (i & 16) ? ((word >> 4) & 0x0F0F0F0Fu) : (word & 0x0F0F0F0Fu);
        return u8_of(m, pos & 3);
    }
    // d * sum((q - 8) x) = d * (sum(q x) - 8 sum(x))
    QG_DEV static float fold(const u32 (&w)[ND], int g, float s, float xs) { return scale(w, g) * fmaf(-8.0f, xs, s); }
    QG_DEV static float value(const u32 (&w)[ND], int i) { return scale(w, i >> 5) * (code(w, i) - 8.0f); }
};

// ---- Q4_K: one block, 36 dwords: [d|dmin] [scales x3] [qs x32] -----------
// qs chunk c (dwords 4+8c .. 4+8c+7): low nibbles are sub-block 2c, high
// nibbles sub-block 2c+1.  The 12 scale bytes hold 6-bit (scale, min) pairs:
// sub-blocks 0..3 use bytes j and j+4; 4..7 take the low/high nibble of byte
// j+4 and the top two bits of bytes j-4 (scale) and j (min).
template <int PH>
struct UQ4_K {
    static constexpr int TYPE = T_Q4_K, VALUES = 256, BYTES = 144, ND = 36;
    static constexpr int GROUPS = 8, GSIZE = 32, SUMS = 32;
    QG_DEV static void load(rsrc_t r, u32 off, u32 (&w)[ND], bool) {
        if constexpr (PH == 0) {
            ldn<36>(r, off, w);
        } else {  // block at 2 mod 4: 37 dwords from 2 bytes earlier, re-aligned
            u32 t[37];
            ldn<37>(r, off, t);
#pragma unroll
            for (int i = 0; i < 36; i++) w[i] = __builtin_amdgcn_alignbyte(t[i + 1], t[i], 2);
        }
    }
    // scale / min bytes for sub-blocks 4h..4h+3 (one per byte)
    QG_DEV static u32 sc4(const u32 (&w)[ND], int h) {
        return h == 0 ? (w[1] & 0x3F3F3F3Fu) : ((w[3] & 0x0F0F0F0Fu) | ((w[1] >> 2) & 0x30303030u));
    }
    QG_DEV static u32 mn4(const u32 (&w)[ND], int h) {
        return h == 0 ? (w[2] & 0x3F3F3F3Fu) : (((w[3] >> 4) & 0x0F0F0F0Fu) | ((w[2] >> 2) & 0x30303030u));
    }
    QG_DEV static float dsc(const u32 (&w)[ND], int g) { return h2f(w[0]) * u8_of(sc4(w, g >> 2), g & 3); }
    QG_DEV static float dmn(const u32 (&w)[ND], int g) { return h2f(w[0] >> 16) * u8_of(mn4(w, g >> 2), g & 3); }
    QG_DEV static float code(const u32 (&w)[ND], int i) {
        const int c = i >> 6, hi = (i >> 5) & 1, k = (i & 31) >> 2;
        const u32 word = w[4 + 8 * c + k];
        const u32 m = hi ? ((word >> 4) & 0x0F0F0F0Fu) : (word & 0x0F0F0F0Fu);
        return u8_of(m, i & 3);
    }
    // d*sc*sum(q x) - dmin*m*sum(x)
    QG_DEV static float fold(const u32 (&w)[ND], int g, float s, float xs) { return fmaf(dsc(w, g), s, -(dmn(w, g) * xs)); }
    // (d*sc)*q - dmin*m with one rounding: both products are exact in f32
    QG_DEV static float value(const u32 (&w)[ND], int i) { return fmaf(dsc(w, i >> 5), code(w, i), -dmn(w, i >> 5)); }
};

// ---- Q6_K: one block, re-aligned to 53 dwords: ql[0..31] qh[32..47] sc[48..51] d[52]
// Half n of the block (values 128n..): value 128n + 32p + l (l < 32) takes the
// low (p = 0, 1) or high (p = 2, 3) nibble of ql[64n + l + 32(p & 1)] and bits
// 2p, 2p+1 of qh[32n + l]; its scale is int8 scales[(value >> 4)].
struct UQ6_K {
    static constexpr int TYPE = T_Q6_K, VALUES = 256, BYTES = 210, ND = 53;
    static constexpr int GROUPS = 16, GSIZE = 16, SUMS = 16;
    // off: the block's byte offset; loads 53 dwords from off & ~3 and shifts.
    QG_DEV static void load(rsrc_t r, u32 off, u32 (&w)[ND], bool) {
        u32 t[54];
        const u32 s = off & 3u;
        ldn<53>(r, off & ~3u, t);
        t[53] = 0;
#pragma unroll
        for (int i = 0; i < 53; i++) w[i] = __builtin_amdgcn_alignbyte(t[i + 1], t[i], s);
    }
    // four 6-bit codes (one per byte) for values 128n + 32p + 4k .. +3
    QG_DEV static u32 code4(const u32 (&w)[ND], int n, int p, int k) {
        const u32 ql = w[16 * n + 8 * (p & 1) + k], qh = w[32 + 8 * n + k];
        const u32 lo = (p >> 1) ? ((ql >> 4) & 0x0F0F0F0Fu) : (ql & 0x0F0F0F0Fu);
        const u32 hb = (p == 0) ? (qh << 4) : (p == 1) ? (qh << 2) : (p == 2) ? qh : (qh >> 2);
        return lo | (hb & 0x30303030u);
    }
    QG_DEV static float code(const u32 (&w)[ND], int i) {  // 0..63
        return u8_of(code4(w, i >> 7, (i >> 5) & 3, (i & 31) >> 2), i & 3);
    }
    QG_DEV static float dsc(const u32 (&w)[ND], int g) { return h2f(w[52]) * s8_at(w, 192 + g); }
    // d*sc*sum((q - 32) x) = d*sc*(sum(q x) - 32 sum(x))
    QG_DEV static float fold(const u32 (&w)[ND], int g, float s, float xs) { return dsc(w, g) * fmaf(-32.0f, xs, s); }
    QG_DEV static float value(const u32 (&w)[ND], int i) { return dsc(w, i >> 4) * (code(w, i) - 32.0f); }
};

}  // namespace qg

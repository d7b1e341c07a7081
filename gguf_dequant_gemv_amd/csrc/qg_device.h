// qg_device.h -- device helpers and the per-type block-unpack layer (gfx950).
//
// A "unit" is the piece of a weight row one lane loads and decodes at a time:
//   Q8_0  one block (32 values, 34 B) or a pair of blocks (64 values, 68 B)
//   Q4_0  one block (32 values, 18 B) or a pair of blocks (64 values, 36 B)
//   Q4_K  one block (256 values, 144 B)
//   Q6_K  one block (256 values, 210 B)
// GGUF blocks sit at 2-byte alignment.  A pair of Q8_0 or Q4_0 blocks is a
// multiple of 4 bytes, so in a tensor that starts 4-byte aligned with an even
// number of blocks per row every pair starts on a dword and every field in it
// sits at a compile-time byte position.  Single blocks and the K-quant blocks
// are loaded from the aligned-down address and shifted into place with
// v_alignbyte (one op per dword).
//
// The GEMV dot products and the dequantization kernel share these decoders.
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

// T_Q8_0P / T_Q6_KP: Q8_0 / Q6_K in their plane layouts
enum { T_Q4_0 = 2, T_Q8_0 = 8, T_Q4_K = 12, T_Q6_K = 14, T_Q8_0P = 264, T_Q6_KP = 270 };

// ---------------------------------------------------------------- scalars --
QG_DEV float h2f(u32 bits) {  // low 16 bits: IEEE binary16 -> f32 (exact)
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
}

// 16-bit field at byte `pos` (even) of a dword array.
QG_DEV u32 half_at(const u32 *w, int pos) { return (w[pos >> 2] >> (8 * (pos & 3))) & 0xFFFFu; }

// Signed / unsigned byte `pos` of a dword array as f32 (one v_cvt with a byte select).
QG_DEV float s8_at(const u32 *w, int pos) { return (float)(int8_t)(w[pos >> 2] >> (8 * (pos & 3))); }
QG_DEV float u8_of(u32 word, int b) { return (float)((word >> (8 * b)) & 0xFFu); }

// The value unchanged, but opaque to the optimiser: a masked word then feeds
// four byte-select converts instead of being re-extracted field by field.
QG_DEV u32 opaque(u32 v) {
    asm("" : "+v"(v));
    return v;
}

// A wave-uniform pointer, kept in scalar registers: a buffer descriptor built
// from it then needs no per-lane loop (the compiler cannot always prove a
// pointer chosen through several paths uniform).
template <class T>
QG_DEV T *uniform_ptr(T *p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const u32 lo = (u32)__builtin_amdgcn_readfirstlane((int)(u32)v);
    const u32 hi = (u32)__builtin_amdgcn_readfirstlane((int)(u32)(v >> 32));
    return (T *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

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

// Sum over the whole wave, every lane getting the same value: DPP within each
// row of 16 lanes, then the four row sums through scalar registers.
QG_DEV float wave_sum(float v) {
    v = group_sum<16>(v);
    const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (a + b) + (c + d);
}

// LDS accesses the compiler does not see as memory operations.  Seen, every
// LDS read or write issued while buffer-to-LDS copies are in flight would
// wait for all of them (the compiler cannot tell which bytes a copy lands
// in), which undoes the copies' lead.  The kernel waits itself: QG_WAIT_VM
// for the copies it is about to read, lds_wait() for these accesses.
QG_DEV u32 lds_off(const void *p) {
    return (u32)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)p;
}
QG_DEV u32 lds_ld32(u32 a) {
    u32 v;
    asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(a));
    return v;
}
QG_DEV u32x4 lds_ld128(u32 a) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(a));
    return v;
}
QG_DEV void lds_st64(u32 a, u32 lo, u32 hi) {
    asm volatile("ds_write_b64 %0, %1" : : "v"(a), "v"(u32x2{lo, hi}) : "memory");
}
QG_DEV void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// after lds_wait(): ties a value read above to the wait, so no use of it is
// scheduled before the wait
template <class T>
QG_DEV void lds_ready(T &v) { asm volatile("" : "+v"(v)); }
// workgroup barrier without the compiler's fence (which would wait for the
// copies in flight): this wave's own LDS accesses are complete first
QG_DEV void lds_barrier() {
    lds_wait();
    __builtin_amdgcn_s_barrier();
}

// N consecutive dwords from LDS byte address a (4-byte aligned), as above
template <int N>
QG_DEV void lds_ldn(u32 a, u32 (&t)[N]) {
#pragma unroll
    for (int i = 0; i + 1 < N; i += 2) {
        u32x2 v;
        asm volatile("ds_read2_b32 %0, %1 offset0:%2 offset1:%3" : "=v"(v) : "v"(a), "i"(i), "i"(i + 1));
        t[i] = v.x;
        t[i + 1] = v.y;
    }
    if constexpr ((N & 1) != 0) asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(t[N - 1]) : "v"(a), "i"(4 * (N - 1)));
}
// 16 bytes at LDS byte address a + O (16-byte aligned)
template <int O>
QG_DEV f32x4 lds_ld128f(u32 a) {
    f32x4 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(a), "i"(O));
    return v;
}

// ------------------------------------------------ x staging layout (LDS) ----
// x values are stored with 4 floats of padding after every 64, so that lanes
// reading the 64- or 256-value spans of different units hit different banks.
QG_DEV int xpad(int c) { return c + ((c >> 6) << 2); }
__host__ __device__ inline int xstride_of(int cols) { return cols + ((cols >> 6) << 2) + 4; }

// ================================================================ units ====
// Every unit type exposes
//   VALUES, BYTES        values and bytes per unit
//   NR, ND               dwords a lane holds for one unit as loaded / decoded
//   GROUPS, GSIZE, SUMS  scale groups (GSIZE values each) and the span of the
//                        x-sums fold() needs (0 = none)
//   issue(r, off, raw)   start the loads of the unit at byte `off`
//   prep(raw, off, w)    the loaded dwords in decode order (after they arrive)
//   load(r, off, w)      issue + prep
//   code(w, i)           integer code of value i as f32 (exact)
//   dcode(w, i)          the code as the dot products use it: times dfix(g, h)^-1
//                        for half h of group g (a high nibble left in place is
//                        16 times the code; the factor is a power of two, so
//                        dcode*x sums scale back exactly)
//   dfix(g, h)           that factor (1 or 1/16)
//   fold(w, g, s, xs)    group g's contribution from s = sum(code*x), xs = sum(x)
//   value(w, i)          the dequantized value as f32 (one rounding)

// Realigned units: the N dwords that start at byte `off` (2-byte aligned) are
// issued as N+1 aligned dwords from off & ~3 (raw_load, kept as they arrive)
// and shifted into place with v_alignbyte only when the unit is consumed
// (realign), so a lane can keep several units' loads in flight.
template <int N, int M>
QG_DEV void raw_load(rsrc_t r, u32 off, u32 (&t)[M]) {
    static_assert(N + 1 <= M, "raw_load: out of range");
    ldn<N>(r, off & ~3u, t);
    // the extra dword is a load of its own: past the tensor's last dword it
    // is out of the descriptor's range and reads 0 without touching memory
    t[N] = __builtin_amdgcn_raw_buffer_load_b32(r, (off & ~3u) + 4 * N, 0, 0);
}
template <int N, int M, int K>
QG_DEV void realign(const u32 (&t)[M], u32 off, u32 (&w)[K]) {
    static_assert(N + 1 <= M && N <= K, "realign: out of range");
    const u32 s = off & 3u;
#pragma unroll
    for (int i = 0; i < N; i++) w[i] = __builtin_amdgcn_alignbyte(t[i + 1], t[i], s);
}

// ---- Q8_0, one block (32 values, 34 B), any 2-byte phase -------------------
struct UQ8_0B {
    static constexpr int TYPE = T_Q8_0, VALUES = 32, BYTES = 34, NR = 10, ND = 9;
    static constexpr int GROUPS = 1, GSIZE = 32, SUMS = 0;
    // 9 dwords from off & ~3 cover the 34 bytes for either phase; the 10th
    // (a separate load) only keeps the shift uniform
    QG_DEV static void issue(rsrc_t r, u32 off, u32 (&t)[NR]) { raw_load<9>(r, off, t); }
    QG_DEV static void prep(const u32 (&t)[NR], u32 off, u32 (&w)[ND]) { realign<9>(t, off, w); }
    QG_DEV static void load(rsrc_t r, u32 off, u32 (&w)[ND]) { u32 t[NR]; issue(r, off, t); prep(t, off, w); }
    QG_DEV static float scale(const u32 (&w)[ND]) { return h2f(w[0]); }
    QG_DEV static float dfix(int, int) { return 1.0f; }
    QG_DEV static float dcode(const u32 (&w)[ND], int i) { return code(w, i); }
    QG_DEV static float code(const u32 (&w)[ND], int i) { return s8_at(w, 2 + i); }
    QG_DEV static float fold(const u32 (&w)[ND], int, float s, float) { return scale(w) * s; }
    QG_DEV static float value(const u32 (&w)[ND], int i) { return scale(w) * code(w, i); }
};

// ---- Q8_0, a pair of blocks (64 values, 68 B) starting 4-byte aligned ------
// Block A at byte 0, block B at byte 34: every field sits at a fixed byte.
struct UQ8_0P {
    static constexpr int TYPE = T_Q8_0, VALUES = 64, BYTES = 68, NR = 17, ND = 17;
    static constexpr int GROUPS = 2, GSIZE = 32, SUMS = 0;
    QG_DEV static void issue(rsrc_t r, u32 off, u32 (&t)[NR]) { ldn<17>(r, off, t); }
    QG_DEV static void prep(const u32 (&t)[NR], u32, u32 (&w)[ND]) {
#pragma unroll
        for (int i = 0; i < ND; i++) w[i] = t[i];
    }
    QG_DEV static void load(rsrc_t r, u32 off, u32 (&w)[ND]) { ldn<17>(r, off, w); }
    QG_DEV static float scale(const u32 (&w)[ND], int g) { return h2f(half_at(w, 34 * g)); }
    QG_DEV static float dfix(int, int) { return 1.0f; }
    QG_DEV static float dcode(const u32 (&w)[ND], int i) { return code(w, i); }
    QG_DEV static float code(const u32 (&w)[ND], int i) { return s8_at(w, 34 * (i >> 5) + 2 + (i & 31)); }
    QG_DEV static float fold(const u32 (&w)[ND], int g, float s, float) { return scale(w, g) * s; }
    QG_DEV static float value(const u32 (&w)[ND], int i) { return scale(w, i >> 5) * code(w, i); }
};

// ---- Q4_0, one block (32 values, 18 B), any 2-byte phase -------------------
// Byte j of the 16 nibble bytes: low nibble = value j, high = value j+16.
struct UQ4_0B {
    static constexpr int TYPE = T_Q4_0, VALUES = 32, BYTES = 18, NR = 6, ND = 5;
    static constexpr int GROUPS = 1, GSIZE = 32, SUMS = 32;
    QG_DEV static void issue(rsrc_t r, u32 off, u32 (&t)[NR]) { raw_load<5>(r, off, t); }
    QG_DEV static void prep(const u32 (&t)[NR], u32 off, u32 (&w)[ND]) { realign<5>(t, off, w); }
    QG_DEV static void load(rsrc_t r, u32 off, u32 (&w)[ND]) { u32 t[NR]; issue(r, off, t); prep(t, off, w); }
    QG_DEV static float scale(const u32 (&w)[ND]) { return h2f(w[0]); }
    QG_DEV static float code(const u32 (&w)[ND], int i) {  // nibble 0..15
        const int pos = 2 + (i & 15);
        const u32 word = w[pos >> 2];
        const u32 m = (i & 16) ? ((word >> 4) & 0x0F0F0F0Fu) : (word & 0x0F0F0F0Fu);
        return u8_of(m, pos & 3);
    }
    // values 16..31 are the high nibbles: 16 * code in place
    QG_DEV static float dfix(int, int h) { return h ? 0.0625f : 1.0f; }
    QG_DEV static float dcode(const u32 (&w)[ND], int i) {
        const int pos = 2 + (i & 15);
        return u8_of(opaque(w[pos >> 2] & ((i & 16) ? 0xF0F0F0F0u : 0x0F0F0F0Fu)), pos & 3);
    }
    // d * sum((q - 8) x) = d * (sum(q x) - 8 sum(x))
    QG_DEV static float fold(const u32 (&w)[ND], int, float s, float xs) { return scale(w) * fmaf(-8.0f, xs, s); }
    QG_DEV static float value(const u32 (&w)[ND], int i) { return scale(w) * (code(w, i) - 8.0f); }
};

// ---- Q4_0, a pair of blocks (64 values, 36 B) starting 4-byte aligned ------
struct UQ4_0P {
    static constexpr int TYPE = T_Q4_0, VALUES = 64, BYTES = 36, NR = 9, ND = 9;
    static constexpr int GROUPS = 2, GSIZE = 32, SUMS = 32;
    QG_DEV static void issue(rsrc_t r, u32 off, u32 (&t)[NR]) { ldn<9>(r, off, t); }
    QG_DEV static void prep(const u32 (&t)[NR], u32, u32 (&w)[ND]) {
#pragma unroll
        for (int i = 0; i < ND; i++) w[i] = t[i];
    }
    QG_DEV static void load(rsrc_t r, u32 off, u32 (&w)[ND]) { ldn<9>(r, off, w); }
    QG_DEV static float scale(const u32 (&w)[ND], int g) { return h2f(half_at(w, 18 * g)); }
    QG_DEV static float code(const u32 (&w)[ND], int i) {
        const int pos = 18 * (i >> 5) + 2 + (i & 15);
        const u32 word = w[pos >> 2];
        const u32 m = (i & 16) ? ((word >> 4) & 0x0F0F0F0Fu) : (word & 0x0F0F0F0Fu);
        return u8_of(m, pos & 3);
    }
    QG_DEV static float dfix(int, int h) { return h ? 0.0625f : 1.0f; }
    QG_DEV static float dcode(const u32 (&w)[ND], int i) {
        const int pos = 18 * (i >> 5) + 2 + (i & 15);
        return u8_of(opaque(w[pos >> 2] & ((i & 16) ? 0xF0F0F0F0u : 0x0F0F0F0Fu)), pos & 3);
    }
    QG_DEV static float fold(const u32 (&w)[ND], int g, float s, float xs) { return scale(w, g) * fmaf(-8.0f, xs, s); }
    QG_DEV static float value(const u32 (&w)[ND], int i) { return scale(w, i >> 5) * (code(w, i) - 8.0f); }
};

// ---- Q4_K: one block (256 values, 144 B), realigned to 36 dwords ----------
// [d|dmin] [scales x3] [qs x32].  qs chunk c (dwords 4+8c .. 4+8c+7): low
// nibbles are sub-block 2c, high nibbles sub-block 2c+1.  The 12 scale bytes
// hold 6-bit (scale, min) pairs: sub-blocks 0..3 use bytes j and j+4; 4..7
// take the low/high nibble of byte j+4 and the top two bits of bytes j-4
// (scale) and j (min).
struct UQ4_K {
    static constexpr int TYPE = T_Q4_K, VALUES = 256, BYTES = 144, NR = 37, ND = 36;
    static constexpr int GROUPS = 8, GSIZE = 32, SUMS = 32;
    QG_DEV static void issue(rsrc_t r, u32 off, u32 (&t)[NR]) { raw_load<36>(r, off, t); }
    QG_DEV static void prep(const u32 (&t)[NR], u32 off, u32 (&w)[ND]) { realign<36>(t, off, w); }
    QG_DEV static void load(rsrc_t r, u32 off, u32 (&w)[ND]) { u32 t[NR]; issue(r, off, t); prep(t, off, w); }
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
    // odd sub-blocks are the high nibbles: 16 * code in place
    QG_DEV static float dfix(int g, int) { return (g & 1) ? 0.0625f : 1.0f; }
    QG_DEV static float dcode(const u32 (&w)[ND], int i) {
        const int c = i >> 6, hi = (i >> 5) & 1, k = (i & 31) >> 2;
        return u8_of(opaque(w[4 + 8 * c + k] & (hi ? 0xF0F0F0F0u : 0x0F0F0F0Fu)), i & 3);
    }
    // d*sc*sum(q x) - dmin*m*sum(x)
    QG_DEV static float fold(const u32 (&w)[ND], int g, float s, float xs) { return fmaf(dsc(w, g), s, -(dmn(w, g) * xs)); }
    // (d*sc)*q - dmin*m with one rounding: both products are exact in f32
    QG_DEV static float value(const u32 (&w)[ND], int i) { return fmaf(dsc(w, i >> 5), code(w, i), -dmn(w, i >> 5)); }
};

// ---- Q6_K: one block (256 values, 210 B), realigned to 53 dwords ----------
// ql[0..31] qh[32..47] sc[48..51] d[52].  Half n of the block (values 128n..):
// value 128n + 32p + l (l < 32) takes the low (p = 0, 1) or high (p = 2, 3)
// nibble of ql[64n + l + 32(p & 1)] and bits 2p, 2p+1 of qh[32n + l]; its
// scale is int8 scales[value >> 4].
struct UQ6_K {
    static constexpr int TYPE = T_Q6_K, VALUES = 256, BYTES = 210, NR = 54, ND = 53;
    static constexpr int GROUPS = 16, GSIZE = 16, SUMS = 16;
    QG_DEV static void issue(rsrc_t r, u32 off, u32 (&t)[NR]) { raw_load<53>(r, off, t); }
    QG_DEV static void prep(const u32 (&t)[NR], u32 off, u32 (&w)[ND]) { realign<53>(t, off, w); }
    QG_DEV static void load(rsrc_t r, u32 off, u32 (&w)[ND]) { u32 t[NR]; issue(r, off, t); prep(t, off, w); }
    // four 6-bit codes (one per byte) for values 128n + 32p + 4k .. +3
    QG_DEV static u32 code4(const u32 (&w)[ND], int n, int p, int k) {
        const u32 ql = w[16 * n + 8 * (p & 1) + k], qh = w[32 + 8 * n + k];
        const u32 lo = (p >> 1) ? ((ql >> 4) & 0x0F0F0F0Fu) : (ql & 0x0F0F0F0Fu);
        const u32 hb = (p == 0) ? (qh << 4) : (p == 1) ? (qh << 2) : (p == 2) ? qh : (qh >> 2);
        return lo | (hb & 0x30303030u);
    }
    QG_DEV static float dfix(int, int) { return 1.0f; }
    QG_DEV static float dcode(const u32 (&w)[ND], int i) {  // one code word per 4 values
        return u8_of(opaque(code4(w, i >> 7, (i >> 5) & 3, (i & 31) >> 2)), i & 3);
    }
    QG_DEV static float code(const u32 (&w)[ND], int i) {  // 0..63
        return u8_of(code4(w, i >> 7, (i >> 5) & 3, (i & 31) >> 2), i & 3);
    }
    QG_DEV static float dsc(const u32 (&w)[ND], int g) { return h2f(w[52]) * s8_at(w, 192 + g); }
    // d*sc*sum((q - 32) x) = d*sc*(sum(q x) - 32 sum(x))
    QG_DEV static float fold(const u32 (&w)[ND], int g, float s, float xs) { return dsc(w, g) * fmaf(-32.0f, xs, s); }
    QG_DEV static float value(const u32 (&w)[ND], int i) { return dsc(w, i >> 4) * (code(w, i) - 32.0f); }
};

// ---------------------------------------------------------- routing ----
// Monotone map f32 -> u32 for the pick order: -0 folded onto +0, and every
// NaN to 0, below -inf (whose key is 0x007FFFFF), so a NaN logit is picked
// only after every number, the lowest index first.
QG_DEV u32 order_key(float f) {
    u32 u = __builtin_bit_cast(u32, f);
    if (u == 0x80000000u) u = 0u;
    const u32 key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return f != f ? 0u : key;
}

// Maximum over the wave, uniform: DPP within each row of 16 lanes, then the
// four row results through scalar registers.
template <int CTRL>
QG_DEV u32 dpp_u(u32 v) {
    return (u32)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
QG_DEV u32 wave_max_u32(u32 v) {
    v = max(v, dpp_u<0xB1>(v));    // lane ^ 1
    v = max(v, dpp_u<0x4E>(v));    // lane ^ 2
    v = max(v, dpp_u<0x141>(v));   // row_half_mirror
    v = max(v, dpp_u<0x140>(v));   // row_mirror
    const u32 a = (u32)__builtin_amdgcn_readlane((int)v, 0), b = (u32)__builtin_amdgcn_readlane((int)v, 16);
    const u32 c = (u32)__builtin_amdgcn_readlane((int)v, 32), d = (u32)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(a, b), max(c, d));
}


}  // namespace qg

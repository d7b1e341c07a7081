"""Second, independent decoders for the four block types (numpy, vectorised).

Each is written from a *different* rendering of the layout on the pages than
the one the oracle follows, so that a transposed index, a wrong shift or a
dropped term in either shows up as a mismatch:

  Q8_0  [qwen3 page] WGSL i8at: value e is byte e&3 of packed word e>>2 of the
        code plane, sign-extended, times the f16 scale of group e>>5.
  Q4_0  [gemma4 page] WGSL matmulQ4T: value kk of a block sits in nibble-plane
        word (kk&15)>>2, at bit shift (kk&3)*8 + (kk>>4)*4; value = (nib-8)*d.
  Q4_K  [bonsai page] packed-weight GEMM WG_GEMM_Q4K: the block as 36 u32
        words: word 0 = (d, dmin), words 1..3 = scales, word 4+8j+i of qs gives
        values 64j+4i+b (low nibble of byte b) and 64j+32+4i+b (high nibble),
        with the (scale, min) pair of sub-blocks 2j and 2j+1 (scmin).
  Q6_K  [gemma4 page] WGSL q6v plane indexer: value t: n=t>>7, r=t&127,
        qd=r>>5, l=r&31; low 4 bits from ql[64n + l + 32(qd&1)] (low nibble for
        qd<2, high for qd>=2); top 2 bits from qh[32n + l] >> 2qd; scale index
        8n + (l>>4) + 2qd; value = d * sc * (q - 32).

All arithmetic is in float64 and exact for these formats.
"""
import numpy as np

Q4_0, Q8_0, Q4_K, Q6_K = 2, 8, 12, 14
QK = {Q4_0: 32, Q8_0: 32, Q4_K: 256, Q6_K: 256}
BB = {Q4_0: 18, Q8_0: 34, Q4_K: 144, Q6_K: 210}


def f16le(lo, hi):
    """Two little-endian bytes -> float64 via numpy's binary16 type."""
    bits = (lo.astype(np.uint16) | (hi.astype(np.uint16) << 8)).astype(np.uint16)
    return bits.view(np.float16).astype(np.float64)


def dec_q8_0(blocks):
    b = blocks.reshape(-1, 34)
    d = f16le(b[:, 0], b[:, 1])
    # the code plane of one block, packed into u32 words as the pages store it
    words = np.ascontiguousarray(b[:, 2:34]).view("<u4")                # [nb, 8]
    e = np.arange(32)
    byte = (words[:, e >> 2] >> ((e & 3) * 8).astype(np.uint32)) & 0xFF
    code = np.where(byte >= 128, byte.astype(np.int64) - 256, byte.astype(np.int64))
    return (d[:, None] * code).ravel()


def dec_q4_0(blocks):
    b = blocks.reshape(-1, 18)
    d = f16le(b[:, 0], b[:, 1])
    words = np.ascontiguousarray(b[:, 2:18]).view("<u4")                # [nb, 4]
    kk = np.arange(32)
    shift = ((kk & 3) * 8 + (kk >> 4) * 4).astype(np.uint32)
    nib = (words[:, (kk & 15) >> 2] >> shift) & 15
    return (d[:, None] * (nib.astype(np.int64) - 8)).ravel()


def _q4k_scmin(s0, s1, s2, j):
    """(scale, min) of sub-block j from the three scale words (scmin rendering)."""
    def sb(i):
        w = s0 if i < 4 else (s1 if i < 8 else s2)
        return (w >> np.uint32(8 * (i & 3))) & 0xFF
    if j < 4:
        return sb(j) & 63, sb(j + 4) & 63
    a, bb, c = sb(j + 4), sb(j - 4), sb(j)
    return (a & 0xF) | ((bb >> 6) << 4), (a >> 4) | ((c >> 6) << 4)


def dec_q4_k(blocks):
    b = np.ascontiguousarray(blocks.reshape(-1, 144))
    W = b.view("<u4")                                                  # [nb, 36]
    nbk = W.shape[0]
    d = f16le(b[:, 0], b[:, 1])
    dmin = f16le(b[:, 2], b[:, 3])
    out = np.empty((nbk, 256), np.float64)
    s0, s1, s2 = W[:, 1], W[:, 2], W[:, 3]
    for j in range(4):
        sl, ml = _q4k_scmin(s0, s1, s2, 2 * j)
        sh, mh = _q4k_scmin(s0, s1, s2, 2 * j + 1)
        for i in range(8):
            w = W[:, 4 + 8 * j + i]
            for byt in range(4):
                lo = (w >> np.uint32(8 * byt)) & 0xF
                hi = (w >> np.uint32(8 * byt + 4)) & 0xF
                k = 64 * j + 4 * i + byt
                out[:, k] = d * sl * lo - dmin * ml
                out[:, k + 32] = d * sh * hi - dmin * mh
    return out.ravel()


def dec_q6_k(blocks):
    b = blocks.reshape(-1, 210)
    ql, qh = b[:, 0:128].astype(np.int64), b[:, 128:192].astype(np.int64)
    sc = b[:, 192:208].view(np.int8).astype(np.int64)
    d = f16le(b[:, 208], b[:, 209])
    t = np.arange(256)
    n, r = t >> 7, t & 127
    qd, l = r >> 5, r & 31
    lo = ql[:, n * 64 + l + (qd & 1) * 32]
    q4 = np.where(qd >= 2, lo >> 4, lo & 15)
    h = (qh[:, n * 32 + l] >> (qd * 2)) & 3
    s = sc[:, n * 8 + (l >> 4) + qd * 2]
    return (d[:, None] * s * ((q4 | (h << 4)) - 32)).ravel()


def dec_q6_k_planes(planes, n):
    """n Q6_K blocks in the plane layout, decoded as the [gemma4 page] q6v
    indexer reads its planes: ql as 32 little-endian words per block (byte
    qb of the block: word qb >> 2, shift 8 (qb & 3)), qh as 16 words, the
    scales as 4 words of int8, d from its own plane (f16 here)."""
    p = np.ascontiguousarray(planes, np.uint8).ravel()
    ql = p[0:128 * n].view("<u4").reshape(n, 32).astype(np.int64)
    qh = p[128 * n:192 * n].view("<u4").reshape(n, 16).astype(np.int64)
    sc = p[192 * n:208 * n].view("<u4").reshape(n, 4).astype(np.int64)
    dd = p[208 * n:210 * n]
    d = f16le(dd[0::2], dd[1::2])
    t = np.arange(256)
    nh, r = t >> 7, t & 127
    qd, l = r >> 5, r & 31
    qb = nh * 64 + l + (qd & 1) * 32
    lo = (ql[:, qb >> 2] >> ((qb & 3) * 8)) & 0xFF
    q4 = np.where(qd >= 2, lo >> 4, lo & 15)
    hb = nh * 32 + l
    h = (qh[:, hb >> 2] >> ((hb & 3) * 8 + qd * 2)) & 3
    si = nh * 8 + (l >> 4) + qd * 2
    s8 = (sc[:, si >> 2] >> ((si & 3) * 8)) & 0xFF
    s = np.where(s8 >= 128, s8 - 256, s8)
    return (d[:, None] * s * ((q4 | (h << 4)) - 32)).ravel()


def dec_q8_0_planes(planes, n):
    """n Q8_0 blocks in the plane layout, decoded as the [qwen3 page] i8at
    reads its code plane: value e is byte e & 3 of little-endian word e >> 2,
    sign-extended, times the f16 scale of group e >> 5 (here from the scale
    plane after the codes)."""
    p = np.ascontiguousarray(planes, np.uint8).ravel()
    words = p[:32 * n].view("<u4").astype(np.int64)
    e = np.arange(32 * n)
    byte = (words[e >> 2] >> ((e & 3) * 8)) & 0xFF
    q = np.where(byte >= 128, byte - 256, byte)
    dd = p[32 * n:34 * n]
    d = f16le(dd[0::2], dd[1::2])
    return d[e >> 5] * q


DEC = {Q8_0: dec_q8_0, Q4_0: dec_q4_0, Q4_K: dec_q4_k, Q6_K: dec_q6_k}


def dequant_matrix(t, W, rows, cols):
    return DEC[t](np.ascontiguousarray(W, np.uint8).ravel()).reshape(rows, cols)

"""Pins for the oracle: it is checked here against things other than itself.

Closed forms, second decoders written from the pages' other renderings of each
block layout, brute force on tiny inputs, bijection and one-hot invariants,
numpy / scipy routines for the special cases that reduce to them, and values
printed on the pages (tests/golden/).  No GPU.
"""
import math
import os

import numpy as np
import pytest
import scipy.special

import gguf_synth as gs
from second_decoders import DEC, dequant_matrix

HERE = os.path.dirname(os.path.abspath(__file__))
TYPES = [gs.Q8_0, gs.Q4_0, gs.Q4_K, gs.Q6_K]


# ---------------------------------------------------------------- f16 -------
def test_f16_all_patterns(orc):
    """Every binary16 pattern decodes as numpy's float16 -> float64 (library routine)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.f16(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zero too
    assert math.copysign(1.0, orc.f16(0x8000)) == -1.0


# ------------------------------------------------------- block layouts ------
@pytest.mark.parametrize("t", TYPES)
def test_dequant_matches_second_decoder(orc, t):
    g = gs.rng(100 + t)
    W = gs.weights(t, g, 7, 2 * gs.QK[t])
    n = W.size // gs.BLOCK_BYTES[t] * gs.QK[t]
    assert np.array_equal(orc.dequant(t, W, n), DEC[t](W.ravel()))


@pytest.mark.parametrize("t", TYPES)
def test_block_sizes(orc, t):
    assert orc.block_bytes(t) == gs.BLOCK_BYTES[t]
    assert orc.block_values(t) == gs.QK[t]


def test_q8_0_round_trip(orc):
    """Q8_0 values are exactly d*q: dividing by the block's d recovers the int8
    code, and re-packing (d, code) gives back the original bytes."""
    W = gs.q8_0(gs.rng(5), 16, 256).reshape(-1, 34)
    v = orc.dequant(gs.Q8_0, W, W.shape[0] * 32).reshape(-1, 32)
    d = W[:, :2].copy().view(np.float16).astype(np.float64)             # [nb, 1]
    nz = d[:, 0] != 0
    q = v[nz] / d[nz]
    assert np.array_equal(q, np.round(q))
    rebuilt = np.concatenate([W[nz, :2], q.astype(np.int8).view(np.uint8)], axis=1)
    assert np.array_equal(rebuilt, W[nz])
    # the f32 value of an exact f64 d*q is that same number (<= 18 significant bits)
    assert np.array_equal(v.astype(np.float32).astype(np.float64), v)


def _q4k_fields(orc, sc_bytes):
    """Decode the 8 scales and 8 mins of a Q4_K block through the oracle:
    with d=1, dmin=0 and all nibbles 1 a sub-block's values equal its scale;
    with d=0, dmin=1 they equal minus its min."""
    one, zero = np.float16(1.0).view(np.uint16), np.float16(0.0).view(np.uint16)

    def blk(d, dm):
        b = np.zeros(144, np.uint8)
        b[0:2] = np.array([d], np.uint16).view(np.uint8)
        b[2:4] = np.array([dm], np.uint16).view(np.uint8)
        b[4:16] = sc_bytes
        b[16:] = 0x11
        return b
    vs = orc.dequant(gs.Q4_K, blk(one, zero), 256).reshape(8, 32)
    vm = orc.dequant(gs.Q4_K, blk(zero, one), 256).reshape(8, 32)
    assert np.all(vs == vs[:, :1]) and np.all(vm == vm[:, :1])
    return vs[:, 0].astype(np.int64), (-vm[:, 0]).astype(np.int64)


def test_q4k_scale_bytes_bijection(orc):
    """96 scale bits <-> eight 6-bit scales + eight 6-bit mins: flipping any one
    bit changes exactly one field, by exactly one power of two."""
    base = gs.rng(9).integers(0, 256, 12).astype(np.uint8)
    s0, m0 = _q4k_fields(orc, base)
    assert s0.max() < 64 and m0.max() < 64
    seen = set()
    for bit in range(96):
        b = base.copy()
        b[bit // 8] ^= np.uint8(1 << (bit % 8))
        s1, m1 = _q4k_fields(orc, b)
        diff = np.concatenate([s1 - s0, m1 - m0])
        nzi = np.flatnonzero(diff)
        assert nzi.size == 1
        dv = abs(int(diff[nzi[0]]))
        assert dv & (dv - 1) == 0
        seen.add((int(nzi[0]), dv))
    assert len(seen) == 96          # every field bit is reached exactly once


def test_q4k_scale_bytes_worked_example(orc):
    """Hand-worked decode of one 12-byte scale field (get_scale_min_k4 rule):
    bytes 0..3 give the low 6 bits of scales 0..3 and their top 2 bits go to
    scales 4..7; bytes 4..7 likewise for the mins; bytes 8..11 give the low
    nibble (scale) and high nibble (min) of sub-blocks 4..7."""
    S = np.array([0xC1, 0x42, 0x83, 0x04,     # scales 0..3 = 1, 2, 3, 4; top bits 3,1,2,0
                  0x85, 0xC6, 0x07, 0x48,     # mins 0..3 = 5, 6, 7, 8; top bits 2,3,0,1
                  0x9A, 0xBC, 0xDE, 0xF0], np.uint8)
    sc, mn = _q4k_fields(orc, S)
    # scale 4+i = (S[8+i] & 15) | (top2(S[i]) << 4); min 4+i = (S[8+i] >> 4) | (top2(S[4+i]) << 4)
    assert list(sc) == [1, 2, 3, 4, 0xA | 3 << 4, 0xC | 1 << 4, 0xE | 2 << 4, 0x0 | 0 << 4]
    assert list(mn) == [5, 6, 7, 8, 0x9 | 2 << 4, 0xB | 3 << 4, 0xD | 0 << 4, 0xF | 1 << 4]


def test_q6k_codes_bijection(orc):
    """ql+qh (1536 bits) <-> 256 six-bit codes: with d=1 and every scale 1 the
    values are q-32; flipping any bit of ql/qh changes one code by 2^b."""
    b = np.zeros(210, np.uint8)
    g = gs.rng(11)
    b[:192] = g.integers(0, 256, 192)
    b[192:208] = 1
    b[208:210] = np.array([np.float16(1.0)]).view(np.uint8)
    v0 = orc.dequant(gs.Q6_K, b, 256)
    assert np.all((v0 >= -32) & (v0 <= 31))
    hit = set()
    for bit in range(192 * 8):
        bb = b.copy()
        bb[bit // 8] ^= np.uint8(1 << (bit % 8))
        d = orc.dequant(gs.Q6_K, bb, 256) - v0
        nzi = np.flatnonzero(d)
        assert nzi.size == 1
        dv = abs(int(d[nzi[0]]))
        assert dv in (1, 2, 4, 8, 16, 32)
        hit.add((int(nzi[0]), dv))
    assert len(hit) == 1536


@pytest.mark.parametrize("t", TYPES)
def test_one_hot_codes(orc, t):
    """A block whose codes are all at the offset value (contributing zero) except
    one, with d=1, dmin=0: exactly one non-zero value, at the index the
    second decoder predicts, and nowhere else."""
    qk, bbytes = gs.QK[t], gs.BLOCK_BYTES[t]
    one = np.array([np.float16(1.0)]).view(np.uint8)
    for pos in range(0, qk, 5):
        b = np.zeros(bbytes, np.uint8)
        if t == gs.Q8_0:
            b[0:2] = one
            b[2 + pos] = 7
        elif t == gs.Q4_0:
            b[0:2] = one
            b[2:18] = 0x88                      # every nibble 8 -> value 0
            j = pos & 15
            b[2 + j] = (b[2 + j] & 0xF0) | 0x3 if pos < 16 else (b[2 + j] & 0x0F) | 0x30
        elif t == gs.Q4_K:
            b[0:2] = one
            b[4:16] = np.array([1, 1, 1, 1, 0, 0, 0, 0, 1, 1, 1, 1], np.uint8)  # all scales 1, mins 0
            c, r = pos // 64, pos % 64
            l = r % 32
            b[16 + 32 * c + l] = 0x5 if r < 32 else 0x50
        else:
            b[192:208] = 1
            b[208:210] = one
            b[0:128] = 0x00
            b[128:192] = 0xAA                   # every top pair = 2 -> q = 32 -> value 0
            n, r = pos // 128, pos % 128
            qd, l = r // 32, r % 32
            idx = 64 * n + l + 32 * (qd & 1)
            b[idx] |= (0x5 if qd < 2 else 0x50)
        v = orc.dequant(t, b, qk)
        nzi = np.flatnonzero(v)
        assert list(nzi) == [pos], (t, pos, nzi)
        assert np.array_equal(v, DEC[t](b))


# ---------------------------------------------------------------- GEMV ------
@pytest.mark.parametrize("t", TYPES)
def test_gemv_brute_force(orc, t):
    """rows 1..3, cols 1..2 blocks, extreme codes, one-hot and random x:
    y equals the second decoder's matrix times x (exact: integer-valued
    products with d=1 and one-hot x)."""
    g = gs.rng(200 + t)
    qk = gs.QK[t]
    for rows in (1, 2, 3):
        for nbk in (1, 2):
            cols = nbk * qk
            W = gs.weights(t, g, rows, cols)
            Wb = W.reshape(-1, gs.BLOCK_BYTES[t])
            # extremes: saturate every code byte in the first block of row 0
            if t == gs.Q8_0:
                Wb[0, 2:] = np.where(np.arange(32) % 2, 0x80, 0x7F)
            elif t == gs.Q4_0:
                Wb[0, 2:] = 0xF0
            elif t == gs.Q4_K:
                Wb[0, 4:16] = 0xFF
                Wb[0, 16:] = 0x0F
            else:
                Wb[0, :192] = 0xFF
                Wb[0, 192:208] = np.array([0x80, 0x7F] * 8, np.uint8)
            M = dequant_matrix(t, W, rows, cols)
            for c in (0, cols - 1, cols // 3):
                x = np.zeros((1, cols), np.float32)
                x[0, c] = 1.0
                y, A = orc.gemv(t, W, x, rows, cols)
                assert np.array_equal(y[0], M[:, c])
                assert np.array_equal(A[0], np.abs(M[:, c]))
            x = gs.activations(g, 2, cols)
            y, A = orc.gemv(t, W, x, rows, cols, ntok=2)
            ref = x.astype(np.float64) @ M.T
            bound = np.abs(x.astype(np.float64)) @ np.abs(M.T)
            assert np.all(np.abs(y - ref) <= 1e-12 * bound)
            assert np.allclose(A, np.abs(x.astype(np.float64)) @ np.abs(M.T), rtol=1e-13, atol=0)


def test_gemv_integer_closed_form(orc):
    """d = 1.0 makes Q8_0 a plain int8 matrix: integer x gives an integer y,
    equal to numpy's int64 matmul exactly; x = ones gives the row sums."""
    g = gs.rng(3)
    rows, cols = 37, 96
    W = gs.q8_0(g, rows, cols).reshape(-1, 34)
    W[:, 0:2] = np.array([np.float16(1.0)]).view(np.uint8)
    codes = W[:, 2:].view(np.int8).astype(np.int64).reshape(rows, cols)
    x = g.integers(-50, 51, size=(1, cols)).astype(np.float32)
    y, _ = orc.gemv(gs.Q8_0, W, x, rows, cols)
    assert np.array_equal(y[0], (codes @ x[0].astype(np.int64)).astype(np.float64))
    y1, _ = orc.gemv(gs.Q8_0, W, np.ones((1, cols), np.float32), rows, cols)
    assert np.array_equal(y1[0], codes.sum(1).astype(np.float64))


@pytest.mark.parametrize("t", TYPES)
def test_gemv_scaling_invariants(orc, t):
    """y(2x) = 2 y(x) bitwise; doubling every block scale (d, and dmin for Q4_K)
    doubles y bitwise (exact powers of two commute with every rounding)."""
    g = gs.rng(300 + t)
    rows, cols = 9, 2 * gs.QK[t]
    W = gs.weights(t, g, rows, cols)
    x = gs.activations(g, 1, cols)
    y, _ = orc.gemv(t, W, x, rows, cols)
    y2, _ = orc.gemv(t, W, 2 * x, rows, cols)
    assert np.array_equal(y2, 2 * y)
    Wb = W.reshape(-1, gs.BLOCK_BYTES[t]).copy()
    offs = {gs.Q8_0: [0], gs.Q4_0: [0], gs.Q4_K: [0, 2], gs.Q6_K: [208]}[t]
    for o in offs:
        h = Wb[:, o:o + 2].copy().view(np.float16)
        Wb[:, o:o + 2] = (h.astype(np.float32) * 2).astype(np.float16).view(np.uint8)
    yd, _ = orc.gemv(t, Wb, x, rows, cols)
    assert np.array_equal(yd, 2 * y)


def test_gemv_row_sample_matches_full(orc):
    g = gs.rng(4)
    W = gs.q4_k(g, 50, 512)
    x = gs.activations(g, 3, 512)
    y, A = orc.gemv(gs.Q4_K, W, x, 50, 512, ntok=3)
    idx = np.array([0, 49, 17, 17, 3])
    ys, As = orc.gemv(gs.Q4_K, W, x, 50, 512, ntok=3, row_idx=idx)
    assert np.array_equal(ys, y[:, idx]) and np.array_equal(As, A[:, idx])


# ---------------------------------------------------------- activations -----
def test_silu_against_library(orc):
    g = np.linspace(-40, 40, 1601)
    ref = g * scipy.special.expit(g)
    got = np.array([orc.silu(v) for v in g])
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-300)
    # silu(g) - silu(-g) = g
    assert np.allclose(got - got[::-1], g, rtol=1e-14, atol=1e-14)


def test_gelu_tanh_pins(orc):
    g = np.linspace(-8, 8, 3201)
    got = np.array([orc.gelu_tanh(v) for v in g])
    # the tanh form approximates the exact GELU g*Phi(g) to a few 1e-4
    exact = g * 0.5 * scipy.special.erfc(-g / np.sqrt(2))
    assert np.max(np.abs(got - exact)) < 1e-3
    # gelu(g) - gelu(-g) = g (tanh is odd; the clamp is symmetric)
    assert np.allclose(got - got[::-1], g, rtol=0, atol=1e-13)
    assert orc.gelu_tanh(0.0) == 0.0
    # past the clamp the value is 0.5*g*(1 + tanh(10)) (and tanh(10) is 1 in f32)
    for v in (12.0, 30.0, -12.0, -30.0):
        assert orc.gelu_tanh(v) == 0.5 * v * (1 + math.tanh(math.copysign(10.0, v)))


# --------------------------------------------------------------- router -----
def test_router_matches_stable_argsort(orc):
    E, k, T = 128, 8, 64
    lg = gs.logits(gs.rng(7), T, E)
    ids, w = orc.router_topk(lg, E, k, T)
    ref = np.argsort(-lg.astype(np.float64), axis=1, kind="stable")[:, :k]
    assert np.array_equal(ids, ref)
    top = np.take_along_axis(lg.astype(np.float64), ref, 1)
    p = np.exp(top - top[:, :1])
    assert np.allclose(w, p / p.sum(1, keepdims=True), rtol=1e-15, atol=0)
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)


def test_router_ties_lowest_index(orc):
    lg = np.zeros((1, 16), np.float32)
    lg[0, [3, 9, 12]] = 2.0
    lg[0, [1, 5]] = 1.0
    ids, w = orc.router_topk(lg, 16, 4, 1)
    assert list(ids[0]) == [3, 9, 12, 1]
    e = math.exp(-1.0)
    assert np.allclose(w[0], np.array([1, 1, 1, e]) / (3 + e), rtol=1e-15)


def test_router_closed_form_two_experts(orc):
    lg = np.array([[0.25, -1.5, 3.0, 0.0]], np.float32)
    ids, w = orc.router_topk(lg, 4, 2, 1)
    assert list(ids[0]) == [2, 0]
    w0 = 1.0 / (1.0 + math.exp(0.25 - 3.0))
    assert abs(w[0, 0] - w0) < 1e-15 and abs(w[0, 1] - (1 - w0)) < 1e-15


def test_router_nan_ranks_below_numbers(orc):
    """Reading of the router on NaN logits (the pages only softmax finite
    ones): a NaN ranks below every number, -inf included, and NaNs among
    themselves go lowest index first.  Checked against numpy's stable argsort
    of the key (NaN -> below -inf)."""
    lg = np.array([[np.nan, 1.0, -np.inf, np.nan, 0.5, -3.0, np.nan, 0.5]], np.float32)
    ids, w = orc.router_topk(lg, 8, 8, 1)
    assert list(ids[0]) == [1, 4, 7, 5, 2, 0, 3, 6]
    key = np.where(np.isnan(lg[0]), -np.inf, lg[0].astype(np.float64))
    order = [i for i in np.argsort(-key, kind="stable") if not np.isnan(lg[0, i])]
    order += [i for i in range(8) if np.isnan(lg[0, i])]
    assert list(ids[0]) == order
    # picks that hold no NaN keep the closed-form weights
    ids3, w3 = orc.router_topk(lg, 8, 3, 1)
    assert list(ids3[0]) == [1, 4, 7]
    e = math.exp(-0.5)
    assert np.allclose(w3[0], np.array([1, e, e]) / (1 + 2 * e), rtol=1e-15, atol=0)
    # a NaN at index 0 is not kept on top
    z = np.array([[np.nan, -1.0, 2.0]], np.float32)
    assert list(orc.router_topk(z, 3, 2, 1)[0][0]) == [2, 1]


# ------------------------------------------------------------------ MoE -----
def _tiny_moe(t, seed, E=6, H=64, F=64, k=2, T=3):
    g = gs.rng(seed)
    if t in (gs.Q4_K, gs.Q6_K):
        H, F = 256, 256
    pool, rec, gu_off, d_off = gs.expert_pool(t, g, E, H, F)
    lg = gs.logits(g, T, E)
    x = gs.activations(g, T, H)
    ds = gs.down_scales(g, E)
    return dict(pool=pool, rec=rec, gu_off=gu_off, d_off=d_off, lg=lg, x=x, ds=ds, E=E, H=H, F=F,
                k=k, T=T)


def _run_moe(orc, t, act, m, slots=None, pool=None, ds=False, want_gu=False):
    pool = m["pool"] if pool is None else pool
    slots = np.arange(m["E"], dtype=np.int32) if slots is None else slots
    return orc.moe_ffn(t, act, m["H"], m["F"], m["E"], pool[m["gu_off"]:], m["rec"],
                       pool[m["d_off"]:], m["rec"], m["ds"] if ds is False else ds, m["lg"], m["k"],
                       slots, m["x"], m["T"], want_gu=want_gu)


@pytest.mark.parametrize("t,act", [(gs.Q8_0, 0), (gs.Q4_0, 1), (gs.Q4_K, 0), (gs.Q6_K, 1)])
def test_moe_brute_force(orc, t, act):
    """The whole routed FFN recomputed in numpy from the second decoders,
    stable argsort and scipy's expit / the tanh GELU with its clamp."""
    m = _tiny_moe(t, 40 + t)
    r = _run_moe(orc, t, act, m)
    H, F, k, T, rec = m["H"], m["F"], m["k"], m["T"], m["rec"]
    for tt in range(T):
        lg = m["lg"][tt].astype(np.float64)
        ids = np.argsort(-lg, kind="stable")[:k]
        p = np.exp(lg[ids] - lg[ids[0]])
        c = p / p.sum()
        assert np.array_equal(r["ids"][tt], ids)
        y = np.zeros(H)
        for j, e in enumerate(ids):
            base = e * rec
            Wgu = dequant_matrix(t, m["pool"][base:base + m["d_off"]], 2 * F, H)
            Wd = dequant_matrix(t, m["pool"][base + m["d_off"]:base + rec], H, F)
            gu = Wgu @ m["x"][tt].astype(np.float64)
            gg, uu = gu[:F], gu[F:]
            if act == 0:
                a = gg * scipy.special.expit(gg) * uu
            else:
                z = np.clip(np.sqrt(2 / np.pi) * (gg + 0.044715 * gg ** 3), -10, 10)
                a = 0.5 * gg * (1 + np.tanh(z)) * uu
            y += (Wd @ a) * float(m["ds"][e]) * c[j]
        assert np.allclose(r["y"][tt], y, rtol=1e-9, atol=1e-9 * np.abs(y).max())


def test_moe_k1_reduces_to_dense_chain(orc):
    """k = 1 (weight 1, scale 1) is the plain dense MLP of the picked expert."""
    t = gs.Q8_0
    m = _tiny_moe(t, 60, k=1)
    r = _run_moe(orc, t, 0, m, ds=None)
    for tt in range(m["T"]):
        e = int(r["ids"][tt, 0])
        assert r["c"][tt, 0] == 1.0
        base = e * m["rec"]
        gu, _ = orc.gemv_f64(t, m["pool"][base:base + m["d_off"]], m["x"][tt].astype(np.float64),
                             2 * m["F"], m["H"])
        a = orc.glu(0, gu, m["F"])
        dn, _ = orc.gemv_f64(t, m["pool"][base + m["d_off"]:base + m["rec"]], a, m["H"], m["F"])
        assert np.array_equal(r["y"][tt], dn)


def test_moe_identical_experts_and_permutation(orc):
    t = gs.Q4_0
    m = _tiny_moe(t, 61, E=5, k=3)
    # identical experts: y = dense MLP * sum(c) = dense MLP
    same = np.tile(m["pool"][:m["rec"]], m["E"])
    r = _run_moe(orc, t, 1, m, pool=same, ds=None)
    gu, _ = orc.gemv_f64(t, same[:m["d_off"]], m["x"][0].astype(np.float64), 2 * m["F"], m["H"])
    dn, _ = orc.gemv_f64(t, same[m["d_off"]:m["rec"]], orc.glu(1, gu, m["F"]), m["H"], m["F"])
    assert np.allclose(r["y"][0], dn, rtol=1e-14, atol=1e-14 * np.abs(dn).max())
    # permuting where each expert lives (pool slots) together with expert_slots
    perm = np.array([3, 0, 4, 1, 2], np.int32)          # expert e lives in slot perm[e]
    pool2 = np.empty_like(m["pool"])
    for e in range(m["E"]):
        pool2[perm[e] * m["rec"]:(perm[e] + 1) * m["rec"]] = m["pool"][e * m["rec"]:(e + 1) * m["rec"]]
    r1 = _run_moe(orc, t, 1, m)
    r2 = _run_moe(orc, t, 1, m, slots=perm, pool=pool2)
    assert np.array_equal(r1["y"], r2["y"])


def test_moe_down_scale_and_absent(orc):
    t = gs.Q8_0
    m = _tiny_moe(t, 62)
    r1 = _run_moe(orc, t, 0, m, ds=np.ones(m["E"], np.float32))
    r2 = _run_moe(orc, t, 0, m, ds=np.full(m["E"], 2.0, np.float32))
    assert np.array_equal(r2["y"], 2 * r1["y"])
    r0 = _run_moe(orc, t, 0, m, ds=None)
    assert np.array_equal(r0["y"], r1["y"])
    # an absent pick skips the token (its row stays as it was: NaN here)
    slots = np.arange(m["E"], dtype=np.int32)
    slots[int(r1["ids"][1, 0])] = -1
    r3 = _run_moe(orc, t, 0, m, slots=slots)
    assert r3["skipped"] >= 1 and np.all(np.isnan(r3["y"][1]))


def test_moe_down_stage_matches_full(orc):
    """The down half fed with the oracle's own gate||up (cast to f32 only where
    exactly representable) reproduces the full FFN."""
    t = gs.Q8_0
    m = _tiny_moe(t, 63)
    r = _run_moe(orc, t, 0, m, want_gu=True)
    gu32 = r["gu"].astype(np.float32)
    y, A, R = orc.moe_down(t, 0, m["H"], m["F"], m["pool"][m["d_off"]:], m["rec"], m["ds"],
                           np.arange(m["E"], dtype=np.int32), r["ids"], r["c"], gu32, m["T"])
    # f32 rounding of gu perturbs y by at most ~ 2^-24 relative per input
    err = np.abs(y - r["y"])
    assert np.all(err <= 1e-6 * (A + R) + 1e-300)
    assert np.all(A > 0) and np.all(R > 0)


# --------------------------------------------------------------- golden -----
def _golden(name):
    vals = {}
    with open(os.path.join(HERE, "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    return vals


def test_golden_record_sizes(orc):
    """Record and block sizes the pages print, reproduced from the block byte
    counts the oracle uses."""
    gv = _golden("page_sizes.txt")
    H, F = 2048, 768                     # Qwen3-30B-A3B expert shape
    rec = (2 * F * H // 32) * orc.block_bytes(gs.Q8_0) + (H * F // 32) * orc.block_bytes(gs.Q8_0)
    assert rec == int(gv["qwen3_moe_expert_record_bytes"])
    assert int(gv["qwen3_moe_experts"]) * rec / 1e9 == pytest.approx(float(gv["qwen3_moe_experts_gb"]), abs=0.5)
    assert orc.block_bytes(gs.Q4_K) == int(gv["q4_k_block_bytes"])
    assert orc.block_bytes(gs.Q6_K) == int(gv["q6_k_block_bytes"])
    assert orc.block_values(gs.Q4_K) == int(gv["k_quant_block_values"])
    assert (orc.block_bytes(gs.Q4_K)) // 4 == int(gv["q4_k_words"])
    assert (orc.block_bytes(gs.Q6_K) + 2) // 4 == int(gv["q6_k_padded_words"])
    # Gemma-4 expert record from the same rule at its shape (Q4_0, H 2816, F 704)
    H4, F4 = 2816, 704
    rec4 = (2 * F4 * H4 // 32) * orc.block_bytes(gs.Q4_0) + (H4 * F4 // 32) * orc.block_bytes(gs.Q4_0)
    assert rec4 == 3345408


def test_golden_tanh_clamp_f32():
    """The gemma4 page notes that tanh at the clamp bound is exactly +-1 in f32."""
    assert np.float32(math.tanh(10.0)) == np.float32(1.0)
    assert np.float32(math.tanh(-10.0)) == np.float32(-1.0)


def test_generator_distributions():
    W = gs.q8_0(gs.rng(0), 64, 256).reshape(-1, 34)
    codes = W[:, 2:].view(np.int8)
    assert codes.min() >= -127 and codes.max() <= 127
    d = W[:, :2].copy().view(np.float16).astype(np.float64)
    assert np.all(d >= 0) and 0.01 < d.mean() < 0.02
    assert gs.row_bytes(gs.Q6_K, 17408) == 14280
    pool, rec, gu, dn = gs.expert_pool(gs.Q8_0, gs.rng(1), 2, 2048, 768)
    assert rec == 5013504 and dn == 3342336

"""Pins for the oracle's steps around the MoE block: f32 weights in the GEMV,
RMS norm, the logistic gate and the shared-expert combine, Gemma's FFN tail,
embedding rows, the logit soft cap and the greedy pick.

Each is checked against something other than its own formula: worked
examples computed by hand, closed forms, invariants, and numpy / scipy
routines for the cases that reduce to them.  No GPU.
"""
import math

import numpy as np
import pytest
import scipy.special

import gguf_synth as gs
from second_decoders import DEC


# ------------------------------------------------------------- f32 weights --
def test_f32_block_format(orc):
    assert orc.block_values(orc.F32) == 1 and orc.block_bytes(orc.F32) == 4
    v = gs.rng(1).standard_normal(37).astype(np.float32)
    v[3] = -0.0
    v[5] = np.float32(1e-40)  # subnormal
    got = orc.dequant(orc.F32, v.view(np.uint8), v.size)
    assert np.array_equal(got, v.astype(np.float64))
    assert math.copysign(1.0, got[3]) == -1.0


def test_f32_gemv_against_matmul(orc):
    """f32 weights: the oracle's GEMV equals numpy's f64 product of the same values."""
    g = gs.rng(2)
    W = g.standard_normal((9, 70)).astype(np.float32)
    x = g.standard_normal((3, 70)).astype(np.float32)
    y, A = orc.gemv(orc.F32, W.view(np.uint8), x, 9, 70, 3)
    ref = x.astype(np.float64) @ W.astype(np.float64).T
    assert np.allclose(y, ref, rtol=1e-14, atol=1e-13)
    assert np.allclose(A, np.abs(x.astype(np.float64)) @ np.abs(W.astype(np.float64)).T, rtol=1e-14)


def test_f32_gemv_integer_closed_form(orc):
    """Small integers: every product and sum is exact, so y is the integer result."""
    W = np.arange(-12, 12, dtype=np.float32).reshape(4, 6)
    x = np.array([1, -2, 3, 0, 5, -1], np.float32)
    y, _ = orc.gemv(orc.F32, W.view(np.uint8), x, 4, 6, 1)
    # row r holds -12+6r .. -7+6r; dot with x by hand:
    # sum(x) = 6, sum(c * x_c) = 0 - 2 + 6 + 0 + 20 - 5 = 19 -> y_r = (-12 + 6r) * 6 + 19
    assert y[0].tolist() == [(-12 + 6 * r) * 6 + 19 for r in range(4)]


# ------------------------------------------------------------------ norms ---
def test_rmsnorm_worked_example(orc):
    """x = (3, 4): mean of squares 12.5, r = 1/sqrt(12.5); w = (1, 2)."""
    y = orc.rmsnorm(np.array([3, 4], np.float32), np.array([1, 2], np.float32), 2, 1, 0.0)
    r = 1.0 / math.sqrt(12.5)
    assert y[0, 0] == pytest.approx(3 * r, rel=1e-15)
    assert y[0, 1] == pytest.approx(8 * r, rel=1e-15)
    # with the factor k (the router's 1/sqrt(H)) and eps
    y2 = orc.rmsnorm(np.array([3, 4], np.float32), np.array([1, 2], np.float32), 2, 1, 0.5, k=0.25)
    r2 = 1.0 / math.sqrt(13.0)
    assert y2[0].tolist() == pytest.approx([3 * r2 * 0.25, 8 * r2 * 0.25], rel=1e-15)


def test_rmsnorm_invariants(orc):
    g = gs.rng(3)
    n = 257
    x = g.standard_normal((4, n)).astype(np.float32)
    one = np.ones(n, np.float32)
    y = orc.rmsnorm(x, one, n, 4, 0.0)
    # unit weights, no eps: every token comes out with mean square 1
    assert np.allclose((y ** 2).mean(axis=1), 1.0, rtol=1e-13)
    # scale invariance (a power of two keeps the f32 input exact)
    y8 = orc.rmsnorm(x * np.float32(8.0), one, n, 4, 0.0)
    assert np.allclose(y8, y, rtol=1e-13)
    # tokens are independent, and the weight multiplies elementwise
    w = g.uniform(0.5, 2.0, n).astype(np.float32)
    yw = orc.rmsnorm(x, w, n, 4, 1e-6)
    for t in range(4):
        assert np.allclose(orc.rmsnorm(x[t], w, n, 1, 1e-6)[0], yw[t], rtol=0, atol=0)
    assert np.allclose(yw / w.astype(np.float64), orc.rmsnorm(x, one, n, 4, 1e-6), rtol=1e-14)
    # a zero vector stays zero while eps > 0
    assert np.array_equal(orc.rmsnorm(np.zeros(n, np.float32), w, n, 1, 1e-6), np.zeros((1, n)))


# ----------------------------------------------------- shared expert gate ---
def test_sigmoid_pins(orc):
    assert orc.sigmoid(0.0) == 0.5
    assert orc.sigmoid(math.log(3.0)) == pytest.approx(0.75, rel=1e-15)
    for v in (-30.0, -2.5, 0.1, 7.0):
        assert orc.sigmoid(v) + orc.sigmoid(-v) == pytest.approx(1.0, rel=1e-15)
        assert orc.sigmoid(v) == pytest.approx(scipy.special.expit(v), rel=1e-14)


def test_shared_combine_worked_example(orc):
    """Two picks with terms 1 and 2, shared output 4, a zero gate logit (sigmoid
    1/2) and residual 10: (1 + 2 + 4 * 0.5) + 10 = 15."""
    H = 3
    terms = np.array([[1, 1, 1], [2, 2, 2]], np.float32)
    sh = np.full(H, 4, np.float32)
    y, A, sg = orc.moe_shared_combine(terms, sh, np.zeros(H, np.float32), np.ones(H, np.float32),
                                      np.full(H, 10, np.float32), H, 1)
    assert y[0].tolist() == [15.0, 15.0, 15.0]
    assert sg[0] == 0.0
    assert A[0].tolist() == [1 + 2 + 2 + 10, 1 + 2 + 2 + 10, 1 + 2 + 2 + 10]


def test_shared_combine_reductions(orc):
    """Against numpy: the gate logit is a dot product, the routed part a sum over
    picks; a zero shared output leaves routed sum + residual."""
    g = gs.rng(4)
    T, k, H = 3, 5, 64
    terms = g.standard_normal((T, k, H)).astype(np.float32)
    sh = g.standard_normal((T, H)).astype(np.float32)
    gi = g.standard_normal(H).astype(np.float32)
    x = g.standard_normal((T, H)).astype(np.float32)
    r = g.standard_normal((T, H)).astype(np.float32)
    y, A, sg = orc.moe_shared_combine(terms, sh, gi, x, r, H, T)
    sg_ref = x.astype(np.float64) @ gi.astype(np.float64)
    assert np.allclose(sg, sg_ref, rtol=1e-13, atol=1e-13)
    gate = scipy.special.expit(sg_ref)[:, None]
    ref = terms.astype(np.float64).sum(axis=1) + sh * gate + r
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
    y0, _, _ = orc.moe_shared_combine(terms, np.zeros_like(sh), gi, x, r, H, T)
    assert np.allclose(y0, terms.astype(np.float64).sum(axis=1) + r, rtol=1e-13, atol=1e-13)
    assert (A >= np.abs(y - r) - 1e-12).all()


# -------------------------------------------------------- Gemma FFN tail ---
def test_post_ffn_constant_closed_form(orc):
    """Positive constant MLP and MoE outputs, unit norm weights, eps 0: each norm
    gives 1, their sum 2 normalises back to 1, so x' = (w + x) * os."""
    n = 40
    g = gs.rng(5)
    w = g.uniform(0.5, 1.5, n).astype(np.float32)
    x = g.standard_normal(n).astype(np.float32)
    one = np.ones(n, np.float32)
    y, _ = orc.post_ffn(np.full(n, 3.0, np.float32), np.full(n, 0.25, np.float32), one, one, w, 0.5, x,
                        n, 1, 0.0)
    assert np.allclose(y[0], (w.astype(np.float64) + x) * 0.5, rtol=1e-14, atol=1e-15)


def test_post_ffn_zero_moe_is_two_norms(orc):
    """With the MoE output zero (and eps > 0) the tail is the MLP's norm followed
    by a second norm: compare with chained rmsnorm calls."""
    n, T, eps = 96, 2, 1e-6
    g = gs.rng(6)
    mlp = g.standard_normal((T, n)).astype(np.float32)
    w1 = g.uniform(0.5, 2, n).astype(np.float32)
    w = g.uniform(0.5, 2, n).astype(np.float32)
    x = g.standard_normal((T, n)).astype(np.float32)
    y, A = orc.post_ffn(mlp, np.zeros((T, n), np.float32), w1, np.ones(n, np.float32), w, 2.0, x, n, T, eps)
    m = orc.rmsnorm(mlp, w1, n, T, eps)
    r = 1.0 / np.sqrt((m ** 2).mean(axis=1, keepdims=True) + eps)
    assert np.allclose(y, ((m * r) * w + x) * 2.0, rtol=1e-13, atol=1e-13)
    assert (A > 0).all()


# ---------------------------------------------------------- embedding rows --
@pytest.mark.parametrize("t", [gs.Q8_0, gs.Q4_0, gs.Q4_K, gs.Q6_K])
def test_embed_rows_match_second_decoder(orc, t):
    """Row gather = the second decoder's row, rounded to f32, times the scale in
    f32 (numpy's float32 multiply)."""
    g = gs.rng(10 + t)
    rows, cols = 6, 2 * gs.QK[t]
    W = gs.weights(t, g, rows, cols)
    tokens = np.array([5, 0, 5, 2], np.int32)
    full = DEC[t](W.ravel()).reshape(rows, cols)
    for scale in (1.0, float(np.float32(math.sqrt(2816.0)))):
        got = orc.embed(t, W, rows, cols, tokens, scale)
        ref = full[tokens].astype(np.float32) * np.float32(scale)
        assert got.dtype == np.float32 and np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_embed_hand_built_q8_0(orc):
    """A Q8_0 row of one block, d = 0.5 (f16 0x3800), codes 0..31 minus 16."""
    blk = np.zeros(34, np.uint8)
    blk[0:2] = np.array([0x00, 0x38], np.uint8)
    blk[2:] = (np.arange(32) - 16).astype(np.int8).view(np.uint8)
    got = orc.embed(gs.Q8_0, blk, 1, 32, np.array([0], np.int32), 1.0)
    assert got[0].tolist() == [(i - 16) * 0.5 for i in range(32)]


def test_embed_rejects_bad_token(orc):
    W = gs.weights(gs.Q8_0, gs.rng(1), 3, 32)
    with pytest.raises(ValueError):
        orc.embed(gs.Q8_0, W, 3, 32, np.array([3], np.int32))


# ---------------------------------------------------------------- head -----
def test_softcap_pins(orc):
    cap = 30.0
    l = np.array([0.0, 1e-3, -1e-3, 300.0, -1e6, 30.0, 15.0], np.float32)
    y = orc.softcap(l, cap)
    inv = np.float32(1.0 / cap)
    assert y[0] == 0.0
    # near zero tanh(a) ~ a: the soft cap is close to the identity
    assert y[1] == pytest.approx(1e-3, rel=1e-6) and y[2] == -y[1]
    # the clamp at |a| = 10, then tanh(10) * cap
    assert y[3] == pytest.approx(math.tanh(10.0) * cap, rel=1e-15)
    assert y[4] == pytest.approx(-math.tanh(10.0) * cap, rel=1e-15)
    # against numpy's tanh away from the clamp
    a = (l[5:].astype(np.float64) * np.float64(inv))
    assert np.allclose(y[5:], np.tanh(a) * cap, rtol=1e-15)


def test_argmax_against_numpy(orc):
    g = gs.rng(7)
    l = g.standard_normal((5, 1000)).astype(np.float32)
    assert orc.argmax(l, 1000, 5).tolist() == np.argmax(l, axis=1).tolist()


def test_argmax_ties_nan_and_degenerate(orc):
    l = np.array([[1, 3, 3, 2], [np.nan, -1, np.nan, -1], [np.nan] * 4, [-np.inf] * 4,
                  [-np.inf, -3.4028235e38, -np.inf, 0.0]], np.float32)
    # ties -> lowest index; NaN never wins; no number -> 0; all -inf -> 0
    assert orc.argmax(l, 4, 5).tolist() == [1, 1, 0, 0, 3]
    l2 = np.array([[-np.inf, -3.4028235e38, -np.inf, -np.inf]], np.float32)
    assert orc.argmax(l2, 4, 1).tolist() == [1]


# ------------------------------------------------------------- Q6_K planes --
from second_decoders import dec_q6_k_planes  # noqa: E402


@pytest.mark.parametrize("n", [1, 3, 68])
def test_q6k_planes_decode_as_the_blocks(orc, n):
    """The plane layout read by a second decoder written from the page's plane
    indexer (words of each plane) gives the blocks' values exactly."""
    W = gs.weights(orc.Q6_K, gs.rng(40 + n), 1, 256 * n)
    P = orc.q6k_planes(W, n)
    assert P.size == W.size
    assert np.array_equal(dec_q6_k_planes(P, n), orc.dequant(orc.Q6_K, W, 256 * n))


def test_q6k_planes_worked_offsets(orc):
    """Two blocks whose bytes name their own place: block b, byte j holds
    (j + 101 b) mod 256.  Each plane's entries sit where the layout says."""
    n = 2
    W = np.array([(j + 101 * b) % 256 for b in range(n) for j in range(210)], np.uint8)
    P = orc.q6k_planes(W, n)
    byte = lambda b, j: (j + 101 * b) % 256  # noqa: E731
    assert P[128 * 1 + 5] == byte(1, 5)                  # ql of block 1
    assert P[128 * n + 64 * 1 + 0] == byte(1, 128)       # qh of block 1
    assert P[128 * n + 63] == byte(0, 191)               # last qh byte of block 0
    assert P[192 * n + 16 * 1 + 15] == byte(1, 207)      # last scale of block 1
    assert P[208 * n + 0] == byte(0, 208) and P[208 * n + 3] == byte(1, 209)   # d bytes
    # a permutation of the bytes, undone by the inverse
    assert np.array_equal(np.sort(P), np.sort(W))
    assert np.array_equal(orc.q6k_unplanes(P, n), W)


def test_q6k_planes_round_trip_random(orc):
    W = gs.rng(44).integers(0, 256, 210 * 37, dtype=np.uint8)
    assert np.array_equal(orc.q6k_unplanes(orc.q6k_planes(W, 37), 37), W)


# ------------------------------------------------------------- Q8_0 planes --
from second_decoders import dec_q8_0_planes  # noqa: E402


@pytest.mark.parametrize("n", [1, 5, 80])
def test_q8_0_planes_decode_as_the_blocks(orc, n):
    """The code and scale planes read by the page's word-wise code-plane
    indexer give the blocks' values exactly."""
    W = gs.weights(orc.Q8_0, gs.rng(60 + n), 1, 32 * n)
    P = orc.q8_0_planes(W, n)
    assert P.size == W.size
    assert np.array_equal(dec_q8_0_planes(P, n), orc.dequant(orc.Q8_0, W, 32 * n))


def test_q8_0_planes_worked_offsets(orc):
    """Three blocks whose bytes name their own place (block b, byte j holds
    (j + 77 b) mod 256): codes row-major at 32 b + j - 2, scales after."""
    n = 3
    W = np.array([(j + 77 * b) % 256 for b in range(n) for j in range(34)], np.uint8)
    P = orc.q8_0_planes(W, n)
    byte = lambda b, j: (j + 77 * b) % 256  # noqa: E731
    assert P[0] == byte(0, 2) and P[31] == byte(0, 33) and P[32 * 2 + 5] == byte(2, 7)
    assert P[32 * n + 0] == byte(0, 0) and P[32 * n + 5] == byte(2, 1)
    assert np.array_equal(np.sort(P), np.sort(W))
    assert np.array_equal(orc.q8_0_unplanes(P, n), W)

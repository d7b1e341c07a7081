"""GPU parity of the plane layouts (QG_Q6_K_PLANES, QG_Q8_0_PLANES) through
the C ABI: the planes qg_prepare writes equal the oracle's byte for byte,
from blocks at either 2-byte phase; qg_unprepare gives the blocks back byte
for byte; dequantized values from the planes are bit-exact against the
oracle over the blocks; one-token GEMV rows from the planes are within
1e-5 * sum |w x| of the oracle over the blocks (several tiles, ragged tails,
odd blocks per row, rows not a multiple of the waves, and the full-size
shapes the GEMVs are measured at, on sampled rows)."""
import numpy as np
import pytest

import gguf_synth as gs
from test_gpu_parity import _torch, check_rows, dev, host, say

pytestmark = pytest.mark.gpu

P = 270   # QG_Q6_K_PLANES
P8 = 264  # QG_Q8_0_PLANES

SHAPES = [(1, 256), (3, 768), (45, 1280), (77, 2816), (129, 4352), (33, 17408), (600, 2816)]


def _prepared(W, rows, cols):
    """(device planes tensor, its pointer) for host blocks W."""
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    Wt, Wp = dev(W)
    Pt = torch.empty(W.size, dtype=torch.uint8, device="cuda")
    qg.qg_prepare(gs.Q6_K, Wp, Pt, rows, cols)
    return Pt, Wt


@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("off", [0, 2])
def test_prepare_bytes_and_round_trip(orc, rows, cols, off):
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    W = gs.weights(gs.Q6_K, gs.rng(5100 + rows + off), rows, cols)
    n = rows * cols // 256
    say("q6_k planes", rows, cols, "blocks offset", off)
    Wt, Wp = dev(W, off)
    Pt = torch.full((W.size,), 0xA5, dtype=torch.uint8, device="cuda")
    qg.qg_prepare(gs.Q6_K, Wp, Pt, rows, cols)
    got = host(Pt)
    assert np.array_equal(got, orc.q6k_planes(W, n))
    back = torch.full((W.size + 16,), 0x5A, dtype=torch.uint8, device="cuda")
    qg.qg_unprepare(gs.Q6_K, Pt, back.data_ptr() + off, rows, cols)
    b = host(back)
    assert np.array_equal(b[off:off + W.size], W.ravel())
    # nothing written outside the blocks
    assert (b[:off] == 0x5A).all() and (b[off + W.size:] == 0x5A).all()


@pytest.mark.parametrize("rows,cols", SHAPES[:5])
def test_planes_dequant_bit_exact(orc, rows, cols):
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    W = gs.weights(gs.Q6_K, gs.rng(5200 + rows), rows, cols)
    say("q6_k planes dequant", rows, cols)
    Pt, Wt = _prepared(W, rows, cols)
    out = torch.full((rows, cols), float("nan"), dtype=torch.float32, device="cuda")
    qg.qg_dequant(P, Pt, out, rows, cols)
    got = host(out)
    ref = orc.dequant(gs.Q6_K, W, rows * cols).reshape(rows, cols).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_planes_gemv_one_token(orc, rows, cols):
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    plan = qg.qg_gemv_plan(P, rows, cols, 1)
    assert plan["kind"] == 4, plan
    g = gs.rng(5300 + rows + cols)
    W = gs.weights(gs.Q6_K, g, rows, cols)
    x = gs.activations(g, 1, cols)
    say("q6_k planes gemv", rows, cols, plan)
    Pt, Wt = _prepared(W, rows, cols)
    xt, xp = dev(x)
    y = torch.full((1, rows), float("nan"), dtype=torch.float32, device="cuda")
    qg.qg_gemv(P, Pt, xp, y, rows, cols, 1)
    yh = host(y)
    y_ref, A = orc.gemv(gs.Q6_K, W, x, rows, cols, 1)
    check_rows(yh, y_ref, A, "planes gemv %dx%d" % (rows, cols))


def _sample(g, rows, n):
    idx = set(g.choice(rows, size=min(n, rows), replace=False).tolist())
    idx.update(range(40))
    idx.update(range(rows - 40, rows))
    return np.array(sorted(idx), dtype=np.int64)


@pytest.mark.parametrize("rows,cols", [(5120, 17408), (262144, 2816)])
def test_planes_gemv_full_size(orc, rows, cols):
    """The shapes the Q6_K GEMV and the Gemma-style head are measured at, on
    sampled rows (the first and last 40 among them)."""
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    g = gs.rng(5400 + rows)
    W = gs.weights(gs.Q6_K, g, rows, cols)
    x = gs.activations(g, 1, cols)
    say("q6_k planes gemv full", rows, cols, qg.qg_gemv_plan(P, rows, cols, 1))
    Pt, Wt = _prepared(W, rows, cols)
    del Wt
    xt, xp = dev(x)
    y = torch.full((1, rows), float("nan"), dtype=torch.float32, device="cuda")
    qg.qg_gemv(P, Pt, xp, y, rows, cols, 1)
    yh = host(y)
    ri = _sample(g, rows, 800)
    y_ref, A = orc.gemv(gs.Q6_K, W, x, rows, cols, 1, row_idx=ri)
    check_rows(yh[:, ri], y_ref, A, "planes gemv %dx%d" % (rows, cols))
    assert np.isfinite(yh).all()


# ------------------------------------------------------------------ Q8_0 ----
# (rows, cols): a 16-byte piece count per row below, at and past 64 lanes, a
# ragged last slot (cols / 16 not a multiple of 64), odd blocks per row, rows
# below one per wave and far past the resident waves
Q8_SHAPES = [(1, 32), (3, 96), (45, 1024), (77, 2560), (129, 1056), (1000, 2048), (33, 9728), (20000, 2560),
             # 8, 10, 12 (x in 12 float4 a thread), 14 and 16 waves a workgroup, last workgroups ragged
             (1500, 64), (2100, 512), (2500, 12288), (3300, 256), (4096, 320)]


def _prepared8(W, rows, cols):
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    Wt, Wp = dev(W)
    Pt = torch.empty(W.size, dtype=torch.uint8, device="cuda")
    qg.qg_prepare(gs.Q8_0, Wp, Pt, rows, cols)
    return Pt, Wt


@pytest.mark.parametrize("rows,cols", Q8_SHAPES[:6])
@pytest.mark.parametrize("off", [0, 2])
def test_q8_prepare_bytes_and_round_trip(orc, rows, cols, off):
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    W = gs.weights(gs.Q8_0, gs.rng(6100 + rows + off), rows, cols)
    n = rows * cols // 32
    say("q8_0 planes", rows, cols, "blocks offset", off)
    Wt, Wp = dev(W, off)
    Pt = torch.full((W.size,), 0xA5, dtype=torch.uint8, device="cuda")
    qg.qg_prepare(gs.Q8_0, Wp, Pt, rows, cols)
    assert np.array_equal(host(Pt), orc.q8_0_planes(W, n))
    back = torch.full((W.size + 16,), 0x5A, dtype=torch.uint8, device="cuda")
    qg.qg_unprepare(gs.Q8_0, Pt, back.data_ptr() + off, rows, cols)
    b = host(back)
    assert np.array_equal(b[off:off + W.size], W.ravel())
    assert (b[:off] == 0x5A).all() and (b[off + W.size:] == 0x5A).all()


@pytest.mark.parametrize("rows,cols", Q8_SHAPES[:5])
def test_q8_planes_dequant_bit_exact(orc, rows, cols):
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    W = gs.weights(gs.Q8_0, gs.rng(6200 + rows), rows, cols)
    say("q8_0 planes dequant", rows, cols)
    Pt, Wt = _prepared8(W, rows, cols)
    out = torch.full((rows, cols), float("nan"), dtype=torch.float32, device="cuda")
    qg.qg_dequant(P8, Pt, out, rows, cols)
    ref = orc.dequant(gs.Q8_0, W, rows * cols).reshape(rows, cols).astype(np.float32)
    assert np.array_equal(host(out).view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("rows,cols", Q8_SHAPES)
def test_q8_planes_gemv_one_token(orc, rows, cols):
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    plan = qg.qg_gemv_plan(P8, rows, cols, 1)
    assert plan["kind"] == 5, plan
    g = gs.rng(6300 + rows + cols)
    W = gs.weights(gs.Q8_0, g, rows, cols)
    x = gs.activations(g, 1, cols)
    say("q8_0 planes gemv", rows, cols, plan)
    Pt, Wt = _prepared8(W, rows, cols)
    xt, xp = dev(x)
    y = torch.full((1, rows), float("nan"), dtype=torch.float32, device="cuda")
    qg.qg_gemv(P8, Pt, xp, y, rows, cols, 1)
    yh = host(y)
    if rows * cols <= 4 * 10 ** 6:
        y_ref, A = orc.gemv(gs.Q8_0, W, x, rows, cols, 1)
        check_rows(yh, y_ref, A, "q8_0 planes gemv %dx%d" % (rows, cols))
    else:
        ri = _sample(g, rows, 800)
        y_ref, A = orc.gemv(gs.Q8_0, W, x, rows, cols, 1, row_idx=ri)
        check_rows(yh[:, ri], y_ref, A, "q8_0 planes gemv %dx%d" % (rows, cols))
    assert np.isfinite(yh).all()


@pytest.mark.parametrize("rows,cols", [(151936, 2560), (2560, 9728)])
def test_q8_planes_gemv_full_size(orc, rows, cols):
    """The tied head and the dense down projection of the Qwen3-style step,
    on sampled rows (the first and last 40 among them), with the workgroups
    of one launch each walking many rows."""
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    g = gs.rng(6400 + rows)
    W = gs.weights(gs.Q8_0, g, rows, cols)
    x = gs.activations(g, 1, cols)
    say("q8_0 planes gemv full", rows, cols, qg.qg_gemv_plan(P8, rows, cols, 1, query_device=True))
    Pt, Wt = _prepared8(W, rows, cols)
    del Wt
    xt, xp = dev(x)
    y = torch.full((1, rows), float("nan"), dtype=torch.float32, device="cuda")
    qg.qg_gemv(P8, Pt, xp, y, rows, cols, 1)
    yh = host(y)
    ri = _sample(g, rows, 1200)
    y_ref, A = orc.gemv(gs.Q8_0, W, x, rows, cols, 1, row_idx=ri)
    check_rows(yh[:, ri], y_ref, A, "q8_0 planes gemv %dx%d" % (rows, cols))
    assert np.isfinite(yh).all()


@pytest.mark.parametrize("act,H,F", [(0, 2560, 9728), (1, 2816, 2112), (0, 96, 64), (1, 12288, 160)])
def test_q8_planes_mlp_stagewise(orc, act, H, F):
    """qg_mlp over three Q8_0 plane tensors, one token, stage by stage: the
    gate and up sums (kept in the workspace) and the activation against the
    oracle, and the down projection fed the GPU's own activation."""
    import gguf_dequant_gemv_amd as qg
    from test_gpu_parity import TOL, _align256, check_act
    torch = _torch()
    g = gs.rng(6500 + H + F)
    Wg, Wu, Wd = gs.weights(gs.Q8_0, g, F, H), gs.weights(gs.Q8_0, g, F, H), gs.weights(gs.Q8_0, g, H, F)
    x = gs.activations(g, 1, H)
    say("q8_0 planes mlp", "act", act, H, F)
    Pg, tg = _prepared8(Wg, F, H)
    Pu, tu = _prepared8(Wu, F, H)
    Pd, td = _prepared8(Wd, H, F)
    xt, _ = dev(x)
    y = torch.full((1, H), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(qg.qg_mlp_workspace_size(P8, H, F, 1) // 4, dtype=torch.float32, device="cuda")
    qg.qg_mlp(P8, act, Pg, Pu, Pd, H, F, xt, y, 1, ws)
    wsh = host(ws)
    gu = wsh[:2 * F].reshape(1, 2 * F)
    a0 = _align256(2 * F * 4) // 4
    check_act(orc, act, gu, wsh[a0:a0 + F].reshape(1, F), F, "planes mlp act")
    yg, Ag = orc.gemv(gs.Q8_0, Wg, x, F, H, 1)
    yu, Au = orc.gemv(gs.Q8_0, Wu, x, F, H, 1)
    check_rows(gu, np.concatenate([yg, yu], 1), np.concatenate([Ag, Au], 1), "planes mlp gate||up")
    yh = host(y)
    a = orc.glu(act, gu[0], F)
    yd, Ad = orc.gemv_f64(gs.Q8_0, Wd, a, H, F)
    R = np.abs(orc.dequant(gs.Q8_0, Wd, H * F).reshape(H, F)) @ np.abs(
        gu[0, :F].astype(np.float64) * gu[0, F:].astype(np.float64))
    err = np.abs(yh[0] - yd)
    assert np.all(err <= TOL * Ad + 1e-6 * R), "planes mlp down: worst err/A %.3g" % (err / Ad).max()


@pytest.mark.parametrize("t,rows,cols", [(gs.Q8_0, 300, 2560), (gs.Q8_0, 7, 96), (gs.Q6_K, 300, 2816), (gs.Q6_K, 5, 256)])
def test_planes_embed_and_argmax_embed(orc, t, rows, cols):
    """Embedding rows from a plane table equal the GGUF table's bit for bit
    (ids in range, and one past the end giving NaN), and the fused pick and
    gather on the planes picks the same token and row as on the blocks."""
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    P_ = P8 if t == gs.Q8_0 else P
    g = gs.rng(6600 + t + rows)
    W = gs.weights(t, g, rows, cols)
    say("planes embed", gs.NAMES[t], rows, cols)
    Pt, Wt = (_prepared8 if t == gs.Q8_0 else _prepared)(W, rows, cols)
    ids = np.array([0, rows - 1, rows // 2, rows], dtype=np.int32)
    it, _ = dev(ids)
    a = torch.empty((4, cols), dtype=torch.float32, device="cuda")
    b = torch.empty((4, cols), dtype=torch.float32, device="cuda")
    qg.qg_embed(t, Wt, rows, cols, it, 4, 1.5, a)
    qg.qg_embed(P_, Pt, rows, cols, it, 4, 1.5, b)
    ah, bh = host(a), host(b)
    assert np.array_equal(ah[:3].view(np.uint32), bh[:3].view(np.uint32))
    assert np.isnan(bh[3]).all()
    ref = orc.embed(t, W, rows, cols, ids[:3], 1.5)
    assert np.array_equal(bh[:3].astype(np.float64), np.asarray(ref).reshape(3, cols))
    # the fused pick over the table's logits (a cap of 30, one clear winner)
    # and the gather of that row
    n, spike = rows, rows // 3
    lg = g.standard_normal((1, n)).astype(np.float32) * 3
    lg[0, spike] = 50.0
    l1, _ = dev(lg)
    l2, _ = dev(lg)
    i1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    i2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(qg.qg_argmax_workspace_size(n, 1) // 4, dtype=torch.float32, device="cuda")
    e1 = torch.empty((1, cols), dtype=torch.float32, device="cuda")
    e2 = torch.empty((1, cols), dtype=torch.float32, device="cuda")
    qg.qg_argmax_embed(l1, n, 1, 30.0, i1, ws, t, Wt, rows, cols, 0.5, e1)
    qg.qg_argmax_embed(l2, n, 1, 30.0, i2, ws, P_, Pt, rows, cols, 0.5, e2)
    assert int(host(i1)[0]) == spike and int(host(i2)[0]) == spike
    assert np.array_equal(host(e1).view(np.uint32), host(e2).view(np.uint32))

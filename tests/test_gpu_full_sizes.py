"""GPU parity at the workloads' full sizes, through the same entry points and
with the same device allocations the bench times.  The oracle computes sampled
rows one by one (plus every row where that is cheap); the bar is the same as
in test_gpu_parity: |y - y_ref| <= 1e-5 * sum|W x| per row, stage by stage,
each stage fed the GPU's own input.
"""
import numpy as np
import pytest

import gguf_synth as gs
from test_gpu_parity import TOL, _torch, check_act, check_rows, dev, host, say, _align256

pytestmark = pytest.mark.gpu


def sample_rows(g, rows, n):
    """n seeded rows, always including the first and the last (the ragged tile)."""
    idx = set(g.choice(rows, size=min(n, rows), replace=False).tolist())
    idx.update({0, rows - 1})
    return np.array(sorted(idx), dtype=np.int64)


def gemv_gpu(t, Wt, xt, rows, cols, T):
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    y = torch.full((T, rows), float("nan"), dtype=torch.float32, device="cuda")
    qg.qg_gemv(t, Wt, xt, y, rows, cols, T)
    return host(y)


def test_q8_0_gemv_1024x2048_every_row(orc):
    t, rows, cols = gs.Q8_0, 1024, 2048
    c = gs.config0(seed=0)
    say("full q8_0 gemv", rows, cols)
    Wt, _ = dev(c["W"])
    xt, _ = dev(c["x"])
    y = gemv_gpu(t, Wt, xt, rows, cols, 1)
    yr, A = orc.gemv(t, c["W"], c["x"], rows, cols, 1)
    check_rows(y, yr, A, "q8_0 1024x2048")


def test_dense_mlp_2560x9728_and_head_151936(orc):
    """The dense Qwen3-style chain at Q8_0, one token: gate||up -> SwiGLU ->
    down (qg_mlp), then the tied head on the GPU's down output (qg_gemv)."""
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    c = gs.config1(seed=0)
    t, H, F, V = gs.Q8_0, c["H"], c["F"], c["head_rows"]
    say("full dense mlp", H, F, "head", V)
    tg, _ = dev(c["Wg"])
    tu, _ = dev(c["Wu"])
    td, _ = dev(c["Wd"])
    xt, _ = dev(c["x"])
    h = torch.full((1, H), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(qg.qg_mlp_workspace_size(t, H, F, 1) // 4, dtype=torch.float32, device="cuda")
    qg.qg_mlp(t, qg.QG_ACT_SILU, tg, tu, td, H, F, xt, h, 1, ws)
    wsh = host(ws)
    gu = wsh[:2 * F].reshape(1, 2 * F)
    a0 = _align256(2 * F * 4) // 4
    act = wsh[a0:a0 + F].reshape(1, F)
    g = gs.rng(11)
    # gate and up rows, sampled
    ri = sample_rows(g, F, 384)
    yg, Ag = orc.gemv(t, c["Wg"], c["x"], F, H, 1, row_idx=ri)
    yu, Au = orc.gemv(t, c["Wu"], c["x"], F, H, 1, row_idx=ri)
    check_rows(gu[:, ri], yg, Ag, "gate rows")
    check_rows(gu[:, F + ri], yu, Au, "up rows")
    # activation, every element
    check_act(orc, 0, gu, act, F, "silu(g)*u")
    # down on the GPU's activation, every row
    hh = host(h)
    yd, Ad = orc.gemv(t, c["Wd"], act, H, F, 1)
    check_rows(hh, yd, Ad, "down")
    # head on the GPU's h, sampled rows
    Wh = c["Wh"]
    th, _ = dev(Wh)
    ht, _ = dev(hh)
    logits = gemv_gpu(t, th, ht, V, H, 1)
    rh = sample_rows(g, V, 1024)
    yh, Ah = orc.gemv(t, Wh, hh, V, H, 1, row_idx=rh)
    check_rows(logits[:, rh], yh, Ah, "head")
    assert np.isfinite(logits).all()


@pytest.mark.parametrize("which", ["q4_k", "q6_k"])
def test_kquant_gemv_full(orc, which):
    c = gs.config3(seed=0)
    if which == "q4_k":
        t, W, x, rows, cols = gs.Q4_K, c["W4"], c["x4"], 17408, 5120
    else:
        t, W, x, rows, cols = gs.Q6_K, c["W6"], c["x6"], 5120, 17408
    say("full", which, rows, cols)
    Wt, _ = dev(W)
    xt, _ = dev(x)
    y = gemv_gpu(t, Wt, xt, rows, cols, 1)
    ri = sample_rows(gs.rng(12), rows, 768)
    yr, A = orc.gemv(t, W, x, rows, cols, 1, row_idx=ri)
    check_rows(y[:, ri], yr, A, which)
    assert np.isfinite(y).all()


def _grid_stride_rows(plan, rows, g, n=400):
    """Rows to check in a grid-stride launch: the first and last 40, seeded
    random rows, and rows from the last tile that several workgroups walk
    (workgroup w takes tiles w, w + grid, ...)."""
    tile_rows = 4 * (64 // plan["lanes_per_row"])
    gx, tiles = plan["workgroups"], plan["row_tiles"]
    assert 0 < gx < tiles, "the launch must give some workgroup more than one tile: %r" % plan
    idx = set(range(40)) | set(range(rows - 40, rows))
    idx |= set(g.choice(rows, size=n, replace=False).tolist())
    for wg in sorted({0, 1, gx // 2, gx - 2, gx - 1}):
        last = wg + ((tiles - 1 - wg) // gx) * gx
        assert last > wg, "workgroup %d walks one tile only" % wg
        r0 = last * tile_rows
        idx |= {min(r0 + j, rows - 1) for j in (0, 1, tile_rows // 2, tile_rows - 1)}
    return np.array(sorted(idx), dtype=np.int64)


@pytest.mark.parametrize("t,rows,cols", [
    # odd Q8_0 block count (per-lane kernel, single blocks), ragged last tile
    (gs.Q8_0, 150001, 33 * 32)])
def test_gemv_multi_tile_workgroups(orc, t, rows, cols):
    """The per-lane kernel's loop over several row tiles per workgroup, which
    runs when the tiles outnumber the workgroups resident at once."""
    import gguf_dequant_gemv_amd as qg
    plan = qg.qg_gemv_plan(t, rows, cols, 1, True, True)
    say("multi-tile gemv", gs.NAMES[t], rows, cols, plan)
    assert plan["kind"] == 0
    g = gs.rng(40 + t)
    W = gs.weights(t, g, rows, cols)
    x = gs.activations(g, 1, cols)
    Wt, _ = dev(W)
    xt, _ = dev(x)
    y = gemv_gpu(t, Wt, xt, rows, cols, 1)
    del Wt
    ri = _grid_stride_rows(plan, rows, g)
    yr, A = orc.gemv(t, W, x, rows, cols, 1, row_idx=ri)
    check_rows(y[:, ri], yr, A, "%s %dx%d multi-tile" % (gs.NAMES[t], rows, cols))
    assert np.isfinite(y).all()


def test_kquant_head_many_rounds(orc):
    """The Q6_K head shape (262144 x 2816) on the quarter-block kernel: many
    more workgroups than are resident at once; the first and last 40 rows and
    seeded random rows against the oracle."""
    import gguf_dequant_gemv_amd as qg
    t, rows, cols = gs.Q6_K, 262144, 2816
    plan = qg.qg_gemv_plan(t, rows, cols, 1, True, True)
    say("q6_k head one token", rows, cols, plan)
    assert plan["kind"] == 4 and plan["workgroups"] > 256 * 8
    g = gs.rng(46)
    W = gs.weights(t, g, rows, cols)
    x = gs.activations(g, 1, cols)
    Wt, _ = dev(W)
    xt, _ = dev(x)
    y = gemv_gpu(t, Wt, xt, rows, cols, 1)
    del Wt
    ri = np.array(sorted(set(range(40)) | set(range(rows - 40, rows)) |
                         set(g.choice(rows, size=600, replace=False).tolist())), dtype=np.int64)
    yr, A = orc.gemv(t, W, x, rows, cols, 1, row_idx=ri)
    check_rows(y[:, ri], yr, A, "q6_k head")
    assert np.isfinite(y).all()


def test_mlp_gate_up_x_chunks(orc):
    """A gated launch whose x (24576 wide) is staged in chunks and whose row
    tiles need more than one round: every tile row walks the chunks twice
    (gate rows, then up rows).  Sampled gate / up rows, every activation, and
    sampled down rows fed the GPU's activations."""
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    t, H, F = gs.Q8_0, 24576, 4128
    g = gs.rng(31)
    Wg, Wu, Wd = gs.weights(t, g, F, H), gs.weights(t, g, F, H), gs.weights(t, g, H, F)
    x = gs.activations(g, 1, H)
    say("mlp x chunks", H, F)
    tg, tu, td = dev(Wg)[0], dev(Wu)[0], dev(Wd)[0]
    xt, _ = dev(x)
    y = torch.full((1, H), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(qg.qg_mlp_workspace_size(t, H, F, 1) // 4, dtype=torch.float32, device="cuda")
    qg.qg_mlp(t, qg.QG_ACT_SILU, tg, tu, td, H, F, xt, y, 1, ws)
    wsh = host(ws)
    gu = wsh[:2 * F].reshape(1, 2 * F)
    a0 = _align256(2 * F * 4) // 4
    act = wsh[a0:a0 + F].reshape(1, F)
    ri = sample_rows(gs.rng(32), F, 300)
    yg, Ag = orc.gemv(t, Wg, x, F, H, 1, row_idx=ri)
    yu, Au = orc.gemv(t, Wu, x, F, H, 1, row_idx=ri)
    check_rows(gu[:, ri], yg, Ag, "gate rows")
    check_rows(gu[:, F + ri], yu, Au, "up rows")
    check_act(orc, 0, gu, act, F, "silu(g)*u")
    # down rows on the GPU's activation, with the activation's rounding term
    rd = sample_rows(gs.rng(33), H, 300)
    yd, Ad = orc.gemv(t, Wd, act, H, F, 1, row_idx=rd)
    rb = gs.row_bytes(t, F)
    gabs = np.abs(gu[0, :F].astype(np.float64) * gu[0, F:].astype(np.float64))
    R = np.array([np.abs(orc.dequant(t, Wd[r * rb:(r + 1) * rb] if Wd.ndim == 1 else Wd[r], F)) @ gabs for r in rd])
    err = np.abs(host(y)[0, rd] - yd[0])
    assert np.all(err <= TOL * Ad[0] + 1e-6 * R), "down rows: worst err/A %.3g" % (err / Ad[0]).max()

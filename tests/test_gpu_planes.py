"""GPU parity of the Q6_K plane layout (QG_Q6_K_PLANES) through the C ABI:
the planes qg_prepare writes equal the oracle's byte for byte, from blocks at
either 2-byte phase; qg_unprepare gives the blocks back byte for byte;
dequantized values from the planes are bit-exact against the oracle over the
blocks; one-token GEMV rows from the planes are within 1e-5 * sum |w x| of the
oracle over the blocks (several tiles, ragged tails, odd blocks per row, the
full 5120 x 17408 and 262144 x 2816 shapes on sampled rows)."""
import numpy as np
import pytest

import gguf_synth as gs
from test_gpu_parity import _torch, check_rows, dev, host, say

pytestmark = pytest.mark.gpu

P = 270   # QG_Q6_K_PLANES

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

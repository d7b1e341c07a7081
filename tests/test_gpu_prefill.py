"""GPU parity of prefill-size products (qg_gemm, and qg_mlp over a prompt
chunk) against the f64 oracle: T = 17..256 tokens, every block type and f32,
ragged row tiles and token chunks, 2-byte-offset weights; the bar is the same
|y - y_ref| <= 1e-5 * sum |W x| per row and token."""
import numpy as np
import pytest

import gguf_synth as gs
from test_gpu_parity import TOL, _align256, _torch, check_act, check_rows, dev, host, say

pytestmark = pytest.mark.gpu

TYPES = [gs.Q8_0, gs.Q4_0, gs.Q4_K, gs.Q6_K]


def gpu_gemm(t, W, x, rows, cols, ntok, w_offset=0):
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    Wt, Wp = dev(W, w_offset)
    xt, _ = dev(x.astype(np.float32))
    y = torch.full((ntok, rows), float("nan"), dtype=torch.float32, device="cuda")
    nws = qg.qg_gemm_workspace_size(t, rows, cols, ntok)
    ws = torch.full((max(nws, 4) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    qg.qg_gemm(t, Wp, xt, y, rows, cols, ntok, ws if nws else None)
    return host(y)


@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("rows,nbk,ntok,off", [(300, 32, 17, 0), (129, 24, 64, 2), (257, 16, 100, 0),
                                               (70, 40, 256, 0), (33, 8, 40, 2),
                                               # 4..16 tokens (Q8_0 / Q4_0 rows split over
                                               # workgroups).  Under a quarter of the CUs'
                                               # worth of tiles: 10 tiles, 13 splits of 16
                                               # with a short last one; 2 tiles, 16 splits of
                                               # 16 with a short last one.  66 tiles: 7 splits
                                               # of 32 with a short last one.  A short row
                                               # left whole.
                                               (300, 200, 8, 0), (33, 250, 16, 2), (2100, 200, 8, 2),
                                               (129, 24, 5, 2)])
def test_gemm_parity(orc, t, rows, nbk, ntok, off):
    if t in (gs.Q4_K, gs.Q6_K):
        nbk = max(1, nbk // 8)
    cols = nbk * gs.QK[t]
    g = gs.rng(8000 + 31 * t + rows + ntok)
    W = gs.weights(t, g, rows, cols)
    x = gs.activations(g, ntok, cols)
    say("gemm", gs.NAMES[t], rows, cols, "T", ntok, "offset", off)
    y = gpu_gemm(t, W, x, rows, cols, ntok, off)
    y_ref, A = orc.gemv(t, W, x, rows, cols, ntok)
    check_rows(y, y_ref, A, "gemm %s %dx%d T=%d" % (gs.NAMES[t], rows, cols, ntok))


@pytest.mark.parametrize("rows,cols,ntok", [(130, 2048, 40), (256, 2816, 256)])
def test_gemm_f32(orc, rows, cols, ntok):
    g = gs.rng(8100 + ntok)
    W = gs.f32_matrix(g, rows, cols, 0.02)
    x = gs.activations(g, ntok, cols)
    say("gemm f32", rows, cols, "T", ntok)
    y = gpu_gemm(0, W.view(np.uint8), x, rows, cols, ntok)
    y_ref, A = orc.gemv(orc.F32, W.view(np.uint8), x, rows, cols, ntok)
    check_rows(y, y_ref, A, "gemm f32")


@pytest.mark.parametrize("t,act,H,F,T", [(gs.Q8_0, 0, 512, 768, 64), (gs.Q4_0, 1, 704, 448, 33),
                                         (gs.Q4_K, 0, 512, 512, 24)])
def test_mlp_prefill_stagewise(orc, t, act, H, F, T):
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    g = gs.rng(8200 + t + T)
    Wg, Wu, Wd = gs.weights(t, g, F, H), gs.weights(t, g, F, H), gs.weights(t, g, H, F)
    x = gs.activations(g, T, H)
    say("mlp prefill", gs.NAMES[t], H, F, "T", T)
    tg, tu, td = dev(Wg)[0], dev(Wu)[0], dev(Wd)[0]
    xt, _ = dev(x)
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(qg.qg_mlp_workspace_size(t, H, F, T) // 4, dtype=torch.float32, device="cuda")
    qg.qg_mlp(t, act, tg, tu, td, H, F, xt, y, T, ws)
    wsh = host(ws)
    gu = wsh[:T * 2 * F].reshape(T, 2 * F)
    a0 = _align256(T * 2 * F * 4) // 4
    check_act(orc, act, gu, wsh[a0:a0 + T * F].reshape(T, F), F, "prefill act")
    yg, Ag = orc.gemv(t, Wg, x, F, H, T)
    yu, Au = orc.gemv(t, Wu, x, F, H, T)
    check_rows(gu, np.concatenate([yg, yu], 1), np.concatenate([Ag, Au], 1), "prefill gate||up")
    yh = host(y)
    Wabs = np.abs(orc.dequant(t, Wd, H * F).reshape(H, F))
    for tt in range(T):
        yd, Ad = orc.gemv_f64(t, Wd, orc.glu(act, gu[tt], F), H, F)
        R = Wabs @ np.abs(gu[tt, :F].astype(np.float64) * gu[tt, F:].astype(np.float64))
        assert np.all(np.abs(yh[tt] - yd) <= TOL * Ad + 1e-6 * R), "prefill down token %d" % tt


def test_gemm_full_size_small_batch_16(orc):
    """The dense down projection at 16 tokens, Q8_0 2560 x 9728: 80 row tiles,
    so each row's 304 blocks go out in 7 splits whose sums a second launch
    adds.  Sampled rows, every token."""
    t, rows, cols, T = gs.Q8_0, 2560, 9728, 16
    g = gs.rng(8310)
    W = gs.weights(t, g, rows, cols)
    x = gs.activations(g, T, cols)
    say("gemm full size small batch", rows, cols, "T", T)
    y = gpu_gemm(t, W, x, rows, cols, T)
    ri = np.array(sorted(set(g.choice(rows, 96, replace=False).tolist()) | {0, rows - 1}), np.int64)
    y_ref, A = orc.gemv(t, W, x, rows, cols, T, row_idx=ri)
    check_rows(y[:, ri], y_ref, A, "gemm 2560x9728 T=16")
    assert np.isfinite(y).all()


def test_gemm_full_size_dense_256(orc):
    """The dense gate projection at a 256-token prefill chunk, Q8_0 9728 x 2560:
    sampled rows, every token."""
    t, rows, cols, T = gs.Q8_0, 9728, 2560, 256
    g = gs.rng(8300)
    W = gs.weights(t, g, rows, cols)
    x = gs.activations(g, T, cols)
    say("gemm full size", rows, cols, "T", T)
    y = gpu_gemm(t, W, x, rows, cols, T)
    ri = np.array(sorted(set(g.choice(rows, 96, replace=False).tolist()) | {0, rows - 1}), np.int64)
    y_ref, A = orc.gemv(t, W, x, rows, cols, T, row_idx=ri)
    check_rows(y[:, ri], y_ref, A, "gemm 9728x2560 T=256")
    assert np.isfinite(y).all()


def test_mlp_full_size_prefill_64(orc):
    """The dense Qwen3-style MLP (2560 x 9728, Q8_0, SwiGLU) on a 64-token
    chunk in the launch configuration the prefill bench times: gate||up split
    along the row 3 ways, down 22 ways, each split's partial sums added by a
    second launch.  Sampled gate / up rows for every token, every activation,
    sampled down rows fed the GPU's activations."""
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    t, act, H, F, T = gs.Q8_0, 0, 2560, 9728, 64
    g = gs.rng(8400)
    Wg, Wu, Wd = gs.weights(t, g, F, H), gs.weights(t, g, F, H), gs.weights(t, g, H, F)
    x = gs.activations(g, T, H)
    say("mlp full size prefill", H, F, "T", T)
    tg, tu, td = dev(Wg)[0], dev(Wu)[0], dev(Wd)[0]
    xt, _ = dev(x)
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(qg.qg_mlp_workspace_size(t, H, F, T) // 4, dtype=torch.float32, device="cuda")
    qg.qg_mlp(t, act, tg, tu, td, H, F, xt, y, T, ws)
    wsh = host(ws)
    gu = wsh[:T * 2 * F].reshape(T, 2 * F)
    a0 = _align256(T * 2 * F * 4) // 4
    check_act(orc, act, gu, wsh[a0:a0 + T * F].reshape(T, F), F, "full prefill act")
    ri = np.array(sorted(set(g.choice(F, 96, replace=False).tolist()) | {0, F - 1}), np.int64)
    yg, Ag = orc.gemv(t, Wg, x, F, H, T, row_idx=ri)
    yu, Au = orc.gemv(t, Wu, x, F, H, T, row_idx=ri)
    check_rows(gu[:, ri], yg, Ag, "full prefill gate")
    check_rows(gu[:, F + ri], yu, Au, "full prefill up")
    rd = np.array(sorted(set(g.choice(H, 96, replace=False).tolist()) | {0, H - 1}), np.int64)
    Wsub = np.ascontiguousarray(Wd[rd])   # the sampled rows' blocks ([rows][row bytes])
    Wabs = np.abs(orc.dequant(t, Wsub, rd.size * F).reshape(rd.size, F))
    yh = host(y)
    assert np.isfinite(yh).all()
    for tt in range(T):
        yd, Ad = orc.gemv_f64(t, Wsub, orc.glu(act, gu[tt], F), rd.size, F)
        R = Wabs @ np.abs(gu[tt, :F].astype(np.float64) * gu[tt, F:].astype(np.float64))
        assert np.all(np.abs(yh[tt, rd] - yd) <= TOL * Ad + 1e-6 * R), "full prefill down token %d" % tt

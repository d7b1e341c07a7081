"""Entry points captured in a HIP graph: every replay (with eager work and
synchronisations in between) must reproduce the eager result bit for bit.
The library records no memset nodes; this checks that nothing it enqueues
depends on state a replay would not restore."""
import numpy as np
import pytest

import gguf_synth as gs
from test_gpu_parity import _torch, dev, host, say

pytestmark = pytest.mark.gpu


def _replays_match(fn, out, n=4):
    torch = _torch()
    fn()
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for i in range(n):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "replay %d differs from the eager result" % i
        fn()                       # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("t,T", [(gs.Q8_0, 1), (gs.Q4_K, 1), (gs.Q4_0, 16)])
def test_gemv_graph(t, T):
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    rows, cols = 1000, 8 * gs.QK[t] * (2 if gs.QK[t] == 32 else 1)
    g = gs.rng(61 + t + T)
    W, _ = dev(gs.weights(t, g, rows, cols))
    x, _ = dev(gs.activations(g, T, cols))
    y = torch.empty((T, rows), dtype=torch.float32, device="cuda")
    say("graph gemv", gs.NAMES[t], rows, cols, "T", T)
    _replays_match(lambda: qg.qg_gemv(t, W, x, y, rows, cols, T), y)


@pytest.mark.parametrize("T", [1, 16])
def test_moe_graph(T):
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    t, act, H, F, E, k = gs.Q4_0, 1, 512, 192, 32, 4
    g = gs.rng(71 + T)
    pool, rec, gu_off, d_off = gs.expert_pool(t, g, E, H, F)
    pt, pp = dev(pool)
    ds, _ = dev(gs.down_scales(g, E))
    m = qg.make_moe(t, act, H, F, E, pp + gu_off, rec, pp + d_off, rec, ds)
    lg, _ = dev(gs.logits(g, T, E))
    x, _ = dev(gs.activations(g, T, H))
    slots, _ = dev(np.arange(E, dtype=np.int32))
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(qg.qg_moe_workspace_size(m, k, T) // 4, dtype=torch.float32, device="cuda")
    say("graph moe T", T)
    _replays_match(lambda: qg.qg_moe_ffn(m, lg, k, slots, x, y, T, ids, w, st, ws), y)
    assert int(host(st)[0]) == 0
    del pt


def test_mlp_split_graph():
    """A 16-token MLP whose down projection splits its rows over workgroups
    (200 blocks a row, 8 row tiles): split sums in the workspace, then the
    reduce launch, all inside the graph."""
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    t, H, F, T = gs.Q8_0, 256, 6400, 16
    g = gs.rng(81)
    Wg, _ = dev(gs.weights(t, g, F, H))
    Wu, _ = dev(gs.weights(t, g, F, H))
    Wd, _ = dev(gs.weights(t, g, H, F))
    x, _ = dev(gs.activations(g, T, H))
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    nws = qg.qg_mlp_workspace_size(t, H, F, T)
    assert nws > (T * 2 * F + T * F) * 4          # the split sums need room
    ws = torch.empty(nws // 4, dtype=torch.float32, device="cuda")
    say("graph mlp split", H, F, "T", T)
    _replays_match(lambda: qg.qg_mlp(t, qg.QG_ACT_SILU, Wg, Wu, Wd, H, F, x, y, T, ws), y)


def test_moe_crowded_graph():
    """Every token on the same four experts: the routing launch's set lists
    (eight chunks per group) are rebuilt on every replay."""
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    t, act, H, F, E, k, T = gs.Q4_0, 1, 256, 128, 64, 4, 16
    g = gs.rng(91)
    pool, rec, gu_off, d_off = gs.expert_pool(t, g, E, H, F)
    pt, pp = dev(pool)
    m = qg.make_moe(t, act, H, F, E, pp + gu_off, rec, pp + d_off, rec, None)
    lg_h = gs.logits(g, T, E).copy()
    lg_h[:, [3, 20, 41, 60]] += np.float32(20.0)
    lg, _ = dev(lg_h)
    x, _ = dev(gs.activations(g, T, H))
    slots, _ = dev(np.arange(E, dtype=np.int32))
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(qg.qg_moe_workspace_size(m, k, T) // 4, dtype=torch.float32, device="cuda")
    say("graph moe crowded")
    _replays_match(lambda: qg.qg_moe_ffn(m, lg, k, slots, x, y, T, ids, w, st, ws), y)
    assert sorted(set(host(ids).flatten().tolist())) == [3, 20, 41, 60]
    del pt

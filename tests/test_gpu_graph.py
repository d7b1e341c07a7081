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

"""The allocation-free MoE entry point (qg_moe_ffn_noalloc, static device
scratch) against the workspace entry point (qg_moe_ffn) on the same inputs:
two calls in a row, the second smaller than the first, each equal bit for bit
(y, ids, weights, status) to qg_moe_ffn with a workspace of its own; ids also
equal the oracle's router."""
import numpy as np
import pytest

import gguf_synth as gs
from test_gpu_parity import _torch, dev, host, say

pytestmark = pytest.mark.gpu


def _case(t, act, H, F, E, k, T, seed):
    g = gs.rng(seed)
    pool, rec, gu_off, d_off = gs.expert_pool(t, g, E, H, F)
    return dict(t=t, act=act, H=H, F=F, E=E, k=k, T=T, pool=pool, rec=rec, gu_off=gu_off, d_off=d_off,
                lg=gs.logits(g, T, E), x=gs.activations(g, T, H), ds=gs.down_scales(g, E))


def _run(c, noalloc):
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    pt, pp = dev(c["pool"])
    dst, _ = dev(c["ds"])
    m = qg.make_moe(c["t"], c["act"], c["H"], c["F"], c["E"], pp + c["gu_off"], c["rec"], pp + c["d_off"],
                    c["rec"], dst)
    lt, _ = dev(c["lg"])
    xt, _ = dev(c["x"])
    slots = torch.arange(c["E"], dtype=torch.int32, device="cuda")
    T, k, H = c["T"], c["k"], c["H"]
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    ids = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    st = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    if noalloc:
        qg.qg_moe_ffn_noalloc(m, lt, k, slots, xt, y, T, ids, w, st)
    else:
        ws = torch.zeros(qg.qg_moe_workspace_size(m, k, T) // 4, dtype=torch.float32, device="cuda")
        qg.qg_moe_ffn(m, lt, k, slots, xt, y, T, ids, w, st, ws)
    return host(y), host(ids), host(w), host(st)


def test_moe_noalloc_two_calls_match_workspace_entry(orc):
    cases = [_case(gs.Q4_0, 1, 1024, 512, 32, 4, 16, 9100),   # first call: 16 tokens
             _case(gs.Q8_0, 0, 512, 256, 16, 2, 1, 9101)]      # second call: one token, smaller shapes
    for c in cases:
        say("moe noalloc", gs.NAMES[c["t"]], c["H"], c["F"], c["E"], "k", c["k"], "T", c["T"])
        got = _run(c, True)
        ref = _run(c, False)
        for a, b, what in zip(got, ref, ("y", "ids", "weights", "status")):
            assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                  b.view(np.uint32) if b.dtype == np.float32 else b), what
        assert int(got[3][0]) == 0
        ids_ref, _ = orc.router_topk(c["lg"], c["E"], c["k"], c["T"])
        assert np.array_equal(got[1], ids_ref)
        assert np.isfinite(got[0]).all()

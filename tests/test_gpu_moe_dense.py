"""GPU parity of qg_moe_ffn_dense (the routed experts and a dense gated MLP
beside them, on inputs of their own) through the C ABI, against the f64
oracle on the same seeded inputs, stage by stage: router picks bit-exact,
every pick's gate||up, the routed sum, the dense MLP's gate||up, activation
and down output, each within 1e-5 * sum |w x| of the oracle fed the GPU's own
input to that stage.  One-token cases whose shapes fit run as two launches
(the MLP's rows riding in the experts' launches); the others as the separate
calls; both must give the same results within the bound.
"""
import numpy as np
import pytest

import gguf_synth as gs
from test_gpu_parity import TOL, _torch, check_act, check_rows, dev, host, say

pytestmark = pytest.mark.gpu


def _case(seed, t, H, F, Fd, E, k, T, td=None, scale=True):
    g = gs.rng(seed)
    td = t if td is None else td
    pool, rec, gu_off, d_off = gs.expert_pool(t, g, E, H, F)
    return dict(type=t, td=td, H=H, F=F, Fd=Fd, E=E, k=k, T=T, pool=pool, record=rec, gu_off=gu_off, d_off=d_off,
                down_scale=gs.down_scales(g, E) if scale else None,
                Wg=gs.weights(td, g, Fd, H), Wu=gs.weights(td, g, Fd, H), Wd=gs.weights(td, g, H, Fd),
                logits=gs.logits(g, T, E), x=gs.activations(g, T, H), xm=gs.activations(g, T, H),
                slots=np.arange(E, dtype=np.int32))


def run_dense_gpu(c, act, dense_off=0):
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    t, td, H, F, Fd, E, k, T = (c[n] for n in ("type", "td", "H", "F", "Fd", "E", "k", "T"))
    pt, pp = dev(c["pool"])
    dst = dev(c["down_scale"])[0] if c["down_scale"] is not None else None
    m = qg.make_moe(t, act, H, F, E, pp + c["gu_off"], c["record"], pp + c["d_off"], c["record"], dst)
    wg, wgp = dev(c["Wg"], dense_off)
    wu, wup = dev(c["Wu"], dense_off)
    wd, wdp = dev(c["Wd"], dense_off)
    d = qg.make_dense_mlp(td, Fd, wgp, wup, wdp)
    st, _ = dev(c["slots"])
    lt, _ = dev(c["logits"])
    xt, _ = dev(c["x"])
    xmt, _ = dev(c["xm"])
    y = torch.full((T, H), 7.0, dtype=torch.float32, device="cuda")
    ym = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    ids = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros((T, k), dtype=torch.float32, device="cuda")
    status = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    nbytes = qg.qg_moe_dense_workspace_size(m, d, k, T)
    base = qg.qg_moe_workspace_size(m, k, T)
    assert nbytes == base + qg.qg_mlp_workspace_size(td, H, Fd, T)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    qg.qg_moe_ffn_dense(m, d, lt, k, st, xt, y, xmt, ym, T, ids, w, status, ws)
    wsh = host(ws)
    b4 = base // 4
    a0 = b4 + (T * 2 * Fd * 4 + 255) // 256 * 64
    out = dict(y=host(y), ym=host(ym), ids=host(ids), w=host(w), status=int(host(status)[0]),
               gu=wsh[:T * k * 2 * F].reshape(T, k, 2 * F),
               dgu=wsh[b4:b4 + T * 2 * Fd].reshape(T, 2 * Fd), dact=wsh[a0:a0 + T * Fd].reshape(T, Fd))
    del pt, wg, wu, wd
    return out


def check_dense_stages(orc, c, r, act, absent=()):
    t, td, H, F, Fd, E, k, T = (c[n] for n in ("type", "td", "H", "F", "Fd", "E", "k", "T"))
    ids, cw = orc.router_topk(c["logits"], E, k, T)
    assert np.array_equal(r["ids"], ids)
    assert np.all(np.abs(r["w"] - cw) <= 1e-6 * cw)
    rec, d_off = c["record"], c["d_off"]
    live = [tt for tt in range(T) if not any(int(e) in absent for e in ids[tt])]
    for tt in live:   # every pick's gate || up
        for j in range(k):
            e = int(ids[tt, j])
            yy, AA = orc.gemv(t, c["pool"][e * rec:e * rec + d_off], c["x"][tt:tt + 1], 2 * F, H, 1)
            check_rows(r["gu"][tt, j][None], yy, AA, "routed gate||up t%d j%d" % (tt, j))
    # the routed sum, fed the GPU's gate || up; absent tokens keep their row
    # (the oracle is given a valid slot for an absent expert: its sums for
    # those tokens are not compared)
    oslots = np.where(c["slots"] < 0, np.arange(E, dtype=np.int32), c["slots"])
    yd, Ad, R = orc.moe_down(t, act, H, F, c["pool"][d_off:], rec, c["down_scale"], oslots, ids,
                             r["w"].astype(np.float64), r["gu"], T)
    for tt in range(T):
        if tt in live:
            e = np.abs(r["y"][tt] - yd[tt])
            assert np.all(e <= TOL * Ad[tt] + 1e-6 * R[tt]), "routed sum t%d: worst %.3g" % (tt, (e / Ad[tt]).max())
        else:
            assert np.all(r["y"][tt] == 7.0), "an absent token's row was written"
    # the dense MLP on its own input, every token
    yg, Ag = orc.gemv(td, c["Wg"], c["xm"], Fd, H, T)
    yu, Au = orc.gemv(td, c["Wu"], c["xm"], Fd, H, T)
    check_rows(r["dgu"], np.concatenate([yg, yu], 1), np.concatenate([Ag, Au], 1), "dense gate||up")
    check_act(orc, act, r["dgu"], r["dact"], Fd, "dense act")
    Wabs = np.abs(orc.dequant(td, c["Wd"], H * Fd).reshape(H, Fd))
    for tt in range(T):
        yy, AA = orc.gemv_f64(td, c["Wd"], orc.glu(act, r["dgu"][tt], Fd), H, Fd)
        Rd = Wabs @ np.abs(r["dgu"][tt, :Fd].astype(np.float64) * r["dgu"][tt, Fd:].astype(np.float64))
        e = np.abs(r["ym"][tt] - yy)
        assert np.all(e <= TOL * AA + 1e-6 * Rd), "dense down t%d: worst err/A %.3g" % (tt, (e / AA).max())


DENSE_CASES = [
    # type, H, F, Fd, E, k, T, dense type, act
    (gs.Q4_0, 2816, 704, 2112, 128, 8, 1, None, 1),   # Gemma4-shaped: three dense row groups, two launches
    (gs.Q8_0, 512, 256, 512, 16, 4, 1, None, 0),      # two groups, Q8_0 units
    (gs.Q4_0, 352, 96, 288, 16, 4, 1, None, 1),       # small, ragged row tiles
    (gs.Q8_0, 256, 256, 4096, 8, 2, 1, None, 0),      # the widest dense row the down launch takes (4 units/lane)
    (gs.Q8_0, 256, 1024, 1024, 16, 8, 1, None, 0),    # 288 (pick, block) columns: the row-walking down launch
    # the separate calls
    (gs.Q8_0, 512, 256, 384, 16, 4, 1, None, 0),      # FD not a multiple of F
    (gs.Q4_0, 352, 96, 288, 16, 4, 3, None, 1),       # several tokens
    (gs.Q4_0, 352, 96, 192, 16, 4, 1, gs.Q8_0, 1),    # the MLP in another block type
    (gs.Q8_0, 256, 1536, 1536, 16, 8, 1, None, 0),    # routed down rows of two units per lane
    (gs.Q8_0, 256, 256, 4352, 8, 2, 1, None, 0),      # dense row past 4 units per lane
]


@pytest.mark.parametrize("t,H,F,Fd,E,k,T,td,act", DENSE_CASES)
def test_moe_dense_stagewise(orc, t, H, F, Fd, E, k, T, td, act):
    c = _case(8000 + H + F + Fd + T, t, H, F, Fd, E, k, T, td)
    say("moe dense", gs.NAMES[t], H, F, Fd, E, k, "T", T, "dense type", gs.NAMES[c["td"]], "act", act)
    r = run_dense_gpu(c, act)
    assert r["status"] == 0
    check_dense_stages(orc, c, r, act)


@pytest.mark.parametrize("dense_off", [2, 4])
def test_moe_dense_offsets(orc, dense_off):
    """Dense matrices off 16-byte alignment beside an aligned pool: the
    experts' gated launch cannot take them, so the MLP runs as its own
    launches after the experts' (same results)."""
    c = _case(8100 + dense_off, gs.Q8_0, 512, 256, 512, 16, 4, 1)
    say("moe dense, dense offset", dense_off)
    r = run_dense_gpu(c, 0, dense_off=dense_off)
    assert r["status"] == 0
    check_dense_stages(orc, c, r, 0)


@pytest.mark.parametrize("T", [1, 2])
def test_moe_dense_absent_expert(orc, T):
    """A pick with no slot: that token's expert row is left as it was and the
    status reads QG_EABSENT; the dense MLP's output is still written."""
    import gguf_dequant_gemv_amd as qg
    c = _case(8200 + T, gs.Q4_0, 352, 96, 288, 16, 4, T)
    ids, _ = orc.router_topk(c["logits"], 16, 4, T)
    e_abs = int(ids[0, 1])
    c["slots"][e_abs] = -1
    say("moe dense absent expert", e_abs, "T", T)
    r = run_dense_gpu(c, 1)
    assert r["status"] == qg.QG_EABSENT
    check_dense_stages(orc, c, r, 1, absent=(e_abs,))

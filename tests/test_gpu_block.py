"""GPU parity of the steps around the routed experts, through the C ABI,
against the f64 oracle on the same seeded inputs:

  * f32-weight GEMV (router, shared gate): |y - y_ref| <= 1e-5 * sum |w x|;
  * RMS norm: |y - y_ref| <= 1e-5 * |y_ref| per element (a product of the
    input, one reduction's factor and the gains: no cancellation);
  * shared-expert MoE block: stage by stage, each stage fed the GPU's own input
    (routed gate||up, activations, down + pick terms, the shared expert's
    gate||up, activation and down, then the combine with the gate and the
    residual: |y - y_ref| <= 1e-5 * A, A the oracle's error scale);
  * Gemma's FFN tail: |x - x_ref| <= 1e-5 * A;
  * embedding rows: bit-exact; soft cap: |l - l_ref| <= 1e-6 * cap; argmax
    exact against the oracle's pick over the GPU's (capped) f32 logits;
  * two whole FFN blocks chained as the pages chain them, each step checked
    on the GPU's own input to it.
"""
import math

import numpy as np
import pytest

import gguf_synth as gs
from test_gpu_parity import TOL, _align256, _torch, check_act, check_rows, dev, host, say

pytestmark = pytest.mark.gpu


def _empty(shape, dtype="float32", fill=float("nan")):
    torch = _torch()
    return torch.full(shape, fill, dtype=getattr(torch, dtype), device="cuda")


# ------------------------------------------------------------ f32 GEMV ------
@pytest.mark.parametrize("rows,cols,T,off", [
    (128, 2048, 1, 0), (128, 2048, 3, 0), (256, 2048, 16, 0), (1, 2816, 1, 0),
    (128, 2816, 16, 0),    # 5.5 column passes shared by a row's 4 waves
    (300, 1000, 5, 0),     # 5 tokens, ragged last pass
    (3, 44, 7, 0),         # one short pass: three of a row's waves add nothing
    (37, 70, 5, 0),        # cols not a multiple of 4: the scalar path
    (9, 256, 2, 4),        # W 4 bytes past a 16-byte boundary: the scalar path
])
def test_f32_gemv(orc, rows, cols, T, off):
    import gguf_dequant_gemv_amd as qg
    g = gs.rng(100 + rows + cols + T)
    W = gs.f32_matrix(g, rows, cols, 1.0 / math.sqrt(cols))
    x = gs.activations(g, T, cols)
    say("f32 gemv", rows, cols, "T", T, "offset", off)
    Wt, Wp = dev(W.view(np.uint8), off)
    xt, _ = dev(x)
    y = _empty((T, rows))
    qg.qg_gemv(qg.QG_F32, Wp, xt, y, rows, cols, T)
    yr, A = orc.gemv(orc.F32, W.view(np.uint8), x, rows, cols, T)
    check_rows(host(y), yr, A, "f32 gemv")


# ------------------------------------------------------------ RMS norm ------
def check_rel(y, ref, what, tol=TOL):
    err = np.abs(y.astype(np.float64) - ref)
    bound = tol * np.abs(ref) + 1e-30
    assert np.all(err <= bound), "%s: worst err/|ref| %.3g" % (what, (err / np.maximum(np.abs(ref), 1e-30)).max())


@pytest.mark.parametrize("n,T,k,inplace", [
    (2048, 1, 1.0, False), (2816, 4, 1.0 / math.sqrt(2816), False), (5, 3, 1.0, False),
    (300, 16, 2.0, True), (5120, 2, 1.0, True)])
def test_rmsnorm(orc, n, T, k, inplace):
    import gguf_dequant_gemv_amd as qg
    g = gs.rng(200 + n + T)
    x = gs.activations(g, T, n) * np.float32(3.0)
    w = gs.norm_weights(g, n)
    say("rmsnorm", n, "T", T, "k", k, "in place", inplace)
    xt, _ = dev(x)
    wt, _ = dev(w)
    y = xt if inplace else _empty((T, n))
    qg.qg_rmsnorm(xt, wt, y, n, T, 1e-6, k)
    check_rel(host(y), orc.rmsnorm(x, w, n, T, 1e-6, k), "rmsnorm")


@pytest.mark.parametrize("n,T,nout", [(2816, 1, 3), (2816, 16, 3), (1000, 3, 4), (64, 2, 1), (4096, 1, 2),
                                      (5000, 2, 2)])
def test_rmsnorm_multi(orc, n, T, nout):
    """Several norms of one row in a launch: bit for bit the separate
    qg_rmsnorm calls, and each against the oracle."""
    import gguf_dequant_gemv_amd as qg
    g = gs.rng(300 + n + T + nout)
    x = gs.activations(g, T, n) * np.float32(2.0)
    ws = [gs.norm_weights(g, n) for _ in range(nout)]
    ks = [1.0, float(1.0 / np.sqrt(n)), 0.5, 3.0][:nout]
    say("rmsnorm multi", n, "T", T, "outputs", nout)
    xt, _ = dev(x)
    wts = [dev(w)[0] for w in ws]
    ys = [_empty((T, n)) for _ in range(nout)]
    qg.qg_rmsnorm_multi(xt, n, T, 1e-6, wts, ks, ys)
    for j in range(nout):
        one = _empty((T, n))
        qg.qg_rmsnorm(xt, wts[j], one, n, T, 1e-6, ks[j])
        assert np.array_equal(host(ys[j]), host(one)), "output %d differs from qg_rmsnorm" % j
        check_rel(host(ys[j]), orc.rmsnorm(x, ws[j], n, T, 1e-6, ks[j]), "rmsnorm multi %d" % j)


@pytest.mark.parametrize("n,E,T,nout", [(2048, 256, 1, 1), (2816, 128, 16, 2), (1000, 37, 3, 0), (1001, 9, 2, 1),
                                         (5000, 8, 2, 3), (1000, 300, 5, 1), (44, 3, 7, 1)])
def test_rmsnorm_router(orc, n, E, T, nout):
    """Norms + router in one launch: the logits and every norm bit for bit
    what qg_rmsnorm / qg_gemv(QG_F32) give separately, and both against the
    oracle."""
    import gguf_dequant_gemv_amd as qg
    g = gs.rng(900 + n + E + T)
    x = gs.activations(g, T, n)
    rw = gs.norm_weights(g, n)
    rk = float(np.float32(1.0 / math.sqrt(n)))
    W = (g.standard_normal((E, n), dtype=np.float32) * np.float32(1.0 / math.sqrt(n))).astype(np.float32)
    ws = [gs.norm_weights(g, n) for _ in range(nout)]
    ks = [1.0, 0.5, 2.0][:nout]
    xt, _ = dev(x)
    rwt, _ = dev(rw)
    Wt, _ = dev(W)
    wts = [dev(w)[0] for w in ws]
    ys = [_empty((T, n)) for _ in range(nout)]
    lg = _empty((T, E))
    say("rmsnorm router", n, E, "T", T, "nout", nout)
    qg.qg_rmsnorm_router(xt, n, T, 1e-6, rwt, rk, Wt, E, lg, wts, ks, ys)
    # the separate launches
    rt = _empty((T, n))
    qg.qg_rmsnorm(xt, rwt, rt, n, T, 1e-6, rk)
    lg2 = _empty((T, E))
    qg.qg_gemv(qg.QG_F32, Wt, rt, lg2, E, n, T)
    assert np.array_equal(host(lg).view(np.uint32), host(lg2).view(np.uint32))
    for j in range(nout):
        one = _empty((T, n))
        qg.qg_rmsnorm(xt, wts[j], one, n, T, 1e-6, ks[j])
        assert np.array_equal(host(ys[j]).view(np.uint32), host(one).view(np.uint32)), "norm %d" % j
        check_rel(host(ys[j]), orc.rmsnorm(x, ws[j], n, T, 1e-6, ks[j]), "norm %d" % j)
    # logits against the oracle's GEMV of the GPU's router input
    rth = host(rt)
    check_rel(rth, orc.rmsnorm(x, rw, n, T, 1e-6, rk), "router input norm")
    y_ref, A = orc.gemv(orc.F32, W.view(np.uint8), rth, E, n, T)
    check_rows(host(lg), y_ref, A, "router logits")


# ------------------------------------------------- shared-expert MoE block --
def run_shared_gpu(c, lt=None, xt=None, resid=None, pool_off=0, sh_off=0):
    """qg_moe_ffn_shared on case c; lt / xt / resid: device tensors to use in
    place of c's logits, input and residual; pool_off / sh_off: byte offsets
    (even) of the expert pool and of the shared expert's matrices.  Returns
    host copies of every stage and the pieces the checks need."""
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    t, H, F, SF, E, k, T = c["type"], c["H"], c["F"], c["SF"], c["E"], c["k"], c["ntok"]
    pt, pp = dev(c["pool"], pool_off)
    m = qg.make_moe(t, qg.QG_ACT_SILU, H, F, E, pp + c["gu_off"], c["record"], pp + c["d_off"], c["record"])
    sgt, sgp = dev(c["sh_gate"], sh_off)
    sut, sup = dev(c["sh_up"], sh_off)
    sdt, sdp = dev(c["sh_down"], sh_off)
    git, _ = dev(c["sh_gate_inp"])
    sh = qg.make_shared_expert(c.get("sh_type", t), SF, sgp, sup, sdp, git)
    st, _ = dev(c["slots"])
    if lt is None:
        lt, _ = dev(c["logits"])
    if xt is None:
        xt, _ = dev(c["x"])
    if resid is None:
        resid, _ = dev(c["resid"])
    r0 = host(resid).copy()
    ids = _empty((T, k), "int32", -1)
    w = _empty((T, k), fill=0.0)
    status = _empty((1,), "int32", 12345)
    nbytes = qg.qg_moe_shared_workspace_size(m, sh, k, T)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    qg.qg_moe_ffn_shared(m, sh, lt, k, st, xt, resid, T, ids, w, status, ws)
    wsh = host(ws)
    P = T * k
    base = qg.qg_moe_workspace_size(m, k, T) // 4
    a0 = _align256(P * 2 * F * 4) // 4
    d0 = a0 + _align256(P * F * 4) // 4
    s_a = base + _align256(T * 2 * SF * 4) // 4
    s_h = (nbytes - _align256(T * H * 4)) // 4      # sh is the last region
    out = dict(resid0=r0, resid=host(resid), ids=host(ids), w=host(w), status=int(host(status)[0]),
               x=host(xt), logits=host(lt),
               gu=wsh[:P * 2 * F].reshape(T, k, 2 * F), act=wsh[a0:a0 + P * F].reshape(T, k, F),
               terms=wsh[d0:d0 + P * H].reshape(T, k, H),
               sh_gu=wsh[base:base + T * 2 * SF].reshape(T, 2 * SF), sh_act=wsh[s_a:s_a + T * SF].reshape(T, SF),
               sh=wsh[s_h:s_h + T * H].reshape(T, H))
    del pt
    return out


def check_shared_stages(orc, c, r):
    t, H, F, SF, E, k, T = c["type"], c["H"], c["F"], c["SF"], c["E"], c["k"], c["ntok"]
    ts = c.get("sh_type", t)
    x = r["x"]
    ids, cw = orc.router_topk(r["logits"], E, k, T)
    assert r["status"] == 0
    assert np.array_equal(r["ids"], ids)
    assert np.all(np.abs(r["w"] - cw) <= 1e-6 * cw)
    rec, d_off = c["record"], c["d_off"]
    # routed gate || up of every pick
    for tt in range(T):
        for j in range(k):
            e = int(ids[tt, j])
            yy, AA = orc.gemv(t, c["pool"][e * rec:e * rec + d_off], x[tt:tt + 1], 2 * F, H, 1)
            check_rows(r["gu"][tt, j][None], yy, AA, "routed gate||up t%d j%d" % (tt, j))
    check_act(orc, 0, r["gu"].reshape(T * k, 2 * F), r["act"].reshape(T * k, F), F, "routed act")
    # routed down and pick weights, summed over the picks, fed the GPU's gate || up
    yd, Ad, R = orc.moe_down(t, 0, H, F, c["pool"][d_off:], rec, None, c["slots"], ids,
                             r["w"].astype(np.float64), r["gu"], T)
    err = np.abs(r["terms"].astype(np.float64).sum(axis=1) - yd)
    assert np.all(err <= TOL * Ad + 1e-6 * R), "routed terms: worst err/A %.3g" % (err / Ad).max()
    # the shared expert on the same input
    yg, Ag = orc.gemv(ts, c["sh_gate"], x, SF, H, T)
    yu, Au = orc.gemv(ts, c["sh_up"], x, SF, H, T)
    check_rows(r["sh_gu"], np.concatenate([yg, yu], 1), np.concatenate([Ag, Au], 1), "shared gate||up")
    check_act(orc, 0, r["sh_gu"], r["sh_act"], SF, "shared act")
    Wabs = np.abs(orc.dequant(ts, c["sh_down"], H * SF).reshape(H, SF))
    for tt in range(T):
        a = orc.glu(0, r["sh_gu"][tt], SF)
        ys, As = orc.gemv_f64(ts, c["sh_down"], a, H, SF)
        Rs = Wabs @ np.abs(r["sh_gu"][tt, :SF].astype(np.float64) * r["sh_gu"][tt, SF:].astype(np.float64))
        e2 = np.abs(r["sh"][tt] - ys)
        assert np.all(e2 <= TOL * As + 1e-6 * Rs), "shared down t%d: worst err/A %.3g" % (tt, (e2 / As).max())
    # combine: routed terms + sigmoid-gated shared output + residual
    yc, Ac, _ = orc.moe_shared_combine(r["terms"], r["sh"], c["sh_gate_inp"], x, r["resid0"], H, T)
    check_rows(r["resid"], yc, Ac, "shared combine")


SHARED_CASES = [
    # type, H, F, SF, E, k, T, shared type
    (gs.Q8_0, 2048, 512, 512, 256, 8, 1, None),     # Qwen3.5/3.6-MoE-style block shape
    (gs.Q8_0, 2048, 512, 512, 64, 8, 16, None),
    (gs.Q4_0, 352, 96, 160, 16, 4, 3, None),        # small, ragged row tiles
    (gs.Q4_K, 512, 256, 96, 8, 2, 2, gs.Q8_0),      # shared expert in another block type
    # one token: a shared expert of the routed experts' shape rides in the
    # routing launch and the one-token down launch (combine included)
    (gs.Q4_0, 352, 96, 96, 16, 4, 1, None),
    (gs.Q8_0, 256, 1536, 1536, 16, 8, 1, None),     # two blocks per lane in the down launch
    (gs.Q8_0, 2336, 512, 512, 16, 8, 1, None),      # 10 rows a down workgroup, the last one ragged
    # one token, other shapes or types: routed down in one launch, then the
    # shared expert and the combine as their own launches
    (gs.Q4_0, 352, 96, 160, 16, 4, 1, None),
    (gs.Q8_0, 512, 256, 256, 16, 4, 1, gs.Q4_0),
]


@pytest.mark.parametrize("t,H,F,SF,E,k,T,ts", SHARED_CASES)
def test_moe_shared_stagewise(orc, t, H, F, SF, E, k, T, ts):
    c = gs.qwen35_block(7000 + H + T + E, T, t, H, E, F, SF, k)
    if ts is not None:
        g = gs.rng(7100 + H)
        c.update(sh_type=ts, sh_gate=gs.weights(ts, g, SF, H), sh_up=gs.weights(ts, g, SF, H),
                 sh_down=gs.weights(ts, g, H, SF))
    c["logits"] = gs.logits(gs.rng(7200 + T), T, E)
    c["resid"] = gs.activations(gs.rng(7300 + T), T, H)
    say("moe shared", gs.NAMES[t], H, F, SF, E, k, "T", T)
    r = run_shared_gpu(c)
    check_shared_stages(orc, c, r)


def test_moe_shared_absent_expert(orc):
    """A token with an absent pick keeps its residual row; the others are updated."""
    import gguf_dequant_gemv_amd as qg
    c = gs.qwen35_block(7400, 3, gs.Q8_0, 256, 10, 64, 96, 3)
    c["logits"] = gs.logits(gs.rng(7401), 3, 10)
    c["resid"] = gs.activations(gs.rng(7402), 3, 256)
    ids, _ = _oracle_ids(c)
    e_abs = int(ids[1, 0])
    c["slots"] = np.arange(10, dtype=np.int32)
    c["slots"][e_abs] = -1
    say("moe shared absent expert", e_abs)
    r = run_shared_gpu(c)
    assert r["status"] == qg.QG_EABSENT
    for tt in range(3):
        if e_abs in ids[tt]:
            assert np.array_equal(r["resid"][tt], r["resid0"][tt])
        else:
            assert not np.array_equal(r["resid"][tt], r["resid0"][tt])


@pytest.mark.parametrize("pool_off,sh_off", [(0, 2), (2, 2), (2, 0)])
def test_moe_shared_one_token_offsets(orc, pool_off, sh_off):
    """One token, shared expert of the routed shape, tensors off 16-byte
    alignment: with an aligned pool (the aligned-copy routing launch) a
    misaligned shared expert runs as its own launches; with a misaligned pool
    it rides in the routing launch at any 2-byte phase."""
    c = gs.qwen35_block(7600 + pool_off + sh_off, 1, gs.Q8_0, 512, 16, 256, 256, 4)
    c["logits"] = gs.logits(gs.rng(7601), 1, 16)
    c["resid"] = gs.activations(gs.rng(7602), 1, 512)
    say("moe shared one token, pool offset", pool_off, "shared offset", sh_off)
    r = run_shared_gpu(c, pool_off=pool_off, sh_off=sh_off)
    check_shared_stages(orc, c, r)


def test_moe_shared_absent_expert_one_token(orc):
    """One token whose first pick has no slot: the fused launches leave its
    residual row as it was and report QG_EABSENT."""
    import gguf_dequant_gemv_amd as qg
    c = gs.qwen35_block(7500, 1, gs.Q8_0, 256, 12, 64, 64, 4)
    c["logits"] = gs.logits(gs.rng(7501), 1, 12)
    c["resid"] = gs.activations(gs.rng(7502), 1, 256)
    ids, _ = _oracle_ids(c)
    c["slots"] = np.arange(12, dtype=np.int32)
    c["slots"][int(ids[0, 0])] = -1
    say("moe shared absent expert, one token", int(ids[0, 0]))
    r = run_shared_gpu(c)
    assert r["status"] == qg.QG_EABSENT
    assert np.array_equal(r["resid"], r["resid0"])


def _oracle_ids(c):
    import oracle
    return oracle.router_topk(c["logits"], c["E"], c["k"], c["ntok"])


# ------------------------------------------------------ Gemma's FFN tail ---
# rows of up to 4096 run from registers (one batch per thread), longer ones in passes
@pytest.mark.parametrize("n,T", [(2816, 1), (2816, 16), (100, 3), (4096, 1), (5000, 2)])
def test_post_ffn(orc, n, T):
    import gguf_dequant_gemv_amd as qg
    g = gs.rng(300 + n + T)
    mlp = gs.activations(g, T, n) * np.float32(0.3)
    moe = gs.activations(g, T, n) * np.float32(2.0)
    x = gs.activations(g, T, n)
    w1, w2, w = gs.norm_weights(g, n), gs.norm_weights(g, n), gs.norm_weights(g, n)
    os_ = np.array([0.75], np.float32)
    say("post ffn", n, "T", T)
    ts = [dev(a)[0] for a in (mlp, moe, w1, w2, w, os_, x)]
    qg.qg_post_ffn(*ts[:6], ts[6], n, T, 1e-6)
    yr, A = orc.post_ffn(mlp, moe, w1, w2, w, float(os_[0]), x, n, T, 1e-6)
    check_rows(host(ts[6]), yr, A, "post ffn")


# --------------------------------------------------------- embedding rows --
@pytest.mark.parametrize("t", [gs.Q8_0, gs.Q4_0, gs.Q4_K, gs.Q6_K])
@pytest.mark.parametrize("blocks,kblocks,off", [(64, 8, 0), (3, 1, 2), (130, 70, 2), (80, 11, 0)])
def test_embed_bit_exact(orc, t, blocks, kblocks, off):
    """A lane per 8 values and a wave per (part, 64 blocks): one and several
    chunks of 64 blocks, a ragged last chunk, odd 2-byte offsets."""
    import gguf_dequant_gemv_amd as qg
    cols_blocks = kblocks if t in (gs.Q4_K, gs.Q6_K) else blocks
    rows, cols = 300, cols_blocks * gs.QK[t]
    W = gs.weights(t, gs.rng(400 + t + cols), rows, cols)
    tokens = np.array([0, 299, 17, 17, 150], np.int32)
    Wt, Wp = dev(W, off)
    tt, _ = dev(tokens)
    for scale in (1.0, float(np.float32(math.sqrt(2816.0)))):
        say("embed", gs.NAMES[t], rows, cols, "offset", off, "scale", scale)
        out = _empty((tokens.size, cols))
        qg.qg_embed(t, Wp, rows, cols, tt, tokens.size, scale, out)
        ref = orc.embed(t, W, rows, cols, tokens, scale)
        assert np.array_equal(host(out).view(np.uint32), ref.view(np.uint32))


def test_embed_out_of_range_token():
    import gguf_dequant_gemv_amd as qg
    W = gs.weights(gs.Q8_0, gs.rng(5), 4, 64)
    Wt, _ = dev(W)
    tt, _ = dev(np.array([1, 4, -1, 3], np.int32))
    out = _empty((4, 64), fill=0.0)
    say("embed out-of-range tokens")
    qg.qg_embed(gs.Q8_0, Wt, 4, 64, tt, 4, 1.0, out)
    o = host(out)
    assert np.isfinite(o[[0, 3]]).all() and np.isnan(o[[1, 2]]).all()


# ------------------------------------------------------- soft cap, argmax --
@pytest.mark.parametrize("n,T,cap", [(151936, 1, 0.0), (262144, 1, 30.0), (151936, 16, 0.0), (262144, 4, 30.0),
                                     (1000, 3, 30.0), (1, 2, 0.0), (5000, 1, 0.0)])
def test_argmax(orc, n, T, cap):
    import gguf_dequant_gemv_amd as qg
    g = gs.rng(500 + n + T)
    l = (g.standard_normal((T, n), dtype=np.float32) * np.float32(8.0)).astype(np.float32)
    if n > 10:
        # a tie for the maximum at two indices, NaN entries, -inf entries
        top = np.float32(l.max() + 50.0)
        l[0, n // 3] = top
        l[0, n - 2] = top
        l[-1, 7] = np.nan
        l[-1, 8] = -np.inf
    say("argmax", n, "T", T, "cap", cap)
    lt, _ = dev(l)
    idx = _empty((T,), "int32", -7)
    ws = _torch().empty(qg.qg_argmax_workspace_size(n, T) // 4, dtype=_torch().float32, device="cuda")
    qg.qg_argmax(lt, n, T, cap, idx, ws)
    got_l = host(lt)
    got = host(idx)
    if cap > 0:
        ref_l = orc.softcap(l, cap).reshape(T, n)
        nan = np.isnan(ref_l)
        assert np.array_equal(np.isnan(got_l), nan)
        assert np.all(np.abs(got_l[~nan] - ref_l[~nan]) <= 1e-6 * cap)
    else:
        assert np.array_equal(got_l.view(np.uint32), l.view(np.uint32))   # untouched
    assert got.tolist() == orc.argmax(got_l, n, T).tolist()
    if n > 10 and cap == 0:
        assert got[0] == n // 3


@pytest.mark.parametrize("t,V,cols,cap,T", [(gs.Q8_0, 151936, 2560, 0.0, 1), (gs.Q6_K, 50000, 2816, 30.0, 1),
                                          (gs.Q4_0, 3000, 96, 0.0, 3), (gs.Q4_K, 700, 512, 30.0, 2)])
def test_argmax_embed(orc, t, V, cols, cap, T):
    """The pick and the gather in two launches equal qg_argmax followed by
    qg_embed bit for bit; the picks against the oracle's."""
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    g = gs.rng(560 + V + T)
    l = (g.standard_normal((T, V), dtype=np.float32) * np.float32(8.0)).astype(np.float32)
    W = gs.weights(t, g, V, cols)
    Wt, _ = dev(W)
    scale = float(np.float32(math.sqrt(cols)))
    say("argmax embed", gs.NAMES[t], V, cols, "cap", cap, "T", T)
    lt1, _ = dev(l)
    lt2, _ = dev(l)
    nws = qg.qg_argmax_workspace_size(V, T)
    ws1 = torch.empty(nws // 4, dtype=torch.float32, device="cuda")
    ws2 = torch.empty(nws // 4, dtype=torch.float32, device="cuda")
    idx1 = _empty((T,), "int32", -1)
    idx2 = _empty((T,), "int32", -1)
    out1 = _empty((T, cols))
    out2 = _empty((T, cols))
    qg.qg_argmax_embed(lt1, V, T, cap, idx1, ws1, t, Wt, V, cols, scale, out1)
    qg.qg_argmax(lt2, V, T, cap, idx2, ws2)
    qg.qg_embed(t, Wt, V, cols, idx2, T, scale, out2)
    assert np.array_equal(host(idx1), host(idx2))
    assert np.array_equal(host(out1).view(np.uint32), host(out2).view(np.uint32))
    assert np.array_equal(host(lt1).view(np.uint32), host(lt2).view(np.uint32))   # the capped logits
    got_l = host(lt1)
    assert host(idx1).tolist() == orc.argmax(got_l, V, T).tolist()
    ref = orc.embed(t, W, V, cols, host(idx1).astype(np.int32), scale)
    assert np.array_equal(host(out1).view(np.uint32), ref.view(np.uint32))


def test_argmax_degenerate_rows():
    import gguf_dequant_gemv_amd as qg
    n = 4099
    l = np.full((3, n), np.nan, np.float32)
    l[1, :] = -np.inf
    l[2, :] = 5.0
    say("argmax degenerate rows")
    lt, _ = dev(l)
    idx = _empty((3,), "int32", -7)
    ws = _torch().empty(qg.qg_argmax_workspace_size(n, 3) // 4, dtype=_torch().float32, device="cuda")
    qg.qg_argmax(lt, n, 3, 0.0, idx, ws)
    assert host(idx).tolist() == [0, 0, 0]


# ----------------------------------------------------- whole FFN blocks ----
def test_qwen35_block_chain(orc):
    """rmsnorm -> f32 router GEMV -> routed + shared experts with the residual,
    each step checked on the GPU's own input to it."""
    import gguf_dequant_gemv_amd as qg
    c = gs.qwen35_block(7500, 2, gs.Q8_0, 2048, 128, 512, 512, 8)
    H, E, T = c["H"], c["E"], c["ntok"]
    say("qwen35 block chain", H, E, "T", T)
    x0 = c["x"]
    resid, _ = dev(x0)
    nt, _ = dev(c["norm"])
    xn = _empty((T, H))
    qg.qg_rmsnorm(resid, nt, xn, H, T, 1e-6, 1.0)
    xnh = host(xn)
    check_rel(xnh, orc.rmsnorm(x0, c["norm"], H, T, 1e-6), "post-attention norm")
    rt, _ = dev(c["router"])
    lg = _empty((T, E))
    qg.qg_gemv(qg.QG_F32, rt, xn, lg, E, H, T)
    yr, A = orc.gemv(orc.F32, c["router"].view(np.uint8), xnh, E, H, T)
    check_rows(host(lg), yr, A, "router logits")
    r = run_shared_gpu(c, lt=lg, xt=xn, resid=resid)
    check_shared_stages(orc, c, r)


def test_gemma_block_chain(orc):
    """Gemma's FFN block: ffn_norm -> dense GELU MLP; pre_ffw_norm_2 -> experts;
    router-input norm -> f32 router; then the FFN tail with the residual."""
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    c = gs.gemma_block(7600, 1, 128)
    t, H, Fd, F, E, k, T = c["type"], c["H"], c["Fd"], c["F"], c["E"], c["k"], c["ntok"]
    say("gemma block chain", H, Fd, F, E, "T", T)
    x0 = c["x"]
    xt, _ = dev(x0)
    wts = {n: dev(c[n])[0] for n in ("w_ffn", "w_pre2", "w_rscale", "w_post1", "w_post2", "w_post", "out_scale")}
    # dense MLP on rmsnorm(x) * ffn_norm
    xn = _empty((T, H))
    qg.qg_rmsnorm(xt, wts["w_ffn"], xn, H, T, 1e-6, 1.0)
    xnh = host(xn)
    check_rel(xnh, orc.rmsnorm(x0, c["w_ffn"], H, T, 1e-6), "ffn_norm")
    tg, tu, td = dev(c["Wg"])[0], dev(c["Wu"])[0], dev(c["Wd"])[0]
    md = _empty((T, H))
    mws = torch.empty(qg.qg_mlp_workspace_size(t, H, Fd, T) // 4, dtype=torch.float32, device="cuda")
    qg.qg_mlp(t, qg.QG_ACT_GELU_TANH, tg, tu, td, H, Fd, xn, md, T, mws)
    wsh = host(mws)
    gu = wsh[:T * 2 * Fd].reshape(T, 2 * Fd)
    yg, Ag = orc.gemv(t, c["Wg"], xnh, Fd, H, T)
    yu, Au = orc.gemv(t, c["Wu"], xnh, Fd, H, T)
    check_rows(gu, np.concatenate([yg, yu], 1), np.concatenate([Ag, Au], 1), "dense gate||up")
    mdh = host(md)
    Wabs = np.abs(orc.dequant(t, c["Wd"], H * Fd).reshape(H, Fd))
    for tt in range(T):
        yd, Ad = orc.gemv_f64(t, c["Wd"], orc.glu(1, gu[tt], Fd), H, Fd)
        R = Wabs @ np.abs(gu[tt, :Fd].astype(np.float64) * gu[tt, Fd:].astype(np.float64))
        assert np.all(np.abs(mdh[tt] - yd) <= TOL * Ad + 1e-6 * R), "dense down"
    # expert input and router input
    xm = _empty((T, H))
    qg.qg_rmsnorm(xt, wts["w_pre2"], xm, H, T, 1e-6, 1.0)
    xmh = host(xm)
    check_rel(xmh, orc.rmsnorm(x0, c["w_pre2"], H, T, 1e-6), "pre_ffw_norm_2")
    rin = _empty((T, H))
    kf = float(np.float32(1.0 / math.sqrt(H)))
    qg.qg_rmsnorm(xt, wts["w_rscale"], rin, H, T, 1e-6, kf)
    rinh = host(rin)
    check_rel(rinh, orc.rmsnorm(x0, c["w_rscale"], H, T, 1e-6, kf), "router input norm")
    rt, _ = dev(c["router"])
    lg = _empty((T, E))
    qg.qg_gemv(qg.QG_F32, rt, rin, lg, E, H, T)
    yr, A = orc.gemv(orc.F32, c["router"].view(np.uint8), rinh, E, H, T)
    lgh = host(lg)
    check_rows(lgh, yr, A, "router logits")
    # routed experts on the GPU's logits and expert input
    pt, pp = dev(c["pool"])
    dst, _ = dev(c["down_scale"])
    m = qg.make_moe(t, qg.QG_ACT_GELU_TANH, H, F, E, pp + c["gu_off"], c["record"], pp + c["d_off"], c["record"],
                    dst)
    st, _ = dev(c["slots"])
    moe = _empty((T, H))
    ids = _empty((T, k), "int32", -1)
    w = _empty((T, k), fill=0.0)
    status = _empty((1,), "int32", 1)
    ws = torch.empty(qg.qg_moe_workspace_size(m, k, T) // 4, dtype=torch.float32, device="cuda")
    qg.qg_moe_ffn(m, lg, k, st, xm, moe, T, ids, w, status, ws)
    idr, cr = orc.router_topk(lgh, E, k, T)
    assert int(host(status)[0]) == 0 and np.array_equal(host(ids), idr)
    wsh = host(ws)
    mgu = wsh[:T * k * 2 * F].reshape(T, k, 2 * F)
    yd, Ad, R = orc.moe_down(t, 1, H, F, c["pool"][c["d_off"]:], c["record"], c["down_scale"], c["slots"], idr,
                             host(w).astype(np.float64), mgu, T)
    moeh = host(moe)
    assert np.all(np.abs(moeh - yd) <= TOL * Ad + 1e-6 * R), "moe sum"
    # the tail: two norms, their sum's norm, the residual and the layer scalar
    qg.qg_post_ffn(md, moe, wts["w_post1"], wts["w_post2"], wts["w_post"], wts["out_scale"], xt, H, T, 1e-6)
    yp, Ap = orc.post_ffn(mdh, moeh, c["w_post1"], c["w_post2"], c["w_post"], float(c["out_scale"][0]), x0, H, T,
                          1e-6)
    check_rows(host(xt), yp, Ap, "ffn tail")
    del pt

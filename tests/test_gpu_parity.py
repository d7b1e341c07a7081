"""GPU parity: the HIP path, called through the C ABI, against the f64 oracle
on the same seeded inputs.

Bars (from the method's contract):
  * dequantized weights bit-exact: each f32 equals the f64 value rounded to f32;
  * router ids exact (same experts, same order); weights |c - c_ref| <= 1e-6 c_ref;
  * every GEMV output row: |y - y_ref| <= 1e-5 * sum_c |W[r][c] x[c]|;
  * chained stages are checked stage by stage, each fed the GPU's own input to
    that stage; the activation's f32 rounding adds at most 1e-6 * R, where
    R = sum |c s| sum_f |W_d[h,f]| |g_f u_f| (see the oracle's moe_down).
"""
import numpy as np
import pytest

import gguf_synth as gs

pytestmark = pytest.mark.gpu

TOL = 1e-5
TYPES = [gs.Q8_0, gs.Q4_0, gs.Q4_K, gs.Q6_K]


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def say(*a):
    print("[case]", *a, flush=True)


def dev(a, offset=0):
    """numpy array -> device tensor; `offset` bytes of padding in front (to
    place the data at a 2-mod-4 address when offset = 2)."""
    torch = _torch()
    if offset:
        raw = np.frombuffer(np.ascontiguousarray(a).tobytes(), np.uint8)
        buf = torch.zeros(raw.size + 16, dtype=torch.uint8, device="cuda")
        buf[offset:offset + raw.size] = torch.from_numpy(raw.copy()).cuda()
        return buf, buf.data_ptr() + offset
    t = torch.from_numpy(np.ascontiguousarray(a).copy()).cuda()
    return t, t.data_ptr()


def host(t):
    _torch().cuda.synchronize()
    return t.cpu().numpy()


def check_rows(y, y_ref, A, what):
    err = np.abs(y.astype(np.float64) - y_ref)
    bound = TOL * A
    bad = err > bound
    ratio = (err / np.maximum(A, 1e-300)).max()
    assert not bad.any(), "%s: %d of %d outputs out of bound; worst err/A = %.3g" % (what, bad.sum(), bad.size, ratio)
    return ratio


def _align256(n):
    return (n + 255) // 256 * 256


def check_act(orc, act, gu, a, F, what):
    """The activation the gated launch wrote against the oracle's f64 act(g)*u
    of the same f32 gate and up sums: f32 evaluation error, a few ulp of |g*u|."""
    for i in range(gu.shape[0]):
        ref = orc.glu(act, gu[i], F)
        bound = 1e-6 * np.abs(gu[i, :F].astype(np.float64) * gu[i, F:].astype(np.float64)) + 1e-30
        err = np.abs(a[i].astype(np.float64) - ref)
        assert np.all(err <= bound), "%s vector %d: worst err/|gu| %.3g" % (what, i, (err / bound).max() * 1e-6)


def gpu_gemv(t, W, x, rows, cols, ntok, w_offset=0):
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    Wt, Wp = dev(W, w_offset)
    xt, _ = dev(x.astype(np.float32))
    y = torch.full((ntok, rows), float("nan"), dtype=torch.float32, device="cuda")
    qg.qg_gemv(t, Wp, xt, y, rows, cols, ntok)
    return host(y)


# ------------------------------------------------------------ dequantize ----
@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("shape,off", [((5, 7), 0), ((3, 9), 2), ((64, 20), 0), ((1, 1), 2)])
def test_dequant_bit_exact(orc, t, shape, off):
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    rows, nbk = shape
    cols = nbk * gs.QK[t]
    W = gs.weights(t, gs.rng(1000 + t + rows), rows, cols)
    say("dequant", gs.NAMES[t], rows, cols, "offset", off)
    Wt, Wp = dev(W, off)
    out = torch.full((rows, cols), float("nan"), dtype=torch.float32, device="cuda")
    qg.qg_dequant(t, Wp, out, rows, cols)
    got = host(out)
    ref = orc.dequant(t, W, rows * cols).reshape(rows, cols).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------------------ GEMV ----
GEMV_CASES = [
    # (rows, blocks per row, ntok, W byte offset): several tiles, ragged tails,
    # odd blocks per row (rows alternate 0 / 2 mod 4), misaligned W
    (1, 1, 1, 0), (7, 3, 1, 0), (130, 20, 1, 0), (257, 9, 1, 2), (96, 64, 1, 0),
    (33, 80, 2, 0), (70, 7, 3, 0), (40, 12, 5, 2), (19, 24, 8, 0), (65, 88, 16, 0), (300, 5, 16, 0),
]


@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("rows,nbk,ntok,off", GEMV_CASES)
def test_gemv_parity(orc, t, rows, nbk, ntok, off):
    if t in (gs.Q4_K, gs.Q6_K):
        nbk = max(1, nbk // 4)
    cols = nbk * gs.QK[t]
    g = gs.rng(2000 + 31 * t + rows + ntok)
    W = gs.weights(t, g, rows, cols)
    x = gs.activations(g, ntok, cols)
    say("gemv", gs.NAMES[t], rows, cols, "T", ntok, "offset", off)
    y = gpu_gemv(t, W, x, rows, cols, ntok, off)
    y_ref, A = orc.gemv(t, W, x, rows, cols, ntok)
    check_rows(y, y_ref, A, "gemv %s %dx%d T=%d" % (gs.NAMES[t], rows, cols, ntok))


# One token against K-quant rows: the quarter-block kernel (plan kind 4) for
# every shape below whose x is 16-byte aligned -- fewer units per row than
# lanes, units not a multiple of the lanes, odd blocks per row (Q6_K rows then
# alternate 0 / 2 mod 4), W at a 2-byte phase, x wide enough for 8-wave
# workgroups; a misaligned x takes the block-unit kernels instead.
KQ1_CASES = [
    # type, rows, cols, W offset, x offset
    (gs.Q4_K, 1, 256, 0, 0), (gs.Q4_K, 37, 768, 0, 0), (gs.Q4_K, 203, 5120, 2, 0), (gs.Q4_K, 130, 20480, 0, 0),
    (gs.Q4_K, 64, 1280, 0, 4),
    (gs.Q6_K, 1, 256, 0, 0), (gs.Q6_K, 45, 1280, 0, 0), (gs.Q6_K, 77, 2816, 2, 0), (gs.Q6_K, 33, 17408, 0, 0),
    (gs.Q6_K, 50, 4352, 0, 4), (gs.Q6_K, 129, 4352, 2, 0),
]


@pytest.mark.parametrize("t,rows,cols,w_off,x_off", KQ1_CASES)
def test_gemv_kquant_one_token(orc, t, rows, cols, w_off, x_off):
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    plan = qg.qg_gemv_plan(t, rows, cols, 1, w_off == 0)
    assert plan["kind"] == 4, plan
    g = gs.rng(2300 + t + rows + cols + w_off + x_off)
    W = gs.weights(t, g, rows, cols)
    x = gs.activations(g, 1, cols)
    say("gemv one token", gs.NAMES[t], rows, cols, "W offset", w_off, "x offset", x_off, plan)
    Wt, Wp = dev(W, w_off)
    xt, xp = dev(x, x_off)
    y = torch.full((1, rows), float("nan"), dtype=torch.float32, device="cuda")
    qg.qg_gemv(t, Wp, xp, y, rows, cols, 1)
    yh = host(y)
    del Wt, xt
    y_ref, A = orc.gemv(t, W, x, rows, cols, 1)
    check_rows(yh, y_ref, A, "gemv %s %dx%d one token" % (gs.NAMES[t], rows, cols))


# x wider than two workgroups' share of LDS, with more row tiles than one
# round at one workgroup per CU holds, is staged in chunks of whole row
# elements (restaged per tile row): T = 1 and 2, aligned and 2-byte-offset
# weights, ragged last tiles; sampled rows plus the first and last 40
XCHUNK_CASES = [
    (gs.Q6_K, 8300, 17408, 1, 0), (gs.Q6_K, 8310, 17408, 2, 2), (gs.Q4_K, 16500, 20480, 1, 0),
    (gs.Q8_0, 4100, 32768, 1, 0), (gs.Q8_0, 4110, 24576, 2, 2), (gs.Q4_0, 4105, 40960, 1, 2),
]


def _sample(g, rows, n):
    idx = set(g.choice(rows, size=min(n, rows), replace=False).tolist())
    idx.update(range(40))
    idx.update(range(rows - 40, rows))
    return np.array(sorted(idx), dtype=np.int64)


@pytest.mark.parametrize("t,rows,cols,ntok,off", XCHUNK_CASES)
def test_gemv_x_chunks(orc, t, rows, cols, ntok, off):
    g = gs.rng(2500 + t + rows + ntok)
    W = gs.weights(t, g, rows, cols)
    x = gs.activations(g, ntok, cols)
    say("gemv x chunks", gs.NAMES[t], rows, cols, "T", ntok, "offset", off)
    y = gpu_gemv(t, W, x, rows, cols, ntok, off)
    ri = _sample(g, rows, 400)
    y_ref, A = orc.gemv(t, W, x, rows, cols, ntok, row_idx=ri)
    check_rows(y[:, ri], y_ref, A, "gemv x chunks %s %dx%d T=%d" % (gs.NAMES[t], rows, cols, ntok))
    assert np.isfinite(y).all()


@pytest.mark.parametrize("t", TYPES)
def test_gemv_scaling_property(t):
    """y(2x) = 2 y(x) bitwise: the kernels' arithmetic commutes with an exact
    power-of-two scale (checked at a size where the oracle is not needed)."""
    rows, cols = 2048, 4096
    g = gs.rng(77 + t)
    W = gs.weights(t, g, rows, cols)
    x = gs.activations(g, 1, cols)
    say("gemv-scale", gs.NAMES[t], rows, cols)
    y1 = gpu_gemv(t, W, x, rows, cols, 1)
    y2 = gpu_gemv(t, W, 2 * x, rows, cols, 1)
    assert np.array_equal(y2, 2 * y1)


# --------------------------------------------------------------- router -----
@pytest.mark.parametrize("E,k,T", [(128, 8, 1), (128, 8, 16), (256, 32, 3), (8, 8, 2), (5, 1, 1)])
def test_router_parity(orc, E, k, T):
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    lg = gs.logits(gs.rng(3000 + E + k + T), T, E)
    lg[0, 1] = lg[0, E - 1] = lg[0].max() + 1.0    # an exact tie at the top
    if E > 20:
        lg[-1, 10:14] = 0.25                       # a tie inside the picks
    say("router", E, k, T)
    lt, _ = dev(lg)
    ids = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros((T, k), dtype=torch.float32, device="cuda")
    qg.qg_router_topk(lt, E, k, T, ids, w)
    ids_ref, w_ref = orc.router_topk(lg, E, k, T)
    assert np.array_equal(host(ids), ids_ref)
    assert np.all(np.abs(host(w) - w_ref) <= 1e-6 * w_ref)


@pytest.mark.parametrize("E,k", [(16, 8), (128, 8), (256, 32)])
def test_router_nan_logits(orc, E, k):
    """NaN logits rank below every number, lowest index first among NaNs
    (the oracle's reading); ids exact, weights NaN exactly where the oracle's
    are (a NaN pick makes the whole token's sum NaN)."""
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    T = 3
    g = gs.rng(3500 + E + k)
    lg = gs.logits(g, T, E)
    lg[0, g.choice(E, size=E - k // 2, replace=False)] = np.nan   # NaNs get picked
    lg[1, [0, 3, E - 1]] = np.nan                                  # NaNs never reached
    lg[2, 0] = np.nan
    lg[2, 1] = -np.inf
    say("router nan", E, k, T)
    lt, _ = dev(lg)
    ids = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros((T, k), dtype=torch.float32, device="cuda")
    qg.qg_router_topk(lt, E, k, T, ids, w)
    ids_ref, w_ref = orc.router_topk(lg, E, k, T)
    assert np.array_equal(host(ids), ids_ref)
    wg = host(w)
    assert np.array_equal(np.isnan(wg), np.isnan(w_ref))
    fin = ~np.isnan(w_ref)
    assert np.all(np.abs(wg[fin] - w_ref[fin]) <= 1e-6 * w_ref[fin])


# --------------------------------------------------------------- dense MLP --
@pytest.mark.parametrize("t,act,H,F,T", [(gs.Q8_0, 0, 256, 320, 1), (gs.Q4_0, 1, 320, 224, 3),
                                         (gs.Q4_K, 0, 512, 768, 2), (gs.Q6_K, 1, 768, 512, 16),
                                         (gs.Q4_0, 1, 2816, 2112, 16), (gs.Q4_0, 1, 2816, 2112, 1),
                                         # gate / up rows of 32 tiles: split 4 ways in 16s
                                         (gs.Q4_0, 1, 2048, 512, 16),
                                         # x too wide for LDS beside two workgroups' stages
                                         (gs.Q6_K, 0, 17408, 256, 1), (gs.Q8_0, 1, 24576, 96, 1)])
def test_mlp_stagewise(orc, t, act, H, F, T):
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    g = gs.rng(4000 + t + H + T)
    Wg, Wu, Wd = gs.weights(t, g, F, H), gs.weights(t, g, F, H), gs.weights(t, g, H, F)
    x = gs.activations(g, T, H)
    say("mlp", gs.NAMES[t], "act", act, H, F, "T", T)
    tg, _ = dev(Wg)
    tu, _ = dev(Wu)
    td, _ = dev(Wd)
    xt, _ = dev(x)
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(qg.qg_mlp_workspace_size(t, H, F, T) // 4, dtype=torch.float32, device="cuda")
    qg.qg_mlp(t, act, tg, tu, td, H, F, xt, y, T, ws)
    wsh = host(ws)
    gu = wsh[:T * 2 * F].reshape(T, 2 * F)
    a0 = _align256(T * 2 * F * 4) // 4
    check_act(orc, act, gu, wsh[a0:a0 + T * F].reshape(T, F), F, "mlp act")
    # stage 1: gate || up
    yg, Ag = orc.gemv(t, Wg, x, F, H, T)
    yu, Au = orc.gemv(t, Wu, x, F, H, T)
    check_rows(gu, np.concatenate([yg, yu], 1), np.concatenate([Ag, Au], 1), "mlp gate||up")
    # stage 2: down fed the GPU's gate||up, with the activation's rounding term
    yh = host(y)
    Wabs = np.abs(orc.dequant(t, Wd, H * F).reshape(H, F))
    for tt in range(T):
        a = orc.glu(act, gu[tt], F)
        yd, Ad = orc.gemv_f64(t, Wd, a, H, F)
        gsum = np.abs(gu[tt, :F].astype(np.float64) * gu[tt, F:].astype(np.float64))
        R = Wabs @ gsum
        err = np.abs(yh[tt] - yd)
        assert np.all(err <= TOL * Ad + 1e-6 * R), "mlp down token %d: worst err/A %.3g" % (
            tt, (err / Ad).max())


# ------------------------------------------------------------------- MoE ----
def _moe_case(t, act, H, F, E, k, T, seed, with_scale):
    g = gs.rng(seed)
    pool, rec, gu_off, d_off = gs.expert_pool(t, g, E, H, F)
    lg = gs.logits(g, T, E)
    x = gs.activations(g, T, H)
    ds = gs.down_scales(g, E) if with_scale else None
    return dict(t=t, act=act, H=H, F=F, E=E, k=k, T=T, pool=pool, rec=rec, gu_off=gu_off, d_off=d_off,
                lg=lg, x=x, ds=ds)


def run_moe_gpu(c, slots=None, perm_pool=None, pool_dev=None, n_slots=0):
    """pool_dev: a device pool (tensor) to read instead of c["pool"], with
    n_slots slots of c["rec"] bytes."""
    import gguf_dequant_gemv_amd as qg
    torch = _torch()
    if pool_dev is not None:
        pt, pp = pool_dev, pool_dev.data_ptr()
    else:
        pool = c["pool"] if perm_pool is None else perm_pool
        pt, pp = dev(pool)
    dst = dev(c["ds"])[0] if c["ds"] is not None else None
    m = qg.make_moe(c["t"], c["act"], c["H"], c["F"], c["E"], pp + c["gu_off"], c["rec"], pp + c["d_off"],
                    c["rec"], dst, n_slots)
    slots = np.arange(c["E"], dtype=np.int32) if slots is None else slots
    st, _ = dev(slots.astype(np.int32))
    lt, _ = dev(c["lg"])
    xt, _ = dev(c["x"])
    T, k, H = c["T"], c["k"], c["H"]
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    ids = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros((T, k), dtype=torch.float32, device="cuda")
    status = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    ws = torch.empty(qg.qg_moe_workspace_size(m, k, T) // 4, dtype=torch.float32, device="cuda")
    qg.qg_moe_ffn(m, lt, k, st, xt, y, T, ids, w, status, ws)
    wsh = host(ws)
    F = c["F"]
    a0 = _align256(T * k * 2 * F * 4) // 4
    out = dict(y=host(y), ids=host(ids), w=host(w), status=int(host(status)[0]),
               gu=wsh[:T * k * 2 * F].reshape(T, k, 2 * F), act=wsh[a0:a0 + T * k * F].reshape(T, k, F))
    del pt
    return out


MOE_CASES = [
    # type, act, H, F, E, k, T, scale
    (gs.Q8_0, 0, 256, 128, 16, 4, 1, False),
    (gs.Q4_0, 1, 320, 96, 12, 3, 5, True),
    (gs.Q4_K, 0, 512, 256, 8, 2, 16, False),
    (gs.Q6_K, 1, 256, 512, 6, 6, 2, True),
    (gs.Q8_0, 0, 2048, 768, 128, 8, 1, False),      # Qwen3-30B-A3B layer shape
    (gs.Q4_0, 1, 2816, 704, 128, 8, 16, True),      # Gemma-4 26B-A4B expert shape, T = 16
    (gs.Q4_0, 1, 2816, 704, 128, 8, 1, True),       # the same, one token
    (gs.Q8_0, 0, 256, 1536, 16, 8, 1, True),        # one token, two blocks per lane in the down launch
    (gs.Q4_0, 1, 320, 96, 12, 1, 1, True),          # one token, one pick
    (gs.Q8_0, 0, 256, 128, 256, 8, 1, False),       # one token, 256 experts: four logits per lane in the routing
    (gs.Q4_0, 1, 320, 96, 200, 8, 1, True),         # one token, a ragged expert count
    (gs.Q8_0, 0, 1088, 256, 32, 8, 1, True),        # one token, 3 rows a down workgroup, the last one ragged
    (gs.Q8_0, 0, 512, 1024, 16, 8, 1, True),        # one token, exactly 256 (pick, block) columns
    (gs.Q8_0, 0, 256, 128, 256, 8, 16, False),      # 16 tokens, 256 experts: the routing launch's four register sets
    (gs.Q4_0, 1, 320, 96, 200, 6, 5, True),         # 5 tokens, 200 experts: four sets, the last one partly empty
]


@pytest.mark.parametrize("t,act,H,F,E,k,T,scale", MOE_CASES)
def test_moe_stagewise(orc, t, act, H, F, E, k, T, scale):
    c = _moe_case(t, act, H, F, E, k, T, 5000 + t + H + T, scale)
    say("moe", gs.NAMES[t], "act", act, H, F, E, k, "T", T)
    _moe_check(orc, c)


@pytest.mark.parametrize("t,act", [(gs.Q8_0, 0), (gs.Q4_0, 1), (gs.Q4_K, 0)])
def test_moe_crowded_experts(orc, t, act):
    """Every token picks the same four experts (their logits lifted by 20):
    four groups of 16 pairs, each split into many chunks of the launches'
    token count, so the routing launch's lists of (group, chunk) sets run
    long and every chunk of a group must land on the right pairs."""
    H, F, E, k, T = 256, 256, 64, 4, 16
    c = _moe_case(t, act, H, F, E, k, T, 6100 + t, act == 1)
    c["lg"] = c["lg"].copy()
    c["lg"][:, [5, 17, 40, 63]] += np.float32(20.0)
    say("moe crowded", gs.NAMES[t], "act", act, H, F, E, k, "T", T)
    _moe_check(orc, c)


def _moe_check(orc, c, **run_kw):
    t, act, H, F, E, k, T = (c[key] for key in ("t", "act", "H", "F", "E", "k", "T"))
    r = run_moe_gpu(c, **run_kw)
    ref = orc.moe_ffn(t, act, H, F, E, c["pool"][c["gu_off"]:], c["rec"], c["pool"][c["d_off"]:], c["rec"],
                      c["ds"], c["lg"], k, np.arange(E, dtype=np.int32), c["x"], T, want_gu=True)
    assert r["status"] == 0
    assert np.array_equal(r["ids"], ref["ids"])
    assert np.all(np.abs(r["w"] - ref["c"]) <= 1e-6 * ref["c"])
    # stage 1: every pair's gate || up against the oracle's GEMV of that expert
    for tt in range(T):
        for j in range(k):
            e = int(ref["ids"][tt, j])
            base = e * c["rec"]
            yy, AA = orc.gemv(t, c["pool"][base:base + c["d_off"]], c["x"][tt:tt + 1], 2 * F, H, 1)
            check_rows(r["gu"][tt, j][None], yy, AA, "moe gate||up t%d j%d" % (tt, j))
    check_act(orc, act, r["gu"].reshape(T * k, 2 * F), r["act"].reshape(T * k, F), F, "moe act")
    # stage 2: down + combine fed the GPU's gate || up
    yd, Ad, R = orc.moe_down(t, act, H, F, c["pool"][c["d_off"]:], c["rec"], c["ds"],
                             np.arange(E, dtype=np.int32), ref["ids"], r["w"].astype(np.float64), r["gu"], T)
    err = np.abs(r["y"] - yd)
    assert np.all(err <= TOL * Ad + 1e-6 * R), "moe down/combine: worst err/A %.3g" % (err / Ad).max()
    # end to end against the independent f64 chain: reported; asserted only as a
    # sanity bound (the contract is the stage-wise check above)
    err2 = np.abs(r["y"] - ref["y"])
    print("[moe end-to-end] worst err/A_y = %.3g" % (err2 / ref["A"]).max(), flush=True)
    assert np.all(err2 <= 1e-3 * (ref["A"] + R))


def test_moe_absent_expert_and_slots(orc):
    t, act, H, F, E, k, T = gs.Q8_0, 0, 256, 128, 10, 3, 4
    c = _moe_case(t, act, H, F, E, k, T, 6001, True)
    say("moe-slots", E, k, T)
    base = run_moe_gpu(c)
    # permuted residency: expert e lives in slot perm[e]; same result bitwise
    perm = np.array([4, 7, 0, 9, 1, 3, 8, 2, 6, 5], np.int32)
    pool2 = np.empty_like(c["pool"])
    rec = c["rec"]
    for e in range(E):
        pool2[perm[e] * rec:(perm[e] + 1) * rec] = c["pool"][e * rec:(e + 1) * rec]
    moved = run_moe_gpu(c, slots=perm, perm_pool=pool2)
    assert np.array_equal(moved["y"], base["y"])
    # an absent picked expert: status word, and that token's row untouched
    slots = np.arange(E, dtype=np.int32)
    e_abs = int(base["ids"][2, 1])
    slots[e_abs] = -1
    r = run_moe_gpu(c, slots=slots)
    assert r["status"] == -2
    hit = [tt for tt in range(T) if e_abs in base["ids"][tt]]
    for tt in range(T):
        if tt in hit:
            assert np.all(np.isnan(r["y"][tt]))
        else:
            assert np.array_equal(r["y"][tt], base["y"][tt])


@pytest.mark.parametrize("t,act,E,k", [(gs.Q8_0, 0, 128, 8), (gs.Q4_0, 1, 200, 8), (gs.Q8_0, 0, 40, 3),
                                      (gs.Q4_0, 1, 256, 5)])
def test_moe_one_token_tied_logits(orc, t, act, E, k):
    """One token, routed inside the gated launch: exact ties among the router
    logits, six at the top and more just below, so the k-th place falls
    inside a run of equal logits (the lowest indices win); the picks, their
    order and the weights equal the oracle's router, then the stage-wise
    checks."""
    H, F, T = 256, 128, 1
    c = _moe_case(t, act, H, F, E, k, T, 6200 + E + k, act == 1)
    lg = c["lg"].copy()
    top = [E - 1, 3, 17, E // 2, 9, 1]
    lg[0, top] = np.float32(6.0)
    nxt = [e for e in ((7 * i + 5) % E for i in range(k + 3)) if e not in top]
    lg[0, nxt] = np.float32(5.5)
    c["lg"] = lg
    say("moe one token tied logits", gs.NAMES[t], "E", E, "k", k)
    _moe_check(orc, c)


@pytest.mark.parametrize("t,act", [(gs.Q8_0, 0), (gs.Q4_0, 1)])
def test_moe_one_token_pool_past_4gib(orc, t, act):
    """One token against an expert pool of a little over 4 GiB whose experts
    sit in its last slots: the column down launch addresses the pool with
    32-bit offsets, so this pool takes the row-walking down launch, and the
    gated launch reaches slots past 4 GiB; the same stage-wise checks as any
    other case."""
    torch = _torch()
    H, F, E, k, T = 256, 128, 6, 3, 1
    c = _moe_case(t, act, H, F, E, k, T, 6004 + t, act == 1)
    rec = c["rec"]
    n_slots = (4 * 2 ** 30 + 64 * 2 ** 20) // rec + E
    slots = np.array([n_slots - 1 - e for e in range(E)], np.int32)
    say("moe pool past 4 GiB", gs.NAMES[t], "slots", n_slots, "record", rec)
    big = torch.empty(n_slots * rec, dtype=torch.uint8, device="cuda")
    src = torch.from_numpy(c["pool"]).cuda()
    for e in range(E):
        s0 = int(slots[e]) * rec
        big[s0:s0 + rec] = src[e * rec:(e + 1) * rec]
    _moe_check(orc, c, slots=slots, pool_dev=big, n_slots=n_slots)
    del big


def test_moe_one_token_absent_expert_and_slots(orc):
    """The one-token down + combine launch: a permuted expert residency gives
    the same y bit for bit, and an absent picked expert leaves y untouched."""
    t, act, H, F, E, k, T = gs.Q4_0, 1, 320, 192, 10, 3, 1
    c = _moe_case(t, act, H, F, E, k, T, 6003, True)
    say("moe-slots one token", E, k)
    base = run_moe_gpu(c)
    assert base["status"] == 0 and not np.any(np.isnan(base["y"]))
    perm = np.array([4, 7, 0, 9, 1, 3, 8, 2, 6, 5], np.int32)
    pool2 = np.empty_like(c["pool"])
    rec = c["rec"]
    for e in range(E):
        pool2[perm[e] * rec:(perm[e] + 1) * rec] = c["pool"][e * rec:(e + 1) * rec]
    moved = run_moe_gpu(c, slots=perm, perm_pool=pool2)
    assert np.array_equal(moved["y"], base["y"])
    slots = np.arange(E, dtype=np.int32)
    slots[int(base["ids"][0, 2])] = -1
    r = run_moe_gpu(c, slots=slots)
    assert r["status"] == -2
    assert np.all(np.isnan(r["y"]))

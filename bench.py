#!/usr/bin/env python3
"""Effective weight-HBM bandwidth of the quantized GEMV / MoE path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 1] [--all] [--no-cpu]

A step is one pass of the named workload over one batch of synthetic inputs
already resident in HBM.  The default workload is the Q8_0 dense Qwen3-style
MLP decode (hidden 2560, ff 9728: gate||up -> SwiGLU -> down) followed by the
tied-head GEMV [151936 x 2560], one token: 492,646,400 weight bytes per step.
Two full copies of the weights alternate between steps so that no step finds
its weights in the 256 MB last-level cache.

Printed: one JSON line with the throughput (algorithmic weight bytes / time),
the roofline of the dominant kernel (the head GEMV, timed with HIP events on
the stream it runs on) and the oracle timed on the host cores.  --all adds one
JSON line per other workload (parity-test shapes timed the same way) to stderr.
"""
import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix rate, published
HERE = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(HERE, "profiles")
CSRC = os.path.join(HERE, "gguf_dequant_gemv_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="1",
                    help="0, 1, 2, 3a, 3b (Q6_K in the plane layout), 3bg (Q6_K as GGUF blocks), 4, 4t16; whole FFN blocks q35, q35t16, gblk, gblkt16; heads head8, "
                         "head6; prefill chunks p64, p256")
    ap.add_argument("--all", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--one-stream", action="store_true",
                    help="issue a step's independent branches in order on one stream (default: two streams)")
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0 = default)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (calibrates the HBM byte counters)")
    ap.add_argument("--dominant-only", action="store_true",
                    help="only launch the dominant kernel, eagerly, --steps times (for counter runs)")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="summarise four rocprofv3 --pmc output folders (FETCH_SIZE and WRITE_SIZE of a "
                         "--dominant-only run of --config with --steps steps, and of a --copy-probe run) into the "
                         "text kept under profiles/ (builds the workload for its name and bytes: needs the GPU)")
    ap.add_argument("--copy-mib", type=int, default=512, help="size of the --copy-probe run summarised")
    ap.add_argument("--counter-summary", nargs="+", metavar="DIR",
                    help="no GPU: per-kernel averages of every counter in rocprofv3 --pmc output folders of "
                         "--dominant-only runs (the measured steps' dispatches), and per-wave ratios of the SQ "
                         "instruction and cycle counters, as the text kept under profiles/")
    ap.add_argument("--stats-summary", nargs=2, metavar=("DIR", "COMMAND"),
                    help="no GPU: summarise the kernel statistics of a rocprofv3 --kernel-trace --stats run "
                         "(output folder DIR, made by COMMAND) into the text kept under profiles/")
    return ap.parse_args()


# --------------------------------------------------------------- workloads --
class Workload:
    name = ""
    bytes_per_step = 0
    dominant = ""            # kernel whose duration the roofline reports
    dominant_bytes = 0
    period = 1               # distinct weight copies the steps rotate through
    dominant_period = 1

    def step(self, i):
        raise NotImplementedError

    def dominant_step(self, i):
        self.step(i)

    def reset(self):
        """Restore state that steps update in place (a residual stream)."""

    def output(self):
        raise NotImplementedError


# Independent branches of a step (the dense MLP beside the routed experts)
# run on a second stream, forked from and joined back into the current one
# with events, as a serving engine would issue them; the graph capture takes
# the fork and join in.  --one-stream issues everything in order instead.
# A workload whose branches are too short for the overlap to pay for the
# cross-queue wait of the join (the Gemma-style block at one token: 54.1 us a
# layer in order, 57.8 us forked) keeps them in order by itself.
TWO_STREAMS = True


class Branches:
    def __init__(self, enabled=True):
        import torch
        self.side = torch.cuda.Stream() if TWO_STREAMS and enabled else None   # default priority

    def run(self, side_fn, main_fn):
        import torch
        if self.side is None:
            side_fn(None)
            main_fn()
            return
        cur = torch.cuda.current_stream()
        self.side.wait_stream(cur)      # fork: after everything already issued
        with torch.cuda.stream(self.side):
            side_fn(self.side)
        main_fn()
        cur.wait_stream(self.side)      # join


def _gen(seed):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return g


class DenseMlpHead(Workload):
    """gate||up -> SwiGLU -> down (qg_mlp) then head GEMV (qg_gemv), Q8_0, T = 1."""

    def __init__(self, copies=2, H=2560, F=9728, V=151936, planes=True):
        import torch
        import gguf_synth as gs
        import gguf_dequant_gemv_amd as qg
        self.qg = qg
        self.H, self.F, self.V = H, F, V
        # the tensors in the Q8_0 plane layout, prepared once as at load time
        # (the same bytes reordered; not part of a step), or GGUF blocks
        self.t = qg.QG_Q8_0_PLANES if planes else qg.QG_Q8_0
        self.sets = []
        for c in range(copies):
            g = _gen(100 + c)
            W = dict(Wg=(F, H), Wu=(F, H), Wd=(H, F), Wh=(V, H))
            for k in ("Wg", "Wu", "Wd", "Wh"):
                W[k] = (gs.device_weights(gs.Q8_0, W[k][0], W[k][1], g), W[k])
            if planes:
                for k in W:
                    src, (r, cc) = W[k]
                    dst = torch.empty_like(src)
                    qg.qg_prepare(qg.QG_Q8_0, src, dst, r, cc)
                    torch.cuda.synchronize()
                    W[k] = (dst, (r, cc))
            self.sets.append({k: v[0] for k, v in W.items()})
        self.x = gs.device_activations(1, H, _gen(7))
        self.h = torch.empty((1, H), dtype=torch.float32, device="cuda")
        self.logits = torch.empty((1, V), dtype=torch.float32, device="cuda")
        self.ws = torch.empty(qg.qg_mlp_workspace_size(self.t, H, F, 1) // 4, dtype=torch.float32, device="cuda")
        rb = gs.row_bytes(gs.Q8_0, H)
        self.mlp_bytes = 2 * F * rb + H * gs.row_bytes(gs.Q8_0, F)
        self.dominant_bytes = V * rb
        self.bytes_per_step = self.mlp_bytes + self.dominant_bytes
        lay = "plane layout" if planes else "GGUF blocks"
        self.name = ("q8_0 dense MLP decode 2560x9728 (gate||up, SwiGLU, down) + tied head 151936x2560, 1 token "
                     "(%s)" % lay)
        self.dominant = "head GEMV Q8_0 151936x2560 (%s)" % lay
        self.key = "head_q8_0_planes_151936x2560" if planes else "head_q8_0_151936x2560"
        self.period = self.dominant_period = copies

    def step(self, i):
        qg = self.qg
        s = self.sets[i % len(self.sets)]
        qg.qg_mlp(self.t, qg.QG_ACT_SILU, s["Wg"], s["Wu"], s["Wd"], self.H, self.F, self.x, self.h, 1, self.ws)
        qg.qg_gemv(self.t, s["Wh"], self.h, self.logits, self.V, self.H, 1)

    def dominant_step(self, i):
        s = self.sets[i % len(self.sets)]
        self.qg.qg_gemv(self.t, s["Wh"], self.h, self.logits, self.V, self.H, 1)

    def output(self):
        return self.logits

    def cpu_baseline(self):
        """The oracle over the whole step (same shapes, numpy-drawn weights):
        one warm-up run, then the median of five, on all the host threads
        the oracle runs with and on one."""
        import numpy as np
        import oracle
        import gguf_synth as gs
        c = gs.config1(seed=0)

        def step():
            yg, _ = oracle.gemv(gs.Q8_0, c["Wg"], c["x"], self.F, self.H)
            yu, _ = oracle.gemv(gs.Q8_0, c["Wu"], c["x"], self.F, self.H)
            a = oracle.glu(oracle.ACT_SILU, np.concatenate([yg[0], yu[0]]), self.F)
            h, _ = oracle.gemv_f64(gs.Q8_0, c["Wd"], a, self.H, self.F)
            oracle.gemv(gs.Q8_0, c["Wh"], h.astype(np.float32), self.V, self.H)

        many = oracle.set_threads(0)
        t_many = _median_run(step)
        oracle.set_threads(1)
        try:
            t_one = _median_run(step)
        finally:
            oracle.set_threads(many)
        rate = lambda t: round(self.bytes_per_step / t / 1e9, 3)
        return dict(value=rate(t_many), unit="GB/s", cores=many, kind="oracle",
                    sample="the whole step (gate||up, SwiGLU, down, head 151936x2560): median of 5 runs after "
                           "1 warm-up, %.3f s a run" % t_many,
                    single_core=dict(value=rate(t_one), unit="GB/s", cores=1,
                                     sample="the same step on one thread: median of 5 after 1 warm-up, "
                                            "%.3f s a run" % t_one))


def _median_run(fn, runs=5):
    """Seconds of fn(): one warm-up call, then the median of `runs` timed calls."""
    fn()
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return sorted(times)[len(times) // 2]


class GemvRot(Workload):
    """One quantized GEMV, T tokens, rotating through distinct weight copies."""

    def __init__(self, t, rows, cols, ntok, total_bytes, label, planes=False):
        import torch
        import gguf_synth as gs
        import gguf_dequant_gemv_amd as qg
        self.qg, self.t, self.rows, self.cols, self.ntok = qg, t, rows, cols, ntok
        wb = rows * gs.row_bytes(t, cols)
        copies = max(2, int(total_bytes // wb))
        g = _gen(300 + t)
        self.W = [gs.device_weights(t, rows, cols, g) for _ in range(copies)]
        if planes:
            # Q6_K in the plane layout, prepared once as at load time (the
            # same bytes reordered; not part of a step)
            self.t = qg.QG_Q6_K_PLANES if t == gs.Q6_K else qg.QG_Q8_0_PLANES
            for i, W in enumerate(self.W):
                P = torch.empty_like(W)
                qg.qg_prepare(t, W, P, rows, cols)
                self.W[i] = P
            torch.cuda.synchronize()
        self.x = gs.device_activations(ntok, cols, g)
        self.y = torch.empty((ntok, rows), dtype=torch.float32, device="cuda")
        self.bytes_per_step = wb
        self.dominant_bytes = wb
        self.name = label
        self.dominant = label
        self.key = "gemv_%s%s_%dx%d_t%d" % (gs.NAMES[t].lower(), "_planes" if planes else "", rows, cols, ntok)
        self.period = self.dominant_period = copies

    def step(self, i):
        self.qg.qg_gemv(self.t, self.W[i % len(self.W)], self.x, self.y, self.rows, self.cols, self.ntok)

    def output(self):
        return self.y


class MoeLayers(Workload):
    """qg_moe_ffn over L independent layers (pools, logits, x), T tokens."""

    def __init__(self, t, act, H, F, E, k, ntok, layers, scale, label, dense_ff=0):
        import torch
        import gguf_synth as gs
        import gguf_dequant_gemv_amd as qg
        self.qg, self.ntok, self.k = qg, ntok, k
        self.t, self.act, self.H, self.dense_ff = t, act, H, dense_ff
        rb_gu, rb_d = gs.row_bytes(t, H), gs.row_bytes(t, F)
        rec = 2 * F * rb_gu + H * rb_d
        self.layers = []
        g = _gen(500 + t)
        for _ in range(layers):
            gu = gs.device_weights(t, E * 2 * F, H, g)        # E records of gate||up
            dn = gs.device_weights(t, E * H, F, g)            # E records of down
            lg = torch.randn((ntok, E), generator=g, device="cuda")
            x = gs.device_activations(ntok, H, g)
            ds = (torch.rand(E, generator=g, device="cuda") * 1.5 + 0.5) if scale else None
            m = qg.make_moe(t, act, H, F, E, gu, 2 * F * rb_gu, dn, H * rb_d, ds)
            L = dict(m=m, gu=gu, dn=dn, lg=lg, x=x, ds=ds)
            if dense_ff:   # the dense MLP that runs beside the experts
                L.update(Wg=gs.device_weights(t, dense_ff, H, g), Wu=gs.device_weights(t, dense_ff, H, g),
                         Wd=gs.device_weights(t, H, dense_ff, g))
            self.layers.append(L)
        self.slots = torch.arange(E, dtype=torch.int32, device="cuda")
        self.y = torch.empty((ntok, H), dtype=torch.float32, device="cuda")
        self.ids = torch.empty((ntok, k), dtype=torch.int32, device="cuda")
        self.w = torch.empty((ntok, k), dtype=torch.float32, device="cuda")
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.ws = torch.empty(qg.qg_moe_workspace_size(self.layers[0]["m"], k, ntok) // 4, dtype=torch.float32,
                              device="cuda")
        # algorithmic bytes: each distinct picked expert's record once
        uniq = []
        for L in self.layers:
            lg = L["lg"].cpu()
            ids = torch.topk(lg, k, dim=1).indices
            uniq.append(len(set(ids.flatten().tolist())))
        self.uniq = uniq
        self.rec = rec
        self.dense_bytes = (2 * dense_ff * rb_gu + H * gs.row_bytes(t, dense_ff)) if dense_ff else 0
        if dense_ff:
            self.branches = Branches()
            self.ym = torch.empty((ntok, H), dtype=torch.float32, device="cuda")
            self.wsm = torch.empty(qg.qg_mlp_workspace_size(t, H, dense_ff, ntok) // 4, dtype=torch.float32,
                                   device="cuda")
            for L in self.layers:
                L["d"] = qg.make_dense_mlp(t, dense_ff, L["Wg"], L["Wu"], L["Wd"])
            self.wsd = torch.empty(qg.qg_moe_dense_workspace_size(self.layers[0]["m"], self.layers[0]["d"], k, ntok)
                                   // 4, dtype=torch.float32, device="cuda")
        self.bytes_per_step = int(sum(uniq) / len(uniq) * rec) + self.dense_bytes
        self.dominant_bytes = self.bytes_per_step
        self.name = label
        self.dominant = label
        self.key = "moe_%s_%d_e%d_t%d" % (gs.NAMES[t].lower(), H, E, ntok)
        self.period = self.dominant_period = layers

    def step(self, i):
        L = self.layers[i % len(self.layers)]
        moe = lambda: self.qg.qg_moe_ffn(L["m"], L["lg"], self.k, self.slots, L["x"], self.y, self.ntok, self.ids,
                                         self.w, self.status, self.ws)
        if not self.dense_ff:
            moe()
            return
        if self.ntok == 1:   # one token: the MLP's rows ride in the experts' two launches
            self.qg.qg_moe_ffn_dense(L["m"], L["d"], L["lg"], self.k, self.slots, L["x"], self.y, L["x"], self.ym,
                                     1, self.ids, self.w, self.status, self.wsd)
            return
        dense = lambda st: self.qg.qg_mlp(self.t, self.act, L["Wg"], L["Wu"], L["Wd"], self.H, self.dense_ff,
                                          L["x"], self.ym, self.ntok, self.wsm, stream=st)
        self.branches.run(dense, moe)

    def output(self):
        return self.y


class Qwen35Block(Workload):
    """A Qwen3.5/3.6-MoE-style FFN block, T tokens, over L independent layers:
    RMS norm of the residual stream, f32 router GEMV, routed experts plus the
    gated shared expert added into the residual (qg_rmsnorm_router at one
    token, else qg_rmsnorm and qg_gemv QG_F32; qg_moe_ffn_shared)."""

    def __init__(self, ntok, layers=16, H=2048, E=256, F=512, SF=512, k=8):
        import torch
        import gguf_synth as gs
        import gguf_dequant_gemv_amd as qg
        t = gs.Q8_0
        self.qg, self.ntok, self.k, self.H, self.E = qg, ntok, k, H, E
        rb_h, rb_f, rb_s = gs.row_bytes(t, H), gs.row_bytes(t, F), gs.row_bytes(t, SF)
        rec = 2 * F * rb_h + H * rb_f
        g = _gen(800 + ntok)
        self.layers = []
        uniq = []
        for _ in range(layers):
            gu = gs.device_weights(t, E * 2 * F, H, g)
            dn = gs.device_weights(t, E * H, F, g)
            L = dict(gu=gu, dn=dn, sg=gs.device_weights(t, SF, H, g), su=gs.device_weights(t, SF, H, g),
                     sd=gs.device_weights(t, H, SF, g),
                     gi=torch.randn(H, generator=g, device="cuda") / H ** 0.5,
                     router=torch.randn((E, H), generator=g, device="cuda") / H ** 0.5,
                     norm=torch.rand(H, generator=g, device="cuda") + 0.5,
                     x0=gs.device_activations(ntok, H, g))
            L["x"] = L["x0"].clone()
            L["m"] = qg.make_moe(t, qg.QG_ACT_SILU, H, F, E, gu, 2 * F * rb_h, dn, H * rb_f)
            L["sh"] = qg.make_shared_expert(t, SF, L["sg"], L["su"], L["sd"], L["gi"])
            self.layers.append(L)
        self.slots = torch.arange(E, dtype=torch.int32, device="cuda")
        self.xn = torch.empty((ntok, H), dtype=torch.float32, device="cuda")
        self.lg = torch.empty((ntok, E), dtype=torch.float32, device="cuda")
        self.ids = torch.empty((ntok, k), dtype=torch.int32, device="cuda")
        self.w = torch.empty((ntok, k), dtype=torch.float32, device="cuda")
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")
        L0 = self.layers[0]
        self.ws = torch.empty(qg.qg_moe_shared_workspace_size(L0["m"], L0["sh"], k, ntok) // 4,
                              dtype=torch.float32, device="cuda")
        # algorithmic bytes: each distinct picked expert's record once, the
        # shared expert, the router and the norm / gate vectors
        for L in self.layers:
            self.step_layer(L)
            uniq.append(len(set(self.ids.cpu().flatten().tolist())))
        self.reset()
        fixed = 2 * SF * rb_h + H * rb_s + E * H * 4 + 2 * H * 4
        self.bytes_per_step = int(sum(uniq) / len(uniq) * rec) + fixed
        self.dominant_bytes = self.bytes_per_step
        self.name = ("q8_0 Qwen3.5-MoE-style FFN block: rmsnorm, f32 router %dx%d, %d experts ff %d top-%d + "
                     "shared expert ff %d, residual; %d token(s)" % (E, H, E, F, k, SF, ntok))
        self.dominant = self.name
        self.key = "qwen35_block_q8_0_%d_e%d_t%d" % (H, E, ntok)
        self.period = self.dominant_period = layers

    def reset(self):
        for L in self.layers:
            L["x"].copy_(L["x0"])

    def step_layer(self, L):
        qg, T = self.qg, self.ntok
        if T == 1:   # the RMS norm and the router on it, one launch
            qg.qg_rmsnorm_router(L["x"], self.H, T, 1e-6, L["norm"], 1.0, L["router"], self.E, self.lg,
                                 [L["norm"]], [1.0], [self.xn])
        else:        # (each workgroup of the fused launch takes every token's norm: slower at 16)
            qg.qg_rmsnorm(L["x"], L["norm"], self.xn, self.H, T, 1e-6, 1.0)
            qg.qg_gemv(qg.QG_F32, L["router"], self.xn, self.lg, self.E, self.H, T)
        qg.qg_moe_ffn_shared(L["m"], L["sh"], self.lg, self.k, self.slots, self.xn, L["x"], T, self.ids, self.w,
                             self.status, self.ws)

    def step(self, i):
        self.step_layer(self.layers[i % len(self.layers)])

    def output(self):
        return torch_cat([L["x"] for L in self.layers])


class GemmaBlock(Workload):
    """Gemma4-26B-A4B-style FFN block at Q4_0, T tokens, over L layers: three
    RMS norms of the residual stream and the f32 router on one of them (one
    launch at one token: qg_rmsnorm_router; else qg_rmsnorm_multi and qg_gemv
    QG_F32), the dense GELU MLP, the routed experts, and the FFN tail into
    the residual (one token: qg_moe_ffn_dense, both in two launches; else
    qg_mlp beside qg_moe_ffn on two streams; then qg_post_ffn)."""

    def __init__(self, ntok, layers=16, H=2816, Fd=2112, E=128, F=704, k=8):
        import torch
        import gguf_synth as gs
        import gguf_dequant_gemv_amd as qg
        t = gs.Q4_0
        self.qg, self.ntok, self.k, self.H, self.E, self.Fd = qg, ntok, k, H, E, Fd
        self.branches = Branches(enabled=ntok > 1)
        rb_h, rb_f, rb_d = gs.row_bytes(t, H), gs.row_bytes(t, F), gs.row_bytes(t, Fd)
        rec = 2 * F * rb_h + H * rb_f
        g = _gen(900 + ntok)
        self.layers = []
        vec = lambda: torch.rand(H, generator=g, device="cuda") + 0.5
        for _ in range(layers):
            gu = gs.device_weights(t, E * 2 * F, H, g)
            dn = gs.device_weights(t, E * H, F, g)
            ds = torch.rand(E, generator=g, device="cuda") * 1.5 + 0.5
            L = dict(gu=gu, dn=dn, ds=ds, Wg=gs.device_weights(t, Fd, H, g), Wu=gs.device_weights(t, Fd, H, g),
                     Wd=gs.device_weights(t, H, Fd, g), router=torch.randn((E, H), generator=g, device="cuda"),
                     w_ffn=vec(), w_pre2=vec(), w_rs=vec(), w1=vec(), w2=vec(), w=vec(),
                     os=torch.rand(1, generator=g, device="cuda") * 0.5 + 0.5, x0=gs.device_activations(ntok, H, g))
            L["x"] = L["x0"].clone()
            L["m"] = qg.make_moe(t, qg.QG_ACT_GELU_TANH, H, F, E, gu, 2 * F * rb_h, dn, H * rb_f, ds)
            L["d"] = qg.make_dense_mlp(t, Fd, L["Wg"], L["Wu"], L["Wd"])
            self.layers.append(L)
        f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device="cuda")
        self.xn, self.xm, self.rt, self.md, self.moe = (f32(ntok, H) for _ in range(5))
        self.lg = f32(ntok, E)
        self.ids = torch.empty((ntok, k), dtype=torch.int32, device="cuda")
        self.w = f32(ntok, k)
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.slots = torch.arange(E, dtype=torch.int32, device="cuda")
        self.wsm = f32(qg.qg_mlp_workspace_size(t, H, Fd, ntok) // 4)
        self.ws = f32(qg.qg_moe_workspace_size(self.layers[0]["m"], k, ntok) // 4)
        self.wsd = f32(qg.qg_moe_dense_workspace_size(self.layers[0]["m"], self.layers[0]["d"], k, ntok) // 4)
        self.kr = 1.0 / H ** 0.5
        uniq = []
        for L in self.layers:
            self.step_layer(L)
            uniq.append(len(set(self.ids.cpu().flatten().tolist())))
        self.reset()
        fixed = 2 * Fd * rb_h + H * rb_d + E * H * 4 + 6 * H * 4
        self.bytes_per_step = int(sum(uniq) / len(uniq) * rec) + fixed
        self.dominant_bytes = self.bytes_per_step
        self.name = ("q4_0 Gemma4-style FFN block: 3 rmsnorms, dense GELU MLP %dx%d, f32 router %dx%d, %d experts "
                     "ff %d top-%d (down scale), FFN tail into the residual; %d token(s)" % (H, Fd, E, H, E, F, k,
                                                                                            ntok))
        self.dominant = self.name
        self.key = "gemma_block_q4_0_%d_e%d_t%d" % (H, E, ntok)
        self.period = self.dominant_period = layers

    def reset(self):
        for L in self.layers:
            L["x"].copy_(L["x0"])

    def step_layer(self, L):
        qg, T, H = self.qg, self.ntok, self.H

        if T == 1:   # ffn_norm, pre_ffw_norm_2 and the router on its scaled norm in one launch
            qg.qg_rmsnorm_router(L["x"], H, T, 1e-6, L["w_rs"], self.kr, L["router"], self.E, self.lg,
                                 [L["w_ffn"], L["w_pre2"]], [1.0, 1.0], [self.xn, self.xm])
        else:        # the three norms in one launch, the router on the third
            qg.qg_rmsnorm_multi(L["x"], H, T, 1e-6, [L["w_ffn"], L["w_pre2"], L["w_rs"]], [1.0, 1.0, self.kr],
                                [self.xn, self.xm, self.rt])
            qg.qg_gemv(qg.QG_F32, L["router"], self.rt, self.lg, self.E, H, T)

        def dense(st):   # the dense GELU MLP
            qg.qg_mlp(qg.QG_Q4_0, qg.QG_ACT_GELU_TANH, L["Wg"], L["Wu"], L["Wd"], H, self.Fd, self.xn, self.md, T,
                      self.wsm, stream=st)

        def experts():   # the routed experts
            qg.qg_moe_ffn(L["m"], self.lg, self.k, self.slots, self.xm, self.moe, T, self.ids, self.w, self.status,
                          self.ws)

        if T == 1:   # the dense MLP's rows ride in the experts' two launches
            qg.qg_moe_ffn_dense(L["m"], L["d"], self.lg, self.k, self.slots, self.xm, self.moe, self.xn, self.md, T,
                                self.ids, self.w, self.status, self.wsd)
        else:
            self.branches.run(dense, experts)
        qg.qg_post_ffn(self.md, self.moe, L["w1"], L["w2"], L["w"], L["os"], L["x"], H, T, 1e-6)

    def step(self, i):
        self.step_layer(self.layers[i % len(self.layers)])

    def output(self):
        return torch_cat([L["x"] for L in self.layers])


class HeadPick(Workload):
    """The decode loop's tail, 1 token: head GEMV, optional logit soft cap,
    greedy pick, and the picked token's (tied) embedding row gathered for the
    next step (qg_gemv, qg_argmax_embed: the pick and the gather in two
    launches), rotating weight copies."""

    def __init__(self, t, V, H, cap, emb_scale, total_bytes, label, planes=False):
        import torch
        import gguf_synth as gs
        import gguf_dequant_gemv_amd as qg
        self.qg, self.t, self.V, self.H, self.cap, self.scale = qg, t, V, H, cap, emb_scale
        wb = V * gs.row_bytes(t, H)
        copies = max(2, int(total_bytes // wb))
        g = _gen(1000 + t)
        self.W = [gs.device_weights(t, V, H, g) for _ in range(copies)]
        if planes:
            # the table in its plane layout, prepared once as at load time
            # (head GEMV and embedding gather both read it)
            for i, W in enumerate(self.W):
                P = torch.empty_like(W)
                qg.qg_prepare(t, W, P, V, H)
                torch.cuda.synchronize()
                self.W[i] = P
            self.t = qg.QG_Q8_0_PLANES if t == gs.Q8_0 else qg.QG_Q6_K_PLANES
        self.x = gs.device_activations(1, H, g)
        self.logits = torch.empty((1, V), dtype=torch.float32, device="cuda")
        self.idx = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.emb = torch.empty((1, H), dtype=torch.float32, device="cuda")
        self.ws = torch.empty(qg.qg_argmax_workspace_size(V, 1) // 4, dtype=torch.float32, device="cuda")
        self.bytes_per_step = wb + gs.row_bytes(t, H)
        self.dominant_bytes = wb
        self.name = label
        self.dominant = "head GEMV %s %dx%d%s" % (gs.NAMES[t], V, H, " (plane layout)" if planes else "")
        self.key = "head_pick_%s%s_%dx%d" % (gs.NAMES[t].lower(), "_planes" if planes else "", V, H)
        self.period = self.dominant_period = copies

    def step(self, i):
        qg = self.qg
        W = self.W[i % len(self.W)]
        qg.qg_gemv(self.t, W, self.x, self.logits, self.V, self.H, 1)
        qg.qg_argmax_embed(self.logits, self.V, 1, self.cap, self.idx, self.ws, self.t, W, self.V, self.H,
                           self.scale, self.emb)

    def dominant_step(self, i):
        self.qg.qg_gemv(self.t, self.W[i % len(self.W)], self.x, self.logits, self.V, self.H, 1)

    def output(self):
        return self.emb


class PrefillMlp(Workload):
    """The dense Qwen3-style MLP (hidden 2560, ff 9728, Q8_0) over a prompt
    chunk of T tokens (qg_mlp: gate||up with SwiGLU, then down), rotating
    weight copies.  Compute-bound from about 64 tokens: its roofline is the
    matrix cores' bf16 rate, counted in the contraction's own flops
    (2 * rows * cols * T per projection; the kernels spend three bf16 MFMAs
    per product for exactness)."""

    def __init__(self, ntok, H=2560, F=9728, copies=4):
        import torch
        import gguf_synth as gs
        import gguf_dequant_gemv_amd as qg
        self.qg, self.H, self.F, self.ntok = qg, H, F, ntok
        g = _gen(1100 + ntok)
        self.sets = [dict(Wg=gs.device_weights(gs.Q8_0, F, H, g), Wu=gs.device_weights(gs.Q8_0, F, H, g),
                          Wd=gs.device_weights(gs.Q8_0, H, F, g)) for _ in range(copies)]
        self.x = gs.device_activations(ntok, H, g)
        self.y = torch.empty((ntok, H), dtype=torch.float32, device="cuda")
        self.ws = torch.empty(qg.qg_mlp_workspace_size(qg.QG_Q8_0, H, F, ntok) // 4, dtype=torch.float32, device="cuda")
        rb = gs.row_bytes(gs.Q8_0, H)
        self.bytes_per_step = 2 * F * rb + H * gs.row_bytes(gs.Q8_0, F)
        self.flops_per_step = 2.0 * 3 * H * F * ntok
        self.dominant_bytes = self.bytes_per_step
        self.name = "q8_0 dense MLP prefill chunk 2560x9728 (gate||up, SwiGLU, down), %d tokens" % ntok
        self.dominant = self.name
        self.key = "prefill_mlp_q8_0_2560x9728_t%d" % ntok
        self.period = self.dominant_period = copies
        self.roof = "mfma"

    def step(self, i):
        s = self.sets[i % len(self.sets)]
        qg = self.qg
        qg.qg_mlp(qg.QG_Q8_0, qg.QG_ACT_SILU, s["Wg"], s["Wu"], s["Wd"], self.H, self.F, self.x, self.y, self.ntok,
                  self.ws)

    def output(self):
        return self.y


def torch_cat(ts):
    import torch
    return torch.cat([t.flatten() for t in ts])


def make_workload(name, copies):
    import gguf_synth as gs
    big = 1.2e9   # bytes of distinct weight copies to rotate through (> 2x the 256 MB cache)
    if name == "1":
        return DenseMlpHead(copies=copies or 2)
    if name == "1g":
        return DenseMlpHead(copies=copies or 2, planes=False)
    if name == "0":
        return GemvRot(gs.Q8_0, 1024, 2048, 1, big, "q8_0 GEMV 1024x2048, 1 token (plane layout)", planes=True)
    if name == "0g":
        return GemvRot(gs.Q8_0, 1024, 2048, 1, big, "q8_0 GEMV 1024x2048, 1 token (GGUF blocks)")
    if name == "3a":
        return GemvRot(gs.Q4_K, 17408, 5120, 1, big, "q4_k GEMV 17408x5120, 1 token")
    if name == "3b":
        return GemvRot(gs.Q6_K, 5120, 17408, 1, big, "q6_k GEMV 5120x17408, 1 token (plane layout)", planes=True)
    if name == "hq8":
        return GemvRot(gs.Q8_0, 151936, 2560, 1, big, "q8_0 GEMV 151936x2560 (tied head), 1 token (GGUF blocks)")
    if name == "hq8p":
        return GemvRot(gs.Q8_0, 151936, 2560, 1, big, "q8_0 GEMV 151936x2560 (tied head), 1 token (plane layout)",
                       planes=True)
    if name == "3bg":
        return GemvRot(gs.Q6_K, 5120, 17408, 1, big, "q6_k GEMV 5120x17408, 1 token (GGUF blocks as stored)")
    if name == "2":
        return MoeLayers(gs.Q8_0, 0, 2048, 768, 128, 8, 1, 16, False,
                         "q8_0 MoE layer 2048, 128 experts ff 768, top-8, 1 token")
    if name in ("4", "4t16"):
        T = 16 if name == "4t16" else 1
        return MoeLayers(gs.Q4_0, 1, 2816, 704, 128, 8, T, 16, True,
                         "q4_0 dense GELU MLP 2816x2112 + MoE layer 2816, 128 experts ff 704 (GELU, down scale), "
                         "top-8, %d token(s)" % T, dense_ff=2112)
    if name in ("q35", "q35t16"):
        return Qwen35Block(16 if name == "q35t16" else 1)
    if name in ("gblk", "gblkt16"):
        return GemmaBlock(16 if name == "gblkt16" else 1)
    if name in ("p64", "p256"):
        return PrefillMlp(int(name[1:]))
    if name in ("head8", "head8g"):
        return HeadPick(gs.Q8_0, 151936, 2560, 0.0, 1.0, big,
                        "q8_0 head 151936x2560 + argmax + tied embedding row, 1 token (%s)"
                        % ("GGUF blocks" if name == "head8g" else "plane layout"), planes=name == "head8")
    if name in ("head6", "head6g"):
        return HeadPick(gs.Q6_K, 262144, 2816, 30.0, float(2816 ** 0.5), big,
                        "q6_k head 262144x2816 + soft cap 30 + argmax + scaled tied embedding row, 1 token (%s)"
                        % ("GGUF blocks" if name == "head6g" else "plane layout"), planes=name == "head6")
    raise SystemExit("unknown config " + name)


def _capture(fn, idxs):
    """One HIP graph holding fn(i) for every i in idxs (captured on torch's
    capture stream, which the binding picks up as the current stream)."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in idxs:
            fn(i)
    return g


def time_workload(wl, steps, warmup):
    """(ms per step, ms per dominant-kernel launch).  Steps run as replays of
    captured graphs (period consecutive steps per graph, so exactly `steps`
    steps are timed); the dominant kernel is timed the same way on its own."""
    import torch
    for i in range(warmup):
        wl.step(i)
    torch.cuda.synchronize()
    # several steps per graph, a whole number of weight-copy rotations, so the
    # graph launch itself is amortised
    per = wl.period * max(1, 16 // wl.period)
    per = max(1, min(per, steps))
    full = _capture(wl.step, range(per))
    rem = steps % per
    tail = _capture(wl.step, range(rem)) if rem else None
    # a replay must reproduce the eager result bit for bit
    wl.reset()
    for i in range(per):
        wl.step(i)
    torch.cuda.synchronize()
    ref = wl.output().clone()
    wl.reset()
    full.replay()
    torch.cuda.synchronize()
    if not torch.equal(ref, wl.output()):
        raise SystemExit("bench: graph replay differs from the eager run")
    # untimed replays until the clocks have settled (at least 0.3 s of work)
    t_w = time.perf_counter()
    nrep = 0
    while nrep < 3 or time.perf_counter() - t_w < 0.3:
        full.replay()
        torch.cuda.synchronize()
        nrep += 1
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps // per):
        full.replay()
    if tail is not None:
        tail.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    log("[bench] %d steps: %.4f ms/step by events, %.4f ms/step by the host clock" % (steps, ms, wall * 1e3 / steps))
    # after the timed region: the spread over replays timed one by one, and
    # one step alone (a graph of a single step: the latency one token sees)
    def timed(g, n):
        out = []
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b))
        return sorted(out)
    reps = timed(full, 20)
    per_step = [r / per for r in reps]
    g1 = _capture(wl.step, range(1))
    one = timed(g1, 20)
    q = lambda v, f: v[min(len(v) - 1, int(f * len(v)))]
    spread = {"p10_ms": round(q(per_step, 0.1), 5), "p50_ms": round(q(per_step, 0.5), 5),
              "p90_ms": round(q(per_step, 0.9), 5), "replays": len(reps), "steps_per_replay": per,
              "single_step_p50_ms": round(q(one, 0.5), 5)}
    del g1
    # dominant kernel alone, same rotation
    dper = wl.dominant_period * max(1, 32 // wl.dominant_period)
    dper = max(1, min(dper, 64))
    dg = _capture(wl.dominant_step, range(dper))
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < 0.1:
        dg.replay()
        torch.cuda.synchronize()
    nrep = max(1, (steps + dper - 1) // dper)
    e0.record()
    for _ in range(nrep):
        dg.replay()
    e1.record()
    torch.cuda.synchronize()
    dom_ms = e0.elapsed_time(e1) / (nrep * dper)
    return ms, dom_ms, spread

# ------------------------------------------------------ counter summaries --
def source_hash():
    """sha256 over the HIP sources: a counter summary holds only for the
    kernels it was taken on."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".h", ".hip")):
            h.update(f.encode())
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def _counter_rows(folder, counter):
    """(dispatch id, kernel name, value) of every dispatch that recorded
    `counter`, in dispatch order."""
    import csv
    out = []
    for root, _, files in os.walk(folder):
        for f in files:
            if f.endswith("counter_collection.csv"):
                with open(os.path.join(root, f)) as fh:
                    for r in csv.DictReader(fh):
                        if r["Counter_Name"] == counter:
                            out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    return sorted(out)


def _step_dispatches(rows):
    """The library's dispatches of the measured steps: those after the last
    dispatch of anything else (the inputs' generation and copies come first;
    the steps launch only this library's kernels)."""
    last_other = max([d for d, n, _ in rows if "qg::" not in n], default=-1)
    return [(d, n, v) for d, n, v in rows if d > last_other and "qg::" in n]


def traffic_summary(fetch_dir, write_dir, cfetch_dir, cwrite_dir, copy_mib, wl_key, bytes_per_launch, steps):
    """Text summary: HBM bytes per dominant launch (one step of the dominant
    part: one kernel, or a step's kernels together) from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) summed over the measured steps' dispatches,
    each counter scaled by what it reads for a plain device copy of known
    size."""
    def per_step(folder, counter):
        rows = _step_dispatches(_counter_rows(folder, counter))
        if not rows:
            raise SystemExit("no %s rows of this library's kernels in %s" % (counter, folder))
        per_kernel = {}
        for _, n, v in rows:
            k = n.replace("void qg::", "").split("(qg::")[0].split("(float")[0]
            per_kernel.setdefault(k, []).append(v)
        return sum(v for _, _, v in rows) / steps, len(rows), per_kernel

    def copy_avg(folder, counter):
        rows = [v for _, n, v in _counter_rows(folder, counter) if "copyBuffer" in n or "copy" in n.lower()]
        if not rows:
            raise SystemExit("no %s rows of a copy kernel in %s" % (counter, folder))
        return sum(rows) / len(rows), len(rows)
    f, nf, kf = per_step(fetch_dir, "FETCH_SIZE")
    w, nw, kw = per_step(write_dir, "WRITE_SIZE")
    cf, ncf = copy_avg(cfetch_dir, "FETCH_SIZE")
    cw, ncw = copy_avg(cwrite_dir, "WRITE_SIZE")
    kib = copy_mib * 1024.0
    ff, fw = kib / cf, kib / cw
    traffic = (f * ff + w * fw) * 1024.0
    lines = [
        "workload: %s" % wl_key,
        "steps: %d (%d dispatches of this library's kernels counted)" % (steps, nf),
    ]
    for k in sorted(kf):
        lines.append("kernel: %s  dispatches %d  fetch_kib_avg %.1f  write_kib_avg %.1f" % (
            k, len(kf[k]), sum(kf[k]) / len(kf[k]), sum(kw.get(k, [0.0])) / max(1, len(kw.get(k, [])))))
    lines += [
        "fetch_kib_per_step: %.1f" % f,
        "write_kib_per_step: %.1f" % w,
        "copy_probe_mib: %d (read %d MiB, write %d MiB per copy)" % (copy_mib, copy_mib, copy_mib),
        "copy_fetch_kib: %.1f (%d dispatches) -> fetch factor %.4f" % (cf, ncf, ff),
        "copy_write_kib: %.1f (%d dispatches) -> write factor %.4f" % (cw, ncw, fw),
        "traffic_bytes_per_launch: %.0f" % traffic,
        "algorithmic_bytes_per_launch: %d" % bytes_per_launch,
        "traffic_over_algorithmic: %.4f" % (traffic / bytes_per_launch),
        "source_sha256: %s" % source_hash(),
    ]
    return "\n".join(lines) + "\n"


def counter_summary(folders):
    """Per kernel: the average of each counter over the measured steps'
    dispatches of this library's kernels (every folder one --pmc pass), and
    per wave: VALU / LDS / SALU / VMEM instructions and the SQ cycle counts
    when those counters were taken (SQ cycle counters tick once per 4 cycles
    on this chip; the ratios are given as counted)."""
    import csv
    per = {}
    for folder in folders:
        rows = {}
        for root, _, files in os.walk(folder):
            for f in files:
                if f.endswith("counter_collection.csv"):
                    with open(os.path.join(root, f)) as fh:
                        for r in csv.DictReader(fh):
                            rows.setdefault(r["Counter_Name"], []).append(
                                (int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
        for counter, rr in rows.items():
            for _, n, v in _step_dispatches(sorted(rr)):
                k = n.replace("void qg::", "").split("(qg::")[0].split("(float")[0]
                per.setdefault(k, {}).setdefault(counter, []).append(v)
    lines = ["source_sha256: %s" % source_hash()]
    for k in sorted(per):
        avg = {c: sum(v) / len(v) for c, v in per[k].items()}
        lines.append("kernel: %s" % k)
        for c in sorted(avg):
            lines.append("  %-28s %16.1f  (%d dispatches)" % (c, avg[c], len(per[k][c])))
        w = avg.get("SQ_WAVES")
        if w:
            for c in ("SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD", "SQ_WAVE_CYCLES",
                      "SQ_ACTIVE_INST_VALU", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_LDS"):
                if c in avg:
                    lines.append("  per wave %-24s %10.1f" % (c, avg[c] / w))
            if "SQ_WAVE_CYCLES" in avg and "SQ_ACTIVE_INST_VALU" in avg:
                lines.append("  VALU issue / wave lifetime: %.3f" % (avg["SQ_ACTIVE_INST_VALU"] / avg["SQ_WAVE_CYCLES"]))
    return "\n".join(lines) + "\n"


def stats_summary(folder, command):
    """Per-kernel table from a rocprofv3 --kernel-trace run: this library's
    kernels by name and grid (one template can serve several shapes), everything
    else (input generation, copies) summed."""
    import csv
    rows = []
    for root, _, files in os.walk(folder):
        for f in files:
            if f.endswith("kernel_trace.csv"):
                with open(os.path.join(root, f)) as fh:
                    rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit("no kernel_trace.csv under " + folder)
    groups, other, n_other = {}, 0.0, 0
    for r in rows:
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if "qg::" not in r["Kernel_Name"]:
            other += dur
            n_other += 1
            continue
        name = r["Kernel_Name"].replace("void qg::", "").split("(qg::")[0].split("(float")[0]
        key = (name, int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]), int(r["Grid_Size_Y"]),
               int(r["Grid_Size_Z"]))
        groups.setdefault(key, []).append(dur)
    out = ["command: " + command, "source_sha256: " + source_hash(), "",
           "%-44s %-16s %6s %10s %10s %10s" % ("kernel", "grid (wg)", "calls", "avg_us", "min_us", "max_us")]
    for key, d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        out.append("%-44s %-16s %6d %10.3f %10.3f %10.3f" % (key[0][:44], "%dx%dx%d" % key[1:], len(d),
                                                            sum(d) / len(d), min(d), max(d)))
    out.append("%-44s %-16s %6d %10s (total %.1f us)" % ("(other kernels: inputs, copies)", "", n_other, "", other))
    return "\n".join(out) + "\n"


def load_traffic(wl_key):
    """Measured HBM bytes per launch for this workload's dominant kernel, or
    None when no summary exists or the kernels changed since it was taken."""
    path = os.path.join(PROFILES, "traffic_%s.txt" % wl_key)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line:
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != source_hash():
        return None
    try:
        return int(float(vals["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def result_line(wl, ms, dom_ms, steps, warmup, cpu=None, spread=None):
    gbs = wl.bytes_per_step / (ms * 1e-3) / 1e9
    dom_gbs = wl.dominant_bytes / (dom_ms * 1e-3) / 1e9
    out = {
        "metric": "effective weight HBM GB/s (and % of peak) per quantized GEMV / MoE layer, 1 tok",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 accumulate over GGUF-quantized weights (q8_0/q4_0/q4_k/q6_k)",
        "data": "synthetic (seeded), inputs resident in HBM",
        "config": {"workload": wl.name, "bytes_per_step": wl.bytes_per_step, "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2)},
        "roofline": {"bound": "hbm", "achieved": round(dom_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": load_traffic(wl.key),
                     "kernel": wl.dominant, "bytes_per_launch": wl.dominant_bytes,
                     "avg_launch_us": round(dom_ms * 1e3, 3)},
    }
    if getattr(wl, "roof", "hbm") == "mfma":
        tf = wl.flops_per_step / (dom_ms * 1e-3) / 1e12
        out["roofline"].update(bound="mfma", achieved=round(tf, 2), peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                               frac=round(tf / MFMA_BF16_PEAK_TFLOPS, 4), flops_per_launch=wl.flops_per_step)
        out["config"]["tokens_per_s"] = round(wl.ntok / (ms * 1e-3), 1)
    if hasattr(wl, "branches"):
        out["config"]["streams"] = 2 if wl.branches.side is not None else 1
    if cpu is not None:
        out["cpu_baseline"] = cpu
    if spread is not None:
        out["spread"] = spread
    return out


def main():
    global TWO_STREAMS
    args = parse()
    TWO_STREAMS = not args.one_stream
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only (the path has no multi-GPU leg); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.stats_summary:
        sys.stdout.write(stats_summary(*args.stats_summary))
        return
    if args.counter_summary:
        sys.stdout.write(counter_summary(args.counter_summary))
        return
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        n = args.copy_probe << 18          # float32 elements
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copied %d MiB five times" % args.copy_probe)
        return
    import gguf_dequant_gemv_amd as qg
    qg.lib()   # fails loudly if the HIP library is not built
    log("[bench] workload", args.config)
    wl = make_workload(args.config, args.copies)
    if args.traffic_summary:   # (the workload built only for its name and algorithmic bytes)
        sys.stdout.write(traffic_summary(*args.traffic_summary, args.copy_mib, wl.key, wl.dominant_bytes,
                                         args.steps))
        return
    if args.dominant_only:
        for i in range(args.steps):
            wl.dominant_step(i)
        torch.cuda.synchronize()
        log("[bench] %d dominant launches: %s" % (args.steps, wl.dominant))
        return
    ms, dom_ms, spread = time_workload(wl, args.steps, args.warmup)
    log("[bench] %.4f ms/step, dominant %.4f ms" % (ms, dom_ms))
    cpu = None
    if not args.no_cpu:
        log("[bench] timing the oracle on the host cores")
        cpu = wl.cpu_baseline() if hasattr(wl, "cpu_baseline") else None
    print(json.dumps(result_line(wl, ms, dom_ms, args.steps, args.warmup, cpu, spread)), flush=True)
    if args.all:
        for name in ("0", "3a", "3b", "3bg", "2", "4", "4t16", "q35", "q35t16", "gblk", "gblkt16", "head8", "head6",
                     "p64", "p256"):
            if name == args.config:
                continue
            log("[bench] workload", name)
            w2 = make_workload(name, 0)
            ms2, dom2, sp2 = time_workload(w2, args.steps, args.warmup)
            log(json.dumps(result_line(w2, ms2, dom2, args.steps, args.warmup, None, sp2)))
            del w2
            torch.cuda.empty_cache()


if __name__ == "__main__":
    main()

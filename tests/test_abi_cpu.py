"""The C ABI without a GPU: the library loads, exports every function the
header declares, reports block sizes, and rejects bad arguments synchronously
(these calls return before any HIP call is made)."""
import ctypes
import os
import re

import pytest

import gguf_dequant_gemv_amd as qg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemv.h")

# a fake, never-dereferenced device address (validation fails before any use)
FAKE = 0x7F0000000000


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(qg_[a-z_0-9]+)\s*\(", src)
    return sorted(set(names))


def test_header_lists_the_binding_exports():
    assert sorted(qg.EXPORTS) == declared_functions()


def test_library_exports_every_declared_symbol():
    L = qg.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_block_sizes():
    assert [qg.qg_block_values(t) for t in (2, 8, 12, 14)] == [32, 32, 256, 256]
    assert [qg.qg_block_bytes(t) for t in (2, 8, 12, 14)] == [18, 34, 144, 210]
    assert qg.qg_block_values(3) == 0 and qg.qg_block_bytes(99) == 0


def test_strerror():
    for c in (0, -1, -2, -3, -4, 7):
        assert isinstance(qg.strerror(c), str) and qg.strerror(c)


@pytest.mark.parametrize("args,code", [
    ((99, FAKE, FAKE, FAKE, 16, 64, 1), qg.QG_EINVAL),          # unknown type
    ((8, FAKE, FAKE, FAKE, 16, 48, 1), qg.QG_EINVAL),           # cols % 32
    ((12, FAKE, FAKE, FAKE, 16, 512 + 32, 1), qg.QG_EINVAL),    # cols % 256
    ((8, FAKE, FAKE, FAKE, 0, 64, 1), qg.QG_EINVAL),            # rows
    ((8, FAKE, FAKE, FAKE, 16, 64, 0), qg.QG_ELIMIT),           # ntok
    ((8, FAKE, FAKE, FAKE, 16, 64, 17), qg.QG_ELIMIT),
    ((8, None, FAKE, FAKE, 16, 64, 1), qg.QG_EINVAL),           # null W
    ((8, FAKE + 1, FAKE, FAKE, 16, 64, 1), qg.QG_EINVAL),       # W odd address
    ((8, FAKE, FAKE + 2, FAKE, 16, 64, 1), qg.QG_EINVAL),       # x misaligned
])
def test_gemv_rejects(args, code):
    assert qg.lib().qg_gemv(*args, None) == code


def test_dequant_rejects():
    L = qg.lib()
    assert L.qg_dequant(14, FAKE, FAKE, 4, 100, None) == qg.QG_EINVAL
    assert L.qg_dequant(2, None, FAKE, 4, 64, None) == qg.QG_EINVAL


def test_router_rejects():
    L = qg.lib()
    assert L.qg_router_topk(FAKE, 257, 8, 1, FAKE, FAKE, None) == qg.QG_ELIMIT
    assert L.qg_router_topk(FAKE, 128, 33, 1, FAKE, FAKE, None) == qg.QG_ELIMIT
    assert L.qg_router_topk(FAKE, 4, 5, 1, FAKE, FAKE, None) == qg.QG_ELIMIT
    assert L.qg_router_topk(FAKE, 128, 8, 17, FAKE, FAKE, None) == qg.QG_ELIMIT
    assert L.qg_router_topk(None, 128, 8, 1, FAKE, FAKE, None) == qg.QG_EINVAL


def test_mlp_rejects_and_sizes():
    L = qg.lib()
    assert qg.qg_mlp_workspace_size(8, 2560, 9728, 1) == 2 * 9728 * 4 + 9728 * 4   # gu, then act
    assert qg.qg_mlp_workspace_size(8, 64, 100, 3) % 256 == 0
    assert qg.qg_mlp_workspace_size(8, 2560, 9728, 0) == 0
    assert qg.qg_mlp_workspace_size(8, 0, 9728, 1) == 0
    ws = qg.qg_mlp_workspace_size(8, 64, 64, 1)
    assert L.qg_mlp(8, 0, FAKE, FAKE, FAKE, 64, 64, FAKE, FAKE, 1, FAKE, ws - 4, None) == qg.QG_EINVAL
    assert L.qg_mlp(8, 5, FAKE, FAKE, FAKE, 64, 64, FAKE, FAKE, 1, FAKE, ws, None) == qg.QG_EINVAL
    assert L.qg_mlp(8, 0, FAKE, FAKE, FAKE, 64, 48, FAKE, FAKE, 1, FAKE, ws, None) == qg.QG_EINVAL
    assert L.qg_mlp(8, 0, FAKE, FAKE, FAKE, 64, 64, FAKE, FAKE, 1, FAKE + 16, ws, None) == qg.QG_EINVAL


def _moe(**kw):
    d = dict(type=8, act=0, hidden=2048, ff=768, n_experts=128, gate_up=FAKE, gate_up_stride=5013504,
             down=FAKE + 3342336, down_stride=5013504, down_scale=None)
    d.update(kw)
    return qg.qg_moe(d["type"], d["act"], d["hidden"], d["ff"], d["n_experts"], d["gate_up"],
                     d["gate_up_stride"], d["down"], d["down_stride"], d["down_scale"])


def test_moe_rejects_and_sizes():
    L = qg.lib()
    m = _moe()
    ws = qg.qg_moe_workspace_size(m, 8, 1)
    assert ws >= 8 * 2 * 768 * 4 + 8 * 768 * 4 + 8 * 2048 * 4   # gu, act, down outputs
    assert ws % 256 == 0
    call = lambda mm, k=8, T=1, w=ws, st=FAKE: L.qg_moe_ffn(ctypes.byref(mm), FAKE, k, FAKE, FAKE, FAKE, T,
                                                           None, None, st, FAKE, w, None)
    assert call(_moe(n_experts=257)) == qg.QG_ELIMIT
    assert call(m, k=33) == qg.QG_ELIMIT
    assert call(m, T=17) == qg.QG_ELIMIT
    assert call(m, w=ws - 256) == qg.QG_EINVAL
    assert call(m, st=None) == qg.QG_EINVAL
    assert call(_moe(act=9)) == qg.QG_EINVAL
    assert call(_moe(ff=100)) == qg.QG_EINVAL                     # ff % 32
    assert call(_moe(gate_up_stride=1000)) == qg.QG_EINVAL        # stride shorter than a record
    assert L.qg_moe_ffn(None, FAKE, 8, FAKE, FAKE, FAKE, 1, None, None, FAKE, FAKE, ws, None) == qg.QG_EINVAL


def test_moe_noalloc_rejects():
    """The allocation-free variant refuses, before any HIP call, shapes whose
    workspace would not fit its static scratch, and the limits qg_moe_ffn
    refuses."""
    L = qg.lib()
    call = lambda mm, k=8, T=1: L.qg_moe_ffn_noalloc(ctypes.byref(mm), FAKE, k, FAKE, FAKE, FAKE, T, None, None,
                                                     FAKE, None)
    assert qg.qg_moe_workspace_size(_moe(), 8, 16) <= qg.QG_NOALLOC_SCRATCH_BYTES
    big = _moe(hidden=8192, ff=8192)
    assert qg.qg_moe_workspace_size(big, 8, 16) > qg.QG_NOALLOC_SCRATCH_BYTES
    assert call(big, T=16) == qg.QG_ELIMIT
    assert call(_moe(), T=17) == qg.QG_ELIMIT
    assert call(_moe(), k=33) == qg.QG_ELIMIT
    assert call(_moe(n_experts=257)) == qg.QG_ELIMIT
    assert L.qg_moe_ffn_noalloc(None, FAKE, 8, FAKE, FAKE, FAKE, 1, None, None, FAKE, None) == qg.QG_EINVAL


def test_f32_block_and_gemv_rejects():
    L = qg.lib()
    assert qg.qg_block_values(qg.QG_F32) == 1 and qg.qg_block_bytes(qg.QG_F32) == 4
    assert L.qg_gemv(0, FAKE, FAKE, FAKE, 128, 2048, 17, None) == qg.QG_ELIMIT
    assert L.qg_gemv(0, FAKE + 2, FAKE, FAKE, 128, 2048, 1, None) == qg.QG_EINVAL   # W not 4-byte aligned
    assert L.qg_gemv(0, FAKE, FAKE, FAKE, 0, 2048, 1, None) == qg.QG_EINVAL
    # f32 is a GEMV weight type only
    assert L.qg_dequant(0, FAKE, FAKE, 4, 64, None) == qg.QG_EINVAL
    assert L.qg_embed(0, FAKE, 4, 64, FAKE, 1, 1.0, FAKE, None) == qg.QG_EINVAL


def test_rmsnorm_post_ffn_rejects():
    L = qg.lib()
    assert L.qg_rmsnorm(FAKE, FAKE, FAKE, 0, 1, 1e-6, 1.0, None) == qg.QG_EINVAL
    assert L.qg_rmsnorm(FAKE, FAKE, FAKE, 64, 0, 1e-6, 1.0, None) == qg.QG_EINVAL
    assert L.qg_rmsnorm(FAKE, FAKE, FAKE, 64, 1, -1.0, 1.0, None) == qg.QG_EINVAL
    assert L.qg_rmsnorm(FAKE, FAKE, FAKE, 64, 1, float("nan"), 1.0, None) == qg.QG_EINVAL
    assert L.qg_rmsnorm(FAKE + 2, FAKE, FAKE, 64, 1, 1e-6, 1.0, None) == qg.QG_EINVAL
    P, f = ctypes.c_void_p, ctypes.c_float
    w3, y3, k3 = (P * 5)(*[FAKE] * 5), (P * 5)(*[FAKE + 4096] * 5), (f * 5)(*[1.0] * 5)
    multi = lambda n=64, T=1, eps=1e-6, m=3, w=w3, k=k3, y=y3, x=FAKE: L.qg_rmsnorm_multi(x, n, T, eps, m, w, k, y,
                                                                                         None)
    assert multi(m=0) == qg.QG_ELIMIT and multi(m=qg.QG_MAX_NORMS + 1) == qg.QG_ELIMIT
    assert multi(n=0) == qg.QG_EINVAL and multi(T=0) == qg.QG_EINVAL and multi(eps=-1.0) == qg.QG_EINVAL
    assert multi(x=FAKE + 2) == qg.QG_EINVAL
    assert multi(w=(P * 3)(FAKE, None, FAKE)) == qg.QG_EINVAL
    assert multi(y=(P * 3)(FAKE, FAKE + 2, FAKE)) == qg.QG_EINVAL
    assert L.qg_post_ffn(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 64, 1, 1e-6, None) == qg.QG_EINVAL
    assert L.qg_post_ffn(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1, 1e-6, None) == qg.QG_EINVAL


def test_embed_argmax_rejects_and_sizes():
    L = qg.lib()
    assert L.qg_embed(14, FAKE, 10, 300, FAKE, 1, 1.0, FAKE, None) == qg.QG_EINVAL    # cols % 256
    assert L.qg_embed(8, FAKE, 10, 64, FAKE, 0, 1.0, FAKE, None) == qg.QG_ELIMIT
    assert L.qg_embed(8, FAKE, 10, 64, None, 1, 1.0, FAKE, None) == qg.QG_EINVAL
    n = 151936
    ws = qg.qg_argmax_workspace_size(n, 2)
    assert ws % 256 == 0 and ws >= 2 * 2 * ((n + 2047) // 2048) * 4
    assert qg.qg_argmax_workspace_size(0, 1) == 0
    assert L.qg_argmax(FAKE, n, 2, 0.0, FAKE, FAKE, ws - 4, None) == qg.QG_EINVAL
    assert L.qg_argmax(FAKE, n, 2, -1.0, FAKE, FAKE, ws, None) == qg.QG_EINVAL
    assert L.qg_argmax(FAKE, n, 2, 0.0, FAKE, FAKE + 16, ws, None) == qg.QG_EINVAL
    assert L.qg_argmax(FAKE, 1 << 31, 1, 0.0, FAKE, FAKE, 1 << 20, None) == qg.QG_ELIMIT


def test_moe_shared_rejects_and_sizes():
    L = qg.lib()
    m = _moe(n_experts=256, ff=512, gate_up_stride=2 * 512 * 64 * 34, down_stride=2048 * 16 * 34)
    sh = qg.qg_shared_expert(8, 512, FAKE, FAKE, FAKE, FAKE)
    base = qg.qg_moe_workspace_size(m, 8, 1)
    ws = qg.qg_moe_shared_workspace_size(m, sh, 8, 1)
    assert ws == base + 2 * 512 * 4 + 512 * 4 + 2048 * 4 + 256   # gu, act, sh, gate logit after the routed part
    call = lambda s, w=ws, T=1: L.qg_moe_ffn_shared(ctypes.byref(m), ctypes.byref(s), FAKE, 8, FAKE, FAKE, FAKE, T,
                                                   None, None, FAKE, FAKE, w, None)
    assert call(sh, w=ws - 256) == qg.QG_EINVAL
    assert call(sh, T=17) == qg.QG_ELIMIT
    assert call(qg.qg_shared_expert(8, 100, FAKE, FAKE, FAKE, FAKE)) == qg.QG_EINVAL   # SF % 32
    assert call(qg.qg_shared_expert(0, 512, FAKE, FAKE, FAKE, FAKE)) == qg.QG_EINVAL   # f32 shared expert
    assert call(qg.qg_shared_expert(8, 512, FAKE, FAKE, FAKE, None)) == qg.QG_EINVAL   # no gate row
    assert L.qg_moe_ffn_shared(ctypes.byref(m), None, FAKE, 8, FAKE, FAKE, FAKE, 1, None, None, FAKE, FAKE, ws,
                               None) == qg.QG_EINVAL


def test_moe_dense_rejects_and_sizes():
    L = qg.lib()
    m = _moe(n_experts=256, ff=512, gate_up_stride=2 * 512 * 64 * 34, down_stride=2048 * 16 * 34)
    d = qg.qg_dense_mlp(8, 1536, FAKE, FAKE, FAKE)
    base = qg.qg_moe_workspace_size(m, 8, 1)
    ws = qg.qg_moe_dense_workspace_size(m, d, 8, 1)
    assert ws == base + qg.qg_mlp_workspace_size(8, 2048, 1536, 1)    # qg_mlp's layout after the routed part
    assert qg.qg_moe_dense_workspace_size(m, qg.qg_dense_mlp(8, 0, FAKE, FAKE, FAKE), 8, 1) == 0
    call = lambda dd, w=ws, T=1, xm=FAKE, ym=FAKE: L.qg_moe_ffn_dense(
        ctypes.byref(m), ctypes.byref(dd), FAKE, 8, FAKE, FAKE, FAKE, xm, ym, T, None, None, FAKE, FAKE, w, None)
    assert call(d, w=ws - 256) == qg.QG_EINVAL                                 # short workspace
    assert call(d, T=17) == qg.QG_ELIMIT
    assert call(qg.qg_dense_mlp(8, 100, FAKE, FAKE, FAKE)) == qg.QG_EINVAL     # FD % 32
    assert call(qg.qg_dense_mlp(8, 1536, FAKE, None, FAKE)) == qg.QG_EINVAL    # no up rows
    assert call(d, xm=None) == qg.QG_EINVAL
    assert call(d, ym=FAKE + 2) == qg.QG_EINVAL                                # misaligned output
    assert L.qg_moe_ffn_dense(ctypes.byref(m), None, FAKE, 8, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None, None, FAKE,
                              FAKE, ws, None) == qg.QG_EINVAL


def test_gemm_token_limits():
    L = qg.lib()
    assert L.qg_gemv(8, FAKE, FAKE, FAKE, 16, 64, 17, None) == qg.QG_ELIMIT
    assert L.qg_gemm(8, FAKE, FAKE, FAKE, 16, 64, qg.QG_MAX_PREFILL + 1, None, 0, None) == qg.QG_ELIMIT
    assert L.qg_gemm(8, FAKE, FAKE, FAKE, 16, 64, 0, None, 0, None) == qg.QG_ELIMIT
    assert L.qg_gemm(8, FAKE, FAKE, FAKE, 16, 48, 64, None, 0, None) == qg.QG_EINVAL     # cols % 32
    assert L.qg_gemm(0, FAKE + 2, FAKE, FAKE, 16, 64, 64, None, 0, None) == qg.QG_EINVAL  # f32 W misaligned
    gu_act = 256 * 2 * 9728 * 4 + 256 * 9728 * 4
    assert qg.qg_mlp_workspace_size(qg.QG_Q4_K, 2560, 9728, 256) == gu_act   # no split on the vector kernels
    assert qg.qg_mlp_workspace_size(8, 2560, 9728, 256) > gu_act             # the 20-tile down splits
    assert qg.qg_mlp_workspace_size(8, 2560, 9728, qg.QG_MAX_PREFILL + 1) == 0
    # 16 tokens: the down projection (80 tiles) splits into 7
    gu_act16 = 16 * 2 * 9728 * 4 + 16 * 9728 * 4
    assert qg.qg_mlp_workspace_size(8, 2560, 9728, 16) == gu_act16 + 7 * 16 * 2560 * 4


def test_rmsnorm_router_rejects():
    L = qg.lib()
    ok = (FAKE, 64, 1, 1e-6, FAKE, 1.0, FAKE, 8, FAKE, 0, None, None, None, None)
    def call(**kw):
        args = list(ok)
        names = ["x", "n", "ntok", "eps", "rw", "rk", "W", "rows", "logits", "nout", "w", "k", "y", "stream"]
        for key, v in kw.items():
            args[names.index(key)] = v
        return L.qg_rmsnorm_router(*args)
    assert call(ntok=17) == qg.QG_ELIMIT
    assert call(ntok=0) == qg.QG_ELIMIT
    assert call(nout=qg.QG_MAX_NORMS + 1) == qg.QG_ELIMIT
    assert call(n=0) == qg.QG_EINVAL
    assert call(rows=0) == qg.QG_EINVAL
    assert call(eps=-1.0) == qg.QG_EINVAL
    assert call(x=None) == qg.QG_EINVAL
    assert call(W=FAKE + 2) == qg.QG_EINVAL
    assert call(nout=1) == qg.QG_EINVAL          # nout outputs but no arrays


def test_argmax_embed_rejects():
    L = qg.lib()
    n = qg.qg_argmax_workspace_size(1000, 1)
    good = [FAKE, 1000, 1, 0.0, FAKE, FAKE, n, 8, FAKE, 1000, 64, 1.0, FAKE, None]
    def call(i, v):
        args = list(good)
        args[i] = v
        return L.qg_argmax_embed(*args)
    assert call(1, 0) == qg.QG_EINVAL             # n
    assert call(2, 0) == qg.QG_EINVAL             # ntok
    assert call(3, -1.0) == qg.QG_EINVAL          # softcap
    assert call(6, n - 4) == qg.QG_EINVAL         # short workspace
    assert call(5, FAKE + 16) == qg.QG_EINVAL     # misaligned workspace
    assert call(7, 99) == qg.QG_EINVAL            # block type
    assert call(10, 48) == qg.QG_EINVAL           # cols % 32
    assert call(8, None) == qg.QG_EINVAL          # W
    assert call(12, FAKE + 2) == qg.QG_EINVAL     # out misaligned


def test_gemm_split_workspace():
    """Prefill-size Q8_0 / Q4_0 launches need scratch: x split into three bf16
    parts (6 bytes per value of the padded chunk), plus whole [split][token][row]
    f32 partial sums when few row tiles make the launch split along the row.
    Small batches (4..16 tokens) on the MFMA kernel split long rows the same
    way when their tiles leave most CUs idle; one to three tokens and the
    vector kernels need none."""
    L = qg.lib()
    n = qg.qg_gemm_workspace_size(8, 2560, 9728, 64)
    xs = 64 * 9728 * 6
    assert n % 256 == 0 and n >= xs + 2 * 64 * 2560 * 4                     # the 20-tile down splits
    assert qg.qg_gemm_workspace_size(2, 2560, 9728, 64) == n                 # Q4_0: the same tiles
    wide = qg.qg_gemm_workspace_size(8, 65536, 9728, 64)                     # enough row tiles already
    assert xs <= wide < xs + 64 * 65536 * 4
    # 2560 rows are 80 tiles of 32: 304 blocks a row go out in 7 splits of 44
    assert qg.qg_gemm_workspace_size(8, 2560, 9728, 16) == 7 * 16 * 2560 * 4
    assert qg.qg_gemm_workspace_size(2, 2560, 9728, 4) == 7 * 4 * 2560 * 4
    assert qg.qg_gemm_workspace_size(8, 9728, 2560, 16) == 0                 # 304 tiles fill the CUs
    assert qg.qg_gemm_workspace_size(8, 2560, 9728, 3) == 0                  # the vector kernel
    assert qg.qg_gemm_workspace_size(qg.QG_Q4_K, 2560, 9728, 16) == 0
    assert qg.qg_gemm_workspace_size(8, 2560, 512, 16) == 0                  # 16 blocks: too short to split
    assert qg.qg_gemm_workspace_size(2, 2816, 2112, 16) == 0                 # 66 blocks: whole rows
    # under a quarter of the CUs' worth of tiles: rows of 64+ blocks split into 16+
    assert qg.qg_gemm_workspace_size(8, 33, 250 * 32, 16) == 16 * 16 * 33 * 4   # 2 tiles: 16 splits of 16
    assert qg.qg_gemm_workspace_size(8, 512, 2048, 16) == 4 * 16 * 512 * 4      # 16 tiles: 4 splits
    assert qg.qg_gemm_workspace_size(8, 512, 63 * 32, 16) == 0                  # 63 blocks: whole rows
    # the shared expert's 512 x 2048 gate and up (32 gated tiles) split 4 ways
    assert qg.qg_mlp_workspace_size(8, 2048, 512, 16) == 16 * 2 * 512 * 4 + 16 * 512 * 4 + 4 * 16 * 2 * 512 * 4
    assert qg.qg_gemm_workspace_size(qg.QG_Q6_K, 2560, 9728, 64) == 0
    assert 64 * 128 * 6 <= qg.qg_gemm_workspace_size(8, 2560, 128, 64) < 2560 * 64 * 4   # too short to split
    assert qg.qg_gemm_workspace_size(8, 2560, 9728, qg.QG_MAX_PREFILL + 1) == 0
    # a tensor past 2 GiB goes out in row launches; its short last launch
    # splits along the row where the full ones do not, and the size covers it
    chunk = (1 << 31) // (8192 // 32 * 34)
    full = qg.qg_gemm_workspace_size(8, chunk, 8192, 64)
    assert qg.qg_gemm_workspace_size(8, chunk + 100, 8192, 64) >= full + 2 * 64 * 100 * 4
    assert qg.qg_gemm_workspace_size(8, 2 * chunk, 8192, 64) == full
    assert L.qg_gemm(8, FAKE, FAKE, FAKE, 2560, 9728, 64, FAKE, n - 256, None) == qg.QG_EINVAL   # short
    assert L.qg_gemm(8, FAKE, FAKE, FAKE, 2560, 9728, 64, FAKE + 16, n, None) == qg.QG_EINVAL    # misaligned
    assert L.qg_gemm(8, FAKE, FAKE, FAKE, 2560, 9728, 64, None, n, None) == qg.QG_EINVAL         # null


def test_gemv_plan_kquant_one_token():
    """One token against K-quant rows takes the quarter-block kernel (kind 4):
    16 lanes a row for the Q4_K 17408 x 5120 shape (5 units each) in
    10-wave workgroups (436: at most 2 on a CU, 5 waves on its busiest SIMD,
    where 8-wave ones put 3 on some CUs), 32 for the Q6_K 5120 x 17408 one
    (8.5 units each) in 256 workgroups of 10 waves, one on every CU (64
    lanes would put two on every CU, each staging all 68 KiB of x; x past
    4096 values takes 8 or more waves a workgroup), and at any 2-byte phase
    of W; more tokens keep the block kernels."""
    p = qg.qg_gemv_plan(qg.QG_Q4_K, 17408, 5120, 1)
    assert (p["kind"], p["lanes_per_row"], p["row_tiles"], p["xchunk"]) == (4, 16, 436, 10)
    p = qg.qg_gemv_plan(qg.QG_Q6_K, 5120, 17408, 1)
    assert (p["kind"], p["lanes_per_row"], p["row_tiles"], p["xchunk"]) == (4, 32, 256, 10)
    # x padded by 4 floats per 64 values (+4), then one sum per 16 (Q6_K) / 32 (Q4_K) values
    assert p["lds_bytes"] == (17408 + 4 * 272 + 4 + 17408 // 16) * 4
    assert qg.qg_gemv_plan(qg.QG_Q4_K, 17408, 5120, 1)["lds_bytes"] == (5120 + 4 * 80 + 4 + 5120 // 32) * 4
    assert qg.qg_gemv_plan(qg.QG_Q4_K, 17408, 5120, 1, w_aligned16=False)["kind"] == 4
    assert qg.qg_gemv_plan(qg.QG_Q6_K, 262144, 2816, 1)["lanes_per_row"] == 16
    assert qg.qg_gemv_plan(qg.QG_Q4_K, 17408, 5120, 2)["kind"] != 4
    assert qg.qg_gemv_plan(qg.QG_Q8_0, 17408, 5120, 1)["kind"] != 4


def test_gemv_plan_multi_tile_shapes():
    """The shapes of the multi-tile parity cases take the per-lane kernel with
    more row tiles than workgroups can be resident at once (256 CUs, at most
    8 workgroups of 4 waves each), so some workgroup walks several tiles."""
    p = qg.qg_gemv_plan(qg.QG_Q8_0, 150001, 33 * 32, 1)
    assert p["kind"] == 0 and p["row_tiles"] > 256 * 8
    # an even block count takes the LDS-staged kernel instead
    assert qg.qg_gemv_plan(qg.QG_Q8_0, 151936, 2560, 1)["kind"] == 1
    assert qg.qg_gemv_plan(qg.QG_Q8_0, 151936, 2560, 1, w_aligned16=False)["kind"] == 2
    assert qg.qg_gemv_plan(qg.QG_Q8_0, 1024, 2048, 8)["kind"] == 3
    with pytest.raises(qg.QgError):
        qg.qg_gemv_plan(qg.QG_Q8_0, 1024, 2047, 1)


def test_q6k_planes_type_and_rejects():
    """The plane layout: block sizes as Q6_K; qg_prepare / qg_unprepare take
    Q6_K (and Q8_0) blocks, 16-byte-aligned planes and non-overlapping buffers; qg_gemv
    takes it at one token with W and x 16-byte aligned; the entry points
    that do not serve it reject it."""
    L, P = qg.lib(), qg.QG_Q6_K_PLANES
    assert (qg.qg_block_values(P), qg.qg_block_bytes(P)) == (256, 210)
    n = 4 * 210 * 2   # bytes of 4 rows x 512 values
    for f in (L.qg_prepare, L.qg_unprepare):
        assert f(qg.QG_Q4_K, FAKE, FAKE + 4096, 4, 512, None) == qg.QG_EINVAL       # type
        assert f(P, FAKE, FAKE + 4096, 4, 512, None) == qg.QG_EINVAL               # the layout is not an input type
        assert f(qg.QG_Q6_K, FAKE, FAKE + 4096, 4, 500, None) == qg.QG_EINVAL       # cols % 256
        assert f(qg.QG_Q6_K, FAKE, FAKE + 4096, 0, 512, None) == qg.QG_EINVAL       # rows
        assert f(qg.QG_Q6_K, None, FAKE + 4096, 4, 512, None) == qg.QG_EINVAL       # null
        assert f(qg.QG_Q6_K, FAKE, FAKE + n - 16, 4, 512, None) == qg.QG_EINVAL     # overlap
    assert L.qg_prepare(qg.QG_Q6_K, FAKE + 1, FAKE + 4096, 4, 512, None) == qg.QG_EINVAL   # blocks odd
    assert L.qg_prepare(qg.QG_Q6_K, FAKE + 2, FAKE + 4104, 4, 512, None) == qg.QG_EINVAL   # planes not 16-aligned
    assert L.qg_unprepare(qg.QG_Q6_K, FAKE + 8, FAKE + 4096, 4, 512, None) == qg.QG_EINVAL  # planes not 16-aligned
    assert L.qg_gemv(P, FAKE, FAKE, FAKE, 16, 512, 2, None) == qg.QG_EINVAL        # one token only
    assert L.qg_gemv(P, FAKE + 2, FAKE, FAKE, 16, 512, 1, None) == qg.QG_EINVAL    # W 16-aligned
    assert L.qg_gemv(P, FAKE, FAKE + 4, FAKE, 16, 512, 1, None) == qg.QG_EINVAL    # x 16-aligned
    assert L.qg_gemv(P, FAKE, FAKE, FAKE, 16, 500, 1, None) == qg.QG_EINVAL        # cols % 256
    assert L.qg_gemv(P, FAKE, FAKE, FAKE, 16, 512, 17, None) == qg.QG_ELIMIT
    assert L.qg_gemv(P, FAKE, FAKE, FAKE, 5 * 2 ** 20, 4096, 1, None) == qg.QG_ELIMIT   # over 2 GiB
    assert L.qg_dequant(P, FAKE + 2, FAKE, 4, 512, None) == qg.QG_EINVAL
    ws = L.qg_mlp_workspace_size(qg.QG_Q6_K, 512, 256, 1)
    assert L.qg_mlp(P, 0, FAKE, FAKE, FAKE, 512, 256, FAKE, FAKE, 1, FAKE, ws, None) == qg.QG_EINVAL
    # embedding rows from the planes: 16-byte aligned tables only
    assert L.qg_embed(P, FAKE + 2, 16, 512, FAKE, 1, ctypes.c_float(1.0), FAKE, None) == qg.QG_EINVAL
    assert L.qg_gemm(P, FAKE, FAKE, FAKE, 16, 512, 32, None, 0, None) == qg.QG_EINVAL


def test_gemv_plan_q6k_planes():
    """The plane layout takes the quarter-block kernel with the raw blocks'
    LDS layout of x; only at one token and from a 16-byte-aligned W."""
    p = qg.qg_gemv_plan(qg.QG_Q6_K_PLANES, 5120, 17408, 1)
    assert p["kind"] == 4 and p["lds_bytes"] == (17408 + 4 * 272 + 4 + 17408 // 16) * 4
    with pytest.raises(qg.QgError):
        qg.qg_gemv_plan(qg.QG_Q6_K_PLANES, 5120, 17408, 1, w_aligned16=False)
    with pytest.raises(qg.QgError):
        qg.qg_gemv_plan(qg.QG_Q6_K_PLANES, 5120, 17408, 2)


def test_q8_0_planes_type_and_rejects():
    """The Q8_0 plane layout: block sizes as Q8_0; qg_prepare takes Q8_0; the
    GEMV and the gated MLP take it at one token with W and x 16-byte aligned
    and up to 12288 values a row (plan kind 5); the entry points that do not
    serve it reject it."""
    L, P = qg.lib(), qg.QG_Q8_0_PLANES
    assert (qg.qg_block_values(P), qg.qg_block_bytes(P)) == (32, 34)
    assert L.qg_prepare(qg.QG_Q8_0, FAKE, FAKE + 4096, 4, 48, None) == qg.QG_EINVAL    # cols % 32
    assert L.qg_prepare(qg.QG_Q8_0, FAKE + 2, FAKE + 4104, 4, 64, None) == qg.QG_EINVAL   # planes not 16-aligned
    assert L.qg_prepare(qg.QG_Q8_0, FAKE, FAKE + 64, 4, 64, None) == qg.QG_EINVAL      # overlap (272 B)
    assert L.qg_unprepare(P, FAKE, FAKE + 4096, 4, 64, None) == qg.QG_EINVAL
    assert L.qg_gemv(P, FAKE, FAKE, FAKE, 16, 512, 2, None) == qg.QG_EINVAL        # one token only
    assert L.qg_gemv(P, FAKE + 2, FAKE, FAKE, 16, 512, 1, None) == qg.QG_EINVAL    # W 16-aligned
    assert L.qg_gemv(P, FAKE, FAKE + 4, FAKE, 16, 512, 1, None) == qg.QG_EINVAL    # x 16-aligned
    assert L.qg_gemv(P, FAKE, FAKE, FAKE, 16, 12288 + 32, 1, None) == qg.QG_EINVAL   # row too long
    assert L.qg_gemv(P, FAKE, FAKE, FAKE, 2 ** 20, 4096, 1, None) == qg.QG_ELIMIT    # 2^32 codes
    assert L.qg_dequant(P, FAKE + 2, FAKE, 4, 64, None) == qg.QG_EINVAL
    # qg_mlp takes the layout at one token, all of W, x 16-byte aligned
    ws = L.qg_mlp_workspace_size(P, 512, 256, 1)
    assert ws == L.qg_mlp_workspace_size(qg.QG_Q8_0, 512, 256, 1)
    assert L.qg_mlp(P, 0, FAKE, FAKE, FAKE, 512, 256, FAKE, FAKE, 2, FAKE, ws, None) == qg.QG_EINVAL
    assert L.qg_mlp(P, 0, FAKE, FAKE + 2, FAKE, 512, 256, FAKE, FAKE, 1, FAKE, ws, None) == qg.QG_EINVAL
    assert L.qg_mlp(P, 0, FAKE, FAKE, FAKE, 512, 256, FAKE + 4, FAKE, 1, FAKE, ws, None) == qg.QG_EINVAL
    assert L.qg_mlp(P, 0, FAKE, FAKE, FAKE, 512, 256, FAKE, FAKE, 1, FAKE, ws - 256, None) == qg.QG_EINVAL
    assert L.qg_mlp(P, 0, FAKE, FAKE, FAKE, 512, 12288 + 32, FAKE, FAKE, 1, FAKE, 1 << 30, None) == qg.QG_EINVAL
    # embedding rows from the planes: 16-byte aligned tables only
    assert L.qg_embed(P, FAKE + 2, 16, 512, FAKE, 1, ctypes.c_float(1.0), FAKE, None) == qg.QG_EINVAL
    p = qg.qg_gemv_plan(P, 151936, 2560, 1)
    assert p["kind"] == 5 and p["lds_bytes"] == (2560 + 2560 // 8) * 4


def test_gemv_plan_q8_0_planes_constants():
    """The plan reports the plane GEMV's own geometry: 2 pieces in flight
    per lane; up to 4096 rows the fewest waves a workgroup (4, 8, 10, 12,
    14, 16) that give every row its own wave within 256 workgroups, beyond
    that 8-wave workgroups walking several rows each."""
    p = qg.qg_gemv_plan(qg.QG_Q8_0_PLANES, 1000, 2048, 1)
    assert (p["kind"], p["lanes_per_row"], p["row_tiles"], p["depth"], p["xchunk"]) == (5, 64, 250, 2, 4)
    for rows, nw in ((1, 4), (1024, 4), (1025, 8), (2048, 8), (2049, 10), (2560, 10), (2816, 12), (3500, 14),
                     (4096, 16), (4097, 8), (151936, 8)):
        p = qg.qg_gemv_plan(qg.QG_Q8_0_PLANES, rows, 256, 1)
        assert p["xchunk"] == nw and p["row_tiles"] == (rows + nw - 1) // nw, (rows, p)

"""Python binding of libqgemv (include/qgemv.h): argument marshalling only.

Every function has the C entry point's name and argument order.  Device
buffers are torch tensors on the GPU (or raw integer device addresses);
`stream` defaults to torch's current stream.  Every step of the path runs in
the HIP library; this module never computes anything itself and raises if the
library is missing or a call fails.
"""
import ctypes
import os

QG_F32, QG_Q4_0, QG_Q8_0, QG_Q4_K, QG_Q6_K = 0, 2, 8, 12, 14
QG_Q6_K_PLANES = 270   # Q6_K in the plane layout qg_prepare writes
QG_Q8_0_PLANES = 264   # Q8_0 as a code plane and a scale plane (qg_prepare)
QG_ACT_SILU, QG_ACT_GELU_TANH = 0, 1
QG_OK, QG_EINVAL, QG_EABSENT, QG_EHIP, QG_ELIMIT = 0, -1, -2, -3, -4
QG_MAX_TOKENS, QG_MAX_EXPERTS, QG_MAX_TOPK, QG_MAX_PREFILL, QG_MAX_NORMS = 16, 256, 32, 4096, 4
QG_NOALLOC_SCRATCH_BYTES = 8 << 20

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqgemv.so")

# Every symbol include/qgemv.h declares.
EXPORTS = ("qg_block_values", "qg_block_bytes", "qg_strerror", "qg_gemv", "qg_gemm_workspace_size", "qg_gemm",
           "qg_dequant", "qg_prepare", "qg_unprepare", "qg_gemv_plan",
           "qg_router_topk", "qg_mlp_workspace_size", "qg_mlp", "qg_moe_workspace_size",
           "qg_moe_ffn", "qg_moe_ffn_noalloc", "qg_rmsnorm", "qg_rmsnorm_multi", "qg_rmsnorm_router", "qg_moe_shared_workspace_size", "qg_moe_ffn_shared",
           "qg_moe_dense_workspace_size", "qg_moe_ffn_dense",
           "qg_post_ffn", "qg_embed", "qg_argmax_workspace_size", "qg_argmax", "qg_argmax_embed")

_lib = None


class QgError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__("%s failed: %d (%s)" % (fn, code, strerror(code)))
        self.code = code


class qg_moe(ctypes.Structure):
    _fields_ = [("type", ctypes.c_int), ("act", ctypes.c_int),
                ("hidden", ctypes.c_int64), ("ff", ctypes.c_int64), ("n_experts", ctypes.c_int),
                ("gate_up", ctypes.c_void_p), ("gate_up_stride", ctypes.c_int64),
                ("down", ctypes.c_void_p), ("down_stride", ctypes.c_int64),
                ("down_scale", ctypes.c_void_p), ("n_slots", ctypes.c_int)]


class qg_shared_expert(ctypes.Structure):
    _fields_ = [("type", ctypes.c_int), ("ff", ctypes.c_int64), ("gate", ctypes.c_void_p),
                ("up", ctypes.c_void_p), ("down", ctypes.c_void_p), ("gate_inp", ctypes.c_void_p)]


class qg_dense_mlp(ctypes.Structure):
    _fields_ = [("type", ctypes.c_int), ("ff", ctypes.c_int64), ("gate", ctypes.c_void_p),
                ("up", ctypes.c_void_p), ("down", ctypes.c_void_p)]


def lib():
    """The loaded libqgemv.so; raises FileNotFoundError if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError("libqgemv.so is not built: run python -m gguf_dequant_gemv_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        L.qg_block_values.argtypes = [i32]
        L.qg_block_bytes.argtypes = [i32]
        L.qg_strerror.argtypes = [i32]
        L.qg_strerror.restype = ctypes.c_char_p
        L.qg_gemv.argtypes = [i32, P, P, P, i64, i64, i32, P]
        L.qg_gemm_workspace_size.argtypes = [i32, i64, i64, i32]
        L.qg_gemm_workspace_size.restype = sz
        L.qg_gemm.argtypes = [i32, P, P, P, i64, i64, i32, P, sz, P]
        L.qg_dequant.argtypes = [i32, P, P, i64, i64, P]
        L.qg_prepare.argtypes = [i32, P, P, i64, i64, P]
        L.qg_unprepare.argtypes = [i32, P, P, i64, i64, P]
        L.qg_gemv_plan.argtypes = [i32, i64, i64, i32, i32, i32, P]
        L.qg_router_topk.argtypes = [P, i32, i32, i32, P, P, P]
        L.qg_mlp_workspace_size.argtypes = [i32, i64, i64, i32]
        L.qg_mlp_workspace_size.restype = sz
        L.qg_mlp.argtypes = [i32, i32, P, P, P, i64, i64, P, P, i32, P, sz, P]
        L.qg_moe_workspace_size.argtypes = [ctypes.POINTER(qg_moe), i32, i32]
        L.qg_moe_workspace_size.restype = sz
        L.qg_moe_ffn.argtypes = [ctypes.POINTER(qg_moe), P, i32, P, P, P, i32, P, P, P, P, sz, P]
        L.qg_moe_ffn_noalloc.argtypes = [ctypes.POINTER(qg_moe), P, i32, P, P, P, i32, P, P, P, P]
        f = ctypes.c_float
        L.qg_rmsnorm.argtypes = [P, P, P, i64, i32, f, f, P]
        L.qg_rmsnorm_multi.argtypes = [P, i64, i32, f, i32, ctypes.POINTER(P), ctypes.POINTER(f),
                                       ctypes.POINTER(P), P]
        L.qg_rmsnorm_router.argtypes = [P, i64, i32, f, P, f, P, i64, P, i32, ctypes.POINTER(P),
                                        ctypes.POINTER(f), ctypes.POINTER(P), P]
        L.qg_moe_shared_workspace_size.argtypes = [ctypes.POINTER(qg_moe), ctypes.POINTER(qg_shared_expert), i32,
                                                   i32]
        L.qg_moe_shared_workspace_size.restype = sz
        L.qg_moe_ffn_shared.argtypes = [ctypes.POINTER(qg_moe), ctypes.POINTER(qg_shared_expert), P, i32, P, P,
                                        P, i32, P, P, P, P, sz, P]
        L.qg_moe_dense_workspace_size.argtypes = [ctypes.POINTER(qg_moe), ctypes.POINTER(qg_dense_mlp), i32, i32]
        L.qg_moe_dense_workspace_size.restype = sz
        L.qg_moe_ffn_dense.argtypes = [ctypes.POINTER(qg_moe), ctypes.POINTER(qg_dense_mlp), P, i32, P, P, P, P, P,
                                       i32, P, P, P, P, sz, P]
        L.qg_post_ffn.argtypes = [P, P, P, P, P, P, P, i64, i32, f, P]
        L.qg_embed.argtypes = [i32, P, i64, i64, P, i32, f, P, P]
        L.qg_argmax_workspace_size.argtypes = [i64, i32]
        L.qg_argmax_workspace_size.restype = sz
        L.qg_argmax.argtypes = [P, i64, i32, f, P, P, sz, P]
        L.qg_argmax_embed.argtypes = [P, i64, i32, f, P, P, sz, i32, P, i64, i64, f, P, P]
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, rc):
    if rc != QG_OK:
        raise QgError(fn, rc)


def strerror(code):
    return lib().qg_strerror(code).decode()


def qg_block_values(t):
    return lib().qg_block_values(t)


def qg_block_bytes(t):
    return lib().qg_block_bytes(t)


def qg_gemv(type, W, x, y, rows, cols, ntok=1, stream=None):
    _check("qg_gemv", lib().qg_gemv(type, _ptr(W), _ptr(x), _ptr(y), rows, cols, ntok, _stream(stream)))


def qg_gemm_workspace_size(type, rows, cols, ntok):
    return lib().qg_gemm_workspace_size(type, rows, cols, ntok)


def qg_gemm(type, W, x, y, rows, cols, ntok, workspace=None, workspace_bytes=None, stream=None):
    nbytes = 0 if workspace is None else _nbytes(workspace, workspace_bytes)
    _check("qg_gemm", lib().qg_gemm(type, _ptr(W), _ptr(x), _ptr(y), rows, cols, ntok, _ptr(workspace), nbytes,
                                    _stream(stream)))


def qg_gemv_plan(type, rows, cols, ntok=1, w_aligned16=True, query_device=False):
    """The plan qg_gemv takes for a shape, as a dict (see include/qgemv.h)."""
    out = (ctypes.c_int32 * 8)()
    _check("qg_gemv_plan", lib().qg_gemv_plan(type, rows, cols, ntok, int(bool(w_aligned16)),
                                              int(bool(query_device)), ctypes.addressof(out)))
    keys = ("kind", "lanes_per_row", "tokens_per_wg", "row_tiles", "workgroups", "lds_bytes", "depth", "xchunk")
    return dict(zip(keys, list(out)))


def qg_dequant(type, W, out, rows, cols, stream=None):
    _check("qg_dequant", lib().qg_dequant(type, _ptr(W), _ptr(out), rows, cols, _stream(stream)))


def qg_prepare(type, src, dst, rows, cols, stream=None):
    """GGUF Q6_K / Q8_0 blocks -> their plane layout (QG_Q6_K_PLANES / QG_Q8_0_PLANES)."""
    _check("qg_prepare", lib().qg_prepare(type, _ptr(src), _ptr(dst), rows, cols, _stream(stream)))


def qg_unprepare(type, src, dst, rows, cols, stream=None):
    """A plane layout -> GGUF blocks (the inverse of qg_prepare)."""
    _check("qg_unprepare", lib().qg_unprepare(type, _ptr(src), _ptr(dst), rows, cols, _stream(stream)))


def qg_router_topk(logits, n_experts, k, ntok, ids, weights, stream=None):
    _check("qg_router_topk", lib().qg_router_topk(_ptr(logits), n_experts, k, ntok, _ptr(ids),
                                                  _ptr(weights), _stream(stream)))


def qg_mlp_workspace_size(type, hidden, ff, ntok):
    return lib().qg_mlp_workspace_size(type, hidden, ff, ntok)


def qg_mlp(type, act, W_gate, W_up, W_down, hidden, ff, x, y, ntok, workspace, workspace_bytes=None,
           stream=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check("qg_mlp", lib().qg_mlp(type, act, _ptr(W_gate), _ptr(W_up), _ptr(W_down), hidden, ff, _ptr(x),
                                  _ptr(y), ntok, _ptr(workspace), workspace_bytes, _stream(stream)))


def make_moe(type, act, hidden, ff, n_experts, gate_up, gate_up_stride, down, down_stride,
             down_scale=None, n_slots=0):
    return qg_moe(type, act, hidden, ff, n_experts, _ptr(gate_up), gate_up_stride, _ptr(down),
                  down_stride, _ptr(down_scale), n_slots)


def qg_moe_workspace_size(m, topk, ntok):
    return lib().qg_moe_workspace_size(ctypes.byref(m), topk, ntok)


def qg_moe_ffn(m, router_logits, topk, expert_slots, x, y, ntok, ids_out, w_out, status, workspace,
               workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check("qg_moe_ffn", lib().qg_moe_ffn(ctypes.byref(m), _ptr(router_logits), topk, _ptr(expert_slots),
                                          _ptr(x), _ptr(y), ntok, _ptr(ids_out), _ptr(w_out), _ptr(status),
                                          _ptr(workspace), workspace_bytes, _stream(stream)))


def qg_moe_ffn_noalloc(m, router_logits, topk, expert_slots, x, y, ntok, ids_out, w_out, status, stream=None):
    _check("qg_moe_ffn_noalloc",
           lib().qg_moe_ffn_noalloc(ctypes.byref(m), _ptr(router_logits), topk, _ptr(expert_slots), _ptr(x), _ptr(y),
                                    ntok, _ptr(ids_out), _ptr(w_out), _ptr(status), _stream(stream)))


def _nbytes(t, given):
    return given if given is not None else t.numel() * t.element_size()


def qg_rmsnorm(x, w, y, n, ntok, eps, k=1.0, stream=None):
    _check("qg_rmsnorm", lib().qg_rmsnorm(_ptr(x), _ptr(w), _ptr(y), n, ntok, eps, k, _stream(stream)))


def qg_rmsnorm_multi(x, n, ntok, eps, ws, ks, ys, stream=None):
    """ws, ys: sequences of device buffers; ks: sequence of floats (host)."""
    m = len(ws)
    if len(ks) != m or len(ys) != m:
        raise ValueError("qg_rmsnorm_multi: ws, ks and ys differ in length")
    P, f = ctypes.c_void_p, ctypes.c_float
    wa = (P * max(m, 1))(*[_ptr(t) for t in ws])
    ya = (P * max(m, 1))(*[_ptr(t) for t in ys])
    ka = (f * max(m, 1))(*ks)
    _check("qg_rmsnorm_multi", lib().qg_rmsnorm_multi(_ptr(x), n, ntok, eps, m, wa, ka, ya, _stream(stream)))


def qg_rmsnorm_router(x, n, ntok, eps, rw, rk, W, rows, logits, ws=(), ks=(), ys=(), stream=None):
    """The router's logits of x's norm (rw, rk) and further norms (ws, ks, ys:
    sequences of device buffers / host floats), one launch."""
    m = len(ws)
    if len(ks) != m or len(ys) != m:
        raise ValueError("qg_rmsnorm_router: ws, ks and ys differ in length")
    P, f = ctypes.c_void_p, ctypes.c_float
    wa = (P * max(m, 1))(*[_ptr(t) for t in ws])
    ya = (P * max(m, 1))(*[_ptr(t) for t in ys])
    ka = (f * max(m, 1))(*ks)
    _check("qg_rmsnorm_router", lib().qg_rmsnorm_router(_ptr(x), n, ntok, eps, _ptr(rw), rk, _ptr(W), rows,
                                                        _ptr(logits), m, wa, ka, ya, _stream(stream)))


def make_shared_expert(type, ff, gate, up, down, gate_inp):
    return qg_shared_expert(type, ff, _ptr(gate), _ptr(up), _ptr(down), _ptr(gate_inp))


def qg_moe_shared_workspace_size(m, sh, topk, ntok):
    return lib().qg_moe_shared_workspace_size(ctypes.byref(m), ctypes.byref(sh), topk, ntok)


def qg_moe_ffn_shared(m, sh, router_logits, topk, expert_slots, x, resid, ntok, ids_out, w_out, status,
                      workspace, workspace_bytes=None, stream=None):
    _check("qg_moe_ffn_shared",
           lib().qg_moe_ffn_shared(ctypes.byref(m), ctypes.byref(sh), _ptr(router_logits), topk, _ptr(expert_slots),
                                   _ptr(x), _ptr(resid), ntok, _ptr(ids_out), _ptr(w_out), _ptr(status),
                                   _ptr(workspace), _nbytes(workspace, workspace_bytes), _stream(stream)))


def make_dense_mlp(type, ff, gate, up, down):
    return qg_dense_mlp(type, ff, _ptr(gate), _ptr(up), _ptr(down))


def qg_moe_dense_workspace_size(m, d, topk, ntok):
    return lib().qg_moe_dense_workspace_size(ctypes.byref(m), ctypes.byref(d), topk, ntok)


def qg_moe_ffn_dense(m, d, router_logits, topk, expert_slots, x, y, x_mlp, y_mlp, ntok, ids_out, w_out, status,
                     workspace, workspace_bytes=None, stream=None):
    _check("qg_moe_ffn_dense",
           lib().qg_moe_ffn_dense(ctypes.byref(m), ctypes.byref(d), _ptr(router_logits), topk, _ptr(expert_slots),
                                  _ptr(x), _ptr(y), _ptr(x_mlp), _ptr(y_mlp), ntok, _ptr(ids_out), _ptr(w_out),
                                  _ptr(status), _ptr(workspace), _nbytes(workspace, workspace_bytes),
                                  _stream(stream)))


def qg_post_ffn(mlp, moe, w1, w2, w, out_scale, x, n, ntok, eps, stream=None):
    _check("qg_post_ffn", lib().qg_post_ffn(_ptr(mlp), _ptr(moe), _ptr(w1), _ptr(w2), _ptr(w), _ptr(out_scale),
                                            _ptr(x), n, ntok, eps, _stream(stream)))


def qg_embed(type, W, rows, cols, tokens, ntok, scale, out, stream=None):
    _check("qg_embed", lib().qg_embed(type, _ptr(W), rows, cols, _ptr(tokens), ntok, scale, _ptr(out),
                                      _stream(stream)))


def qg_argmax_workspace_size(n, ntok):
    return lib().qg_argmax_workspace_size(n, ntok)


def qg_argmax(logits, n, ntok, softcap, idx, workspace, workspace_bytes=None, stream=None):
    _check("qg_argmax", lib().qg_argmax(_ptr(logits), n, ntok, softcap, _ptr(idx), _ptr(workspace),
                                        _nbytes(workspace, workspace_bytes), _stream(stream)))


def qg_argmax_embed(logits, n, ntok, softcap, idx, workspace, type, W, rows, cols, scale, out,
                    workspace_bytes=None, stream=None):
    _check("qg_argmax_embed", lib().qg_argmax_embed(_ptr(logits), n, ntok, softcap, _ptr(idx), _ptr(workspace),
                                                    _nbytes(workspace, workspace_bytes), type, _ptr(W), rows, cols,
                                                    scale, _ptr(out), _stream(stream)))

"""The oracle: TEST INFRASTRUCTURE ONLY.

A plain CPU implementation in f64 of the quantized GEMV / MoE path (see
oracle.c).  Only the tests, the smoke check and the bench's CPU-baseline leg
import it; the product library never does, and it shares no code with the
product library.  This module is ctypes marshalling around liboracle.so.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, Q4_0, Q8_0, Q4_K, Q6_K = 0, 2, 8, 12, 14
ACT_SILU, ACT_GELU_TANH = 0, 1

_lib = None


def lib():
    """Load liboracle.so, building it first if it is missing or stale."""
    global _lib
    if _lib is None:
        so = _build.LIB
        if (not os.path.exists(so)) or os.path.getmtime(so) < os.path.getmtime(_build.SRC):
            _build.build()
        L = ctypes.CDLL(so)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int
        L.or_f16.restype = ctypes.c_double
        L.or_f16.argtypes = [ctypes.c_uint16]
        L.or_block_values.argtypes = [i32]
        L.or_block_bytes.argtypes = [i32]
        L.or_dequant.argtypes = [i32, P, i64, P]
        L.or_gemv.argtypes = [i32, P, P, i64, i64, i32, P, P]
        L.or_gemv_rows.argtypes = [i32, P, P, i64, i64, i32, P, i64, P, P]
        L.or_gemv_f64.argtypes = [i32, P, P, i64, i64, P, P]
        L.or_silu.restype = ctypes.c_double
        L.or_silu.argtypes = [ctypes.c_double]
        L.or_gelu_tanh.restype = ctypes.c_double
        L.or_gelu_tanh.argtypes = [ctypes.c_double]
        L.or_glu.argtypes = [i32, P, i64, P]
        L.or_glu.restype = None
        L.or_glu_f32.argtypes = [i32, P, i64, P]
        L.or_glu_f32.restype = None
        L.or_router_topk.argtypes = [P, i32, i32, i32, P, P]
        L.or_moe_ffn.argtypes = [i32, i32, i64, i64, i32, P, i64, P, i64, P, P, i32, P, P, i32,
                                 P, P, P, P, P]
        L.or_moe_down.argtypes = [i32, i32, i64, i64, P, i64, P, P, P, P, i32, P, i32, P, P, P]
        d = ctypes.c_double
        L.or_rmsnorm.argtypes = [P, P, i64, i32, d, d, P]
        L.or_sigmoid.restype = d
        L.or_sigmoid.argtypes = [d]
        L.or_moe_shared_combine.argtypes = [P, i32, P, P, P, P, i64, i32, P, P, P]
        L.or_post_ffn.argtypes = [P, P, P, P, P, d, P, i64, i32, d, P, P]
        L.or_embed.argtypes = [i32, P, i64, i64, P, i32, ctypes.c_float, P]
        L.or_softcap.argtypes = [P, i64, ctypes.c_float, P]
        L.or_argmax.argtypes = [P, i64, i32, P]
        L.or_set_threads.argtypes = [i32]
        L.or_q6k_planes.argtypes = [P, i64, P]
        L.or_q8_0_planes.argtypes = [P, i64, P]
        L.or_q8_0_unplanes.argtypes = [P, i64, P]
        L.or_q6k_unplanes.argtypes = [P, i64, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def block_values(t):
    return lib().or_block_values(t)


def block_bytes(t):
    return lib().or_block_bytes(t)


def f16(bits):
    """binary16 bit pattern -> float (f64), exact."""
    return lib().or_f16(int(bits) & 0xFFFF)


def dequant(t, blocks, n):
    """First n values of a block stream, exact in f64."""
    b = _c(blocks, np.uint8)
    out = np.empty(n, np.float64)
    if lib().or_dequant(t, _p(b), n, _p(out)):
        raise ValueError("or_dequant: bad type or size")
    return out


def gemv(t, W, x, rows, cols, ntok=1, row_idx=None):
    """(y, A): y[t][r] = sum_c W[r][c] x[t][c], A = sum |W x|, both f64 [ntok][n]."""
    Wb = _c(W, np.uint8)
    xf = _c(x, np.float32)
    assert xf.size == ntok * cols
    if row_idx is None:
        y = np.empty((ntok, rows), np.float64)
        A = np.empty((ntok, rows), np.float64)
        rc = lib().or_gemv(t, _p(Wb), _p(xf), rows, cols, ntok, _p(y), _p(A))
    else:
        ri = _c(row_idx, np.int64)
        y = np.empty((ntok, ri.size), np.float64)
        A = np.empty((ntok, ri.size), np.float64)
        rc = lib().or_gemv_rows(t, _p(Wb), _p(xf), rows, cols, ntok, _p(ri), ri.size, _p(y), _p(A))
    if rc:
        raise ValueError("or_gemv: bad arguments")
    return y, A


def gemv_f64(t, W, x, rows, cols):
    Wb = _c(W, np.uint8)
    xd = _c(x, np.float64)
    y = np.empty(rows, np.float64)
    A = np.empty(rows, np.float64)
    if lib().or_gemv_f64(t, _p(Wb), _p(xd), rows, cols, _p(y), _p(A)):
        raise ValueError("or_gemv_f64: bad arguments")
    return y, A


def silu(g):
    return lib().or_silu(float(g))


def gelu_tanh(g):
    return lib().or_gelu_tanh(float(g))


def glu(act, gu, F):
    """act(gu[:F]) * gu[F:2F] in f64; gu f64 (exact inputs) or f32 (stage input)."""
    out = np.empty(F, np.float64)
    if gu.dtype == np.float32:
        g = _c(gu, np.float32)
        lib().or_glu_f32(act, _p(g), F, _p(out))
    else:
        g = _c(gu, np.float64)
        lib().or_glu(act, _p(g), F, _p(out))
    return out


def router_topk(logits, E, k, ntok):
    lg = _c(logits, np.float32)
    ids = np.empty((ntok, k), np.int32)
    w = np.empty((ntok, k), np.float64)
    if lib().or_router_topk(_p(lg), E, k, ntok, _p(ids), _p(w)):
        raise ValueError("or_router_topk: bad arguments")
    return ids, w


def moe_ffn(t, act, H, F, E, gate_up, gu_stride, down, d_stride, down_scale, logits, k, slots,
            x, ntok, want_gu=False):
    """Returns dict(y, A, ids, c, gu, skipped); gate_up/down are byte arrays indexed by slot."""
    gub = _c(gate_up, np.uint8)
    db = _c(down, np.uint8)
    ds = None if down_scale is None else _c(down_scale, np.float32)
    lg = _c(logits, np.float32)
    sl = _c(slots, np.int32)
    xf = _c(x, np.float32)
    y = np.full((ntok, H), np.nan, np.float64)
    A = np.full((ntok, H), np.nan, np.float64)
    gu = np.empty((ntok, k, 2 * F), np.float64) if want_gu else None
    ids = np.empty((ntok, k), np.int32)
    c = np.empty((ntok, k), np.float64)
    rc = lib().or_moe_ffn(t, act, H, F, E, _p(gub), gu_stride, _p(db), d_stride, _p(ds), _p(lg),
                          k, _p(sl), _p(xf), ntok, _p(y), _p(A), _p(gu), _p(ids), _p(c))
    if rc < 0:
        raise ValueError("or_moe_ffn: bad arguments")
    return dict(y=y, A=A, ids=ids, c=c, gu=gu, skipped=rc)


def moe_down(t, act, H, F, down, d_stride, down_scale, slots, ids, c, gu_f32, ntok):
    """Down half fed with an f32 gate||up stage: returns (y, A, R), each [ntok][H]."""
    db = _c(down, np.uint8)
    ds = None if down_scale is None else _c(down_scale, np.float32)
    sl = _c(slots, np.int32)
    idc = _c(ids, np.int32)
    cc = _c(c, np.float64)
    k = idc.shape[-1]
    g = _c(gu_f32, np.float32)
    assert g.size == ntok * k * 2 * F
    y = np.empty((ntok, H), np.float64)
    A = np.empty((ntok, H), np.float64)
    R = np.empty((ntok, H), np.float64)
    rc = lib().or_moe_down(t, act, H, F, _p(db), d_stride, _p(ds), _p(sl), _p(idc), _p(cc), k,
                           _p(g), ntok, _p(y), _p(A), _p(R))
    if rc:
        raise ValueError("or_moe_down: bad arguments")
    return y, A, R


# ------------------------------------------------------ around the MoE step


def rmsnorm(x, w, n, ntok, eps, k=1.0):
    """((x * r) * k) * w per token, r = 1/sqrt(mean x^2 + eps); f64 [ntok][n]."""
    xf = _c(x, np.float32)
    wf = _c(w, np.float32)
    assert xf.size == n * ntok and wf.size == n
    y = np.empty((ntok, n), np.float64)
    if lib().or_rmsnorm(_p(xf), _p(wf), n, ntok, float(eps), float(k), _p(y)):
        raise ValueError("or_rmsnorm: bad arguments")
    return y


def sigmoid(g):
    return lib().or_sigmoid(float(g))


def moe_shared_combine(terms, sh, gate_inp, x, resid, H, ntok):
    """(y, A, sg): y = (sum_j terms_j + sh * sigmoid(gate_inp . x)) + resid, f64 [ntok][H]."""
    tf = _c(terms, np.float32)
    k = tf.size // (ntok * H)
    assert tf.size == ntok * k * H
    shf = _c(sh, np.float32)
    gf = _c(gate_inp, np.float32)
    xf = _c(x, np.float32)
    rf = _c(resid, np.float32)
    y = np.empty((ntok, H), np.float64)
    A = np.empty((ntok, H), np.float64)
    sg = np.empty(ntok, np.float64)
    if lib().or_moe_shared_combine(_p(tf), k, _p(shf), _p(gf), _p(xf), _p(rf), H, ntok, _p(y), _p(A), _p(sg)):
        raise ValueError("or_moe_shared_combine: bad arguments")
    return y, A, sg


def post_ffn(mlp, moe, w1, w2, w, os_, x, n, ntok, eps):
    """Gemma's FFN tail: (y, A), f64 [ntok][n]."""
    a = [_c(v, np.float32) for v in (mlp, moe, w1, w2, w, x)]
    y = np.empty((ntok, n), np.float64)
    A = np.empty((ntok, n), np.float64)
    if lib().or_post_ffn(_p(a[0]), _p(a[1]), _p(a[2]), _p(a[3]), _p(a[4]), float(os_), _p(a[5]), n, ntok,
                         float(eps), _p(y), _p(A)):
        raise ValueError("or_post_ffn: bad arguments")
    return y, A


# ---------------------------------------------------- embedding and head


def embed(t, W, rows, cols, tokens, scale=1.0):
    """f32 [ntok][cols]: each row's values rounded to f32, times scale in f32."""
    Wb = _c(W, np.uint8)
    tk = _c(tokens, np.int32).ravel()
    out = np.empty((tk.size, cols), np.float32)
    if lib().or_embed(t, _p(Wb), rows, cols, _p(tk), tk.size, float(scale), _p(out)):
        raise ValueError("or_embed: bad arguments")
    return out


def softcap(l, cap):
    lf = _c(l, np.float32)
    out = np.empty(lf.shape, np.float64)
    if lib().or_softcap(_p(lf), lf.size, float(cap), _p(out)):
        raise ValueError("or_softcap: bad arguments")
    return out


def argmax(l, n, ntok):
    lf = _c(l, np.float32)
    assert lf.size == n * ntok
    idx = np.empty(ntok, np.int32)
    if lib().or_argmax(_p(lf), n, ntok, _p(idx)):
        raise ValueError("or_argmax: bad arguments")
    return idx


def q6k_planes(blocks, n):
    """The Q6_K plane layout of n blocks (uint8 [210 n]): ql, qh, scales, d."""
    b = _c(blocks, np.uint8).ravel()
    assert b.size >= 210 * n
    out = np.empty(210 * n, np.uint8)
    if lib().or_q6k_planes(_p(b), n, _p(out)):
        raise ValueError("or_q6k_planes: bad size")
    return out


def q6k_unplanes(planes, n):
    """Blocks back from the plane layout (the inverse of q6k_planes)."""
    p = _c(planes, np.uint8).ravel()
    assert p.size >= 210 * n
    out = np.empty(210 * n, np.uint8)
    if lib().or_q6k_unplanes(_p(p), n, _p(out)):
        raise ValueError("or_q6k_unplanes: bad size")
    return out


def q8_0_planes(blocks, n):
    """The Q8_0 plane layout of n blocks (uint8 [34 n]): codes, then scales."""
    b = _c(blocks, np.uint8).ravel()
    assert b.size >= 34 * n
    out = np.empty(34 * n, np.uint8)
    if lib().or_q8_0_planes(_p(b), n, _p(out)):
        raise ValueError("or_q8_0_planes: bad size")
    return out


def q8_0_unplanes(planes, n):
    """Blocks back from the Q8_0 plane layout."""
    p = _c(planes, np.uint8).ravel()
    assert p.size >= 34 * n
    out = np.empty(34 * n, np.uint8)
    if lib().or_q8_0_unplanes(_p(p), n, _p(out)):
        raise ValueError("or_q8_0_unplanes: bad size")
    return out


def set_threads(n):
    """Set the host threads the oracle's loops use (n > 0); returns the count
    in force afterwards (n = 0 only reads it)."""
    return lib().or_set_threads(int(n))

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

Q4_0, Q8_0, Q4_K, Q6_K = 2, 8, 12, 14
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

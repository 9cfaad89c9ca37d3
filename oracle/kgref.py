"""ctypes binding of the CPU oracle (oracle/libkgref.so).

TEST INFRASTRUCTURE: only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module. Argument marshalling only; all the
arithmetic is in kgref.c (fp64, see its header for the method and the readings
of the pages it follows).
"""
import ctypes
import os

import numpy as np

from . import build as _build

OK, ERR_NULL, ERR_SHAPE, ERR_GRAN, ERR_DTYPE, ERR_KSUM = 0, -1, -2, -3, -4, -9
E4M3_F32SCALE, E4M3_UE8M0, BF16 = 0, 1, 2
SRC_BF16, SRC_E4M3_1X128 = 0, 1
SCALE_F32, SCALE_UE8M0 = 0, 1

_lib = None


def lib():
    """Load the oracle library, compiling it first only if it is not built.
    KGREF_LIB names another build of kgref.c (the test suite's planted-mistake
    check loads deliberately broken copies that way)."""
    global _lib
    if _lib is None:
        path = os.environ.get("KGREF_LIB") or _build.LIB
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.kgref_e4m3.restype = ctypes.c_double
        L.kgref_e4m3.argtypes = [ctypes.c_uint8]
        L.kgref_e8m0.restype = ctypes.c_double
        L.kgref_e8m0.argtypes = [ctypes.c_uint8]
        L.kgref_bf16.restype = ctypes.c_double
        L.kgref_bf16.argtypes = [ctypes.c_uint16]
        L.kgref_validate.restype = ctypes.c_int
        L.kgref_validate.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, i64,
                                     ctypes.c_int, ctypes.c_int]
        L.kgref_offsets.restype = ctypes.c_int
        L.kgref_offsets.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp, vp]
        L.kgref_wgrad.restype = ctypes.c_int
        L.kgref_wgrad.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, i64, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  vp, vp, ctypes.c_int]
        L.kgref_wgrad_sampled.restype = ctypes.c_int
        L.kgref_wgrad_sampled.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, i64, ctypes.c_int, ctypes.c_int,
                                          i64, vp, vp, vp, vp, vp, ctypes.c_int]
        L.kgref_last_threads.restype = ctypes.c_int
        L.kgref_last_threads.argtypes = []
        L.kgref_e4m3_encode.restype = ctypes.c_uint8
        L.kgref_e4m3_encode.argtypes = [ctypes.c_double]
        L.kgref_bf16_round.restype = ctypes.c_uint16
        L.kgref_bf16_round.argtypes = [ctypes.c_double]
        L.kgref_bf16_round_array.restype = None
        L.kgref_bf16_round_array.argtypes = [vp, vp, i64]
        L.kgref_dgrad_validate.restype = ctypes.c_int
        L.kgref_dgrad_validate.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, i64]
        L.kgref_dgrad.restype = ctypes.c_int
        L.kgref_dgrad.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  i64, i64, i64, vp, vp, ctypes.c_int]
        L.kgref_dgrad_sampled.restype = ctypes.c_int
        L.kgref_dgrad_sampled.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, i64, i64, vp, vp, vp, vp, ctypes.c_int]
        L.kgref_requant.restype = ctypes.c_int
        L.kgref_requant.argtypes = [vp, vp, vp, ctypes.c_int, ctypes.c_int, i64, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, vp, vp]
        _lib = L
        del i32
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


def _inputs(A, sa, B, sb, C, ks, dtype):
    ks = np.ascontiguousarray(np.asarray(ks, dtype=np.int32))
    adt = np.uint16 if dtype == BF16 else np.uint8
    A = _c(A, adt)
    B = _c(B, adt)
    if dtype == E4M3_F32SCALE:
        sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    elif dtype == E4M3_UE8M0:
        sa, sb = _c(sa, np.uint8), _c(sb, np.uint8)
    C = _c(C, np.float32)
    return A, sa, B, sb, C, ks


def e4m3(byte):
    return lib().kgref_e4m3(int(byte))


def e8m0(byte):
    return lib().kgref_e8m0(int(byte))


def bf16(bits):
    return lib().kgref_bf16(int(bits))


def validate(ks, G, M, N, K_total, gran_k, dtype):
    ks = np.ascontiguousarray(np.asarray(ks, dtype=np.int32))
    return lib().kgref_validate(_ptr(ks) if G > 0 else None, G, M, N, K_total, gran_k, dtype)


def offsets(ks, gran_k):
    ks = np.ascontiguousarray(np.asarray(ks, dtype=np.int32))
    G = ks.size
    off = np.zeros(G + 1, np.int64)
    boff = np.zeros(G + 1, np.int32)
    rc = lib().kgref_offsets(_ptr(ks), G, gran_k, _ptr(off), _ptr(boff))
    if rc != OK:
        raise ValueError(f"kgref_offsets failed: {rc}")
    return off, boff


def wgrad(A, sa, B, sb, C, ks, M, N, gran_k, dtype, g_range=None, m_range=None,
          threads=0, K_total=None):
    """Reference D and bound (fp64) for groups g_range and rows m_range.

    Returns (rc, D, bound); D and bound have shape [g_hi-g_lo, m_hi-m_lo, N].
    """
    A, sa, B, sb, C, ks = _inputs(A, sa, B, sb, C, ks, dtype)
    G = ks.size
    if K_total is None:
        K_total = int(ks.astype(np.int64).sum())
    g_lo, g_hi = g_range if g_range is not None else (0, G)
    m_lo, m_hi = m_range if m_range is not None else (0, M)
    shape = (max(g_hi - g_lo, 0), max(m_hi - m_lo, 0), N)
    D = np.zeros(shape, np.float64)
    bound = np.zeros(shape, np.float64)
    rc = lib().kgref_wgrad(_ptr(A), _ptr(sa), _ptr(B), _ptr(sb), _ptr(C),
                           _ptr(ks) if G > 0 else None, G, M, N, K_total, gran_k, dtype,
                           g_lo, g_hi, m_lo, m_hi, _ptr(D), _ptr(bound), threads)
    return rc, D, bound


def wgrad_sampled(A, sa, B, sb, C, ks, M, N, gran_k, dtype, sg, sm, sn, threads=0,
                  K_total=None):
    """Reference value and bound for the elements (sg[i], sm[i], sn[i])."""
    A, sa, B, sb, C, ks = _inputs(A, sa, B, sb, C, ks, dtype)
    G = ks.size
    if K_total is None:
        K_total = int(ks.astype(np.int64).sum())
    sg = np.ascontiguousarray(sg, dtype=np.int32)
    sm = np.ascontiguousarray(sm, dtype=np.int32)
    sn = np.ascontiguousarray(sn, dtype=np.int32)
    ns = sg.size
    if sm.size != ns or sn.size != ns:
        raise ValueError("sample index arrays differ in length")
    out = np.zeros(ns, np.float64)
    bound = np.zeros(ns, np.float64)
    rc = lib().kgref_wgrad_sampled(_ptr(A), _ptr(sa), _ptr(B), _ptr(sb), _ptr(C),
                                   _ptr(ks) if G > 0 else None, G, M, N, K_total, gran_k,
                                   dtype, ns, _ptr(sg), _ptr(sm), _ptr(sn), _ptr(out),
                                   _ptr(bound), threads)
    return rc, out, bound


def last_threads():
    return lib().kgref_last_threads()


def e4m3_encode(v):
    return int(lib().kgref_e4m3_encode(float(v)))


def requant(X, xs, ks, H, gran_k, src, scale_kind, K_total=None):
    """Reference requantisation: returns (rc, Q uint8 [K_total, H], S [nblocks, H])."""
    ks = np.ascontiguousarray(np.asarray(ks, dtype=np.int32))
    G = ks.size
    if K_total is None:
        K_total = int(ks.astype(np.int64).sum())
    X = _c(X, np.uint16 if src == SRC_BF16 else np.uint8)
    xs = _c(xs, np.float32)
    nblk = int(sum((int(k) + gran_k - 1) // gran_k for k in ks))
    Q = np.zeros((K_total, H), np.uint8)
    S = np.zeros((nblk, H), np.float32 if scale_kind == SCALE_F32 else np.uint8)
    rc = lib().kgref_requant(_ptr(X), _ptr(xs), _ptr(ks) if G > 0 else None, G, H, K_total,
                             gran_k, src, scale_kind, _ptr(Q), _ptr(S))
    return rc, Q, S


def bf16_round(v):
    """Nearest bf16 codes (uint16) to the fp64 values v (kgref_bf16_round)."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().kgref_bf16_round_array(_ptr(v), _ptr(out), v.size)
    return out


def bf16_value(codes):
    """fp64 values of bf16 codes (kgref_bf16, elementwise)."""
    c = np.ascontiguousarray(codes, dtype=np.uint16)
    return (c.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dgrad(A, sa, W, sw, ms, N, K, rows=None, threads=0):
    """M-grouped dgrad reference: (rc, D [rows, N] fp64, bound [rows, N]) for token
    rows `rows` = (t_lo, t_hi) (default: all). A uint8 [M_total, K], sa float32
    [K/128, M_total], W uint8 [G, K, N], sw float32 [G, K/128, N/128], ms int32 [G]."""
    A = _c(A, np.uint8)
    sa = _c(sa, np.float32)
    W = _c(W, np.uint8)
    sw = _c(sw, np.float32)
    ms = _c(ms, np.int32)
    M_total = int(ms.astype(np.int64).sum())
    t_lo, t_hi = (0, M_total) if rows is None else rows
    D = np.zeros((max(t_hi - t_lo, 0), N), np.float64)
    bound = np.zeros_like(D)
    rc = lib().kgref_dgrad(_ptr(A), _ptr(sa), _ptr(W), _ptr(sw), _ptr(ms), ms.size, N, K,
                           M_total, t_lo, t_hi, _ptr(D), _ptr(bound), threads)
    return rc, D, bound


def dgrad_sampled(A, sa, W, sw, ms, N, K, st, sn, threads=0):
    """The dgrad reference for the elements (st[i], sn[i])."""
    A = _c(A, np.uint8)
    sa = _c(sa, np.float32)
    W = _c(W, np.uint8)
    sw = _c(sw, np.float32)
    ms = _c(ms, np.int32)
    M_total = int(ms.astype(np.int64).sum())
    st = np.ascontiguousarray(st, dtype=np.int64)
    sn = np.ascontiguousarray(sn, dtype=np.int32)
    out = np.zeros(st.size, np.float64)
    bound = np.zeros(st.size, np.float64)
    rc = lib().kgref_dgrad_sampled(_ptr(A), _ptr(sa), _ptr(W), _ptr(sw), _ptr(ms), ms.size, N, K,
                                   M_total, st.size, _ptr(st), _ptr(sn), _ptr(out), _ptr(bound),
                                   threads)
    return rc, out, bound


def token_major(Xt, K_total):
    """The K-major (NT) operand layout: channel m's K_total token values are
    contiguous, Xt[m, t] (rows may be longer than K_total; the rest is padding and
    is never read). Returns the same matrix token-major, X[t, m] = Xt[m, t] (issue
    page: dw = dy^t x with dy^t as A [M, K] and x^t as B [N, K], K = tokens)."""
    Xt = np.asarray(Xt)
    if Xt.ndim != 2 or Xt.shape[1] < K_total:
        raise ValueError("K-major operand must be [channels, >= K_total]")
    return np.ascontiguousarray(Xt[:, :K_total].T)


def wgrad_nt(At, sa, Bt, sb, C, ks, M, N, gran_k, dtype, K_total=None, **kw):
    """wgrad with K-major operands At [M, >= K_total] and Bt [N, >= K_total]: the
    same D as wgrad on their token-major forms; scales keep their [blocks, M] and
    [blocks, N] layout."""
    if K_total is None:
        K_total = int(np.asarray(ks, np.int64).sum())
    return wgrad(token_major(At, K_total), sa, token_major(Bt, K_total), sb, C, ks, M, N,
                 gran_k, dtype, K_total=K_total, **kw)


def wgrad_sampled_nt(At, sa, Bt, sb, C, ks, M, N, gran_k, dtype, sg, sm, sn, K_total=None,
                     **kw):
    """wgrad_sampled with K-major operands (see wgrad_nt)."""
    if K_total is None:
        K_total = int(np.asarray(ks, np.int64).sum())
    return wgrad_sampled(token_major(At, K_total), sa, token_major(Bt, K_total), sb, C, ks, M,
                         N, gran_k, dtype, sg, sm, sn, K_total=K_total, **kw)

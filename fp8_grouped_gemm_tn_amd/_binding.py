"""ctypes binding of libkgwgrad.so (the C ABI in include/kgwgrad.h).

Argument marshalling only: every step of the computation runs in the library's
HIP kernels. There is no fallback: if the library is missing or cannot be
loaded, the calls raise.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkgwgrad.so")

KG_E4M3_F32SCALE, KG_E4M3_UE8M0, KG_BF16 = 0, 1, 2
KG_FLAG_FP8_MFMA = 0x100
KG_FLAG_D_BF16 = 0x200
KG_OK = 0
KG_ERR_NULL, KG_ERR_SHAPE, KG_ERR_GRAN, KG_ERR_DTYPE = -1, -2, -3, -4
KG_ERR_ALIGN, KG_ERR_ALIAS, KG_ERR_UNSUPPORTED, KG_ERR_HIP, KG_ERR_KSUM = -5, -6, -7, -8, -9
KG_ERR_SPLIT = -10
KG_ERR_SCALE_ROWS = -11
KG_ERR_SCALE_RANGE = -12
KG_SRC_BF16, KG_SRC_E4M3_1X128 = 0, 1
ERROR_NAMES = {0: "KG_OK", -1: "KG_ERR_NULL", -2: "KG_ERR_SHAPE", -3: "KG_ERR_GRAN",
               -4: "KG_ERR_DTYPE", -5: "KG_ERR_ALIGN", -6: "KG_ERR_ALIAS",
               -7: "KG_ERR_UNSUPPORTED", -8: "KG_ERR_HIP", -9: "KG_ERR_KSUM",
               -10: "KG_ERR_SPLIT", -11: "KG_ERR_SCALE_ROWS",
               -12: "KG_ERR_SCALE_RANGE"}

# name -> (restype, argtypes): the symbols include/kgwgrad.h declares
_vp, _i32, _i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
SIGNATURES = {
    "kg_wgrad": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i64, _i64, _i32,
                        _i32, _vp]),
    "kg_wgrad_ws": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i64, _i64, _i32,
                           _i32, _vp, _i64, _vp]),
    "kg_wgrad_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i64, _i64,
                                _i32, _i32, _vp]),
    "kg_wgrad_nt": (_i32, [_vp, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i64,
                           _i64, _i32, _i32, _vp]),
    "kg_wgrad_nt_ws": (_i32, [_vp, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                              _i64, _i64, _i32, _i32, _vp, _i64, _vp]),
    "kg_wgrad_workspace_bytes": (_i64, []),
    "kg_wgrad_workspace_flag_bytes": (_i64, []),
    "kg_status": (_i32, [_vp]),
    "kg_debug_offsets": (_i32, [_vp, _i32, _i32, _vp, _vp, _vp]),
    "kg_max_groups": (_i32, []),
    "kg_requant": (_i32, [_vp, _vp, _vp, _i32, _i32, _i64, _i32, _i32, _i32, _vp, _vp, _i64,
                          _vp]),
    "kg_dgrad": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i64, _i32, _vp]),
}

_lib = None


class KgError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"{what} failed: {ERROR_NAMES.get(code, code)}")
        self.code = code


def lib():
    """The loaded library. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m fp8_grouped_gemm_tn_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _tensors_on_gpu(ref, **named):
    """Every given tensor contiguous (or, for the names in `strided`, checked by the
    caller) and on `ref`'s GPU. Checked after the shapes, so that shape errors
    show on any device."""
    for name, t in named.items():
        if t is None:
            continue
        _need(t.is_cuda, f"{name} must be a GPU tensor")
        _need(t.device == ref.device, f"{name} is on {t.device}, D on {ref.device}")


def _operand_dtype_ok(t, dtype):
    import torch
    if dtype == KG_BF16:
        return t.dtype == torch.bfloat16
    return t.element_size() == 1 and t.dtype != torch.bool


def _scale_dtype_ok(t, dtype):
    import torch
    return t.dtype == (torch.float32 if dtype == KG_E4M3_F32SCALE else torch.uint8)


def scale_rows_of(sa, sb):
    """The scale_rows argument: rows that both scale tensors hold (0 without scales).
    The library checks it against the rows the experts' blocks need."""
    if sa is None or sb is None:
        return 0
    return int(min(sa.shape[0], sb.shape[0]))


def _check_wgrad(A_cols, B_cols, sa, sb, C, D, ks, K_total, gran_k, dtype, A, B, kmajor):
    """Shapes and dtypes of a kg_wgrad / kg_wgrad_nt call (the C ABI takes plain
    pointers and cannot see extents). The scale tensors need at least
    ceil(K_total / gran_k) rows here; their row count goes to the library, which
    checks the exact need, sum ceil(ks / gran_k), on the device."""
    import torch
    base = dtype & 0xFF
    _need(base in (KG_E4M3_F32SCALE, KG_E4M3_UE8M0, KG_BF16), f"unknown dtype {base}")
    _need(D.dim() == 3, "D must be [G, M, N]")
    _need(D.dtype in (torch.float32, torch.bfloat16), "D must be float32 or bfloat16")
    _need(D.is_contiguous(), "D must be contiguous")
    G, M, N = D.shape
    _need(ks.dim() == 1 and ks.numel() == G and ks.dtype == torch.int32 and ks.is_contiguous(),
          "ks must be a contiguous int32 [G] tensor")
    if C is not None:
        _need(C.shape == D.shape and C.dtype == D.dtype and C.is_contiguous(),
              "C must be a contiguous tensor of D's shape and dtype")
    _need(A.dim() == 2 and B.dim() == 2, "A and B must be 2-D")
    _need(A_cols == M and B_cols == N, "A and B must have M and N channels (D is [G, M, N])")
    _need(_operand_dtype_ok(A, base) and _operand_dtype_ok(B, base),
          "A and B must be bfloat16 for KG_BF16, 1-byte fp8 codes otherwise")
    if kmajor:
        _need(A.shape[1] >= K_total and B.shape[1] >= K_total, "At and Bt hold fewer tokens than K_total")
    else:
        _need(A.is_contiguous() and B.is_contiguous(), "A and B must be contiguous")
        _need(A.shape[0] >= K_total and B.shape[0] >= K_total, "A and B hold fewer rows than K_total")
    if base == KG_BF16:
        _need(sa is None and sb is None, "bf16 operands take no scales")
    elif K_total > 0:
        _need(sa is not None and sb is not None, "fp8 operands need sa and sb")
        nmin = -(-int(K_total) // int(gran_k)) if gran_k > 0 else 0
        _need(sa.dim() == 2 and sa.shape[1] == M and sb.dim() == 2 and sb.shape[1] == N,
              "sa must be [nblk, M] and sb [nblk, N]")
        _need(sa.shape[0] >= nmin and sb.shape[0] >= nmin,
              f"sa and sb need at least ceil(K_total / gran_k) = {nmin} rows")
        _need(_scale_dtype_ok(sa, base) and _scale_dtype_ok(sb, base),
              "scales must be float32 (fp32 scales) or uint8 (UE8M0)")
        _need(sa.is_contiguous() and sb.is_contiguous(), "sa and sb must be contiguous")
    _tensors_on_gpu(D, A=A, B=B, sa=sa, sb=sb, C=C, ks=ks)


def kg_wgrad_raw(A, sa, B, sb, C, D, ks, G, M, N, K_total, gran_k, dtype, stream=None,
                 scale_rows=None):
    """Call kg_wgrad with torch device tensors (or None); returns the status code.
    scale_rows defaults to the rows the scale tensors hold."""
    if scale_rows is None:
        scale_rows = scale_rows_of(sa, sb)
    return lib().kg_wgrad(_ptr(A), _ptr(sa), _ptr(B), _ptr(sb), _ptr(C), _ptr(D), _ptr(ks),
                          int(G), int(M), int(N), int(K_total), int(scale_rows), int(gran_k),
                          int(dtype), _stream(stream))


def kg_wgrad_ws_raw(A, sa, B, sb, C, D, ks, G, M, N, K_total, gran_k, dtype, ws, ws_bytes,
                    stream=None, scale_rows=None):
    """Call kg_wgrad_ws with torch device tensors (or None); returns the status code."""
    if scale_rows is None:
        scale_rows = scale_rows_of(sa, sb)
    return lib().kg_wgrad_ws(_ptr(A), _ptr(sa), _ptr(B), _ptr(sb), _ptr(C), _ptr(D), _ptr(ks),
                             int(G), int(M), int(N), int(K_total), int(scale_rows), int(gran_k),
                             int(dtype), _ptr(ws), int(ws_bytes), _stream(stream))


def kg_wgrad_noalloc_raw(A, sa, B, sb, C, D, ks, G, M, N, K_total, gran_k, dtype, stream=None,
                         scale_rows=None):
    """Call kg_wgrad_noalloc (the library's static scratch instead of a workspace) with
    torch device tensors (or None); returns the status code."""
    if scale_rows is None:
        scale_rows = scale_rows_of(sa, sb)
    return lib().kg_wgrad_noalloc(_ptr(A), _ptr(sa), _ptr(B), _ptr(sb), _ptr(C), _ptr(D),
                                  _ptr(ks), int(G), int(M), int(N), int(K_total),
                                  int(scale_rows), int(gran_k), int(dtype), _stream(stream))


def kg_wgrad_workspace_bytes():
    n = lib().kg_wgrad_workspace_bytes()
    if n < 0:
        raise KgError(KG_ERR_HIP, "kg_wgrad_workspace_bytes")
    return n


def kg_wgrad_workspace_flag_bytes():
    n = lib().kg_wgrad_workspace_flag_bytes()
    if n < 0:
        raise KgError(KG_ERR_HIP, "kg_wgrad_workspace_flag_bytes")
    return n


def new_workspace(device=None):
    """A zeroed workspace tensor for kg_wgrad(..., workspace=...) on `device`."""
    import torch
    return torch.zeros(kg_wgrad_workspace_bytes(), dtype=torch.uint8, device=device or "cuda")


def kg_wgrad(A, sa, B, sb, C, D, ks, gran_k, dtype, K_total=None, stream=None, workspace=None):
    """D = C + K-grouped A^T B. Shapes are read from the tensors:
    A [K_total, M], B [K_total, N], D [G, M, N], ks [G] int32 (all on the GPU).
    A bfloat16 D (and C) selects the bf16-output variant (KG_FLAG_D_BF16).
    `workspace` (from new_workspace) lets problems with few tiles use every CU."""
    import torch
    if K_total is None:
        K_total = A.shape[0]
    if C is not None and C.dtype != D.dtype:
        raise TypeError("C and D must have the same dtype")
    _check_wgrad(A.shape[1] if A.dim() == 2 else -1, B.shape[1] if B.dim() == 2 else -1, sa, sb,
                 C, D, ks, K_total, gran_k, dtype, A, B, kmajor=False)
    if workspace is not None:
        _need(workspace.is_contiguous(), "workspace must be contiguous")
        _tensors_on_gpu(D, workspace=workspace)
    G, M, N = D.shape
    if D.dtype == torch.bfloat16:
        dtype |= KG_FLAG_D_BF16
    if workspace is None:
        rc = kg_wgrad_raw(A, sa, B, sb, C, D, ks, G, M, N, K_total, gran_k, dtype, stream)
    else:
        rc = kg_wgrad_ws_raw(A, sa, B, sb, C, D, ks, G, M, N, K_total, gran_k, dtype, workspace,
                             workspace.numel() * workspace.element_size(), stream)
    if rc != KG_OK:
        raise KgError(rc, "kg_wgrad")
    return D


def kg_wgrad_nt_raw(At, lda, sa, Bt, ldb, sb, C, D, ks, G, M, N, K_total, gran_k, dtype,
                    ws=None, ws_bytes=0, stream=None, scale_rows=None):
    """Call kg_wgrad_nt (or kg_wgrad_nt_ws when `ws` is given); returns the status."""
    if scale_rows is None:
        scale_rows = scale_rows_of(sa, sb)
    if ws is None:
        return lib().kg_wgrad_nt(_ptr(At), int(lda), _ptr(sa), _ptr(Bt), int(ldb), _ptr(sb),
                                 _ptr(C), _ptr(D), _ptr(ks), int(G), int(M), int(N), int(K_total),
                                 int(scale_rows), int(gran_k), int(dtype), _stream(stream))
    return lib().kg_wgrad_nt_ws(_ptr(At), int(lda), _ptr(sa), _ptr(Bt), int(ldb), _ptr(sb),
                                _ptr(C), _ptr(D), _ptr(ks), int(G), int(M), int(N), int(K_total),
                                int(scale_rows), int(gran_k), int(dtype), _ptr(ws), int(ws_bytes),
                                _stream(stream))


def kg_wgrad_nt(At, sa, Bt, sb, C, D, ks, gran_k, dtype, stream=None, workspace=None):
    """kg_wgrad with K-major operands: At [M, K_total] and Bt [N, K_total] with unit
    stride along tokens (row strides, e.g. of a padded buffer, are passed as lda and
    ldb). D [G, M, N]; a bfloat16 D selects the bf16-output variant."""
    import torch
    if At.dim() != 2 or Bt.dim() != 2 or At.stride(1) != 1 or Bt.stride(1) != 1:
        raise ValueError("At and Bt must be 2-D with unit stride along tokens")
    if At.shape[1] != Bt.shape[1]:
        raise ValueError("At and Bt must have the same number of tokens")
    _need(At.stride(0) >= At.shape[1] and Bt.stride(0) >= Bt.shape[1],
          "At and Bt rows must not overlap (row stride >= tokens)")
    if C is not None and C.dtype != D.dtype:
        raise TypeError("C and D must have the same dtype")
    _check_wgrad(At.shape[0], Bt.shape[0], sa, sb, C, D, ks, At.shape[1], gran_k, dtype, At, Bt,
                 kmajor=True)
    if workspace is not None:
        _need(workspace.is_contiguous(), "workspace must be contiguous")
        _tensors_on_gpu(D, workspace=workspace)
    G, M, N = D.shape
    if D.dtype == torch.bfloat16:
        dtype |= KG_FLAG_D_BF16
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = kg_wgrad_nt_raw(At, At.stride(0), sa, Bt, Bt.stride(0), sb, C, D, ks, G, M, N,
                         At.shape[1], gran_k, dtype, workspace, ws_bytes, stream)
    if rc != KG_OK:
        raise KgError(rc, "kg_wgrad_nt")
    return D


def kg_status(stream=None):
    return lib().kg_status(_stream(stream))


def kg_debug_offsets(ks, gran_k, off, boff, stream=None):
    rc = lib().kg_debug_offsets(_ptr(ks), int(ks.numel()), int(gran_k), _ptr(off), _ptr(boff),
                                _stream(stream))
    if rc != KG_OK:
        raise KgError(rc, "kg_debug_offsets")


def kg_max_groups():
    return lib().kg_max_groups()


def kg_requant_raw(X, xs, ks, G, H, K_total, gran_k, src, scale_kind, Q, S, stream=None,
                   s_rows=None):
    """Call kg_requant with torch device tensors (or None); returns the status code.
    s_rows defaults to the rows S holds."""
    if s_rows is None:
        s_rows = 0 if S is None else S.shape[0]
    return lib().kg_requant(_ptr(X), _ptr(xs), _ptr(ks), int(G), int(H), int(K_total), int(gran_k),
                            int(src), int(scale_kind), _ptr(Q), _ptr(S), int(s_rows),
                            _stream(stream))


def kg_requant(X, xs, ks, gran_k, scale_kind, nblk, Q=None, S=None, stream=None):
    """fp8 operand and per-(expert block, channel) scales for kg_wgrad from X.

    X: bf16 [K_total, H] (xs None) or e4m3fn bytes / float8 [K_total, H] with xs fp32
    [K_total, H/128]; ks int32 [G] on the GPU; nblk = sum(ceil(ks / gran_k)) (the scale
    rows; the caller knows ks). Returns (Q uint8 [K_total, H], S [nblk, H])."""
    import torch
    _need(X.dim() == 2 and X.is_contiguous(), "X must be a contiguous [K_total, H] tensor")
    K_total, H = X.shape
    src = KG_SRC_BF16 if X.dtype == torch.bfloat16 else KG_SRC_E4M3_1X128
    _need(src == KG_SRC_BF16 or (X.element_size() == 1 and X.dtype != torch.bool),
          "X must be bfloat16 or 1-byte e4m3 codes")
    if src == KG_SRC_BF16:
        _need(xs is None, "a bf16 source takes no xs")
    else:
        _need(xs is not None and xs.dtype == torch.float32 and xs.is_contiguous() and
              tuple(xs.shape) == (K_total, -(-H // 128)),
              "an fp8 source needs contiguous float32 xs [K_total, H / 128]")
    _need(ks.dim() == 1 and ks.dtype == torch.int32 and ks.is_contiguous(),
          "ks must be a contiguous int32 [G] tensor")
    sdt = torch.float32 if scale_kind == KG_E4M3_F32SCALE else torch.uint8
    if Q is None:
        Q = torch.empty((K_total, H), dtype=torch.uint8, device=X.device)
    if S is None:
        S = torch.empty((nblk, H), dtype=sdt, device=X.device)
    _need(tuple(Q.shape) == (K_total, H) and Q.element_size() == 1 and Q.is_contiguous(),
          "Q must be a contiguous 1-byte [K_total, H] tensor")
    _need(tuple(S.shape) == (nblk, H) and S.dtype == sdt and S.is_contiguous(),
          f"S must be a contiguous {sdt} [nblk, H] tensor")
    _tensors_on_gpu(X, xs=xs, ks=ks, Q=Q, S=S)
    rc = kg_requant_raw(X, xs, ks, ks.numel(), H, K_total, gran_k, src, scale_kind, Q, S, stream)
    if rc != KG_OK:
        raise KgError(rc, "kg_requant")
    return Q, S


def kg_dgrad_raw(A, sa, W, sw, D, ms, G, N, K, M_total, flags, stream=None):
    """Call kg_dgrad with torch device tensors (or None); returns the status code."""
    return lib().kg_dgrad(_ptr(A), _ptr(sa), _ptr(W), _ptr(sw), _ptr(D), _ptr(ms), int(G), int(N),
                          int(K), int(M_total), int(flags), _stream(stream))


def kg_dgrad(A, sa, W, sw, D, ms, flags=0, stream=None):
    """D = M-grouped dy . w: A (dy) [M_total, K] fp8 bytes, sa [K/128, M_total] fp32,
    W [G, K, N] fp8 bytes, sw [G, K/128, N/128] fp32, ms [G] int32, D [M_total, N]
    (float32, or bfloat16 for the bf16 output). All on the GPU."""
    import torch
    _need(W.dim() == 3 and W.element_size() == 1 and W.is_contiguous(),
          "W must be contiguous fp8 codes [G, K, N]")
    G, K, N = W.shape
    _need(A.dim() == 2 and A.shape[1] == K and A.element_size() == 1 and A.is_contiguous(),
          "A must be contiguous fp8 codes [M_total, K]")
    M_total = A.shape[0]
    _need(tuple(sa.shape) == (-(-K // 128), M_total) and sa.dtype == torch.float32 and
          sa.is_contiguous(), "sa must be contiguous float32 [K / 128, M_total]")
    _need(tuple(sw.shape) == (G, -(-K // 128), -(-N // 128)) and sw.dtype == torch.float32 and
          sw.is_contiguous(), "sw must be contiguous float32 [G, K / 128, N / 128]")
    _need(ms.dim() == 1 and ms.numel() == G and ms.dtype == torch.int32 and ms.is_contiguous(),
          "ms must be a contiguous int32 [G] tensor")
    _need(tuple(D.shape) == (M_total, N) and D.dtype in (torch.float32, torch.bfloat16) and
          D.is_contiguous(), "D must be a contiguous float32 or bfloat16 [M_total, N] tensor")
    _tensors_on_gpu(D, A=A, sa=sa, W=W, sw=sw, ms=ms)
    if D.dtype == torch.bfloat16:
        flags |= KG_FLAG_D_BF16
    rc = kg_dgrad_raw(A, sa, W, sw, D, ms, G, N, K, A.shape[0], flags, stream)
    if rc != KG_OK:
        raise KgError(rc, "kg_dgrad")
    return D

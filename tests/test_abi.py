"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching any GPU (all the
argument sets below fail validation, so no HIP call is made)."""
import ctypes
import os
import re

import numpy as np
import pytest

import fp8_grouped_gemm_tn_amd as kg
from fp8_grouped_gemm_tn_amd import _binding as B
from fp8_grouped_gemm_tn_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kgwgrad.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|int64_t)\s+(kg_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_symbols()
    assert names == sorted(B.SIGNATURES)
    lib = B.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_header_enums_match_binding():
    text = open(HEADER).read()
    for name, val in re.findall(r"(KG_\w+)\s*=\s*(-?\d+)", text):
        assert getattr(B, name) == int(val), name
    for name, val in re.findall(r"#define\s+(KG_\w+)\s+(0x[0-9a-fA-F]+|\d+)", text):
        assert getattr(B, name) == int(val, 0), name


def test_max_groups():
    assert kg.kg_max_groups() == 1024


FAKE = 0x100000  # an aligned, never dereferenced address


def call(A=FAKE, sa=FAKE, Bp=FAKE, sb=FAKE, C=None, D=FAKE + (1 << 30), ks=FAKE + (1 << 31),
         G=3, M=64, N=128, K=104, gran=128, dtype=kg.KG_E4M3_F32SCALE, rows=3):
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return B.lib().kg_wgrad(v(A), v(sa), v(Bp), v(sb), v(C), v(D), v(ks), G, M, N, K, rows, gran,
                            dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), B.KG_ERR_DTYPE),
    (dict(dtype=kg.KG_BF16 | kg.KG_FLAG_FP8_MFMA, sa=None, sb=None), B.KG_ERR_DTYPE),
    (dict(dtype=kg.KG_E4M3_F32SCALE | 0x400), B.KG_ERR_DTYPE),
    # bf16 output: the same checks with 2-byte C and D
    (dict(dtype=kg.KG_E4M3_F32SCALE | kg.KG_FLAG_D_BF16, C=FAKE + (1 << 30) + 32),
     B.KG_ERR_ALIAS),
    (dict(dtype=kg.KG_E4M3_F32SCALE | kg.KG_FLAG_D_BF16, D=FAKE + 4096), B.KG_ERR_ALIAS),
    (dict(dtype=kg.KG_BF16 | kg.KG_FLAG_D_BF16, sa=None, sb=None, D=FAKE + (1 << 30) + 2),
     B.KG_ERR_ALIGN),
    (dict(dtype=kg.KG_E4M3_F32SCALE | kg.KG_FLAG_D_BF16, M=40), B.KG_ERR_ALIGN),
    (dict(G=-1), B.KG_ERR_SHAPE),
    (dict(M=-16), B.KG_ERR_SHAPE),
    (dict(K=-1), B.KG_ERR_SHAPE),
    (dict(gran=64), B.KG_ERR_GRAN),
    (dict(G=1025), B.KG_ERR_UNSUPPORTED),
    (dict(D=None), B.KG_ERR_NULL),
    (dict(ks=None), B.KG_ERR_NULL),
    (dict(A=None), B.KG_ERR_NULL),
    (dict(sb=None), B.KG_ERR_NULL),
    (dict(dtype=kg.KG_BF16), B.KG_ERR_NULL),  # scales given for bf16
    (dict(M=72), B.KG_ERR_ALIGN),
    (dict(N=8), B.KG_ERR_ALIGN),
    (dict(A=FAKE + 4), B.KG_ERR_ALIGN),
    (dict(D=FAKE + (1 << 30) + 8), B.KG_ERR_ALIGN),
    (dict(C=FAKE + (1 << 30) + 64), B.KG_ERR_ALIAS),  # partial overlap of C and D
    (dict(D=FAKE + 4096), B.KG_ERR_ALIAS),  # D overlaps A
    # scale rows: fewer than ceil(K_total / gran_k) (1 here, 4 at gran 32)
    (dict(rows=0), B.KG_ERR_SCALE_ROWS),
    (dict(rows=-5), B.KG_ERR_SCALE_ROWS),
    (dict(rows=3, gran=32), B.KG_ERR_SCALE_ROWS),
    (dict(rows=0, dtype=kg.KG_E4M3_UE8M0, gran=32), B.KG_ERR_SCALE_ROWS),
    # ... and scale tensors of that many rows overlapping D
    (dict(sb=FAKE + (1 << 30) - 1024, rows=3), B.KG_ERR_ALIAS),
    (dict(sa=FAKE + (1 << 30) + 1024, rows=3), B.KG_ERR_ALIAS),
])
def test_synchronous_errors(kw, code):
    assert call(**kw) == code


def call_ws(ws=FAKE + (1 << 32), ws_bytes=1 << 26, **kw):
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    a = dict(A=FAKE, sa=FAKE, Bp=FAKE, sb=FAKE, C=None, D=FAKE + (1 << 30), ks=FAKE + (1 << 31),
             G=3, M=64, N=128, K=104, rows=3, gran=128, dtype=kg.KG_E4M3_F32SCALE)
    a.update(kw)
    return B.lib().kg_wgrad_ws(v(a["A"]), v(a["sa"]), v(a["Bp"]), v(a["sb"]), v(a["C"]), v(a["D"]),
                               v(a["ks"]), a["G"], a["M"], a["N"], a["K"], a["rows"], a["gran"],
                               a["dtype"], v(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(ws=FAKE + (1 << 32) + 16), B.KG_ERR_ALIGN),        # workspace not 256-byte aligned
    (dict(ws=FAKE + (1 << 30) - 256), B.KG_ERR_ALIAS),       # workspace overlaps D
    (dict(ws_bytes=-1), B.KG_ERR_SHAPE),
    (dict(M=1 << 15, N=1 << 15), B.KG_ERR_UNSUPPORTED),      # M * N above 2^29
    (dict(gran=64), B.KG_ERR_GRAN),
    (dict(rows=0), B.KG_ERR_SCALE_ROWS),
])
def test_workspace_entry_point_errors(kw, code):
    assert call_ws(**kw) == code


def call_nt(ws=None, ws_bytes=0, **kw):
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    a = dict(A=FAKE, lda=112, sa=FAKE, Bp=FAKE, ldb=112, sb=FAKE, C=None, D=FAKE + (1 << 30),
             ks=FAKE + (1 << 31), G=3, M=64, N=128, K=104, rows=3, gran=128,
             dtype=kg.KG_E4M3_F32SCALE)
    a.update(kw)
    args = (v(a["A"]), a["lda"], v(a["sa"]), v(a["Bp"]), a["ldb"], v(a["sb"]), v(a["C"]),
            v(a["D"]), v(a["ks"]), a["G"], a["M"], a["N"], a["K"], a["rows"], a["gran"],
            a["dtype"])
    if ws is None:
        return B.lib().kg_wgrad_nt(*args, None)
    return B.lib().kg_wgrad_nt_ws(*args, v(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(lda=100), B.KG_ERR_SHAPE),                         # row shorter than K_total
    (dict(ldb=96), B.KG_ERR_SHAPE),
    (dict(lda=104), B.KG_ERR_ALIGN),                         # 104 fp8 bytes: not whole 16 B
    (dict(ldb=120), B.KG_ERR_ALIGN),
    (dict(lda=(1 << 24) + 16), B.KG_ERR_UNSUPPORTED),        # 256 rows of offsets >= 2^32
    (dict(ldb=(1 << 23) + 8, dtype=kg.KG_BF16, sa=None, sb=None), B.KG_ERR_UNSUPPORTED),
    (dict(D=FAKE + 4096), B.KG_ERR_ALIAS),                   # D inside A's 64 rows of 112
    (dict(gran=64), B.KG_ERR_GRAN),
    (dict(A=FAKE + 8), B.KG_ERR_ALIGN),
    (dict(dtype=kg.KG_BF16, sa=None, sb=None, lda=108), B.KG_ERR_ALIGN),  # 216 bytes
    (dict(ws=FAKE + (1 << 32) + 16, ws_bytes=1 << 26), B.KG_ERR_ALIGN),
    (dict(rows=0), B.KG_ERR_SCALE_ROWS),
])
def test_nt_synchronous_errors(kw, code):
    assert call_nt(**kw) == code


def call_rq(X=FAKE, xs=None, ks=FAKE + (1 << 31), G=2, H=256, K=300, gran=128,
            src=B.KG_SRC_BF16, kind=kg.KG_E4M3_F32SCALE, Q=FAKE + (1 << 32), S=FAKE + (1 << 33),
            rows=4):
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return B.lib().kg_requant(v(X), v(xs), v(ks), G, H, K, gran, src, kind, v(Q), v(S), rows,
                              None)


@pytest.mark.parametrize("kw,code", [
    (dict(src=5), B.KG_ERR_DTYPE),
    (dict(kind=kg.KG_BF16), B.KG_ERR_DTYPE),
    (dict(G=-1), B.KG_ERR_SHAPE),
    (dict(H=-128), B.KG_ERR_SHAPE),
    (dict(gran=64), B.KG_ERR_GRAN),
    (dict(G=1025), B.KG_ERR_UNSUPPORTED),
    (dict(H=(1 << 23) + 128, K=3), B.KG_ERR_UNSUPPORTED),  # 32-bit buffer offsets
    (dict(Q=None), B.KG_ERR_NULL),
    (dict(ks=None), B.KG_ERR_NULL),
    (dict(src=B.KG_SRC_E4M3_1X128), B.KG_ERR_NULL),      # 1x128 source without its scales
    (dict(xs=FAKE), B.KG_ERR_NULL),                        # scales given for a bf16 source
    (dict(H=192), B.KG_ERR_ALIGN),
    (dict(Q=FAKE + (1 << 32) + 8), B.KG_ERR_ALIGN),
    (dict(Q=FAKE + 4096), B.KG_ERR_ALIAS),                 # Q overlaps X
    (dict(rows=2), B.KG_ERR_SCALE_ROWS),                   # S: fewer rows than ceil(300 / 128)
    (dict(rows=-1), B.KG_ERR_SCALE_ROWS),
    (dict(S=FAKE + (1 << 32) + 300 * 256 - 512), B.KG_ERR_ALIAS),  # S overlaps Q's end
])
def test_requant_synchronous_errors(kw, code):
    assert call_rq(**kw) == code


def test_requant_empty_is_ok_without_launch():
    assert call_rq(G=0) == B.KG_OK
    assert call_rq(H=0) == B.KG_OK


def test_empty_shapes_are_ok_without_launch():
    assert call(G=0) == B.KG_OK
    assert call(M=0) == B.KG_OK
    assert call(N=0) == B.KG_OK


def test_debug_offsets_errors():
    L = B.lib()
    v = ctypes.c_void_p
    assert L.kg_debug_offsets(v(FAKE), -1, 128, v(FAKE), v(FAKE), None) == B.KG_ERR_SHAPE
    assert L.kg_debug_offsets(v(FAKE), 1025, 128, v(FAKE), v(FAKE), None) == B.KG_ERR_SHAPE
    assert L.kg_debug_offsets(v(FAKE), 3, 0, v(FAKE), v(FAKE), None) == B.KG_ERR_GRAN
    assert L.kg_debug_offsets(None, 3, 128, v(FAKE), v(FAKE), None) == B.KG_ERR_NULL


# ---------------------------------------------------------------- generators

def test_routing_generators():
    for name in inputs.WORKLOADS:
        ks = inputs.workload_ks(name)
        assert ks.dtype == np.int32 and (ks >= 0).all()
    assert inputs.workload_ks("worked").tolist() == [32, 45, 27]
    ks = inputs.workload_ks("bf16")
    assert ks.size == 4 and ks[1] == 0 and ks.sum() == 16384
    ks = inputs.workload_ks("zipf_fp8")
    assert ks.size == 32 and ks.sum() == 65536 and ks.max() > 10 * max(ks.min(), 1)
    ks = inputs.workload_ks("ue8m0_many")
    assert ks.size == 256 and ks.sum() == 131072 and (ks == 0).sum() == 51
    ks = inputs.workload_ks("local_share")
    assert ks.size == 8 and ks.sum() == 262144


def test_quantizer_blocks_restart_per_group_and_fit_e4m3():
    import torch
    ks = np.array([130, 0, 5], np.int32)
    x = torch.randn(135, 16) * 3
    q, s = inputs.quantize_fp8(x, ks, 128, pow2=False)
    assert s.shape == (2 + 1, 16)  # ceil(130/128) + ceil(5/128)
    deq = q.view(torch.float8_e4m3fn).float()
    rows = torch.tensor([0] * 128 + [1] * 2 + [2] * 5)
    err = (deq * s[rows] - x).abs()
    assert (err <= x.abs() * 2 ** -3 + s[rows] * 2 ** -9).all()
    q2, e = inputs.quantize_fp8(x, ks, 32, pow2=True)
    assert e.dtype == torch.uint8 and e.shape == (5 + 1, 16)
    sc = torch.ldexp(torch.ones(e.shape), e.to(torch.int32) - 127)
    rows = torch.tensor([0] * 32 + [1] * 32 + [2] * 32 + [3] * 32 + [4] * 2 + [5] * 5)
    assert (q2.view(torch.float8_e4m3fn).float().abs() <= 448).all()
    assert ((q2.view(torch.float8_e4m3fn).float() * sc[rows] - x).abs() <= x.abs() * 2 ** -3 + sc[rows] * 2 ** -9).all()


def dcall(A=FAKE, sa=FAKE, W=FAKE + (1 << 28), sw=FAKE, D=FAKE + (1 << 30), ms=FAKE + (1 << 31),
          G=3, N=256, K=384, M=100, flags=0):
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return B.lib().kg_dgrad(v(A), v(sa), v(W), v(sw), v(D), v(ms), G, N, K, M, flags, None)


@pytest.mark.parametrize("kw,code", [
    (dict(flags=0x400), B.KG_ERR_DTYPE),
    (dict(G=-1), B.KG_ERR_SHAPE),
    (dict(K=-128), B.KG_ERR_SHAPE),
    (dict(M=-1), B.KG_ERR_SHAPE),
    (dict(G=1025), B.KG_ERR_UNSUPPORTED),
    (dict(K=200), B.KG_ERR_ALIGN),
    (dict(N=64), B.KG_ERR_ALIGN),
    (dict(D=None), B.KG_ERR_NULL),
    (dict(ms=None), B.KG_ERR_NULL),
    (dict(W=None), B.KG_ERR_NULL),
    (dict(sa=None), B.KG_ERR_NULL),
    (dict(A=FAKE + 8), B.KG_ERR_ALIGN),
    (dict(D=FAKE + (1 << 30) + 4), B.KG_ERR_ALIGN),
    (dict(D=FAKE + 4096), B.KG_ERR_ALIAS),                 # D overlaps A
    (dict(D=FAKE + (1 << 28), flags=kg.KG_FLAG_D_BF16), B.KG_ERR_ALIAS),  # D on W
    (dict(N=2097152, M=1, D=FAKE + (1 << 40)), B.KG_ERR_UNSUPPORTED),    # 256 x N x 4 >= 2^31
    (dict(K=8388608, M=1, W=FAKE + (1 << 40), D=FAKE + (1 << 44)),
     B.KG_ERR_UNSUPPORTED),                                              # 256 x K >= 2^31
])
def test_dgrad_synchronous_errors(kw, code):
    assert dcall(**kw) == code


def test_dgrad_empty_problems_launch_nothing():
    assert dcall(G=0) == B.KG_OK
    assert dcall(N=0) == B.KG_OK
    assert dcall(M=0) == B.KG_OK


# ---------------------------------------------------------------- binding checks
# The C ABI takes plain pointers; the Python wrappers check tensor shapes, dtypes,
# layout and device before calling it. CPU tensors: a well-formed call ends at the
# device check.

def _wgrad_args(**over):
    import torch
    M, N, K = 32, 48, 100
    a = dict(A=torch.zeros((K, M), dtype=torch.uint8), sa=torch.zeros((2, M)),
             B=torch.zeros((K, N), dtype=torch.uint8), sb=torch.zeros((2, N)), C=None,
             D=torch.zeros((2, M, N)), ks=torch.tensor([60, 40], dtype=torch.int32),
             gran_k=128, dtype=kg.KG_E4M3_F32SCALE)
    a.update(over)
    return a


def _bad_wgrad_cases():
    import torch
    return [
        (dict(A=torch.zeros((100, 16), dtype=torch.uint8)), "channels"),
        (dict(ks=torch.tensor([100], dtype=torch.int32)), "ks must"),
        (dict(ks=torch.tensor([60, 40], dtype=torch.int64)), "ks must"),
        (dict(sa=torch.zeros((2, 16))), "sa must be"),
        (dict(sa=torch.zeros((0, 32)), sb=torch.zeros((0, 48))), "rows"),
        (dict(sa=torch.zeros((2, 32), dtype=torch.uint8)), "scales must"),
        (dict(A=torch.zeros((100, 32), dtype=torch.bfloat16)), "1-byte"),
        (dict(A=torch.zeros((50, 32), dtype=torch.uint8), K_total=100), "fewer rows"),
        (dict(C=torch.zeros((2, 32, 16))), "C must"),
        (dict(D=torch.zeros((2, 48, 32)).transpose(1, 2)), "contiguous"),
        (dict(D=torch.zeros((2, 32, 48), dtype=torch.float64)), "float32 or bfloat16"),
        (dict(dtype=kg.KG_BF16, A=torch.zeros((100, 32), dtype=torch.bfloat16),
              B=torch.zeros((100, 48), dtype=torch.bfloat16)), "no scales"),
        (dict(), "GPU tensor"),
    ]


def test_wgrad_binding_rejects_bad_tensors():
    for over, msg in _bad_wgrad_cases():
        with pytest.raises(ValueError, match=msg):
            kg.kg_wgrad(**_wgrad_args(**over))


def test_wgrad_nt_binding_rejects_bad_tensors():
    import torch
    a = _wgrad_args()
    At = torch.zeros((32, 112), dtype=torch.uint8)[:, :100]
    Bt = torch.zeros((48, 112), dtype=torch.uint8)[:, :100]
    call = lambda **o: kg.kg_wgrad_nt(o.get("At", At), a["sa"], o.get("Bt", Bt), a["sb"], None,
                                      o.get("D", a["D"]), a["ks"], 128, a["dtype"])
    with pytest.raises(ValueError, match="unit stride"):
        call(At=torch.zeros((100, 32), dtype=torch.uint8).t())
    with pytest.raises(ValueError, match="same number of tokens"):
        call(Bt=torch.zeros((48, 112), dtype=torch.uint8)[:, :90])
    with pytest.raises(ValueError, match="channels"):
        call(At=torch.zeros((16, 112), dtype=torch.uint8)[:, :100])
    with pytest.raises(ValueError, match="must not overlap"):
        call(At=torch.zeros((32 * 50 + 50,), dtype=torch.uint8).as_strided((32, 100), (50, 1)))
    with pytest.raises(ValueError, match="GPU tensor"):
        call()


def test_dgrad_binding_rejects_bad_tensors():
    import torch
    G, K, N, Mt = 2, 256, 128, 40
    ok = dict(A=torch.zeros((Mt, K), dtype=torch.uint8), sa=torch.zeros((2, Mt)),
              W=torch.zeros((G, K, N), dtype=torch.uint8), sw=torch.zeros((G, 2, 1)),
              D=torch.zeros((Mt, N)), ms=torch.tensor([30, 10], dtype=torch.int32))
    for over, msg in [(dict(A=torch.zeros((Mt, 128), dtype=torch.uint8)), "A must"),
                      (dict(sa=torch.zeros((Mt, 2))), "sa must"),
                      (dict(sw=torch.zeros((G, 2, 2))), "sw must"),
                      (dict(ms=torch.tensor([40], dtype=torch.int32)), "ms must"),
                      (dict(D=torch.zeros((Mt, 256))), "D must"),
                      (dict(W=torch.zeros((G, K, N))), "W must"),
                      (dict(), "GPU tensor")]:
        a = dict(ok, **over)
        with pytest.raises(ValueError, match=msg):
            kg.kg_dgrad(a["A"], a["sa"], a["W"], a["sw"], a["D"], a["ms"])


def test_requant_binding_rejects_bad_tensors():
    import torch
    ks = torch.tensor([60, 40], dtype=torch.int32)
    X = torch.zeros((100, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="no xs"):
        kg.kg_requant(X, torch.zeros((100, 2)), ks, 128, kg.KG_E4M3_F32SCALE, 2)
    with pytest.raises(ValueError, match="xs"):
        kg.kg_requant(torch.zeros((100, 256), dtype=torch.uint8), None, ks, 128,
                      kg.KG_E4M3_F32SCALE, 2)
    with pytest.raises(ValueError, match="S must"):
        kg.kg_requant(X, None, ks, 128, kg.KG_E4M3_F32SCALE, 2, S=torch.zeros((2, 256), dtype=torch.uint8))
    with pytest.raises(ValueError, match="X must"):
        kg.kg_requant(X.t(), None, ks, 128, kg.KG_E4M3_F32SCALE, 2)
    with pytest.raises(ValueError, match="GPU tensor"):
        kg.kg_requant(X, None, ks, 128, kg.KG_E4M3_F32SCALE, 2)

"""kg_wgrad_noalloc (the library's static device scratch instead of a caller-owned
workspace) against kg_wgrad_ws, through the C ABI: two calls in a row, the second
with a smaller problem, each bit-identical to the workspace entry point's result on
the same inputs and within the tolerance of the CPU oracle."""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_tn_amd as kg
from fp8_grouped_gemm_tn_amd import inputs
from oracle import kgref

pytestmark = pytest.mark.gpu

RTOL, ATOL, FROB = 1e-5, 1e-6, 1e-5
FAST_RTOL, FAST_FROB = 2.0 ** -10, 1e-4

# (dtype, gran, flags, ks, M, N): both take the stream-K mode (few tiles), the second
# is the smaller one; then a problem of whole tiles
CALLS = [
    (kg.KG_E4M3_F32SCALE, 128, 0, [4000, 1234], 512, 1024),
    (kg.KG_E4M3_F32SCALE, 128, 0, [300, 0, 517], 256, 256),
    (kg.KG_BF16, 128, 0, [640, 0, 129, 77], 128, 256),
    (kg.KG_E4M3_UE8M0, 32, kg.KG_FLAG_FP8_MFMA, [33, 0, 1000], 256, 512),
]


def check(case, D, fast):
    h = case.host()
    rc, D_ref, bound = kgref.wgrad(h["A"], h["sa"], h["B"], h["sb"], h["C"], h["ks"], case.M,
                                   case.N, case.gran_k, case.dtype)
    assert rc == kgref.OK
    got = D.cpu().numpy().astype(np.float64)
    err = np.abs(got - D_ref)
    assert (err <= (FAST_RTOL if fast else RTOL) * bound + ATOL).all()
    assert np.linalg.norm(got - D_ref) <= (FAST_FROB if fast else FROB) * np.linalg.norm(D_ref)


def test_noalloc_matches_workspace_entry_point_twice():
    d = torch.device("cuda:0")
    ws = kg.new_workspace(d)
    for i, (dtype, gran, flags, ks, M, N) in enumerate(CALLS):
        print(f"[case] noalloc call {i}: dtype {dtype} gran {gran} flags {flags} ks {ks} "
              f"M {M} N {N}", flush=True)
        case = inputs.make_case("noalloc", ks, M, N, dtype, gran, with_c=True, seed=50 + i,
                                b_std=1e-3, a_outlier_p=0.01)
        mv = lambda t: None if t is None else t.to(d)
        A, B, sa, sb, C = mv(case.A), mv(case.B), mv(case.sa), mv(case.sb), mv(case.C)
        ksd = torch.from_numpy(case.ks).to(d)
        D_ws = torch.full((case.G, M, N), float("nan"), device=d)
        rc = kg.kg_wgrad_ws_raw(A, sa, B, sb, C, D_ws, ksd, case.G, M, N, case.K_total, gran,
                                dtype | flags, ws, ws.numel())
        assert rc == kg.KG_OK and kg.kg_status() == kg.KG_OK
        D_na = torch.full_like(D_ws, float("nan"))
        rc = kg.kg_wgrad_noalloc_raw(A, sa, B, sb, C, D_na, ksd, case.G, M, N, case.K_total,
                                     gran, dtype | flags)
        assert rc == kg.KG_OK and kg.kg_status() == kg.KG_OK
        torch.cuda.synchronize()
        assert torch.equal(D_na.view(torch.int32), D_ws.view(torch.int32)), f"call {i}"
        check(case, D_na, bool(flags))

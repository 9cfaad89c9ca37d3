"""GPU parity: libkgwgrad (through its C ABI) against the CPU oracle.

Default (precise) paths, from the fp32 accumulation of exact fp8 or bf16 products:
|D - D_ref| <= 1e-5 * sum_t |a(t,m) b(t,n)| + 1e-6 and ||D - D_ref||_F <=
1e-5 ||D_ref||_F. Offsets and empty experts are bit-exact.

Fast fp8-MFMA mode (KG_FLAG_FP8_MFMA): gfx950's fp8 MFMA adds each group of 8
products aligned to the largest with about 13 bits, so a group loses less than
8 * 2^-13 of its largest product, i.e. at most 2^-10 of its sum of |products|:
|D - D_ref| <= 2^-10 * sum|ab| + 1e-6, and ||D - D_ref||_F <= 1e-4 ||D_ref||_F.
"""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_tn_amd as kg
from fp8_grouped_gemm_tn_amd import inputs
from oracle import kgref

pytestmark = pytest.mark.gpu

F32, UE8, BF = kg.KG_E4M3_F32SCALE, kg.KG_E4M3_UE8M0, kg.KG_BF16
FAST = kg.KG_FLAG_FP8_MFMA
RTOL, ATOL, FROB = 1e-5, 1e-6, 1e-5
FAST_RTOL, FAST_FROB = 2.0 ** -10, 1e-4


def say(*a):
    print("[case]", *a, flush=True)


def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def to_dev(case):
    d = dev()
    mv = lambda t: None if t is None else t.to(d)
    return dict(A=mv(case.A), B=mv(case.B), sa=mv(case.sa), sb=mv(case.sb), C=mv(case.C),
                ks=torch.from_numpy(case.ks).to(d))


def run_gpu(case, t, D=None, C="default", check_status=True, flags=0):
    if D is None:
        D = torch.full((case.G, case.M, case.N), float("nan"), dtype=torch.float32, device=dev())
    Cp = t["C"] if isinstance(C, str) else C
    kg.kg_wgrad(t["A"], t["sa"], t["B"], t["sb"], Cp, D, t["ks"], case.gran_k,
                case.dtype | flags, K_total=case.K_total)
    if check_status:
        assert kg.kg_status() == kg.KG_OK
    torch.cuda.synchronize()
    return D


def oracle_full(case, C="default"):
    h = case.host()
    Ch = h["C"] if isinstance(C, str) else C
    rc, D, bound = kgref.wgrad(h["A"], h["sa"], h["B"], h["sb"], Ch, h["ks"], case.M, case.N,
                               case.gran_k, case.dtype)
    assert rc == kgref.OK
    return D, bound


def check_close(D_gpu, D_ref, bound, what="", fast=False):
    D = D_gpu.detach().cpu().numpy().astype(np.float64)
    assert np.isfinite(D).all(), f"{what}: non-finite output"
    err = np.abs(D - D_ref)
    lim = (FAST_RTOL if fast else RTOL) * bound + ATOL
    bad = err > lim
    assert not bad.any(), (f"{what}: {bad.sum()} elements out of tolerance, worst "
                           f"{(err - lim).max():.3e} at {np.unravel_index(np.argmax(err - lim), err.shape)}")
    ref_norm = np.linalg.norm(D_ref)
    if ref_norm > 0:
        rel = np.linalg.norm(D - D_ref) / ref_norm
        assert rel <= (FAST_FROB if fast else FROB), f"{what}: Frobenius {rel:.3e}"


def small_case(dtype, gran, ks, M, N, with_c=True, seed=1, **kw):
    return inputs.make_case("small", ks, M, N, dtype, gran, with_c=with_c, seed=seed, **kw)


# ---------------------------------------------------------------- offsets

def test_device_offsets_bit_exact():
    for ks, gran in [([32, 45, 27], 128), ([32, 45, 27], 32), ([0, 5, 0, 300, 1, 0, 4096], 128),
                     (list(np.random.default_rng(0).integers(0, 3000, 1024)), 32), ([], 128)]:
        say("offsets", len(ks), gran)
        ks_np = np.asarray(ks, np.int32)
        G = ks_np.size
        off = torch.full((G + 1,), -7, dtype=torch.int64, device=dev())
        boff = torch.full((G + 1,), -7, dtype=torch.int32, device=dev())
        kg.kg_debug_offsets(torch.from_numpy(ks_np).to(dev()), gran, off, boff)
        torch.cuda.synchronize()
        if G == 0:
            assert off.cpu().tolist() == [0] and boff.cpu().tolist() == [0]
            continue
        r_off, r_boff = kgref.offsets(ks_np, gran)
        assert off.cpu().numpy().tolist() == r_off.tolist()
        assert boff.cpu().numpy().tolist() == r_boff.tolist()


# ---------------------------------------------------------------- worked shape

def test_worked_shape_full():
    say("worked shape")
    case = inputs.workload("worked")
    t = to_dev(case)
    D = run_gpu(case, t)
    D_ref, bound = oracle_full(case)
    check_close(D, D_ref, bound, "worked")


# ---------------------------------------------------------------- multi-tile ragged

RAGGED = [300, 0, 129, 1, 513, 64]
PATHS = [(F32, 128), (F32, 32), (UE8, 32), (UE8, 128), (BF, 128)]


@pytest.mark.parametrize("dtype,gran", PATHS)
@pytest.mark.parametrize("with_c", [True, False])
def test_ragged_multi_tile(dtype, gran, with_c):
    say("ragged", dtype, gran, with_c)
    # M spans two m-tiles (the second partial), N spans two n-tiles (partial)
    case = small_case(dtype, gran, RAGGED, 320, 272, with_c=with_c, seed=3)
    t = to_dev(case)
    D = run_gpu(case, t)
    D_ref, bound = oracle_full(case)
    check_close(D, D_ref, bound, f"ragged {dtype} {gran}")
    # empty expert: bit-exact passthrough of C, or +0.0
    g = RAGGED.index(0)
    Dg = D[g].cpu()
    if with_c:
        assert torch.equal(Dg.view(torch.int32), case.C[g].view(torch.int32))
    else:
        assert torch.equal(Dg.view(torch.int32), torch.zeros_like(Dg).view(torch.int32))


@pytest.mark.parametrize("dtype,gran", PATHS)
def test_outliers_and_small_gradients(dtype, gran):
    say("outliers", dtype, gran)
    case = small_case(dtype, gran, [700, 77, 1000], 256, 512, seed=4, b_std=1e-3,
                      a_outlier_p=0.01)
    t = to_dev(case)
    D = run_gpu(case, t)
    D_ref, bound = oracle_full(case)
    check_close(D, D_ref, bound, "outliers")


FAST_PATHS = [(F32, 128), (F32, 32), (UE8, 32), (UE8, 128)]


@pytest.mark.parametrize("dtype,gran", FAST_PATHS)
@pytest.mark.parametrize("with_c", [True, False])
def test_fast_fp8_mfma_mode(dtype, gran, with_c):
    say("fast", dtype, gran, with_c)
    case = small_case(dtype, gran, RAGGED, 320, 272, with_c=with_c, seed=13, b_std=1e-3,
                      a_outlier_p=0.01)
    t = to_dev(case)
    D = run_gpu(case, t, flags=FAST)
    D_ref, bound = oracle_full(case)
    check_close(D, D_ref, bound, f"fast {dtype} {gran}", fast=True)
    g = RAGGED.index(0)
    if with_c:
        assert torch.equal(D[g].cpu().view(torch.int32), case.C[g].view(torch.int32))


def test_bf16_many_tiles_large_tile_config():
    # enough 256 x 256 tiles (G * 1 * 1 >= 2 per CU) that the bf16 path takes its
    # full-size tile configuration; ragged and empty experts throughout
    say("bf16 many tiles")
    rng = np.random.default_rng(14)
    ks = rng.integers(0, 97, 600).astype(np.int32)
    ks[rng.choice(600, 60, replace=False)] = 0
    case = small_case(BF, 128, ks, 256, 256, seed=14)
    t = to_dev(case)
    D = run_gpu(case, t)
    D_ref, bound = oracle_full(case)
    check_close(D, D_ref, bound, "bf16 many tiles")
    for g in np.nonzero(ks == 0)[0]:
        assert torch.equal(D[g].cpu().view(torch.int32), case.C[g].view(torch.int32))


def _ws_clean(ws):
    """The workspace's flag area is zero again after a successful call."""
    torch.cuda.synchronize()
    return int(ws[:kg.kg_wgrad_workspace_flag_bytes()].count_nonzero()) == 0


SPLIT_SHAPES = [
    ([300, 0, 517], 256, 256, True),      # few stages over every CU: tiles cut into 1-stage units
    ([4000, 1234], 512, 1024, False),     # several tiles per expert, cuts inside tiles
    ([0, 1, 33, 0], 256, 512, True),      # tiny and empty experts
    # the largest group count stream-K takes (64), and one more (whole tiles although
    # a workspace is given); ragged experts, every ninth one empty
    ([0 if i % 9 == 0 else (37 * i) % 301 + 1 for i in range(64)], 128, 256, True),
    ([0 if i % 9 == 0 else (37 * i) % 301 + 1 for i in range(65)], 128, 256, False),
]


@pytest.mark.parametrize("dtype,gran,flags", [(BF, 128, 0), (F32, 128, 0), (UE8, 32, 0),
                                              (UE8, 128, 0), (F32, 128, FAST), (UE8, 32, FAST),
                                              (F32, 32, 0), (F32, 32, FAST)])
@pytest.mark.parametrize("ks,M,N,with_c", SPLIT_SHAPES)
def test_stream_k_workspace(ks, M, N, with_c, dtype, gran, flags):
    say("stream-K", dtype, gran, flags, ks, M, N, with_c)
    case = small_case(dtype, gran, ks, M, N, with_c=with_c, seed=15, b_std=1e-3, a_outlier_p=0.01)
    t = to_dev(case)
    ws = kg.new_workspace()
    D = torch.full((case.G, M, N), float("nan"), device=dev())
    kg.kg_wgrad(t["A"], t["sa"], t["B"], t["sb"], t["C"], D, t["ks"], gran, dtype | flags,
                workspace=ws)
    assert kg.kg_status() == kg.KG_OK
    assert _ws_clean(ws), "workspace flags not left zero"
    D_ref, bound = oracle_full(case)
    check_close(D, D_ref, bound, "stream-K", fast=bool(flags))
    for g in np.nonzero(np.asarray(ks) == 0)[0]:
        want = case.C[g] if with_c else torch.zeros_like(case.C[g] if with_c else D[g].cpu())
        assert torch.equal(D[g].cpu().view(torch.int32), want.view(torch.int32))
    # same bits on a second call through the same workspace
    D2 = torch.full_like(D, float("nan"))
    kg.kg_wgrad(t["A"], t["sa"], t["B"], t["sb"], t["C"], D2, t["ks"], gran, dtype | flags,
                workspace=ws)
    assert kg.kg_status() == kg.KG_OK
    assert torch.equal(D.view(torch.int32), D2.view(torch.int32))
    assert _ws_clean(ws)


@pytest.mark.parametrize("dtype,gran,flags", [(F32, 128, 0), (BF, 128, 0), (UE8, 32, FAST)])
def test_stream_k_beside_a_long_kernel_on_another_stream(dtype, gran, flags):
    """Stream-K needs no co-resident workgroups: with matrix products occupying the GPU
    from another stream, a stream-K call on its own stream completes with the oracle's
    result (to the tolerance), the same bits as on an idle GPU, and clean counters."""
    say("stream-K beside", dtype, gran, flags)
    case = small_case(dtype, gran, [4000, 1234], 512, 1024, seed=43, b_std=1e-3,
                      a_outlier_p=0.01)
    t = to_dev(case)
    ws = kg.new_workspace(dev())
    D_idle = torch.full((case.G, case.M, case.N), float("nan"), device=dev())
    kg.kg_wgrad(t["A"], t["sa"], t["B"], t["sb"], t["C"], D_idle, t["ks"], gran, dtype | flags,
                workspace=ws)
    assert kg.kg_status() == kg.KG_OK
    X = torch.randn((8192, 8192), device=dev()).to(torch.bfloat16)
    busy, mine = torch.cuda.Stream(), torch.cuda.Stream()
    D = torch.full_like(D_idle, float("nan"))
    torch.cuda.synchronize()
    with torch.cuda.stream(busy):
        Y = X
        for _ in range(12):
            Y = torch.mm(Y, X) * 1e-2
    with torch.cuda.stream(mine):
        kg.kg_wgrad(t["A"], t["sa"], t["B"], t["sb"], t["C"], D, t["ks"], gran, dtype | flags,
                    workspace=ws)
    torch.cuda.synchronize()
    assert kg.kg_status() == kg.KG_OK
    assert _ws_clean(ws)
    assert torch.equal(D.view(torch.int32), D_idle.view(torch.int32))
    D_ref, bound = oracle_full(case)
    check_close(D, D_ref, bound, "stream-K beside", fast=bool(flags))
    del X, Y


def test_bf16_stream_k_full_workload_and_in_place():
    say("stream-K full bf16 workload")
    case = inputs.workload("bf16", device="cuda")
    t = to_dev(case)
    ws = kg.new_workspace()
    D = torch.empty((case.G, case.M, case.N), dtype=torch.float32, device=dev())
    kg.kg_wgrad(t["A"], None, t["B"], None, t["C"], D, t["ks"], 128, BF, workspace=ws)
    assert kg.kg_status() == kg.KG_OK and _ws_clean(ws)
    sampled_check(case, t, D)
    # in place: D starts as C
    Di = t["C"].clone()
    kg.kg_wgrad(t["A"], None, t["B"], None, Di, Di, t["ks"], 128, BF, workspace=ws)
    assert kg.kg_status() == kg.KG_OK and _ws_clean(ws)
    assert torch.equal(Di.view(torch.int32), D.view(torch.int32))


@pytest.mark.parametrize("dtype,gran", [(F32, 128), (BF, 128)])
def test_in_place_accumulate(dtype, gran):
    say("in place", dtype)
    case = small_case(dtype, gran, [200, 0, 57], 64, 128, seed=5)
    t = to_dev(case)
    D = t["C"].clone()
    run_gpu(case, t, D=D, C=D)
    D_ref, bound = oracle_full(case)
    check_close(D, D_ref, bound, "in place")


def test_guard_canaries_and_determinism():
    say("canaries")
    case = small_case(F32, 128, [129, 0, 400], 128, 256, seed=6)
    t = to_dev(case)
    n = case.G * case.M * case.N
    pad = 4096
    buf = torch.full((n + 2 * pad,), 12345.0, dtype=torch.float32, device=dev())
    D = buf[pad:pad + n].view(case.G, case.M, case.N)
    run_gpu(case, t, D=D)
    assert (buf[:pad] == 12345.0).all() and (buf[pad + n:] == 12345.0).all()
    D2 = run_gpu(case, t)
    assert torch.equal(D.view(torch.int32), D2.view(torch.int32)), "run-to-run bits differ"


CANARY_PATHS = [(F32, 128, 0), (F32, 128, FAST), (F32, 32, 0), (F32, 32, FAST), (UE8, 32, 0),
                (UE8, 32, FAST), (UE8, 128, 0), (UE8, 128, FAST), (BF, 128, 0)]


def guarded(shape, dtype, pad=4096):
    """A tensor of `shape` inside a buffer whose `pad` elements before and after hold a
    canary pattern; returns (tensor, check) where check() asserts the canaries."""
    n = int(np.prod(shape))
    if dtype == torch.float32:
        buf = torch.full((n + 2 * pad,), 12345.0, dtype=torch.float32, device=dev())
        pat = torch.tensor(12345.0).view(torch.int32).item()
        raw = buf.view(torch.int32)
    else:
        raw = torch.full((n + 2 * pad,), 0x3F8F, dtype=torch.int16, device=dev())
        buf, pat = raw.view(torch.bfloat16), 0x3F8F
    check = lambda: (raw[:pad] == pat).all().item() and (raw[pad + n:] == pat).all().item()
    return buf[pad:pad + n].view(*shape), check


@pytest.mark.parametrize("dtype,gran,flags", CANARY_PATHS)
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("split", [False, True])
def test_canaries_every_path(dtype, gran, flags, out, split):
    """Every kind and mode, fp32 and bf16 output, whole tiles and (with the workspace,
    fp32 output) stream-K: ragged tiles in both dimensions, an empty and a one-token
    expert, with C. Nothing is written outside D, two runs give the same bits, and the
    result matches the oracle."""
    say("canaries", dtype, gran, flags, out, split)
    case = small_case(dtype, gran, [129, 0, 400, 1], 272, 144, seed=17)
    t = to_dev(case)
    C = t["C"] if out == torch.float32 else t["C"].to(torch.bfloat16)
    ws = kg.new_workspace(dev()) if split else None
    D, intact = guarded((case.G, case.M, case.N), out)
    runs = []
    for _ in range(2):
        kg.kg_wgrad(t["A"], t["sa"], t["B"], t["sb"], C, D, t["ks"], gran, dtype | flags,
                    workspace=ws)
        assert kg.kg_status() == kg.KG_OK
        torch.cuda.synchronize()
        assert intact(), "a write landed outside D"
        runs.append(D.clone())
    assert torch.equal(runs[0].view(torch.int16), runs[1].view(torch.int16)), "run-to-run bits differ"
    D_ref, bound = oracle_full(case, C=C.float().cpu().numpy())
    if out == torch.float32:
        check_close(D, D_ref, bound, "canaries", fast=bool(flags))
    else:
        check_bf16_out(D, D_ref, bound, "canaries", fast=bool(flags))


def test_power_of_two_scales_bit_exact_on_gpu():
    say("power of two")
    case = small_case(F32, 128, [300, 45], 128, 128, with_c=False, seed=7)
    t = to_dev(case)
    D = run_gpu(case, t)
    t2 = dict(t, sa=t["sa"] * 8.0)
    D8 = run_gpu(case, t2)
    assert torch.equal(D8, D * 8.0)
    case = small_case(UE8, 32, [300, 45], 128, 128, with_c=False, seed=7)
    t = to_dev(case)
    D = run_gpu(case, t)
    t2 = dict(t, sb=(t["sb"].to(torch.int32) - 3).to(torch.uint8))
    Dm = run_gpu(case, t2)
    assert torch.equal(Dm, D / 8.0)


def test_k_split_invariant_on_gpu():
    say("k split")
    case = small_case(F32, 128, [50, 3 * 128 + 17, 9], 128, 256, seed=8)
    t = to_dev(case)
    D = run_gpu(case, t)
    ks2 = torch.tensor([50, 256, 128 + 17, 9], dtype=torch.int32, device=dev())
    C2 = torch.cat([t["C"][:2], torch.zeros_like(t["C"][:1]), t["C"][2:]])
    D2 = torch.empty((4, case.M, case.N), dtype=torch.float32, device=dev())
    kg.kg_wgrad(t["A"], t["sa"], t["B"], t["sb"], C2, D2, ks2, 128, F32, K_total=case.K_total)
    assert kg.kg_status() == kg.KG_OK
    torch.cuda.synchronize()
    # D2[1] + D2[2] must equal D[1] to the tolerance, measured against sum|ab|
    _, bound = oracle_full(case)
    s = (D2[1] + D2[2]).double().cpu().numpy()
    ref = D[1].double().cpu().numpy()
    assert (np.abs(s - ref) <= 2e-5 * bound[1] + 2e-6).all()
    assert torch.equal(D2[0], D[0]) and torch.equal(D2[3], D[2])


# ---------------------------------------------------------------- edge cases

def test_all_groups_empty_and_single_group():
    say("all empty")
    case = small_case(F32, 128, [0, 0, 0], 64, 64, seed=9)
    t = to_dev(case)
    D = run_gpu(case, t)
    assert torch.equal(D.cpu().view(torch.int32), case.C.view(torch.int32))
    say("single group, minimal 16x16")
    case = small_case(BF, 128, [1], 16, 16, seed=10)
    t = to_dev(case)
    D = run_gpu(case, t)
    D_ref, bound = oracle_full(case)
    check_close(D, D_ref, bound, "16x16")


def test_max_groups():
    say("G = 1024")
    rng = np.random.default_rng(11)
    ks = rng.integers(0, 40, 1024).astype(np.int32)
    ks[rng.choice(1024, 100, replace=False)] = 0
    case = small_case(UE8, 32, ks, 16, 32, seed=11)
    t = to_dev(case)
    D = run_gpu(case, t)
    D_ref, bound = oracle_full(case)
    check_close(D, D_ref, bound, "G=1024")


def test_ksum_mismatch_is_reported_and_writes_nothing():
    say("ksum mismatch")
    case = small_case(F32, 128, [100, 28], 64, 64, seed=12)
    t = to_dev(case)
    D = torch.full((2, 64, 64), float("nan"), device=dev())
    rc = kg.kg_wgrad_raw(t["A"], t["sa"], t["B"], t["sb"], t["C"], D, t["ks"], 2, 64, 64,
                         case.K_total - 1, 128, F32)
    assert rc == kg.KG_OK
    assert kg.kg_status() == kg.KG_ERR_KSUM
    assert torch.isnan(D).all()
    assert kg.kg_status() == kg.KG_OK  # cleared
    bad = torch.tensor([130, -2], dtype=torch.int32, device=dev())
    rc = kg.kg_wgrad_raw(t["A"], t["sa"], t["B"], t["sb"], t["C"], D, bad, 2, 64, 64,
                         case.K_total, 128, F32)
    assert rc == kg.KG_OK and kg.kg_status() == kg.KG_ERR_KSUM
    assert torch.isnan(D).all()


@pytest.mark.parametrize("dtype,gran", [(F32, 128), (F32, 32), (UE8, 32), (UE8, 128)])
def test_too_few_scale_rows_is_reported_and_writes_nothing(dtype, gran):
    """The experts' blocks need sum ceil(ks / gran_k) scale rows (12 at gran 128 here):
    with fewer, but at least ceil(K_total / gran_k), the host cannot tell, and the
    kernel reports KG_ERR_SCALE_ROWS without writing D or reading past the rows."""
    say("scale rows", dtype, gran)
    case = small_case(dtype, gran, RAGGED, 64, 128, seed=12)
    t = to_dev(case)
    need = int(sum(-(-k // gran) for k in RAGGED))
    low = -(-case.K_total // gran)
    assert low < need
    D = torch.full((case.G, 64, 128), float("nan"), device=dev())
    for rows in (need - 1, low):
        rc = kg.kg_wgrad_raw(t["A"], t["sa"][:rows].contiguous(), t["B"], t["sb"][:rows].contiguous(),
                             t["C"], D, t["ks"], case.G, 64, 128, case.K_total, gran, dtype,
                             scale_rows=rows)
        assert rc == kg.KG_OK
        assert kg.kg_status() == kg.KG_ERR_SCALE_ROWS
        assert torch.isnan(D).all()
    rc = kg.kg_wgrad_raw(t["A"], t["sa"], t["B"], t["sb"], t["C"], D, t["ks"], case.G, 64, 128,
                         case.K_total, gran, dtype, scale_rows=low - 1)
    assert rc == kg.KG_ERR_SCALE_ROWS  # caught on the host
    # exactly enough rows: the normal result
    run_gpu(case, t, D=D)
    D_ref, bound = oracle_full(case)
    check_close(D, D_ref, bound, "exact scale rows")


def test_fp8_mfma_mode_accumulation_pin():
    """What the fp8-MFMA mode's looser bound rests on, through kg_wgrad: gfx950's fp8
    MFMA adds each group of 8 consecutive products aligned to the largest of them, so
    448 * 448 + 1 * 1 in one group gives 200704, while the default mode (exact bf16
    products, fp32 sums) and the oracle give 200705. One expert of 8 tokens, unit
    scales, every output element the same dot product."""
    say("fp8 mfma pin")
    M = N = 16
    code448, code1 = 0x7E, 0x38  # e4m3fn 448 and 1.0
    A = torch.zeros((8, M), dtype=torch.uint8)
    B = torch.zeros((8, N), dtype=torch.uint8)
    A[0], B[0] = code448, code448
    A[1], B[1] = code1, code1
    sa = torch.ones((1, M), dtype=torch.float32)
    sb = torch.ones((1, N), dtype=torch.float32)
    d = dev()
    ks = torch.tensor([8], dtype=torch.int32, device=d)
    out = {}
    for flags in (0, FAST):
        D = torch.empty((1, M, N), device=d)
        kg.kg_wgrad(A.to(d), sa.to(d), B.to(d), sb.to(d), None, D, ks, 128, F32 | flags)
        assert kg.kg_status() == kg.KG_OK
        out[flags] = D.cpu()
    rc, D_ref, _ = kgref.wgrad(A.numpy(), sa.numpy(), B.numpy(), sb.numpy(), None,
                               np.array([8], np.int32), M, N, 128, F32)
    assert rc == kgref.OK and (D_ref == 200705.0).all()
    assert (out[0] == 200705.0).all()
    assert (out[FAST] == 200704.0).all()


@pytest.mark.parametrize("dtype,gran,flags,ks,M,N,use_ws", [
    (F32, 128, 0, [300, 0, 517], 256, 256, True),       # stream-K with the workspace
    (BF, 128, 0, RAGGED, 320, 272, False),               # kg_wgrad, whole tiles
    (UE8, 32, FAST, [4000, 1234], 512, 1024, True),      # stream-K, fp8-MFMA mode
    (UE8, 32, 0, [0] + [70] * 299, 256, 256, False),     # several rounds, empty expert
])
def test_hip_graph_capture_and_replay(dtype, gran, flags, ks, M, N, use_ws):
    """kg_wgrad (and kg_wgrad_ws) inside a captured HIP graph: the library allocates,
    synchronises and memsets nothing, so a capture holds only its kernel launch (index
    page, "DeepGEMM CUDA Graph Compatibility for Masked Grouped GEMMs"). Three replays,
    with eager work and synchronisations between them, each bit-identical to the eager
    call, within the tolerance of the oracle, and leaving the workspace flags zero."""
    say("graph", dtype, gran, flags, ks, M, N)
    case = small_case(dtype, gran, ks, M, N, seed=41, b_std=1e-3, a_outlier_p=0.01)
    t = to_dev(case)
    ws = kg.new_workspace(dev()) if use_ws else None
    D_eager = torch.full((case.G, M, N), float("nan"), device=dev())
    kg.kg_wgrad(t["A"], t["sa"], t["B"], t["sb"], t["C"], D_eager, t["ks"], gran, dtype | flags,
                workspace=ws)
    assert kg.kg_status() == kg.KG_OK
    D = torch.full_like(D_eager, float("nan"))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            kg.kg_wgrad(t["A"], t["sa"], t["B"], t["sb"], t["C"], D, t["ks"], gran, dtype | flags,
                        workspace=ws)
    torch.cuda.synchronize()
    D_ref, bound = oracle_full(case)
    for rep in range(3):
        D.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert kg.kg_status() == kg.KG_OK
        assert torch.equal(D.view(torch.int32), D_eager.view(torch.int32)), f"replay {rep}"
        assert ws is None or _ws_clean(ws)
        check_close(D, D_ref, bound, f"graph replay {rep}", fast=bool(flags))
    del g


# ---------------------------------------------------------------- full-size workloads

def sampled_check(case, t, D, n=1500, seed=0, fast=False, tile=128):
    """n random outputs of the live experts, tile corners, and one output at a random
    position inside every tile x tile block of every live expert (a tile-indexing or
    scheduling fault that shows only at full size lands in some block)."""
    rng = np.random.default_rng(seed)
    G, M, N = case.G, case.M, case.N
    live = np.nonzero(case.ks > 0)[0]
    sg = rng.choice(live, n)
    sm = rng.integers(0, M, n)
    sn = rng.integers(0, N, n)
    # one per tile x tile block of every live expert
    tm, tn = -(-M // tile), -(-N // tile)
    bg = np.repeat(live, tm * tn)
    bi = np.tile(np.repeat(np.arange(tm), tn), live.size)
    bj = np.tile(np.tile(np.arange(tn), tm), live.size)
    bm = np.minimum(bi * tile + rng.integers(0, tile, bi.size), M - 1)
    bn = np.minimum(bj * tile + rng.integers(0, tile, bj.size), N - 1)
    sg, sm, sn = np.concatenate([sg, bg]), np.concatenate([sm, bm]), np.concatenate([sn, bn])
    # every 16 x 16 sub-tile (the MFMA's output unit) of two 256 x 256 tiles
    for g in rng.choice(live, 2):
        m0 = int(rng.integers(0, max(1, -(-M // 256)))) * 256
        n0 = int(rng.integers(0, max(1, -(-N // 256)))) * 256
        si, sj = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
        sub_m = np.minimum(m0 + 16 * si.ravel() + rng.integers(0, 16, 256), M - 1)
        sub_n = np.minimum(n0 + 16 * sj.ravel() + rng.integers(0, 16, 256), N - 1)
        sg = np.concatenate([sg, np.full(256, g)])
        sm, sn = np.concatenate([sm, sub_m]), np.concatenate([sn, sub_n])
    # corners of tiles and the last row / column of a few experts
    corners = [(0, 0), (M - 1, N - 1), (min(255, M - 1), min(256, N - 1)),
               (min(256, M - 1), min(255, N - 1))]
    cg = [g for g in live[:4] for _ in corners]
    cm = [m for _ in live[:4] for m, _n in corners]
    cn = [n for _ in live[:4] for _m, n in corners]
    sg = np.concatenate([sg, cg]).astype(np.int64)
    sm = np.concatenate([sm, cm]).astype(np.int64)
    sn = np.concatenate([sn, cn]).astype(np.int64)
    assert sg.size == sm.size == sn.size
    h = case.host()
    rc, ref, bound = kgref.wgrad_sampled(h["A"], h["sa"], h["B"], h["sb"], h["C"], h["ks"], M,
                                         N, case.gran_k, case.dtype, sg, sm, sn)
    assert rc == kgref.OK
    got = D[torch.from_numpy(sg).to(D.device), torch.from_numpy(sm).to(D.device),
            torch.from_numpy(sn).to(D.device)].double().cpu().numpy()
    err = np.abs(got - ref)
    lim = (FAST_RTOL if fast else RTOL) * bound + ATOL
    assert (err <= lim).all(), f"{(err > lim).sum()} sampled elements out of tolerance"
    assert np.linalg.norm(got - ref) <= (FAST_FROB if fast else FROB) * np.linalg.norm(ref)
    # every empty expert is bit-exact C (or +0.0)
    for g in np.nonzero(case.ks == 0)[0]:
        if case.C is not None:
            assert torch.equal(D[g].view(torch.int32), t["C"][g].view(torch.int32))
        else:
            assert (D[g].view(torch.int32) == 0).all()


@pytest.mark.parametrize("with_c", [True, False])
def test_wide_precise_tile_for_long_experts(with_c):
    """fp32 scales per 128 tokens, precise mode, experts of 4096+ tokens on average:
    the 256 x 256 tile (KG_PRINT_CONFIG names it), with partial tiles in M and N, an
    empty and a one-token expert, against the full oracle."""
    say("wide precise tile", with_c)
    case = small_case(F32, 128, [9000, 0, 8200, 1], 320, 272, with_c=with_c, seed=17)
    t = to_dev(case)
    D = run_gpu(case, t)
    D_ref, bound = oracle_full(case)
    check_close(D, D_ref, bound, "wide precise tile")
    if case.C is not None:
        assert torch.equal(D[1].view(torch.int32), t["C"][1].view(torch.int32))
    else:
        assert (D[1].view(torch.int32) == 0).all()


def test_wide_precise_tile_bf16_output():
    """The wide precise tile with bf16 C and D: every output within its rounding
    interval of the oracle; the empty expert passes C through bit for bit."""
    say("wide precise tile, bf16 output")
    case = small_case(F32, 128, [9000, 0, 8200, 1], 320, 272, with_c=True, seed=18)
    t = to_dev(case)
    Cb = t["C"].to(torch.bfloat16)
    D = torch.full((case.G, case.M, case.N), float("nan"), dtype=torch.bfloat16, device=dev())
    kg.kg_wgrad(t["A"], t["sa"], t["B"], t["sb"], Cb, D, t["ks"], 128, F32, K_total=case.K_total)
    assert kg.kg_status() == kg.KG_OK
    torch.cuda.synchronize()
    D_ref, bound = oracle_full(case, C=Cb.float().cpu().numpy().astype(np.float32))
    check_bf16_out(D, D_ref, bound, "wide bf16 out")
    assert torch.equal(D[1].view(torch.int16), Cb[1].view(torch.int16))


@pytest.mark.parametrize("dtype,gran", [(F32, 128), (UE8, 32), (BF, 128)])
def test_long_expert_random_data_within_accuracy_envelope(dtype, gran):
    """An expert of 10^6 tokens of N(0, 1) data (the accuracy envelope's stated
    length) beside a short one: sampled outputs within 1e-5 sum |ab| per element and
    1e-5 in Frobenius norm of the oracle."""
    say("long expert random data", dtype, gran)
    ks = [1_000_000, 37]
    case = inputs.make_case("long_random", ks, 64, 96, dtype, gran, with_c=True, seed=41,
                            device="cuda")
    t = to_dev(case)
    D = run_gpu(case, t)
    torch.cuda.synchronize()
    sampled_check(case, t, D, n=400, seed=5, tile=32)
    del D, t, case
    torch.cuda.empty_cache()


# M or N at 2^24 (the largest accepted) and M x N at 2^29 (the largest expert output
# whose byte offsets fit 32 bits): one stage's rows of a 2^24-wide operand span 2^31
# bytes, and the epilogue's offsets in one expert's C reach 2^31.
LIMIT_CASES = [(F32, 128, 1 << 24, 16), (UE8, 32, 1 << 24, 16), (BF, 128, 1 << 24, 16),
               (F32, 128, 16, 1 << 24), (BF, 128, 16, 1 << 24),
               (F32, 128, 1 << 14, 1 << 15), (BF, 128, 1 << 15, 1 << 14)]


@pytest.mark.parametrize("dtype,gran,M,N", LIMIT_CASES)
def test_size_limits_sampled(dtype, gran, M, N):
    """Largest accepted shapes, ragged experts (37 and 91 tokens) around an empty one,
    with C; sampled outputs (tile corners included) in both modes, empty expert bit-exact."""
    say("size limit", dtype, gran, M, N)
    case = inputs.make_case("limit", [37, 0, 91], M, N, dtype, gran, with_c=True, seed=21,
                            device="cuda")
    t = to_dev(case)
    D = torch.empty((case.G, M, N), dtype=torch.float32, device=dev())
    for flags in ((0, FAST) if dtype != BF else (0,)):
        say("size limit run", dtype, gran, M, N, flags)
        run_gpu(case, t, D=D, flags=flags)
        sampled_check(case, t, D, n=600, seed=M ^ N, fast=bool(flags))
    del D, t, case
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["bf16", "zipf_fp8", "ue8m0_many", "local_share"])
def test_full_size_workloads_sampled(name):
    say("full size", name)
    case = inputs.workload(name, device="cuda")
    t = to_dev(case)
    D = torch.empty((case.G, case.M, case.N), dtype=torch.float32, device=dev())
    run_gpu(case, t, D=D)
    assert torch.isfinite(D).all()
    sampled_check(case, t, D)
    if case.dtype != BF:
        say("full size fast", name)
        run_gpu(case, t, D=D, flags=FAST)
        sampled_check(case, t, D, fast=True)
    del D, t, case
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", list(inputs.SINGLE))
def test_single_group_issue_shapes_sampled(name):
    """The issue page's non-grouped 1D1D shapes as one group (ragged N tiles for
    n = 2112, 512-token and 16384-token contractions), in the launch configuration
    bench.py times (with the stream-K workspace)."""
    say("single group", name)
    case = inputs.workload(name, device="cuda")
    t = to_dev(case)
    ws = kg.new_workspace(dev())
    D = torch.empty((case.G, case.M, case.N), dtype=torch.float32, device=dev())
    for flags in (0, FAST):
        kg.kg_wgrad(t["A"], t["sa"], t["B"], t["sb"], None, D, t["ks"], case.gran_k,
                    case.dtype | flags, K_total=case.K_total, workspace=ws)
        assert kg.kg_status() == kg.KG_OK
        torch.cuda.synchronize()
        assert torch.isfinite(D).all()
        sampled_check(case, t, D, fast=bool(flags))
    del D, t, case, ws
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- bf16 output

def check_bf16_out(D_gpu, D_ref, bound, what="", fast=False):
    """D_gpu (bf16) must lie between the oracle's bf16 roundings of D_ref -+ the fp32
    tolerance: the kernel rounds its fp32 sum (within the tolerance of D_ref) once to
    the nearest bf16, and rounding is monotone."""
    tol = (FAST_RTOL if fast else RTOL) * bound + ATOL
    got = kgref.bf16_value(D_gpu.view(torch.int16).cpu().numpy().view(np.uint16))
    lo = kgref.bf16_value(kgref.bf16_round(D_ref - tol))
    hi = kgref.bf16_value(kgref.bf16_round(D_ref + tol))
    bad = (got < lo) | (got > hi)
    assert not bad.any(), (f"{what}: {bad.sum()} bf16 outputs outside their rounding interval, "
                           f"first at {np.unravel_index(np.argmax(bad), bad.shape)}")
    if not fast:
        # most intervals hold a single bf16 value, which the output then equals
        assert (lo == hi).mean() > 0.5, f"{what}: tolerance interval too wide to be a check"


@pytest.mark.parametrize("dtype,gran", [(F32, 128), (F32, 32), (UE8, 32), (UE8, 128), (BF, 128)])
@pytest.mark.parametrize("with_c", [False, True])
@pytest.mark.parametrize("flags", [0, FAST])
def test_bf16_output_variant(dtype, gran, with_c, flags):
    if dtype == BF and flags:
        pytest.skip("the fp8-MFMA flag applies to fp8 inputs")
    ks = [300, 0, 129, 1, 517]
    say("bf16 out", dtype, gran, with_c, flags)
    case = small_case(dtype, gran, ks, 272, 400, with_c=with_c, seed=11)
    t = to_dev(case)
    Cb = None if case.C is None else t["C"].to(torch.bfloat16)
    D = torch.full((case.G, case.M, case.N), float("nan"), dtype=torch.bfloat16, device=dev())
    kg.kg_wgrad(t["A"], t["sa"], t["B"], t["sb"], Cb, D, t["ks"], case.gran_k, case.dtype | flags,
                K_total=case.K_total)
    assert kg.kg_status() == kg.KG_OK
    torch.cuda.synchronize()
    h = case.host()
    C32 = None if Cb is None else Cb.float().cpu().numpy()
    rc, D_ref, bound = kgref.wgrad(h["A"], h["sa"], h["B"], h["sb"], C32, h["ks"], case.M, case.N,
                                   case.gran_k, case.dtype)
    assert rc == kgref.OK
    check_bf16_out(D, D_ref, bound, "bf16 out", fast=bool(flags))
    # the empty expert: C bit for bit, or +0.0
    want = Cb[1] if Cb is not None else torch.zeros_like(D[1])
    assert torch.equal(D[1].view(torch.int16), want.view(torch.int16))


def test_bf16_output_in_place_and_workspace():
    ks = [640, 0, 200]
    case = small_case(F32, 128, ks, 512, 256, with_c=True, seed=5)
    t = to_dev(case)
    Cb = t["C"].to(torch.bfloat16)
    D = Cb.clone()
    ws = kg.new_workspace(dev())
    # in place (C == D), with a workspace that the bf16 output never uses for stream-K
    kg.kg_wgrad(t["A"], t["sa"], t["B"], t["sb"], D, D, t["ks"], case.gran_k, case.dtype,
                K_total=case.K_total, workspace=ws)
    assert kg.kg_status() == kg.KG_OK
    torch.cuda.synchronize()
    h = case.host()
    rc, D_ref, bound = kgref.wgrad(h["A"], h["sa"], h["B"], h["sb"], Cb.float().cpu().numpy(),
                                   h["ks"], case.M, case.N, case.gran_k, case.dtype)
    assert rc == kgref.OK
    check_bf16_out(D, D_ref, bound, "bf16 in place")
    assert torch.equal(D[1].view(torch.int16), Cb[1].view(torch.int16))
    assert (ws[:kg.kg_wgrad_workspace_flag_bytes()] == 0).all()


def test_bf16_output_full_size_default_workload_sampled():
    say("bf16 out full size")
    case = inputs.workload("bf16", device="cuda")
    t = to_dev(case)
    Cb = t["C"].to(torch.bfloat16)
    D = torch.empty((case.G, case.M, case.N), dtype=torch.bfloat16, device=dev())
    kg.kg_wgrad(t["A"], t["sa"], t["B"], t["sb"], Cb, D, t["ks"], case.gran_k, case.dtype,
                K_total=case.K_total, workspace=kg.new_workspace(dev()))
    assert kg.kg_status() == kg.KG_OK
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    live = np.nonzero(case.ks > 0)[0]
    n = 2000
    sg, sm, sn = rng.choice(live, n), rng.integers(0, case.M, n), rng.integers(0, case.N, n)
    h = case.host()
    C32 = Cb.float().cpu().numpy()
    rc, ref, bound = kgref.wgrad_sampled(h["A"], h["sa"], h["B"], h["sb"], C32, h["ks"], case.M,
                                         case.N, case.gran_k, case.dtype, sg, sm, sn)
    assert rc == kgref.OK
    got = D[torch.from_numpy(sg).to(D.device), torch.from_numpy(sm).to(D.device),
            torch.from_numpy(sn).to(D.device)]
    check_bf16_out(got, ref, bound, "bf16 out full size")
    g0 = int(np.nonzero(case.ks == 0)[0][0])
    assert torch.equal(D[g0].view(torch.int16), Cb[g0].view(torch.int16))


def test_f32_scales_per_32_tokens_full_size_sampled():
    """fp32 scales per 32 tokens on the Zipf-routed shape (G = 32, M = 7168, N = 4096,
    65536 tokens), both modes, sampled against the oracle."""
    say("full size f32/32")
    ks = inputs.workload_ks("zipf_fp8")
    case = inputs.make_case("zipf_f32_32", ks, 7168, 4096, F32, 32, with_c=True, seed=0,
                            device="cuda", b_std=1e-3, a_outlier_p=0.01)
    t = to_dev(case)
    D = torch.empty((case.G, case.M, case.N), dtype=torch.float32, device=dev())
    run_gpu(case, t, D=D)
    sampled_check(case, t, D)
    run_gpu(case, t, D=D, flags=FAST)
    sampled_check(case, t, D, fast=True)
    del D, t, case
    torch.cuda.empty_cache()


def test_print_config_switch():
    """KG_PRINT_CONFIG=1 prints each launch's configuration on stderr (read once per
    process, so the call runs in a child process)."""
    import os
    import subprocess
    import sys
    say("KG_PRINT_CONFIG")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "import torch, numpy as np\n"
        "import fp8_grouped_gemm_tn_amd as kg\n"
        "from fp8_grouped_gemm_tn_amd import inputs\n"
        "c = inputs.workload('worked', device='cuda')\n"
        "D = torch.empty((c.G, c.M, c.N), device='cuda')\n"
        "kg.kg_wgrad(c.A, c.sa, c.B, c.sb, None, D, torch.from_numpy(c.ks).cuda(), 128, c.dtype)\n"
        "assert kg.kg_status() == kg.KG_OK\n"
        "w = inputs.make_case('long', [4096], 64, 128, c.dtype, 128, with_c=False, device='cuda')\n"
        "Dw = torch.empty((1, 64, 128), device='cuda')\n"
        "kg.kg_wgrad(w.A, w.sa, w.B, w.sb, None, Dw, torch.from_numpy(w.ks).cuda(), 128, w.dtype)\n"
        "assert kg.kg_status() == kg.KG_OK\n")
    env = dict(os.environ, KG_PRINT_CONFIG="1", PYTHONPATH=root)
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                         timeout=300, cwd=root)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [l for l in res.stderr.splitlines() if l.startswith("kgwgrad:")]
    assert len(lines) == 2, res.stderr[-2000:]
    assert "token-major e4m3+f32 gran 128 precise G 3 M 64 N 128 K_total 104" in lines[0]
    assert "whole tiles" in lines[0] and "tile 256x128" in lines[0]
    # 4096 tokens per expert: the wide precise tile
    assert "precise G 1 M 64 N 128 K_total 4096" in lines[1] and "tile 256x256" in lines[1]

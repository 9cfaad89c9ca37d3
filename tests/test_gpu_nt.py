"""GPU parity of the K-major (NT) entry points (kg_wgrad_nt, kg_wgrad_nt_ws) against
the CPU oracle (kgref.wgrad_nt), with the tolerances of the token-major path
(precise: 1e-5 * sum|ab| + 1e-6 per element, Frobenius 1e-5; fp8-MFMA mode:
2^-10 * sum|ab| + 1e-6, Frobenius 1e-4). The K-major operands sit in row buffers
padded with NaN codes, so a read past an expert's tokens or into the padding shows.
Where both layouts hand every MFMA the same operands (the fp8 kinds, except fp32
scales per 128 tokens), the K-major result in whole-tile mode also equals the
token-major kernel's bit for bit. bf16 and fp32 scales per 128 tokens (both modes)
give the MFMA a step's tokens in another order (16-byte LDS reads per lane), whose
sums round differently: they are held to the oracle's tolerance (and are exact
wherever the sums are, see test_nt_limit_row_length).
"""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_tn_amd as kg
from fp8_grouped_gemm_tn_amd import inputs
from oracle import kgref
from tests.test_gpu_parity import (FAST, FAST_FROB, FAST_RTOL, FROB, RTOL, ATOL, BF, F32, UE8,
                                   check_bf16_out, check_close, dev, say, small_case, to_dev)

pytestmark = pytest.mark.gpu

PATHS = [(F32, 128, 0), (F32, 128, FAST), (F32, 32, 0), (F32, 32, FAST), (UE8, 32, 0),
         (UE8, 32, FAST), (UE8, 128, 0), (UE8, 128, FAST), (BF, 128, 0)]


def same_order(dtype, gran, flags):
    """True where the K-major kernel hands the MFMA a step's tokens in the
    token-major kernel's order (its whole-tile results then have the same bits):
    not for bf16, nor for fp32 scales per 128 tokens (either mode), whose K-major
    fragments come from single 16-byte LDS reads."""
    return dtype != BF and not (dtype == F32 and gran == 128)


def nt_dev(case, t, extra=5):
    """K-major copies of A and B on the device (NaN-padded rows)."""
    return inputs.k_major(t["A"], extra), inputs.k_major(t["B"], extra + 11)


def nt_oracle(case, At, Bt, C="default"):
    h = case.host()
    bits = lambda x: x.view(torch.int16).cpu().numpy().view(np.uint16) \
        if x.dtype == torch.bfloat16 else x.cpu().numpy()
    Ch = h["C"] if isinstance(C, str) else C
    rc, D, bound = kgref.wgrad_nt(bits(At), h["sa"], bits(Bt), h["sb"], Ch, h["ks"], case.M,
                                  case.N, case.gran_k, case.dtype)
    assert rc == kgref.OK
    return D, bound


def run_nt(case, t, At, Bt, flags=0, out=torch.float32, C="default", workspace=None):
    D = torch.full((case.G, case.M, case.N), float("nan"), dtype=out, device=dev())
    Cp = t["C"] if isinstance(C, str) else C
    if Cp is not None and out == torch.bfloat16:
        Cp = Cp.to(torch.bfloat16)
    kg.kg_wgrad_nt(At, t["sa"], Bt, t["sb"], Cp, D, t["ks"], case.gran_k, case.dtype | flags,
                   workspace=workspace)
    assert kg.kg_status() == kg.KG_OK
    torch.cuda.synchronize()
    return D


# unaligned expert starts (45, 176, 179, ...), an empty expert, 1- and 3-token experts,
# tails of every length mod 16, M and N with partial tiles
NT_KS = [45, 0, 131, 3, 300, 1, 17, 128, 143]


@pytest.mark.parametrize("dtype,gran,flags", PATHS)
def test_nt_ragged_matches_oracle_and_token_major(dtype, gran, flags):
    say("nt ragged", dtype, gran, flags)
    case = small_case(dtype, gran, NT_KS, 320, 272, with_c=True, seed=21)
    t = to_dev(case)
    At, Bt = nt_dev(case, t)
    D = run_nt(case, t, At, Bt, flags)
    D_ref, bound = nt_oracle(case, At, Bt)
    check_close(D, D_ref, bound, f"nt {dtype} {gran} {flags}", fast=bool(flags))
    g = NT_KS.index(0)
    assert torch.equal(D[g].cpu().view(torch.int32), case.C[g].view(torch.int32))
    # the token-major kernel on the same matrices: the same bits (fp8 kinds)
    if same_order(dtype, gran, flags):
        D_tn = torch.full_like(D, float("nan"))
        kg.kg_wgrad(t["A"], t["sa"], t["B"], t["sb"], t["C"], D_tn, t["ks"], gran, dtype | flags)
        torch.cuda.synchronize()
        assert torch.equal(D.view(torch.int32), D_tn.view(torch.int32))


def test_nt_wide_precise_tile_for_long_experts():
    """fp32 scales, precise mode, experts of 4096+ tokens on average (the 256 x 256
    tile) with K-major operands, unaligned expert starts and partial tiles: the oracle,
    and the token-major kernel's bits."""
    say("nt wide precise tile")
    ks = [9001, 0, 8200, 3]
    case = small_case(F32, 128, ks, 320, 272, with_c=True, seed=23)
    t = to_dev(case)
    At, Bt = nt_dev(case, t)
    D = run_nt(case, t, At, Bt, 0)
    D_ref, bound = nt_oracle(case, At, Bt)
    check_close(D, D_ref, bound, "nt wide")
    assert torch.equal(D[1].cpu().view(torch.int32), case.C[1].view(torch.int32))
    if same_order(F32, 128, 0):
        D_tn = torch.full_like(D, float("nan"))
        kg.kg_wgrad(t["A"], t["sa"], t["B"], t["sb"], t["C"], D_tn, t["ks"], 128, F32)
        torch.cuda.synchronize()
        assert torch.equal(D.view(torch.int32), D_tn.view(torch.int32))


@pytest.mark.parametrize("dtype,gran,flags", [(F32, 128, 0), (UE8, 32, FAST), (BF, 128, 0)])
def test_nt_every_tail_length(dtype, gran, flags):
    # one expert per tail length 1..16 (mod 16) after an unaligned start, no C
    ks = [7] + [16 * (i % 3) + i for i in range(1, 17)]
    say("nt tails", dtype, gran, flags, ks)
    case = small_case(dtype, gran, ks, 64, 128, with_c=False, seed=23)
    t = to_dev(case)
    At, Bt = nt_dev(case, t, extra=0)
    D = run_nt(case, t, At, Bt, flags, C=None)
    D_ref, bound = nt_oracle(case, At, Bt, C=None)
    check_close(D, D_ref, bound, "nt tails", fast=bool(flags))


@pytest.mark.parametrize("dtype,gran,flags", PATHS)
def test_nt_bf16_output(dtype, gran, flags):
    say("nt bf16 out", dtype, gran, flags)
    case = small_case(dtype, gran, NT_KS, 256, 144, with_c=True, seed=25)
    t = to_dev(case)
    At, Bt = nt_dev(case, t)
    D = run_nt(case, t, At, Bt, flags, out=torch.bfloat16)
    # the oracle's C is the bf16 C the kernel read
    Cb = t["C"].to(torch.bfloat16).float().cpu().numpy()
    D_ref, bound = nt_oracle(case, At, Bt, C=Cb)
    check_bf16_out(D, D_ref, bound, "nt bf16 out", fast=bool(flags))


SPLIT = [([300, 0, 517], 256, 256), ([4001, 1237], 512, 1024), ([0, 1, 33, 0], 256, 512)]


@pytest.mark.parametrize("dtype,gran,flags", [(BF, 128, 0), (F32, 128, 0), (F32, 128, FAST),
                                              (UE8, 32, 0), (F32, 32, 0)])
@pytest.mark.parametrize("ks,M,N", SPLIT)
def test_nt_stream_k(ks, M, N, dtype, gran, flags):
    say("nt stream-K", dtype, gran, flags, ks, M, N)
    case = small_case(dtype, gran, ks, M, N, with_c=True, seed=27)
    t = to_dev(case)
    At, Bt = nt_dev(case, t)
    ws = kg.new_workspace()
    D = run_nt(case, t, At, Bt, flags, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws[:kg.kg_wgrad_workspace_flag_bytes()].count_nonzero()) == 0
    D_ref, bound = nt_oracle(case, At, Bt)
    check_close(D, D_ref, bound, "nt stream-K", fast=bool(flags))
    D2 = run_nt(case, t, At, Bt, flags, workspace=ws)
    assert torch.equal(D.view(torch.int32), D2.view(torch.int32))


def test_nt_worked_example_and_in_place():
    # the how-to page's example shape, accumulated in place (C == D)
    case = inputs.workload("worked")
    t = to_dev(case)
    At, Bt = nt_dev(case, t)
    D = run_nt(case, t, At, Bt, C=None)
    D_ref, bound = nt_oracle(case, At, Bt, C=None)
    check_close(D, D_ref, bound, "nt worked")
    C0 = torch.randn_like(D)
    Di = C0.clone()
    kg.kg_wgrad_nt(At, t["sa"], Bt, t["sb"], Di, Di, t["ks"], 128, case.dtype)
    torch.cuda.synchronize()
    D_ref2, bound2 = nt_oracle(case, At, Bt, C=C0.cpu().numpy())
    check_close(Di, D_ref2, bound2, "nt in place")


def test_nt_ksum_mismatch_is_reported_and_writes_nothing():
    case = small_case(F32, 128, [100, 60], 64, 128, with_c=False, seed=29)
    t = to_dev(case)
    At, Bt = nt_dev(case, t)
    bad = torch.tensor([100, 61], dtype=torch.int32, device=dev())
    D = torch.full((2, 64, 128), float("nan"), device=dev())
    rc = kg.kg_wgrad_nt_raw(At, At.stride(0), t["sa"], Bt, Bt.stride(0), t["sb"], None, D, bad,
                            2, 64, 128, case.K_total, 128, F32)
    assert rc == kg.KG_OK
    assert kg.kg_status() == kg.KG_ERR_KSUM
    assert torch.isnan(D).all()


@pytest.mark.parametrize("name", ["bf16", "zipf_fp8", "ue8m0_many", "local_share"])
def test_nt_full_size_sampled(name):
    """Full-size workloads with K-major operands (the layout transposed on the GPU),
    in the configuration bench.py --nt times, sampled against the oracle on the
    token-major host copies (the K-major arrays are checked to be their transposes)."""
    say("nt full size", name)
    case = inputs.workload(name, device="cuda")
    t = to_dev(case)
    At, Bt = inputs.k_major(t["A"]), inputs.k_major(t["B"])
    assert torch.equal(At, t["A"].t()) and torch.equal(Bt, t["B"].t())
    ws = kg.new_workspace(dev())
    rng = np.random.default_rng(3)
    live = np.nonzero(case.ks > 0)[0]
    n = 1200
    sg = rng.choice(live, n)
    sm = rng.integers(0, case.M, n)
    sn = rng.integers(0, case.N, n)
    sm[:4], sn[:4] = [0, case.M - 1, 255, 256], [0, case.N - 1, 256, 255]
    h = case.host()
    rc, ref, bound = kgref.wgrad_sampled(h["A"], h["sa"], h["B"], h["sb"], h["C"], h["ks"],
                                         case.M, case.N, case.gran_k, case.dtype, sg, sm, sn)
    assert rc == kgref.OK
    idx = [torch.from_numpy(x).to(dev()) for x in (sg, sm, sn)]
    for flags in ((0, FAST) if case.dtype != BF else (0,)):
        say("nt full size", name, flags)
        D = torch.empty((case.G, case.M, case.N), dtype=torch.float32, device=dev())
        kg.kg_wgrad_nt(At, t["sa"], Bt, t["sb"], t["C"], D, t["ks"], case.gran_k,
                       case.dtype | flags, workspace=ws)
        assert kg.kg_status() == kg.KG_OK
        torch.cuda.synchronize()
        assert torch.isfinite(D).all()
        got = D[idx[0], idx[1], idx[2]].double().cpu().numpy()
        lim = (FAST_RTOL if flags else RTOL) * bound + ATOL
        assert (np.abs(got - ref) <= lim).all()
        assert np.linalg.norm(got - ref) <= (FAST_FROB if flags else FROB) * np.linalg.norm(ref)
        for g in np.nonzero(case.ks == 0)[0]:
            if case.C is not None:
                assert torch.equal(D[g].view(torch.int32), t["C"][g].view(torch.int32))
            else:
                assert (D[g].view(torch.int32) == 0).all()
        del D
    del At, Bt, t, case, ws
    torch.cuda.empty_cache()


def test_nt_edge_cases():
    # every expert empty (K_total = 0, rows of length 0): D = C bit for bit
    say("nt all empty")
    case = small_case(F32, 128, [0, 0, 0], 64, 64, seed=31)
    t = to_dev(case)
    At = torch.zeros((64, 16), dtype=torch.uint8, device=dev())[:, :0]  # row stride 16
    Bt = torch.zeros((64, 16), dtype=torch.uint8, device=dev())[:, :0]
    D = torch.full((3, 64, 64), float("nan"), device=dev())
    kg.kg_wgrad_nt(At, t["sa"], Bt, t["sb"], t["C"], D, t["ks"], 128, F32)
    assert kg.kg_status() == kg.KG_OK
    torch.cuda.synchronize()
    assert torch.equal(D.cpu().view(torch.int32), case.C.view(torch.int32))
    # one expert of one token, the smallest tile (bf16: the 8-element row unit)
    say("nt single token 16x16")
    case = small_case(BF, 128, [1], 16, 16, seed=32)
    t = to_dev(case)
    At, Bt = nt_dev(case, t, extra=0)
    D = run_nt(case, t, At, Bt)
    D_ref, bound = nt_oracle(case, At, Bt)
    check_close(D, D_ref, bound, "nt 16x16")
    # 1024 experts, UE8M0 per 32 tokens, many tiny and empty experts
    say("nt G = 1024")
    rng = np.random.default_rng(33)
    ks = rng.integers(0, 40, 1024).astype(np.int32)
    ks[rng.choice(1024, 100, replace=False)] = 0
    case = small_case(UE8, 32, ks, 16, 32, seed=33)
    t = to_dev(case)
    At, Bt = nt_dev(case, t)
    D = run_nt(case, t, At, Bt, FAST)
    D_ref, bound = nt_oracle(case, At, Bt)
    check_close(D, D_ref, bound, "nt G=1024", fast=True)


# ---------------------------------------------------------------- size limits

@pytest.mark.parametrize("dtype,gran,flags", [(F32, 128, 0), (F32, 128, FAST), (BF, 128, 0)])
def test_nt_limit_m_2p24_bit_identical(dtype, gran, flags):
    """M = 2^24 (the largest accepted), ragged experts around an empty one, with C:
    sampled outputs match the oracle, and the fp8 kinds equal the token-major kernel
    bit for bit (whole tiles)."""
    from tests.test_gpu_parity import sampled_check
    M, N = 1 << 24, 16
    say("nt limit M", dtype, gran, flags)
    case = inputs.make_case("limit", [37, 0, 91], M, N, dtype, gran, with_c=True, seed=23,
                            device="cuda")
    t = to_dev(case)
    At, Bt = nt_dev(case, t)
    D = run_nt(case, t, At, Bt, flags)
    if same_order(dtype, gran, flags):
        D_tn = torch.full_like(D, float("nan"))
        kg.kg_wgrad(t["A"], t["sa"], t["B"], t["sb"], t["C"], D_tn, t["ks"], gran, dtype | flags)
        torch.cuda.synchronize()
        assert torch.equal(D.view(torch.int32), D_tn.view(torch.int32))
        del D_tn
    del At, Bt
    sampled_check(case, t, D, n=300, seed=1, fast=bool(flags))
    del D, t, case
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,K", [(F32, 16_000_000), (BF, 8_000_000)])
def test_nt_limit_row_length(dtype, K):
    """K-major rows near the longest accepted (256 rows of one load span just under
    2^32 bytes), three experts (one empty) over K tokens, M and N below one tile:
    with bf16 (exact sums) whole tiles equal the token-major kernel bit for bit (fp32
    scales per 128 tokens take another token order there); whole tiles and stream-K
    (with the workspace) match the oracle on sampled outputs. The bf16 operands are
    ternary with integer C, so that its experts of 2.7M and 5.3M tokens have exact
    fp32 sums and the outputs must equal the oracle's exactly (with N(0, 1) data,
    fp32 accumulation over 5.3M tokens is ~2e-5 off in relative Frobenius norm)."""
    from tests.test_gpu_parity import sampled_check
    ks = [K // 3 + 1, 0, K - K // 3 - 1]
    say("nt limit rows", dtype, K)
    if dtype == BF:
        case = inputs.make_ternary_bf16_case("long", ks, 32, 48, seed=24, device="cuda")
    else:
        case = inputs.make_case("long", ks, 32, 48, dtype, 128, with_c=True, seed=24,
                                device="cuda")
    t = to_dev(case)
    At, Bt = nt_dev(case, t)
    elt = 2 if dtype == BF else 1
    assert 256 * At.stride(0) * elt <= 0xFFFFFF00 and 256 * Bt.stride(0) * elt <= 0xFFFFFF00
    h = case.host()
    rng = np.random.default_rng(4)
    sg = np.array([0, 2] * 20, np.int64)
    sm = np.concatenate([rng.integers(0, 32, 36), [0, 31, 0, 31]]).astype(np.int64)
    sn = np.concatenate([rng.integers(0, 48, 36), [0, 47, 47, 0]]).astype(np.int64)
    rc, ref, bound = kgref.wgrad_sampled(h["A"], h["sa"], h["B"], h["sb"], h["C"], h["ks"], 32,
                                         48, 128, dtype, sg, sm, sn)
    assert rc == kgref.OK

    def check(D):
        got = D[torch.from_numpy(sg).to(D.device), torch.from_numpy(sm).to(D.device),
                torch.from_numpy(sn).to(D.device)].double().cpu().numpy()
        if dtype == BF:
            assert np.array_equal(got, ref), f"{(got != ref).sum()} sampled outputs not exact"
        else:
            assert (np.abs(got - ref) <= RTOL * bound + ATOL).all()
            assert np.linalg.norm(got - ref) <= FROB * np.linalg.norm(ref)
        assert torch.equal(D[1].view(torch.int32), t["C"][1].view(torch.int32))

    D = run_nt(case, t, At, Bt)
    if same_order(dtype, 128, 0) or dtype == BF:
        # the same token order, or exact sums (ternary bf16): the token-major bits
        D_tn = torch.full_like(D, float("nan"))
        kg.kg_wgrad(t["A"], t["sa"], t["B"], t["sb"], t["C"], D_tn, t["ks"], 128, dtype)
        torch.cuda.synchronize()
        assert torch.equal(D.view(torch.int32), D_tn.view(torch.int32))
        del D_tn
    check(D)
    ws = kg.new_workspace(dev())
    say("nt limit rows stream-K", dtype, K)
    D = run_nt(case, t, At, Bt, workspace=ws)
    check(D)
    del D, At, Bt, ws, t, case
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,gran,flags", PATHS)
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("split", [False, True])
def test_nt_canaries_every_path(dtype, gran, flags, out, split):
    """K-major: nothing written outside D (guard regions), two runs give the same
    bits; whole tiles of the fp8 kinds equal the token-major kernel's bits in the same
    mode; bf16 and stream-K match the oracle."""
    from tests.test_gpu_parity import guarded
    say("nt canaries", dtype, gran, flags, out, split)
    case = small_case(dtype, gran, [129, 0, 400, 1], 272, 144, seed=17)
    t = to_dev(case)
    At, Bt = nt_dev(case, t)
    C = t["C"] if out == torch.float32 else t["C"].to(torch.bfloat16)
    ws = kg.new_workspace(dev()) if split else None
    D, intact = guarded((case.G, case.M, case.N), out)
    runs = []
    for _ in range(2):
        kg.kg_wgrad_nt(At, t["sa"], Bt, t["sb"], C, D, t["ks"], gran, dtype | flags, workspace=ws)
        assert kg.kg_status() == kg.KG_OK
        torch.cuda.synchronize()
        assert intact(), "a write landed outside D"
        runs.append(D.clone())
    assert torch.equal(runs[0].view(torch.int16), runs[1].view(torch.int16))
    if split:
        # stream-K cuts ranges in stages, whose length may differ between the layouts
        D_ref, bound = nt_oracle(case, At, Bt, C=C.float().cpu().numpy())
        if out == torch.float32:
            check_close(D, D_ref, bound, "nt canaries", fast=bool(flags))
        else:
            check_bf16_out(D, D_ref, bound, "nt canaries", fast=bool(flags))
        return
    if not same_order(dtype, gran, flags):
        D_ref, bound = nt_oracle(case, At, Bt, C=C.float().cpu().numpy())
        if out == torch.float32:
            check_close(D, D_ref, bound, "nt canaries", fast=bool(flags))
        else:
            check_bf16_out(D, D_ref, bound, "nt canaries", fast=bool(flags))
        return
    D_tn = torch.empty_like(D)
    kg.kg_wgrad(t["A"], t["sa"], t["B"], t["sb"], C, D_tn, t["ks"], gran, dtype | flags)
    torch.cuda.synchronize()
    assert torch.equal(D.view(torch.int16), D_tn.view(torch.int16))

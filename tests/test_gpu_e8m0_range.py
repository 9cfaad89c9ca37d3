"""GPU parity of the UE8M0 (power-of-two scale) paths across the exponent range.

The scale byte e means 2^(e - 127) and is applied to each block's partial sum (GitHub
issue "Is DeepGEMM directly applicable to backward in training?", qijiaxing
2025-03-26; index page, "UE8M0 Format in DeepGEMM ..."). Exponent pairs whose scale
product 2^(ea + eb - 254) is moderate must give the oracle's result to the usual
tolerance even when each exponent alone is extreme: (0, 254), (254, 0), (1, 253),
(250, 5), (5, 250) and (127, 127), per block, per expert, with ragged tails and tiles
that run past M and N.
"""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_tn_amd as kg
from fp8_grouped_gemm_tn_amd import inputs
from oracle import kgref

pytestmark = pytest.mark.gpu

UE8 = kg.KG_E4M3_UE8M0
FAST = kg.KG_FLAG_FP8_MFMA
RTOL, ATOL, FROB = 1e-5, 1e-6, 1e-5
FAST_RTOL, FAST_FROB = 2.0 ** -10, 1e-4

PAIRS = [(0, 254), (254, 0), (1, 253), (253, 1), (250, 5), (5, 250), (127, 127), (20, 240)]


def say(*a):
    print("[case]", *a, flush=True)


def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def with_exponents(case, ea_rows, eb_rows):
    """The case with its scale exponents replaced: ea_rows [nblk, M], eb_rows [nblk, N]
    (uint8 numpy arrays). The fp8 codes stay as quantised."""
    case.sa = torch.from_numpy(np.ascontiguousarray(ea_rows, dtype=np.uint8))
    case.sb = torch.from_numpy(np.ascontiguousarray(eb_rows, dtype=np.uint8))
    return case


def jittered(rng, base, shape):
    """Exponents base + {-2 .. 2}, kept in [0, 254]."""
    return np.clip(base + rng.integers(-2, 3, shape), 0, 254).astype(np.uint8)


def run_and_check(case, flags, what):
    d = dev()
    t = {k: (None if v is None else v.to(d)) for k, v in
         dict(A=case.A, B=case.B, sa=case.sa, sb=case.sb, C=case.C).items()}
    ks = torch.from_numpy(case.ks).to(d)
    D = torch.full((case.G, case.M, case.N), float("nan"), device=d)
    kg.kg_wgrad(t["A"], t["sa"], t["B"], t["sb"], t["C"], D, ks, case.gran_k, UE8 | flags,
                K_total=case.K_total)
    assert kg.kg_status() == kg.KG_OK
    torch.cuda.synchronize()
    h = case.host()
    rc, D_ref, bound = kgref.wgrad(h["A"], h["sa"], h["B"], h["sb"], h["C"], h["ks"], case.M,
                                   case.N, case.gran_k, UE8)
    assert rc == kgref.OK
    assert np.isfinite(D_ref).all()
    got = D.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    fast = bool(flags)
    err = np.abs(got - D_ref)
    lim = (FAST_RTOL if fast else RTOL) * bound + ATOL
    bad = err > lim
    assert not bad.any(), (f"{what}: {bad.sum()} elements out of tolerance, worst "
                           f"{(err - lim).max():.3e} at {np.unravel_index(np.argmax(err - lim), err.shape)}")
    rel = np.linalg.norm(got - D_ref) / np.linalg.norm(D_ref)
    assert rel <= (FAST_FROB if fast else FROB), f"{what}: Frobenius {rel:.3e}"


@pytest.mark.parametrize("gran", [32, 128])
@pytest.mark.parametrize("ea0,eb0", PAIRS)
@pytest.mark.parametrize("flags", [0, FAST])
def test_extreme_exponent_pairs(ea0, eb0, gran, flags):
    """One exponent pair (+-2) for every block and channel; ragged experts (an empty
    one, a one-token one), M and N with partial tiles."""
    say("e8m0 range", ea0, eb0, gran, flags)
    ks = [300, 0, 129, 1, 517, 64]
    case = inputs.make_case("e8range", ks, 272, 400, UE8, gran, with_c=True, seed=31)
    rng = np.random.default_rng(ea0 * 1000 + eb0 + gran)
    nblk = case.sa.shape[0]
    with_exponents(case, jittered(rng, ea0, (nblk, case.M)), jittered(rng, eb0, (nblk, case.N)))
    run_and_check(case, flags, f"pair ({ea0}, {eb0}) gran {gran}")


@pytest.mark.parametrize("gran", [32, 128])
@pytest.mark.parametrize("flags", [0, FAST])
def test_exponent_pairs_change_per_block(gran, flags):
    """Consecutive blocks take different pairs, so that stages in the fold window,
    stages that need a shift and shifts of both signs alternate inside one expert."""
    say("e8m0 range per block", gran, flags)
    ks = [1000, 77, 0, 611]
    case = inputs.make_case("e8range_blocks", ks, 256, 512, UE8, gran, with_c=True, seed=32)
    rng = np.random.default_rng(gran + 7)
    nblk = case.sa.shape[0]
    ea = np.empty((nblk, case.M), np.uint8)
    eb = np.empty((nblk, case.N), np.uint8)
    for r in range(nblk):
        a0, b0 = PAIRS[r % len(PAIRS)]
        ea[r] = jittered(rng, a0, case.M)
        eb[r] = jittered(rng, b0, case.N)
    with_exponents(case, ea, eb)
    run_and_check(case, flags, f"per-block pairs gran {gran}")


@pytest.mark.parametrize("gran", [32, 128])
@pytest.mark.parametrize("flags", [0, FAST])
def test_exponent_rows_and_columns_spread(gran, flags):
    """Within one block the rows' exponents span 0 .. 60 and the columns' 194 .. 254:
    both leave the fold window, one shift brings them all inside, and every product's
    scale 2^(ea + eb - 254) lies in 2^-60 .. 2^60."""
    say("e8m0 range spread", gran, flags)
    ks = [260, 130]
    case = inputs.make_case("e8range_spread", ks, 256, 256, UE8, gran, with_c=False, seed=33)
    nblk = case.sa.shape[0]
    ea = np.tile((np.arange(case.M) * 60 // (case.M - 1)).astype(np.uint8), (nblk, 1))
    eb = np.tile((194 + np.arange(case.N) * 60 // (case.N - 1)).astype(np.uint8), (nblk, 1))
    with_exponents(case, ea, eb)
    run_and_check(case, flags, "spread")


def test_unfoldable_spread_is_reported():
    """Rows of one block at exponents 0 and 254 side by side: no single shift keeps both
    in bf16's normal range, so the default mode reports KG_ERR_SCALE_RANGE (the result
    is not checked: its terms reach 2^127)."""
    say("e8m0 unfoldable")
    case = inputs.make_case("e8range_bad", [200], 64, 128, UE8, 32, with_c=False, seed=34)
    nblk = case.sa.shape[0]
    ea = np.tile(np.where(np.arange(case.M) % 2 == 0, 0, 254).astype(np.uint8), (nblk, 1))
    eb = np.full((nblk, case.N), 127, np.uint8)
    with_exponents(case, ea, eb)
    d = dev()
    D = torch.empty((1, case.M, case.N), device=d)
    kg.kg_wgrad(case.A.to(d), case.sa.to(d), case.B.to(d), case.sb.to(d), None, D,
                torch.from_numpy(case.ks).to(d), 32, UE8, K_total=case.K_total)
    assert kg.kg_status() == kg.KG_ERR_SCALE_RANGE
    assert kg.kg_status() == kg.KG_OK  # cleared

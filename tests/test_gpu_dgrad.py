"""GPU parity of the M-grouped dgrad GEMM (kg_dgrad, through the C ABI) against the
CPU oracle.

Precise mode: |D - D_ref| <= 1e-5 * sum_k |a w| + 1e-6 element-wise and Frobenius
1e-5 (fp32 accumulation of exact fp8 products, as for the K-grouped GEMM); fp8-MFMA
mode: 2^-10 * sum|a w| + 1e-6 and Frobenius 1e-4 (the fp8 MFMA's accumulation, see
kgwgrad.h). bf16 output: between the oracle's bf16 roundings of D_ref -+ the
tolerance.
"""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_tn_amd as kg
from fp8_grouped_gemm_tn_amd import inputs
from oracle import kgref

pytestmark = pytest.mark.gpu

FAST = kg.KG_FLAG_FP8_MFMA
RTOL, ATOL, FROB = 1e-5, 1e-6, 1e-5
FAST_RTOL, FAST_FROB = 2.0 ** -10, 1e-4


def say(*a):
    print("[case]", *a, flush=True)


def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def to_dev(c):
    d = dev()
    return dict(A=c.A.to(d), sa=c.sa.to(d), W=c.W.to(d), sw=c.sw.to(d),
                ms=torch.from_numpy(c.ms).to(d))


def run(c, t, flags=0, out=torch.float32, D=None):
    if D is None:
        D = torch.full((c.M_total, c.N), float("nan"), dtype=out, device=dev())
    kg.kg_dgrad(t["A"], t["sa"], t["W"], t["sw"], D, t["ms"], flags)
    assert kg.kg_status() == kg.KG_OK
    torch.cuda.synchronize()
    return D


def check(D, ref, bound, fast=False, what=""):
    tol = (FAST_RTOL if fast else RTOL) * bound + ATOL
    if D.dtype == torch.bfloat16:
        got = kgref.bf16_value(D.view(torch.int16).cpu().numpy().view(np.uint16))
        lo = kgref.bf16_value(kgref.bf16_round(ref - tol))
        hi = kgref.bf16_value(kgref.bf16_round(ref + tol))
        bad = (got < lo) | (got > hi)
        assert not bad.any(), f"{what}: {bad.sum()} bf16 outputs outside their rounding interval"
        return
    got = D.double().cpu().numpy()
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bad = err > tol
    assert not bad.any(), (f"{what}: {bad.sum()} out of tolerance, worst {(err - tol).max():.3e} "
                           f"at {np.unravel_index(np.argmax(err - tol), err.shape)}")
    nrm = np.linalg.norm(ref)
    if nrm > 0:
        assert np.linalg.norm(got - ref) <= (FAST_FROB if fast else FROB) * nrm


@pytest.mark.parametrize("ms,N,K", [
    ([300, 0, 1, 517, 256], 384, 512),   # ragged experts, an empty one, several m-tiles
    ([40], 128, 128),                    # one partial tile, one stage
    ([0, 257, 0], 256, 1024),            # 257 rows: a full tile and a one-row tile
    ([300, 0, 1, 517, 256], 768, 384),   # N a multiple of 256: the wide tile (fp8 MFMA)
    # the largest group count of the wide tile (512), one more, and the most groups
    # (1024): 0-5 rows per expert, every seventh one empty
    ([0 if i % 7 == 0 else i % 5 + 1 for i in range(512)], 256, 128),
    ([0 if i % 7 == 0 else i % 5 + 1 for i in range(513)], 256, 128),
    ([0 if i % 7 == 0 else i % 5 + 1 for i in range(1024)], 128, 256),
])
@pytest.mark.parametrize("flags", [0, FAST])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_dgrad_matches_oracle(ms, N, K, flags, out):
    say("dgrad", ms, N, K, flags, out)
    c = inputs.make_dgrad_case("t", ms, N, K, seed=3)
    t = to_dev(c)
    D = run(c, t, flags, out)
    h = c.host()
    rc, ref, bound = kgref.dgrad(h["A"], h["sa"], h["W"], h["sw"], h["ms"], c.N, c.K)
    assert rc == kgref.OK
    check(D, ref, bound, fast=bool(flags), what="dgrad")


def test_dgrad_writes_only_its_rows_and_is_deterministic():
    c = inputs.make_dgrad_case("t", [129, 0, 300], 256, 384, seed=5)
    t = to_dev(c)
    guard = 64
    big = torch.full((c.M_total + 2 * guard, c.N), float("nan"), device=dev())
    D = big[guard:guard + c.M_total]
    run(c, t, D=D)
    assert torch.isnan(big[:guard]).all() and torch.isnan(big[guard + c.M_total:]).all()
    assert torch.isfinite(D).all()
    D2 = run(c, t)
    assert torch.equal(D.view(torch.int32), D2.view(torch.int32))


def test_dgrad_ms_mismatch_is_reported_and_writes_nothing():
    c = inputs.make_dgrad_case("t", [100, 60], 128, 256, seed=1)
    t = to_dev(c)
    bad = torch.tensor([100, 61], dtype=torch.int32, device=dev())
    D = torch.full((c.M_total, c.N), float("nan"), device=dev())
    rc = kg.kg_dgrad_raw(t["A"], t["sa"], t["W"], t["sw"], D, bad, 2, c.N, c.K, c.M_total, 0)
    assert rc == kg.KG_OK
    assert kg.kg_status() == kg.KG_ERR_KSUM
    assert torch.isnan(D).all()
    assert kg.kg_status() == kg.KG_OK


def test_dgrad_power_of_two_scales_bit_exact():
    c = inputs.make_dgrad_case("t", [200, 77], 256, 512, seed=9)
    t = to_dev(c)
    D = run(c, t)
    t2 = dict(t, sa=t["sa"] * 4.0, sw=t["sw"] * 0.5)
    D2 = run(c, t2)
    assert torch.equal(D2, D * 2.0)


@pytest.mark.parametrize("name", inputs.DGRAD_WORKLOADS)
def test_dgrad_full_size_sampled(name):
    say("dgrad full size", name)
    c = inputs.dgrad_workload(name, device="cuda")
    t = to_dev(c)
    h = {k: (v.cpu().numpy() if torch.is_tensor(v) else v) for k, v in
         dict(A=c.A, sa=c.sa, W=c.W, sw=c.sw, ms=c.ms).items()}
    rng = np.random.default_rng(0)
    n = 1500
    st = rng.integers(0, c.M_total, n)
    sn = rng.integers(0, c.N, n)
    # the first and last row of every non-empty expert, first and last column
    off = np.concatenate([[0], np.cumsum(c.ms)])
    edges = [r for g in range(c.G) if c.ms[g] > 0 for r in (off[g], off[g + 1] - 1)]
    st = np.concatenate([st, edges, edges])
    sn = np.concatenate([sn, np.zeros(len(edges), np.int64), np.full(len(edges), c.N - 1)])
    rc, ref, bound = kgref.dgrad_sampled(h["A"], h["sa"], h["W"], h["sw"], h["ms"], c.N, c.K,
                                         st, sn)
    assert rc == kgref.OK
    for flags, out in ((0, torch.float32), (0, torch.bfloat16), (FAST, torch.bfloat16)):
        say("dgrad full size", name, flags, out)
        D = torch.empty((c.M_total, c.N), dtype=out, device=dev())
        run(c, t, flags, D=D)
        got = D[torch.from_numpy(st).to(D.device), torch.from_numpy(sn).to(D.device)]
        check(got, ref, bound, fast=bool(flags), what=name)
        del D
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- size limits

def sampled(c, t, flags, out, n, seed):
    h = {k: (v.cpu().numpy() if torch.is_tensor(v) else v) for k, v in
         dict(A=c.A, sa=c.sa, W=c.W, sw=c.sw, ms=c.ms).items()}
    rng = np.random.default_rng(seed)
    st = rng.integers(0, c.M_total, n)
    sn = rng.integers(0, c.N, n)
    off = np.concatenate([[0], np.cumsum(c.ms)])
    edges = [r for g in range(c.G) if c.ms[g] > 0 for r in (off[g], off[g + 1] - 1)]
    st = np.concatenate([st, edges, edges])
    sn = np.concatenate([sn, np.zeros(len(edges), np.int64), np.full(len(edges), c.N - 1)])
    rc, ref, bound = kgref.dgrad_sampled(h["A"], h["sa"], h["W"], h["sw"], h["ms"], c.N, c.K,
                                         st, sn)
    assert rc == kgref.OK
    D = run(c, t, flags, out=out)
    got = D[torch.from_numpy(st).to(D.device), torch.from_numpy(sn).to(D.device)]
    check(got, ref, bound, fast=bool(flags), what=f"limit N={c.N} K={c.K}")


# N = 2097024 is the largest multiple of 128 whose 256-row output tile has byte
# offsets below 2^31 (2096896, a multiple of 256, takes the fp8-MFMA mode's wide
# tile); K = 8388480 the largest whose 256-row activation tile does.
@pytest.mark.parametrize("ms,N,K,flags,out", [
    ([37, 0, 91, 1], 2097024, 128, 0, torch.float32),
    ([37, 0, 91, 1], 2097024, 128, FAST, torch.bfloat16),
    ([37, 0, 91, 1], 2096896, 128, FAST, torch.float32),
    ([37, 0, 91], 128, 8388480, 0, torch.bfloat16),
    ([37, 0, 91], 256, 8388480, FAST, torch.float32),
])
def test_dgrad_size_limits_sampled(ms, N, K, flags, out):
    say("dgrad limit", ms, N, K, flags, out)
    c = inputs.make_dgrad_case("limit", ms, N, K, seed=25, device="cuda")
    t = to_dev(c)
    sampled(c, t, flags, out, n=60, seed=N ^ K)
    del t, c
    torch.cuda.empty_cache()


def draw_dgrad(seed):
    """A seeded random dgrad configuration: expert count, rows per expert (long, short
    with empty and one-row experts, or heavy-tailed), N and K (multiples of 128), mode
    and output type."""
    rng = np.random.default_rng(2000 + seed)
    G = int(rng.integers(1, 65))
    style = rng.integers(0, 3)
    if style == 0:
        ms = rng.integers(0, 700, G)
    elif style == 1:
        ms = rng.choice([0, 1, 2, 63, 64, 65, 127, 128, 129, 255, 256, 257], G)
    else:
        ms = np.minimum((rng.pareto(1.2, G) * 50).astype(np.int64), 2000)
    ms[rng.random(G) < 0.15] = 0
    N = 128 * int(rng.integers(1, 7))
    K = 128 * int(rng.integers(1, 9))
    flags = FAST if rng.random() < 0.4 else 0
    out = torch.bfloat16 if rng.random() < 0.5 else torch.float32
    return [int(m) for m in ms], N, K, flags, out


@pytest.mark.parametrize("seed", range(24))
def test_dgrad_random_configuration(seed):
    ms, N, K, flags, out = draw_dgrad(seed)
    say("dgrad random", seed, "G", len(ms), "rows", sum(ms), N, K, flags, out)
    c = inputs.make_dgrad_case("t", ms, N, K, seed=seed)
    t = to_dev(c)
    D = run(c, t, flags, out)
    h = c.host()
    rc, ref, bound = kgref.dgrad(h["A"], h["sa"], h["W"], h["sw"], h["ms"], c.N, c.K)
    assert rc == kgref.OK
    check(D, ref, bound, fast=bool(flags), what=f"dgrad random {seed}")

"""Seeded random configurations through kg_wgrad against the oracle: every input kind
and scale granularity, both math modes, with and without C, with and without the
stream-K workspace, fp32 or bf16 output, over random expert counts (empty and
one-token experts included), token counts and M, N (multiples of 16, partial tiles).
Each configuration is drawn from its seed alone, so a failure names a case that can
be rerun by itself."""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_tn_amd as kg
from fp8_grouped_gemm_tn_amd import inputs
from tests.test_gpu_parity import (FAST, check_bf16_out, check_close, dev, oracle_full, say,
                                   to_dev)

pytestmark = pytest.mark.gpu

KINDS = [(kg.KG_E4M3_F32SCALE, 128), (kg.KG_E4M3_F32SCALE, 32), (kg.KG_E4M3_UE8M0, 32),
         (kg.KG_E4M3_UE8M0, 128), (kg.KG_BF16, 128)]


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    dtype, gran = KINDS[seed % len(KINDS)]
    G = int(rng.integers(1, 41))
    style = rng.integers(0, 3)
    if style == 0:    # a few long experts
        ks = rng.integers(0, 1200, G)
    elif style == 1:  # many short ones, some empty or of one token
        ks = rng.choice([0, 1, 2, 31, 32, 33, 127, 128, 129, 255], G)
    else:             # heavy-tailed
        ks = np.minimum((rng.pareto(1.2, G) * 60).astype(np.int64), 3000)
    ks[rng.random(G) < 0.15] = 0
    M = 16 * int(rng.integers(1, 40))
    N = 16 * int(rng.integers(1, 40))
    with_c = bool(rng.random() < 0.5)
    fast = dtype != kg.KG_BF16 and bool(rng.random() < 0.4)
    use_ws = bool(rng.random() < 0.5)
    bf16_out = not use_ws and bool(rng.random() < 0.25)
    return dict(dtype=dtype, gran=gran, ks=[int(k) for k in ks], M=M, N=N, with_c=with_c,
                fast=fast, use_ws=use_ws, bf16_out=bf16_out)


@pytest.mark.parametrize("seed", range(40))
def test_random_configuration(seed):
    cfg = draw(seed)
    say("random config", seed, {k: v for k, v in cfg.items() if k != "ks"}, "G", len(cfg["ks"]),
        "tokens", sum(cfg["ks"]))
    case = inputs.make_case("random", cfg["ks"], cfg["M"], cfg["N"], cfg["dtype"], cfg["gran"],
                            with_c=cfg["with_c"], seed=seed)
    t = to_dev(case)
    flags = FAST if cfg["fast"] else 0
    ws = kg.new_workspace(dev()) if cfg["use_ws"] else None
    if cfg["bf16_out"]:
        C = None if case.C is None else t["C"].to(torch.bfloat16)
        D = torch.full((case.G, case.M, case.N), float("nan"), dtype=torch.bfloat16, device=dev())
    else:
        C = t["C"]
        D = torch.full((case.G, case.M, case.N), float("nan"), dtype=torch.float32, device=dev())
    kg.kg_wgrad(t["A"], t["sa"], t["B"], t["sb"], C, D, t["ks"], case.gran_k,
                case.dtype | flags, K_total=case.K_total, workspace=ws)
    assert kg.kg_status() == kg.KG_OK
    torch.cuda.synchronize()
    if cfg["bf16_out"]:
        Ch = None if C is None else C.float().cpu().numpy().astype(np.float32)
        D_ref, bound = oracle_full(case, C=Ch)
        check_bf16_out(D, D_ref, bound, f"random {seed}", fast=cfg["fast"])
    else:
        D_ref, bound = oracle_full(case)
        check_close(D, D_ref, bound, f"random {seed}", fast=cfg["fast"])
    if ws is not None:
        # the workspace's arrival counters are back at zero after the call
        nflag = kg.kg_wgrad_workspace_flag_bytes()
        assert (ws[:nflag] == 0).all()


@pytest.mark.parametrize("seed", range(100, 124))
def test_random_configuration_k_major(seed):
    """The same random draws through kg_wgrad_nt: K-major copies of A and B in rows
    padded (by a seeded amount) with NaN codes, so that a read past an expert's tokens
    or into the padding shows, against the oracle's K-major entry."""
    from tests.test_gpu_nt import nt_oracle, run_nt
    cfg = draw(seed)
    say("random k-major config", seed, {k: v for k, v in cfg.items() if k != "ks"}, "G",
        len(cfg["ks"]), "tokens", sum(cfg["ks"]))
    case = inputs.make_case("random", cfg["ks"], cfg["M"], cfg["N"], cfg["dtype"], cfg["gran"],
                            with_c=cfg["with_c"], seed=seed)
    t = to_dev(case)
    rng = np.random.default_rng(seed)
    At = inputs.k_major(t["A"], int(rng.integers(0, 40)))
    Bt = inputs.k_major(t["B"], int(rng.integers(0, 40)))
    flags = FAST if cfg["fast"] else 0
    ws = kg.new_workspace(dev()) if cfg["use_ws"] else None
    out = torch.bfloat16 if cfg["bf16_out"] else torch.float32
    D = run_nt(case, t, At, Bt, flags, out=out, workspace=ws)
    if cfg["bf16_out"]:
        Ch = None if case.C is None else t["C"].to(torch.bfloat16).float().cpu().numpy()
        D_ref, bound = nt_oracle(case, At, Bt, C=Ch)
        check_bf16_out(D, D_ref, bound, f"random k-major {seed}", fast=cfg["fast"])
    else:
        D_ref, bound = nt_oracle(case, At, Bt)
        check_close(D, D_ref, bound, f"random k-major {seed}", fast=cfg["fast"])
    if ws is not None:
        assert (ws[:kg.kg_wgrad_workspace_flag_bytes()] == 0).all()

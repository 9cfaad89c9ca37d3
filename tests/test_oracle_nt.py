"""Pins of the oracle's K-major (NT) entry (kgref.wgrad_nt).

The issue page ("Is DeepGEMM directly applicable to backward in training?",
qijiaxing 2025-04-03) writes the weight gradient dw = dy^t x as a GEMM whose
operands are dy^t [h_out, tokens] and x^t [h_in, tokens]: the token (contraction)
index is the contiguous one. The how-to page names the SM90 entry point of this
layout k_grouped_fp8_gemm_nt_contiguous ("API Entry Points", FAQ on NT and TN).
Here At [M, ld] and Bt [N, ld] hold token t of channel m at At[m, t], ld >= K_total
(columns past K_total are padding). The pins index the K-major arrays directly with
exact rationals, so a transposed operand or a read of the padding fails them.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import kgref
from tests.test_oracle import BF, F32, UE8, e8m0_def, rand_problem, torch_bf16, torch_e4m3


def k_major(X, ld, junk):
    """[K, C] token-major -> [C, ld] K-major, padding columns set to `junk`."""
    K, Cn = X.shape
    out = np.full((Cn, ld), junk, dtype=X.dtype)
    out[:, :K] = X.T
    return out


def exact_nt(At, sa, Bt, sb, C, ks, M, N, gran, dtype):
    """The definition read straight from the K-major arrays: D[g, m, n] = C + sum over
    the group's tokens t of dec(At[m, t]) SA(m) dec(Bt[n, t]) SB(n)."""
    dec = torch_bf16 if dtype == BF else torch_e4m3
    Ad, Bd = dec(At), dec(Bt)
    G = len(ks)
    out = np.zeros((G, M, N), dtype=object)
    t0 = 0
    srow = 0
    for g in range(G):
        for m in range(M):
            for n in range(N):
                s = Fraction(float(C[g, m, n])) if C is not None else Fraction(0)
                for i in range(int(ks[g])):
                    r = srow + i // gran
                    if dtype == F32:
                        sc = Fraction(float(sa[r, m])) * Fraction(float(sb[r, n]))
                    elif dtype == UE8:
                        sc = Fraction(e8m0_def(sa[r, m])) * Fraction(e8m0_def(sb[r, n]))
                    else:
                        sc = Fraction(1)
                    s += Fraction(float(Ad[m, t0 + i])) * Fraction(float(Bd[n, t0 + i])) * sc
                out[g, m, n] = s
        t0 += int(ks[g])
        srow += (int(ks[g]) + gran - 1) // gran
    return out


@pytest.mark.parametrize("dtype,gran", [(F32, 128), (F32, 32), (UE8, 32), (UE8, 128), (BF, 128)])
def test_nt_brute_force_exact_with_junk_padding(dtype, gran):
    rng = np.random.default_rng(31 + 7 * dtype + gran)
    ks = np.array([45, 0, 131, 3], np.int32)  # unaligned group starts, an empty group
    M, N = 4, 6
    p = rand_problem(rng, ks, M, N, dtype, gran)
    K = int(ks.sum())
    junk = 0x7FC0 if dtype == BF else 0x7F  # NaN codes: a read of the padding shows
    At = k_major(p["A"], K + 13, junk)
    Bt = k_major(p["B"], K + 5, junk)
    rc, D, bound = kgref.wgrad_nt(At, p["sa"], Bt, p["sb"], p["C"], ks, M, N, gran, dtype)
    assert rc == kgref.OK
    ref = exact_nt(At, p["sa"], Bt, p["sb"], p["C"], ks, M, N, gran, dtype)
    for g in range(len(ks)):
        for m in range(M):
            for n in range(N):
                err = abs(Fraction(D[g, m, n]) - ref[g, m, n])
                assert err <= Fraction(1e-14) * Fraction(bound[g, m, n] + 1.0), (g, m, n)


def test_nt_worked_example_shape_and_sampled():
    # the how-to page's example shape: ks = [32, 45, 27], M = 64, N = 128
    rng = np.random.default_rng(5)
    ks = np.array([32, 45, 27], np.int32)
    M, N = 64, 128
    p = rand_problem(rng, ks, M, N, F32, 128, with_c=False)
    At, Bt = k_major(p["A"], 112, 0x7F), k_major(p["B"], 104, 0x7F)
    rc, D, _ = kgref.wgrad_nt(At, p["sa"], Bt, p["sb"], None, ks, M, N, 128, F32)
    assert rc == kgref.OK and np.isfinite(D).all()
    # three samples against the exact definition
    for g, m, n in [(0, 0, 0), (1, 63, 127), (2, 17, 90)]:
        t0 = int(ks[:g].sum())
        s = Fraction(0)
        for i in range(int(ks[g])):
            s += (Fraction(float(torch_e4m3(At[m, t0 + i]))) * Fraction(float(p["sa"][g, m]))
                  * Fraction(float(torch_e4m3(Bt[n, t0 + i]))) * Fraction(float(p["sb"][g, n])))
        assert abs(Fraction(D[g, m, n]) - s) <= Fraction(1e-12) * (abs(s) + 1)
    sg, sm, sn = np.array([0, 1, 2]), np.array([0, 63, 17]), np.array([0, 127, 90])
    rc, v, _ = kgref.wgrad_sampled_nt(At, p["sa"], Bt, p["sb"], None, ks, M, N, 128, F32,
                                      sg, sm, sn)
    assert rc == kgref.OK
    np.testing.assert_array_equal(v, D[sg, sm, sn])


def test_nt_rejects_short_rows():
    with pytest.raises(ValueError):
        kgref.token_major(np.zeros((4, 10), np.uint8), 11)

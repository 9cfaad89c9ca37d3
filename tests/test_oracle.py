"""Pins of the CPU oracle against facts other than the oracle itself.

Each test names what fixes the expected value: the e4m3fn format definition
(golden landmarks) and torch's own float8/bf16 conversions; exact rational
arithmetic (brute force with Python Fractions on tiny inputs); numpy's fp64
matrix product for the special case G = 1 with unit scales; closed forms; and
invariants of the definition (K-split, permutations, power-of-two scaling,
transposition, empty-group passthrough, linearity in C).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import kgref

HERE = os.path.dirname(os.path.abspath(__file__))
F32, UE8, BF = kgref.E4M3_F32SCALE, kgref.E4M3_UE8M0, kgref.BF16


def golden(name):
    with open(os.path.join(HERE, "golden", name)) as f:
        return json.load(f)


# ------------------------------------------------------------ independent decoders

def torch_e4m3(byte_array):
    t = torch.from_numpy(np.asarray(byte_array, np.uint8).copy())
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_bf16(bits):
    t = torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16).copy())
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def e8m0_def(e):
    return math.ldexp(1.0, int(e) - 127)


# ------------------------------------------------------------ random inputs

def rand_fp8(rng, shape):
    x = rng.integers(0, 256, size=shape, dtype=np.uint8)
    x[(x & 0x7F) == 0x7F] = 0x38  # keep NaN codes out
    return x


def rand_problem(rng, ks, M, N, dtype, gran, with_c=True):
    ks = np.asarray(ks, np.int32)
    K = int(ks.sum())
    nb = int(sum((int(k) + gran - 1) // gran for k in ks))
    if dtype == BF:
        A = torch.randn(K, M, dtype=torch.float32).to(torch.bfloat16)
        B = torch.randn(K, N, dtype=torch.float32).to(torch.bfloat16)
        A = A.view(torch.int16).numpy().view(np.uint16).copy()
        B = B.view(torch.int16).numpy().view(np.uint16).copy()
        sa = sb = None
    else:
        A, B = rand_fp8(rng, (K, M)), rand_fp8(rng, (K, N))
        if dtype == F32:
            sa = np.exp(rng.normal(0, 2, (nb, M))).astype(np.float32)
            sb = np.exp(rng.normal(0, 2, (nb, N))).astype(np.float32)
        else:
            sa = rng.integers(117, 138, (nb, M)).astype(np.uint8)
            sb = rng.integers(117, 138, (nb, N)).astype(np.uint8)
    C = rng.normal(0, 1, (ks.size, M, N)).astype(np.float32) if with_c else None
    return dict(A=A, sa=sa, B=B, sb=sb, C=C, ks=ks)


def run(p, M, N, gran, dtype, **kw):
    rc, D, bound = kgref.wgrad(p["A"], p["sa"], p["B"], p["sb"], p["C"], p["ks"], M, N,
                               gran, dtype, **kw)
    assert rc == kgref.OK
    return D, bound


# ------------------------------------------------------------ decoders

def test_e4m3_landmarks_from_format_definition():
    g = golden("e4m3fn_landmarks.json")
    for code, val in g["values"].items():
        assert kgref.e4m3(int(code, 16)) == val, code
    for code in g["nan"]:
        assert math.isnan(kgref.e4m3(int(code, 16)))
    nz = kgref.e4m3(int(g["negative_zero"], 16))
    assert nz == 0.0 and math.copysign(1.0, nz) < 0


def test_e4m3_all_codes_match_torch_and_are_monotone():
    codes = np.arange(256, dtype=np.uint8)
    ours = np.array([kgref.e4m3(c) for c in codes])
    ref = torch_e4m3(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    pos = ours[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(ours[0x80:0xFF], -ours[:0x7F])


def test_e8m0_and_bf16_decoders():
    assert kgref.e8m0(127) == 1.0 and kgref.e8m0(128) == 2.0
    assert kgref.e8m0(0) == 2.0 ** -127 and kgref.e8m0(254) == 2.0 ** 127
    assert math.isnan(kgref.e8m0(255))
    bits = np.arange(0, 65536, 97, dtype=np.uint16)
    ours = np.array([kgref.bf16(b) for b in bits])
    ref = torch_bf16(bits)
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


# ------------------------------------------------------------ offsets and checks

def test_worked_shape_offsets_golden():
    g = golden("worked_shape.json")
    off, boff = kgref.offsets(g["ks"], 128)
    assert off.tolist() == g["off"] and boff.tolist() == g["boff_gran128"]
    off, boff = kgref.offsets(g["ks"], 32)
    assert off.tolist() == g["off"] and boff.tolist() == g["boff_gran32"]
    assert 2 * g["K_total"] * g["M"] * g["N"] == g["flops"]


def test_validation_codes():
    v = kgref.validate
    assert v([1, 2], 2, 16, 16, 3, 128, F32) == kgref.OK
    assert v([1, 2], 2, 16, 16, 4, 128, F32) == kgref.ERR_KSUM
    assert v([1, -1], 2, 16, 16, 0, 128, F32) == kgref.ERR_KSUM
    assert v([1, 2], 2, 16, 16, 3, 64, F32) == kgref.ERR_GRAN
    assert v([1, 2], 2, 16, 16, 3, 64, BF) == kgref.OK
    assert v([1, 2], 2, 16, 16, 3, 128, 7) == kgref.ERR_DTYPE
    assert v([1, 2], 2, -1, 16, 3, 128, F32) == kgref.ERR_SHAPE
    assert v([], 0, 16, 16, 0, 32, UE8) == kgref.OK
    p = rand_problem(np.random.default_rng(0), [3, 4], 8, 8, F32, 128)
    rc, _, _ = kgref.wgrad(p["A"], p["sa"], p["B"], p["sb"], p["C"], p["ks"], 8, 8, 128, F32,
                           K_total=8)
    assert rc == kgref.ERR_KSUM


# ------------------------------------------------------------ brute force, exact

def exact_reference(p, M, N, gran, dtype):
    """Plain definition with exact rationals: every token dequantised on its own,
    no blocking; the scale row of token t is found by walking the groups."""
    ks = p["ks"]
    G = ks.size
    if dtype == BF:
        Ad, Bd = torch_bf16(p["A"]), torch_bf16(p["B"])
    else:
        Ad, Bd = torch_e4m3(p["A"]), torch_e4m3(p["B"])
    out = np.zeros((G, M, N), dtype=object)
    t = 0
    srow = 0
    for g in range(G):
        acc = [[Fraction(0)] * N for _ in range(M)]
        for i in range(int(ks[g])):
            r = srow + i // gran
            for m in range(M):
                if dtype == F32:
                    sa = Fraction(float(p["sa"][r, m]))
                elif dtype == UE8:
                    sa = Fraction(e8m0_def(p["sa"][r, m]))
                else:
                    sa = Fraction(1)
                a = Fraction(float(Ad[t + i, m])) * sa
                if a == 0:
                    continue
                for n in range(N):
                    if dtype == F32:
                        sb = Fraction(float(p["sb"][r, n]))
                    elif dtype == UE8:
                        sb = Fraction(e8m0_def(p["sb"][r, n]))
                    else:
                        sb = Fraction(1)
                    acc[m][n] += a * Fraction(float(Bd[t + i, n])) * sb
        for m in range(M):
            for n in range(N):
                c = Fraction(float(p["C"][g, m, n])) if p["C"] is not None else Fraction(0)
                out[g, m, n] = c + acc[m][n]
        t += int(ks[g])
        srow += (int(ks[g]) + gran - 1) // gran
    return out


@pytest.mark.parametrize("dtype,gran", [(F32, 128), (F32, 32), (UE8, 32), (UE8, 128), (BF, 128)])
def test_brute_force_exact_tiny(dtype, gran):
    rng = np.random.default_rng(11 + dtype * 10 + gran)
    ks = [37, 0, 150, 5]
    M, N = 5, 7
    p = rand_problem(rng, ks, M, N, dtype, gran)
    D, bound = run(p, M, N, gran, dtype)
    ref = exact_reference(p, M, N, gran, dtype)
    for g in range(len(ks)):
        for m in range(M):
            for n in range(N):
                err = abs(Fraction(D[g, m, n]) - ref[g, m, n])
                tol = Fraction(1e-14) * Fraction(bound[g, m, n] + 1.0)
                assert err <= tol, (g, m, n, float(err), bound[g, m, n])


def test_block_partial_is_exact_in_fp64():
    """One block, unit scales, no C: the oracle's fp64 result equals the exact
    integer sum (e4m3fn values are multiples of 2^-9) bit for bit."""
    rng = np.random.default_rng(5)
    ks = np.array([128], np.int32)
    M, N = 6, 9
    A, B = rand_fp8(rng, (128, M)), rand_fp8(rng, (128, N))
    sa, sb = np.ones((1, M), np.float32), np.ones((1, N), np.float32)
    rc, D, _ = kgref.wgrad(A, sa, B, sb, None, ks, M, N, 128, F32)
    assert rc == kgref.OK
    Ai = (torch_e4m3(A) * 512).astype(np.int64)
    Bi = (torch_e4m3(B) * 512).astype(np.int64)
    assert np.array_equal(Ai.astype(np.float64), torch_e4m3(A) * 512)
    exact = Ai.T @ Bi  # int64, units of 2^-18
    assert np.array_equal(D[0], exact.astype(np.float64) / 2.0 ** 18)


def test_bound_is_sum_of_abs_products():
    rng = np.random.default_rng(6)
    ks = [70, 200]
    M, N = 4, 3
    p = rand_problem(rng, ks, M, N, F32, 128, with_c=False)
    _, bound = run(p, M, N, 128, F32)
    p_abs = dict(p)
    p_abs["A"] = p["A"] & 0x7F
    p_abs["B"] = p["B"] & 0x7F
    D_abs, _ = run(p_abs, M, N, 128, F32)
    np.testing.assert_allclose(bound, D_abs, rtol=1e-14)


# ------------------------------------------------------------ special cases

def test_single_group_unit_scales_is_numpy_matmul():
    rng = np.random.default_rng(7)
    K, M, N = 300, 24, 40
    A, B = rand_fp8(rng, (K, M)), rand_fp8(rng, (K, N))
    nb = (K + 127) // 128
    sa, sb = np.ones((nb, M), np.float32), np.ones((nb, N), np.float32)
    rc, D, _ = kgref.wgrad(A, sa, B, sb, None, [K], M, N, 128, F32)
    assert rc == kgref.OK
    ref = torch_e4m3(A).T @ torch_e4m3(B)
    np.testing.assert_allclose(D[0], ref, rtol=1e-13, atol=1e-12)


def test_single_group_bf16_is_numpy_matmul_plus_c():
    rng = np.random.default_rng(8)
    p = rand_problem(rng, [333], 16, 48, BF, 128)
    D, _ = run(p, 16, 48, 128, BF)
    ref = torch_bf16(p["A"]).T @ torch_bf16(p["B"]) + p["C"][0].astype(np.float64)
    np.testing.assert_allclose(D[0], ref, rtol=1e-13, atol=1e-12)


def test_closed_form_all_ones():
    ks = np.array([32, 45, 0, 27, 300], np.int32)
    K, M, N = int(ks.sum()), 8, 16
    A = np.full((K, M), 0x38, np.uint8)
    B = np.full((K, N), 0x38, np.uint8)
    for gran in (32, 128):
        nb = int(sum((k + gran - 1) // gran for k in ks))
        sa, sb = np.ones((nb, M), np.float32), np.ones((nb, N), np.float32)
        C = np.arange(ks.size * M * N, dtype=np.float32).reshape(ks.size, M, N)
        rc, D, _ = kgref.wgrad(A, sa, B, sb, C, ks, M, N, gran, F32)
        assert rc == kgref.OK
        for g, k in enumerate(ks):
            assert np.array_equal(D[g], C[g] + float(k))
        e = np.full((nb, M), 127, np.uint8), np.full((nb, N), 127, np.uint8)
        rc, D2, _ = kgref.wgrad(A, e[0], B, e[1], None, ks, M, N, gran, UE8)
        assert rc == kgref.OK
        for g, k in enumerate(ks):
            assert np.all(D2[g] == float(k))


def test_closed_form_one_hot_rows():
    """A[t] is the unit vector e_{m_t}: D[g][m] = sum of b(t,.) over the tokens of
    g routed to m (scaled by each token's block scales)."""
    rng = np.random.default_rng(9)
    ks = np.array([130, 64, 1], np.int32)
    K, M, N = int(ks.sum()), 8, 5
    mt = rng.integers(0, M, K)
    A = np.zeros((K, M), np.uint8)
    A[np.arange(K), mt] = 0x38
    B = rand_fp8(rng, (K, N))
    gran = 128
    nb = int(sum((k + gran - 1) // gran for k in ks))
    sa = np.ones((nb, M), np.float32)
    sb = np.exp(rng.normal(0, 1, (nb, N))).astype(np.float32)
    rc, D, _ = kgref.wgrad(A, sa, B, sb, None, ks, M, N, gran, F32)
    assert rc == kgref.OK
    Bd = torch_e4m3(B)
    t = 0
    r = 0
    for g, k in enumerate(ks):
        exp = np.zeros((M, N))
        for i in range(k):
            exp[mt[t + i]] += Bd[t + i] * sb[r + i // gran].astype(np.float64)
        np.testing.assert_allclose(D[g], exp, rtol=1e-14, atol=0)
        t += k
        r += (k + gran - 1) // gran


# ------------------------------------------------------------ invariants

@pytest.mark.parametrize("dtype,gran", [(F32, 128), (UE8, 32), (F32, 32)])
def test_k_split_at_block_boundary(dtype, gran):
    rng = np.random.default_rng(12)
    ks = np.array([50, 3 * gran + 17, 9], np.int32)
    M, N = 12, 20
    p = rand_problem(rng, ks, M, N, dtype, gran)
    D, _ = run(p, M, N, gran, dtype)
    # split group 1 after 2 blocks: scale rows stay where they are
    ks2 = np.array([50, 2 * gran, gran + 17, 9], np.int32)
    C2 = np.concatenate([p["C"][:2], np.zeros((1, M, N), np.float32), p["C"][2:]])
    p2 = dict(p, ks=ks2, C=C2)
    D2, _ = run(p2, M, N, gran, dtype)
    np.testing.assert_array_equal(D2[0], D[0])
    np.testing.assert_allclose(D2[1] + D2[2], D[1], rtol=1e-13, atol=1e-12)
    np.testing.assert_array_equal(D2[3], D[2])


def test_bf16_k_split_anywhere():
    rng = np.random.default_rng(13)
    p = rand_problem(rng, [211], 8, 8, BF, 128)
    D, _ = run(p, 8, 8, 128, BF)
    p2 = dict(p, ks=np.array([77, 134], np.int32),
              C=np.stack([p["C"][0], np.zeros((8, 8), np.float32)]))
    D2, _ = run(p2, 8, 8, 128, BF)
    np.testing.assert_allclose(D2[0] + D2[1], D[0], rtol=1e-13, atol=1e-12)


@pytest.mark.parametrize("dtype,gran", [(F32, 128), (UE8, 32)])
def test_token_permutation_within_block_is_bit_exact(dtype, gran):
    rng = np.random.default_rng(14)
    ks = np.array([2 * gran + 11, gran], np.int32)
    M, N = 10, 6
    p = rand_problem(rng, ks, M, N, dtype, gran)
    D, _ = run(p, M, N, gran, dtype)
    perm = np.arange(int(ks.sum()))
    starts = [0, gran, 2 * gran, 2 * gran + 11, 3 * gran + 11]
    for a, b in zip(starts[:-1], starts[1:]):
        perm[a:b] = a + rng.permutation(b - a)
    p2 = dict(p, A=p["A"][perm], B=p["B"][perm])
    D2, _ = run(p2, M, N, gran, dtype)
    np.testing.assert_array_equal(D2, D)


def test_block_permutation_with_scale_rows():
    rng = np.random.default_rng(15)
    gran = 128
    ks = np.array([4 * gran + 9], np.int32)
    M, N = 7, 9
    p = rand_problem(rng, ks, M, N, F32, gran)
    D, _ = run(p, M, N, gran, F32)
    order = [2, 0, 3, 1]  # full blocks only; the tail block stays last
    tok = np.concatenate([np.arange(b * gran, (b + 1) * gran) for b in order]
                         + [np.arange(4 * gran, 4 * gran + 9)])
    rows = np.array(order + [4])
    p2 = dict(p, A=p["A"][tok], B=p["B"][tok], sa=p["sa"][rows], sb=p["sb"][rows])
    D2, _ = run(p2, M, N, gran, F32)
    np.testing.assert_allclose(D2, D, rtol=1e-14, atol=1e-13)


def test_empty_groups_pass_c_through_bit_exact():
    rng = np.random.default_rng(16)
    ks = np.array([0, 40, 0, 0], np.int32)
    M, N = 8, 8
    p = rand_problem(rng, ks, M, N, F32, 128)
    D, _ = run(p, M, N, 128, F32)
    for g in (0, 2, 3):
        np.testing.assert_array_equal(D[g], p["C"][g].astype(np.float64))
    p0 = dict(p, C=None)
    D0, _ = run(p0, M, N, 128, F32)
    for g in (0, 2, 3):
        assert np.all(D0[g] == 0.0) and not np.any(np.signbit(D0[g]))


@pytest.mark.parametrize("j", [-3, 1, 5])
def test_power_of_two_scale_is_bit_exact(j):
    rng = np.random.default_rng(17)
    ks = np.array([129, 64, 300], np.int32)
    M, N = 6, 10
    p = rand_problem(rng, ks, M, N, F32, 128, with_c=False)
    D, _ = run(p, M, N, 128, F32)
    p2 = dict(p, sa=(p["sa"] * np.float32(2.0 ** j)).astype(np.float32))
    D2, _ = run(p2, M, N, 128, F32)
    np.testing.assert_array_equal(D2, D * 2.0 ** j)
    q = rand_problem(rng, ks, M, N, UE8, 32, with_c=False)
    E, _ = run(q, M, N, 32, UE8)
    q2 = dict(q, sb=(q["sb"].astype(np.int32) + j).astype(np.uint8))
    E2, _ = run(q2, M, N, 32, UE8)
    np.testing.assert_array_equal(E2, E * 2.0 ** j)


def test_linear_in_c():
    rng = np.random.default_rng(18)
    ks = np.array([100, 28], np.int32)
    p = rand_problem(rng, ks, 8, 8, F32, 32)
    D, _ = run(p, 8, 8, 32, F32)
    D0, _ = run(dict(p, C=None), 8, 8, 32, F32)
    np.testing.assert_allclose(D - D0, p["C"], rtol=0, atol=1e-12 * (1 + np.abs(D0).max()))


@pytest.mark.parametrize("dtype,gran", [(F32, 128), (UE8, 32), (BF, 128)])
def test_swapping_operands_transposes_d(dtype, gran):
    rng = np.random.default_rng(19)
    ks = np.array([45, 140], np.int32)
    M, N = 6, 11
    p = rand_problem(rng, ks, M, N, dtype, gran, with_c=False)
    D, _ = run(p, M, N, gran, dtype)
    q = dict(p, A=p["B"], B=p["A"], sa=p["sb"], sb=p["sa"])
    Dt, _ = run(q, N, M, gran, dtype)
    np.testing.assert_array_equal(Dt, np.transpose(D, (0, 2, 1)))


# ------------------------------------------------------------ oracle plumbing

def test_sampled_equals_full_and_threads_do_not_matter():
    rng = np.random.default_rng(20)
    ks = np.array([200, 0, 77], np.int32)
    M, N = 16, 32
    p = rand_problem(rng, ks, M, N, F32, 128)
    D1, b1 = run(p, M, N, 128, F32, threads=1)
    D8, b8 = run(p, M, N, 128, F32, threads=8)
    np.testing.assert_array_equal(D1, D8)
    np.testing.assert_array_equal(b1, b8)
    sg = rng.integers(0, 3, 50)
    sm = rng.integers(0, M, 50)
    sn = rng.integers(0, N, 50)
    rc, v, b = kgref.wgrad_sampled(p["A"], p["sa"], p["B"], p["sb"], p["C"], ks, M, N, 128,
                                   F32, sg, sm, sn)
    assert rc == kgref.OK
    np.testing.assert_array_equal(v, D1[sg, sm, sn])
    np.testing.assert_array_equal(b, b1[sg, sm, sn])
    # sub-ranges of groups and rows
    rc, Dp, _ = kgref.wgrad(p["A"], p["sa"], p["B"], p["sb"], p["C"], ks, M, N, 128, F32,
                            g_range=(1, 3), m_range=(4, 9))
    assert rc == kgref.OK
    np.testing.assert_array_equal(Dp, D1[1:3, 4:9])


# ---------------------------------------------------------------- bf16 output rounding

# (value, code) from the bf16 format: 1 = 0x3F80 and the spacing just above 1 is
# 2^-7; 1 + 2^-8 is the midpoint of 0x3F80 and 0x3F81 (tie -> even 0x3F80);
# 1 + 3*2^-8 is the midpoint of 0x3F81 and 0x3F82 (tie -> even 0x3F82); the
# smallest subnormal is 2^-133 (0x0001), its half is a tie with zero (-> 0x0000),
# 1.5 * 2^-133 ties between 0x0001 and 0x0002 (-> 0x0002); the midpoint between the
# largest finite value (2 - 2^-7) * 2^127 = 0x7F7F and 2^128 ties to the even
# code, which is 2^128 itself, i.e. infinity (0x7F80).
BF16_LANDMARKS = [
    (1.0, 0x3F80), (-2.5, 0xC020), (1 + 2.0 ** -8, 0x3F80), (1 + 3 * 2.0 ** -8, 0x3F82),
    (1 + 2.0 ** -8 + 2.0 ** -40, 0x3F81), (2.0 ** -133, 0x0001), (2.0 ** -134, 0x0000),
    (1.5 * 2.0 ** -133, 0x0002), (2.0 ** 128 * (1 - 2.0 ** -9), 0x7F80),
    ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F), (-0.0, 0x8000), (0.0, 0x0000),
    (float("inf"), 0x7F80), (float("-inf"), 0xFF80),
]


@pytest.mark.parametrize("v,code", BF16_LANDMARKS)
def test_bf16_round_landmarks(v, code):
    assert kgref.lib().kgref_bf16_round(v) == code


def test_bf16_round_nan():
    c = kgref.lib().kgref_bf16_round(float("nan"))
    assert (c & 0x7F80) == 0x7F80 and (c & 0x007F) != 0


def test_bf16_round_matches_torch_on_binary32_inputs():
    # binary32 inputs round once either way, so torch's float32 -> bfloat16
    # conversion (round to nearest even) is an independent check
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(20000) * 1e-39).astype(np.float32),        # subnormals
        (rng.standard_normal(20000) * 5e37).astype(np.float32),
        # exact midpoints between neighbouring bf16 values
        ((rng.integers(0x0001, 0x7F7F, 20000).astype(np.uint32) << 16) | 0x8000).view(np.float32),
    ])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = kgref.bf16_round(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_bf16_round_once_from_fp64_not_through_binary32():
    # just above a midpoint by less than binary32's resolution: binary32 rounding
    # first would land on the midpoint and then go to the even code
    base = (np.arange(0x3F00, 0x4100, 2, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    spacing = 2.0 ** (np.floor(np.log2(base)) - 7)
    v = base + spacing / 2 + spacing * 2.0 ** -30
    got = kgref.bf16_round(v)
    even = (base.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(got, even + 1)
    assert np.array_equal(kgref.bf16_round(base + spacing / 2), even)


def test_bf16_round_is_monotone_and_nearest():
    rng = np.random.default_rng(3)
    v = np.sort(rng.standard_normal(100000) * 10.0)
    c = kgref.bf16_round(v)
    val = kgref.bf16_value(c)
    assert (np.diff(val) >= 0).all()
    # nearest: no bf16 value lies strictly closer (neighbour codes one step away)
    pos = v > 0
    up = kgref.bf16_value(np.where(pos, c + 1, c - 1).astype(np.uint16))
    dn = kgref.bf16_value(np.where(pos, c - 1, c + 1).astype(np.uint16))
    err = np.abs(val - v)
    assert (err <= np.abs(up - v)).all() and (err <= np.abs(dn - v)).all()

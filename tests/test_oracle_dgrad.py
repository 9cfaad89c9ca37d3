"""Pins of the CPU oracle for the M-grouped data-gradient GEMM (dgrad).

What the oracle computes (GitHub issue "Is DeepGEMM directly applicable to backward
in training?": the backward pass of a GEMM is two GEMMs; activations carry 1x128
scales, weights 128x128 block scales): for token t of expert g and column n,
D[t][n] = sum over 128-channel blocks kb of SA[kb][t] * SW[g][kb][n/128] *
sum_{k in kb} dec(A[t][k]) dec(W[g][k][n]).

Each pin below checks the oracle against something other than its own formula:
exact rational arithmetic, the separately pinned K-grouped oracle, numpy's matmul,
closed forms and invariants.
"""
from fractions import Fraction

import numpy as np
import pytest

from fp8_grouped_gemm_tn_amd import inputs
from oracle import kgref

ONE = 0x38  # e4m3fn 1.0


def dec_table():
    return np.array([kgref.lib().kgref_e4m3(b) for b in range(256)], np.float64)


def small(ms, N=256, K=384, seed=0):
    c = inputs.make_dgrad_case("t", ms, N, K, seed=seed)
    return c, c.host()


def run(h, N, K):
    rc, D, bound = kgref.dgrad(h["A"], h["sa"], h["W"], h["sw"], h["ms"], N, K)
    assert rc == kgref.OK
    return D, bound


def test_exact_rational_brute_force():
    # per-element dequantisation and one exact sum per output, no blocking
    c, h = small([3, 0, 2, 1], N=256, K=256, seed=3)
    D, bound = run(h, c.N, c.K)
    tab = [Fraction(float(v)) if np.isfinite(v) else None for v in dec_table()]  # NaN codes unused
    off = np.concatenate([[0], np.cumsum(c.ms)])
    rng = np.random.default_rng(0)
    for _ in range(120):
        t = int(rng.integers(0, c.M_total))
        n = int(rng.integers(0, c.N))
        g = int(np.searchsorted(off, t, side="right") - 1)
        while c.ms[g] == 0:
            g += 1
        s = Fraction(0)
        sabs = Fraction(0)
        for k in range(c.K):
            a = tab[h["A"][t, k]] * Fraction(float(h["sa"][k // 128, t]))
            w = tab[h["W"][g, k, n]] * Fraction(float(h["sw"][g, k // 128, n // 128]))
            s += a * w
            sabs += abs(a) * abs(w)
        assert abs(D[t, n] - float(s)) <= 1e-12 * float(sabs) + 1e-300
        assert abs(bound[t, n] - float(sabs)) <= 1e-12 * float(sabs)


def test_each_row_equals_the_k_grouped_oracle():
    # the K-grouped oracle (pinned on its own) computes one dgrad row when the
    # contraction channels play the role of tokens: A_w [K, 1] = dy row, B_w = W[g],
    # per-block scales sa_w[kb] = SA[kb][t], sb_w[kb][n] = SW[g][kb][n/128]
    c, h = small([4, 0, 3], N=256, K=384, seed=5)
    D, _ = run(h, c.N, c.K)
    off = np.concatenate([[0], np.cumsum(c.ms)])
    nkb = c.K // 128
    for t in range(c.M_total):
        g = int(np.searchsorted(off, t, side="right") - 1)
        while c.ms[g] == 0:
            g += 1
        A_w = np.ascontiguousarray(h["A"][t].reshape(c.K, 1))
        sa_w = np.ascontiguousarray(h["sa"][:, t].reshape(nkb, 1))
        B_w = np.ascontiguousarray(h["W"][g])
        sb_w = np.ascontiguousarray(np.repeat(h["sw"][g], 128, axis=1))
        rc, Dw, _ = kgref.wgrad(A_w, sa_w, B_w, sb_w, None, np.array([c.K], np.int32), 1, c.N,
                                128, kgref.E4M3_F32SCALE)
        assert rc == kgref.OK
        assert np.array_equal(Dw[0, 0], D[t])


def test_unit_scales_single_expert_is_numpy_matmul():
    c, h = small([37], N=384, K=512, seed=2)
    h["sa"][:] = 1.0
    h["sw"][:] = 1.0
    D, _ = run(h, c.N, c.K)
    tab = dec_table()
    ref = tab[h["A"]] @ tab[h["W"][0]]
    assert np.allclose(D, ref, rtol=1e-13, atol=1e-9)


def test_closed_form_all_ones():
    ms = [2, 0, 3]
    K, N = 256, 128
    A = np.full((5, K), ONE, np.uint8)
    W = np.full((3, K, N), ONE, np.uint8)
    sa = np.ones((K // 128, 5), np.float32)
    sw = np.ones((3, K // 128, N // 128), np.float32)
    sw[2] = 0.5
    rc, D, bound = kgref.dgrad(A, sa, W, sw, np.array(ms, np.int32), N, K)
    assert rc == kgref.OK
    assert (D[:2] == K).all() and (D[2:] == K / 2).all()
    assert np.array_equal(bound, D)


def test_token_permutation_within_expert_permutes_rows_bit_exactly():
    c, h = small([6, 5], seed=7)
    D, _ = run(h, c.N, c.K)
    perm = np.concatenate([np.random.default_rng(1).permutation(6), 6 + np.arange(5)[::-1]])
    h2 = dict(h, A=np.ascontiguousarray(h["A"][perm]), sa=np.ascontiguousarray(h["sa"][:, perm]))
    D2, _ = run(h2, c.N, c.K)
    assert np.array_equal(D2, D[perm])


def test_splitting_an_expert_or_adding_an_empty_one_changes_nothing():
    c, h = small([7, 4], seed=9)
    D, _ = run(h, c.N, c.K)
    # expert 0 split into 3 + 4 tokens that share its weight; an empty expert in front
    W2 = np.ascontiguousarray(np.stack([h["W"][1], h["W"][0], h["W"][0], h["W"][1]]))
    sw2 = np.ascontiguousarray(np.stack([h["sw"][1], h["sw"][0], h["sw"][0], h["sw"][1]]))
    D2, _ = run(dict(h, W=W2, sw=sw2, ms=np.array([0, 3, 4, 4], np.int32)), c.N, c.K)
    assert np.array_equal(D2, D)


@pytest.mark.parametrize("j", [-3, 5])
def test_power_of_two_scales_are_exact(j):
    c, h = small([5, 3], seed=11)
    D, _ = run(h, c.N, c.K)
    # one token's activation scales times 2^j: its row times 2^j
    sa2 = h["sa"].copy()
    sa2[:, 2] *= np.float32(2.0 ** j)
    D2, _ = run(dict(h, sa=sa2), c.N, c.K)
    assert np.array_equal(D2[2], D[2] * 2.0 ** j)
    assert np.array_equal(np.delete(D2, 2, axis=0), np.delete(D, 2, axis=0))
    # all of expert 1's weight scales times 2^j: its rows times 2^j
    sw2 = h["sw"].copy()
    sw2[1] *= np.float32(2.0 ** j)
    D3, _ = run(dict(h, sw=sw2), c.N, c.K)
    assert np.array_equal(D3[5:], D[5:] * 2.0 ** j)
    assert np.array_equal(D3[:5], D[:5])


def test_sampled_equals_full_and_threads_do_not_matter():
    c, h = small([9, 0, 4], seed=13)
    D, bound = run(h, c.N, c.K)
    rng = np.random.default_rng(2)
    st = rng.integers(0, c.M_total, 300)
    sn = rng.integers(0, c.N, 300)
    rc, out, b = kgref.dgrad_sampled(h["A"], h["sa"], h["W"], h["sw"], h["ms"], c.N, c.K, st, sn)
    assert rc == kgref.OK
    assert np.array_equal(out, D[st, sn]) and np.array_equal(b, bound[st, sn])
    rc, D1, _ = kgref.dgrad(h["A"], h["sa"], h["W"], h["sw"], h["ms"], c.N, c.K, threads=1)
    assert rc == kgref.OK and np.array_equal(D1, D)
    rc, Dr, _ = kgref.dgrad(h["A"], h["sa"], h["W"], h["sw"], h["ms"], c.N, c.K, rows=(4, 11))
    assert rc == kgref.OK and np.array_equal(Dr, D[4:11])


def test_validation_codes():
    L = kgref.lib()
    ms = np.array([3, 4], np.int32)
    p = ms.ctypes.data
    assert L.kgref_dgrad_validate(p, 2, 256, 384, 7) == kgref.OK
    assert L.kgref_dgrad_validate(p, 2, 256, 300, 7) == kgref.ERR_SHAPE   # K % 128
    assert L.kgref_dgrad_validate(p, 2, 200, 384, 7) == kgref.ERR_SHAPE   # N % 128
    assert L.kgref_dgrad_validate(p, 2, 256, 384, 8) == kgref.ERR_KSUM
    neg = np.array([3, -1], np.int32)
    assert L.kgref_dgrad_validate(neg.ctypes.data, 2, 256, 384, 2) == kgref.ERR_KSUM
    assert L.kgref_dgrad_validate(None, 2, 256, 384, 7) == kgref.ERR_NULL


def test_quantisers_of_the_inputs():
    # the generator's 1x128 and 128x128 quantisers: every run's largest magnitude
    # encodes to +-448 and dequantisation is within half an e4m3 step (1/16 relative)
    import torch
    g = torch.Generator().manual_seed(0)
    x = torch.randn((5, 256), generator=g)
    q, s = inputs.quantize_rows_1x128(x)
    tab = dec_table()
    deq = tab[q.numpy()] * np.repeat(s.numpy().T, 128, axis=1)
    assert (np.abs(tab[q.numpy()]).reshape(5, 2, 128).max(axis=2) == 448).all()
    assert np.all(np.abs(deq - x.numpy()) <= np.abs(x.numpy()) / 16 + 1e-6 * s.numpy().max())
    w = torch.randn((2, 256, 128), generator=g)
    qw, sw = inputs.quantize_blocks_128x128(w)
    assert (np.abs(tab[qw.numpy()]).reshape(2, 2, 128, 1, 128).max(axis=(2, 4)) == 448).all()

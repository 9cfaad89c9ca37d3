"""Pins of the requantiser oracle (kgref_requant, kgref_e4m3_encode) against facts
other than the oracle itself: torch's float8 e4m3fn conversion (round to nearest,
ties to even) for the encoder; a second, independent implementation in numpy
float32 arithmetic plus torch's conversion for whole problems; closed forms (the
block maximum maps to +-448, all-zero blocks); and invariants (expert-aligned
blocks, power-of-two scale bounds, dequantisation error within half an e4m3 step).
"""
import math

import numpy as np
import pytest
import torch

from oracle import kgref

F32S, UE8 = kgref.SCALE_F32, kgref.SCALE_UE8M0
SBF, S8 = kgref.SRC_BF16, kgref.SRC_E4M3_1X128


def torch_enc(x32):
    """fp32 -> e4m3fn bytes by torch's conversion (values must be within +-448)."""
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def dec(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


# ------------------------------------------------------------ the encoder

def test_encoder_round_trips_every_code():
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            assert kgref.e4m3_encode(float("nan")) == 0x7F
            continue
        assert kgref.e4m3_encode(float(dec([c])[0])) == c, hex(c)


def test_encoder_matches_torch_conversion():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 1e-2,
        rng.standard_normal(5000) * 2.0 ** -9,
        # exact midpoints between neighbouring codes: ties go to the even code
        (dec(np.arange(0, 126)) + dec(np.arange(1, 127))) / 2,
        -(dec(np.arange(0, 126)) + dec(np.arange(1, 127))) / 2,
    ]).astype(np.float32)
    mine = np.array([kgref.e4m3_encode(float(v)) for v in x], np.uint8)
    assert np.array_equal(mine, torch_enc(x))


def test_encoder_saturates_and_keeps_sign():
    assert kgref.e4m3_encode(448.0) == 0x7E
    assert kgref.e4m3_encode(464.0) == 0x7E
    assert kgref.e4m3_encode(1e30) == 0x7E
    assert kgref.e4m3_encode(-1e30) == 0xFE
    assert kgref.e4m3_encode(-0.0) == 0x80
    assert kgref.e4m3_encode(-2.0 ** -12) == 0x80
    assert kgref.e4m3_encode(2.0 ** -10) == 0x00       # midpoint of 0 and 2^-9: even code
    assert kgref.e4m3_encode(3 * 2.0 ** -10) == 0x02   # midpoint of 2^-9 and 2^-8: even code


# ------------------------------------------------------------ an independent implementation

def numpy_requant(x32, ks, gran, scale_kind):
    """The same definition written with numpy float32 arithmetic and torch's encoder."""
    K, H = x32.shape
    rows_q = np.zeros((K, H), np.uint8)
    scales = []
    t0 = 0
    for k in ks:
        for b0 in range(t0, t0 + int(k), gran):
            b1 = min(b0 + gran, t0 + int(k))
            blk = x32[b0:b1]
            # largest magnitude with NaNs skipped (0 for an all-NaN column)
            amax = np.fmax.reduce(np.abs(blk), axis=0).astype(np.float32)
            amax = np.where(np.isnan(amax), np.float32(0), amax).astype(np.float32)
            if scale_kind == F32S:
                s = np.where(amax == 0, np.float32(1.0), amax / np.float32(448.0)).astype(np.float32)
                with np.errstate(divide="ignore", invalid="ignore"):
                    y = (blk / s[None, :]).astype(np.float32)
                q = np.where(np.isnan(y), np.uint8(0x7F), torch_enc(np.clip(y, -448, 448)))
                scales.append(s)
            else:
                r = (amax / np.float32(448.0)).astype(np.float32)
                e = np.full(H, 127, np.int64)
                nz = amax > 0
                # smallest k with 2^k >= r, from r's binary32 exponent and mantissa bits
                bits = r.view(np.uint32)
                ex = ((bits >> 23) & 0xFF).astype(np.int64)
                mant = (bits & 0x7FFFFF)
                k2 = np.where(ex > 0, ex - 127 + (mant != 0), 0)
                sub = (ex == 0) & (mant != 0) & nz
                if sub.any():  # subnormal quotients
                    k2[sub] = np.ceil(np.log2(r[sub].astype(np.float64))).astype(np.int64)
                k2[nz & (r == 0)] = -1000  # amax / 448 underflowed: any k, clamped to 0
                e[nz] = np.clip(k2[nz] + 127, 0, 254)
                y = (blk.astype(np.float64) * np.exp2(127.0 - e)[None, :]).astype(np.float32)
                q = np.where(np.isnan(y), np.uint8(0x7F), torch_enc(np.clip(y, -448, 448)))
                scales.append(e.astype(np.uint8))
            rows_q[b0:b1] = q
        t0 += int(k)
    S = np.stack(scales) if scales else np.zeros((0, H), np.float32 if scale_kind == F32S else np.uint8)
    return rows_q, S


def bf16_input(rng, K, H, outliers=False):
    x = rng.standard_normal((K, H)).astype(np.float32)
    if outliers:
        x[rng.random((K, H)) < 0.01] *= 50
    x[rng.random((K, H)) < 0.01] = 0.0
    b = torch.from_numpy(x).to(torch.bfloat16)
    return b.view(torch.int16).numpy().view(np.uint16), b.to(torch.float32).numpy()


@pytest.mark.parametrize("gran", [32, 128])
@pytest.mark.parametrize("scale_kind", [F32S, UE8])
def test_bf16_source_matches_independent_numpy(gran, scale_kind):
    rng = np.random.default_rng(1)
    ks = [300, 0, 129, 1, 64]
    K, H = sum(ks), 48
    xb, x32 = bf16_input(rng, K, H, outliers=True)
    rc, Q, S = kgref.requant(xb, None, ks, H, gran, SBF, scale_kind)
    assert rc == kgref.OK
    Qn, Sn = numpy_requant(x32, ks, gran, scale_kind)
    assert np.array_equal(Q, Qn)
    assert np.array_equal(S.view(np.uint8), Sn.view(np.uint8))


@pytest.mark.parametrize("scale_kind", [F32S, UE8])
def test_fp8_1x128_source_matches_independent_numpy(scale_kind):
    rng = np.random.default_rng(2)
    ks = [200, 77, 0]
    K, H = sum(ks), 256
    X = rng.integers(0, 256, (K, H), dtype=np.uint8)
    X[(X & 0x7F) == 0x7F] = 0x30
    xs = (rng.random((K, H // 128)) * 0.01 + 1e-4).astype(np.float32)
    rc, Q, S = kgref.requant(X, xs, ks, H, 128, S8, scale_kind)
    assert rc == kgref.OK
    x32 = (dec(X).astype(np.float32) * np.repeat(xs, 128, axis=1)).astype(np.float32)
    Qn, Sn = numpy_requant(x32, ks, 128, scale_kind)
    assert np.array_equal(Q, Qn)
    assert np.array_equal(S.view(np.uint8), Sn.view(np.uint8))


# ------------------------------------------------------------ closed forms and invariants

def test_block_maximum_maps_to_448_and_zero_blocks():
    rng = np.random.default_rng(3)
    ks = [130, 70]
    K, H = 200, 32
    xb, x32 = bf16_input(rng, K, H)
    x32[128:130, 5] = 0.0
    xb[128:130, 5] = 0
    rc, Q, S = kgref.requant(xb, None, ks, H, 128, SBF, F32S)
    assert rc == kgref.OK
    for (b0, b1, row) in [(0, 128, 0), (128, 130, 1), (130, 200, 2)]:
        blk = np.abs(x32[b0:b1])
        for h in range(H):
            if blk[:, h].max() == 0:
                assert S[row, h] == 1.0 and (Q[b0:b1, h] & 0x7F == 0).all()
                continue
            t = b0 + int(np.argmax(blk[:, h]))
            assert Q[t, h] & 0x7F == 0x7E


def test_dequantisation_error_and_scale_bounds():
    rng = np.random.default_rng(4)
    ks = [257, 3]
    K, H = sum(ks), 40
    xb, x32 = bf16_input(rng, K, H, outliers=True)
    for kind in (F32S, UE8):
        rc, Q, S = kgref.requant(xb, None, ks, H, 32, SBF, kind)
        assert rc == kgref.OK
        rows = np.concatenate([np.full(min(32, 257 - b), i) for i, b in enumerate(range(0, 257, 32))] +
                              [np.full(3, 9)])
        s = S.astype(np.float64) if kind == F32S else np.exp2(S.astype(np.float64) - 127)
        back = dec(Q) * s[rows]
        # half an e4m3 step: 2^-4 relative for normals, 2^-10 * s absolute below 2^-6 * s
        assert (np.abs(back - x32) <= np.abs(x32) * 2.0 ** -4 + s[rows] * 2.0 ** -10 + 1e-30).all()
        if kind == UE8:
            amax = np.array([np.abs(x32[rows == r]).max(axis=0) for r in range(S.shape[0])])
            lim = (amax.astype(np.float32) / np.float32(448)).astype(np.float64)
            nz = amax > 0
            assert (s[nz] >= lim[nz]).all() and (s[nz] < 2 * lim[nz]).all()


def test_blocks_restart_at_each_expert():
    # the same token rows quantised as one expert or as two experts differ only
    # through the block boundaries: splitting at a multiple of gran_k changes nothing
    rng = np.random.default_rng(5)
    xb, _ = bf16_input(rng, 256 + 40, 24)
    rc1, Q1, S1 = kgref.requant(xb, None, [296], 24, 128, SBF, F32S)
    rc2, Q2, S2 = kgref.requant(xb, None, [256, 40], 24, 128, SBF, F32S)
    assert rc1 == rc2 == kgref.OK
    assert np.array_equal(Q1, Q2) and np.array_equal(S1, S2)
    # a split off the block grid starts a new block at the second expert's first token
    rc3, Q3, S3 = kgref.requant(xb, None, [100, 196], 24, 128, SBF, F32S)
    assert rc3 == kgref.OK and S3.shape[0] == 1 + 2
    rc4, Q4, S4 = kgref.requant(xb[100:], None, [196], 24, 128, SBF, F32S)
    assert np.array_equal(Q3[100:], Q4) and np.array_equal(S3[1:], S4)


def test_requant_validation():
    x = np.zeros((4, 128), np.uint16)
    assert kgref.requant(x, None, [4], 128, 64, SBF, F32S)[0] == kgref.ERR_GRAN
    assert kgref.requant(x, None, [3], 128, 128, SBF, F32S, K_total=4)[0] == kgref.ERR_KSUM
    assert kgref.requant(x, None, [4], 128, 128, SBF, 7)[0] == kgref.ERR_DTYPE
    x8 = np.zeros((4, 96), np.uint8)
    assert kgref.requant(x8, np.zeros((4, 1), np.float32), [4], 96, 128, S8, F32S)[0] == kgref.ERR_SHAPE


# ------------------------------------------------------------ special values

@pytest.mark.parametrize("gran", [32, 128])
@pytest.mark.parametrize("scale_kind", [F32S, UE8])
def test_edge_values_match_independent_numpy(gran, scale_kind):
    """Infinities, NaNs, signed zeros, bf16 subnormals, maxima whose scale is
    subnormal, and exact rounding ties x / s = o * 2^k, against the numpy twin (NaNs
    skipped by amax and encoded 0x7F; IEEE binary32 arithmetic for the rest)."""
    from fp8_grouped_gemm_tn_amd import inputs
    ks = [200, 0, 37, 64, 1]
    K, H = sum(ks), 128
    x32 = inputs.requant_edge_source(K, H, seed=gran + scale_kind)
    xb = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    rc, Q, S = kgref.requant(xb, None, ks, H, gran, SBF, scale_kind)
    assert rc == kgref.OK
    Qn, Sn = numpy_requant(x32, ks, gran, scale_kind)
    assert np.array_equal(Q, Qn)
    assert np.array_equal(S.view(np.uint8), Sn.view(np.uint8))


def test_edge_values_closed_forms():
    """What IEEE arithmetic fixes for the special columns, block by block."""
    from fp8_grouped_gemm_tn_amd import inputs
    K, H = 128, 128
    x32 = inputs.requant_edge_source(K, H, seed=3)
    xb = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    _, Qf, Sf = kgref.requant(xb, None, [K], H, 128, SBF, F32S)
    _, Qe, Se = kgref.requant(xb, None, [K], H, 128, SBF, UE8)
    for h in range(H):
        col, fam = x32[:, h], h % 16
        fin = np.isfinite(col)
        if fam == 0:   # +inf present: s = inf, finite values -> signed zeros, inf -> NaN
            assert np.isinf(Sf[0, h]) and Se[0, h] == 254
            assert (Qf[fin, h] & 0x7F == 0).all() and (Qf[~fin, h] == 0x7F).all()
            assert (Qe[np.isposinf(col), h] == 0x7E).all()
        if fam == 2:   # all NaN: amax 0, unit scale / byte 127, codes NaN
            assert Sf[0, h] == 1.0 and Se[0, h] == 127 and (Qf[:, h] == 0x7F).all()
        if fam == 3:   # zeros: sign kept
            assert Sf[0, h] == 1.0 and Se[0, h] == 127
            assert np.array_equal(Qf[:, h], np.where(np.signbit(col), 0x80, 0x00))
        if fam == 6:   # amax 448: s = 1, e = 127, the codes are the values' own
            assert Sf[0, h] == 1.0 and Se[0, h] == 127
            assert np.array_equal(Qf[:, h], torch_enc(col)) and np.array_equal(Qe[:, h], Qf[:, h])
        if fam in (7, 8, 9):  # amax 448 f: s = f exactly, x / s = o * 2^k exactly
            f = (3.0, 5.0, 7.0)[fam - 7]
            assert Sf[0, h] == f
            assert np.array_equal(Qf[:, h], torch_enc((col / np.float32(f)).astype(np.float32)))


@pytest.mark.parametrize("gran", [32, 128])
@pytest.mark.parametrize("scale_kind", [F32S, UE8])
def test_fp8_edge_source_matches_independent_numpy(gran, scale_kind):
    """The fp8 source with NaN codes and per-token scales whose products overflow, are
    subnormal or zero; runs whose fp32 scale amax / 448 underflows to 0."""
    from fp8_grouped_gemm_tn_amd import inputs
    ks = [300, 0, 129, 1, 200]
    K, H = sum(ks), 256
    X, xs = inputs.requant_edge_fp8_source(K, H, seed=gran + scale_kind)
    rc, Q, S = kgref.requant(X, xs, ks, H, gran, S8, scale_kind)
    assert rc == kgref.OK
    with np.errstate(over="ignore", invalid="ignore"):
        x32 = (dec(X).astype(np.float32) * np.repeat(xs, 128, axis=1)).astype(np.float32)
    Qn, Sn = numpy_requant(x32, ks, gran, scale_kind)
    assert np.array_equal(Q, Qn)
    assert np.array_equal(S.view(np.uint8), Sn.view(np.uint8))
    if scale_kind == F32S:
        assert (S == 0).any() and np.isinf(S).any()

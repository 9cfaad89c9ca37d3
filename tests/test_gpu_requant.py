"""GPU parity of the requantiser (kg_requant, through the C ABI) against the CPU
oracle: fp8 codes and scales must agree bit for bit (integer/byte work), for both
sources (bf16; e4m3 with 1x128 per-token scales), both scale kinds and both block
sizes, on ragged experts with empty ones, and on a larger routed shape."""
import numpy as np
import pytest
import torch

import fp8_grouped_gemm_tn_amd as kg
from fp8_grouped_gemm_tn_amd import inputs
from oracle import kgref

pytestmark = pytest.mark.gpu

SRC = {kg.KG_SRC_BF16: kgref.SRC_BF16, kg.KG_SRC_E4M3_1X128: kgref.SRC_E4M3_1X128}
KIND = {kg.KG_E4M3_F32SCALE: kgref.SCALE_F32, kg.KG_E4M3_UE8M0: kgref.SCALE_UE8M0}


def say(*a):
    print("[case]", *a, flush=True)


def make_source(src, K, H, seed):
    g = torch.Generator().manual_seed(seed)
    if src == kg.KG_SRC_BF16:
        x = torch.randn(K, H, generator=g)
        x = torch.where(torch.rand(K, H, generator=g) < 0.01, x * 50, x)
        x = torch.where(torch.rand(K, H, generator=g) < 0.01, torch.zeros_like(x), x)
        xb = x.to(torch.bfloat16)
        return xb, None, xb.view(torch.int16).numpy().view(np.uint16), None
    codes = torch.randint(0, 256, (K, H), generator=g, dtype=torch.int32).to(torch.uint8)
    codes = torch.where((codes & 0x7F) == 0x7F, torch.full_like(codes, 0x30), codes)
    xs = torch.rand(K, H // 128, generator=g) * 0.01 + 1e-4
    return codes, xs, codes.numpy(), xs.numpy()


def run_case(src, kind, gran, ks, H, seed):
    K = int(np.asarray(ks, np.int64).sum())
    run_source(src, kind, gran, ks, H, *make_source(src, K, H, seed))


def run_source(src, kind, gran, ks, H, X, xs, Xh, xsh):
    """X, xs: the source as torch CPU tensors (bf16, or uint8 codes with fp32 scales);
    Xh, xsh: the same as numpy arrays for the oracle."""
    ks = np.asarray(ks, np.int32)
    K = int(ks.sum())
    nblk = int(sum((int(k) + gran - 1) // gran for k in ks))
    d = torch.device("cuda:0")
    Xd = X.to(d)
    xsd = None if xs is None else xs.to(d)
    ksd = torch.from_numpy(ks).to(d)
    sdt = torch.float32 if kind == kg.KG_E4M3_F32SCALE else torch.uint8
    # Q and S inside guarded buffers (4 KB of 0x5A bytes before and after each)
    pad = 4096
    qbuf = torch.full((K * H + 2 * pad,), 0x5A, dtype=torch.uint8, device=d)
    Q = qbuf[pad:pad + K * H].view(K, H)
    ssz = nblk * H * (4 if sdt == torch.float32 else 1)
    sbuf = torch.full((ssz + 2 * pad,), 0x5A, dtype=torch.uint8, device=d)
    S = sbuf[pad:pad + ssz].view(sdt).view(nblk, H)
    if sdt == torch.float32:
        S.fill_(float("nan"))
    rc = kg.kg_requant_raw(Xd, xsd, ksd, ks.size, H, K, gran, src, kind, Q, S)
    assert rc == kg.KG_OK
    assert kg.kg_status() == kg.KG_OK
    for buf, n in ((qbuf, K * H), (sbuf, ssz)):
        assert (buf[:pad] == 0x5A).all() and (buf[pad + n:] == 0x5A).all(), "write outside Q or S"
    rc, Qr, Sr = kgref.requant(Xh, xsh, ks, H, gran, SRC[src], KIND[kind])
    assert rc == kgref.OK
    Qg = Q.cpu().numpy()
    Sg = S.cpu().numpy()
    bad = np.nonzero(Qg != Qr)
    assert bad[0].size == 0, f"{bad[0].size} fp8 codes differ, first at {bad[0][0], bad[1][0]}: " \
                             f"{Qg[bad][0]:#x} vs {Qr[bad][0]:#x}"
    assert np.array_equal(Sg.view(np.uint8), Sr.view(np.uint8)), "scales differ"


@pytest.mark.parametrize("gran", [32, 128])
@pytest.mark.parametrize("kind", [kg.KG_E4M3_F32SCALE, kg.KG_E4M3_UE8M0])
@pytest.mark.parametrize("src", [kg.KG_SRC_BF16, kg.KG_SRC_E4M3_1X128])
def test_requant_bit_exact_ragged(src, kind, gran):
    say("requant", src, kind, gran)
    run_case(src, kind, gran, [300, 0, 129, 1, 513, 64, 0], 384, seed=gran + 7 * kind + 31 * src)


@pytest.mark.parametrize("kind", [kg.KG_E4M3_F32SCALE, kg.KG_E4M3_UE8M0])
def test_requant_bit_exact_routed_shape(kind):
    say("requant routed", kind)
    rng = np.random.default_rng(5)
    p = 1.0 / np.arange(1, 17) ** 1.2
    ks = rng.multinomial(16384, p / p.sum()).astype(np.int32)
    run_case(kg.KG_SRC_BF16, kind, 128 if kind == kg.KG_E4M3_F32SCALE else 32, ks, 1024, seed=9)


@pytest.mark.parametrize("kind,gran", [(kg.KG_E4M3_F32SCALE, 128), (kg.KG_E4M3_UE8M0, 32)])
def test_requant_bit_exact_most_groups(kind, gran):
    # G = 1024 (the most accepted): 0-40 tokens per expert, every seventh one empty
    say("requant 1024 groups", kind, gran)
    ks = [0 if i % 7 == 0 else (13 * i) % 41 for i in range(1024)]
    run_case(kg.KG_SRC_BF16, kind, gran, ks, 256, seed=12)


@pytest.mark.parametrize("gran", [32, 128])
@pytest.mark.parametrize("kind", [kg.KG_E4M3_F32SCALE, kg.KG_E4M3_UE8M0])
def test_requant_bit_exact_edge_values(kind, gran):
    """Infinities, NaNs, signed zeros, bf16 subnormals, block maxima whose scale is
    subnormal (its reciprocal overflows), exact rounding ties x / s = o * 2^k for
    s = 1, 3, 5, 7, and a wide dynamic range, on ragged experts."""
    say("requant edge values bf16", kind, gran)
    ks = [300, 0, 129, 1, 513, 64, 7]
    K, H = sum(ks), 512
    x32 = inputs.requant_edge_source(K, H, seed=gran + kind)
    xb = torch.from_numpy(x32).to(torch.bfloat16)
    run_source(kg.KG_SRC_BF16, kind, gran, ks, H, xb, None,
               xb.view(torch.int16).numpy().view(np.uint16), None)


@pytest.mark.parametrize("gran", [32, 128])
@pytest.mark.parametrize("kind", [kg.KG_E4M3_F32SCALE, kg.KG_E4M3_UE8M0])
def test_requant_bit_exact_edge_values_fp8_source(kind, gran):
    """The fp8 source with every code (NaN codes included) and per-token scales whose
    products overflow to infinity, are subnormal, or are zero (scale 0: the block's
    fp32 scale amax / 448 can underflow to 0)."""
    say("requant edge values fp8", kind, gran)
    ks = [300, 0, 129, 1, 200]
    K, H = sum(ks), 384
    codes, xs = inputs.requant_edge_fp8_source(K, H, seed=gran + kind)
    run_source(kg.KG_SRC_E4M3_1X128, kind, gran, ks, H, torch.from_numpy(codes),
               torch.from_numpy(xs), codes, xs)


def test_requant_ksum_mismatch_writes_nothing():
    say("requant ksum")
    d = torch.device("cuda:0")
    X = torch.randn(100, 128, device=d).to(torch.bfloat16)
    ks = torch.tensor([60, 30], dtype=torch.int32, device=d)
    Q = torch.full((100, 128), 7, dtype=torch.uint8, device=d)
    S = torch.full((2, 128), 3.0, device=d)
    assert kg.kg_requant_raw(X, None, ks, 2, 128, 100, 128, kg.KG_SRC_BF16, kg.KG_E4M3_F32SCALE,
                             Q, S) == kg.KG_OK
    assert kg.kg_status() == kg.KG_ERR_KSUM
    assert (Q == 7).all() and (S == 3.0).all()


def test_requant_too_few_scale_rows_writes_nothing():
    """ks [60, 30, 10] at gran 128 needs 3 scale rows, while the host can only require
    ceil(100 / 128) = 1: S with 1 or 2 rows passes the host check and the kernel reports
    KG_ERR_SCALE_ROWS without writing. At gran 32 the host bound, ceil(100 / 32) = 4,
    already rejects 3 rows."""
    say("requant scale rows")
    d = torch.device("cuda:0")
    X = torch.randn(100, 128, device=d).to(torch.bfloat16)
    ks = torch.tensor([60, 30, 10], dtype=torch.int32, device=d)
    Q = torch.full((100, 128), 7, dtype=torch.uint8, device=d)
    S = torch.full((3, 128), 3.0, device=d)
    for rows in (1, 2):
        assert kg.kg_requant_raw(X, None, ks, 3, 128, 100, 128, kg.KG_SRC_BF16,
                                 kg.KG_E4M3_F32SCALE, Q, S[:rows], s_rows=rows) == kg.KG_OK
        assert kg.kg_status() == kg.KG_ERR_SCALE_ROWS
        assert (Q == 7).all() and (S == 3.0).all()
    assert kg.kg_requant_raw(X, None, ks, 3, 128, 100, 32, kg.KG_SRC_BF16,
                             kg.KG_E4M3_F32SCALE, Q, S, s_rows=3) == kg.KG_ERR_SCALE_ROWS
    assert kg.kg_requant_raw(X, None, ks, 3, 128, 100, 128, kg.KG_SRC_BF16,
                             kg.KG_E4M3_F32SCALE, Q, S) == kg.KG_OK
    assert kg.kg_status() == kg.KG_OK
    assert not (S == 3.0).any()


def test_requant_feeds_wgrad():
    # the requantised operands run through kg_wgrad and match the oracle GEMM on them
    say("requant -> wgrad")
    d = torch.device("cuda:0")
    ks = np.array([200, 0, 77], np.int32)
    K, M, N = 277, 128, 256
    g = torch.Generator().manual_seed(3)
    a = torch.randn(K, M, generator=g).to(torch.bfloat16)
    b = (torch.randn(K, N, generator=g) * 1e-3).to(torch.bfloat16)
    ksd = torch.from_numpy(ks).to(d)
    A, sa = kg.kg_requant(a.to(d), None, ksd, 128, kg.KG_E4M3_F32SCALE, 3)
    B, sb = kg.kg_requant(b.to(d), None, ksd, 128, kg.KG_E4M3_F32SCALE, 3)
    D = torch.empty((3, M, N), device=d)
    kg.kg_wgrad(A, sa, B, sb, None, D, ksd, 128, kg.KG_E4M3_F32SCALE)
    assert kg.kg_status() == kg.KG_OK
    rc, Dr, bound = kgref.wgrad(A.cpu().numpy(), sa.cpu().numpy(), B.cpu().numpy(), sb.cpu().numpy(),
                                None, ks, M, N, 128, kgref.E4M3_F32SCALE)
    assert rc == kgref.OK
    err = np.abs(D.cpu().numpy().astype(np.float64) - Dr)
    assert (err <= 1e-5 * bound + 1e-6).all()
    # and the fp8 product stays close to the bf16 one (quantisation error only)
    ref = [a[:200].float().T @ b[:200].float(), torch.zeros(M, N), a[200:].float().T @ b[200:].float()]
    for gi in (0, 2):
        rel = (D[gi].cpu() - ref[gi]).norm() / ref[gi].norm()
        assert rel < 0.1, float(rel)


@pytest.mark.parametrize("name", list(inputs.REQUANT_WORKLOADS))
def test_requant_full_size_sampled_blocks(name):
    """The bench workloads at full size, in the launch configuration bench.py times:
    16 random blocks (scale rows) plus the first and last block of three experts are
    compared bit for bit (codes and scales, all channels) with the oracle run on just
    those blocks' token rows."""
    say("requant full size", name)
    wl, H, gran, kind, src = inputs.REQUANT_WORKLOADS[name]
    d = torch.device("cuda:0")
    X, xs, ks = inputs.requant_source(name, device=d, seed=0)
    K = int(ks.astype(np.int64).sum())
    nblk = int(sum((int(k) + gran - 1) // gran for k in ks))
    Q = torch.empty((K, H), dtype=torch.uint8, device=d)
    S = torch.empty((nblk, H), dtype=torch.float32 if kind == kg.KG_E4M3_F32SCALE else torch.uint8,
                    device=d)
    rc = kg.kg_requant_raw(X, xs, torch.from_numpy(ks).to(d), ks.size, H, K, gran, src, kind, Q, S)
    assert rc == kg.KG_OK
    assert kg.kg_status() == kg.KG_OK
    # blocks: (scale row, first token, tokens)
    off = np.concatenate([[0], np.cumsum(ks.astype(np.int64))])
    blocks = []
    for g in range(ks.size):
        for kb in range((int(ks[g]) + gran - 1) // gran):
            t0 = int(off[g]) + kb * gran
            blocks.append((len(blocks), t0, min(gran, int(off[g + 1]) - t0)))
    rng = np.random.default_rng(11)
    pick = set(rng.choice(len(blocks), 16, replace=False).tolist())
    live = np.nonzero(ks > 0)[0]
    for g in live[[0, live.size // 2, -1]]:
        first = int(sum((int(k) + gran - 1) // gran for k in ks[:g]))
        pick |= {first, first + (int(ks[g]) + gran - 1) // gran - 1}
    for b in sorted(pick):
        row, t0, n = blocks[b]
        Xh = X[t0:t0 + n].cpu()
        Xh = (Xh.view(torch.int16).numpy().view(np.uint16) if src == kg.KG_SRC_BF16
              else Xh.numpy())
        xsh = None if xs is None else np.ascontiguousarray(xs[t0:t0 + n].cpu().numpy())
        rc, Qr, Sr = kgref.requant(Xh, xsh, [n], H, gran, SRC[src], KIND[kind])
        assert rc == kgref.OK
        assert np.array_equal(Q[t0:t0 + n].cpu().numpy(), Qr), f"block {b}: codes differ"
        assert np.array_equal(S[row].cpu().numpy().view(np.uint8), Sr[0].view(np.uint8)), \
            f"block {b}: scales differ"
    del X, xs, Q, S
    torch.cuda.empty_cache()


@pytest.mark.parametrize("seed", range(24))
def test_requant_random_configuration(seed):
    """Seeded random requantiser configurations, bit-exact against the oracle: source,
    scale kind, block size, expert count and token counts (long, short with empty and
    one-token experts, or heavy-tailed) and channel count."""
    rng = np.random.default_rng(3000 + seed)
    src = [kg.KG_SRC_BF16, kg.KG_SRC_E4M3_1X128][seed % 2]
    kind = [kg.KG_E4M3_F32SCALE, kg.KG_E4M3_UE8M0][(seed // 2) % 2]
    gran = [32, 128][(seed // 4) % 2]
    G = int(rng.integers(1, 65))
    style = rng.integers(0, 3)
    if style == 0:
        ks = rng.integers(0, 600, G)
    elif style == 1:
        ks = rng.choice([0, 1, 2, 31, 32, 33, 127, 128, 129], G)
    else:
        ks = np.minimum((rng.pareto(1.2, G) * 40).astype(np.int64), 2000)
    ks[rng.random(G) < 0.15] = 0
    H = 128 * int(rng.integers(1, 9))
    say("requant random", seed, src, kind, gran, "G", G, "tokens", int(ks.sum()), "H", H)
    run_case(src, kind, gran, [int(k) for k in ks], H, seed)

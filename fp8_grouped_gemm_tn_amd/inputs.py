"""Seeded synthetic inputs for the K-grouped weight-gradient GEMM.

This module makes inputs only: per-expert token counts (routing), fp32 values,
and their quantisation to fp8 e4m3fn with per-(block, channel) scales or to
bf16. It contains none of the GEMM's arithmetic, and both the GPU path's tests
and the CPU oracle's tests draw their inputs from it.

Workloads (named by what they are):
  worked       - the how-to page's worked shape: ks = [32, 45, 27], M = 64, N = 128,
                 fp8 with fp32 scales per 128 tokens, no C.
  bf16         - G = 4, M = 1024, N = 2048, 16384 tokens routed uniformly over three
                 experts (the second expert gets none), bf16 N(0,1)*0.1, C ~ N(0,1).
  zipf_fp8     - G = 32, M = 7168, N = 4096, 65536 tokens with Zipf(1.2) routing, A
                 N(0,1) with 1% of entries x50, B N(0,1)*1e-3, fp8 + fp32 scales per
                 128 tokens, C ~ N(0,1).
  ue8m0_many   - G = 256, M = 2048, N = 7168, 16384 tokens each routed to 8 distinct
                 experts among 205 active ones (51 experts empty), A, B ~ N(0,1), fp8 +
                 power-of-two scales per 32 tokens, no C.
  local_share  - G = 8, M = 7168, N = 4096, 262144 tokens with per-expert counts drawn
                 from N(32768, 8192), clipped at 0 and rescaled, values as zipf_fp8.
  single_m{m}_n{n}_k{k} - one group (G = 1): the six non-grouped fp8 GEMM shapes
                 (m, n, k) of the GitHub issue page's 1D1D kernel table (thefacetakt,
                 2025-03-20), mapped onto this operation as M = m, N = n and k
                 contraction tokens; A, B ~ N(0,1), fp8 + fp32 scales per 128 tokens
                 (the table's 1x128 scales on both operands), no C.

Quantiser (input preparation, not part of the measured path): for each run of
gran_k tokens of one expert (runs restart at each expert's first token) and each
channel, amax = max |x|; fp32 scale = amax / 448 (1 if amax == 0) and
q = e4m3fn(RNE(clamp(x / scale, +-448))); power-of-two scales use
e = ceil(log2(amax / 448)) + 127 clamped to [0, 254] (127 if amax == 0), scale
2^(e-127).
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

E4M3_F32SCALE, E4M3_UE8M0, BF16 = 0, 1, 2
DTYPE_NAMES = {E4M3_F32SCALE: "e4m3+f32scale", E4M3_UE8M0: "e4m3+ue8m0", BF16: "bf16"}
FP8_MAX = 448.0


@dataclass
class Case:
    name: str
    G: int
    M: int
    N: int
    ks: np.ndarray          # int32 [G]
    dtype: int
    gran_k: int
    A: torch.Tensor         # uint8 [K_total, M] (fp8 bytes) or bfloat16 [K_total, M]
    B: torch.Tensor         # uint8 [K_total, N] or bfloat16 [K_total, N]
    sa: Optional[torch.Tensor]  # float32 or uint8 [nblocks, M]; None for bf16
    sb: Optional[torch.Tensor]  # float32 or uint8 [nblocks, N]; None for bf16
    C: Optional[torch.Tensor]   # float32 [G, M, N] or None
    meta: dict = field(default_factory=dict)

    @property
    def K_total(self) -> int:
        return int(self.ks.astype(np.int64).sum())

    @property
    def flops(self) -> int:
        return 2 * self.K_total * self.M * self.N

    def host(self):
        """numpy copies in the layouts the oracle reads (fp8 / bf16 as raw bits)."""
        def bits(t):
            if t is None:
                return None
            t = t.detach().cpu()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16)
            return t.numpy()
        return dict(A=bits(self.A), B=bits(self.B), sa=bits(self.sa), sb=bits(self.sb),
                    C=bits(self.C), ks=self.ks.copy())

    def algorithmic_bytes(self, out_bytes: int = 4) -> int:
        """Bytes the method must move once: A, B, scales, C (if given) and D, with
        `out_bytes` per element of C and D (4: fp32, 2: the bf16-output variant)."""
        elt = 2 if self.dtype == BF16 else 1
        nbytes = self.K_total * (self.M + self.N) * elt
        if self.sa is not None:
            nbytes += self.sa.numel() * self.sa.element_size()
            nbytes += self.sb.numel() * self.sb.element_size()
        out = self.G * self.M * self.N * out_bytes
        nbytes += out + (out if self.C is not None else 0)
        return nbytes


def k_major(X: torch.Tensor, extra: int = 0) -> torch.Tensor:
    """K-major (NT) copy of a token-major operand X [K_total, C]: a [C, K_total] view
    (stride ld) of a [C, ld] buffer whose rows are whole 16-byte units with at least
    `extra` columns of padding; the padding holds NaN codes (e4m3 0x7F, bf16 0x7FC0),
    so a kernel that reads it shows NaN."""
    K, Cn = X.shape
    elt = X.element_size()
    unit = 16 // elt
    ld = (K + extra + unit - 1) // unit * unit
    if X.dtype == torch.bfloat16:
        buf = torch.full((Cn, ld), 0x7FC0, dtype=torch.int16, device=X.device).view(torch.bfloat16)
    else:
        buf = torch.full((Cn, ld), 0x7F, dtype=X.dtype, device=X.device)
    buf[:, :K] = X.t()
    return buf[:, :K]


# ----------------------------------------------------------------- routing

def ks_worked():
    return np.array([32, 45, 27], np.int32)


def ks_uniform_with_empty(total, G, empty, seed):
    rng = np.random.default_rng(seed)
    live = [g for g in range(G) if g not in set(empty)]
    counts = rng.multinomial(total, [1.0 / len(live)] * len(live))
    ks = np.zeros(G, np.int64)
    ks[live] = counts
    return ks.astype(np.int32)


def ks_zipf(total, G, s, seed):
    rng = np.random.default_rng(seed)
    ranks = rng.permutation(G) + 1
    p = ranks.astype(np.float64) ** (-s)
    p /= p.sum()
    return rng.multinomial(total, p).astype(np.int32)


def ks_topk(tokens, G, topk, n_empty, seed):
    rng = np.random.default_rng(seed)
    empty = rng.choice(G, n_empty, replace=False)
    active = np.setdiff1d(np.arange(G), empty)
    picks = np.argsort(rng.random((tokens, active.size)), axis=1)[:, :topk]
    counts = np.bincount(picks.ravel(), minlength=active.size)
    ks = np.zeros(G, np.int64)
    ks[active] = counts
    return ks.astype(np.int32)


def ks_normal(total, G, mean, std, seed):
    rng = np.random.default_rng(seed)
    x = np.clip(rng.normal(mean, std, G), 0.0, None)
    if x.sum() == 0:
        x[:] = 1.0
    x = x * (total / x.sum())
    base = np.floor(x).astype(np.int64)
    rem = total - int(base.sum())
    order = np.argsort(-(x - base), kind="stable")
    base[order[:rem]] += 1
    return base.astype(np.int32)


# ----------------------------------------------------------------- quantiser

def _block_rows(ks, gran):
    return int(sum((int(k) + gran - 1) // gran for k in ks))


def quantize_fp8(x: torch.Tensor, ks, gran: int, pow2: bool):
    """x fp32 [K_total, W] -> (uint8 [K_total, W], scales [nblocks, W])."""
    K_total, W = x.shape
    q = torch.empty((K_total, W), dtype=torch.uint8, device=x.device)
    nb = _block_rows(ks, gran)
    s = torch.empty((nb, W), dtype=torch.uint8 if pow2 else torch.float32, device=x.device)
    t0 = 0
    r0 = 0
    for k in ks:
        k = int(k)
        if k == 0:
            continue
        nbk = (k + gran - 1) // gran
        xg = x[t0:t0 + k]
        pad = nbk * gran - k
        if pad:
            xg = torch.cat([xg, torch.zeros((pad, W), dtype=x.dtype, device=x.device)])
        xb = xg.view(nbk, gran, W)
        amax = xb.abs().amax(dim=1)                      # [nbk, W]
        if pow2:
            v = amax / FP8_MAX
            mant, ex = torch.frexp(v)                    # v = mant * 2^ex, mant in [0.5, 1)
            e = torch.where(mant == 0.5, ex - 1, ex)     # ceil(log2 v)
            e = torch.clamp(e + 127, 0, 254)
            e = torch.where(amax == 0, torch.full_like(e, 127), e)
            scale = torch.ldexp(torch.ones_like(amax), (e - 127).to(torch.int32))
            s[r0:r0 + nbk] = e.to(torch.uint8)
        else:
            scale = torch.where(amax == 0, torch.ones_like(amax), amax / FP8_MAX)
            s[r0:r0 + nbk] = scale
        y = torch.clamp(xb / scale[:, None, :], -FP8_MAX, FP8_MAX)
        y = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(nbk * gran, W)
        q[t0:t0 + k] = y[:k]
        t0 += k
        r0 += nbk
    return q, s


# ----------------------------------------------------------------- cases

def _normal(gen, shape, device, std=1.0):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std


def make_case(name, ks, M, N, dtype, gran_k=128, with_c=True, seed=0, device="cpu",
              a_std=1.0, b_std=1.0, a_outlier_p=0.0, a_outlier_mul=50.0, scale_values=None):
    """Seeded inputs of one problem. Draw order: A, outlier mask, B, C."""
    ks = np.asarray(ks, dtype=np.int32)
    G = ks.size
    K_total = int(ks.astype(np.int64).sum())
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    a = _normal(gen, (K_total, M), dev, a_std)
    if a_outlier_p > 0:
        mask = torch.rand((K_total, M), generator=gen, device=dev) < a_outlier_p
        a = torch.where(mask, a * a_outlier_mul, a)
        del mask
    b = _normal(gen, (K_total, N), dev, b_std)
    C = _normal(gen, (G, M, N), dev) if with_c else None
    if dtype == BF16:
        A, B, sa, sb = a.to(torch.bfloat16), b.to(torch.bfloat16), None, None
    else:
        pow2 = dtype == E4M3_UE8M0
        A, sa = quantize_fp8(a, ks, gran_k, pow2)
        del a
        B, sb = quantize_fp8(b, ks, gran_k, pow2)
        del b
    return Case(name=name, G=G, M=M, N=N, ks=ks, dtype=dtype, gran_k=gran_k,
                A=A.contiguous(), B=B.contiguous(), sa=sa, sb=sb, C=C,
                meta=dict(seed=seed, device=str(dev)))


def make_ternary_bf16_case(name, ks, M, N, seed=0, device="cpu"):
    """bf16 operands with values in {-1, 0, +1} and integer C in [-64, 64]: every
    partial sum of up to 2^24 tokens is an integer that fp32 holds exactly, so a
    result must equal the exact one bit for bit, however long the experts. Draw
    order: A, B, C."""
    ks = np.asarray(ks, dtype=np.int32)
    G = ks.size
    K_total = int(ks.astype(np.int64).sum())
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    A = torch.randint(-1, 2, (K_total, M), generator=gen, device=dev, dtype=torch.int8)
    B = torch.randint(-1, 2, (K_total, N), generator=gen, device=dev, dtype=torch.int8)
    C = torch.randint(-64, 65, (G, M, N), generator=gen, device=dev, dtype=torch.int32)
    return Case(name=name, G=G, M=M, N=N, ks=ks, dtype=BF16, gran_k=128,
                A=A.to(torch.bfloat16), B=B.to(torch.bfloat16), sa=None, sb=None,
                C=C.to(torch.float32), meta=dict(seed=seed, device=str(dev), ternary=True))


# (m, n, k) of the issue page's non-grouped 1D1D fp8 GEMM table
SINGLE_SHAPES = ((4096, 2112, 7168), (4096, 24576, 1536), (4096, 32768, 512),
                 (4096, 7168, 16384), (4096, 4096, 7168), (4096, 7168, 2048))


def single_name(m, n, k):
    return f"single_m{m}_n{n}_k{k}"


SINGLE = {single_name(*mnk): mnk for mnk in SINGLE_SHAPES}
WORKLOADS = ("worked", "bf16", "zipf_fp8", "ue8m0_many", "local_share") + tuple(SINGLE)


def workload(name, device="cpu", seed=0, gran_k=None):
    """The named workloads (see the module docstring). `gran_k` replaces an fp8
    workload's scale granularity (e.g. 32 for fp32 scales per 32 tokens)."""
    if gran_k is not None:
        return _regran(name, device, seed, gran_k)
    if name == "worked":
        return make_case(name, ks_worked(), 64, 128, E4M3_F32SCALE, 128, with_c=False,
                         seed=seed, device=device)
    if name == "bf16":
        ks = ks_uniform_with_empty(16384, 4, [1], seed)
        return make_case(name, ks, 1024, 2048, BF16, 128, with_c=True, seed=seed,
                         device=device, a_std=0.1, b_std=0.1)
    if name == "zipf_fp8":
        ks = ks_zipf(65536, 32, 1.2, seed)
        return make_case(name, ks, 7168, 4096, E4M3_F32SCALE, 128, with_c=True, seed=seed,
                         device=device, b_std=1e-3, a_outlier_p=0.01)
    if name == "ue8m0_many":
        ks = ks_topk(16384, 256, 8, 51, seed)
        return make_case(name, ks, 2048, 7168, E4M3_UE8M0, 32, with_c=False, seed=seed,
                         device=device)
    if name == "local_share":
        ks = ks_normal(262144, 8, 32768.0, 8192.0, seed)
        return make_case(name, ks, 7168, 4096, E4M3_F32SCALE, 128, with_c=True, seed=seed,
                         device=device, b_std=1e-3, a_outlier_p=0.01)
    if name in SINGLE:
        m, n, k = SINGLE[name]
        return make_case(name, np.array([k], np.int32), m, n, E4M3_F32SCALE, 128, with_c=False,
                         seed=seed, device=device)
    raise KeyError(name)


def _regran(name, device, seed, gran_k):
    spec = {"zipf_fp8": (7168, 4096, E4M3_F32SCALE, True, dict(b_std=1e-3, a_outlier_p=0.01)),
            "local_share": (7168, 4096, E4M3_F32SCALE, True, dict(b_std=1e-3, a_outlier_p=0.01)),
            "ue8m0_many": (2048, 7168, E4M3_UE8M0, False, {})}
    if name not in spec and name not in SINGLE:
        raise KeyError(f"{name}: no scale granularity to replace")
    if name in SINGLE:
        m, n, k = SINGLE[name]
        return make_case(name, np.array([k], np.int32), m, n, E4M3_F32SCALE, gran_k,
                         with_c=False, seed=seed, device=device)
    M, N, dt, with_c, kw = spec[name]
    return make_case(name, workload_ks(name, seed), M, N, dt, gran_k, with_c=with_c, seed=seed,
                     device=device, **kw)


def workload_ks(name, seed=0):
    """Routing of a named workload without generating its values."""
    if name in SINGLE:
        return np.array([SINGLE[name][2]], np.int32)
    return {
        "worked": lambda: ks_worked(),
        "bf16": lambda: ks_uniform_with_empty(16384, 4, [1], seed),
        "zipf_fp8": lambda: ks_zipf(65536, 32, 1.2, seed),
        "ue8m0_many": lambda: ks_topk(16384, 256, 8, 51, seed),
        "local_share": lambda: ks_normal(262144, 8, 32768.0, 8192.0, seed),
    }[name]()


# ----------------------------------------------------------------- M-grouped dgrad inputs

@dataclass
class DgradCase:
    """Inputs of the M-grouped data-gradient GEMM: expert g owns token rows
    [off[g], off[g+1]) of A = dy [M_total, K] (fp8, one fp32 scale per token per 128
    channels, stored [K/128, M_total]); W [G, K, N] is each expert's weight as the
    forward pass stores it (fp8, one fp32 scale per 128 x 128 block, [G, K/128, N/128])."""
    name: str
    G: int
    N: int
    K: int
    ms: np.ndarray          # int32 [G]
    A: torch.Tensor         # uint8 [M_total, K]
    sa: torch.Tensor        # float32 [K/128, M_total]
    W: torch.Tensor         # uint8 [G, K, N]
    sw: torch.Tensor        # float32 [G, K/128, N/128]

    @property
    def M_total(self) -> int:
        return int(self.ms.astype(np.int64).sum())

    @property
    def flops(self) -> int:
        return 2 * self.M_total * self.N * self.K

    def algorithmic_bytes(self, out_bytes: int = 2) -> int:
        """A, the weights of experts that have tokens, their scales and D (out_bytes per
        element) once."""
        live = int((self.ms > 0).sum())
        return (self.M_total * self.K + live * self.K * self.N + self.sa.numel() * 4
                + live * (self.K // 128) * (self.N // 128) * 4 + self.M_total * self.N * out_bytes)

    def host(self):
        cpu = lambda t: t.detach().cpu().numpy()
        return dict(A=cpu(self.A), sa=cpu(self.sa), W=cpu(self.W), sw=cpu(self.sw),
                    ms=self.ms.copy())


def quantize_rows_1x128(x: torch.Tensor):
    """x fp32 [R, K] -> (uint8 [R, K], fp32 scales [K/128, R]): one scale per row per
    128 columns, amax / 448 (1 for an all-zero run)."""
    R, K = x.shape
    xb = x.view(R, K // 128, 128)
    amax = xb.abs().amax(dim=2)
    scale = torch.where(amax == 0, torch.ones_like(amax), amax / FP8_MAX)
    y = torch.clamp(xb / scale[:, :, None], -FP8_MAX, FP8_MAX)
    q = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(R, K)
    return q, scale.t().contiguous()


def quantize_blocks_128x128(w: torch.Tensor):
    """w fp32 [G, K, N] -> (uint8 [G, K, N], fp32 scales [G, K/128, N/128])."""
    G, K, N = w.shape
    wb = w.view(G, K // 128, 128, N // 128, 128)
    amax = wb.abs().amax(dim=(2, 4))
    scale = torch.where(amax == 0, torch.ones_like(amax), amax / FP8_MAX)
    y = torch.clamp(wb / scale[:, :, None, :, None], -FP8_MAX, FP8_MAX)
    q = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(G, K, N)
    return q, scale


def make_dgrad_case(name, ms, N, K, seed=0, device="cpu", a_std=1.0, w_std=1.0):
    """Seeded dgrad inputs. Draw order: A (dy), then W."""
    ms = np.asarray(ms, dtype=np.int32)
    G = ms.size
    M_total = int(ms.astype(np.int64).sum())
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    a = _normal(gen, (M_total, K), dev, a_std)
    w = _normal(gen, (G, K, N), dev, w_std)
    A, sa = quantize_rows_1x128(a)
    del a
    W, sw = quantize_blocks_128x128(w)
    del w
    return DgradCase(name=name, G=G, N=N, K=K, ms=ms, A=A.contiguous(), sa=sa, W=W.contiguous(),
                     sw=sw.contiguous())


DGRAD_WORKLOADS = ("dgrad_local_share", "dgrad_ue8m0_many_down")


def dgrad_workload(name, device="cpu", seed=0):
    """dgrad_local_share: the data gradient paired with the local_share weight
    gradient (fused gate+up projection w [4096, 7168]: dx [262144, 7168] = dy
    [262144, 4096] w), routing of local_share. dgrad_ue8m0_many_down: the
    down projection of the many-expert layer (w [7168, 2048]: dx [131072, 2048] =
    dy [131072, 7168] w), routing of ue8m0_many (51 empty experts)."""
    if name == "dgrad_local_share":
        return make_dgrad_case(name, workload_ks("local_share", seed), 7168, 4096, seed=seed,
                               device=device)
    if name == "dgrad_ue8m0_many_down":
        return make_dgrad_case(name, workload_ks("ue8m0_many", seed), 2048, 7168, seed=seed,
                               device=device)
    raise KeyError(name)


def requant_edge_source(K, H, seed=0):
    """Requantiser edge-case source: fp32 [K, H], every value exactly representable in
    bf16. Column h follows pattern h % 16, each row-periodic so that any run of 8 or
    more tokens holds the pattern's largest magnitude:
      0  N(0,1) with +inf at every 32nd row
      1  N(0,1) with -inf at every 32nd row and NaN at every 5th
      2  all NaN
      3  zeros, every other one negative
      4  bf16 subnormals: +-j * 2^-133, j in 1..127
      5  small normals +-(1 + j/128) * 2^-120 .. 2^-125 (amax / 448 is subnormal)
      6-9  f * o * 2^k with f = 1, 3, 5, 7, o odd in 1..31, k in -12..3, and
           +-448 f at every 8th row (so that x / (amax / 448) = o * 2^k exactly)
      10 N(0,1) * 2^u, u uniform in -30..30
      11-15 N(0,1), 1% of entries x 50
    """
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((K, H)).astype(np.float32)
    fam = np.arange(H) % 16
    rows = np.arange(K)[:, None]
    sign = np.where(rng.random((K, H)) < 0.5, -1.0, 1.0).astype(np.float32)
    def put(mask_cols, vals):
        x[:, mask_cols] = vals[:, mask_cols]
    c = fam == 0
    x[:, c] = np.where(rows % 32 == 0, np.float32(np.inf), x[:, c])
    c = fam == 1
    v = np.where(rows % 5 == 0, np.float32(np.nan), x[:, c])
    x[:, c] = np.where(rows % 32 == 3, np.float32(-np.inf), v)
    x[:, fam == 2] = np.nan
    c = fam == 3
    x[:, c] = np.where(rows % 2 == 0, np.float32(0.0), np.float32(-0.0))
    j = rng.integers(1, 128, (K, H)).astype(np.float64)
    put(fam == 4, (sign * np.ldexp(j, -133)).astype(np.float32))
    e = rng.integers(-125, -119, (K, H))
    put(fam == 5, (sign * np.ldexp(1.0 + j / 128.0, e)).astype(np.float32))
    o = (2 * rng.integers(0, 16, (K, H)) + 1).astype(np.float64)
    k = rng.integers(-12, 4, (K, H))
    for f_id, f in zip((6, 7, 8, 9), (1.0, 3.0, 5.0, 7.0)):
        c = fam == f_id
        vals = (sign * f * np.ldexp(o, k)).astype(np.float32)
        vals = np.where(rows % 8 == 0, (sign * np.float32(448.0 * f)).astype(np.float32), vals)
        x[:, c] = vals[:, c]
    u = rng.integers(-30, 31, (K, H))
    put(fam == 10, np.ldexp(x.astype(np.float64), u).astype(np.float32))
    c = fam >= 11
    big = rng.random((K, H)) < 0.01
    x[:, c] = np.where(big[:, c], x[:, c] * 50, x[:, c])
    # every value to the nearest bf16 (the patterns above are exact already)
    return torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()


def requant_edge_fp8_source(K, H, seed=0):
    """Requantiser edge cases for the fp8 source with 1x128 per-token scales: e4m3fn
    bytes [K, H] (uint8) of every code, NaN codes 0x7F and 0xFF included, and fp32
    scales [K, H/128]: mostly 1e-4 .. 1e-2, with rows at 3e38 (products above 1
    overflow to infinity), 1e-40 (subnormal products) and 0. The last 80 rows hold
    codes of magnitude at most 224 with scales alternately 2^-149 (the smallest
    subnormal) and 0, so that the largest magnitude of a run there is at most
    224 * 2^-149."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, (K, H), dtype=np.uint8)
    xs = (rng.random((K, H // 128)) * 0.01 + 1e-4).astype(np.float32)
    xs[5::17] = np.float32(3e38)
    xs[7::19] = np.float32(1e-40)
    xs[11::23] = np.float32(0.0)
    tail = codes[-80:]
    codes[-80:] = np.where((tail & 0x7F) > 0x77, tail & 0xF7, tail)
    xs[-80:] = np.float32(2.0 ** -149)
    xs[-80::2] = np.float32(0.0)
    return codes, xs


# Requantiser workloads: (routing workload, H, gran_k, scale kind, source kind), the
# kinds as in the C ABI (scale: 0 fp32, 1 UE8M0; source: 0 bf16, 1 e4m3 with 1x128
# per-token scales)
REQUANT_WORKLOADS = {
    "local_share_A": ("local_share", 7168, 128, 0, 0),
    "local_share_A_fp8": ("local_share", 7168, 128, 0, 1),
    "ue8m0_many_B": ("ue8m0_many", 7168, 32, 1, 0),
}


def requant_source(name, device="cpu", seed=0):
    """The requantiser's source for a named workload: (X, xs, ks). X is N(0, 1) values
    [tokens, H] as bf16, or (source kind 1) as the forward pass's e4m3 copy with one
    fp32 scale per token per 128 channels (amax / 448, amax floored at 1e-30), xs
    [tokens, H / 128]; ks the workload's routing (numpy int32)."""
    wl, H, gran, kind, src = REQUANT_WORKLOADS[name]
    ks = workload_ks(wl, seed)
    K = int(ks.astype(np.int64).sum())
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    x = torch.randn((K, H), generator=gen, device=dev)
    if src == 0:
        return x.to(torch.bfloat16), None, ks
    amax = x.abs().view(K, H // 128, 128).amax(dim=2).clamp_min(1e-30)
    xs = (amax / FP8_MAX).float()
    X = (x.view(K, H // 128, 128) / xs[:, :, None]).view(K, H).to(torch.float8_e4m3fn)
    return X.view(torch.uint8), xs, ks

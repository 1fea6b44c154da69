"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module only draws random numbers and rounds them to the workload's
storage type; it holds none of the codec's arithmetic.  Every workload draws
its values in fp64 from NumPy's PCG64, one independent child stream per block
of rows (``SeedSequence(seed).spawn``), and rounds them (round-to-nearest-even)
to its dtype: fp32, or fp32 -> bfloat16.  A block of rows can therefore be
regenerated on its own, which lets a test rebuild any sampled row of a large
workload without drawing the rest.

bfloat16 values are returned as fp32 arrays whose values are exactly
representable in bfloat16 (``dtype`` says which type the GPU receives).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BLOCK = 4096  # rows per independent child stream


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp64/fp32 -> fp32 (RNE) -> bfloat16 (RNE); returned as fp32 values."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32)


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(dtype)


def _streams(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


@dataclass
class Gaussian:
    """Rows of i.i.d. N(0,1) vectors, optionally with per-group outlier channels
    and per-(group, token) log-normal row scales."""
    seed: int
    n_rows: int
    d: int
    dtype: str = "f32"
    # outliers: every `group_rows` consecutive rows share `n_outliers` channels x `outlier_scale`
    group_rows: int = 0
    n_outliers: int = 0
    outlier_scale: float = 1.0
    # log-normal token scale: scale index = row // heads_per_token_block ... see token_scale_of
    lognormal_sigma: float = 0.0
    token_layout: tuple = ()  # (batch, heads, tokens): row = (b*heads + h)*tokens + t
    _outlier_channels: np.ndarray | None = field(default=None, repr=False)

    def __post_init__(self):
        s_main, s_aux = np.random.SeedSequence(self.seed).spawn(2)
        self._main_seed = s_main
        self._aux_seed = s_aux
        n_blocks = max(1, math.ceil(self.n_rows / BLOCK))
        self._block_seeds = s_main.spawn(n_blocks)
        if self.n_outliers:
            rng = np.random.Generator(np.random.PCG64(s_aux))
            n_groups = self.n_rows // self.group_rows
            self._outlier_channels = np.stack(
                [rng.choice(self.d, self.n_outliers, replace=False) for _ in range(n_groups)])
        if self.lognormal_sigma:
            b, h, t = self.token_layout
            rng = np.random.Generator(np.random.PCG64(s_aux.spawn(1)[0]))
            self._token_scale = rng.lognormal(0.0, self.lognormal_sigma, size=(b, t))

    def rows64(self, lo: int, hi: int) -> np.ndarray:
        out = np.empty((hi - lo, self.d))
        b0, b1 = lo // BLOCK, (hi - 1) // BLOCK
        for blk in range(b0, b1 + 1):
            rng = np.random.Generator(np.random.PCG64(self._block_seeds[blk]))
            base = blk * BLOCK
            n = min(BLOCK, self.n_rows - base)
            vals = rng.standard_normal((n, self.d))
            s, e = max(lo, base), min(hi, base + n)
            out[s - lo:e - lo] = vals[s - base:e - base]
        rows = np.arange(lo, hi)
        if self.n_outliers:
            ch = self._outlier_channels[rows // self.group_rows]
            np.put_along_axis(out, ch, np.take_along_axis(out, ch, axis=1) * self.outlier_scale, axis=1)
        if self.lognormal_sigma:
            b, h, t = self.token_layout
            bi = rows // (h * t)
            ti = rows % t
            out *= self._token_scale[bi, ti][:, None]
        return out

    def rows(self, lo: int = 0, hi: int | None = None) -> np.ndarray:
        hi = self.n_rows if hi is None else hi
        return _cast(self.rows64(lo, hi), self.dtype)


@dataclass
class GaussianMixtureUnit:
    """Unit-length rows x = (μ_k + ε)/||μ_k + ε||, μ_k ~ N(0, I_d) for k < n_centers,
    k uniform, ε ~ N(0, I_d)."""
    seed: int
    n_rows: int
    d: int
    n_centers: int = 256
    dtype: str = "f32"
    centers_seed: int | None = None

    def __post_init__(self):
        s_c, s_main = np.random.SeedSequence(self.seed).spawn(2)
        cs = s_c if self.centers_seed is None else np.random.SeedSequence(self.centers_seed).spawn(2)[0]
        self.centers = np.random.Generator(np.random.PCG64(cs)).standard_normal((self.n_centers, self.d))
        self._block_seeds = s_main.spawn(max(1, math.ceil(self.n_rows / BLOCK)))

    def rows64(self, lo: int, hi: int) -> np.ndarray:
        out = np.empty((hi - lo, self.d))
        for blk in range(lo // BLOCK, (hi - 1) // BLOCK + 1):
            rng = np.random.Generator(np.random.PCG64(self._block_seeds[blk]))
            base = blk * BLOCK
            n = min(BLOCK, self.n_rows - base)
            comp = rng.integers(0, self.n_centers, size=n)
            x = self.centers[comp] + rng.standard_normal((n, self.d))
            x /= np.linalg.norm(x, axis=1, keepdims=True)
            s, e = max(lo, base), min(hi, base + n)
            out[s - lo:e - lo] = x[s - base:e - base]
        return out

    def rows(self, lo: int = 0, hi: int | None = None) -> np.ndarray:
        hi = self.n_rows if hi is None else hi
        return _cast(self.rows64(lo, hi), self.dtype)


@dataclass
class NeedleKeys:
    """Rows of a Gaussian workload plus beta · u_g on a seeded Bernoulli(p)
    subset of rows ("needles"), u_g a given unit vector per group of
    `group_rows` consecutive rows."""
    base: Gaussian
    directions: np.ndarray  # [n_groups][d], unit vectors
    group_rows: int
    p: float
    beta: float
    seed: int
    dtype: str = "bf16"

    def __post_init__(self):
        self.n_rows, self.d = self.base.n_rows, self.base.d
        self._block_seeds = np.random.SeedSequence(self.seed).spawn(max(1, math.ceil(self.n_rows / BLOCK)))

    def needles(self, lo: int = 0, hi: int | None = None) -> np.ndarray:
        hi = self.n_rows if hi is None else hi
        out = np.empty(hi - lo, dtype=bool)
        for blk in range(lo // BLOCK, (hi - 1) // BLOCK + 1):
            rng = np.random.Generator(np.random.PCG64(self._block_seeds[blk]))
            base = blk * BLOCK
            n = min(BLOCK, self.n_rows - base)
            m = rng.random(n) < self.p
            s, e = max(lo, base), min(hi, base + n)
            out[s - lo:e - lo] = m[s - base:e - base]
        return out

    def rows64(self, lo: int, hi: int) -> np.ndarray:
        out = self.base.rows64(lo, hi)
        m = self.needles(lo, hi)
        rows = np.arange(lo, hi)[m]
        out[m] += self.beta * self.directions[rows // self.group_rows]
        return out

    def rows(self, lo: int = 0, hi: int | None = None) -> np.ndarray:
        hi = self.n_rows if hi is None else hi
        return _cast(self.rows64(lo, hi), self.dtype)


# ---------------------------------------------------------------------------
# The five workloads (sizes can be shrunk for fast tests; defaults are full).
# Codec seed 1234 everywhere; data seed = workload number.
# ---------------------------------------------------------------------------
CODEC_SEED = 1234


def tiny_ref(n_keys=4096, d=128):
    """1 head, d=128, one fp32 query, 4096 fp32 keys N(0,1); 3-bit."""
    keys = Gaussian(seed=101, n_rows=n_keys, d=d, dtype="f32")
    q = Gaussian(seed=102, n_rows=1, d=d, dtype="f32")
    return dict(name="tiny_ref_4096x128_f32", bits=3, d=d, keys=keys, queries=q,
                batch=1, n_q_heads=1, n_kv_heads=1, n_queries=1, ctx=n_keys)


def llama8b_decode(ctx=32768, bits=3, batch=1, n_q_heads=32, n_kv_heads=8, d=128):
    """Llama-3.1-8B-shaped decode logits: 32 q heads / 8 KV heads, bf16 keys
    N(0,1) with 4 outlier channels per KV head scaled x10."""
    keys = Gaussian(seed=201, n_rows=batch * n_kv_heads * ctx, d=d, dtype="bf16",
                    group_rows=ctx, n_outliers=4, outlier_scale=10.0)
    q = Gaussian(seed=202, n_rows=batch * n_q_heads, d=d, dtype="bf16")
    return dict(name=f"llama8b_decode_ctx{ctx}_{bits}bit", bits=bits, d=d, keys=keys,
                queries=q, batch=batch, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                n_queries=1, ctx=ctx)


def prefill_encode(batch=16, ctx=8192, n_kv_heads=8, n_queries=16, d=128, bits=3):
    """bf16 K and V [batch][heads][ctx][d]: per (batch, token) one
    LogNormal(0, 0.5) scale shared by that token's heads times N(0, I) rows;
    16 decode queries per sequence (one query head per KV head)."""
    lay = (batch, n_kv_heads, ctx)
    keys = Gaussian(seed=301, n_rows=batch * n_kv_heads * ctx, d=d, dtype="bf16",
                    lognormal_sigma=0.5, token_layout=lay)
    vals = Gaussian(seed=302, n_rows=batch * n_kv_heads * ctx, d=d, dtype="bf16",
                    lognormal_sigma=0.5, token_layout=lay)
    q = Gaussian(seed=303, n_rows=batch * n_queries * n_kv_heads, d=d, dtype="bf16")
    return dict(name=f"prefill_b{batch}_ctx{ctx}_{bits}bit", bits=bits, d=d, keys=keys,
                values=vals, queries=q, batch=batch, n_q_heads=n_kv_heads,
                n_kv_heads=n_kv_heads, n_queries=n_queries, ctx=ctx)


def long_decode(ctx=131072, batch=1, n_q_heads=32, n_kv_heads=8, d=128, bits=3):
    """Fused decode attention: bf16 K, V N(0,1), 32 q heads / 8 KV heads,
    temperature 1/sqrt(128), bf16 output."""
    keys = Gaussian(seed=401, n_rows=batch * n_kv_heads * ctx, d=d, dtype="bf16")
    vals = Gaussian(seed=402, n_rows=batch * n_kv_heads * ctx, d=d, dtype="bf16")
    q = Gaussian(seed=403, n_rows=batch * n_q_heads, d=d, dtype="bf16")
    return dict(name=f"long_decode_ctx{ctx}_{bits}bit", bits=bits, d=d, keys=keys, values=vals,
                queries=q, batch=batch, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                n_queries=1, ctx=ctx, scale=1.0 / math.sqrt(d))


def long_decode_needles(ctx=131072, batch=1, n_q_heads=32, n_kv_heads=8, d=128, bits=3, p=1.0 / 512,
                        beta=64.0):
    """The long-context decode workload with peaked attention: the same bf16
    queries, haystack keys and values, plus, with probability p per (KV head,
    position), a needle key z + beta·u, u the unit vector of the sum of that
    KV head's query heads.  A needle then scores about beta/2 above a
    haystack key for every query head of the group, so almost all of the
    softmax weight sits on the needles."""
    w = long_decode(ctx=ctx, batch=batch, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, d=d, bits=bits)
    G = n_q_heads // n_kv_heads
    q = w["queries"].rows().astype(np.float64).reshape(batch, n_kv_heads, G, d).sum(axis=2)
    u = (q / np.linalg.norm(q, axis=-1, keepdims=True)).reshape(batch * n_kv_heads, d)
    w["keys"] = NeedleKeys(base=w["keys"], directions=u, group_rows=ctx, p=p, beta=beta, seed=404)
    w["name"] = f"long_decode_needles_ctx{ctx}_{bits}bit"
    w["needle_p"], w["needle_beta"] = p, beta
    return w


def vector_search(n_db=1_000_000, n_queries=1024, d=1536, n_centers=256, bits=4, k=10):
    """fp32 unit vectors from a 256-centre Gaussian mixture; 4-bit; top-10."""
    db = GaussianMixtureUnit(seed=501, n_rows=n_db, d=d, n_centers=n_centers)
    q = GaussianMixtureUnit(seed=502, n_rows=n_queries, d=d, n_centers=n_centers, centers_seed=501)
    return dict(name=f"search_{n_db}x{d}_{bits}bit", bits=bits, d=d, db=db, queries=q, k=k)


def vector_search_torch(device, n_db=1_000_000, n_queries=1024, d=1536, n_centers=256, chunk=65536):
    """The vector-search workload drawn on the GPU (torch Philox, seeded), for
    full-size runs where drawing 1.5e9 normals in NumPy would dominate:
    centres μ_k ~ N(0, I_d) (k < 256), row = μ_k + N(0, I_d) with k uniform,
    normalised to unit length; fp32.  Database seed 501, query seed 502,
    centres from the database generator."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(501)
    centers = torch.randn((n_centers, d), generator=g, device=device)
    db = torch.empty((n_db, d), dtype=torch.float32, device=device)
    for s in range(0, n_db, chunk):
        e = min(n_db, s + chunk)
        comp = torch.randint(0, n_centers, (e - s,), generator=g, device=device)
        x = centers[comp] + torch.randn((e - s, d), generator=g, device=device)
        db[s:e] = x / x.norm(dim=1, keepdim=True)
    gq = torch.Generator(device=device)
    gq.manual_seed(502)
    comp = torch.randint(0, n_centers, (n_queries,), generator=gq, device=device)
    q = centers[comp] + torch.randn((n_queries, d), generator=gq, device=device)
    q = q / q.norm(dim=1, keepdim=True)
    return db, q.contiguous()

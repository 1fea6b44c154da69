"""TurboQuant oracle: fp64 NumPy, step by step, CPU only (test infrastructure).

Pages cited (each comment names the page title and the section):

* 「TurboQuant 学习路径：论文 → 技术 → 数学」 (zzszmyf.github.io notes) —
  二.2 JL transforms (Gaussian JL, FJLT y = P·H·D·x), 三.1 table (orthogonal
  matrices, Hadamard recursion), 三.4 (Lloyd-Max).
* 「谷歌 TurboQuant 深度拆解：LLM 内存压缩 6 倍、推理加速 8 倍、零精度损失，
  它是怎么做到的？」 (juejin.cn) — 第二部分 (two-stage method: random rotation,
  optimal scalar quantizer with no per-block constants, QJL sign bits and an
  unbiased estimator), 第六部分 (distortion lower bounds, the post-rotation
  coordinate density, unbiasedness of the QJL estimator).
* 「TurboQuant+ 深度解析：当前 Google 工程师决定单挑大厂」 (zhichai.net) —
  第二部分 (the rotation is a random-sign Walsh–Hadamard transform),
  第四部分 (the rotation needs high precision), 第五部分 (K and V compressed
  the same way), 第六部分 (Sparse V).

Readings where the pages leave a step open are marked "Reading:".

Parity status: every function here is pinned by a CPU test in
``tests/test_oracle_*.py`` (closed forms, textbook special cases, brute force,
invariants, Monte-Carlo unbiasedness) except the absolute per-key values,
which depend on the seeded rotation and projection and which the pages give no
worked example for: those are "parity unpinned" beyond the pins of their parts.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
from scipy import integrate, special

__all__ = [
    "splitmix64", "rademacher_signs", "gaussian_matrix",
    "sylvester_hadamard", "paley_hadamard_12", "hadamard", "rotation_matrix",
    "sphere_coordinate_density", "sphere_coordinate_cdf",
    "sphere_coordinate_first_moment", "lloyd_max", "walsh_plane_coefficients",
    "Codec", "make_codec", "make_mse_codec", "qjl_constant",
    "pack_planes", "unpack_planes", "pack_bits", "unpack_bits",
    "encode", "encode_given_codes", "dequantize",
    "prepare_query", "score", "attn_logits",
    "decode_attn_materialized", "decode_attn_accumulated", "decode_attn_sparse_v",
    "decode_attn_sparse_v_plain",
    "paged_row", "append_paged", "gather_paged", "decode_attn_paged",
    "vblock_pack", "vblock_unpack",
    "polar_angle_cdf", "polar_angle_density", "polar_lloyd_max", "polar_transform", "polar_reconstruct",
    "polar_slots", "PolarCodec", "make_polar_codec", "polar_encode", "polar_encode_given_codes",
    "polar_dequantize", "polar_score",
    "search_topk", "bf16_round",
]

_MASK64 = (1 << 64) - 1
_GOLDEN = 0x9E3779B97F4A7C15
TAG_SIGNS = 1
TAG_GAUSS = 2


# --------------------------------------------------------------------------
# O1. Seeded randomness: SplitMix64 (Steele, Lea & Flood, OOPSLA 2014).
# The pages only ask for "random signs" (学习路径 二.2 FJLT, D) and a Gaussian
# JL matrix with i.i.d. N(0,1) entries (学习路径 二.2 standard JL).
# Reading: both come from a counter-based SplitMix64 stream keyed by
# (seed XOR tag); Gaussians by Box–Muller (Box & Muller 1958).
# --------------------------------------------------------------------------
def splitmix64(seed: int, tag: int, idx) -> np.ndarray:
    """Output number ``idx`` (0-based) of SplitMix64 seeded with seed ^ tag.

    SplitMix64 adds the golden-ratio increment to its state before each output,
    so output i is the mix function applied to state0 + (i+1)*0x9E37...7C15.
    """
    idx = np.asarray(idx, dtype=np.uint64)
    s0 = np.uint64((int(seed) ^ int(tag)) & _MASK64)
    with np.errstate(over="ignore"):
        z = s0 + (idx + np.uint64(1)) * np.uint64(_GOLDEN)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        z = z ^ (z >> np.uint64(31))
    return z


def rademacher_signs(d: int, seed: int) -> np.ndarray:
    """D_j = +1 when the top bit of word(seed, 1, j) is 0, else -1 (fp64)."""
    w = splitmix64(seed, TAG_SIGNS, np.arange(d, dtype=np.uint64))
    top = (w >> np.uint64(63)).astype(np.int64)
    return np.where(top == 0, 1.0, -1.0)


def gaussian_matrix(m: int, d: int, seed: int) -> np.ndarray:
    """QJL matrix S (m x d), i.i.d. N(0,1), rounded to fp32 (canonical values).

    Entry k = i*d + j (row-major) belongs to pair P = k // 2, which draws
    w1 = word(seed, 2, 2P), w2 = word(seed, 2, 2P+1);
    u1 = ((w1 >> 11) + 1) * 2^-53 in (0, 1], u2 = (w2 >> 11) * 2^-53 in [0, 1);
    even k takes sqrt(-2 ln u1) cos(2 pi u2), odd k the sine (Box–Muller).
    """
    n = m * d
    assert n % 2 == 0
    pairs = np.arange(n // 2, dtype=np.uint64)
    w1 = splitmix64(seed, TAG_GAUSS, 2 * pairs)
    w2 = splitmix64(seed, TAG_GAUSS, 2 * pairs + np.uint64(1))
    u1 = ((w1 >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53
    u2 = (w2 >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    rad = np.sqrt(-2.0 * np.log(u1))
    ang = 2.0 * math.pi * u2
    out = np.empty(n, dtype=np.float64)
    out[0::2] = rad * np.cos(ang)
    out[1::2] = rad * np.sin(ang)
    return out.astype(np.float32).reshape(m, d)


# --------------------------------------------------------------------------
# O2. Rotation R = H D / sqrt(d)  (学习路径 二.2: FJLT is P·H·D·x; 三.1: an
# orthogonal R has R^T R = I and keeps norms, and H_n = H_1 ⊗ H_{n-1};
# TurboQuant+ 深度解析 第二部分: the rotation is a Walsh–Hadamard transform).
# Reading: no subsampling P (it would not be orthogonal); Sylvester natural
# order; for d = 12 * 2^k (d = 1536) H = H12 ⊗ H_{2^k} with H12 the Paley
# type-I matrix (Paley 1933, q = 11), since no Sylvester matrix of that order
# exists.
# --------------------------------------------------------------------------
def sylvester_hadamard(n: int) -> np.ndarray:
    """H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]] (natural order), int64."""
    if n < 1 or n & (n - 1):
        raise ValueError("Sylvester order must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def _legendre(a: int, q: int) -> int:
    a %= q
    if a == 0:
        return 0
    return 1 if pow(a, (q - 1) // 2, q) == 1 else -1


def paley_hadamard_12() -> np.ndarray:
    """Paley type-I Hadamard matrix of order 12 (q = 11, q ≡ 3 mod 4).

    Q_ij = chi(j - i) over GF(11) (chi = quadratic character, chi(0) = 0);
    S = [[0, 1^T], [-1, Q]] is skew-symmetric and H = I + S.
    """
    q = 11
    Q = np.array([[_legendre(j - i, q) for j in range(q)] for i in range(q)],
                 dtype=np.int64)
    S = np.zeros((q + 1, q + 1), dtype=np.int64)
    S[0, 1:] = 1
    S[1:, 0] = -1
    S[1:, 1:] = Q
    return np.eye(q + 1, dtype=np.int64) + S


def hadamard(d: int) -> np.ndarray:
    """Dense ±1 Hadamard matrix of order d (power of two, or 12 * power of two)."""
    if d >= 1 and d & (d - 1) == 0:
        return sylvester_hadamard(d)
    if d % 12 == 0 and (d // 12) & (d // 12 - 1) == 0:
        return np.kron(paley_hadamard_12(), sylvester_hadamard(d // 12))
    raise ValueError(f"no Hadamard construction for d={d}")


def rotation_matrix(d: int, seed: int) -> np.ndarray:
    """R = H diag(D) / sqrt(d), fp64, applied as y = R u."""
    H = hadamard(d).astype(np.float64)
    D = rademacher_signs(d, seed)
    return H * D[None, :] / math.sqrt(d)


# --------------------------------------------------------------------------
# O3. Codebook: Lloyd-Max (学习路径 三.4) for the coordinate law of a rotated
# unit vector (深度拆解 第六部分: f(x) = Γ(d/2)/(√π Γ((d-1)/2)) (1-x²)^((d-3)/2)
# on [-1, 1]; 深度拆解 第二部分: fixed known law, so no per-block constants).
# Reading: the sphere law itself (not its Gaussian limit); X = 2B - 1 with
# B ~ Beta((d-1)/2, (d-1)/2), so its CDF is a regularized incomplete beta.
# --------------------------------------------------------------------------
def _log_norm_const(d: int) -> float:
    return math.lgamma(d / 2) - 0.5 * math.log(math.pi) - math.lgamma((d - 1) / 2)


def sphere_coordinate_density(x, d: int):
    x = np.asarray(x, dtype=np.float64)
    alpha = (d - 3) / 2
    return math.exp(_log_norm_const(d)) * np.power(np.clip(1 - x * x, 0, None), alpha)


def sphere_coordinate_cdf(t, d: int):
    a = (d - 1) / 2
    t = np.clip(np.asarray(t, dtype=np.float64), -1.0, 1.0)
    return special.betainc(a, a, (1.0 + t) / 2.0)


def sphere_coordinate_first_moment(lo, hi, d: int):
    """∫_lo^hi x f(x) dx in closed form: the antiderivative of x(1-x²)^α is
    -(1-x²)^(α+1) / (2(α+1))."""
    a1 = (d - 1) / 2  # alpha + 1
    lo = np.asarray(lo, dtype=np.float64)
    hi = np.asarray(hi, dtype=np.float64)
    c = math.exp(_log_norm_const(d))
    g = lambda x: np.power(np.clip(1 - x * x, 0, None), a1)
    return c / (2 * a1) * (g(lo) - g(hi))


def lloyd_max(d: int, b: int, tol: float = 1e-13, max_iter: int = 5000):
    """Lloyd-Max quantizer with 2^b levels for the sphere coordinate law.

    Start at Gaussian quantiles (k+1/2)/2^b scaled by 1/sqrt(d); iterate
    boundaries = midpoints (nearest neighbour), centroids = conditional means
    (centroid condition), keep the codebook symmetric; stop when the largest
    centroid change, in units of 1/sqrt(d), is below ``tol``.  Returns (centroids, boundaries, iters),
    centroids ascending, fp64.
    """
    L = 1 << b
    c = special.ndtri((np.arange(L) + 0.5) / L) / math.sqrt(d)
    it = 0
    for it in range(1, max_iter + 1):
        t = 0.5 * (c[:-1] + c[1:])
        edges = np.concatenate([[-1.0], t, [1.0]])
        mass = sphere_coordinate_cdf(edges[1:], d) - sphere_coordinate_cdf(edges[:-1], d)
        mom = sphere_coordinate_first_moment(edges[:-1], edges[1:], d)
        new = mom / mass
        new = 0.5 * (new - new[::-1])
        delta = float(np.max(np.abs(new - c))) * math.sqrt(d)
        c = new
        if delta < tol:
            break
    t = 0.5 * (c[:-1] + c[1:])
    return c, t, it


def walsh_plane_coefficients(centroids: np.ndarray) -> dict:
    """Expansion of c[idx] over the bits of idx (Walsh basis x_i = 2 b_i - 1).

    Returns {frozenset(S): coefficient} for every subset S of bit positions;
    for a symmetric codebook only odd |S| are non-zero.  Used by tests only.
    """
    L = len(centroids)
    b = L.bit_length() - 1
    out = {}
    for mask in range(L):
        S = frozenset(i for i in range(b) if mask >> i & 1)
        acc = 0.0
        for idx in range(L):
            sgn = 1.0
            for i in S:
                sgn *= 2 * ((idx >> i) & 1) - 1
            acc += centroids[idx] * sgn
        out[S] = acc / L
    return out


def qjl_constant(m: int) -> float:
    """sqrt(pi/2)/m.  For g ~ N(0, I) and any r ≠ 0,
    E[<g, q> sign(<g, r>)] = sqrt(2/pi) <q, r>/||r||, so
    sqrt(pi/2)/m * ||r|| * sum_i <s_i, q> sign(<s_i, r>) is unbiased for <q, r>
    (深度拆解 第二部分/第六部分: the QJL estimator is unbiased, variance ~ 1/m)."""
    return math.sqrt(math.pi / 2) / m


# --------------------------------------------------------------------------
# Codec = everything fixed by (d, bits, m, seed); data-oblivious
# (深度拆解 第二部分: no training, no calibration).
# Reading: bits = 1 + b, b bits of Lloyd-Max code plus 1 QJL bit per
# projected coordinate with m = d ("2 bits + 1 bit = 3 bits").
# --------------------------------------------------------------------------
@dataclass
class Codec:
    d: int
    bits: int
    m: int
    seed: int
    D: np.ndarray           # (d,) ±1
    R: np.ndarray           # (d, d) fp64 rotation
    S: np.ndarray           # (m, d) fp32 canonical
    centroids: np.ndarray   # (2^b,) fp64 ascending
    bounds: np.ndarray      # (2^b - 1,) fp64
    iters: int
    qjl: bool = True        # False: first stage only (see make_mse_codec)

    @property
    def b(self) -> int:
        return self.bits - 1 if self.qjl else self.bits

    @property
    def c32(self) -> np.ndarray:
        return self.centroids.astype(np.float32)

    @property
    def t32(self) -> np.ndarray:
        return self.bounds.astype(np.float32)

    @property
    def code_words(self) -> int:
        return self.b * self.d // 32

    @property
    def sign_words(self) -> int:
        return self.m // 32

    @property
    def record_bytes(self) -> int:
        return 4 * (self.code_words + self.sign_words) + (8 if self.qjl else 4)


def make_codec(d: int, bits: int, m: int | None = None, seed: int = 1234) -> Codec:
    m = d if m is None else m
    if bits < 2:
        raise ValueError("bits must be >= 2 (b >= 1 MSE bits plus 1 QJL bit)")
    c, t, it = lloyd_max(d, bits - 1)
    return Codec(d=d, bits=bits, m=m, seed=seed, D=rademacher_signs(d, seed),
                 R=rotation_matrix(d, seed), S=gaussian_matrix(m, d, seed),
                 centroids=c, bounds=t, iters=it)


# --------------------------------------------------------------------------
# MSE-only codec for values.  TurboQuant+ 深度解析 第五部分 reports that the
# value cache tolerates much coarser compression than the key cache (keys route
# attention, values only carry what is read).  Reading: a value codec may drop
# the QJL stage and give all `bits` to the first stage's Lloyd-Max code (the
# two-stage split of 深度拆解 第二部分 exists to make inner products with a
# query unbiased, which the value path does not need).  The record is the
# codes and ν only, and v̂ = ν Rᵀ c[idx], the reconstruction of least mean
# squared error for the codebook.  Such a codec has no unbiased score, so it
# never serves as a key codec.
# --------------------------------------------------------------------------
def make_mse_codec(d: int, bits: int, seed: int = 1234) -> Codec:
    if bits < 1:
        raise ValueError("bits must be >= 1")
    c, t, it = lloyd_max(d, bits)
    return Codec(d=d, bits=bits, m=0, seed=seed, D=rademacher_signs(d, seed),
                 R=rotation_matrix(d, seed), S=np.zeros((0, d), np.float32),
                 centroids=c, bounds=t, iters=it, qjl=False)


# --------------------------------------------------------------------------
# Packed record format (学习路径 二.4: pack low-bit integers into 32-bit words).
# Codes: bit-planes.  Plane p holds bit p of every code; coordinate j of plane
# p is bit (j % 32) of word p*(d/32) + j//32.  Signs: QJL bit i is bit (i % 32)
# of word i//32.  Norms ν = ||x|| and γ = ||r|| are fp32 side arrays.
# --------------------------------------------------------------------------
def pack_bits(bits: np.ndarray) -> np.ndarray:
    """(n, L) array of 0/1 -> (n, L/32) uint32, bit i -> word i//32, bit i%32."""
    n, L = bits.shape
    assert L % 32 == 0
    b = bits.astype(np.uint64).reshape(n, L // 32, 32)
    w = (b << np.arange(32, dtype=np.uint64)).sum(axis=2)
    return w.astype(np.uint32)


def unpack_bits(words: np.ndarray, L: int) -> np.ndarray:
    n = words.shape[0]
    w = words.astype(np.uint64).reshape(n, -1, 1)
    bits = (w >> np.arange(32, dtype=np.uint64)) & np.uint64(1)
    return bits.reshape(n, -1)[:, :L].astype(np.int64)


def pack_planes(idx: np.ndarray, b: int) -> np.ndarray:
    n, d = idx.shape
    planes = [pack_bits((idx >> p) & 1) for p in range(b)]
    return np.concatenate(planes, axis=1) if planes else np.zeros((n, 0), np.uint32)


def unpack_planes(codes: np.ndarray, b: int, d: int) -> np.ndarray:
    wpp = d // 32
    idx = np.zeros((codes.shape[0], d), dtype=np.int64)
    for p in range(b):
        idx |= unpack_bits(codes[:, p * wpp:(p + 1) * wpp], d) << p
    return idx


# --------------------------------------------------------------------------
# O4. Encode (深度拆解 第二部分: rotate, quantize each coordinate with the
# fixed optimal scalar quantizer, project the residual with a JL matrix and
# keep one sign bit per projected coordinate).
# Readings: store ν = ||x|| and quantize u = x/ν (学习路径 三.1 polar split
# x = r·x̂); the residual and S act in the rotated domain; idx_j counts the
# boundaries strictly below y_j (ties go low); sign(0) = +1; ν = 0 gives y = 0.
# Decisions (idx, sign) are taken in fp32, the kernels' precision: y and the
# boundaries are rounded to fp32 before comparing.
# --------------------------------------------------------------------------
def encode(codec: Codec, x: np.ndarray, chunk: int = 16384) -> dict:
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    out = {k: [] for k in ("codes", "signs", "norm", "rnorm", "y", "idx", "z", "r")}
    for s in range(0, n, chunk):
        xs = x[s:s + chunk]
        nu = np.sqrt(np.sum(xs * xs, axis=1))
        safe = np.where(nu > 0, nu, 1.0)
        u = np.where(nu[:, None] > 0, xs / safe[:, None], 0.0)
        y = u @ codec.R.T
        idx = np.sum(codec.t32.astype(np.float64)[None, None, :]
                     < y.astype(np.float32).astype(np.float64)[:, :, None], axis=2)
        r, gamma, z, sbits = _residual_and_signs(codec, y, idx)
        out["codes"].append(pack_planes(idx, codec.b))
        out["signs"].append(pack_bits(sbits))
        out["norm"].append(nu.astype(np.float32))
        out["rnorm"].append(gamma.astype(np.float32))
        out["y"].append(y)
        out["idx"].append(idx)
        out["z"].append(z)
        out["r"].append(r)
    return {k: (np.concatenate(v, axis=0) if v else v) for k, v in out.items()}


def _residual_and_signs(codec: Codec, y, idx):
    yhat = codec.c32.astype(np.float64)[idx]
    r = y - yhat
    gamma = np.sqrt(np.sum(r * r, axis=1))
    z = r @ codec.S.astype(np.float64).T
    sbits = (z >= 0).astype(np.int64)
    return r, gamma, z, sbits


def encode_given_codes(codec: Codec, x: np.ndarray, idx: np.ndarray) -> dict:
    """Re-derive r, γ, z and the signs of x when its codes are fixed to ``idx``
    (used when a code legitimately differs within the boundary band)."""
    x = np.asarray(x, dtype=np.float64)
    nu = np.sqrt(np.sum(x * x, axis=1))
    safe = np.where(nu > 0, nu, 1.0)
    u = np.where(nu[:, None] > 0, x / safe[:, None], 0.0)
    y = u @ codec.R.T
    r, gamma, z, sbits = _residual_and_signs(codec, y, np.asarray(idx, np.int64))
    return {"signs": pack_bits(sbits), "rnorm": gamma.astype(np.float32), "z": z,
            "y": y, "r": r}


def _unpack_record(codec: Codec, packed: dict):
    idx = unpack_planes(np.asarray(packed["codes"]), codec.b, codec.d)
    nu = np.asarray(packed["norm"], dtype=np.float32).astype(np.float64)
    if not codec.qjl:  # MSE-only records hold no signs and no γ
        n = idx.shape[0]
        return idx, np.zeros((n, 0)), nu, np.zeros(n)
    tau = 2 * unpack_bits(np.asarray(packed["signs"]), codec.m) - 1
    gamma = np.asarray(packed["rnorm"], dtype=np.float32).astype(np.float64)
    return idx, tau.astype(np.float64), nu, gamma


def dequantize(codec: Codec, packed: dict) -> np.ndarray:
    """v̂ = ν Rᵀ (c[idx] + sqrt(pi/2)/m · γ · Sᵀ τ): the unbiased reconstruction
    (E_S[Sᵀ sign(S r)] = sqrt(2/pi) m r/||r||); ν Rᵀ c[idx] for an MSE-only codec."""
    if isinstance(codec, PolarCodec):  # the recursive polar first stage (O8)
        return polar_dequantize(codec, packed)
    idx, tau, nu, gamma = _unpack_record(codec, packed)
    chat = codec.c32.astype(np.float64)[idx]
    if not codec.qjl:
        return nu[:, None] * (chat @ codec.R)
    corr = qjl_constant(codec.m) * gamma[:, None] * (tau @ codec.S.astype(np.float64))
    return nu[:, None] * ((chat + corr) @ codec.R)


# --------------------------------------------------------------------------
# O5. Score (深度拆解 第二部分: a full-precision query against the compressed
# key, unbiased): q' = R q, p = S q',
# ℓ = ν (Σ_j q'_j c[idx_j] + sqrt(pi/2)/m · γ · Σ_i p_i τ_i),
# with the fp32-stored ν, γ and the fp32 centroids.
# --------------------------------------------------------------------------
def prepare_query(codec: Codec, q: np.ndarray):
    q = np.asarray(q, dtype=np.float64)
    qr = q @ codec.R.T
    p = qr @ codec.S.astype(np.float64).T
    return qr, p


def score(codec: Codec, q: np.ndarray, packed: dict) -> np.ndarray:
    """Logits of every query row against every packed key: (n_q, n_keys) fp64."""
    if isinstance(codec, PolarCodec):  # the recursive polar first stage (O8)
        return polar_score(codec, q, packed)
    if not codec.qjl:
        raise ValueError("an MSE-only codec has no unbiased score; keys take the two-stage codec")
    qr, p = prepare_query(codec, np.atleast_2d(q))
    idx, tau, nu, gamma = _unpack_record(codec, packed)
    chat = codec.c32.astype(np.float64)[idx]
    mse = qr @ chat.T
    qjl = p @ tau.T
    return nu[None, :] * (mse + qjl_constant(codec.m) * gamma[None, :] * qjl)


def _slice_packed(packed: dict, lo: int, hi: int) -> dict:
    return {k: np.asarray(packed[k])[lo:hi] for k in ("codes", "signs", "norm", "rnorm")}


def attn_logits(codec: Codec, q: np.ndarray, packed: dict, batch: int,
                n_q_heads: int, n_kv_heads: int, n_queries: int, ctx_len: int):
    """q: (batch, n_queries, n_q_heads, d); key rows ordered (batch, kv_head, t).
    Returns logits (batch, n_q_heads, n_queries, ctx_len).  Query head h reads
    KV head h // (n_q_heads // n_kv_heads) (consecutive grouping)."""
    G = n_q_heads // n_kv_heads
    q = np.asarray(q, dtype=np.float64).reshape(batch, n_queries, n_q_heads, codec.d)
    out = np.zeros((batch, n_q_heads, n_queries, ctx_len))
    for bi in range(batch):
        for kh in range(n_kv_heads):
            row0 = (bi * n_kv_heads + kh) * ctx_len
            keys = _slice_packed(packed, row0, row0 + ctx_len)
            for g in range(G):
                h = kh * G + g
                out[bi, h] = score(codec, q[bi, :, h, :], keys)
    return out


# --------------------------------------------------------------------------
# O6. Fused decode attention: w = softmax(scale · ℓ) over the context,
# o = Σ_i w_i v̂_i (V compressed like K: TurboQuant+ 深度解析 第五部分).
# Two formulations that must agree: materialize every v̂_i, or accumulate
# M = Σ w ν c[idx] and J = Σ w ν γ τ first and map back once.  Either codec
# may take the recursive polar first stage of O8 instead (深度拆解 第二部分
# 第三步 compresses the whole KV cache that way): its score and v̂ keep the
# same form with ŷ, rebuilt from the angle codes, in place of c[idx].
# --------------------------------------------------------------------------
def _softmax_weights(logits: np.ndarray, scale: float):
    s = scale * logits
    mx = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - mx)
    return e, np.sum(e, axis=-1, keepdims=True)


def decode_attn_materialized(codec_k: Codec, codec_v: Codec, q, k_packed, v_packed,
                             batch, n_q_heads, n_kv_heads, ctx_len, scale):
    q = np.asarray(q, dtype=np.float64).reshape(batch, n_q_heads, codec_k.d)
    G = n_q_heads // n_kv_heads
    out = np.zeros((batch, n_q_heads, codec_v.d))
    for bi in range(batch):
        for kh in range(n_kv_heads):
            row0 = (bi * n_kv_heads + kh) * ctx_len
            keys = _slice_packed(k_packed, row0, row0 + ctx_len)
            vals = dequantize(codec_v, _slice_packed(v_packed, row0, row0 + ctx_len))
            hs = slice(kh * G, (kh + 1) * G)
            lg = score(codec_k, q[bi, hs], keys)
            e, l = _softmax_weights(lg, scale)
            out[bi, hs] = (e / l) @ vals
    return out


def decode_attn_accumulated(codec_k: Codec, codec_v: Codec, q, k_packed, v_packed,
                            batch, n_q_heads, n_kv_heads, ctx_len, scale):
    q = np.asarray(q, dtype=np.float64).reshape(batch, n_q_heads, codec_k.d)
    G = n_q_heads // n_kv_heads
    out = np.zeros((batch, n_q_heads, codec_v.d))
    kv = qjl_constant(codec_v.m) if codec_v.qjl else 0.0
    S = codec_v.S.astype(np.float64)
    for bi in range(batch):
        for kh in range(n_kv_heads):
            row0 = (bi * n_kv_heads + kh) * ctx_len
            keys = _slice_packed(k_packed, row0, row0 + ctx_len)
            vals = _slice_packed(v_packed, row0, row0 + ctx_len)
            if isinstance(codec_v, PolarCodec):  # ŷ rebuilt from the angle codes (O8)
                chat, tau, nu, gamma = _polar_unpack(codec_v, vals)
            else:
                idx, tau, nu, gamma = _unpack_record(codec_v, vals)
                chat = codec_v.c32.astype(np.float64)[idx]
            hs = slice(kh * G, (kh + 1) * G)
            lg = score(codec_k, q[bi, hs], keys)
            e, l = _softmax_weights(lg, scale)
            M = (e * nu[None, :]) @ chat
            o_rot = M / l
            if codec_v.qjl:
                J = (e * (nu * gamma)[None, :]) @ tau
                o_rot = o_rot + kv * (J @ S) / l
            out[bi, hs] = o_rot @ codec_v.R
    return out


# --------------------------------------------------------------------------
# O6b. Sparse V (TurboQuant+ 深度解析 第六部分 Sparse V Dequant): the
# attention weights act as a gate, and a position whose weight is below a
# threshold (1e-6 on that page) does not have its value decompressed or added.
#
# Reading: the weight the gate tests is the one known where the value is
# accumulated.  Decode attention is split over the context into chunks of
# `chunk` consecutive positions; inside a chunk the weight of position t for
# query head h is exp(s_ht - m_hc) / l_hc, with m_hc and l_hc the maximum and
# the sum of exp(s - m_hc) of head h's scaled scores over that chunk.  Since
# the whole-context normaliser satisfies l·e^m >= l_hc·e^(m_hc), this
# chunk-local weight is never below the final softmax weight, so every
# position the gate drops has a final weight below the threshold too.  The
# gate is taken per (query head, position); the normaliser l still sums every
# position, only the value term is dropped.  With one chunk spanning the
# context the gate is exactly "final weight < threshold".
# --------------------------------------------------------------------------
def decode_attn_sparse_v(codec_k: Codec, codec_v: Codec, q, k_packed, v_packed,
                         batch, n_q_heads, n_kv_heads, ctx_len, scale, gate, chunk):
    """Returns (out [batch][n_q_heads][d], keep [batch][n_q_heads][ctx_len]
    bool, local [batch][n_q_heads][ctx_len] chunk-local weights)."""
    q = np.asarray(q, dtype=np.float64).reshape(batch, n_q_heads, codec_k.d)
    G = n_q_heads // n_kv_heads
    out = np.zeros((batch, n_q_heads, codec_v.d))
    keep = np.zeros((batch, n_q_heads, ctx_len), dtype=bool)
    local = np.zeros((batch, n_q_heads, ctx_len))
    for bi in range(batch):
        for kh in range(n_kv_heads):
            row0 = (bi * n_kv_heads + kh) * ctx_len
            keys = _slice_packed(k_packed, row0, row0 + ctx_len)
            vals = dequantize(codec_v, _slice_packed(v_packed, row0, row0 + ctx_len))
            hs = slice(kh * G, (kh + 1) * G)
            s = scale * score(codec_k, q[bi, hs], keys)          # [G][T]
            e = np.exp(s - np.max(s, axis=-1, keepdims=True))
            l = np.sum(e, axis=-1, keepdims=True)               # every position
            for c0 in range(0, ctx_len, chunk):
                sc = s[:, c0:c0 + chunk]
                ec = np.exp(sc - np.max(sc, axis=-1, keepdims=True))
                local[bi, hs, c0:c0 + chunk] = ec / np.sum(ec, axis=-1, keepdims=True)
            k = local[bi, hs] >= gate
            keep[bi, hs] = k
            out[bi, hs] = (e * k / l) @ vals
    return out, keep, local


def decode_attn_sparse_v_plain(codec_k: Codec, codec_v: Codec, q, k_packed, v_packed,
                               batch, n_q_heads, n_kv_heads, ctx_len, scale, gate):
    """Sparse V exactly as TurboQuant+ 深度解析 第六部分 states it: the value of
    a position is neither decompressed nor added when its attention weight --
    the final softmax weight over the whole context -- is below the gate; the
    normaliser still sums every position.  No chunking: this is the page's
    rule, which the split kernels bound from above (the chunk-local weight of
    decode_attn_sparse_v is never below this one, so they keep a superset of
    these positions).  Returns (out [batch][n_q_heads][d], keep
    [batch][n_q_heads][ctx_len] bool, w [batch][n_q_heads][ctx_len] final
    weights)."""
    q = np.asarray(q, dtype=np.float64).reshape(batch, n_q_heads, codec_k.d)
    G = n_q_heads // n_kv_heads
    out = np.zeros((batch, n_q_heads, codec_v.d))
    keep = np.zeros((batch, n_q_heads, ctx_len), dtype=bool)
    w = np.zeros((batch, n_q_heads, ctx_len))
    for bi in range(batch):
        for kh in range(n_kv_heads):
            row0 = (bi * n_kv_heads + kh) * ctx_len
            keys = _slice_packed(k_packed, row0, row0 + ctx_len)
            vals = dequantize(codec_v, _slice_packed(v_packed, row0, row0 + ctx_len))
            hs = slice(kh * G, (kh + 1) * G)
            e, l = _softmax_weights(score(codec_k, q[bi, hs], keys), scale)
            wt = e / l
            w[bi, hs] = wt
            keep[bi, hs] = wt >= gate
            out[bi, hs] = (wt * keep[bi, hs]) @ vals
    return out, keep, w


# --------------------------------------------------------------------------
# O6c. Paged cache (the KV cache of 深度拆解 第一部分 "KV 缓存是什么" grows by one
# token per decode step).  Reading: the cache is split into pages of
# `page_size` positions; page p holds, for every KV head kh, the records of
# its positions at rows (p * n_kv_heads + kh) * page_size + slot, and
# page_table[b][i] names the page holding positions [i*page_size,
# (i+1)*page_size) of sequence b.  New tokens are encoded like any other
# vector and written at positions ctx_lens[b], ctx_lens[b] + 1, ...  Decode
# attention of sequence b runs over its first ctx_lens[b] positions; an empty
# context gives a zero output (the pages never consider one).
# --------------------------------------------------------------------------
def paged_row(page_table, b: int, kh: int, pos: int, n_kv_heads: int, page_size: int) -> int:
    page = int(np.asarray(page_table)[b][pos // page_size])
    return (page * n_kv_heads + kh) * page_size + pos % page_size


def append_paged(codec: Codec, cache: dict, x, ctx_lens, page_table, page_size: int):
    """x: (batch, n_kv_heads, n_new, d).  Writes the records into `cache`
    (numpy arrays, modified in place) and returns it."""
    x = np.asarray(x, dtype=np.float64)
    batch, hkv, n_new, d = x.shape
    enc = encode(codec, x.reshape(-1, d))
    i = 0
    for b in range(batch):
        for kh in range(hkv):
            for t in range(n_new):
                row = paged_row(page_table, b, kh, int(ctx_lens[b]) + t, hkv, page_size)
                for key in ("codes", "signs", "norm", "rnorm"):
                    cache[key][row] = enc[key][i]
                i += 1
    return cache


def gather_paged(cache: dict, page_table, b: int, n_kv_heads: int, ctx_len: int, page_size: int) -> dict:
    """Sequence b's records as contiguous rows [kv_head][position]."""
    rows = [paged_row(page_table, b, kh, t, n_kv_heads, page_size)
            for kh in range(n_kv_heads) for t in range(ctx_len)]
    return {k: np.asarray(cache[k])[rows] for k in ("codes", "signs", "norm", "rnorm")}


def decode_attn_paged(codec_k: Codec, codec_v: Codec, q, k_cache, v_cache, page_table, ctx_lens,
                      n_q_heads, n_kv_heads, page_size, scale, gate=None, chunk=None):
    """q: (batch, n_q_heads, d).  gate=None: plain attention; else Sparse V
    (O6b) with the given gate and chunk."""
    q = np.asarray(q, dtype=np.float64)
    batch = q.shape[0]
    out = np.zeros((batch, n_q_heads, codec_v.d))
    for b in range(batch):
        n = int(ctx_lens[b])
        if n == 0:
            continue
        kr = gather_paged(k_cache, page_table, b, n_kv_heads, n, page_size)
        vr = gather_paged(v_cache, page_table, b, n_kv_heads, n, page_size)
        if gate is None:
            out[b] = decode_attn_accumulated(codec_k, codec_v, q[b:b + 1], kr, vr, 1, n_q_heads, n_kv_heads, n,
                                             scale)[0]
        else:
            out[b] = decode_attn_sparse_v(codec_k, codec_v, q[b:b + 1], kr, vr, 1, n_q_heads, n_kv_heads, n,
                                          scale, gate, chunk)[0][0]
    return out


# --------------------------------------------------------------------------
# O7b. Value records in blocks of 32 rows.  A storage order of the same bits
# as O4's row records (the pages fix no memory layout; this one puts each
# coordinate's bits of 32 consecutive rows in one word, the operand a
# contraction over keys needs).  d = 128.  Block B holds rows 32B..32B+31.
# Planes: the b code planes of O4, then the QJL sign plane (if any).  For
# coordinate j = 16c + n (n < 16, c < 8):
#   codes word (B*b + p)*128 + 8n + c,  signs word B*128 + 8n + c,
# and row 32B + 8r + i (i < 8, r < 4) is bit 4i + r of that word.  The arrays
# keep the row layout's sizes: n rows (a multiple of 32) of code_words and
# sign_words words.  ν and γ stay per row.
# Parity: a layout defined here, not by the pages; pinned by bits placed by
# hand and by the round trip with vblock_unpack.
# --------------------------------------------------------------------------
def _vblock_word_of_coordinate(j):
    j = np.asarray(j)
    return 8 * (j % 16) + j // 16


def _vblock_bit_of_row(tau: int) -> int:
    return 4 * (tau % 8) + tau // 8


def _record_planes(rec: dict, b: int, d: int) -> np.ndarray:
    """(n, planes, d) 0/1 array: the code planes of O4, then the signs."""
    wpp = d // 32
    codes = np.asarray(rec["codes"], dtype=np.uint32)
    planes = [unpack_bits(codes[:, p * wpp:(p + 1) * wpp], d) for p in range(b)]
    signs = np.asarray(rec["signs"], dtype=np.uint32)
    if signs.shape[1]:
        planes.append(unpack_bits(signs, d))
    return np.stack(planes, axis=1)


def vblock_pack(rec: dict, b: int, d: int = 128) -> dict:
    """Row records (O4) -> the same records in 32-row blocks."""
    assert d == 128
    bits = _record_planes(rec, b, d)
    n, n_planes, _ = bits.shape
    assert n % 32 == 0
    nblk = n // 32
    out = np.zeros((nblk, n_planes, 128), dtype=np.uint64)
    w = _vblock_word_of_coordinate(np.arange(d))
    for tau in range(32):
        sh = np.uint64(_vblock_bit_of_row(tau))
        for p in range(n_planes):
            out[:, p, w] |= bits[tau::32, p, :].astype(np.uint64) << sh
    out = out.astype(np.uint32)
    codes = out[:, :b, :].reshape(n, b * d // 32)
    signs = out[:, b, :].reshape(n, d // 32) if n_planes > b else np.zeros((n, 0), np.uint32)
    return {"codes": codes, "signs": signs, "norm": np.asarray(rec["norm"]).copy(),
            "rnorm": np.asarray(rec["rnorm"]).copy()}


def vblock_unpack(blocked: dict, b: int, d: int = 128) -> dict:
    """The inverse of vblock_pack."""
    assert d == 128
    codes = np.asarray(blocked["codes"], dtype=np.uint32)
    n = codes.shape[0]
    nblk = n // 32
    signs = np.asarray(blocked["signs"], dtype=np.uint32)
    words = [codes.reshape(nblk, b, 128)[:, p, :] for p in range(b)]
    if signs.shape[1]:
        words.append(signs.reshape(nblk, 128))
    w = _vblock_word_of_coordinate(np.arange(d))
    bits = np.zeros((n, len(words), d), dtype=np.int64)
    for tau in range(32):
        sh = np.uint64(_vblock_bit_of_row(tau))
        for p, wp in enumerate(words):
            bits[tau::32, p, :] = (wp[:, w].astype(np.uint64) >> sh) & np.uint64(1)
    idx = np.zeros((n, d), dtype=np.int64)
    for p in range(b):
        idx |= bits[:, p, :] << p
    return {"codes": pack_planes(idx, b),
            "signs": pack_bits(bits[:, b, :]) if len(words) > b else np.zeros((n, 0), np.uint32),
            "norm": np.asarray(blocked["norm"]).copy(), "rnorm": np.asarray(blocked["rnorm"]).copy()}


# --------------------------------------------------------------------------
# O8. PolarQuant first stage (深度拆解 第二部分 PolarQuant; vocus 第一階段):
# rotate, write the rotated vector in polar form by pairing coordinates into
# (radius, angle), pair the radii again and recurse until one radius is left,
# and quantize every angle with a Lloyd-Max quantizer fitted to that angle's
# known law; then the same residual QJL stage as before.
#
# Readings.
# * y = R x/ν as in O4 (unit vector), d a power of two: log2(d) levels.  Level
#   1 pairs (y_2i, y_2i+1); level l > 1 pairs the radii (r_2i, r_2i+1) of level
#   l-1; angle θ = atan2(second, first), radius = hypot.  The last radius is
#   ‖y‖ = 1 and is not stored (ν is).
# * Angle laws for y uniform on the sphere: level 1 is uniform on the circle
#   (taken in [0, 2π)); for l > 1 with n = 2^(l-1) coordinates per half,
#   sin²θ ~ Beta(n/2, n/2), i.e. f(θ) = 2/B(n/2, n/2) (sin θ cos θ)^(n-1) on
#   [0, π/2] (the ratio of the norms of two independent Gaussian halves).
# * b bits for every angle: d-1 angles in about the b·d bits the scalar stage
#   spends, so "bits" keeps its meaning (b angle bits + 1 QJL bit).  Level 1's
#   optimal quantizer is the uniform one (centroids (k+1/2)·2π/2^b); levels > 1
#   run Lloyd-Max on f (MSE in the angle).
# * Code slots: level l's d/2^l angles take slots [d - d/2^(l-1), d - d/2^l) in
#   order, slot d-1 is unused (code 0); the codes are packed in bit planes as in
#   O4.  The stored reconstruction tables are cos and sin of every centroid
#   rounded to fp32; ŷ is rebuilt top-down from radius 1 with them.
# * Decisions are taken in fp64 here; the kernels take them in fp32, so an
#   angle within 1e-5 rad of a boundary may legitimately get the other code.
# --------------------------------------------------------------------------
def polar_angle_density(theta, level: int):
    theta = np.asarray(theta, dtype=np.float64)
    if level == 1:
        return np.where((theta >= 0) & (theta < 2 * math.pi), 1.0 / (2 * math.pi), 0.0)
    n = 1 << (level - 1)
    with np.errstate(divide="ignore"):
        logf = (math.log(2.0) - special.betaln(n / 2, n / 2)
                + (n - 1) * np.log(np.clip(np.sin(theta) * np.cos(theta), 0, None)))
    return np.where((theta >= 0) & (theta <= math.pi / 2), np.exp(logf), 0.0)


def polar_angle_cdf(theta, level: int):
    theta = np.asarray(theta, dtype=np.float64)
    if level == 1:
        return np.clip(theta / (2 * math.pi), 0.0, 1.0)
    n = 1 << (level - 1)
    t = np.clip(theta, 0.0, math.pi / 2)
    return special.betainc(n / 2, n / 2, np.sin(t) ** 2)


def _polar_first_moment(lo: float, hi: float, level: int) -> float:
    mid = math.pi / 4
    pts = [mid] if lo < mid < hi else None
    val, _ = integrate.quad(lambda t: t * float(polar_angle_density(t, level)), lo, hi, points=pts,
                            epsabs=0.0, epsrel=1e-13, limit=200)
    return val


def polar_lloyd_max(level: int, b: int, tol: float = 1e-13, max_iter: int = 5000):
    """(centroids, boundaries, iterations) of the 2^b-level quantizer of the
    level's angle, ascending, fp64."""
    L = 1 << b
    if level == 1:
        step = 2 * math.pi / L
        return (np.arange(L) + 0.5) * step, np.arange(1, L) * step, 0
    n = 1 << (level - 1)
    c = np.arcsin(np.sqrt(special.betaincinv(n / 2, n / 2, (np.arange(L) + 0.5) / L)))
    it = 0
    for it in range(1, max_iter + 1):
        t = 0.5 * (c[:-1] + c[1:])
        edges = np.concatenate([[0.0], t, [math.pi / 2]])
        mass = polar_angle_cdf(edges[1:], level) - polar_angle_cdf(edges[:-1], level)
        mom = np.array([_polar_first_moment(edges[k], edges[k + 1], level) for k in range(L)])
        new = mom / mass
        new = 0.5 * (new + (math.pi / 2 - new[::-1]))      # symmetric about π/4
        delta = float(np.max(np.abs(new - c)))
        c = new
        if delta < tol:
            break
    return c, 0.5 * (c[:-1] + c[1:]), it


def polar_transform(y):
    """y: (n, d), d a power of two.  Returns (angles, radius): angles[l-1] is
    the (n, d/2^l) array of level-l angles, radius the (n,) final radius."""
    r = np.asarray(y, dtype=np.float64)
    angles = []
    level = 1
    while r.shape[1] > 1:
        a, b = r[:, 0::2], r[:, 1::2]
        th = np.arctan2(b, a)
        if level == 1:
            th = np.where(th < 0, th + 2 * math.pi, th)
        angles.append(th)
        r = np.hypot(a, b)
        level += 1
    return angles, r[:, 0]


def polar_reconstruct(cos_tabs, sin_tabs, idx_levels, radius=None):
    """Top-down rebuild: cos_tabs[l-1][k], sin_tabs[l-1][k] = cos, sin of the
    level's centroid k; idx_levels[l-1] = (n, d/2^l) codes.  Returns (n, d)."""
    n = idx_levels[0].shape[0]
    r = np.ones((n, 1)) if radius is None else np.asarray(radius, dtype=np.float64).reshape(n, 1)
    for lv in range(len(idx_levels), 0, -1):
        k = idx_levels[lv - 1]
        ca = np.asarray(cos_tabs[lv - 1], dtype=np.float64)[k]
        sa = np.asarray(sin_tabs[lv - 1], dtype=np.float64)[k]
        nxt = np.empty((n, 2 * r.shape[1]))
        nxt[:, 0::2] = r * ca
        nxt[:, 1::2] = r * sa
        r = nxt
    return r


def polar_slots(d: int):
    """Slot ranges [lo, hi) of each level's angles in the code vector."""
    out, lo, cnt = [], 0, d // 2
    while cnt >= 1:
        out.append((lo, lo + cnt))
        lo += cnt
        cnt //= 2
    return out


@dataclass
class PolarCodec:
    d: int
    bits: int
    m: int
    seed: int
    D: np.ndarray
    R: np.ndarray
    S: np.ndarray
    centroids: list       # per level, fp64 ascending
    bounds: list          # per level, fp64
    iters: list

    @property
    def b(self) -> int:
        return self.bits - 1

    @property
    def qjl(self) -> bool:  # the residual always takes the QJL stage
        return True

    @property
    def levels(self) -> int:
        return len(self.centroids)

    @property
    def cos32(self) -> list:
        return [np.cos(c).astype(np.float32) for c in self.centroids]

    @property
    def sin32(self) -> list:
        return [np.sin(c).astype(np.float32) for c in self.centroids]

    @property
    def code_words(self) -> int:
        return self.b * self.d // 32

    @property
    def sign_words(self) -> int:
        return self.m // 32

    @property
    def record_bytes(self) -> int:
        return 4 * (self.code_words + self.sign_words) + 8


def make_polar_codec(d: int, bits: int, m: int | None = None, seed: int = 1234) -> PolarCodec:
    if d < 2 or d & (d - 1):
        raise ValueError("the recursive polar stage needs d a power of two")
    if bits < 2:
        raise ValueError("bits must be >= 2")
    m = d if m is None else m
    books = [polar_lloyd_max(lv, bits - 1) for lv in range(1, int(math.log2(d)) + 1)]
    return PolarCodec(d=d, bits=bits, m=m, seed=seed, D=rademacher_signs(d, seed), R=rotation_matrix(d, seed),
                      S=gaussian_matrix(m, d, seed), centroids=[c for c, _, _ in books],
                      bounds=[t for _, t, _ in books], iters=[i for _, _, i in books])


def _polar_yhat_from_slots(codec: PolarCodec, idx):
    levels = [idx[:, lo:hi] for lo, hi in polar_slots(codec.d)]
    return polar_reconstruct(codec.cos32, codec.sin32, levels)


def polar_encode(codec: PolarCodec, x: np.ndarray) -> dict:
    x = np.asarray(x, dtype=np.float64)
    nu = np.sqrt(np.sum(x * x, axis=1))
    safe = np.where(nu > 0, nu, 1.0)
    u = np.where(nu[:, None] > 0, x / safe[:, None], 0.0)
    y = u @ codec.R.T
    angles, _ = polar_transform(y)
    idx = np.zeros((x.shape[0], codec.d), dtype=np.int64)
    for lv, ((lo, hi), th) in enumerate(zip(polar_slots(codec.d), angles), start=1):
        idx[:, lo:hi] = np.sum(codec.bounds[lv - 1][None, None, :] < th[:, :, None], axis=2)
    out = polar_encode_given_codes(codec, x, idx)
    out.update(codes=pack_planes(idx, codec.b), norm=nu.astype(np.float32), idx=idx, angles=angles)
    return out


def polar_encode_given_codes(codec: PolarCodec, x: np.ndarray, idx: np.ndarray) -> dict:
    x = np.asarray(x, dtype=np.float64)
    nu = np.sqrt(np.sum(x * x, axis=1))
    safe = np.where(nu > 0, nu, 1.0)
    u = np.where(nu[:, None] > 0, x / safe[:, None], 0.0)
    y = u @ codec.R.T
    yhat = _polar_yhat_from_slots(codec, np.asarray(idx, np.int64))
    r = y - yhat
    gamma = np.sqrt(np.sum(r * r, axis=1))
    z = r @ codec.S.astype(np.float64).T
    return {"signs": pack_bits((z >= 0).astype(np.int64)), "rnorm": gamma.astype(np.float32), "z": z,
            "y": y, "yhat": yhat, "r": r}


def _polar_unpack(codec: PolarCodec, packed: dict):
    idx = unpack_planes(np.asarray(packed["codes"]), codec.b, codec.d)
    tau = (2 * unpack_bits(np.asarray(packed["signs"]), codec.m) - 1).astype(np.float64)
    nu = np.asarray(packed["norm"], dtype=np.float32).astype(np.float64)
    gamma = np.asarray(packed["rnorm"], dtype=np.float32).astype(np.float64)
    return _polar_yhat_from_slots(codec, idx), tau, nu, gamma


def polar_dequantize(codec: PolarCodec, packed: dict) -> np.ndarray:
    yhat, tau, nu, gamma = _polar_unpack(codec, packed)
    corr = qjl_constant(codec.m) * gamma[:, None] * (tau @ codec.S.astype(np.float64))
    return nu[:, None] * ((yhat + corr) @ codec.R)


def polar_score(codec: PolarCodec, q: np.ndarray, packed: dict) -> np.ndarray:
    """ℓ = ν (⟨q', ŷ⟩ + sqrt(pi/2)/m · γ · ⟨p, τ⟩), q' = R q, p = S q'."""
    q = np.atleast_2d(np.asarray(q, dtype=np.float64))
    qr = q @ codec.R.T
    p = qr @ codec.S.astype(np.float64).T
    yhat, tau, nu, gamma = _polar_unpack(codec, packed)
    return nu[None, :] * (qr @ yhat.T + qjl_constant(codec.m) * gamma[None, :] * (p @ tau.T))


# --------------------------------------------------------------------------
# O7. Exhaustive search (深度拆解 第三部分 向量搜索: the compressed database is
# the index, nothing is trained): scores by O5, top-k by descending score,
# ties to the lower database index.
# --------------------------------------------------------------------------
def search_topk(codec: Codec, db_packed: dict, queries: np.ndarray, k: int,
                chunk: int = 65536):
    queries = np.atleast_2d(np.asarray(queries, dtype=np.float64))
    n_db = np.asarray(db_packed["norm"]).shape[0]
    scores = np.empty((queries.shape[0], n_db))
    for s in range(0, n_db, chunk):
        scores[:, s:s + chunk] = score(codec, queries, _slice_packed(db_packed, s, s + chunk))
    order = np.argsort(-scores, axis=1, kind="stable")[:, :k]
    return order.astype(np.int64), np.take_along_axis(scores, order, axis=1), scores


# --------------------------------------------------------------------------
# Numerics helper: round-to-nearest-even to bfloat16 (returned as fp32 values).
# An fp64 input is first rounded to fp32 (RNE), as torch does for a double ->
# bfloat16 cast; an fp32 input is rounded once.  Ties go to the even
# significand; values at or above the overflow threshold become ±Inf; ±0,
# subnormals and ±Inf keep their class; NaN stays NaN.
# --------------------------------------------------------------------------
def bf16_round(x: np.ndarray) -> np.ndarray:
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    out = u.astype(np.uint32).view(np.float32)
    return np.where(np.isnan(f), f, out)

"""Comparison helpers for the GPU-vs-oracle parity tests.

Bars (stated once here, used by every GPU test):
* codes: bit-exact except coordinates whose fp32 rotated value lies within
  1e-5 of the boundary between the two codes; at most 1e-5 of all coordinates
  may differ.  A vector with a differing code is re-derived by the oracle
  given the GPU's codes (r, γ, signs all depend on them).
* signs: bit-exact except where the oracle's |z| < 1e-5.
* ν and γ: relative error <= 2e-6 (fp32 accumulation of d terms).
* logits / attention outputs: per row max_i|a_i - b_i| / max_i|b_i| <= 1e-3
  for bf16 inputs, 1e-4 for fp32 inputs.
"""
from __future__ import annotations

import numpy as np

import oracle as O

BAND = 1e-5
NORM_RTOL = 2e-6


def tol_for(dtype: str) -> float:
    return 1e-4 if dtype == "f32" else 1e-3


def row_rel_err(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    a = np.asarray(a, np.float64).reshape(-1, np.shape(a)[-1])
    b = np.asarray(b, np.float64).reshape(-1, np.shape(b)[-1])
    den = np.maximum(np.max(np.abs(b), axis=1), 1e-30)
    return np.max(np.abs(a - b), axis=1) / den


def check_encode(cd: O.Codec, x64: np.ndarray, gpu: dict, label: str = "") -> dict:
    """Compare one GPU encode (numpy dict) with the oracle on inputs x64."""
    ref = O.encode(cd, x64)
    n, d = x64.shape
    gi = O.unpack_planes(gpu["codes"], cd.b, d)
    ri = ref["idx"]
    diff = gi != ri
    n_diff = int(diff.sum())
    assert n_diff <= max(1, int(1e-5 * diff.size)), f"{label}: {n_diff} codes differ of {diff.size}"
    if n_diff:
        y32 = ref["y"].astype(np.float32).astype(np.float64)
        t32 = cd.t32.astype(np.float64)
        vv, jj = np.nonzero(diff)
        for v, j in zip(vv, jj):
            a, b = int(gi[v, j]), int(ri[v, j])
            assert abs(a - b) == 1, f"{label}: code jump {b}->{a} at ({v},{j})"
            tb = t32[min(a, b)]
            assert abs(y32[v, j] - tb) < BAND, f"{label}: mismatch at ({v},{j}) y={y32[v,j]} boundary {tb}"
    # norms
    assert np.allclose(gpu["norm"], ref["norm"], rtol=NORM_RTOL, atol=0), f"{label}: norm"
    if not cd.qjl:  # an MSE-only record ends here: codes and ν
        return {"code_mismatch": n_diff, "sign_mismatch": 0, "ref": ref}
    # re-derive rows whose codes differ
    rows = np.unique(np.nonzero(diff)[0]) if n_diff else np.array([], np.int64)
    exp_signs = ref["signs"].copy()
    exp_rnorm = ref["rnorm"].copy()
    z = ref["z"].copy()
    if rows.size:
        rd = O.encode_given_codes(cd, x64[rows], gi[rows])
        exp_signs[rows] = rd["signs"]
        exp_rnorm[rows] = rd["rnorm"]
        z[rows] = rd["z"]
    assert np.allclose(gpu["rnorm"], exp_rnorm, rtol=NORM_RTOL, atol=1e-7), f"{label}: rnorm"
    gs = O.unpack_bits(gpu["signs"], cd.m)
    es = O.unpack_bits(exp_signs, cd.m)
    sd = gs != es
    if sd.any():
        assert np.all(np.abs(z[sd]) < BAND), f"{label}: {int(sd.sum())} sign bits differ outside the band " \
                                             f"(max |z| {np.max(np.abs(z[sd]))})"
    return {"code_mismatch": n_diff, "sign_mismatch": int(sd.sum()), "ref": ref}


def oracle_records_like(cd: O.Codec, x64: np.ndarray, gpu: dict) -> dict:
    """The oracle's records for x64, conditioned on the GPU's legitimate
    choices (checked by check_encode first): the GPU's codes on rows where a
    coordinate sits in the boundary band, with r and γ re-derived from those
    codes, and the GPU's sign bits, which differ from the oracle's only where
    |z| is inside the band.  (Over a long context such in-band sign choices
    are not negligible: an attention output that averages 10^5 values is
    ~300x smaller than one value, so a dozen legitimately flipped bits show
    up at the 1e-4 level.)"""
    check_encode(cd, x64, gpu, "conditioned")
    ref = O.encode(cd, x64)
    gi = O.unpack_planes(gpu["codes"], cd.b, x64.shape[1])
    rows = np.nonzero(np.any(gi != ref["idx"], axis=1))[0]
    out = {k: ref[k].copy() for k in ("codes", "signs", "norm", "rnorm")}
    if rows.size:
        rd = O.encode_given_codes(cd, x64[rows], gi[rows])
        out["codes"][rows] = gpu["codes"][rows]
        out["rnorm"][rows] = rd["rnorm"]
    out["signs"] = np.asarray(gpu["signs"]).copy()
    return out


def assert_sparse_v_close(out, ref, local, gate, vhat, hkv, ctx, tol):  # batch 1
    """out vs the gated oracle to `tol` of each row's maximum, plus, for the
    positions within 1% of the gate (a floating-point decision either side
    may take), the most their value terms can move the output: the
    chunk-local weight bounds the final one."""
    G = out.shape[1] // hkv
    amb = np.abs(np.log(np.maximum(local[0], 1e-300) / gate)) < 1e-2      # [hq][ctx]
    slack = np.zeros_like(ref[0])
    for h in np.nonzero(amb.any(axis=1))[0]:
        kh = h // G
        t = np.nonzero(amb[h])[0]
        slack[h] = local[0, h, t] @ np.abs(vhat[kh * ctx + t])
    diff = np.abs(out[0] - ref[0])
    bound = tol * np.max(np.abs(ref[0]), axis=-1, keepdims=True) + 1.01 * slack
    print(f"  positions near the gate {int(amb.sum())}, max row err {row_rel_err(out, ref).max():.2e}, "
          f"worst diff/bound {np.max(diff / bound):.3f}", flush=True)
    assert np.all(diff <= bound)


def assert_sparse_v_within_plain_rule(out, plain, w, gate, vhat, hkv, ctx, tol):  # batch 1
    """out (a kernel's gated attention) vs the page's own rule, which drops the
    value term of every position whose final softmax weight w is below the
    gate (oracle decode_attn_sparse_v_plain).  A split kernel may keep some of
    those positions (its chunk-local weight bounds w from above) and, within
    1% of the gate, take a floating-point decision either way, so the two
    differ by at most the value mass of the positions with w < 1.01·gate,
    per (head, coordinate), plus `tol` of each row's maximum.  Also checks the
    coarser bound gate × (positions dropped by the plain rule) × max|v̂|."""
    G = out.shape[1] // hkv
    slack = np.zeros_like(plain[0])
    coarse = np.zeros(plain.shape[1])
    vmax = np.abs(vhat).max()
    for h in range(out.shape[1]):
        kh = h // G
        t = np.nonzero(w[0, h] < 1.01 * gate)[0]
        slack[h] = w[0, h, t] @ np.abs(vhat[kh * ctx + t])
        coarse[h] = gate * np.count_nonzero(w[0, h] < gate) * vmax
    diff = np.abs(out[0] - plain[0])
    scale = tol * np.max(np.abs(plain[0]), axis=-1, keepdims=True)
    bound = scale + 1.01 * slack
    print(f"  plain rule: dropped (head, key) {np.mean(w < gate):.4f}, max |out - plain| {diff.max():.2e}, "
          f"worst diff/bound {np.max(diff / bound):.3f}, coarse bound {coarse.max():.2e}", flush=True)
    assert np.all(diff <= bound)
    assert np.all(diff.max(axis=-1) <= scale[:, 0] + coarse * 1.01)


ANGLE_BAND = 1e-5  # rad


def check_polar_encode(pc: O.PolarCodec, x64: np.ndarray, gpu: dict, label: str = "", max_rate=None) -> dict:
    """Compare a GPU encode with a polar codec against the oracle.  Angle
    codes: bit-exact except angles within ANGLE_BAND of the boundary between
    the two codes (for level 1 also of the wrap 0 = 2π), each checked.  With
    max_rate (Gaussian rows) the differing codes are also capped at that
    fraction of all codes (at least one); without it (rows built to sit on
    boundaries: a basis vector's rotated coordinates share one magnitude, so
    its angles fall on multiples of π/4) only the per-code check applies.
    Vectors with a differing code are re-derived by the oracle given the
    GPU's codes.  ν and γ: relative 2e-6 and 1e-5 (γ carries
    the fp32 products of the reconstruction); signs: bit-exact except |z| < BAND."""
    ref = O.polar_encode(pc, x64)
    n, d = x64.shape
    gi = O.unpack_planes(gpu["codes"], pc.b, d)
    ri = ref["idx"]
    diff = gi != ri
    n_diff = int(diff.sum())
    if max_rate is not None:
        assert n_diff <= max(1, int(max_rate * diff.size)), f"{label}: {n_diff} angle codes differ of {diff.size}"
    if n_diff:
        L = 1 << pc.b
        for v, s in zip(*np.nonzero(diff)):
            lv = next(i for i, (lo, hi) in enumerate(O.polar_slots(d), start=1) if lo <= s < hi)
            lo = O.polar_slots(d)[lv - 1][0]
            th = ref["angles"][lv - 1][v, s - lo]
            a, b = sorted((int(gi[v, s]), int(ri[v, s])))
            if lv == 1 and (a, b) == (0, L - 1):
                dist = min(th, 2 * np.pi - th)
            else:
                assert b == a + 1, f"{label}: code jump at ({v},{s})"
                dist = abs(th - pc.bounds[lv - 1][a])
            assert dist < ANGLE_BAND, f"{label}: angle code differs at ({v},{s}), {dist:.2e} rad from the boundary"
    assert np.allclose(gpu["norm"], ref["norm"], rtol=NORM_RTOL, atol=0), f"{label}: norm"
    rows = np.unique(np.nonzero(diff)[0]) if n_diff else np.array([], np.int64)
    exp_signs, exp_rnorm, z = ref["signs"].copy(), ref["rnorm"].copy(), ref["z"].copy()
    if rows.size:
        rd = O.polar_encode_given_codes(pc, x64[rows], gi[rows])
        exp_signs[rows], exp_rnorm[rows], z[rows] = rd["signs"], rd["rnorm"], rd["z"]
    assert np.allclose(gpu["rnorm"], exp_rnorm, rtol=1e-5, atol=1e-7), f"{label}: rnorm"
    sd = O.unpack_bits(gpu["signs"], pc.m) != O.unpack_bits(exp_signs, pc.m)
    if sd.any():
        assert np.all(np.abs(z[sd]) < BAND), f"{label}: {int(sd.sum())} sign bits differ outside the band"
    return {"code_mismatch": n_diff, "sign_mismatch": int(sd.sum()), "ref": ref}


def polar_records_like(pc: O.PolarCodec, x64: np.ndarray, gpu: dict) -> dict:
    """The oracle's polar records for x64 conditioned on the GPU's legitimate
    choices (its angle codes and its sign bits), after check_polar_encode."""
    check_polar_encode(pc, x64, gpu, "conditioned")
    gi = O.unpack_planes(gpu["codes"], pc.b, x64.shape[1])
    rd = O.polar_encode_given_codes(pc, x64, gi)
    nu = np.sqrt(np.sum(np.asarray(x64, np.float64) ** 2, axis=1)).astype(np.float32)
    return {"codes": np.asarray(gpu["codes"]).copy(), "signs": np.asarray(gpu["signs"]).copy(), "norm": nu,
            "rnorm": rd["rnorm"]}


def fill_pages(rec_by_seq, page_table, hkv, P, n_pages, junk):
    """A numpy cache with sequence b's records (rows [kv_head][position]) at
    their page slots; every other row holds a junk record."""
    cache = {k: np.asarray(junk[k])[np.arange(n_pages * hkv * P) % len(junk["norm"])].copy()
             for k in ("codes", "signs", "norm", "rnorm")}
    for b, rec in enumerate(rec_by_seq):
        n = len(rec["norm"]) // hkv
        for kh in range(hkv):
            for t in range(n):
                row = O.paged_row(page_table, b, kh, t, hkv, P)
                for k in cache:
                    cache[k][row] = np.asarray(rec[k])[kh * n + t]
    return cache

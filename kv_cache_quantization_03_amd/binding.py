"""Thin Python binding over libtq.so (ctypes).  Argument marshalling only.

Every function keeps the name of the C entry point it wraps.  Device buffers
are torch tensors (torch is used for device memory and streams only); the
calls run on torch's current stream of the tensors' device.  There is no CPU
fallback: importing this module without the built library raises.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

TQ_F32, TQ_BF16, TQ_F16 = 0, 1, 2


class TQError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


class tq_packed_t(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("signs", C.c_void_p), ("norm", C.c_void_p), ("rnorm", C.c_void_p)]


class tq_codec_info_t(C.Structure):
    _fields_ = [("head_dim", C.c_int32), ("bits", C.c_int32), ("mse_bits", C.c_int32),
                ("qjl_dim", C.c_int32), ("code_words", C.c_int32), ("sign_words", C.c_int32),
                ("record_bytes", C.c_int32), ("lloyd_max_iterations", C.c_int32),
                ("seed", C.c_uint64), ("centroids", C.c_double * 16), ("bounds", C.c_double * 15),
                ("stage1", C.c_int32), ("layout", C.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m kv_cache_quantization_03_amd.build` (hipcc, gfx950)")
    lib = C.CDLL(LIB_PATH)
    vp, i32, i64, u64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_uint64, C.c_size_t
    P = tq_packed_t
    sig = {
        "tq_status_string": (C.c_char_p, [C.c_int]),
        "tq_last_error": (C.c_char_p, []),
        "tq_abi_version": (i32, []),
        "tq_codec_build_host": (C.c_int, [i32, i32, i32, u64, vp, vp, vp, vp, vp]),
        "tq_codec_create": (C.c_int, [i32, i32, i32, u64, C.POINTER(vp)]),
        "tq_codec_destroy": (C.c_int, [vp]),
        "tq_codec_info": (C.c_int, [vp, C.POINTER(tq_codec_info_t)]),
        "tq_codec_create_polar": (C.c_int, [i32, i32, i32, C.c_uint64, C.POINTER(C.c_void_p)]),
        "tq_codec_create_mse": (C.c_int, [i32, i32, C.c_uint64, C.POINTER(C.c_void_p)]),
        "tq_codec_create_vblock": (C.c_int, [i32, i32, i32, C.c_uint64, C.POINTER(C.c_void_p)]),
        "tq_polar_book_host": (C.c_int, [i32, i32, i32, C.POINTER(C.c_double), C.POINTER(C.c_double),
                                         C.POINTER(i32)]),
        "tq_encode_workspace": (sz, [vp, i64]),
        "tq_encode_kv": (C.c_int, [vp, vp, vp, C.c_int, i64, P, P, vp, sz, vp]),
        "tq_attn_logits_workspace": (sz, [vp, i32, i32, i32, i32]),
        "tq_attn_logits": (C.c_int, [vp, vp, C.c_int, i32, i32, i32, i32, P, i64, vp, vp, sz, vp]),
        "tq_attn_query_prep": (C.c_int, [vp, vp, C.c_int, i32, i32, i32, i32, vp, sz, vp]),
        "tq_attn_logits_prepped": (C.c_int, [vp, vp, sz, i32, i32, i32, i32, P, i64, vp, vp]),
        "tq_decode_attn_workspace": (sz, [vp, vp, i32, i32, i32, i64]),
        "tq_decode_attn": (C.c_int, [vp, vp, vp, C.c_int, i32, i32, i32, P, P, i64, C.c_float, vp, C.c_int,
                                     vp, sz, vp]),
        "tq_decode_attn_sparse_v": (C.c_int, [vp, vp, vp, C.c_int, i32, i32, i32, P, P, i64, C.c_float, C.c_float,
                                              vp, C.c_int, vp, sz, vp]),
        "tq_decode_attn_chunk": (i32, [i32, i32]),
        "tq_decode_attn_no_alloc": (C.c_int, [vp, vp, vp, C.c_int, i32, i32, i32, P, P, i64, C.c_float, vp,
                                              C.c_int, vp]),
        "tq_encode_append_paged_workspace": (sz, [vp, i32, i32, i32]),
        "tq_encode_append_paged": (C.c_int, [vp, vp, C.c_int, i32, i32, i32, vp, vp, i32, i32, i32, P, vp, sz, vp]),
        "tq_decode_attn_paged_workspace": (sz, [vp, vp, i32, i32, i32, i64]),
        "tq_attn_logits_paged_workspace": (sz, [vp, i32, i32, i32, i32]),
        "tq_attn_logits_paged": (C.c_int, [vp, vp, C.c_int, i32, i32, i32, i32, P, vp, vp, i32, i32, i64, vp, vp, sz,
                                           vp]),
        "tq_decode_attn_paged": (C.c_int, [vp, vp, vp, C.c_int, i32, i32, i32, P, P, vp, vp, i32, i32, i64,
                                           C.c_float, C.c_float, vp, C.c_int, vp, sz, vp]),
        "tq_search_workspace": (sz, [vp, i64, i32, i32]),
        "tq_search_topk": (C.c_int, [vp, P, i64, vp, i32, i32, vp, vp, vp, sz, vp]),
        "tq_diag_stream_sink_words": (i64, [sz]),
        "tq_diag_stream": (C.c_int, [vp, sz, vp, sz, vp, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()
EXPORTED = ("tq_status_string", "tq_last_error", "tq_abi_version", "tq_codec_build_host", "tq_codec_create",
            "tq_codec_destroy", "tq_codec_info", "tq_codec_create_polar", "tq_codec_create_mse", "tq_codec_create_vblock",
            "tq_polar_book_host", "tq_encode_workspace", "tq_encode_kv",
            "tq_attn_logits_workspace", "tq_attn_logits", "tq_attn_query_prep", "tq_attn_logits_prepped",
            "tq_decode_attn_workspace", "tq_decode_attn", "tq_decode_attn_sparse_v", "tq_decode_attn_chunk",
            "tq_decode_attn_no_alloc",
            "tq_encode_append_paged_workspace", "tq_encode_append_paged", "tq_decode_attn_paged_workspace",
            "tq_decode_attn_paged", "tq_attn_logits_paged_workspace", "tq_attn_logits_paged",
            "tq_search_workspace", "tq_search_topk", "tq_diag_stream_sink_words", "tq_diag_stream")


def _check(status: int, where: str):
    if status != 0:
        raise TQError(status, where, f"{lib.tq_status_string(status).decode()}: {lib.tq_last_error().decode()}")


def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    return {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16, torch.float16: TQ_F16}[t.dtype]


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(t):
    torch = _torch()
    return C.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


# ---------------------------------------------------------------- codec
def tq_codec_build_host(head_dim: int, bits: int, qjl_dim: int = 0, seed: int = 1234) -> dict:
    """Host-only tables (no GPU): D, S (fp32), centroids, bounds (fp64), iterations."""
    m = head_dim if qjl_dim == 0 else qjl_dim
    b = bits - 1
    D = np.zeros(head_dim, np.float32)
    S = np.zeros((m, head_dim), np.float32)
    c = np.zeros(1 << b, np.float64)
    t = np.zeros((1 << b) - 1, np.float64)
    it = C.c_int32(0)
    st = lib.tq_codec_build_host(head_dim, bits, qjl_dim, seed, D.ctypes.data, S.ctypes.data, c.ctypes.data,
                                 t.ctypes.data if t.size else None, C.byref(it))
    _check(st, "tq_codec_build_host")
    return {"D": D, "S": S, "centroids": c, "bounds": t, "iterations": it.value}


class Codec:
    """Owns a tq_codec_t handle (destroyed with the object)."""

    def __init__(self, handle, info: tq_codec_info_t):
        self.handle = handle
        self.d = info.head_dim
        self.bits = info.bits
        self.b = info.mse_bits
        self.m = info.qjl_dim
        self.code_words = info.code_words
        self.sign_words = info.sign_words
        self.record_bytes = info.record_bytes
        self.seed = info.seed
        self.iterations = info.lloyd_max_iterations
        self.centroids = np.array(info.centroids[:1 << self.b])
        self.bounds = np.array(info.bounds[:(1 << self.b) - 1])
        self.polar = info.stage1 == 1
        self.qjl = info.qjl_dim > 0  # False: MSE-only value codec (records: codes and ν)
        self.vblock = info.layout == 1  # codes and signs in 32-row blocks of transposed words

    def __del__(self):
        if getattr(self, "handle", None) and lib is not None:
            lib.tq_codec_destroy(self.handle)
            self.handle = None


def tq_codec_create(head_dim: int, bits: int, qjl_dim: int = 0, seed: int = 1234) -> Codec:
    h = C.c_void_p()
    _check(lib.tq_codec_create(head_dim, bits, qjl_dim, seed, C.byref(h)), "tq_codec_create")
    info = tq_codec_info_t()
    _check(lib.tq_codec_info(h, C.byref(info)), "tq_codec_info")
    return Codec(h, info)


def tq_codec_create_polar(head_dim: int, bits: int, qjl_dim: int = 0, seed: int = 1234) -> Codec:
    h = C.c_void_p()
    _check(lib.tq_codec_create_polar(head_dim, bits, qjl_dim, seed, C.byref(h)), "tq_codec_create_polar")
    info = tq_codec_info_t()
    _check(lib.tq_codec_info(h, C.byref(info)), "tq_codec_info")
    return Codec(h, info)


def tq_codec_create_mse(head_dim: int, bits: int, seed: int = 1234) -> Codec:
    h = C.c_void_p()
    _check(lib.tq_codec_create_mse(head_dim, bits, seed, C.byref(h)), "tq_codec_create_mse")
    info = tq_codec_info_t()
    _check(lib.tq_codec_info(h, C.byref(info)), "tq_codec_info")
    return Codec(h, info)


def tq_codec_create_vblock(head_dim: int, bits: int, mse_only: bool = False, seed: int = 1234) -> Codec:
    h = C.c_void_p()
    _check(lib.tq_codec_create_vblock(head_dim, bits, int(mse_only), seed, C.byref(h)), "tq_codec_create_vblock")
    info = tq_codec_info_t()
    _check(lib.tq_codec_info(h, C.byref(info)), "tq_codec_info")
    return Codec(h, info)


def tq_polar_book_host(head_dim: int, bits: int, level: int):
    """(centroids, bounds, iterations) of one level's angle codebook, fp64 (host only)."""
    n = 1 << (bits - 1)
    c = (C.c_double * n)()
    t = (C.c_double * max(n - 1, 1))()
    it = C.c_int32()
    _check(lib.tq_polar_book_host(head_dim, bits, level, c, t, C.byref(it)), "tq_polar_book_host")
    return np.array(c[:]), np.array(t[:n - 1]), it.value


# ---------------------------------------------------------------- packed arrays
@dataclass
class Packed:
    codes: object   # torch uint32-compatible int32 [n][code_words]
    signs: object   # [n][sign_words]; None for an MSE-only codec
    norm: object    # float32 [n]
    rnorm: object   # float32 [n]; None for an MSE-only codec

    @property
    def n(self) -> int:
        return self.norm.shape[0]

    def c(self) -> tq_packed_t:
        return tq_packed_t(self.codes.data_ptr(), None if self.signs is None else self.signs.data_ptr(),
                           self.norm.data_ptr(), None if self.rnorm is None else self.rnorm.data_ptr())

    def rows(self, lo: int, hi: int) -> "Packed":
        return Packed(self.codes[lo:hi], None if self.signs is None else self.signs[lo:hi], self.norm[lo:hi],
                      None if self.rnorm is None else self.rnorm[lo:hi])

    def numpy(self) -> dict:
        n = self.n
        return {"codes": self.codes.cpu().numpy().view(np.uint32),
                "signs": (np.zeros((n, 0), np.uint32) if self.signs is None
                          else self.signs.cpu().numpy().view(np.uint32)),
                "norm": self.norm.cpu().numpy(),
                "rnorm": np.zeros(n, np.float32) if self.rnorm is None else self.rnorm.cpu().numpy()}


def alloc_packed(codec: Codec, n: int, device="cuda") -> Packed:
    torch = _torch()
    q = getattr(codec, "qjl", True)
    return Packed(torch.empty((n, codec.code_words), dtype=torch.int32, device=device),
                  torch.empty((n, codec.sign_words), dtype=torch.int32, device=device) if q else None,
                  torch.empty(n, dtype=torch.float32, device=device),
                  torch.empty(n, dtype=torch.float32, device=device) if q else None)


def packed_from_numpy(rec: dict, device="cuda") -> Packed:
    torch = _torch()
    return Packed(torch.from_numpy(np.ascontiguousarray(rec["codes"]).view(np.int32)).to(device),
                  torch.from_numpy(np.ascontiguousarray(rec["signs"]).view(np.int32)).to(device),
                  torch.from_numpy(np.ascontiguousarray(rec["norm"], dtype=np.float32)).to(device),
                  torch.from_numpy(np.ascontiguousarray(rec["rnorm"], dtype=np.float32)).to(device))


def _workspace(nbytes: int, device):
    torch = _torch()
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- encode
def tq_encode_workspace(codec: Codec, n: int) -> int:
    return lib.tq_encode_workspace(codec.handle, n)


def tq_encode_kv(codec: Codec, k, v=None, k_out: Packed | None = None, v_out: Packed | None = None, ws=None):
    n = k.shape[0] if k.dim() == 2 else int(np.prod(k.shape[:-1]))
    assert k.shape[-1] == codec.d and k.is_contiguous()
    if v is not None:
        assert v.shape == k.shape and v.dtype == k.dtype and v.is_contiguous()
    k_out = k_out or alloc_packed(codec, n, k.device)
    if v is not None:
        v_out = v_out or alloc_packed(codec, n, k.device)
    need = tq_encode_workspace(codec, n)
    ws = ws if ws is not None else _workspace(need, k.device)
    vo = v_out.c() if v is not None else tq_packed_t()
    st = lib.tq_encode_kv(codec.handle, _ptr(k), _ptr(v), _dt(k), n, k_out.c(), vo, _ptr(ws), ws.numel(),
                          _stream(k))
    _check(st, "tq_encode_kv")
    return k_out, v_out


# ---------------------------------------------------------------- logits
def tq_attn_logits_workspace(codec: Codec, batch: int, n_q_heads: int, n_kv_heads: int, n_queries: int) -> int:
    return lib.tq_attn_logits_workspace(codec.handle, batch, n_q_heads, n_kv_heads, n_queries)


def tq_attn_logits(codec: Codec, q, k: Packed, ctx_len: int, n_kv_heads: int, logits=None, ws=None):
    """q: [batch][n_queries][n_q_heads][d]; k rows [batch][n_kv_heads][ctx_len].
    Returns logits fp32 [batch][n_q_heads][n_queries][ctx_len]."""
    torch = _torch()
    batch, nq, hq, d = q.shape
    assert d == codec.d and q.is_contiguous()
    if logits is None:
        logits = torch.empty((batch, hq, nq, ctx_len), dtype=torch.float32, device=q.device)
    need = tq_attn_logits_workspace(codec, batch, hq, n_kv_heads, nq)
    ws = ws if ws is not None else _workspace(need, q.device)
    st = lib.tq_attn_logits(codec.handle, _ptr(q), _dt(q), batch, hq, n_kv_heads, nq, k.c(), ctx_len, _ptr(logits),
                            _ptr(ws), ws.numel(), _stream(q))
    _check(st, "tq_attn_logits")
    return logits


def tq_attn_query_prep(codec: Codec, q, n_kv_heads: int, prep=None):
    """Prepares q [batch][n_queries][n_q_heads][d] for tq_attn_logits_prepped."""
    batch, nq, hq, d = q.shape
    assert d == codec.d and q.is_contiguous()
    need = tq_attn_logits_workspace(codec, batch, hq, n_kv_heads, nq)
    prep = prep if prep is not None else _workspace(need, q.device)
    st = lib.tq_attn_query_prep(codec.handle, _ptr(q), _dt(q), batch, hq, n_kv_heads, nq, _ptr(prep), prep.numel(),
                                _stream(q))
    _check(st, "tq_attn_query_prep")
    return prep


def tq_attn_logits_prepped(codec: Codec, prep, shape, k: Packed, ctx_len: int, n_kv_heads: int, logits=None):
    """shape = (batch, n_queries, n_q_heads) of the prepared queries."""
    torch = _torch()
    batch, nq, hq = shape
    if logits is None:
        logits = torch.empty((batch, hq, nq, ctx_len), dtype=torch.float32, device=prep.device)
    st = lib.tq_attn_logits_prepped(codec.handle, _ptr(prep), prep.numel(), batch, hq, n_kv_heads, nq, k.c(),
                                    ctx_len, _ptr(logits), _stream(prep))
    _check(st, "tq_attn_logits_prepped")
    return logits


# ---------------------------------------------------------------- decode attention
def tq_decode_attn_workspace(ck: Codec, cv: Codec, batch: int, n_q_heads: int, n_kv_heads: int, ctx_len: int) -> int:
    return lib.tq_decode_attn_workspace(ck.handle, cv.handle, batch, n_q_heads, n_kv_heads, ctx_len)


def tq_decode_attn(ck: Codec, cv: Codec, q, k: Packed, v: Packed, ctx_len: int, n_kv_heads: int,
                   softmax_scale: float, out_dtype=None, out=None, ws=None):
    """q: [batch][n_q_heads][d]; returns out [batch][n_q_heads][d] (fp32 or bf16)."""
    torch = _torch()
    batch, hq, d = q.shape
    out_dtype = out_dtype or torch.bfloat16
    if out is None:
        out = torch.empty((batch, hq, d), dtype=out_dtype, device=q.device)
    need = tq_decode_attn_workspace(ck, cv, batch, hq, n_kv_heads, ctx_len)
    ws = ws if ws is not None else _workspace(need, q.device)
    st = lib.tq_decode_attn(ck.handle, cv.handle, _ptr(q), _dt(q), batch, hq, n_kv_heads, k.c(), v.c(), ctx_len,
                            float(softmax_scale), _ptr(out), _dt(out), _ptr(ws), ws.numel(), _stream(q))
    _check(st, "tq_decode_attn")
    return out


def tq_decode_attn_no_alloc(ck: Codec, cv: Codec, q, k: Packed, v: Packed, ctx_len: int, n_kv_heads: int,
                            softmax_scale: float, out):
    """tq_decode_attn without a workspace (the library's static scratch);
    `out` [batch][n_q_heads][d] is the caller's, so nothing is allocated."""
    batch, hq, d = q.shape
    st = lib.tq_decode_attn_no_alloc(ck.handle, cv.handle, _ptr(q), _dt(q), batch, hq, n_kv_heads, k.c(), v.c(),
                                     ctx_len, float(softmax_scale), _ptr(out), _dt(out), _stream(q))
    _check(st, "tq_decode_attn_no_alloc")
    return out


def tq_decode_attn_sparse_v(ck: Codec, cv: Codec, q, k: Packed, v: Packed, ctx_len: int, n_kv_heads: int,
                            softmax_scale: float, v_gate: float, out_dtype=None, out=None, ws=None):
    """tq_decode_attn with the value term of (head, position) dropped when its
    chunk-local weight is below v_gate."""
    torch = _torch()
    batch, hq, d = q.shape
    out_dtype = out_dtype or torch.bfloat16
    if out is None:
        out = torch.empty((batch, hq, d), dtype=out_dtype, device=q.device)
    need = tq_decode_attn_workspace(ck, cv, batch, hq, n_kv_heads, ctx_len)
    ws = ws if ws is not None else _workspace(need, q.device)
    st = lib.tq_decode_attn_sparse_v(ck.handle, cv.handle, _ptr(q), _dt(q), batch, hq, n_kv_heads, k.c(), v.c(),
                                     ctx_len, float(softmax_scale), float(v_gate), _ptr(out), _dt(out), _ptr(ws),
                                     ws.numel(), _stream(q))
    _check(st, "tq_decode_attn_sparse_v")
    return out


def tq_decode_attn_chunk(n_q_heads: int, n_kv_heads: int) -> int:
    return lib.tq_decode_attn_chunk(n_q_heads, n_kv_heads)


# ---------------------------------------------------------------- paged cache
def tq_encode_append_paged(codec: Codec, x, ctx_lens, page_table, page_size: int, n_pages: int, cache: Packed,
                           ws=None):
    """x: [batch][n_kv_heads][n_new][d]; ctx_lens int32 [batch], page_table
    int32 [batch][max_pages] (device).  Writes into `cache` in place."""
    batch, hkv, n_new, d = x.shape
    assert d == codec.d and x.is_contiguous() and page_table.is_contiguous()
    need = lib.tq_encode_append_paged_workspace(codec.handle, batch, hkv, n_new)
    ws = ws if ws is not None else _workspace(need, x.device)
    st = lib.tq_encode_append_paged(codec.handle, _ptr(x), _dt(x), batch, hkv, n_new, _ptr(ctx_lens),
                                    _ptr(page_table), page_table.shape[1], page_size, n_pages, cache.c(), _ptr(ws),
                                    ws.numel(), _stream(x))
    _check(st, "tq_encode_append_paged")
    return cache


def tq_decode_attn_paged(ck: Codec, cv: Codec, q, k_cache: Packed, v_cache: Packed, ctx_lens, page_table,
                         page_size: int, max_ctx: int, n_kv_heads: int, softmax_scale: float, v_gate: float = 0.0,
                         out_dtype=None, out=None, ws=None):
    """q: [batch][n_q_heads][d]; returns out [batch][n_q_heads][d]."""
    torch = _torch()
    batch, hq, d = q.shape
    out_dtype = out_dtype or torch.bfloat16
    if out is None:
        out = torch.empty((batch, hq, d), dtype=out_dtype, device=q.device)
    need = lib.tq_decode_attn_paged_workspace(ck.handle, cv.handle, batch, hq, n_kv_heads, max_ctx)
    ws = ws if ws is not None else _workspace(need, q.device)
    st = lib.tq_decode_attn_paged(ck.handle, cv.handle, _ptr(q), _dt(q), batch, hq, n_kv_heads, k_cache.c(),
                                  v_cache.c(), _ptr(ctx_lens), _ptr(page_table), page_table.shape[1], page_size,
                                  max_ctx, float(softmax_scale), float(v_gate), _ptr(out), _dt(out), _ptr(ws),
                                  ws.numel(), _stream(q))
    _check(st, "tq_decode_attn_paged")
    return out


def tq_attn_logits_paged(codec: Codec, q, k_cache: Packed, ctx_lens, page_table, page_size: int, max_ctx: int,
                         n_kv_heads: int, logits=None, ws=None):
    """q: [batch][n_queries][n_q_heads][d]; returns logits [batch][n_q_heads][n_queries][max_ctx] (fp32);
    positions at or past ctx_lens[b] are not written."""
    torch = _torch()
    batch, nq, hq, d = q.shape
    if logits is None:
        logits = torch.zeros((batch, hq, nq, max_ctx), dtype=torch.float32, device=q.device)
    need = lib.tq_attn_logits_paged_workspace(codec.handle, batch, hq, n_kv_heads, nq)
    ws = ws if ws is not None else _workspace(need, q.device)
    st = lib.tq_attn_logits_paged(codec.handle, _ptr(q), _dt(q), batch, hq, n_kv_heads, nq, k_cache.c(),
                                  _ptr(ctx_lens), _ptr(page_table), page_table.shape[1], page_size, max_ctx,
                                  _ptr(logits), _ptr(ws), ws.numel(), _stream(q))
    _check(st, "tq_attn_logits_paged")
    return logits


# ---------------------------------------------------------------- search
def tq_search_workspace(codec: Codec, n_db: int, n_queries: int, topk: int) -> int:
    return lib.tq_search_workspace(codec.handle, n_db, n_queries, topk)


def tq_search_topk(codec: Codec, db: Packed, queries, topk: int, out_idx=None, out_score=None, ws=None):
    torch = _torch()
    nq = queries.shape[0]
    assert queries.dtype == torch.float32 and queries.is_contiguous()
    if out_idx is None:
        out_idx = torch.empty((nq, topk), dtype=torch.int64, device=queries.device)
    if out_score is None:
        out_score = torch.empty((nq, topk), dtype=torch.float32, device=queries.device)
    need = tq_search_workspace(codec, db.n, nq, topk)
    ws = ws if ws is not None else _workspace(need, queries.device)
    st = lib.tq_search_topk(codec.handle, db.c(), db.n, _ptr(queries), nq, topk, _ptr(out_idx), _ptr(out_score),
                            _ptr(ws), ws.numel(), _stream(queries))
    _check(st, "tq_search_topk")
    return out_idx, out_score


def tq_diag_stream(src, dst=None, sink=None):
    """Streaming ceiling (measurement helper, not part of the method): reads
    the device tensor src and writes dst (if given) in one launch.  sink:
    int32 device tensor of tq_diag_stream_sink_words() words (allocated when
    None); returns it."""
    torch = _torch()
    rb = src.numel() * src.element_size()
    wb = 0 if dst is None else dst.numel() * dst.element_size()
    if sink is None:
        sink = torch.empty(max(1, lib.tq_diag_stream_sink_words(rb)), dtype=torch.int32, device=src.device)
    st = lib.tq_diag_stream(_ptr(src), rb, None if dst is None else _ptr(dst), wb, _ptr(sink), _stream(src))
    _check(st, "tq_diag_stream")
    return sink

// C-ABI layer: argument validation, workspace sizing, error strings, and the
// dispatch to the kernel launchers.  Validation happens before any HIP call, so
// an invalid request has no side effect.
#include <cstdio>
#include <cstdlib>
#include <string>

#include "tq_internal.h"

namespace tq {

namespace {
thread_local std::string g_last_error;
}

void set_error(const std::string& msg) { g_last_error = msg; }
void clear_error() { g_last_error.clear(); }

}  // namespace tq

using tq::set_error;

extern "C" const char* tq_status_string(tq_status_t s) {
  switch (s) {
    case TQ_SUCCESS: return "TQ_SUCCESS";
    case TQ_ERROR_INVALID_VALUE: return "TQ_ERROR_INVALID_VALUE";
    case TQ_ERROR_NOT_SUPPORTED: return "TQ_ERROR_NOT_SUPPORTED";
    case TQ_ERROR_MISALIGNED: return "TQ_ERROR_MISALIGNED";
    case TQ_ERROR_WORKSPACE_TOO_SMALL: return "TQ_ERROR_WORKSPACE_TOO_SMALL";
    case TQ_ERROR_OUT_OF_MEMORY: return "TQ_ERROR_OUT_OF_MEMORY";
    case TQ_ERROR_HIP: return "TQ_ERROR_HIP";
  }
  return "TQ_ERROR_UNKNOWN";
}

extern "C" const char* tq_last_error(void) { return tq::g_last_error.c_str(); }
extern "C" int32_t tq_abi_version(void) { return TQ_ABI_VERSION; }

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t dtype_size(tq_dtype_t dt) { return dt == TQ_F32 ? 4 : 2; }

bool valid_dtype(tq_dtype_t dt) { return dt == TQ_F32 || dt == TQ_BF16 || dt == TQ_F16; }

// The kernels read and write record words and input vectors with 16-byte
// vector loads and stores, so codes, signs and the q/k/v/x arrays must be
// 16-byte aligned; ν and γ are read as floats (4 bytes).  This check runs
// first in every call that takes packed arrays, before the codec is looked
// at, on every non-NULL pointer (a NULL one is reported later, once the codec
// says whether the array is needed).
tq_status_t check_packed_alignment(const tq_packed_t& p, const char* name) {
  if (!aligned(p.codes, 16) || !aligned(p.signs, 16) || !aligned(p.norm, 4) || !aligned(p.rnorm, 4)) {
    set_error(std::string(name) + ": codes and signs must be 16-byte aligned, norm and rnorm 4-byte aligned");
    return TQ_ERROR_MISALIGNED;
  }
  return TQ_SUCCESS;
}

// Records of an MSE-only codec (qjl false) have no signs and no γ: those two
// pointers are ignored and may be NULL.
tq_status_t check_packed(const tq_packed_t& p, const char* name, bool qjl = true) {
  if (!p.codes || !p.norm || (qjl && (!p.signs || !p.rnorm))) {
    set_error(std::string(name) + ": a packed array pointer is NULL");
    return TQ_ERROR_INVALID_VALUE;
  }
  return check_packed_alignment(p, name);
}

// Input vectors (q, k, v, x, search queries): 16-byte aligned, see above.
bool vec_aligned(const void* p) { return aligned(p, 16); }

tq_status_t check_ws(void* ws, size_t have, size_t need) {
  if (have < need) {
    set_error("workspace too small: need " + std::to_string(need) + " bytes, got " + std::to_string(have));
    return TQ_ERROR_WORKSPACE_TOO_SMALL;
  }
  if (need > 0 && (!ws || !aligned(ws, 16))) {
    set_error("workspace must be non-NULL and 16-byte aligned");
    return ws ? TQ_ERROR_MISALIGNED : TQ_ERROR_INVALID_VALUE;
  }
  return TQ_SUCCESS;
}

tq_status_t finish(hipError_t e, const char* what) {
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) {
    set_error(std::string(what) + ": " + hipGetErrorString(e));
    return TQ_ERROR_HIP;
  }
  return TQ_SUCCESS;
}

bool log_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("TQ_LOG");
    return v && v[0] == '1';
  }();
  return on;
}

tq_status_t check_heads(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads) {
  if (batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0) {
    set_error("need batch >= 0, n_q_heads > 0, n_kv_heads > 0 and n_q_heads % n_kv_heads == 0");
    return TQ_ERROR_INVALID_VALUE;
  }
  return TQ_SUCCESS;
}

// The logits kernels index keys within a head in 32 bits (a grid row spans at
// most 2^31 keys, with room for the last block's rounding).
constexpr int64_t kMaxLogitsCtx = (int64_t{1} << 31) - (int64_t{1} << 16);

// The logits and search estimators need the QJL stage (an MSE-only codec's
// inner products are biased); such codecs serve as value codecs only.
tq_status_t need_qjl(const tq_codec_s* c, const char* what) {
  if (c->qjl) return TQ_SUCCESS;
  set_error(std::string(what) + " needs a two-stage codec (an MSE-only codec is a value codec)");
  return TQ_ERROR_NOT_SUPPORTED;
}

// Scoring reads row records: a codec whose records are stored in 32-row
// blocks is a value codec (decode attention's cv) only.
tq_status_t need_rows(const tq_codec_s* c, const char* what) {
  if (!c->vblock) return TQ_SUCCESS;
  set_error(std::string(what) + " reads row records; a codec in 32-row blocks serves as the value codec of decode attention only");
  return TQ_ERROR_NOT_SUPPORTED;
}

}  // namespace

// ---------------------------------------------------------------- encode
extern "C" size_t tq_encode_workspace(tq_codec_t c, int64_t n_vec) {
  if (!c || n_vec < 0) return 0;
  return tq::encode_ws_bytes(c, n_vec);
}

extern "C" tq_status_t tq_encode_kv(tq_codec_t c, const void* k, const void* v, tq_dtype_t dt,
                                    int64_t n_vec, tq_packed_t k_out, tq_packed_t v_out, void* ws,
                                    size_t ws_bytes, void* stream) {
  tq::clear_error();
  tq_status_t st = check_packed_alignment(k_out, "k_out");
  if (st != TQ_SUCCESS) return st;
  if (v && (st = check_packed_alignment(v_out, "v_out")) != TQ_SUCCESS) return st;
  if (!vec_aligned(k) || !vec_aligned(v)) { set_error("k/v must be 16-byte aligned"); return TQ_ERROR_MISALIGNED; }
  if (!c) { set_error("codec is NULL"); return TQ_ERROR_INVALID_VALUE; }
  if (!valid_dtype(dt)) { set_error("bad dtype"); return TQ_ERROR_INVALID_VALUE; }
  if (n_vec < 0) { set_error("n_vec < 0"); return TQ_ERROR_INVALID_VALUE; }
  if (c->vblock && n_vec % 32 != 0) {
    set_error("a codec in 32-row blocks encodes whole blocks: n_vec must be a multiple of 32");
    return TQ_ERROR_INVALID_VALUE;
  }
  if (n_vec == 0) return TQ_SUCCESS;
  if (!k) { set_error("k is NULL"); return TQ_ERROR_INVALID_VALUE; }
  st = check_packed(k_out, "k_out", c->qjl);
  if (st != TQ_SUCCESS) return st;
  if (v && (st = check_packed(v_out, "v_out", c->qjl)) != TQ_SUCCESS) return st;
  if ((st = check_ws(ws, ws_bytes, tq::encode_ws_bytes(c, n_vec))) != TQ_SUCCESS) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (log_enabled()) std::fprintf(stderr, "[tq] encode n=%lld d=%d bits=%d v=%d\n", (long long)n_vec, c->prm.d, c->host.bits, v != nullptr);
  hipError_t e = tq::launch_encode(c, k, dt, n_vec, k_out, ws, s);
  if (e == hipSuccess && v) e = tq::launch_encode(c, v, dt, n_vec, v_out, ws, s);
  return finish(e, "tq_encode_kv launch");
}

// ---------------------------------------------------------------- logits
extern "C" size_t tq_attn_logits_workspace(tq_codec_t c, int32_t batch, int32_t n_q_heads,
                                           int32_t n_kv_heads, int32_t n_queries) {
  if (!c || batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || n_queries < 0) return 0;
  return tq::logits_ws_bytes(c, batch, n_q_heads, n_kv_heads, n_queries);
}

extern "C" tq_status_t tq_attn_logits(tq_codec_t c, const void* q, tq_dtype_t q_dt, int32_t batch,
                                      int32_t n_q_heads, int32_t n_kv_heads, int32_t n_queries,
                                      tq_packed_t k, int64_t ctx_len, float* logits, void* ws,
                                      size_t ws_bytes, void* stream) {
  tq::clear_error();
  tq_status_t st = check_packed_alignment(k, "k");
  if (st != TQ_SUCCESS) return st;
  if (!vec_aligned(q)) { set_error("q must be 16-byte aligned"); return TQ_ERROR_MISALIGNED; }
  if (!c) { set_error("codec is NULL"); return TQ_ERROR_INVALID_VALUE; }
  if (!valid_dtype(q_dt)) { set_error("bad q dtype"); return TQ_ERROR_INVALID_VALUE; }
  if ((st = need_qjl(c, "tq_attn_logits")) != TQ_SUCCESS) return st;
  if ((st = need_rows(c, "tq_attn_logits")) != TQ_SUCCESS) return st;
  if ((st = check_heads(batch, n_q_heads, n_kv_heads)) != TQ_SUCCESS) return st;
  if (n_queries < 0 || ctx_len < 0) { set_error("n_queries and ctx_len must be >= 0"); return TQ_ERROR_INVALID_VALUE; }
  if (ctx_len > kMaxLogitsCtx) { set_error("ctx_len must be below 2^31 - 2^16"); return TQ_ERROR_NOT_SUPPORTED; }
  if (batch == 0 || n_queries == 0 || ctx_len == 0) return TQ_SUCCESS;
  if (!q || !logits) { set_error("q or logits is NULL"); return TQ_ERROR_INVALID_VALUE; }
  if (!aligned(logits, 4)) { set_error("logits misaligned"); return TQ_ERROR_MISALIGNED; }
  if ((st = check_packed(k, "k")) != TQ_SUCCESS) return st;
  if ((st = check_ws(ws, ws_bytes, tq::logits_ws_bytes(c, batch, n_q_heads, n_kv_heads, n_queries))) != TQ_SUCCESS) return st;
  if (log_enabled()) std::fprintf(stderr, "[tq] logits b=%d hq=%d hkv=%d nq=%d ctx=%lld\n", batch, n_q_heads, n_kv_heads, n_queries, (long long)ctx_len);
  hipError_t e = tq::launch_logits(c, q, q_dt, batch, n_q_heads, n_kv_heads, n_queries, k, ctx_len,
                                   logits, ws, static_cast<hipStream_t>(stream));
  return finish(e, "tq_attn_logits launch");
}

extern "C" tq_status_t tq_attn_query_prep(tq_codec_t c, const void* q, tq_dtype_t q_dt, int32_t batch,
                                          int32_t n_q_heads, int32_t n_kv_heads, int32_t n_queries, void* prep,
                                          size_t prep_bytes, void* stream) {
  tq::clear_error();
  if (!vec_aligned(q)) { set_error("q must be 16-byte aligned"); return TQ_ERROR_MISALIGNED; }
  if (!c) { set_error("codec is NULL"); return TQ_ERROR_INVALID_VALUE; }
  if (!valid_dtype(q_dt)) { set_error("bad q dtype"); return TQ_ERROR_INVALID_VALUE; }
  tq_status_t st = need_qjl(c, "tq_attn_query_prep");
  if (st != TQ_SUCCESS) return st;
  if ((st = check_heads(batch, n_q_heads, n_kv_heads)) != TQ_SUCCESS) return st;
  if (n_queries < 0) { set_error("n_queries must be >= 0"); return TQ_ERROR_INVALID_VALUE; }
  if (batch == 0 || n_queries == 0) return TQ_SUCCESS;
  if (!q) { set_error("q is NULL"); return TQ_ERROR_INVALID_VALUE; }
  if ((st = check_ws(prep, prep_bytes, tq::logits_ws_bytes(c, batch, n_q_heads, n_kv_heads, n_queries))) != TQ_SUCCESS) return st;
  hipError_t e = tq::launch_logits_prep(c, q, q_dt, batch, n_q_heads, n_kv_heads, n_queries, prep,
                                        static_cast<hipStream_t>(stream));
  return finish(e, "tq_attn_query_prep launch");
}

extern "C" tq_status_t tq_attn_logits_prepped(tq_codec_t c, const void* prep, size_t prep_bytes, int32_t batch,
                                              int32_t n_q_heads, int32_t n_kv_heads, int32_t n_queries,
                                              tq_packed_t k, int64_t ctx_len, float* logits, void* stream) {
  tq::clear_error();
  tq_status_t st = check_packed_alignment(k, "k");
  if (st != TQ_SUCCESS) return st;
  if (!c) { set_error("codec is NULL"); return TQ_ERROR_INVALID_VALUE; }
  if ((st = need_qjl(c, "tq_attn_logits_prepped")) != TQ_SUCCESS) return st;
  if ((st = need_rows(c, "tq_attn_logits_prepped")) != TQ_SUCCESS) return st;
  if ((st = check_heads(batch, n_q_heads, n_kv_heads)) != TQ_SUCCESS) return st;
  if (n_queries < 0 || ctx_len < 0) { set_error("n_queries and ctx_len must be >= 0"); return TQ_ERROR_INVALID_VALUE; }
  if (ctx_len > kMaxLogitsCtx) { set_error("ctx_len must be below 2^31 - 2^16"); return TQ_ERROR_NOT_SUPPORTED; }
  if (batch == 0 || n_queries == 0 || ctx_len == 0) return TQ_SUCCESS;
  if (!logits) { set_error("logits is NULL"); return TQ_ERROR_INVALID_VALUE; }
  if (!aligned(logits, 4)) { set_error("logits misaligned"); return TQ_ERROR_MISALIGNED; }
  if ((st = check_packed(k, "k")) != TQ_SUCCESS) return st;
  if ((st = check_ws(const_cast<void*>(prep), prep_bytes, tq::logits_ws_bytes(c, batch, n_q_heads, n_kv_heads, n_queries))) != TQ_SUCCESS) return st;
  hipError_t e = tq::launch_logits_prepped(c, prep, batch, n_q_heads, n_kv_heads, n_queries, k, ctx_len, logits,
                                           static_cast<hipStream_t>(stream));
  return finish(e, "tq_attn_logits_prepped launch");
}

// ---------------------------------------------------------------- decode attention
extern "C" size_t tq_decode_attn_workspace(tq_codec_t ck, tq_codec_t cv, int32_t batch,
                                           int32_t n_q_heads, int32_t n_kv_heads, int64_t ctx_len) {
  if (!ck || !cv || batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || ctx_len < 0) return 0;
  return tq::decode_ws_bytes(ck, cv, batch, n_q_heads, n_kv_heads, ctx_len);
}

namespace {
tq_status_t decode_common(tq_codec_t ck, tq_codec_t cv, const void* q, tq_dtype_t q_dt, int32_t batch,
                          int32_t n_q_heads, int32_t n_kv_heads, tq_packed_t k, tq_packed_t v, int64_t ctx_len,
                          float softmax_scale, bool sparse_v, float v_gate, const tq::PageMap* pm, void* out,
                          tq_dtype_t out_dt, void* ws, size_t ws_bytes, void* stream, const char* name,
                          bool no_alloc = false) {
  tq_status_t st = check_packed_alignment(k, "k");
  if (st != TQ_SUCCESS) return st;
  if ((st = check_packed_alignment(v, "v")) != TQ_SUCCESS) return st;
  if (!vec_aligned(q)) { set_error("q must be 16-byte aligned"); return TQ_ERROR_MISALIGNED; }
  if (!ck || !cv) { set_error("codec is NULL"); return TQ_ERROR_INVALID_VALUE; }
  if (ck->prm.d != cv->prm.d) { set_error("K and V codecs must share head_dim"); return TQ_ERROR_INVALID_VALUE; }
  if (ck->polar || cv->polar) {
    if (!tq::decode_polar_shape_ok(ck, cv)) {
      set_error("decode attention with a polar codec needs head_dim 128 or 256 (the same for K and V), qjl_dim equal "
                "to head_dim and V in row records");
      return TQ_ERROR_NOT_SUPPORTED;
    }
  }
  if (!ck->qjl) { set_error("the K codec must be a two-stage codec (an MSE-only codec is a value codec)"); return TQ_ERROR_NOT_SUPPORTED; }
  if (!valid_dtype(q_dt) || (out_dt != TQ_F32 && out_dt != TQ_BF16)) { set_error("bad dtype"); return TQ_ERROR_INVALID_VALUE; }
  if ((st = check_heads(batch, n_q_heads, n_kv_heads)) != TQ_SUCCESS) return st;
  if (ctx_len < 1) { set_error("ctx_len must be >= 1"); return TQ_ERROR_INVALID_VALUE; }
  if (ck->vblock) {
    set_error("the K codec must store row records (a codec in 32-row blocks is a value codec)");
    return TQ_ERROR_NOT_SUPPORTED;
  }
  if (cv->vblock && !tq::decode_paged_supported(ck, cv, n_q_heads, n_kv_heads)) {
    set_error("a V cache in 32-row blocks needs head_dim 128 for K and V, qjl_dim 128 and at most 4 query heads per KV head");
    return TQ_ERROR_NOT_SUPPORTED;
  }
  if (cv->vblock && !pm && ctx_len % 32 != 0) {
    set_error("a contiguous V cache in 32-row blocks needs ctx_len % 32 == 0 (each head's rows start a block)");
    return TQ_ERROR_NOT_SUPPORTED;
  }
  if (!(softmax_scale == softmax_scale)) { set_error("softmax_scale is NaN"); return TQ_ERROR_INVALID_VALUE; }
  const char* why = nullptr;
  if (!tq::decode_supported(cv, n_q_heads, n_kv_heads, ctx_len, &why)) { set_error(why); return TQ_ERROR_NOT_SUPPORTED; }
  if (batch == 0) return TQ_SUCCESS;
  if (!q || !out) { set_error("q or out is NULL"); return TQ_ERROR_INVALID_VALUE; }
  if (!aligned(out, dtype_size(out_dt))) { set_error("out misaligned"); return TQ_ERROR_MISALIGNED; }
  if ((st = check_packed(k, "k")) != TQ_SUCCESS) return st;
  if ((st = check_packed(v, "v", cv->qjl)) != TQ_SUCCESS) return st;
  if (no_alloc) {
    // the static scratch replaces the workspace: refuse what does not fit it
    const size_t need = tq::decode_ws_bytes(ck, cv, batch, n_q_heads, n_kv_heads, ctx_len);
    if (need > tq::kNoAllocScratchBytes) {
      set_error(std::string(name) + ": this call needs " + std::to_string(need) +
                " bytes of scratch, above the static maximum of " + std::to_string(tq::kNoAllocScratchBytes) +
                " bytes (call tq_decode_attn with a workspace instead)");
      return TQ_ERROR_NOT_SUPPORTED;
    }
    const hipError_t e = tq::no_alloc_scratch(&ws);
    if (e != hipSuccess) {
      set_error(std::string(name) + ": looking up the static scratch failed: " + hipGetErrorString(e));
      return TQ_ERROR_HIP;
    }
    ws_bytes = tq::kNoAllocScratchBytes;
  }
  if ((st = check_ws(ws, ws_bytes, tq::decode_ws_bytes(ck, cv, batch, n_q_heads, n_kv_heads, ctx_len))) != TQ_SUCCESS) return st;
  if (log_enabled())
    std::fprintf(stderr, "[tq] %s b=%d hq=%d hkv=%d ctx=%lld gate=%g\n", name, batch, n_q_heads, n_kv_heads,
                 (long long)ctx_len, sparse_v ? v_gate : 0.0);
  hipError_t e = tq::launch_decode(ck, cv, q, q_dt, batch, n_q_heads, n_kv_heads, k, v, ctx_len, softmax_scale,
                                   sparse_v, v_gate, pm, out, out_dt, ws, static_cast<hipStream_t>(stream));
  return finish(e, name);
}
}  // namespace

extern "C" tq_status_t tq_decode_attn(tq_codec_t ck, tq_codec_t cv, const void* q, tq_dtype_t q_dt,
                                      int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                      tq_packed_t k, tq_packed_t v, int64_t ctx_len,
                                      float softmax_scale, void* out, tq_dtype_t out_dt, void* ws,
                                      size_t ws_bytes, void* stream) {
  tq::clear_error();
  return decode_common(ck, cv, q, q_dt, batch, n_q_heads, n_kv_heads, k, v, ctx_len, softmax_scale, false, 0.f,
                       nullptr, out, out_dt, ws, ws_bytes, stream, "tq_decode_attn");
}

extern "C" tq_status_t tq_decode_attn_no_alloc(tq_codec_t ck, tq_codec_t cv, const void* q, tq_dtype_t q_dt,
                                               int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                               tq_packed_t k, tq_packed_t v, int64_t ctx_len, float softmax_scale,
                                               void* out, tq_dtype_t out_dt, void* stream) {
  tq::clear_error();
  return decode_common(ck, cv, q, q_dt, batch, n_q_heads, n_kv_heads, k, v, ctx_len, softmax_scale, false, 0.f,
                       nullptr, out, out_dt, nullptr, 0, stream, "tq_decode_attn_no_alloc", true);
}

extern "C" tq_status_t tq_decode_attn_sparse_v(tq_codec_t ck, tq_codec_t cv, const void* q, tq_dtype_t q_dt,
                                               int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                               tq_packed_t k, tq_packed_t v, int64_t ctx_len,
                                               float softmax_scale, float v_gate, void* out, tq_dtype_t out_dt,
                                               void* ws, size_t ws_bytes, void* stream) {
  tq::clear_error();
  if (!(v_gate >= 0.f && v_gate < 1.f)) { set_error("v_gate must be in [0, 1)"); return TQ_ERROR_INVALID_VALUE; }
  return decode_common(ck, cv, q, q_dt, batch, n_q_heads, n_kv_heads, k, v, ctx_len, softmax_scale, true, v_gate,
                       nullptr, out, out_dt, ws, ws_bytes, stream, "tq_decode_attn_sparse_v");
}

extern "C" int32_t tq_decode_attn_chunk(int32_t n_q_heads, int32_t n_kv_heads) {
  if (n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0) return 0;
  return tq::decode_chunk(n_q_heads, n_kv_heads);
}

// ---------------------------------------------------------------- paged cache
extern "C" size_t tq_encode_append_paged_workspace(tq_codec_t c, int32_t batch, int32_t n_kv_heads, int32_t n_new) {
  if (!c || batch < 0 || n_kv_heads <= 0 || n_new < 0) return 0;
  return tq::append_paged_ws_bytes(c, static_cast<int64_t>(batch) * n_kv_heads * n_new);
}

extern "C" tq_status_t tq_encode_append_paged(tq_codec_t c, const void* x, tq_dtype_t dt, int32_t batch,
                                              int32_t n_kv_heads, int32_t n_new, const int32_t* ctx_lens,
                                              const int32_t* page_table, int32_t max_pages, int32_t page_size,
                                              int32_t n_pages, tq_packed_t cache, void* ws, size_t ws_bytes,
                                              void* stream) {
  tq::clear_error();
  tq_status_t st = check_packed_alignment(cache, "cache");
  if (st != TQ_SUCCESS) return st;
  if (!vec_aligned(x)) { set_error("x must be 16-byte aligned"); return TQ_ERROR_MISALIGNED; }
  if (!c) { set_error("codec is NULL"); return TQ_ERROR_INVALID_VALUE; }
  if (!valid_dtype(dt)) { set_error("bad dtype"); return TQ_ERROR_INVALID_VALUE; }
  if (batch < 0 || n_kv_heads <= 0 || n_new < 0) {
    set_error("need batch >= 0, n_kv_heads > 0, n_new >= 0");
    return TQ_ERROR_INVALID_VALUE;
  }
  if (max_pages <= 0 || page_size <= 0 || n_pages <= 0) {
    set_error("max_pages, page_size and n_pages must be > 0");
    return TQ_ERROR_INVALID_VALUE;
  }
  if (c->vblock && page_size % 32 != 0) {
    set_error("a cache in 32-row blocks needs page_size % 32 == 0 (a block must not span pages)");
    return TQ_ERROR_INVALID_VALUE;
  }
  if (batch == 0 || n_new == 0) return TQ_SUCCESS;
  if (!x || !ctx_lens || !page_table) { set_error("x, ctx_lens or page_table is NULL"); return TQ_ERROR_INVALID_VALUE; }
  if (!aligned(ctx_lens, 4) || !aligned(page_table, 4)) {
    set_error("ctx_lens or page_table misaligned");
    return TQ_ERROR_MISALIGNED;
  }
  if ((st = check_packed(cache, "cache", c->qjl)) != TQ_SUCCESS) return st;
  const int64_t n = static_cast<int64_t>(batch) * n_kv_heads * n_new;
  if ((st = check_ws(ws, ws_bytes, tq::append_paged_ws_bytes(c, n))) != TQ_SUCCESS) return st;
  hipError_t e = tq::launch_append_paged(c, x, dt, batch, n_kv_heads, n_new, ctx_lens, page_table, max_pages,
                                         page_size, n_pages, cache, ws, static_cast<hipStream_t>(stream));
  return finish(e, "tq_encode_append_paged launch");
}

extern "C" size_t tq_decode_attn_paged_workspace(tq_codec_t ck, tq_codec_t cv, int32_t batch, int32_t n_q_heads,
                                                 int32_t n_kv_heads, int64_t max_ctx) {
  return tq_decode_attn_workspace(ck, cv, batch, n_q_heads, n_kv_heads, max_ctx);
}

extern "C" tq_status_t tq_decode_attn_paged(tq_codec_t ck, tq_codec_t cv, const void* q, tq_dtype_t q_dt,
                                            int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                            tq_packed_t k_cache, tq_packed_t v_cache, const int32_t* ctx_lens,
                                            const int32_t* page_table, int32_t max_pages, int32_t page_size,
                                            int64_t max_ctx, float softmax_scale, float v_gate, void* out,
                                            tq_dtype_t out_dt, void* ws, size_t ws_bytes, void* stream) {
  tq::clear_error();
  tq_status_t st = check_packed_alignment(k_cache, "k_cache");
  if (st != TQ_SUCCESS) return st;
  if ((st = check_packed_alignment(v_cache, "v_cache")) != TQ_SUCCESS) return st;
  if (!vec_aligned(q)) { set_error("q must be 16-byte aligned"); return TQ_ERROR_MISALIGNED; }
  if (!ck || !cv) { set_error("codec is NULL"); return TQ_ERROR_INVALID_VALUE; }
  if (!(v_gate >= 0.f && v_gate < 1.f)) { set_error("v_gate must be in [0, 1)"); return TQ_ERROR_INVALID_VALUE; }
  if (max_pages <= 0 || page_size <= 0 || page_size % 128 != 0) {
    set_error("need max_pages > 0 and page_size a positive multiple of 128");
    return TQ_ERROR_INVALID_VALUE;
  }
  if (max_ctx < 1 || max_ctx > static_cast<int64_t>(max_pages) * page_size) {
    set_error("need 1 <= max_ctx <= max_pages * page_size");
    return TQ_ERROR_INVALID_VALUE;
  }
  if (batch > 0 && (!ctx_lens || !page_table)) { set_error("ctx_lens or page_table is NULL"); return TQ_ERROR_INVALID_VALUE; }
  if (batch > 0 && (!aligned(ctx_lens, 4) || !aligned(page_table, 4))) {
    set_error("ctx_lens or page_table misaligned");
    return TQ_ERROR_MISALIGNED;
  }
  const tq::PageMap pm{page_table, ctx_lens, max_pages, page_size};
  return decode_common(ck, cv, q, q_dt, batch, n_q_heads, n_kv_heads, k_cache, v_cache, max_ctx, softmax_scale,
                       v_gate > 0.f, v_gate, &pm, out, out_dt, ws, ws_bytes, stream, "tq_decode_attn_paged");
}

extern "C" size_t tq_attn_logits_paged_workspace(tq_codec_t c, int32_t batch, int32_t n_q_heads,
                                                 int32_t n_kv_heads, int32_t n_queries) {
  if (!c || batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || n_queries < 0 || !tq::logits_paged_supported(c)) return 0;
  return tq::logits_paged_ws_bytes(c, batch, n_q_heads, n_kv_heads, n_queries);
}

extern "C" tq_status_t tq_attn_logits_paged(tq_codec_t c, const void* q, tq_dtype_t q_dt, int32_t batch,
                                            int32_t n_q_heads, int32_t n_kv_heads, int32_t n_queries,
                                            tq_packed_t k_cache, const int32_t* ctx_lens, const int32_t* page_table,
                                            int32_t max_pages, int32_t page_size, int64_t max_ctx, float* logits,
                                            void* ws, size_t ws_bytes, void* stream) {
  tq::clear_error();
  tq_status_t st = check_packed_alignment(k_cache, "k_cache");
  if (st != TQ_SUCCESS) return st;
  if (!vec_aligned(q)) { set_error("q must be 16-byte aligned"); return TQ_ERROR_MISALIGNED; }
  if (!c) { set_error("codec is NULL"); return TQ_ERROR_INVALID_VALUE; }
  if (!valid_dtype(q_dt)) { set_error("bad q dtype"); return TQ_ERROR_INVALID_VALUE; }
  if ((st = need_qjl(c, "tq_attn_logits_paged")) != TQ_SUCCESS) return st;
  if ((st = need_rows(c, "tq_attn_logits_paged")) != TQ_SUCCESS) return st;
  if (!tq::logits_paged_supported(c)) {
    set_error("paged logits need a polar codec, or a per-coordinate codec with head_dim 128 or 256 and qjl_dim = "
              "head_dim");
    return TQ_ERROR_NOT_SUPPORTED;
  }
  if ((st = check_heads(batch, n_q_heads, n_kv_heads)) != TQ_SUCCESS) return st;
  if (n_queries < 0) { set_error("n_queries must be >= 0"); return TQ_ERROR_INVALID_VALUE; }
  if (max_pages <= 0 || page_size <= 0 || page_size % 128 != 0) {
    set_error("need max_pages > 0 and page_size a positive multiple of 128");
    return TQ_ERROR_INVALID_VALUE;
  }
  if (max_ctx < 1 || max_ctx > static_cast<int64_t>(max_pages) * page_size) {
    set_error("need 1 <= max_ctx <= max_pages * page_size");
    return TQ_ERROR_INVALID_VALUE;
  }
  if (max_ctx > kMaxLogitsCtx) { set_error("max_ctx must be below 2^31 - 2^16"); return TQ_ERROR_NOT_SUPPORTED; }
  if (batch == 0 || n_queries == 0) return TQ_SUCCESS;
  if (!q || !logits || !ctx_lens || !page_table) {
    set_error("q, logits, ctx_lens or page_table is NULL");
    return TQ_ERROR_INVALID_VALUE;
  }
  if (!aligned(logits, 4) || !aligned(ctx_lens, 4) || !aligned(page_table, 4)) {
    set_error("logits, ctx_lens or page_table misaligned");
    return TQ_ERROR_MISALIGNED;
  }
  if ((st = check_packed(k_cache, "k_cache")) != TQ_SUCCESS) return st;
  if ((st = check_ws(ws, ws_bytes, tq::logits_paged_ws_bytes(c, batch, n_q_heads, n_kv_heads, n_queries))) !=
      TQ_SUCCESS)
    return st;
  const tq::PageMap pm{page_table, ctx_lens, max_pages, page_size};
  hipError_t e = tq::launch_logits_paged(c, q, q_dt, batch, n_q_heads, n_kv_heads, n_queries, k_cache, max_ctx, pm,
                                         logits, ws, static_cast<hipStream_t>(stream));
  return finish(e, "tq_attn_logits_paged launch");
}

// ---------------------------------------------------------------- search
extern "C" size_t tq_search_workspace(tq_codec_t c, int64_t n_db, int32_t n_queries, int32_t topk) {
  if (!c || n_db < 0 || n_queries < 0 || topk < 1) return 0;
  return tq::search_ws_bytes(c, n_db, n_queries, topk);
}

extern "C" tq_status_t tq_search_topk(tq_codec_t c, tq_packed_t db, int64_t n_db, const float* queries,
                                      int32_t n_queries, int32_t topk, int64_t* out_idx,
                                      float* out_score, void* ws, size_t ws_bytes, void* stream) {
  tq::clear_error();
  tq_status_t st = check_packed_alignment(db, "db");
  if (st != TQ_SUCCESS) return st;
  if (!vec_aligned(queries)) { set_error("queries must be 16-byte aligned"); return TQ_ERROR_MISALIGNED; }
  if (!c) { set_error("codec is NULL"); return TQ_ERROR_INVALID_VALUE; }
  if (!c->qjl) return need_qjl(c, "tq_search_topk");
  if ((st = need_rows(c, "tq_search_topk")) != TQ_SUCCESS) return st;
  if (n_db < 1 || n_queries < 0) { set_error("need n_db >= 1 and n_queries >= 0"); return TQ_ERROR_INVALID_VALUE; }
  if (topk < 1 || topk > 1024 || topk > n_db) { set_error("need 1 <= topk <= min(n_db, 1024)"); return TQ_ERROR_INVALID_VALUE; }
  if (n_queries == 0) return TQ_SUCCESS;
  if (!queries || !out_idx || !out_score) { set_error("queries/out_idx/out_score is NULL"); return TQ_ERROR_INVALID_VALUE; }
  if (!aligned(out_idx, 8) || !aligned(out_score, 4)) { set_error("search outputs misaligned"); return TQ_ERROR_MISALIGNED; }
  if ((st = check_packed(db, "db")) != TQ_SUCCESS) return st;
  if ((st = check_ws(ws, ws_bytes, tq::search_ws_bytes(c, n_db, n_queries, topk))) != TQ_SUCCESS) return st;
  if (log_enabled()) std::fprintf(stderr, "[tq] search n_db=%lld nq=%d k=%d\n", (long long)n_db, n_queries, topk);
  hipError_t e = tq::launch_search(c, db, n_db, queries, n_queries, topk, out_idx, out_score, ws,
                                   static_cast<hipStream_t>(stream));
  return finish(e, "tq_search_topk launch");
}

namespace tq {
int64_t diag_stream_sink_words(size_t read_bytes);
hipError_t launch_stream(const void* src, size_t read_bytes, void* dst, size_t write_bytes, uint32_t* sink,
                         hipStream_t s);
}  // namespace tq

extern "C" int64_t tq_diag_stream_sink_words(size_t read_bytes) { return tq::diag_stream_sink_words(read_bytes); }

extern "C" tq_status_t tq_diag_stream(const void* src, size_t read_bytes, void* dst, size_t write_bytes,
                                      uint32_t* sink, void* stream) {
  tq::clear_error();
  if (read_bytes % 16 != 0 || write_bytes % 16 != 0) {
    set_error("read_bytes and write_bytes must be multiples of 16");
    return TQ_ERROR_INVALID_VALUE;
  }
  if ((read_bytes && (!src || !sink)) || (write_bytes && !dst)) {
    set_error("src and sink (with read_bytes > 0) and dst (with write_bytes > 0) must be non-NULL");
    return TQ_ERROR_INVALID_VALUE;
  }
  if (!aligned(src, 16) || !aligned(dst, 16) || !aligned(sink, 4)) {
    set_error("src and dst must be 16-byte aligned, sink 4-byte aligned");
    return TQ_ERROR_MISALIGNED;
  }
  if (static_cast<uint64_t>(tq::diag_stream_sink_words(read_bytes)) +
          (write_bytes + 16383) / 16384 > 0x7FFFFFFFull) {
    set_error("read_bytes + write_bytes too large for one launch");
    return TQ_ERROR_INVALID_VALUE;
  }
  return finish(tq::launch_stream(src, read_bytes, dst, write_bytes, sink, static_cast<hipStream_t>(stream)),
                "tq_diag_stream launch");
}

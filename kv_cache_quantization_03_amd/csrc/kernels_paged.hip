// Paged KV cache: append-encode of new tokens into pages.
//
// A decode step adds one token per (sequence, KV head) to the cache
// (「谷歌 TurboQuant 深度拆解」 第一部分: the cache keeps every past token's K
// and V).  The cache is split into pages of page_size positions; page p holds,
// for every KV head kh, the records of its positions at rows
// (p * n_kv_heads + kh) * page_size + slot, and page_table[b][i] names the
// page of positions [i*page_size, (i+1)*page_size) of sequence b.
//
// The new tokens are encoded by the ordinary encode kernels into a staging
// area of the workspace, then one scatter kernel copies every record to its
// page slot: the encode stays the one tested path, and a decode step's few
// hundred records cost one more small launch.
#include "kernels_common.h"

namespace tq {

namespace {

// One thread per (record, 32-bit word); words of a record: code words, sign
// words, ν, γ (an MSE-only codec: code words and ν; sw = 0, qjl = 0).  Records
// whose position falls outside the page table, or whose page id is outside
// [0, n_pages), are not written.
__global__ __launch_bounds__(256) void scatter_paged_kernel(tq_packed_t src, int cw, int sw, int qjl, int n_kv_heads,
                                                            int n_new, int64_t n_rec,
                                                            const int32_t* __restrict__ ctx_lens,
                                                            const int32_t* __restrict__ page_table, int max_pages,
                                                            int page_size, int n_pages, tq_packed_t dst) {
  const int words = cw + sw + 1 + qjl;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= n_rec * words) return;
  const int64_t i = e / words;
  const int w = static_cast<int>(e % words);
  const int t = static_cast<int>(i % n_new);
  const int kh = static_cast<int>((i / n_new) % n_kv_heads);
  const int b = static_cast<int>(i / (static_cast<int64_t>(n_new) * n_kv_heads));
  const int64_t pos = static_cast<int64_t>(ctx_lens[b]) + t;
  if (pos < 0 || pos / page_size >= max_pages) return;
  const int page = page_table[static_cast<int64_t>(b) * max_pages + pos / page_size];
  if (page < 0 || page >= n_pages) return;
  const int64_t row = (static_cast<int64_t>(page) * n_kv_heads + kh) * page_size + pos % page_size;
  if (w < cw) {
    dst.codes[row * cw + w] = src.codes[i * cw + w];
  } else if (w < cw + sw) {
    dst.signs[row * sw + (w - cw)] = src.signs[i * sw + (w - cw)];
  } else if (w == cw + sw) {
    dst.norm[row] = src.norm[i];
  } else {
    dst.rnorm[row] = src.rnorm[i];
  }
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

// Staging records (codes, signs, ν, γ, each 256-byte aligned), then the encode's own workspace.
size_t append_paged_ws_bytes(const tq_codec_s* c, int64_t n_rec) {
  const size_t cw = c->prm.code_words, sw = c->prm.sign_words;
  return align256(n_rec * cw * 4) + align256(n_rec * sw * 4) + 2 * align256(n_rec * 4) + encode_rows_ws_bytes(c, n_rec);
}

hipError_t launch_append_paged(const tq_codec_s* c, const void* x, tq_dtype_t dt, int batch, int n_kv_heads,
                               int n_new, const int32_t* ctx_lens, const int32_t* page_table, int max_pages,
                               int page_size, int n_pages, tq_packed_t cache, void* ws, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(batch) * n_kv_heads * n_new;
  const int cw = c->prm.code_words, sw = c->prm.sign_words;
  uint8_t* p = static_cast<uint8_t*>(ws);
  tq_packed_t st;
  st.codes = reinterpret_cast<uint32_t*>(p);
  p += align256(n * cw * 4);
  st.signs = reinterpret_cast<uint32_t*>(p);
  p += align256(n * sw * 4);
  st.norm = reinterpret_cast<float*>(p);
  p += align256(n * 4);
  st.rnorm = reinterpret_cast<float*>(p);
  p += align256(n * 4);
  hipError_t e = launch_encode_rows(c, x, dt, n, st, reinterpret_cast<float*>(p), s);
  if (e != hipSuccess) return e;
  if (c->vblock)  // merge each record's bits into its 32-row block
    return launch_vblock_append(c, st, n_kv_heads, n_new, n, ctx_lens, page_table, max_pages, page_size, n_pages,
                                cache, s);
  const int qjl = c->qjl ? 1 : 0;
  const int64_t total = n * (cw + sw + 1 + qjl);
  hipLaunchKernelGGL(scatter_paged_kernel, dim3(static_cast<unsigned>(ceil_div(total, 256))), dim3(256), 0, s, st,
                     cw, sw, qjl, n_kv_heads, n_new, n, ctx_lens, page_table, max_pages, page_size, n_pages, cache);
  return hipGetLastError();
}

}  // namespace tq

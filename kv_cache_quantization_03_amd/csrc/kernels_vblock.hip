// Value cache in 32-row blocks (tq_codec_create_vblock; d = m = 128).
//
// Decode attention accumulates V as a contraction over keys on the matrix
// cores (「TurboQuant+ 深度解析」 第五部分: V is compressed like K; 第六部分:
// V dequantization is a large share of long-context decode), so each lane needs
// the bits of one coordinate across 32 keys, while a row record holds 32
// coordinates of one key.  Transposing in the decode kernel costs about a third
// of its instructions at every step; this layout stores the transposed words
// once, at encode:
//   block B = rows 32B..32B+31; for plane p (the b code planes, then the sign
//   plane in the signs array) and coordinate j = 16cb + n (n < 16, cb < 8):
//     codes[(B*b + p)*128 + 8n + cb], signs[B*128 + 8n + cb]
//   hold, at bit 4i + r, the bit of row 32B + 8r + i (the order of the FP4 B
//   operand: nibble i of mask r is contraction element 8r + i).
// ν and γ stay one float per row.  The arrays have the sizes of row records.
#include "mfma_common.h"

namespace tq {

namespace {

// One wave per 128 rows: the decode kernel's lane-to-key order and bit
// transpose (v_key_of_row, transpose32), then 16-byte stores of each lane's
// eight words per plane.  n is a multiple of 32 (checked by the caller), so
// every block is whole; a wave's blocks at or past n are not stored.
template <int NB, bool QJL>
__global__ __launch_bounds__(256) void vblock_from_rows_kernel(tq_packed_t rows, int64_t n, uint32_t* __restrict__ codes,
                                                               uint32_t* __restrict__ signs) {
  const int lane = threadIdx.x & 63, g = lane >> 4, kl = lane & 15;
  const int64_t r0 = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * 128;
  if (r0 >= n) return;  // wave-uniform
  v4u cv[2][NB], sv[2];
#pragma unroll
  for (int reg = 0; reg < 2; ++reg) {
    const int64_t key = r0 + 32 * g + v_key_of_row(kl + 16 * reg);
    const bool ok = key < n;
    const int64_t row = ok ? key : n - 1;
#pragma unroll
    for (int p = 0; p < NB; ++p) {
      const v4u w = reinterpret_cast<const v4u*>(rows.codes)[row * NB + p];
      cv[reg][p] = ok ? w : v4u{0u, 0u, 0u, 0u};
    }
    if constexpr (QJL) {
      const v4u w = reinterpret_cast<const v4u*>(rows.signs)[row];
      sv[reg] = ok ? w : v4u{0u, 0u, 0u, 0u};
    }
  }
  const int64_t blk = r0 / 32 + g;
  const bool store = blk * 32 < n;
#pragma unroll
  for (int p = 0; p < NB + (QJL ? 1 : 0); ++p) {
    uint32_t tw[8];
#pragma unroll
    for (int wb = 0; wb < 4; ++wb) {
      uint32_t a = p < NB ? cv[0][p < NB ? p : 0][wb] : sv[0][wb];
      uint32_t b = p < NB ? cv[1][p < NB ? p : 0][wb] : sv[1][wb];
      transpose32(a, b, lane);
      tw[2 * wb] = a;
      tw[2 * wb + 1] = b;
    }
    if (store) {
      uint32_t* dst = p < NB ? codes + ((blk * NB + p) * 128 + kl * 8) : signs + (blk * 128 + kl * 8);
      reinterpret_cast<v4u*>(dst)[0] = v4u{tw[0], tw[1], tw[2], tw[3]};
      reinterpret_cast<v4u*>(dst)[1] = v4u{tw[4], tw[5], tw[6], tw[7]};
    }
  }
}

// Paged append into a blocked cache: one thread per (new record, bit plane,
// coordinate), plus one per record for ν and γ.  The record's bit is merged
// into its block word with an atomic AND (clear) and OR (set): other threads
// merge other rows' bits into the same words at the same time.  Positions
// outside the page table or the pool are not written (as the row layout).
__global__ __launch_bounds__(256) void vblock_append_kernel(tq_packed_t src, int nb, int qjl, int n_kv_heads,
                                                            int n_new, int64_t n_rec,
                                                            const int32_t* __restrict__ ctx_lens,
                                                            const int32_t* __restrict__ page_table, int max_pages,
                                                            int page_size, int n_pages, tq_packed_t dst) {
  const int planes = nb + qjl;
  const int per = planes * 128 + 1;  // bits, then ν and γ
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= n_rec * per) return;
  const int64_t i = e / per;
  const int w = static_cast<int>(e % per);
  const int t = static_cast<int>(i % n_new);
  const int kh = static_cast<int>((i / n_new) % n_kv_heads);
  const int b = static_cast<int>(i / (static_cast<int64_t>(n_new) * n_kv_heads));
  const int64_t pos = static_cast<int64_t>(ctx_lens[b]) + t;
  if (pos < 0 || pos / page_size >= max_pages) return;
  const int page = page_table[static_cast<int64_t>(b) * max_pages + pos / page_size];
  if (page < 0 || page >= n_pages) return;
  const int64_t row = (static_cast<int64_t>(page) * n_kv_heads + kh) * page_size + pos % page_size;
  if (w == planes * 128) {
    dst.norm[row] = src.norm[i];
    if (qjl) dst.rnorm[row] = src.rnorm[i];
    return;
  }
  const int p = w >> 7, j = w & 127;
  const uint32_t word = p < nb ? src.codes[i * nb * 4 + p * 4 + (j >> 5)] : src.signs[i * 4 + (j >> 5)];
  const uint32_t bit = (word >> (j & 31)) & 1u;
  const int tau = static_cast<int>(row & 31);
  const uint32_t m = 1u << (4 * (tau & 7) + (tau >> 3));
  const int64_t blk = row >> 5;
  uint32_t* at = p < nb ? dst.codes + (blk * nb + p) * 128 + (j & 15) * 8 + (j >> 4)
                        : dst.signs + blk * 128 + (j & 15) * 8 + (j >> 4);
  atomicAnd(at, ~m);
  if (bit) atomicOr(at, m);
}

}  // namespace

hipError_t launch_vblock_from_rows(const tq_codec_s* c, tq_packed_t rows, int64_t n, tq_packed_t out, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(ceil_div(n, 512)));
  const int nb = c->prm.b;
  auto go = [&]<int NB>() -> hipError_t {
    if (c->qjl)
      hipLaunchKernelGGL((vblock_from_rows_kernel<NB, true>), grid, dim3(256), 0, s, rows, n, out.codes, out.signs);
    else
      hipLaunchKernelGGL((vblock_from_rows_kernel<NB, false>), grid, dim3(256), 0, s, rows, n, out.codes,
                         static_cast<uint32_t*>(nullptr));
    return hipGetLastError();
  };
  switch (nb) {
    case 1: return go.template operator()<1>();
    case 2: return go.template operator()<2>();
    case 3: return go.template operator()<3>();
  }
  return hipErrorInvalidValue;
}

hipError_t launch_vblock_append(const tq_codec_s* c, tq_packed_t rows, int n_kv_heads, int n_new, int64_t n_rec,
                                const int32_t* ctx_lens, const int32_t* page_table, int max_pages, int page_size,
                                int n_pages, tq_packed_t cache, hipStream_t s) {
  const int nb = c->prm.b, qjl = c->qjl ? 1 : 0;
  const int64_t total = n_rec * ((nb + qjl) * 128 + 1);
  hipLaunchKernelGGL(vblock_append_kernel, dim3(static_cast<unsigned>(ceil_div(total, 256))), dim3(256), 0, s, rows,
                     nb, qjl, n_kv_heads, n_new, n_rec, ctx_lens, page_table, max_pages, page_size, n_pages, cache);
  return hipGetLastError();
}

// ---------------------------------------------------------------- encode for any layout
namespace {
size_t align256v(size_t x) { return (x + 255) / 256 * 256; }
}  // namespace

size_t encode_ws_bytes(const tq_codec_s* c, int64_t n) {
  if (!c->vblock) return encode_rows_ws_bytes(c, n);
  // row records staged in the workspace (codes, signs), then the row encoder's own
  return align256v(static_cast<size_t>(n) * c->prm.code_words * 4) +
         align256v(static_cast<size_t>(n) * c->prm.sign_words * 4) + encode_rows_ws_bytes(c, n);
}

hipError_t launch_encode(const tq_codec_s* c, const void* x, tq_dtype_t dt, int64_t n, tq_packed_t out, void* ws,
                         hipStream_t s) {
  if (!c->vblock) return launch_encode_rows(c, x, dt, n, out, static_cast<float*>(ws), s);
  uint8_t* p = static_cast<uint8_t*>(ws);
  tq_packed_t st;
  st.codes = reinterpret_cast<uint32_t*>(p);
  p += align256v(static_cast<size_t>(n) * c->prm.code_words * 4);
  st.signs = c->qjl ? reinterpret_cast<uint32_t*>(p) : nullptr;
  p += align256v(static_cast<size_t>(n) * c->prm.sign_words * 4);
  st.norm = out.norm;    // ν and γ are per row in both layouts
  st.rnorm = out.rnorm;
  hipError_t e = launch_encode_rows(c, x, dt, n, st, reinterpret_cast<float*>(p), s);
  if (e != hipSuccess) return e;
  return launch_vblock_from_rows(c, st, n, out, s);
}

}  // namespace tq

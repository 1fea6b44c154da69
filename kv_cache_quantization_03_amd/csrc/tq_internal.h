// Internal declarations shared by the host codec builder, the C-ABI layer and
// the kernel launchers.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/tq.h"

namespace tq {

// Thread-local error message (tq_last_error).
void set_error(const std::string& msg);
void clear_error();

// Host tables of one codec (fp64 fit, fp32 canonical where stated).
struct HostTables {
  int d = 0, bits = 0, b = 0, m = 0;
  uint64_t seed = 0;
  std::vector<float> D;          // [d] ±1
  std::vector<float> S;          // [m*d] row-major, canonical fp32
  std::vector<double> centroids; // [2^b] ascending
  std::vector<double> bounds;    // [2^b-1]
  int iterations = 0;
  // recursive polar first stage (when polar): per level (1..log2 d) the angle
  // codebook, ascending, and its boundaries
  bool polar = false;
  std::vector<std::vector<double>> pcent, pbound;
  std::vector<int> piters;
};

// Builds every table on the host.  Returns TQ_SUCCESS or an error status (and
// sets the thread-local message).
tq_status_t build_host_tables(int d, int bits, int m, uint64_t seed, HostTables* out);
// The same plus the per-level angle codebooks of the recursive polar stage.
tq_status_t build_polar_tables(int d, int bits, int m, uint64_t seed, HostTables* out);
// First stage only (MSE-only value codec): b = bits Lloyd-Max bits, m = 0, no S.
tq_status_t build_mse_tables(int d, int bits, uint64_t seed, HostTables* out);
bool supported_dim(int d);

// Device constant block of one codec: everything a kernel needs besides S.
// Laid out for a single struct-by-value kernel argument.
struct DevParams {
  float cent[8];       // fp32 centroids (2^b <= 8)
  float bound[8];      // fp32 boundaries (2^b - 1 used)
  float plane_coef[4]; // MSE plane weights of the bit-plane expansion of c[idx]
  float plane_bias;    // constant term of that expansion
  float qjl_kappa;     // sqrt(pi/2)/m
  float inv_sqrt_d;    // 1/sqrt(d)
  float mrow_bound;    // max_i ||row i of M = S R||_2 (fp32 M, rounded up): |(M q)_i| <= mrow_bound ||q||
  int d, b, m, code_words, sign_words, n_planes;
};

// Tables of the recursive polar stage for the kernels: per level l (index
// l-1), cos and sin of every centroid (fp32) and the boundaries (unused +inf);
// bcs: the boundary tests of the encode, (cos β, sin β) at level 1 and
// (cos² β, sin² β) above (from the fp64 boundaries).
constexpr int kPolarMaxLevels = 8;
struct PolarParams {
  float cosc[kPolarMaxLevels][16];
  float sinc[kPolarMaxLevels][16];
  float bound[kPolarMaxLevels][16];
  float2 bcs[kPolarMaxLevels][16];
  int levels, nl;  // log2 d, 2^b
};

// A paged cache (see tq_decode_attn_paged): page_table[b][i] holds positions
// [i*page_size, (i+1)*page_size) of sequence b; page p, KV head kh, slot s is
// row (p * n_kv_heads + kh) * page_size + s.  ctx_lens[b]: positions in use.
struct PageMap {
  const int32_t* table;
  const int32_t* ctx_lens;
  int max_pages, page_size;
};

}  // namespace tq

namespace tq {
// Paley type-I Hadamard matrix of order 12 (q = 11): H = I + S with
// S = [[0, 1ᵀ], [-1, Q]], Q_ab = χ(b - a), χ the quadratic character mod 11.
__host__ __device__ constexpr int legendre11(int a) {
  a = ((a % 11) + 11) % 11;
  if (a == 0) return 0;
  int r = 1;
  for (int k = 0; k < 5; ++k) r = (r * a) % 11;  // Euler's criterion: a^5 mod 11
  return r == 1 ? 1 : -1;
}
__host__ __device__ constexpr int paley12(int a, int b) {
  return a == b ? 1 : (a == 0 ? 1 : (b == 0 ? -1 : legendre11(b - a)));
}
}  // namespace tq

struct tq_codec_s {
  tq::HostTables host;
  tq::DevParams prm;
  int device = 0;
  // device tables (one allocation)
  void* dev_block = nullptr;
  float* dS = nullptr;   // [m][d] row-major
  float* dMt = nullptr;  // [d][m]: (S R)ᵀ, so that p = S R q needs no rotated query
  float* dD = nullptr;   // [d] ±1
  _Float16* dS16 = nullptr;  // [2][m][d]: S = hi + lo in fp16 (m = d, d a multiple of 128; else nullptr)
  bool polar = false;        // first stage: recursive polar angles instead of per-coordinate codes
  bool qjl = true;           // false: MSE-only codec (m = 0: records hold codes and ν, no signs, no γ)
  bool vblock = false;       // codes and signs stored in 32-row blocks of transposed words (a value-cache layout)
  tq::PolarParams pol{};
};

namespace tq {

// Static device scratch of tq_decode_attn_no_alloc (scratch.hip): its size,
// and its device address on the current device (looked up on the first call
// per device; no allocation).
constexpr size_t kNoAllocScratchBytes = TQ_NO_ALLOC_SCRATCH_BYTES;
hipError_t no_alloc_scratch(void** out);

// ---- kernel launchers (kernels_*.hip).  All arguments were validated. ----
// Encode: rotate + quantize (codes, norm, rnorm) and write the residual r (fp32
// [n][d]) into ws_r; then the QJL projection writes the sign words.
hipError_t launch_encode(const tq_codec_s* c, const void* x, tq_dtype_t dt, int64_t n,
                         tq_packed_t out, void* ws, hipStream_t s);
size_t encode_ws_bytes(const tq_codec_s* c, int64_t n);
// The same in row records whatever the codec's layout (the blocked layout's
// first step; the paged append's staging).
hipError_t launch_encode_rows(const tq_codec_s* c, const void* x, tq_dtype_t dt, int64_t n, tq_packed_t out,
                              float* ws_r, hipStream_t s);
size_t encode_rows_ws_bytes(const tq_codec_s* c, int64_t n);
// Blocked value layout (kernels_vblock.hip): row records -> 32-row blocks; the
// paged append's bit merge.
hipError_t launch_vblock_from_rows(const tq_codec_s* c, tq_packed_t rows, int64_t n, tq_packed_t out,
                                   hipStream_t s);
hipError_t launch_vblock_append(const tq_codec_s* c, tq_packed_t rows, int n_kv_heads, int n_new, int64_t n_rec,
                                const int32_t* ctx_lens, const int32_t* page_table, int max_pages, int page_size,
                                int n_pages, tq_packed_t cache, hipStream_t s);

// Query prep: q' = R q and p = S q' for n query vectors (fp32 outputs [n][d],[n][m]).
hipError_t launch_qprep(const tq_codec_s* c, const void* q, tq_dtype_t dt, int64_t n, float* qrot,
                        float* proj, hipStream_t s);

// Logits for the [batch][n_q_heads][n_queries][ctx] layout (prepped queries
// in ws).
size_t logits_ws_bytes(const tq_codec_s* c, int batch, int n_q_heads, int n_kv_heads, int n_queries);
bool logits_paged_supported(const tq_codec_s* c);
size_t logits_paged_ws_bytes(const tq_codec_s* c, int batch, int n_q_heads, int n_kv_heads, int n_queries);
hipError_t launch_logits_paged(const tq_codec_s* c, const void* q, tq_dtype_t dt, int batch, int n_q_heads,
                               int n_kv_heads, int n_queries, tq_packed_t k, int64_t max_ctx, const PageMap& pm,
                               float* logits, void* ws, hipStream_t s);
hipError_t launch_logits(const tq_codec_s* c, const void* q, tq_dtype_t dt, int batch, int n_q_heads,
                         int n_kv_heads, int n_queries, tq_packed_t k, int64_t ctx, float* logits,
                         void* ws, hipStream_t s);
hipError_t launch_logits_prep(const tq_codec_s* c, const void* q, tq_dtype_t dt, int batch, int n_q_heads,
                              int n_kv_heads, int n_queries, void* ws, hipStream_t s);
hipError_t launch_logits_prepped(const tq_codec_s* c, const void* ws, int batch, int n_q_heads, int n_kv_heads,
                                 int n_queries, tq_packed_t k, int64_t ctx, float* logits, hipStream_t s);
// The polar scorer on prepped queries; pm set: a paged cache (ctx: the
// largest context and the logits row stride).
hipError_t launch_logits_polar(const tq_codec_s* c, const void* ws, int batch, int n_q_heads, int n_kv_heads,
                               int n_queries, tq_packed_t k, int64_t ctx, float* logits, hipStream_t s,
                               const PageMap* pm = nullptr);

bool decode_supported(const tq_codec_s* cv, int n_q_heads, int n_kv_heads, int64_t ctx, const char** why);
size_t decode_ws_bytes(const tq_codec_s* ck, const tq_codec_s* cv, int batch, int n_q_heads,
                       int n_kv_heads, int64_t ctx);
int decode_chunk(int n_q_heads, int n_kv_heads);
// pm: nullptr for a contiguous cache [batch][kv_head][ctx]; else a paged
// cache read through pm, ctx being the largest context (grid size).
hipError_t launch_decode(const tq_codec_s* ck, const tq_codec_s* cv, const void* q, tq_dtype_t q_dt,
                         int batch, int n_q_heads, int n_kv_heads, tq_packed_t k, tq_packed_t v,
                         int64_t ctx, float scale, bool sparse_v, float v_gate, const PageMap* pm, void* out,
                         tq_dtype_t out_dt, void* ws, hipStream_t s);
bool decode_paged_supported(const tq_codec_s* ck, const tq_codec_s* cv, int n_q_heads, int n_kv_heads);
// Either codec polar (the logits by the key scorer, then V from them): d = m =
// 128 or 256, the same for K and V, and V in row records.
bool decode_polar_shape_ok(const tq_codec_s* ck, const tq_codec_s* cv);

size_t append_paged_ws_bytes(const tq_codec_s* c, int64_t n_rec);
hipError_t launch_append_paged(const tq_codec_s* c, const void* x, tq_dtype_t dt, int batch, int n_kv_heads,
                               int n_new, const int32_t* ctx_lens, const int32_t* page_table, int max_pages,
                               int page_size, int n_pages, tq_packed_t cache, void* ws, hipStream_t s);

size_t search_ws_bytes(const tq_codec_s* c, int64_t n_db, int n_queries, int topk);
hipError_t launch_search(const tq_codec_s* c, tq_packed_t db, int64_t n_db, const float* queries,
                         int n_queries, int topk, int64_t* out_idx, float* out_score, void* ws,
                         hipStream_t s);

}  // namespace tq

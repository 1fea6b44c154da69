/*
 * tq.h — TurboQuant KV-cache and vector codec for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only.  Every compute call is asynchronous on
 * the caller's HIP stream.  Every device pointer is owned by the caller: the
 * library never allocates or frees it.  tq_codec_create is the one synchronous
 * call: it builds the codec tables on the host and uploads them.
 *
 * Method (pages cited by title and section):
 *   「谷歌 TurboQuant 深度拆解：LLM 内存压缩 6 倍、推理加速 8 倍、零精度损失，
 *    它是怎么做到的？」 第二部分, the two-stage method:
 *     (1) a random rotation, after which each coordinate follows a known law,
 *         so an optimal scalar (Lloyd-Max) quantizer needs no per-block scale
 *         or zero-point;
 *     (2) QJL: the residual is projected with a Gaussian JL matrix and only
 *         one sign bit is kept per projected coordinate; a full-precision
 *         query scores the compressed key with an unbiased estimator.
 *   Same page, 第六部分: the coordinate density
 *     f(x) = Γ(d/2)/(√π Γ((d-1)/2)) (1-x²)^((d-3)/2), and the estimator is
 *     unbiased with variance falling as 1/m.
 *   「TurboQuant+ 深度解析：当前 Google 工程师决定单挑大厂」 第二部分: the
 *     rotation is a random-sign Walsh–Hadamard transform.
 *   「TurboQuant 学习路径：论文 → 技术 → 数学」 二.2: FJLT y = P·H·D·x and
 *     Gaussian JL; 三.1: Hadamard recursion H_n = H_1 ⊗ H_{n-1}.
 *
 * Codec parameters: head_dim d, total bits B (2, 3 or 4) = b Lloyd-Max bits
 * (b = B-1) + 1 QJL bit per projected coordinate, QJL dimension m = d, seed.
 *   R = H diag(D)/√d.  H is Sylvester natural order for d = 2^k; for d = 1536
 *     it is H12 ⊗ H128, with H12 the Paley type-I matrix.  D = ±1 from
 *     SplitMix64(seed ^ 1).
 *   S = m x d i.i.d. N(0,1): SplitMix64(seed ^ 2) fed to Box–Muller, then
 *     rounded to fp32.
 *   c, t = the Lloyd-Max centroids and boundaries of f (fp64 fit, fp32 on the
 *     device).
 *
 * Encode, per vector x:
 *   ν = ||x||, y = R x/ν, idx_j = #{k : t_k < y_j}, r = y - c[idx], γ = ||r||,
 *   sign bit i = [(S r)_i >= 0].
 * Score against a query q:
 *   q' = R q, p = S q',
 *   ℓ = ν (Σ_j q'_j c[idx_j] + √(π/2)/m · γ · Σ_i p_i (2 bit_i - 1)).
 *
 * Packed record layout (tq_packed_t).  Each array has one row per vector, in
 * the caller's row order (for a KV cache: [batch][kv_head][token]):
 *   codes[n][b*d/32] u32  bit-planes.  Word p*(d/32) + j/32, bit j%32 holds
 *                         bit p of idx_j.
 *   signs[n][m/32]   u32  word i/32, bit i%32 holds sign bit i.
 *   norm[n]  f32          ν = ||x||.
 *   rnorm[n] f32          γ = ||r|| of the unit-vector residual.
 * Bytes per vector: d·B/8 + 8 (3-bit, d=128: 48 + 8 = 56 B, vs 256 B of fp16).
 *
 * Alignment.  The kernels move record words and input vectors with 16-byte
 * loads and stores, so codes, signs and every input vector array (q, k, v, x,
 * search queries) must be 16-byte aligned; ν, γ, logits and fp32 outputs
 * 4-byte aligned; workspaces 16-byte aligned.  Any other pointer gives
 * TQ_ERROR_MISALIGNED.  A row offset into a cache keeps 16-byte alignment
 * whenever a row's code and sign words are multiples of 16 bytes (every
 * head_dim >= 128); for head_dim 64 only even row offsets keep it.  The
 * alignment of the array arguments is checked first, before the codec
 * handle.
 *
 * Errors.  Every call returns a tq_status_t and never throws.  Arguments are
 * validated on the host before any launch, so an invalid call has no side
 * effect.  tq_last_error() returns a thread-local message for the last failing
 * call on this thread.  Launch failures map to TQ_ERROR_HIP.
 */
#ifndef TQ_H_
#define TQ_H_

/* Environment switches (read at each call; for comparisons and tests, not
 * needed in normal use).  Each forces the general VALU kernel of one step, or
 * the two-kernel form, instead of the matrix-core or fused one:
 *   TQ_LOGITS_KERNEL=valu   logits (any head_dim)
 *   TQ_LOGITS_FUSED=0       logits: query-prep launch + logits launch
 *   TQ_DECODE_KERNEL=valu   decode attention (contiguous caches only)
 *   TQ_ENCODE_KERNEL=split  encode: rotate/quantize, then the projection
 *   TQ_SPROJ_KERNEL=valu    encode's QJL projection on the fp32 VALU
 *   TQ_SEARCH_KERNEL=valu   search scores
 *   TQ_LOG=1                one line per call on stderr. */

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_ABI_VERSION 2

typedef struct tq_codec_s* tq_codec_t; /* opaque; immutable after create, usable from any stream */

typedef enum {
  TQ_SUCCESS = 0,
  TQ_ERROR_INVALID_VALUE = 1,        /* NULL handle/pointer, negative size, bad enum, bad shape */
  TQ_ERROR_NOT_SUPPORTED = 2,        /* a valid request the library does not implement */
  TQ_ERROR_MISALIGNED = 3,           /* a pointer breaks the alignment stated below */
  TQ_ERROR_WORKSPACE_TOO_SMALL = 4,  /* ws_bytes < the matching *_workspace() size */
  TQ_ERROR_OUT_OF_MEMORY = 5,        /* host or device allocation inside tq_codec_create failed */
  TQ_ERROR_HIP = 6                   /* a HIP runtime call or kernel launch failed */
} tq_status_t;

typedef enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 } tq_dtype_t;

/* Device pointers to one packed cache or database; all arrays have n rows.
 * Records of an MSE-only codec (tq_codec_create_mse) have no signs and no γ:
 * signs and rnorm are ignored and may be NULL. */
typedef struct {
  uint32_t* codes; /* [n][code_words], 16-byte aligned */
  uint32_t* signs; /* [n][sign_words], 16-byte aligned */
  float* norm;     /* [n], 4-byte aligned */
  float* rnorm;    /* [n], 4-byte aligned */
} tq_packed_t;

typedef struct {
  int32_t head_dim;     /* d */
  int32_t bits;         /* B = b + 1 (an MSE-only codec: B = b) */
  int32_t mse_bits;     /* b */
  int32_t qjl_dim;      /* m (0: MSE-only codec, no QJL stage) */
  int32_t code_words;   /* b*d/32 */
  int32_t sign_words;   /* m/32 */
  int32_t record_bytes; /* 4*(code_words+sign_words) + 8 */
  int32_t lloyd_max_iterations;
  uint64_t seed;
  double centroids[16]; /* 2^b entries, ascending, fp64 */
  double bounds[15];    /* 2^b - 1 entries, midpoints of the centroids */
  int32_t stage1;       /* 0: per-coordinate Lloyd-Max codes; 1: recursive polar angles */
  int32_t layout;       /* 0: row records; 1: 32-row blocks (tq_codec_create_vblock) */
} tq_codec_info_t;

/* ---------------------------------------------------------------- status */
const char* tq_status_string(tq_status_t s);
/* Thread-local message for the last failing call on this thread ("" if none). */
const char* tq_last_error(void);
int32_t tq_abi_version(void);

/* ---------------------------------------------------------------- codec
 * Supported: head_dim in {64, 128, 256, 512, 1024, 1536}; bits in {2, 3, 4};
 * qjl_dim 0 (meaning d) or d.  Other values -> TQ_ERROR_NOT_SUPPORTED.
 * The tables depend only on (head_dim, bits, qjl_dim, seed): the codec is
 * data-oblivious (深度拆解 第二部分: no training, tuning or calibration).
 */

/* Host only, no GPU needed: writes the codec tables into caller-owned host
 * buffers.  Any output pointer may be NULL.
 * D_out[d] (±1), S_out[m*d] (row-major fp32), centroids[2^b], bounds[2^b-1],
 * iterations = number of Lloyd-Max iterations. */
tq_status_t tq_codec_build_host(int32_t head_dim, int32_t bits, int32_t qjl_dim, uint64_t seed,
                                float* D_out, float* S_out, double* centroids, double* bounds,
                                int32_t* iterations);

/* Builds the tables on the host and uploads them to the current HIP device
 * (synchronous).  *out receives the handle.  The handle stays bound to that
 * device. */
tq_status_t tq_codec_create(int32_t head_dim, int32_t bits, int32_t qjl_dim, uint64_t seed,
                            tq_codec_t* out);
/* A codec whose first stage is PolarQuant's recursive polar form
 * (深度拆解 第二部分 PolarQuant; vocus 第一階段: 3- or 4-bit angles): after
 * the same rotation y = R x/ν, level 1 pairs the coordinates (y_2i, y_2i+1)
 * into (radius, angle), each further level pairs the radii of the level
 * below, down to one radius (‖y‖ = 1, not stored).  Every angle gets b =
 * bits-1 bits: level 1's angles (in [0, 2π)) the uniform quantizer of the
 * circle, level l > 1's (in [0, π/2], sin²θ ~ Beta(n/2, n/2), n = 2^(l-1))
 * the Lloyd-Max quantizer of that law.  Codes: level l's d/2^l angles in
 * slots [d - d/2^(l-1), d - d/2^l) of the usual bit-plane record, slot d-1
 * unused (0); ŷ is rebuilt from radius 1 with cos and sin of the centroids
 * (fp32), and the residual y - ŷ takes the same QJL stage, so the record size
 * and the score ν(⟨q', ŷ⟩ + √(π/2)/m γ ⟨p, τ⟩) keep their form.
 * head_dim 64, 128 or 256 (log2 head_dim levels); bits 2, 3 or 4.  Such
 * codecs are accepted by tq_encode_kv, tq_encode_append_paged,
 * tq_attn_logits, its split form and tq_attn_logits_paged, by tq_search_topk
 * (the polar score against every database record), and, at head_dim 128 or
 * 256, as either codec (ck, cv or both) of tq_decode_attn,
 * tq_decode_attn_no_alloc, tq_decode_attn_sparse_v and tq_decode_attn_paged
 * (深度拆解 第二部分 第三步: the whole KV cache in polar form;
 * v̂ = ν Rᵀ (ŷ + √(π/2)/m γ Sᵀ τ)). */
tq_status_t tq_codec_create_polar(int32_t head_dim, int32_t bits, int32_t qjl_dim, uint64_t seed,
                                  tq_codec_t* out);
/* An MSE-only value codec: the same rotation and per-coordinate Lloyd-Max
 * stage with all `bits` (2 or 3) given to the code, and no QJL stage
 * (TurboQuant+ 深度解析 第五部分: the value cache tolerates coarser
 * compression than the key cache, which routes attention).  A record is the
 * codes (d*bits/8 bytes) and ν; the value reconstruction is v̂ = ν Rᵀ c[idx]
 * (least mean squared error; biased for inner products).  Accepted by
 * tq_encode_kv, tq_encode_append_paged and as the V codec (cv) of the decode
 * attention calls; tq_attn_logits, its split form, tq_search_topk and the K
 * codec role return TQ_ERROR_NOT_SUPPORTED.  head_dim as tq_codec_create;
 * tq_codec_info reports qjl_dim = 0 and sign_words = 0. */
tq_status_t tq_codec_create_mse(int32_t head_dim, int32_t bits, uint64_t seed, tq_codec_t* out);
/* A value codec whose records are stored in blocks of 32 rows (head_dim 128;
 * bits 2, 3 or 4 as tq_codec_create, or with mse_only != 0 the MSE-only codec
 * of tq_codec_create_mse).  Decode attention accumulates the attention-weighted
 * values as a contraction over keys (TurboQuant+ 深度解析 第五部分 compresses V
 * like K; 第六部分: V dequantization is a large share of long-context decode),
 * which needs each coordinate's bits across 32 consecutive rows; this layout
 * stores them so:
 *   block B = rows 32B..32B+31, b = mse_bits planes of codes (bit plane p of
 *   every code index), then the sign plane.  For coordinate j = 16c + n
 *   (n < 16, c < 8):
 *     codes[(B*b + p)*128 + 8n + c]   (words, counting from the array start)
 *     signs[B*128 + 8n + c]
 *   bit 4i + r of such a word is the bit of row 32B + 8r + i.
 *   norm[row] and rnorm[row] stay one float per row.
 * The arrays have the sizes of row records (codes [n][code_words], ...), and
 * rows 32B.. of the row layout and block B cover the same words, so offsets
 * by a multiple of 32 rows work as for row records.  tq_encode_kv writes whole
 * blocks (n_vec a multiple of 32, else TQ_ERROR_INVALID_VALUE), so an append
 * through it starts at a multiple of 32 rows; tq_encode_append_paged merges
 * single rows into their blocks (page_size a multiple of 32; two calls that
 * write rows of one block may not run concurrently).  Accepted by tq_encode_kv, tq_encode_append_paged and as
 * the V codec (cv) of the decode attention calls (the contiguous ones need
 * ctx_len % 32 == 0); every other call returns TQ_ERROR_NOT_SUPPORTED.
 * Decode results equal those with the row-record codec of the same head_dim,
 * bits and seed (the codec tables are the same), bit for bit. */
tq_status_t tq_codec_create_vblock(int32_t head_dim, int32_t bits, int32_t mse_only, uint64_t seed,
                                   tq_codec_t* out);
/* Host only (no GPU needed): level l's (1..log2 head_dim) angle codebook of
 * the polar stage for head_dim 64, 128 or 256 and the given bits:
 * centroids[2^b] and bounds[2^b - 1], fp64, ascending, and the Lloyd-Max
 * iterations (0 for the uniform level 1).  Level l's law depends on l only,
 * not on head_dim.  Any output pointer may be NULL. */
tq_status_t tq_polar_book_host(int32_t head_dim, int32_t bits, int32_t level, double* centroids,
                               double* bounds, int32_t* iterations);
/* The caller guarantees that no work using c is still in flight. */
tq_status_t tq_codec_destroy(tq_codec_t c);
tq_status_t tq_codec_info(tq_codec_t c, tq_codec_info_t* info);

/* ---------------------------------------------------------------- encode
 * Compresses n_vec rows of k (and of v if v != NULL) with codec c: the
 * two-stage encode of 深度拆解 第二部分 (random rotation, then the optimal
 * scalar code of each rotated coordinate with no per-block constants, then
 * the QJL sign bits of the projected residual), applied to the KV cache that
 * 第一部分 (KV 缓存是什么) describes: every past token's K and V.
 *   k, v : device [n_vec][d] in dtype dt, 16-byte aligned.
 *   k_out, v_out : device packed arrays with n_vec rows.  To append to an
 *          existing cache, offset each pointer by the first row to write.
 *   ws   : device workspace of at least tq_encode_workspace(c, n_vec) bytes,
 *          16-byte aligned (may be NULL when that size is 0).
 * n_vec = 0 is a valid no-op.  To give K and V different codecs (for example
 * 4-bit K and 3-bit V), call once per codec with v = NULL.
 */
size_t tq_encode_workspace(tq_codec_t c, int64_t n_vec);
tq_status_t tq_encode_kv(tq_codec_t c, const void* k, const void* v, tq_dtype_t dt, int64_t n_vec,
                         tq_packed_t k_out, tq_packed_t v_out, void* ws, size_t ws_bytes,
                         void* stream);

/* ---------------------------------------------------------------- logits
 * Unbiased attention logits of every query against every compressed key
 * (深度拆解 第二部分: full-precision query against the compressed key;
 * 第三部分 推理速度: attention logits are bound by memory bandwidth).
 *   q      : device [batch][n_queries][n_q_heads][d], dtype q_dt.
 *   k      : packed rows [batch][n_kv_heads][ctx_len].
 *   logits : device fp32 [batch][n_q_heads][n_queries][ctx_len].  These are
 *            raw <q,k> estimates: no 1/sqrt(d) scaling is applied.
 * GQA: query head h reads KV head h / (n_q_heads / n_kv_heads); n_q_heads
 * must be a multiple of n_kv_heads.  ctx_len = 0 is a valid no-op; ctx_len
 * above 2^31 - 2^16 returns TQ_ERROR_NOT_SUPPORTED.
 * Workspace: tq_attn_logits_workspace(...) bytes, 16-byte aligned.
 */
size_t tq_attn_logits_workspace(tq_codec_t c, int32_t batch, int32_t n_q_heads,
                                int32_t n_kv_heads, int32_t n_queries);
tq_status_t tq_attn_logits(tq_codec_t c, const void* q, tq_dtype_t q_dt, int32_t batch,
                           int32_t n_q_heads, int32_t n_kv_heads, int32_t n_queries,
                           tq_packed_t k, int64_t ctx_len, float* logits, void* ws,
                           size_t ws_bytes, void* stream);

/* Split form of tq_attn_logits for callers that score one set of queries
 * against several caches, or that time the two stages apart.
 * tq_attn_query_prep writes the prepared queries (q' = R q, p = S q' and
 * their scoring operands) into `prep`, a device buffer of at least
 * tq_attn_logits_workspace(...) bytes, 16-byte aligned.
 * tq_attn_logits_prepped reads `prep` and writes the logits exactly as
 * tq_attn_logits does.  Both calls must use the same shape arguments. */
tq_status_t tq_attn_query_prep(tq_codec_t c, const void* q, tq_dtype_t q_dt, int32_t batch,
                               int32_t n_q_heads, int32_t n_kv_heads, int32_t n_queries, void* prep,
                               size_t prep_bytes, void* stream);
tq_status_t tq_attn_logits_prepped(tq_codec_t c, const void* prep, size_t prep_bytes, int32_t batch,
                                   int32_t n_q_heads, int32_t n_kv_heads, int32_t n_queries,
                                   tq_packed_t k, int64_t ctx_len, float* logits, void* stream);

/* ---------------------------------------------------------------- decode attention
 * One decode step of attention over a compressed K/V cache:
 *   out[b][h] = Σ_t softmax_t(softmax_scale · ℓ_t) · v̂_t
 * where v̂ = ν Rᵀ (c[idx] + √(π/2)/m · γ · Sᵀ τ) is the value's unbiased
 * reconstruction.  K and V use the same codec layout
 * (TurboQuant+ 深度解析 第五部分: K and V are compressed the same way).  V is
 * accumulated in the codec domain and mapped back once per head.
 *   ck, cv : codecs of K and V (they may be the same handle; their bits may
 *            differ; head_dim must match).  cv may be an MSE-only codec
 *            (tq_codec_create_mse): then v̂ = ν Rᵀ c[idx] and v.signs,
 *            v.rnorm are not read.  Either may be a polar codec
 *            (tq_codec_create_polar; then both have head_dim 128 or 256 and
 *            cv is not a codec in 32-row blocks): the logits then come from the
 *            key codec's scorer and are held in the workspace, and a polar
 *            value's ŷ is rebuilt per position from its angle codes.
 *   q      : device [batch][n_q_heads][d], dtype q_dt.
 *   k, v   : packed rows [batch][n_kv_heads][ctx_len].
 *   out    : device [batch][n_q_heads][d], dtype out_dt (TQ_F32 or TQ_BF16,
 *            the latter rounded to nearest even).
 *   ctx_len >= 1.  Workspace: tq_decode_attn_workspace(...) bytes.
 */
size_t tq_decode_attn_workspace(tq_codec_t ck, tq_codec_t cv, int32_t batch, int32_t n_q_heads,
                                int32_t n_kv_heads, int64_t ctx_len);
tq_status_t tq_decode_attn(tq_codec_t ck, tq_codec_t cv, const void* q, tq_dtype_t q_dt,
                           int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, tq_packed_t k,
                           tq_packed_t v, int64_t ctx_len, float softmax_scale, void* out,
                           tq_dtype_t out_dt, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- decode attention, no allocation
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.
 * tq_decode_attn with the same arguments and results, minus the workspace:
 * its partial results live in a static device array of the library,
 * TQ_NO_ALLOC_SCRATCH_BYTES (16 MiB) per GPU, held from the library's load
 * until the process ends.  The call allocates and frees nothing.
 * A call that would need more than that (tq_decode_attn_workspace(...) >
 * TQ_NO_ALLOC_SCRATCH_BYTES; e.g. 32 query heads, 8 KV heads and more than
 * 4 million positions) returns TQ_ERROR_NOT_SUPPORTED before any launch.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (different streams, or threads)
 * race and must be serialised by the caller.  Nothing in the array needs to
 * start at zero (every value is written before it is read). */
#define TQ_NO_ALLOC_SCRATCH_BYTES ((size_t)16 << 20)
tq_status_t tq_decode_attn_no_alloc(tq_codec_t ck, tq_codec_t cv, const void* q, tq_dtype_t q_dt, int32_t batch,
                                    int32_t n_q_heads, int32_t n_kv_heads, tq_packed_t k, tq_packed_t v,
                                    int64_t ctx_len, float softmax_scale, void* out, tq_dtype_t out_dt,
                                    void* stream);

/* ---------------------------------------------------------------- Sparse V decode attention
 * tq_decode_attn with the value dequantization gated by the attention weights
 * (TurboQuant+ 深度解析, 第六部分 Sparse V Dequant: positions whose weight is
 * negligible, below about 1e-6, are not decompressed).
 * The context is processed in chunks of tq_decode_attn_chunk(n_q_heads,
 * n_kv_heads) consecutive positions.  For query head h and position t in
 * chunk c, with s = softmax_scale · ℓ, m_hc = max of s over the chunk and
 * l_hc = Σ_chunk exp(s - m_hc):
 *   the term of v̂_t is dropped for head h iff exp(s_ht - m_hc) < v_gate · l_hc.
 * This chunk-local weight is never below the final softmax weight, so every
 * dropped position has a final weight below v_gate and the output differs from
 * tq_decode_attn by at most v_gate · (dropped positions) · max ||v̂||_∞ per
 * element.  The softmax normaliser still sums every position.  A run of keys
 * dropped for every head of a KV group is not read from V at all.
 *   v_gate : in [0, 1); 0 drops nothing (the result then equals tq_decode_attn
 *            up to fp32 rounding order).
 * Other arguments, workspace and errors as tq_decode_attn; TQ_ERROR_INVALID_VALUE
 * for v_gate outside [0, 1) or NaN. */
tq_status_t tq_decode_attn_sparse_v(tq_codec_t ck, tq_codec_t cv, const void* q, tq_dtype_t q_dt,
                                    int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, tq_packed_t k,
                                    tq_packed_t v, int64_t ctx_len, float softmax_scale, float v_gate,
                                    void* out, tq_dtype_t out_dt, void* ws, size_t ws_bytes, void* stream);
/* Positions per chunk of the decode split (the Sparse V gate's normalisation
 * window): 1024 for at most 4 query heads per KV head, 512 for at most 8, 256
 * above.  0 for invalid head counts. */
int32_t tq_decode_attn_chunk(int32_t n_q_heads, int32_t n_kv_heads);

/* ---------------------------------------------------------------- paged cache
 * A KV cache that grows by one token per decode step (深度拆解 第一部分: the
 * cache keeps the K and V of every past token), stored in pages so that
 * sequences of different lengths share one pool.
 * Layout.  A cache is one set of packed arrays of n_pages * n_kv_heads *
 * page_size rows.  Page p holds, for KV head kh, the records of page_size
 * consecutive positions at rows (p * n_kv_heads + kh) * page_size + slot.
 * page_table (device int32 [batch][max_pages]): page_table[b][i] is the page
 * holding positions [i*page_size, (i+1)*page_size) of sequence b.
 * ctx_lens (device int32 [batch]): positions in use per sequence.
 *
 * tq_encode_append_paged encodes x (device [batch][n_kv_heads][n_new][d],
 * dtype dt) and writes token t of sequence b, KV head kh at position
 * ctx_lens[b] + t.  The records are exactly those tq_encode_kv writes for the
 * same rows.  A position whose page index is >= max_pages, or whose page id is
 * outside [0, n_pages), is not written.  ctx_lens is read, not updated: the
 * caller advances it (for example by n_new) before the next step.  Call once
 * per cache (K and V may use different codecs).  page_size >= 1 here; decode
 * needs a multiple of 128.  Workspace: tq_encode_append_paged_workspace(...)
 * bytes, 16-byte aligned.  batch = 0 or n_new = 0 is a no-op. */
size_t tq_encode_append_paged_workspace(tq_codec_t c, int32_t batch, int32_t n_kv_heads, int32_t n_new);
tq_status_t tq_encode_append_paged(tq_codec_t c, const void* x, tq_dtype_t dt, int32_t batch,
                                   int32_t n_kv_heads, int32_t n_new, const int32_t* ctx_lens,
                                   const int32_t* page_table, int32_t max_pages, int32_t page_size,
                                   int32_t n_pages, tq_packed_t cache, void* ws, size_t ws_bytes,
                                   void* stream);

/* tq_decode_attn over paged K and V caches (same layout and page table):
 * sequence b attends over its first ctx_lens[b] positions (clamped to
 * [0, max_ctx]); an empty context gives a zero output.  max_ctx (host) bounds
 * every ctx_lens[b] and sizes the grid and the workspace:
 * tq_decode_attn_paged_workspace(..., max_ctx) bytes.  v_gate > 0 applies the
 * Sparse V gate of tq_decode_attn_sparse_v (0: plain attention).  Shapes as
 * tq_decode_attn (head_dim = qjl_dim = 128 with at most 4 query heads per KV
 * head runs on the matrix cores, other shapes on the general kernel; a V
 * cache in 32-row blocks needs the former; polar codecs as tq_decode_attn
 * takes them: the key scorer's logits through the page table, then the
 * value kernel reading its rows through it), page_size a multiple of 128 and
 * 1 <= max_ctx <= max_pages * page_size (else TQ_ERROR_INVALID_VALUE).  Page
 * ids in the used part of the page table must be valid pages of the caches. */
size_t tq_decode_attn_paged_workspace(tq_codec_t ck, tq_codec_t cv, int32_t batch, int32_t n_q_heads,
                                      int32_t n_kv_heads, int64_t max_ctx);
tq_status_t tq_decode_attn_paged(tq_codec_t ck, tq_codec_t cv, const void* q, tq_dtype_t q_dt,
                                 int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, tq_packed_t k_cache,
                                 tq_packed_t v_cache, const int32_t* ctx_lens, const int32_t* page_table,
                                 int32_t max_pages, int32_t page_size, int64_t max_ctx, float softmax_scale,
                                 float v_gate, void* out, tq_dtype_t out_dt, void* ws, size_t ws_bytes,
                                 void* stream);

/* Logits over a paged cache (the layout of tq_decode_attn_paged: page p holds,
 * for KV head kh, rows (p * n_kv_heads + kh) * page_size + slot;
 * page_table[b][i] names the page of positions [i*page_size, (i+1)*page_size)
 * of sequence b).  q and the logits as tq_attn_logits with max_ctx as the
 * context: logits [batch][n_q_heads][n_queries][max_ctx] fp32; sequence b
 * scores its first min(ctx_lens[b], max_ctx) positions, and the logits of the
 * positions past them are not written.  Needs a polar codec (any head_dim it
 * takes) or a per-coordinate two-stage codec with head_dim 128 or 256,
 * page_size a positive multiple of 128 and
 * 1 <= max_ctx <= max_pages * page_size (else an error, no launch).
 * ctx_lens [batch] and page_table [batch][max_pages] are device int32 arrays
 * that must hold valid page ids for every position below ctx_lens[b].
 * Workspace: tq_attn_logits_paged_workspace(...) bytes, 16-byte aligned. */
size_t tq_attn_logits_paged_workspace(tq_codec_t c, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                      int32_t n_queries);
tq_status_t tq_attn_logits_paged(tq_codec_t c, const void* q, tq_dtype_t q_dt, int32_t batch, int32_t n_q_heads,
                                 int32_t n_kv_heads, int32_t n_queries, tq_packed_t k_cache,
                                 const int32_t* ctx_lens, const int32_t* page_table, int32_t max_pages,
                                 int32_t page_size, int64_t max_ctx, float* logits, void* ws, size_t ws_bytes,
                                 void* stream);

/* ---------------------------------------------------------------- search
 * Exhaustive inner-product search over a compressed database
 * (深度拆解 第三部分 向量搜索: the compressed vectors are the index; nothing
 * is trained).  Scores use the same estimator as tq_attn_logits.
 *   db        : packed rows [n_db].
 *   queries   : device fp32 [n_queries][d].
 *   out_idx   : device int64 [n_queries][topk], best first.  Ties go to the
 *               lower index.
 *   out_score : device fp32 [n_queries][topk].
 * 1 <= topk <= min(n_db, 1024).  Workspace: tq_search_workspace(...) bytes.
 */
size_t tq_search_workspace(tq_codec_t c, int64_t n_db, int32_t n_queries, int32_t topk);
tq_status_t tq_search_topk(tq_codec_t c, tq_packed_t db, int64_t n_db, const float* queries,
                           int32_t n_queries, int32_t topk, int64_t* out_idx, float* out_score,
                           void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- measurement
 * Not part of the method: the streaming ceiling the kernels' HBM rates are
 * compared with.  One launch reads read_bytes at src and writes write_bytes
 * (a fixed pattern) at dst, with the access pattern that keeps the most bytes
 * in flight: blocks of 256 threads, each thread issuing four independent
 * 16-byte non-temporal loads (or stores) before using any.  One XOR word per
 * 16 KiB read block goes to the device array sink[tq_diag_stream_sink_words(
 * read_bytes)], so the loads are not removed.  Both byte counts must be
 * multiples of 16 (else TQ_ERROR_INVALID_VALUE), src and dst 16-byte aligned
 * (else TQ_ERROR_MISALIGNED); either count may be 0. */
int64_t tq_diag_stream_sink_words(size_t read_bytes);
tq_status_t tq_diag_stream(const void* src, size_t read_bytes, void* dst, size_t write_bytes, uint32_t* sink,
                           void* stream);

#ifdef __cplusplus
}
#endif
#endif /* TQ_H_ */

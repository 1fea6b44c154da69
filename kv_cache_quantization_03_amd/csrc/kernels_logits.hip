// Attention logits over a compressed K cache: the unbiased estimator
//   ℓ = ν (Σ_j q'_j c[idx_j] + √(π/2)/m · γ · Σ_i p_i τ_i),
// q' = R q and p = S q' prepared once per query (「谷歌 TurboQuant 深度拆解」
// 第二部分: a full-precision query against the compressed key, unbiased).
//
// This file holds the general VALU kernel (one thread per key, any head_dim,
// any number of query vectors per KV head).  It is the reference kernel on the
// GPU and covers shapes the MFMA kernel does not.
#include "kernels_common.h"

namespace tq {

constexpr int kLogitsQC = 8;  // query vectors per block (grid.z splits the rest)

// Prepped query rows: qrot[row][d], proj[row][m] with row = (b*nq + qi)*Hq + h.
__global__ __launch_bounds__(256) void logits_valu_kernel(DevParams P, const float* __restrict__ qrot,
                                                          const float* __restrict__ proj, int Hq, int nq,
                                                          int G, int nkv, int64_t ctx, tq_packed_t k,
                                                          float* __restrict__ logits) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int bk = blockIdx.y;
  const int b = bk / nkv, kh = bk % nkv;
  const int nqv = nq * G;
  const int qv0 = blockIdx.z * kLogitsQC;
  const bool valid = t < ctx;
  const int64_t row = static_cast<int64_t>(bk) * ctx + (valid ? t : 0);
  const int d = P.d, m = P.m, W = d / 32, CW = P.code_words, SW = P.sign_words;
  const int L = 1 << P.b;

  int64_t qrow[kLogitsQC];
  int hq[kLogitsQC], qiq[kLogitsQC];
  bool qok[kLogitsQC];
#pragma unroll
  for (int c = 0; c < kLogitsQC; ++c) {
    const int qv = qv0 + c;
    qok[c] = qv < nqv;
    const int qi = qok[c] ? qv / G : 0, g = qok[c] ? qv % G : 0;
    hq[c] = kh * G + g;
    qiq[c] = qi;
    qrow[c] = (static_cast<int64_t>(b) * nq + qi) * Hq + hq[c];
  }
  float cent[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) cent[i] = P.cent[i];

  float mse[kLogitsQC] = {}, qjl[kLogitsQC] = {};
  const uint32_t* crow = k.codes + row * CW;
  for (int w = 0; w < W; ++w) {
    uint32_t pw[3] = {0, 0, 0};
    for (int p = 0; p < P.b; ++p) pw[p] = crow[p * W + w];
    for (int bit = 0; bit < 32; ++bit) {
      int idx = 0;
#pragma unroll
      for (int p = 0; p < 3; ++p) idx |= ((pw[p] >> bit) & 1u) << p;
      float cv = cent[0];
#pragma unroll
      for (int l = 1; l < 8; ++l) cv = (idx == l && l < L) ? cent[l] : cv;
      const int j = w * 32 + bit;
#pragma unroll
      for (int c = 0; c < kLogitsQC; ++c) mse[c] = fmaf(qrot[(qok[c] ? qrow[c] : 0) * d + j], cv, mse[c]);
    }
  }
  const uint32_t* srow = k.signs + row * SW;
  for (int w = 0; w < m / 32; ++w) {
    const uint32_t sw = srow[w];
    for (int bit = 0; bit < 32; ++bit) {
      const float tau = ((sw >> bit) & 1u) ? 1.f : -1.f;
      const int i = w * 32 + bit;
#pragma unroll
      for (int c = 0; c < kLogitsQC; ++c) qjl[c] = fmaf(proj[(qok[c] ? qrow[c] : 0) * m + i], tau, qjl[c]);
    }
  }
  if (!valid) return;
  const float nu = k.norm[row], ga = k.rnorm[row];
#pragma unroll
  for (int c = 0; c < kLogitsQC; ++c) {
    if (!qok[c]) continue;
    const int64_t o = ((static_cast<int64_t>(b) * Hq + hq[c]) * nq + qiq[c]) * ctx + t;
    logits[o] = nu * (mse[c] + P.qjl_kappa * ga * qjl[c]);
  }
}

// ----------------------------------------------------------------------------
// Logits for a codec with the recursive polar first stage (d = 128): the MSE
// term is ⟨q', ŷ⟩ with ŷ rebuilt from the angle codes, the QJL term is the
// usual one.  One thread per key: it walks the 64 level-1 pairs in order,
// keeping the products of the upper levels' factors along its path (the
// factors of levels <= ctz(i) + 2 change at pair i, two per pair on average),
// so ŷ costs about four multiplications per pair.  The query values are the
// same for every thread of the block, so they are read as scalar operands;
// the loops are unrolled, so every code's slot and bit are constants.  Up to
// 4 query vectors per block (grid.z splits the rest).  The QJL sums
// Σ_{τ_i = +1} p_i come from tables in LDS: for each byte g of the 128 sign
// bits and each of its 256 values, the four vectors' sums of p over the set
// bits (built once per block of 1024 keys), so a key takes 16 table reads
// instead of 128 multiply-adds per vector.  Likewise the level-1 pair i with
// code c contributes r_i (q'_2i cos θ_c + q'_2i+1 sin θ_c) to each vector's
// MSE sum, r_i the product of the upper levels' factors: the bracket is read
// from a table of the four vectors' values for every (pair, code); with at
// most 4 codes per angle the same is done one level up, per (level-2 node,
// its code, its two pairs' codes).
// ----------------------------------------------------------------------------
constexpr int kPolarKeys = 1024;

template <int B>
__global__ __launch_bounds__(kPolarKeys) void logits_polar_kernel(DevParams P, PolarParams PP, const float* __restrict__ qrot,
                                                           const float* __restrict__ proj, int Hq, int nq, int G,
                                                           int nkv, int64_t ctx, tq_packed_t k,
                                                           float* __restrict__ logits) {
  constexpr int d = 128, NL = 1 << B;
  __shared__ float2 tab[7][NL];     // (cos, sin) of every level's centroids
  __shared__ float psum[4];         // Σ_i p_i of each tile vector
  __shared__ float4 pj[d];          // p_j of the four tile vectors
  __shared__ float4 ptab[16][256];  // [byte g][value]: Σ over the set bits k of p_{8g+k}
  __shared__ float4 qtab[64][NL];   // [pair i][code c]: q'_2i cos θ_c + q'_2i+1 sin θ_c
  constexpr bool L2T = NL <= 4;     // level-2 table: 32 nodes x NL^3 entries
  constexpr int N3 = L2T ? NL * NL * NL : 1;
  __shared__ float4 q2tab[L2T ? 32 : 1][N3];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bk = blockIdx.y, b = bk / nkv, kh = bk % nkv;
  const int nqv = nq * G, qv0 = blockIdx.z * 4;
  const float* qp[4];
  const float* pp[4];
  int64_t orow[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int v = qv0 + t;
    const bool ok = v < nqv;
    const int qi = ok ? v / G : 0, h = kh * G + (ok ? v % G : 0);
    const int64_t qr = (static_cast<int64_t>(b) * nq + qi) * Hq + h;
    qp[t] = qrot + qr * d;
    pp[t] = proj + qr * d;
    orow[t] = ok ? ((static_cast<int64_t>(b) * Hq + h) * nq + qi) * ctx : -1;
  }
  if (tid < 7 * NL) tab[tid / NL][tid % NL] = float2{PP.cosc[tid / NL][tid % NL], PP.sinc[tid / NL][tid % NL]};
  if (wv < 4) {
    const float s = wave_sum(pp[wv][lane] + pp[wv][lane + 64]);  // wave w: tile vector w
    if (lane == 0) psum[wv] = s;
  }
  if (tid < d) pj[tid] = float4{pp[0][tid], pp[1][tid], pp[2][tid], pp[3][tid]};
  if (tid < 64 * NL) {
    const int i = tid / NL, c = tid % NL;
    const float cs = PP.cosc[0][c], sn = PP.sinc[0][c];
    qtab[i][c] = float4{fmaf(qp[0][2 * i + 1], sn, qp[0][2 * i] * cs), fmaf(qp[1][2 * i + 1], sn, qp[1][2 * i] * cs),
                        fmaf(qp[2][2 * i + 1], sn, qp[2][2 * i] * cs), fmaf(qp[3][2 * i + 1], sn, qp[3][2 * i] * cs)};
  }
  __syncthreads();
  for (int e = tid; e < 16 * 256; e += kPolarKeys) {
    const int g = e >> 8, v = e & 255;
    float4 a = float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      if ((v >> kb) & 1) {
        const float4 x = pj[8 * g + kb];
        a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
      }
    }
    ptab[g][v] = a;
  }
  if constexpr (L2T) {
    // node n, codes (c2, ca, cb): cos θ2_c2 · qtab[2n][ca] + sin θ2_c2 · qtab[2n+1][cb].
    // Entry r = c2·4^B + Σ_p q_p·4^p with q_p the two bits of plane p at the
    // slots 2n, 2n+1 (bit 0: pair 2n), so a key forms r with one extract per plane.
    for (int e = tid; e < 32 * N3; e += kPolarKeys) {
      const int n = e / N3, r = e % N3, c2 = r >> (2 * B);
      int ca = 0, cb = 0;
#pragma unroll
      for (int p = 0; p < B; ++p) {
        ca |= ((r >> (2 * p)) & 1) << p;
        cb |= ((r >> (2 * p + 1)) & 1) << p;
      }
      const float cs = PP.cosc[1][c2], sn = PP.sinc[1][c2];
      const float4 a = qtab[2 * n][ca], b = qtab[2 * n + 1][cb];
      q2tab[n][r] = float4{fmaf(sn, b.x, cs * a.x), fmaf(sn, b.y, cs * a.y), fmaf(sn, b.z, cs * a.z),
                           fmaf(sn, b.w, cs * a.w)};
    }
  }
  __syncthreads();
  const int64_t key = static_cast<int64_t>(blockIdx.x) * kPolarKeys + tid;
  if (key >= ctx) return;
  const int64_t row = static_cast<int64_t>(bk) * ctx + key;
  uint32_t w[B][4];
#pragma unroll
  for (int p = 0; p < B; ++p) {
    const uint4 u = reinterpret_cast<const uint4*>(k.codes + row * (4 * B))[p];
    w[p][0] = u.x; w[p][1] = u.y; w[p][2] = u.z; w[p][3] = u.w;
  }
  const uint4 sg = reinterpret_cast<const uint4*>(k.signs)[row];
  const uint32_t sw[4] = {sg.x, sg.y, sg.z, sg.w};
  auto code = [&](int slot) {  // slot is a constant after unrolling
    int c = 0;
#pragma unroll
    for (int p = 0; p < B; ++p) c |= static_cast<int>((w[p][slot >> 5] >> (slot & 31)) & 1u) << p;
    return c;
  };
  float mse[4] = {0.f, 0.f, 0.f, 0.f}, qj[4] = {0.f, 0.f, 0.f, 0.f};
  float prod[9];  // prod[lv]: product of the factors of levels 7..lv along the current path
  prod[8] = 1.f;
  if constexpr (L2T) {
#pragma unroll
    for (int n = 0; n < 32; ++n) {
      // levels whose factor changes at level-2 node n: lv <= ctz(n) + 3 (all at n = 0)
      const int hi = n == 0 ? 7 : (__builtin_ctz(n) + 3 < 7 ? __builtin_ctz(n) + 3 : 7);
#pragma unroll
      for (int lv = 7; lv >= 3; --lv) {
        if (lv > hi) continue;
        const int node = n >> (lv - 2), side = (n >> (lv - 3)) & 1;
        const float2 cs = tab[lv - 1][code(128 - (256 >> lv) + node)];
        prod[lv] = prod[lv + 1] * (side ? cs.y : cs.x);
      }
      int r = code(64 + n) << (2 * B);
#pragma unroll
      for (int p = 0; p < B; ++p) r |= static_cast<int>((w[p][n >> 4] >> (2 * (n & 15))) & 3u) << (2 * p);
      const float4 b = q2tab[n][r];
      mse[0] = fmaf(prod[3], b.x, mse[0]);
      mse[1] = fmaf(prod[3], b.y, mse[1]);
      mse[2] = fmaf(prod[3], b.z, mse[2]);
      mse[3] = fmaf(prod[3], b.w, mse[3]);
#pragma unroll
      for (int t = 0; t < 4; ++t) asm volatile("" : "+v"(mse[t]));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int i = 0; i < (L2T ? 0 : 64); ++i) {
    // levels whose factor changes at pair i: lv <= ctz(i) + 2 (all at i = 0)
    const int hi = i == 0 ? 7 : (__builtin_ctz(i) + 2 < 7 ? __builtin_ctz(i) + 2 : 7);
#pragma unroll
    for (int lv = 7; lv >= 2; --lv) {
      if (lv > hi) continue;
      const int node = i >> (lv - 1), side = (i >> (lv - 2)) & 1;
      const int slot = 128 - (256 >> lv) + node;  // level lv's angles start at 128 - 2^(8-lv)
      const float2 cs = tab[lv - 1][code(slot)];
      prod[lv] = prod[lv + 1] * (side ? cs.y : cs.x);
    }
    const float4 b = qtab[i][code(i)];
    mse[0] = fmaf(prod[2], b.x, mse[0]);
    mse[1] = fmaf(prod[2], b.y, mse[1]);
    mse[2] = fmaf(prod[2], b.z, mse[2]);
    mse[3] = fmaf(prod[2], b.w, mse[3]);
    // one pair's work stays together: without these the compiler keeps all
    // 128 ŷ values live and forms the dot products afterwards (256 registers)
#pragma unroll
    for (int t = 0; t < 4; ++t) asm volatile("" : "+v"(mse[t]));
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int g = 0; g < 16; ++g) {
    const float4 x = ptab[g][(sw[g >> 2] >> (8 * (g & 3))) & 255u];
    qj[0] += x.x; qj[1] += x.y; qj[2] += x.z; qj[3] += x.w;
  }
  const float nu = k.norm[row], ga = k.rnorm[row];
#pragma unroll
  for (int t = 0; t < 4; ++t)  // Σ p τ = 2 Σ_{τ=+1} p - Σ p
    if (orow[t] >= 0) logits[orow[t] + key] = nu * (mse[t] + P.qjl_kappa * ga * (2.f * qj[t] - psum[t]));
}

hipError_t launch_logits_polar(const tq_codec_s* c, const void* ws, int batch, int n_q_heads, int n_kv_heads,
                               int n_queries, tq_packed_t k, int64_t ctx, float* logits, hipStream_t s) {
  const int64_t nv = static_cast<int64_t>(batch) * n_queries * n_q_heads;
  const float* qrot = static_cast<const float*>(ws);
  const float* proj = qrot + nv * c->prm.d;
  const int G = n_q_heads / n_kv_heads;
  const dim3 grid(static_cast<unsigned>(ceil_div(ctx, kPolarKeys)), batch * n_kv_heads,
                  static_cast<unsigned>(ceil_div(static_cast<int64_t>(n_queries) * G, 4)));
  auto go = [&]<int B>() -> hipError_t {
    hipLaunchKernelGGL((logits_polar_kernel<B>), grid, dim3(kPolarKeys), 0, s, c->prm, c->pol, qrot, proj, n_q_heads,
                       n_queries, G, n_kv_heads, ctx, k, logits);
    return hipGetLastError();
  };
  switch (c->prm.b) {
    case 1: return go.template operator()<1>();
    case 2: return go.template operator()<2>();
    case 3: return go.template operator()<3>();
  }
  return hipErrorInvalidValue;
}

bool logits_mfma_eligible(const tq_codec_s* c);
size_t logits_mfma_ws_bytes(const tq_codec_s* c, int batch, int n_q_heads, int n_kv_heads, int n_queries);
hipError_t launch_logits_mfma_prep(const tq_codec_s* c, const void* q, tq_dtype_t dt, int batch, int n_q_heads,
                                   int n_kv_heads, int n_queries, void* ws, hipStream_t s);
hipError_t launch_logits_mfma(const tq_codec_s* c, const void* ws, int batch, int n_q_heads, int n_kv_heads,
                              int n_queries, tq_packed_t k, int64_t ctx, float* logits, hipStream_t s,
                              const PageMap* pm = nullptr);
bool logits_fused_eligible(const tq_codec_s* c, int batch, int n_q_heads, int n_kv_heads, int n_queries,
                           int64_t ctx);
hipError_t launch_logits_fused(const tq_codec_s* c, const void* q, tq_dtype_t dt, int batch, int n_q_heads,
                               int n_kv_heads, int n_queries, tq_packed_t k, int64_t ctx, float* logits,
                               hipStream_t s);

size_t logits_ws_bytes(const tq_codec_s* c, int batch, int n_q_heads, int n_kv_heads, int n_queries) {
  if (!c->polar && logits_mfma_eligible(c)) return logits_mfma_ws_bytes(c, batch, n_q_heads, n_kv_heads, n_queries);
  const size_t nv = static_cast<size_t>(batch) * n_queries * n_q_heads;
  return nv * (c->prm.d + c->prm.m) * sizeof(float);
}

hipError_t launch_qprep128(const tq_codec_s* c, const void* q, tq_dtype_t dt, int batch, int n_q_heads, int n_kv_heads,
                           int n_queries, float* qrot, float* proj, hipStream_t s);

hipError_t launch_logits_prep(const tq_codec_s* c, const void* q, tq_dtype_t dt, int batch, int n_q_heads,
                              int n_kv_heads, int n_queries, void* ws, hipStream_t s) {
  if (c->polar) {  // fp32 q' and p for the polar scorer (d = 128)
    float* qrot = static_cast<float*>(ws);
    float* proj = qrot + static_cast<int64_t>(batch) * n_queries * n_q_heads * c->prm.d;
    return launch_qprep128(c, q, dt, batch, n_q_heads, n_kv_heads, n_queries, qrot, proj, s);
  }
  if (!c->polar && logits_mfma_eligible(c))
    return launch_logits_mfma_prep(c, q, dt, batch, n_q_heads, n_kv_heads, n_queries, ws, s);
  const int64_t nv = static_cast<int64_t>(batch) * n_queries * n_q_heads;
  float* qrot = static_cast<float*>(ws);
  float* proj = qrot + nv * c->prm.d;
  return launch_qprep(c, q, dt, nv, qrot, proj, s);
}

hipError_t launch_logits(const tq_codec_s* c, const void* q, tq_dtype_t dt, int batch, int n_q_heads,
                         int n_kv_heads, int n_queries, tq_packed_t k, int64_t ctx, float* logits, void* ws,
                         hipStream_t s) {
  if (!c->polar && logits_fused_eligible(c, batch, n_q_heads, n_kv_heads, n_queries, ctx))
    return launch_logits_fused(c, q, dt, batch, n_q_heads, n_kv_heads, n_queries, k, ctx, logits, s);
  hipError_t e = launch_logits_prep(c, q, dt, batch, n_q_heads, n_kv_heads, n_queries, ws, s);
  if (e != hipSuccess) return e;
  return launch_logits_prepped(c, ws, batch, n_q_heads, n_kv_heads, n_queries, k, ctx, logits, s);
}

hipError_t launch_logits_prepped(const tq_codec_s* c, const void* ws, int batch, int n_q_heads, int n_kv_heads,
                                 int n_queries, tq_packed_t k, int64_t ctx, float* logits, hipStream_t s) {
  if (c->polar) return launch_logits_polar(c, ws, batch, n_q_heads, n_kv_heads, n_queries, k, ctx, logits, s);
  if (logits_mfma_eligible(c))
    return launch_logits_mfma(c, ws, batch, n_q_heads, n_kv_heads, n_queries, k, ctx, logits, s);
  const DevParams& P = c->prm;
  const int64_t nv = static_cast<int64_t>(batch) * n_queries * n_q_heads;
  const float* qrot = static_cast<const float*>(ws);
  const float* proj = qrot + nv * P.d;
  const int G = n_q_heads / n_kv_heads;
  dim3 grid(static_cast<unsigned>(ceil_div(ctx, 256)), batch * n_kv_heads,
            static_cast<unsigned>(ceil_div(static_cast<int64_t>(n_queries) * G, kLogitsQC)));
  hipLaunchKernelGGL(logits_valu_kernel, grid, dim3(256), 0, s, P, qrot, proj, n_q_heads, n_queries, G,
                     n_kv_heads, ctx, k, logits);
  return hipGetLastError();
}

// Paged cache: the query operands, then the matrix-core scorer reading each
// 64-key group from its page (per-sequence context lengths).
bool logits_paged_supported(const tq_codec_s* c) {
  return !c->polar && c->qjl && (c->prm.d == 128 || c->prm.d == 256) && c->prm.m == c->prm.d;
}

size_t logits_paged_ws_bytes(const tq_codec_s* c, int batch, int n_q_heads, int n_kv_heads, int n_queries) {
  return logits_mfma_ws_bytes(c, batch, n_q_heads, n_kv_heads, n_queries);
}

hipError_t launch_logits_paged(const tq_codec_s* c, const void* q, tq_dtype_t dt, int batch, int n_q_heads,
                               int n_kv_heads, int n_queries, tq_packed_t k, int64_t max_ctx, const PageMap& pm,
                               float* logits, void* ws, hipStream_t s) {
  hipError_t e = launch_logits_mfma_prep(c, q, dt, batch, n_q_heads, n_kv_heads, n_queries, ws, s);
  if (e != hipSuccess) return e;
  return launch_logits_mfma(c, ws, batch, n_q_heads, n_kv_heads, n_queries, k, max_ctx, logits, s, &pm);
}

// Scores of nq prepped query vectors against n packed rows: scores[q][t].
hipError_t launch_scores(const tq_codec_s* c, const float* qrot, const float* proj, int nq, tq_packed_t db,
                         int64_t n, float* scores, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(ceil_div(n, 256)), 1, static_cast<unsigned>(ceil_div(nq, kLogitsQC)));
  hipLaunchKernelGGL(logits_valu_kernel, grid, dim3(256), 0, s, c->prm, qrot, proj, nq, 1, nq, 1, n, db, scores);
  return hipGetLastError();
}

}  // namespace tq

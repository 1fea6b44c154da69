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
// usual one.  16 lanes per key, lane l rebuilding ŷ_8l..ŷ_8l+7 from the codes
// of its path (levels 7..4: nodes l >> (k+1), level 3: slot 96 + l, level 2:
// slots 64 + 2l + i, level 1: slots 4l + i) with the cos and sin tables in
// LDS; a block of 256 threads scores kPolarKeys keys against up to 4 query
// vectors.  VALU-bound: ~200 lane-instructions per key and lane.
// ----------------------------------------------------------------------------
constexpr int kPolarKeys = 256;

template <int B>
__global__ __launch_bounds__(256) void logits_polar_kernel(DevParams P, PolarParams PP, const float* __restrict__ qrot,
                                                           const float* __restrict__ proj, int Hq, int nq, int G,
                                                           int nkv, int64_t ctx, tq_packed_t k,
                                                           float* __restrict__ logits) {
  constexpr int d = 128, NL = 1 << B;
  __shared__ float tab[2][7][NL];
  for (int e = threadIdx.x; e < 7 * NL; e += 256) {
    tab[0][e / NL][e % NL] = PP.cosc[e / NL][e % NL];
    tab[1][e / NL][e % NL] = PP.sinc[e / NL][e % NL];
  }
  __syncthreads();
  const int l = threadIdx.x & 15, grp = threadIdx.x >> 4;
  const int bk = blockIdx.y, b = bk / nkv, kh = bk % nkv;
  const int nqv = nq * G, qv0 = blockIdx.z * 4;
  float qv[4][8], pv[4][8];
  int64_t orow[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int v = qv0 + t;
    const bool ok = v < nqv;
    const int qi = ok ? v / G : 0, h = kh * G + (ok ? v % G : 0);
    const int64_t qr = (static_cast<int64_t>(b) * nq + qi) * Hq + h;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qv[t][e] = ok ? qrot[qr * d + 8 * l + e] : 0.f;
      pv[t][e] = ok ? proj[qr * d + 8 * l + e] : 0.f;
    }
    orow[t] = ok ? ((static_cast<int64_t>(b) * Hq + h) * nq + qi) * ctx : -1;
  }
  const int64_t k0 = static_cast<int64_t>(blockIdx.x) * kPolarKeys;
  const int64_t k1 = min(ctx, k0 + kPolarKeys);
  for (int64_t key = k0 + grp; key < k1; key += 16) {  // uniform within the 16-lane group
    const int64_t row = static_cast<int64_t>(bk) * ctx + key;
    uint32_t w[B][4];
#pragma unroll
    for (int p = 0; p < B; ++p) {
      const uint4 u = reinterpret_cast<const uint4*>(k.codes + row * (4 * B))[p];
      w[p][0] = u.x; w[p][1] = u.y; w[p][2] = u.z; w[p][3] = u.w;
    }
    auto code = [&](int slot) {
      int c = 0;
#pragma unroll
      for (int p = 0; p < B; ++p) c |= static_cast<int>((w[p][slot >> 5] >> (slot & 31)) & 1u) << p;
      return c;
    };
    float R = 1.f;
#pragma unroll
    for (int kk = 3; kk >= 0; --kk) {  // levels 7..4
      const int c = code(128 - (16 >> kk) + (l >> (kk + 1)));
      R *= ((l >> kk) & 1) ? tab[1][3 + kk][c] : tab[0][3 + kk][c];
    }
    const int c3 = code(96 + l);
    const float q2[2] = {R * tab[0][2][c3], R * tab[1][2][c3]};
    float yh[8];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c2 = code(64 + 2 * l + i);
      const float qa = q2[i] * tab[0][1][c2], qb = q2[i] * tab[1][1][c2];
      const int ca = code(4 * l + 2 * i), cb = code(4 * l + 2 * i + 1);
      yh[4 * i] = qa * tab[0][0][ca];
      yh[4 * i + 1] = qa * tab[1][0][ca];
      yh[4 * i + 2] = qb * tab[0][0][cb];
      yh[4 * i + 3] = qb * tab[1][0][cb];
    }
    const uint32_t sw = k.signs[row * 4 + (l >> 2)] >> (8 * (l & 3));
    const float nu = k.norm[row], ga = k.rnorm[row];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float mse = 0.f, qj = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        mse = fmaf(qv[t][e], yh[e], mse);
        qj += ((sw >> e) & 1u) ? pv[t][e] : -pv[t][e];
      }
      mse = row_sum(mse);
      qj = row_sum(qj);
      if (l == 0 && orow[t] >= 0) logits[orow[t] + key] = nu * (mse + P.qjl_kappa * ga * qj);
    }
  }
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
    hipLaunchKernelGGL((logits_polar_kernel<B>), grid, dim3(256), 0, s, c->prm, c->pol, qrot, proj, n_q_heads,
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
                              int n_queries, tq_packed_t k, int64_t ctx, float* logits, hipStream_t s);
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

hipError_t launch_logits_prep(const tq_codec_s* c, const void* q, tq_dtype_t dt, int batch, int n_q_heads,
                              int n_kv_heads, int n_queries, void* ws, hipStream_t s) {
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

// Scores of nq prepped query vectors against n packed rows: scores[q][t].
hipError_t launch_scores(const tq_codec_s* c, const float* qrot, const float* proj, int nq, tq_packed_t db,
                         int64_t n, float* scores, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(ceil_div(n, 256)), 1, static_cast<unsigned>(ceil_div(nq, kLogitsQC)));
  hipLaunchKernelGGL(logits_valu_kernel, grid, dim3(256), 0, s, c->prm, qrot, proj, nq, 1, nq, 1, n, db, scores);
  return hipGetLastError();
}

}  // namespace tq

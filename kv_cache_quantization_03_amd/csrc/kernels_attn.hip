// Fused decode attention over a compressed K/V cache, split over context chunks.
//
//   split kernel, one block per (batch*kv_head, chunk):
//     logits of the G query heads for the chunk's keys, scaled; chunk max and
//     exp-sum per head; V accumulated in the codec domain:
//       M[j] += w ν c[idx_j]   (rotated domain)
//       J[i] += w ν γ τ_i       (QJL domain)
//   combine kernel, one block per (batch, q head):
//     log-sum-exp merge of the chunks, o' = (M + √(π/2)/m · Sᵀ J) / l,
//     o = Rᵀ o' = D ⊙ (Hᵀ o')/√d, fp32 or bf16 (round to nearest even) store.
//
// Pages: 「谷歌 TurboQuant 深度拆解」 第二部分 (unbiased scores); the unbiased
// value reconstruction uses E[Sᵀ sign(S r)] = √(2/π) m r/||r|| for Gaussian S;
// 「TurboQuant+ 深度解析」 第五部分 (V compressed like K) and 第六部分 (most
// attention weights at long context are tiny, so V dequantization dominates).
#include <algorithm>

#include "kernels_common.h"

namespace tq {

namespace {
constexpr int kAttnThreads = 256;

int attn_chunk(int G) { return G <= 4 ? 1024 : (G <= 8 ? 512 : 256); }

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  v = is_max ? wave_max(v) : wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wv] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < kAttnThreads / 64; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
  return r;
}
}  // namespace

// Partials per (bk, chunk, g): [mx, l, M[d], J[m]].  gate > 0 (Sparse V): the
// value term of (head, key) is dropped when exp(s - mx) < gate · l, l keeps
// every key, and a key dropped for every head is not read.  A paged cache
// (pm.table set): sequence b uses its first min(ctx_lens[b], ctx) positions; a
// chunk past them writes mx = -inf, l = 0 and zero sums.
__global__ __launch_bounds__(kAttnThreads) void decode_split_kernel(
    DevParams PK, DevParams PV, const float* __restrict__ qrot, const float* __restrict__ proj, int Hq, int nkv,
    int64_t ctx, int CH, tq_packed_t K, tq_packed_t V, float scale, float gate, PageMap pm,
    float* __restrict__ part) {
  extern __shared__ float smem[];  // s[G][CH] then red[4]
  const int G = Hq / nkv;
  const int bk = blockIdx.y, chunk = blockIdx.x;
  const int b = bk / nkv, kh = bk % nkv;
  const int64_t t0 = static_cast<int64_t>(chunk) * CH;
  const int64_t ctx_b = pm.table ? max<int64_t>(0, min<int64_t>(pm.ctx_lens[b], ctx)) : ctx;
  const int n_in = static_cast<int>(max<int64_t>(0, min<int64_t>(CH, ctx_b - t0)));
  float* s = smem;
  float* red = smem + G * CH;
  const int d = PK.d, m = PK.m, W = d / 32;
  const int LK = 1 << PK.b;

  // ---- logits of G heads for this chunk (one key per thread per pass)
  for (int tl = threadIdx.x; tl < CH; tl += kAttnThreads) {
    if (tl >= n_in) {
      for (int g = 0; g < G; ++g) s[g * CH + tl] = -INFINITY;
      continue;
    }
    const int64_t row = kv_row(pm, bk, nkv, ctx, t0 + tl);
    const uint32_t* crow = K.codes + row * PK.code_words;
    const uint32_t* srow = K.signs + row * PK.sign_words;
    const float nu = K.norm[row], ga = K.rnorm[row];
    for (int g = 0; g < G; ++g) {
      const int64_t qr = static_cast<int64_t>(b) * Hq + kh * G + g;
      const float* qq = qrot + qr * d;
      const float* pp = proj + qr * m;
      float mse = 0.f, qjl = 0.f;
      for (int w = 0; w < W; ++w) {
        uint32_t pw[3] = {0, 0, 0};
        for (int p = 0; p < PK.b; ++p) pw[p] = crow[p * W + w];
        for (int bit = 0; bit < 32; ++bit) {
          int idx = 0;
#pragma unroll
          for (int p = 0; p < 3; ++p) idx |= ((pw[p] >> bit) & 1u) << p;
          float cv = PK.cent[0];
#pragma unroll
          for (int l = 1; l < 8; ++l) cv = (idx == l && l < LK) ? PK.cent[l] : cv;
          mse = fmaf(qq[w * 32 + bit], cv, mse);
        }
      }
      for (int w = 0; w < m / 32; ++w) {
        const uint32_t sw = srow[w];
        for (int bit = 0; bit < 32; ++bit) qjl = fmaf(pp[w * 32 + bit], ((sw >> bit) & 1u) ? 1.f : -1.f, qjl);
      }
      s[g * CH + tl] = scale * nu * (mse + PK.qjl_kappa * ga * qjl);
    }
  }
  __syncthreads();
  // ---- per-head chunk max and exp weights
  float mx[16], lsum[16];
  for (int g = 0; g < G; ++g) {
    float v = -INFINITY;
    for (int tl = threadIdx.x; tl < n_in; tl += kAttnThreads) v = fmaxf(v, s[g * CH + tl]);
    mx[g] = block_reduce(v, red, true);
    float acc = 0.f;
    for (int tl = threadIdx.x; tl < CH; tl += kAttnThreads) {
      const float e = tl < n_in ? __expf(s[g * CH + tl] - mx[g]) : 0.f;
      s[g * CH + tl] = e;
      acc += e;
    }
    lsum[g] = block_reduce(acc, red, false);
    if (gate > 0.f) {  // the same threads rewrite the weights they wrote
      const float thr = gate * lsum[g];
      for (int tl = threadIdx.x; tl < CH; tl += kAttnThreads)
        if (s[g * CH + tl] < thr) s[g * CH + tl] = 0.f;
    }
  }
  __syncthreads();
  // ---- V accumulation: threads [0,128) own coordinates of M, [128,256) QJL indices of J
  const int dv = PV.d, mv = PV.m, Wv = dv / 32;
  const int LV = 1 << PV.b;
  const bool is_m = threadIdx.x < 128;
  const int lt = threadIdx.x & 127;
  const int per = (is_m ? dv : mv) / 128;  // 1..12 coordinates per thread
  float acc[16][12];
  for (int g = 0; g < G; ++g)
    for (int u = 0; u < per; ++u) acc[g][u] = 0.f;
  for (int tl = 0; tl < n_in; ++tl) {
    if (gate > 0.f) {  // uniform over the block: every thread reads the same weights
      bool any = false;
      for (int g = 0; g < G; ++g) any = any || s[g * CH + tl] > 0.f;
      if (!any) continue;
    }
    const int64_t row = kv_row(pm, bk, nkv, ctx, t0 + tl);
    const float nu = V.norm[row];
    const float scl = is_m ? nu : (per > 0 ? nu * V.rnorm[row] : 0.f);  // an MSE-only V codec has no γ (mv = 0)
    for (int u = 0; u < per; ++u) {
      const int j = lt + u * 128;
      float val;
      if (is_m) {
        const uint32_t* crow = V.codes + row * PV.code_words;
        int idx = 0;
        for (int p = 0; p < PV.b; ++p) idx |= ((crow[p * Wv + j / 32] >> (j % 32)) & 1u) << p;
        val = PV.cent[0];
#pragma unroll
        for (int l = 1; l < 8; ++l) val = (idx == l && l < LV) ? PV.cent[l] : val;
      } else {
        val = ((V.signs[row * PV.sign_words + j / 32] >> (j % 32)) & 1u) ? 1.f : -1.f;
      }
      val *= scl;
      for (int g = 0; g < G; ++g) acc[g][u] = fmaf(s[g * CH + tl], val, acc[g][u]);
    }
  }
  const int rec = 2 + dv + mv;
  for (int g = 0; g < G; ++g) {
    float* out = part + ((static_cast<int64_t>(bk) * gridDim.x + chunk) * G + g) * rec;
    if (threadIdx.x == 0) {
      out[0] = mx[g];
      out[1] = lsum[g];
    }
    for (int u = 0; u < per; ++u) out[2 + (is_m ? 0 : dv) + lt + u * 128] = acc[g][u];
  }
}

// Combine: one block of 1024 threads per (batch, q head).  Every loop that
// reads chunk partials is spread over the threads (the chunk loads are
// independent), so the kernel is not a chain of dependent L2 round trips.
constexpr int kCombThreads = 1024;

template <int E>
__global__ __launch_bounds__(kCombThreads) void decode_combine_kernel(DevParams PV, const float* __restrict__ part,
                                                                      int Hq, int nkv, int n_chunks,
                                                                      const float* __restrict__ S,
                                                                      const float* __restrict__ Dsign, void* out,
                                                                      int out_bf16) {
  constexpr int d = E * kWave;
  constexpr int NW = kCombThreads / kWave;
  __shared__ float Jsh[d];
  __shared__ float osh[d];
  __shared__ float wsh[1024];           // chunk weights exp(m_c - max)
  __shared__ float red[NW];
  __shared__ float acc_sh[4][256];     // partial sums (d = m = 128 paths below)
  const int G = Hq / nkv;
  const int bh = blockIdx.x;  // b*Hq + h
  const int b = bh / Hq, h = bh % Hq;
  const int kh = h / G, g = h % G;
  const int bk = b * nkv + kh;
  const int m = PV.m;
  const int rec = 2 + d + m;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const float* base = part + (static_cast<int64_t>(bk) * n_chunks * G + g) * rec;
  const int64_t cstride = static_cast<int64_t>(G) * rec;
  // global max over chunks
  float gm = -INFINITY;
  for (int c = tid; c < n_chunks; c += kCombThreads) gm = fmaxf(gm, base[c * cstride]);
  gm = wave_max(gm);
  if (lane == 0) red[wv] = gm;
  __syncthreads();
  gm = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) gm = fmaxf(gm, red[w]);
  __syncthreads();
  // chunk weights and the total weight
  float lt = 0.f;
  for (int c = tid; c < n_chunks; c += kCombThreads) {
    const float mc = base[c * cstride];
    const float wc = mc != -INFINITY ? __expf(mc - gm) : 0.f;  // a chunk with no position weighs 0
    wsh[c] = wc;
    lt = fmaf(wc, base[c * cstride + 1], lt);
  }
  lt = wave_sum(lt);
  if (lane == 0) red[wv] = lt;
  __syncthreads();
  float ltot = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) ltot += red[w];
  // M and J: value j = tid % (d + m) over a quarter of the chunks each
  const int nv = d + m;
  if (nv <= 2 * 128 && d == 128) {
    const int j = tid & 255, qtr = tid >> 8;
    float a = 0.f;
    if (j < nv) {  // records hold nv = d + m values (m = 0 for an MSE-only V codec)
#pragma unroll 8
      for (int c = qtr; c < n_chunks; c += 4) a = fmaf(wsh[c], base[c * cstride + 2 + j], a);
    }
    acc_sh[qtr][j] = a;
    __syncthreads();
    if (tid < nv) {
      const float v = acc_sh[0][tid] + acc_sh[1][tid] + acc_sh[2][tid] + acc_sh[3][tid];
      if (tid < d)
        osh[tid] = v;
      else
        Jsh[tid - d] = v;
    }
  } else {
    for (int j = tid; j < nv; j += kCombThreads) {
      float a = 0.f;
#pragma unroll 8
      for (int c = 0; c < n_chunks; ++c) a = fmaf(wsh[c], base[c * cstride + 2 + j], a);
      if (j < d)
        osh[j] = a;
      else
        Jsh[j - d] = a;
    }
  }
  __syncthreads();
  // o' = (M + κ Sᵀ J)/l: coordinate j over four slices of i (an empty context gives 0)
  const float inv_l = ltot > 0.f ? 1.0f / ltot : 0.f;
  if (d == 128) {
    const int j = tid & 127, part4 = tid >> 7;  // 8 slices of i
    const int i0 = part4 * (m / 8), i1 = i0 + m / 8;
    float a = 0.f;
#pragma unroll 8
    for (int i = i0; i < i1; ++i) a = fmaf(S[static_cast<int64_t>(i) * d + j], Jsh[i], a);
    reinterpret_cast<float*>(acc_sh)[part4 * 128 + j] = a;
    __syncthreads();
    if (tid < d) {
      float t = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) t += reinterpret_cast<float*>(acc_sh)[q * 128 + tid];
      osh[tid] = (osh[tid] + PV.qjl_kappa * t) * inv_l;
    }
  } else {
    for (int j = tid; j < d; j += kCombThreads) {
      float a = 0.f;
#pragma unroll 8
      for (int i = 0; i < m; ++i) a = fmaf(S[static_cast<int64_t>(i) * d + j], Jsh[i], a);
      osh[j] = (osh[j] + PV.qjl_kappa * a) * inv_l;
    }
  }
  __syncthreads();
  if (tid < kWave) {
    float v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = osh[e * kWave + lane];
    hadamard_wave<E, true>(v, lane);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = e * kWave + lane;
      const float o = v[e] * PV.inv_sqrt_d * Dsign[j];
      const int64_t oi = static_cast<int64_t>(bh) * d + j;
      if (out_bf16) {
        reinterpret_cast<__hip_bfloat16*>(out)[oi] = __float2bfloat16(o);
      } else {
        reinterpret_cast<float*>(out)[oi] = o;
      }
    }
  }
}

// Combine for d = m = 128 with one round of global loads: every thread issues
// its chunk's (max, Σw), its value j = t % 256 (M below 128, J above) of every
// fourth chunk, and its slice of S for Sᵀ J before using any of them; the
// chunk weights then go through LDS.  (Contexts over 128 chunks load the
// values of the further chunks in more rounds.)  With an MSE-only V codec
// (VQ = false) the records hold M only: value j = t % 128 of every eighth
// chunk, and no Sᵀ J.
// ctx_lens (paged caches, else nullptr): sequence b uses its first
// ceil(ctx_lens[b] / chunk) chunks; the decode kernel did not write the rest.
template <bool VQ>
__global__ __launch_bounds__(kCombThreads) void decode_combine128_kernel(DevParams PV, const float* __restrict__ part,
                                                                         int Hq, int nkv, int n_chunks_grid,
                                                                         const int32_t* __restrict__ ctx_lens,
                                                                         int chunk,
                                                                         const float* __restrict__ S,
                                                                         const float* __restrict__ Dsign, void* out,
                                                                         int out_bf16) {
  constexpr int d = 128, NW = kCombThreads / kWave;
  constexpr int NV = VQ ? 2 * d : d;    // values per record
  constexpr int NS = kCombThreads / NV;  // chunk slices (4 or 8)
  constexpr int U = 128 / NS;            // chunks per thread in the first round
  __shared__ float wsh[kCombThreads];  // chunk weights exp(m_c - max)
  __shared__ float red[NW], red2[NW];
  __shared__ float qa[NS][NV];
  __shared__ float osh[d], Jsh[d];
  __shared__ float sj[8][d];
  const int G = Hq / nkv;
  const int bh = blockIdx.x, b = bh / Hq, h = bh % Hq;
  const int bk = b * nkv + h / G, g = h % G;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, j = tid % NV, qtr = tid / NV;
  // (64-bit: a length near 2^31 must not wrap when rounded up)
  const int n_chunks =
      ctx_lens ? static_cast<int>(min(static_cast<int64_t>(n_chunks_grid),
                                      (static_cast<int64_t>(max(ctx_lens[b], 0)) + chunk - 1) / chunk))
               : n_chunks_grid;
  const int rec = 2 + NV;
  const float* base = part + (static_cast<int64_t>(bk) * n_chunks_grid * G + g) * rec;
  // unsigned 32-bit offsets from the block's base: the loads take the scalar base plus one offset register
  const unsigned cstride = static_cast<unsigned>(G * rec);
  // ---- loads
  const bool has_c = tid < n_chunks;
  const float* own = base + (has_c ? static_cast<unsigned>(tid) : 0u) * cstride;
  const float m_own = has_c ? own[0] : -INFINITY;
  const float l_own = has_c ? own[1] : 0.f;
  const int jj = tid & 127, pp = tid >> 7;  // o'_jj += Σ_{i in [16pp, 16pp+16)} S[i][jj] J_i
  float sv[16];
  if constexpr (VQ) {
#pragma unroll
    for (int u = 0; u < 16; ++u) sv[u] = S[static_cast<unsigned>((pp * 16 + u) * d + jj)];
  }
  float vc[U];
#pragma unroll
  for (int u = 0; u < U; ++u)
    vc[u] = base[static_cast<unsigned>(max(0, min(qtr + NS * u, n_chunks - 1))) * cstride + 2u + j];
  // ---- global max and chunk weights
  float m = wave_max(m_own);
  if (lane == 0) red[wv] = m;
  __syncthreads();
  float gm = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) gm = fmaxf(gm, red[w]);
  // chunks with no position (m = -inf; an empty context has only those) weigh 0
  const float w_own = has_c && m_own != -INFINITY ? __expf(m_own - gm) : 0.f;
  wsh[tid] = w_own;
  const float lw = wave_sum(w_own * l_own);
  if (lane == 0) red2[wv] = lw;
  __syncthreads();
  float ltot = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) ltot += red2[w];
  // ---- weighted sum of the thread's chunks
  float acc = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = qtr + NS * u;
    if (c < n_chunks) acc = fmaf(wsh[c], vc[u], acc);
  }
  for (int c0 = qtr + NS * U; c0 < n_chunks; c0 += NS * U) {  // contexts over 128 chunks
#pragma unroll
    for (int u = 0; u < U; ++u)
      vc[u] = base[static_cast<unsigned>(max(0, min(c0 + NS * u, n_chunks - 1))) * cstride + 2u + j];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + NS * u;
      if (c < n_chunks) acc = fmaf(wsh[c], vc[u], acc);
    }
  }
  qa[qtr][j] = acc;
  __syncthreads();
  if (tid < NV) {
    float a = 0.f;
#pragma unroll
    for (int q = 0; q < NS; ++q) a += qa[q][tid];
    if (tid < d) osh[tid] = a;
    else Jsh[tid - d] = a;
  }
  __syncthreads();
  if constexpr (VQ) {
    float a = 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) a = fmaf(sv[u], Jsh[pp * 16 + u], a);
    sj[pp][jj] = a;
    __syncthreads();
  }
  if (tid < kWave) {
    const float inv_l = ltot > 0.f ? 1.0f / ltot : 0.f;  // an empty context gives 0
    float v[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int jo = e * kWave + tid;
      float t = 0.f;
      if constexpr (VQ) {
#pragma unroll
        for (int q = 0; q < 8; ++q) t += sj[q][jo];
      }
      v[e] = (osh[jo] + PV.qjl_kappa * t) * inv_l;
    }
    hadamard_wave<2, true>(v, tid);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int jo = e * kWave + tid;
      const float o = v[e] * PV.inv_sqrt_d * Dsign[jo];
      const int64_t oi = static_cast<int64_t>(bh) * d + jo;
      if (out_bf16) {
        reinterpret_cast<__hip_bfloat16*>(out)[oi] = __float2bfloat16(o);
      } else {
        reinterpret_cast<float*>(out)[oi] = o;
      }
    }
  }
}

// The combine over contiguous chunk partials [mx, l, M[d], J[m]] (J absent
// for an MSE-only value codec): the d = m = 128 kernel, else the general one.
hipError_t launch_decode_combine_contig(const tq_codec_s* cv, const float* part, int batch, int n_q_heads,
                                        int n_kv_heads, int n_chunks, int chunk, void* out, tq_dtype_t out_dt,
                                        hipStream_t s) {
  if (cv->prm.d == 128 && (cv->prm.m == 128 || !cv->qjl)) {
    auto kern = cv->qjl ? decode_combine128_kernel<true> : decode_combine128_kernel<false>;
    hipLaunchKernelGGL(kern, dim3(batch * n_q_heads), dim3(kCombThreads), 0, s, cv->prm, part, n_q_heads,
                       n_kv_heads, n_chunks, static_cast<const int32_t*>(nullptr), chunk, cv->dS, cv->dD, out,
                       out_dt == TQ_BF16 ? 1 : 0);
    return hipGetLastError();
  }
  auto run = [&]<int E>() -> hipError_t {
    hipLaunchKernelGGL((decode_combine_kernel<E>), dim3(batch * n_q_heads), dim3(kCombThreads), 0, s, cv->prm,
                       part, n_q_heads, n_kv_heads, n_chunks, cv->dS, cv->dD, out, out_dt == TQ_BF16 ? 1 : 0);
    return hipGetLastError();
  };
  return dispatch_E(cv->prm.d, run);
}

bool decode_supported(const tq_codec_s* cv, int n_q_heads, int n_kv_heads, int64_t ctx, const char** why) {
  const int G = n_q_heads / n_kv_heads;
  if (G > 16) { *why = "at most 16 query heads per KV head"; return false; }
  if (G * (cv->prm.d / 128) > 16 * 12 || cv->prm.d < 128) { *why = "head_dim must be >= 128 and G*d/128 <= 192"; return false; }
  if (ceil_div(ctx, attn_chunk(G)) > 1024) { *why = "context too long for one call (max 1024 chunks)"; return false; }
  return true;
}

size_t logits_mfma_ws_bytes(const tq_codec_s* c, int batch, int n_q_heads, int n_kv_heads, int n_queries);
hipError_t launch_logits_mfma_prep(const tq_codec_s* c, const void* q, tq_dtype_t dt, int batch, int n_q_heads,
                                   int n_kv_heads, int n_queries, void* ws, hipStream_t s);

// Workspace: the prepared queries (rotated and projected fp32 queries for the
// general kernel, or the matrix-core operands), then the chunk partials.
static size_t decode_prep_region(const tq_codec_s* ck, int batch, int n_q_heads, int n_kv_heads) {
  const size_t nq = static_cast<size_t>(batch) * n_q_heads;
  const size_t valu = nq * (ck->prm.d + ck->prm.m) * sizeof(float);
  const size_t mfma = ck->prm.d == 128 ? logits_mfma_ws_bytes(ck, batch, n_q_heads, n_kv_heads, 1) : 0;
  return (std::max(valu, mfma) + 255) / 256 * 256;
}

size_t decode_polar_ws_bytes(const tq_codec_s* ck, const tq_codec_s* cv, int batch, int n_q_heads, int n_kv_heads,
                             int64_t ctx, int CH);
hipError_t launch_decode_polar(const tq_codec_s* ck, const tq_codec_s* cv, const void* q, tq_dtype_t q_dt,
                               int batch, int n_q_heads, int n_kv_heads, tq_packed_t k, tq_packed_t v, int64_t ctx,
                               float scale, bool sparse_v, float v_gate, const PageMap* pm, void* out,
                               tq_dtype_t out_dt, void* ws, int CH, hipStream_t s);

size_t decode_ws_bytes(const tq_codec_s* ck, const tq_codec_s* cv, int batch, int n_q_heads, int n_kv_heads,
                       int64_t ctx) {
  const int G = n_q_heads / n_kv_heads;
  const int CH = attn_chunk(G);
  if (ck->polar || cv->polar) return decode_polar_ws_bytes(ck, cv, batch, n_q_heads, n_kv_heads, ctx, CH);
  const int64_t n_chunks = ceil_div(ctx, CH);
  const size_t part = static_cast<size_t>(batch) * n_kv_heads * n_chunks * G * (2 + cv->prm.d + cv->prm.m) * sizeof(float);
  return decode_prep_region(ck, batch, n_q_heads, n_kv_heads) + part;
}

bool decode_mfma_eligible(const tq_codec_s* ck, const tq_codec_s* cv, int n_q_heads, int n_kv_heads);
bool decode_mfma_shape_ok(const tq_codec_s* ck, const tq_codec_s* cv, int n_q_heads, int n_kv_heads);
int decode_mfma_chunk();
hipError_t launch_decode_mfma(const tq_codec_s* ck, const tq_codec_s* cv, int batch, int n_q_heads, int n_kv_heads,
                              tq_packed_t k, tq_packed_t v, int64_t ctx, float scale, bool sparse_v, float v_gate,
                              const PageMap* pm, const uint8_t* prep, float* part, int n_chunks, hipStream_t s);

// Paged caches and V caches in 32-row blocks are read by the matrix-core
// kernel only (d = 128, at most 4 query heads per KV head), with the
// d = m = 128 combine.
bool decode_paged_supported(const tq_codec_s* ck, const tq_codec_s* cv, int n_q_heads, int n_kv_heads) {
  return decode_mfma_shape_ok(ck, cv, n_q_heads, n_kv_heads) && decode_mfma_chunk() == attn_chunk(n_q_heads / n_kv_heads);
}

int decode_chunk(int n_q_heads, int n_kv_heads) { return attn_chunk(n_q_heads / n_kv_heads); }

hipError_t launch_decode(const tq_codec_s* ck, const tq_codec_s* cv, const void* q, tq_dtype_t q_dt, int batch,
                         int n_q_heads, int n_kv_heads, tq_packed_t k, tq_packed_t v, int64_t ctx, float scale,
                         bool sparse_v, float v_gate, const PageMap* pm, void* out, tq_dtype_t out_dt, void* ws,
                         hipStream_t s) {
  const int G = n_q_heads / n_kv_heads;
  const int CH = attn_chunk(G);
  if (ck->polar || cv->polar)  // logits by the key codec's scorer, then V from them (kernels_attn_polar.hip)
    return launch_decode_polar(ck, cv, q, q_dt, batch, n_q_heads, n_kv_heads, k, v, ctx, scale, sparse_v, v_gate,
                               pm, out, out_dt, ws, CH, s);
  int n_chunks = static_cast<int>(ceil_div(ctx, CH));
  const int64_t nq = static_cast<int64_t>(batch) * n_q_heads;
  float* qrot = static_cast<float*>(ws);
  float* proj = qrot + nq * ck->prm.d;
  float* part = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) +
                                         decode_prep_region(ck, batch, n_q_heads, n_kv_heads));
  hipError_t e;
  // paged caches take the matrix-core kernel where its shape fits (else the
  // general kernel below, through the page table); a V cache in 32-row blocks
  // always does (the caller checked its shape)
  const bool mfma = decode_mfma_eligible(ck, cv, n_q_heads, n_kv_heads) && decode_mfma_chunk() == CH;
  if (cv->vblock || (pm && decode_paged_supported(ck, cv, n_q_heads, n_kv_heads)) || mfma) {
    // matrix-core split kernel, same partial layout.  The query operands are
    // prepared once per KV head by their own launch (rebuilding them in every
    // block measured 58.7 against 55.5 us at 32 heads x 128K keys).
    if ((e = launch_logits_mfma_prep(ck, q, q_dt, batch, n_q_heads, n_kv_heads, 1, ws, s)) != hipSuccess) return e;
    e = launch_decode_mfma(ck, cv, batch, n_q_heads, n_kv_heads, k, v, ctx, scale, sparse_v, v_gate, pm,
                           static_cast<const uint8_t*>(ws), part, n_chunks, s);
    if (e != hipSuccess) return e;
  } else {
    e = launch_qprep(ck, q, q_dt, nq, qrot, proj, s);
    if (e != hipSuccess) return e;
    const size_t sh = (static_cast<size_t>(G) * CH + 8) * sizeof(float);
    hipLaunchKernelGGL(decode_split_kernel, dim3(n_chunks, batch * n_kv_heads), dim3(kAttnThreads), sh, s, ck->prm,
                       cv->prm, qrot, proj, n_q_heads, n_kv_heads, ctx, CH, k, v, scale, sparse_v ? v_gate : 0.f,
                       pm ? *pm : PageMap{nullptr, nullptr, 0, 0}, part);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (cv->prm.d == 128 && (cv->prm.m == 128 || !cv->qjl)) {
    auto kern = cv->qjl ? decode_combine128_kernel<true> : decode_combine128_kernel<false>;
    hipLaunchKernelGGL(kern, dim3(batch * n_q_heads), dim3(kCombThreads), 0, s, cv->prm, part, n_q_heads, n_kv_heads,
                       n_chunks, pm ? pm->ctx_lens : nullptr, CH, cv->dS, cv->dD, out, out_dt == TQ_BF16 ? 1 : 0);
    return hipGetLastError();
  }
  auto run = [&]<int E>() -> hipError_t {
    hipLaunchKernelGGL((decode_combine_kernel<E>), dim3(batch * n_q_heads), dim3(kCombThreads), 0, s, cv->prm,
                       part, n_q_heads, n_kv_heads, n_chunks, cv->dS, cv->dD, out, out_dt == TQ_BF16 ? 1 : 0);
    return hipGetLastError();
  };
  return dispatch_E(cv->prm.d, run);
}

}  // namespace tq

// Attention logits over a compressed K cache: the unbiased estimator
//   ℓ = ν (Σ_j q'_j c[idx_j] + √(π/2)/m · γ · Σ_i p_i τ_i),
// q' = R q and p = S q' prepared once per query (「谷歌 TurboQuant 深度拆解」
// 第二部分: a full-precision query against the compressed key, unbiased).
//
// This file holds the general VALU kernel (one thread per key, any head_dim,
// any number of query vectors per KV head).  It is the reference kernel on the
// GPU and covers shapes the MFMA kernel does not.
#include <algorithm>

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
// Logits for a codec with the recursive polar first stage (d = 2^LD, 64 to
// 256): the MSE term is ⟨q', ŷ⟩ with ŷ rebuilt from the angle codes, the QJL
// term is the usual one.  One thread per key: it walks the d/2 level-1 pairs
// in order, keeping the products of the upper levels' factors along its path
// (the factors of levels <= ctz(i) + 2 change at pair i, two per pair on
// average), so ŷ costs about four multiplications per pair.  The query values
// are the same for every thread of the block, so they are read as scalar
// operands; the loops are unrolled, so every code's slot and bit are
// constants.  Up to 4 query vectors per block (grid.z splits the rest).  The
// QJL sums Σ_{τ_i = +1} p_i come from tables in LDS: for each 4-bit group h of
// the d sign bits and each of its 16 values, the four vectors' sums of p over
// the set bits (built once per block), so a key takes d/4 table reads instead
// of d multiply-adds per vector; a group's 16 entries (256 bytes) sit in
// distinct LDS banks, so lanes that read different entries do not collide
// (8-bit groups at d = 256: d/8 reads).  Likewise the level-1 pair i
// with code c contributes r_i (q'_2i cos θ_c + q'_2i+1 sin θ_c) to each
// vector's MSE sum, r_i the product of the upper levels' factors: the bracket
// is read from a table of the four vectors' values for every (pair, code);
// with at most 4 codes per angle and d <= 128 the same is done one level up,
// per (level-2 node, its code, its two pairs' codes).  Level l's angles sit
// in slots d - 2d/2^l + node.
// ----------------------------------------------------------------------------
// Keys (and threads) per block: 512.  Up to d = 128 two blocks share a
// compute unit (tables of at most 46 KB, at most 128 registers), so one
// block's table reads run under the other's VALU work; at d = 256 the records
// and path products take up to 254 registers and a block has the unit alone.
template <int LD>
constexpr int polar_keys() { return 512; }
template <int LD>
constexpr int polar_blocks_per_cu() { return LD <= 7 ? 2 : 1; }
// Sign bits per QJL table index: 4 (16-entry tables) up to d = 128; 8 at
// d = 256, whose registers cannot take twice the table reads (the block has
// the unit's LDS to itself there).
template <int LD>
constexpr int polar_tab_bits() { return LD <= 7 ? 4 : 8; }

// NW consecutive 32-bit words (NW = 2: one 8-byte load; else 16-byte loads).
template <int NW>
__device__ __forceinline__ void load_words(const uint32_t* p, uint32_t (&w)[NW]) {
  if constexpr (NW == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x;
    w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[i];
      w[4 * i] = v.x;
      w[4 * i + 1] = v.y;
      w[4 * i + 2] = v.z;
      w[4 * i + 3] = v.w;
    }
  }
}

// One key's record into registers (nothing past the sequence's context;
// a paged cache looks the key's row up in the page table).
template <int B, int NW>
__device__ __forceinline__ void polar_fetch(const tq_packed_t& k, const PageMap& pm, int bk, int nkv, int64_t ctx,
                                            int64_t ctx_v, int64_t key, uint32_t (&nc)[B][NW], uint32_t (&ns)[NW],
                                            float& nn, float& ng) {
  if (key < ctx_v) {
    const int64_t row = kv_row(pm, bk, nkv, ctx, key);
#pragma unroll
    for (int p = 0; p < B; ++p) load_words<NW>(k.codes + row * (NW * B) + NW * p, nc[p]);
    load_words<NW>(k.signs + row * NW, ns);
    nn = k.norm[row];
    ng = k.rnorm[row];
  }
}

// pm.table set (a paged cache): sequence b scores its first
// min(ctx_lens[b], ctx) positions; ctx is the stride of the logits rows.
template <int B, int LD>
__global__ __launch_bounds__(polar_keys<LD>())
__attribute__((amdgpu_waves_per_eu(polar_blocks_per_cu<LD>() * polar_keys<LD>() / 256))) void logits_polar_kernel(DevParams P, PolarParams PP, const float* __restrict__ qrot,
                                                           const float* __restrict__ proj, int Hq, int nq, int G,
                                                           int nkv, int64_t ctx, tq_packed_t k,
                                                           float* __restrict__ logits, PageMap pm) {
  constexpr int d = 1 << LD, NL = 1 << B, NW = d / 32, kPolarKeys = polar_keys<LD>();
  __shared__ float2 tab[LD][NL];      // (cos, sin) of every level's centroids
  __shared__ float psum[4];           // Σ_i p_i of each tile vector
  __shared__ float4 pj[d];            // p_j of the four tile vectors
  constexpr int PB = polar_tab_bits<LD>(), PV = 1 << PB, PG = 32 / PB;  // PG: groups per sign word
  __shared__ float4 ptab[d / PB][PV];  // [group h][value]: Σ over the set bits k of p_{PB h + k}
  __shared__ float4 qtab[d / 2][NL];  // [pair i][code c]: q'_2i cos θ_c + q'_2i+1 sin θ_c
  constexpr bool L2T = NL <= 4 && d <= 128;  // level-2 table: d/4 nodes x NL^3 entries
  constexpr int N3 = L2T ? NL * NL * NL : 1;
  __shared__ float4 q2tab[L2T ? d / 4 : 1][N3];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bk = blockIdx.y, b = bk / nkv, kh = bk % nkv;
  const int64_t ctx_v = pm.table ? max<int64_t>(0, min<int64_t>(pm.ctx_lens[b], ctx)) : ctx;
  if (static_cast<int64_t>(blockIdx.x) * kPolarKeys >= ctx_v) return;  // no key of this sequence for the block
  uint32_t nc[B][NW], ns[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) ns[i] = 0u;
  float nn = 0.f, ng = 0.f;
  polar_fetch<B, NW>(k, pm, bk, nkv, ctx, ctx_v, static_cast<int64_t>(blockIdx.x) * kPolarKeys + tid, nc, ns, nn, ng);
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
  if (tid < LD * NL) tab[tid / NL][tid % NL] = float2{PP.cosc[tid / NL][tid % NL], PP.sinc[tid / NL][tid % NL]};
  if (wv < 4) {
    float a = pp[wv][lane];
#pragma unroll
    for (int u = 1; u < d / 64; ++u) a += pp[wv][lane + 64 * u];
    const float s = wave_sum(a);  // wave w: tile vector w
    if (lane == 0) psum[wv] = s;
  }
  for (int e = tid; e < d; e += kPolarKeys) pj[e] = float4{pp[0][e], pp[1][e], pp[2][e], pp[3][e]};
  for (int e = tid; e < (d / 2) * NL; e += kPolarKeys) {
    const int i = e / NL, c = e % NL;
    const float cs = PP.cosc[0][c], sn = PP.sinc[0][c];
    qtab[i][c] = float4{fmaf(qp[0][2 * i + 1], sn, qp[0][2 * i] * cs), fmaf(qp[1][2 * i + 1], sn, qp[1][2 * i] * cs),
                        fmaf(qp[2][2 * i + 1], sn, qp[2][2 * i] * cs), fmaf(qp[3][2 * i + 1], sn, qp[3][2 * i] * cs)};
  }
  __syncthreads();
  for (int e = tid; e < (d / PB) * PV; e += kPolarKeys) {
    const int h = e >> PB, v = e & (PV - 1);
    float4 a = float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < PB; ++kb) {
      if ((v >> kb) & 1) {
        const float4 x = pj[PB * h + kb];
        a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
      }
    }
    ptab[h][v] = a;
  }
  if constexpr (L2T) {
    // node n, codes (c2, ca, cb): cos θ2_c2 · qtab[2n][ca] + sin θ2_c2 · qtab[2n+1][cb].
    // Entry r = c2·4^B + Σ_p q_p·4^p with q_p the two bits of plane p at the
    // slots 2n, 2n+1 (bit 0: pair 2n), so a key forms r with one extract per plane.
    for (int e = tid; e < (d / 4) * N3; e += kPolarKeys) {
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
  // blocks stride over the context's 512-key blocks; each thread's next
  // record is loaded while the current one is scored (the first one while
  // the tables are built)
  const int64_t nkb = (ctx_v + kPolarKeys - 1) / kPolarKeys;
  for (int64_t kb = blockIdx.x; kb < nkb; kb += gridDim.x) {
  const int64_t key = kb * kPolarKeys + tid;
  uint32_t w[B][NW], sw[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
#pragma unroll
    for (int p = 0; p < B; ++p) w[p][i] = nc[p][i];
    sw[i] = ns[i];
  }
  const float nu = nn, ga = ng;
  polar_fetch<B, NW>(k, pm, bk, nkv, ctx, ctx_v, key + static_cast<int64_t>(gridDim.x) * kPolarKeys, nc, ns, nn, ng);
  if (key < ctx_v) {
  auto code = [&](int slot) {  // slot is a constant after unrolling
    int c = 0;
#pragma unroll
    for (int p = 0; p < B; ++p) c |= static_cast<int>((w[p][slot >> 5] >> (slot & 31)) & 1u) << p;
    return c;
  };
  float mse[4] = {0.f, 0.f, 0.f, 0.f}, qj[4] = {0.f, 0.f, 0.f, 0.f};
  float prod[LD + 2];  // prod[lv]: product of the factors of levels LD..lv along the current path
  prod[LD + 1] = 1.f;
  if constexpr (L2T) {
    // Level-4 node m at a time (level-2 nodes 4m..4m+3): its factors of levels
    // LD..3 and its four level-2 brackets are read together, one LDS round
    // trip per group of four nodes; the products keep the top-down order.
    const float2 ftop = tab[LD - 1][code(d - 2)];
#pragma unroll
    for (int m = 0; m < d / 16; ++m) {
      float2 fu[LD > 5 ? LD - 5 : 1];  // levels LD-1 .. 5
#pragma unroll
      for (int lv = LD - 1; lv >= 5; --lv) fu[LD - 1 - lv] = tab[lv - 1][code(d - ((2 * d) >> lv) + (m >> (lv - 4)))];
      const float2 f4 = tab[3][code(d - d / 8 + m)];
      const float2 f3a = tab[2][code(d - d / 4 + 2 * m)], f3b = tab[2][code(d - d / 4 + 1 + 2 * m)];
      float4 bq[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = 4 * m + i;
        int r = code(d / 2 + n) << (2 * B);
#pragma unroll
        for (int p = 0; p < B; ++p) r |= static_cast<int>((w[p][n >> 4] >> (2 * (n & 15))) & 3u) << (2 * p);
        bq[i] = q2tab[n][r];
      }
      float p5 = ((m >> (LD - 5)) & 1) ? ftop.y : ftop.x;
#pragma unroll
      for (int lv = LD - 1; lv >= 5; --lv) p5 = p5 * (((m >> (lv - 5)) & 1) ? fu[LD - 1 - lv].y : fu[LD - 1 - lv].x);
      const float p4a = p5 * f4.x, p4b = p5 * f4.y;
      const float p3[4] = {p4a * f3a.x, p4a * f3a.y, p4b * f3b.x, p4b * f3b.y};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        mse[0] = fmaf(p3[i], bq[i].x, mse[0]);
        mse[1] = fmaf(p3[i], bq[i].y, mse[1]);
        mse[2] = fmaf(p3[i], bq[i].z, mse[2]);
        mse[3] = fmaf(p3[i], bq[i].w, mse[3]);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) asm volatile("" : "+v"(mse[t]));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if constexpr (!L2T) static_for<d / 2>([&]<int i>() {
    // levels whose factor changes at pair i: lv <= ctz(i) + 2 (all at i = 0)
    const int hi = i == 0 ? LD : (__builtin_ctz(i) + 2 < LD ? __builtin_ctz(i) + 2 : LD);
#pragma unroll
    for (int lv = LD; lv >= 2; --lv) {
      if (lv > hi) continue;
      const int node = i >> (lv - 1), side = (i >> (lv - 2)) & 1;
      const float2 cs = tab[lv - 1][code(d - ((2 * d) >> lv) + node)];
      prod[lv] = prod[lv + 1] * (side ? cs.y : cs.x);
    }
    const float4 b = qtab[i][code(i)];
    mse[0] = fmaf(prod[2], b.x, mse[0]);
    mse[1] = fmaf(prod[2], b.y, mse[1]);
    mse[2] = fmaf(prod[2], b.z, mse[2]);
    mse[3] = fmaf(prod[2], b.w, mse[3]);
    // one pair's work stays together: without these the compiler keeps all
    // d ŷ values live and forms the dot products afterwards
#pragma unroll
    for (int t = 0; t < 4; ++t) asm volatile("" : "+v"(mse[t]));
    __builtin_amdgcn_sched_barrier(0);
  });
#pragma unroll
  for (int h = 0; h < d / PB; ++h) {
    const float4 x = ptab[h][(sw[h / PG] >> (PB * (h % PG))) & (PV - 1u)];
    qj[0] += x.x; qj[1] += x.y; qj[2] += x.z; qj[3] += x.w;
    if (h % 8 == 7) {  // eight reads in flight at a time: all of them at once would spill
#pragma unroll
      for (int t = 0; t < 4; ++t) asm volatile("" : "+v"(qj[t]));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int t = 0; t < 4; ++t)  // Σ p τ = 2 Σ_{τ=+1} p - Σ p
    if (orow[t] >= 0) logits[orow[t] + key] = nu * (mse[t] + P.qjl_kappa * ga * (2.f * qj[t] - psum[t]));
  }
  }
}

hipError_t launch_logits_polar(const tq_codec_s* c, const void* ws, int batch, int n_q_heads, int n_kv_heads,
                               int n_queries, tq_packed_t k, int64_t ctx, float* logits, hipStream_t s,
                               const PageMap* pm) {
  const PageMap pmv = pm ? *pm : PageMap{nullptr, nullptr, 0, 0};
  const int64_t nv = static_cast<int64_t>(batch) * n_queries * n_q_heads;
  const float* qrot = static_cast<const float*>(ws);
  const float* proj = qrot + nv * c->prm.d;
  const int G = n_q_heads / n_kv_heads;
  // polar_blocks_per_cu blocks per compute unit in all; each block then
  // scores several key blocks with the tables it built
  const int64_t nz = ceil_div(static_cast<int64_t>(n_queries) * G, 4);
  auto go = [&]<int B, int LD>() -> hipError_t {
    const int64_t per = std::max<int64_t>(
        1, polar_blocks_per_cu<LD>() * device_cu_count() / std::max<int64_t>(1, batch * n_kv_heads * nz));
    const int64_t nkb = ceil_div(ctx, polar_keys<LD>());
    const dim3 grid(static_cast<unsigned>(std::min(nkb, per)), batch * n_kv_heads, static_cast<unsigned>(nz));
    hipLaunchKernelGGL((logits_polar_kernel<B, LD>), grid, dim3(polar_keys<LD>()), 0, s, c->prm, c->pol, qrot, proj,
                       n_q_heads, n_queries, G, n_kv_heads, ctx, k, logits, pmv);
    return hipGetLastError();
  };
  auto byd = [&]<int B>() -> hipError_t {
    switch (c->prm.d) {
      case 64: return go.template operator()<B, 6>();
      case 128: return go.template operator()<B, 7>();
      case 256: return go.template operator()<B, 8>();
    }
    return hipErrorInvalidValue;
  };
  switch (c->prm.b) {
    case 1: return byd.template operator()<1>();
    case 2: return byd.template operator()<2>();
    case 3: return byd.template operator()<3>();
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
                               hipStream_t s, const PageMap* pm = nullptr);

size_t logits_ws_bytes(const tq_codec_s* c, int batch, int n_q_heads, int n_kv_heads, int n_queries) {
  if (!c->polar && logits_mfma_eligible(c)) return logits_mfma_ws_bytes(c, batch, n_q_heads, n_kv_heads, n_queries);
  const size_t nv = static_cast<size_t>(batch) * n_queries * n_q_heads;
  return nv * (c->prm.d + c->prm.m) * sizeof(float);
}

hipError_t launch_qprep128(const tq_codec_s* c, const void* q, tq_dtype_t dt, int batch, int n_q_heads, int n_kv_heads,
                           int n_queries, float* qrot, float* proj, hipStream_t s);

hipError_t launch_logits_prep(const tq_codec_s* c, const void* q, tq_dtype_t dt, int batch, int n_q_heads,
                              int n_kv_heads, int n_queries, void* ws, hipStream_t s) {
  if (c->polar && c->prm.d == 128) {  // fp32 q' and p for the polar scorer (other d: the general prep below)
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
// A polar codec (any head_dim it takes): its query prep, then the polar
// scorer reading each key's row through the page table.
bool logits_paged_supported(const tq_codec_s* c) {
  if (c->polar) return true;
  return c->qjl && (c->prm.d == 128 || c->prm.d == 256) && c->prm.m == c->prm.d;
}

size_t logits_paged_ws_bytes(const tq_codec_s* c, int batch, int n_q_heads, int n_kv_heads, int n_queries) {
  if (c->polar) return logits_ws_bytes(c, batch, n_q_heads, n_kv_heads, n_queries);
  return logits_mfma_ws_bytes(c, batch, n_q_heads, n_kv_heads, n_queries);
}

hipError_t launch_logits_paged(const tq_codec_s* c, const void* q, tq_dtype_t dt, int batch, int n_q_heads,
                               int n_kv_heads, int n_queries, tq_packed_t k, int64_t max_ctx, const PageMap& pm,
                               float* logits, void* ws, hipStream_t s) {
  if (c->polar) {
    hipError_t e = launch_logits_prep(c, q, dt, batch, n_q_heads, n_kv_heads, n_queries, ws, s);
    if (e != hipSuccess) return e;
    return launch_logits_polar(c, ws, batch, n_q_heads, n_kv_heads, n_queries, k, max_ctx, logits, s, &pm);
  }
  // one launch where the fused kernel takes the shape (its records through the page table)
  if (logits_fused_eligible(c, batch, n_q_heads, n_kv_heads, n_queries, max_ctx))
    return launch_logits_fused(c, q, dt, batch, n_q_heads, n_kv_heads, n_queries, k, max_ctx, logits, s, &pm);
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

// Decode attention when either codec takes the recursive polar first stage.
//
// 「谷歌 TurboQuant 深度拆解」 第二部分 第三步 compresses the whole KV cache with
// the recursive polar form: a value record then holds angle codes, and its
// rotated-domain reconstruction ŷ is the product of the cos/sin factors along
// each coordinate's path from the root (「TurboQuant+ 深度解析」 第五部分: V is
// compressed like K).  The score and v̂ keep their two-stage form with ŷ in
// place of c[idx], so the step is:
//   1. the logits of every (query head, position), by the key codec's own
//      scorer (the polar scorer, or the per-coordinate kernels), into the
//      workspace;
//   2. a split kernel, one block per (batch*KV head, chunk of positions):
//      scaled logits, chunk max and exp-sum per query head (the Sparse V gate
//      as in the other split kernels), then V accumulated in the codec domain:
//        M[j] += w ν ŷ_j   (ŷ rebuilt per position from its angle codes, or
//                           c[idx_j] for a per-coordinate value codec)
//        J[i] += w ν γ τ_i
//   3. the d = m = 128 combine shared with the other decode paths.
// Eight threads share a position, each one level-4 subtree (16 coordinates):
// it rebuilds those ŷ values in registers (the three factors above the
// subtree, then its 30 products below, top-down) and accumulates them, with
// its 16 sign bits, into per-thread M and J for up to four query heads; the
// threads of a coordinate block are summed across lanes and waves once, at
// the end.  Records are loaded one step ahead; the chunk's logits, ν and γ at
// once, before any is used.
#include "kernels_common.h"

namespace tq {

namespace {
constexpr int kPvThreads = 256;
constexpr int kD = 128;

__device__ __forceinline__ int plane_code(const uint32_t* a, int NB, int bit) {
  int c = 0;
  for (int p = 0; p < NB; ++p) c |= static_cast<int>((a[p] >> bit) & 1u) << p;
  return c;
}

// The polar ŷ of coordinates [16o, 16o + 16) of one record (level-4 node o),
// rebuilt top-down from radius 1 with the fp32 cos/sin of the angle
// centroids.  Code slots of level l start at 128 - 2^(8-l): the subtree reads
// slot 126 (level 7), 124 + o/4, 120 + o/2, 112 + o, 96 + 2o + s, 64 + 4o + u
// and 8o + v (levels 6 down to 1).  All 18 table reads are issued before the
// first product.
template <int NB, int NL>
__device__ __forceinline__ void polar_subtree16(const uint32_t (&w)[NB][4], int o, const float2 (*tab)[NL],
                                                float (&y)[16]) {
  uint32_t a1[NB], a2[NB], a3[NB];
#pragma unroll
  for (int p = 0; p < NB; ++p) {
    // (the empty asm keeps the two words in registers: a select between two
    // elements of w would otherwise become an indexed load from scratch)
    uint32_t w0 = w[p][0], w1 = w[p][1];
    asm volatile("" : "+v"(w0), "+v"(w1));
    a1[p] = ((o >> 2) ? w1 : w0) >> (8 * (o & 3));  // level 1: bits 0..7
    a2[p] = w[p][2] >> (4 * o);   // level 2: bits 0..3
    a3[p] = w[p][3];              // levels 3..7
  }
  float2 f[18];  // levels 7, 6, 5, 4, then 3 (2), 2 (4), 1 (8)
  f[0] = tab[6][plane_code(a3, NB, 30)];
  f[1] = tab[5][plane_code(a3, NB, 28 + (o >> 2))];
  f[2] = tab[4][plane_code(a3, NB, 24 + (o >> 1))];
  f[3] = tab[3][plane_code(a3, NB, 16 + o)];
#pragma unroll
  for (int s = 0; s < 2; ++s) f[4 + s] = tab[2][plane_code(a3, NB, 2 * o + s)];
#pragma unroll
  for (int u = 0; u < 4; ++u) f[6 + u] = tab[1][plane_code(a2, NB, u)];
#pragma unroll
  for (int v = 0; v < 8; ++v) f[10 + v] = tab[0][plane_code(a1, NB, v)];
  const float r = (((o >> 2) ? f[0].y : f[0].x) * (((o >> 1) & 1) ? f[1].y : f[1].x)) * ((o & 1) ? f[2].y : f[2].x);
  const float r4[2] = {r * f[3].x, r * f[3].y};
  float r3[4], r2[8];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    r3[2 * s] = r4[s] * f[4 + s].x;
    r3[2 * s + 1] = r4[s] * f[4 + s].y;
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    r2[2 * u] = r3[u] * f[6 + u].x;
    r2[2 * u + 1] = r3[u] * f[6 + u].y;
  }
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    y[2 * v] = r2[v] * f[10 + v].x;
    y[2 * v + 1] = r2[v] * f[10 + v].y;
  }
}

// Loads the code planes (all four words; the subtree reads three of them) and
// the sign word of coordinates [32(o/2), 32(o/2) + 32) of chunk position tl,
// unless it is past the chunk or the Sparse V gate dropped it for every head
// of the block.
template <int NB, bool VQ, int GT>
__device__ __forceinline__ bool fetch_record(const tq_packed_t& V, int64_t row0, int tl, int n_in, int CH,
                                             const float* wm, float gate, int o, uint4 (&cw)[NB], uint32_t& sw) {
  bool need = tl < n_in;
  if (need && gate > 0.f) {
    bool any = false;
#pragma unroll
    for (int t = 0; t < GT; ++t) any = any || wm[t * CH + tl] != 0.f;
    need = any;
  }
  if (need) {
    const int64_t row = row0 + tl;
#pragma unroll
    for (int p = 0; p < NB; ++p) cw[p] = reinterpret_cast<const uint4*>(V.codes + row * (4 * NB))[p];
    if constexpr (VQ) sw = V.signs[row * 4 + (o >> 1)];
  }
  return need;
}

// Partials per (bk, chunk, g): [mx, l, M[128], J[128]] (J absent when VQ is
// false: an MSE-only value codec).  Block (chunk, bk, z) serves query heads
// z·GT .. z·GT + GT - 1 of the KV group (heads past G weigh 0).  Thread
// (kq = tid/8, o = tid%8) takes positions kq, kq + 32, ... of the chunk and
// coordinates [16o, 16o + 16).  Dynamic LDS (at most 36 KB): wm[GT][CH] = w ν,
// gam[CH] = γ, then the cross-wave sums [4][GT][256].  NB: the value codec's
// code planes.
template <int NB, bool VP, bool VQ, int GT>
__global__ __launch_bounds__(kPvThreads) void decode_from_logits_kernel(
    DevParams PV, PolarParams PP, const float* __restrict__ logits, int Hq, int nkv, int64_t ctx, int CH,
    tq_packed_t V, float scale, float gate, float* __restrict__ part) {
  constexpr int NL = 1 << NB;
  constexpr int NV = VQ ? 2 * kD : kD;  // values per partial record after (mx, l)
  extern __shared__ float4 smem4[];
  float* smem = reinterpret_cast<float*>(smem4);
  __shared__ float2 tab[7][NL];   // polar: (cos, sin) of every level's centroids
  __shared__ float cent[8];       // per-coordinate: the centroids
  __shared__ float red[kPvThreads / kWave];
  __shared__ float mxs[4], ls[4];
  const int G = Hq / nkv;
  const int bk = blockIdx.y, chunk = blockIdx.x, g0 = blockIdx.z * GT;
  const int b = bk / nkv, kh = bk % nkv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t t0 = static_cast<int64_t>(chunk) * CH;
  const int n_in = static_cast<int>(min<int64_t>(CH, ctx - t0));
  float* wm = smem;
  float* gam = wm + GT * CH;
  float* wsum = gam + CH;  // [4 waves][GT][NV]
  if constexpr (VP) {
    if (tid < 7 * NL) tab[tid / NL][tid % NL] = float2{PP.cosc[tid / NL][tid % NL], PP.sinc[tid / NL][tid % NL]};
  } else {
    if (tid < 8) cent[tid] = PV.cent[tid];
  }
  // ---- scaled logits, chunk max and exp weights per query head
  const int64_t row0 = static_cast<int64_t>(bk) * ctx + t0;
  const int lch = __builtin_ctz(CH);  // CH is a power of two
  float nv[4];
  {
    float lv[16], gv[4];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = tid + kPvThreads * u, t = e >> lch, tl = e & (CH - 1);
      lv[u] = t < GT && g0 + t < G && tl < n_in
                  ? logits[(static_cast<int64_t>(b) * Hq + kh * G + g0 + t) * ctx + t0 + tl]
                  : -INFINITY;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tl = tid + kPvThreads * r;
      nv[r] = tl < n_in ? V.norm[row0 + tl] : 0.f;
      gv[r] = VQ && tl < n_in ? V.rnorm[row0 + tl] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = tid + kPvThreads * u;
      if (e < GT * CH) wm[e] = scale * lv[u];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tl = tid + kPvThreads * r;
      if (VQ && tl < CH) gam[tl] = gv[r];
    }
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < GT; ++t) {
    if (g0 + t >= G) {  // a padding head: weight 0 everywhere (uniform branch)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tl = tid + kPvThreads * r;
        if (tl < CH) wm[t * CH + tl] = 0.f;
      }
      continue;
    }
    float v = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tl = tid + kPvThreads * r;
      if (tl < n_in) v = fmaxf(v, wm[t * CH + tl]);
    }
    v = wave_max(v);
    if (lane == 0) red[wv] = v;
    __syncthreads();
    float mx = red[0];
#pragma unroll
    for (int w = 1; w < kPvThreads / kWave; ++w) mx = fmaxf(mx, red[w]);
    __syncthreads();
    float ev[4], acc = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tl = tid + kPvThreads * r;
      ev[r] = tl < n_in ? __expf(wm[t * CH + tl] - mx) : 0.f;
      acc += ev[r];
    }
    acc = wave_sum(acc);
    if (lane == 0) red[wv] = acc;
    __syncthreads();
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kPvThreads / kWave; ++w) l += red[w];
    __syncthreads();
    if (tid == 0) {
      mxs[t] = mx;
      ls[t] = l;
    }
    // the Sparse V gate, then w ν (the same threads rewrite the weights they read)
    const float thr = gate * l;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tl = tid + kPvThreads * r;
      if (tl < CH) wm[t * CH + tl] = gate > 0.f && ev[r] < thr ? 0.f : ev[r] * nv[r];
    }
  }
  __syncthreads();
  // ---- V accumulation
  const int kq = tid >> 3, o = tid & 7;
  float am[GT][16], aj[GT][16];
#pragma unroll
  for (int t = 0; t < GT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) am[t][e] = aj[t][e] = 0.f;
  uint4 cw[NB];
  uint32_t sw = 0u;
  bool need = fetch_record<NB, VQ, GT>(V, row0, kq, n_in, CH, wm, gate, o, cw, sw);
  for (int s0 = 0; s0 < n_in; s0 += kPvThreads / 8) {
    const int tl = s0 + kq;
    uint32_t w[NB][4];
#pragma unroll
    for (int p = 0; p < NB; ++p) {
      w[p][0] = cw[p].x;
      w[p][1] = cw[p].y;
      w[p][2] = cw[p].z;
      w[p][3] = cw[p].w;
    }
    const bool have = need;
    const uint32_t sig = sw >> (16 * (o & 1));  // bit e: coordinate 16o + e
    need = fetch_record<NB, VQ, GT>(V, row0, tl + kPvThreads / 8, n_in, CH, wm, gate, o, cw, sw);
    if (have) {
      float y[16];
      if constexpr (VP) {
        polar_subtree16<NB, NL>(w, o, tab, y);
      } else {
        uint32_t a[NB];
#pragma unroll
        for (int p = 0; p < NB; ++p) a[p] = ((o >> 2) ? ((o >> 1) & 1 ? w[p][3] : w[p][2])
                                                      : ((o >> 1) & 1 ? w[p][1] : w[p][0])) >> (16 * (o & 1));
#pragma unroll
        for (int e = 0; e < 16; ++e) y[e] = cent[plane_code(a, NB, e)];
      }
      float wk[GT];
#pragma unroll
      for (int t = 0; t < GT; ++t) wk[t] = wm[t * CH + tl];
      if constexpr (VQ) {
        const float gm = gam[tl];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float tg = ((sig >> e) & 1u) ? gm : -gm;
#pragma unroll
          for (int t = 0; t < GT; ++t) aj[t][e] = fmaf(wk[t], tg, aj[t][e]);
        }
      }
#pragma unroll
      for (int t = 0; t < GT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) am[t][e] = fmaf(wk[t], y[e], am[t][e]);
    }
  }
  // ---- sum the 8 lanes of each coordinate block in the wave (lane bits 3..5), then the 4 waves
  const bool up16 = (lane >> 4) & 1, up32 = (lane >> 5) & 1;
#pragma unroll
  for (int t = 0; t < GT; ++t) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
#pragma unroll
      for (int q = 0; q < (VQ ? 2 : 1); ++q) {
        float x = q ? aj[t][e] : am[t][e];
        x += __int_as_float(row_ror_dpp<0x128>(__float_as_int(x), 0));  // lane ^ 8
        {
          const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
          x += __uint_as_float(up16 ? r16[0] : r16[1]);
        }
        {
          const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
          x += __uint_as_float(up32 ? r32[0] : r32[1]);
        }
        if (lane < 8) wsum[(wv * GT + t) * NV + q * kD + 16 * o + e] = x;
      }
    }
  }
  __syncthreads();
  constexpr int rec = 2 + NV;
  float* base = part + (static_cast<int64_t>(bk) * gridDim.x + chunk) * G * rec;
#pragma unroll
  for (int t = 0; t < GT; ++t) {
    if (g0 + t < G) {
      for (int v = tid; v < NV; v += kPvThreads)
        base[(g0 + t) * rec + 2 + v] = ((wsum[(0 * GT + t) * NV + v] + wsum[(1 * GT + t) * NV + v]) +
                                        wsum[(2 * GT + t) * NV + v]) + wsum[(3 * GT + t) * NV + v];
    }
  }
  if (tid < GT && g0 + tid < G) {
    base[(g0 + tid) * rec] = mxs[tid];
    base[(g0 + tid) * rec + 1] = ls[tid];
  }
}

size_t align256p(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t logits_ws_bytes(const tq_codec_s* c, int batch, int n_q_heads, int n_kv_heads, int n_queries);
hipError_t launch_logits(const tq_codec_s* c, const void* q, tq_dtype_t dt, int batch, int n_q_heads,
                         int n_kv_heads, int n_queries, tq_packed_t k, int64_t ctx, float* logits, void* ws,
                         hipStream_t s);
hipError_t launch_decode_combine128(const tq_codec_s* cv, const float* part, int batch, int n_q_heads,
                                    int n_kv_heads, int n_chunks, int chunk, void* out, tq_dtype_t out_dt,
                                    hipStream_t s);

bool decode_polar_shape_ok(const tq_codec_s* ck, const tq_codec_s* cv) {
  return ck->prm.d == kD && cv->prm.d == kD && (!cv->qjl || cv->prm.m == kD) && !cv->vblock;
}

static size_t polar_chunk_part_bytes(const tq_codec_s* cv, int batch, int n_q_heads, int n_kv_heads, int64_t ctx,
                                     int CH) {
  const int64_t n_chunks = ceil_div(ctx, CH);
  const int rec = 2 + kD + (cv->qjl ? kD : 0);
  return static_cast<size_t>(batch) * n_q_heads * n_chunks * rec * sizeof(float);
}

// Workspace: the key scorer's own, the logits [batch][n_q_heads][ctx] fp32,
// then the chunk partials.
size_t decode_polar_ws_bytes(const tq_codec_s* ck, const tq_codec_s* cv, int batch, int n_q_heads, int n_kv_heads,
                             int64_t ctx, int CH) {
  return align256p(logits_ws_bytes(ck, batch, n_q_heads, n_kv_heads, 1)) +
         align256p(static_cast<size_t>(batch) * n_q_heads * ctx * sizeof(float)) +
         polar_chunk_part_bytes(cv, batch, n_q_heads, n_kv_heads, ctx, CH);
}

hipError_t launch_decode_polar(const tq_codec_s* ck, const tq_codec_s* cv, const void* q, tq_dtype_t q_dt,
                               int batch, int n_q_heads, int n_kv_heads, tq_packed_t k, tq_packed_t v, int64_t ctx,
                               float scale, bool sparse_v, float v_gate, void* out, tq_dtype_t out_dt, void* ws,
                               int CH, hipStream_t s) {
  uint8_t* p = static_cast<uint8_t*>(ws);
  void* lws = p;
  p += align256p(logits_ws_bytes(ck, batch, n_q_heads, n_kv_heads, 1));
  float* logits = reinterpret_cast<float*>(p);
  p += align256p(static_cast<size_t>(batch) * n_q_heads * ctx * sizeof(float));
  float* part = reinterpret_cast<float*>(p);
  hipError_t e = launch_logits(ck, q, q_dt, batch, n_q_heads, n_kv_heads, 1, k, ctx, logits, lws, s);
  if (e != hipSuccess) return e;
  const int G = n_q_heads / n_kv_heads;
  const int n_chunks = static_cast<int>(ceil_div(ctx, CH));
  const int GT = G == 1 ? 1 : G == 2 ? 2 : 4;  // query heads per block (grid z covers the rest)
  const int nz = static_cast<int>(ceil_div(G, GT));
  const size_t sh = (static_cast<size_t>(GT + 1) * CH + 4 * GT * (cv->qjl ? 2 * kD : kD)) * sizeof(float);
  const float gate = sparse_v ? v_gate : 0.f;
  const dim3 grid(n_chunks, batch * n_kv_heads, nz);
  auto go = [&]<int NB, bool VP, bool VQ>() -> hipError_t {
    auto run = [&]<int H>() -> hipError_t {
      hipLaunchKernelGGL((decode_from_logits_kernel<NB, VP, VQ, H>), grid, dim3(kPvThreads), sh, s, cv->prm,
                         cv->pol, logits, n_q_heads, n_kv_heads, ctx, CH, v, scale, gate, part);
      return hipGetLastError();
    };
    switch (GT) {
      case 1: return run.template operator()<1>();
      case 2: return run.template operator()<2>();
      default: return run.template operator()<4>();
    }
  };
  const int nb = cv->prm.b;
  if (cv->polar) {
    switch (nb) {
      case 1: e = go.template operator()<1, true, true>(); break;
      case 2: e = go.template operator()<2, true, true>(); break;
      case 3: e = go.template operator()<3, true, true>(); break;
      default: return hipErrorInvalidValue;
    }
  } else if (cv->qjl) {
    switch (nb) {
      case 1: e = go.template operator()<1, false, true>(); break;
      case 2: e = go.template operator()<2, false, true>(); break;
      case 3: e = go.template operator()<3, false, true>(); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (nb) {
      case 2: e = go.template operator()<2, false, false>(); break;
      case 3: e = go.template operator()<3, false, false>(); break;
      default: return hipErrorInvalidValue;
    }
  }
  if (e != hipSuccess) return e;
  return launch_decode_combine128(cv, part, batch, n_q_heads, n_kv_heads, n_chunks, CH, out, out_dt, s);
}

}  // namespace tq

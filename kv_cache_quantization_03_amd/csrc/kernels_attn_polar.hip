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
//   3. the combine shared with the other decode paths.
// d/16 threads share a position (8 at d = 128, 16 at d = 256), each one
// level-4 subtree (16 coordinates): it rebuilds those ŷ values in registers
// (the factors above the subtree, then its 30 products below, top-down) and
// accumulates them, with its 16 sign bits, into per-thread M and J for up to
// four query heads; the threads of a coordinate block are summed across lanes
// and waves once, at the end.  Records are loaded one step ahead; the chunk's
// logits, ν and γ at once, before any is used.
#include <algorithm>

#include "kernels_common.h"

namespace tq {

namespace {
constexpr int kPvThreads = 256;

__device__ __forceinline__ int plane_code(const uint32_t* a, int NB, int bit) {
  int c = 0;
  for (int p = 0; p < NB; ++p) c |= static_cast<int>((a[p] >> bit) & 1u) << p;
  return c;
}

// w[i] for a lane-dependent i < N by selects between registers (the empty
// asm keeps the words in registers: a select between two elements of an
// array would otherwise become an indexed load from scratch).
template <int N>
__device__ __forceinline__ uint32_t pick_word(const uint32_t* w, int i) {
  if constexpr (N == 1) {
    return w[0];
  } else if constexpr (N == 2) {
    uint32_t w0 = w[0], w1 = w[1];
    asm volatile("" : "+v"(w0), "+v"(w1));
    return i ? w1 : w0;
  } else if constexpr (N == 4) {
    uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3];
    asm volatile("" : "+v"(w0), "+v"(w1), "+v"(w2), "+v"(w3));
    return (i & 2) ? ((i & 1) ? w3 : w2) : ((i & 1) ? w1 : w0);
  } else {
    static_assert(N == 8, "2, 4 or 8 words");
    return (i & 4) ? pick_word<4>(w + 4, i & 3) : pick_word<4>(w, i & 3);
  }
}

// The polar ŷ of coordinates [16o, 16o + 16) of one record (level-4 node o,
// D = 128 or 256, LD = log2 D levels), rebuilt top-down from radius 1 with
// the fp32 cos/sin of the angle centroids.  Level l's slots start at
// D - 2D/2^l: the subtree reads, for level l >= 5, slot D - 2D/2^l + (o >>
// (l - 4)) (all in the record's last word), then 7D/8 + o (level 4), 3D/4 +
// 2o + s, D/2 + 4o + u and 8o + v (levels 3 to 1).  All table reads are
// issued before the first product.
template <int NB, int NL, int D>
__device__ __forceinline__ void polar_subtree16(const uint32_t (&w)[NB][D / 32], int o, const float2 (*tab)[NL],
                                                float (&y)[16]) {
  constexpr int NWD = D / 32, LD = D == 128 ? 7 : 8, NU = LD - 4;  // NU: levels LD..5
  uint32_t a1[NB], a2[NB], a3[NB], a4[NB], at[NB];
#pragma unroll
  for (int p = 0; p < NB; ++p) {
    a1[p] = pick_word<NWD / 2 < 4 ? NWD / 2 : 4>(w[p], o >> 2) >> (8 * (o & 3));  // level 1: bits 0..7
    a2[p] = pick_word<NWD / 4 < 2 ? 1 : 2>(w[p] + D / 64, o >> 3) >> (4 * (o & 7));  // level 2: bits 0..3
    a3[p] = w[p][(3 * D / 4) >> 5];  // level 3
    a4[p] = w[p][(7 * D / 8) >> 5];  // level 4
    at[p] = w[p][NWD - 1];           // levels 5..LD
  }
  float2 f[NU + 15];  // levels LD..5, 4, then 3 (2), 2 (4), 1 (8)
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int lv = LD - u;
    f[u] = tab[lv - 1][plane_code(at, NB, 32 - ((2 * D) >> lv) + (o >> (lv - 4)))];
  }
  f[NU] = tab[3][plane_code(a4, NB, ((7 * D / 8) & 31) + o)];
#pragma unroll
  for (int s = 0; s < 2; ++s) f[NU + 1 + s] = tab[2][plane_code(a3, NB, ((3 * D / 4) & 31) + 2 * o + s)];
#pragma unroll
  for (int u = 0; u < 4; ++u) f[NU + 3 + u] = tab[1][plane_code(a2, NB, u)];
#pragma unroll
  for (int v = 0; v < 8; ++v) f[NU + 7 + v] = tab[0][plane_code(a1, NB, v)];
  float r = ((o >> (LD - 5)) & 1) ? f[0].y : f[0].x;
#pragma unroll
  for (int u = 1; u < NU; ++u) r = r * (((o >> (LD - 5 - u)) & 1) ? f[u].y : f[u].x);
  const float r4[2] = {r * f[NU].x, r * f[NU].y};
  float r3[4], r2[8];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    r3[2 * s] = r4[s] * f[NU + 1 + s].x;
    r3[2 * s + 1] = r4[s] * f[NU + 1 + s].y;
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    r2[2 * u] = r3[u] * f[NU + 3 + u].x;
    r2[2 * u + 1] = r3[u] * f[NU + 3 + u].y;
  }
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    y[2 * v] = r2[v] * f[NU + 7 + v].x;
    y[2 * v + 1] = r2[v] * f[NU + 7 + v].y;
  }
}

// Loads the code planes (every word; the subtree reads some of them) and the
// sign word of coordinates [32(o/2), 32(o/2) + 32) of chunk position tl,
// unless it is past the chunk or the Sparse V gate dropped it for every head
// of the block.
template <int NB, bool VQ, int GT, int D>
__device__ __forceinline__ bool fetch_record(const tq_packed_t& V, const PageMap& pm, int bk, int nkv, int64_t ctx,
                                             int64_t t0, int tl, int n_in, int CH, const float* wm, float gate, int o,
                                             uint32_t (&cw)[NB][D / 32], uint32_t& sw) {
  constexpr int NWD = D / 32;
  bool need = tl < n_in;
  if (need && gate > 0.f) {
    bool any = false;
#pragma unroll
    for (int t = 0; t < GT; ++t) any = any || wm[t * CH + tl] != 0.f;
    need = any;
  }
  if (need) {
    const int64_t row = kv_row(pm, bk, nkv, ctx, t0 + tl);
#pragma unroll
    for (int p = 0; p < NB; ++p)
#pragma unroll
      for (int i = 0; i < NWD / 4; ++i) {
        const uint4 x = reinterpret_cast<const uint4*>(V.codes + row * (NWD * NB) + NWD * p)[i];
        cw[p][4 * i] = x.x;
        cw[p][4 * i + 1] = x.y;
        cw[p][4 * i + 2] = x.z;
        cw[p][4 * i + 3] = x.w;
      }
    if constexpr (VQ) sw = V.signs[row * NWD + (o >> 1)];
  }
  return need;
}

// Partials per (bk, chunk, g): [mx, l, M[D], J[D]] (J absent when VQ is
// false: an MSE-only value codec).  Block (chunk, bk, z) serves query heads
// z·GT .. z·GT + GT - 1 of the KV group (heads past G weigh 0).  Thread
// (kq = tid/NO, o = tid%NO), NO = D/16, takes positions kq, kq + 256/NO, ...
// of the chunk and coordinates [16o, 16o + 16).  Dynamic LDS (at most 52 KB):
// wm[GT][CH] = w ν, gam[CH] = γ, then the cross-wave sums [4][GT][2D].  NB:
// the value codec's code planes.  A paged cache (pm.table set): sequence b
// uses its first min(ctx_lens[b], ctx) positions, rows through the page
// table; a chunk past them writes mx = -inf, l = 0 and zero sums.  ctx is
// the logits row stride either way.
template <int NB, bool VP, bool VQ, int GT, int D>
__global__ __launch_bounds__(kPvThreads) void decode_from_logits_kernel(
    DevParams PV, PolarParams PP, const float* __restrict__ logits, int Hq, int nkv, int64_t ctx, int CH,
    tq_packed_t V, float scale, float gate, PageMap pm, float* __restrict__ part) {
  constexpr int NL = 1 << NB, NWD = D / 32, LD = D == 128 ? 7 : 8;
  constexpr int NO = D / 16, PS = kPvThreads / NO;  // threads per position, positions per step
  constexpr int NV = VQ ? 2 * D : D;  // values per partial record after (mx, l)
  extern __shared__ float4 smem4[];
  float* smem = reinterpret_cast<float*>(smem4);
  __shared__ float2 tab[LD][NL];  // polar: (cos, sin) of every level's centroids
  __shared__ float cent[8];       // per-coordinate: the centroids
  __shared__ float red[kPvThreads / kWave];
  __shared__ float mxs[4], ls[4];
  const int G = Hq / nkv;
  const int bk = blockIdx.y, chunk = blockIdx.x, g0 = blockIdx.z * GT;
  const int b = bk / nkv, kh = bk % nkv;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t t0 = static_cast<int64_t>(chunk) * CH;
  const int64_t ctx_v = pm.table ? max<int64_t>(0, min<int64_t>(pm.ctx_lens[b], ctx)) : ctx;
  const int n_in = static_cast<int>(max<int64_t>(0, min<int64_t>(CH, ctx_v - t0)));
  float* wm = smem;
  float* gam = wm + GT * CH;
  float* wsum = gam + CH;  // [4 waves][GT][NV]
  if constexpr (VP) {
    if (tid < LD * NL) tab[tid / NL][tid % NL] = float2{PP.cosc[tid / NL][tid % NL], PP.sinc[tid / NL][tid % NL]};
  } else {
    if (tid < 8) cent[tid] = PV.cent[tid];
  }
  // ---- scaled logits, chunk max and exp weights per query head
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
      const int64_t row = tl < n_in ? kv_row(pm, bk, nkv, ctx, t0 + tl) : 0;
      nv[r] = tl < n_in ? V.norm[row] : 0.f;
      gv[r] = VQ && tl < n_in ? V.rnorm[row] : 0.f;
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
  const int kq = tid / NO, o = tid % NO;
  float am[GT][16], aj[GT][16];
#pragma unroll
  for (int t = 0; t < GT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) am[t][e] = aj[t][e] = 0.f;
  uint32_t cw[NB][NWD];
  uint32_t sw = 0u;
  bool need = fetch_record<NB, VQ, GT, D>(V, pm, bk, nkv, ctx, t0, kq, n_in, CH, wm, gate, o, cw, sw);
  for (int s0 = 0; s0 < n_in; s0 += PS) {
    const int tl = s0 + kq;
    uint32_t w[NB][NWD];
#pragma unroll
    for (int p = 0; p < NB; ++p)
#pragma unroll
      for (int i = 0; i < NWD; ++i) w[p][i] = cw[p][i];
    const bool have = need;
    const uint32_t sig = sw >> (16 * (o & 1));  // bit e: coordinate 16o + e
    need = fetch_record<NB, VQ, GT, D>(V, pm, bk, nkv, ctx, t0, tl + PS, n_in, CH, wm, gate, o, cw, sw);
    if (have) {
      float y[16];
      if constexpr (VP) {
        polar_subtree16<NB, NL, D>(w, o, tab, y);
      } else {
        uint32_t a[NB];
#pragma unroll
        for (int p = 0; p < NB; ++p) a[p] = pick_word<NWD>(w[p], o >> 1) >> (16 * (o & 1));
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
  // ---- sum the lanes of each coordinate block in the wave (lane bits log2(NO)..5), then the 4 waves
  const bool up16 = (lane >> 4) & 1, up32 = (lane >> 5) & 1;
#pragma unroll
  for (int t = 0; t < GT; ++t) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
#pragma unroll
      for (int q = 0; q < (VQ ? 2 : 1); ++q) {
        float x = q ? aj[t][e] : am[t][e];
        if constexpr (NO == 8) x += __int_as_float(row_ror_dpp<0x128>(__float_as_int(x), 0));  // lane ^ 8
        {
          const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
          x += __uint_as_float(up16 ? r16[0] : r16[1]);
        }
        {
          const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
          x += __uint_as_float(up32 ? r32[0] : r32[1]);
        }
        if (lane < NO) wsum[(wv * GT + t) * NV + q * D + 16 * o + e] = x;
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

hipError_t launch_decode_combine_contig(const tq_codec_s* cv, const float* part, int batch, int n_q_heads,
                                        int n_kv_heads, int n_chunks, int chunk, void* out, tq_dtype_t out_dt,
                                        hipStream_t s);

bool decode_polar_shape_ok(const tq_codec_s* ck, const tq_codec_s* cv) {
  const int d = cv->prm.d;
  return (d == 128 || d == 256) && ck->prm.d == d && (!cv->qjl || cv->prm.m == d) && !cv->vblock;
}

static size_t polar_chunk_part_bytes(const tq_codec_s* cv, int batch, int n_q_heads, int n_kv_heads, int64_t ctx,
                                     int CH) {
  const int64_t n_chunks = ceil_div(ctx, CH);
  const int rec = 2 + cv->prm.d + (cv->qjl ? cv->prm.d : 0);
  return static_cast<size_t>(batch) * n_q_heads * n_chunks * rec * sizeof(float);
}

// Workspace: the key scorer's own (the larger of the contiguous and the paged
// scorer's), the logits [batch][n_q_heads][ctx] fp32, then the chunk partials.
static size_t scorer_ws_bytes(const tq_codec_s* ck, int batch, int n_q_heads, int n_kv_heads) {
  size_t b = logits_ws_bytes(ck, batch, n_q_heads, n_kv_heads, 1);
  if (logits_paged_supported(ck)) b = std::max(b, logits_paged_ws_bytes(ck, batch, n_q_heads, n_kv_heads, 1));
  return align256p(b);
}

size_t decode_polar_ws_bytes(const tq_codec_s* ck, const tq_codec_s* cv, int batch, int n_q_heads, int n_kv_heads,
                             int64_t ctx, int CH) {
  return scorer_ws_bytes(ck, batch, n_q_heads, n_kv_heads) +
         align256p(static_cast<size_t>(batch) * n_q_heads * ctx * sizeof(float)) +
         polar_chunk_part_bytes(cv, batch, n_q_heads, n_kv_heads, ctx, CH);
}

hipError_t launch_decode_polar(const tq_codec_s* ck, const tq_codec_s* cv, const void* q, tq_dtype_t q_dt,
                               int batch, int n_q_heads, int n_kv_heads, tq_packed_t k, tq_packed_t v, int64_t ctx,
                               float scale, bool sparse_v, float v_gate, const PageMap* pm, void* out,
                               tq_dtype_t out_dt, void* ws, int CH, hipStream_t s) {
  uint8_t* p = static_cast<uint8_t*>(ws);
  void* lws = p;
  p += scorer_ws_bytes(ck, batch, n_q_heads, n_kv_heads);
  float* logits = reinterpret_cast<float*>(p);
  p += align256p(static_cast<size_t>(batch) * n_q_heads * ctx * sizeof(float));
  float* part = reinterpret_cast<float*>(p);
  hipError_t e = pm ? launch_logits_paged(ck, q, q_dt, batch, n_q_heads, n_kv_heads, 1, k, ctx, *pm, logits, lws, s)
                    : launch_logits(ck, q, q_dt, batch, n_q_heads, n_kv_heads, 1, k, ctx, logits, lws, s);
  if (e != hipSuccess) return e;
  const PageMap pmv = pm ? *pm : PageMap{nullptr, nullptr, 0, 0};
  const int G = n_q_heads / n_kv_heads;
  const int n_chunks = static_cast<int>(ceil_div(ctx, CH));
  const int GT = G == 1 ? 1 : G == 2 ? 2 : 4;  // query heads per block (grid z covers the rest)
  const int nz = static_cast<int>(ceil_div(G, GT));
  const int D = cv->prm.d;
  const size_t sh = (static_cast<size_t>(GT + 1) * CH + 4 * GT * (cv->qjl ? 2 * D : D)) * sizeof(float);
  const float gate = sparse_v ? v_gate : 0.f;
  const dim3 grid(n_chunks, batch * n_kv_heads, nz);
  auto go = [&]<int NB, bool VP, bool VQ>() -> hipError_t {
    auto run = [&]<int H>() -> hipError_t {
      if (D == 128)
        hipLaunchKernelGGL((decode_from_logits_kernel<NB, VP, VQ, H, 128>), grid, dim3(kPvThreads), sh, s, cv->prm,
                           cv->pol, logits, n_q_heads, n_kv_heads, ctx, CH, v, scale, gate, pmv, part);
      else
        hipLaunchKernelGGL((decode_from_logits_kernel<NB, VP, VQ, H, 256>), grid, dim3(kPvThreads), sh, s, cv->prm,
                           cv->pol, logits, n_q_heads, n_kv_heads, ctx, CH, v, scale, gate, pmv, part);
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
  return launch_decode_combine_contig(cv, part, batch, n_q_heads, n_kv_heads, n_chunks, CH, out, out_dt, s);
}

}  // namespace tq

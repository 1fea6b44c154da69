// Exhaustive-search scores on the CDNA4 matrix cores.
//
// Vector search scores every query against every database record with the
// attention estimator (「谷歌 TurboQuant 深度拆解」 第三部分 向量搜索; the
// estimator is 第二部分):
//   score = ν (Σ_j q'_j c[idx_j] + √(π/2)/m · γ · Σ_i p_i τ_i).
// At 10^3 queries x 10^6 records x d = 1536 that is a dense contraction of
// about 3·10^12 multiply-adds, far beyond the fp32 vector units, so it runs
// as fp8 x fp4 matrix products (v_mfma_scale_f32_16x16x128_f8f6f4):
//
// * B operands are the packed bit planes themselves (the b code planes, their
//   parity for b = 3, the QJL signs), made FP4 by the AND masks of the logits
//   kernel: the word's bits 4j+v become nibble j of operand dword v with value
//   0 or 0.5, 1, 2 (v = 0, 1, 2), and ±1 (v = 3).
// * A operands are the queries in fixed point.  Per (query, 32-coordinate
//   block) with |a| < 2^E, a is rounded to a B-bit integer times 2^(E-B) and
//   split into B/4 base-16 digits with the sign (B = 16 for q'; B = 12 for p,
//   whose term carries the factor √(π/2)/m).  A digit times the nibble
//   compensation (2, 1, 1/2, -1/2) is an exact e4m3 number, and the digit's
//   weight 16^(B/4-1-l) 2^(E-B) is the op's E8M0 block scale (the scale of lane
//   16b + r covers row r, contraction elements 32b..32b+31).  Every product is
//   then a multiple of 1/2 below 16, so the op's group sums are exact and the
//   only error is the 2^-(B+1) rounding of the digits, relative to the block
//   maximum.  (Sums of eight products are aligned to their maximum and cut 13
//   bits below it on gfx950, so floating-point limbs would lose more; twelve
//   bits of q' leave errors of 1e-4 of the score for Gaussian queries.)
// * Every code plane multiplies the same query digits, so one accumulator per
//   plane keeps one A operand set per contraction step; the plane weights of the
//   codebook expansion c(idx) = bias + Σ_P coef_P plane_P(idx) are applied with
//   the record's ν when the scores are written.
// * The -1/2 compensation of the ±1 nibbles adds -1/2 Σ_{v=3} â to each plane
//   sum; the prep kernel folds that, the bias term and the -Σ p of
//   τ = 2·bit - 1 into one constant per query and estimator part.
//
// Work split.  The digits of one 16-query tile for every contraction step
// (d/128 steps x 4 digits x 2 KiB = 96 KiB for q' at d = 1536) stay in LDS for
// a block of 4096 records.  q' and p together would not fit the 160 KiB of LDS,
// so the MSE part and the QJL part are two launches of one kernel: the first
// writes ν(Σ q'c) and the second adds ν κ γ Σ p τ.  Each of the 8 waves takes
// a few record tiles of 16 at a time and streams their plane words with 8- or
// 16-byte loads (lane group g reads words NS·g + s of every plane, so step s's
// B operand for contraction block g is the word itself).
#include "mfma_common.h"

namespace tq {

namespace {
constexpr int kDigQ = 4;            // base-16 digits of q' (16 bits)
constexpr int kDigP = 3;            // base-16 digits of p (12 bits: the QJL term carries a factor 1/m)
constexpr int kSWaves = 8;
#ifndef TQ_MSE_TILES
#define TQ_MSE_TILES 4
#define TQ_MSE_LW 2
#define TQ_QJL_TILES 4
#define TQ_QJL_LW 4
#endif
// record tiles per wave and plane words per lane and load, per estimator part
constexpr int kMseTiles = TQ_MSE_TILES, kMseLW = TQ_MSE_LW, kQjlTiles = TQ_QJL_TILES, kQjlLW = TQ_QJL_LW;
constexpr int kSPrepThreads = 256;
constexpr int64_t kSPerBlock = 4096;  // records per block

// Prepared operands of query tile qt for vector vec (0: q', 1: p) with DIG
// digits: aop[qt][s][l][lane][32] fp8 digits, ascl[qt][s][l][lane] E8M0
// scales, qconst[qt*16 + row][vec] the constant of the estimator part.
template <int NS, int DIG>
__global__ __launch_bounds__(kSPrepThreads) void search_prep_kernel(DevParams P, const float* __restrict__ src,
                                                                   int vec, int nq, uint8_t* __restrict__ aop,
                                                                   uint8_t* __restrict__ ascl,
                                                                   float* __restrict__ qconst) {
  constexpr int W = 4 * NS, d = 128 * NS, HW = kSPrepThreads / 32;
  __shared__ float part[HW][16][3];  // per half-wave and row: Σ_{v=3} â, Σ â, Σ_{v=3} â without its last digit
  constexpr int BITS = 4 * DIG;
  const int qt = blockIdx.x;
  const int hw = threadIdx.x >> 5, l32 = threadIdx.x & 31;
  for (int i = threadIdx.x; i < HW * 16 * 3; i += kSPrepThreads) (&part[0][0][0])[i] = 0.f;
  __syncthreads();
  uint8_t* A = aop + static_cast<size_t>(qt) * NS * DIG * kOpBytes;
  uint8_t* SC = ascl + static_cast<size_t>(qt) * NS * DIG * 64;
  const int v = l32 & 3, j = l32 >> 2;  // nibble class and nibble of coordinate bit l32 of the word
  const float comp = v == 0 ? 2.f : (v == 1 ? 1.f : (v == 2 ? 0.5f : -0.5f));
  for (int pi = hw; pi < 16 * W; pi += HW) {  // (row, word) pairs, one per half-wave
    const int row = pi / W, w = pi % W;
    const int q = qt * 16 + row;
    const float a = q < nq ? src[static_cast<int64_t>(q) * d + 32 * w + l32] : 0.f;
    float mx = fabsf(a);
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 32));
    int E = -111;  // keeps every digit scale 2^(E-BITS+4(DIG-1-l)) inside E8M0
    if (mx > 0.f) {
      int e;
      (void)frexpf(mx, &e);  // mx in [2^(e-1), 2^e)
      E = max(e, -111);
    }
    const float V = fminf(rintf(ldexpf(fabsf(a), BITS - E)), static_cast<float>((1 << BITS) - 1));
    const int vi = static_cast<int>(V);
    const float sg = a < 0.f ? -1.f : 1.f;
    const int b = w / NS, s = w % NS;  // word w feeds contraction block b of step s
    const int k = 32 * b + 8 * v + j;  // contraction index of this coordinate
    const int lane = 16 * ((k & 63) >> 4) + row;
    const int byte = (k & 15) + 16 * (k >> 6);
#pragma unroll
    for (int l = 0; l < DIG; ++l) {
      const int dig = (vi >> (4 * (DIG - 1 - l))) & 15;
      const float x = sg * static_cast<float>(dig) * comp;
      const int f8 = __builtin_amdgcn_cvt_pk_fp8_f32(x, 0.f, 0, false);
      A[((static_cast<size_t>(s) * DIG + l) * 64 + lane) * 32 + byte] = static_cast<uint8_t>(f8 & 0xFF);
      if (l32 == 0) SC[(s * DIG + l) * 64 + 16 * b + row] = static_cast<uint8_t>(127 + E - BITS + 4 * (DIG - 1 - l));
    }
    const float ahat = sg * ldexpf(V, E - BITS);  // the value the digits carry
    const float ahat_t = sg * ldexpf(static_cast<float>(vi & ~15), E - BITS);  // without the last digit
    float c3 = v == 3 ? ahat : 0.f, sa = ahat, c3t = v == 3 ? ahat_t : 0.f;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) {
      c3 += __shfl_xor(c3, o, 32);
      sa += __shfl_xor(sa, o, 32);
      c3t += __shfl_xor(c3t, o, 32);
    }
    if (l32 == 0) {
      part[hw][row][0] += c3;
      part[hw][row][1] += sa;
      part[hw][row][2] += c3t;
    }
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    float c3 = 0.f, sa = 0.f, c3t = 0.f;
    for (int h = 0; h < HW; ++h) {
      c3 += part[h][threadIdx.x][0];
      sa += part[h][threadIdx.x][1];
      c3t += part[h][threadIdx.x][2];
    }
    c3 *= 0.5f;  // the ±1 nibbles' offset: true Σ â·bit = op sum + c3
    c3t *= 0.5f;
    float cst;
    if (vec == 0) {
      float csum = 0.f;
      for (int i = 0; i < P.n_planes; ++i) csum += P.plane_coef[i];
      cst = P.plane_bias * sa + csum * c3;
      if (P.n_planes == 4) cst += P.plane_coef[3] * (c3t - c3);  // the parity plane drops the last digit
    } else {
      cst = 2.f * c3 - sa;  // Σ p τ = 2 Σ p·bit - Σ p
    }
    qconst[(static_cast<size_t>(qt) * 16 + threadIdx.x) * 2 + vec] = cst;
  }
}

typedef uint32_t v2u __attribute__((ext_vector_type(2)));
template <int SG>
__device__ __forceinline__ void load_words(const uint32_t* p, uint32_t (&o)[SG]) {
  if constexpr (SG == 4) {
    const v4u x = *reinterpret_cast<const v4u*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = x[i];
  } else if constexpr (SG == 2) {
    const v2u x = *reinterpret_cast<const v2u*>(p);
    o[0] = x[0];
    o[1] = x[1];
  } else {
    o[0] = p[0];
  }
}

// One estimator part for (16-query tile blockIdx.x) x (records of block y).
// QJL = false: the NB code planes (+ parity), A = q' digits; writes
//   scores = ν (const_q + Σ_P coef_P ⟨plane_P, q̂'⟩).
// QJL = true: the sign plane, A = p digits; adds ν κ γ (2 ⟨bits, p̂⟩ + const_p).
template <int NS, int NB, bool QJL, int TILES, int DIG, int LW>
__global__ __launch_bounds__(kSWaves * 64) void search_part_kernel(DevParams P, const uint8_t* __restrict__ aop,
                                                                  const uint8_t* __restrict__ ascl,
                                                                  const float* __restrict__ qconst, int nq,
                                                                  tq_packed_t db, int64_t n,
                                                                  float* __restrict__ scores, int64_t ld) {
  constexpr int NW = QJL ? 1 : NB;                   // planes loaded per record
  constexpr int NPL = QJL ? 1 : (NB == 3 ? 4 : NB);  // planes multiplied (+ parity for b = 3)
  constexpr int W = 4 * NS, RW = NW * W;             // words per plane, per record
  constexpr int SG = NS % LW == 0 ? LW : 1;  // contraction steps per record load
  constexpr int ABYTES = NS * DIG * kOpBytes, SBYTES = NS * DIG * 64;
  __shared__ __attribute__((aligned(16))) uint8_t sa[ABYTES];
  __shared__ __attribute__((aligned(16))) uint8_t ss[SBYTES];
  const int qt = blockIdx.x;
  {
    const v4u* src = reinterpret_cast<const v4u*>(aop + static_cast<size_t>(qt) * ABYTES);
    for (int i = threadIdx.x; i < ABYTES / 16; i += kSWaves * 64) reinterpret_cast<v4u*>(sa)[i] = src[i];
    const v4u* ssrc = reinterpret_cast<const v4u*>(ascl + static_cast<size_t>(qt) * SBYTES);
    for (int i = threadIdx.x; i < SBYTES / 16; i += kSWaves * 64) reinterpret_cast<v4u*>(ss)[i] = ssrc[i];
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, col = lane & 15;
  float cst[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) cst[r] = qconst[(static_cast<size_t>(qt) * 16 + 4 * g + r) * 2 + (QJL ? 1 : 0)];
  float coef[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) coef[i] = QJL ? 2.f : P.plane_coef[i];
  const uint32_t* words = QJL ? db.signs : db.codes;
  __syncthreads();

  const int64_t lo = static_cast<int64_t>(blockIdx.y) * kSPerBlock;
  const int64_t hi = min(n, lo + kSPerBlock);
  for (int64_t t0 = lo + wv * (16 * TILES); t0 < hi; t0 += kSWaves * 16 * TILES) {
    v4f acc[TILES][NPL];
#pragma unroll
    for (int t = 0; t < TILES; ++t)
#pragma unroll
      for (int i = 0; i < NPL; ++i) acc[t][i] = v4f{0.f, 0.f, 0.f, 0.f};
    int64_t rec[TILES];  // this lane's record of tile t (the last one past the end: read, never written)
#pragma unroll
    for (int t = 0; t < TILES; ++t) rec[t] = min(t0 + 16 * t + col, n - 1);
#pragma unroll 1
    for (int s0 = 0; s0 < NS; s0 += SG) {
      uint32_t wd[TILES][NW][SG];
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        const uint32_t* rp = words + rec[t] * RW + NS * g + s0;
#pragma unroll
        for (int pl = 0; pl < NW; ++pl) load_words<SG>(rp + pl * W, wd[t][pl]);
      }
#pragma unroll
      for (int s1 = 0; s1 < SG; ++s1) {
        const int s = s0 + s1;
        v8i a[DIG];
        int sc[DIG];
#pragma unroll
        for (int l = 0; l < DIG; ++l) {
          a[l] = *reinterpret_cast<const v8i*>(sa + ((s * DIG + l) * 64 + lane) * 32);
          sc[l] = ss[(s * DIG + l) * 64 + lane];
        }
        // plane-major, so only one plane's B operands (one per tile) are live
#pragma unroll
        for (int pl = 0; pl < NPL; ++pl) {
#pragma unroll
          for (int t = 0; t < TILES; ++t) {
            uint32_t w;
            if (NB == 3 && !QJL && pl == 3) w = wd[t][0][s1] ^ wd[t][NW > 1 ? 1 : 0][s1] ^ wd[t][NW - 1][s1];
            else w = wd[t][pl < NW ? pl : 0][s1];
            const v8i bo = fp4_operand(w);
            // the parity plane's weight is ~1/16 of the largest bit plane's (Lloyd-Max
            // codebooks are close to uniform), so its last digit is below the others' error
            const int ND = (!QJL && pl == 3) ? DIG - 1 : DIG;  // pl is unrolled: constant
#pragma unroll
            for (int l = 0; l < ND; ++l) acc[t][pl] = mfma_fp8_fp4_scaled(a[l], bo, acc[t][pl], sc[l]);
          }
        }
      }
    }
    // lane L, register r holds query row 4(L/16) + r of record column L%16
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      const int64_t r = t0 + 16 * t + col;
      if (r >= hi) continue;
      const float f = QJL ? P.qjl_kappa * db.norm[r] * db.rnorm[r] : db.norm[r];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int q = qt * 16 + 4 * g + rr;
        if (q >= nq) continue;
        float x = cst[rr];
#pragma unroll
        for (int pl = 0; pl < NPL; ++pl) x = fmaf(coef[pl], acc[t][pl][rr], x);
        float* o = scores + static_cast<int64_t>(q) * ld + r;
        if constexpr (QJL)
          *o = fmaf(f, x, *o);
        else
          *o = f * x;
      }
    }
  }
}

// Calls f.template operator()<NS>() for the supported step counts.
template <typename F>
hipError_t dispatch_ns(int ns, F&& f) {
  switch (ns) {
    case 1: return f.template operator()<1>();
    case 2: return f.template operator()<2>();
    case 4: return f.template operator()<4>();
    case 8: return f.template operator()<8>();
    case 12: return f.template operator()<12>();
  }
  return hipErrorInvalidValue;
}

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct PrepLayout {
  size_t aq, ap, sq, sp, qconst, total;  // q' digits, p digits, their scales, constants
};
PrepLayout prep_layout(const tq_codec_s* c, int nq) {
  const size_t nqt = static_cast<size_t>(ceil_div(nq, 16));
  const size_t ns = c->prm.d / 128;
  PrepLayout L{};
  L.aq = 0;
  L.ap = L.aq + align256(nqt * ns * kDigQ * kOpBytes);
  L.sq = L.ap + align256(nqt * ns * kDigP * kOpBytes);
  L.sp = L.sq + align256(nqt * ns * kDigQ * 64);
  L.qconst = L.sp + align256(nqt * ns * kDigP * 64);
  L.total = L.qconst + align256(nqt * 16 * 2 * sizeof(float));
  return L;
}
}  // namespace

bool search_mfma_eligible(const tq_codec_s* c) {
  const char* v = std::getenv("TQ_SEARCH_KERNEL");
  if (v && std::string(v) == "valu") return false;
  const DevParams& P = c->prm;
  if (P.d % 128 != 0 || P.m != P.d || (P.b != 2 && P.b != 3)) return false;
  const int ns = P.d / 128;
  return ns == 1 || ns == 2 || ns == 4 || ns == 8 || ns == 12;
}

// Bytes of the prepared query operands (digits, scales, constants).
size_t search_mfma_prep_bytes(const tq_codec_s* c, int nq) { return prep_layout(c, nq).total; }

hipError_t launch_search_mfma_prep(const tq_codec_s* c, const float* qrot, const float* proj, int nq, void* prep,
                                   hipStream_t s) {
  const DevParams& P = c->prm;
  const int nqt = static_cast<int>(ceil_div(nq, 16));
  const PrepLayout L = prep_layout(c, nq);
  uint8_t* base = static_cast<uint8_t*>(prep);
  float* qc = reinterpret_cast<float*>(base + L.qconst);
  auto run = [&]<int NS>() -> hipError_t {
    hipLaunchKernelGGL((search_prep_kernel<NS, kDigQ>), dim3(nqt), dim3(kSPrepThreads), 0, s, P, qrot, 0, nq,
                       base + L.aq, base + L.sq, qc);
    hipLaunchKernelGGL((search_prep_kernel<NS, kDigP>), dim3(nqt), dim3(kSPrepThreads), 0, s, P, proj, 1, nq,
                       base + L.ap, base + L.sp, qc);
    return hipGetLastError();
  };
  return dispatch_ns(P.d / 128, run);
}

// scores[q][r] (row stride ld) for the n records of db and the nq prepared queries.
hipError_t launch_search_mfma_scores(const tq_codec_s* c, const void* prep, int nq, tq_packed_t db, int64_t n,
                                     float* scores, int64_t ld, hipStream_t s) {
  const DevParams& P = c->prm;
  const int nqt = static_cast<int>(ceil_div(nq, 16));
  const PrepLayout L = prep_layout(c, nq);
  const uint8_t* base = static_cast<const uint8_t*>(prep);
  const float* qc = reinterpret_cast<const float*>(base + L.qconst);
  const dim3 grid(nqt, static_cast<unsigned>(ceil_div(n, kSPerBlock)));
  const dim3 block(kSWaves * 64);
  auto run = [&]<int NS>() -> hipError_t {
    if (P.b == 3)
      hipLaunchKernelGGL((search_part_kernel<NS, 3, false, kMseTiles, kDigQ, kMseLW>), grid, block, 0, s, P, base + L.aq,
                         base + L.sq, qc, nq, db, n, scores, ld);
    else
      hipLaunchKernelGGL((search_part_kernel<NS, 2, false, kMseTiles, kDigQ, kMseLW>), grid, block, 0, s, P, base + L.aq,
                         base + L.sq, qc, nq, db, n, scores, ld);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((search_part_kernel<NS, 2, true, kQjlTiles, kDigP, kQjlLW>), grid, block, 0, s, P, base + L.ap, base + L.sp,
                       qc, nq, db, n, scores, ld);
    return hipGetLastError();
  };
  return dispatch_ns(P.d / 128, run);
}

}  // namespace tq

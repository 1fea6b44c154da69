// Encode (rotate, quantize, pack, residual, QJL signs), the query-side rotation,
// and the S-projection GEMM used by both.
//
// Pages: 「谷歌 TurboQuant 深度拆解」 第二部分 (rotation, fixed scalar quantizer,
// 1-bit QJL signs of the projected residual); 「TurboQuant+ 深度解析」 第二部分
// (random-sign Walsh–Hadamard rotation) and 第四部分 (the rotation must be
// computed in high precision: here fp32 throughout); 「TurboQuant 学习路径」
// 二.4 (bit-packing into 32-bit words).
#include <cmath>
#include <cstdlib>
#include <string>

#include "kernels_common.h"

namespace tq {

// ----------------------------------------------------------------------------
// Rotate + quantize: one wavefront per vector.
//   ν = ||x||, y = H (D ⊙ x/ν)/√d, idx_j = #{k : t_k < y_j} (ties low),
//   r = y - c[idx] -> rbuf (fp32), γ = ||r||, codes packed as bit-planes.
// ----------------------------------------------------------------------------
// The residual goes to rbuf as fp32 [n][d] (RM = kResF32) or, for the
// matrix-core projection, as r·rscale split into an fp16 pair [n][hi, lo][d]
// (RM = kResF16; the same bytes).  An MSE-only codec (RM = kResNone) keeps
// neither the residual nor γ: its record is the codes and ν.
enum ResidualMode { kResF32, kResF16, kResNone };

// Bit-plane packing of one vector's codes (code of coordinate e*64 + lane in
// idx[e] of that lane): plane p, register e -> words p*(d/32) + 2e (+1), the
// ballot's two halves selected into lane (word % 64) of register word / 64.
template <int E>
__device__ __forceinline__ void pack_code_planes(const int (&idx)[E], int lane, int nb, uint32_t* __restrict__ crow,
                                                 int W) {
  constexpr int d = E * kWave;
  constexpr int WMAX = 3 * d / 32;                  // words of the widest record (b = 3)
  constexpr int NW = (WMAX + kWave - 1) / kWave;    // registers of words per lane
  uint32_t words[NW];
#pragma unroll
  for (int r = 0; r < NW; ++r) words[r] = 0u;
  static_for<3>([&]<int p>() {
    if (p >= nb) return;  // uniform
    static_for<E>([&]<int e>() {
      const uint64_t m = __ballot((idx[e] >> p) & 1);
      constexpr int w0 = p * (d / 32) + 2 * e;  // even: both halves land in one register
      uint32_t& wr = words[w0 / kWave];
      wr = lane == w0 % kWave ? static_cast<uint32_t>(m) : wr;
      wr = lane == w0 % kWave + 1 ? static_cast<uint32_t>(m >> 32) : wr;
      __builtin_amdgcn_sched_barrier(0);  // each ballot's two scalar registers are used at once
    });
  });
#pragma unroll
  for (int r = 0; r < NW; ++r)
    if (r * kWave + lane < W) crow[r * kWave + lane] = words[r];
}

template <int E, typename T, int RM>
__global__ __launch_bounds__(256) void encode_rq_kernel(const T* __restrict__ x, int64_t n, DevParams P,
                                                        const float* __restrict__ Dsign,
                                                        uint32_t* __restrict__ codes, float* __restrict__ norm,
                                                        float* __restrict__ rnorm, float* __restrict__ rbuf,
                                                        float rscale) {
  constexpr int d = E * kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t vec = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (vec >= n) return;  // wave-uniform
  const T* xr = x + vec * d;
  float v[E];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    v[e] = load_elem(xr, e * kWave + lane);
    ss = fmaf(v[e], v[e], ss);
  }
  ss = wave_sum(ss);
  const float nu = sqrtf(ss);
  const float inv = nu > 0.f ? 1.0f / nu : 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] *= inv * Dsign[e * kWave + lane];
  hadamard_wave<E, false, true>(v, lane);

  // quantize (idx = #{k : t_k < y}, ties low).  The codebook is symmetric
  // (c[L-1-k] = -c[k], middle boundary 0): with s = [y > 0] and m = #{positive
  // boundaries below |y|} (at or below it when y <= 0, hence |y| one ulp up
  // there), idx = s ? L/2 + m : L/2-1 - m and c[idx] = ±c[L/2 + m].  At most 3
  // positive boundaries (L <= 8); the unused ones are +inf.
  const int H = (1 << P.b) / 2;
  float tb[3], tc[4];  // the positive boundaries and centroids (uniform; read once)
#pragma unroll
  for (int j = 0; j < 3; ++j) tb[j] = P.bound[H + j];
#pragma unroll
  for (int j = 0; j < 4; ++j) tc[j] = P.cent[min(H + j, 7)];
  int idx[E];
  float rs = 0.f;
  float* rr = rbuf + vec * d;
  _Float16* rh = reinterpret_cast<_Float16*>(rbuf) + vec * 2 * d;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float y = v[e] * P.inv_sqrt_d;
    const bool pos = y > 0.f;
    const float a = __uint_as_float((__float_as_uint(y) & 0x7FFFFFFFu) + (pos ? 0u : 1u));
    int mm = 0;
    float mag = tc[0];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const bool gt = tb[j] < a;
      mm += gt;
      mag = gt ? tc[j + 1] : mag;
    }
    idx[e] = pos ? H + mm : H - 1 - mm;
    asm volatile("" : "+v"(idx[e]));  // a vector register now, not lane masks kept for the packing
    const float yh = pos ? mag : -mag;
    const float r = y - yh;
    if constexpr (RM == kResF16) {
      const float rsc = r * rscale;
      const _Float16 hi = static_cast<_Float16>(rsc);
      rh[e * kWave + lane] = hi;
      rh[d + e * kWave + lane] = static_cast<_Float16>(rsc - static_cast<float>(hi));
    } else if constexpr (RM == kResF32) {
      rr[e * kWave + lane] = r;
    }
    rs = fmaf(r, r, rs);
  }
  if constexpr (RM != kResNone) rs = wave_sum(rs);

  pack_code_planes<E>(idx, lane, P.b, codes + vec * P.code_words, P.code_words);
  if (lane == 0) {
    norm[vec] = nu;
    if constexpr (RM != kResNone) rnorm[vec] = sqrtf(rs);
  }
}

// q' = H (D ⊙ q)/√d (no normalisation): one wavefront per vector.
template <int E, typename T>
__global__ __launch_bounds__(256) void rotate_kernel(const T* __restrict__ x, int64_t n, float inv_sqrt_d,
                                                     const float* __restrict__ Dsign, float* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t vec = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (vec >= n) return;
  constexpr int d = E * kWave;
  float v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] = load_elem(x + vec * d, e * kWave + lane) * Dsign[e * kWave + lane];
  hadamard_wave<E, false, true>(v, lane);
#pragma unroll
  for (int e = 0; e < E; ++e) out[vec * d + e * kWave + lane] = v[e] * inv_sqrt_d;
}

// ----------------------------------------------------------------------------
// S-projection: Z[v][i] = Σ_j A[v][j] S[i][j]  (A: [n][K], S: [M][K] row-major).
// 64x64 output tile per 256-thread block, 4x4 per thread, K in chunks of 16
// through LDS.  Epilogue: fp32 store, or the sign bits [Z >= 0] packed into
// words (bit i%32 of word i/32).
// ----------------------------------------------------------------------------
constexpr int kTileV = 64, kTileI = 64, kTileK = 16;

template <bool kSigns>
__global__ __launch_bounds__(256) void sproj_kernel(const float* __restrict__ A, int64_t n, int K, int M,
                                                    const float* __restrict__ S, float* __restrict__ Z,
                                                    uint32_t* __restrict__ signs) {
  __shared__ float As[kTileK][kTileV + 4];
  __shared__ float Bs[kTileK][kTileI + 4];
  __shared__ uint8_t sg[kSigns ? kTileV : 1][kSigns ? kTileI + 4 : 1];
  const int tid = threadIdx.x;
  const int tv = tid / 16, ti = tid % 16;  // 16x16 threads, 4x4 each
  const int64_t v0 = static_cast<int64_t>(blockIdx.x) * kTileV;
  const int i0 = blockIdx.y * kTileI;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += kTileK) {
    // load A tile: 64 rows x 16 k (4 per thread)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int li = tid + r * 256;  // 0..1023
      const int row = li / kTileK, kk = li % kTileK;
      const int64_t gv = v0 + row;
      As[kk][row] = (gv < n) ? A[gv * K + k0 + kk] : 0.f;
      const int gi = i0 + row;
      Bs[kk][row] = S[static_cast<int64_t>(gi) * K + k0 + kk];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kTileK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        a[r] = As[kk][tv * 4 + r];
        b[r] = Bs[kk][ti * 4 + r];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(a[r], b[c], acc[r][c]);
    }
    __syncthreads();
  }
  if constexpr (!kSigns) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t gv = v0 + tv * 4 + r;
      if (gv >= n) continue;
#pragma unroll
      for (int c = 0; c < 4; ++c) Z[gv * M + i0 + ti * 4 + c] = acc[r][c];
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) sg[tv * 4 + r][ti * 4 + c] = acc[r][c] >= 0.f ? 1 : 0;
    __syncthreads();
    if (tid < 2 * kTileV) {
      const int row = tid / 2, half = tid % 2;
      const int64_t gv = v0 + row;
      if (gv < n) {
        uint32_t w = 0;
#pragma unroll
        for (int b = 0; b < 32; ++b) w |= static_cast<uint32_t>(sg[row][half * 32 + b]) << b;
        signs[gv * (M / 32) + i0 / 32 + half] = w;
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Fused encode for d = m = 128: rotate, quantize, pack and the QJL signs in
// one pass, with S·r on the matrix cores.
//
// * 16 lanes per vector, lane l holding coordinates 8l..8l+7 (one 16-byte
//   load of a bf16/fp16 row): the Walsh-Hadamard butterflies of coordinate
//   bits 0-2 run between registers, bits 3-6 between lanes through DPP.
// * The residual r (scaled by 2^6) goes to LDS as an fp16 pair hi + lo; with
//   S = S_hi + S_lo prepared in fp16 at codec creation, z = S r is
//   S_hi r_hi + S_hi r_lo + S_lo r_hi on v_mfma_f32_16x16x32_f16, whose sums
//   keep fp32 precision (measured), so z carries ~1e-7 absolute error
//   against the 1e-5 band the sign decisions are held to.
// * A block encodes 16 vectors per pass; wave w owns outputs 32w..32w+31 of
//   z and keeps its fp16 rows of S in registers for all passes.
// ----------------------------------------------------------------------------
typedef float f4v __attribute__((ext_vector_type(4)));
constexpr int kEncPasses = 8;

// Angle codes, #{boundaries β of the level below θ} (ties low), decided
// without forming θ.
// Level 1, θ = atan2(b, a) taken into [0, 2π) for the pair (a, b): sin(θ - β)
// has the sign of b cos β - a sin β, and θ > β holds iff θ lies in the later
// half-turn (θ >= π > β) or in β's half-turn with sin(θ - β) > 0.
template <int NL>
__device__ __forceinline__ int polar_code_l1(const PolarParams& PP, float a, float b) {
  const bool up = b < 0.f || (b == 0.f && a < 0.f);  // θ in [π, 2π)
  int c = 0;
#pragma unroll
  for (int k = 0; k + 1 < NL; ++k) {
    const float2 t = PP.bcs[0][k];
    const bool pos = fmaf(b, t.x, -(a * t.y)) > 0.f;
    c += PP.bound[0][k] < 3.14159265358979324f ? (up || pos) : (up && pos);
  }
  return c;
}
// Upper levels, θ = atan2(√rb2, √ra2) in [0, π/2] from the children's squared
// radii; the boundaries lie inside (0, π/2), where θ > β iff rb2 cos²β > ra2 sin²β.
template <int NL>
__device__ __forceinline__ int polar_code_up(const float2 (&t)[16], float ra2, float rb2) {
  int c = 0;
#pragma unroll
  for (int k = 0; k + 1 < NL; ++k) c += fmaf(rb2, t[k].x, -(ra2 * t[k].y)) > 0.f;
  return c;
}

// POLAR: the recursive polar first stage (「谷歌 TurboQuant 深度拆解」 第二部分
// PolarQuant) replaces the per-coordinate quantizer.  Lane l holds y_8l..y_8l+7:
// levels 1-3 pair registers (4, 2, 1 angles per lane), levels 4-7 pair the
// lanes l and l ^ 2^(level-4) (both lanes of a pair compute the same angle
// from the same two radii).  Codes go to their slots in LDS (level 1: 4l + i,
// level 2: 64 + 2l + i, level 3: 96 + l, level k >= 4: 128 - 2^(8-k) + node),
// and ŷ is rebuilt top-down from radius 1 with the fp32 cos and sin tables.
// QJL = false (an MSE-only codec): codes and ν only, no residual, no S·r.
template <typename T, int B, bool POLAR, bool QJL>
__global__ __launch_bounds__(256) void encode_fused_kernel(const T* __restrict__ x, int64_t n, DevParams P,
                                                           PolarParams PP, const float* __restrict__ Dsign,
                                                           const _Float16* __restrict__ S16,
                                                           uint32_t* __restrict__ codes, uint32_t* __restrict__ signs,
                                                           float* __restrict__ norm, float* __restrict__ rnorm) {
  constexpr int d = 128, NL = 1 << B;
  __shared__ __attribute__((aligned(16))) _Float16 rh[2][16][d + 8];  // r hi / lo of the pass's 16 vectors
  __shared__ float ptab[POLAR ? 2 : 1][POLAR ? 7 : 1][POLAR ? NL : 1];  // cos, sin of every level's centroids
  __shared__ uint8_t pcode[POLAR ? 16 : 1][POLAR ? d : 1];            // angle codes by slot
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, l = lane & 15;
  const int vrow = 4 * wv + (lane >> 4);  // the lane's vector within the pass
  if constexpr (POLAR) {
    for (int e = threadIdx.x; e < 7 * NL; e += blockDim.x) {
      ptab[0][e / NL][e % NL] = PP.cosc[e / NL][e % NL];
      ptab[1][e / NL][e % NL] = PP.sinc[e / NL][e % NL];
    }
    __syncthreads();
  }
  // fp16 S rows of this wave's outputs: A fragments [row block][K step][hi, lo]
  h8 sf[2][4][2];
  if constexpr (QJL) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int hl = 0; hl < 2; ++hl)
          sf[rb][ks][hl] = *reinterpret_cast<const h8*>(S16 + hl * d * d + (32 * wv + 16 * rb + l) * d + 32 * ks +
                                                        8 * (lane >> 4));
  }
  float dsg[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) dsg[e] = Dsign[8 * l + e];

  for (int pass = 0; pass < kEncPasses; ++pass) {
    const int64_t tile0 = (static_cast<int64_t>(blockIdx.x) * kEncPasses + pass) * 16;
    if (tile0 >= n) break;  // block-uniform
    const int64_t vec = tile0 + vrow;
    const bool valid = vec < n;
    float v[8];
    load8(x + (valid ? vec : n - 1) * d + 8 * l, v);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
    const float nu = sqrtf(row_sum(ss));
    // 1/(ν √d) by the hardware reciprocal (1 ulp; the codes tolerate far more)
    const float kscale = nu > 0.f ? __builtin_amdgcn_rcpf(nu) * P.inv_sqrt_d : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] *= dsg[e];
    // y = H (D ⊙ x)/(ν √d): coordinate bits 0-2 in registers, 3-6 across lanes
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (e & h) continue;
        const float a = v[e], b = v[e + h];
        v[e] = a + b;
        v[e + h] = a - b;
      }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool upper = (l >> k) & 1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float o = lane_xor_f(v[e], k);
        v[e] = upper ? (o - v[e]) : (v[e] + o);
      }
    }
    // quantize (idx = #{k : t_k < y}, ties low), residual, bit planes.  The
    // codebook is symmetric (c[L-1-k] = -c[k], middle boundary 0), so with
    // s = [y > 0] and m = #{positive boundaries t below |y|} (at or below it
    // when y <= 0, hence |y| one ulp up there): idx = s ? L/2 + m : L/2-1 - m,
    // c[idx] = ±c[L/2 + m], the top bit is s and the others are m's, inverted
    // when y <= 0.
    uint32_t bits[B];
#pragma unroll
    for (int p = 0; p < B; ++p) bits[p] = 0u;
    float rr[8], rs = 0.f;
    if constexpr (POLAR) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = v[e] * kscale;
      int c1[4], c2[2];
      float r1[4], r2[2];  // squared radii
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // level 1: angles in [0, 2π)
        c1[i] = polar_code_l1<NL>(PP, y[2 * i], y[2 * i + 1]);
        r1[i] = fmaf(y[2 * i], y[2 * i], y[2 * i + 1] * y[2 * i + 1]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        c2[i] = polar_code_up<NL>(PP.bcs[1], r1[2 * i], r1[2 * i + 1]);
        r2[i] = r1[2 * i] + r1[2 * i + 1];
      }
      const int c3 = polar_code_up<NL>(PP.bcs[2], r2[0], r2[1]);
      float rad = r2[0] + r2[1];
      int ck[4];  // levels 4..7: lanes l and l ^ 2^k (the same sum on both)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float o = lane_xor_f(rad, k);
        const bool hi = (l >> k) & 1;
        const float a = hi ? o : rad, b = hi ? rad : o;
        ck[k] = polar_code_up<NL>(PP.bcs[3 + k], a, b);
        rad = a + b;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) pcode[vrow][4 * l + i] = static_cast<uint8_t>(c1[i]);
#pragma unroll
      for (int i = 0; i < 2; ++i) pcode[vrow][64 + 2 * l + i] = static_cast<uint8_t>(c2[i]);
      pcode[vrow][96 + l] = static_cast<uint8_t>(c3);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if ((l & ((2 << k) - 1)) == 0) pcode[vrow][128 - (16 >> k) + (l >> (k + 1))] = static_cast<uint8_t>(ck[k]);
      if (l == 0) pcode[vrow][127] = 0;
      // ŷ top-down from radius 1
      float R = 1.f;
#pragma unroll
      for (int k = 3; k >= 0; --k) R *= ((l >> k) & 1) ? ptab[1][3 + k][ck[k]] : ptab[0][3 + k][ck[k]];
      float q2[2] = {R * ptab[0][2][c3], R * ptab[1][2][c3]};
      float q1[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        q1[2 * i] = q2[i] * ptab[0][1][c2[i]];
        q1[2 * i + 1] = q2[i] * ptab[1][1][c2[i]];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rr[2 * i] = y[2 * i] - q1[i] * ptab[0][0][c1[i]];
        rr[2 * i + 1] = y[2 * i + 1] - q1[i] * ptab[1][0][c1[i]];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) rs = fmaf(rr[e], rr[e], rs);
      __builtin_amdgcn_wave_barrier();  // a vector's 16 lanes are one wave's: its LDS writes land first
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int cd = pcode[vrow][8 * l + e];
#pragma unroll
        for (int p = 0; p < B; ++p) bits[p] |= static_cast<uint32_t>((cd >> p) & 1) << e;
      }
    } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float y = v[e] * kscale;
      const bool pos = y > 0.f;
      const float a = __uint_as_float((__float_as_uint(y) & 0x7FFFFFFFu) + (pos ? 0u : 1u));
      int mm = 0;
      float mag = P.cent[NL / 2];
#pragma unroll
      for (int j = 0; j < NL / 2 - 1; ++j) {
        const bool gt = P.bound[NL / 2 + j] < a;
        mm += gt;
        mag = gt ? P.cent[NL / 2 + j + 1] : mag;
      }
      const float yh = pos ? mag : -mag;
      const int lowbits = pos ? mm : ~mm;
#pragma unroll
      for (int p = 0; p + 1 < B; ++p) bits[p] |= static_cast<uint32_t>((lowbits >> p) & 1) << e;
      bits[B - 1] |= static_cast<uint32_t>(pos) << e;
      if constexpr (QJL) {
        rr[e] = y - yh;
        rs = fmaf(rr[e], rr[e], rs);
      }
    }
    }  // POLAR
    if constexpr (QJL) rs = row_sum(rs);
    // code word w (coordinates 32w..32w+31) of plane p from lanes 4w..4w+3
#pragma unroll
    for (int p = 0; p < B; ++p) {
      uint32_t word = bits[p] << (8 * (l & 3));
      word |= lane_xor<0>(word);
      word |= lane_xor<1>(word);
      if (valid && (l & 3) == 0) codes[vec * (B * 4) + 4 * p + (l >> 2)] = word;
    }
    if (valid && l == 0) {
      norm[vec] = nu;
      if constexpr (QJL) rnorm[vec] = sqrtf(rs);
    }
    if constexpr (!QJL) continue;  // an MSE-only record is complete
    h8 hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float rsc = rr[e] * 64.f;
      hi[e] = static_cast<_Float16>(rsc);
      lo[e] = static_cast<_Float16>(rsc - static_cast<float>(hi[e]));
    }
    *reinterpret_cast<h8*>(&rh[0][vrow][8 * l]) = hi;
    *reinterpret_cast<h8*>(&rh[1][vrow][8 * l]) = lo;
    __syncthreads();
    // z = S r: rows = this wave's outputs, columns = the pass's 16 vectors
    f4v acc[2] = {f4v{0.f, 0.f, 0.f, 0.f}, f4v{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const h8 bh = *reinterpret_cast<const h8*>(&rh[0][l][32 * ks + 8 * (lane >> 4)]);
      const h8 bl = *reinterpret_cast<const h8*>(&rh[1][l][32 * ks + 8 * (lane >> 4)]);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sf[rb][ks][0], bh, acc[rb], 0, 0, 0);
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sf[rb][ks][0], bl, acc[rb], 0, 0, 0);
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sf[rb][ks][1], bh, acc[rb], 0, 0, 0);
      }
    }
    asm volatile("" : "+v"(acc[0]), "+v"(acc[1]));  // matrix ops stay in wave-uniform flow
    // sign bits [z >= 0]: lane (g, v) holds outputs 32w + 16rb + 4g + r of vector v
    uint32_t part = 0u;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) part |= static_cast<uint32_t>(acc[rb][r] >= 0.f) << (16 * rb + 4 * (lane >> 4) + r);
    part |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(part), 16, kWave));
    part |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(part), 32, kWave));
    if (lane < 16 && tile0 + lane < n) signs[(tile0 + lane) * 4 + wv] = part;
    __syncthreads();  // the next pass rewrites rh
  }
}

// ----------------------------------------------------------------------------
// Rotate + recursive polar quantize (「谷歌 TurboQuant 深度拆解」 第二部分
// PolarQuant) for d = 64 and 256, the split encode's first step (d = 128 has
// the fused kernel above): one wavefront per vector, lane holding the E
// consecutive coordinates E*lane .. E*lane + E-1.  Level l (1..log2 d) pairs
// the two children of each node, whose coordinates differ in bit l-1: the
// lane's registers for l <= log2 E (each angle once), lanes lane ^
// 2^(l-1-log2 E) above (both lanes of a pair compute the same code from the
// same two radii).  Level 1: the angle of (y_2n, y_2n+1) in [0, 2π); above:
// that of the two child radii, in [0, π/2]; code = #{level boundaries below
// the angle}, found by sign tests (polar_code_l1, polar_code_up).  The rotation's butterflies run over the register bits, then the
// lane bits (the Sylvester matrix is a product over coordinate bits, so the
// order is free).  ŷ_j is the fp32 product, top-down from radius 1, of cos or
// sin (bit l-1 of j) of level l's centroid at node j >> l.  The codes reach
// their slots (level l: d - 2d/2^l + node; slot d-1 holds 0) through LDS and
// are packed as bit-planes like the per-coordinate codes; the residual y - ŷ,
// γ and ν leave as in encode_rq_kernel.
template <int E, typename T, int RM, int B>
__global__ __launch_bounds__(256) void encode_polar_rq_kernel(const T* __restrict__ x, int64_t n, DevParams P,
                                                              PolarParams PP, const float* __restrict__ Dsign,
                                                              uint32_t* __restrict__ codes, float* __restrict__ norm,
                                                              float* __restrict__ rnorm, float* __restrict__ rbuf,
                                                              float rscale) {
  static_assert(E == 1 || E == 2 || E == 4, "d = 64, 128 or 256");
  constexpr int d = E * kWave, NL = 1 << B;
  constexpr int RL = E == 1 ? 0 : (E == 2 ? 1 : 2);  // levels inside a lane's registers
  constexpr int LV = 6 + RL;                          // log2 d
  __shared__ float2 tab[LV][NL];    // (cos, sin) of every level's centroids
  __shared__ uint8_t pcode[4][d];   // each wave's codes by slot
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < LV * NL; e += blockDim.x)
    tab[e / NL][e % NL] = float2{PP.cosc[e / NL][e % NL], PP.sinc[e / NL][e % NL]};
  __syncthreads();
  const int64_t vec = static_cast<int64_t>(blockIdx.x) * 4 + wv;
  if (vec >= n) return;  // wave-uniform
  const T* xr = x + vec * d + E * lane;
  float v[E];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    v[e] = load_elem(xr, e);
    ss = fmaf(v[e], v[e], ss);
  }
  ss = wave_sum(ss);
  const float nu = sqrtf(ss);
  const float inv = nu > 0.f ? 1.0f / nu : 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] *= inv * Dsign[E * lane + e];
  fwht_regs<E>(v);
  fwht_lanes_dpp<E>(v, lane);
  float y[E];
#pragma unroll
  for (int e = 0; e < E; ++e) y[e] = v[e] * P.inv_sqrt_d;
  // register levels: node u of level l holds registers [u 2^l, (u+1) 2^l)
  int creg[RL > 0 ? RL : 1][E > 1 ? E / 2 : 1];
  float rad[E];
#pragma unroll
  for (int e = 0; e < E; ++e) rad[e] = y[e];
  // (rad: the coordinates, then from level 1 on the squared radii)
  static_for<RL>([&]<int k>() {  // level k + 1
    constexpr int W = 1 << k;     // child spacing in registers
#pragma unroll
    for (int u = 0; u < E / (2 * W); ++u) {
      const float a = rad[2 * W * u], b = rad[2 * W * u + W];
      if constexpr (k == 0) {
        creg[k][u] = polar_code_l1<NL>(PP, a, b);
        rad[2 * W * u] = fmaf(a, a, b * b);
      } else {
        creg[k][u] = polar_code_up<NL>(PP.bcs[k], a, b);
        rad[2 * W * u] = a + b;
      }
    }
  });
  // lane levels: the lane's node (squared) radius in rad[0]
  int clane[6];
  {
    float r = rad[0];
    static_for<6>([&]<int k>() {  // level RL + k + 1: partner lane ^ 2^k
      const bool hi = (lane >> k) & 1;
      const float o = __shfl_xor(r, 1 << k, kWave);
      const float a = hi ? o : r, b = hi ? r : o;  // the same on both lanes of the pair
      if constexpr (RL + k == 0) {
        clane[k] = polar_code_l1<NL>(PP, a, b);
        r = fmaf(a, a, b * b);
      } else {
        clane[k] = polar_code_up<NL>(PP.bcs[RL + k], a, b);
        r = a + b;
      }
    });
  }
  // each node's code from the member holding its first coordinate
  static_for<RL>([&]<int k>() {
    constexpr int l = k + 1, base = d - ((2 * d) >> l);
#pragma unroll
    for (int u = 0; u < E / (2 << k); ++u)
      pcode[wv][base + ((E * lane + (2 << k) * u) >> l)] = static_cast<uint8_t>(creg[k][u]);
  });
  static_for<6>([&]<int k>() {
    constexpr int l = RL + k + 1, base = d - ((2 * d) >> l);
    if (((E * lane) & ((1 << l) - 1)) == 0) pcode[wv][base + ((E * lane) >> l)] = static_cast<uint8_t>(clane[k]);
  });
  if (lane == 0) pcode[wv][d - 1] = 0;
  // ŷ top-down from radius 1: the lane levels, then the register levels
  float R = 1.f;
  static_for<6>([&]<int k>() {
    constexpr int kk = 5 - k, l = RL + kk + 1;  // level l = LV down to RL + 1
    const float2 f = tab[l - 1][clane[kk]];
    R *= (((E * lane) >> (l - 1)) & 1) ? f.y : f.x;
  });
  float rs = 0.f;
  float* rr = rbuf + vec * d;
  _Float16* rh = reinterpret_cast<_Float16*>(rbuf) + vec * 2 * d;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    float Re = R;
    static_for<RL>([&]<int k>() {
      constexpr int kk = RL - 1 - k, l = kk + 1;  // level l = RL down to 1
      const float2 f = tab[l - 1][creg[kk][e >> l]];
      Re *= ((e >> (l - 1)) & 1) ? f.y : f.x;
    });
    const float r = y[e] - Re;
    if constexpr (RM == kResF16) {
      const float rsc = r * rscale;
      const _Float16 hi = static_cast<_Float16>(rsc);
      rh[E * lane + e] = hi;
      rh[d + E * lane + e] = static_cast<_Float16>(rsc - static_cast<float>(hi));
    } else if constexpr (RM == kResF32) {
      rr[E * lane + e] = r;
    }
    rs = fmaf(r, r, rs);
  }
  if constexpr (RM != kResNone) rs = wave_sum(rs);
  __builtin_amdgcn_wave_barrier();  // the wave's code writes land before its reads
  int idx[E];
#pragma unroll
  for (int e = 0; e < E; ++e) idx[e] = pcode[wv][e * kWave + lane];
  pack_code_planes<E>(idx, lane, B, codes + vec * P.code_words, P.code_words);
  if (lane == 0) {
    norm[vec] = nu;
    if constexpr (RM != kResNone) rnorm[vec] = sqrtf(rs);
  }
}

// The QJL projection z = S r with its sign bits on the fp16 matrix cores
// (v_mfma_f32_16x16x32_f16), for d = m a multiple of 128: the split encode's
// second step.  S = S_hi + S_lo (fp16 pair, made at codec creation) and
// r·2^sc = r_hi + r_lo (written so by encode_rq_kernel; 2^sc keeps r_lo out
// of the fp16 subnormals and does not change a sign); z·2^sc = S_hi r_hi +
// S_hi r_lo + S_lo r_hi in fp32, about 2^-22 of |S_i||r| from the fp32 product.
//
// Block: 128 outputs x 128 vectors, 4 waves of 64 x 64 (4 x 4 tiles of 16),
// contraction in steps of 32 through double-buffered LDS (one barrier a step).
// The result tile holds output 4(L/16)+reg of vector L%16 in lane L, so sign
// words are ORed over the four lane groups.
namespace {
constexpr int kPjB = 128;   // outputs and vectors per block
constexpr int kPjK = 32;    // contraction step
constexpr int kPjRow = 32;  // LDS row stride in halfs: no padding, so two blocks fit a CU's LDS
// The 16-byte chunk c of LDS row r sits at chunk c ^ ((r >> 1) & 3): the eight
// rows one ds_read_b128 phase touches (same c) then land in eight distinct
// 4-bank groups, as the row stores do.
__device__ __forceinline__ int pj_col(int row, int col) { return ((col >> 3) ^ ((row >> 1) & 3)) << 3; }

__global__ __launch_bounds__(256) void sproj_mfma_kernel(const _Float16* __restrict__ r16, int64_t n, int d, int m,
                                                         const _Float16* __restrict__ S16,
                                                         uint32_t* __restrict__ signs) {
  __shared__ __attribute__((aligned(16))) _Float16 sa[2][2][kPjB][kPjRow];  // [buffer][hi, lo][output][k]
  __shared__ __attribute__((aligned(16))) _Float16 sb[2][2][kPjB][kPjRow];  // [buffer][hi, lo][vector][k]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv & 1, wn = wv >> 1;  // the wave's 64 outputs and 64 vectors
  // Blocks go to the 8 XCDs round-robin (block p to XCD p % 8).  The XCDs split
  // into go output groups x vparts vector parts: XCD x keeps the S rows of its
  // tpg output tiles (tpg·128·d·4 bytes hi+lo: 2.4 MB at d = 1536) in its L2
  // and streams every vparts-th vector tile, whose tpg output tiles run there
  // back to back, so the L2 also serves the tile's r after the first read.
  const int nob = m / kPjB;
  const int go = nob % 4 == 0 ? 4 : (nob % 2 == 0 ? 2 : 1), vparts = 8 / go, tpg = nob / go;
  const int64_t p = blockIdx.x, xcd = p % 8, kq = p / 8;
  const int ot = static_cast<int>((xcd % go) * tpg + kq % tpg);
  const int64_t vt = (xcd / go) + vparts * (kq / tpg);
  const int o0 = ot * kPjB;
  const int64_t v0 = vt * kPjB;
  if (v0 >= n) return;  // block-uniform: vector tiles past the end (the last round of each part)
  // staging: thread t moves row t/2, contraction elements 16(t%2)..+15 of both operands
  const int srow = tid >> 1, sk = 16 * (tid & 1);
  const _Float16* sp_hi = S16 + static_cast<int64_t>(o0 + srow) * d + sk;
  const _Float16* sp_lo = sp_hi + static_cast<int64_t>(m) * d;
  const _Float16* rp_hi = r16 + min(v0 + srow, n - 1) * 2 * d + sk;
  const _Float16* rp_lo = rp_hi + d;
  h8 ga[2][2], gb[2][2];  // S and r, hi/lo, two 8-half pieces each
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      ga[0][i] = *reinterpret_cast<const h8*>(sp_hi + k0 + 8 * i);
      ga[1][i] = *reinterpret_cast<const h8*>(sp_lo + k0 + 8 * i);
      gb[0][i] = *reinterpret_cast<const h8*>(rp_hi + k0 + 8 * i);
      gb[1][i] = *reinterpret_cast<const h8*>(rp_lo + k0 + 8 * i);
    }
  };
  auto sstore = [&](int b) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int hl = 0; hl < 2; ++hl) {
        *reinterpret_cast<h8*>(&sa[b][hl][srow][pj_col(srow, sk + 8 * i)]) = ga[hl][i];
        *reinterpret_cast<h8*>(&sb[b][hl][srow][pj_col(srow, sk + 8 * i)]) = gb[hl][i];
      }
  };
  f4v acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f4v{0.f, 0.f, 0.f, 0.f};
  const int nk = d / kPjK;
  gload(0);
  sstore(0);
  __syncthreads();
  const int fr = lane & 15, fk = 8 * (lane >> 4);  // fragment row and first contraction element
#pragma unroll 1
  for (int ks = 0; ks < nk; ++ks) {
    const int b = ks & 1;
    if (ks + 1 < nk) gload(kPjK * (ks + 1));
    h8 ah[4], al[4], bh[4], bl[4];
    const int fc = pj_col(fr, fk);  // rows 16i + fr: (row >> 1) & 3 depends on fr only
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ah[i] = *reinterpret_cast<const h8*>(&sa[b][0][64 * wm + 16 * i + fr][fc]);
      al[i] = *reinterpret_cast<const h8*>(&sa[b][1][64 * wm + 16 * i + fr][fc]);
      bh[i] = *reinterpret_cast<const h8*>(&sb[b][0][64 * wn + 16 * i + fr][fc]);
      bl[i] = *reinterpret_cast<const h8*>(&sb[b][1][64 * wn + 16 * i + fr][fc]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[i], bh[j], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[i], bl[j], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[i], bh[j], acc[i][j], 0, 0, 0);
      }
    if (ks + 1 < nk) sstore(b ^ 1);  // that buffer was last read before the previous barrier
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(acc[i][j]));  // matrix ops stay in wave-uniform flow
  // sign words: outputs o0 + 64wm + 16i + 4(lane/16) + reg of vector v0 + 64wn + 16j + lane%16
  const int g = lane >> 4, sw = m / 32;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t w0 = 0u, w1 = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t bit = static_cast<uint32_t>(acc[i][j][q] >= 0.f) << (16 * (i & 1) + 4 * g + q);
        if (i < 2) w0 |= bit; else w1 |= bit;
      }
    w0 |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(w0), 16, kWave));
    w0 |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(w0), 32, kWave));
    w1 |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(w1), 16, kWave));
    w1 |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(w1), 32, kWave));
    const int64_t vec = v0 + 64 * wn + 16 * j + fr;
    if (g < 2 && vec < n) signs[vec * sw + (o0 + 64 * wm) / 32 + g] = g == 0 ? w0 : w1;
  }
}
}  // namespace

bool sproj_mfma_eligible(const tq_codec_s* c) {
  const char* v = std::getenv("TQ_SPROJ_KERNEL");
  if (v && std::string(v) == "valu") return false;
  return c->dS16 != nullptr && c->prm.m == c->prm.d && c->prm.d % kPjB == 0;
}

bool encode_fused_eligible(const tq_codec_s* c) {
  if (c->polar) return c->prm.d == 128;  // d = 64 and 256: the split path with the polar quantizer
  const char* v = std::getenv("TQ_ENCODE_KERNEL");
  if (v && std::string(v) == "split") return false;
  if (!c->qjl) return c->prm.d == 128;  // MSE-only: no projection
  return c->prm.d == 128 && c->prm.m == 128 && c->dS16 != nullptr;
}

size_t encode_rows_ws_bytes(const tq_codec_s* c, int64_t n) {
  if (encode_fused_eligible(c)) return 0;  // the fused kernel keeps r on chip
  if (!c->qjl) return 0;                   // MSE-only: no residual to project
  return static_cast<size_t>(n) * c->prm.d * sizeof(float);
}

namespace {
template <typename T>
hipError_t encode_typed(const tq_codec_s* c, const T* x, int64_t n, tq_packed_t out, float* ws_r,
                        hipStream_t s) {
  const DevParams& P = c->prm;
  if (encode_fused_eligible(c)) {
    const dim3 grid(static_cast<unsigned>(ceil_div(n, 16 * kEncPasses)));
    auto go = [&]<int B>() -> hipError_t {
      if (c->polar)
        hipLaunchKernelGGL((encode_fused_kernel<T, B, true, true>), grid, dim3(256), 0, s, x, n, P, c->pol, c->dD,
                           c->dS16, out.codes, out.signs, out.norm, out.rnorm);
      else if (c->qjl)
        hipLaunchKernelGGL((encode_fused_kernel<T, B, false, true>), grid, dim3(256), 0, s, x, n, P, c->pol, c->dD,
                           c->dS16, out.codes, out.signs, out.norm, out.rnorm);
      else
        hipLaunchKernelGGL((encode_fused_kernel<T, B, false, false>), grid, dim3(256), 0, s, x, n, P, c->pol, c->dD,
                           static_cast<const _Float16*>(nullptr), out.codes, static_cast<uint32_t*>(nullptr),
                           out.norm, static_cast<float*>(nullptr));
      return hipGetLastError();
    };
    switch (P.b) {
      case 1: return go.template operator()<1>();
      case 2: return go.template operator()<2>();
      case 3: return go.template operator()<3>();
    }
    return hipErrorInvalidValue;
  }
  const bool mfma = sproj_mfma_eligible(c);
  // 2^sc with sc = ceil(log2 sqrt(d)) + 4: r·2^sc is O(1) per coordinate and below 2^11
  const int sc = static_cast<int>(std::ceil(std::log2(std::sqrt(static_cast<double>(P.d))))) + 4;
  const dim3 grid_rq(static_cast<unsigned>(ceil_div(n, 4)));
  if (c->polar) {  // d = 64 or 256 (d = m, the QJL stage always present)
    auto prun = [&]<int E, int B>() -> hipError_t {
      if (mfma)
        hipLaunchKernelGGL((encode_polar_rq_kernel<E, T, kResF16, B>), grid_rq, dim3(256), 0, s, x, n, P, c->pol,
                           c->dD, out.codes, out.norm, out.rnorm, ws_r, std::ldexp(1.0f, sc));
      else
        hipLaunchKernelGGL((encode_polar_rq_kernel<E, T, kResF32, B>), grid_rq, dim3(256), 0, s, x, n, P, c->pol,
                           c->dD, out.codes, out.norm, out.rnorm, ws_r, 1.0f);
      return hipGetLastError();
    };
    auto pb = [&]<int E>() -> hipError_t {
      switch (P.b) {
        case 1: return prun.template operator()<E, 1>();
        case 2: return prun.template operator()<E, 2>();
        case 3: return prun.template operator()<E, 3>();
      }
      return hipErrorInvalidValue;
    };
    hipError_t e = P.d == 64 ? pb.template operator()<1>() : P.d == 256 ? pb.template operator()<4>()
                                                                       : hipErrorInvalidValue;
    if (e != hipSuccess) return e;
  }
  auto run = [&]<int E>() -> hipError_t {
    if (!c->qjl)
      hipLaunchKernelGGL((encode_rq_kernel<E, T, kResNone>), grid_rq, dim3(256), 0, s, x, n, P, c->dD, out.codes,
                         out.norm, static_cast<float*>(nullptr), static_cast<float*>(nullptr), 1.0f);
    else if (mfma)
      hipLaunchKernelGGL((encode_rq_kernel<E, T, kResF16>), grid_rq, dim3(256), 0, s, x, n, P, c->dD, out.codes,
                         out.norm, out.rnorm, ws_r, std::ldexp(1.0f, sc));
    else
      hipLaunchKernelGGL((encode_rq_kernel<E, T, kResF32>), grid_rq, dim3(256), 0, s, x, n, P, c->dD, out.codes,
                         out.norm, out.rnorm, ws_r, 1.0f);
    return hipGetLastError();
  };
  hipError_t e = c->polar ? hipSuccess : dispatch_E(P.d, run);
  if (e != hipSuccess || !c->qjl) return e;
  if (mfma) {
    const _Float16* r16 = reinterpret_cast<const _Float16*>(ws_r);
    const int64_t per_launch = static_cast<int64_t>(1) << 24;  // vectors per launch (grid size well inside 2^32)
    for (int64_t v0 = 0; v0 < n; v0 += per_launch) {
      const int64_t nv = std::min(per_launch, n - v0);
      // one-dimensional grid: 8 XCDs x tpg output tiles x the vector tiles of each vector part
      const int nob = P.m / kPjB;
      const int go = nob % 4 == 0 ? 4 : (nob % 2 == 0 ? 2 : 1);
      const dim3 grid(static_cast<unsigned>(8 * (nob / go) * ceil_div(ceil_div(nv, kPjB), 8 / go)));
      hipLaunchKernelGGL(sproj_mfma_kernel, grid, dim3(256), 0, s, r16 + v0 * 2 * P.d, nv, P.d, P.m, c->dS16,
                         out.signs + v0 * P.sign_words);
      const hipError_t e2 = hipGetLastError();
      if (e2 != hipSuccess) return e2;
    }
    return hipSuccess;
  }
  dim3 grid(static_cast<unsigned>(ceil_div(n, kTileV)), P.m / kTileI);
  hipLaunchKernelGGL((sproj_kernel<true>), grid, dim3(256), 0, s, ws_r, n, P.d, P.m, c->dS,
                     static_cast<float*>(nullptr), out.signs);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_encode_rows(const tq_codec_s* c, const void* x, tq_dtype_t dt, int64_t n, tq_packed_t out,
                              float* ws_r, hipStream_t s) {
  switch (dt) {
    case TQ_F32: return encode_typed(c, static_cast<const float*>(x), n, out, ws_r, s);
    case TQ_BF16: return encode_typed(c, static_cast<const __hip_bfloat16*>(x), n, out, ws_r, s);
    case TQ_F16: return encode_typed(c, static_cast<const __half*>(x), n, out, ws_r, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_qprep(const tq_codec_s* c, const void* q, tq_dtype_t dt, int64_t n, float* qrot,
                        float* proj, hipStream_t s) {
  const DevParams& P = c->prm;
  auto rot = [&]<typename T>(const T* x) {
    auto run = [&]<int E>() -> hipError_t {
      hipLaunchKernelGGL((rotate_kernel<E, T>), dim3(static_cast<unsigned>(ceil_div(n, 4))), dim3(256), 0, s, x,
                         n, P.inv_sqrt_d, c->dD, qrot);
      return hipGetLastError();
    };
    return dispatch_E(P.d, run);
  };
  hipError_t e = hipErrorInvalidValue;
  switch (dt) {
    case TQ_F32: e = rot(static_cast<const float*>(q)); break;
    case TQ_BF16: e = rot(static_cast<const __hip_bfloat16*>(q)); break;
    case TQ_F16: e = rot(static_cast<const __half*>(q)); break;
  }
  if (e != hipSuccess) return e;
  dim3 grid(static_cast<unsigned>(ceil_div(n, kTileV)), P.m / kTileI);
  hipLaunchKernelGGL((sproj_kernel<false>), grid, dim3(256), 0, s, qrot, n, P.d, P.m, c->dS, proj,
                     static_cast<uint32_t*>(nullptr));
  return hipGetLastError();
}

}  // namespace tq

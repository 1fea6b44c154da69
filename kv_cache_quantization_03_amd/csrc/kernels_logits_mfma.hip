// Attention logits on the CDNA4 matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4).
//
// The estimator (「谷歌 TurboQuant 深度拆解」 第二部分) is a dense contraction of
// every query of a KV-head group with every compressed key of that head:
//   ℓ = ν (Σ_j q'_j c[idx_j] + √(π/2)/m · γ · Σ_i p_i τ_i).
// Decoding each key to floats costs several VALU instructions per coordinate,
// more than the memory time allows at 4 query heads per key, so the kernel
// never decodes: the packed bits themselves become FP4 (e2m1) matrix operands.
//
// * Bit-plane form of the codebook.  A symmetric codebook is, over the bits of
//   idx, c(idx) = bias + Σ_P coef_P · plane_P(idx), with planes the b bits
//   (and, for b = 3, their parity).  So the MSE sum is Σ_P coef_P ⟨plane_P, q'⟩
//   plus a query constant, and the QJL sum is 2⟨bits, p⟩ - Σ p.
// * FP4 without unpacking.  In a 32-bit word w holding 32 plane bits, the
//   nibbles of (w & 0x11111111 << v) are FP4 numbers 0 or 2^(v-1) for v = 0, 1, 2,
//   and (w & 0x88888888) | 0x22222222 gives ±1.  Four AND/AND-OR instructions turn
//   one word into the 32-element FP4 B operand of one lane; the query side
//   divides by the nibble's value and absorbs the ±1 offset into a constant.
// * FP32-grade query operand.  Each query value is split into four fp8 (e4m3)
//   limbs R0 + R1/16 + R2/256 + R3/4096 (after a power-of-two scale), and the 16
//   rows of the A operand are (4 query vectors) x (4 limbs).  The limb sum is
//   taken in fp32 after the MFMA, so the contraction is exact up to about 2^-16
//   of the largest query element.
//
// Lane layout of the instruction (measured on gfx950 with a probe): contraction
// index k of the fp4 B operand sits in lane group k/32 (lanes 16(k/32)..+15,
// one per column), nibble k%32; of the fp8 A operand in lane group (k%64)/16,
// byte k%16 + 16(k/64).  The 16x16 result: lane L, register r = row 4(L/16)+r,
// column L%16.  Here column = key L%16 and row 4h+r = (query vector h, limb r),
// so each lane ends with all four limbs of one (key, query vector).  Lane L
// loads word L/16 of each plane of key L%16, and that dword is its B operand
// after four AND/AND-OR instructions.  The A operands (queries) stay in VGPRs.
#include <cstdlib>
#include <string>

#include "kernels_common.h"

namespace tq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));  // 16-byte record piece (a plain vector, kept in VGPRs)

namespace {

constexpr int kOpBytes = 64 * 32;  // one K-block of A for one M-tile: 64 lanes x 32 bytes
// Per M-tile after the operands: float[4][4] (scale_m, scale_q, bias_m, bias_q)
// per query vector, then int32[4] output rows ((b*Hq + h)*nq + qi, or -1 for
// a padding slot), padded to 128 bytes.
constexpr int kConstBytes = 128;
constexpr int kKeysPerTile = 16;

__device__ __forceinline__ v4f mfma_fp8_fp4(const v8i& a, const v8i& b, const v4f& c) {
  // cbsz = 0: A is fp8 e4m3; blgp = 4: B is fp4 e2m1; E8M0 scales 127 = 2^0.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, 127, 0, 127);
}

__device__ __forceinline__ v8i fp4_operand(uint32_t w) {
  v8i b;
  b[0] = static_cast<int>(w & 0x11111111u);                 // 0 or 0.5
  b[1] = static_cast<int>(w & 0x22222222u);                 // 0 or 1
  b[2] = static_cast<int>(w & 0x44444444u);                 // 0 or 2
  b[3] = static_cast<int>((w & 0x88888888u) | 0x22222222u);  // +1 (bit 0) or -1 (bit 1)
  b[4] = b[5] = b[6] = b[7] = 0;
  return b;
}

// fp32 -> fp8 (e4m3, hardware round to nearest even) and back.
__device__ __forceinline__ uint32_t to_fp8(float x) {
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.f, 0, false)) & 0xFFu;
}
__device__ __forceinline__ float from_fp8(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(byte), 0);
}

// Power-of-two scale 2^E with sigma * 2^E < 256 (E = 8 - exponent of sigma).
__device__ __forceinline__ int limb_exponent(float sigma) {
  if (!(sigma > 0.f)) return 0;
  int k;
  (void)frexpf(sigma, &k);
  return 8 - k;
}

}  // namespace

// ----------------------------------------------------------------------------
// Query prep: one block (4 waves) per (batch*kv_head, M-tile of 4 query vectors).
// q' = H (D ⊙ q)/√d, p = S q', then the fp8 limb operands and constants.
// ----------------------------------------------------------------------------
template <int E, typename T>
__global__ __launch_bounds__(256) void attn_prep_mfma_kernel(const T* __restrict__ q, DevParams P,
                                                             const float* __restrict__ Dsign,
                                                             const float* __restrict__ Mt, int Hq, int nq, int G,
                                                             int nkv, int n_mt, uint8_t* __restrict__ prep) {
  constexpr int d = E * kWave;
  constexpr int W = d / 32;
  constexpr int TPO = 256 / d >= 1 ? 256 / d : 1;  // threads per output of p (2 for d=128, 1 for d=256)
  constexpr int JPT = d / TPO;                      // inputs per thread
  constexpr int CH = JPT < 64 ? JPT : 64;           // loads per batch
  __shared__ float qs[4][d];  // q' = R q
  __shared__ float qr[4][d];  // q
  __shared__ float ps[4][d];  // p = S R q
  __shared__ float mx[4][2];
  __shared__ __attribute__((aligned(16))) uint8_t opst[5 * (d / 128) * kOpBytes];  // A operands being built
  const int blk = blockIdx.x;
  const int mt = blk % n_mt, bk = blk / n_mt;
  const int b = bk / nkv, kh = bk % nkv;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int Gq = nq * G;
  // The first batch of M = S R (transposed) loads goes out before anything else:
  // p = M q needs no rotated query, so it overlaps the query load and rotation.
  const int pi = threadIdx.x % d, part = threadIdx.x / d;
  float mv[CH];
#pragma unroll
  for (int u = 0; u < CH; ++u) mv[u] = Mt[static_cast<int64_t>(part * JPT + u) * d + pi];
  {
    const int qv = mt * 4 + wv;
    float v[E];
    if (qv < Gq) {
      const int qi = qv / G, g = qv % G;
      const int64_t row = (static_cast<int64_t>(b) * nq + qi) * Hq + kh * G + g;
#pragma unroll
      for (int e = 0; e < E; ++e) v[e] = load_elem(q + row * d, e * kWave + lane);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) v[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      qr[wv][e * kWave + lane] = v[e];
      v[e] *= Dsign[e * kWave + lane];
    }
    hadamard_wave<E>(v, lane);
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      v[e] *= P.inv_sqrt_d;
      qs[wv][e * kWave + lane] = v[e];
      amax = fmaxf(amax, fabsf(v[e]));
    }
    amax = wave_max(amax);
    if (lane == 0) mx[wv][0] = amax;
  }
  __syncthreads();
  {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j0 = part * JPT; j0 < (part + 1) * JPT; j0 += CH) {
      if (j0 != part * JPT) {
#pragma unroll
        for (int u = 0; u < CH; ++u) mv[u] = Mt[static_cast<int64_t>(j0 + u) * d + pi];
      }
#pragma unroll
      for (int u = 0; u < CH; ++u) {
#pragma unroll
        for (int vq = 0; vq < 4; ++vq) acc[vq] = fmaf(mv[u], qr[vq][j0 + u], acc[vq]);
      }
    }
    if (TPO == 1) {
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) ps[vq][pi] = acc[vq];
    } else {
      // two partial sums per output: the upper half parks its sums in ps, the lower adds them
      if (part == 1) {
#pragma unroll
        for (int vq = 0; vq < 4; ++vq) ps[vq][pi] = acc[vq];
      }
      __syncthreads();
      if (part == 0) {
#pragma unroll
        for (int vq = 0; vq < 4; ++vq) ps[vq][pi] += acc[vq];
      }
    }
  }
  __syncthreads();
  {
    float amax = 0.f;
    for (int j = lane; j < d; j += kWave) amax = fmaxf(amax, fabsf(ps[wv][j]));
    amax = wave_max(amax);
    if (lane == 0) mx[wv][1] = amax;
  }
  __syncthreads();

  const int NP = P.n_planes;
  const int NKB = (NP + 1) * (W / 4);
  float cmax = 0.f, csum = 0.f;
  for (int k = 0; k < NP; ++k) {
    cmax = fmaxf(cmax, fabsf(P.plane_coef[k]));
    csum += P.plane_coef[k];
  }
  uint8_t* base = prep + (static_cast<int64_t>(bk) * n_mt + mt) * (NKB * kOpBytes + kConstBytes);
  // Operands.  Every (query vector hl, K-block kbi, coordinate j) value is cut
  // into its four fp8 limbs once, and each limb byte is placed at its slot of
  // the A layout in LDS: limb l of vector hl is row 4hl+l; coordinate j of
  // word wi (0..3 in the block) at bit 4i+v is contraction index
  // kk = 32wi + 8v + i (the B nibble order), held by A lane group (kk%64)/16,
  // byte kk%16 + 16(kk/64) (A byte order measured on gfx950).
  for (int e = threadIdx.x; e < 4 * NKB * 128; e += 256) {
    const int jl = e & 127, kbi = (e >> 7) % NKB, hl = (e >> 7) / NKB;
    const int plane = kbi / (W / 4), kb = kbi % (W / 4);
    const bool qjl = plane >= NP;
    const float kappa = qjl ? 2.f : P.plane_coef[plane];
    const float sigma = qjl ? 4.f * mx[hl][1] : 2.f * cmax * mx[hl][0];
    const int wi = jl >> 5, rr = jl & 31, i = rr >> 2, v = rr & 3;
    const float inv_val = v == 0 ? 2.f : (v == 1 ? 1.f : (v == 2 ? 0.5f : -0.5f));
    const float* src = qjl ? ps[hl] : qs[hl];
    float R = ldexpf(kappa * src[128 * kb + jl] * inv_val, limb_exponent(sigma));
    const int kk = 32 * wi + 8 * v + i;
    const int grp = (kk & 63) >> 4, byte = (kk & 15) + 16 * (kk >> 6);
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      const uint32_t bl = to_fp8(R);
      opst[kbi * kOpBytes + (16 * grp + 4 * hl + l) * 32 + byte] = static_cast<uint8_t>(bl);
      R = (R - from_fp8(bl)) * 16.f;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < NKB * kOpBytes / 16; e += 256)
    reinterpret_cast<uint4*>(base)[e] = reinterpret_cast<const uint4*>(opst)[e];
  // constants per query vector of the tile: wave hl reduces vector hl
  {
    const int hl = wv;
    float sall = 0.f, s3 = 0.f, pall = 0.f, p3 = 0.f;
    for (int j = lane; j < d; j += kWave) {
      const float a = qs[hl][j], pj = ps[hl][j];
      sall += a;
      pall += pj;
      if ((j & 3) == 3) {
        s3 += a;
        p3 += pj;
      }
    }
    sall = wave_sum(sall);
    s3 = wave_sum(s3);
    pall = wave_sum(pall);
    p3 = wave_sum(p3);
    if (lane == 0) {
      const int qv = mt * 4 + hl;
      int orow = -1;
      if (qv < Gq) orow = (b * Hq + kh * G + qv % G) * nq + qv / G;
      reinterpret_cast<int*>(base + NKB * kOpBytes + 64)[hl] = orow;
      float* cst = reinterpret_cast<float*>(base + NKB * kOpBytes);
      cst[hl * 4 + 0] = ldexpf(1.f, -limb_exponent(2.f * cmax * mx[hl][0]));
      cst[hl * 4 + 1] = ldexpf(1.f, -limb_exponent(4.f * mx[hl][1]));
      // slots with j%4 = 3 hold -x/2 against the +-1 nibble: add the x/2 back
      cst[hl * 4 + 2] = P.plane_bias * sall + 0.5f * csum * s3;
      cst[hl * 4 + 3] = -pall + p3;
    }
  }
}

// ----------------------------------------------------------------------------
// Records and scoring, shared by the two logits kernels.
//
// Each wave scores 64 consecutive keys (4 tiles of 16) of one (batch, kv head).
// Memory: the wave's records are contiguous in each array (64 rows), so they
// are read with fully coalesced 16-byte loads (one instruction covers 1 KB),
// staged in the wave's own LDS slice, and read back in the MFMA lane layout
// (lane L: word L/16 of key L%16 of a tile).  Rows are padded by 4 words in
// LDS to spread the reads over the banks.  The wave's 64 norms ν and γ are
// loaded one per lane and moved to the owning lane with a cross-lane read.
// Reading the words in the MFMA layout straight from global memory touches
// every cache line from several instructions and costs ~1.7x the time.
// ----------------------------------------------------------------------------
constexpr int kKeysPerWave = 64;

template <int NP, int WB>
struct RecLayout {
  static constexpr int W = 4 * WB;            // words per plane (d/32)
  static constexpr int NB = NP > 3 ? 3 : NP;  // stored planes (the parity plane is computed)
  static constexpr int CW = NB * W;           // code words per key
  static constexpr int SW = W;                // sign words per key
  static constexpr int CS = CW + 4, SS = SW + 4;  // LDS row strides (words)
  static constexpr int NKB = (NP + 1) * WB;   // K-blocks: MSE planes x word blocks, then QJL word blocks
};

// Issue the wave's record loads (pointers at the wave's first row): 16 B per
// lane per instruction; rows past the end of the context re-read the last
// valid row (branch-free, always in bounds) and are never stored.
// cv, sv: the wave's code and sign words as 16-byte pieces; nu, ga: ν and γ of
// key `lane`.
template <int NP, int WB, int NC, int NS>
__device__ __forceinline__ void load_wave_records(v4u (&cv)[NC], v4u (&sv)[NS], float& nu, float& ga,
                                                  const uint32_t* __restrict__ codes,
                                                  const uint32_t* __restrict__ signs,
                                                  const float* __restrict__ norm,
                                                  const float* __restrict__ rnorm, int nvalid, int lane) {
  using L = RecLayout<NP, WB>;
  static_assert(NC == L::CW / 4 && NS == L::SW / 4, "record pieces");
#pragma unroll
  for (int i = 0; i < L::CW / 4; ++i) {
    const int w = 4 * (i * 64 + lane);
    const int kk = min(w / L::CW, nvalid - 1);
    cv[i] = reinterpret_cast<const v4u*>(codes)[(kk * L::CW + w % L::CW) / 4];
  }
#pragma unroll
  for (int i = 0; i < L::SW / 4; ++i) {
    const int w = 4 * (i * 64 + lane);
    const int kk = min(w / L::SW, nvalid - 1);
    sv[i] = reinterpret_cast<const v4u*>(signs)[(kk * L::SW + w % L::SW) / 4];
  }
  const int ln = min(lane, nvalid - 1);
  nu = norm[ln];
  ga = rnorm[ln];
}

// Scatter the records into the wave's LDS slice, then score the 64 keys
// against NMT M-tiles: a = A operands, cst = (scale_m, scale_q, bias_m,
// bias_q) of query vector `lane/16` per tile, out = its logits row at the
// wave's first key (nullptr: padding slot, not stored).
template <int NP, int WB, int NMT, int NC, int NS, int NKB>
__device__ __forceinline__ void score_wave(const v4u (&cv)[NC], const v4u (&sv)[NS], float nu_l, float ga_l,
                                           uint32_t* __restrict__ s_codes,
                                           uint32_t* __restrict__ s_signs, const v8i (&a)[NMT][NKB],
                                           const float4 (&cst)[NMT], float* const (&out)[NMT], int nvalid,
                                           float kappa, int lane) {
  using L = RecLayout<NP, WB>;
  const int g = lane >> 4, kl = lane & 15;
#pragma unroll
  for (int i = 0; i < L::CW / 4; ++i) {
    const int w = 4 * (i * 64 + lane);
    *reinterpret_cast<v4u*>(&s_codes[(w / L::CW) * L::CS + w % L::CW]) = cv[i];
  }
#pragma unroll
  for (int i = 0; i < L::SW / 4; ++i) {
    const int w = 4 * (i * 64 + lane);
    *reinterpret_cast<v4u*>(&s_signs[(w / L::SW) * L::SS + w % L::SW]) = sv[i];
  }
  // the wave reads back only what it wrote: LDS ops of one wave complete in
  // order; the barrier keeps the compiler from moving the reads above the writes
  __builtin_amdgcn_wave_barrier();

#pragma unroll
  for (int t = 0; t < kKeysPerWave / kKeysPerTile; ++t) {
    const int kk = t * kKeysPerTile + kl;
    const uint32_t* crow = &s_codes[kk * L::CS];
    const uint32_t* srow = &s_signs[kk * L::SS];
    const float nu = __shfl(nu_l, kk, kWave), ga = __shfl(ga_l, kk, kWave);
    v4f acc_m[NMT], acc_q[NMT];
#pragma unroll
    for (int i = 0; i < NMT; ++i) {
      acc_m[i] = v4f{0.f, 0.f, 0.f, 0.f};
      acc_q[i] = v4f{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int wb = 0; wb < WB; ++wb) {
      uint32_t pw[L::NB];
#pragma unroll
      for (int p = 0; p < L::NB; ++p) pw[p] = crow[p * L::W + 4 * wb + g];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        constexpr int NB = L::NB;
        const uint32_t w = (p < NB) ? pw[p < NB ? p : 0] : (pw[0] ^ pw[NB > 1 ? 1 : 0] ^ pw[NB > 2 ? 2 : 0]);
        const v8i bop = fp4_operand(w);
#pragma unroll
        for (int i = 0; i < NMT; ++i) acc_m[i] = mfma_fp8_fp4(a[i][p * WB + wb], bop, acc_m[i]);
      }
      const v8i bop = fp4_operand(srow[4 * wb + g]);
#pragma unroll
      for (int i = 0; i < NMT; ++i) acc_q[i] = mfma_fp8_fp4(a[i][NP * WB + wb], bop, acc_q[i]);
    }
    // An MFMA reads operands from all 64 lanes, so it must run with the full
    // EXEC mask: pin every accumulator here, in wave-uniform control flow, so
    // the compiler cannot sink the matrix ops into the lane-divergent stores.
#pragma unroll
    for (int i = 0; i < NMT; ++i) asm volatile("" : "+v"(acc_m[i]), "+v"(acc_q[i]));
#pragma unroll
    for (int i = 0; i < NMT; ++i) {
      const float mse = cst[i].x * (acc_m[i][0] + acc_m[i][1] * 0.0625f + acc_m[i][2] * 0.00390625f +
                                    acc_m[i][3] * 0.000244140625f) + cst[i].z;
      const float qj = cst[i].y * (acc_q[i][0] + acc_q[i][1] * 0.0625f + acc_q[i][2] * 0.00390625f +
                                   acc_q[i][3] * 0.000244140625f) + cst[i].w;
      if (out[i] != nullptr && kk < nvalid) out[i][kk] = nu * (mse + kappa * ga * qj);
    }
  }
}

// ----------------------------------------------------------------------------
// Logits from prepared query operands: each wave scores its 64 keys against
// NMT M-tiles of its query group, operands and constants read from `prep`.
// ----------------------------------------------------------------------------
template <int NP, int WB, int NMT, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void logits_mfma_kernel(const uint8_t* __restrict__ prep, int n_mt, int ctx,
                                                                 const uint32_t* __restrict__ codes,
                                                                 const uint32_t* __restrict__ signs,
                                                                 const float* __restrict__ norm,
                                                                 const float* __restrict__ rnorm, float kappa,
                                                                 float* __restrict__ logits) {
  using L = RecLayout<NP, WB>;
  constexpr int NKB = L::NKB;
  constexpr int MT_BYTES = NKB * kOpBytes + kConstBytes;
  __shared__ uint32_t s_codes[WAVES][kKeysPerWave * L::CS];
  __shared__ uint32_t s_signs[WAVES][kKeysPerWave * L::SS];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int bk = blockIdx.y;
  const int key0 = (blockIdx.x * WAVES + wv) * kKeysPerWave;
  if (key0 >= ctx) return;  // wave-uniform
  const int nvalid = min(kKeysPerWave, ctx - key0);
  const int64_t row0 = static_cast<int64_t>(bk) * ctx + key0;
  v4u cv[L::CW / 4], sv[L::SW / 4];
  float nu_l, ga_l;
  load_wave_records<NP, WB>(cv, sv, nu_l, ga_l, codes + row0 * L::CW, signs + row0 * L::SW, norm + row0,
                            rnorm + row0, nvalid, lane);

  // ---- query operands, constants and output rows (from L2)
  const int mt0 = blockIdx.z * NMT;
  v8i a[NMT][NKB];
  float4 cst[NMT];
  float* out[NMT];
#pragma unroll
  for (int i = 0; i < NMT; ++i) {
    const int mt = min(mt0 + i, n_mt - 1);
    const uint8_t* base = prep + (static_cast<int64_t>(bk) * n_mt + mt) * MT_BYTES;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const uint4* src = reinterpret_cast<const uint4*>(base + kb * kOpBytes + lane * 32);
      const uint4 x = src[0], y = src[1];
      a[i][kb][0] = x.x; a[i][kb][1] = x.y; a[i][kb][2] = x.z; a[i][kb][3] = x.w;
      a[i][kb][4] = y.x; a[i][kb][5] = y.y; a[i][kb][6] = y.z; a[i][kb][7] = y.w;
    }
    cst[i] = reinterpret_cast<const float4*>(base + NKB * kOpBytes)[g];
    const int orow = reinterpret_cast<const int*>(base + NKB * kOpBytes + 64)[g];
    out[i] = (mt0 + i < n_mt && orow >= 0) ? logits + static_cast<int64_t>(orow) * ctx + key0 : nullptr;
  }
  score_wave<NP, WB, NMT>(cv, sv, nu_l, ga_l, s_codes[wv], s_signs[wv], a, cst, out, nvalid, kappa, lane);
}

// Wave-wide sum / max of non-negative values through DPP (no LDS round
// trips): butterflies inside quads, half-row and row mirrors, then the
// row broadcasts; the total lands in lane 63 and is read back as a scalar.
#define TQ_DPP_F(x, ctrl, rmask) \
  __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), (ctrl), (rmask), 0xF, false))
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += TQ_DPP_F(v, 0xB1, 0xF);   // quad_perm [1,0,3,2]
  v += TQ_DPP_F(v, 0x4E, 0xF);   // quad_perm [2,3,0,1]
  v += TQ_DPP_F(v, 0x141, 0xF);  // row_half_mirror
  v += TQ_DPP_F(v, 0x140, 0xF);  // row_mirror
  v += TQ_DPP_F(v, 0x142, 0xA);  // row_bcast:15 into rows 1, 3
  v += TQ_DPP_F(v, 0x143, 0xC);  // row_bcast:31 into rows 2, 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_max_dpp(float v) {  // v >= 0
  v = fmaxf(v, TQ_DPP_F(v, 0xB1, 0xF));
  v = fmaxf(v, TQ_DPP_F(v, 0x4E, 0xF));
  v = fmaxf(v, TQ_DPP_F(v, 0x141, 0xF));
  v = fmaxf(v, TQ_DPP_F(v, 0x140, 0xF));
  v = fmaxf(v, TQ_DPP_F(v, 0x142, 0xA));
  v = fmaxf(v, TQ_DPP_F(v, 0x143, 0xC));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
#undef TQ_DPP_F

// ----------------------------------------------------------------------------
// Fused logits (d = 128, one M-tile of 4 query vectors per KV head): every
// block rebuilds the query operands of its (batch, kv head) in LDS while its
// records are in flight, so a decode step is one launch.
//
// Because the fp8 limbs are floating point, the power-of-two operand scales
// need only upper bounds of the operands, not their maxima: with
// β = √d max_k |q_k| >= ||q||, |q'_j| <= β (R is orthogonal) and
// |p_i| <= max_i ||M_i|| β (Cauchy-Schwarz), so one max over the raw query
// replaces the reductions over q' and p.  The two constant
// sums of q' come from the Hadamard matrix's row sums: Σ_j q'_j = √d D_0 q_0
// and Σ_{j≡3 mod 4} q'_j = (√d/4)(D_0q_0 - D_1q_1 - D_2q_2 + D_3q_3).  Each
// thread then cuts the limbs of its own (vector, coordinate).
// ----------------------------------------------------------------------------
template <int NP, int WAVES, typename T>
__global__ __launch_bounds__(WAVES * 64) void logits_fused_kernel(
    const T* q, DevParams P, const float* Dsign, const float* Mt, int Hq,
    int nq, int G, int nkv, int ctx, const uint32_t* __restrict__ codes, const uint32_t* __restrict__ signs,
    const float* __restrict__ norm, const float* __restrict__ rnorm, float* __restrict__ logits) {
  using L = RecLayout<NP, 1>;
  constexpr int d = 128, NT = WAVES * 64, PARTS = NT / d, JP = d / PARTS, NKB = L::NKB;
  static_assert(NT >= 4 * d, "one thread per (query vector, coordinate) of the tile");
  __shared__ uint32_t s_codes[WAVES][kKeysPerWave * L::CS];
  __shared__ uint32_t s_signs[WAVES][kKeysPerWave * L::SS];
  __shared__ float qr[4][d];         // q
  __shared__ float qs[4][d];         // D ⊙ q, then q' = R q
  __shared__ float pp[PARTS][4][d];  // partial sums of p = M q over slices of j
  __shared__ float qmx[4][2];        // max |q_k| per vector, per half
  __shared__ float dq4[4][4];        // (D ⊙ q)_0..3 per vector
  __shared__ float psum[4][2][2];    // Σ p and Σ_{i%4=3} p per vector, per half
  __shared__ __attribute__((aligned(16))) uint8_t opst[NKB * kOpBytes];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bk = blockIdx.y, mt = blockIdx.z;
  const int b = bk / nkv, kh = bk % nkv, Gq = nq * G;
  const int key0 = (blockIdx.x * WAVES + wv) * kKeysPerWave;
  const bool active = key0 < ctx;  // wave-uniform; idle waves still help with the operands
  const int nvalid = active ? min(kKeysPerWave, ctx - key0) : 0;

  // Operand-side loads go out first, all unconditional.  Loads complete in
  // issue order as far as the wait counter is concerned, so the operand math
  // below waits for these while the record loads issued after them are still
  // in flight.  p_i = Σ_j M_ij q_j: thread (part, i) sums its slice of j for
  // all four vectors.
  const int pi = tid & (d - 1), part = tid / d;
  float mv[JP];
#pragma unroll
  for (int u = 0; u < JP; ++u) mv[u] = Mt[(part * JP + u) * d + pi];
  // the thread's (vector, coordinate) of the tile; threads past 4d repeat vector 3
  const int lv = min(tid / d, 3), qv = mt * 4 + lv, qc = min(qv, Gq - 1);
  const float qraw =
      load_elem(q + ((static_cast<int64_t>(b) * nq + qc / G) * Hq + kh * G + qc % G) * d, pi);
  const float dx = Dsign[pi];
  // The vector memory path returns data in request order, so an operand load
  // queued behind record loads (HBM misses) would wait for them: every wave's
  // operand loads are queued before any wave issues its records.  The barrier
  // waits for no data; q, D and M are not declared __restrict__ so that their
  // loads are not sunk below it.
  __syncthreads();
  // Records: every wave loads (an idle wave re-reads the last key and never
  // uses it), so no branch sits around the loads.
  v4u cv[L::CW / 4], sv[L::SW / 4];
  float nu_l, ga_l;
  {
    const int k0 = active ? key0 : ctx - 1;
    const int64_t row0 = static_cast<int64_t>(bk) * ctx + k0;
    load_wave_records<NP, 1>(cv, sv, nu_l, ga_l, codes + row0 * L::CW, signs + row0 * L::SW, norm + row0,
                             rnorm + row0, active ? nvalid : 1, lane);
  }
  const float qx = qv < Gq ? qraw : 0.f;
  if (NT == 4 * d || tid < 4 * d) {
    qr[lv][pi] = qx;
    qs[lv][pi] = qx * dx;
    if (pi < 4) dq4[lv][pi] = qx * dx;
    const float mx = wave_max_dpp(fabsf(qx));
    if (lane == 0) qmx[lv][(tid >> 6) & 1] = mx;
  }
  __syncthreads();

  // q' = H (D ⊙ q)/√d in place by waves 0..3 (one vector each); p partial sums by all
  if (wv < 4) {
    float v[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) v[e] = qs[wv][e * kWave + lane];
    hadamard_wave<2>(v, lane);
#pragma unroll
    for (int e = 0; e < 2; ++e) qs[wv][e * kWave + lane] = v[e] * P.inv_sqrt_d;
  }
  {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < JP; ++u) {
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) acc[vq] = fmaf(mv[u], qr[vq][part * JP + u], acc[vq]);
    }
#pragma unroll
    for (int vq = 0; vq < 4; ++vq) pp[part][vq][pi] = acc[vq];
  }
  float cmax = 0.f, csum = 0.f;
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    cmax = fmaxf(cmax, fabsf(P.plane_coef[k]));
    csum += P.plane_coef[k];
  }
  __syncthreads();

  // Limbs of the thread's own (vector lv, coordinate pi): the MSE planes from
  // q'_pi and the QJL block from p_pi.  Coordinate j of K-block kbi sits at
  // bit 4i+v of word wi (j = 32wi + 4i + v), contraction index kk = 32wi + 8v + i
  // (the B nibble order), held by A lane group (kk%64)/16 at byte
  // kk%16 + 16(kk/64) (the A byte order measured on gfx950).
  if (NT == 4 * d || tid < 4 * d) {
    const float beta = fmaxf(qmx[lv][0], qmx[lv][1]) * (sqrtf(static_cast<float>(d)) * 1.001f);
    const int em = limb_exponent(2.f * cmax * beta);
    const int eq = limb_exponent(4.f * P.mrow_bound * beta);
    float pv = 0.f;
#pragma unroll
    for (int u = 0; u < PARTS; ++u) pv += pp[u][lv][pi];
    const int wi = pi >> 5, i8 = (pi & 31) >> 2, vb = pi & 3;
    const int kk = 32 * wi + 8 * vb + i8;
    const int slot = (16 * ((kk & 63) >> 4) + 4 * lv) * 32 + (kk & 15) + 16 * (kk >> 6);
    const float inv_val = vb == 0 ? 2.f : (vb == 1 ? 1.f : (vb == 2 ? 0.5f : -0.5f));
    const float qp = qs[lv][pi];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const float kappa = kb < NP ? P.plane_coef[kb < NP ? kb : 0] : 2.f;
      float R = ldexpf(kappa * (kb < NP ? qp : pv) * inv_val, kb < NP ? em : eq);
#pragma unroll
      for (int l = 0; l < 4; ++l) {
        const uint32_t bl = to_fp8(R);
        opst[kb * kOpBytes + slot + 32 * l] = static_cast<uint8_t>(bl);
        R = (R - from_fp8(bl)) * 16.f;
      }
    }
    const float s_all = wave_sum_dpp(pv);
    const float s_3 = wave_sum_dpp(vb == 3 ? pv : 0.f);
    if (lane == 0) {
      psum[lv][(tid >> 6) & 1][0] = s_all;
      psum[lv][(tid >> 6) & 1][1] = s_3;
    }
  }
  __syncthreads();
  if (!active) return;  // wave-uniform

  // A operands of the wave's lanes and the constants of query vector g = lane/16
  const int g = lane >> 4;
  v8i a[1][NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const uint4* src = reinterpret_cast<const uint4*>(opst + kb * kOpBytes + lane * 32);
    const uint4 x = src[0], y = src[1];
    a[0][kb][0] = x.x; a[0][kb][1] = x.y; a[0][kb][2] = x.z; a[0][kb][3] = x.w;
    a[0][kb][4] = y.x; a[0][kb][5] = y.y; a[0][kb][6] = y.z; a[0][kb][7] = y.w;
  }
  float4 cst[1];
  {
    const float sq = sqrtf(static_cast<float>(d));
    const float beta = fmaxf(qmx[g][0], qmx[g][1]) * (sq * 1.001f);
    const float s_all = sq * dq4[g][0];                                     // Σ_j q'_j
    const float s_3 = 0.25f * sq * (dq4[g][0] - dq4[g][1] - dq4[g][2] + dq4[g][3]);  // Σ_{j%4=3} q'_j
    const float p_all = psum[g][0][0] + psum[g][1][0], p_3 = psum[g][0][1] + psum[g][1][1];
    // slots with j%4 = 3 hold -x/2 against the +-1 nibble: add the x/2 back
    cst[0] = float4{ldexpf(1.f, -limb_exponent(2.f * cmax * beta)), ldexpf(1.f, -limb_exponent(4.f * P.mrow_bound * beta)),
                    P.plane_bias * s_all + 0.5f * csum * s_3, -p_all + p_3};
  }
  const int qvg = mt * 4 + g;
  float* const out[1] = {qvg < Gq ? logits + (static_cast<int64_t>(b * Hq + kh * G + qvg % G) * nq + qvg / G) * ctx + key0
                                  : nullptr};
  score_wave<NP, 1, 1>(cv, sv, nu_l, ga_l, s_codes[wv], s_signs[wv], a, cst, out, nvalid, P.qjl_kappa, lane);
}

// TQ_LOGITS_KERNEL=valu selects the general VALU kernel (A/B comparisons).
bool logits_mfma_eligible(const tq_codec_s* c) {
  const char* v = std::getenv("TQ_LOGITS_KERNEL");
  const bool forced_valu = v && std::string(v) == "valu";
  return !forced_valu && (c->prm.d == 128 || c->prm.d == 256);
}

size_t logits_mfma_ws_bytes(const tq_codec_s* c, int batch, int n_q_heads, int n_kv_heads, int n_queries) {
  const int G = n_q_heads / n_kv_heads;
  const int n_mt = static_cast<int>(ceil_div(static_cast<int64_t>(n_queries) * G, 4));
  const int NKB = (c->prm.n_planes + 1) * (c->prm.d / 128);
  return static_cast<size_t>(batch) * n_kv_heads * n_mt * (NKB * kOpBytes + kConstBytes);
}

hipError_t launch_logits_mfma_prep(const tq_codec_s* c, const void* q, tq_dtype_t dt, int batch, int n_q_heads,
                                   int n_kv_heads, int n_queries, void* ws, hipStream_t s) {
  const int G = n_q_heads / n_kv_heads;
  const int n_mt = static_cast<int>(ceil_div(static_cast<int64_t>(n_queries) * G, 4));
  const dim3 grid(static_cast<unsigned>(batch * n_kv_heads * n_mt));
  auto go = [&]<int E, typename T>(const T* qq) -> hipError_t {
    hipLaunchKernelGGL((attn_prep_mfma_kernel<E, T>), grid, dim3(256), 0, s, qq, c->prm, c->dD, c->dMt, n_q_heads,
                       n_queries, G, n_kv_heads, n_mt, static_cast<uint8_t*>(ws));
    return hipGetLastError();
  };
  auto by_type = [&]<int E>() -> hipError_t {
    switch (dt) {
      case TQ_F32: return go.template operator()<E>(static_cast<const float*>(q));
      case TQ_BF16: return go.template operator()<E>(static_cast<const __hip_bfloat16*>(q));
      case TQ_F16: return go.template operator()<E>(static_cast<const __half*>(q));
    }
    return hipErrorInvalidValue;
  };
  return c->prm.d == 128 ? by_type.template operator()<2>() : by_type.template operator()<4>();
}

hipError_t launch_logits_mfma(const tq_codec_s* c, const void* ws, int batch, int n_q_heads, int n_kv_heads,
                              int n_queries, tq_packed_t k, int64_t ctx, float* logits, hipStream_t s) {
  const int G = n_q_heads / n_kv_heads;
  const int n_mt = static_cast<int>(ceil_div(static_cast<int64_t>(n_queries) * G, 4));
  auto go = [&]<int NP, int WB, int NMT>() -> hipError_t {
    constexpr int WAVES = WB == 1 ? 8 : 4;
    const dim3 grid(static_cast<unsigned>(ceil_div(ctx, WAVES * kKeysPerWave)), batch * n_kv_heads,
                    static_cast<unsigned>(ceil_div(n_mt, NMT)));
    hipLaunchKernelGGL((logits_mfma_kernel<NP, WB, NMT, WAVES>), grid, dim3(WAVES * 64), 0, s,
                       static_cast<const uint8_t*>(ws), n_mt, static_cast<int>(ctx), k.codes, k.signs, k.norm,
                       k.rnorm, c->prm.qjl_kappa, logits);
    return hipGetLastError();
  };
  const int NP = c->prm.n_planes;
  const int WB = c->prm.d / 128;
  auto by_mt = [&]<int NPc, int WBc>() -> hipError_t {
    constexpr int NKB = (NPc + 1) * WBc;
    if (n_mt >= 4 && NKB * 4 <= 12) return go.template operator()<NPc, WBc, 4>();
    if (n_mt >= 2 && NKB * 2 <= 12) return go.template operator()<NPc, WBc, 2>();
    return go.template operator()<NPc, WBc, 1>();
  };
  if (WB == 1) {
    if (NP == 1) return by_mt.template operator()<1, 1>();
    if (NP == 2) return by_mt.template operator()<2, 1>();
    if (NP == 4) return by_mt.template operator()<4, 1>();
  } else {
    if (NP == 1) return by_mt.template operator()<1, 2>();
    if (NP == 2) return by_mt.template operator()<2, 2>();
    if (NP == 4) return by_mt.template operator()<4, 2>();
  }
  return hipErrorInvalidValue;
}

// One launch for prep and logits when the query group is one M-tile (at most
// 4 query vectors per KV head) and d = 128; TQ_LOGITS_FUSED=0 turns it off.
bool logits_fused_eligible(const tq_codec_s* c, int n_q_heads, int n_kv_heads, int n_queries) {
  const char* v = std::getenv("TQ_LOGITS_FUSED");
  if (v && std::string(v) == "0") return false;
  const int64_t nv = static_cast<int64_t>(n_queries) * (n_q_heads / n_kv_heads);
  return logits_mfma_eligible(c) && c->prm.d == 128 && nv <= 4;
}

hipError_t launch_logits_fused(const tq_codec_s* c, const void* q, tq_dtype_t dt, int batch, int n_q_heads,
                               int n_kv_heads, int n_queries, tq_packed_t k, int64_t ctx, float* logits,
                               hipStream_t s) {
  // 16 waves (1024 keys) per block: one block per CU at the decode shapes, so
  // the operand rebuild is paid once per CU rather than twice (measured 8.7 us
  // against 9.2 us for 8-wave blocks at 32 query heads x 32K keys).
  constexpr int WAVES = 16;
  const int G = n_q_heads / n_kv_heads;
  auto go = [&]<int NP, typename T>(const T* qq) -> hipError_t {
    const dim3 grid(static_cast<unsigned>(ceil_div(ctx, WAVES * kKeysPerWave)), batch * n_kv_heads, 1);
    hipLaunchKernelGGL((logits_fused_kernel<NP, WAVES, T>), grid, dim3(WAVES * 64), 0, s, qq, c->prm, c->dD, c->dMt,
                       n_q_heads, n_queries, G, n_kv_heads, static_cast<int>(ctx), k.codes, k.signs, k.norm,
                       k.rnorm, logits);
    return hipGetLastError();
  };
  auto by_np = [&]<typename T>(const T* qq) -> hipError_t {
    switch (c->prm.n_planes) {
      case 1: return go.template operator()<1>(qq);
      case 2: return go.template operator()<2>(qq);
      case 4: return go.template operator()<4>(qq);
    }
    return hipErrorInvalidValue;
  };
  switch (dt) {
    case TQ_F32: return by_np(static_cast<const float*>(q));
    case TQ_BF16: return by_np(static_cast<const __hip_bfloat16*>(q));
    case TQ_F16: return by_np(static_cast<const __half*>(q));
  }
  return hipErrorInvalidValue;
}

}  // namespace tq

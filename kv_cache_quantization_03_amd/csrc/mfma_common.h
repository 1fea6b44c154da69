// Matrix-core building blocks shared by the logits and decode-attention
// kernels (v_mfma_scale_f32_16x16x128_f8f6f4 on gfx950).
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
#pragma once

#include "kernels_common.h"

namespace tq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));  // 16-byte record piece (a plain vector, kept in VGPRs)

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
// The same with a per-lane E8M0 scale for A: the scale of lane 16b + r applies
// to row r, contraction elements 32b..32b+31 (measured on gfx950).
__device__ __forceinline__ v4f mfma_fp8_fp4_scaled(const v8i& a, const v8i& b, const v4f& c, int scale_a) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, scale_a, 0, 127);
}

// A pointer the caller knows to be wave-uniform, moved to scalar registers
// (for buffer resources, whose base must be scalar).
template <typename T>
__device__ __forceinline__ T* uniform_ptr(const T* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(u & 0xFFFFFFFFu)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(u >> 32)));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
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
    cv[i] = __builtin_nontemporal_load(&reinterpret_cast<const v4u*>(codes)[(kk * L::CW + w % L::CW) / 4]);
  }
#pragma unroll
  for (int i = 0; i < L::SW / 4; ++i) {
    const int w = 4 * (i * 64 + lane);
    const int kk = min(w / L::SW, nvalid - 1);
    sv[i] = __builtin_nontemporal_load(&reinterpret_cast<const v4u*>(signs)[(kk * L::SW + w % L::SW) / 4]);
  }
  const int ln = min(lane, nvalid - 1);
  nu = __builtin_nontemporal_load(&norm[ln]);
  ga = __builtin_nontemporal_load(&rnorm[ln]);
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
      if (out[i] != nullptr && kk < nvalid) __builtin_nontemporal_store(nu * (mse + kappa * ga * qj), &out[i][kk]);
    }
  }
}

// Scores of the wave's 64 keys (records as loaded by load_wave_records)
// against one M-tile, kept in registers: val[t] = ℓ of key 16t + lane%16 for
// tile vector lane/16.  Same staging and matrix ops as score_wave.
template <int NP, int WB, int NC, int NS, int NKB>
__device__ __forceinline__ void score_wave_values(const v4u (&cv)[NC], const v4u (&sv)[NS], float nu_l, float ga_l,
                                                  uint32_t* __restrict__ s_codes, uint32_t* __restrict__ s_signs,
                                                  const v8i (&a)[1][NKB], const float4& cst, float kappa, int lane,
                                                  float (&val)[kKeysPerWave / kKeysPerTile]) {
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
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int t = 0; t < kKeysPerWave / kKeysPerTile; ++t) {
    const int kk = t * kKeysPerTile + kl;
    const uint32_t* crow = &s_codes[kk * L::CS];
    const uint32_t* srow = &s_signs[kk * L::SS];
    const float nu = __shfl(nu_l, kk, kWave), ga = __shfl(ga_l, kk, kWave);
    v4f acc_m = v4f{0.f, 0.f, 0.f, 0.f}, acc_q = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int wb = 0; wb < WB; ++wb) {
      uint32_t pw[L::NB];
#pragma unroll
      for (int p = 0; p < L::NB; ++p) pw[p] = crow[p * L::W + 4 * wb + g];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        constexpr int NB = L::NB;
        const uint32_t w = (p < NB) ? pw[p < NB ? p : 0] : (pw[0] ^ pw[NB > 1 ? 1 : 0] ^ pw[NB > 2 ? 2 : 0]);
        acc_m = mfma_fp8_fp4(a[0][p * WB + wb], fp4_operand(w), acc_m);
      }
      acc_q = mfma_fp8_fp4(a[0][NP * WB + wb], fp4_operand(srow[4 * wb + g]), acc_q);
    }
    asm volatile("" : "+v"(acc_m), "+v"(acc_q));
    const float mse = cst.x * (acc_m[0] + acc_m[1] * 0.0625f + acc_m[2] * 0.00390625f + acc_m[3] * 0.000244140625f) + cst.z;
    const float qj = cst.y * (acc_q[0] + acc_q[1] * 0.0625f + acc_q[2] * 0.00390625f + acc_q[3] * 0.000244140625f) + cst.w;
    val[t] = nu * (mse + kappa * ga * qj);
  }
  __builtin_amdgcn_wave_barrier();
}

// ----------------------------------------------------------------------------
// V bits as matrix operands (decode attention, and the 32-token blocked V
// layout written at encode).  The contraction over keys needs, in each lane,
// the bits of one coordinate across 32 keys, while a row record holds 32
// coordinates of one key: a 32x32 bit transpose in registers (four lane
// stages with DPP partners within rows of 16 lanes, one stage between the
// lane's two registers).
// ----------------------------------------------------------------------------
// One stage of the bit transpose: swap row bit K (lane bit K) with column bit K.
template <int K>
__device__ __forceinline__ uint32_t transpose_stage(uint32_t w, int lane) {
  constexpr uint32_t M = K == 0 ? 0x55555555u : (K == 1 ? 0x33333333u : (K == 2 ? 0x0F0F0F0Fu : 0x00FF00FFu));
  constexpr int s = 1 << K;
  const uint32_t x = lane_xor<K>(w);
  const bool hi = (lane >> K) & 1;
  const uint32_t t = hi ? (x >> s) : (x << s);
  const uint32_t keep = hi ? ~M : M;
  return (w & keep) | (t & ~keep);
}

// 32x32 bit transpose within each row of 16 lanes: input row ρ = lane%16 + 16·reg
// (r0: reg 0, r1: reg 1), column = bit; output lane%16 + 16·reg = column,
// bit = row.
__device__ __forceinline__ void transpose32(uint32_t& r0, uint32_t& r1, int lane) {
  r0 = transpose_stage<0>(r0, lane);
  r1 = transpose_stage<0>(r1, lane);
  r0 = transpose_stage<1>(r0, lane);
  r1 = transpose_stage<1>(r1, lane);
  r0 = transpose_stage<2>(r0, lane);
  r1 = transpose_stage<2>(r1, lane);
  r0 = transpose_stage<3>(r0, lane);
  r1 = transpose_stage<3>(r1, lane);
  const uint32_t t = ((r0 >> 16) ^ r1) & 0x0000FFFFu;
  r1 ^= t;
  r0 ^= t << 16;
}

// Key (within the lane group's 32) whose words lane%16 + 16·reg loads: row
// ρ = 4i + r carries key 8r + i, so that after the transpose bit 4i + r of the
// word — FP4 nibble i of mask r, contraction index 8r + i — is that key.
__device__ __forceinline__ int v_key_of_row(int rho) { return 8 * (rho & 3) + (rho >> 2); }

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
// In-block query operands (d = 128, one M-tile of 4 query vectors).
//
// Every block that scores keys of one (batch, kv head) rebuilds the fp8 limb
// operands of that head's query vectors in LDS while its records are in
// flight.  Because the limbs are floating point, the power-of-two operand
// scales need only upper bounds of the operands, not their maxima: with
// β = √d max_k |q_k| >= ||q||, |q'_j| <= β (R is orthogonal) and
// |p_i| <= max_i ||M_i|| β (Cauchy-Schwarz), so one max over the raw query
// replaces the reductions over q' and p.  The two constant sums of q' come
// from the Sylvester matrix's row sums: Σ_j q'_j = √d D_0 q_0 and
// Σ_{j≡3 mod 4} q'_j = (√d/4)(D_0q_0 - D_1q_1 - D_2q_2 + D_3q_3).  Each thread
// cuts the limbs of its own (vector, coordinate).
// ----------------------------------------------------------------------------
constexpr int kPrepD = 128;

template <int NT, int NKB>
struct QueryPrepShared {
  static constexpr int PARTS = NT / kPrepD;
  float qr[4][kPrepD];         // q
  float qs[4][kPrepD];         // D ⊙ q, then q' = R q
  float pp[PARTS][4][kPrepD];  // partial sums of p = M q over slices of j
  float qmx[4][2];             // max |q_k| per vector, per half
  float dq4[4][4];             // (D ⊙ q)_0..3 per vector
  float psum[4][2][2];         // Σ p and Σ_{i%4=3} p per vector, per half
  __attribute__((aligned(16))) uint8_t opst[NKB * kOpBytes];
};

// Where the tile's query vectors live: vector v of the tile is query slot
// mt*4 + v of KV head kh, i.e. query index slot/G and head kh*G + slot%G of
// q[batch][nq][Hq][d]; slots past Gq = nq*G are padding (zero).
struct QueryTile {
  int b, nq, Hq, G, kh, mt, Gq;
};

template <int NT>
struct QueryPrepRegs {
  float mv[kPrepD / (NT / kPrepD)];  // the thread's slice of column pi of Mᵀ
  float qraw, dx;                    // q and D at (vector tid/d, coordinate tid%d)
};

// The operand-side loads of the calling thread; issue them before the record
// loads.  q, D and M are not __restrict__ so the compiler keeps these loads
// above the barrier that follows them.
template <int NT, typename T>
__device__ __forceinline__ void query_prep_load(QueryPrepRegs<NT>& r, const T* q, const float* Dsign,
                                                const float* Mt, const QueryTile& t) {
  constexpr int d = kPrepD, JP = d / (NT / d);
  const int tid = threadIdx.x, pi = tid & (d - 1), part = tid / d;
#pragma unroll
  for (int u = 0; u < JP; ++u) r.mv[u] = Mt[(part * JP + u) * d + pi];
  const int lv = min(tid / d, 3), qc = min(t.mt * 4 + lv, t.Gq - 1);
  r.qraw = load_elem(q + ((static_cast<int64_t>(t.b) * t.nq + qc / t.G) * t.Hq + t.kh * t.G + qc % t.G) * d, pi);
  r.dx = Dsign[pi];
}

// Builds the A operands of the tile in sh.opst (NKB K-blocks: NP MSE planes,
// then the QJL block).  Every thread of the block calls it; it holds three
// block barriers and ends with the operands visible to the whole block.
template <int NT, int NP, int NKB>
__device__ __forceinline__ void query_prep_build(QueryPrepShared<NT, NKB>& sh, const QueryPrepRegs<NT>& r,
                                                 const DevParams& P, const QueryTile& t) {
  constexpr int d = kPrepD, PARTS = NT / d, JP = d / PARTS;
  static_assert(NT >= 4 * d, "one thread per (query vector, coordinate) of the tile");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, pi = tid & (d - 1), part = tid / d;
  const int lv = min(tid / d, 3), qv = t.mt * 4 + lv;
  if (NT == 4 * d || tid < 4 * d) {
    const float qx = qv < t.Gq ? r.qraw : 0.f;
    sh.qr[lv][pi] = qx;
    sh.qs[lv][pi] = qx * r.dx;
    if (pi < 4) sh.dq4[lv][pi] = qx * r.dx;
    const float mx = wave_max_dpp(fabsf(qx));
    if (lane == 0) sh.qmx[lv][wv & 1] = mx;
  }
  __syncthreads();

  // q' = H (D ⊙ q)/√d in place by waves 0..3 (one vector each); p partial sums by all
  if (wv < 4) {
    float v[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) v[e] = sh.qs[wv][e * kWave + lane];
    hadamard_wave<2, false, true>(v, lane);
#pragma unroll
    for (int e = 0; e < 2; ++e) sh.qs[wv][e * kWave + lane] = v[e] * P.inv_sqrt_d;
  }
  {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < JP; ++u) {
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) acc[vq] = fmaf(r.mv[u], sh.qr[vq][part * JP + u], acc[vq]);
    }
#pragma unroll
    for (int vq = 0; vq < 4; ++vq) sh.pp[part][vq][pi] = acc[vq];
  }
  float cmax = 0.f;
#pragma unroll
  for (int k = 0; k < NP; ++k) cmax = fmaxf(cmax, fabsf(P.plane_coef[k]));
  __syncthreads();

  // Limbs of the thread's own (vector lv, coordinate pi): the MSE planes from
  // q'_pi and the QJL block from p_pi.  Coordinate j of K-block kbi sits at
  // bit 4i+v of word wi (j = 32wi + 4i + v), contraction index kk = 32wi + 8v + i
  // (the B nibble order), held by A lane group (kk%64)/16 at byte
  // kk%16 + 16(kk/64) (the A byte order measured on gfx950).
  if (NT == 4 * d || tid < 4 * d) {
    const float beta = fmaxf(sh.qmx[lv][0], sh.qmx[lv][1]) * (sqrtf(static_cast<float>(d)) * 1.001f);
    const int em = limb_exponent(2.f * cmax * beta);
    const int eq = limb_exponent(4.f * P.mrow_bound * beta);
    float pv = 0.f;
#pragma unroll
    for (int u = 0; u < PARTS; ++u) pv += sh.pp[u][lv][pi];
    const int wi = pi >> 5, i8 = (pi & 31) >> 2, vb = pi & 3;
    const int kk = 32 * wi + 8 * vb + i8;
    const int slot = (16 * ((kk & 63) >> 4) + 4 * lv) * 32 + (kk & 15) + 16 * (kk >> 6);
    const float inv_val = vb == 0 ? 2.f : (vb == 1 ? 1.f : (vb == 2 ? 0.5f : -0.5f));
    const float qp = sh.qs[lv][pi];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const float kappa = kb < NP ? P.plane_coef[kb < NP ? kb : 0] : 2.f;
      float R = ldexpf(kappa * (kb < NP ? qp : pv) * inv_val, kb < NP ? em : eq);
#pragma unroll
      for (int l = 0; l < 4; ++l) {
        const uint32_t bl = to_fp8(R);
        sh.opst[kb * kOpBytes + slot + 32 * l] = static_cast<uint8_t>(bl);
        R = (R - from_fp8(bl)) * 16.f;
      }
    }
    const float s_all = wave_sum_dpp(pv);
    const float s_3 = wave_sum_dpp(vb == 3 ? pv : 0.f);
    if (lane == 0) {
      sh.psum[lv][wv & 1][0] = s_all;
      sh.psum[lv][wv & 1][1] = s_3;
    }
  }
  __syncthreads();
}

// The lane's K-block operands (lane L holds 32 bytes of each) from sh.opst.
template <int NT, int NKB>
__device__ __forceinline__ void query_prep_operands(const QueryPrepShared<NT, NKB>& sh, v8i (&a)[1][NKB], int lane) {
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const uint4* src = reinterpret_cast<const uint4*>(sh.opst + kb * kOpBytes + lane * 32);
    const uint4 x = src[0], y = src[1];
    a[0][kb][0] = x.x; a[0][kb][1] = x.y; a[0][kb][2] = x.z; a[0][kb][3] = x.w;
    a[0][kb][4] = y.x; a[0][kb][5] = y.y; a[0][kb][6] = y.z; a[0][kb][7] = y.w;
  }
}

// (scale_m, scale_q, bias_m, bias_q) of tile vector g: the limb scales undo
// the operand scales; slots with j%4 = 3 hold -x/2 against the ±1 nibble, so
// the biases add the x/2 back (and the codebook's constant term for the MSE sum).
template <int NT, int NP, int NKB>
__device__ __forceinline__ float4 query_prep_constants(const QueryPrepShared<NT, NKB>& sh, const DevParams& P, int g) {
  constexpr int d = kPrepD;
  float cmax = 0.f, csum = 0.f;
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    cmax = fmaxf(cmax, fabsf(P.plane_coef[k]));
    csum += P.plane_coef[k];
  }
  const float sq = sqrtf(static_cast<float>(d));
  const float beta = fmaxf(sh.qmx[g][0], sh.qmx[g][1]) * (sq * 1.001f);
  const float s_all = sq * sh.dq4[g][0];                                                   // Σ_j q'_j
  const float s_3 = 0.25f * sq * (sh.dq4[g][0] - sh.dq4[g][1] - sh.dq4[g][2] + sh.dq4[g][3]);  // Σ_{j%4=3} q'_j
  const float p_all = sh.psum[g][0][0] + sh.psum[g][1][0], p_3 = sh.psum[g][0][1] + sh.psum[g][1][1];
  return float4{ldexpf(1.f, -limb_exponent(2.f * cmax * beta)), ldexpf(1.f, -limb_exponent(4.f * P.mrow_bound * beta)),
                P.plane_bias * s_all + 0.5f * csum * s_3, -p_all + p_3};
}

}  // namespace tq

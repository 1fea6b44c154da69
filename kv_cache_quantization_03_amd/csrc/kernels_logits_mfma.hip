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

namespace {

constexpr int kOpBytes = 64 * 32;  // one K-block of A for one M-tile: 64 lanes x 32 bytes
constexpr int kConstFloats = 16;   // per M-tile: 4 query vectors x (scale_m, scale_q, bias_m, bias_q)
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

// Limb `limb` of R = R0 + R1/16 + R2/256 + R3/4096 (|R| <= 256).
__device__ __forceinline__ uint32_t fp8_limb(float R, int limb) {
  uint32_t out = 0;
#pragma unroll
  for (int l = 0; l < 4; ++l) {
    const uint32_t b = to_fp8(R);
    if (l == limb) out = b;
    R = (R - from_fp8(b)) * 16.f;
  }
  return out;
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
                                                             const float* __restrict__ St, int Hq, int nq, int G,
                                                             int nkv, int n_mt, uint8_t* __restrict__ prep) {
  constexpr int d = E * kWave;
  constexpr int W = d / 32;
  __shared__ float qs[4][d];
  __shared__ float ps[4][d];
  __shared__ float mx[4][2];
  const int blk = blockIdx.x;
  const int mt = blk % n_mt, bk = blk / n_mt;
  const int b = bk / nkv, kh = bk % nkv;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int Gq = nq * G;
  {
    const int qv = mt * 4 + wv;
    float v[E];
    if (qv < Gq) {
      const int qi = qv / G, g = qv % G;
      const int64_t row = (static_cast<int64_t>(b) * nq + qi) * Hq + kh * G + g;
#pragma unroll
      for (int e = 0; e < E; ++e) v[e] = load_elem(q + row * d, e * kWave + lane) * Dsign[e * kWave + lane];
      hadamard_wave<E>(v, lane);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) v[e] = 0.f;
    }
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
  for (int i = threadIdx.x; i < d; i += 256) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int j = 0; j < d; ++j) {
      const float s = St[static_cast<int64_t>(j) * d + i];
      a0 = fmaf(s, qs[0][j], a0);
      a1 = fmaf(s, qs[1][j], a1);
      a2 = fmaf(s, qs[2][j], a2);
      a3 = fmaf(s, qs[3][j], a3);
    }
    ps[0][i] = a0;
    ps[1][i] = a1;
    ps[2][i] = a2;
    ps[3][i] = a3;
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
  uint8_t* base = prep + (static_cast<int64_t>(bk) * n_mt + mt) * (NKB * kOpBytes + kConstFloats * 4);
  // operands: K-block kbi -> (plane, word block); wave wv builds kbi = wv, wv+4, ...
  for (int kbi = wv; kbi < NKB; kbi += 4) {
    const int plane = kbi / (W / 4), kb = kbi % (W / 4);
    const bool qjl = plane >= NP;
    const float kappa = qjl ? 2.f : P.plane_coef[plane];
    const int row = lane & 15, hl = row >> 2, limb = row & 3, g = lane >> 4;
    const float sigma = qjl ? 4.f * mx[hl][1] : 2.f * cmax * mx[hl][0];
    const float scale = ldexpf(1.f, limb_exponent(sigma));
    const float* src = qjl ? ps[hl] : qs[hl];
    uint32_t words[8];
#pragma unroll
    for (int dw = 0; dw < 8; ++dw) {
      uint32_t wbits = 0;
#pragma unroll
      for (int by = 0; by < 4; ++by) {
        // A byte s of lane group g holds contraction index kk; B nibble kk%32
        // of lane group kk/32 holds the same kk (lane layout measured on gfx950)
        const int s = dw * 4 + by;
        const int kk = s < 16 ? 16 * g + s : 64 + 16 * g + (s - 16);
        const int wi = kk >> 5, sp = kk & 31;
        const int v = sp >> 3, i = sp & 7;  // nibble i of B VGPR v = bit 4i+v of the word
        const int j = 32 * (4 * kb + wi) + 4 * i + v;
        const float inv_val = v == 0 ? 2.f : (v == 1 ? 1.f : (v == 2 ? 0.5f : -0.5f));
        const float x = kappa * src[j] * inv_val * scale;
        wbits |= fp8_limb(x, limb) << (8 * by);
      }
      words[dw] = wbits;
    }
    uint4* dst = reinterpret_cast<uint4*>(base + static_cast<int64_t>(kbi) * kOpBytes + lane * 32);
    dst[0] = make_uint4(words[0], words[1], words[2], words[3]);
    dst[1] = make_uint4(words[4], words[5], words[6], words[7]);
  }
  // constants per query vector of the tile
  if (threadIdx.x < 4) {
    const int hl = threadIdx.x;
    float sall = 0.f, s3 = 0.f, pall = 0.f, p3 = 0.f;
    for (int j = 0; j < d; ++j) {
      sall += qs[hl][j];
      pall += ps[hl][j];
      if ((j & 3) == 3) {
        s3 += qs[hl][j];
        p3 += ps[hl][j];
      }
    }
    float* cst = reinterpret_cast<float*>(base + NKB * kOpBytes);
    cst[hl * 4 + 0] = ldexpf(1.f, -limb_exponent(2.f * cmax * mx[hl][0]));
    cst[hl * 4 + 1] = ldexpf(1.f, -limb_exponent(4.f * mx[hl][1]));
    cst[hl * 4 + 2] = P.plane_bias * sall + 0.5f * csum * s3;  // slots j%4 = 3 hold -x/2 against 1-2bit
    cst[hl * 4 + 3] = -pall + p3;
  }
}

// ----------------------------------------------------------------------------
// Logits: block = 4 waves, each wave scores T tiles of 16 keys of one
// (batch, kv head) against NMT M-tiles of its query group.
// ----------------------------------------------------------------------------
template <int NP, int WB, int NMT, int T>
__global__ __launch_bounds__(256) void logits_mfma_kernel(const uint8_t* __restrict__ prep, DevParams P, int Hq,
                                                          int nq, int G, int nkv, int n_mt, int64_t ctx,
                                                          tq_packed_t k, float* __restrict__ logits) {
  constexpr int NKB = (NP + 1) * WB;  // K-blocks: MSE planes x word blocks, then QJL word blocks
  constexpr int W = 4 * WB;           // words per plane
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane >> 4, kl = lane & 15;
  const int bk = blockIdx.y;
  const int b = bk / nkv, kh = bk % nkv;
  const int mt0 = blockIdx.z * NMT;
  const int64_t key0 = (static_cast<int64_t>(blockIdx.x) * 4 + wv) * (T * kKeysPerTile);
  if (key0 >= ctx) return;
  const int CW = P.code_words, SW = P.sign_words;

  // ---- loads for all T tiles first (memory-level parallelism)
  constexpr int NB = NP > 3 ? 3 : NP;  // stored planes (the parity plane is computed)
  uint32_t cw[T][NB * WB];
  uint32_t sw[T][WB];
  float nu[T], ga[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    int64_t key = key0 + t * kKeysPerTile + kl;
    key = key < ctx ? key : ctx - 1;
    const int64_t row = static_cast<int64_t>(bk) * ctx + key;
    const uint32_t* crow = k.codes + row * CW;
#pragma unroll
    for (int p = 0; p < NB; ++p)
#pragma unroll
      for (int wb = 0; wb < WB; ++wb) cw[t][p * WB + wb] = crow[p * W + 4 * wb + g];
#pragma unroll
    for (int wb = 0; wb < WB; ++wb) sw[t][wb] = k.signs[row * SW + 4 * wb + g];
    nu[t] = k.norm[row];
    ga[t] = k.rnorm[row];
  }
  // ---- query operands and constants (shared by every tile)
  v8i a[NMT][NKB];
  float sc_m[NMT], sc_q[NMT], bi_m[NMT], bi_q[NMT];
  bool mt_ok[NMT];
#pragma unroll
  for (int i = 0; i < NMT; ++i) {
    const int mt = mt0 + i;
    mt_ok[i] = mt < n_mt;
    const int mtc = mt_ok[i] ? mt : 0;
    const uint8_t* base = prep + (static_cast<int64_t>(bk) * n_mt + mtc) * (NKB * kOpBytes + kConstFloats * 4);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const uint4* src = reinterpret_cast<const uint4*>(base + kb * kOpBytes + lane * 32);
      const uint4 x = src[0], y = src[1];
      a[i][kb][0] = x.x; a[i][kb][1] = x.y; a[i][kb][2] = x.z; a[i][kb][3] = x.w;
      a[i][kb][4] = y.x; a[i][kb][5] = y.y; a[i][kb][6] = y.z; a[i][kb][7] = y.w;
    }
    const float* cst = reinterpret_cast<const float*>(base + NKB * kOpBytes) + g * 4;
    sc_m[i] = cst[0];
    sc_q[i] = cst[1];
    bi_m[i] = cst[2];
    bi_q[i] = cst[3];
  }
  const float kappa = P.qjl_kappa;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int64_t key = key0 + t * kKeysPerTile + kl;
    v4f acc_m[NMT], acc_q[NMT];
#pragma unroll
    for (int i = 0; i < NMT; ++i) {
      acc_m[i] = v4f{0.f, 0.f, 0.f, 0.f};
      acc_q[i] = v4f{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
#pragma unroll
      for (int wb = 0; wb < WB; ++wb) {
        uint32_t w;
        if (p < 3 && p < NB) {
          w = cw[t][p * WB + wb];
        } else {  // parity plane of a 3-bit code
          w = cw[t][0 * WB + wb] ^ cw[t][1 * WB + wb] ^ cw[t][2 * WB + wb];
        }
        const v8i bop = fp4_operand(w);
#pragma unroll
        for (int i = 0; i < NMT; ++i) acc_m[i] = mfma_fp8_fp4(a[i][p * WB + wb], bop, acc_m[i]);
      }
    }
#pragma unroll
    for (int wb = 0; wb < WB; ++wb) {
      const v8i bop = fp4_operand(sw[t][wb]);
#pragma unroll
      for (int i = 0; i < NMT; ++i) acc_q[i] = mfma_fp8_fp4(a[i][NP * WB + wb], bop, acc_q[i]);
    }
    // An MFMA reads operands from all 64 lanes, so it must run with the full
    // EXEC mask: pin every accumulator here, in wave-uniform control flow, so
    // the compiler cannot sink the matrix ops into the lane-divergent stores.
#pragma unroll
    for (int i = 0; i < NMT; ++i) asm volatile("" : "+v"(acc_m[i]), "+v"(acc_q[i]));
    if (key >= ctx) continue;
#pragma unroll
    for (int i = 0; i < NMT; ++i) {
      const int qv = (mt0 + i) * 4 + g;
      if (!mt_ok[i] || qv >= nq * G) continue;
      const float mse = sc_m[i] * (acc_m[i][0] + acc_m[i][1] * 0.0625f + acc_m[i][2] * 0.00390625f +
                                   acc_m[i][3] * 0.000244140625f) + bi_m[i];
      const float qj = sc_q[i] * (acc_q[i][0] + acc_q[i][1] * 0.0625f + acc_q[i][2] * 0.00390625f +
                                  acc_q[i][3] * 0.000244140625f) + bi_q[i];
      const int qi = qv / G, gg = qv % G;
      const int h = kh * G + gg;
      logits[((static_cast<int64_t>(b) * Hq + h) * nq + qi) * ctx + key] = nu[t] * (mse + kappa * ga[t] * qj);
    }
  }
}

// ----------------------------------------------------------------------------
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
  return static_cast<size_t>(batch) * n_kv_heads * n_mt * (NKB * kOpBytes + kConstFloats * 4);
}

hipError_t launch_logits_mfma_prep(const tq_codec_s* c, const void* q, tq_dtype_t dt, int batch, int n_q_heads,
                                   int n_kv_heads, int n_queries, void* ws, hipStream_t s) {
  const int G = n_q_heads / n_kv_heads;
  const int n_mt = static_cast<int>(ceil_div(static_cast<int64_t>(n_queries) * G, 4));
  const dim3 grid(static_cast<unsigned>(batch * n_kv_heads * n_mt));
  auto go = [&]<int E, typename T>(const T* qq) -> hipError_t {
    hipLaunchKernelGGL((attn_prep_mfma_kernel<E, T>), grid, dim3(256), 0, s, qq, c->prm, c->dD, c->dSt, n_q_heads,
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
  constexpr int T = 4;
  auto go = [&]<int NP, int WB, int NMT>() -> hipError_t {
    const dim3 grid(static_cast<unsigned>(ceil_div(ctx, 4 * T * kKeysPerTile)), batch * n_kv_heads,
                    static_cast<unsigned>(ceil_div(n_mt, NMT)));
    hipLaunchKernelGGL((logits_mfma_kernel<NP, WB, NMT, T>), grid, dim3(256), 0, s,
                       static_cast<const uint8_t*>(ws), c->prm, n_q_heads, n_queries, G, n_kv_heads, n_mt, ctx, k,
                       logits);
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

}  // namespace tq

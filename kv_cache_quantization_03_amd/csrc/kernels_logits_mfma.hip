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

#include "mfma_common.h"

namespace tq {

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
    hadamard_wave<E, false, true>(v, lane);
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
// Query prep for d = 128 with the in-block operand builder of the fused kernel
// (query_prep_*: operand scales from bounds, DPP reductions, 1024 threads), one
// block per (batch*kv_head, M-tile); same output layout as attn_prep_mfma_kernel.
// 7.5 us for the 8 KV heads of a decode step with 256-thread blocks that
// reduce the exact maxima; this one is bounded by one L2 round trip for M.
// ----------------------------------------------------------------------------
template <int NP, typename T>
__global__ __launch_bounds__(1024) void attn_prep_inblock_kernel(const T* q, DevParams P, const float* Dsign,
                                                                 const float* Mt, int Hq, int nq, int G, int nkv,
                                                                 int n_mt, uint8_t* __restrict__ prep) {
  constexpr int NT = 1024, NKB = NP + 1;
  __shared__ QueryPrepShared<NT, NKB> sh;
  const int mt = blockIdx.x % n_mt, bk = blockIdx.x / n_mt;
  const QueryTile tile{bk / nkv, nq, Hq, G, bk % nkv, mt, nq * G};
  QueryPrepRegs<NT> pr;
  query_prep_load<NT>(pr, q, Dsign, Mt, tile);
  query_prep_build<NT, NP, NKB>(sh, pr, P, tile);  // ends with a block barrier
  uint8_t* base = prep + (static_cast<int64_t>(bk) * n_mt + mt) * (NKB * kOpBytes + kConstBytes);
  for (int e = threadIdx.x; e < NKB * kOpBytes / 16; e += NT)
    reinterpret_cast<uint4*>(base)[e] = reinterpret_cast<const uint4*>(sh.opst)[e];
  if (threadIdx.x < 4) {  // constants and output row of tile vector v
    const int v = threadIdx.x, qv = mt * 4 + v;
    reinterpret_cast<float4*>(base + NKB * kOpBytes)[v] = query_prep_constants<NT, NP, NKB>(sh, P, v);
    reinterpret_cast<int*>(base + NKB * kOpBytes + 64)[v] =
        qv < tile.Gq ? (tile.b * Hq + tile.kh * G + qv % G) * nq + qv / G : -1;
  }
}

// The same builder writing q' = R q and p = S q' in fp32 (rows (b*nq + qi)*Hq
// + h of qrot[.][128], proj[.][128]) for the VALU scorers (the PolarQuant
// first stage), instead of the rotate kernel and the general fp32 projection
// (21 us for a decode step's 32 query vectors).
template <typename T>
__global__ __launch_bounds__(1024) void attn_prep_fp32_kernel(const T* q, DevParams P, const float* Dsign,
                                                              const float* Mt, int Hq, int nq, int G, int nkv,
                                                              int n_mt, float* __restrict__ qrot,
                                                              float* __restrict__ proj) {
  constexpr int NT = 1024, d = kPrepD;
  __shared__ QueryPrepShared<NT, 3> sh;
  const int mt = blockIdx.x % n_mt, bk = blockIdx.x / n_mt;
  const QueryTile tile{bk / nkv, nq, Hq, G, bk % nkv, mt, nq * G};
  QueryPrepRegs<NT> pr;
  query_prep_load<NT>(pr, q, Dsign, Mt, tile);
  query_prep_build<NT, 2, 3>(sh, pr, P, tile);  // ends with a block barrier; its operands are not used
  if (threadIdx.x < 4 * d) {
    const int v = threadIdx.x / d, j = threadIdx.x % d, qv = mt * 4 + v;
    if (qv < tile.Gq) {
      const int64_t row = (static_cast<int64_t>(tile.b) * nq + qv / G) * Hq + tile.kh * G + qv % G;
      float pv = 0.f;
#pragma unroll
      for (int u = 0; u < NT / d; ++u) pv += sh.pp[u][v][j];
      qrot[row * d + j] = sh.qs[v][j];
      proj[row * d + j] = pv;
    }
  }
}

hipError_t launch_qprep128(const tq_codec_s* c, const void* q, tq_dtype_t dt, int batch, int n_q_heads, int n_kv_heads,
                           int n_queries, float* qrot, float* proj, hipStream_t s) {
  const int G = n_q_heads / n_kv_heads;
  const int n_mt = static_cast<int>(ceil_div(static_cast<int64_t>(n_queries) * G, 4));
  const dim3 grid(static_cast<unsigned>(batch * n_kv_heads * n_mt));
  auto go = [&]<typename T>(const T* qq) -> hipError_t {
    hipLaunchKernelGGL((attn_prep_fp32_kernel<T>), grid, dim3(1024), 0, s, qq, c->prm, c->dD, c->dMt, n_q_heads,
                       n_queries, G, n_kv_heads, n_mt, qrot, proj);
    return hipGetLastError();
  };
  switch (dt) {
    case TQ_F32: return go(static_cast<const float*>(q));
    case TQ_BF16: return go(static_cast<const __hip_bfloat16*>(q));
    case TQ_F16: return go(static_cast<const __half*>(q));
  }
  return hipErrorInvalidValue;
}

// ----------------------------------------------------------------------------
// Logits from prepared query operands: each wave scores NG consecutive groups
// of 64 keys against NMT M-tiles of its query group, operands and constants
// read once from `prep`; the next group's records load while the current one
// is scored.  With one M-tile and d = 128 the logits leave in whole lines as
// in logits_fused_kernel below (vec_out).
// ----------------------------------------------------------------------------
// PAGED: the keys of (batch b, KV head kh) live in the pages of a paged cache
// (see PageMap; page_size a multiple of 64, so a 64-key group lies in one
// page); sequence b scores its first ctx_lens[b] keys, and ctx is the row
// stride of the logits.
template <int NP, int WB, int NMT, int WAVES, int NG, bool PAGED>
__global__ __launch_bounds__(WAVES * 64) void logits_mfma_kernel(const uint8_t* __restrict__ prep, int n_mt, int ctx,
                                                                 const uint32_t* __restrict__ codes,
                                                                 const uint32_t* __restrict__ signs,
                                                                 const float* __restrict__ norm,
                                                                 const float* __restrict__ rnorm, float kappa,
                                                                 float* __restrict__ logits, PageMap pm, int nkv,
                                                                 int vec_out) {
  using L = RecLayout<NP, WB>;
  constexpr int NKB = L::NKB;
  constexpr int MT_BYTES = NKB * kOpBytes + kConstBytes;
  __shared__ uint32_t s_codes[WAVES][kKeysPerWave * L::CS];
  __shared__ uint32_t s_signs[WAVES][kKeysPerWave * L::SS];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int bk = blockIdx.y;
  const int key0 = (blockIdx.x * WAVES + wv) * (NG * kKeysPerWave);
  int ctx_v = ctx;  // keys to score in this row
  // paged: the sequence's own length, clamped to max_ctx (ctx here), which the
  // host bounds by max_pages * page_size
  if constexpr (PAGED) ctx_v = max(0, min(pm.ctx_lens[bk / nkv], ctx));
  if (key0 >= ctx_v) return;  // wave-uniform
  v4u cv[2][L::CW / 4], sv[2][L::SW / 4];
  float nu_l[2], ga_l[2];
  auto load_group = [&](int i, int buf) {
    const int k0 = key0 + i * kKeysPerWave;
    int64_t r0 = static_cast<int64_t>(bk) * ctx + k0;
    if constexpr (PAGED) {
      const int page = pm.table[static_cast<int64_t>(bk / nkv) * pm.max_pages + k0 / pm.page_size];
      r0 = (static_cast<int64_t>(page) * nkv + bk % nkv) * pm.page_size + k0 % pm.page_size;
    }
    load_wave_records<NP, WB>(cv[buf], sv[buf], nu_l[buf], ga_l[buf], codes + r0 * L::CW, signs + r0 * L::SW,
                              norm + r0, rnorm + r0, min(kKeysPerWave, ctx_v - k0), lane);
  };
  load_group(0, 0);

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
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int k0 = key0 + i * kKeysPerWave;
    if (k0 >= ctx_v) break;  // wave-uniform
    if (i + 1 < NG && k0 + kKeysPerWave < ctx_v) load_group(i + 1, (i + 1) & 1);
    const int nvalid = min(kKeysPerWave, ctx_v - k0);
    if constexpr (NMT == 1 && WB == 1) {
      if (vec_out) {
        // the group's scores in registers, then out in whole lines: val[t] is
        // key 16t + lane%16; through the wave's LDS slice to keys 4(lane%16)..+3,
        // so 16 lanes write a 64-key row piece with 16-byte stores
        float val[kKeysPerWave / kKeysPerTile];
        score_wave_values<NP, 1>(cv[i & 1], sv[i & 1], nu_l[i & 1], ga_l[i & 1], s_codes[wv], s_signs[wv], a,
                                 cst[0], kappa, lane, val);
        const int kl = lane & 15;
        float* st = reinterpret_cast<float*>(s_codes[wv]) + g * kKeysPerWave;
#pragma unroll
        for (int t = 0; t < kKeysPerWave / kKeysPerTile; ++t) st[kKeysPerTile * t + kl] = val[t];
        __builtin_amdgcn_wave_barrier();
        const v4f o = *reinterpret_cast<const v4f*>(st + 4 * kl);
        __builtin_amdgcn_wave_barrier();  // read before the next group's staging
        if (out[0] != nullptr) {
          float* orow = out[0] + i * kKeysPerWave;
          if (4 * kl + 3 < nvalid) {
            __builtin_nontemporal_store(o, reinterpret_cast<v4f*>(orow + 4 * kl));
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (4 * kl + e < nvalid) __builtin_nontemporal_store(o[e], orow + 4 * kl + e);
          }
        }
        continue;
      }
    }
    float* oi[NMT];
#pragma unroll
    for (int j = 0; j < NMT; ++j) oi[j] = out[j] ? out[j] + i * kKeysPerWave : nullptr;
    score_wave<NP, WB, NMT>(cv[i & 1], sv[i & 1], nu_l[i & 1], ga_l[i & 1], s_codes[wv], s_signs[wv], a, cst, oi,
                            nvalid, kappa, lane);
    __builtin_amdgcn_wave_barrier();  // the next group's LDS staging follows this group's reads
  }
}

// ----------------------------------------------------------------------------
// Fused logits (d = 128, one M-tile of 4 query vectors per KV head): every
// block rebuilds the query operands of its (batch, kv head) in LDS while its
// records are in flight (query_prep_*), so a decode step is one launch.
// The logits leave in whole lines: each wave's four 16-key tiles go through
// its LDS slice and come back as four consecutive keys per lane, so a row of
// 64 keys is written by 16 lanes with 16-byte stores (two full 128-byte
// lines) instead of four 64-byte pieces.  vec_out = 0 (ctx not a multiple of
// 4, or logits not 16-byte aligned) keeps the scalar stores.
// ----------------------------------------------------------------------------
// PAGED: the records of sequence b's position t sit at row
// (page_table[b][t / page_size] * nkv + kh) * page_size + t % page_size, and b
// scores its first min(ctx_lens[b], ctx) positions (ctx = max_ctx, the logits
// row length); page_size is a multiple of 128, so a 64-key group lies in one
// page.  A block past its sequence's end exits before any barrier.
template <int NP, int WAVES, typename T, bool LOOP, bool PAGED>
__global__ __launch_bounds__(WAVES * 64) void logits_fused_kernel(
    const T* q, DevParams P, const float* Dsign, const float* Mt, int Hq, int nq, int G, int nkv, int ctx,
    const uint32_t* __restrict__ codes, const uint32_t* __restrict__ signs, const float* __restrict__ norm,
    const float* __restrict__ rnorm, float* __restrict__ logits, int vec_out, int ngw, PageMap pm) {
  using L = RecLayout<NP, 1>;
  constexpr int NT = WAVES * 64, NKB = L::NKB;
  __shared__ uint32_t s_codes[WAVES][kKeysPerWave * L::CS];
  __shared__ uint32_t s_signs[WAVES][kKeysPerWave * L::SS];
  __shared__ QueryPrepShared<NT, NKB> sh;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int bk = blockIdx.y;
  const QueryTile tile{bk / nkv, nq, Hq, G, bk % nkv, static_cast<int>(blockIdx.z), nq * G};
  // The block's keys: ngw rounds of WAVES consecutive 64-key groups, wave wv
  // taking group wv of each round (every round reads one contiguous range).
  const int blk0 = blockIdx.x * ngw * (WAVES * kKeysPerWave);
  int ctx_v = ctx;  // keys this row scores
  if constexpr (PAGED) {
    ctx_v = max(0, min(pm.ctx_lens[bk / nkv], ctx));
    if (blk0 >= ctx_v) return;  // block-uniform, before any barrier
  }
  auto group_key = [&](int i) { return blk0 + (i * WAVES + wv) * kKeysPerWave; };
  const int key0 = group_key(0);
  const bool active = key0 < ctx_v;  // wave-uniform; idle waves still help with the operands

  // The vector memory path returns data in request order, so an operand load
  // queued behind record loads (HBM misses) would wait for them: every wave's
  // operand loads are queued before any wave issues its records.  The barrier
  // waits for no data.
  QueryPrepRegs<NT> pr;
  query_prep_load<NT>(pr, q, Dsign, Mt, tile);
  __syncthreads();
  // Records, double-buffered: group i + 1 loads while group i is scored.  Every
  // wave loads its first group (an idle wave re-reads the last key and never
  // uses it), so no branch sits around the loads.
  v4u cvA[L::CW / 4], svA[L::SW / 4], cvB[L::CW / 4], svB[L::SW / 4];
  float nuA, gaA, nuB, gaB;
  auto load = [&](int k0, v4u (&cv)[L::CW / 4], v4u (&sv)[L::SW / 4], float& nu, float& ga) {
    const bool ok = k0 < ctx_v;
    const int key = ok ? k0 : ctx_v - 1;  // ctx_v >= 1 here (the block holds a key)
    int64_t row0 = static_cast<int64_t>(bk) * ctx + key;
    if constexpr (PAGED) {
      const int page = pm.table[static_cast<int64_t>(bk / nkv) * pm.max_pages + key / pm.page_size];
      row0 = (static_cast<int64_t>(page) * nkv + bk % nkv) * pm.page_size + key % pm.page_size;
    }
    load_wave_records<NP, 1>(cv, sv, nu, ga, codes + row0 * L::CW, signs + row0 * L::SW, norm + row0, rnorm + row0,
                             ok ? min(kKeysPerWave, ctx_v - k0) : 1, lane);
  };
  load(key0, cvA, svA, nuA, gaA);
  query_prep_build<NT, NP, NKB>(sh, pr, P, tile);
  if (!active) return;  // wave-uniform

  const int g = lane >> 4, kl = lane & 15;
  v8i a[1][NKB];
  query_prep_operands<NT, NKB>(sh, a, lane);
  const float4 cst = query_prep_constants<NT, NP, NKB>(sh, P, g);
  const int qvg = tile.mt * 4 + g;
  // a padding slot of the tile scores like the others (the matrix ops need
  // every lane) but stores nothing
  const bool store = qvg < tile.Gq;
  float* const orow0 =
      logits + (static_cast<int64_t>(tile.b * Hq + tile.kh * G + (store ? qvg % G : 0)) * nq + qvg / G) * ctx;
  // score group i from (cv, sv, nu, ga); group i + 1 loads into (cvn, ...)
  // before the scoring (prefetch) or after it (the same registers)
  auto step = [&](int i, v4u (&cv)[L::CW / 4], v4u (&sv)[L::SW / 4], float& nu, float& ga, v4u (&cvn)[L::CW / 4],
                  v4u (&svn)[L::SW / 4], float& nun, float& gan, bool prefetch) {
    const int k0 = group_key(i);
    const bool more = i + 1 < ngw && group_key(i + 1) < ctx_v;
    if (prefetch && more) load(group_key(i + 1), cvn, svn, nun, gan);
    const int nvalid = min(kKeysPerWave, ctx_v - k0);
    float val[kKeysPerWave / kKeysPerTile];
    score_wave_values<NP, 1>(cv, sv, nu, ga, s_codes[wv], s_signs[wv], a, cst, P.qjl_kappa, lane, val);
    if (!prefetch && more) load(group_key(i + 1), cvn, svn, nun, gan);
    float* orow = orow0 + k0;
    if (vec_out) {
      // val[t] is key 16t + kl; through the wave's LDS slice to keys 4kl..4kl+3
      float* st = reinterpret_cast<float*>(s_codes[wv]) + g * kKeysPerWave;
#pragma unroll
      for (int t = 0; t < kKeysPerWave / kKeysPerTile; ++t) st[kKeysPerTile * t + kl] = val[t];
      __builtin_amdgcn_wave_barrier();
      const v4f o = *reinterpret_cast<const v4f*>(st + 4 * kl);
      __builtin_amdgcn_wave_barrier();  // read before the next group's staging
      if (store) {
        if (4 * kl + 3 < nvalid) {
          __builtin_nontemporal_store(o, reinterpret_cast<v4f*>(orow + 4 * kl));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * kl + e < nvalid) __builtin_nontemporal_store(o[e], orow + 4 * kl + e);
        }
      }
    } else if (store) {
#pragma unroll
      for (int t = 0; t < kKeysPerWave / kKeysPerTile; ++t)
        if (kKeysPerTile * t + kl < nvalid) __builtin_nontemporal_store(val[t], orow + kKeysPerTile * t + kl);
    }
  };
  if constexpr (LOOP) {
    for (int i = 0; i < ngw; i += 2) {
      if (group_key(i) >= ctx_v) break;  // wave-uniform
      step(i, cvA, svA, nuA, gaA, cvB, svB, nuB, gaB, true);
      if (i + 1 >= ngw || group_key(i + 1) >= ctx_v) break;
      step(i + 1, cvB, svB, nuB, gaB, cvA, svA, nuA, gaA, true);
    }
  } else {  // one round (ngw = 1)
    step(0, cvA, svA, nuA, gaA, cvB, svB, nuB, gaB, false);
  }
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
  if (c->prm.d != 128) return by_type.template operator()<4>();
  auto go128 = [&]<int NP, typename T>(const T* qq) -> hipError_t {
    hipLaunchKernelGGL((attn_prep_inblock_kernel<NP, T>), grid, dim3(1024), 0, s, qq, c->prm, c->dD, c->dMt,
                       n_q_heads, n_queries, G, n_kv_heads, n_mt, static_cast<uint8_t*>(ws));
    return hipGetLastError();
  };
  auto by_np = [&]<typename T>(const T* qq) -> hipError_t {
    switch (c->prm.n_planes) {
      case 1: return go128.template operator()<1>(qq);
      case 2: return go128.template operator()<2>(qq);
      case 4: return go128.template operator()<4>(qq);
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

constexpr int kFusedWaves = 16;  // 1024 keys per fused block

// Rounds of 64-key groups per wave of the fused kernel: enough that the grid
// is about one block per compute unit (each block then rebuilds its operands
// once and streams ngw rounds of records), never more rounds than the context
// holds.
static int fused_groups_per_wave(int batch, int n_kv_heads, int64_t ctx) {
  const int64_t rounds = ceil_div(ctx, static_cast<int64_t>(kFusedWaves) * kKeysPerWave);
  const int64_t blocks1 = rounds * batch * n_kv_heads;
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(rounds, ceil_div(blocks1, device_cu_count()))));
}

hipError_t launch_logits_mfma(const tq_codec_s* c, const void* ws, int batch, int n_q_heads, int n_kv_heads,
                              int n_queries, tq_packed_t k, int64_t ctx, float* logits, hipStream_t s,
                              const PageMap* pm) {
  const PageMap pmv = pm ? *pm : PageMap{nullptr, nullptr, 0, 0};
  const int G = n_q_heads / n_kv_heads;
  const int n_mt = static_cast<int>(ceil_div(static_cast<int64_t>(n_queries) * G, 4));
  // whole-line stores need 16-byte aligned rows: ctx % 4 == 0 and aligned logits
  const int vec_out = ctx % 4 == 0 && reinterpret_cast<uintptr_t>(logits) % 16 == 0;
  auto go = [&]<int NP, int WB, int NMT>() -> hipError_t {
    constexpr int WAVES = WB == 1 ? 8 : 4;
    auto launch = [&]<int NG>() -> hipError_t {
      const dim3 grid(static_cast<unsigned>(ceil_div(ctx, WAVES * NG * kKeysPerWave)), batch * n_kv_heads,
                      static_cast<unsigned>(ceil_div(n_mt, NMT)));
      if (pm)
        hipLaunchKernelGGL((logits_mfma_kernel<NP, WB, NMT, WAVES, NG, true>), grid, dim3(WAVES * 64), 0, s,
                           static_cast<const uint8_t*>(ws), n_mt, static_cast<int>(ctx), k.codes, k.signs, k.norm,
                           k.rnorm, c->prm.qjl_kappa, logits, pmv, n_kv_heads, vec_out);
      else
        hipLaunchKernelGGL((logits_mfma_kernel<NP, WB, NMT, WAVES, NG, false>), grid, dim3(WAVES * 64), 0, s,
                           static_cast<const uint8_t*>(ws), n_mt, static_cast<int>(ctx), k.codes, k.signs, k.norm,
                           k.rnorm, c->prm.qjl_kappa, logits, pmv, n_kv_heads, vec_out);
      return hipGetLastError();
    };
    // Four groups per wave read the operands once per 256 keys (measured 49.8
    // against 56.9 us for the 16 x 8 x 8192-key, 16-query prefill scores) when
    // the grid still holds at least two blocks per compute unit.
    const int64_t blocks4 = ceil_div(ctx, WAVES * 4 * kKeysPerWave) * batch * n_kv_heads * ceil_div(n_mt, NMT);
    if (blocks4 >= 2 * device_cu_count()) return launch.template operator()<4>();
    return launch.template operator()<1>();
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
// 4 query vectors per KV head) and d = 128: about one block per compute unit,
// each rebuilding its operands in LDS while its first records are in flight,
// then streaming up to 4 rounds of records.  Measured at 32 heads x 32K keys
// (kernel times, same box): batch 2 11.6 us against 4.5 + 9.7 split, batch 4
// 17.4 against 4.2 + 17.1; at batch 16 (16 rounds) 66.5 against 5.4 + 54.4,
// so longer streams take the split form, whose 2048 blocks balance better.
// TQ_LOGITS_FUSED=0 turns it off.
bool logits_fused_eligible(const tq_codec_s* c, int batch, int n_q_heads, int n_kv_heads, int n_queries,
                           int64_t ctx) {
  const char* v = std::getenv("TQ_LOGITS_FUSED");
  if (v && std::string(v) == "0") return false;
  const int64_t nv = static_cast<int64_t>(n_queries) * (n_q_heads / n_kv_heads);
  const int ngw = fused_groups_per_wave(batch, n_kv_heads, ctx);
  return logits_mfma_eligible(c) && c->prm.d == 128 && nv <= 4 && ngw <= 4 && (ngw == 1 || c->prm.n_planes < 4);
}

hipError_t launch_logits_fused(const tq_codec_s* c, const void* q, tq_dtype_t dt, int batch, int n_q_heads,
                               int n_kv_heads, int n_queries, tq_packed_t k, int64_t ctx, float* logits,
                               hipStream_t s, const PageMap* pm) {
  // 16 waves (1024 keys) per block: one block per CU at the decode shapes, so
  // the operand rebuild is paid once per CU rather than twice (measured 8.7 us
  // against 9.2 us for 8-wave blocks at 32 query heads x 32K keys).
  constexpr int WAVES = kFusedWaves;
  const int G = n_q_heads / n_kv_heads;
  const int vec_out = ctx % 4 == 0 && reinterpret_cast<uintptr_t>(logits) % 16 == 0;
  const int ngw = fused_groups_per_wave(batch, n_kv_heads, ctx);
  auto go = [&]<int NP, typename T>(const T* qq) -> hipError_t {
    const dim3 grid(static_cast<unsigned>(ceil_div(ctx, static_cast<int64_t>(WAVES) * kKeysPerWave * ngw)),
                    batch * n_kv_heads, 1);
    // several rounds: the double-buffered loop (not for 72-byte records: their
    // second buffer does not fit 128 registers, and the split form takes them)
    auto pick = [&]<bool PG>() {
      auto kern = logits_fused_kernel<NP, WAVES, T, false, PG>;
      if constexpr (NP < 4) {
        if (ngw > 1) kern = logits_fused_kernel<NP, WAVES, T, true, PG>;
      }
      return kern;
    };
    auto kern = pm ? pick.template operator()<true>() : pick.template operator()<false>();
    hipLaunchKernelGGL(kern, grid, dim3(WAVES * 64), 0, s, qq, c->prm, c->dD, c->dMt, n_q_heads, n_queries, G,
                       n_kv_heads, static_cast<int>(ctx), k.codes, k.signs, k.norm, k.rnorm, logits, vec_out, ngw,
                       pm ? *pm : PageMap{nullptr, nullptr, 0, 0});
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

// Fused decode attention on the CDNA4 matrix cores (d = 128 for K and V, at
// most 4 query heads per KV head).
//
// One block per (batch*kv_head, chunk of 1024 keys), 8 waves of 128 keys:
//   1. the K records load; the K query operands of the head (prepared once per
//      KV head by attn_prep_mfma_kernel, the logits path's prep) come from L2;
//   2. each wave scores its 128 keys on the matrix cores (score_wave_values);
//   3. softmax against the chunk's per-head maximum;
//   4. V is accumulated in the codec domain on the matrix cores:
//        M[g][j] = Σ_k w_gk ν_k c(idx_kj),   J[g][i] = Σ_k w_gk ν_k γ_k τ_ki,
//      a contraction over keys, with the softmax weights as fp8 limb A
//      operands and the V bit planes as fp4 B operands;
//   5. the chunk partials (max, Σw, M, J) go to the combine kernel, which
//      merges the chunks (log-sum-exp) and maps back to the input domain.
// The Sparse V variant (GATE) drops the value term of a (query head, key)
// whose weight normalised within the chunk, exp(s - m_c) / l_c, is below the
// gate, and a wave whose 128 keys are all dropped for every head of its group
// loads no V record and runs none of step 4.  The normaliser keeps every key.
// With an MSE-only V codec (VQ = false) the V records hold codes and ν only:
// step 4 has no J, and the partials are (max, Σw, M).
// Pages: 「谷歌 TurboQuant 深度拆解」 第二部分 (the unbiased estimator);
// 「TurboQuant+ 深度解析」 第五部分 (V compressed like K) and 第六部分 (V
// dequantization dominates long-context decode).
//
// V as a matrix operand.  The contraction over keys needs, in each lane, the
// bits of one coordinate across 32 keys, while a row record holds 32
// coordinates of one key.  With row records (VB = false) each lane loads the V
// records of two keys and a 32x32 bit transpose runs in registers: four lane
// stages (lane bits 0-3, partners through DPP within rows of 16) and one
// stage between the lane's two registers.  The key each lane loads is chosen
// so that the transposed words land exactly in the B-operand layout with
// contraction index = key index (see v_key_of_row).  A V cache in 32-key
// blocks (VB, tq_codec_create_vblock) holds those transposed words already,
// written once at encode by the same transpose, and the lanes load them as
// they are.  The parity plane of a 3-bit codebook is the XOR of the stored
// planes' words.
#include <cstdlib>
#include <string>

#include "mfma_common.h"

namespace tq {

namespace {

constexpr int kDecWaves = 8;
constexpr int kDecKeysPerWave = 128;
constexpr int kDecChunk = kDecWaves * kDecKeysPerWave;  // keys per block

}  // namespace

template <int NPK, int NPV, bool GATE, bool PAGED, bool VQ, bool VB>
__global__ __launch_bounds__(kDecWaves * 64) void decode_mfma_kernel(
    const uint8_t* __restrict__ prep, DevParams PK, DevParams PV, PageMap pm, int Hq, int nkv, int ctx_max,
    int n_chunks, float scale, float gate, const uint32_t* __restrict__ kc, const uint32_t* __restrict__ ks,
    const float* __restrict__ kn, const float* __restrict__ kr, const uint32_t* __restrict__ vc,
    const uint32_t* __restrict__ vs, const float* __restrict__ vn, const float* __restrict__ vr,
    float* __restrict__ part) {
  using LK = RecLayout<NPK, 1>;
  using LV = RecLayout<NPV, 1>;
  constexpr int NT = kDecWaves * 64, NKB = LK::NKB, NBV = LV::NB;
  constexpr int KSTAGE = kKeysPerWave * (LK::CS + LK::SS);
  constexpr int SCR = KSTAGE > 1024 ? KSTAGE : 1024;  // words of per-wave scratch
  constexpr int NTY = VQ ? 2 : 1;                      // V weight types: MSE (and QJL)
  constexpr int REC = 2 + (VQ ? 2 : 1) * kPrepD;       // floats per partial record
  __shared__ __attribute__((aligned(16))) uint32_t wsc[kDecWaves][SCR];
  __shared__ float hmax[kDecWaves][4];
  __shared__ int ubexp[kDecWaves][2][4][4];  // V weight block exponents [type][head][key block]
  __shared__ float hsum[kDecWaves][4][4];
  // wave index through readfirstlane: every per-wave quantity is then known uniform (scalar registers)
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int g = lane >> 4, kl = lane & 15;
  int bk = blockIdx.y, chunk = blockIdx.x;
  if constexpr (PAGED) {
    // Blocks take the (sequence, KV head, chunk) items that hold positions in
    // order, so the grid's empty chunks (it is sized by the longest context)
    // all come last and exit at once instead of sitting between the work.
    // Every wave derives the same item from ctx_lens (no LDS, no barrier).
    const int batch = gridDim.y / nkv;
    const int64_t item = blockIdx.x + static_cast<int64_t>(blockIdx.y) * gridDim.x;
    int64_t base = 0;
    bool found = false;
    for (int b0 = 0; b0 < batch && !found; b0 += 64) {
      const int b = b0 + lane;
      const int cb = b < batch ? (max(0, min(pm.ctx_lens[b], ctx_max)) + kDecChunk - 1) / kDecChunk : 0;
      const int64_t items = static_cast<int64_t>(cb) * nkv;
      int64_t incl = items;  // inclusive prefix over the lanes
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int64_t o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
      }
      const int64_t total = __shfl(incl, 63, 64);
      if (item < base + total) {
        const unsigned long long hit = __ballot(base + incl > item);
        const int bl = __builtin_ctzll(hit);  // the item's sequence, lane of this round
        const int64_t excl = base + __shfl(incl - items, bl, 64);
        const int cbl = __shfl(cb, bl, 64);
        const int r = static_cast<int>(item - excl);
        bk = __builtin_amdgcn_readfirstlane((b0 + bl) * nkv + r / cbl);
        chunk = __builtin_amdgcn_readfirstlane(r % cbl);
        found = true;
      }
      base += total;
    }
    if (!found) return;  // past every sequence's positions (block-uniform)
  }
  const int G = Hq / nkv;
  const int kbase = chunk * kDecChunk + wv * kDecKeysPerWave;  // first key of the wave (within the head)
  const int64_t hrow = static_cast<int64_t>(bk) * ctx_max;     // first row of the head (contiguous cache)
  // the sequence's context: ctx_max for a contiguous cache; for a paged one its
  // own length, clamped to the grid (the host checks ctx_max <= max_pages *
  // page_size, so the clamp keeps every position inside the page table)
  int ctx = ctx_max;
  if constexpr (PAGED) ctx = max(0, min(pm.ctx_lens[bk / nkv], ctx_max));
  // a chunk past a shorter sequence's end: the combine reads only the chunks in use
  if (PAGED && chunk * kDecChunk >= ctx) return;  // block-uniform
  // Record rows.  Every key the wave touches, clamped to ctx - 1, lies in the
  // wave's 128-key block, or for a wave past the end in the block of key
  // ctx - 1; page_size is a multiple of 128, so that block sits in one page,
  // found with one page-table read per wave: row(key) = wrow + key - wkey.
  const int wkey = kbase < ctx ? kbase : ((ctx - 1) & ~(kDecKeysPerWave - 1));
  int64_t wrow = hrow + wkey;
  if constexpr (PAGED) {
    const int page = pm.table[static_cast<int64_t>(bk / nkv) * pm.max_pages + wkey / pm.page_size];
    wrow = (static_cast<int64_t>(page) * nkv + bk % nkv) * pm.page_size + wkey % pm.page_size;
  }
  auto row_of = [&](int key) -> int64_t { return wrow + (key - wkey); };

  // ---- loads: the K records, then the head's query operands (prepared once
  // per KV head by attn_prep_inblock_kernel; L2-resident)
  v4u kcv[2][LK::CW / 4], ksv[2][LK::SW / 4];
  float knu[2], kga[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k0 = kbase + 64 * h;
    const int nv = min(64, ctx - k0);  // may be <= 0: then re-read the last key, never used
    const int64_t r0 = row_of(nv > 0 ? k0 : ctx - 1);
    load_wave_records<NPK, 1>(kcv[h], ksv[h], knu[h], kga[h], kc + r0 * LK::CW, ks + r0 * LK::SW, kn + r0,
                              kr + r0, nv > 0 ? nv : 1, lane);
  }

  // ---- K query operands, then logits of the wave's 128 keys (8 per lane)
  float s[8];
  {
    v8i a[1][NKB];
    const uint8_t* base = prep + static_cast<int64_t>(bk) * (NKB * kOpBytes + kConstBytes);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const uint4* src = reinterpret_cast<const uint4*>(base + kb * kOpBytes + lane * 32);
      const uint4 x = src[0], y = src[1];
      a[0][kb][0] = x.x; a[0][kb][1] = x.y; a[0][kb][2] = x.z; a[0][kb][3] = x.w;
      a[0][kb][4] = y.x; a[0][kb][5] = y.y; a[0][kb][6] = y.z; a[0][kb][7] = y.w;
    }
    const float4 cst = reinterpret_cast<const float4*>(base + NKB * kOpBytes)[g];
    uint32_t* stage = wsc[wv];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float val[4];
      score_wave_values<NPK, 1>(kcv[h], ksv[h], knu[h], kga[h], stage, stage + kKeysPerWave * LK::CS, a, cst,
                                PK.qjl_kappa, lane, val);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int key = kbase + 64 * h + 16 * t + kl;
        s[4 * h + t] = (key < ctx && g < G) ? scale * val[t] : -INFINITY;
      }
    }
  }

  // V: lane loads the whole records of keys kbase + 32·(lane/16) + v_key_of_row(lane%16 + 16·reg),
  // and ν, γ of V for the scoring layout (key 16t + lane%16 of the wave).
  // Issued only after the scores: held through the query prep they push the
  // kernel past 128 registers, and then a CU runs one 8-wave block instead of
  // two.  The gated kernel issues them once the gate has kept the wave.
  // VB (V in 32-key blocks, written so at encode): the lane's words are
  // already the B operands: words 8·(lane%16)..+7 of each plane of its block
  // (keys kbase + 32·(lane/16)..+31), coordinate 16·cb + lane%16 in word cb;
  // vcv[0] holds cb 0..3, vcv[1] cb 4..7.
  v4u vcv[2][NBV], vsv[2];
  float vnu[8], vga[8];
  auto load_v = [&]() {
    if constexpr (VB) {
      const int key = min(kbase + 32 * g, (ctx - 1) & ~31);  // a block past the end re-reads the last one
      const int64_t blk = row_of(key) >> 5;
#pragma unroll
      for (int p = 0; p < NBV; ++p) {
        const v4u* src = reinterpret_cast<const v4u*>(vc + ((blk * NBV + p) * 128 + kl * 8));
        vcv[0][p] = src[0];
        vcv[1][p] = src[1];
      }
      if constexpr (VQ) {
        const v4u* src = reinterpret_cast<const v4u*>(vs + (blk * 128 + kl * 8));
        vsv[0] = src[0];
        vsv[1] = src[1];
      }
    } else {
#pragma unroll
      for (int reg = 0; reg < 2; ++reg) {
        const int key = min(kbase + 32 * g + v_key_of_row(kl + 16 * reg), ctx - 1);
        const int64_t row = row_of(key);
#pragma unroll
        for (int p = 0; p < NBV; ++p) vcv[reg][p] = reinterpret_cast<const v4u*>(vc)[row * NBV + p];
        if constexpr (VQ) vsv[reg] = reinterpret_cast<const v4u*>(vs)[row];
      }
    }
    // ν, γ through buffers over the wave's rows from wkey (scalar base), one
    // offset register: keys at or past ctx read 0 (their weight is 0)
    {
      const int nb = __builtin_amdgcn_readfirstlane(min(max(ctx - wkey, 0), 2 * kDecKeysPerWave) * 4);
      const __amdgpu_buffer_rsrc_t rn = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(vn + wrow), 0, nb, 0x00020000);
      const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(vr + wrow), 0, nb, 0x00020000);
      const int off = (kbase - wkey + kl) * 4;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        vnu[t] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rn, off + 64 * t, 0, 0));
        if constexpr (VQ) vga[t] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rr, off + 64 * t, 0, 0));
      }
    }
  };
  if constexpr (!GATE) load_v();

  // ---- chunk maximum per head
  {
    float m = s[0];
#pragma unroll
    for (int t = 1; t < 8; ++t) m = fmaxf(m, s[t]);
    m = row_max_rot(m);
    if (kl == 0) hmax[wv][g] = m;
  }
  __syncthreads();
  float mg = hmax[0][g];
#pragma unroll
  for (int w = 1; w < kDecWaves; ++w) mg = fmaxf(mg, hmax[w][g]);

  // ---- softmax weights against the chunk maximum; the sum keeps every key
  float wt[8];
  float l_sum = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    wt[t] = s[t] == -INFINITY ? 0.f : __expf(s[t] - mg);
    l_sum += wt[t];
  }
  l_sum = row_sum_rot(l_sum);  // lane kl = 0's is stored
  if (kl == 0) hsum[wv][g][0] = l_sum;
  bool wave_on = true;
  if constexpr (GATE) {
    // Sparse V gate: keep (head, key) iff exp(s - m_c) >= gate · l_c
    __syncthreads();
    float lc = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) lc += hsum[w][g][0];
    const float thr = gate * lc;
    bool any = false;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      wt[t] = wt[t] >= thr ? wt[t] : 0.f;
      any = any || wt[t] > 0.f;
    }
    wave_on = __builtin_amdgcn_ballot_w64(any) != 0;  // heads g >= G have no weight
  }
  float macc[8], jacc[8];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) macc[cb] = jacc[cb] = 0.f;
  if (!wave_on) {
    if (kl == 0) hsum[wv][g][1] = hsum[wv][g][2] = hsum[wv][g][3] = 0.f;
  } else {
    if constexpr (GATE) load_v();

    // ---- the V weight operands.
    // The matrix op aligns the products of each group of 8 contraction
    // elements to the largest and keeps 13 bits below it (measured on gfx950),
    // so floating-point limbs of weights that span many octaves lose the small
    // ones.  Instead u = w ν (MSE) and u = 2 w ν γ (QJL) become 16-bit fixed
    // point V relative to the maximum of their (head, 32-key block): four
    // base-16 digits, each an exact fp8 integer (times the nibble's 1/value),
    // so every product sum is exact.  The block exponent and the digit weight
    // go into the op's per-block E8M0 scale (row r, keys 32b..32b+31: lane
    // 16b + r).  LW[type][g][key] = the key's four digit bytes, byte j = digit
    // of weight 16^j; ub = block exponents.
    // Digit bytes in integer arithmetic: the nibbles of V spread to bytes, then
    // a byte-wise table lookup: v_perm over the lane's 8-entry table of
    // fp8(d / value) for d < 8, and fp8(d / value) = d + C for d >= 8 (the
    // exponent is then fixed: fp8 e4m3 of 8..15 times 2^k is 0x48 + 8k + d).
    // The key's FP4 mask index r = 2·(t odd) + (lane%16 >= 8) fixes the value
    // 1/2, 1, 2 or -2 (r = 0..3) the op multiplies the digit by.
    uint32_t* LW = wsc[wv];
    {
      const bool hi8 = kl >= 8;
      // tables for t even (r = 0 or 1) and t odd (r = 2 or 3): fp8 of d·{2, 1, 0.5, -0.5}
      const uint32_t tlo_e = hi8 ? 0x44403800u : 0x4C484000u, thi_e = hi8 ? 0x4E4C4A48u : 0x56545250u;
      const uint32_t tlo_o = hi8 ? 0xBCB8B080u : 0x3C383000u, thi_o = hi8 ? 0xC6C4C2C0u : 0x46444240u;
      const uint32_t c8_e = hi8 ? 0x48484848u : 0x50505050u, c8_o = hi8 ? 0xC0C0C0C0u : 0x40404040u;
      float u[NTY][8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        u[0][t] = wt[t] * vnu[t];
        if constexpr (VQ) u[NTY - 1][t] = 2.f * u[0][t] * vga[t];
      }
      float w_all = 0.f, w_3 = 0.f, q_n3 = 0.f;
#pragma unroll
      for (int ty = 0; ty < NTY; ++ty) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {  // block kb = keys 32kb..32kb+31 = tiles 2kb, 2kb+1
          const float m = row_max_nonneg(__uint_as_float(max(__float_as_uint(u[ty][2 * kb]), __float_as_uint(u[ty][2 * kb + 1]))));
          int e = 0;
          (void)frexpf(m, &e);               // m in [2^(e-1), 2^e); 0 for m = 0
          const int eb = max(e - 1, -100);   // every u of the block is below 2^(eb+1)
          if (kl == 0) ubexp[wv][ty][g][kb] = eb;
          const float scl = __uint_as_float(static_cast<uint32_t>(127 + 15 - eb) << 23);  // 2^(15 - eb)
          const float isc = __uint_as_float(static_cast<uint32_t>(127 - 15 + eb) << 23);  // 2^(eb - 15)
          uint32_t V[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int t = 2 * kb + h;
            // round to nearest (u >= 0), 16 bits
            V[h] = min(static_cast<uint32_t>(fmaf(u[ty][t], scl, 0.5f)), 65535u);
            const uint32_t y = (V[h] | (V[h] << 8)) & 0x00FF00FFu;
            const uint32_t z = (y | (y << 4)) & 0x0F0F0F0Fu;  // byte j = nibble j
            const uint32_t lo = __builtin_amdgcn_perm(h ? thi_o : thi_e, h ? tlo_o : tlo_e, z);  // d < 8
            const uint32_t hi = z + (h ? c8_o : c8_e);                                           // d >= 8
            // byte j from lo (selector j) or, where d >= 8, from hi (selector 4 + j)
            const uint32_t sel = ((z >> 1) & 0x04040404u) | 0x03020100u;
            LW[(ty * 4 + g) * kDecKeysPerWave + 16 * t + kl] = __builtin_amdgcn_perm(hi, lo, sel);
          }
          // the values the digits carry, for the constant terms: every key
          // (MSE), the r = 3 keys (MSE), the r != 3 keys (QJL, halved)
          if (ty == 0) {
            w_all = fmaf(static_cast<float>(V[0] + V[1]), isc, w_all);
            w_3 = fmaf(static_cast<float>(hi8 ? V[1] : 0u), isc, w_3);
          } else {
            q_n3 = fmaf(static_cast<float>(V[0] + (hi8 ? 0u : V[1])), 0.5f * isc, q_n3);
          }
        }
      }
      w_all = row_sum_rot(w_all);  // lane kl = 0's are stored
      w_3 = row_sum_rot(w_3);
      q_n3 = row_sum_rot(q_n3);
      if (kl == 0) {
        hsum[wv][g][1] = w_all;
        hsum[wv][g][2] = w_3;
        hsum[wv][g][3] = q_n3;
      }
    }
    __builtin_amdgcn_wave_barrier();
    // A operands: lane (row 4g'+l, group grp) holds digit l (weight 16^(3-l),
    // byte 3 - l of the LW words) of keys 16grp..+15 and 64+16grp..+15 (A byte
    // order measured on gfx950); its E8M0 scale serves row 4g'+l of key block
    // grp: 2^(block exponent - 3 - 4l).
    v8i av[NTY];
    int sav[NTY];
    {
      const int row = lane & 15, grp = lane >> 4, gq = row >> 2, l = row & 3;
      const uint32_t sel = static_cast<uint32_t>(3 - l) | (static_cast<uint32_t>(7 - l) << 8) | 0x0C0C0000u;
#pragma unroll
      for (int ty = 0; ty < NTY; ++ty) {
        const uint32_t* src = LW + (ty * 4 + gq) * kDecKeysPerWave;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int key0 = (j < 4 ? 16 * grp + 4 * j : 64 + 16 * grp + 4 * (j - 4));
          const v4u d4 = *reinterpret_cast<const v4u*>(src + key0);
          const uint32_t lo = __builtin_amdgcn_perm(d4[1], d4[0], sel);
          const uint32_t hi = __builtin_amdgcn_perm(d4[3], d4[2], sel);
          av[ty][j] = static_cast<int>((lo & 0xFFFFu) | (hi << 16));
        }
        sav[ty] = 127 + ubexp[wv][ty][gq][grp] - 3 - 4 * l;
      }
    }
    __builtin_amdgcn_wave_barrier();

    // ---- V on the matrix cores: per plane and 16-coordinate block cb,
    // Σ_k A[row][k] B[k][n] with B the transposed bits of coordinate 16cb + n
    uint32_t par[8];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) par[cb] = 0u;
    const v4f zero = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < NBV + (VQ ? 1 : 0); ++p) {  // stored planes, then the signs
      uint32_t tw[8];
      if constexpr (VB) {
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) tw[cb] = p < NBV ? vcv[cb >> 2][p < NBV ? p : 0][cb & 3] : vsv[cb >> 2][cb & 3];
      } else {
#pragma unroll
        for (int wb = 0; wb < 4; ++wb) {
          uint32_t r0 = p < NBV ? vcv[0][p < NBV ? p : 0][wb] : vsv[0][wb];
          uint32_t r1 = p < NBV ? vcv[1][p < NBV ? p : 0][wb] : vsv[1][wb];
          transpose32(r0, r1, lane);
          tw[2 * wb] = r0;
          tw[2 * wb + 1] = r1;
        }
      }
      // two halves of four 16-coordinate blocks keep the live accumulators at 8 registers
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        v4f acc[4], accp[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[c] = mfma_fp8_fp4_scaled(p < NBV ? av[0] : av[NTY - 1], fp4_operand(tw[4 * hb + c]), zero,
                                       p < NBV ? sav[0] : sav[NTY - 1]);
        if constexpr (NPV > NBV) {  // parity plane once the last stored plane is in
          if (p == NBV - 1) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
              accp[c] = mfma_fp8_fp4_scaled(av[0], fp4_operand(par[4 * hb + c] ^ tw[4 * hb + c]), zero, sav[0]);
          }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) asm volatile("" : "+v"(acc[c]));
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int cb = 4 * hb + c;
          const float v = (acc[c][0] + acc[c][1]) + (acc[c][2] + acc[c][3]);  // digit weights are in the scales
          if (p < NBV) {
            macc[cb] = fmaf(PV.plane_coef[p < NBV ? p : 0], v, macc[cb]);
            par[cb] ^= tw[cb];
          } else {
            jacc[cb] = v;
          }
        }
        if constexpr (NPV > NBV) {
          if (p == NBV - 1) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              asm volatile("" : "+v"(accp[c]));
              const float v = (accp[c][0] + accp[c][1]) + (accp[c][2] + accp[c][3]);
              macc[4 * hb + c] = fmaf(PV.plane_coef[NPV - 1], v, macc[4 * hb + c]);
            }
          }
        }
      }
    }

  }  // wave_on

  // ---- chunk partials: sum the 8 waves, add the per-head constant terms
  __syncthreads();  // every wave is done with its scratch
  {
    float* red = reinterpret_cast<float*>(wsc[wv]);
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      red[cb * 64 + lane] = macc[cb];
      if constexpr (VQ) red[(8 + cb) * 64 + lane] = jacc[cb];
    }
  }
  __syncthreads();
  float csum = 0.f;
#pragma unroll
  for (int k = 0; k < NPV; ++k) csum += PV.plane_coef[k];
  for (int e = threadIdx.x; e < (VQ ? 16 : 8) * 64; e += NT) {
    const int slot = e >> 6, L = e & 63, gh = L >> 4;
    if (gh >= G) continue;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) v += reinterpret_cast<const float*>(wsc[w])[e];
    float l_sum = 0.f, w_all = 0.f, w_3 = 0.f, q_n3 = 0.f, m = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      l_sum += hsum[w][gh][0];
      w_all += hsum[w][gh][1];
      w_3 += hsum[w][gh][2];
      q_n3 += hsum[w][gh][3];
      m = fmaxf(m, hmax[w][gh]);
    }
    const bool is_m = slot < 8;
    const int j = 16 * (slot & 7) + (L & 15);
    v += is_m ? PV.plane_bias * w_all + 0.5f * csum * w_3 : -q_n3;
    float* out = part + ((static_cast<int64_t>(bk) * n_chunks + chunk) * G + gh) * REC;
    out[2 + (is_m ? 0 : kPrepD) + j] = v;
    if (e == gh * 16) {  // one thread per head writes the max and the weight sum
      out[0] = m;
      out[1] = l_sum;
    }
  }
}

// d = 128 for K and V (QJL dimension 128, or an MSE-only V codec), at most 4
// query heads per KV head.
bool decode_mfma_shape_ok(const tq_codec_s* ck, const tq_codec_s* cv, int n_q_heads, int n_kv_heads) {
  const int G = n_q_heads / n_kv_heads;
  return ck->prm.d == 128 && cv->prm.d == 128 && ck->prm.m == 128 && (cv->prm.m == 128 || !cv->qjl) && G <= 4;
}

// The same, unless TQ_DECODE_KERNEL=valu asks for the general kernel (which
// reads row records only, so paged and blocked V caches ignore it).
bool decode_mfma_eligible(const tq_codec_s* ck, const tq_codec_s* cv, int n_q_heads, int n_kv_heads) {
  const char* v = std::getenv("TQ_DECODE_KERNEL");
  if (v && std::string(v) == "valu") return false;
  return decode_mfma_shape_ok(ck, cv, n_q_heads, n_kv_heads);
}

int decode_mfma_chunk() { return kDecChunk; }

// `prep`: the query operands of every (batch, KV head), as attn_prep_mfma_kernel writes them.
hipError_t launch_decode_mfma(const tq_codec_s* ck, const tq_codec_s* cv, int batch, int n_q_heads, int n_kv_heads,
                              tq_packed_t k, tq_packed_t v, int64_t ctx, float scale, bool sparse_v, float v_gate,
                              const PageMap* pm, const uint8_t* prep, float* part, int n_chunks, hipStream_t s) {
  const PageMap pmv = pm ? *pm : PageMap{nullptr, nullptr, 0, 0};
  auto go = [&]<int NPK, int NPV, bool VQ>() -> hipError_t {
    auto pick = [&]<bool VB>() {
      return pm ? (sparse_v ? decode_mfma_kernel<NPK, NPV, true, true, VQ, VB>
                            : decode_mfma_kernel<NPK, NPV, false, true, VQ, VB>)
                : (sparse_v ? decode_mfma_kernel<NPK, NPV, true, false, VQ, VB>
                            : decode_mfma_kernel<NPK, NPV, false, false, VQ, VB>);
    };
    auto kern = cv->vblock ? pick.template operator()<true>() : pick.template operator()<false>();
    hipLaunchKernelGGL(kern, dim3(n_chunks, batch * n_kv_heads), dim3(kDecWaves * 64),
                       0, s, prep, ck->prm, cv->prm, pmv, n_q_heads, n_kv_heads, static_cast<int>(ctx),
                       n_chunks, scale, v_gate, k.codes, k.signs, k.norm, k.rnorm, v.codes, v.signs, v.norm, v.rnorm,
                       part);
    return hipGetLastError();
  };
  auto by_v = [&]<int NPK>() -> hipError_t {
    if (!cv->qjl) {  // MSE-only V codecs: 2 or 3 code bits
      switch (cv->prm.n_planes) {
        case 2: return go.template operator()<NPK, 2, false>();
        case 4: return go.template operator()<NPK, 4, false>();
      }
      return hipErrorInvalidValue;
    }
    switch (cv->prm.n_planes) {
      case 1: return go.template operator()<NPK, 1, true>();
      case 2: return go.template operator()<NPK, 2, true>();
      case 4: return go.template operator()<NPK, 4, true>();
    }
    return hipErrorInvalidValue;
  };
  switch (ck->prm.n_planes) {
    case 1: return by_v.template operator()<1>();
    case 2: return by_v.template operator()<2>();
    case 4: return by_v.template operator()<4>();
  }
  return hipErrorInvalidValue;
}

}  // namespace tq

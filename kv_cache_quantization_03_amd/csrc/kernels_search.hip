// Exhaustive search over a compressed database: estimator scores per DB chunk,
// exact top-k per (query, chunk) by radix select on the score bits, then the
// same selection over the per-chunk candidates.
//
// Pages: 「谷歌 TurboQuant 深度拆解」 第三部分 向量搜索 (the compressed vectors
// are the index; nothing is trained) and 第二部分 (unbiased inner-product
// estimate from a full-precision query).
#include "kernels_common.h"

namespace tq {

hipError_t launch_scores(const tq_codec_s* c, const float* qrot, const float* proj, int nq, tq_packed_t db,
                         int64_t n, float* scores, hipStream_t s);
bool search_mfma_eligible(const tq_codec_s* c);
size_t search_mfma_prep_bytes(const tq_codec_s* c, int nq);
hipError_t launch_search_mfma_prep(const tq_codec_s* c, const float* qrot, const float* proj, int nq, void* prep,
                                   hipStream_t s);
hipError_t launch_search_mfma_scores(const tq_codec_s* c, const void* prep, int nq, tq_packed_t db, int64_t n,
                                     float* scores, int64_t ld, hipStream_t s);

// A polar codec's scores come from the polar scorer (the queries as the query
// heads of one KV head); the matrix-core search scorer reads per-coordinate codes.
static bool search_use_mfma(const tq_codec_s* c) { return !c->polar && search_mfma_eligible(c); }

namespace {
constexpr int64_t kSearchChunk = 65536;
constexpr int kSelThreads = 256;

// Sort key: ascending order of the key = descending order of the score.
__device__ __forceinline__ uint32_t desc_key(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;
}
__device__ __forceinline__ float key_to_score(uint32_t k) {
  const uint32_t asc = ~k;
  const uint32_t u = (asc & 0x80000000u) ? (asc & 0x7FFFFFFFu) : ~asc;
  return __uint_as_float(u);
}
}  // namespace

// One block per row.  Row r: scores src[r*src_stride + pos], pos < len_r;
// global index = idx_in ? idx_in[r*src_stride + pos] : idx_base + pos.
// Writes the k best (score desc, index asc) to out_score/out_idx[r*k ...].
// When len_r < k the tail is filled with (-inf, INT64_MAX).
__global__ __launch_bounds__(kSelThreads) void topk_rows_kernel(const float* __restrict__ src,
                                                                const int64_t* __restrict__ idx_in,
                                                                int64_t src_stride, int64_t len, int64_t idx_base,
                                                                int k, float* __restrict__ out_score,
                                                                int64_t* __restrict__ out_idx, int64_t out_stride) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sel_key[1024];
  __shared__ int64_t sel_idx[1024];
  __shared__ uint32_t sh_prefix, sh_need, sh_cnt_lt;
  __shared__ uint32_t scan[kSelThreads];
  const int r = blockIdx.x;
  const float* row = src + static_cast<int64_t>(r) * src_stride;
  const int64_t* irow = idx_in ? idx_in + static_cast<int64_t>(r) * src_stride : nullptr;
  const int tid = threadIdx.x;
  const int kk = static_cast<int>(min<int64_t>(k, len));
  auto gidx = [&](int64_t pos) -> int64_t { return irow ? irow[pos] : idx_base + pos; };

  uint32_t prefix = 0, mask = 0, need = kk;
  for (int pass = 0; pass < 4 && kk > 0; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    for (int64_t pos = tid; pos < len; pos += kSelThreads) {
      const uint32_t key = desc_key(row[pos]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t cum = 0, sel = 255;
      for (int bsel = 0; bsel < 256; ++bsel) {
        if (cum + hist[bsel] >= need) { sel = bsel; break; }
        cum += hist[bsel];
      }
      sh_prefix = prefix | (sel << shift);
      sh_need = need - cum;
    }
    __syncthreads();
    prefix = sh_prefix;
    need = sh_need;
    mask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t T = prefix;           // key of the kk-th best
  const uint32_t n_lt = kk - need;     // strictly better than T
  if (tid == 0) sh_cnt_lt = 0;
  __syncthreads();
  for (int64_t pos = tid; pos < len && kk > 0; pos += kSelThreads) {
    const uint32_t key = desc_key(row[pos]);
    if (key < T) {
      const uint32_t slot = atomicAdd(&sh_cnt_lt, 1u);
      sel_key[slot] = key;
      sel_idx[slot] = gidx(pos);
    }
  }
  // equal to T: the first `need` of them in position order (position order is
  // index order for both call sites)
  uint32_t taken = 0;
  for (int64_t base = 0; base < len && taken < need; base += kSelThreads) {
    const int64_t pos = base + tid;
    const uint32_t f = (pos < len && desc_key(row[pos]) == T) ? 1u : 0u;
    scan[tid] = f;
    __syncthreads();
    for (int off = 1; off < kSelThreads; off <<= 1) {
      const uint32_t v = tid >= off ? scan[tid - off] : 0u;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const uint32_t incl = scan[tid];
    const uint32_t total = scan[kSelThreads - 1];
    if (f && taken + incl - 1 < need) {
      const uint32_t slot = n_lt + taken + incl - 1;
      sel_key[slot] = T;
      sel_idx[slot] = gidx(pos);
    }
    taken += total;
    __syncthreads();
  }
  // pad and bitonic-sort by (key, idx)
  int P2 = 1;
  while (P2 < k) P2 <<= 1;
  for (int i = tid; i < P2; i += kSelThreads)
    if (i >= kk) {
      sel_key[i] = 0xFFFFFFFFu;
      sel_idx[i] = INT64_MAX;
    }
  __syncthreads();
  for (int size = 2; size <= P2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < P2; i += kSelThreads) {
        const int jx = i ^ stride;
        if (jx > i) {
          const bool up = (i & size) == 0;
          const uint32_t ka = sel_key[i], kb = sel_key[jx];
          const int64_t ia = sel_idx[i], ib = sel_idx[jx];
          const bool a_gt_b = (ka > kb) || (ka == kb && ia > ib);
          if (a_gt_b == up) {
            sel_key[i] = kb; sel_key[jx] = ka;
            sel_idx[i] = ib; sel_idx[jx] = ia;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < k; i += kSelThreads) {
    const int64_t o = static_cast<int64_t>(r) * out_stride + i;
    const bool real = i < kk;
    out_score[o] = real ? key_to_score(sel_key[i]) : -INFINITY;
    out_idx[o] = real ? sel_idx[i] : INT64_MAX;
  }
}

namespace {
constexpr int kTopThreads = 1024;
constexpr int kTopCap = 4096;  // candidates sorted in LDS
constexpr int kTopVPT = static_cast<int>(kSearchChunk / kTopThreads);  // scores per thread

// The want-th smallest (1-based) of the values val(i) with ok(i), over the
// VPT slots of every thread of the block, by 8-bit radix passes
// from the top.  Returns T and need = want - #(values < T) (>= 1).  Every
// thread of the block calls it; hist[257] and sel[2] are LDS scratch.
template <int PASSES, int VPT, typename V, typename OK>
__device__ __forceinline__ void block_radix_select(V val, OK ok, uint32_t want, uint32_t* hist, uint32_t* sel,
                                                   uint32_t& T, uint32_t& need) {
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t prefix = 0, mask = 0;
  need = want;
  for (int pass = 0; pass < PASSES; ++pass) {
    const int shift = 8 * (PASSES - 1 - pass);
    if (tid <= 256) hist[tid] = 0;
    __syncthreads();
    for (int i = 0; i < VPT; ++i) {  // values outside the prefix count in bin 256
      const uint32_t v = val(i);
      const bool in = ok(i) && (v & mask) == prefix;
      atomicAdd(&hist[in ? (v >> shift) & 255u : 256u], 1u);
    }
    __syncthreads();
    if (tid < 64) {  // wave 0: lane l scans bins 4l..4l+3
      uint32_t h[4], sum = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        h[b] = hist[4 * lane + b];
        sum += h[b];
      }
      uint32_t inc = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(inc, o, 64);
        if (lane >= o) inc += y;
      }
      uint32_t cum = inc - sum;
      if (cum < need && need <= inc) {  // exactly one lane
        int b = 0;
        while (cum + h[b] < need) cum += h[b++];
        sel[0] = 4 * lane + b;
        sel[1] = cum;
      }
    }
    __syncthreads();
    prefix |= sel[0] << shift;
    need -= sel[1];
    mask |= 255u << shift;
    __syncthreads();
  }
  T = prefix;
}
}  // namespace

// Top-k of one row of up to kSearchChunk scores per block, the row held in
// registers (one read of the scores).  Row r: src[r*len + pos]; global index
// idx_base + pos.  Writes the k best (score desc, index asc) to
// out_score/out_idx[r*out_stride ...]; when len < k the tail is (-inf, INT64_MAX).
//
// Candidates first: every thread's best key is a real score, so the k-th best
// of those 1024 bests, T0, has at least k scores at or above it and every
// member of the top k scores at least T0.  The scores at or above T0 (about
// 64k of them for k << 1024) go to LDS and are sorted there by (score desc,
// position asc).  When more than kTopCap pass (massive ties), the block falls
// back to an exact radix selection that re-reads the row.
__global__ __launch_bounds__(kTopThreads) void topk_regs_kernel(const float* __restrict__ src, int64_t len,
                                                                int64_t idx_base, int k,
                                                                float* __restrict__ out_score,
                                                                int64_t* __restrict__ out_idx, int64_t out_stride) {
  __shared__ uint32_t hist[257];
  __shared__ uint32_t sel[2];
  __shared__ uint32_t ck[kTopCap];
  __shared__ uint32_t cpos[kTopCap];
  __shared__ uint32_t cnt;
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  // buffer loads: one VGPR offset for all kTopVPT loads (the slot stride goes in
  // the scalar offset), and reads past the row's end return 0
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(src + static_cast<int64_t>(r) * len), 0, static_cast<int>(len * sizeof(float)), 0x00020000);
  const int nslot = static_cast<int>((len - tid + kTopThreads - 1) / kTopThreads);  // slots of this thread in the row
  // 0xFFFFFFFF marks an empty slot; a real score never maps there (a NaN that
  // would is moved one step up)
  auto load_key = [&](int i) {
    const uint32_t u = __builtin_amdgcn_raw_buffer_load_b32(rsrc, tid * 4, i * kTopThreads * 4, 0);
    return min(desc_key(__uint_as_float(u)), 0xFFFFFFFEu) | (i < nslot ? 0u : 0xFFFFFFFFu);
  };
  uint32_t key[kTopVPT];
#pragma unroll
  for (int i = 0; i < kTopVPT; ++i) key[i] = load_key(i);
  const uint32_t kk = static_cast<uint32_t>(min<int64_t>(k, len));
  uint32_t total = 0;
  if (kk > 0) {
    uint32_t best = key[0];
#pragma unroll
    for (int i = 1; i < kTopVPT; ++i) best = min(best, key[i]);
    uint32_t T0, need0;  // at least kk threads hold a key (kk <= min(len, kTopThreads))
    block_radix_select<4, 1>([&](int) { return best; }, [&](int) { return best != 0xFFFFFFFFu; }, kk, hist, sel,
                             T0, need0);
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < kTopVPT; ++i) c += key[i] <= T0 ? 1u : 0u;
    if (tid == 0) cnt = 0;
    __syncthreads();
    c = static_cast<uint32_t>(wave_sum(static_cast<float>(c)));  // exact: counts < 2^24
    if (lane == 0 && c) atomicAdd(&cnt, c);
    __syncthreads();
    total = cnt;
    __syncthreads();
    if (tid == 0) cnt = 0;
    __syncthreads();
    if (total <= kTopCap) {
#pragma unroll
      for (int i = 0; i < kTopVPT; ++i) {
        if (key[i] <= T0) {
          const uint32_t slot = atomicAdd(&cnt, 1u);
          ck[slot] = key[i];
          cpos[slot] = static_cast<uint32_t>(i * kTopThreads + tid);
        }
      }
    } else {
      // exact radix selection over the row, re-read from memory (no register copy
      // of the row is kept live through this path)
      asm volatile("" ::: "memory");
      uint32_t T, need;
      block_radix_select<4, kTopVPT>(load_key, [&](int i) { return i < nslot; }, kk, hist, sel, T, need);
      if (tid <= 256) hist[tid] = 0;
      __syncthreads();
      uint32_t my_eq = 0;
      for (int i = 0; i < nslot; ++i) my_eq += load_key(i) == T ? 1u : 0u;
      if (my_eq) atomicAdd(&hist[0], my_eq);
      __syncthreads();
      const uint32_t total_eq = hist[0];
      __syncthreads();  // hist is reused below
      uint32_t pos_cut = 0xFFFFFFFFu;  // keys equal to T with position <= pos_cut are taken
      if (total_eq > need) {
        uint32_t Tp, needp;
        block_radix_select<3, kTopVPT>([&](int i) { return static_cast<uint32_t>(i * kTopThreads + tid); },
                                       [&](int i) { return i < nslot && load_key(i) == T; }, need, hist, sel, Tp,
                                       needp);
        pos_cut = Tp;
      }
      for (int i = 0; i < nslot; ++i) {
        const uint32_t kx = load_key(i), pos = static_cast<uint32_t>(i * kTopThreads + tid);
        if (kx < T || (kx == T && pos <= pos_cut)) {
          const uint32_t slot = atomicAdd(&cnt, 1u);
          ck[slot] = kx;
          cpos[slot] = pos;
        }
      }
      total = kk;
    }
  }
  // sort the candidates by (key, position) and write the first kk
  int P2 = 1;
  while (P2 < static_cast<int>(max<uint32_t>(total, static_cast<uint32_t>(k)))) P2 <<= 1;
  __syncthreads();
  for (int i = static_cast<int>(total) + tid; i < P2; i += kTopThreads) {
    ck[i] = 0xFFFFFFFFu;
    cpos[i] = 0xFFFFFFFFu;
  }
  __syncthreads();
  for (int size = 2; size <= P2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < P2; i += kTopThreads) {
        const int jx = i ^ stride;
        if (jx > i) {
          const bool up = (i & size) == 0;
          const uint32_t ka = ck[i], kb = ck[jx], pa = cpos[i], pb = cpos[jx];
          const bool a_gt_b = (ka > kb) || (ka == kb && pa > pb);
          if (a_gt_b == up) {
            ck[i] = kb; ck[jx] = ka;
            cpos[i] = pb; cpos[jx] = pa;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < k; i += kTopThreads) {
    const int64_t o = static_cast<int64_t>(r) * out_stride + i;
    const bool real = i < static_cast<int>(kk);
    out_score[o] = real ? key_to_score(ck[i]) : -INFINITY;
    out_idx[o] = real ? idx_base + cpos[i] : INT64_MAX;
  }
}

namespace {
inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
struct SearchLayout {
  size_t qrot, proj, prep, scores, cand_idx, cand_score, total;
};
SearchLayout search_layout(const tq_codec_s* c, int64_t n_db, int nq, int topk) {
  const int64_t chunk = std::min<int64_t>(kSearchChunk, n_db);
  const int64_t n_chunks = ceil_div(n_db, chunk);
  SearchLayout L{};
  L.qrot = 0;
  L.proj = align256(L.qrot + static_cast<size_t>(nq) * c->prm.d * sizeof(float));
  L.prep = align256(L.proj + static_cast<size_t>(nq) * c->prm.m * sizeof(float));
  L.scores = L.prep + (search_use_mfma(c) ? search_mfma_prep_bytes(c, nq) : 0);
  L.cand_idx = align256(L.scores + static_cast<size_t>(nq) * chunk * sizeof(float));
  L.cand_score = align256(L.cand_idx + static_cast<size_t>(nq) * n_chunks * topk * sizeof(int64_t));
  L.total = align256(L.cand_score + static_cast<size_t>(nq) * n_chunks * topk * sizeof(float));
  return L;
}
}  // namespace

size_t search_ws_bytes(const tq_codec_s* c, int64_t n_db, int n_queries, int topk) {
  return search_layout(c, n_db, n_queries, topk).total;
}

hipError_t launch_search(const tq_codec_s* c, tq_packed_t db, int64_t n_db, const float* queries, int nq, int topk,
                         int64_t* out_idx, float* out_score, void* ws, hipStream_t s) {
  const DevParams& P = c->prm;
  const int64_t chunk = std::min<int64_t>(kSearchChunk, n_db);
  const int64_t n_chunks = ceil_div(n_db, chunk);
  char* w = static_cast<char*>(ws);
  const SearchLayout SL = search_layout(c, n_db, nq, topk);
  float* qrot = reinterpret_cast<float*>(w + SL.qrot);
  float* proj = reinterpret_cast<float*>(w + SL.proj);
  float* scores = reinterpret_cast<float*>(w + SL.scores);
  int64_t* cand_idx = reinterpret_cast<int64_t*>(w + SL.cand_idx);
  float* cand_score = reinterpret_cast<float*>(w + SL.cand_score);
  const bool mfma = search_use_mfma(c);
  hipError_t e = launch_qprep(c, queries, TQ_F32, nq, qrot, proj, s);
  if (e != hipSuccess) return e;
  if (mfma && (e = launch_search_mfma_prep(c, qrot, proj, nq, w + SL.prep, s)) != hipSuccess) return e;
  for (int64_t ci = 0; ci < n_chunks; ++ci) {
    const int64_t lo = ci * chunk;
    const int64_t len = std::min<int64_t>(chunk, n_db - lo);
    tq_packed_t sub{db.codes + lo * P.code_words, db.signs + lo * P.sign_words, db.norm + lo, db.rnorm + lo};
    // (qrot and proj are contiguous: nq·d floats is a multiple of 256 bytes)
    e = c->polar ? launch_logits_polar(c, qrot, 1, nq, 1, 1, sub, len, scores, s)
        : mfma   ? launch_search_mfma_scores(c, w + SL.prep, nq, sub, len, scores, len, s)
                 : launch_scores(c, qrot, proj, nq, sub, len, scores, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_regs_kernel, dim3(nq), dim3(kTopThreads), 0, s, scores, len, lo, topk,
                       cand_score + ci * topk, cand_idx + ci * topk, static_cast<int64_t>(n_chunks * topk));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(topk_rows_kernel, dim3(nq), dim3(kSelThreads), 0, s, cand_score, cand_idx,
                     static_cast<int64_t>(n_chunks * topk), static_cast<int64_t>(n_chunks * topk),
                     static_cast<int64_t>(0), topk, out_score, out_idx, static_cast<int64_t>(topk));
  return hipGetLastError();
}

}  // namespace tq

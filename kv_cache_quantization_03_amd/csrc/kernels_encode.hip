// Encode (rotate, quantize, pack, residual, QJL signs), the query-side rotation,
// and the S-projection GEMM used by both.
//
// Pages: 「谷歌 TurboQuant 深度拆解」 第二部分 (rotation, fixed scalar quantizer,
// 1-bit QJL signs of the projected residual); 「TurboQuant+ 深度解析」 第二部分
// (random-sign Walsh–Hadamard rotation) and 第四部分 (the rotation must be
// computed in high precision: here fp32 throughout); 「TurboQuant 学习路径」
// 二.4 (bit-packing into 32-bit words).
#include "kernels_common.h"

namespace tq {

// ----------------------------------------------------------------------------
// Rotate + quantize: one wavefront per vector.
//   ν = ||x||, y = H (D ⊙ x/ν)/√d, idx_j = #{k : t_k < y_j} (ties low),
//   r = y - c[idx] -> rbuf (fp32), γ = ||r||, codes packed as bit-planes.
// ----------------------------------------------------------------------------
template <int E, typename T>
__global__ __launch_bounds__(256) void encode_rq_kernel(const T* __restrict__ x, int64_t n, DevParams P,
                                                        const float* __restrict__ Dsign,
                                                        uint32_t* __restrict__ codes, float* __restrict__ norm,
                                                        float* __restrict__ rnorm, float* __restrict__ rbuf) {
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
  hadamard_wave<E>(v, lane);

  const int L = 1 << P.b;
  int idx[E];
  float rs = 0.f;
  float* rr = rbuf + vec * d;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float y = v[e] * P.inv_sqrt_d;
    int c = 0;
    float yh = P.cent[0];
    for (int k = 0; k < L - 1; ++k) {
      const bool gt = P.bound[k] < y;
      c += gt;
      yh = gt ? P.cent[k + 1] : yh;
    }
    idx[e] = c;
    const float r = y - yh;
    rr[e * kWave + lane] = r;
    rs = fmaf(r, r, rs);
  }
  rs = wave_sum(rs);

  // bit-plane packing: plane p, register e -> words p*(d/32) + 2e (+1)
  const int W = P.code_words;
  uint32_t* crow = codes + vec * W;
  for (int base = 0; base < W; base += kWave) {
    const int w = base + lane;
    uint32_t word = 0;
    for (int p = 0; p < P.b; ++p) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint64_t m = __ballot((idx[e] >> p) & 1);
        const int w0 = p * (d / 32) + 2 * e;
        word = (w == w0) ? static_cast<uint32_t>(m) : word;
        word = (w == w0 + 1) ? static_cast<uint32_t>(m >> 32) : word;
      }
    }
    if (w < W) crow[w] = word;
  }
  if (lane == 0) {
    norm[vec] = nu;
    rnorm[vec] = sqrtf(rs);
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
  hadamard_wave<E>(v, lane);
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

size_t encode_ws_bytes(const tq_codec_s* c, int64_t n) {
  return static_cast<size_t>(n) * c->prm.d * sizeof(float);
}

namespace {
template <typename T>
hipError_t encode_typed(const tq_codec_s* c, const T* x, int64_t n, tq_packed_t out, float* ws_r,
                        hipStream_t s) {
  const DevParams& P = c->prm;
  auto run = [&]<int E>() -> hipError_t {
    hipLaunchKernelGGL((encode_rq_kernel<E, T>), dim3(static_cast<unsigned>(ceil_div(n, 4))), dim3(256), 0, s,
                       x, n, P, c->dD, out.codes, out.norm, out.rnorm, ws_r);
    return hipGetLastError();
  };
  hipError_t e = dispatch_E(P.d, run);
  if (e != hipSuccess) return e;
  dim3 grid(static_cast<unsigned>(ceil_div(n, kTileV)), P.m / kTileI);
  hipLaunchKernelGGL((sproj_kernel<true>), grid, dim3(256), 0, s, ws_r, n, P.d, P.m, c->dS,
                     static_cast<float*>(nullptr), out.signs);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_encode(const tq_codec_s* c, const void* x, tq_dtype_t dt, int64_t n, tq_packed_t out,
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

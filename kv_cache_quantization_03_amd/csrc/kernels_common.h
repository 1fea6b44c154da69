// Device helpers shared by the gfx950 kernels: element loads, wavefront
// reductions, and the in-register Walsh–Hadamard rotation.
//
// Wavefront layout used for one d-vector: lane l of a 64-wide wave holds the
// E = d/64 coordinates j = e*64 + l (e = 0..E-1).  With this layout a ballot
// over the wave packs 64 consecutive coordinates into two 32-bit words.
#pragma once

#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "tq_internal.h"

namespace tq {

constexpr int kWave = 64;

__device__ __forceinline__ float load_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const __hip_bfloat16* p, int64_t i) {
  const uint16_t u = reinterpret_cast<const uint16_t*>(p)[i];
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}
__device__ __forceinline__ float load_elem(const __half* p, int64_t i) { return __half2float(p[i]); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

// Value of lane (lane ^ 2^K) within rows of 16 lanes, through DPP.
template <int K>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x) {
  const int v = static_cast<int>(x);
  if constexpr (K == 0) return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));
  if constexpr (K == 1) return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));
  if constexpr (K == 2) {  // quad reverse (i^3), then half-row mirror (i^7): i^4
    const int y = __builtin_amdgcn_update_dpp(0, v, 0x1B, 0xF, 0xF, false);
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, y, 0x141, 0xF, 0xF, false));
  }
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false));  // row_ror:8 = i^8
}

__device__ __forceinline__ float lane_xor_f(float x, int k) {
  switch (k) {
    case 0: return __uint_as_float(lane_xor<0>(__float_as_uint(x)));
    case 1: return __uint_as_float(lane_xor<1>(__float_as_uint(x)));
    case 2: return __uint_as_float(lane_xor<2>(__float_as_uint(x)));
    default: return __uint_as_float(lane_xor<3>(__float_as_uint(x)));
  }
}

// Max / sum over the 16 lanes of each row (all 16 lanes get the result).
__device__ __forceinline__ float row_max(float v) {
#pragma unroll
  for (int k = 0; k < 4; ++k) v = fmaxf(v, lane_xor_f(v, k));
  return v;
}
__device__ __forceinline__ float row_sum(float v) {
#pragma unroll
  for (int k = 0; k < 4; ++k) v += lane_xor_f(v, k);
  return v;
}

// Unnormalised Walsh–Hadamard transform along the 64 lanes (bits 0..5 of j):
// butterfly partner = lane ^ mask; lower lane keeps a+b, upper keeps a-b.
template <int E>
__device__ __forceinline__ void fwht_lanes(float (&v)[E], int lane) {
#pragma unroll
  for (int mask = 1; mask < kWave; mask <<= 1) {
    const bool upper = lane & mask;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float o = __shfl_xor(v[e], mask, kWave);
      v[e] = upper ? (o - v[e]) : (v[e] + o);
    }
  }
}

// Butterflies between registers (bits of e, i.e. bits 6.. of j) for a
// power-of-two E: Sylvester H_E applied across the registers of each lane.
template <int E>
__device__ __forceinline__ void fwht_regs(float (&v)[E]) {
#pragma unroll
  for (int h = 1; h < E; h <<= 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (e & h) continue;
      const float a = v[e], b = v[e + h];
      v[e] = a + b;
      v[e + h] = a - b;
    }
  }
}

// y = H v for the wave layout.  E a power of two: Sylvester H_{64E}.  E = 24
// (d = 1536): j = a*128 + i with a = e/2, i = (e%2)*64 + lane, H = H12 ⊗ H128;
// `transpose` applies Hᵀ (H12 is not symmetric; Sylvester matrices are).
template <int E, bool kTranspose = false>
__device__ __forceinline__ void hadamard_wave(float (&v)[E], int lane) {
  if constexpr (E == 24) {
    // H128 on i: register pairs (2a, 2a+1) then the lanes
#pragma unroll
    for (int a = 0; a < 12; ++a) {
      const float x = v[2 * a], y = v[2 * a + 1];
      v[2 * a] = x + y;
      v[2 * a + 1] = x - y;
    }
    fwht_lanes<24>(v, lane);
    // H12 on a, separately for each half of i
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      float w[12];
#pragma unroll
      for (int a = 0; a < 12; ++a) {
        float acc = 0.f;
#pragma unroll
        for (int b = 0; b < 12; ++b) {
          const int h = kTranspose ? paley12(b, a) : paley12(a, b);
          acc += h > 0 ? v[2 * b + par] : -v[2 * b + par];
        }
        w[a] = acc;
      }
#pragma unroll
      for (int a = 0; a < 12; ++a) v[2 * a + par] = w[a];
    }
  } else {
    fwht_regs<E>(v);
    fwht_lanes<E>(v, lane);
  }
}

template <typename T>
struct DtypeOf;
template <>
struct DtypeOf<float> { static constexpr tq_dtype_t v = TQ_F32; };
template <>
struct DtypeOf<__hip_bfloat16> { static constexpr tq_dtype_t v = TQ_BF16; };
template <>
struct DtypeOf<__half> { static constexpr tq_dtype_t v = TQ_F16; };

// Calls f.template operator()<E>() for the register count of head_dim d.
template <typename F>
__host__ inline hipError_t dispatch_E(int d, F&& f) {
  switch (d) {
    case 64: return f.template operator()<1>();
    case 128: return f.template operator()<2>();
    case 256: return f.template operator()<4>();
    case 512: return f.template operator()<8>();
    case 1024: return f.template operator()<16>();
    case 1536: return f.template operator()<24>();
    default: return hipErrorInvalidValue;
  }
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace tq

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

#include <utility>

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

// Eight consecutive elements as fp32 (p 16-byte aligned), in two steps so a
// caller can issue the load early and convert after a barrier: load_raw8
// keeps the loaded bits, unpack8 converts them.
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
template <typename T>
struct Raw8;
template <>
struct Raw8<float> { float4 a, b; };
template <>
struct Raw8<__hip_bfloat16> { uint4 a; };
template <>
struct Raw8<__half> { h8 a; };

__device__ __forceinline__ void load_raw8(const float* p, Raw8<float>& r) {
  r.a = reinterpret_cast<const float4*>(p)[0];
  r.b = reinterpret_cast<const float4*>(p)[1];
}
__device__ __forceinline__ void load_raw8(const __hip_bfloat16* p, Raw8<__hip_bfloat16>& r) {
  r.a = *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void load_raw8(const __half* p, Raw8<__half>& r) { r.a = *reinterpret_cast<const h8*>(p); }

__device__ __forceinline__ void unpack8(const Raw8<float>& r, float (&v)[8]) {
  v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w; v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
}
__device__ __forceinline__ void unpack8(const Raw8<__hip_bfloat16>& r, float (&v)[8]) {
  const uint32_t w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void unpack8(const Raw8<__half>& r, float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = static_cast<float>(r.a[i]);
}

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]) {
  Raw8<T> r;
  load_raw8(p, r);
  unpack8(r, v);
}

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

// Row (16-lane) reductions through the rotations row_ror 1, 2, 4, 8: the
// compiler folds each DPP move into the reducing op (one VALU op per step;
// the lane_xor forms above take up to four).  row_max_rot is exact and equal
// in every lane (-0 ranks below +0); row_max_nonneg is the same for v >= 0
// (the float order is the integer order of the bits).  In row_sum_rot each
// lane adds the 16 values in its own order: lanes may differ in the last
// bits, so use it where one lane's sum is taken.
template <int CTRL>
__device__ __forceinline__ int row_ror_dpp(int x, int old) {
  return __builtin_amdgcn_update_dpp(old, x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float row_max_nonneg(float v) {
  uint32_t x = __float_as_uint(v);
  x = max(x, static_cast<uint32_t>(row_ror_dpp<0x121>(static_cast<int>(x), 0)));
  x = max(x, static_cast<uint32_t>(row_ror_dpp<0x122>(static_cast<int>(x), 0)));
  x = max(x, static_cast<uint32_t>(row_ror_dpp<0x124>(static_cast<int>(x), 0)));
  x = max(x, static_cast<uint32_t>(row_ror_dpp<0x128>(static_cast<int>(x), 0)));
  return __uint_as_float(x);
}
__device__ __forceinline__ float row_max_rot(float v) {
  const int b = __float_as_int(v);
  int x = b ^ ((b >> 31) & 0x7FFFFFFF);  // monotone map of the float order to the signed order
  constexpr int lo = static_cast<int>(0x80000000u);
  x = max(x, row_ror_dpp<0x121>(x, lo));
  x = max(x, row_ror_dpp<0x122>(x, lo));
  x = max(x, row_ror_dpp<0x124>(x, lo));
  x = max(x, row_ror_dpp<0x128>(x, lo));
  return __int_as_float(x ^ ((x >> 31) & 0x7FFFFFFF));
}
__device__ __forceinline__ float row_sum_rot(float v) {
  v += __int_as_float(row_ror_dpp<0x121>(__float_as_int(v), 0));
  v += __int_as_float(row_ror_dpp<0x122>(__float_as_int(v), 0));
  v += __int_as_float(row_ror_dpp<0x124>(__float_as_int(v), 0));
  v += __int_as_float(row_ror_dpp<0x128>(__float_as_int(v), 0));
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

// The same transform with the partners fetched without LDS: lane distances
// 1-8 through DPP within rows of 16, 16 and 32 through v_permlane16_swap /
// v_permlane32_swap (with a = b = v the first result holds the other half of
// the lane's pair for an upper lane, the second for a lower one).  The same
// additions in the same order as fwht_lanes, so the results are identical.
template <int K, int E>
__device__ __forceinline__ void fwht_stage_dpp(float (&v)[E], int lane) {
  const bool upper = (lane >> K) & 1;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float o = __uint_as_float(lane_xor<K>(__float_as_uint(v[e])));
    v[e] = upper ? (o - v[e]) : (v[e] + o);
  }
}
template <int E>
__device__ __forceinline__ void fwht_lanes_dpp(float (&v)[E], int lane) {
  fwht_stage_dpp<0>(v, lane);
  fwht_stage_dpp<1>(v, lane);
  fwht_stage_dpp<2>(v, lane);
  fwht_stage_dpp<3>(v, lane);
  const bool up16 = (lane >> 4) & 1;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t x = __float_as_uint(v[e]);
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    const float o = __uint_as_float(up16 ? r[0] : r[1]);
    v[e] = up16 ? (o - v[e]) : (v[e] + o);
  }
  const bool up32 = (lane >> 5) & 1;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t x = __float_as_uint(v[e]);
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    const float o = __uint_as_float(up32 ? r[0] : r[1]);
    v[e] = up32 ? (o - v[e]) : (v[e] + o);
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
// kDpp: the lane stages through DPP and permlane swaps (fwht_lanes_dpp).
template <int E, bool kTranspose = false, bool kDpp = false>
__device__ __forceinline__ void hadamard_wave(float (&v)[E], int lane) {
  if constexpr (E == 24) {
    // H128 on i: register pairs (2a, 2a+1) then the lanes
#pragma unroll
    for (int a = 0; a < 12; ++a) {
      const float x = v[2 * a], y = v[2 * a + 1];
      v[2 * a] = x + y;
      v[2 * a + 1] = x - y;
    }
    if constexpr (kDpp) fwht_lanes_dpp<24>(v, lane);
    else fwht_lanes<24>(v, lane);
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
    if constexpr (kDpp) fwht_lanes_dpp<E>(v, lane);
    else fwht_lanes<E>(v, lane);
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

// Row of position t of (sequence b, KV head kh), bk = b * nkv + kh:
// [batch][kv_head][ctx] rows for a contiguous cache (pm.table null), else
// through the page table.
__device__ __forceinline__ int64_t kv_row(const PageMap& pm, int bk, int nkv, int64_t ctx, int64_t t) {
  if (!pm.table) return static_cast<int64_t>(bk) * ctx + t;
  const int page = pm.table[static_cast<int64_t>(bk / nkv) * pm.max_pages + t / pm.page_size];
  return (static_cast<int64_t>(page) * nkv + bk % nkv) * pm.page_size + t % pm.page_size;
}

// f.template operator()<I>() for I = 0..N-1, I a constant expression in each
// call (an unrolling that does not depend on the optimizer's size limits).
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  [&]<int... I>(std::integer_sequence<int, I...>) { (f.template operator()<I>(), ...); }(
      std::make_integer_sequence<int, N>{});
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device (256 on MI355X; that if the query fails).
inline int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

}  // namespace tq

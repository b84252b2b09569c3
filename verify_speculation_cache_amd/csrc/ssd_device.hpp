// Device-side helpers shared by the gfx950 kernels: chunk loads, orderable
// keys, wave64 / workgroup reductions and the cross-workgroup completion
// counter.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssd_internal.hpp"

namespace ssd {

// dtype tags: 0 = float32 logits, 1 = bfloat16 logits
template <int DT> struct Dt;
template <> struct Dt<0> {
  using T = float;
  static constexpr int kPerVec = 4;      // elements per 16-byte load
  static constexpr int kKeyBits = 32;
  __device__ static float to_f(T v) { return v; }
};
template <> struct Dt<1> {
  using T = uint16_t;
  static constexpr int kPerVec = 8;
  static constexpr int kKeyBits = 16;
  __device__ static float to_f(T v) { return __uint_as_float(uint32_t(v) << 16); }
};

__device__ __forceinline__ bool is_finite_f(float x) { return __builtin_isfinite(x); }
__device__ __forceinline__ float pivot_of(float m) { return is_finite_f(m) ? m : 0.0f; }

// Order-preserving integer image of a logit (dtype bits; -0 folded onto +0),
// so larger key <=> larger value. bf16 values are exact in float, so the key
// is taken from the top 16 bits of the widened value.
template <int DT> __device__ __forceinline__ uint32_t key_of(float x);
template <> __device__ __forceinline__ uint32_t key_of<0>(float x) {
  uint32_t b = __float_as_uint(x);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
template <> __device__ __forceinline__ uint32_t key_of<1>(float x) {
  uint32_t b = __float_as_uint(x) >> 16;
  if (b == 0x8000u) b = 0u;
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}
template <int DT> __device__ __forceinline__ float value_of_key(uint32_t k);
template <> __device__ __forceinline__ float value_of_key<0>(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
template <> __device__ __forceinline__ float value_of_key<1>(uint32_t k) {
  uint32_t b = (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
  return __uint_as_float(b << 16);
}

// 64-bit rank key: key descending, then token index ascending.
__device__ __forceinline__ uint64_t rank_key(uint32_t key, int32_t idx) {
  return (uint64_t(key) << 32) | uint64_t(0xFFFFFFFFu - uint32_t(idx));
}

// Chunk of kChunk entries starting at c0, strided layout: thread t holds
// vector g = j * kThreads + t (j = 0..NV-1) of kPerVec consecutive entries,
// so each load instruction of a wave covers one contiguous 1 KiB span.
template <int DT>
struct Strided {
  static constexpr int PV = Dt<DT>::kPerVec;
  static constexpr int NV = kPerThread / PV;
  __device__ static int64_t index(int64_t c0, int tid, int k) {
    const int j = k / PV, e = k % PV;
    return c0 + int64_t(j * kThreads + tid) * PV + e;
  }
};

template <int DT>
__device__ __forceinline__ void load_strided(const typename Dt<DT>::T* __restrict__ row, int64_t c0,
                                             int64_t V, bool vec, int tid, float (&x)[kPerThread]) {
  using S = Strided<DT>;
  if (vec) {
    const uint4* p = reinterpret_cast<const uint4*>(row + c0);
    uint4 raw[S::NV];
#pragma unroll
    for (int j = 0; j < S::NV; ++j) raw[j] = p[j * kThreads + tid];
#pragma unroll
    for (int j = 0; j < S::NV; ++j) {
      const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (DT == 1) {
          x[j * 8 + 2 * q] = __uint_as_float(w[q] << 16);
          x[j * 8 + 2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
        } else {
          x[j * 4 + q] = __uint_as_float(w[q]);
        }
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int64_t i = S::index(c0, tid, k);
      x[k] = (i < V) ? Dt<DT>::to_f(row[i]) : -__builtin_inff();
    }
  }
}

// Contiguous layout: thread t holds entries c0 + t*kPerThread + k.
template <int DT>
__device__ __forceinline__ void load_run(const typename Dt<DT>::T* __restrict__ row, int64_t c0,
                                         int64_t V, bool vec, int tid, float (&x)[kPerThread]) {
  const int64_t base = c0 + int64_t(tid) * kPerThread;
  if (vec) {
    constexpr int PV = Dt<DT>::kPerVec;
    constexpr int NV = kPerThread / PV;
    const uint4* p = reinterpret_cast<const uint4*>(row + base);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const uint4 r = p[j];
      const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (DT == 1) {
          x[j * 8 + 2 * q] = __uint_as_float(w[q] << 16);
          x[j * 8 + 2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
        } else {
          x[j * 4 + q] = __uint_as_float(w[q]);
        }
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int64_t i = base + k;
      x[k] = (i < V) ? Dt<DT>::to_f(row[i]) : -__builtin_inff();
    }
  }
}

// ---- wave64 reductions (butterflies: every lane ends with the same bits) ----
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
// inclusive prefix sum over lanes 0..63
__device__ __forceinline__ int wave_incl_scan_i(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}
__device__ __forceinline__ double wave_incl_scan_d(double v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// ---- workgroup (4 waves) reductions; all threads must call ----
__device__ __forceinline__ float block_max(float v, float* sm4) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm4[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(sm4[0], sm4[1]), fmaxf(sm4[2], sm4[3]));
}
__device__ __forceinline__ double block_sum(double v, double* sm4) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm4[w] = v;
  __syncthreads();
  return (sm4[0] + sm4[1]) + (sm4[2] + sm4[3]);
}
__device__ __forceinline__ int block_sum_i(int v, int* sm4) {
  v = wave_sum_i(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm4[w] = v;
  __syncthreads();
  return (sm4[0] + sm4[1]) + (sm4[2] + sm4[3]);
}

// Publish this workgroup's results and count it in; returns true in every
// thread of the workgroup that arrives last (it then sees all the others'
// writes). The last arrival also re-arms the counter for the next call.
// No workgroup ever waits for another, so this cannot deadlock.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t expected, int* sm_flag) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = atomicAdd(counter, 1u);
    const bool last = (prev == expected - 1u);
    if (last) *counter = 0u;
    *sm_flag = last ? 1 : 0;
  }
  __syncthreads();
  const bool last = *sm_flag != 0;
  if (last) __threadfence();
  return last;
}

}  // namespace ssd

// Kernels of the speculation-cache build, the cache lookup and the
// per-length hit counts; the device code of the build is in ssd_cache.hpp.
#include "ssd_cache.hpp"

namespace ssd {

template <int DT>
__global__ __launch_bounds__(kThreads) void k_cache_merge(CacheArgs a) {
  cache_merge_wg<DT>(a, blockIdx.x);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void k_cache_chunk(CacheArgs a) {
  cache_chunk_wg<DT>(a, blockIdx.x);
}

// One wave per batch row. Everything the row needs (its accepted length,
// its outcome tokens and, when the row's cache holds at most 256 tokens, the
// whole cache row) is loaded in one round trip; the outcome (k, t*) is then
// matched against segment k with a ballot. Segment tokens are distinct, so
// at most one slot matches.
constexpr int kLookupPre = 4;   // cache slots per lane loaded up front

__global__ __launch_bounds__(kThreads) void k_lookup(LookupArgs a) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (b >= a.B) return;   // whole wave
  const int32_t* orow = a.out_tokens + int64_t(b) * (a.K + 1);
  const int32_t* crow = a.cache_tokens + int64_t(b) * a.sumF;
  const bool pre = a.sumF <= 64 * kLookupPre;
  const int av = a.accepted[b];
  const int32_t ot = lane <= a.K ? orow[lane] : -1;
  const int32_t ot64 = (lane == 0 && a.K >= 64) ? orow[64] : -1;
  int32_t cv[kLookupPre];
#pragma unroll
  for (int r = 0; r < kLookupPre; ++r) {
    const int idx = r * 64 + lane;
    cv[r] = (pre && idx < a.sumF) ? crow[idx] : -1;
  }
  uint8_t h = 0;
  int32_t s = -1;
  if (av >= 0 && av <= a.K) {   // wave-uniform
    const int32_t t = av < 64 ? __shfl(ot, av) : __shfl(ot64, 0);
    const int lo = a.off[av], n = a.F[av];
    if (t >= 0 && n > 0) {
      if (pre) {
#pragma unroll
        for (int r = 0; r < kLookupPre; ++r) {
          const int idx = r * 64 + lane;
          const uint64_t m = __ballot(idx >= lo && idx < lo + n && cv[r] == t);
          if (m != 0 && s < 0) s = r * 64 + (__ffsll((unsigned long long)m) - 1) - lo;
        }
      } else {
        const uint64_t m = __ballot(lane < n && crow[lo + lane] == t);
        if (m != 0) s = __ffsll((unsigned long long)m) - 1;
      }
      h = s >= 0 ? 1 : 0;
    }
  }
  if (lane == 0) {
    a.hit[b] = h;
    if (a.slot) a.slot[b] = s;
  }
}

// Per-length outcome and hit counts of one round: one workgroup, LDS
// histogram with integer atomics (exact, order-independent), fully written.
__global__ __launch_bounds__(kThreads) void k_cache_stats(CacheStatsArgs a) {
  __shared__ uint32_t h[SSD_MAX_K + 1][2];
  for (int i = threadIdx.x; i < (a.K + 1) * 2; i += kThreads) h[i >> 1][i & 1] = 0u;
  __syncthreads();
  for (int b = threadIdx.x; b < a.B; b += kThreads) {
    const int av = a.accepted[b];
    if (av >= 0 && av <= a.K) {
      atomicAdd(&h[av][0], 1u);
      if (a.hit[b]) atomicAdd(&h[av][1], 1u);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < (a.K + 1) * 2; i += kThreads) a.counts[i] = h[i >> 1][i & 1];
}

hipError_t launch_cache_stats(const CacheStatsArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_cache_stats, dim3(1), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_cache(const CacheArgs& a0, int dtype, hipStream_t st) {
  CacheArgs a = a0;
  a.div_pb = make_fastdiv(uint32_t((a.K + 1) * a.S));
  a.div_s = make_fastdiv(uint32_t(a.S));
  a.div_kp = make_fastdiv(uint32_t(a.K + 1));
  const unsigned grid = unsigned(int64_t(a.B) * (a.K + 1) * a.S);
  const unsigned rows = unsigned(int64_t(a.B) * (a.K + 1));
  if (dtype == SSD_BF16) {
    hipLaunchKernelGGL(k_cache_chunk<1>, dim3(grid), dim3(kThreads), 0, st, a);
    hipLaunchKernelGGL(k_cache_merge<1>, dim3(rows), dim3(kThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL(k_cache_chunk<0>, dim3(grid), dim3(kThreads), 0, st, a);
    hipLaunchKernelGGL(k_cache_merge<0>, dim3(rows), dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_lookup(const LookupArgs& a, hipStream_t st) {
  const unsigned rows_per_wg = kThreads / 64;
  const unsigned grid = unsigned((a.B + rows_per_wg - 1) / rows_per_wg);
  hipLaunchKernelGGL(k_lookup, dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace ssd

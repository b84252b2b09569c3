// One verification round of speculative speculative decoding on the GPU:
// the speculation cache is built from the draft rows (papernotes.org
// "Speculative Speculative Decoding", framework and key designs 1-2), the
// drafted tokens are verified against the sigma-reshaped draft distribution
// (brentwoodlivery.com "Speculative decoding", The Algorithm, step 3), and
// the realised outcome is looked up in the cache.
//
// The separate entry points need five launches (cache chunk pass, cache
// merge, row statistics, residual, lookup). Here:
//  k_round_chunks  the cache chunk pass over draft rows 0..K and the row
//                  statistics' chunk pass over target rows 0..K in one grid
//                  (they read different rows and depend on nothing), so the
//                  two streams share one launch and one tail;
//  k_round_merge   the cache merge of every (b, k); the last merge of batch
//                  row b to finish runs that row's accept scan, which needs
//                  the sigma statistics of all K+1 merges;
//  k_resid         the residual / bonus draw, whose last workgroup per row
//                  also looks the outcome up in the cache.
// The arithmetic is that of the separate entry points: the cache is
// bit-identical to ssd_build_cache's; the row statistics here sum 8192-entry
// chunk partials (ssd_verify's pass sums 16384-entry ones, a register budget
// this launch cannot afford next to the cache pass), so accept decisions and
// draws agree with ssd_verify's except at rounding-level ties.
#include "ssd_cache.hpp"
#include "ssd_stats.hpp"

namespace ssd {

template <int DT>
__global__ __launch_bounds__(kThreads) void k_round_chunks(RoundArgs a) {
  const uint32_t per_b = a.ncw + a.nsw;
  const uint32_t b = blockIdx.x / per_b;
  const uint32_t rem = blockIdx.x - b * per_b;
  // uniform per workgroup; the statistics chunks are 8192 entries here (32
  // per thread, as the cache chunks), which keeps the launch at the cache
  // pass's register budget
  if (rem < a.ncw) cache_chunk_wg<DT>(a.c, b * a.ncw + rem);
  else stats_chunk_wg<DT, kPerThread>(a.s, b * a.nsw + (rem - a.ncw));
}

template <int DT>
__global__ __launch_bounds__(kThreads) void k_round_merge(RoundArgs a) {
  __shared__ int sm_last;
  const int64_t rowid = blockIdx.x;   // b * (K+1) + k
  cache_merge_wg<DT>(a.c, rowid);
  const int b = int(rowid / (a.c.K + 1));
  if (!arrive_last(&a.cnt[int64_t(b) * kCntStride], uint32_t(a.c.K + 1), &sm_last)) return;
  stats_epilogue<DT>(a.s, b);
}

hipError_t launch_round_chunks(const RoundArgs& a, int dtype, hipStream_t st) {
  const unsigned grid = unsigned(int64_t(a.c.B) * (a.ncw + a.nsw));
  if (dtype == SSD_BF16) hipLaunchKernelGGL(k_round_chunks<1>, dim3(grid), dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL(k_round_chunks<0>, dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_round_merge(const RoundArgs& a, int dtype, hipStream_t st) {
  const unsigned grid = unsigned(int64_t(a.c.B) * (a.c.K + 1));
  if (dtype == SSD_BF16) hipLaunchKernelGGL(k_round_merge<1>, dim3(grid), dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL(k_round_merge<0>, dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace ssd

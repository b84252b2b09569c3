// The row-statistics chunk pass: kernel and launcher; the device code is in
// ssd_stats.hpp.
#include "ssd_stats.hpp"

namespace ssd {

// The chunk pass: partials and gathered logits for a consumer in a later
// launch that merges them itself (the residual kernels).
// PT entries per thread: 64 (16384-entry chunks), or 16 for small grids.
template <int DT, int PT>
__global__ __launch_bounds__(kThreads) void k_stats_chunks(StatsArgs a) {
  stats_chunk_wg<DT, PT>(a, blockIdx.x);
}

hipError_t launch_stats_chunks(const StatsArgs& a0, int dtype, hipStream_t st) {
  StatsArgs a = a0;
  a.div_pb = make_fastdiv(uint32_t(a.NR * a.S));
  a.div_s = make_fastdiv(uint32_t(a.S));
  const dim3 grid(unsigned(int64_t(a.B) * a.NR * a.S));
  const bool small = a.pt == kSmallPerThread;
  if (dtype == SSD_BF16) {
    if (small) hipLaunchKernelGGL((k_stats_chunks<1, kSmallPerThread>), grid, dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((k_stats_chunks<1, kStatsPerThread>), grid, dim3(kThreads), 0, st, a);
  } else {
    if (small) hipLaunchKernelGGL((k_stats_chunks<0, kSmallPerThread>), grid, dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((k_stats_chunks<0, kStatsPerThread>), grid, dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace ssd

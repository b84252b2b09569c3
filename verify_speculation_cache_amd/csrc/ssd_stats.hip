// The row-statistics chunk pass: kernel and launcher; the device code is in
// ssd_stats.hpp.
#include "ssd_stats.hpp"

namespace ssd {

// The chunk pass: partials and gathered logits for a consumer in a later
// launch that merges them itself (the residual kernels).
template <int DT>
__global__ __launch_bounds__(kThreads) void k_stats_chunks(StatsArgs a) {
  stats_chunk_wg<DT>(a, blockIdx.x);
}

hipError_t launch_stats_chunks(const StatsArgs& a, int dtype, hipStream_t st) {
  const int64_t grid = int64_t(a.B) * a.NR * a.S;
  if (dtype == SSD_BF16)
    hipLaunchKernelGGL(k_stats_chunks<1>, dim3(unsigned(grid)), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(k_stats_chunks<0>, dim3(unsigned(grid)), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace ssd

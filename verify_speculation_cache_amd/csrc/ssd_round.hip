// One verification round of speculative speculative decoding on the GPU:
// the speculation cache is built from the draft rows (papernotes.org
// "Speculative Speculative Decoding", framework and key designs 1-2), the
// drafted tokens are verified against the sigma-reshaped draft distribution
// (brentwoodlivery.com "Speculative decoding", The Algorithm, step 3), and
// the realised outcome is looked up in the cache.
//
// The separate entry points need five launches (cache chunk pass, cache
// merge, row statistics, residual, lookup). Here three:
//  k_round_chunks  the cache chunk pass over draft rows 0..K and the row
//                  statistics' chunk pass over target rows 0..na-1 in one
//                  grid (they read different rows and depend on nothing), so
//                  the two streams share one launch and one tail;
//  k_round_merge_stats  the cache merge of every (b, k), as in the cache
//                  build, first in the grid, then the statistics chunks of
//                  target rows na..K: the merges' round trips run beside
//                  streaming work instead of alone (the merge holds four
//                  candidate slots per thread in registers here instead of
//                  sixteen, so the launch stays near the streaming pass's
//                  register budget, and visits them in the same order);
//                  na = floor(2(K+1)/3) balanced the two launches best at
//                  B=64 K=5 V=128256 (60.5 us per round against 61.2 for
//                  half and 61.6 for a third of the rows);
//  k_round_resid   every workgroup of batch row b first runs the row's accept
//                  scan itself (it needs the sigma statistics of all K+1
//                  merges and the target rows' chunk partials, a few KiB),
//                  then its share of the residual / bonus draw; the last
//                  workgroup per row also looks the outcome up in the cache.
//                  Repeating the small scan in each of the row's workgroups
//                  costs less than a cross-workgroup hand-off of its result
//                  while the draw's workgroups are all resident at once;
//                  draws of kScanOnceWgs or more workgroups (several
//                  generations of them) instead run the scan once per row in
//                  k_row_scan, a launch of its own, and read its RowInfo.
// The arithmetic is that of the separate entry points: the cache is
// bit-identical to ssd_build_cache's; the row statistics here sum 8192-entry
// chunk partials (ssd_verify's pass sums 16384-entry ones, a register budget
// this launch cannot afford next to the cache pass), so accept decisions and
// draws agree with ssd_verify's except at rounding-level ties.
#include <hip/hip_ext.h>

#include "ssd_cache.hpp"
#include "ssd_resid.hpp"
#include "ssd_stats.hpp"

namespace ssd {

template <int DT>
__global__ __launch_bounds__(kThreads) void k_round_chunks(RoundArgs a) {
  const uint32_t per_b = a.ncw + a.na * uint32_t(a.s.S);
  const uint32_t b = fdiv(blockIdx.x, a.div_pb);
  const uint32_t rem = blockIdx.x - b * per_b;
  // uniform per workgroup; the statistics chunks are 8192 entries here (32
  // per thread, as the cache chunks), which keeps the launch at the cache
  // pass's register budget
  if (rem < a.ncw) {
    const uint32_t k = fdiv(rem, a.c.div_s);
    cache_chunk_at<DT>(a.c, int(b), int(k), int(rem - k * uint32_t(a.c.S)));
  } else {
    const uint32_t r = fdiv(rem - a.ncw, a.s.div_s);
    stats_chunk_at<DT, kPerThread>(a.s, int(b), int(r), int(rem - a.ncw - r * uint32_t(a.s.S)));
  }
}

// The cache merges of every (b, k) (first in the grid, so they start at
// once), then the statistics chunks of target rows na..K: the merges' round
// trips overlap the streaming workgroups.
template <int DT>
__global__ __launch_bounds__(kThreads) void k_round_merge_stats(RoundArgs a) {
  const uint32_t nmerge = uint32_t(a.c.B) * uint32_t(a.c.K + 1);
  if (blockIdx.x < nmerge) {
    cache_merge_wg<DT, false, kHoldLean>(a.c, blockIdx.x);
    return;
  }
  const uint32_t j = blockIdx.x - nmerge;
  const uint32_t per_b = (uint32_t(a.s.NR) - a.na) * uint32_t(a.s.S);
  const uint32_t b = fdiv(j, a.div_pbb);
  const uint32_t rem = j - b * per_b;
  const uint32_t r = fdiv(rem, a.s.div_s);
  stats_chunk_at<DT, kPerThread>(a.s, int(b), int(a.na + r), int(rem - r * uint32_t(a.s.S)));
}

// Also the second launch of ssd_verify (after its statistics chunk pass),
// with SIG as the caller's sigma switch and no lookup. ONCE: k_row_scan ran
// the accept scan before this launch and left each row's RowInfo in the
// workspace (large grids).
template <int DT, bool SIG, int PT, bool ONCE>
__global__ __launch_bounds__(kThreads) void k_round_resid(RoundResidArgs a) {
  const int nw = resid_wgs_per_row(a.r.S, PT);
  const int b = int(fdiv(blockIdx.x, a.r.div_nw));
  const int c4 = blockIdx.x - b * nw;
  RowInfo inf;
  if constexpr (ONCE) {
    inf = a.r.info[b];   // the same address in every lane
  } else {
    __shared__ float e_piv[kMaxRows];
    __shared__ double e_s[kMaxRows];
    __shared__ RowInfo sm_inf;
    // the row's first workgroup also stores accepted[b], out_tokens, probs
    // and the optional row log-normalisers
    inf = accept_scan<DT, true>(a.s, b, c4 == 0, e_piv, e_s, &sm_inf);
    if (c4 == 0) write_row_lse(a.s, b, e_piv, e_s);
  }
  resid_row_wg<DT, SIG, PT>(a.r, inf, b, c4);
}

// The accept scan of batch row b = blockIdx.x on its own (large grids): it
// stores accepted[b], out_tokens (position a too, which the draw of the next
// launch then overwrites), probs and the optional row log-normalisers, and
// leaves the row's RowInfo in the workspace for k_round_resid<.., true>.
template <int DT>
__global__ __launch_bounds__(kThreads) void k_row_scan(RoundResidArgs a) {
  __shared__ float e_piv[kMaxRows];
  __shared__ double e_s[kMaxRows];
  const int b = blockIdx.x;
  const RowInfo inf = accept_scan<DT, false>(a.s, b, true, e_piv, e_s, nullptr);
  write_row_lse(a.s, b, e_piv, e_s);
  if (threadIdx.x == 0) a.s.info[b] = inf;   // wave 0 holds the result
}

static RoundArgs round_divs(const RoundArgs& a0) {
  RoundArgs a = a0;
  a.div_pb = make_fastdiv(a.ncw + a.na * uint32_t(a.s.S));
  a.div_pbb = make_fastdiv((uint32_t(a.s.NR) - a.na) * uint32_t(a.s.S));
  a.c.div_s = make_fastdiv(uint32_t(a.c.S));
  a.c.div_kp = make_fastdiv(uint32_t(a.c.K + 1));
  a.s.div_s = make_fastdiv(uint32_t(a.s.S));
  return a;
}

hipError_t launch_round_chunks(const RoundArgs& a0, int dtype, hipStream_t st, hipEvent_t start, hipEvent_t stop) {
  const RoundArgs a = round_divs(a0);
  const unsigned grid = unsigned(int64_t(a.c.B) * (a.ncw + a.na * uint32_t(a.s.S)));
  if (start != nullptr || stop != nullptr) {
    if (dtype == SSD_BF16)
      hipExtLaunchKernelGGL(k_round_chunks<1>, dim3(grid), dim3(kThreads), 0, st, start, stop, 0, a);
    else
      hipExtLaunchKernelGGL(k_round_chunks<0>, dim3(grid), dim3(kThreads), 0, st, start, stop, 0, a);
  } else if (dtype == SSD_BF16) {
    hipLaunchKernelGGL(k_round_chunks<1>, dim3(grid), dim3(kThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL(k_round_chunks<0>, dim3(grid), dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_round_merge_stats(const RoundArgs& a0, int dtype, hipStream_t st) {
  const RoundArgs a = round_divs(a0);
  const unsigned grid =
      unsigned(int64_t(a.c.B) * (a.c.K + 1) + int64_t(a.c.B) * (a.s.NR - int64_t(a.na)) * a.s.S);
  if (dtype == SSD_BF16) hipLaunchKernelGGL(k_round_merge_stats<1>, dim3(grid), dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL(k_round_merge_stats<0>, dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int DT, bool SIG>
static void launch_round_resid_t(const RoundResidArgs& a, unsigned grid, bool once, hipStream_t st) {
  if (a.r.span_pt == kSmallPerThread)
    hipLaunchKernelGGL((k_round_resid<DT, SIG, kSmallPerThread, false>), dim3(grid), dim3(kThreads), 0, st, a);
  else if (once)
    hipLaunchKernelGGL((k_round_resid<DT, SIG, kStatsPerThread, true>), dim3(grid), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((k_round_resid<DT, SIG, kStatsPerThread, false>), dim3(grid), dim3(kThreads), 0, st, a);
}

hipError_t launch_round_resid(const RoundResidArgs& a0, int dtype, bool sigma, hipStream_t st) {
  RoundResidArgs a = a0;
  const int64_t nw = resid_wgs_per_row(a.r.S, a.r.span_pt);
  a.r.div_nw = make_fastdiv(uint32_t(nw));
  const unsigned grid = unsigned(int64_t(a.r.B) * nw);
  const bool once = a.r.span_pt != kSmallPerThread && int64_t(a.r.B) * nw >= kScanOnceWgs;
  if (once) {
    if (dtype == SSD_BF16) hipLaunchKernelGGL(k_row_scan<1>, dim3(unsigned(a.r.B)), dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL(k_row_scan<0>, dim3(unsigned(a.r.B)), dim3(kThreads), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dtype == SSD_BF16) {
    if (sigma) launch_round_resid_t<1, true>(a, grid, once, st);
    else launch_round_resid_t<1, false>(a, grid, once, st);
  } else {
    if (sigma) launch_round_resid_t<0, true>(a, grid, once, st);
    else launch_round_resid_t<0, false>(a, grid, once, st);
  }
  return hipGetLastError();
}

hipError_t launch_round(const RoundArgs& a, const RoundResidArgs& rr, int dtype, hipStream_t st,
                        void* const* marks) {
  auto mark = [&](int i) -> hipError_t {
    return marks != nullptr ? hipEventRecord(static_cast<hipEvent_t>(marks[i]), st) : hipSuccess;
  };
  hipError_t e;
  // marks 0 and 1: the first launch's own start and end (recorded by the
  // launch, so their interval is that kernel's execution time); marks 2
  // and 3: recorded after the second and the last launch
  if (marks != nullptr)
    e = launch_round_chunks(a, dtype, st, static_cast<hipEvent_t>(marks[0]), static_cast<hipEvent_t>(marks[1]));
  else
    e = launch_round_chunks(a, dtype, st);
  if (e != hipSuccess) return e;
  if ((e = launch_round_merge_stats(a, dtype, st)) != hipSuccess) return e;
  if ((e = mark(2)) != hipSuccess) return e;
  if ((e = launch_round_resid(rr, dtype, true, st)) != hipSuccess) return e;
  return mark(3);
}

}  // namespace ssd

// Correction / bonus draw by inverse CDF.
//
// After a rejection at position a the replacement token is drawn from
// max(0, p_a - q_a)/Z; after a full accept the bonus is drawn from p_K
// (brentwoodlivery.com "Speculative decoding", The Algorithm, step 3, and
// Derivation of Acceptance Criterion; til.phipham141.dev "Why does
// speculative decoding exist?", Fix 2 and Fix 3). The draw is the smallest
// token v (in index order) whose running residual mass exceeds u * Z.
//
// Masses are in target units (ssd_resid.hpp) with rho = s_t / s_d.
//
// Phase A (all workgroups): one workgroup per (batch row, 16384-entry span)
// sums r and e_t over each 4096-entry chunk of its span (per-thread float
// sums, double across threads).
// Phase B (last workgroup of the batch row): walks the chunk masses in order
// to find the chunk holding u*Z, re-reads that chunk with each thread owning
// 16 consecutive tokens, scans thread totals in double and picks the token.
// If rounding leaves no crossing inside the chosen chunk the last token of
// that chunk with positive mass is taken. With no residual mass at all the
// draw uses p (e_t) instead; with no mass in p either the token is -1.
#include "ssd_resid.hpp"
#include "ssd_stats.hpp"

namespace ssd {

// ssd_residual_sample's draw, after the statistics chunk pass over the row
// pair of each batch row (rows mode): every workgroup of batch row b merges
// the pair's partials itself (a few hundred bytes) before its share of the
// draw, so no workgroup of the chunk pass waits on a counter.
template <int DT, bool SIG, int PT>
__global__ __launch_bounds__(kThreads) void k_rows_resid(RoundResidArgs a) {
  __shared__ float e_piv[2];
  __shared__ double e_s[2];
  __shared__ RowInfo sm_inf;
  const int nw = resid_wgs_per_row(a.r.S, PT);
  const int b = int(fdiv(blockIdx.x, a.r.div_nw));
  const RowInfo inf = rows_mode_info(a.s, b, e_piv, e_s, &sm_inf);
  resid_row_wg<DT, SIG, PT>(a.r, inf, b, blockIdx.x - b * nw);
}

template <int DT, bool SIG>
static void launch_rows_resid_t(const RoundResidArgs& a, unsigned grid, hipStream_t st) {
  if (a.r.span_pt == kSmallPerThread)
    hipLaunchKernelGGL((k_rows_resid<DT, SIG, kSmallPerThread>), dim3(grid), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((k_rows_resid<DT, SIG, kStatsPerThread>), dim3(grid), dim3(kThreads), 0, st, a);
}

hipError_t launch_rows_resid(const RoundResidArgs& a0, int dtype, bool sigma, hipStream_t st) {
  RoundResidArgs a = a0;
  a.r.div_nw = make_fastdiv(uint32_t(resid_wgs_per_row(a.r.S, a.r.span_pt)));
  const unsigned grid = unsigned(int64_t(a.r.B) * resid_wgs_per_row(a.r.S, a.r.span_pt));
  if (dtype == SSD_BF16) {
    if (sigma) launch_rows_resid_t<1, true>(a, grid, st);
    else launch_rows_resid_t<1, false>(a, grid, st);
  } else {
    if (sigma) launch_rows_resid_t<0, true>(a, grid, st);
    else launch_rows_resid_t<0, false>(a, grid, st);
  }
  return hipGetLastError();
}

}  // namespace ssd

// Inverse-CDF building blocks shared by the residual/bonus draw and the draft
// sampler: the draw is the smallest token v (index order) whose running mass
// exceeds u * Z, found in two levels, chunk then token.
#pragma once

#include "ssd_device.hpp"

namespace ssd {

// Wave-level search over per-chunk masses: the first chunk whose running mass
// (chunk order, fixed wave scans) exceeds `target`; also the mass before it.
// mass(cc, g) gives chunk cc's mass (0 for cc >= S) and is called once per
// group g of 64 chunks, lane-parallel. If rounding leaves `target` past every
// crossing, the last chunk with mass is taken. cs = -1 when no chunk has mass.
template <class MassFn>
__device__ __forceinline__ void chunk_crossing(MassFn mass, int S, double target, int lane, int& cs, double& pre) {
  cs = -1;
  pre = 0.0;
  double base = 0.0, lastpre = 0.0;
  int lastpos = -1;
  for (int g = 0; g < S && cs < 0; g += 64) {
    const int cc = g + lane;
    const double mc = mass(cc, g);
    const double incl = wave_incl_scan_d(mc, lane);
    const double excl = base + wave_shift_up1_d(incl);
    const uint64_t crossing = __ballot(cc < S && base + incl > target);
    const uint64_t pos = __ballot(cc < S && mc > 0.0);
    if (crossing) {
      const int l = __ffsll((unsigned long long)crossing) - 1;
      cs = g + l;
      pre = lane_d(excl, l);
    } else if (pos) {
      const int l = 63 - __clzll((long long)pos);
      lastpos = g + l;
      lastpre = lane_d(excl, l);
    }
    base += lane_d(incl, 63);
  }
  if (cs < 0) {
    cs = lastpos;
    pre = lastpre;
  }
}

template <int DT, int NROW, int PT = kPerThread>
struct PickLds {
  double scan[4];
  int pick[4];
  int best[4];
  double base;
  int lastpos;
  int tok;
  float vals[PT];   // the crossing thread's masses, token order
};

// Token pick inside chunk [c0, c0 + 256 PT) whose running mass starts at
// `pre`: every thread owns PT (32 or 64) consecutive tokens of NROW rows (raw
// vectors in cv, contiguous layout); value(x, idx) is the mass of token idx
// from its NROW logits x. Thread totals are scanned in double; the crossing
// thread then recomputes its PT masses from the vectors it still holds and
// hands them to wave 0 through LDS for a parallel rescan (no second memory
// round trip; the same values as in the totals, bit for bit). If rounding keeps
// the running mass at or below `target` through a run, the run's last token
// with mass is taken (the chunk's, if no thread crosses). Called by every
// thread of the workgroup; returns the token (-1: no mass).
template <int DT, int NROW, int PT, class ValueFn>
__device__ __forceinline__ int chunk_pick(const ChunkVecs<DT, false, PT> (&cv)[NROW], int64_t c0, double pre,
                                          double target, ValueFn value, PickLds<DT, NROW, PT>& L) {
  static_assert(PT <= 64, "the rescan holds one token per lane");
  constexpr int PV = Dt<DT>::kPerVec;
  constexpr int NV = PT / PV;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i0 = int(c0) + tid * PT;
  double tot = 0.0;
  int lastpos = -1;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    float xv[NROW][PV];
#pragma unroll
    for (int r = 0; r < NROW; ++r) cv[r].get(j, xv[r]);
#pragma unroll
    for (int e = 0; e < PV; ++e) {
      float x[NROW];
#pragma unroll
      for (int r = 0; r < NROW; ++r) x[r] = xv[r][e];
      const float v = value(x, i0 + j * PV + e);
      tot += double(v);
      if (v > 0.0f) lastpos = j * PV + e;
    }
    // one vector at a time: keeps the unpacked values of later vectors out
    // of registers, so this tail of the kernel needs no more of them than
    // the streaming part
    __builtin_amdgcn_sched_barrier(0);
  }
  // exclusive scan of thread totals (thread order = token order)
  const double incl_w = wave_incl_scan_d(tot, lane);
  if (lane == 63) L.scan[w] = incl_w;
  __syncthreads();
  double wbase = 0.0;
  for (int ww = 0; ww < w; ++ww) wbase += L.scan[ww];
  const double base = pre + wbase + (incl_w - tot);
  // first thread whose running mass crosses the target
  const uint64_t cm = __ballot((base + tot) > target);
  if (lane == 0) L.pick[w] = cm ? (w * 64 + __ffsll((unsigned long long)cm) - 1) : 0x7FFFFFFF;
  __syncthreads();
  const int first = min(min(L.pick[0], L.pick[1]), min(L.pick[2], L.pick[3]));
  if (first != 0x7FFFFFFF) {
    if (tid == first) {
      L.base = base;
      L.lastpos = lastpos;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        float xv[NROW][PV];
#pragma unroll
        for (int r = 0; r < NROW; ++r) cv[r].get(j, xv[r]);
#pragma unroll
        for (int e = 0; e < PV; ++e) {
          float x[NROW];
#pragma unroll
          for (int r = 0; r < NROW; ++r) x[r] = xv[r][e];
          L.vals[j * PV + e] = value(x, i0 + j * PV + e);
        }
      }
    }
    __syncthreads();
    if (w == 0) {
      const int q = lane & (PT - 1);
      const int f0 = int(c0) + first * PT;
      const float v = L.vals[q];
      const double cum = L.base + wave_incl_scan_d(lane < PT ? double(v) : 0.0, lane);
      const uint64_t cr = __ballot(lane < PT && cum > target);
      if (lane == 0) L.tok = f0 + (cr ? __ffsll((unsigned long long)cr) - 1 : L.lastpos);
    }
  } else {
    int best = lastpos >= 0 ? i0 + lastpos : -1;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) best = max(best, __shfl_xor(best, o));
    if (lane == 0) L.best[w] = best;
    __syncthreads();
    if (tid == 0) L.tok = max(max(L.best[0], L.best[1]), max(L.best[2], L.best[3]));
  }
  __syncthreads();
  return L.tok;
}

}  // namespace ssd

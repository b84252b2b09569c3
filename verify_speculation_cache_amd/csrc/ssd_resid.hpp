// Residual / bonus mass of one (target row, draft row) pair and the two
// phases of its inverse-CDF draw, shared by the one-path residual kernel and
// the token-tree rounds.
//
// Units: everything is kept relative to the target row, e_t(v) =
// exp((z_t(v) - pivot_t)/tau), so p = e_t / s_t and the residual mass is
// r(v) = max(0, e_t(v) - rho_w * e_d(v)) with rho_w = w * rho (w = C for
// sigma members, else 1); rho is split into two floats so the subtraction
// keeps double-precision scaling. With every rho zero (set_plain) the mass
// is e_t itself: fma(-0, e_d, e_t) = e_t, so no select is needed and the
// per-entry code stays branch-free.
#pragma once

#include "ssd_cdf.hpp"

namespace ssd {

struct ResidConsts {
  float piv_t, piv_d, c32;
  float rho_hi, rho_lo, rhoC_hi, rhoC_lo;
  float thr_val;     // sigma threshold as a logit value (key order = value order)
  int32_t thr_idx;
};

// Mass = e_t (bonus draw, or a residual without mass).
__device__ __forceinline__ void set_plain(ResidConsts& k) {
  k.rho_hi = k.rho_lo = k.rhoC_hi = k.rhoC_lo = 0.0f;
}

__device__ __forceinline__ void split2(double v, float& hi, float& lo) {
  hi = float(v);
  lo = float(v - double(hi));
}

// Residual mass of one entry in target units (e_t when plain).
// Sigma membership "key > thr, or key == thr and index <= thr_idx" is taken
// on values: for non-NaN logits the order of keys is the order of values,
// with -0 and +0 equal in both.
template <bool SIG>
__device__ __forceinline__ float resid_elem(const ResidConsts& k, float xt, float xd, int idx) {
  const float et = __builtin_amdgcn_exp2f((xt - k.piv_t) * k.c32);
  const float ed = __builtin_amdgcn_exp2f((xd - k.piv_d) * k.c32);
  float hi = k.rho_hi, lo = k.rho_lo;
  if constexpr (SIG) {
    // bitwise, not short-circuit: keeps the test branch-free
    const bool mem = (xd > k.thr_val) | ((xd == k.thr_val) & (idx <= k.thr_idx));
    hi = mem ? k.rhoC_hi : hi;
    lo = mem ? k.rhoC_lo : lo;
  }
  float r = __builtin_fmaf(-hi, ed, et);
  r = __builtin_fmaf(-lo, ed, r);
  return fmaxf(r, 0.0f);
}

__device__ __forceinline__ float target_elem(const ResidConsts& k, float xt) {
  return __builtin_amdgcn_exp2f((xt - k.piv_t) * k.c32);
}

// Phase A: residual mass and target mass of the 8192-entry chunk at c0
// (per-thread float sums, double across threads). Called by every thread;
// the two workgroup totals are returned in thread 0 (sm_pair: 8 doubles of
// LDS; one barrier).
template <int DT, bool SIG>
__device__ __forceinline__ void resid_chunk_masses(const ResidConsts& k, const typename Dt<DT>::T* rowT,
                                                   const typename Dt<DT>::T* rowD, int64_t c0, int V,
                                                   double* sm_pair, double& R, double& P) {
  constexpr int PV = Dt<DT>::kPerVec;
  constexpr int NV = kPerThread / PV;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  ChunkVecs<DT, true> vt, vd;
  load_pair(vt, rowT, vd, rowD, c0, V, tid);
  float rs = 0.0f, ts = 0.0f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    float xt[PV], xd[PV];
    vt.get(j, xt);
    vd.get(j, xd);
    const int i0 = int(c0) + ChunkVecs<DT, true>::local(tid, j);
#pragma unroll
    for (int e = 0; e < PV; ++e) {
      ts += target_elem(k, xt[e]);
      rs += resid_elem<SIG>(k, xt[e], xd[e], i0 + e);
    }
  }
  // both sums across the workgroup with one barrier
  const double Rw = wave_sum(double(rs));
  const double Pw = wave_sum(double(ts));
  if (lane == 0) {
    sm_pair[w] = Rw;
    sm_pair[4 + w] = Pw;
  }
  __syncthreads();
  R = (sm_pair[0] + sm_pair[1]) + (sm_pair[2] + sm_pair[3]);
  P = (sm_pair[4] + sm_pair[5]) + (sm_pair[6] + sm_pair[7]);
}

// Phase A over two consecutive 8192-chunks at once (a 16384-entry span at
// c0, 64 entries per thread, strided: vectors j < NV/2 lie in the first
// chunk): the masses of each chunk, so the draw keeps 8192-entry chunks while
// a workgroup moves twice the bytes per round trip. R[h], P[h] for half h are
// returned in every thread (sm: 16 doubles of LDS; one barrier).
template <int DT, bool SIG>
__device__ __forceinline__ void resid_chunk_masses2(const ResidConsts& k, const typename Dt<DT>::T* rowT,
                                                    const typename Dt<DT>::T* rowD, int64_t c0, int V,
                                                    double* sm, double (&R)[2], double (&P)[2]) {
  constexpr int PV = Dt<DT>::kPerVec;
  using CV = ChunkVecs<DT, true, kStatsPerThread>;
  constexpr int NVH = CV::NV / 2;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  CV vt, vd;
  load_pair(vt, rowT, vd, rowD, c0, V, tid);
  float rs[2] = {0.0f, 0.0f}, ts[2] = {0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < CV::NV; ++j) {
    float xt[PV], xd[PV];
    vt.get(j, xt);
    vd.get(j, xd);
    const int i0 = int(c0) + CV::local(tid, j);
#pragma unroll
    for (int e = 0; e < PV; ++e) {
      ts[j / NVH] += target_elem(k, xt[e]);
      rs[j / NVH] += resid_elem<SIG>(k, xt[e], xd[e], i0 + e);
    }
    __builtin_amdgcn_sched_barrier(0);   // one vector pair at a time
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const double Rw = wave_sum(double(rs[h]));
    const double Pw = wave_sum(double(ts[h]));
    if (lane == 0) {
      sm[8 * h + w] = Rw;
      sm[8 * h + 4 + w] = Pw;
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    R[h] = (sm[8 * h] + sm[8 * h + 1]) + (sm[8 * h + 2] + sm[8 * h + 3]);
    P[h] = (sm[8 * h + 4] + sm[8 * h + 5]) + (sm[8 * h + 6] + sm[8 * h + 7]);
  }
}

// Phase B, first level (wave 0): from per-chunk (residual, target) masses at
// cmw[2*cc], cmw[2*cc+1] (one lane per chunk, one round trip for S <= 64),
// the totals Z_res and Z_tgt, and the chunk holding target = u * Z of the
// residual (or of p when the residual has no mass). cs = -1 if neither has
// mass. All lanes of wave 0 call it; results are valid in every lane.
__device__ __forceinline__ void resid_find_chunk(const uint64_t* cmw, int S, float u, int lane, double& zres,
                                                 double& ztgt, int& useres, double& target, int& cs,
                                                 double& pre) {
  zres = 0.0;
  ztgt = 0.0;
  double r0 = 0.0, t0 = 0.0;   // this lane's masses in the first group
  for (int g = 0; g < S; g += 64) {
    const int cc = g + lane;
    const double r = cc < S ? bits_d(dev_load(cmw + cc * 2)) : 0.0;
    const double t = cc < S ? bits_d(dev_load(cmw + cc * 2 + 1)) : 0.0;
    if (g == 0) {
      r0 = r;
      t0 = t;
    }
    zres += __shfl(wave_incl_scan_d(r, lane), 63);
    ztgt += __shfl(wave_incl_scan_d(t, lane), 63);
  }
  useres = zres > 0.0 ? 1 : 0;
  const double tot = useres ? zres : ztgt;
  target = double(u) * tot;
  cs = -1;
  pre = 0.0;
  if (tot > 0.0) {
    const int ur = useres;
    chunk_crossing(
        [&](int cc, int g) -> double {
          if (g == 0) return ur ? r0 : t0;
          return cc < S ? bits_d(dev_load(cmw + cc * 2 + (ur ? 0 : 1))) : 0.0;
        },
        S, target, lane, cs, pre);
  }
}

// Phase B, second level (every thread): re-read chunk cs of both rows and
// pick the token whose running mass crosses target.
template <int DT, bool SIG>
__device__ __forceinline__ int resid_pick(const ResidConsts& k, const typename Dt<DT>::T* rowT,
                                          const typename Dt<DT>::T* rowD, int cs, double pre, double target,
                                          int V, PickLds<DT, 2>& pk) {
  const int64_t c0 = int64_t(cs) * kChunk;
  // each thread owns 32 consecutive tokens of the chunk
  ChunkVecs<DT, false> cv[2];
  load_pair(cv[0], rowT, cv[1], rowD, c0, V, threadIdx.x);
  const typename Dt<DT>::T* const rows[2] = {rowT, rowD};
  return chunk_pick<DT, 2>(cv, rows, V, c0, pre, target,
                           [&](const float (&x)[2], int idx) { return resid_elem<SIG>(k, x[0], x[1], idx); }, pk);
}

}  // namespace ssd

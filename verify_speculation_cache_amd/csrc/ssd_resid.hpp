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
//
// Per entry the exponentials are taken in scaled form (scaled_mass: one
// fused multiply-add for the argument): e_t = fix_t * e'_t and e_d = fix_d *
// e'_d with row constants fix_t, fix_d, so r = fix_t * max(0, e'_t - rho' *
// e'_d) with rho' = rho_w * fix_d / fix_t. The per-entry values are r / fix_t
// (and e_t / fix_t); chunk masses are returned in target units (times
// fix_t), and the in-chunk pick compares running sums of the per-entry
// values against targets divided by fix_t.
#pragma once

#include "ssd_cdf.hpp"

namespace ssd {

struct ResidConsts {
  float Pt, Pd, c32;   // scaled pivots of the target and draft rows, log2(e)/tau
  float fix_t;         // e_t = fix_t * (per-entry target value)
  double dratio;       // fix_d / fix_t
  float rho_hi, rho_lo, rhoC_hi, rhoC_lo;
  float thr_val;     // sigma threshold as a logit value (key order = value order)
  int32_t thr_idx;
};

__device__ __forceinline__ void split2(double v, float& hi, float& lo) {
  hi = float(v);
  lo = float(v - double(hi));
}

// Row constants from the target and draft rows' pivots (raw logit units).
__device__ __forceinline__ void set_rows(ResidConsts& k, float piv_t, float piv_d, float c32) {
  const ScaledPivot st = scaled_pivot(piv_t, c32), sd = scaled_pivot(piv_d, c32);
  k.c32 = c32;
  k.Pt = st.P;
  k.Pd = sd.P;
  k.fix_t = st.fix;
  k.dratio = double(sd.fix) / double(st.fix);
}

// The residual's weights: rho for non-members, rho * C for sigma members.
__device__ __forceinline__ void set_rho(ResidConsts& k, double rho, double C) {
  split2(rho * k.dratio, k.rho_hi, k.rho_lo);
  split2(rho * C * k.dratio, k.rhoC_hi, k.rhoC_lo);
}

// Mass = e_t (bonus draw, or a residual without mass).
__device__ __forceinline__ void set_plain(ResidConsts& k) {
  k.rho_hi = k.rho_lo = k.rhoC_hi = k.rhoC_lo = 0.0f;
}

// Residual mass of one entry in target units (e_t when plain).
// Sigma membership "key > thr, or key == thr and index <= thr_idx" is taken
// on values: for non-NaN logits the order of keys is the order of values,
// with -0 and +0 equal in both.
template <bool SIG>
__device__ __forceinline__ float resid_elem(const ResidConsts& k, float xt, float xd, int idx) {
  const float et = scaled_mass(xt, k.c32, k.Pt);
  const float ed = scaled_mass(xd, k.c32, k.Pd);
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
  return scaled_mass(xt, k.c32, k.Pt);
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
  R = ((sm_pair[0] + sm_pair[1]) + (sm_pair[2] + sm_pair[3])) * double(k.fix_t);
  P = ((sm_pair[4] + sm_pair[5]) + (sm_pair[6] + sm_pair[7])) * double(k.fix_t);
}

// Phase A over one span of 256 * PT entries at c0 (PT per thread, strided:
// the first NV/NQ vectors of every thread lie in the first 4096 entries,
// the next NV/NQ in the second, and so on): the masses of each of its NQ =
// PT/16 pick chunks. PT = 64 lets a workgroup move 64 KiB (bf16) per round
// trip; small grids use PT = 16 (one pick chunk per workgroup). R[h], P[h]
// for chunk h are returned in every thread (sm: 8 NQ doubles of LDS; one
// barrier).
template <int DT, bool SIG, int PT>
__device__ __forceinline__ void resid_span_masses(const ResidConsts& k, const typename Dt<DT>::T* rowT,
                                                  const typename Dt<DT>::T* rowD, int64_t c0, int V, double* sm,
                                                  double (&R)[PT / kPickPerThread],
                                                  double (&P)[PT / kPickPerThread]) {
  constexpr int PV = Dt<DT>::kPerVec;
  constexpr int NQ = PT / kPickPerThread;
  using CV = ChunkVecs<DT, true, PT>;
  constexpr int NVQ = CV::NV / NQ;   // vectors per pick chunk
  static_assert(NVQ * NQ == CV::NV, "pick chunks must split the vectors evenly");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  CV vt, vd;
  load_pair(vt, rowT, vd, rowD, c0, V, tid);
  float rs[NQ], ts[NQ];
#pragma unroll
  for (int h = 0; h < NQ; ++h) rs[h] = ts[h] = 0.0f;
#pragma unroll
  for (int j = 0; j < CV::NV; ++j) {
    float xt[PV], xd[PV];
    vt.get(j, xt);
    vd.get(j, xd);
    const int i0 = int(c0) + CV::local(tid, j);
#pragma unroll
    for (int e = 0; e < PV; ++e) {
      ts[j / NVQ] += target_elem(k, xt[e]);
      rs[j / NVQ] += resid_elem<SIG>(k, xt[e], xd[e], i0 + e);
    }
    __builtin_amdgcn_sched_barrier(0);   // one vector pair at a time
  }
#pragma unroll
  for (int h = 0; h < NQ; ++h) {
    const double Rw = wave_sum(double(rs[h]));
    const double Pw = wave_sum(double(ts[h]));
    if (lane == 0) {
      sm[8 * h + w] = Rw;
      sm[8 * h + 4 + w] = Pw;
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < NQ; ++h) {
    R[h] = ((sm[8 * h] + sm[8 * h + 1]) + (sm[8 * h + 2] + sm[8 * h + 3])) * double(k.fix_t);
    P[h] = ((sm[8 * h + 4] + sm[8 * h + 5]) + (sm[8 * h + 6] + sm[8 * h + 7])) * double(k.fix_t);
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
    zres += lane_d(wave_incl_scan_d(r, lane), 63);
    ztgt += lane_d(wave_incl_scan_d(t, lane), 63);
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

// Phase B, second level (every thread): re-read chunk cs (chunks of
// 256 * PT entries) of both rows and pick the token whose running mass
// crosses target (pre and target in target units; the per-entry values are
// those units divided by fix_t).
template <int DT, bool SIG, int PT = kPerThread>
__device__ __forceinline__ int resid_pick(const ResidConsts& k, const typename Dt<DT>::T* rowT,
                                          const typename Dt<DT>::T* rowD, int cs, double pre, double target,
                                          int V, PickLds<DT, 2, PT>& pk) {
  const int64_t c0 = int64_t(cs) * (kThreads * PT);
  // each thread owns PT consecutive tokens of the chunk
  ChunkVecs<DT, false, PT> cv[2];
  load_pair(cv[0], rowT, cv[1], rowD, c0, V, threadIdx.x);
  const double inv = 1.0 / double(k.fix_t);
  return chunk_pick<DT, 2>(cv, c0, pre * inv, target * inv,
                           [&](const float (&x)[2], int idx) { return resid_elem<SIG>(k, x[0], x[1], idx); }, pk);
}

// Row pointers and constants of the draw of batch row b described by inf
// (validated: a row index the accept scan could not have written is taken
// as a flagged row, so stale state can never address outside the inputs).
template <int DT, bool SIG>
__device__ __forceinline__ void resid_setup(const ResidArgs& a, RowInfo& inf, int b, ResidConsts& k,
                                            const typename Dt<DT>::T*& rowT, const typename Dt<DT>::T*& rowD) {
  using T = typename Dt<DT>::T;
  if (inf.a < -1 || inf.a > a.K) inf.a = -1;
  if (inf.a == a.K || a.draft == nullptr) inf.bonus = 1;

  // A bonus row has no draft: it reads the target row twice with rho = 0,
  // so both rows take the same load and arithmetic path.
  k = ResidConsts{};
  rowT = nullptr;
  rowD = nullptr;
  if (inf.a >= 0) {
    rowT = static_cast<const T*>(a.target) + int64_t(b) * a.tb + int64_t(inf.a) * a.V;
    k.thr_val = value_of_key<DT>(inf.thr_key);
    k.thr_idx = inf.thr_idx;
    if (inf.bonus) {
      rowD = rowT;
      set_rows(k, inf.piv_t, inf.piv_t, a.c32);
      set_plain(k);
    } else {
      rowD = static_cast<const T*>(a.draft) + int64_t(b) * a.db + int64_t(inf.a) * a.V;
      set_rows(k, inf.piv_t, inf.piv_d, a.c32);
      set_rho(k, inf.s_d > 0.0 ? inf.s_t / inf.s_d : 0.0, double(inf.C));
    }
  }
  // sigma thresholds that admit no entry (key above that of +inf)
  if (SIG && inf.thr_key > key_of<DT>(__builtin_inff())) k.thr_val = __builtin_nanf("");
}

// Phase A of the draw of batch row b by its workgroup c4 (span c4 of 256 *
// PT entries: pick chunks NQ c4 .. NQ c4 + NQ - 1): the residual and target
// masses of those chunks, left in a.cmass by thread 0 with device-scope
// stores. Every thread calls it.
template <int DT, bool SIG, int PT>
__device__ __forceinline__ void resid_phase_a(const ResidArgs& a, RowInfo inf, int b, int c4) {
  using T = typename Dt<DT>::T;
  constexpr int NQ = PT / kPickPerThread;
  __shared__ double sm_pair[8 * NQ];
  const int tid = threadIdx.x;
  ResidConsts k;
  const T* rowT;
  const T* rowD;
  resid_setup<DT, SIG>(a, inf, b, k, rowT, rowD);
  if (inf.a >= 0) {
    double R[NQ], P[NQ];
    resid_span_masses<DT, SIG, PT>(k, rowT, rowD, int64_t(c4) * (kThreads * PT), a.V, sm_pair, R, P);
    if (tid == 0) {
      const int c = NQ * c4;
      uint64_t* wp = reinterpret_cast<uint64_t*>(a.cmass + (int64_t(b) * a.S + c) * 2);
#pragma unroll
      for (int h = 0; h < NQ; ++h) {
        if (c + h < a.S) {
          dev_store(wp + 2 * h, dbits(R[h]));
          dev_store(wp + 2 * h + 1, dbits(P[h]));
        }
      }
    }
  }
}

// Phase B of the draw of batch row b, once every chunk mass of the row is in
// a.cmass: the chunk holding u * Z, then the token inside it (and the cache
// hit when a lookup is attached). Every thread calls it.
template <int DT, bool SIG>
__device__ __forceinline__ void resid_phase_b(const ResidArgs& a, RowInfo inf, int b) {
  using T = typename Dt<DT>::T;
  __shared__ double sm_pre, sm_target;
  __shared__ int sm_c, sm_useres;
  __shared__ PickLds<DT, 2, kPickPerThread> sm_pk;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  ResidConsts k;
  const T* rowT;
  const T* rowD;
  resid_setup<DT, SIG>(a, inf, b, k, rowT, rowD);
  if (inf.a < 0) {
    if (tid == 0 && !a.tok_at_a) {
      a.tok_out[int64_t(b) * a.tok_stride] = -1;
      if (a.mass_out) a.mass_out[b] = __builtin_nanf("");
    }
    if (tid == 0 && a.hit) {
      a.hit[b] = 0;
      if (a.slot) a.slot[b] = -1;
    }
    return;
  }
  // the cache segment of length a (at most 64 tokens, lane i holds slot i),
  // requested first so that its round trip overlaps those of the draw
  int32_t seg_tok = -1;
  if (a.hit && w == 0) {
    const int n = a.lk_F[inf.a];
    // device-scope: the cache may come from another workgroup of this launch
    seg_tok = lane < n ? int32_t(dev_load32(reinterpret_cast<const uint32_t*>(a.cache_tokens) +
                                            int64_t(b) * a.sumF + a.lk_off[inf.a] + lane))
                       : -1;
  }
  // chunk masses, then the first chunk whose running mass exceeds u * Z
  if (w == 0) {
    double zres, ztgt, target, pre;
    int useres, cs;
    resid_find_chunk(reinterpret_cast<const uint64_t*>(a.cmass + int64_t(b) * a.S * 2), a.S, a.u[b], lane, zres,
                     ztgt, useres, target, cs, pre);
    if (lane == 0) {
      sm_c = cs;
      sm_pre = pre;
      sm_target = target;
      sm_useres = useres;
      if (a.mass_out) a.mass_out[b] = useres ? float(zres / inf.s_t) : 0.0f;
    }
  }
  __syncthreads();
  const int cs = sm_c;
  int tok = -1;
  if (cs >= 0) {
    if (!sm_useres) set_plain(k);
    tok = resid_pick<DT, SIG, kPickPerThread>(k, rowT, rowD, cs, sm_pre, sm_target, a.V, sm_pk);
  }
  if (tid == 0) a.tok_out[int64_t(b) * a.tok_stride + (a.tok_at_a ? inf.a : 0)] = tok;
  if (a.hit && w == 0) {
    // cache hit of the outcome (a, t*)
    const uint64_t m = __ballot(tok >= 0 && seg_tok == tok);
    if (lane == 0) {
      a.hit[b] = m != 0 ? 1 : 0;
      if (a.slot) a.slot[b] = m != 0 ? __ffsll((unsigned long long)m) - 1 : -1;
    }
  }
}

// Workgroups of the draw per batch row (one per span of 256 * span_pt
// entries, span_pt / 16 pick chunks each).
__host__ __device__ __forceinline__ int resid_wgs_per_row(int S, int span_pt) {
  const int nq = span_pt / kPickPerThread;
  return (S + nq - 1) / nq;
}

// The residual / bonus draw of batch row b by one of its resid_wgs_per_row
// workgroups (c4: its span), given the row's RowInfo as written by the
// accept scan: phase A, then phase B in the workgroup that arrives last.
// Every thread calls it; returns true in the workgroup that finished the
// row.
template <int DT, bool SIG, int PT>
__device__ __forceinline__ bool resid_row_wg(const ResidArgs& a, RowInfo inf, int b, int c4) {
  __shared__ int sm_last;
  resid_phase_a<DT, SIG, PT>(a, inf, b, c4);
  if (!arrive_last(&a.cnt[int64_t(b) * kCntStride], uint32_t(resid_wgs_per_row(a.S, PT)), &sm_last)) return false;
  resid_phase_b<DT, SIG>(a, inf, b);
  return true;
}

}  // namespace ssd

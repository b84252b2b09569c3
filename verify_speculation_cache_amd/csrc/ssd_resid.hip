// Correction / bonus draw by inverse CDF.
//
// After a rejection at position a the replacement token is drawn from
// max(0, p_a - q_a)/Z; after a full accept the bonus is drawn from p_K
// (brentwoodlivery.com "Speculative decoding", The Algorithm, step 3, and
// Derivation of Acceptance Criterion; til.phipham141.dev "Why does
// speculative decoding exist?", Fix 2 and Fix 3). The draw is the smallest
// token v (in index order) whose running residual mass exceeds u * Z.
//
// Units: everything is kept relative to the target row, e_t(v) =
// exp((z_t(v) - pivot_t)/tau), so p = e_t / s_t and the residual mass is
// r(v) = max(0, e_t(v) - rho_w * e_d(v)) with rho_w = w * s_t / s_d (w = C
// for sigma members, else 1); rho is split into two floats so the
// subtraction keeps double-precision scaling.
//
// Phase A (all workgroups): one workgroup per (batch row, chunk) sums r and
// e_t over its chunk (per-thread float sums, double across threads).
// Phase B (last workgroup of the batch row): walks the chunk masses in order
// to find the chunk holding u*Z, re-reads that chunk with each thread owning
// 32 consecutive tokens, scans thread totals in double and picks the token.
// If rounding leaves no crossing inside the chosen chunk the last token of
// that chunk with positive mass is taken. With no residual mass at all the
// draw uses p (e_t) instead; with no mass in p either the token is -1.
#include "ssd_cdf.hpp"

namespace ssd {

struct ResidConsts {
  float piv_t, piv_d, c32;
  float rho_hi, rho_lo, rhoC_hi, rhoC_lo;
  float thr_val;     // sigma threshold as a logit value (key order = value order)
  int32_t thr_idx;
  bool plain;        // value is e_t itself (bonus draw, or no residual mass)
};

__device__ __forceinline__ void split2(double v, float& hi, float& lo) {
  hi = float(v);
  lo = float(v - double(hi));
}

// Residual (or, when plain, target) mass of one entry in target units.
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
  return k.plain ? et : fmaxf(r, 0.0f);
}

__device__ __forceinline__ float target_elem(const ResidConsts& k, float xt) {
  return __builtin_amdgcn_exp2f((xt - k.piv_t) * k.c32);
}

template <int DT, bool SIG>
__global__ __launch_bounds__(kThreads) void k_resid(ResidArgs a) {
  using T = typename Dt<DT>::T;
  constexpr int PV = Dt<DT>::kPerVec;
  constexpr int NV = kPerThread / PV;
  __shared__ double sm_pair[8];
  __shared__ int sm_last;
  __shared__ double sm_pre, sm_target;
  __shared__ int sm_c, sm_useres;
  __shared__ PickLds<DT, 2> sm_pk;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = blockIdx.x / a.S;
  const int c = blockIdx.x - b * a.S;
  RowInfo inf = a.info[b];
  // Only trust a row index the stats kernel could have written: anything
  // else (a workspace that was not zero-filled for this shape) is treated
  // as a flagged row, so stale state can never address outside the inputs.
  if (inf.a < -1 || inf.a > a.K) inf.a = -1;
  if (inf.a == a.K || a.draft == nullptr) inf.bonus = 1;

  // A bonus row has no draft: it reads the target row twice with rho = 0,
  // so both rows take the same load and arithmetic path.
  ResidConsts k{};
  const T* rowT = nullptr;
  const T* rowD = nullptr;
  if (inf.a >= 0) {
    rowT = static_cast<const T*>(a.target) + int64_t(b) * a.tb + int64_t(inf.a) * a.V;
    k.piv_t = inf.piv_t;
    k.c32 = a.c32;
    k.thr_val = value_of_key<DT>(inf.thr_key);
    k.thr_idx = inf.thr_idx;
    if (inf.bonus) {
      rowD = rowT;
      k.piv_d = inf.piv_t;
      k.plain = true;
    } else {
      rowD = static_cast<const T*>(a.draft) + int64_t(b) * a.db + int64_t(inf.a) * a.V;
      k.piv_d = inf.piv_d;
      const double rho = inf.s_d > 0.0 ? inf.s_t / inf.s_d : 0.0;
      split2(rho, k.rho_hi, k.rho_lo);
      split2(rho * double(inf.C), k.rhoC_hi, k.rhoC_lo);
    }
  }
  // sigma thresholds that admit no entry (key above that of +inf)
  if (SIG && inf.thr_key > key_of<DT>(__builtin_inff())) k.thr_val = __builtin_nanf("");

  // ---------------- phase A: chunk masses ----------------
  if (inf.a >= 0) {
    const int64_t c0 = int64_t(c) * kChunk;
    ChunkVecs<DT, true> vt, vd;
    load_pair(vt, rowT, vd, rowD, c0, a.V, tid);
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
    const double R = wave_sum(double(rs));
    const double P = wave_sum(double(ts));
    if (lane == 0) {
      sm_pair[w] = R;
      sm_pair[4 + w] = P;
    }
    __syncthreads();
    if (tid == 0) {
      uint64_t* wp = reinterpret_cast<uint64_t*>(a.cmass + (int64_t(b) * a.S + c) * 2);
      dev_store(wp, dbits((sm_pair[0] + sm_pair[1]) + (sm_pair[2] + sm_pair[3])));
      dev_store(wp + 1, dbits((sm_pair[4] + sm_pair[5]) + (sm_pair[6] + sm_pair[7])));
    }
  }

  if (!arrive_last(&a.cnt[int64_t(b) * kCntStride], uint32_t(a.S), &sm_last)) return;

  // ---------------- phase B: last workgroup of batch row b ----------------
  if (inf.a < 0) {
    if (tid == 0 && !a.tok_at_a) {
      a.tok_out[int64_t(b) * a.tok_stride] = -1;
      if (a.mass_out) a.mass_out[b] = __builtin_nanf("");
    }
    return;
  }
  // chunk masses (one lane per chunk, one round trip for S <= 64), prefix
  // sums by a fixed wave scan, then the first chunk whose running mass
  // exceeds u * Z
  if (w == 0) {
    const uint64_t* cmw = reinterpret_cast<const uint64_t*>(a.cmass + int64_t(b) * a.S * 2);
    double zres = 0.0, ztgt = 0.0;   // totals over chunk groups
    double r0 = 0.0, t0 = 0.0;        // this lane's masses in the first group
    for (int g = 0; g < a.S; g += 64) {
      const int cc = g + lane;
      const double r = cc < a.S ? bits_d(dev_load(cmw + cc * 2)) : 0.0;
      const double t = cc < a.S ? bits_d(dev_load(cmw + cc * 2 + 1)) : 0.0;
      if (g == 0) {
        r0 = r;
        t0 = t;
      }
      zres += __shfl(wave_incl_scan_d(r, lane), 63);
      ztgt += __shfl(wave_incl_scan_d(t, lane), 63);
    }
    const int useres = zres > 0.0 ? 1 : 0;
    const double tot = useres ? zres : ztgt;
    const double target = double(a.u[b]) * tot;
    int cs = -1;
    double pre = 0.0;
    if (tot > 0.0) {
      chunk_crossing(
          [&](int cc, int g) -> double {
            if (g == 0) return useres ? r0 : t0;
            return cc < a.S ? bits_d(dev_load(cmw + cc * 2 + (useres ? 0 : 1))) : 0.0;
          },
          a.S, target, lane, cs, pre);
    }
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
    if (!sm_useres) k.plain = true;
    const int64_t c0 = int64_t(cs) * kChunk;
    // each thread owns 32 consecutive tokens of the chunk
    ChunkVecs<DT, false> cv[2];
    load_pair(cv[0], rowT, cv[1], rowD, c0, a.V, tid);
    tok = chunk_pick<DT, 2>(cv, c0, sm_pre, sm_target,
                            [&](const float (&x)[2], int idx) { return resid_elem<SIG>(k, x[0], x[1], idx); },
                            sm_pk);
  }
  if (tid == 0) a.tok_out[int64_t(b) * a.tok_stride + (a.tok_at_a ? inf.a : 0)] = tok;
}

hipError_t launch_resid(const ResidArgs& a, int dtype, bool sigma, hipStream_t st) {
  const unsigned grid = unsigned(int64_t(a.B) * a.S);
  if (dtype == SSD_BF16) {
    if (sigma) hipLaunchKernelGGL((k_resid<1, true>), dim3(grid), dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((k_resid<1, false>), dim3(grid), dim3(kThreads), 0, st, a);
  } else {
    if (sigma) hipLaunchKernelGGL((k_resid<0, true>), dim3(grid), dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((k_resid<0, false>), dim3(grid), dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace ssd

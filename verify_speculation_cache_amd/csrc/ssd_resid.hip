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
#include "ssd_device.hpp"

namespace ssd {

struct ResidConsts {
  float piv_t, piv_d, c32;
  float rho_hi, rho_lo, rhoC_hi, rhoC_lo;
  uint32_t thr_key;
  int32_t thr_idx;
  int bonus;
};

__device__ __forceinline__ void split2(double v, float& hi, float& lo) {
  hi = float(v);
  lo = float(v - double(hi));
}

template <int DT, bool SIG>
__device__ __forceinline__ float resid_elem(const ResidConsts& k, float xt, float xd, int64_t idx) {
  const float et = __builtin_amdgcn_exp2f((xt - k.piv_t) * k.c32);
  const float ed = __builtin_amdgcn_exp2f((xd - k.piv_d) * k.c32);
  float hi = k.rho_hi, lo = k.rho_lo;
  if constexpr (SIG) {
    const uint32_t kk = key_of<DT>(xd);
    const bool mem = (kk > k.thr_key) || (kk == k.thr_key && idx <= int64_t(k.thr_idx));
    hi = mem ? k.rhoC_hi : hi;
    lo = mem ? k.rhoC_lo : lo;
  }
  float r = __builtin_fmaf(-hi, ed, et);
  r = __builtin_fmaf(-lo, ed, r);
  return fmaxf(r, 0.0f);
}

template <int DT>
__device__ __forceinline__ float target_elem(const ResidConsts& k, float xt) {
  return __builtin_amdgcn_exp2f((xt - k.piv_t) * k.c32);
}

template <int DT, bool SIG>
__global__ __launch_bounds__(kThreads) void k_resid(ResidArgs a) {
  using T = typename Dt<DT>::T;
  __shared__ double sm_d[4];
  __shared__ int sm_i[4];
  __shared__ int sm_last;
  __shared__ double sm_scan[4];
  __shared__ int sm_pick[4];
  __shared__ double sm_pre, sm_target;
  __shared__ int sm_c, sm_useres, sm_tok;

  const int tid = threadIdx.x;
  const int b = blockIdx.x / a.S;
  const int c = blockIdx.x - b * a.S;
  RowInfo inf = a.info[b];
  // Only trust a row index the stats kernel could have written: anything
  // else (a workspace that was not zero-filled for this shape) is treated
  // as a flagged row, so stale state can never address outside the inputs.
  if (inf.a < -1 || inf.a > a.K) inf.a = -1;
  if (inf.a == a.K || a.draft == nullptr) inf.bonus = 1;

  ResidConsts k{};
  const T* rowT = nullptr;
  const T* rowD = nullptr;
  if (inf.a >= 0) {
    rowT = static_cast<const T*>(a.target) + int64_t(b) * a.tb + int64_t(inf.a) * a.V;
    k.piv_t = inf.piv_t;
    k.piv_d = inf.piv_d;
    k.c32 = a.c32;
    k.bonus = inf.bonus;
    k.thr_key = inf.thr_key;
    k.thr_idx = inf.thr_idx;
    if (!inf.bonus) {
      rowD = static_cast<const T*>(a.draft) + int64_t(b) * a.db + int64_t(inf.a) * a.V;
      const double rho = inf.s_d > 0.0 ? inf.s_t / inf.s_d : 0.0;
      split2(rho, k.rho_hi, k.rho_lo);
      split2(rho * double(inf.C), k.rhoC_hi, k.rhoC_lo);
    }
  }

  // ---------------- phase A: chunk masses ----------------
  if (inf.a >= 0) {
    const int64_t c0 = int64_t(c) * kChunk;
    const bool full = c0 + kChunk <= a.V;
    const bool vt = (reinterpret_cast<uintptr_t>(rowT) & 15u) == 0;
    float xt[kPerThread];
    load_strided<DT>(rowT, c0, a.V, vt, tid, xt);
    float rs = 0.0f, ts = 0.0f;
    if (inf.bonus) {
#pragma unroll
      for (int q = 0; q < kPerThread; ++q) ts += target_elem<DT>(k, xt[q]);
      rs = ts;
    } else {
      const bool vd = (reinterpret_cast<uintptr_t>(rowD) & 15u) == 0;
      float xd[kPerThread];
      load_strided<DT>(rowD, c0, a.V, vd, tid, xd);
#pragma unroll
      for (int q = 0; q < kPerThread; ++q) {
        ts += target_elem<DT>(k, xt[q]);
        rs += resid_elem<DT, SIG>(k, xt[q], xd[q], Strided<DT>::index(c0, tid, q));
      }
    }
    const double R = block_sum(double(rs), sm_d);
    const double P = block_sum(double(ts), sm_d);
    if (tid == 0) {
      uint64_t* w = reinterpret_cast<uint64_t*>(a.cmass + (int64_t(b) * a.S + c) * 2);
      dev_store(w, dbits(R));
      dev_store(w + 1, dbits(P));
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
  // chunk masses in parallel (one lane per chunk), prefix sums by a fixed
  // wave scan, then the first chunk whose running mass exceeds u * Z.
  if (tid < 64) {
    const int lane = tid;
    const uint64_t* cmw = reinterpret_cast<const uint64_t*>(a.cmass + int64_t(b) * a.S * 2);
    double zres = 0.0, ztgt = 0.0;   // running totals over chunk groups
    for (int g = 0; g < a.S; g += 64) {
      const int cc = g + lane;
      const double r = cc < a.S ? bits_d(dev_load(cmw + cc * 2)) : 0.0;
      const double t = cc < a.S ? bits_d(dev_load(cmw + cc * 2 + 1)) : 0.0;
      zres += __shfl(wave_incl_scan_d(r, lane), 63);
      ztgt += __shfl(wave_incl_scan_d(t, lane), 63);
    }
    const int useres = zres > 0.0 ? 1 : 0;
    const double tot = useres ? zres : ztgt;
    const double target = double(a.u[b]) * tot;
    int cs = -1;
    double pre = 0.0;
    if (tot > 0.0) {
      double base = 0.0;
      int lastpos = -1;
      double lastpre = 0.0;
      for (int g = 0; g < a.S && cs < 0; g += 64) {
        const int cc = g + lane;
        const double mc = cc < a.S ? bits_d(dev_load(cmw + cc * 2 + (useres ? 0 : 1))) : 0.0;
        const double incl = wave_incl_scan_d(mc, lane);
        const double prev = __shfl_up(incl, 1);   // all lanes shuffle (lane 0 reads itself)
        const double excl = base + (lane > 0 ? prev : 0.0);
        const uint64_t crossing = __ballot(cc < a.S && base + incl > target);
        const uint64_t pos = __ballot(cc < a.S && mc > 0.0);
        if (crossing) {
          const int l = __ffsll((unsigned long long)crossing) - 1;
          cs = g + l;
          pre = __shfl(excl, l);
        } else if (pos) {
          const int l = 63 - __clzll((long long)pos);
          lastpos = g + l;
          lastpre = __shfl(excl, l);
        }
        base += __shfl(incl, 63);
      }
      if (cs < 0) {   // rounding left u*Z past the last crossing: last chunk with mass
        cs = lastpos;
        pre = lastpre;
      }
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
    const int64_t c0 = int64_t(cs) * kChunk;
    const bool full = c0 + kChunk <= a.V;
    const bool useres = sm_useres != 0 && !inf.bonus;
    float xt[kPerThread], xd[kPerThread];
    load_run<DT>(rowT, c0, a.V, (reinterpret_cast<uintptr_t>(rowT) & 15u) == 0, tid, xt);
    if (useres)
      load_run<DT>(rowD, c0, a.V, (reinterpret_cast<uintptr_t>(rowD) & 15u) == 0, tid, xd);
    const int64_t base_idx = c0 + int64_t(tid) * kPerThread;
    float v[kPerThread];
#pragma unroll
    for (int q = 0; q < kPerThread; ++q)
      v[q] = useres ? resid_elem<DT, SIG>(k, xt[q], xd[q], base_idx + q) : target_elem<DT>(k, xt[q]);
    double tot = 0.0;
    int lastpos = -1;
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
      tot += double(v[q]);
      if (v[q] > 0.0f) lastpos = q;
    }
    // exclusive scan of thread totals (thread order = token order)
    const int lane = tid & 63, w = tid >> 6;
    const double incl_w = wave_incl_scan_d(tot, lane);
    if (lane == 63) sm_scan[w] = incl_w;
    __syncthreads();
    double wbase = 0.0;
    for (int ww = 0; ww < w; ++ww) wbase += sm_scan[ww];
    const double excl = wbase + (incl_w - tot);
    const double base = sm_pre + excl;
    const double target = sm_target;
    const bool cross = (base + tot) > target;
    // first crossing thread
    const uint64_t cm = __ballot(cross);
    if (lane == 0) sm_pick[w] = cm ? (w * 64 + __ffsll((unsigned long long)cm) - 1) : 0x7FFFFFFF;
    __syncthreads();
    const int first = min(min(sm_pick[0], sm_pick[1]), min(sm_pick[2], sm_pick[3]));
    __syncthreads();
    if (first != 0x7FFFFFFF) {
      if (tid == first) {
        double run = 0.0;   // same association as `tot`, so q = 31 reproduces `cross`
        int pick = lastpos;
        for (int q = 0; q < kPerThread; ++q) {
          run += double(v[q]);
          if (base + run > target) {
            pick = q;
            break;
          }
        }
        sm_tok = int(base_idx + pick);
      }
    } else {
      // rounding left u*Z past this chunk's scan: last token with mass
      const int cand = lastpos >= 0 ? int(base_idx + lastpos) : -1;
      int best = cand;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) best = max(best, __shfl_xor(best, o));
      if (lane == 0) sm_i[w] = best;
      __syncthreads();
      if (tid == 0) sm_tok = max(max(sm_i[0], sm_i[1]), max(sm_i[2], sm_i[3]));
    }
    __syncthreads();
    tok = sm_tok;
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

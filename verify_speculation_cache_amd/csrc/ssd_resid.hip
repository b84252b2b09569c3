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
// Phase A (all workgroups): one workgroup per (batch row, pair of chunks)
// sums r and e_t over each chunk (per-thread float sums, double across
// threads).
// Phase B (last workgroup of the batch row): walks the chunk masses in order
// to find the chunk holding u*Z, re-reads that chunk with each thread owning
// 32 consecutive tokens, scans thread totals in double and picks the token.
// If rounding leaves no crossing inside the chosen chunk the last token of
// that chunk with positive mass is taken. With no residual mass at all the
// draw uses p (e_t) instead; with no mass in p either the token is -1.
#include "ssd_resid.hpp"

namespace ssd {

template <int DT, bool SIG>
__global__ __launch_bounds__(kThreads) void k_resid(ResidArgs a) {
  using T = typename Dt<DT>::T;
  __shared__ double sm_pair[16];
  __shared__ int sm_last;
  __shared__ double sm_pre, sm_target;
  __shared__ int sm_c, sm_useres;
  __shared__ PickLds<DT, 2> sm_pk;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int S2 = (a.S + 1) / 2;   // workgroups per batch row, two 8192-chunks each
  const int b = blockIdx.x / S2;
  const int c2 = blockIdx.x - b * S2;
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
      set_plain(k);
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
    double R[2], P[2];
    resid_chunk_masses2<DT, SIG>(k, rowT, rowD, int64_t(c2) * kStatsChunk, a.V, sm_pair, R, P);
    if (tid == 0) {
      const int c = 2 * c2;
      uint64_t* wp = reinterpret_cast<uint64_t*>(a.cmass + (int64_t(b) * a.S + c) * 2);
      dev_store(wp, dbits(R[0]));
      dev_store(wp + 1, dbits(P[0]));
      if (c + 1 < a.S) {
        dev_store(wp + 2, dbits(R[1]));
        dev_store(wp + 3, dbits(P[1]));
      }
    }
  }

  if (!arrive_last(&a.cnt[int64_t(b) * kCntStride], uint32_t(S2), &sm_last)) return;

  // ---------------- phase B: last workgroup of batch row b ----------------
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
    seg_tok = lane < n ? a.cache_tokens[int64_t(b) * a.sumF + a.lk_off[inf.a] + lane] : -1;
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
    tok = resid_pick<DT, SIG>(k, rowT, rowD, cs, sm_pre, sm_target, a.V, sm_pk);
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

hipError_t launch_resid(const ResidArgs& a, int dtype, bool sigma, hipStream_t st) {
  const unsigned grid = unsigned(int64_t(a.B) * ((a.S + 1) / 2));
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

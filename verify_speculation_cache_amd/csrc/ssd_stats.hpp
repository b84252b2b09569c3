// Device code of the row-statistics pass and its per-row epilogue (shared
// by the verification kernels and the fused verification round).
//
// Row statistics and the accept scan.
//
// Grid: one workgroup per (batch row b, logit row r, vocabulary chunk c),
// b slowest, so each batch row's workgroups are dispatched together and its
// epilogue runs while later batch rows still stream. A workgroup reads its
// 8192-entry chunk once (16-byte loads, one 1 KiB span per wave
// instruction), reduces the chunk max and the chunk sum of
// exp((z - max)/tau), and writes them. The last workgroup of a batch row to
// finish merges the chunk partials in chunk order and then:
//  - verify: takes p and q at the drafted tokens and runs the accept scan
//    (keep d iff u*q(d) < p(d), stop at the first rejection) of
//    brentwoodlivery.com "Speculative decoding", The Algorithm, step 3, with
//    q optionally the sigma_{F,C} form of papernotes.org "Speculative
//    Speculative Decoding", key design 2;
//  - rows mode: records the statistics of the one position to sample from.
// Either way it leaves a RowInfo for the residual / bonus kernel.
#pragma once

#include "ssd_device.hpp"

namespace ssd {

template <int DT>
__device__ const typename Dt<DT>::T* stats_row_ptr(const StatsArgs& a, int b, int r) {
  using T = typename Dt<DT>::T;
  const T* tgt = static_cast<const T*>(a.target);
  const T* dft = static_cast<const T*>(a.draft);
  if (a.mode != kModeRows) {
    if (r <= a.K) return tgt + int64_t(b) * a.tb + int64_t(r) * a.V;
    return dft + int64_t(b) * a.db + int64_t(r - a.K - 1) * a.V;
  }
  const int j = a.rows_in[b];
  if (j < 0 || j > a.K) return nullptr;
  if (r == 0) return tgt + int64_t(b) * a.tb + int64_t(j) * a.V;
  if (a.use_draft && !a.use_sigma && j < a.K) return dft + int64_t(b) * a.db + int64_t(j) * a.V;
  return nullptr;
}

template <int DT>
__device__ __forceinline__ float load_one(const void* base, int64_t off) {
  return Dt<DT>::to_f(static_cast<const typename Dt<DT>::T*>(base)[off]);
}

// sigma membership of token idx (value x) in the top-F set bounded by thr
template <int DT>
__device__ __forceinline__ bool in_top(float x, int32_t idx, uint32_t tkey, int32_t tidx) {
  const uint32_t k = key_of<DT>(x);
  return (k > tkey) || (k == tkey && idx <= tidx);
}

// sigma statistics of draft row i of batch row b (written by the cache
// merge, possibly by another workgroup of the same launch): the max logit,
// S_top, S_rest, and the threshold key of the top-F set
__device__ __forceinline__ void load_sigma(const StatsArgs& a, int b, int i, double& zmax, double& stop,
                                           double& srest, ssd_rowkey& tk) {
  const uint64_t* sp = reinterpret_cast<const uint64_t*>(a.dstats + (int64_t(b) * (a.K + 1) + i) * 3);
  zmax = bits_d(dev_load(sp));
  stop = bits_d(dev_load(sp + 1));
  srest = bits_d(dev_load(sp + 2));
  const uint64_t t = dev_load(reinterpret_cast<const uint64_t*>(a.thr + int64_t(b) * (a.K + 1) + i));
  tk.key = uint32_t(t);
  tk.idx = int32_t(uint32_t(t >> 32));
}

// The chunk pass of one workgroup over chunk c of logit row r of batch row
// b (chunks of kThreads * PT entries, a.S of them per row). The partial and
// any gathered logits are left with device-scope stores by thread 0.
template <int DT, int PT = kStatsPerThread>
__device__ __forceinline__ void stats_chunk_at(const StatsArgs& a, int b, int r, int c) {
  constexpr int kSpan = kThreads * PT;
  __shared__ float sm_f[4];
  __shared__ double sm_s[4];

  const int tid = threadIdx.x;
  const typename Dt<DT>::T* row = stats_row_ptr<DT>(a, b, r);
  if (row != nullptr) {  // uniform per workgroup
    using CV = ChunkVecs<DT, true, PT>;
    const int64_t c0 = int64_t(c) * kSpan;
    CV cv;
    cv.load(row, c0, a.V, (reinterpret_cast<uintptr_t>(row) & 15u) == 0, tid);
    // the chunk's loads are in flight before the drafted token is read
    __builtin_amdgcn_sched_barrier(0);
    // The workgroup whose chunk holds drafted token d_r (target row r < K)
    // also fetches z_t(d_r) and z_d(d_r) for the accept test, so the
    // epilogue finds them with the partials.
    int32_t dtok = -1;
    if (a.mode != kModeRows && r < a.K) dtok = a.tokens[int64_t(b) * a.K + r];
    const bool owns = dtok >= 0 && dtok < a.V && int64_t(dtok) >= c0 && int64_t(dtok) < c0 + kSpan;
    float gzt = 0.0f, gzd = 0.0f;
    if (owns && tid == 0) {
      gzt = load_one<DT>(a.target, int64_t(b) * a.tb + int64_t(r) * a.V + dtok);
      gzd = load_one<DT>(a.draft, int64_t(b) * a.db + int64_t(r) * a.V + dtok);
    }
    float m;
    double sd;
    chunk_max_sum(cv, a.c32, sm_f, sm_s, m, sd);
    if (tid == 0) {
      uint64_t* wp = reinterpret_cast<uint64_t*>(a.part + (int64_t(b) * a.NR + r) * a.S + c);
      dev_store(wp, pack2(m, 0.0f));
      dev_store(wp + 1, dbits(sd));
      if (owns) dev_store(a.zg + int64_t(b) * a.K + r, pack2(gzt, gzd));
    }
  }
}

// The same for workgroup blk = (b * NR + r) * S + c of a one-chunk-per-
// workgroup grid.
template <int DT, int PT = kStatsPerThread>
__device__ __forceinline__ void stats_chunk_wg(const StatsArgs& a, uint32_t blk) {
  const uint32_t b = fdiv(blk, a.div_pb);
  const uint32_t rem = blk - b * uint32_t(a.NR * a.S);
  const uint32_t r = fdiv(rem, a.div_s);
  stats_chunk_at<DT, PT>(a, int(b), int(r), int(rem - r * uint32_t(a.S)));
}

// Row max pivots and sums of the a.NR logit rows of batch row b, merged
// from their chunk partials (loaded with device-scope loads: the partials
// may come from other workgroups of the same launch). Called by every
// thread; the results are in e_piv / e_s after the caller's barrier.
__device__ __forceinline__ void merge_row_partials(const StatsArgs& a, int b, float* e_piv, double* e_s) {
  const uint64_t* pb = reinterpret_cast<const uint64_t*>(a.part) + int64_t(b) * a.NR * a.S * 2;
  if (a.S <= 64) merge_rows_seg(pb, a.NR, a.S, a.c32, e_piv, e_s);
  else merge_rows<2>(pb, a.NR, a.S, a.c32, e_piv, e_s, nullptr);
}

// exp2((z - piv) * c32) of one token in the scaled form of the streaming
// sums (one rounding in the argument, the pivot's product error restored by
// a second factor), returned in double for the division by the row sum.
// Its relative error (a few float ulps, plus |argument| * 2^-24) stays far
// below the 1e-6 absolute margin that decides an accept test and the 1e-5
// relative tolerance of the reported probabilities.
__device__ __forceinline__ double token_mass(float z, float piv, float c32) {
  const ScaledPivot sp = scaled_pivot(piv, c32);
  return double(scaled_mass(z, c32, sp.P)) * double(sp.fix);
}

// The accept scan of batch row b (verify mode): merges the target rows'
// partials, takes p and q at the drafted tokens, keeps d iff u*q(d) < p(d)
// up to the first rejection, and fills the RowInfo of the row to sample
// from (wave 0, lane i for drafted position i; the sigma statistics of the
// sampled row come out of the lane that loaded them). With `write`, wave 0
// also stores accepted[b], out_tokens and probs. Called by every thread;
// the RowInfo is returned in every thread (through *sm_inf, one barrier)
// when BCAST, else only in wave 0. BCAST is for a caller that draws in the
// same launch: out_tokens at the accepted length is then not written here
// (the draw stores it). e_piv / e_s stay valid for the caller.
template <int DT, bool BCAST>
__device__ __forceinline__ RowInfo accept_scan(const StatsArgs& a, int b, bool write, float* e_piv, double* e_s,
                                               RowInfo* sm_inf) {
  const int tid = threadIdx.x;
  const int K = a.K;
  // per drafted position (wave 0, lane i < K): inputs of the accept test,
  // loaded before the merge so that all loads share one round trip
  int32_t d = -1;
  float ua = 0.0f, zt = 0.0f, zd = 0.0f;
  double sp0 = 0.0, sp1 = 0.0, sp2 = 0.0;
  ssd_rowkey tk{0xFFFFFFFFu, -1};
  if (tid < K) {
    const int i = tid;
    d = a.tokens[int64_t(b) * K + i];
    ua = a.u_acc[int64_t(b) * K + i];
    const uint64_t g = dev_load(a.zg + int64_t(b) * K + i);   // valid only for 0 <= d < V
    zt = lo_f(g);
    zd = __uint_as_float(uint32_t(g >> 32));
    if (a.use_sigma) load_sigma(a, b, i, sp0, sp1, sp2, tk);
  }
  merge_row_partials(a, b, e_piv, e_s);
  __syncthreads();

  RowInfo inf{};
  if (tid < 64) {
    const int i = tid;
    bool bad = false, acc = true;
    double pd = 0.0, qd = 0.0;
    if (i < K) {
      bad = (d < 0 || d >= a.V);
      if (!bad) {
        const double st = e_s[i];
        pd = st > 0.0 ? token_mass(zt, e_piv[i], a.c32) / st : 0.0;
        double pivd, sdn, wgt = 1.0;
        if (a.use_sigma) {
          pivd = double(pivot_of(float(sp0)));
          sdn = double(a.C) * sp1 + sp2;
          if (in_top<DT>(zd, d, tk.key, tk.idx)) wgt = double(a.C);
        } else {
          pivd = double(e_piv[K + 1 + i]);
          sdn = e_s[K + 1 + i];
        }
        qd = sdn > 0.0 ? wgt * token_mass(zd, float(pivd), a.c32) / sdn : 0.0;
        acc = double(ua) * qd < pd;
      }
    }
    const uint64_t badm = __ballot(i < K && bad);
    const uint64_t rej = __ballot(i < K && !acc);
    const int av = badm ? -1 : (rej ? (__ffsll((unsigned long long)rej) - 1) : K);   // wave-uniform
    if (write) {
      if (i < K && a.probs != nullptr) {
        a.probs[(int64_t(b) * K + i) * 2 + 0] = float(pd);
        a.probs[(int64_t(b) * K + i) * 2 + 1] = float(qd);
      }
      // positions 0..K: the kept drafts (lane ii < av <= K holds d_ii), then
      // -1; position av is left to the draw when BCAST (the draw runs in the
      // same launch and stores the token there)
      for (int ii = i; ii <= K; ii += 64)
        if (!BCAST || ii != av) a.out_tokens[int64_t(b) * (K + 1) + ii] = (av >= 0 && ii < av) ? d : -1;
      if (i == 0) a.accepted[b] = av;
    }

    inf.a = av;
    inf.C = 1.0f;
    inf.thr_key = 0xFFFFFFFFu;
    inf.thr_idx = -1;
    if (av >= 0) {
      inf.bonus = (av == K) ? 1 : 0;
      inf.piv_t = e_piv[av];
      inf.s_t = e_s[av];
      if (!inf.bonus) {
        if (a.use_sigma) {   // av < K <= 64: lane av holds draft row av's statistics
          auto rl_d = [av](double v) {
            const uint64_t u = dbits(v);
            const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(u)), av));
            const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(u >> 32)), av));
            return bits_d(uint64_t(lo) | (uint64_t(hi) << 32));
          };
          inf.piv_d = pivot_of(float(rl_d(sp0)));
          inf.s_d = double(a.C) * rl_d(sp1) + rl_d(sp2);
          inf.thr_key = uint32_t(__builtin_amdgcn_readlane(int(tk.key), av));
          inf.thr_idx = __builtin_amdgcn_readlane(tk.idx, av);
          inf.C = a.C;
        } else {
          inf.piv_d = e_piv[K + 1 + av];
          inf.s_d = e_s[K + 1 + av];
        }
      }
    }
    if (BCAST && i == 0) *sm_inf = inf;
  }
  if (BCAST) {
    __syncthreads();
    // the same in every lane: kept in scalar registers
    auto u32 = [](const void* p) { return uint32_t(__builtin_amdgcn_readfirstlane(*static_cast<const int*>(p))); };
    auto f32 = [&](const float* p) { return __uint_as_float(u32(p)); };
    auto f64 = [&](const double* p) {
      const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
      return bits_d(uint64_t(u32(q)) | (uint64_t(u32(q + 1)) << 32));
    };
    inf.a = int32_t(u32(&sm_inf->a));
    inf.bonus = int32_t(u32(&sm_inf->bonus));
    inf.piv_t = f32(&sm_inf->piv_t);
    inf.piv_d = f32(&sm_inf->piv_d);
    inf.s_t = f64(&sm_inf->s_t);
    inf.s_d = f64(&sm_inf->s_d);
    inf.thr_key = u32(&sm_inf->thr_key);
    inf.thr_idx = int32_t(u32(&sm_inf->thr_idx));
    inf.C = f32(&sm_inf->C);
  }
  return inf;
}

// Optional log-normalisers of batch row b's 2K+1 rows (verify mode), from
// the merged partials in e_piv / e_s (target rows 0..K, and draft rows
// without sigma) or the sigma statistics (draft rows with sigma):
// lse = pivot / tau + ln(sum). Called by every thread after accept_scan.
__device__ __forceinline__ void write_row_lse(const StatsArgs& a, int b, const float* e_piv, const double* e_s) {
  if (a.row_lse == nullptr) return;
  const int K = a.K;
  for (int rr = threadIdx.x; rr < 2 * K + 1; rr += kThreads) {
    double l;
    if (rr <= K || !a.use_sigma) {
      const double s = e_s[rr];
      l = s > 0.0 ? double(e_piv[rr]) * a.inv_tau + log(s) : -__builtin_inf();
    } else {
      double z0, st1, st2;
      ssd_rowkey tk;
      load_sigma(a, b, rr - K - 1, z0, st1, st2, tk);
      const double s = double(a.C) * st1 + st2;
      l = s > 0.0 ? double(pivot_of(float(z0))) * a.inv_tau + log(s) : -__builtin_inf();
    }
    a.row_lse[int64_t(b) * (2 * K + 1) + rr] = float(l);
  }
}

// RowInfo of the draw ssd_residual_sample makes for batch row b (rows mode:
// logit row 0 = target row j = rows_in[b], row 1 = draft row j): merges the
// two rows' chunk partials (loaded with device-scope loads) and takes the
// sigma statistics of draft row j when sigma is given. Every thread calls
// it; the result is returned in every thread (through *sm_inf, one barrier).
__device__ __forceinline__ RowInfo rows_mode_info(const StatsArgs& a, int b, float* e_piv, double* e_s,
                                                  RowInfo* sm_inf) {
  const int K = a.K;
  merge_row_partials(a, b, e_piv, e_s);
  __syncthreads();
  if (threadIdx.x == 0) {
    RowInfo inf{};
    const int j = a.rows_in[b];
    inf.C = 1.0f;
    inf.thr_key = 0xFFFFFFFFu;
    inf.thr_idx = -1;
    if (j < 0 || j > K) {
      inf.a = -1;
    } else {
      inf.a = j;
      inf.bonus = (a.use_draft && j < K) ? 0 : 1;
      inf.piv_t = e_piv[0];
      inf.s_t = e_s[0];
      if (!inf.bonus) {
        if (a.use_sigma) {
          double z0, st1, st2;
          ssd_rowkey tk;
          load_sigma(a, b, j, z0, st1, st2, tk);
          inf.piv_d = pivot_of(float(z0));
          inf.s_d = double(a.C) * st1 + st2;
          inf.thr_key = tk.key;
          inf.thr_idx = tk.idx;
          inf.C = a.C;
        } else {
          inf.piv_d = e_piv[1];
          inf.s_d = e_s[1];
        }
      }
    }
    *sm_inf = inf;
  }
  __syncthreads();
  return *sm_inf;
}

}  // namespace ssd

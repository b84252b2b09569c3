// Speculation-cache build (top-F_k per acceptance length, sigma statistics)
// and the cache-hit lookup.
//
// The cache holds, for each acceptance length k, the F_k tokens the draft
// ranks highest on draft row k: the guessed bonus tokens for outcomes
// (k, t*) (papernotes.org "Speculative Speculative Decoding", framework and
// key designs 1-2; the cache picks its tokens by draft logit). sigma_{F,C}
// then needs, per row, S_top = sum of exp((z - zmax)/tau) over those tokens
// and S_rest over the others; both are summed directly (no subtraction), so
// C * S_top + S_rest keeps full relative accuracy for any C.
//
// Build grid: one workgroup per (batch row b, length k, chunk c), b slowest.
// Per chunk:
//  1. 8192 logits into registers, chunk max.
//  2. Per wave: the F-th largest per-lane maximum T0 (bitwise search with
//     wave ballots). Any entry of the wave's top-F has at least... fewer than
//     F strictly larger entries, hence is >= T0, so "value >= T0" keeps a
//     superset of the wave's top-F (typically F to 2F entries of 2048).
//  3. Survivors are compacted into LDS and ranked exactly by (key, index);
//     the first F become this chunk's candidates. If ties make the survivor
//     set too large for LDS, an exact bitwise search for the chunk's F-th
//     (key, index) replaces step 2.
//  4. Mass of every entry that is not a chunk candidate goes to S_rest.
// The last workgroup of a row merges the per-chunk sorted candidate lists
// (rank = own position + binary-search counts in the other lists), writes
// the F_k tokens in order, the threshold key and (zmax, S_top, S_rest).
#include "ssd_device.hpp"

namespace ssd {

constexpr int kSurvCap = 1024;    // survivor list capacity (entries)
constexpr int kMergeCap = 4096;   // candidates staged in LDS for the merge

__device__ __forceinline__ uint64_t cand_bits(Cand e) {
  return uint64_t(e.key) | (uint64_t(uint32_t(e.idx)) << 32);
}
__device__ __forceinline__ Cand bits_cand(uint64_t w) {
  Cand e;
  e.key = uint32_t(w);
  e.idx = int32_t(uint32_t(w >> 32));
  return e;
}

// Position of entry q of thread tid inside its chunk (strided layout).
template <int DT>
__device__ __forceinline__ int local_of(int tid, int q) {
  constexpr int PV = Dt<DT>::kPerVec;
  return ((q / PV) * kThreads + tid) * PV + (q % PV);
}

// chunk-local rank key for the exact search: key, then the smaller offset
template <int DT>
__device__ __forceinline__ uint64_t local_comp(float x, int loc) {
  return (uint64_t(key_of<DT>(x)) << 13) | uint64_t(kChunk - 1 - loc);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void k_cache(CacheArgs a) {
  using T = typename Dt<DT>::T;
  __shared__ Cand s_list[kMergeCap];
  __shared__ float sm_f[4];
  __shared__ double sm_d[4];
  __shared__ int sm_i[4];
  __shared__ int sm_wcnt[4];
  __shared__ int sm_last;
  __shared__ double s_sel_e[SSD_MAX_F];
  __shared__ Cand s_sel[SSD_MAX_F];
  __shared__ float sm_mrow;
  __shared__ double sm_srest;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int KP = a.K + 1;
  const int per_b = KP * a.S;
  const int b = blockIdx.x / per_b;
  const int rem = blockIdx.x - b * per_b;
  const int k = rem / a.S;
  const int c = rem - k * a.S;
  const int F = a.F[k];
  const int64_t rowid = int64_t(b) * KP + k;
  const T* row = static_cast<const T*>(a.draft) + int64_t(b) * a.db + int64_t(k) * a.V;

  const int64_t c0 = int64_t(c) * kChunk;
  const int nvalid = int(min(int64_t(kChunk), int64_t(a.V) - c0));   // entries of this chunk
  const bool full = nvalid == kChunk;
  const bool vec = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
  float x[kPerThread];
  load_strided<DT>(row, c0, a.V, vec, tid, x);
  float lm = x[0];
#pragma unroll
  for (int q = 1; q < kPerThread; ++q) lm = fmaxf(lm, x[q]);
  const float mc = block_max(lm, sm_f);
  const float piv = pivot_of(mc);
  const float c32 = a.c32;

  // ---- per-wave threshold from lane maxima ----
  float f0 = __builtin_inff();   // F == 0: no survivors
  if (F > 0) {
    const uint32_t kl = local_of<DT>(tid, 0) < nvalid ? key_of<DT>(lm) : 0u;
    uint32_t t = 0;
    for (int bit = Dt<DT>::kKeyBits - 1; bit >= 0; --bit) {
      const uint32_t cand = t | (1u << bit);
      if (__popcll(__ballot(kl >= cand)) >= F) t = cand;
    }
    f0 = (t <= key_of<DT>(-__builtin_inff())) ? -__builtin_inff() : value_of_key<DT>(t);
  }
  // survivor mask: bit q set when entry q may be among the chunk's top-F
  uint32_t smask = 0;
#pragma unroll
  for (int q = 0; q < kPerThread; ++q)
    if (x[q] >= f0 && (full || local_of<DT>(tid, q) < nvalid)) smask |= 1u << q;
  int n = block_sum_i(__popc(smask), sm_i);

  // ---- exact fallback (ties beyond LDS capacity): chunk-level F-th (key, offset) ----
  if (n > kSurvCap) {   // uniform per workgroup
    constexpr int kBits = Dt<DT>::kKeyBits + 13;
    uint64_t thr = 0;
    for (int bit = kBits - 1; bit >= 0; --bit) {
      const uint64_t cand = thr | (uint64_t(1) << bit);
      int cnt = 0;
#pragma unroll
      for (int q = 0; q < kPerThread; ++q) {
        const int loc = local_of<DT>(tid, q);
        if (loc < nvalid && local_comp<DT>(x[q], loc) >= cand) ++cnt;
      }
      if (block_sum_i(cnt, sm_i) >= F) thr = cand;
    }
    smask = 0;
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
      const int loc = local_of<DT>(tid, q);
      if (loc < nvalid && local_comp<DT>(x[q], loc) >= thr) smask |= 1u << q;
    }
  }

  // ---- mass of the entries that are not survivors ----
  float sn = 0.0f;
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const float e = __builtin_amdgcn_exp2f((x[q] - piv) * c32);
    sn += ((smask >> q) & 1u) ? 0.0f : e;
  }

  // ---- compaction of survivors into LDS ----
  const int nt = __popc(smask);
  const int incl = wave_incl_scan_i(nt, lane);
  __syncthreads();
  if (lane == 63) sm_wcnt[w] = incl;
  __syncthreads();
  int woff = 0;
  for (int ww = 0; ww < w; ++ww) woff += sm_wcnt[ww];
  n = (sm_wcnt[0] + sm_wcnt[1]) + (sm_wcnt[2] + sm_wcnt[3]);
  int pos = woff + incl - nt;
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    if ((smask >> q) & 1u) {
      Cand e;
      e.key = key_of<DT>(x[q]);
      e.idx = int32_t(c0) + local_of<DT>(tid, q);
      s_list[pos++] = e;
    }
  }
  __syncthreads();

  // rank survivors exactly; the first F are this chunk's candidates
  Cand* out = a.cand + (rowid * a.S + c) * SSD_MAX_F;
  double sdrop = 0.0;
  for (int i = tid; i < n; i += kThreads) {
    const Cand e = s_list[i];
    const uint64_t rk = rank_key(e.key, e.idx);
    int rank = 0;
    for (int j = 0; j < n; ++j) rank += (rank_key(s_list[j].key, s_list[j].idx) > rk) ? 1 : 0;
    if (rank < F) dev_store(reinterpret_cast<uint64_t*>(out + rank), cand_bits(e));
    else sdrop += double(__builtin_amdgcn_exp2f((value_of_key<DT>(e.key) - piv) * c32));
  }
  for (int r = n + tid; r < F; r += kThreads) {
    Cand e;
    e.key = 0u;
    e.idx = -1;
    dev_store(reinterpret_cast<uint64_t*>(out + r), cand_bits(e));
  }
  const double s_rest = block_sum(double(sn), sm_d) + block_sum(sdrop, sm_d);
  if (tid == 0) {
    uint64_t* wp = reinterpret_cast<uint64_t*>(a.part + rowid * a.S + c);
    dev_store(wp, pack2(mc, 0.0f));
    dev_store(wp + 1, dbits(s_rest));
  }

  if (!arrive_last(&a.cnt[rowid * kCntStride], uint32_t(a.S), &sm_last)) return;

  // ---------------- merge: last workgroup of row (b, k) ----------------
  const double c64 = a.c64;
  const uint64_t* cl = reinterpret_cast<const uint64_t*>(a.cand + rowid * a.S * SSD_MAX_F);
  const int L = a.S * F;
  const bool staged = L <= kMergeCap;
  if (w == 0) {   // chunk maxima and non-candidate masses, one lane per chunk
    __shared__ float sm_pv;
    merge_rows<1>(reinterpret_cast<const uint64_t*>(a.part + rowid * a.S), 1, a.S, c32, &sm_pv,
                  &sm_srest, &sm_mrow);
  }
  if (staged) {
    for (int i = tid; i < L; i += kThreads) s_list[i] = bits_cand(dev_load(cl + (i / F) * SSD_MAX_F + (i % F)));
  }
  __syncthreads();
  auto cand_at = [&](int list, int i) -> Cand {
    return staged ? s_list[list * F + i] : bits_cand(dev_load(cl + list * SSD_MAX_F + i));
  };
  const float mrow = sm_mrow;
  const float prow = pivot_of(mrow);
  double s_unsel = 0.0;
  for (int e = tid; e < L; e += kThreads) {
    const int li = e / F, ii = e - li * F;
    const Cand me = cand_at(li, ii);
    if (me.idx < 0) continue;   // padding
    const uint64_t rk = rank_key(me.key, me.idx);
    int rank = ii;
    for (int ol = 0; ol < a.S; ++ol) {
      if (ol == li) continue;
      int lo = 0, hi = F;   // first position whose key is not above rk (lists descend)
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const Cand o = cand_at(ol, mid);
        const uint64_t ok = o.idx < 0 ? 0ull : rank_key(o.key, o.idx);
        if (ok > rk) lo = mid + 1;
        else hi = mid;
      }
      rank += lo;
    }
    const double ev = exp2(double(value_of_key<DT>(me.key) - prow) * double(c32));
    if (rank < F) {
      s_sel[rank] = me;
      s_sel_e[rank] = ev;
    } else {
      s_unsel += ev;
    }
  }
  const double unsel = block_sum(s_unsel, sm_d);
  int32_t* ct = a.cache_tokens + int64_t(b) * a.sumF + a.off[k];
  for (int r = tid; r < F; r += kThreads) ct[r] = s_sel[r].idx;
  if (tid == 0) {
    double s_top = 0.0;
    for (int r = 0; r < F; ++r) s_top += s_sel_e[r];
    ssd_rowkey tk;
    if (F > 0) {
      tk.key = s_sel[F - 1].key;
      tk.idx = s_sel[F - 1].idx;
    } else {
      tk.key = 0xFFFFFFFFu;
      tk.idx = -1;
    }
    a.thr[rowid] = tk;
    double* ds = a.dstats + rowid * 3;
    ds[0] = double(mrow);
    ds[1] = s_top;
    ds[2] = sm_srest + unsel;
  }
}

__global__ __launch_bounds__(kThreads) void k_lookup(LookupArgs a) {
  const int b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= a.B) return;
  const int av = a.accepted[b];
  uint8_t h = 0;
  int32_t s = -1;
  if (av >= 0 && av <= a.K) {
    const int32_t t = a.out_tokens[int64_t(b) * (a.K + 1) + av];
    const int32_t* seg = a.cache_tokens + int64_t(b) * a.sumF + a.off[av];
    if (t >= 0) {
      for (int j = 0; j < a.F[av]; ++j) {
        if (seg[j] == t) {
          h = 1;
          s = j;
          break;
        }
      }
    }
  }
  a.hit[b] = h;
  if (a.slot) a.slot[b] = s;
}

hipError_t launch_cache(const CacheArgs& a, int dtype, hipStream_t st) {
  const unsigned grid = unsigned(int64_t(a.B) * (a.K + 1) * a.S);
  if (dtype == SSD_BF16) hipLaunchKernelGGL(k_cache<1>, dim3(grid), dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL(k_cache<0>, dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_lookup(const LookupArgs& a, hipStream_t st) {
  const unsigned grid = unsigned((a.B + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(k_lookup, dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace ssd

// Device code of the speculation-cache build (shared by the build's own
// kernels and the fused verification round).
//
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
// Order: logit descending, then token index ascending, on order-preserving
// integer keys (exact, no tolerance).
//
// Thresholds. Any key t such that at least F lanes of a chunk hold an entry
// >= t (their lane maximum) bounds the chunk's F-th largest entry from
// below, and so the row's: an entry below it can never be in the top F. In a
// wave (2048 entries, 32 per lane) let Q_w be any value that at least
// ceil(F/4) lane maxima reach; min_w Q_w is such a bound (4 x ceil(F/4) >= F
// lanes) and is the chunk's T0. The tightest Q_w is the ceil(F/4)-th largest
// lane maximum; a full chunk settles for a few bisection steps towards it
// (about 21 candidates per chunk on the B=64 K=5 rows against 19 for the
// exact value, for far fewer serial steps), a partial chunk finds it
// exactly. (The F-th largest lane maximum of one wave, max over waves, is
// another bound; on the synthetic rows it kept 3 % fewer candidates, and its
// bitwise search cost more than that saved.)
//
// Two launches.
//  k_cache_chunk, one workgroup per (batch row b, length k, chunk c): 8192
//  logits in registers; chunk max and T0; entries >= T0 (about F of 8192 for
//  the synthetic logits) are written out unsorted as candidates, and the exp-mass of all
//  other entries is summed. If ties push the candidates past kCandCap the
//  chunk is only flagged.
//  k_cache_merge, one workgroup per row (b, k): re-reads flagged chunks and
//  keeps exactly their top F (bitwise searches for the F-th key and, among
//  entries tied at it, for the offset bound); loads every candidate and the
//  chunk records in one round trip; ranks the candidates at or above the
//  largest chunk T0 by (key, index) (when too many remain, after finding
//  the row's F-th largest key exactly with 8-bit radix histograms); the
//  first F are the cache tokens.
#pragma once

#include "ssd_device.hpp"

namespace ssd {

constexpr int kFiltCap = 256;   // filtered candidates ranked in LDS by the merge
constexpr uint64_t kOverflow = 0xFFFFFFFFull;   // chunk record: candidates not written

__device__ __forceinline__ uint64_t cand_bits(uint32_t key, int32_t idx) {
  return uint64_t(key) | (uint64_t(uint32_t(idx)) << 32);
}
__device__ __forceinline__ uint32_t cand_key(uint64_t w) { return uint32_t(w); }
__device__ __forceinline__ int32_t cand_idx(uint64_t w) { return int32_t(uint32_t(w >> 32)); }

// Offset of entry q of thread tid inside its chunk (strided layout).
template <int DT>
__device__ __forceinline__ int local_of(int tid, int q) {
  constexpr int PV = Dt<DT>::kPerVec;
  return ((q / PV) * kThreads + tid) * PV + (q % PV);
}

// Float threshold equivalent to "key >= k" for logits: keys at or below that
// of -inf accept every entry, keys above that of +inf accept none.
template <int DT>
__device__ __forceinline__ float threshold_value(uint32_t k) {
  if (k <= key_of<DT>(-__builtin_inff())) return -__builtin_inff();
  if (k > key_of<DT>(__builtin_inff())) return __builtin_nanf("");
  return value_of_key<DT>(k);
}

// exp((z - pivot)/tau) of a candidate, from its key
template <int DT>
__device__ __forceinline__ double cand_mass(uint64_t e, float prow, float c32) {
  return double(__builtin_amdgcn_exp2f((value_of_key<DT>(cand_key(e)) - prow) * c32));
}

// Entries j*PV .. j*PV+PV-1 of this thread (strided layout), NaN past the end.
template <int DT>
__device__ __forceinline__ void load_vec(const typename Dt<DT>::T* row, int64_t c0, int nvalid, int tid,
                                         int j, float (&v)[Dt<DT>::kPerVec]) {
  constexpr int PV = Dt<DT>::kPerVec;
  const typename Dt<DT>::T* base = row + c0;   // uniform; per-entry 32-bit offsets
  const int loc0 = (j * kThreads + tid) * PV;
#pragma unroll
  for (int e = 0; e < PV; ++e) {
    const int loc = loc0 + e;
    const float val = Dt<DT>::to_f(base[loc < nvalid ? loc : nvalid - 1]);
    v[e] = loc < nvalid ? val : __builtin_nanf("");
  }
}

// Exact top-F of one chunk when ties overflow the candidate slots: bitwise
// search for the F-th largest key (counting by float comparison), then the
// entries tied at it are taken in offset order (vector row j, thread, entry)
// until F are in. Returns the thread's selection bitmask (bit j*PV + e) and
// the key of the F-th entry. Every pass re-reads the chunk.
template <int DT>
__device__ __forceinline__ uint32_t exact_top_f(const typename Dt<DT>::T* row, int64_t c0, int nvalid, int F,
                                                int tid, int lane, int w, int* sm_i, int* sm_wcnt,
                                                uint32_t& key_out) {
  constexpr int PV = Dt<DT>::kPerVec;
  constexpr int NV = kPerThread / PV;
  uint32_t t = 0;
  for (int bit = Dt<DT>::kKeyBits - 1; bit >= 0; --bit) {
    const uint32_t cand = t | (1u << bit);
    const float fv = threshold_value<DT>(cand);
    int cnt = 0;
#pragma unroll 1
    for (int j = 0; j < NV; ++j) {
      float v[PV];
      load_vec<DT>(row, c0, nvalid, tid, j, v);
#pragma unroll
      for (int e = 0; e < PV; ++e) cnt += v[e] >= fv ? 1 : 0;
    }
    if (block_sum_i(cnt, sm_i) >= F) t = cand;
  }
  const float ft = threshold_value<DT>(t);
  uint32_t gmask = 0, tmask = 0;
#pragma unroll 1
  for (int j = 0; j < NV; ++j) {
    float v[PV];
    load_vec<DT>(row, c0, nvalid, tid, j, v);
#pragma unroll
    for (int e = 0; e < PV; ++e) {
      if (v[e] > ft) gmask |= 1u << (j * PV + e);
      if (v[e] == ft) tmask |= 1u << (j * PV + e);
    }
  }
  const int need = F - block_sum_i(__popc(gmask), sm_i);
  uint32_t keep = 0;
  int before = 0;   // ties in earlier vector rows
#pragma unroll 1
  for (int j = 0; j < NV; ++j) {
    const uint32_t bits = (tmask >> (j * PV)) & ((1u << PV) - 1u);
    const int cj = __popc(bits);
    const int inc = wave_incl_scan_i(cj, lane);
    if (lane == 63) sm_wcnt[w] = inc;
    __syncthreads();
    int wb = 0;
    for (int ww = 0; ww < w; ++ww) wb += sm_wcnt[ww];
    const int tot = (sm_wcnt[0] + sm_wcnt[1]) + (sm_wcnt[2] + sm_wcnt[3]);
    __syncthreads();
    const int first = before + wb + inc - cj;   // rank of this thread's first tie in row j
#pragma unroll
    for (int e = 0; e < PV; ++e)
      if (((bits >> e) & 1u) && first + __popc(bits & ((1u << e) - 1u)) < need) keep |= 1u << (j * PV + e);
    before += tot;
  }
  key_out = t;
  return gmask | keep;
}

constexpr int kHold = 16;        // candidate slots a merge thread holds in registers (own launch)
constexpr int kHoldLean = 4;     // the same where the merge shares a launch with streaming work
constexpr int kCountLds = 256;   // chunk candidate counts kept in LDS by the merge
constexpr int kHeldChunks = 32;  // rows of at most this many chunks use the chunk-major map

// The candidate slots of one row, as seen by one merge thread. Rows of at
// most kHeldChunks chunks use a chunk-major map: with G the chunk count
// rounded up to a power of two and P = 256 / G, thread tid serves chunk
// tid / P at positions tid % P + P * i, i < 128 / P, which covers every
// slot of the chunk. A thread's valid slots are a prefix of its i, a
// chunk's candidates spread over its P threads, and one wave load
// instruction reads 64 / P runs of P consecutive slots. The first HOLD
// positions (kHold, or kHoldLean where the merge shares a launch) are loaded
// in the round trip of the chunk records and kept in registers (they hold
// every candidate of a chunk with up to HOLD * P of them); later positions
// are read when a visit reaches them, in the same order, and only while
// some lane of the wave has one. Longer rows stream their slots on every
// visit (thread tid: slots tid, tid + 256, ...). Either way each thread
// meets its candidates in the same order for every HOLD, so both forms of
// the merge give bit-identical results.
template <int HOLD>
struct RowCands {
  uint64_t v[HOLD];
  uint32_t ok;          // bit i: slot i holds a written candidate
  const uint64_t* base; // this thread's chunk's slots
  int pos, step, nc;    // first position, position step, the chunk's candidate count
};

struct HeldMap {
  int chunk, pos, step;   // this thread's chunk, first position, position step
};
__device__ __forceinline__ HeldMap held_map(int S, int tid) {
  const int lg = S <= 1 ? 0 : min(8, 32 - __clz(S - 1));   // ceil(log2 S), at most 8
  const int P = kThreads >> lg;
  return HeldMap{tid / P, tid % P, P};
}

// f(e) for every written candidate of the row, each visited by one thread
// (a thread's candidates in the order of its positions).
template <bool COH, int HOLD, typename Fn>
__device__ __forceinline__ void visit(const RowCands<HOLD>& rc, bool held, const uint64_t* pp, const int* cnt_lds,
                                      const uint64_t* cl, int S, Fn f) {
  if (held) {
#pragma unroll
    for (int i = 0; i < HOLD; ++i)
      if ((rc.ok >> i) & 1u) f(rc.v[i]);
    for (int i0 = HOLD; rc.step * i0 < kCandCap; i0 += HOLD) {
      if (__builtin_amdgcn_ballot_w64(rc.pos + rc.step * i0 < rc.nc) == 0) break;   // wave-uniform
      uint64_t e[HOLD];
      bool ok[HOLD];
#pragma unroll
      for (int i = 0; i < HOLD; ++i) {
        const int p = rc.pos + rc.step * (i0 + i);
        ok[i] = p < rc.nc;
        e[i] = ok[i] ? ld64<COH>(rc.base + p) : 0ull;
      }
#pragma unroll
      for (int i = 0; i < HOLD; ++i)
        if (ok[i]) f(e[i]);
    }
    return;
  }
  const int slots = S * kCandCap;
  for (int base = 0; base < slots; base += kThreads * HOLD) {
    uint64_t e[HOLD];
    bool ok[HOLD];
#pragma unroll
    for (int i = 0; i < HOLD; ++i) {
      const int sidx = base + i * kThreads + int(threadIdx.x);
      ok[i] = false;
      if (sidx < slots) {
        const int cc = sidx / kCandCap;
        const int n = cc < kCountLds ? cnt_lds[cc] : int(uint32_t(ld64<COH>(pp + cc * 4 + 2)));
        ok[i] = (sidx - cc * kCandCap) < n;
      }
      e[i] = ok[i] ? ld64<COH>(cl + sidx) : 0ull;
    }
#pragma unroll
    for (int i = 0; i < HOLD; ++i)
      if (ok[i]) f(e[i]);
  }
}

// The same candidates as visit, a batch at a time: fb(e, okm) gets up to
// HOLD slots of the thread (bit i of okm: e[i] holds a written candidate),
// in the order visit meets them. Every thread of the workgroup calls it and
// fb is called by all lanes of a wave together.
template <bool COH, int HOLD, typename Fb>
__device__ __forceinline__ void visit_batches(const RowCands<HOLD>& rc, bool held, const uint64_t* pp,
                                              const int* cnt_lds, const uint64_t* cl, int S, Fb fb) {
  if (held) {
    fb(rc.v, rc.ok);
    for (int i0 = HOLD; rc.step * i0 < kCandCap; i0 += HOLD) {
      if (__builtin_amdgcn_ballot_w64(rc.pos + rc.step * i0 < rc.nc) == 0) break;   // wave-uniform
      uint64_t e[HOLD];
      uint32_t okm = 0;
#pragma unroll
      for (int i = 0; i < HOLD; ++i) {
        const int p = rc.pos + rc.step * (i0 + i);
        const bool ok = p < rc.nc;
        e[i] = ok ? ld64<COH>(rc.base + p) : 0ull;
        okm |= ok ? 1u << i : 0u;
      }
      fb(e, okm);
    }
    return;
  }
  const int slots = S * kCandCap;
  for (int base = 0; base < slots; base += kThreads * HOLD) {
    uint64_t e[HOLD];
    uint32_t okm = 0;
#pragma unroll
    for (int i = 0; i < HOLD; ++i) {
      const int sidx = base + i * kThreads + int(threadIdx.x);
      bool ok = false;
      if (sidx < slots) {
        const int cc = sidx / kCandCap;
        const int n = cc < kCountLds ? cnt_lds[cc] : int(uint32_t(ld64<COH>(pp + cc * 4 + 2)));
        ok = (sidx - cc * kCandCap) < n;
      }
      e[i] = ok ? ld64<COH>(cl + sidx) : 0ull;
      okm |= ok ? 1u << i : 0u;
    }
    fb(e, okm);
  }
}

// Appends the entries e[i] with bit i of km set to the LDS list: one prefix
// count over the wave and one LDS atomic per wave and batch (entries past
// kFiltCap are counted but not stored). Called by all lanes of a wave
// together; the list order is the wave's lane order, then i.
template <int HOLD>
__device__ __forceinline__ void batch_append(const uint64_t (&e)[HOLD], uint32_t km, int lane, int* n,
                                             uint64_t* list) {
  const int cnt = __popc(km);
  const int incl = wave_incl_scan_i(cnt, lane);
  const int tot = __builtin_amdgcn_readlane(incl, 63);
  if (tot == 0) return;   // wave-uniform
  int base = 0;
  if (lane == 0) base = atomicAdd(n, tot);
  int slot = __builtin_amdgcn_readlane(base, 0) + incl - cnt;
#pragma unroll
  for (int i = 0; i < HOLD; ++i) {
    if ((km >> i) & 1u) {
      if (slot < kFiltCap) list[slot] = e[i];
      ++slot;
    }
  }
}

// Every thread's first HOLD slots, loaded unconditionally (slots past a
// chunk's count are masked out later; the chunk and position are clamped
// into the row's slots, so there is no branch around the loads).
template <bool COH, int HOLD>
__device__ __forceinline__ void load_held(RowCands<HOLD>& rc, const uint64_t* cl, const HeldMap& hm, int S) {
  rc.base = cl + min(hm.chunk, S - 1) * kCandCap;
  rc.pos = hm.pos;
  rc.step = hm.step;
#pragma unroll
  for (int i = 0; i < HOLD; ++i) rc.v[i] = ld64<COH>(rc.base + min(hm.pos + hm.step * i, kCandCap - 1));
}

// Appends e to the LDS list when keep holds: one LDS atomic per wave (the
// lowest selected lane reserves the wave's slots), entries past kFiltCap
// are counted but not stored. Called by the active lanes of a wave together.
__device__ __forceinline__ void wave_append(uint64_t e, bool keep, int lane, int* n, uint64_t* list) {
  const uint64_t m = __builtin_amdgcn_ballot_w64(keep);
  if (m == 0) return;   // uniform over the active lanes
  const int leader = __builtin_ctzll(m);
  int base = 0;
  if (lane == leader) base = atomicAdd(n, __popcll(m));
  base = __builtin_amdgcn_readlane(base, leader);
  if (keep) {
    const int slot = base + int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
    if (slot < kFiltCap) list[slot] = e;
  }
}

// The merge of row rowid = b * (K+1) + k.
//
// Every chunk's T0 bounds the row's F-th largest key from below (the chunk
// holds at least F entries at or above it), and so does the F-th largest of
// the chunk maxima when F <= S (they are F distinct entries of the row).
// The larger of the largest T0 and that maximum, Tmax, is the bound used:
// the row's top F are among the candidates at or above Tmax, and every
// candidate below it only adds to S_rest. Those at or above Tmax (from F to
// a few times F on the synthetic rows) are ranked directly by (key,
// index). Only when more than kFiltCap of them remain is the row's F-th
// largest key found exactly first (8-bit radix passes over LDS histograms),
// and then the candidates tied at it by a bitwise search over the index.
// thr and draft_stats are stored by thread 0 with device-scope stores, so a
// workgroup of the same launch that arrives after this one (arrive_last) may
// read them. COH: the chunk records and candidates were written by other
// workgroups of the same launch, so they are read (and rewritten) with
// device-scope accesses, and so are the cache tokens written.
template <int DT, bool COH = false, int HOLD = kHold>
__device__ __forceinline__ void cache_merge_wg(const CacheArgs& a, int64_t rowid) {
  using T = typename Dt<DT>::T;
  const int KP = a.K + 1;
  const int b = int(fdiv(uint32_t(rowid), a.div_kp));   // rowid < 2^31 (the grid)
  const int k = int(rowid) - b * KP;
  const int F = a.F[k];
  __shared__ uint64_t s_list[kFiltCap];
  __shared__ double s_exp[kFiltCap];
  __shared__ int s_hist[256];
  __shared__ int s_cnt[kCountLds];
  __shared__ int s_n2;
  __shared__ float s_mrow;
  __shared__ double s_srest;
  __shared__ uint32_t s_prefix, s_tmax;
  __shared__ int s_need;
  __shared__ double sm_d2[4];
  __shared__ int sm_i2[4];
  __shared__ int sm_wcnt2[4];
  __shared__ int s_anyovf;
  __shared__ uint64_t s_thrw;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float c32 = a.c32;
  uint64_t* pw = reinterpret_cast<uint64_t*>(a.part + rowid * a.S);
  const uint64_t* pp = pw;
  uint64_t* clw = reinterpret_cast<uint64_t*>(a.cand + rowid * a.S * kCandCap);
  const uint64_t* cl = clw;
  const bool held = a.S <= kHeldChunks;
  const HeldMap hm = held_map(a.S, tid);

  // The chunk records (wave 0, one lane per chunk) are requested first and
  // every thread's candidate slots right after, so both arrive in one round
  // trip and wave 0 folds the records while the candidates are in flight.
  // Both are issued without branches (indices clamped into the row) so that
  // the fold waits only for the records.
  // Lane l < S of wave 0 holds chunk l's record; every thread also reads
  // the candidate count of the chunk it holds.
  const bool rec = w == 0 && lane < a.S;
  const int rl = min(lane, a.S - 1);
  const uint64_t r0 = ld64<COH>(pp + rl * 4), r1 = ld64<COH>(pp + rl * 4 + 1), r2 = ld64<COH>(pp + rl * 4 + 2);
  const uint64_t own_cnt = ld64<COH>(pp + min(hm.chunk, a.S - 1) * 4 + 2);
  __builtin_amdgcn_sched_barrier(0);
  RowCands<HOLD> rc;
  rc.ok = 0;
  load_held<COH, HOLD>(rc, cl, hm, a.S);
  __builtin_amdgcn_sched_barrier(0);

  // row max, the chunks' non-candidate mass (lane-local fold in chunk order,
  // then butterflies), Tmax; candidate counts to LDS
  if (w == 0) {
    float ml = -__builtin_inff();
    double sl = 0.0;
    int ovf = 0;
    uint32_t tmax = 0;
    auto fold = [&](int cc, uint64_t w0, uint64_t w1, uint64_t w2) {
      const double sc = bits_d(w1);
      const int nc = w2 == kOverflow ? 0 : int(uint32_t(w2));
      ovf |= w2 == kOverflow ? 1 : 0;
      if (cc < kCountLds) s_cnt[cc] = nc;
      tmax = max(tmax, uint32_t(w0 >> 32));
      const float qm = lo_f(w0);
      const float nm = fmaxf(ml, qm);
      const float pn = pivot_of(nm);
      double acc = 0.0;
      if (sl > 0.0) acc += sl * rescale(pivot_of(ml), pn, c32);
      if (sc > 0.0) acc += sc * rescale(pivot_of(qm), pn, c32);
      ml = nm;
      sl = acc;
    };
    if (rec) fold(lane, r0, r1, r2);
    for (int cc = lane + 64; cc < a.S; cc += 64)
      fold(cc, ld64<COH>(pp + cc * 4), ld64<COH>(pp + cc * 4 + 1), ld64<COH>(pp + cc * 4 + 2));
    const float m = wave_max(ml);
    const double t = sl > 0.0 ? sl * rescale(pivot_of(ml), pivot_of(m), c32) : 0.0;
    const double srest = wave_sum(t);
    tmax = wave_max_u32(tmax);
    // the F-th largest chunk maximum (the F largest are F distinct entries
    // of the row), by a bitwise search over the lanes' chunk-max keys
    if (F > 0 && F <= a.S && a.S <= 64) {
      const uint32_t km = rec ? key_of<DT>(lo_f(r0)) : 0u;
      uint32_t mf = 0;
      for (int bit = Dt<DT>::kKeyBits - 1; bit >= 0; --bit) {
        const uint32_t cand = mf | (1u << bit);
        if (__popcll(__ballot(km >= cand)) >= F) mf = cand;
      }
      tmax = max(tmax, mf);
    }
    const bool anyovf = __ballot(ovf != 0) != 0;
    if (lane == 0) {
      s_mrow = m;
      s_srest = srest;
      s_n2 = 0;
      s_prefix = 0;
      s_need = F;
      s_tmax = tmax;
      s_anyovf = anyovf ? 1 : 0;
      s_thrw = cand_bits(0xFFFFFFFFu, -1);
    }
  }
  __syncthreads();
  const float mrow = s_mrow;
  const float prow = pivot_of(mrow);
  double s_unsel = 0.0;

  // chunks whose candidates overflowed (ties): re-read them and keep exactly
  // their top F; the other entries >= T0 of such a chunk add to S_rest
  if (__builtin_expect(s_anyovf != 0, 0)) {   // rare: ties overflowed a chunk's slots
    const T* row = static_cast<const T*>(a.draft) + int64_t(b) * a.db + int64_t(k) * a.V;
    for (int cc = 0; cc < a.S; ++cc) {
      if (ld64<COH>(pp + cc * 4 + 2) != kOverflow) continue;   // uniform
      const int64_t c0 = int64_t(cc) * kChunk;
      const int nvalid = int(min(int64_t(kChunk), int64_t(a.V) - c0));
      uint32_t key_unused;
      const uint32_t sel = exact_top_f<DT>(row, c0, nvalid, F, tid, lane, w, sm_i2, sm_wcnt2, key_unused);
      const float f0 = threshold_value<DT>(uint32_t(ld64<COH>(pp + cc * 4) >> 32));
      const int nt = __popc(sel);
      const int incl = wave_incl_scan_i(nt, lane);
      if (lane == 63) sm_wcnt2[w] = incl;
      __syncthreads();
      int pos = incl - nt;
      for (int ww = 0; ww < w; ++ww) pos += sm_wcnt2[ww];
      const int nsel = (sm_wcnt2[0] + sm_wcnt2[1]) + (sm_wcnt2[2] + sm_wcnt2[3]);
      __syncthreads();
      // the chunk again, a vector at a time (entry order as in the pass):
      // selected entries to the slots, the rest at or above T0 to S_rest
      constexpr int PV = Dt<DT>::kPerVec;
#pragma unroll 1
      for (int j = 0; j < kPerThread / PV; ++j) {
        float v[PV];
        load_vec<DT>(row, c0, nvalid, tid, j, v);
#pragma unroll
        for (int e = 0; e < PV; ++e) {
          const int q = j * PV + e;
          const int loc = local_of<DT>(tid, q);
          if ((sel >> q) & 1u) {
            st64<COH>(clw + int64_t(cc) * kCandCap + pos, cand_bits(key_of<DT>(v[e]), int32_t(c0) + loc));
            ++pos;
          } else if (loc < nvalid && v[e] >= f0) {
            s_unsel += double(__builtin_amdgcn_exp2f((v[e] - prow) * c32));
          }
        }
      }
      if (tid == 0) {
        st64<COH>(pw + cc * 4 + 2, uint64_t(uint32_t(nsel)));
        if (cc < kCountLds) s_cnt[cc] = nsel;
      }
      __syncthreads();
    }
    __threadfence();
    __syncthreads();
    load_held<COH, HOLD>(rc, cl, hm, a.S);   // the rewritten lists
  }

  if (held) {
    // this thread's chunk count: from its own record, or from LDS where an
    // overflowed chunk was rewritten
    int nc = hm.chunk < a.S ? (own_cnt == kOverflow ? 0 : int(uint32_t(own_cnt))) : 0;
    if (s_anyovf && hm.chunk < a.S) nc = s_cnt[hm.chunk];
    rc.nc = nc;
#pragma unroll
    for (int i = 0; i < HOLD; ++i)
      if (hm.pos + hm.step * i < nc) rc.ok |= 1u << i;
  }
  int32_t* ct = a.cache_tokens + int64_t(b) * a.sumF + a.off[k];

  // candidates at or above Tmax go to the ranked list; the others only add
  // to S_rest
  const uint32_t tcut = s_tmax;
  visit_batches<COH, HOLD>(rc, held, pp, s_cnt, cl, a.S, [&](const uint64_t (&e)[HOLD], uint32_t okm) {
    uint32_t km = 0;
#pragma unroll
    for (int i = 0; i < HOLD; ++i) {
      if ((okm >> i) & 1u) {
        if (F > 0 && cand_key(e[i]) >= tcut) km |= 1u << i;
        else s_unsel += cand_mass<DT>(e[i], prow, c32);
      }
    }
    batch_append(e, km, lane, &s_n2, s_list);
  });
  __syncthreads();
  int n2 = __builtin_amdgcn_readfirstlane(s_n2);   // uniform
  __syncthreads();

  if (__builtin_expect(n2 > kFiltCap, 0)) {
    // too many at or above Tmax: the row's F-th largest key, exactly, 8 bits
    // at a time from the top (it is >= Tmax, so only those are re-sorted)
    constexpr int KB = Dt<DT>::kKeyBits;
    for (int shift = KB - 8; shift >= 0; shift -= 8) {
      s_hist[tid] = 0;
      __syncthreads();
      const uint32_t prefix = s_prefix;
      visit<COH, HOLD>(rc, held, pp, s_cnt, cl, a.S, [&](uint64_t e) {
        const uint32_t key = cand_key(e);
        const uint32_t hi = (shift + 8 < 32) ? (key >> (shift + 8)) : 0u;
        if (hi == prefix) atomicAdd(&s_hist[(key >> shift) & 255u], 1);
      });
      __syncthreads();
      if (w == 0) {   // bin holding the need-th largest: suffix counts over 4 bins per lane
        const int need = s_need;
        const int h0 = s_hist[4 * lane], h1 = s_hist[4 * lane + 1], h2 = s_hist[4 * lane + 2],
                  h3 = s_hist[4 * lane + 3];
        const int lane_tot = h0 + h1 + h2 + h3;
        int v = lane_tot;   // inclusive suffix scan over lanes 63..0
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int t2 = __shfl_down(v, o);
          if (lane + o < 64) v += t2;
        }
        const int above = v - lane_tot;   // counts in bins of higher lanes
        int binsel = -1, rem_need = 0;
        int acc = above;
        const int hh[4] = {h3, h2, h1, h0};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (binsel < 0 && acc + hh[i] >= need && acc < need) {
            binsel = 4 * lane + 3 - i;
            rem_need = need - acc;
          }
          acc += hh[i];
        }
        const uint64_t hitm = __ballot(binsel >= 0);
        if (hitm) {
          const int l = __ffsll((unsigned long long)hitm) - 1;
          if (lane == l) {
            s_prefix = (prefix << 8) | uint32_t(binsel);
            s_need = rem_need;
          }
        } else if (lane == 0) {   // fewer than F candidates: keep them all
          s_prefix = 0;
          s_need = 0;
        }
      }
      __syncthreads();
      if (s_need == 0) break;
    }
    const uint32_t cut = s_need == 0 && s_prefix == 0 ? tcut : s_prefix;   // the F-th key
    if (tid == 0) s_n2 = 0;
    __syncthreads();
    visit<COH, HOLD>(rc, held, pp, s_cnt, cl, a.S, [&](uint64_t e) {
      if (cand_key(e) < tcut) return;   // already counted
      const bool keep = cand_key(e) >= cut;
      wave_append(e, keep, lane, &s_n2, s_list);
      if (!keep) s_unsel += cand_mass<DT>(e, prow, c32);
    });
    __syncthreads();
    n2 = s_n2;
    __syncthreads();

    if (n2 > kFiltCap) {
      // more ties at the F-th key than the list holds: the needed ties are
      // the ones with the smallest indices (bitwise search for the index bound)
      int c = 0;
      visit<COH, HOLD>(rc, held, pp, s_cnt, cl, a.S, [&](uint64_t e) { c += cand_key(e) > cut ? 1 : 0; });
      const int need = F - block_sum_i(c, sm_i2);
      int lim = 0;   // largest bound with fewer than `need` ties below it
      for (int bit = 30; bit >= 0; --bit) {
        const int cand = lim | (1 << bit);
        int cnt = 0;
        visit<COH, HOLD>(rc, held, pp, s_cnt, cl, a.S, [&](uint64_t e) {
          cnt += (cand_key(e) == cut && cand_idx(e) < cand) ? 1 : 0;
        });
        if (block_sum_i(cnt, sm_i2) < need) lim = cand;
      }
      // ties with index <= lim are exactly `need` of them
      if (tid == 0) s_n2 = 0;
      __syncthreads();
      visit<COH, HOLD>(rc, held, pp, s_cnt, cl, a.S, [&](uint64_t e) {
        if (cand_key(e) < cut) return;   // already counted
        const bool keep = cand_key(e) > cut || cand_idx(e) <= lim;
        wave_append(e, keep, lane, &s_n2, s_list);
        if (!keep) s_unsel += cand_mass<DT>(e, prow, c32);
      });
      __syncthreads();
      n2 = min(s_n2, kFiltCap);   // == F
      __syncthreads();
    }
  }

  // exact ranks among the kept candidates; ranks are unique, so nothing
  // below depends on the order in which the list was filled
  auto place = [&](uint64_t e, int rank) {
    s_exp[rank] = cand_mass<DT>(e, prow, c32);
    if (rank < F) st32<COH>(ct + rank, cand_idx(e));
    if (rank == F - 1) s_thrw = e;
  };
  if (__builtin_expect(n2 <= 64, 1)) {
    // entry i in lane i of every wave; wave w counts the larger keys among
    // entries w, w + 4, ... (broadcast LDS reads), wave 0 adds the four
    // counts (in s_hist, unused on this path) and places the entries
    const uint64_t e = lane < n2 ? s_list[lane] : 0ull;
    const uint64_t rk = rank_key(cand_key(e), cand_idx(e));
    int part = 0;
    for (int j = w; j < n2; j += 4) {
      const uint64_t o = s_list[j];
      part += rank_key(cand_key(o), cand_idx(o)) > rk ? 1 : 0;
    }
    s_hist[tid] = part;
    __syncthreads();
    if (w == 0) {
      const int rank = (s_hist[lane] + s_hist[64 + lane]) + (s_hist[128 + lane] + s_hist[192 + lane]);
      if (lane < n2) place(e, rank);
    }
  } else {
    for (int i = tid; i < n2; i += kThreads) {
      const uint64_t e = s_list[i];
      const uint64_t rk = rank_key(cand_key(e), cand_idx(e));
      int rank = 0;
      for (int j = 0; j < n2; ++j) {
        const uint64_t o = s_list[j];
        rank += rank_key(cand_key(o), cand_idx(o)) > rk ? 1 : 0;
      }
      place(e, rank);
    }
  }
  const double unsel = block_sum(s_unsel, sm_d2);   // its barriers also publish s_exp
  if (w == 0) {
    // S_top over ranks < F, the ranked rest into S_rest (lane-strided, then
    // butterflies)
    double top = 0.0, more = 0.0;
    for (int r = lane; r < n2; r += 64) {
      if (r < F) top += s_exp[r];
      else more += s_exp[r];
    }
    top = wave_sum_u(top);
    more = wave_sum_u(more);
    if (lane == 0) {
      // the F-th member (key | index << 32, the ssd_rowkey layout), or the
      // empty marker when F = 0
      const uint64_t tw = F == 0 ? cand_bits(0xFFFFFFFFu, -1) : s_thrw;
      dev_store(reinterpret_cast<uint64_t*>(a.thr + rowid), tw);
      uint64_t* ds = reinterpret_cast<uint64_t*>(a.dstats + rowid * 3);
      dev_store(ds, dbits(double(mrow)));
      dev_store(ds + 1, dbits(top));
      dev_store(ds + 2, dbits(s_srest + unsel + more));
    }
  }
}


// Scaled exp-mass (scaled_mass) of the entries below f0 (the
// non-candidates); the caller applies the chunk's fix. Entries past the row
// end read as -inf and add nothing; with f0 = NaN (no candidates) every
// entry counts. Bit j of cvec is set when vector j holds a candidate in some
// lane of the wave (wave_compact's ballots): the other vectors skip the
// per-entry test, since it passes every entry there (a padding entry it
// would drop adds exp2(-inf) = 0 either way), and the sum is the same.
template <int DT>
__device__ __forceinline__ float chunk_rest_mass(const float (&x)[kPerThread], float f0, float P, float c32,
                                                 uint32_t cvec) {
  constexpr int PV = Dt<DT>::kPerVec;
  float sn = 0.0f;
#pragma unroll
  for (int j = 0; j < kPerThread / PV; ++j) {
    if (cvec & (1u << j)) {   // wave-uniform
#pragma unroll
      for (int e = 0; e < PV; ++e) {
        const float m = scaled_mass(x[j * PV + e], c32, P);
        sn += (x[j * PV + e] >= f0) ? 0.0f : m;
      }
    } else {
#pragma unroll
      for (int e = 0; e < PV; ++e) sn += scaled_mass(x[j * PV + e], c32, P);
    }
    // a vector at a time: keeps the exp temporaries short-lived
    __builtin_amdgcn_sched_barrier(0);
  }
  return sn;
}

// Compacts one wave's candidates (entries >= f0; with CHECK also inside the
// row) into its LDS staging lists, in (entry, lane) order: the value's raw
// bits in wv and the token index in wi (the copy-out forms the keyed
// records, so the rare taken branch stays short). Entries past kCandCap are
// counted and written to the spare slot kCandCap, which is never read.
// Returns the wave's count; bit j of cvec marks vector j (entries j PV ..
// j PV + PV - 1 of every lane) as holding a candidate in some lane.
template <int DT, bool CHECK>
__device__ __forceinline__ uint32_t wave_compact(const float (&x)[kPerThread], float f0, int tid, int nvalid, int c0,
                                                 uint32_t* wv, int32_t* wi, uint32_t& cvec) {
  constexpr int PV = Dt<DT>::kPerVec;
  uint32_t cw = 0;
  cvec = 0;
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int loc = local_of<DT>(tid, q);
    const bool cand = CHECK ? ((x[q] >= f0) & (loc < nvalid)) : (x[q] >= f0);
    const uint64_t m = __builtin_amdgcn_ballot_w64(cand);
    if (m != 0) {   // wave-uniform
      if (cand) {
        const uint32_t p = min(cw + __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)),
                               uint32_t(kCandCap));
        wv[p] = __float_as_uint(x[q]);
        wi[p] = c0 + loc;
      }
      cw += uint32_t(__popcll(m));
      cvec |= 1u << (q / PV);
    }
  }
  return cw;
}

constexpr int kBisectSteps = 5;   // value bisection steps of a full chunk's per-wave bound

// Largest key of the dtype whose value is <= v (v not NaN). For bfloat16
// the float key's top half is that key when the low half is 0xFFFF (a
// negative value that is exactly a bfloat16) or the value is positive;
// otherwise a negative v lies strictly between two bfloat16 values and the
// next smaller one is one key below.
template <int DT> __device__ __forceinline__ uint32_t floor_key(float v);
template <> __device__ __forceinline__ uint32_t floor_key<0>(float v) { return key_of<0>(v); }
template <> __device__ __forceinline__ uint32_t floor_key<1>(float v) {
  const uint32_t k32 = key_of<0>(v);
  uint32_t k = k32 >> 16;
  if (k32 < 0x80000000u && (k32 & 0xFFFFu) != 0xFFFFu) k -= 1u;
  return k;
}

// The chunk pass of one workgroup over chunk c of draft row k of batch row
// b. COH: the record and candidates are read by a merge in the same launch,
// so they are stored with device-scope stores.
template <int DT, bool COH = false>
__device__ __forceinline__ void cache_chunk_at(const CacheArgs& a, int b, int k, int c) {
  using T = typename Dt<DT>::T;
  constexpr int PV = Dt<DT>::kPerVec;
  constexpr int NV = kPerThread / PV;
  __shared__ float sm_wmax[4];
  __shared__ uint32_t sm_wthq[4];
  __shared__ int sm_wcnt[4];
  __shared__ double sm_ws[4];
  __shared__ uint32_t sm_lv[4][kCandCap + 1];   // per-wave candidate staging: value bits,
  __shared__ int32_t sm_li[4][kCandCap + 1];    // token index (+1: spill slot)

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int KP = a.K + 1;
  const int F = a.F[k];
  const int64_t rowid = int64_t(b) * KP + k;
  const T* row = static_cast<const T*>(a.draft) + int64_t(b) * a.db + int64_t(k) * a.V;

  const int64_t c0 = int64_t(c) * kChunk;
  const int nvalid = int(min(int64_t(kChunk), int64_t(a.V) - c0));
  float x[kPerThread];
  float vm[NV];   // per-vector maxima (padding is -inf)
  {
    ChunkVecs<DT, true> cv;
    cv.load(row, c0, a.V, (reinterpret_cast<uintptr_t>(row) & 15u) == 0, tid);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      float v[PV];
      cv.get(j, v);
      float m = v[0];
#pragma unroll
      for (int e = 0; e < PV; ++e) {
        x[j * PV + e] = v[e];
        m = fmaxf(m, v[e]);
      }
      vm[j] = m;
    }
  }
  float lm = vm[0];
#pragma unroll
  for (int j = 1; j < NV; ++j) lm = fmaxf(lm, vm[j]);
  const float c32 = a.c32;

  // ---- per-wave max and threshold; chunk max and T0 ----
  // A key t with at least F lanes whose maximum is >= t bounds the chunk's
  // top F from below. Each wave finds a key that ceil(F/4) of its lane
  // maxima reach; the smallest over the four waves is such a bound (4 x
  // ceil(F/4) >= F lanes). It is the chunk's T0.
  // In the exact search every lane's key lies between the wave's smallest
  // key and the key of its maximum, so all keys share those two keys'
  // common leading bits, and the full search would set exactly those: it
  // starts from that prefix and tests only the bits below it (same result,
  // typically half the steps; lanes past the row end have key 0, which
  // leaves no common prefix).
  {
    const float wm = wave_max_u(lm);
    uint32_t tq = 0;
    if (F > 0 && nvalid == kChunk) {
      // Full chunk: five bisection steps on values between the wave's
      // smallest finite and largest lane maximum. lo starts at a value at
      // least Fq lanes reach (the smallest finite lane maximum, or -inf when
      // fewer than Fq lanes have a finite entry) and only ever takes a
      // midpoint that at least Fq lanes reach, so it stays a valid bound;
      // its key is rounded down to a logit of the row's dtype. A handful
      // of steps keeps the candidates within a few of the exact bound's.
      const int Fq = (F + 3) >> 2;
      float lo = -wave_max_u(lm > -__builtin_inff() ? -lm : -__builtin_inff()), hi = wm;
      if (__popcll(__ballot(lm >= lo)) < Fq) lo = -__builtin_inff();
#pragma unroll
      for (int it = 0; it < kBisectSteps; ++it) {
        const float mid = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(0.5f * (lo + hi))));
        const bool ok = __popcll(__ballot(lm >= mid)) >= Fq;
        lo = ok ? mid : lo;
        hi = ok ? hi : mid;
      }
      tq = floor_key<DT>(lo);
    } else if (F > 0) {
      // Partial chunk (lanes past the row end hold no entry): the exact
      // ceil(F/4)-th largest lane maximum, by a bitwise search.
      const int Fq = (F + 3) >> 2;
      const uint32_t kl = local_of<DT>(tid, 0) < nvalid ? key_of<DT>(lm) : 0u;
      const uint32_t diff = wave_min_u32(kl) ^ key_of<DT>(wm);
      const int h = diff == 0 ? 0 : 32 - __clz(diff);   // bits below h may differ
      tq = h >= 32 ? 0u : (key_of<DT>(wm) >> h) << h;
      for (int bit = h - 1; bit >= 0; --bit) {
        const uint32_t cand = tq | (1u << bit);
        if (__popcll(__ballot(kl >= cand)) >= Fq) tq = cand;
      }
    }
    if (lane == 0) {
      sm_wmax[w] = wm;
      sm_wthq[w] = tq;
    }
  }
  __syncthreads();
  // lane i < 4 reads wave i's values; the combination happens on scalars
  // (one register each instead of a copy of all eight per thread)
  float mc;
  uint32_t t0;
  {
    const int li = lane & 3;
    const float vm = sm_wmax[li];
    const uint32_t vq = sm_wthq[li];
    auto rlf = [](float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); };
    auto rlu = [](uint32_t v, int l) { return uint32_t(__builtin_amdgcn_readlane(int(v), l)); };
    mc = fmaxf(fmaxf(rlf(vm, 0), rlf(vm, 1)), fmaxf(rlf(vm, 2), rlf(vm, 3)));
    t0 = min(min(rlu(vq, 0), rlu(vq, 1)), min(rlu(vq, 2), rlu(vq, 3)));
  }
  const ScaledPivot sp = scaled_pivot(pivot_of(mc), c32);
  float f0 = __builtin_nanf("");   // F == 0: compares false, nothing is a candidate
  if (F > 0) f0 = (t0 <= key_of<DT>(-__builtin_inff())) ? -__builtin_inff() : value_of_key<DT>(t0);

  // ---- candidates (per-wave compaction) and exp-mass of the rest ----
  uint32_t cw, cvec;
  if (nvalid < kChunk && f0 == -__builtin_inff())   // padding would pass the test
    cw = wave_compact<DT, true>(x, f0, tid, nvalid, int(c0), sm_lv[w], sm_li[w], cvec);
  else
    cw = wave_compact<DT, false>(x, f0, tid, nvalid, int(c0), sm_lv[w], sm_li[w], cvec);
  const float sn = chunk_rest_mass<DT>(x, f0, sp.P, c32, cvec);
  const double ws = wave_sum_u(double(sn));   // double across threads
  if (lane == 0) {
    sm_wcnt[w] = int(cw);
    sm_ws[w] = ws;
  }
  __syncthreads();
  int woff = 0;
  for (int ww = 0; ww < w; ++ww) woff += sm_wcnt[ww];
  const int n = (sm_wcnt[0] + sm_wcnt[1]) + (sm_wcnt[2] + sm_wcnt[3]);
  const bool overflow = n > kCandCap;   // ties: the merge re-reads this chunk

  // ---- candidates out: each wave copies its list, in order ----
  if (!overflow) {
    uint64_t* out = reinterpret_cast<uint64_t*>(a.cand + (rowid * a.S + c) * kCandCap) + woff;
    for (int i = lane; i < int(cw); i += 64)
      st64<COH>(out + i, cand_bits(key_of<DT>(__uint_as_float(sm_lv[w][i])), sm_li[w][i]));
  }
  if (tid == 0) {
    const double s_rest = ((sm_ws[0] + sm_ws[1]) + (sm_ws[2] + sm_ws[3])) * double(sp.fix);
    uint64_t* wp = reinterpret_cast<uint64_t*>(a.part + rowid * a.S + c);
    st64<COH>(wp, uint64_t(__float_as_uint(mc)) | (uint64_t(t0) << 32));
    st64<COH>(wp + 1, dbits(s_rest));
    st64<COH>(wp + 2, overflow ? kOverflow : uint64_t(uint32_t(n)));
  }
}

// The same for workgroup blk = (b * (K+1) + k) * S + c of a one-chunk-per-
// workgroup grid.
template <int DT, bool COH = false>
__device__ __forceinline__ void cache_chunk_wg(const CacheArgs& a, uint32_t blk) {
  const uint32_t b = fdiv(blk, a.div_pb);
  const uint32_t rem = blk - b * uint32_t((a.K + 1) * a.S);
  const uint32_t k = fdiv(rem, a.div_s);
  cache_chunk_at<DT, COH>(a, int(b), int(k), int(rem - k * uint32_t(a.S)));
}

}  // namespace ssd

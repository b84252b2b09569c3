// Drafting from the sigma-reshaped draft distribution.
//
// SAGUARO reshapes the draft distribution before sampling: the top-F tokens
// of draft row k (the tokens the cache prepares for) keep weight C, all
// others weight 1, and the drafted token d_{k+1} is drawn from the
// renormalised result (papernotes.org "Speculative Speculative Decoding",
// key design 2). The verifier then uses the same q_sigma, which keeps the
// output distribution exact (brentwoodlivery.com "Speculative decoding",
// Derivation of Acceptance Criterion). Without sigma the draw is from the
// plain softmax of draft row k at temperature tau.
//
// The draw is by inverse CDF in token-index order: the smallest v whose
// running mass exceeds u * Z. Two launches: k_sample_chunks, one workgroup
// per (batch row b, position i, 16384-entry span), sums the weighted mass of
// each of the span's four 4096-entry chunks against that chunk's own max;
// k_sample_pick, one workgroup per (b, i), rescales the chunk masses to the
// row max, finds the crossing chunk and picks the token inside it (16
// entries per thread). A row without mass (all logits -inf) draws -1. The
// second launch replaces an arrival count in the first (the last workgroup
// of a row drawing): that count and the draw's latency kept workgroup slots
// of the streaming pass busy.
#include "ssd_cdf.hpp"

namespace ssd {

struct SigmaTest {
  float val;   // threshold as a logit value (NaN: no member)
  int32_t idx;
  float C;
  // sigma weight of token idx with logit x: C for members (key above the
  // threshold, or equal with index at most idx), else 1; bitwise tests keep
  // it branch-free
  __device__ float weight(float x, int i) const {
    const bool mem = (x > val) | ((x == val) & (i <= idx));
    return mem ? C : 1.0f;
  }
};

template <int DT, bool SIG>
__device__ __forceinline__ SigmaTest sigma_test(const SampleArgs& a, int b, int i) {
  SigmaTest t{__builtin_nanf(""), -1, 1.0f};
  if (SIG) {
    const ssd_rowkey tk = a.thr[int64_t(b) * (a.K + 1) + i];
    t.val = tk.key > key_of<DT>(__builtin_inff()) ? __builtin_nanf("") : value_of_key<DT>(tk.key);
    t.idx = tk.idx;
    t.C = a.C;
  }
  return t;
}

template <int DT, bool SIG>
__global__ __launch_bounds__(kThreads) void k_sample_chunks(SampleArgs a) {
  using T = typename Dt<DT>::T;
  using CV = ChunkVecs<DT, true, kStatsPerThread>;
  constexpr int PV = Dt<DT>::kPerVec;
  constexpr int NQ = kStatsPerThread / kPickPerThread;   // pick chunks per span
  constexpr int NVQ = CV::NV / NQ;                      // vectors per pick chunk
  __shared__ float sm_f[4 * NQ];
  __shared__ double sm_s[4 * NQ];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int S4 = (a.S + NQ - 1) / NQ;   // workgroups per row
  const int64_t rowid = fdiv(blockIdx.x, a.div_s4);
  const int c4 = int(blockIdx.x - rowid * S4);
  const int b = int(fdiv(uint32_t(rowid), a.div_k));
  const int i = int(rowid - int64_t(b) * a.K);
  const T* row = static_cast<const T*>(a.draft) + int64_t(b) * a.db + int64_t(i) * a.V;
  const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
  const SigmaTest sg = sigma_test<DT, SIG>(a, b, i);

  // max and weighted mass of four 4096-chunks: a workgroup reads 16384
  // entries (64 per thread, strided: vectors j < NVQ lie in the first
  // 4096, the next NVQ in the second, and so on) and writes one partial per
  // 4096-chunk, the chunks the draw picks in.
  const int64_t c0 = int64_t(c4) * kStatsChunk;
  CV cv;
  cv.load(row, c0, a.V, aligned, tid);
  float m[NQ];
#pragma unroll
  for (int h = 0; h < NQ; ++h) m[h] = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < CV::NV; ++j) {
    float v[PV];
    cv.get(j, v);
#pragma unroll
    for (int e = 0; e < PV; ++e) m[j / NVQ] = fmaxf(m[j / NVQ], v[e]);
  }
#pragma unroll
  for (int h = 0; h < NQ; ++h) {
    m[h] = wave_max_u(m[h]);
    if (lane == 0) sm_f[4 * h + w] = m[h];
  }
  __syncthreads();
  float pc[NQ];
#pragma unroll
  for (int h = 0; h < NQ; ++h) {
    m[h] = fmaxf(fmaxf(sm_f[4 * h], sm_f[4 * h + 1]), fmaxf(sm_f[4 * h + 2], sm_f[4 * h + 3]));
    pc[h] = pivot_of(m[h]);
  }
  float sum[NQ];
#pragma unroll
  for (int h = 0; h < NQ; ++h) sum[h] = 0.0f;
#pragma unroll
  for (int j = 0; j < CV::NV; ++j) {
    float v[PV];
    cv.get(j, v);
    const int i0 = int(c0) + CV::local(tid, j);
    // a sigma member has a logit at or above the threshold value, so a
    // vector whose maximum lies below it in every lane of the wave has
    // none: its entries take weight 1 without the per-entry test (1 * ex
    // is ex exactly, so the sums are unchanged)
    bool member_possible = false;
    if (SIG) {
      float vmax = v[0];
#pragma unroll
      for (int e = 1; e < PV; ++e) vmax = fmaxf(vmax, v[e]);
      member_possible = __builtin_amdgcn_ballot_w64(vmax >= sg.val) != 0;
    }
    if (member_possible) {
#pragma unroll
      for (int e = 0; e < PV; ++e) {
        const float ex = __builtin_amdgcn_exp2f((v[e] - pc[j / NVQ]) * a.c32);
        sum[j / NVQ] += sg.weight(v[e], i0 + e) * ex;
      }
    } else {
#pragma unroll
      for (int e = 0; e < PV; ++e) sum[j / NVQ] += __builtin_amdgcn_exp2f((v[e] - pc[j / NVQ]) * a.c32);
    }
  }
#pragma unroll
  for (int h = 0; h < NQ; ++h) {
    const double ws = wave_sum_u(double(sum[h]));
    if (lane == 0) sm_s[4 * h + w] = ws;
  }
  __syncthreads();
  if (tid == 0) {
    const int cq = NQ * c4;
    uint64_t* wp = reinterpret_cast<uint64_t*>(a.part + rowid * a.S + cq);
#pragma unroll
    for (int h = 0; h < NQ; ++h) {
      if (cq + h < a.S) {
        dev_store(wp + 2 * h, pack2(m[h], 0.0f));
        dev_store(wp + 2 * h + 1, dbits((sm_s[4 * h] + sm_s[4 * h + 1]) + (sm_s[4 * h + 2] + sm_s[4 * h + 3])));
      }
    }
  }
}

// The draw of row (b, i) = blockIdx.x from its chunk partials.
template <int DT, bool SIG>
__global__ __launch_bounds__(kThreads) void k_sample_pick(SampleArgs a) {
  using T = typename Dt<DT>::T;
  __shared__ int sm_c;
  __shared__ double sm_pre, sm_target;
  __shared__ float sm_piv;
  __shared__ PickLds<DT, 1, kPickPerThread> sm_pk;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t rowid = blockIdx.x;
  const int b = int(fdiv(uint32_t(rowid), a.div_k));
  const int i = int(rowid - int64_t(b) * a.K);
  const T* row = static_cast<const T*>(a.draft) + int64_t(b) * a.db + int64_t(i) * a.V;
  const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
  const SigmaTest sg = sigma_test<DT, SIG>(a, b, i);
  if (w == 0) {
    const uint64_t* pw = reinterpret_cast<const uint64_t*>(a.part + rowid * a.S);
    // chunk partials (the first 64 stay in registers: one round trip for S <= 64)
    float m0 = -__builtin_inff();
    double s0 = 0.0;
    float mx = -__builtin_inff();
    for (int g = 0; g < a.S; g += 64) {
      const int cc = g + lane;
      const float mc = cc < a.S ? lo_f(dev_load(pw + cc * 2)) : -__builtin_inff();
      if (g == 0) {
        m0 = mc;
        s0 = cc < a.S ? bits_d(dev_load(pw + cc * 2 + 1)) : 0.0;
      }
      mx = fmaxf(mx, mc);
    }
    const float P = pivot_of(wave_max(mx));
    auto mass = [&](int cc, int g) -> double {
      float mc = m0;
      double sc = s0;
      if (g != 0) {
        mc = cc < a.S ? lo_f(dev_load(pw + cc * 2)) : -__builtin_inff();
        sc = cc < a.S ? bits_d(dev_load(pw + cc * 2 + 1)) : 0.0;
      }
      return sc > 0.0 ? sc * rescale(pivot_of(mc), P, a.c32) : 0.0;
    };
    double Z = 0.0;
    for (int g = 0; g < a.S; g += 64) Z += lane_d(wave_incl_scan_d(mass(g + lane, g), lane), 63);
    const double target = double(a.u[rowid]) * Z;
    int cs = -1;
    double pre = 0.0;
    if (Z > 0.0) chunk_crossing(mass, a.S, target, lane, cs, pre);
    if (lane == 0) {
      sm_c = cs;
      sm_pre = pre;
      sm_target = target;
      sm_piv = P;
    }
  }
  __syncthreads();
  const int cs = sm_c;
  int tok = -1;
  if (cs >= 0) {
    const int64_t c0 = int64_t(cs) * kPickChunk;
    const float P = sm_piv, c32 = a.c32;
    ChunkVecs<DT, false, kPickPerThread> cv[1];
    cv[0].load(row, c0, a.V, aligned, tid);
    tok = chunk_pick<DT, 1, kPickPerThread>(cv, c0, sm_pre, sm_target,
                            [&](const float (&x)[1], int idx) {
                              const float ex = __builtin_amdgcn_exp2f((x[0] - P) * c32);
                              return SIG ? sg.weight(x[0], idx) * ex : ex;
                            },
                            sm_pk);
  }
  if (tid == 0) a.tok_out[rowid] = tok;
}

template <int DT, bool SIG>
static hipError_t launch_sample_t(const SampleArgs& a0, hipStream_t st) {
  SampleArgs a = a0;
  constexpr int NQ = kStatsPerThread / kPickPerThread;
  const int S4 = (a.S + NQ - 1) / NQ;
  a.div_s4 = make_fastdiv(uint32_t(S4));
  a.div_k = make_fastdiv(uint32_t(a.K));
  const int64_t rows = int64_t(a.B) * a.K;
  hipLaunchKernelGGL((k_sample_chunks<DT, SIG>), dim3(unsigned(rows * S4)), dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_sample_pick<DT, SIG>), dim3(unsigned(rows)), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_sample(const SampleArgs& a, int dtype, hipStream_t st) {
  const bool sig = a.thr != nullptr;
  if (dtype == SSD_BF16) return sig ? launch_sample_t<1, true>(a, st) : launch_sample_t<1, false>(a, st);
  return sig ? launch_sample_t<0, true>(a, st) : launch_sample_t<0, false>(a, st);
}

}  // namespace ssd

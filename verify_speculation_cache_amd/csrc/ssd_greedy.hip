// Greedy verification: a drafted token is kept iff it is the target's argmax
// at its position, the scan stops at the first mismatch, and the target's
// argmax at the stopping position is emitted (til.phipham141.dev "Why does
// speculative decoding exist?", How it works, Fix 2). Argmax order: largest
// logit, ties to the smaller token index; a row with no finite logit has no
// argmax (-1). Temperature plays no part, and no draft logits are read.
//
// One workgroup per (batch row b, target row i = 0..K, 16384-entry chunk):
// chunk max and the smallest index holding it. The last workgroup of batch
// row b takes, per target row, the max over chunks and the first chunk
// (lowest indices) holding it, then runs the scan.
#include "ssd_device.hpp"

namespace ssd {

template <int DT>
__global__ __launch_bounds__(kThreads) void k_greedy(GreedyArgs a) {
  using T = typename Dt<DT>::T;
  using CV = ChunkVecs<DT, true, kStatsPerThread>;
  constexpr int PV = Dt<DT>::kPerVec;
  __shared__ float sm_f[4];
  __shared__ int sm_i[4];
  __shared__ int sm_last;
  __shared__ int e_arg[SSD_MAX_K + 1];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int KP = a.K + 1;
  const int per_b = KP * a.S;
  const int b = int(fdiv(blockIdx.x, a.div_pb));
  const int rem = blockIdx.x - b * per_b;
  const int r = int(fdiv(uint32_t(rem), a.div_s));
  const int c = rem - r * a.S;
  const T* row = static_cast<const T*>(a.target) + int64_t(b) * a.tb + int64_t(r) * a.V;

  // ---- chunk max and its smallest index ----
  {
    const int64_t c0 = int64_t(c) * kStatsChunk;
    CV cv;
    cv.load(row, c0, a.V, (reinterpret_cast<uintptr_t>(row) & 15u) == 0, tid);
    float lm = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < CV::NV; ++j) {
      float v[PV];
      cv.get(j, v);
#pragma unroll
      for (int e = 0; e < PV; ++e) lm = fmaxf(lm, v[e]);
    }
    float m = wave_max_u(lm);
    if (lane == 0) sm_f[w] = m;
    __syncthreads();
    m = fmaxf(fmaxf(sm_f[0], sm_f[1]), fmaxf(sm_f[2], sm_f[3]));
    // smallest local index equal to the max (vector order is index order
    // within a thread; across threads the minimum is taken); only a wave
    // with a lane whose maximum is the chunk's can hold it
    int best = 0x7FFFFFFF;
    if (__builtin_amdgcn_ballot_w64(lm == m) != 0) {   // wave-uniform
#pragma unroll
      for (int j = CV::NV - 1; j >= 0; --j) {
        float v[PV];
        cv.get(j, v);
#pragma unroll
        for (int e = PV - 1; e >= 0; --e) best = (v[e] == m) ? CV::local(tid, j) + e : best;
      }
      best = int(wave_min_u32(uint32_t(best)));
    }
    if (lane == 0) sm_i[w] = best;
    __syncthreads();
    if (tid == 0) {
      best = min(min(sm_i[0], sm_i[1]), min(sm_i[2], sm_i[3]));
      // a chunk whose max is -inf holds no argmax
      const int32_t idx = (m > -__builtin_inff()) ? int32_t(c0 + best) : -1;
      dev_store(a.part + (int64_t(b) * KP + r) * a.S + c,
                uint64_t(__float_as_uint(m)) | (uint64_t(uint32_t(idx)) << 32));
    }
  }
  if (!arrive_last(&a.cnt[int64_t(b) * kCntStride], uint32_t(per_b), &sm_last)) return;

  // ---- last workgroup of batch row b: argmax per target row, then the scan ----
  for (int rr = w; rr < KP; rr += 4) {   // one wave per target row
    const uint64_t* pp = a.part + (int64_t(b) * KP + rr) * a.S;
    float best_m = -__builtin_inff();
    int best_idx = -1;
    for (int g = 0; g < a.S; g += 64) {   // chunks in index order
      const int cc = g + lane;
      const uint64_t e = cc < a.S ? dev_load(pp + cc) : (uint64_t(0xFF800000u) | (uint64_t(0xFFFFFFFFu) << 32));
      const float mc = __uint_as_float(uint32_t(e));
      const float gm = wave_max(mc);
      // the first chunk of this group attaining the group max
      const uint64_t hit = __ballot(cc < a.S && mc == gm && gm > -__builtin_inff());
      if (hit && gm > best_m) {   // a later group must be strictly larger to win
        const int l = __ffsll((unsigned long long)hit) - 1;
        best_m = gm;
        best_idx = __shfl(int32_t(e >> 32), l);
      }
    }
    if (lane == 0) e_arg[rr] = best_idx;
  }
  __syncthreads();
  if (w == 0) {
    const int K = a.K;
    bool bad = false, keep = true;
    int32_t d = -1;
    if (lane < K) {
      d = a.tokens[int64_t(b) * K + lane];
      bad = d < 0 || d >= a.V;
      keep = !bad && d == e_arg[lane];
    }
    const uint64_t badm = __ballot(lane < K && bad);
    const uint64_t rej = __ballot(lane < K && !keep);
    const int av = badm ? -1 : (rej ? __ffsll((unsigned long long)rej) - 1 : K);
    for (int ii = lane; ii <= K; ii += 64) {
      int32_t o = -1;
      if (av >= 0) {
        if (ii < av) o = a.tokens[int64_t(b) * K + ii];
        else if (ii == av) o = e_arg[av];
      }
      a.out_tokens[int64_t(b) * (K + 1) + ii] = o;
    }
    if (lane == 0) a.accepted[b] = av;
  }
}

hipError_t launch_greedy(const GreedyArgs& a0, int dtype, hipStream_t st) {
  GreedyArgs a = a0;
  a.div_pb = make_fastdiv(uint32_t((a.K + 1) * a.S));
  a.div_s = make_fastdiv(uint32_t(a.S));
  const unsigned grid = unsigned(int64_t(a.B) * (a.K + 1) * a.S);
  if (dtype == SSD_BF16) hipLaunchKernelGGL(k_greedy<1>, dim3(grid), dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL(k_greedy<0>, dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace ssd

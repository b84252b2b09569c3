// Token-tree verification: the target checks every drafted branch of a tree
// in one pass (brentwoodlivery.com "Speculative decoding", Extensions and
// Variants, Multi-candidate speculation; shivam2003.com "Speculative
// Speculative Decoding", Where SSD sits in the inference stack).
//
// Each batch row walks its tree from the root. The children of the current
// node are tested in index order with the one-candidate rule (keep child x
// iff u * q(x) < P(x); brentwoodlivery.com "Speculative decoding", The
// Algorithm, step 3), P being p of the node for the first child and, after
// each rejection, the normalised residual max(0, P - q) / Z of the previous
// test. A kept child becomes the current node. When no child is left, one
// token is drawn from the last P by inverse CDF (token order).
//
// The residual after j rejections at a node is max(0, p - c_j q) / N(c_j)
// with c_1 = 1, c_{j+1} = c_j + N(c_j) and N(c) = sum_v max(0, p - c q):
// since max(0, max(0, p - c q)/N - q) = max(0, p - (c + N) q)/N, every
// residual is one scalar c away from p and q. Testing a child needs p and q
// at its token only (gathered once), so only N(c) and the final draw need a
// pass over the vocabulary.
//
// Kernels:
//  k_tree_stats  one workgroup per (batch row, statistics row, 16384-entry
//                chunk): chunk max and sum of every target row and every
//                draft row of an inner node.
//  k_tree_round  one workgroup per (batch row, 8192-entry chunk): the
//                residual mass max(0, e_t - c rho e_d) and the target mass of
//                the pending node over the chunk; the last workgroup of the
//                batch row either takes N(c) and walks on, or (no child left)
//                picks the token and writes the row's outputs. Rows without a
//                pending pass exit at once. The host launches as many rounds
//                as the topology can need. In the first round every
//                workgroup of a batch row starts by merging the row's
//                statistics partials, gathering p and q at every node's token
//                and walking until the walk needs a pass (the row's first
//                workgroup stores what later rounds read); repeating that in
//                each workgroup costs less than an arrival count and a
//                last-workgroup tail in the statistics pass.
#include "ssd_resid.hpp"

namespace ssd {

template <int DT>
__device__ __forceinline__ const typename Dt<DT>::T* tree_row(const TreeArgs& a, int b, int r) {
  using T = typename Dt<DT>::T;
  if (r < a.N) return static_cast<const T*>(a.target) + int64_t(b) * a.tb + int64_t(r) * a.V;
  return static_cast<const T*>(a.draft) + int64_t(b) * a.db + int64_t(a.rnode[r - a.N]) * a.V;
}

// Tests children of st.node until one pass over the vocabulary is needed:
// after a rejection (N of the new c, or the final draw when no sibling is
// left) or at a node without children (the bonus draw). Single thread.
__device__ void tree_walk(const TreeArgs& a, TreeState& st, const double* sP, const double* sQ, const float* sU) {
  for (;;) {
    const int ch = st.nxt;
    if (ch < 0) break;
    const double px = sP[ch], qx = sQ[ch];
    const double pc = st.c > 0.0 ? fmax(0.0, px - st.c * qx) / st.nc : px;
    if (double(sU[ch]) * qx < pc) {
      st.node = ch;
      st.depth += 1;
      st.nxt = a.first_child[ch];
      st.c = 0.0;
      st.nc = 1.0;
      continue;
    }
    st.c += st.nc;
    st.nxt = a.next_sib[ch];
    break;
  }
  st.status = 1;
}

template <int DT>
__global__ __launch_bounds__(kThreads) void k_tree_stats(TreeArgs a) {
  __shared__ float sm_f[4];
  __shared__ double sm_s[4];

  const int tid = threadIdx.x;
  const int per_b = a.NR * a.SS;
  const int b = int(fdiv(blockIdx.x, a.div_pb));
  const int rem = blockIdx.x - b * per_b;
  const int r = int(fdiv(uint32_t(rem), a.div_ss));
  const int c = rem - r * a.SS;

  const typename Dt<DT>::T* row = tree_row<DT>(a, b, r);
  ChunkVecs<DT, true, kStatsPerThread> cv;
  const int64_t c0 = int64_t(c) * kStatsChunk;
  cv.load(row, c0, a.V, (reinterpret_cast<uintptr_t>(row) & 15u) == 0, tid);
  float m;
  double sd;
  chunk_max_sum(cv, a.c32, sm_f, sm_s, m, sd);
  if (tid == 0) {
    uint64_t* wp = reinterpret_cast<uint64_t*>(a.part + (int64_t(b) * a.NR + r) * a.SS + c);
    dev_store(wp, pack2(m, 0.0f));
    dev_store(wp + 1, dbits(sd));
  }
}

// Start of batch row b's walk (every thread of a first-round workgroup):
// merges the row's statistics partials into e_piv / e_s, puts p and q of
// every node's token under its parent's rows and the node uniforms into
// sP / sQ / sU, and walks from the root until a pass is needed; the state
// comes back in *sm_st. With `writer` (one workgroup per row) it also stores
// the merged statistics and p, q for later rounds, and the outputs of a
// flagged row (a token outside [0, V)). Returns false for a flagged row.
template <int DT>
__device__ __forceinline__ bool tree_start(const TreeArgs& a, int b, bool writer, float* e_piv, double* e_s,
                                           double* sP, double* sQ, float* sU, TreeState* sm_st, int* sm_bad) {
  const int tid = threadIdx.x;
  const int N = a.N;
  int32_t x = 0;
  float u = 0.0f;
  if (tid < N) {   // node tid's token and uniform, loaded before the merge
    x = a.tokens[int64_t(b) * N + tid];
    u = a.u_acc[int64_t(b) * N + tid];
  }
  {
    const uint64_t* pb = reinterpret_cast<const uint64_t*>(a.part) + int64_t(b) * a.NR * a.SS * 2;
    if (a.SS <= 64) merge_rows_seg(pb, a.NR, a.SS, a.c32, e_piv, e_s);
    else merge_rows<2>(pb, a.NR, a.SS, a.c32, e_piv, e_s, nullptr);
  }
  __syncthreads();
  if (writer) {
    for (int rr = tid; rr < a.NR; rr += kThreads) {
      RowPartial rp{};
      rp.m = e_piv[rr];
      rp.s = e_s[rr];
      a.rstat[int64_t(b) * a.NR + rr] = rp;
    }
  }
  if (tid < 64) {
    // p and q of node n's token under its parent's rows (lane n, n >= 1)
    const int n = tid;
    const bool node = n >= 1 && n < N;
    const bool bad = node && (x < 0 || x >= a.V);
    double P = 0.0, Q = 0.0;
    if (node && !bad) {
      const int pn = a.parent[n], dr = a.drow[pn];
      const float zt = Dt<DT>::to_f(tree_row<DT>(a, b, pn)[x]);
      const float zd = Dt<DT>::to_f(tree_row<DT>(a, b, dr)[x]);
      const double st = e_s[pn], sd = e_s[dr];
      P = st > 0.0 ? exp2(double(zt - e_piv[pn]) * double(a.c32)) / st : 0.0;
      Q = sd > 0.0 ? exp2(double(zd - e_piv[dr]) * double(a.c32)) / sd : 0.0;
      if (writer) {
        a.pq[(int64_t(b) * N + n) * 2 + 0] = P;
        a.pq[(int64_t(b) * N + n) * 2 + 1] = Q;
      }
    }
    sP[n] = P;
    sQ[n] = Q;
    sU[n] = u;
    const uint64_t badm = __ballot(bad);
    if (n == 0) *sm_bad = badm != 0 ? 1 : 0;
  }
  __syncthreads();
  if (*sm_bad) {   // a token outside [0, V): the row is flagged
    if (writer) {
      for (int i = tid; i < N; i += kThreads) {
        a.out_tokens[int64_t(b) * N + i] = -1;
        if (a.out_nodes) a.out_nodes[int64_t(b) * N + i] = -1;
      }
      if (tid == 0) {
        a.accepted[b] = -1;
        TreeState st{};
        a.state[b] = st;   // status 0: no pass
      }
    }
    return false;
  }
  if (tid == 0) {
    TreeState st{};
    st.node = 0;
    st.nxt = a.first_child[0];
    st.depth = 0;
    st.c = 0.0;
    st.nc = 1.0;
    tree_walk(a, st, sP, sQ, sU);
    *sm_st = st;
  }
  __syncthreads();
  return true;
}

template <int DT, bool FIRST>
__global__ __launch_bounds__(kThreads) void k_tree_round(TreeArgs a) {
  using T = typename Dt<DT>::T;
  __shared__ double sm_pair[8];
  __shared__ int sm_last;
  __shared__ double sm_pre, sm_target;
  __shared__ int sm_c, sm_useres;
  __shared__ PickLds<DT, 2> sm_pk;
  __shared__ double sP[kMaxTree], sQ[kMaxTree];
  __shared__ float sU[kMaxTree];
  __shared__ int path[kMaxTree];
  __shared__ float e_piv[FIRST ? kMaxRows : 1];
  __shared__ double e_s[FIRST ? kMaxRows : 1];
  __shared__ TreeState sm_st;
  __shared__ int sm_bad;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = int(fdiv(blockIdx.x, a.div_s));
  const int c = blockIdx.x - b * a.S;
  TreeState st;
  if (FIRST) {
    if (!tree_start<DT>(a, b, c == 0, e_piv, e_s, sP, sQ, sU, &sm_st, &sm_bad)) return;
    st = sm_st;
  } else {
    st = a.state[b];
  }
  // Only a state the walk could have written is trusted; anything else (a
  // workspace not zero-filled for this shape) ends the row's rounds.
  if (st.status != 1 || st.node < 0 || st.node >= a.N || st.nxt >= a.N || st.depth < 0 || st.depth >= a.N)
    return;
  const int node = st.node;
  // merged statistics of a row: in LDS in the first round, else as stored
  auto rstat = [&](int r) {
    if (FIRST) {
      RowPartial rp{};
      rp.m = e_piv[r];
      rp.s = e_s[r];
      return rp;
    }
    return a.rstat[int64_t(b) * a.NR + r];
  };
  const RowPartial rt = rstat(node);
  const T* rowT = tree_row<DT>(a, b, node);
  const T* rowD = rowT;
  ResidConsts k{};
  set_rows(k, rt.m, rt.m, a.c32);
  set_plain(k);
  const int dr = a.drow[node];
  if (st.c > 0.0 && dr >= 0) {
    const RowPartial rd = rstat(dr);
    rowD = tree_row<DT>(a, b, dr);
    set_rows(k, rt.m, rd.m, a.c32);
    set_rho(k, rd.s > 0.0 ? st.c * rt.s / rd.s : 0.0, 1.0);
  }

  // ---------------- phase A: chunk masses ----------------
  {
    double R, P;
    resid_chunk_masses<DT, false>(k, rowT, rowD, int64_t(c) * kChunk, a.V, sm_pair, R, P);
    if (tid == 0) {
      uint64_t* wp = reinterpret_cast<uint64_t*>(a.cmass + (int64_t(b) * a.S + c) * 2);
      dev_store(wp, dbits(R));
      dev_store(wp + 1, dbits(P));
    }
  }
  if (!arrive_last(&a.cnt_round[int64_t(b) * kCntStride], uint32_t(a.S), &sm_last)) return;

  // ---------------- phase B: last workgroup of batch row b ----------------
  const int N = a.N;
  const uint64_t* cmw = reinterpret_cast<const uint64_t*>(a.cmass + int64_t(b) * a.S * 2);
  if (st.nxt >= 0) {
    // N(c) for the next sibling's test, then walk on
    __shared__ double sm_z;
    if (w == 0) {
      const int n = lane;
      // p, q and u of every node (already in LDS in the first round)
      double P = 0.0, Q = 0.0;
      float u = 0.0f;
      if (!FIRST && n >= 1 && n < N) {
        P = a.pq[(int64_t(b) * N + n) * 2 + 0];
        Q = a.pq[(int64_t(b) * N + n) * 2 + 1];
        u = a.u_acc[int64_t(b) * N + n];
      }
      double zres = 0.0;
      for (int g = 0; g < a.S; g += 64) {
        const int cc = g + lane;
        const double r = cc < a.S ? bits_d(dev_load(cmw + cc * 2)) : 0.0;
        zres += lane_d(wave_incl_scan_d(r, lane), 63);
      }
      if (!FIRST) {
        sP[n] = P;
        sQ[n] = Q;
        sU[n] = u;
      }
      if (lane == 0) sm_z = zres;
    }
    __syncthreads();
    if (tid == 0) {
      const double nc = rt.s > 0.0 ? sm_z / rt.s : 0.0;
      if (nc > 0.0) {
        st.nc = nc;
      } else {   // the residual has no mass: test the next sibling against p
        st.c = 0.0;
        st.nc = 1.0;
      }
      tree_walk(a, st, sP, sQ, sU);
      a.state[b] = st;
    }
    return;
  }

  // no child left: draw from max(0, p - c q) (p when c = 0 or it has no mass)
  if (w == 0) {
    double zres, ztgt, target, pre;
    int useres, cs;
    resid_find_chunk(cmw, a.S, a.u_res[b], lane, zres, ztgt, useres, target, cs, pre);
    if (lane == 0) {
      sm_c = cs;
      sm_pre = pre;
      sm_target = target;
      sm_useres = useres;
      // nodes on the kept path, root first
      int v = node;
      for (int d = st.depth; d >= 0; --d) {
        path[d] = v;
        v = v > 0 ? a.parent[v] : 0;
      }
    }
  }
  __syncthreads();
  const int cs = sm_c;
  int tok = -1;
  if (cs >= 0) {
    if (!sm_useres) set_plain(k);
    tok = resid_pick<DT, false>(k, rowT, rowD, cs, sm_pre, sm_target, a.V, sm_pk);
  }
  const int depth = st.depth;
  for (int i = tid; i < N; i += kThreads) {
    int32_t o = -1;
    if (i < depth) o = a.tokens[int64_t(b) * N + path[i + 1]];
    else if (i == depth) o = tok;
    a.out_tokens[int64_t(b) * N + i] = o;
    if (a.out_nodes) a.out_nodes[int64_t(b) * N + i] = i <= depth ? path[i] : -1;
  }
  if (tid == 0) {
    a.accepted[b] = depth;
    TreeState done = st;
    done.status = 0;
    a.state[b] = done;
  }
}

hipError_t launch_tree_stats(const TreeArgs& a0, int dtype, hipStream_t st) {
  TreeArgs a = a0;
  a.div_pb = make_fastdiv(uint32_t(a.NR * a.SS));
  a.div_ss = make_fastdiv(uint32_t(a.SS));
  const unsigned grid = unsigned(int64_t(a.B) * a.NR * a.SS);
  if (dtype == SSD_BF16) hipLaunchKernelGGL(k_tree_stats<1>, dim3(grid), dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL(k_tree_stats<0>, dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_tree_round(const TreeArgs& a0, int dtype, bool first, hipStream_t st) {
  TreeArgs a = a0;
  a.div_s = make_fastdiv(uint32_t(a.S));
  const unsigned grid = unsigned(int64_t(a.B) * a.S);
  if (dtype == SSD_BF16) {
    if (first) hipLaunchKernelGGL((k_tree_round<1, true>), dim3(grid), dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((k_tree_round<1, false>), dim3(grid), dim3(kThreads), 0, st, a);
  } else {
    if (first) hipLaunchKernelGGL((k_tree_round<0, true>), dim3(grid), dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((k_tree_round<0, false>), dim3(grid), dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace ssd

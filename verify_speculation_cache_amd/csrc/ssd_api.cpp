// C-ABI layer of libssdv: argument checks, workspace carving and kernel
// launches on the caller's stream. Every check runs on the host before the
// first HIP call, so bad arguments never reach the device.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "ssd_internal.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return SSD_OK;
}

constexpr double kLog2e = 1.4426950408889634073599246810018921;

bool dtype_ok(int dtype) { return dtype == SSD_F32 || dtype == SSD_BF16; }

int check_shape(int32_t B, int32_t K, int32_t V) {
  if (B < 1 || B >= (1 << 24)) return fail(SSD_EINVAL, "B=%d outside [1, 2^24)", B);
  if (K < 1 || K > SSD_MAX_K) return fail(SSD_EINVAL, "K=%d outside [1, %d]", K, SSD_MAX_K);
  if (V < 1) return fail(SSD_EINVAL, "V=%d must be >= 1", V);
  return SSD_OK;
}

int check_tau(float tau) {
  if (!(tau > 0.0f) || !std::isfinite(tau)) return fail(SSD_EINVAL, "tau=%g must be finite and > 0", double(tau));
  return SSD_OK;
}

int check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return SSD_OK;
  if (ws == nullptr) return fail(SSD_EWORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(SSD_EWORKSPACE, "workspace not 256-byte aligned");
  if (have < need) return fail(SSD_EWORKSPACE, "workspace %zu bytes < %zu needed", have, need);
  return SSD_OK;
}

int check_sigma(const ssd_sigma* s) {
  if (s == nullptr) return SSD_OK;
  if (!(s->C >= 0.0f && s->C <= 1.0f)) return fail(SSD_EINVAL, "sigma C=%g outside [0, 1]", double(s->C));
  if (s->thr == nullptr || s->draft_stats == nullptr) return fail(SSD_EINVAL, "sigma thr/draft_stats is NULL");
  return SSD_OK;
}

// grid dimension x is limited to 2^32-1 workgroups
int check_grid(int64_t wgs) {
  if (wgs > int64_t(0xFFFFFFFFll)) return fail(SSD_EINVAL, "problem too large for one launch (%lld workgroups)", (long long)wgs);
  return SSD_OK;
}

int check_fanout_vec(const int32_t* F, int32_t K, int32_t V, int* sumF) {
  if (F == nullptr) return fail(SSD_EINVAL, "F is NULL");
  long long s = 0;
  for (int k = 0; k <= K; ++k) {
    if (F[k] < 0 || F[k] > SSD_MAX_F || F[k] > V)
      return fail(SSD_EINVAL, "F[%d]=%d outside [0, min(V=%d, %d)]", k, F[k], V, SSD_MAX_F);
    s += F[k];
  }
  *sumF = int(s);
  return SSD_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SSD_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Argument blocks shared by the separate entry points and the fused round.
using namespace ssd;

CacheArgs cache_args(const void* draft, int64_t db, int32_t B, int32_t K, int32_t V, float tau, const int32_t* F,
                     int sumF, int32_t* cache_tokens, ssd_rowkey* thr, double* dstats, char* ws, const CacheWs& cw) {
  CacheArgs a{};
  a.draft = draft;
  a.db = db;
  a.B = B;
  a.K = K;
  a.V = V;
  a.S = int(chunks_per_row(V));
  a.sumF = sumF;
  a.c64 = kLog2e / double(tau);
  a.c32 = float(a.c64);
  int acc = 0;
  for (int k = 0; k <= K; ++k) {
    a.F[k] = F[k];
    a.off[k] = acc;
    acc += F[k];
  }
  a.off[K + 1] = acc;
  a.cache_tokens = cache_tokens;
  a.thr = thr;
  a.dstats = dstats;
  a.part = reinterpret_cast<CachePartial*>(ws + cw.part);
  a.cand = reinterpret_cast<Cand*>(ws + cw.cand);
  a.cnt = reinterpret_cast<uint32_t*>(ws + cw.cnt);
  return a;
}

StatsArgs verify_stats_args(const void* target, int64_t tb, const void* draft, int64_t db, int32_t B, int32_t K,
                            int32_t V, float tau, const int32_t* tokens, const float* u_acc, const ssd_sigma* sigma,
                            int32_t* accepted, int32_t* out_tokens, float* probs, float* row_lse, char* ws,
                            const StatsWs& sw, int pt) {
  const bool sig = sigma != nullptr;
  StatsArgs a{};
  a.target = target;
  a.tb = tb;
  a.draft = draft;
  a.db = db;
  a.B = B;
  a.K = K;
  a.V = V;
  a.pt = pt;
  a.S = int(chunks_of(V, pt));
  a.NR = sig ? K + 1 : 2 * K + 1;
  a.mode = sig ? kModeVerifySigma : kModeVerify;
  a.c64 = kLog2e / double(tau);
  a.c32 = float(a.c64);
  a.inv_tau = 1.0 / double(tau);
  a.tokens = tokens;
  a.u_acc = u_acc;
  a.use_sigma = sig ? 1 : 0;
  a.C = sig ? sigma->C : 1.0f;
  a.thr = sig ? sigma->thr : nullptr;
  a.dstats = sig ? sigma->draft_stats : nullptr;
  a.accepted = accepted;
  a.out_tokens = out_tokens;
  a.probs = probs;
  a.row_lse = row_lse;
  a.part = reinterpret_cast<RowPartial*>(ws + sw.part);
  a.cnt = reinterpret_cast<uint32_t*>(ws + sw.cnt);
  a.info = reinterpret_cast<RowInfo*>(ws + sw.info);
  a.zg = reinterpret_cast<uint64_t*>(ws + sw.zg);
  return a;
}

ResidArgs verify_resid_args(const StatsArgs& a, const float* u_res, float* resid_mass, char* ws_r,
                            const ResidWs& rw) {
  ResidArgs r{};
  r.target = a.target;
  r.tb = a.tb;
  r.draft = a.draft;
  r.db = a.db;
  r.B = a.B;
  r.K = a.K;
  r.V = a.V;
  r.S = int(pick_chunks_per_row(a.V));
  // small grids take one pick chunk per first-phase workgroup
  r.span_pt = a.pt == kSmallPerThread ? kSmallPerThread : kStatsPerThread;
  r.c32 = a.c32;
  r.u = u_res;
  r.info = a.info;
  r.cmass = reinterpret_cast<double*>(ws_r + rw.cmass);
  r.cnt = reinterpret_cast<uint32_t*>(ws_r + rw.cnt);
  r.tok_out = a.out_tokens;
  r.tok_stride = a.K + 1;
  r.tok_at_a = 1;
  r.mass_out = resid_mass;
  return r;
}

// Token-tree topology from a host parent array: children lists in index
// order, the statistics rows (targets of all nodes, then drafts of inner
// nodes) and the number of rounds a walk can need.
struct TreeTopo {
  int N = 0, NR = 0, rounds = 0;
  int8_t first_child[SSD_MAX_TREE], next_sib[SSD_MAX_TREE], parent[SSD_MAX_TREE];
  int8_t drow[SSD_MAX_TREE], rnode[SSD_MAX_TREE];
};

int tree_topology(const int32_t* parent, int32_t N, TreeTopo& t) {
  if (N < 1 || N > SSD_MAX_TREE) return fail(SSD_EINVAL, "N=%d outside [1, %d]", N, SSD_MAX_TREE);
  if (parent == nullptr) return fail(SSD_EINVAL, "parent is NULL");
  if (parent[0] != -1) return fail(SSD_EINVAL, "parent[0]=%d, the root's must be -1", parent[0]);
  for (int n = 1; n < N; ++n)
    if (parent[n] < 0 || parent[n] >= n)
      return fail(SSD_EINVAL, "parent[%d]=%d outside [0, %d)", n, parent[n], n);
  t.N = N;
  int nch[SSD_MAX_TREE] = {0};
  for (int n = 0; n < N; ++n) {
    t.first_child[n] = -1;
    t.next_sib[n] = -1;
    t.parent[n] = int8_t(parent[n]);
    t.drow[n] = -1;
    t.rnode[n] = 0;
  }
  for (int n = N - 1; n >= 1; --n) {   // prepend in reverse: lists end up in index order
    const int p = parent[n];
    t.next_sib[n] = t.first_child[p];
    t.first_child[p] = int8_t(n);
    nch[p] += 1;
  }
  int inner = 0;
  for (int n = 0; n < N; ++n)
    if (nch[n] > 0) {
      t.drow[n] = int8_t(N + inner);
      t.rnode[inner] = int8_t(n);
      ++inner;
    }
  t.NR = N + inner;
  // A walk ending at node n made one pass per rejected sibling before each
  // kept node on its path (the siblings with smaller index) and then
  // max(children, 1) passes at n (every child rejected, or the bonus draw at
  // a leaf); the largest such count over n is the number of rounds.
  int extra[SSD_MAX_TREE], seen[SSD_MAX_TREE] = {0};
  t.rounds = 0;
  for (int n = 0; n < N; ++n) {
    extra[n] = n == 0 ? 0 : extra[parent[n]] + seen[parent[n]]++;
    t.rounds = std::max(t.rounds, extra[n] + std::max(nch[n], 1));
  }
  return SSD_OK;
}

}  // namespace

using namespace ssd;

extern "C" {

// Status message setter for entry points defined in other source files.
int ssd_internal_fail(int code, const char* msg) { return fail(code, "%s", msg); }

SSD_API const char* ssd_last_error(void) { return g_err.c_str(); }

SSD_API int ssd_fanout(int32_t n_budget, int32_t K, double a_p, double r, int32_t* F_out) {
  if (F_out == nullptr) return fail(SSD_EINVAL, "F_out is NULL");
  if (n_budget < 0) return fail(SSD_EINVAL, "budget %d < 0", n_budget);
  if (K < 1 || K > SSD_MAX_K) return fail(SSD_EINVAL, "K=%d outside [1, %d]", K, SSD_MAX_K);
  if (!(a_p > 0.0 && a_p < 1.0) || !std::isfinite(a_p)) return fail(SSD_EINVAL, "a_p=%g outside (0, 1)", a_p);
  if (!(r > -1.0) || !std::isfinite(r)) return fail(SSD_EINVAL, "r=%g must be finite and > -1", r);
  // weights of the geometric shape: a_p^(k/(1+r)) for k < K, and the
  // all-accept length a_p^(K/(1+r)) (1 - a_p)^(-1/(1+r))
  const double e = 1.0 / (1.0 + r);
  std::vector<double> wgt(K + 1);
  double tot = 0.0;
  for (int k = 0; k < K; ++k) {
    wgt[k] = std::pow(a_p, double(k) * e);
    tot += wgt[k];
  }
  wgt[K] = std::pow(a_p, double(K) * e) * std::pow(1.0 - a_p, -e);
  tot += wgt[K];
  const double f0 = double(n_budget) / tot;
  std::vector<double> frac(K + 1);
  long long used = 0;
  for (int k = 0; k <= K; ++k) {
    const double v = f0 * wgt[k];
    const double fl = std::floor(v);
    F_out[k] = int32_t(fl);
    frac[k] = v - fl;
    used += F_out[k];
  }
  // leftover units to the largest fractional parts, ties to the smaller k
  long long left = (long long)n_budget - used;
  std::vector<char> taken(K + 1, 0);
  for (; left > 0; --left) {
    int best = -1;
    for (int k = 0; k <= K; ++k)
      if (!taken[k] && (best < 0 || frac[k] > frac[best])) best = k;
    if (best < 0) break;
    taken[best] = 1;
    F_out[best] += 1;
  }
  ok();
  return n_budget;
}

SSD_API int ssd_fanout_uniform(int32_t n_budget, int32_t K, int32_t* F_out) {
  if (F_out == nullptr) return fail(SSD_EINVAL, "F_out is NULL");
  if (n_budget < 0) return fail(SSD_EINVAL, "budget %d < 0", n_budget);
  if (K < 1 || K > SSD_MAX_K) return fail(SSD_EINVAL, "K=%d outside [1, %d]", K, SSD_MAX_K);
  // equal real shares; every fractional part ties, so the leftover units go
  // to the smallest lengths
  const int32_t base = n_budget / (K + 1), left = n_budget - base * (K + 1);
  for (int k = 0; k <= K; ++k) F_out[k] = base + (k < left ? 1 : 0);
  ok();
  return n_budget;
}

SSD_API int ssd_speedup(double p_hit, double e_hit, double e_miss, double t_p, double t_b, int32_t batch,
                        double* out) {
  if (out == nullptr) return fail(SSD_EINVAL, "out is NULL");
  if (!(p_hit >= 0.0 && p_hit <= 1.0)) return fail(SSD_EINVAL, "p_hit=%g outside [0, 1]", p_hit);
  if (!(e_hit >= 0.0) || !(e_miss >= 0.0) || !std::isfinite(e_hit) || !std::isfinite(e_miss))
    return fail(SSD_EINVAL, "E_hit, E_miss must be finite and >= 0");
  if (!(t_p >= 0.0) || !(t_b >= 0.0) || !std::isfinite(t_p) || !std::isfinite(t_b))
    return fail(SSD_EINVAL, "T_p, T_b must be finite and >= 0");
  if (batch < 1) return fail(SSD_EINVAL, "batch=%d < 1", batch);
  const double q = std::pow(p_hit, double(batch));   // every sequence of the batch hits
  *out = (p_hit * e_hit + (1.0 - p_hit) * e_miss) / (q * std::max(1.0, t_p) + (1.0 - q) * (1.0 + t_b));
  ok();
  return SSD_OK;
}

SSD_API int ssd_cache_stats(const int32_t* accepted, const uint8_t* hit, int32_t B, int32_t K,
                            uint32_t* counts, void* hip_stream) {
  if (!accepted || !hit || !counts) return fail(SSD_EINVAL, "a required pointer is NULL");
  if (B < 1 || B >= (1 << 24)) return fail(SSD_EINVAL, "B=%d outside [1, 2^24)", B);
  if (K < 1 || K > SSD_MAX_K) return fail(SSD_EINVAL, "K=%d outside [1, %d]", K, SSD_MAX_K);
  CacheStatsArgs a{};
  a.accepted = accepted;
  a.hit = hit;
  a.B = B;
  a.K = K;
  a.counts = counts;
  return hip_status(launch_cache_stats(a, as_stream(hip_stream)), "cache stats launch");
}

SSD_API size_t ssd_verify_workspace_size(int32_t B, int32_t K, int32_t V, int dtype) {
  if (check_shape(B, K, V) != SSD_OK || !dtype_ok(dtype)) return 0;
  const StatsWs sw(B, 2 * K + 1, chunks_of(V, stats_pt(B, 2 * K + 1, V)), K);
  const ResidWs rw(B, pick_chunks_per_row(V));
  return sw.total + rw.total;
}

SSD_API size_t ssd_residual_workspace_size(int32_t B, int32_t K, int32_t V, int dtype) {
  if (check_shape(B, K, V) != SSD_OK || !dtype_ok(dtype)) return 0;
  const StatsWs sw(B, 2, chunks_of(V, stats_pt(B, 2, V)), K);
  const ResidWs rw(B, pick_chunks_per_row(V));
  return sw.total + rw.total;
}

SSD_API size_t ssd_build_cache_workspace_size(int32_t B, int32_t K, int32_t V, int dtype) {
  if (check_shape(B, K, V) != SSD_OK || !dtype_ok(dtype)) return 0;
  return CacheWs(B, K, chunks_per_row(V)).total;
}

SSD_API int ssd_verify(const void* target_logits, int64_t target_bstride,
                       const void* draft_logits, int64_t draft_bstride, int dtype,
                       int32_t B, int32_t K, int32_t V, float tau,
                       const int32_t* draft_tokens, const float* u_acc, const float* u_res,
                       const ssd_sigma* sigma,
                       int32_t* accepted, int32_t* out_tokens, float* probs,
                       float* resid_mass, float* row_lse,
                       void* workspace, size_t ws_bytes, void* hip_stream) {
  int st;
  if (!dtype_ok(dtype)) return fail(SSD_EDTYPE, "unknown dtype %d", dtype);
  if ((st = check_shape(B, K, V)) != SSD_OK) return st;
  if ((st = check_tau(tau)) != SSD_OK) return st;
  if ((st = check_sigma(sigma)) != SSD_OK) return st;
  if (!target_logits || !draft_logits || !draft_tokens || !u_acc || !u_res || !accepted || !out_tokens)
    return fail(SSD_EINVAL, "a required pointer is NULL");
  if (target_bstride < 0 || draft_bstride < 0) return fail(SSD_EINVAL, "negative batch stride");
  const int64_t SP = pick_chunks_per_row(V);
  const int pt = stats_pt(B, 2 * K + 1, V);
  const int64_t SS = chunks_of(V, pt);
  const bool sig = sigma != nullptr;
  const int NR = sig ? K + 1 : 2 * K + 1;
  const StatsWs sw(B, 2 * K + 1, SS, K);
  const ResidWs rw(B, SP);
  if ((st = check_ws(workspace, ws_bytes, sw.total + rw.total)) != SSD_OK) return st;
  if ((st = check_grid(int64_t(B) * NR * SS)) != SSD_OK) return st;
  char* ws = static_cast<char*>(workspace);
  const StatsArgs a = verify_stats_args(target_logits, target_bstride, draft_logits, draft_bstride, B, K, V, tau,
                                        draft_tokens, u_acc, sigma, accepted, out_tokens, probs, row_lse, ws, sw,
                                        pt);
  hipStream_t stream = as_stream(hip_stream);
  // two launches: the statistics chunk pass, then per batch row the accept
  // scan (repeated in each of the row's residual workgroups, or for large
  // draws once per row in a launch of its own) and the draw
  if ((st = hip_status(launch_stats_chunks(a, dtype, stream), "stats launch")) != SSD_OK) return st;
  const RoundResidArgs rr{verify_resid_args(a, u_res, resid_mass, ws + sw.total, rw), a};
  return hip_status(launch_round_resid(rr, dtype, sig, stream), "residual launch");
}

SSD_API int ssd_residual_sample(const void* target_logits, int64_t target_bstride,
                                const void* draft_logits, int64_t draft_bstride, int dtype,
                                int32_t B, int32_t K, int32_t V, float tau,
                                const int32_t* row, const ssd_sigma* sigma, const float* u,
                                int32_t* token_out, float* mass_out,
                                void* workspace, size_t ws_bytes, void* hip_stream) {
  int st;
  if (!dtype_ok(dtype)) return fail(SSD_EDTYPE, "unknown dtype %d", dtype);
  if ((st = check_shape(B, K, V)) != SSD_OK) return st;
  if ((st = check_tau(tau)) != SSD_OK) return st;
  if ((st = check_sigma(sigma)) != SSD_OK) return st;
  if (!target_logits || !row || !u || !token_out) return fail(SSD_EINVAL, "a required pointer is NULL");
  if (sigma && !draft_logits) return fail(SSD_EINVAL, "sigma given without draft logits");
  if (target_bstride < 0 || draft_bstride < 0) return fail(SSD_EINVAL, "negative batch stride");
  const int64_t SP = pick_chunks_per_row(V);
  const int pt = stats_pt(B, 2, V);
  const int64_t SS = chunks_of(V, pt);
  const StatsWs sw(B, 2, SS, K);
  const ResidWs rw(B, SP);
  if ((st = check_ws(workspace, ws_bytes, sw.total + rw.total)) != SSD_OK) return st;
  if ((st = check_grid(int64_t(B) * 2 * SS)) != SSD_OK) return st;
  char* ws = static_cast<char*>(workspace);
  const bool sig = sigma != nullptr;

  StatsArgs a{};
  a.target = target_logits;
  a.tb = target_bstride;
  a.draft = draft_logits;
  a.db = draft_bstride;
  a.B = B;
  a.K = K;
  a.V = V;
  a.pt = pt;
  a.S = int(SS);
  a.NR = 2;
  a.mode = kModeRows;
  a.c64 = kLog2e / double(tau);
  a.c32 = float(a.c64);
  a.inv_tau = 1.0 / double(tau);
  a.rows_in = row;
  a.use_draft = draft_logits != nullptr ? 1 : 0;
  a.use_sigma = sig ? 1 : 0;
  a.C = sig ? sigma->C : 1.0f;
  a.thr = sig ? sigma->thr : nullptr;
  a.dstats = sig ? sigma->draft_stats : nullptr;
  a.part = reinterpret_cast<RowPartial*>(ws + sw.part);
  a.cnt = reinterpret_cast<uint32_t*>(ws + sw.cnt);
  a.info = reinterpret_cast<RowInfo*>(ws + sw.info);
  a.zg = reinterpret_cast<uint64_t*>(ws + sw.zg);
  hipStream_t stream = as_stream(hip_stream);
  // two launches: the statistics chunk pass over each batch row's pair of
  // rows, then the draw, every workgroup of which merges its row's partials
  if ((st = hip_status(launch_stats_chunks(a, dtype, stream), "stats launch")) != SSD_OK) return st;

  RoundResidArgs rr{};
  rr.s = a;
  ResidArgs& r = rr.r;
  r.target = target_logits;
  r.tb = target_bstride;
  r.draft = draft_logits;
  r.db = draft_bstride;
  r.B = B;
  r.K = K;
  r.V = V;
  r.S = int(SP);
  r.span_pt = pt == kSmallPerThread ? kSmallPerThread : kStatsPerThread;
  r.c32 = a.c32;
  r.u = u;
  r.info = a.info;
  r.cmass = reinterpret_cast<double*>(ws + sw.total + rw.cmass);
  r.cnt = reinterpret_cast<uint32_t*>(ws + sw.total + rw.cnt);
  r.tok_out = token_out;
  r.tok_stride = 1;
  r.tok_at_a = 0;
  r.mass_out = mass_out;
  return hip_status(launch_rows_resid(rr, dtype, sig, stream), "residual launch");
}

SSD_API size_t ssd_verify_greedy_workspace_size(int32_t B, int32_t K, int32_t V, int dtype) {
  if (check_shape(B, K, V) != SSD_OK || !dtype_ok(dtype)) return 0;
  return GreedyWs(B, K, stats_chunks_per_row(V)).total;
}

SSD_API int ssd_verify_greedy(const void* target_logits, int64_t target_bstride, int dtype,
                              int32_t B, int32_t K, int32_t V, const int32_t* draft_tokens,
                              int32_t* accepted, int32_t* out_tokens,
                              void* workspace, size_t ws_bytes, void* hip_stream) {
  int st;
  if (!dtype_ok(dtype)) return fail(SSD_EDTYPE, "unknown dtype %d", dtype);
  if ((st = check_shape(B, K, V)) != SSD_OK) return st;
  if (!target_logits || !draft_tokens || !accepted || !out_tokens)
    return fail(SSD_EINVAL, "a required pointer is NULL");
  if (target_bstride < 0) return fail(SSD_EINVAL, "negative batch stride");
  const int64_t SS = stats_chunks_per_row(V);
  const GreedyWs gw(B, K, SS);
  if ((st = check_ws(workspace, ws_bytes, gw.total)) != SSD_OK) return st;
  if ((st = check_grid(int64_t(B) * (K + 1) * SS)) != SSD_OK) return st;
  char* ws = static_cast<char*>(workspace);
  GreedyArgs a{};
  a.target = target_logits;
  a.tb = target_bstride;
  a.B = B;
  a.K = K;
  a.V = V;
  a.S = int(SS);
  a.tokens = draft_tokens;
  a.accepted = accepted;
  a.out_tokens = out_tokens;
  a.part = reinterpret_cast<uint64_t*>(ws + gw.part);
  a.cnt = reinterpret_cast<uint32_t*>(ws + gw.cnt);
  return hip_status(launch_greedy(a, dtype, as_stream(hip_stream)), "greedy launch");
}

SSD_API size_t ssd_draft_sample_workspace_size(int32_t B, int32_t K, int32_t V, int dtype) {
  if (check_shape(B, K, V) != SSD_OK || !dtype_ok(dtype)) return 0;
  return SampleWs(int64_t(B) * K, pick_chunks_per_row(V)).total;
}

SSD_API int ssd_draft_sample(const void* draft_logits, int64_t draft_bstride, int dtype,
                             int32_t B, int32_t K, int32_t V, float tau, const ssd_sigma* sigma,
                             const float* u, int32_t* tokens_out,
                             void* workspace, size_t ws_bytes, void* hip_stream) {
  int st;
  if (!dtype_ok(dtype)) return fail(SSD_EDTYPE, "unknown dtype %d", dtype);
  if ((st = check_shape(B, K, V)) != SSD_OK) return st;
  if ((st = check_tau(tau)) != SSD_OK) return st;
  if (sigma != nullptr && (!(sigma->C >= 0.0f && sigma->C <= 1.0f) || sigma->thr == nullptr))
    return fail(SSD_EINVAL, "sigma needs C in [0, 1] and thr");
  if (!draft_logits || !u || !tokens_out) return fail(SSD_EINVAL, "a required pointer is NULL");
  if (draft_bstride < 0) return fail(SSD_EINVAL, "negative batch stride");
  // one partial per 4096-entry pick chunk, four per 16384-entry workgroup
  const int64_t S = pick_chunks_per_row(V);
  const SampleWs sw(int64_t(B) * K, S);
  if ((st = check_ws(workspace, ws_bytes, sw.total)) != SSD_OK) return st;
  if ((st = check_grid(int64_t(B) * K * stats_chunks_per_row(V))) != SSD_OK) return st;
  char* ws = static_cast<char*>(workspace);
  SampleArgs a{};
  a.draft = draft_logits;
  a.db = draft_bstride;
  a.B = B;
  a.K = K;
  a.V = V;
  a.S = int(S);
  a.c32 = float(kLog2e / double(tau));
  a.C = sigma ? sigma->C : 1.0f;
  a.thr = sigma ? sigma->thr : nullptr;
  a.u = u;
  a.tok_out = tokens_out;
  a.part = reinterpret_cast<RowPartial*>(ws + sw.part);
  return hip_status(launch_sample(a, dtype, as_stream(hip_stream)), "sample launch");
}

SSD_API int ssd_build_cache(const void* draft_logits, int64_t draft_bstride, int dtype,
                            int32_t B, int32_t K, int32_t V, float tau, const int32_t* F,
                            int32_t* cache_tokens, ssd_rowkey* thr, double* draft_stats,
                            void* workspace, size_t ws_bytes, void* hip_stream) {
  int st;
  if (!dtype_ok(dtype)) return fail(SSD_EDTYPE, "unknown dtype %d", dtype);
  if ((st = check_shape(B, K, V)) != SSD_OK) return st;
  if ((st = check_tau(tau)) != SSD_OK) return st;
  int sumF = 0;
  if ((st = check_fanout_vec(F, K, V, &sumF)) != SSD_OK) return st;
  if (!draft_logits || !thr || !draft_stats || (sumF > 0 && !cache_tokens))
    return fail(SSD_EINVAL, "a required pointer is NULL");
  if (draft_bstride < 0) return fail(SSD_EINVAL, "negative batch stride");
  const int64_t S = chunks_per_row(V);
  const CacheWs cw(B, K, S);
  if ((st = check_ws(workspace, ws_bytes, cw.total)) != SSD_OK) return st;
  if ((st = check_grid(int64_t(B) * (K + 1) * S)) != SSD_OK) return st;
  char* ws = static_cast<char*>(workspace);
  const CacheArgs a = cache_args(draft_logits, draft_bstride, B, K, V, tau, F, sumF, cache_tokens, thr, draft_stats,
                                 ws, cw);
  return hip_status(launch_cache(a, dtype, as_stream(hip_stream)), "cache build launch");
}

SSD_API int ssd_cache_lookup(const int32_t* cache_tokens, const int32_t* F, int32_t B, int32_t K,
                             const int32_t* accepted, const int32_t* out_tokens,
                             uint8_t* hit, int32_t* slot, void* hip_stream) {
  if (B < 1 || B >= (1 << 24)) return fail(SSD_EINVAL, "B=%d outside [1, 2^24)", B);
  if (K < 1 || K > SSD_MAX_K) return fail(SSD_EINVAL, "K=%d outside [1, %d]", K, SSD_MAX_K);
  if (F == nullptr) return fail(SSD_EINVAL, "F is NULL");
  LookupArgs a{};
  int acc = 0;
  for (int k = 0; k <= K; ++k) {
    if (F[k] < 0 || F[k] > SSD_MAX_F) return fail(SSD_EINVAL, "F[%d]=%d outside [0, %d]", k, F[k], SSD_MAX_F);
    a.F[k] = F[k];
    a.off[k] = acc;
    acc += F[k];
  }
  a.off[K + 1] = acc;
  if (!accepted || !out_tokens || !hit || (acc > 0 && !cache_tokens))
    return fail(SSD_EINVAL, "a required pointer is NULL");
  a.cache_tokens = cache_tokens;
  a.B = B;
  a.K = K;
  a.sumF = acc;
  a.accepted = accepted;
  a.out_tokens = out_tokens;
  a.hit = hit;
  a.slot = slot;
  return hip_status(launch_lookup(a, as_stream(hip_stream)), "lookup launch");
}

SSD_API int ssd_tree_rounds(const int32_t* parent, int32_t N) {
  TreeTopo t;
  const int st = tree_topology(parent, N, t);
  return st != SSD_OK ? st : t.rounds;
}

SSD_API size_t ssd_verify_tree_workspace_size(int32_t B, int32_t N, int32_t V, int dtype) {
  if (B < 1 || B >= (1 << 24) || N < 1 || N > SSD_MAX_TREE || V < 1 || !dtype_ok(dtype)) return 0;
  return TreeWs(B, N, 2 * N - 1, stats_chunks_per_row(V), chunks_per_row(V)).total;
}

SSD_API int ssd_verify_tree(const void* target_logits, int64_t target_bstride,
                            const void* draft_logits, int64_t draft_bstride, int dtype,
                            int32_t B, int32_t N, int32_t V, float tau, const int32_t* parent,
                            const int32_t* tokens, const float* u_acc, const float* u_res,
                            int32_t* accepted, int32_t* out_tokens, int32_t* out_nodes,
                            void* workspace, size_t ws_bytes, void* hip_stream) {
  int st;
  if (!dtype_ok(dtype)) return fail(SSD_EDTYPE, "unknown dtype %d", dtype);
  if (B < 1 || B >= (1 << 24)) return fail(SSD_EINVAL, "B=%d outside [1, 2^24)", B);
  if (V < 1) return fail(SSD_EINVAL, "V=%d must be >= 1", V);
  if ((st = check_tau(tau)) != SSD_OK) return st;
  TreeTopo t;
  if ((st = tree_topology(parent, N, t)) != SSD_OK) return st;
  if (!target_logits || !tokens || !u_acc || !u_res || !accepted || !out_tokens)
    return fail(SSD_EINVAL, "a required pointer is NULL");
  if (N > 1 && !draft_logits) return fail(SSD_EINVAL, "draft_logits is NULL for a tree with inner nodes");
  if (target_bstride < 0 || draft_bstride < 0) return fail(SSD_EINVAL, "negative batch stride");
  const int64_t SS = stats_chunks_per_row(V), S = chunks_per_row(V);
  // laid out for the largest statistics row count of N nodes, as the size query
  const TreeWs tw(B, N, 2 * N - 1, SS, S);
  if ((st = check_ws(workspace, ws_bytes, tw.total)) != SSD_OK) return st;
  if ((st = check_grid(int64_t(B) * t.NR * SS)) != SSD_OK) return st;
  if ((st = check_grid(int64_t(B) * S)) != SSD_OK) return st;
  char* ws = static_cast<char*>(workspace);
  TreeArgs a{};
  a.target = target_logits;
  a.tb = target_bstride;
  a.draft = draft_logits;
  a.db = draft_bstride;
  a.B = B;
  a.N = N;
  a.V = V;
  a.NR = t.NR;
  a.SS = int(SS);
  a.S = int(S);
  a.c32 = float(kLog2e / double(tau));
  std::memcpy(a.first_child, t.first_child, sizeof(a.first_child));
  std::memcpy(a.next_sib, t.next_sib, sizeof(a.next_sib));
  std::memcpy(a.parent, t.parent, sizeof(a.parent));
  std::memcpy(a.drow, t.drow, sizeof(a.drow));
  std::memcpy(a.rnode, t.rnode, sizeof(a.rnode));
  a.tokens = tokens;
  a.u_acc = u_acc;
  a.u_res = u_res;
  a.accepted = accepted;
  a.out_tokens = out_tokens;
  a.out_nodes = out_nodes;
  a.part = reinterpret_cast<RowPartial*>(ws + tw.part);
  a.rstat = reinterpret_cast<RowPartial*>(ws + tw.rstat);
  a.pq = reinterpret_cast<double*>(ws + tw.pq);
  a.state = reinterpret_cast<TreeState*>(ws + tw.state);
  a.cmass = reinterpret_cast<double*>(ws + tw.cmass);
  a.cnt_round = reinterpret_cast<uint32_t*>(ws + tw.cnt_round);
  hipStream_t stream = as_stream(hip_stream);
  if ((st = hip_status(launch_tree_stats(a, dtype, stream), "tree stats launch")) != SSD_OK) return st;
  // the first round also starts every row's walk (rounds >= 1: the walk
  // always ends in a draw)
  for (int r = 0; r < t.rounds; ++r)
    if ((st = hip_status(launch_tree_round(a, dtype, r == 0, stream), "tree round launch")) != SSD_OK) return st;
  return ok();
}

SSD_API size_t ssd_verify_round_workspace_size(int32_t B, int32_t K, int32_t V, int dtype) {
  if (check_shape(B, K, V) != SSD_OK || !dtype_ok(dtype)) return 0;
  const int64_t S = chunks_per_row(V);
  return CacheWs(B, K, S).total + StatsWs(B, K + 1, S, K).total + ResidWs(B, pick_chunks_per_row(V)).total;
}

SSD_API int ssd_verify_round_marked(const void* target_logits, int64_t target_bstride,
                                    const void* draft_logits, int64_t draft_bstride, int dtype,
                                    int32_t B, int32_t K, int32_t V, float tau, const int32_t* F, float C,
                                    const int32_t* draft_tokens, const float* u_acc, const float* u_res,
                                    int32_t* cache_tokens, ssd_rowkey* thr, double* draft_stats,
                                    int32_t* accepted, int32_t* out_tokens, uint8_t* hit, int32_t* slot,
                                    void* workspace, size_t ws_bytes, void* hip_stream, void* const* marks) {
  int st;
  if (!dtype_ok(dtype)) return fail(SSD_EDTYPE, "unknown dtype %d", dtype);
  if ((st = check_shape(B, K, V)) != SSD_OK) return st;
  if ((st = check_tau(tau)) != SSD_OK) return st;
  if (!(C >= 0.0f && C <= 1.0f)) return fail(SSD_EINVAL, "C=%g outside [0, 1]", double(C));
  int sumF = 0;
  if ((st = check_fanout_vec(F, K, V, &sumF)) != SSD_OK) return st;
  if (!target_logits || !draft_logits || !draft_tokens || !u_acc || !u_res || !thr || !draft_stats ||
      !accepted || !out_tokens || !hit || (sumF > 0 && !cache_tokens))
    return fail(SSD_EINVAL, "a required pointer is NULL");
  if (target_bstride < 0 || draft_bstride < 0) return fail(SSD_EINVAL, "negative batch stride");
  // the statistics chunks of the round are 8192 entries, like the cache's
  const int64_t S = chunks_per_row(V);
  const CacheWs cw(B, K, S);
  const StatsWs sw(B, K + 1, S, K);
  const ResidWs rw(B, pick_chunks_per_row(V));
  const size_t off_s = cw.total, off_r = off_s + sw.total;
  if ((st = check_ws(workspace, ws_bytes, off_r + rw.total)) != SSD_OK) return st;
  if ((st = check_grid(int64_t(B) * (K + 1) * 2 * S)) != SSD_OK) return st;
  char* ws = static_cast<char*>(workspace);
  RoundArgs a{};
  a.c = cache_args(draft_logits, draft_bstride, B, K, V, tau, F, sumF, cache_tokens, thr, draft_stats, ws, cw);
  const ssd_sigma sig{C, thr, draft_stats};
  a.s = verify_stats_args(target_logits, target_bstride, draft_logits, draft_bstride, B, K, V, tau, draft_tokens,
                          u_acc, &sig, accepted, out_tokens, nullptr, nullptr, ws + off_s, sw, kPerThread);
  a.s.S = int(S);
  a.ncw = uint32_t((K + 1) * S);
  a.na = uint32_t(2 * (K + 1) / 3);   // target rows whose statistics share the cache's chunk pass
  RoundResidArgs rr{};
  rr.s = a.s;
  ResidArgs& r = rr.r;
  r = verify_resid_args(a.s, u_res, nullptr, ws + off_r, rw);
  r.cache_tokens = cache_tokens;
  r.sumF = sumF;
  for (int k = 0; k <= K; ++k) {
    r.lk_F[k] = F[k];
    r.lk_off[k] = a.c.off[k];
  }
  r.hit = hit;
  r.slot = slot;
  return hip_status(launch_round(a, rr, dtype, as_stream(hip_stream), marks), "round launch");
}

SSD_API int ssd_verify_round(const void* target_logits, int64_t target_bstride,
                             const void* draft_logits, int64_t draft_bstride, int dtype,
                             int32_t B, int32_t K, int32_t V, float tau, const int32_t* F, float C,
                             const int32_t* draft_tokens, const float* u_acc, const float* u_res,
                             int32_t* cache_tokens, ssd_rowkey* thr, double* draft_stats,
                             int32_t* accepted, int32_t* out_tokens, uint8_t* hit, int32_t* slot,
                             void* workspace, size_t ws_bytes, void* hip_stream) {
  return ssd_verify_round_marked(target_logits, target_bstride, draft_logits, draft_bstride, dtype, B, K, V, tau,
                                 F, C, draft_tokens, u_acc, u_res, cache_tokens, thr, draft_stats, accepted,
                                 out_tokens, hit, slot, workspace, ws_bytes, hip_stream, nullptr);
}

}  // extern "C"

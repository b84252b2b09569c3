// Internal interface between the C-ABI layer (ssd_api.cpp) and the HIP
// kernels: argument blocks, workspace layout and launcher declarations.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ssd.h"

namespace ssd {

// One workgroup = 256 lanes = four wave64s; every thread holds 32 logits of
// its chunk in registers, so a chunk is 8192 vocabulary entries.
constexpr int kThreads = 256;
constexpr int kPerThread = 32;
constexpr int kChunk = kThreads * kPerThread;   // 8192
constexpr int kMaxRows = 2 * SSD_MAX_K + 1;     // rows one verify batch element touches

inline int64_t chunks_per_row(int64_t V) { return (V + kChunk - 1) / kChunk; }

// Division by a divisor 1 <= d <= 2^31 fixed at launch, for dividends n
// below 2^31 (workgroup indices): with s = ceil(log2 d) and M =
// ceil(2^(32+s) / d) = 2^32 + m (m < 2^32 since d > 2^(s-1)), n / d =
// floor(n * M / 2^(32+s)) = (mulhi(n, m) + n) >> s, the sum staying below
// 2^32. It is exact: with M * d = 2^(32+s) + e, 0 <= e < d <= 2^s, the term
// n * e / (d * 2^(32+s)) is below 1/d, less than the gap from n/d to the
// next integer. The launchers fill these from the argument block's own
// sizes, so the kernels split a linear workgroup index with a scalar high
// multiply, an add and a shift instead of a division.
struct FastDiv {
  uint32_t m, s;
};
inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f{0u, 0u};
  if (d < 1 || d > (1u << 31)) return f;   // outside the sizes the launchers pass
  while ((uint64_t(1) << f.s) < d) ++f.s;
  f.m = uint32_t(((uint64_t(1) << (32 + f.s)) + d - 1) / d - (uint64_t(1) << 32));
  return f;
}

// The row-statistics pass reads 64 entries per thread: twice the bytes per
// workgroup, half the workgroups (dispatching workgroups, not HBM, bounds a
// one-chunk-per-workgroup pass at this size).
constexpr int kStatsPerThread = 64;
constexpr int kStatsChunk = kThreads * kStatsPerThread;   // 16384
inline int64_t stats_chunks_per_row(int64_t V) { return (V + kStatsChunk - 1) / kStatsChunk; }

// The residual / bonus draw keeps its chunk masses per 4096 entries: a
// workgroup of its first phase covers one 16384-entry statistics span (four
// such chunks; one on small grids), and the in-chunk pick of the second
// phase, which runs on one workgroup per row with nothing else on its
// compute unit, has 16 tokens per thread to scan instead of 32.
constexpr int kPickPerThread = 16;
constexpr int kPickChunk = kThreads * kPickPerThread;      // 4096
inline int64_t pick_chunks_per_row(int64_t V) { return (V + kPickChunk - 1) / kPickChunk; }

// Small grids: when a verification's statistics pass would have fewer than
// kSmallGridWgs workgroups of 16384 entries (about two per compute unit),
// its statistics chunks and the draw's first-phase spans are 4096 entries
// instead: four times the workgroups with a quarter of the bytes each,
// since at that size one workgroup's own loads, not HBM, set the time.
constexpr int64_t kSmallGridWgs = 512;
// Residual grids of at least this many workgroups (more than stay resident
// at once) run the accept scan once per batch row in a launch of their own
// and leave its RowInfo in the workspace; smaller grids repeat it in every
// residual workgroup (no extra launch on the latency path).
#ifndef SSD_SCAN_ONCE_WGS
#define SSD_SCAN_ONCE_WGS 2048
#endif
constexpr int64_t kScanOnceWgs = SSD_SCAN_ONCE_WGS;
constexpr int kSmallPerThread = kPickPerThread;   // 16: a span of one pick chunk
inline int stats_pt(int64_t B, int64_t NR, int64_t V) {
  return B * NR * stats_chunks_per_row(V) < kSmallGridWgs ? kSmallPerThread : kStatsPerThread;
}
inline int64_t chunks_of(int64_t V, int pt) {
  const int64_t span = int64_t(kThreads) * pt;
  return (V + span - 1) / span;
}

// Per-(row, chunk) statistics: chunk max of the raw logits and the chunk's
// sum of exp2((z - pivot) * log2(e)/tau), pivot = chunk max (0 if -inf).
struct alignas(16) RowPartial {
  float m;
  float pad;
  double s;
};

// Everything the residual kernel needs about one batch row.
struct alignas(16) RowInfo {
  int32_t a;        // accepted length (-1: flagged row, skip)
  int32_t bonus;    // 1: draw from p of target row `a`; 0: from max(0, p - q)
  float piv_t;      // pivot of target row a (raw logit units)
  float piv_d;      // pivot of draft row a
  double s_t;       // sum exp2((z - piv_t) c) over target row a
  double s_d;       // sigma-weighted draft normaliser of row a (same units)
  uint32_t thr_key; // sigma membership threshold of draft row a
  int32_t thr_idx;
  float C;          // weight of members (1 when no sigma)
  int32_t pad;
};

// Per-(row, chunk) record of the cache build, four 64-bit words:
//  [0] chunk max (low 32 bits, float) | chunk threshold key T0 (high 32 bits)
//  [1] sum of exp2((z - max) * c) over the chunk entries that are not candidates
//  [2] number of candidates written for the chunk
struct alignas(32) CachePartial {
  uint64_t w[4];
};
constexpr int kCandCap = 128;   // candidate slots per (row, chunk)

struct Cand {
  uint32_t key;
  int32_t idx;
};

enum StatsMode { kModeVerify = 0, kModeVerifySigma = 1, kModeRows = 2 };

struct StatsArgs {
  const void* target;
  int64_t tb;
  const void* draft;
  int64_t db;
  int B, K, V, S, NR, mode;
  int pt;           // entries per thread of a statistics chunk (S = chunks of 256 * pt)
  float c32;        // log2(e) / tau
  double c64;       // log2(e) / tau in double
  double inv_tau;   // 1 / tau
  const int32_t* tokens;
  const float* u_acc;
  const int32_t* rows_in;   // kModeRows: position per batch row
  int use_draft;            // kModeRows: residual form (else bonus form)
  int use_sigma;
  float C;
  const ssd_rowkey* thr;
  const double* dstats;
  int32_t* accepted;
  int32_t* out_tokens;
  float* probs;
  float* row_lse;
  RowPartial* part;   // [B, NR, S] (S = stats chunks per row)
  uint32_t* cnt;      // [B] (kCntStride apart)
  RowInfo* info;      // [B]
  uint64_t* zg;       // [B, K]: target | draft logit at the drafted token (floats)
  FastDiv div_pb, div_s;   // by NR*S and by S: set by the launchers
};

struct ResidArgs {
  const void* target;
  int64_t tb;
  const void* draft;
  int64_t db;
  int B, K, V, S;
  int span_pt;         // entries per thread of a first-phase span: 64 (four pick chunks) or 16 (one)
  float c32;
  const float* u;
  const RowInfo* info;
  double* cmass;       // [B, S, 2]: residual mass, target mass per chunk (S chunks of kPickChunk
                       // for the one-path draw, of kChunk for the token-tree rounds)
  uint32_t* cnt;       // [B] (kCntStride apart)
  FastDiv div_nw;      // by the first-phase workgroups per row: set by the launchers
  int32_t* tok_out;    // token written at tok_out[b * tok_stride + (tok_at_a ? a : 0)]
  int64_t tok_stride;
  int tok_at_a;
  float* mass_out;     // nullable [B]
  // optional cache lookup of the drawn token (when hit != nullptr): hit[b] =
  // 1 iff it lies in segment a of cache row b, slot[b] = its position
  const int32_t* cache_tokens;   // [B, sumF]
  int sumF;
  int lk_F[SSD_MAX_K + 1];
  int lk_off[SSD_MAX_K + 1];
  uint8_t* hit;
  int32_t* slot;       // nullable
};

struct CacheArgs {
  const void* draft;
  int64_t db;
  int B, K, V, S, sumF;
  float c32;
  double c64;
  int F[SSD_MAX_K + 1];
  int off[SSD_MAX_K + 2];
  int32_t* cache_tokens;
  ssd_rowkey* thr;
  double* dstats;
  CachePartial* part;   // [B, K+1, S]
  Cand* cand;           // [B, K+1, S, kCandCap]
  uint32_t* cnt;        // [B, K+1] (kCntStride apart)
  FastDiv div_pb, div_s, div_kp;   // by (K+1)*S, by S, by K+1: set by the launchers
};

struct SampleArgs {
  const void* draft;
  int64_t db;
  int B, K, V, S;
  float c32;
  float C;                  // sigma weight of the top-F members (1: plain softmax)
  const ssd_rowkey* thr;    // [B, K+1] sigma thresholds (nullptr: plain)
  const float* u;           // [B, K]
  int32_t* tok_out;         // [B, K]
  RowPartial* part;         // [B*K, S]
  FastDiv div_s4, div_k;    // by (S+3)/4 and by K: set by the launcher
};

struct LookupArgs {
  const int32_t* cache_tokens;
  int B, K, sumF;
  int F[SSD_MAX_K + 1];
  int off[SSD_MAX_K + 2];
  const int32_t* accepted;
  const int32_t* out_tokens;
  uint8_t* hit;
  int32_t* slot;
};

// Workspace layouts (byte offsets, each 256-aligned).
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Completion counters sit kCntStride uint32 apart (4 KiB): device-scope
// atomics on one cache line serialise, so every counter gets its own line
// and memory channel.
constexpr int kCntStride = 1024;

struct StatsWs {
  size_t part, cnt, info, zg, total;
  StatsWs(int64_t B, int64_t NR, int64_t S, int64_t K) {
    part = 0;
    cnt = align256(part + sizeof(RowPartial) * B * NR * S);
    info = align256(cnt + sizeof(uint32_t) * kCntStride * B);
    zg = align256(info + sizeof(RowInfo) * B);
    total = align256(zg + sizeof(uint64_t) * B * K);
  }
};

struct ResidWs {
  size_t cmass, cnt, total;
  ResidWs(int64_t B, int64_t S) {
    cmass = 0;
    cnt = align256(cmass + sizeof(double) * 2 * B * S);
    total = align256(cnt + sizeof(uint32_t) * kCntStride * B);
  }
};

struct CacheWs {
  size_t part, cand, cnt, total;
  CacheWs(int64_t B, int64_t K, int64_t S) {
    part = 0;
    cand = align256(part + sizeof(CachePartial) * B * (K + 1) * S);
    cnt = align256(cand + sizeof(Cand) * B * (K + 1) * S * kCandCap);
    total = align256(cnt + sizeof(uint32_t) * kCntStride * B * (K + 1));
  }
};

struct CacheStatsArgs {
  const int32_t* accepted;
  const uint8_t* hit;
  int B, K;
  uint32_t* counts;   // [K+1, 2]
};

struct GreedyArgs {
  const void* target;
  int64_t tb;
  int B, K, V, S;            // S = stats chunks per row
  const int32_t* tokens;     // [B, K]
  int32_t* accepted;         // [B]
  int32_t* out_tokens;       // [B, K+1]
  uint64_t* part;            // [B, K+1, S]: chunk max (float bits) | argmax index << 32
  uint32_t* cnt;             // [B] (kCntStride apart)
  FastDiv div_pb, div_s;     // by (K+1)*S and by S: set by the launcher
};

struct GreedyWs {
  size_t part, cnt, total;
  GreedyWs(int64_t B, int64_t K, int64_t S) {
    part = 0;
    cnt = align256(part + sizeof(uint64_t) * B * (K + 1) * S);
    total = align256(cnt + sizeof(uint32_t) * kCntStride * B);
  }
};

struct SampleWs {
  size_t part, total;
  SampleWs(int64_t rows, int64_t S) {
    part = 0;
    total = align256(part + sizeof(RowPartial) * rows * S);
  }
};

// Token-tree verification. The topology is shared by the batch and fixed
// on the host (node 0 = root, parent[n] < n); every node has a target row,
// every node with children a draft row.
constexpr int kMaxTree = SSD_MAX_TREE;

// Walk state of one batch row between the rounds of a tree verification.
// The distribution the next child of `node` is tested against is
// max(0, p - c q) / nc (p itself when c = 0, nc = 1).
struct alignas(16) TreeState {
  int32_t node;     // current node
  int32_t nxt;      // next child of node to test (-1: none left)
  int32_t depth;    // accepted tokens so far
  int32_t status;   // 1: a pass over (node, c) is pending; 0: row finished
  double c, nc;
};

struct TreeArgs {
  const void* target;
  int64_t tb;
  const void* draft;
  int64_t db;
  int B, N, V, NR, SS, S;   // NR statistics rows, SS stats chunks, S residual chunks
  float c32;                // log2(e) / tau
  int8_t first_child[kMaxTree];   // -1: leaf
  int8_t next_sib[kMaxTree];      // -1: last child
  int8_t parent[kMaxTree];        // -1 for the root
  int8_t drow[kMaxTree];          // statistics row of the node's draft row (-1: leaf)
  int8_t rnode[kMaxTree];         // node of statistics row N + j
  const int32_t* tokens;    // [B, N]
  const float* u_acc;       // [B, N]
  const float* u_res;       // [B]
  int32_t* accepted;        // [B]
  int32_t* out_tokens;      // [B, N]
  int32_t* out_nodes;       // [B, N] or nullptr
  RowPartial* part;         // [B, NR, SS]
  RowPartial* rstat;        // [B, NR]: merged (pivot, sum) per row
  double* pq;               // [B, N, 2]: p and q of node n's token under its parent's rows
  TreeState* state;         // [B]
  double* cmass;            // [B, S, 2]
  uint32_t* cnt_round;      // [B] (kCntStride apart)
  FastDiv div_pb, div_ss, div_s;   // by NR*SS, by SS, by S: set by the launchers
};

struct TreeWs {
  size_t part, rstat, pq, state, cmass, cnt_round, total;
  TreeWs(int64_t B, int64_t N, int64_t NR, int64_t SS, int64_t S) {
    part = 0;
    rstat = align256(part + sizeof(RowPartial) * B * NR * SS);
    pq = align256(rstat + sizeof(RowPartial) * B * NR);
    state = align256(pq + sizeof(double) * 2 * B * N);
    cmass = align256(state + sizeof(TreeState) * B);
    cnt_round = align256(cmass + sizeof(double) * 2 * B * S);
    total = align256(cnt_round + sizeof(uint32_t) * kCntStride * B);
  }
};

// One verification round with the speculation cache (ssd_verify_round):
// the cache build's and the row statistics' chunk passes in one launch, the
// cache merges with the accept scan in a second, the residual draw with the
// cache lookup in a third.
struct RoundArgs {
  CacheArgs c;
  StatsArgs s;
  uint32_t ncw;         // cache chunk workgroups per batch row
  uint32_t na;          // target rows whose statistics run in the first launch (the rest in the second)
  FastDiv div_pb, div_pbb;   // by the first and second launch's chunk workgroups per batch row
};
struct RoundResidArgs {
  ResidArgs r;
  StatsArgs s;          // the accept scan's inputs (partials, sigma statistics)
};

// Launchers (return the hipError_t of the launch).
hipError_t launch_stats_chunks(const StatsArgs& a, int dtype, hipStream_t st);
hipError_t launch_cache(const CacheArgs& a, int dtype, hipStream_t st);
hipError_t launch_lookup(const LookupArgs& a, hipStream_t st);
hipError_t launch_sample(const SampleArgs& a, int dtype, hipStream_t st);
hipError_t launch_greedy(const GreedyArgs& a, int dtype, hipStream_t st);
hipError_t launch_cache_stats(const CacheStatsArgs& a, hipStream_t st);
hipError_t launch_tree_stats(const TreeArgs& a, int dtype, hipStream_t st);
hipError_t launch_tree_round(const TreeArgs& a, int dtype, bool first, hipStream_t st);
// start / stop (may be null): events the launch itself records at the
// kernel's start and end (hipExtLaunchKernel), for callers that time it
hipError_t launch_round_chunks(const RoundArgs& a, int dtype, hipStream_t st, hipEvent_t start = nullptr,
                               hipEvent_t stop = nullptr);
hipError_t launch_round_merge_stats(const RoundArgs& a, int dtype, hipStream_t st);
hipError_t launch_round_resid(const RoundResidArgs& a, int dtype, bool sigma, hipStream_t st);
hipError_t launch_rows_resid(const RoundResidArgs& a, int dtype, bool sigma, hipStream_t st);
// The three launches of a verification round; with marks (hipEvent_t[4],
// else NULL) the events are recorded on st before the chunk pass and after
// each launch.
hipError_t launch_round(const RoundArgs& a, const RoundResidArgs& rr, int dtype, hipStream_t st,
                        void* const* marks);

}  // namespace ssd

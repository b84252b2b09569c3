/*
 * ssd.h - C ABI of libssdv: batched speculative-decoding verification and the
 * SAGUARO speculation-cache build on one AMD MI355X (gfx950) GPU.
 *
 * Sources (page title, then section):
 *   [SD-notes]  brentwoodlivery.com, "Speculative decoding" study notes
 *   [SD-why]    til.phipham141.dev, "Why does speculative decoding exist?"
 *   [SSD-notes] papernotes.org, "Speculative Speculative Decoding" (ICLR 2026 notes)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Logits.  Row-major [B, rows, V] with the vocabulary contiguous; rows of one
 *   batch element are V elements apart; consecutive batch elements are
 *   `*_bstride` ELEMENTS apart (0 broadcasts one batch element to all B).
 *   dtype is SSD_F32 (float) or SSD_BF16 (bfloat16 bits). Values must be
 *   finite or -inf (a masked token); NaN and +inf are undefined.
 * Temperature.  x = logits / tau for target and draft alike, tau > 0 finite
 *   ([SD-notes] Temperature and Sampling).
 * Memory.  Every pointer documented "device" is device memory owned by the
 *   caller; "host" pointers are read during the call only. The library never
 *   allocates. Workspace: a device buffer (256-byte aligned) of at least the
 *   size returned by the matching *_workspace_size query. Its layout depends
 *   on the entry point and on (B, K, V, dtype); it must be ZERO-FILLED before
 *   its first use with a given entry point and shape. Each completed call
 *   leaves the completion counters it uses at zero, so the buffer can be
 *   reused for the same entry point and shape without clearing; zero it again
 *   before using it with another entry point or shape. A workspace that was
 *   not zero-filled gives wrong outputs but never makes the kernels address
 *   memory outside the caller's buffers. One workspace must not be used by
 *   two calls that may run at the same time.
 * Streams.  Calls enqueue kernels on `hip_stream` (a hipStream_t; NULL = the
 *   default stream) and return without synchronising. ssd_fanout,
 *   ssd_fanout_uniform, ssd_speedup and ssd_tree_rounds run on the host only.
 *   Graph capture is supported (no memset or allocation inside).
 * Errors.  Functions return SSD_OK (0) or a negative status; arguments are
 *   checked on the host before anything is enqueued, and ssd_last_error()
 *   gives a message for the calling thread's last failure. A drafted token
 *   outside [0, V) is a data error found on the device: that batch row gets
 *   accepted = -1, all its out_tokens = -1, hit = 0 and slot = -1; other rows
 *   are unaffected.
 * Determinism.  No floating-point atomics; identical inputs on the same
 *   device give bit-identical outputs.
 * Limits.  1 <= B < 2^24, 1 <= K <= 64, 1 <= V < 2^31, 0 <= F_k <= min(V, 64),
 *   token trees of 1 <= N <= 64 nodes.
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define SSD_API __attribute__((visibility("default")))
#else
#define SSD_API
#endif

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

enum {
  SSD_OK = 0,
  SSD_EINVAL = -1,     /* bad size, pointer, temperature, C, fan-out ... */
  SSD_EDTYPE = -2,     /* unknown dtype */
  SSD_EWORKSPACE = -3, /* workspace missing, too small or misaligned (256 B) */
  SSD_EHIP = -4        /* the HIP runtime refused a launch */
};

enum { SSD_MAX_K = 64, SSD_MAX_F = 64, SSD_MAX_TREE = 64 };

/* Position of one token in the top-F order of a draft row: an order-preserving
 * integer image of the logit (dtype specific) and the token index. Produced
 * by ssd_build_cache, consumed by ssd_verify / ssd_residual_sample; opaque. */
typedef struct {
  uint32_t key;
  int32_t idx;
} ssd_rowkey;

/* sigma_{F,C} reshaping of the draft distribution ([SSD-notes] key design 2):
 * q(t) is proportional to C*exp(x_t) for t among the F_k largest draft logits
 * of row k (ties: smaller index first), exp(x_t) otherwise. Passed to verify
 * and residual sampling to use the reshaped q; both arrays come from
 * ssd_build_cache run on the same draft logits with the same tau. */
typedef struct {
  float C;                    /* down-weight in [0, 1] */
  const ssd_rowkey* thr;      /* device [B, K+1]: last member of each top-F_k set */
  const double* draft_stats;  /* device [B, K+1, 3]: zmax, S_top, S_rest (see ssd_build_cache) */
} ssd_sigma;

/* Message for the calling thread's last non-OK return ("" if none). */
SSD_API const char* ssd_last_error(void);

/* Geometric fan-out of a cache budget over acceptance lengths k = 0..K
 * ([SSD-notes] key design 1): real-valued F_k = F_0 a_p^(k/(1+r)) for k < K,
 * F_K = F_0 a_p^(K/(1+r)) (1-a_p)^(-1/(1+r)), with F_0 chosen so the values
 * sum to n_budget; rounded by largest remainder (ties to the smaller k), so
 * the integers sum to n_budget exactly.
 * n_budget >= 0, 1 <= K <= 64, 0 < a_p < 1, r > -1, both finite.
 * F_out: host int32[K+1]. Returns sum(F) (= n_budget) or a negative status. */
SSD_API int ssd_fanout(int32_t n_budget, int32_t K, double a_p, double r, int32_t* F_out);

/* Uniform fan-out, the baseline cache shape of [SSD-notes] (ablation: cache
 * topology): n_budget split evenly over k = 0..K, the remainder going to the
 * smallest k (largest remainder with ties to the smaller k, as ssd_fanout).
 * F_out: host int32[K+1]. Returns sum(F) (= n_budget) or a negative status. */
SSD_API int ssd_fanout_uniform(int32_t n_budget, int32_t K, int32_t* F_out);

/* Expected speedup of SSD over the verifier alone ([SSD-notes] theoretical
 * analysis): (p E_hit + (1-p) E_miss) / (q max(1, T_p) + (1-q)(1 + T_b)) with
 * p = p_hit, and q = p_hit^batch the probability that every sequence of a
 * batch hits ([SSD-notes] batch-size-aware fallback); batch = 1 is the
 * single-sequence formula. T_p, T_b: primary and backup speculator times
 * relative to one verification; E_hit, E_miss: tokens per round on a hit or
 * a miss. 0 <= p_hit <= 1, E_* >= 0, T_* >= 0, batch >= 1. Writes *out;
 * returns SSD_OK or a negative status. Host only. */
SSD_API int ssd_speedup(double p_hit, double e_hit, double e_miss, double t_p, double t_b, int32_t batch,
                        double* out);

/* Per-length cache statistics of one round: counts[k][0] = rows whose
 * accepted length is k, counts[k][1] = those among them that hit (hit[b] = 1),
 * k = 0..K; flagged rows (accepted < 0) are not counted. Exact integer
 * counts (order-independent).
 *   accepted device int32 [B]; hit device uint8 [B]
 *   counts device uint32 [K+1, 2] (fully written). One kernel launch. */
SSD_API int ssd_cache_stats(const int32_t* accepted, const uint8_t* hit, int32_t B, int32_t K,
                            uint32_t* counts, void* hip_stream);

/* Bytes of workspace ssd_verify needs for this shape (any mode). */
SSD_API size_t ssd_verify_workspace_size(int32_t B, int32_t K, int32_t V, int dtype);

/* Batched verification ([SD-notes] The Algorithm, step 3; Batching
 * Speculation; [SD-why] How it works, Fixes 2 and 3).
 * For each batch row b and position i = 0..K-1, with p_i = softmax(target row
 * i / tau) and q_i = softmax(draft row i / tau) (or its sigma_{F_i,C} form):
 * the drafted token d = draft_tokens[b,i] is kept iff u_acc[b,i]*q_i(d) <
 * p_i(d) (accept with probability min(1, p/q)); the scan stops at the first
 * rejection. With a = number kept, the extra token t* is drawn from
 * max(0, p_a - q_a)/Z if a < K, or from p_K if a = K, by inverse CDF in token
 * order: the smallest v whose running mass exceeds u_res[b]*Z. If that
 * residual has no mass the draw uses p_a; if p_a has none, t* = -1.
 *   target_logits  device [B, K+1, V]  (row K feeds the bonus)
 *   draft_logits   device [B, >=K, V]  (rows 0..K-1 used; ignored with sigma
 *                                        except row a for the residual)
 *   draft_tokens   device int32 [B, K]
 *   u_acc          device float [B, K] in [0, 1);  u_res device float [B] in [0, 1)
 *   sigma          NULL for plain softmax q, else host pointer (see ssd_sigma)
 * Outputs (device):
 *   accepted    int32 [B]: a in 0..K, or -1 for a flagged row
 *   out_tokens  int32 [B, K+1]: d_1..d_a, t*, then -1 padding
 *   probs       float [B, K, 2] or NULL: (p_i(d), q_i(d)) for every i < K
 *   resid_mass  float [B] or NULL: Z of the final draw (probability units;
 *               1 for a bonus, 0 when the residual was empty)
 *   row_lse     float [B, 2K+1] or NULL: log-sum-exp of x over target rows
 *               0..K, then draft rows 0..K-1 (sigma form when sigma given)
 * Launches two kernels on hip_stream: the row statistics' chunk pass, then
 * one in which every workgroup of a batch row runs the row's accept scan
 * before its share of the draw. Draws of 2048 or more workgroups (B times
 * ceil(V / 16384)) run the accept scan once per batch row in a kernel of its
 * own between the two (three launches). */
SSD_API int ssd_verify(const void* target_logits, int64_t target_bstride,
                       const void* draft_logits, int64_t draft_bstride, int dtype,
                       int32_t B, int32_t K, int32_t V, float tau,
                       const int32_t* draft_tokens, const float* u_acc, const float* u_res,
                       const ssd_sigma* sigma,
                       int32_t* accepted, int32_t* out_tokens, float* probs,
                       float* resid_mass, float* row_lse,
                       void* workspace, size_t ws_bytes, void* hip_stream);

/* ssd_verify without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc). The workspace is a file-scope device array of
 * ssd_noalloc_scratch_bytes() bytes (SSD_NOALLOC_SCRATCH_BYTES, 16 MiB), one
 * copy per GPU the library runs on, held until the process ends; its
 * address on the current device is looked up on the first call on that
 * device. Every call clears the part it uses with a fill kernel before the
 * kernels of ssd_verify run (no memset, no allocation, so it can be
 * captured), so what an earlier call left there never matters. Arguments,
 * outputs and errors are those of ssd_verify; a shape whose workspace
 * (ssd_verify_workspace_size) exceeds the array returns SSD_EINVAL with a
 * message. All calls on one GPU share the array: calls that may overlap in
 * time on one GPU (other streams, other threads) race and give wrong
 * results. Launches the fill kernel, then ssd_verify's kernels, on
 * hip_stream (the current device's). */
#define SSD_NOALLOC_SCRATCH_BYTES (16u << 20)
SSD_API size_t ssd_noalloc_scratch_bytes(void);
SSD_API int ssd_verify_noalloc(const void* target_logits, int64_t target_bstride,
                               const void* draft_logits, int64_t draft_bstride, int dtype,
                               int32_t B, int32_t K, int32_t V, float tau,
                               const int32_t* draft_tokens, const float* u_acc, const float* u_res,
                               const ssd_sigma* sigma,
                               int32_t* accepted, int32_t* out_tokens, float* probs,
                               float* resid_mass, float* row_lse, void* hip_stream);

/* Bytes of workspace ssd_residual_sample needs. */
SSD_API size_t ssd_residual_workspace_size(int32_t B, int32_t K, int32_t V, int dtype);

/* One draw per batch row from position row[b] (0..K) ([SD-notes] step 3 and
 * Derivation of Acceptance Criterion): from max(0, p - q)/Z when row[b] < K
 * and draft_logits is given (q optionally sigma-reshaped), otherwise from p
 * of that target row (the bonus form). Same inverse-CDF convention and
 * fallbacks as ssd_verify. The rows' log-normalisers are recomputed from the
 * logits (one statistics pass over the row pair) rather than taken from the
 * caller: an fp32 log-normaliser carries about |lse| * 2^-24 of relative
 * error into every probability, more than the draws tolerate.
 *   target_logits device [B, K+1, V]; draft_logits device [B, >=K, V] or NULL
 *   row device int32 [B]; u device float [B]
 *   token_out device int32 [B]; mass_out device float [B] or NULL (Z).
 * Two kernel launches on hip_stream: the statistics chunk pass over each
 * batch row's pair of rows, then the draw (every workgroup of a batch row
 * merges the pair's partials itself). */
SSD_API int ssd_residual_sample(const void* target_logits, int64_t target_bstride,
                                const void* draft_logits, int64_t draft_bstride, int dtype,
                                int32_t B, int32_t K, int32_t V, float tau,
                                const int32_t* row, const ssd_sigma* sigma, const float* u,
                                int32_t* token_out, float* mass_out,
                                void* workspace, size_t ws_bytes, void* hip_stream);

/* Bytes of workspace ssd_verify_greedy needs. */
SSD_API size_t ssd_verify_greedy_workspace_size(int32_t B, int32_t K, int32_t V, int dtype);

/* Greedy verification ([SD-why] How it works, Fix 2: the drafted token is
 * kept iff it is also the target's argmax): for each batch row b, d_i =
 * draft_tokens[b,i] is kept iff it is the argmax of target row i (largest
 * logit, ties to the smaller index); the scan stops at the first mismatch a,
 * and the argmax of target row a (the correction, or the bonus from row K
 * when a = K) is emitted. A target row with no finite logit has no argmax:
 * its drafted token is rejected and the emitted token is -1. No temperature
 * and no draft logits.
 *   target_logits device [B, K+1, V]; draft_tokens device int32 [B, K]
 *   accepted device int32 [B]: a in 0..K, or -1 for a flagged row
 *   out_tokens device int32 [B, K+1]: d_1..d_a, argmax of row a, then -1
 * One kernel launch on hip_stream. */
SSD_API int ssd_verify_greedy(const void* target_logits, int64_t target_bstride, int dtype,
                              int32_t B, int32_t K, int32_t V, const int32_t* draft_tokens,
                              int32_t* accepted, int32_t* out_tokens,
                              void* workspace, size_t ws_bytes, void* hip_stream);

/* Bytes of workspace ssd_draft_sample needs. */
SSD_API size_t ssd_draft_sample_workspace_size(int32_t B, int32_t K, int32_t V, int dtype);

/* The draft phase's sampling ([SD-notes] The Algorithm, step 1; with sigma,
 * [SSD-notes] key design 2: the top-F_i tokens of draft row i keep weight C,
 * the others weight 1, and the draw is from the renormalised result): for
 * every batch row b and position i = 0..K-1, d[b,i] is drawn from
 * q_i = softmax(draft row i / tau), or its sigma_{F_i,C} form, by inverse CDF
 * in token order with u[b,i] (the smallest v whose running mass exceeds
 * u*Z). A row without mass (all -inf) draws -1.
 *   draft_logits device [B, >=K, V] (rows 0..K-1 read)
 *   sigma        NULL for the plain softmax, else host pointer whose thr comes
 *                from ssd_build_cache on the same draft rows (draft_stats is
 *                not read)
 *   u            device float [B, K] in [0, 1)
 *   tokens_out   device int32 [B, K]
 * Two kernel launches on hip_stream (chunk masses, then the per-row draw);
 * the workspace holds only chunk partials, written before they are read. */
SSD_API int ssd_draft_sample(const void* draft_logits, int64_t draft_bstride, int dtype,
                             int32_t B, int32_t K, int32_t V, float tau, const ssd_sigma* sigma,
                             const float* u, int32_t* tokens_out,
                             void* workspace, size_t ws_bytes, void* hip_stream);

/* Number of round kernels ssd_verify_tree launches for this topology (the
 * most vocabulary passes one walk can need), or a negative status for an
 * invalid parent array. Host only. */
SSD_API int ssd_tree_rounds(const int32_t* parent, int32_t N);

/* Bytes of workspace ssd_verify_tree needs (any topology of N nodes). */
SSD_API size_t ssd_verify_tree_workspace_size(int32_t B, int32_t N, int32_t V, int dtype);

/* Token-tree verification ([SD-notes] Extensions and Variants, Multi-
 * candidate speculation: the draft proposes a tree of candidates and the
 * target checks every path in one pass).
 * Topology (host, shared by the batch): N nodes, node 0 the root (the
 * position after the committed context), parent[0] = -1, 0 <= parent[n] < n.
 * Node n >= 1 holds token tokens[b,n], drawn from the draft distribution at
 * its parent; siblings are expected to be independent draws. For each batch
 * row the walk starts at the root with P = p of the node (softmax of its
 * target row / tau) and tests the node's children in index order with the
 * one-candidate rule ([SD-notes] The Algorithm, step 3): child x is kept iff
 * u_acc[b,x] * q(x) < P(x), q = softmax of the node's draft row / tau. After
 * a rejection P becomes max(0, P - q)/Z (or p of the node if that has no
 * mass) and the next sibling is tested. A kept child becomes the current
 * node and its token is emitted. When the current node has no child left to
 * test, one more token is drawn from P by inverse CDF in token order with
 * u_res[b]: the residual of the last rejection, or p of the node (the bonus)
 * when none of its children was tested; -1 if P has no mass.
 *   target_logits device [B, N, V]: row n = target logits after node n's path
 *   draft_logits  device [B, N, V]: row n = draft logits at node n (read only
 *                 for nodes with children; may be NULL when N = 1)
 *   tokens device int32 [B, N]; u_acc device float [B, N] in [0, 1) (entry 0
 *   of both unused); u_res device float [B] in [0, 1)
 * Outputs (device):
 *   accepted   int32 [B]: depth a of the final node (tokens kept), -1 flagged
 *   out_tokens int32 [B, N]: the a kept tokens, the drawn token, then -1
 *   out_nodes  int32 [B, N] or NULL: nodes on the kept path, root first
 *              (a+1 entries), then -1
 * A token outside [0, V) at any node >= 1 flags the row (everything -1).
 * Launches 1 + ssd_tree_rounds(parent, N) kernels on hip_stream. */
SSD_API int ssd_verify_tree(const void* target_logits, int64_t target_bstride,
                            const void* draft_logits, int64_t draft_bstride, int dtype,
                            int32_t B, int32_t N, int32_t V, float tau, const int32_t* parent,
                            const int32_t* tokens, const float* u_acc, const float* u_res,
                            int32_t* accepted, int32_t* out_tokens, int32_t* out_nodes,
                            void* workspace, size_t ws_bytes, void* hip_stream);

/* Bytes of workspace ssd_build_cache needs. */
SSD_API size_t ssd_build_cache_workspace_size(int32_t B, int32_t K, int32_t V, int dtype);

/* Speculation-cache keys ([SSD-notes] framework; key designs 1 and 2): for
 * every batch row b and acceptance length k = 0..K, the F_k tokens with the
 * largest draft logits on draft row k (order: logit descending, index
 * ascending) - the guessed bonus tokens prepared for outcome (k, t*).
 *   draft_logits device [B, >=K+1, V] (rows 0..K read)
 *   F host int32 [K+1] (e.g. from ssd_fanout), 0 <= F_k <= min(V, 64)
 * Outputs (device):
 *   cache_tokens int32 [B, sum F]: row b holds the K+1 segments in k order,
 *                segment k sorted in top-F order
 *   thr          ssd_rowkey [B, K+1]: the F_k-th member (or an empty marker)
 *   draft_stats  double [B, K+1, 3]: zmax = max logit of the row; S_top and
 *                S_rest = sums of exp((z - zmax)/tau) over the top-F_k set and
 *                over the other tokens (zmax taken as 0 if the row is all
 *                -inf). ln(C S_top + S_rest) + zmax/tau is the log-normaliser
 *                of sigma_{F_k,C}.
 * Two kernel launches on hip_stream (chunk pass, then per-row merge). */
SSD_API int ssd_build_cache(const void* draft_logits, int64_t draft_bstride, int dtype,
                            int32_t B, int32_t K, int32_t V, float tau, const int32_t* F,
                            int32_t* cache_tokens, ssd_rowkey* thr, double* draft_stats,
                            void* workspace, size_t ws_bytes, void* hip_stream);

/* Bytes of workspace ssd_verify_round needs. */
SSD_API size_t ssd_verify_round_workspace_size(int32_t B, int32_t K, int32_t V, int dtype);

/* One verification round with the speculation cache ([SSD-notes] framework
 * and key designs 1-2; [SD-notes] The Algorithm, step 3): the cache of
 * ssd_build_cache on draft rows 0..K, verification of the drafted tokens
 * against q = sigma_{F_i,C}(draft row i / tau) as ssd_verify with that
 * sigma, and the hit of the realised outcome as ssd_cache_lookup. The cache
 * outputs are bit-identical to ssd_build_cache's; the row sums of the
 * verification add 8192-entry chunk partials (ssd_verify: 16384), so an
 * outcome can differ from the three calls' only where a decision lies within
 * rounding of its threshold. Three launches instead of five: the first
 * streams draft rows 0..K for the cache and target rows 0..na-1 for the row
 * statistics (na = floor(2(K+1)/3)); the second runs every cache merge
 * beside the statistics of target rows na..K; and each residual workgroup
 * runs its batch row's accept scan before its share of the draw (the lookup
 * in the draw's last workgroup). As in ssd_verify, draws of 2048 or more
 * workgroups take the accept scan once per batch row in a launch of its own
 * before the residual launch.
 *   target_logits device [B, K+1, V]; draft_logits device [B, >=K+1, V]
 *   F host int32 [K+1] (0 <= F_k <= min(V, 64)); C in [0, 1]
 *   draft_tokens device int32 [B, K] (drawn from q_sigma, e.g. by
 *   ssd_draft_sample); u_acc device float [B, K]; u_res device float [B]
 * Outputs (device): cache_tokens int32 [B, sum F], thr ssd_rowkey [B, K+1],
 *   draft_stats double [B, K+1, 3] (as ssd_build_cache); accepted int32 [B],
 *   out_tokens int32 [B, K+1] (as ssd_verify); hit uint8 [B], slot int32 [B]
 *   or NULL (as ssd_cache_lookup).
 * Three kernel launches on hip_stream (four for the large draws above). */
SSD_API int ssd_verify_round(const void* target_logits, int64_t target_bstride,
                             const void* draft_logits, int64_t draft_bstride, int dtype,
                             int32_t B, int32_t K, int32_t V, float tau, const int32_t* F, float C,
                             const int32_t* draft_tokens, const float* u_acc, const float* u_res,
                             int32_t* cache_tokens, ssd_rowkey* thr, double* draft_stats,
                             int32_t* accepted, int32_t* out_tokens, uint8_t* hit, int32_t* slot,
                             void* workspace, size_t ws_bytes, void* hip_stream);

/* ssd_verify_round for callers that time its launches (profilers, the
 * bench): marks is NULL or a host array of four hipEvent_t (created by the
 * caller on the device of hip_stream, with timing). marks[0] and marks[1]
 * are the start and the end of the first launch (the cache chunk pass with
 * the statistics of target rows 0..na-1), recorded by that launch itself
 * (hipExtLaunchKernel), so their interval is the kernel's execution time;
 * marks[2] and marks[3] are recorded on hip_stream after the second launch
 * (the cache merges with the statistics of target rows na..K) and after the
 * residual launch, so those intervals also hold the gap before each launch
 * (the last one the accept-scan launch too where there is one). With marks,
 * call it on a stream that is not being captured into a graph (a launch
 * that records its own events is not a graph node); with marks NULL it is
 * ssd_verify_round. Everything else, the arguments and the outputs, are
 * those of ssd_verify_round. */
SSD_API int ssd_verify_round_marked(const void* target_logits, int64_t target_bstride,
                                    const void* draft_logits, int64_t draft_bstride, int dtype,
                                    int32_t B, int32_t K, int32_t V, float tau, const int32_t* F, float C,
                                    const int32_t* draft_tokens, const float* u_acc, const float* u_res,
                                    int32_t* cache_tokens, ssd_rowkey* thr, double* draft_stats,
                                    int32_t* accepted, int32_t* out_tokens, uint8_t* hit, int32_t* slot,
                                    void* workspace, size_t ws_bytes, void* hip_stream, void* const* marks);

/* Cache hit of the realised outcome ([SSD-notes] framework: the round's
 * outcome (k, t*) hits iff it is among the prepared keys): hit[b] = 1 iff
 * t* = out_tokens[b, a] lies in segment a of cache_tokens row b, with
 * a = accepted[b]; slot[b] = its position in that segment, else -1.
 *   cache_tokens device int32 [B, sum F]; F host int32 [K+1]
 *   accepted device int32 [B]; out_tokens device int32 [B, K+1]
 *   hit device uint8 [B]; slot device int32 [B] or NULL. One kernel launch. */
SSD_API int ssd_cache_lookup(const int32_t* cache_tokens, const int32_t* F, int32_t B, int32_t K,
                             const int32_t* accepted, const int32_t* out_tokens,
                             uint8_t* hit, int32_t* slot, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */

"""Plain float64 reference for batched speculative verification and the SAGUARO cache.

TEST INFRASTRUCTURE ONLY: used by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the GPU library. It is written from the
source pages, one step per function, in float64, with Python loops over batch
rows and positions and NumPy only for whole-row vector operations.

Sources (page title, then section):
  [SD-notes]  brentwoodlivery.com, "Speculative decoding" study notes
  [SD-why]    til.phipham141.dev, "Why does speculative decoding exist?"
  [SSD-notes] papernotes.org, "Speculative Speculative Decoding" (ICLR 2026 notes)
  [SSD-yc]    shivam2003.com, "Speculative Speculative Decoding - Guessing the
              Guess Before It Lands"

Inputs are the stored logits exactly as the GPU reads them: float32 values,
or bfloat16 bit patterns held in uint16 arrays (widened exactly).

Readings where the pages leave a step open (each is listed, with reasons, in
the design notes of this repository):
  - accept test: a drafted token is kept iff u * q < p, with u in [0, 1);
    this is "accept with probability min(1, p/q)" without a division, and it
    rejects when p = q = 0;
  - correction / bonus token: inverse CDF in token-index order, the smallest v
    whose running sum of the unnormalised mass exceeds u * Z;
  - if a rejection leaves no residual mass (Z <= 0, only possible through
    rounding or fully masked rows), the token is drawn from p of that row;
    if that row has no mass either, the token is -1;
  - top-F order: raw logit descending, then token index ascending;
  - sigma reshaping applies to draft rows 0..K-1 (the rows drafts are drawn
    from) and the cache's top-F set of length k is taken on draft row k;
  - fan-out rounding: largest remainder, ties to the smaller k;
  - a row whose drafted token lies outside [0, V) is flagged: accepted = -1
    and all its emitted tokens are -1.

Where a function has no independent pin, its docstring says "parity unpinned".
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "as_f64", "row_stats", "softmax", "top_f", "sigma_weights", "draft_probs",
    "sigma_row_stats", "accept_scan", "inverse_cdf", "verify_row", "verify",
    "residual_sample", "fanout", "fanout_real", "build_cache", "cache_lookup",
    "alpha", "expected_tokens", "p_hit_row", "sample_draft", "draft_sample", "segment_offsets",
    "argmax_token", "verify_greedy", "fanout_uniform", "cache_stats", "ssd_speedup",
    "tree_children", "tree_depth", "verify_tree_row", "verify_tree",
]


# ---------------------------------------------------------------------------
# input widening
# ---------------------------------------------------------------------------
def as_f64(z: np.ndarray) -> np.ndarray:
    """Stored logits -> float64. uint16 arrays are bfloat16 bit patterns."""
    z = np.asarray(z)
    if z.dtype == np.uint16:
        return (z.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if z.dtype == np.float32 or z.dtype == np.float64:
        return z.astype(np.float64)
    raise TypeError(f"unsupported logits dtype {z.dtype}")


# ---------------------------------------------------------------------------
# O1: temperature softmax   [SD-notes] Temperature and Sampling
# ---------------------------------------------------------------------------
def row_stats(z: np.ndarray, tau: float):
    """Max, sum and log-sum-exp of x = z / tau over one row.

    Both models divide their logits by the same temperature before the
    softmax ([SD-notes] Temperature and Sampling). Returns (m, s, lse) with
    m = max x, s = sum exp(x - m), lse = m + ln s. A row whose entries are all
    -inf has no mass: (-inf, 0, -inf).
    """
    x = as_f64(z) / float(tau)
    m = float(np.max(x))
    if m == -math.inf:
        return m, 0.0, -math.inf
    s = float(np.sum(np.exp(x - m)))
    return m, s, m + math.log(s)


def softmax(z: np.ndarray, tau: float) -> np.ndarray:
    """p = softmax(z / tau) in float64 ([SD-notes] Temperature and Sampling)."""
    x = as_f64(z) / float(tau)
    m, s, lse = row_stats(z, tau)
    if s == 0.0:
        return np.zeros_like(x)
    return np.exp(x - lse)


# ---------------------------------------------------------------------------
# O2 / O3: top-F and sigma_{F,C}   [SSD-notes] key design 2 (SAGUARO sampling)
# ---------------------------------------------------------------------------
def top_f(z: np.ndarray, F: int) -> np.ndarray:
    """The F tokens with the largest draft logits.

    Order: logit value descending, ties broken by the smaller token index.
    The page selects the cache tokens as the top draft tokens by draft logit
    ([SSD-notes] key design 2); the tie order is a reading.
    """
    zf = as_f64(z)
    order = np.lexsort((np.arange(zf.shape[0]), -zf))
    return order[:int(F)]


def sigma_weights(V: int, T: np.ndarray, C: float) -> np.ndarray:
    """Per-token weight of sigma_{F,C}: C on the top-F set T, 1 elsewhere."""
    w = np.ones(V, dtype=np.float64)
    w[np.asarray(T, dtype=np.int64)] = float(C)
    return w


def draft_probs(z: np.ndarray, tau: float, F: Optional[int] = None, C: float = 1.0) -> np.ndarray:
    """Draft distribution q at temperature tau, optionally reshaped by sigma_{F,C}.

    sigma_{F,C}(x)_t is proportional to C*exp(x_t) for t in top_F, and to
    exp(x_t) otherwise ([SSD-notes] key design 2). F=None or C=1 gives the
    plain softmax. The normaliser is summed directly over all tokens.
    """
    x = as_f64(z) / float(tau)
    m = float(np.max(x))
    if m == -math.inf:
        return np.zeros_like(x)
    e = np.exp(x - m)
    if F is not None and F > 0:
        e = e * sigma_weights(x.shape[0], top_f(z, F), C)
    s = float(np.sum(e))
    if s == 0.0:
        return np.zeros_like(x)
    return e / s


def sigma_row_stats(z: np.ndarray, tau: float, F: int, C: float):
    """Statistics the cache build reports for one draft row.

    Returns (zmax, S_top, S_rest, lse_sigma) with, for pivot = zmax (0 if the
    row is all -inf):
      S_top  = sum over top_F of exp((z - pivot) / tau)
      S_rest = sum over the other tokens of exp((z - pivot) / tau)
      lse_sigma = pivot / tau + ln(C * S_top + S_rest)
    """
    zf = as_f64(z)
    zmax = float(np.max(zf))
    piv = 0.0 if zmax == -math.inf else zmax
    e = np.exp((zf - piv) / float(tau))
    inT = np.zeros(zf.shape[0], dtype=bool)
    if F > 0:
        inT[top_f(z, F)] = True
    s_top = float(np.sum(e[inT]))
    s_rest = float(np.sum(e[~inT]))
    tot = float(C) * s_top + s_rest
    lse = piv / float(tau) + math.log(tot) if tot > 0 else -math.inf
    return zmax, s_top, s_rest, lse


# ---------------------------------------------------------------------------
# O5: accept scan   [SD-notes] The Algorithm, step 3; [SD-why] How it works, Fix 2/3
# ---------------------------------------------------------------------------
def accept_scan(p_tok: Sequence[float], q_tok: Sequence[float], u: Sequence[float]):
    """Walk the drafted tokens in order; stop at the first rejection.

    Token i is kept with probability min(1, p_i/q_i) ([SD-notes] step 3),
    decided against the supplied uniform as u_i * q_i < p_i. Returns
    (a, margins): a = number of leading tokens kept (K if none rejected),
    margins[i] = |p_i - u_i q_i| for the decisions actually taken (i <= a),
    nan for positions after the rejection.
    """
    K = len(p_tok)
    margins = np.full(K, np.nan)
    for i in range(K):
        p, q, ui = float(p_tok[i]), float(q_tok[i]), float(u[i])
        margins[i] = abs(p - ui * q)
        if not (ui * q < p):
            return i, margins
    return K, margins


# ---------------------------------------------------------------------------
# O6: residual / bonus draw   [SD-notes] step 3 and Derivation; [SD-why] Fix 3
# ---------------------------------------------------------------------------
def inverse_cdf(r: np.ndarray, u: float):
    """Draw a token from the (unnormalised) mass vector r with uniform u.

    Returns (t, Z, margin): Z = sum r, t = smallest index whose running sum
    exceeds u*Z (token-index order; a zero-mass token is never chosen), and
    margin = distance from u*Z to the nearest end of t's CDF interval.
    t = -1 when r has no positive mass.
    """
    cdf = np.cumsum(r)           # sequential running sum, float64
    Z = float(cdf[-1]) if cdf.shape[0] else 0.0
    if not Z > 0.0:
        return -1, Z, math.inf
    target = float(u) * Z
    t = int(np.searchsorted(cdf, target, side="right"))
    if t >= cdf.shape[0]:        # u*Z == Z cannot happen for u < 1; keep t valid
        t = int(np.flatnonzero(r > 0)[-1])
    lo = float(cdf[t - 1]) if t > 0 else 0.0
    margin = min(target - lo, float(cdf[t]) - target)
    return t, Z, margin


def _residual(p_row: np.ndarray, q_row: Optional[np.ndarray], u: float):
    """max(0, p - q) normalised, or p itself for the bonus (q_row None).

    On rejection the replacement comes from max(0, p - q) / Z ([SD-notes]
    step 3 and the Derivation of the acceptance criterion); after a full
    accept the bonus comes from the target distribution of the next position
    ([SD-notes] step 3, [SD-why] Fix 2). If the residual has no mass the draw
    falls back to p (reading).
    Returns (t, Z, margin, used_fallback).
    """
    if q_row is None:
        t, Z, mg = inverse_cdf(p_row, u)
        return t, Z, mg, False
    r = np.maximum(0.0, p_row - q_row)
    t, Z, mg = inverse_cdf(r, u)
    if Z > 0.0:
        return t, Z, mg, False
    t, _, mg = inverse_cdf(p_row, u)
    return t, Z, mg, True


def verify_row(target: np.ndarray, draft: np.ndarray, tokens: Sequence[int],
               u_acc: Sequence[float], u_res: float, tau: float,
               sigma: Optional[dict] = None) -> dict:
    """Verify one sequence's K drafted tokens ([SD-notes] The Algorithm).

    target [K+1, V]: target logits at positions 0..K (row K feeds the bonus).
    draft  [>=K, V]: draft logits; row i is the distribution d_{i+1} came from.
    sigma: None, or {"F": [K+1 ints], "C": float}; then q_i = sigma_{F_i,C}
    of draft row i ([SSD-notes] key design 2).
    Returns a, the emitted tokens [K+1] (d_1..d_a, then t*, then -1 padding
    as in [SD-notes] Batching Speculation), p/q at the drafted tokens, the
    accept and residual margins, Z, and the row log-sum-exps.
    """
    K = len(tokens)
    V = target.shape[-1]
    out = np.full(K + 1, -1, dtype=np.int64)
    res = {"a": -1, "out": out, "p_tok": np.full(K, np.nan), "q_tok": np.full(K, np.nan),
           "acc_margin": np.full(K, np.nan), "Z": math.nan, "res_margin": math.nan,
           "fallback": False, "lse_t": np.full(K + 1, np.nan), "lse_d": np.full(K, np.nan)}
    if any((int(d) < 0 or int(d) >= V) for d in tokens):
        return res
    P = [softmax(target[i], tau) for i in range(K + 1)]
    if sigma is None:
        Q = [softmax(draft[i], tau) for i in range(K)]
    else:
        Q = [draft_probs(draft[i], tau, int(sigma["F"][i]), float(sigma["C"])) for i in range(K)]
    for i in range(K + 1):
        res["lse_t"][i] = row_stats(target[i], tau)[2]
    for i in range(K):
        if sigma is None:
            res["lse_d"][i] = row_stats(draft[i], tau)[2]
        else:
            res["lse_d"][i] = sigma_row_stats(draft[i], tau, int(sigma["F"][i]), float(sigma["C"]))[3]
    p_tok = np.array([P[i][int(tokens[i])] for i in range(K)])
    q_tok = np.array([Q[i][int(tokens[i])] for i in range(K)])
    a, margins = accept_scan(p_tok, q_tok, u_acc)
    if a < K:
        t, Z, mg, fb = _residual(P[a], Q[a], u_res)
    else:
        t, Z, mg, fb = _residual(P[K], None, u_res)
    out[:a] = np.asarray(tokens[:a], dtype=np.int64)
    out[a] = t
    res.update(a=a, p_tok=p_tok, q_tok=q_tok, acc_margin=margins, Z=Z, res_margin=mg,
               fallback=fb)
    return res


def verify(target: np.ndarray, draft: np.ndarray, tokens: np.ndarray, u_acc: np.ndarray,
           u_res: np.ndarray, tau: float, sigma: Optional[dict] = None) -> dict:
    """Batched verification: every sequence accepts 0..K tokens independently
    ([SD-notes] Batching Speculation). Loops over the batch."""
    B, K = tokens.shape
    rows = [verify_row(target[b], draft[b], tokens[b], u_acc[b], float(u_res[b]), tau, sigma)
            for b in range(B)]
    return {
        "accepted": np.array([r["a"] for r in rows], dtype=np.int64),
        "out_tokens": np.stack([r["out"] for r in rows]),
        "probs": np.stack([np.stack([r["p_tok"], r["q_tok"]], axis=-1) for r in rows]),
        "acc_margin": np.stack([r["acc_margin"] for r in rows]),
        "res_margin": np.array([r["res_margin"] for r in rows]),
        "Z": np.array([r["Z"] for r in rows]),
        "fallback": np.array([r["fallback"] for r in rows]),
        "lse_t": np.stack([r["lse_t"] for r in rows]),
        "lse_d": np.stack([r["lse_d"] for r in rows]),
    }


def residual_sample(target: np.ndarray, draft: Optional[np.ndarray], rows: np.ndarray,
                    u: np.ndarray, tau: float, sigma: Optional[dict] = None) -> dict:
    """Draw one token per sequence from position rows[b].

    rows[b] < K with a draft: from max(0, p - q) of that position (the
    correction after a rejection); rows[b] == K, or no draft: from p of that
    position (the bonus). K is taken as target.shape[1] - 1.
    """
    B = target.shape[0]
    K = target.shape[1] - 1
    toks = np.full(B, -1, dtype=np.int64)
    Zs = np.full(B, np.nan)
    mgs = np.full(B, np.nan)
    for b in range(B):
        j = int(rows[b])
        P = softmax(target[b, j], tau)
        if draft is None or j == K:
            t, Z, mg, _ = _residual(P, None, float(u[b]))
        else:
            if sigma is None:
                Q = softmax(draft[b, j], tau)
            else:
                Q = draft_probs(draft[b, j], tau, int(sigma["F"][j]), float(sigma["C"]))
            t, Z, mg, _ = _residual(P, Q, float(u[b]))
        toks[b], Zs[b], mgs[b] = t, Z, mg
    return {"tokens": toks, "Z": Zs, "margin": mgs}


# ---------------------------------------------------------------------------
# O8: fan-out   [SSD-notes] key design 1 (verification cache and fan-out)
# ---------------------------------------------------------------------------
def fanout_real(n_budget: int, K: int, a_p: float, r: float) -> np.ndarray:
    """Real-valued geometric fan-out whose sum equals the budget.

    F_k = F_0 * a_p^(k/(1+r)) for k < K, and the all-accept length gets
    F_K = F_0 * a_p^(K/(1+r)) * (1 - a_p)^(-1/(1+r)) ([SSD-notes] key
    design 1). F_0 is set so that sum_k F_k equals the budget.
    """
    e = 1.0 / (1.0 + float(r))
    w = [float(a_p) ** (k * e) for k in range(K)]
    w.append(float(a_p) ** (K * e) * (1.0 - float(a_p)) ** (-e))
    F0 = float(n_budget) / sum(w)
    return np.array([F0 * wk for wk in w])


def fanout(n_budget: int, K: int, a_p: float, r: float) -> list:
    """Integer fan-out F[0..K]: floors of the real values, then the leftover
    budget one unit at a time to the largest fractional parts (ties to the
    smaller k), so the sum equals the budget (reading of the budget
    constraint sum F_k <= B in [SSD-notes] key design 1)."""
    real = fanout_real(n_budget, K, a_p, r)
    F = [int(math.floor(v)) for v in real]
    left = int(n_budget) - sum(F)
    order = sorted(range(K + 1), key=lambda k: (-(real[k] - math.floor(real[k])), k))
    for k in order[:left]:
        F[k] += 1
    return F


def segment_offsets(F: Sequence[int]) -> np.ndarray:
    """Start of each length-k segment in a row of cache_tokens."""
    return np.concatenate([[0], np.cumsum(np.asarray(F, dtype=np.int64))])


# ---------------------------------------------------------------------------
# A18 / A22: cache build and lookup   [SSD-notes] framework; key designs 1-2
# ---------------------------------------------------------------------------
def build_cache(draft: np.ndarray, tau: float, F: Sequence[int], C: float) -> dict:
    """For each sequence b and acceptance length k = 0..K: the F_k guessed
    bonus tokens (top-F_k of draft row k), the last one's index, and the
    row statistics (zmax, S_top, S_rest) used by the sigma-reshaped q.
    """
    B = draft.shape[0]
    K = len(F) - 1
    off = segment_offsets(F)
    cache = np.full((B, int(off[-1])), -1, dtype=np.int64)
    thr_idx = np.full((B, K + 1), -1, dtype=np.int64)
    stats = np.zeros((B, K + 1, 3))
    for b in range(B):
        for k in range(K + 1):
            T = top_f(draft[b, k], F[k])
            cache[b, off[k]:off[k + 1]] = T
            if F[k] > 0:
                thr_idx[b, k] = T[-1]
            zmax, s_top, s_rest, _ = sigma_row_stats(draft[b, k], tau, F[k], C)
            stats[b, k] = (zmax, s_top, s_rest)
    return {"cache_tokens": cache, "thr_idx": thr_idx, "stats": stats}


def cache_lookup(cache_tokens: np.ndarray, F: Sequence[int], accepted: np.ndarray,
                 out_tokens: np.ndarray):
    """Hit test of the realised outcome (a, t*) against the cache.

    The outcome of a round is the accepted length plus the correction/bonus
    token; it hits iff it is one of the prepared keys ([SSD-notes]
    framework). Returns hit [B] (0/1) and slot [B] (position of t* within
    the length-a segment, -1 on a miss or a flagged row).
    """
    off = segment_offsets(F)
    B = accepted.shape[0]
    hit = np.zeros(B, dtype=np.uint8)
    slot = np.full(B, -1, dtype=np.int64)
    for b in range(B):
        a = int(accepted[b])
        if a < 0:
            continue
        t = int(out_tokens[b, a])
        seg = cache_tokens[b, off[a]:off[a + 1]]
        where = np.flatnonzero(seg == t)
        if t >= 0 and where.shape[0] > 0:
            hit[b] = 1
            slot[b] = int(where[0])
    return hit, slot


# ---------------------------------------------------------------------------
# exact expectations   [SD-notes] Speedup Analysis; [SSD-yc] P_hit
# ---------------------------------------------------------------------------
def alpha(p: np.ndarray, q: np.ndarray) -> float:
    """Acceptance probability of one position when the drafted token is drawn
    from q: sum_x q(x) min(1, p(x)/q(x)) = sum_x min(p(x), q(x)) (the
    accepted term of [SD-notes] Derivation of Acceptance Criterion)."""
    return float(np.sum(np.minimum(p, q)))


def expected_tokens(alphas: Sequence[float]) -> float:
    """Expected emitted tokens (accepted + 1) when position i is accepted with
    probability alphas[i] independently: sum_{i=0..K} prod_{j<i} alphas[j].
    With a constant alpha this is the closed form of [SD-notes] Expected
    Acceptance Rate."""
    tot, run = 0.0, 1.0
    for i in range(len(alphas) + 1):
        tot += run
        if i < len(alphas):
            run *= float(alphas[i])
    return tot


def p_hit_row(target: np.ndarray, draft: np.ndarray, tau: float, F: Sequence[int],
              C: float, sigma_in_q: bool = True) -> dict:
    """Exact probability that the outcome (a, t*) of one sequence hits its cache.

    P(hit) = sum_{k<K} (prod_{j<k} alpha_j)(1 - alpha_k) R_k(T_k)
             + (prod_{j<K} alpha_j) p_K(T_K),
    where R_k is the normalised residual of position k and T_k the cached
    tokens for length k. This is the P_hit = sum over prepared outcomes of
    their probability ([SSD-yc] expected drafting overhead eliminated) taken
    over (k, t*) keys. It holds because the synthetic rows do not depend on
    the emitted tokens. Also returns the per-position alphas and E[tokens].
    """
    K = len(F) - 1
    P = [softmax(target[i], tau) for i in range(K + 1)]
    if sigma_in_q:
        Q = [draft_probs(draft[i], tau, int(F[i]), float(C)) for i in range(K)]
    else:
        Q = [softmax(draft[i], tau) for i in range(K)]
    al = [alpha(P[i], Q[i]) for i in range(K)]
    ph, run = 0.0, 1.0
    for k in range(K):
        r = np.maximum(0.0, P[k] - Q[k])
        Z = float(np.sum(r))
        Tk = top_f(draft[k], F[k])
        share = float(np.sum(r[Tk])) / Z if Z > 0 else 0.0
        ph += run * (1.0 - al[k]) * share
        run *= al[k]
    ph += run * float(np.sum(P[K][top_f(draft[K], F[K])]))
    return {"p_hit": ph, "alphas": al, "e_tokens": expected_tokens(al)}


def sample_draft(z: np.ndarray, tau: float, u: float, F: Optional[int] = None,
                 C: float = 1.0) -> int:
    """Draw a drafted token from the (optionally sigma-reshaped) draft
    distribution by inverse CDF; used by statistical tests that need drafts
    from q_sigma ([SSD-notes] key design 2)."""
    q = draft_probs(z, tau, F, C)
    t, _, _ = inverse_cdf(q, u)
    return t


def draft_sample(draft: np.ndarray, tau: float, u: np.ndarray, F: Optional[Sequence[int]] = None,
                 C: float = 1.0):
    """The draft phase for a batch ([SD-notes] The Algorithm, step 1; with F,
    the sigma_{F_i,C} reshaping of [SSD-notes] key design 2): for every
    sequence b and position i < K, d[b, i] is drawn from the draft
    distribution of row i by inverse CDF with u[b, i]. Returns tokens [B, K]
    (-1 for a row without mass) and the margins of the draws."""
    B, K = u.shape
    tokens = np.full((B, K), -1, dtype=np.int64)
    margins = np.full((B, K), math.inf)
    for b in range(B):
        for i in range(K):
            q = draft_probs(draft[b, i], tau, None if F is None else int(F[i]), C)
            t, _, mg = inverse_cdf(q, float(u[b, i]))
            tokens[b, i] = t
            margins[b, i] = mg
    return tokens, margins


# ---------------------------------------------------------------------------
# greedy verification   [SD-why] How it works, Fix 2
# ---------------------------------------------------------------------------
def argmax_token(z: np.ndarray) -> int:
    """The target's greedy token: the largest logit, ties to the smaller index
    (the same order as top_f). A row with no finite logit has none: -1."""
    zf = as_f64(z)
    if not np.any(zf > -math.inf):
        return -1
    return int(top_f(z, 1)[0])


def verify_greedy(target: np.ndarray, tokens: np.ndarray) -> dict:
    """Greedy verification: keep drafted token d_i iff it is the target's
    argmax at position i, stop at the first mismatch, and emit the target's
    argmax at the stopping position (the correction, or the bonus from row K
    when all K are kept). Temperature plays no part. A row with a drafted
    token outside [0, V) is flagged (accepted -1, all outputs -1).
    Returns accepted [B] and out_tokens [B, K+1]."""
    B, K = tokens.shape
    V = target.shape[-1]
    acc = np.full(B, -1, dtype=np.int64)
    out = np.full((B, K + 1), -1, dtype=np.int64)
    for b in range(B):
        if any(int(d) < 0 or int(d) >= V for d in tokens[b]):
            continue
        g = [argmax_token(target[b, i]) for i in range(K + 1)]
        a = K
        for i in range(K):
            if int(tokens[b, i]) != g[i]:
                a = i
                break
        acc[b] = a
        out[b, :a] = tokens[b, :a]
        out[b, a] = g[a]
    return {"accepted": acc, "out_tokens": out}


# ---------------------------------------------------------------------------
# cache statistics and policy   [SSD-notes] theoretical analysis; ablations
# ---------------------------------------------------------------------------
def fanout_uniform(n_budget: int, K: int) -> list:
    """The uniform cache shape (the baseline of the cache-topology ablation):
    real F_k = budget / (K+1) for every k, rounded like fanout (floors, then
    the leftover to the largest fractional parts, ties to the smaller k)."""
    real = [float(n_budget) / (K + 1)] * (K + 1)
    F = [int(math.floor(v)) for v in real]
    left = int(n_budget) - sum(F)
    order = sorted(range(K + 1), key=lambda k: (-(real[k] - math.floor(real[k])), k))
    for k in order[:left]:
        F[k] += 1
    return F


def cache_stats(accepted: np.ndarray, hit: np.ndarray, K: int) -> np.ndarray:
    """counts[k] = (rows with accepted length k, hits among them), k = 0..K;
    flagged rows (accepted < 0) are not counted."""
    counts = np.zeros((K + 1, 2), dtype=np.int64)
    for a, h in zip(accepted, hit):
        if 0 <= int(a) <= K:
            counts[int(a), 0] += 1
            counts[int(a), 1] += int(h != 0)
    return counts


def ssd_speedup(p_hit: float, e_hit: float, e_miss: float, t_p: float, t_b: float, batch: int = 1) -> float:
    """Expected SSD speedup ([SSD-notes] theoretical analysis):
    (p E_hit + (1-p) E_miss) / (p max(1, T_p) + (1-p)(1 + T_b)); for a batch
    of b sequences the round waits on a miss unless every sequence hits, so
    the time terms use p_hit^b ([SSD-notes] batch-size-aware fallback) while
    the tokens per sequence keep p_hit (a reading: the page states only that
    p_hit^b takes over the latency expectation)."""
    q = float(p_hit) ** int(batch)
    num = float(p_hit) * e_hit + (1.0 - float(p_hit)) * e_miss
    return num / (q * max(1.0, float(t_p)) + (1.0 - q) * (1.0 + float(t_b)))


# ---------------------------------------------------------------------------
# token-tree verification   [SD-notes] Extensions and Variants, Multi-candidate
#                           speculation; [SSD-yc] Where SSD sits in the
#                           inference stack (token trees)
# ---------------------------------------------------------------------------
def tree_children(parent: Sequence[int]) -> list:
    """Children of every node of a token tree, in node-index order.
    parent[0] = -1 (the root, the position after the committed context) and
    0 <= parent[n] < n for n >= 1."""
    ch = [[] for _ in range(len(parent))]
    for n in range(1, len(parent)):
        ch[int(parent[n])].append(n)
    return ch


def tree_depth(parent: Sequence[int]) -> list:
    """Depth of every node (root 0)."""
    d = [0] * len(parent)
    for n in range(1, len(parent)):
        d[n] = d[int(parent[n])] + 1
    return d


def _after_rejection(P: np.ndarray, q: np.ndarray, p: np.ndarray):
    """The distribution the next sibling is tested against once a child drawn
    from q was rejected under P: max(0, P - q) / Z ([SD-notes] step 3 and the
    Derivation of the acceptance criterion), or p of the node when the
    residual has no mass (reading, as for one candidate). Returns (P', r) with
    r the unnormalised residual (None on the fallback)."""
    r = np.maximum(0.0, P - q)
    Z = float(np.sum(r))
    if Z > 0.0:
        return r / Z, r
    return p, None


def verify_tree_row(target: np.ndarray, draft: np.ndarray, parent: Sequence[int],
                    tokens: Sequence[int], u_acc: Sequence[float], u_res: float,
                    tau: float) -> dict:
    """Verify one sequence's token tree ([SD-notes] Extensions and Variants,
    Multi-candidate speculation: the target checks every drafted branch in
    one pass).

    target [N, V]: target logits after each node's path; draft [N, V]: draft
    logits at each node (the distribution its children were drawn from; rows
    of leaves are not read). tokens[n] is node n's token (n >= 1), u_acc[n]
    the uniform of node n's test, u_res the uniform of the final draw.

    The walk applies the page's one-candidate rule ([SD-notes] The Algorithm,
    step 3) to the children of the current node in index order, each against
    the distribution left by the previous rejection (readings):
      P = p of the node; for each child c: keep c iff u_acc[c] q(x_c) < P(x_c);
      on a rejection P <- max(0, P - q) / Z; if that leaves no mass
      (Z <= 0) P <- p of the node.
    A kept child becomes the current node (its token is emitted); when every
    child of the current node was rejected, or it has none, one more token is
    drawn from the last P by inverse CDF with u_res: the residual
    max(0, P - q) of the last rejection, or p of the node (the bonus) when
    nothing was rejected there. With siblings drawn independently from q this
    keeps the emitted token distributed as p.
    Returns a = depth reached, out [N] (emitted tokens, -1 padding), nodes [N]
    (nodes on the kept path, root first, -1 padding), the margin of every
    test taken (nan for nodes not tested), the residual margin and Z.
    A token outside [0, V) at any node >= 1 flags the row (a = -1, all -1).
    """
    N = len(parent)
    V = target.shape[-1]
    out = np.full(N, -1, dtype=np.int64)
    nodes = np.full(N, -1, dtype=np.int64)
    res = {"a": -1, "out": out, "nodes": nodes, "acc_margin": np.full(N, np.nan),
           "res_margin": math.nan, "Z": math.nan}
    if any(int(tokens[n]) < 0 or int(tokens[n]) >= V for n in range(1, N)):
        return res
    ch = tree_children(parent)
    node, depth = 0, 0
    nodes[0] = 0
    while True:
        p = softmax(target[node], tau)
        P = p
        last_r = None                    # unnormalised residual of the last rejection
        kept = None
        if ch[node]:
            q = softmax(draft[node], tau)
            for c in ch[node]:
                x = int(tokens[c])
                u = float(u_acc[c])
                res["acc_margin"][c] = abs(P[x] - u * q[x])
                if u * q[x] < P[x]:
                    kept = c
                    break
                P, last_r = _after_rejection(P, q, p)
        if kept is None:
            t, Z, mg = inverse_cdf(P if last_r is None else last_r, u_res)
            out[depth] = t
            res.update(a=depth, res_margin=mg, Z=Z)
            return res
        out[depth] = int(tokens[kept])
        depth += 1
        nodes[depth] = kept
        node = kept


def verify_tree(target: np.ndarray, draft: np.ndarray, parent: Sequence[int], tokens: np.ndarray,
                u_acc: np.ndarray, u_res: np.ndarray, tau: float) -> dict:
    """Batched token-tree verification: every sequence walks its own tree
    (same topology, its own tokens, logits and uniforms). Loops over the batch."""
    B, N = tokens.shape
    rows = [verify_tree_row(target[b], draft[b], parent, tokens[b], u_acc[b], float(u_res[b]), tau)
            for b in range(B)]
    return {
        "accepted": np.array([r["a"] for r in rows], dtype=np.int64),
        "out_tokens": np.stack([r["out"] for r in rows]),
        "out_nodes": np.stack([r["nodes"] for r in rows]),
        "acc_margin": np.stack([r["acc_margin"] for r in rows]),
        "res_margin": np.array([r["res_margin"] for r in rows]),
        "Z": np.array([r["Z"] for r in rows]),
    }

"""Pins of the float64 oracle against facts the pages and mathematics fix.

Each check is independent of the oracle's own formula: library routines
(scipy logsumexp/softmax, numerical optimisation), brute force on tiny
inputs, printed worked examples (tests/golden), closed forms and exact
invariants (the output distribution of verification equals p). The planted-
mistake tests at the end show each pin fails when a plausible error is put
into the oracle.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.optimize
import scipy.special

import oracle.ssd_oracle as O
OM = O

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _ln_rows(rows):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(rows, dtype=np.float64)).astype(np.float32)


# ---------------------------------------------------------------------------
# O1: temperature softmax against scipy
# ---------------------------------------------------------------------------
def check_row_stats():
    rng = np.random.default_rng(11)
    for V, tau in ((1, 1.0), (7, 0.5), (1000, 0.7), (32000, 1.3)):
        z = (rng.standard_normal(V) * 4).astype(np.float32)
        if V > 3:
            z[rng.integers(0, V, size=V // 4)] = -np.inf
        m, s, lse = O.row_stats(z, tau)
        x = z.astype(np.float64) / tau
        assert abs(lse - scipy.special.logsumexp(x)) < 1e-12 * max(1, abs(lse))
        p = O.softmax(z, tau)
        assert np.allclose(p, scipy.special.softmax(x), rtol=1e-12, atol=1e-300)
        assert m == np.max(x)
    # bf16 bit patterns widen exactly
    bits = np.array([0x3F80, 0xBF80, 0x4000, 0xFF80, 0x0000, 0x8000], dtype=np.uint16)
    assert list(O.as_f64(bits)) == [1.0, -1.0, 2.0, -np.inf, 0.0, -0.0]
    # fully masked row has no mass
    m, s, lse = O.row_stats(np.full(5, -np.inf, dtype=np.float32), 1.0)
    assert s == 0.0 and lse == -np.inf
    assert not O.softmax(np.full(5, -np.inf, dtype=np.float32), 1.0).any()


def test_row_stats_matches_scipy():
    check_row_stats()


# ---------------------------------------------------------------------------
# O2: top-F order against brute-force rank counting
# ---------------------------------------------------------------------------
def _bruteforce_top(z, F):
    z = O.as_f64(z)
    V = len(z)
    rank = [sum(1 for u in range(V) if z[u] > z[v] or (z[u] == z[v] and u < v)) for v in range(V)]
    order = sorted(range(V), key=lambda v: rank[v])
    return order[:F]


def check_top_f():
    rng = np.random.default_rng(5)
    for trial in range(200):
        V = int(rng.integers(1, 40))
        z = rng.integers(-3, 4, size=V).astype(np.float32)      # many ties
        if trial % 5 == 0:
            z[rng.integers(0, V)] = -np.inf
        F = int(rng.integers(0, V + 1))
        assert list(O.top_f(z, F)) == _bruteforce_top(z, F)
    # all-equal row -> lowest indices; -0 ties with +0
    assert list(O.top_f(np.zeros(9, dtype=np.float32), 4)) == [0, 1, 2, 3]
    z = np.array([-0.0, 0.0, -0.0, 0.0], dtype=np.float32)
    assert list(O.top_f(z, 4)) == [0, 1, 2, 3]
    # bf16 bits
    bits = np.array([0x3F80, 0x4000, 0x3F80, 0xFF80], dtype=np.uint16)
    assert list(O.top_f(bits, 3)) == [1, 0, 2]


def test_top_f_matches_bruteforce():
    check_top_f()


# ---------------------------------------------------------------------------
# O3: sigma_{F,C} special cases
# ---------------------------------------------------------------------------
def check_sigma():
    rng = np.random.default_rng(3)
    z = (rng.standard_normal(50) * 2).astype(np.float32)
    tau = 0.7
    x = z.astype(np.float64) / tau
    sm = scipy.special.softmax(x)
    assert np.allclose(O.draft_probs(z, tau, 7, 1.0), sm, rtol=1e-12)
    assert np.allclose(O.draft_probs(z, tau, 0, 0.3), sm, rtol=1e-12)
    assert np.allclose(O.draft_probs(z, tau, 50, 0.3), sm, rtol=1e-12)
    q0 = O.draft_probs(z, tau, 7, 0.0)
    T = O.top_f(z, 7)
    assert not q0[T].any()
    rest = np.setdiff1d(np.arange(50), T)
    assert np.allclose(q0[rest], scipy.special.softmax(x[rest]), rtol=1e-12)
    # general C against scipy on log weights
    for C in (0.5, 0.3, 1e-3):
        w = np.ones(50)
        w[T] = C
        ref = scipy.special.softmax(x + np.log(w))
        assert np.allclose(O.draft_probs(z, tau, 7, C), ref, rtol=1e-12)
        zmax, s_top, s_rest, lse = O.sigma_row_stats(z, tau, 7, C)
        assert abs(lse - scipy.special.logsumexp(x + np.log(w))) < 1e-12
        assert abs(math.log(s_top + s_rest) + zmax / tau - scipy.special.logsumexp(x)) < 1e-12
    # cache tokens are scaled by C relative to the rest
    qC = O.draft_probs(z, tau, 7, 0.5)
    ratio = (qC / sm)
    assert np.allclose(ratio[T] / ratio[rest][0], 0.5, rtol=1e-12)


def test_sigma_special_cases():
    check_sigma()


# ---------------------------------------------------------------------------
# O4-O6: worked examples printed on the pages
# ---------------------------------------------------------------------------
def _run_golden(fx, case, u_res):
    tgt = _ln_rows(fx["p_rows"])
    dft = _ln_rows(fx["q_rows"])
    return O.verify_row(tgt, dft, fx["draft_tokens"], case["u_acc"], u_res, fx["tau"])


def check_worked_example(golden_dir):
    fx = _load(golden_dir, "worked_example_4token.json")
    c0 = fx["cases"][0]
    for u_res in np.linspace(0.0, 0.999, 37):
        r = _run_golden(fx, c0, float(u_res))
        assert r["a"] == c0["expect_accepted"]
        assert list(r["out"]) == c0["expect_out"]
        ratios = r["p_tok"][:3] / r["q_tok"][:3]
        assert np.allclose(ratios, c0["expect_ratios"], rtol=1e-6)
        assert np.all(r["acc_margin"][:3] >= 0.1 - 1e-6)
        assert abs(r["Z"] - 0.4) < 1e-6          # residual 0.5 - 0.1 on '.'
        assert int(np.sum(r["out"] >= 0)) == fx["printed"]["tokens_generated"]
    c1 = fx["cases"][1]
    r = _run_golden(fx, c1, 0.5)
    assert r["a"] >= c1["expect_accepted_at_least"]


def test_worked_example(golden_dir):
    check_worked_example(golden_dir)


def check_paris(golden_dir):
    fx = _load(golden_dir, "paris_example.json")
    c = fx["cases"][0]
    for u_res in (0.0, 0.3, 0.77, 0.999):
        r = _run_golden(fx, c, u_res)
        assert r["a"] == fx["printed"]["accepted_length"] == c["expect_accepted"]
        assert list(r["out"]) == c["expect_out"]
        assert fx["names"][r["out"][3]] == fx["printed"]["substitute"]


def test_paris_example(golden_dir):
    check_paris(golden_dir)


# ---------------------------------------------------------------------------
# O5+O6 distribution: output of verification equals p (losslessness)
# ---------------------------------------------------------------------------
def check_lossless(N=3000, seed=0):
    rng = np.random.default_rng(seed)
    grid = (np.arange(N) + 0.5) / N
    for V, tau in ((3, 1.0), (4, 0.7)):
        zt = (rng.standard_normal((2, V)) * 1.5).astype(np.float32)
        zd = (zt[:1] + rng.standard_normal((1, V)).astype(np.float32)).astype(np.float32)
        p0 = scipy.special.softmax(zt[0].astype(np.float64) / tau)
        q0 = scipy.special.softmax(zd[0].astype(np.float64) / tau)
        acc = np.zeros(V)
        for x in range(V):
            acc[x] = np.mean([O.verify_row(zt, zd, [x], [u], 0.5, tau)["a"] == 1 for u in grid])
        # resample histogram after a forced rejection (a token with p<q, top uniform)
        xr = int(np.argmax(q0 - p0))
        hist = np.zeros(V)
        for u in grid:
            r = O.verify_row(zt, zd, [xr], [0.999999], float(u), tau)
            assert r["a"] == 0
            hist[r["out"][0]] += 1.0 / N
        first = np.zeros(V)
        for x in range(V):
            first[x] += q0[x] * acc[x]
            first += q0[x] * (1.0 - acc[x]) * hist
        assert np.max(np.abs(first - p0)) < 3.0 / N, (first, p0)
        # bonus branch: every token kept -> the extra token follows p of the next position
        pK = scipy.special.softmax(zt[1].astype(np.float64) / tau)
        hb = np.zeros(V)
        x = int(np.argmax(p0 - q0))            # p >= q: always kept
        for u in grid:
            r = O.verify_row(zt, zd, [x], [0.999999], float(u), tau)
            assert r["a"] == 1
            hb[r["out"][1]] += 1.0 / N
        assert np.max(np.abs(hb - pK)) < 2.0 / N


def test_lossless_bruteforce():
    check_lossless()


# ---------------------------------------------------------------------------
# expected tokens: closed form at constant alpha
# ---------------------------------------------------------------------------
def check_expected_tokens(golden_dir, n=20000, seed=1):
    fx = _load(golden_dir, "expected_tokens_alpha07.json")
    p = np.array(fx["p"])
    q = np.array(fx["q"])
    assert abs(O.alpha(p, q) - fx["alpha"]) < 1e-15
    rng = np.random.default_rng(seed)
    lp, lq = np.log(p).astype(np.float32), np.log(q).astype(np.float32)
    for item in fx["printed_approx"]:
        K = item["K"]
        closed = (1 - fx["alpha"] ** (K + 1)) / (1 - fx["alpha"])
        assert abs(closed - item["e_tokens"]) < fx["printed_rounding"]
        assert abs(O.expected_tokens([fx["alpha"]] * K) - closed) < 1e-12
        tgt = np.tile(lp, (K + 1, 1))
        dft = np.tile(lq, (K, 1))
        q32 = scipy.special.softmax(lq.astype(np.float64))
        toks = (rng.random((n, K)) >= q32[0]).astype(np.int64)   # drafts ~ q
        ua = rng.random((n, K)).astype(np.float32)
        ur = rng.random(n).astype(np.float32)
        emitted = np.array([O.verify_row(tgt, dft, toks[i], ua[i], float(ur[i]), 1.0)["a"] + 1
                            for i in range(n)])
        se = emitted.std() / math.sqrt(n)
        assert abs(emitted.mean() - closed) < 4 * se, (K, emitted.mean(), closed, se)


def test_expected_tokens_closed_form(golden_dir):
    check_expected_tokens(golden_dir)


# ---------------------------------------------------------------------------
# O8: fan-out is the optimum of the budgeted hit-probability problem
# ---------------------------------------------------------------------------
def _fanout_by_optimiser(N, K, a_p, r):
    # outcome probabilities of the acceptance length: geometric for k < K, tail at K
    pk = np.array([a_p ** k * (1 - a_p) for k in range(K)] + [a_p ** K])
    # hit probability with a power-law miss rate: sum_k pk (1 - F_k^-r); maximise under sum F = N
    def neg(F):
        return -np.sum(pk * (1.0 - np.power(F, -r)))
    x0 = np.full(K + 1, N / (K + 1))
    res = scipy.optimize.minimize(neg, x0, method="SLSQP", bounds=[(1e-6, N)] * (K + 1),
                                  constraints=[{"type": "eq", "fun": lambda F: np.sum(F) - N}],
                                  options={"ftol": 1e-15, "maxiter": 2000})
    return res.x


def check_fanout():
    for (N, K, a_p, r) in ((64, 7, 0.8, 1.0), (128, 8, 0.7, 0.5), (64, 5, 0.8, 1.0),
                           (40, 3, 0.6, 2.0), (17, 2, 0.9, 0.25)):
        real = O.fanout_real(N, K, a_p, r)
        assert abs(real.sum() - N) < 1e-9
        opt = _fanout_by_optimiser(N, K, a_p, r)
        assert np.allclose(real, opt, rtol=2e-3, atol=2e-3), (real, opt)
        F = O.fanout(N, K, a_p, r)
        assert sum(F) == N and all(f >= 0 for f in F)
        assert all(abs(F[k] - real[k]) < 1.0 for k in range(K + 1))
        for k in range(K - 1):
            assert abs(real[k + 1] / real[k] - a_p ** (1 / (1 + r))) < 1e-12
    # largest remainder: the units left after flooring go to the largest fractions
    real = O.fanout_real(64, 7, 0.8, 1.0)
    F = O.fanout(64, 7, 0.8, 1.0)
    fl = np.floor(real).astype(int)
    got = set(np.flatnonzero(np.array(F) - fl))
    want = set(np.argsort(-(real - fl), kind="stable")[:64 - fl.sum()])
    assert got == want


def test_fanout_optimum():
    check_fanout()


# ---------------------------------------------------------------------------
# O9 / hit: lookup against rank counting; P(hit) and E[tokens] against Monte Carlo
# ---------------------------------------------------------------------------
def check_hit_montecarlo(n=1500, seed=7):
    rng = np.random.default_rng(seed)
    V, K, tau, C = 24, 3, 0.8, 0.4
    F = O.fanout(12, K, 0.7, 1.0)
    zt = (rng.standard_normal((K + 1, V)) * 1.5).astype(np.float32)
    zd = (zt + rng.standard_normal((K + 1, V)).astype(np.float32) * 0.7).astype(np.float32)
    ex = O.p_hit_row(zt, zd, tau, F, C)
    cache = O.build_cache(zd[None], tau, F, C)
    sigma = {"F": F, "C": C}
    hits, emitted = [], []
    for i in range(n):
        toks = [O.sample_draft(zd[k], tau, rng.random(), F[k], C) for k in range(K)]
        r = O.verify_row(zt, zd, toks, rng.random(K), rng.random(), tau, sigma)
        h, s = O.cache_lookup(cache["cache_tokens"], F, np.array([r["a"]]), r["out"][None])
        # cross-check by rank: hit iff fewer than F_a tokens beat t* on draft row a
        a, t = r["a"], r["out"][r["a"]]
        za = O.as_f64(zd[a])
        rank = int(np.sum((za > za[t]) | ((za == za[t]) & (np.arange(V) < t))))
        assert bool(h[0]) == (rank < F[a])
        if h[0]:
            assert s[0] == rank
        hits.append(h[0])
        emitted.append(r["a"] + 1)
    hits, emitted = np.array(hits, float), np.array(emitted, float)
    se_h = math.sqrt(ex["p_hit"] * (1 - ex["p_hit"]) / n)
    assert abs(hits.mean() - ex["p_hit"]) < 4 * se_h + 1e-9
    se_e = emitted.std() / math.sqrt(n)
    assert abs(emitted.mean() - ex["e_tokens"]) < 4 * se_e


def test_hit_rate_montecarlo():
    check_hit_montecarlo()


# ---------------------------------------------------------------------------
# degenerate cases
# ---------------------------------------------------------------------------
def test_inverse_cdf_edges():
    r = np.array([0.0, 0.0, 0.3, 0.0, 0.7, 0.0])
    assert O.inverse_cdf(r, 0.0)[0] == 2            # u = 0 gives the first positive token
    assert O.inverse_cdf(r, 0.9999999)[0] == 4
    for u in np.linspace(0, 0.999, 101):
        t = O.inverse_cdf(r, u)[0]
        assert r[t] > 0
        assert t == (2 if u * 1.0 < 0.3 else 4)
    assert O.inverse_cdf(np.zeros(4), 0.5)[0] == -1


def test_draft_sample_distribution():
    # Drafts over a stratified grid of u reproduce q (plain) and q_sigma: the
    # sigma form written out by hand here (top-2 by logit get weight C).
    z = np.log(np.array([[0.30, 0.05, 0.25, 0.10, 0.20, 0.10]], dtype=np.float64)).astype(np.float32)
    draft = np.broadcast_to(z, (1, 1, 6))
    N = 20000
    u = ((np.arange(N) + 0.5) / N).reshape(N, 1)
    for F, C in ((None, 1.0), ([2], 0.3), ([2], 0.0), ([6], 0.5)):
        toks, _ = O.draft_sample(np.broadcast_to(draft, (N, 1, 6)), 1.0, u, F, C)
        hist = np.bincount(toks[:, 0], minlength=6) / N
        w = np.exp(z[0].astype(np.float64))
        if F is not None:
            w[[0, 2]] *= C if F[0] == 2 else 1.0
            if F[0] == 6:
                w = w * C
        q = w / w.sum()
        assert np.max(np.abs(hist - q)) <= 1.0 / N + 1e-12, (F, C, hist, q)
    toks, _ = O.draft_sample(np.full((1, 1, 4), -np.inf, dtype=np.float32), 1.0, np.array([[0.5]]))
    assert toks[0, 0] == -1


def test_greedy_is_the_zero_temperature_limit():
    # With well separated target logits, sampling verification at a tiny
    # temperature has one-hot p: it keeps d iff d is the argmax, and the
    # residual max(0, p - q) (or p_K) puts all mass on the argmax. So the
    # sampling oracle at tau -> 0 must reproduce greedy verification.
    rng = np.random.default_rng(7)
    B, K, V = 40, 4, 12
    target = rng.permuted(np.tile(np.arange(V, dtype=np.float32) * 3.0, (B, K + 1, 1)), axis=2)
    draft = (target[:, :K] + rng.standard_normal((B, K, V)).astype(np.float32)).astype(np.float32)
    g = np.argmax(target, axis=2)
    tokens = np.where(rng.random((B, K)) < 0.7, g[:, :K], rng.integers(0, V, (B, K))).astype(np.int32)
    gr = O.verify_greedy(target, tokens)
    sm = O.verify(target, draft, tokens, rng.random((B, K)).astype(np.float32),
                  rng.random(B).astype(np.float32), 1e-3)
    assert np.array_equal(gr["accepted"], sm["accepted"])
    assert np.array_equal(gr["out_tokens"], sm["out_tokens"])
    # the argmax order and the degenerate rows
    assert O.argmax_token(np.array([1.0, 3.0, 3.0, 2.0], dtype=np.float32)) == 1
    assert O.argmax_token(np.full(5, -np.inf, dtype=np.float32)) == -1
    t = np.zeros((1, 3, 4), dtype=np.float32)
    t[0, :, 2] = 1.0
    r = O.verify_greedy(t, np.array([[2, 0]], dtype=np.int32))
    assert r["accepted"][0] == 1 and list(r["out_tokens"][0]) == [2, 2, -1]
    r = O.verify_greedy(t, np.array([[2, 2]], dtype=np.int32))
    assert r["accepted"][0] == 2 and list(r["out_tokens"][0]) == [2, 2, 2]
    r = O.verify_greedy(t, np.array([[2, 9]], dtype=np.int32))
    assert r["accepted"][0] == -1 and list(r["out_tokens"][0]) == [-1, -1, -1]


def test_cache_policy_helpers():
    # uniform shape: sums to the budget, differs by at most one, extra units first
    for n, K in ((64, 7), (128, 8), (5, 3), (0, 4), (9, 8)):
        F = O.fanout_uniform(n, K)
        assert sum(F) == n and max(F) - min(F) <= 1 and F == sorted(F, reverse=True)
    assert O.fanout_uniform(10, 3) == [3, 3, 2, 2]
    # speedup: all hits with a primary no slower than the verifier give E_hit;
    # all misses give E_miss / (1 + T_b); batch 1 is the single-sequence form;
    # a large batch almost never has every sequence hit
    assert O.ssd_speedup(1.0, 4.0, 1.5, 0.5, 0.2) == 4.0
    assert O.ssd_speedup(1.0, 4.0, 1.5, 2.0, 0.2) == 2.0
    assert abs(O.ssd_speedup(0.0, 4.0, 1.5, 0.5, 0.2) - 1.5 / 1.2) < 1e-15
    p, Eh, Em, Tp, Tb = 0.8, 3.6, 1.9, 0.7, 0.1
    single = (p * Eh + (1 - p) * Em) / (p * 1.0 + (1 - p) * (1 + Tb))
    assert abs(O.ssd_speedup(p, Eh, Em, Tp, Tb, 1) - single) < 1e-15
    big = O.ssd_speedup(p, Eh, Em, Tp, Tb, 200)
    assert abs(big - (p * Eh + (1 - p) * Em) / (1 + Tb)) < 1e-12
    assert O.ssd_speedup(p, Eh, Em, Tp, Tb, 2) < single
    # per-length counts on a hand example
    acc = np.array([0, 2, 2, -1, 3, 2, 0])
    hit = np.array([1, 0, 1, 1, 1, 1, 0], dtype=np.uint8)
    assert O.cache_stats(acc, hit, 3).tolist() == [[2, 1], [0, 0], [3, 2], [1, 1]]


def test_zero_residual_falls_back_to_p():
    # identical target and draft rows, drafted token masked in both: p = q = 0 -> reject,
    # the residual is empty, the draw comes from p of that row
    z = np.array([0.0, 1.0, -np.inf, 0.5], dtype=np.float32)
    tgt = np.stack([z, z])
    r = O.verify_row(tgt, z[None], [2], [0.0], 0.99, 1.0)
    assert r["a"] == 0 and r["fallback"] and r["Z"] == 0.0
    assert r["out"][0] == O.inverse_cdf(O.softmax(z, 1.0), 0.99)[0]


def test_bad_token_flags_row():
    z = np.zeros((3, 4), dtype=np.float32)
    r = O.verify_row(z, z, [1, 4], [0.1, 0.1], 0.5, 1.0)
    assert r["a"] == -1 and list(r["out"]) == [-1, -1, -1]
    hit, slot = O.cache_lookup(np.zeros((1, 2), dtype=np.int64), [1, 1], np.array([-1]),
                               np.array([[-1, -1]]))
    assert hit[0] == 0 and slot[0] == -1


# ---------------------------------------------------------------------------
# planted mistakes: each pin must fail when the oracle is wrong
# ---------------------------------------------------------------------------
def _expect_fail(check, *args):
    with pytest.raises(AssertionError):
        check(*args)


def test_planted_mistakes_are_caught(monkeypatch, golden_dir):
    # 1) accept test with the comparison reversed
    with monkeypatch.context() as m:
        def bad_scan(p_tok, q_tok, u):
            K = len(p_tok)
            for i in range(K):
                if not (u[i] * q_tok[i] > p_tok[i]):
                    return i, np.zeros(K)
            return K, np.zeros(K)
        m.setattr(OM, "accept_scan", bad_scan)
        _expect_fail(check_worked_example, golden_dir)
        _expect_fail(check_lossless, 400)
    # 2) residual with the operands swapped
    with monkeypatch.context() as m:
        orig = OM._residual
        m.setattr(OM, "_residual", lambda p, q, u: orig(q if q is not None else p,
                                                        p if q is not None else None, u))
        _expect_fail(check_worked_example, golden_dir)
        _expect_fail(check_lossless, 400)
    # 3) temperature multiplied instead of divided
    with monkeypatch.context() as m:
        orig_sm = OM.softmax
        m.setattr(OM, "softmax", lambda z, tau: orig_sm(z, 1.0 / tau))
        _expect_fail(check_lossless, 400)
    # 4) inverse CDF that can land on a zero-mass token (left-closed search)
    with monkeypatch.context() as m:
        def bad_icdf(r, u):
            cdf = np.cumsum(r)
            Z = float(cdf[-1])
            if not Z > 0:
                return -1, Z, math.inf
            return int(np.searchsorted(cdf, u * Z, side="left")), Z, 0.0
        m.setattr(OM, "inverse_cdf", bad_icdf)
        with pytest.raises(AssertionError):
            test_inverse_cdf_edges()
    # 5) fan-out exponent without the (1+r)
    with monkeypatch.context() as m:
        def bad_real(N, K, a_p, r):
            w = [a_p ** k for k in range(K)] + [a_p ** K / (1 - a_p)]
            return np.array([N / sum(w) * x for x in w])
        m.setattr(OM, "fanout_real", bad_real)
        _expect_fail(check_fanout)
    # 6) top-F ties broken by the larger index
    with monkeypatch.context() as m:
        def bad_top(z, F):
            zf = O.as_f64(z)
            return np.lexsort((-np.arange(zf.shape[0]), -zf))[:int(F)]
        m.setattr(OM, "top_f", bad_top)
        _expect_fail(check_top_f)
    # 7) sigma applied with 1/C instead of C
    with monkeypatch.context() as m:
        orig_dp = OM.draft_probs
        m.setattr(OM, "draft_probs", lambda z, tau, F=None, C=1.0:
                  orig_dp(z, tau, F, 1.0 / C if C > 0 else C))
        _expect_fail(check_sigma)
    # 8) bonus drawn from the last drafted position instead of the next one
    with monkeypatch.context() as m:
        orig_vr = OM.verify_row
        def bad_vr(target, draft, tokens, u_acc, u_res, tau, sigma=None):
            t2 = np.array(target, copy=True)
            t2[len(tokens)] = t2[len(tokens) - 1]
            return orig_vr(t2, draft, tokens, u_acc, u_res, tau, sigma)
        m.setattr(OM, "verify_row", bad_vr)
        _expect_fail(check_lossless, 400)


# ---------------------------------------------------------------------------
# token-tree verification
# ---------------------------------------------------------------------------
def _tree_logits(prob_rows):
    return _ln_rows(prob_rows)


def check_tree_hand_cases():
    """Small trees worked by hand from the one-candidate rule applied to each
    sibling in turn (temperature 1, logits ln(prob)).

    p = (0.5, 0.3, 0.2), q = (0.2, 0.2, 0.6) at the root; root children are
    nodes 1 and 2, both leaves. A token-2 child is kept iff 0.6 u < 0.2.
    After rejecting it the residual is (0.3, 0.1, 0)/0.4 = (0.75, 0.25, 0),
    where a token-1 child is kept iff 0.2 u < 0.25 (always) and a token-2
    child never; rejecting that as well leaves max(0, (0.75, 0.25, 0) - q) =
    (0.55, 0.05, 0), Z = 0.6, so the final draw is token 0 for u_res Z < 0.55
    and token 1 above.
    """
    p = [0.5, 0.3, 0.2]
    q = [0.2, 0.2, 0.6]
    leaf1 = [0.5, 0.5, 0.0]      # target after node 1 (bonus row)
    leaf2 = [0.1, 0.1, 0.8]      # target after node 2
    T = _tree_logits([p, leaf1, leaf2])
    D = _tree_logits([q, q, q])
    par = [-1, 0, 0]
    cases = [
        # tokens, u_acc, u_res, a, out, nodes
        ([0, 2, 1], [0, 0.5, 0.9], 0.3, 1, [1, 2, -1], [0, 2, -1]),   # reject, keep, bonus 2
        ([0, 2, 2], [0, 0.5, 0.2], 0.5, 0, [0, -1, -1], [0, -1, -1]),  # both rejected, 0.30 < 0.55
        ([0, 2, 2], [0, 0.5, 0.2], 0.95, 0, [1, -1, -1], [0, -1, -1]), # 0.57 in (0.55, 0.6]
        ([0, 2, 2], [0, 0.2, 0.2], 0.9, 1, [2, 1, -1], [0, 1, -1]),   # 0.12 < 0.2: keep node 1
    ]
    for toks, ua, ur, a, out, nodes in cases:
        r = O.verify_tree_row(T, D, par, toks, ua, ur, 1.0)
        assert r["a"] == a and list(r["out"]) == out and list(r["nodes"]) == nodes, (toks, ua, ur, r)
    r = O.verify_tree_row(T, D, par, [0, 2, 2], [0, 0.5, 0.2], 0.5, 1.0)
    assert abs(r["Z"] - 0.6) < 1e-6
    # empty residual: p = q = (1, 0); a token-1 child has p = q = 0 and is
    # rejected; max(0, p - q) = 0, so the draw uses p: token 0
    one = _tree_logits([[1.0, 0.0]] * 2)
    r = O.verify_tree_row(one, one, [-1, 0], [0, 1], [0, 0.3], 0.7, 1.0)
    assert r["a"] == 0 and list(r["out"]) == [0, -1]
    # root only: the bonus from p of the root, (0.5, 0.8, 1.0] -> token 1
    r = O.verify_tree_row(_tree_logits([p]), _tree_logits([q]), [-1], [0], [0.0], 0.6, 1.0)
    assert r["a"] == 0 and list(r["out"]) == [1]
    # a token outside [0, V) anywhere flags the row
    r = O.verify_tree_row(T, D, par, [0, 1, 3], [0, 0.1, 0.1], 0.5, 1.0)
    assert r["a"] == -1 and list(r["out"]) == [-1, -1, -1]


def test_tree_hand_cases():
    check_tree_hand_cases()


def check_tree_chain(n=150, seed=3):
    """A tree that is one chain is the single-path algorithm: same kept
    length and tokens as verify_row on the same rows and uniforms."""
    rng = np.random.default_rng(seed)
    for it in range(n):
        K = int(rng.integers(1, 6))
        V = int(rng.integers(2, 40))
        tau = float(rng.choice([0.5, 0.8, 1.3]))
        zt = (rng.standard_normal((K + 1, V)) * 1.5).astype(np.float32)
        zd = (zt + rng.standard_normal((K + 1, V)).astype(np.float32) * 0.7).astype(np.float32)
        toks = rng.integers(0, V, K)
        ua = rng.random(K)
        ur = float(rng.random())
        lin = O.verify_row(zt, zd[:K], toks, ua, ur, tau)
        par = [-1] + list(range(K))
        tr = O.verify_tree_row(zt, zd, par, [0] + list(toks), [0.0] + list(ua), ur, tau)
        assert tr["a"] == lin["a"], it
        assert list(tr["out"]) == list(lin["out"]), it
        assert list(tr["nodes"][:tr["a"] + 1]) == list(range(tr["a"] + 1))


def test_tree_chain_is_linear_verification():
    check_tree_chain()


def check_tree_lossless(T=12000, seed=11):
    """Siblings drawn independently from the draft: the first emitted token
    follows p of the root, and after a kept first token x the next emitted
    token follows p after x (chi-square at 1e-4, fixed seed). Rows depend on
    the token path only, as a model's would."""
    import scipy.stats
    rng = np.random.default_rng(seed)
    V = 4
    dirich = lambda: rng.dirichlet(np.full(V, 0.8))
    p0, q0 = dirich(), dirich()
    p1 = [dirich() for _ in range(V)]           # target after token x
    q1 = [dirich() for _ in range(V)]           # draft after token x
    p2 = [[dirich() for _ in range(V)] for _ in range(V)]
    lg = lambda v: _tree_logits([v])[0]
    # root with 3 children, each child with 2 children: N = 10
    par = [-1, 0, 0, 0, 1, 1, 2, 2, 3, 3]
    first = np.zeros(V)
    second = np.zeros((V, V))
    for _ in range(T):
        toks = [0] * 10
        for c in (1, 2, 3):
            toks[c] = int(rng.choice(V, p=q0))
        for c in range(4, 10):
            toks[c] = int(rng.choice(V, p=q1[toks[par[c]]]))
        tgt = np.zeros((10, V), dtype=np.float32)
        dft = np.zeros((10, V), dtype=np.float32)
        tgt[0], dft[0] = lg(p0), lg(q0)
        for c in range(1, 10):
            if par[c] == 0:
                tgt[c], dft[c] = lg(p1[toks[c]]), lg(q1[toks[c]])
            else:
                tgt[c], dft[c] = lg(p2[toks[par[c]]][toks[c]]), lg(q0)
        r = O.verify_tree_row(tgt, dft, par, toks, rng.random(10), float(rng.random()), 1.0)
        first[r["out"][0]] += 1
        if r["a"] >= 1:
            second[r["out"][0], r["out"][1]] += 1
    assert scipy.stats.chisquare(first, p0 * T).pvalue > 1e-4, (first / T, p0)
    for x in range(V):
        n = second[x].sum()
        if n >= 200:
            assert scipy.stats.chisquare(second[x], p1[x] * n).pvalue > 1e-4, (x, second[x] / n, p1[x])


def test_tree_lossless_montecarlo():
    check_tree_lossless()


def test_tree_planted_mistakes_are_caught(monkeypatch):
    # siblings all tested against p (no residual update between them)
    with monkeypatch.context() as m:
        m.setattr(OM, "_after_rejection", lambda P, q, p: (P, None))
        _expect_fail(check_tree_hand_cases)
        _expect_fail(check_tree_lossless, 6000)
    # residual left unnormalised
    with monkeypatch.context() as m:
        def unnorm(P, q, p):
            r = np.maximum(0.0, P - q)
            return (r, r) if r.sum() > 0 else (p, None)
        m.setattr(OM, "_after_rejection", unnorm)
        _expect_fail(check_tree_lossless, 6000)
    # residual taken from p of the node instead of the current distribution
    with monkeypatch.context() as m:
        def from_p(P, q, p):
            r = np.maximum(0.0, p - q)
            return (r / r.sum(), r) if r.sum() > 0 else (p, None)
        m.setattr(OM, "_after_rejection", from_p)
        _expect_fail(check_tree_hand_cases)
        _expect_fail(check_tree_lossless, 6000)

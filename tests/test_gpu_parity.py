"""GPU parity: the HIP library (through its C ABI) against the float64 oracle.

Integer outputs (accepted length, emitted tokens, cache tokens, hits, slots)
must match exactly, except batch rows whose deciding margin in the oracle is
below 1e-6 (counted and printed); probabilities within 1e-5 relative, row
log-sum-exps within 1e-5, residual mass within 1e-5 relative.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_utils import (EXCUSE, compare_cache, compare_hits, compare_verify, fvec, golden_inputs, ivec, log,
                       to_dev)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def S():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import verify_speculation_cache_amd as lib
    lib.lib()
    return lib


def _ln(rows):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(rows, dtype=np.float64)).astype(np.float32)


def _run_verify(S, d, sigma=None, oracle_sigma=None, rows=None, label=""):
    tgt, dft = to_dev(d["target"], torch), to_dev(d["draft"], torch)
    got = S.ssd_verify(tgt, dft, ivec(d["tokens"], torch), fvec(d["u_acc"], torch),
                       fvec(d["u_res"], torch), d["tau"], sigma)
    torch.cuda.synchronize()
    sel = list(range(d["tokens"].shape[0])) if rows is None else list(rows)
    ref = O.verify(d["target"][sel], d["draft"][sel], d["tokens"][sel], d["u_acc"][sel],
                   d["u_res"][sel], d["tau"], oracle_sigma)
    n_exc = compare_verify(ref, got, d["tokens"].shape[1], rows=sel, label=label)
    return got, ref, n_exc


# ---------------------------------------------------------------------------
# printed worked examples
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["worked_example_4token.json", "paris_example.json"])
def test_worked_examples(S, name):
    fx = json.load(open(os.path.join(GOLDEN, name)))
    log(f"[gpu] worked example {name}")
    for case in fx["cases"]:
        n = 16
        us = np.linspace(0.0, 0.999, n).astype(np.float32)
        d = {"target": np.broadcast_to(_ln(fx["p_rows"]), (n, fx["K"] + 1, fx["V"])).copy(),
             "draft": np.broadcast_to(_ln(fx["q_rows"]), (n, fx["K"], fx["V"])).copy(),
             "tokens": np.tile(np.array(fx["draft_tokens"], dtype=np.int32), (n, 1)),
             "u_acc": np.tile(np.array(case["u_acc"], dtype=np.float32), (n, 1)),
             "u_res": us, "tau": fx["tau"]}
        got, ref, _ = _run_verify(S, d, label=name)
        acc = got["accepted"].cpu().numpy()
        out = got["out_tokens"].cpu().numpy()
        if "expect_accepted" in case:
            assert np.all(acc == case["expect_accepted"])
            assert np.all(out == np.array(case["expect_out"]))
        else:
            assert np.all(acc >= case["expect_accepted_at_least"])


# ---------------------------------------------------------------------------
# small sizes the oracle finishes quickly, spanning several chunks with a ragged tail
# ---------------------------------------------------------------------------
def _random_case(seed, B, K, V, dtype, tau, mask_frac=0.0, draft_sd=0.7, Kd=None):
    rng = np.random.default_rng(seed)
    Kd = K if Kd is None else Kd
    t = (rng.standard_normal((B, K + 1, V)) * 2.5).astype(np.float32)
    d = (t[:, :Kd] + rng.standard_normal((B, Kd, V)).astype(np.float32) * draft_sd).astype(np.float32)
    if mask_frac > 0:
        t[rng.random(t.shape) < mask_frac] = -np.inf
        d[rng.random(d.shape) < mask_frac] = -np.inf
    if dtype == "bf16":
        t, d = W.f32_to_bf16_bits(t), W.f32_to_bf16_bits(d)
    toks = np.zeros((B, K), dtype=np.int32)
    for b in range(B):
        for i in range(K):
            toks[b, i] = O.sample_draft(d[b, i], tau, rng.random())
    return {"target": t, "draft": d, "tokens": toks,
            "u_acc": rng.random((B, K)).astype(np.float32),
            "u_res": rng.random(B).astype(np.float32), "tau": float(np.float32(tau))}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V,K,B", [(20000, 4, 6), (8192, 3, 4), (16385, 2, 3), (1000, 5, 8),
                                   (61, 6, 5), (7, 1, 9), (1, 2, 3)])
def test_verify_small(S, dtype, V, K, B):
    log(f"[gpu] verify small dtype={dtype} V={V} K={K} B={B}")
    d = _random_case(V * 7 + K, B, K, V, dtype, 0.8)
    _run_verify(S, d, label=f"small-{dtype}-{V}")


def test_verify_masked_and_unaligned(S):
    # masked tokens and an odd V (rows not 16-byte aligned -> scalar loads)
    for V, dtype in ((12347, "bf16"), (9001, "f32"), (33, "bf16")):
        log(f"[gpu] masked V={V} {dtype}")
        d = _random_case(V, 5, 3, V, dtype, 0.6, mask_frac=0.3)
        _run_verify(S, d, label=f"mask-{V}")


def test_verify_extremes(S):
    # K = 64 (largest), identical target/draft (everything accepted), tau extremes
    log("[gpu] K=64")
    d = _random_case(1, 2, 64, 3000, "bf16", 1.0, draft_sd=0.05)
    _run_verify(S, d, label="K64")
    for tau in (0.05, 5.0):
        log(f"[gpu] tau={tau}")
        d = _random_case(2, 4, 3, 5000, "f32", tau)
        _run_verify(S, d, label=f"tau{tau}")
    log("[gpu] identical rows")
    d = _random_case(3, 4, 4, 4000, "bf16", 0.7, draft_sd=0.0)
    got, _, _ = _run_verify(S, d, label="identical")
    assert np.all(got["accepted"].cpu().numpy() == 4)


def test_verify_flagged_tokens(S):
    log("[gpu] out-of-range drafted tokens")
    d = _random_case(4, 6, 3, 2000, "bf16", 1.0)
    d["tokens"][1, 2] = 2000
    d["tokens"][3, 0] = -5
    got, _, _ = _run_verify(S, d, label="flagged")
    acc = got["accepted"].cpu().numpy()
    out = got["out_tokens"].cpu().numpy()
    assert acc[1] == -1 and acc[3] == -1 and np.all(out[1] == -1) and np.all(out[3] == -1)
    assert np.all(acc[[0, 2, 4, 5]] >= 0)


def test_fully_masked_rows(S):
    # a target row with no mass: p = 0 there, so its drafted token is rejected and
    # the residual (from p = 0) is empty -> token -1
    log("[gpu] fully masked target row")
    d = _random_case(5, 3, 2, 3000, "f32", 1.0)
    d["target"][1, 0, :] = -np.inf
    got, _, _ = _run_verify(S, d, label="fullmask")
    assert got["accepted"].cpu().numpy()[1] == 0
    assert got["out_tokens"].cpu().numpy()[1, 0] == -1


def test_determinism(S):
    log("[gpu] determinism")
    d = _random_case(6, 8, 4, 30000, "bf16", 0.7)
    tgt, dft = to_dev(d["target"], torch), to_dev(d["draft"], torch)
    args = (ivec(d["tokens"], torch), fvec(d["u_acc"], torch), fvec(d["u_res"], torch), d["tau"])
    r1 = S.ssd_verify(tgt, dft, *args)
    o1 = {k: v.clone() for k, v in r1.items() if v is not None}
    # another shape in between (its own workspace)
    d2 = _random_case(7, 3, 2, 500, "bf16", 0.7)
    S.ssd_verify(to_dev(d2["target"], torch), to_dev(d2["draft"], torch), ivec(d2["tokens"], torch),
                 fvec(d2["u_acc"], torch), fvec(d2["u_res"], torch), d2["tau"])
    r2 = S.ssd_verify(tgt, dft, *args)
    torch.cuda.synchronize()
    for k, v in o1.items():
        assert torch.equal(v, r2[k]), k


def test_verify_large_draw_scan_once(S):
    # 128 batch rows x 16 spans of 16384 entries = 2048 residual workgroups:
    # the accept scan runs once per batch row in a launch of its own and the
    # draw reads its result; every output (probs, Z, log-normalisers) of every
    # row against the oracle, with two flagged rows and a fully masked target
    # row among them
    B, K, V = 128, 2, 262144
    log(f"[gpu] verify large draw B={B} K={K} V={V} bf16")
    d = _random_case(11, B, K, V, "bf16", 0.8)
    d["tokens"][5, 1] = V
    d["tokens"][77, 0] = -1
    d["target"][9, 0, :] = W.f32_to_bf16_bits(np.full(V, -np.inf, dtype=np.float32))
    got, _, _ = _run_verify(S, d, label="large-draw")
    acc = got["accepted"].cpu().numpy()
    out = got["out_tokens"].cpu().numpy()
    assert acc[5] == -1 and acc[77] == -1 and np.all(out[[5, 77]] == -1)
    assert acc[9] == 0 and out[9, 0] == -1


def test_verify_large_draw_scan_once_sigma(S):
    # the same 2048-workgroup draw with sigma: cache build, sigma verification
    # and lookup against the oracle on every row
    B, K, V = 128, 2, 262144
    log(f"[gpu] sigma verify large draw B={B} K={K} V={V} bf16")
    d = _random_case(12, B, K, V, "bf16", 0.8, Kd=K + 1)
    _cache_case(S, d, [6, 5, 9], 0.5, label="large-draw-sigma")


# ---------------------------------------------------------------------------
# residual sampling entry point
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_residual_sample(S, dtype):
    log(f"[gpu] residual_sample {dtype}")
    d = _random_case(8, 10, 3, 17000, dtype, 0.9)
    rows = np.array([0, 1, 2, 3, 0, 1, 2, 3, 1, 0], dtype=np.int32)
    u = np.random.default_rng(1).random(10).astype(np.float32)
    tgt, dft = to_dev(d["target"], torch), to_dev(d["draft"], torch)
    for use_draft in (True, False):
        got = S.ssd_residual_sample(tgt, dft if use_draft else None, ivec(rows, torch), fvec(u, torch),
                                    d["tau"])
        torch.cuda.synchronize()
        ref = O.residual_sample(d["target"], d["draft"] if use_draft else None, rows, u, d["tau"])
        tg = got["tokens"].cpu().numpy()
        mg = got["mass"].cpu().numpy()
        for b in range(10):
            if tg[b] != ref["tokens"][b]:
                assert ref["margin"][b] < 1e-6, (b, tg[b], ref["tokens"][b], ref["margin"][b])
            if ref["Z"][b] >= 1e-2:
                assert abs(mg[b] - ref["Z"][b]) <= 1e-5 * ref["Z"][b]


# ---------------------------------------------------------------------------
# cache build, sigma verify and lookup
# ---------------------------------------------------------------------------
def _check_cache(cache, ref, F, rows, label):
    compare_cache(cache, ref, F, rows, label)


def _cache_case(S, d, F, C, rows=None, label=""):
    K = d["tokens"].shape[1]
    sel = list(range(d["tokens"].shape[0])) if rows is None else list(rows)
    dft = to_dev(d["draft"], torch)
    cache = S.ssd_build_cache(dft, d["tau"], F)
    torch.cuda.synchronize()
    ref = O.build_cache(d["draft"][sel], d["tau"], F, C)
    _check_cache(cache, ref, F, sel, label)
    sigma = S.sigma_from_cache(cache, C)
    got, vref, n_exc = _run_verify(S, d, sigma, {"F": F, "C": C}, rows=sel, label=label)
    look = S.ssd_cache_lookup(cache["cache_tokens"], F, got["accepted"], got["out_tokens"])
    torch.cuda.synchronize()
    hg = look["hit"].cpu().numpy()
    sg = look["slot"].cpu().numpy()
    acc_g = got["accepted"].cpu().numpy()
    out_g = got["out_tokens"].cpu().numpy()
    hit_r, _ = O.cache_lookup(ref["cache_tokens"], F, vref["accepted"], vref["out_tokens"])
    vref = dict(vref, hit=hit_r)
    compare_hits(hg[sel], sg[sel], ref["cache_tokens"], F, acc_g[sel], out_g[sel], vref, label)
    return cache, got, hg


def test_cache_small(S):
    for (V, K, B, dtype, N, C) in ((20000, 3, 5, "bf16", 40, 0.5), (9000, 2, 4, "f32", 30, 0.0),
                                   (300, 4, 6, "bf16", 64, 1.0), (70, 2, 3, "bf16", 9, 0.3)):
        log(f"[gpu] cache small V={V} K={K} B={B} {dtype} N={N} C={C}")
        F = S.ssd_fanout(N, K, 0.75, 1.0)
        F = [min(f, 64, V) for f in F]
        d = _random_case(V + K, B, K, V, dtype, 0.7, Kd=K + 1)
        _cache_case(S, d, F, C, label=f"cache-{V}")


def test_cache_ties_and_limits(S):
    # all-equal rows (every token ties), F_k = 0 and F_k = 64 segments
    log("[gpu] cache ties")
    B, K, V = 3, 3, 20000
    d = _random_case(11, B, K, V, "bf16", 1.0, Kd=K + 1)
    d["draft"][0, :, :] = W.f32_to_bf16_bits(np.full((K + 1, V), 0.5, dtype=np.float32))
    d["draft"][1, 1, ::2] = W.f32_to_bf16_bits(np.full(V // 2, 3.0, dtype=np.float32))
    F = [64, 0, 17, 64]
    _cache_case(S, d, F, 0.4, label="ties")
    log("[gpu] cache f32 ties")
    d = _random_case(12, B, K, 5000, "f32", 1.0, Kd=K + 1)
    d["draft"][2] = np.round(d["draft"][2])
    _cache_case(S, d, [5, 64, 1, 33], 0.2, label="ties-f32")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_cache_masked_full_chunks(S, dtype):
    """Full 8192-entry chunks whose lanes are mostly or wholly masked: the
    chunk bound must stay valid with -inf lane maxima (rows with 99 % of
    the tokens masked, a wholly masked first chunk, a chunk with two finite
    tokens, and negative-only and positive-only rows)."""
    log(f"[gpu] cache masked full chunks {dtype}")
    B, K, V = 6, 3, 3 * 8192 + 77
    rng = np.random.default_rng(4242)
    d = _random_case(4243, B, K, V, "f32", 0.9, Kd=K + 1)
    dr = d["draft"]
    dr[0][rng.random((K + 1, V)) < 0.99] = -np.inf
    dr[1, :, :8192] = -np.inf
    dr[2, :, 8192:16384] = -np.inf
    dr[2, :, 8192 + 5] = 1.5
    dr[2, :, 8192 + 4000] = -7.25
    dr[3] = -np.abs(dr[3]) - 1.0
    dr[4] = np.abs(dr[4]) + 1.0
    dr[5][rng.random((K + 1, V)) < 0.5] = -np.inf
    if dtype == "bf16":
        d["target"], d["draft"] = W.f32_to_bf16_bits(d["target"]), W.f32_to_bf16_bits(dr)
    for b in range(B):   # drafts from the masked rows (token 0 for a row without mass)
        for i in range(K):
            d["tokens"][b, i] = max(O.sample_draft(d["draft"][b, i], d["tau"], rng.random()), 0)
    _cache_case(S, d, [64, 13, 1, 0], 0.3, label=f"masked-{dtype}")


@pytest.mark.parametrize("K,F", [(64, [5] * 65), (4, [64] * 5), (3, [0, 10, 0, 64]), (1, [1, 0])])
def test_cache_lookup_direct(S, K, F):
    """Lookup against the oracle on synthetic caches: rows whose cache holds
    more than 256 tokens, K = 64 (outcome at position 64), empty segments,
    flagged rows and misses."""
    log(f"[gpu] lookup K={K} sumF={sum(F)}")
    rng = np.random.default_rng(1000 + K)
    B, V = 97, 50000
    off = np.concatenate([[0], np.cumsum(F)])
    cache = np.full((B, sum(F)), -1, dtype=np.int32)
    for b in range(B):
        for k in range(K + 1):
            cache[b, off[k]:off[k + 1]] = rng.choice(V, size=F[k], replace=False)
    acc = rng.integers(-1, K + 1, size=B).astype(np.int32)
    acc[:3] = K
    out = rng.integers(0, V, size=(B, K + 1)).astype(np.int32)
    for b in range(B):
        a = int(acc[b])
        if a >= 0 and F[a] > 0 and b % 2 == 0:
            out[b, a] = cache[b, off[a] + rng.integers(0, F[a])]
        if b % 7 == 3 and a >= 0:
            out[b, a] = -1
    got = S.ssd_cache_lookup(torch.from_numpy(cache).cuda(), F, torch.from_numpy(acc).cuda(),
                             torch.from_numpy(out).cuda())
    torch.cuda.synchronize()
    hit_r, slot_r = O.cache_lookup(cache, F, acc, out)
    assert np.array_equal(got["hit"].cpu().numpy(), hit_r)
    assert np.array_equal(got["slot"].cpu().numpy().astype(np.int64), slot_r)
    assert hit_r.sum() >= 10   # the case exercises hits, not only misses


# ---------------------------------------------------------------------------
# the five workloads at full size
# ---------------------------------------------------------------------------
def test_workload_B1_K4_V32000_f32(S):
    cfg = W.get_config(1)
    log(f"[gpu] {cfg.name}")
    d = W.make_inputs(cfg)
    _run_verify(S, d, label=cfg.name)
    # many uniform draws on the same logits (batch stride 0 broadcast)
    n = 256
    ua = np.random.default_rng(5).random((n, cfg.K)).astype(np.float32)
    ur = np.random.default_rng(6).random(n).astype(np.float32)
    tgt = to_dev(d["target"], torch).expand(n, -1, -1)
    dft = to_dev(d["draft"], torch).expand(n, -1, -1)
    toks = np.tile(d["tokens"], (n, 1))
    got = S.ssd_verify(tgt, dft, ivec(toks, torch), fvec(ua, torch), fvec(ur, torch), d["tau"])
    torch.cuda.synchronize()
    ref = O.verify(np.broadcast_to(d["target"], (n,) + d["target"].shape[1:]),
                   np.broadcast_to(d["draft"], (n,) + d["draft"].shape[1:]), toks, ua, ur, d["tau"])
    compare_verify(ref, got, cfg.K, label="B1-broadcast")


def test_workload_B64_K5_V128256(S):
    cfg = W.get_config(2)
    log(f"[gpu] {cfg.name}")
    d = W.make_inputs(cfg)
    _run_verify(S, d, label=cfg.name)


def _golden_step(S, name, label):
    """Every batch row of a cache workload, against the oracle's stored
    outputs: the separate calls (ssd_build_cache, ssd_verify with sigma,
    ssd_cache_lookup), the fused ssd_verify_round, and the GPU's own sigma
    drafts (ssd_draft_sample) against the oracle's draws that the golden
    verification used."""
    cfg, d, g = golden_inputs(name)
    K, tau, F, C = cfg.K, d["tau"], g["F"], g["C"]
    assert F == S.ssd_fanout(cfg.n_budget, K, cfg.a_p, cfg.r)
    rows = list(range(cfg.B))
    tgt, dft = to_dev(d["target"], torch), to_dev(d["draft"][:, :K + 1], torch)
    toks, ua, ur = ivec(d["tokens"], torch), fvec(d["u_acc"], torch), fvec(d["u_res"], torch)

    cache = S.ssd_build_cache(dft, tau, F)
    sg = S.sigma_from_cache(cache, C)
    sep = S.ssd_verify(tgt, dft, toks, ua, ur, tau, sg)
    look = S.ssd_cache_lookup(cache["cache_tokens"], F, sep["accepted"], sep["out_tokens"])
    torch.cuda.synchronize()
    compare_cache(cache, g, F, rows, label + " build")
    n_sep = compare_verify(g, sep, K, label=label + " verify")
    acc, out = sep["accepted"].cpu().numpy(), sep["out_tokens"].cpu().numpy()
    compare_hits(look["hit"].cpu().numpy(), look["slot"].cpu().numpy(), g["cache_tokens"], F, acc, out, g,
                 label + " lookup")

    rnd = S.ssd_verify_round(tgt, dft, F, C, toks, ua, ur, tau)
    torch.cuda.synchronize()
    compare_cache(rnd, g, F, rows, label + " round cache")
    n_rnd = compare_verify(g, rnd, K, check_lse=False, label=label + " round")
    acc, out = rnd["accepted"].cpu().numpy(), rnd["out_tokens"].cpu().numpy()
    compare_hits(rnd["hit"].cpu().numpy(), rnd["slot"].cpu().numpy(), g["cache_tokens"], F, acc, out, g,
                 label + " round lookup")

    u_draft = W.make_draft_uniforms(cfg, tau)
    drafts = S.ssd_draft_sample(dft, fvec(u_draft, torch), tau, sg).cpu().numpy()
    bad = (drafts != g["tokens"]) & ~(g["draft_margin"] < EXCUSE)
    assert not bad.any(), (label, np.argwhere(bad))
    hits = rnd["hit"].cpu().numpy()
    log(f"[gpu] {label}: {cfg.B} rows, excused verify {n_sep} round {n_rnd}, "
        f"draft ties {int((drafts != g['tokens']).sum())}, mean a+1 {np.mean(acc + 1):.4f}, hit rate {hits.mean():.4f}")
    return rnd


def test_step_B64_K5_V128256_all_rows(S):
    """The measured step (cache on draft rows 0..5 with budget 64, a_p 0.8,
    r 1, C 0.5; verification against q_sigma; lookup) on every batch row."""
    log("[gpu] step B=64 K=5 V=128256 (golden)")
    rnd = _golden_step(S, "step_B64_K5_V128256_bf16", "B64-step")
    assert [int(x) for x in S.ssd_fanout(64, 5, 0.8, 1.0)] == [12, 11, 10, 8, 8, 15]
    assert rnd["cache_tokens"].shape[1] == 64


def test_workload_B32_K7_cache(S):
    cfg = W.get_config(3)
    log(f"[gpu] {cfg.name}")
    d = W.make_inputs(cfg)
    F = S.ssd_fanout(cfg.n_budget, cfg.K, cfg.a_p, cfg.r)
    assert F == [10, 9, 8, 8, 7, 6, 5, 11]
    _, _, hits = _cache_case(S, d, F, cfg.C, label=cfg.name)
    log(f"[gpu] B=32 cache hit rate {hits.mean():.3f} (softmax drafts)")
    _run_verify(S, d, label=cfg.name + "-plain")
    _golden_step(S, "cache_B32_K7_V128256_bf16", "B32-cache-sigma-drafts")


def test_workload_B512_K4_V151936(S):
    log("[gpu] verify B=512 K=4 V=151936 (golden, every row)")
    cfg, d, g = golden_inputs("verify_B512_K4_V151936_bf16")
    got = S.ssd_verify(to_dev(d["target"], torch), to_dev(d["draft"], torch), ivec(d["tokens"], torch),
                       fvec(d["u_acc"], torch), fvec(d["u_res"], torch), d["tau"])
    torch.cuda.synchronize()
    n = compare_verify(g, got, cfg.K, label=cfg.name)
    log(f"[gpu] {cfg.name}: {cfg.B} rows, {n} excused")


@pytest.mark.parametrize("tau", [0.5, 1.0])
def test_workload_B256_K8_cache(S, tau):
    log(f"[gpu] cache B=256 K=8 V=256000 tau={tau} (golden, every row)")
    rnd = _golden_step(S, f"cache_B256_K8_V256000_bf16_tau{tau}", f"B256-{tau}")
    assert rnd["cache_tokens"].shape[1] == 128


# ---------------------------------------------------------------------------
# the draft phase on the GPU (sigma-aware drafting)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V,K,B,sig", [(20000, 3, 5, True), (20000, 3, 5, False), (16385, 2, 3, True),
                                       (300, 4, 6, True), (8192, 2, 4, False), (7, 2, 4, False),
                                       (70000, 2, 3, True)])
def test_draft_sample(S, dtype, V, K, B, sig):
    log(f"[gpu] draft sample V={V} K={K} B={B} {dtype} sigma={sig}")
    d = _random_case(V + 3 * K + B, B, K, V, dtype, 0.7, Kd=K + 1)
    rng = np.random.default_rng(V + K)
    u = rng.random((B, K)).astype(np.float32)
    u[0, 0] = 0.0
    u[-1, -1] = np.float32(0.99999994)
    draft = to_dev(d["draft"], torch)
    C = 0.3 if sig else 1.0
    F = [min(f, 64, V) for f in S.ssd_fanout(40, K, 0.75, 1.0)] if sig else None
    sg = S.sigma_from_cache(S.ssd_build_cache(draft, d["tau"], F), C) if sig else None
    got = S.ssd_draft_sample(draft, fvec(u, torch), d["tau"], sg).cpu().numpy()
    ref, mg = O.draft_sample(d["draft"], d["tau"], u, F, C)
    bad = (got != ref) & ~(mg < EXCUSE)
    assert not bad.any(), (np.argwhere(bad), got[bad], ref[bad])
    log(f"[gpu] draft sample excused {int(((got != ref) & (mg < EXCUSE)).sum())}")


def test_draft_sample_masked_rows(S):
    log("[gpu] draft sample masked rows")
    B, K, V = 3, 2, 9000
    d = _random_case(5, B, K, V, "bf16", 1.0, Kd=K)
    dd = W.bf16_bits_to_f32(d["draft"])
    dd[0, 0, :] = -np.inf               # no mass: draws -1
    dd[1, 1, ::3] = -np.inf             # masked tokens are never drawn
    dd[2, 0, :-1] = -np.inf             # only the last token has mass
    d["draft"] = W.f32_to_bf16_bits(dd)
    u = np.array([[0.5, 0.0], [0.3, 0.7], [0.9, 0.1]], dtype=np.float32)
    got = S.ssd_draft_sample(to_dev(d["draft"], torch), fvec(u, torch), 1.0).cpu().numpy()
    ref, mg = O.draft_sample(d["draft"], 1.0, u)
    assert got[0, 0] == -1 and got[2, 0] == V - 1 and got[1, 1] % 3 != 0
    assert np.array_equal(got[mg >= EXCUSE], ref[mg >= EXCUSE])


@pytest.mark.slow
@pytest.mark.parametrize("tau", [0.5, 1.0])
def test_B256_K8_expected_tokens_and_hits(S, tau):
    """Config 5's statistical checks: the empirical mean of (accepted + 1)
    and the empirical cache-hit rate over many uniform draws (drafts sampled
    on the GPU from q_sigma, verified against q_sigma) fall within 4 standard
    errors of the exact expectations mean_b E_b[tokens] and mean_b P_b(hit)
    computed by the oracle; the closed form with the mean alpha is printed."""
    cfg = W.get_config(5)
    nb, reps, rounds = 32, 32, 16            # 32 rows x 32 copies x 16 rounds = 16384 samples
    log(f"[gpu] B=256 statistics tau={tau}: {nb} rows x {reps * rounds} draws")
    d = W.make_inputs(cfg, tau=tau, draw_tokens=False, b_rows=range(nb))
    F = S.ssd_fanout(cfg.n_budget, cfg.K, cfg.a_p, cfg.r)
    K, tau32 = cfg.K, d["tau"]
    ex = [O.p_hit_row(d["target"][b], d["draft"][b], tau32, F, cfg.C) for b in range(nb)]
    e_tok = float(np.mean([e["e_tokens"] for e in ex]))
    p_hit = float(np.mean([e["p_hit"] for e in ex]))
    abar = float(np.mean([np.mean(e["alphas"]) for e in ex]))
    closed = (1 - abar ** (K + 1)) / (1 - abar)
    tgt = to_dev(d["target"], torch).repeat(reps, 1, 1)
    dft = to_dev(d["draft"], torch).repeat(reps, 1, 1)
    B = nb * reps
    cache = S.ssd_build_cache(dft, tau32, F)
    sg = S.sigma_from_cache(cache, cfg.C)
    rng = np.random.default_rng(4000 + int(tau * 10))
    lens, hits = [], []
    for _ in range(rounds):
        toks = S.ssd_draft_sample(dft, fvec(rng.random((B, K)), torch), tau32, sg)
        res = S.ssd_verify(tgt, dft, toks, fvec(rng.random((B, K)), torch), fvec(rng.random(B), torch),
                           tau32, sg)
        look = S.ssd_cache_lookup(cache["cache_tokens"], F, res["accepted"], res["out_tokens"])
        lens.append(res["accepted"].cpu().numpy() + 1)
        hits.append(look["hit"].cpu().numpy())
    lens = np.concatenate(lens).astype(np.float64)
    hits = np.concatenate(hits).astype(np.float64)
    assert lens.min() >= 1
    se_t = lens.std(ddof=1) / math.sqrt(lens.size)
    se_h = math.sqrt(max(p_hit * (1 - p_hit), 1e-12) / hits.size)
    log(f"[gpu] B=256 tau={tau}: mean tokens {lens.mean():.4f} vs exact {e_tok:.4f} (4 SE {4 * se_t:.4f}); "
        f"closed form with mean alpha {abar:.4f}: {closed:.4f}; hit rate {hits.mean():.4f} vs exact "
        f"{p_hit:.4f} (4 SE {4 * se_h:.4f})")
    assert abs(lens.mean() - e_tok) <= 4 * se_t
    assert abs(hits.mean() - p_hit) <= 4 * se_h


# ---------------------------------------------------------------------------
# greedy verification
# ---------------------------------------------------------------------------
def _greedy_case(seed, B, K, V, dtype, ties=False):
    rng = np.random.default_rng(seed)
    t = (rng.standard_normal((B, K + 1, V)) * 2.5).astype(np.float32)
    if ties:
        t = np.round(t).astype(np.float32)   # many equal maxima: the smaller index wins
    if dtype == "bf16":
        t = W.bf16_bits_to_f32(W.f32_to_bf16_bits(t))
    g = np.array([[O.argmax_token(t[b, i]) for i in range(K)] for b in range(B)], dtype=np.int32).reshape(B, K)
    toks = np.where(rng.random((B, K)) < 0.75, g, rng.integers(0, max(V, 1), (B, K))).astype(np.int32)
    tt = W.f32_to_bf16_bits(t) if dtype == "bf16" else t
    return tt, toks


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V,K,B,ties", [(20000, 4, 6, False), (20000, 4, 6, True), (16385, 2, 3, True),
                                        (40000, 3, 4, True), (7, 3, 5, True), (1, 2, 3, False),
                                        (100, 64, 2, True)])
def test_verify_greedy(S, dtype, V, K, B, ties):
    log(f"[gpu] greedy V={V} K={K} B={B} {dtype} ties={ties}")
    t, toks = _greedy_case(V + K + B, B, K, V, dtype, ties)
    if B >= 3 and V > 4:
        t[1, 0] = W.f32_to_bf16_bits(np.full(V, -np.inf, np.float32)) if dtype == "bf16" else -np.inf
        toks[2, K - 1] = V + 5                          # flagged row
    got = S.ssd_verify_greedy(to_dev(t, torch), ivec(toks, torch))
    torch.cuda.synchronize()
    ref = O.verify_greedy(t, toks)
    assert np.array_equal(got["accepted"].cpu().numpy(), ref["accepted"])
    assert np.array_equal(got["out_tokens"].cpu().numpy(), ref["out_tokens"])


def test_verify_greedy_B64_K5(S):
    cfg = W.get_config(2)
    log("[gpu] greedy B=64 K=5")
    d = W.make_inputs(cfg, draw_tokens=False)
    g = np.array([[O.argmax_token(d["target"][b, i]) for i in range(cfg.K)] for b in range(cfg.B)],
                 dtype=np.int32)
    rng = np.random.default_rng(22)
    toks = np.where(rng.random(g.shape) < 0.8, g, rng.integers(0, cfg.V, g.shape)).astype(np.int32)
    got = S.ssd_verify_greedy(to_dev(d["target"], torch), ivec(toks, torch))
    ref = O.verify_greedy(d["target"], toks)
    assert np.array_equal(got["accepted"].cpu().numpy(), ref["accepted"])
    assert np.array_equal(got["out_tokens"].cpu().numpy(), ref["out_tokens"])


# ---------------------------------------------------------------------------
# per-length cache statistics
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,K", [(1, 1), (97, 5), (5000, 8), (3, 64)])
def test_cache_stats(S, B, K):
    log(f"[gpu] cache stats B={B} K={K}")
    rng = np.random.default_rng(B + K)
    acc = rng.integers(-1, K + 1, size=B).astype(np.int32)
    hit = (rng.random(B) < 0.6).astype(np.uint8)
    got = S.ssd_cache_stats(torch.from_numpy(acc).cuda(), torch.from_numpy(hit).cuda(), K)
    assert np.array_equal(got.cpu().numpy().astype(np.int64), O.cache_stats(acc, hit, K))


def test_uniform_fanout_cache_hits(S):
    # the uniform shape drives the same cache build and lookup (B=32 cache workload)
    cfg = W.get_config(3)
    log("[gpu] uniform fan-out cache on the B=32 cache workload")
    F = S.ssd_fanout_uniform(cfg.n_budget, cfg.K)
    assert F == O.fanout_uniform(cfg.n_budget, cfg.K)
    d = W.make_inputs(cfg, b_rows=range(0, 32, 4))
    _cache_case(S, d, F, cfg.C, label="B32-uniform")


# ---------------------------------------------------------------------------
# the fused verification round: bit-identical to the separate calls
# ---------------------------------------------------------------------------
def _round_vs_separate(S, d, F, C, label, oracle_rows=True):
    """The fused round builds the cache bit-identically to ssd_build_cache (the
    same code) and its outcomes equal the oracle's on every row, except rows
    whose oracle margin at the first diverging decision is below EXCUSE; the
    separate calls are held to the same bar."""
    tgt, dft = to_dev(d["target"], torch), to_dev(d["draft"], torch)
    toks, ua, ur = ivec(d["tokens"], torch), fvec(d["u_acc"], torch), fvec(d["u_res"], torch)
    cache = S.ssd_build_cache(dft, d["tau"], F)
    sep = S.ssd_verify(tgt, dft, toks, ua, ur, d["tau"], S.sigma_from_cache(cache, C))
    look = S.ssd_cache_lookup(cache["cache_tokens"], F, sep["accepted"], sep["out_tokens"])
    rnd = S.ssd_verify_round(tgt, dft, F, C, toks, ua, ur, d["tau"])
    again = S.ssd_verify_round(tgt, dft, F, C, toks, ua, ur, d["tau"])   # workspace reused
    torch.cuda.synchronize()
    for k in ("cache_tokens", "thr", "draft_stats"):
        assert torch.equal(rnd[k], cache[k]), (label, k)
    for k in rnd:
        assert torch.equal(again[k], rnd[k]), (label, k, "second call")
    K = d["tokens"].shape[1]
    rows = list(range(d["tokens"].shape[0]))
    ref_c = O.build_cache(d["draft"], d["tau"], F, C)
    compare_cache(rnd, ref_c, F, rows, label + " cache")
    vref = O.verify(d["target"], d["draft"], d["tokens"], d["u_acc"], d["u_res"], d["tau"], {"F": list(F), "C": C})
    hit_r, _ = O.cache_lookup(ref_c["cache_tokens"], F, vref["accepted"], vref["out_tokens"])
    vref = dict(vref, hit=hit_r)
    for name, got, hs in (("round", rnd, (rnd["hit"], rnd["slot"])), ("separate", sep, (look["hit"], look["slot"]))):
        compare_verify(vref, got, K, check_lse=False, label=f"{label} {name}")
        compare_hits(hs[0].cpu().numpy(), hs[1].cpu().numpy(), ref_c["cache_tokens"], F,
                     got["accepted"].cpu().numpy(), got["out_tokens"].cpu().numpy(), vref, f"{label} {name}")
    return rnd


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V,K,B,F,mask", [(20000, 4, 6, [3, 2, 5, 1, 4], 0.0), (16385, 2, 3, [0, 7, 64], 0.0),
                                          (300, 5, 4, [64, 1, 0, 2, 3, 5], 0.3), (8192, 3, 5, [10, 9, 8, 11], 0.0),
                                          (1, 1, 3, [1, 1], 0.0), (40000, 6, 7, [1] * 7, 0.05)])
def test_verify_round_matches_separate_calls(S, dtype, V, K, B, F, mask):
    log(f"[gpu] verify round V={V} K={K} B={B} F={F} {dtype} mask={mask}")
    d = _random_case(V * 7 + K + B, B, K, V, dtype, 0.8, mask_frac=mask, Kd=K + 1)
    if B >= 3:
        d["tokens"][B - 1, K - 1] = V + 2                # a flagged row
    rnd = _round_vs_separate(S, d, F, 0.4, f"round V={V}")
    acc = rnd["accepted"].cpu().numpy()
    if B >= 3:
        assert acc[B - 1] == -1 and rnd["hit"].cpu().numpy()[B - 1] == 0


def test_verify_round_extremes(S):
    # K = 64 with 65 cache segments (F_k up to 64), and a fully masked row
    log("[gpu] verify round K=64")
    K = 64
    d = _random_case(5, 3, K, 3000, "bf16", 1.0, draft_sd=0.05, Kd=K + 1)
    F = [(k * 7) % 65 for k in range(K + 1)]
    _round_vs_separate(S, d, F, 0.5, "round K64")
    log("[gpu] verify round masked rows, tau extremes")
    for tau in (0.05, 5.0):
        d = _random_case(6, 4, 3, 5000, "f32", tau, Kd=4)
        d["target"][1] = -np.inf                      # a row without mass: empty p
        d["draft"][2, 0] = -np.inf                    # a draft row without mass
        _round_vs_separate(S, d, [4, 0, 64, 3], 0.0, f"round tau{tau}")


@pytest.mark.parametrize("V", [16 * 8192, 32 * 8192])
def test_verify_round_tied_chunks(S, V):
    """Chunks whose candidates (entries at or above the chunk bound) fill
    more of their slots than the merge keeps in registers (four positions of
    P = 256 / G threads: 64 slots at 16 chunks, 32 at 32), more than the 128
    slots (the exact top-F rewrite), and ties spread over several chunks
    (more than 64 kept candidates, ranked in LDS). The round's merge (four
    held slots) and ssd_build_cache's (sixteen) must agree bit for bit, and
    both with the oracle."""
    log(f"[gpu] verify round tied chunks V={V}")
    B, K = 5, 2
    rng = np.random.default_rng(V + 17)
    d = _random_case(V + 3, B, K, V, "f32", 0.9, Kd=K + 1)
    dr = d["draft"]
    c = 8192

    def ties(b, k, chunk, n, val=20.0):   # far above every other logit of the row
        pos = rng.choice(c, size=n, replace=False)
        dr[b, k, chunk * c + pos] = val

    for k in range(K + 1):
        ties(0, k, 3, 100)               # 64 < n <= 128 at 16 chunks (32 < n at 32)
        ties(1, k, 5, 200)               # past the 128 slots: the exact top-F rewrite
        for ch in range(4):
            ties(2, k, ch, 50)           # 200 ties at the row maximum over four chunks
        ties(3, k, 1, 40)                # 32 < n <= 64: a continuation only at 32 chunks
        ties(3, k, 2, 40, 19.0)
    d["target"], d["draft"] = W.f32_to_bf16_bits(d["target"]), W.f32_to_bf16_bits(dr)
    for b in range(B):
        for i in range(K):
            d["tokens"][b, i] = O.sample_draft(d["draft"][b, i], d["tau"], rng.random())
    _round_vs_separate(S, d, [64, 40, 8], 0.5, f"round ties V={V}")


def test_verify_round_marked_matches_round(S):
    """ssd_verify_round_marked: the same outputs as ssd_verify_round, and the
    four events recorded in launch order (non-negative elapsed times)."""
    log("[gpu] verify round marked")
    B, K, V = 9, 3, 20000
    d = _random_case(77, B, K, V, "bf16", 0.8, Kd=K + 1)
    F = [5, 4, 3, 6]
    tgt, dft = to_dev(d["target"], torch), to_dev(d["draft"], torch)
    toks, ua, ur = ivec(d["tokens"], torch), fvec(d["u_acc"], torch), fvec(d["u_res"], torch)
    plain = S.ssd_verify_round(tgt, dft, F, 0.5, toks, ua, ur, d["tau"])
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    marked = S.ssd_verify_round(tgt, dft, F, 0.5, toks, ua, ur, d["tau"], marks=marks)
    torch.cuda.synchronize()
    for k in plain:
        if isinstance(plain[k], torch.Tensor):
            assert torch.equal(plain[k], marked[k]), k
    for i in range(3):
        assert marks[i].elapsed_time(marks[i + 1]) >= 0.0

"""Property tier: hypothesis-generated tiny problems, HIP library vs the oracle.

Shapes V 1-64, K 1-8, B 1-6 in both dtypes; logits with ties (values on a
coarse grid), masked (-inf) tokens and whole masked rows; uniforms at the
edges (u_acc = 0, u_res = 0 and 1 - 2^-24, the largest float below 1) as
well as inside (0, 1); with and without the sigma_{F,C} reshaping (random
fan-out F_k <= min(V, 64) and C in [0, 1]). Each example runs ssd_verify,
ssd_build_cache + sigma ssd_verify + ssd_cache_lookup, ssd_verify_round and
ssd_residual_sample, and compares them with the oracle at the same bar as
the other parity tests (integers exact unless the oracle's margin at the
first differing decision is below 1e-6; cache tokens exact).
"""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_utils import EXCUSE, compare_cache, compare_hits, compare_verify, fvec, ivec, to_dev

torch = pytest.importorskip("torch")
hyp = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

pytestmark = pytest.mark.gpu

U_TOP = float(np.float32(1.0 - 2.0 ** -24))


@pytest.fixture(scope="module")
def S():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import verify_speculation_cache_amd as lib
    lib.lib()
    return lib


@st.composite
def problems(draw):
    B = draw(st.integers(1, 6))
    K = draw(st.integers(1, 8))
    V = draw(st.integers(1, 64))
    dtype = draw(st.sampled_from(["bf16", "f32"]))
    tau = draw(st.sampled_from([0.3, 0.7, 1.0, 2.5]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    grid = draw(st.sampled_from([0.0, 0.5, 1.0]))      # 0: continuous values; else ties on a grid
    mask = draw(st.sampled_from([0.0, 0.2, 0.6]))
    u_mode = draw(st.sampled_from(["random", "zero", "top", "mixed"]))
    sigma = draw(st.booleans())
    C = draw(st.sampled_from([0.0, 0.3, 0.5, 1.0]))
    rng = np.random.default_rng(seed)
    t = (rng.standard_normal((B, K + 1, V)) * 2.0).astype(np.float32)
    d = (t + rng.standard_normal((B, K + 1, V)).astype(np.float32) * 0.6).astype(np.float32)
    if grid > 0:
        t = (np.round(t / grid) * grid).astype(np.float32)
        d = (np.round(d / grid) * grid).astype(np.float32)
    if mask > 0:
        t[rng.random(t.shape) < mask] = -np.inf
        d[rng.random(d.shape) < mask] = -np.inf
    if B > 1 and rng.random() < 0.3:
        t[B - 1, rng.integers(0, K + 1)] = -np.inf        # a target row with no mass
    if dtype == "bf16":
        t, d = W.f32_to_bf16_bits(t), W.f32_to_bf16_bits(d)
    F = [int(x) for x in rng.integers(0, min(V, 64) + 1, size=K + 1)]
    u_acc = rng.random((B, K)).astype(np.float32)
    u_res = rng.random(B).astype(np.float32)
    if u_mode in ("zero", "mixed"):
        u_acc[rng.random((B, K)) < 0.5] = 0.0
        u_res[0] = 0.0
    if u_mode in ("top", "mixed"):
        u_acc[rng.random((B, K)) < 0.5] = U_TOP
        u_res[-1] = U_TOP
    # drafted tokens: inverse CDF of the (reshaped) draft distribution; rows
    # without mass draw -1, which the library flags, so use token 0 there
    toks = np.zeros((B, K), dtype=np.int32)
    for b in range(B):
        for i in range(K):
            x = O.sample_draft(d[b, i], float(np.float32(tau)), rng.random(), F[i] if sigma else None,
                               C if sigma else 1.0)
            toks[b, i] = x if x >= 0 else 0
    return {"target": t, "draft": d, "tokens": toks, "u_acc": u_acc, "u_res": u_res,
            "tau": float(np.float32(tau)), "F": F, "C": C, "sigma": sigma}


@settings(max_examples=60, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(p=problems())
def test_tiny_problems_match_oracle(S, p):
    B, K = p["tokens"].shape
    tau, F, C = p["tau"], p["F"], p["C"]
    rows = list(range(B))
    tgt, dft = to_dev(p["target"], torch), to_dev(p["draft"], torch)
    toks, ua, ur = ivec(p["tokens"], torch), fvec(p["u_acc"], torch), fvec(p["u_res"], torch)
    label = f"B={B} K={K} V={p['target'].shape[2]} tau={tau} sigma={p['sigma']}"

    # plain verification
    got = S.ssd_verify(tgt, dft, toks, ua, ur, tau)
    torch.cuda.synchronize()
    ref = O.verify(p["target"], p["draft"], p["tokens"], p["u_acc"], p["u_res"], tau)
    compare_verify(ref, got, K, label=label + " plain")

    # residual draws from every position, residual and bonus forms
    pos = np.arange(B, dtype=np.int32) % (K + 1)
    for use_draft in (True, False):
        rs = S.ssd_residual_sample(tgt, dft if use_draft else None, ivec(pos, torch), ur, tau)
        torch.cuda.synchronize()
        rr = O.residual_sample(p["target"], p["draft"] if use_draft else None, pos, p["u_res"], tau)
        tg = rs["tokens"].cpu().numpy()
        bad = (tg != rr["tokens"]) & ~(rr["margin"] < EXCUSE)
        assert not bad.any(), (label, "residual_sample", tg, rr["tokens"], rr["margin"])

    if not p["sigma"]:
        return
    # cache build, sigma verification and lookup; the fused round
    cache = S.ssd_build_cache(dft, tau, F)
    sg = S.sigma_from_cache(cache, C)
    sv = S.ssd_verify(tgt, dft, toks, ua, ur, tau, sg)
    look = S.ssd_cache_lookup(cache["cache_tokens"], F, sv["accepted"], sv["out_tokens"])
    rnd = S.ssd_verify_round(tgt, dft, F, C, toks, ua, ur, tau)
    torch.cuda.synchronize()
    rc = O.build_cache(p["draft"], tau, F, C)
    compare_cache(cache, rc, F, rows, label + " cache")
    compare_cache(rnd, rc, F, rows, label + " round cache")
    vref = O.verify(p["target"], p["draft"], p["tokens"], p["u_acc"], p["u_res"], tau, {"F": F, "C": C})
    hit_r, _ = O.cache_lookup(rc["cache_tokens"], F, vref["accepted"], vref["out_tokens"])
    vref = dict(vref, hit=hit_r)
    compare_verify(vref, sv, K, label=label + " sigma")
    compare_verify(vref, rnd, K, check_lse=False, label=label + " round")
    for name, res, hs in (("lookup", sv, look), ("round", rnd, rnd)):
        compare_hits(hs["hit"].cpu().numpy(), hs["slot"].cpu().numpy(), rc["cache_tokens"], F,
                     res["accepted"].cpu().numpy(), res["out_tokens"].cpu().numpy(), vref, label + " " + name)

"""Host-side checks of libssdv (no GPU needed): the library loads, exports
every entry point declared in include/ssd.h, its host-only fan-out agrees
with the oracle, and argument checks reject bad calls before any device
work (pointer arguments below are never dereferenced)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
import verify_speculation_cache_amd as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x1000)   # non-null, never dereferenced: validation fails first


def _declared():
    src = open(os.path.join(ROOT, "include", "ssd.h")).read()
    return sorted(set(re.findall(r"SSD_API\s+[\w\s\*]+?\b(ssd_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = S.lib()
    names = _declared()
    assert set(names) == set(S.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n


def test_fanout_matches_oracle():
    rng = np.random.default_rng(0)
    cases = [(64, 7, 0.8, 1.0), (128, 8, 0.7, 0.5), (64, 5, 0.8, 1.0), (0, 3, 0.5, 0.0),
             (1, 1, 0.5, 0.0), (11, 1, 0.5, 0.0), (1000, 64, 0.95, 3.0)]
    for _ in range(200):
        cases.append((int(rng.integers(0, 500)), int(rng.integers(1, 65)),
                      float(rng.uniform(0.01, 0.99)), float(rng.uniform(-0.9, 4.0))))
    for N, K, a_p, r in cases:
        got = S.ssd_fanout(N, K, a_p, r)
        assert got == O.fanout(N, K, a_p, r), (N, K, a_p, r)
        assert sum(got) == N


def test_fanout_workload_vectors():
    # the cache workloads' fan-outs (largest-remainder rounding of the geometric shape)
    assert S.ssd_fanout(64, 7, 0.8, 1.0) == [10, 9, 8, 8, 7, 6, 5, 11]
    assert S.ssd_fanout(128, 8, 0.7, 0.5) == [29, 23, 18, 15, 11, 9, 7, 6, 10]
    assert S.ssd_fanout(64, 5, 0.8, 1.0) == [12, 11, 10, 8, 8, 15]


@pytest.mark.parametrize("args", [(-1, 3, 0.5, 1.0), (10, 0, 0.5, 1.0), (10, 65, 0.5, 1.0),
                                  (10, 3, 0.0, 1.0), (10, 3, 1.0, 1.0), (10, 3, 0.5, -1.0),
                                  (10, 3, float("nan"), 1.0), (10, 3, 0.5, float("inf"))])
def test_fanout_rejects_bad_arguments(args):
    with pytest.raises(S.SsdError) as e:
        S.ssd_fanout(*args)
    assert e.value.code == -1


def test_workspace_queries():
    for dt in (S.SSD_F32, S.SSD_BF16):
        for (B, K, V) in ((1, 4, 32000), (64, 5, 128256), (256, 8, 256000), (3, 1, 1)):
            for q in (S.ssd_verify_workspace_size, S.ssd_residual_workspace_size,
                      S.ssd_build_cache_workspace_size):
                n = q(B, K, V, dt)
                assert n > 0 and n % 256 == 0
    assert S.ssd_verify_workspace_size(0, 4, 10, 0) == 0
    assert S.ssd_verify_workspace_size(1, 4, 10, 7) == 0


def _verify(**kw):
    a = dict(t=FAKE, tb=0, d=FAKE, db=0, dtype=S.SSD_BF16, B=2, K=3, V=100, tau=1.0,
             tok=FAKE, ua=FAKE, ur=FAKE, sigma=None, acc=FAKE, out=FAKE, ws=None, wsz=0)
    a.update(kw)
    L = S.lib()
    return L.ssd_verify(a["t"], a["tb"], a["d"], a["db"], a["dtype"], a["B"], a["K"], a["V"],
                        a["tau"], a["tok"], a["ua"], a["ur"], a["sigma"], a["acc"], a["out"],
                        None, None, None, a["ws"], a["wsz"], None)


def test_verify_argument_checks():
    assert _verify(dtype=5) == -2
    assert _verify(B=0) == -1
    assert _verify(K=0) == -1
    assert _verify(K=65) == -1
    assert _verify(V=0) == -1
    assert _verify(tau=0.0) == -1
    assert _verify(tau=float("nan")) == -1
    assert _verify(tau=float("inf")) == -1
    assert _verify(t=None) == -1
    assert _verify(tok=None) == -1
    assert _verify(tb=-1) == -1
    assert _verify(ws=None) == -3                       # workspace missing
    assert _verify(ws=ctypes.c_void_p(0x1001), wsz=1 << 30) == -3   # misaligned
    assert _verify(ws=ctypes.c_void_p(0x1000), wsz=16) == -3        # too small
    sig = S._Sigma(1.5, 0x1000, 0x1000)
    assert _verify(sigma=ctypes.byref(sig)) == -1      # C outside [0, 1]
    sig = S._Sigma(0.5, None, 0x1000)
    assert _verify(sigma=ctypes.byref(sig)) == -1
    assert b"thr" in S.lib().ssd_last_error()


def test_build_cache_and_lookup_argument_checks():
    L = S.lib()
    F = (ctypes.c_int32 * 4)(3, 2, 1, 65)
    r = L.ssd_build_cache(FAKE, 0, S.SSD_BF16, 2, 3, 100, 1.0, F, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert r == -1 and b"F[3]" in L.ssd_last_error()
    F = (ctypes.c_int32 * 4)(3, 2, 1, 5)
    r = L.ssd_build_cache(FAKE, 0, S.SSD_BF16, 2, 3, 4, 1.0, F, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert r == -1                                      # F_k > V
    F = (ctypes.c_int32 * 4)(-1, 2, 1, 5)
    r = L.ssd_build_cache(FAKE, 0, S.SSD_BF16, 2, 3, 100, 1.0, F, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert r == -1
    F = (ctypes.c_int32 * 4)(3, 2, 1, 5)
    r = L.ssd_build_cache(FAKE, 0, S.SSD_BF16, 2, 3, 100, 1.0, F, FAKE, FAKE, FAKE, None, 0, None)
    assert r == -3
    r = L.ssd_cache_lookup(FAKE, None, 2, 3, FAKE, FAKE, FAKE, None, None)
    assert r == -1
    F = (ctypes.c_int32 * 4)(3, 2, 1, 99)
    r = L.ssd_cache_lookup(FAKE, F, 2, 3, FAKE, FAKE, FAKE, None, None)
    assert r == -1
    r = L.ssd_residual_sample(FAKE, 0, None, 0, S.SSD_BF16, 2, 3, 100, -1.0, FAKE, None, FAKE,
                              FAKE, None, FAKE, 1 << 30, None)
    assert r == -1
    sig = S._Sigma(0.5, 0x1000, 0x1000)
    r = L.ssd_residual_sample(FAKE, 0, None, 0, S.SSD_BF16, 2, 3, 100, 1.0, FAKE, ctypes.byref(sig),
                              FAKE, FAKE, None, FAKE, 1 << 30, None)
    assert r == -1                                      # sigma without draft


def test_draft_sample_argument_checks():
    L = S.lib()

    def call(**kw):
        a = dict(d=FAKE, db=0, dtype=S.SSD_BF16, B=2, K=3, V=100, tau=1.0, sigma=None, u=FAKE, out=FAKE,
                 ws=FAKE, wsz=1 << 30)
        a.update(kw)
        return L.ssd_draft_sample(a["d"], a["db"], a["dtype"], a["B"], a["K"], a["V"], a["tau"], a["sigma"],
                                  a["u"], a["out"], a["ws"], a["wsz"], None)

    assert call(tau=0.0) == -1
    assert call(tau=float("inf")) == -1
    assert call(dtype=7) == -2
    assert call(K=0) == -1 and call(K=65) == -1
    assert call(u=None) == -1 and call(out=None) == -1 and call(d=None) == -1
    assert call(db=-1) == -1
    assert call(ws=None, wsz=0) == -3
    assert call(wsz=16) == -3
    sig = S._Sigma(-0.1, 0x1000, None)
    assert call(sigma=ctypes.byref(sig)) == -1
    sig = S._Sigma(0.5, None, None)
    assert call(sigma=ctypes.byref(sig)) == -1 and b"thr" in L.ssd_last_error()
    assert S.ssd_draft_sample_workspace_size(2, 3, 100, S.SSD_BF16) > 0
    assert S.ssd_draft_sample_workspace_size(0, 3, 100, S.SSD_BF16) == 0


def test_verify_greedy_argument_checks():
    L = S.lib()

    def call(**kw):
        a = dict(t=FAKE, tb=0, dtype=S.SSD_F32, B=2, K=3, V=100, tok=FAKE, acc=FAKE, out=FAKE, ws=FAKE, wsz=1 << 30)
        a.update(kw)
        return L.ssd_verify_greedy(a["t"], a["tb"], a["dtype"], a["B"], a["K"], a["V"], a["tok"], a["acc"],
                                   a["out"], a["ws"], a["wsz"], None)

    assert call(dtype=5) == -2
    assert call(B=0) == -1 and call(K=65) == -1 and call(V=0) == -1
    assert call(t=None) == -1 and call(tok=None) == -1 and call(acc=None) == -1 and call(out=None) == -1
    assert call(tb=-4) == -1
    assert call(ws=None, wsz=0) == -3 and call(wsz=8) == -3
    assert S.ssd_verify_greedy_workspace_size(2, 3, 100, S.SSD_F32) > 0


def test_cache_policy_host_calls_match_oracle():
    for n, K in ((64, 7), (128, 8), (5, 3), (0, 4), (1000, 64)):
        assert S.ssd_fanout_uniform(n, K) == O.fanout_uniform(n, K)
    for args in ((0.8, 3.6, 1.9, 0.7, 0.1, 1), (0.95, 4.0, 1.2, 1.5, 0.0, 16), (0.0, 2.0, 1.0, 0.3, 0.4, 3),
                 (1.0, 5.0, 1.0, 0.0, 2.0, 64)):
        assert abs(S.ssd_speedup(*args) - O.ssd_speedup(*args)) <= 1e-15 * O.ssd_speedup(*args)
    L = S.lib()
    out = ctypes.c_double()
    assert L.ssd_speedup(1.5, 1.0, 1.0, 0.0, 0.0, 1, ctypes.byref(out)) == -1
    assert L.ssd_speedup(0.5, -1.0, 1.0, 0.0, 0.0, 1, ctypes.byref(out)) == -1
    assert L.ssd_speedup(0.5, 1.0, 1.0, 0.0, 0.0, 0, ctypes.byref(out)) == -1
    assert L.ssd_speedup(0.5, 1.0, 1.0, float("nan"), 0.0, 1, ctypes.byref(out)) == -1
    assert L.ssd_speedup(0.5, 1.0, 1.0, 0.0, 0.0, 1, None) == -1
    F = (ctypes.c_int32 * 2)()
    assert L.ssd_fanout_uniform(-1, 1, F) == -1 and L.ssd_fanout_uniform(4, 0, F) == -1
    assert L.ssd_cache_stats(FAKE, FAKE, 0, 3, FAKE, None) == -1
    assert L.ssd_cache_stats(FAKE, None, 4, 3, FAKE, None) == -1
    assert L.ssd_cache_stats(FAKE, FAKE, 4, 65, FAKE, None) == -1


def test_oracle_not_imported_by_product():
    import sys
    src_dir = os.path.join(ROOT, "verify_speculation_cache_amd")
    for dirpath, _, files in os.walk(src_dir):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.replace("oracle-free", ""), f


def _max_passes(children, node):
    # brute force over walk outcomes: each rejection costs one vocabulary
    # pass; all children rejected ends with the draw in the last one's pass;
    # a node without children needs one pass for its bonus draw
    ch = children[node]
    best = max(len(ch), 1)
    for i, c in enumerate(ch):
        best = max(best, i + _max_passes(children, c))
    return best


def test_tree_rounds_match_bruteforce():
    rng = np.random.default_rng(4)
    cases = [[-1], [-1, 0], [-1, 0, 1, 2, 3], [-1] + [0] * 63, [-1, 0, 0, 1, 1, 2, 2]]
    for _ in range(300):
        N = int(rng.integers(1, 65))
        cases.append([-1] + [int(rng.integers(0, n)) for n in range(1, N)])
    for par in cases:
        ch = O.tree_children(par)
        assert S.ssd_tree_rounds(par) == _max_passes(ch, 0), par


def test_verify_tree_argument_checks():
    L = S.lib()

    def call(parent=(-1, 0, 0), **kw):
        a = dict(t=FAKE, tb=0, d=FAKE, db=0, dtype=S.SSD_BF16, B=2, V=100, tau=1.0, tok=FAKE, ua=FAKE, ur=FAKE,
                 acc=FAKE, out=FAKE, nodes=None, ws=FAKE, wsz=1 << 30)
        a.update(kw)
        N = kw.pop("N", len(parent))
        arr = (ctypes.c_int32 * max(len(parent), 1))(*parent)
        return L.ssd_verify_tree(a["t"], a["tb"], a["d"], a["db"], a["dtype"], a["B"], N, a["V"], a["tau"], arr,
                                 a["tok"], a["ua"], a["ur"], a["acc"], a["out"], a["nodes"], a["ws"], a["wsz"],
                                 None)

    assert call(dtype=3) == -2
    assert call(B=0) == -1 and call(V=0) == -1
    assert call(tau=0.0) == -1 and call(tau=float("nan")) == -1
    assert call(parent=(0, 0, 0)) == -1 and b"root" in L.ssd_last_error()
    assert call(parent=(-1, 0, 2)) == -1 and b"parent[2]" in L.ssd_last_error()
    assert call(parent=(-1, 1)) == -1
    assert call(parent=(-1,) + (0,) * 64) == -1                  # N = 65
    assert call(d=None) == -1 and b"draft" in L.ssd_last_error()
    assert call(tok=None) == -1 and call(ur=None) == -1 and call(out=None) == -1
    assert call(tb=-2) == -1
    assert call(ws=None, wsz=0) == -3 and call(wsz=64) == -3
    assert S.ssd_verify_tree_workspace_size(2, 3, 100, S.SSD_BF16) > 0
    assert S.ssd_verify_tree_workspace_size(2, 65, 100, S.SSD_BF16) == 0
    with pytest.raises(S.SsdError):
        S.ssd_tree_rounds([-1, 0, 5])


def test_verify_round_argument_checks():
    L = S.lib()

    def call(F=(3, 2, 1), **kw):
        a = dict(t=FAKE, tb=0, d=FAKE, db=0, dtype=S.SSD_BF16, B=2, K=2, V=100, tau=1.0, C=0.5, tok=FAKE, ua=FAKE,
                 ur=FAKE, ct=FAKE, thr=FAKE, ds=FAKE, acc=FAKE, out=FAKE, hit=FAKE, slot=None, ws=FAKE, wsz=1 << 30)
        a.update(kw)
        Fa = (ctypes.c_int32 * len(F))(*F)
        return L.ssd_verify_round(a["t"], a["tb"], a["d"], a["db"], a["dtype"], a["B"], a["K"], a["V"], a["tau"],
                                  Fa, a["C"], a["tok"], a["ua"], a["ur"], a["ct"], a["thr"], a["ds"], a["acc"],
                                  a["out"], a["hit"], a["slot"], a["ws"], a["wsz"], None)

    assert call(dtype=4) == -2
    assert call(C=1.5) == -1 and call(C=float("nan")) == -1
    assert call(tau=-1.0) == -1
    assert call(F=(3, 2, 65)) == -1 and b"F[2]" in L.ssd_last_error()
    assert call(F=(3, -1, 1)) == -1
    assert call(hit=None) == -1 and call(thr=None) == -1 and call(ct=None) == -1
    assert call(tb=-1) == -1
    assert call(ws=None, wsz=0) == -3 and call(wsz=128) == -3
    assert S.ssd_verify_round_workspace_size(2, 2, 100, S.SSD_BF16) > S.ssd_build_cache_workspace_size(2, 2, 100, S.SSD_BF16)

"""The stored expected outputs under tests/golden/*.npz are the oracle's.

Sampled batch rows of every golden case are recomputed here with the oracle
(inputs regenerated from the seeded generator) and must equal what is stored,
bit for bit; the stored shapes and summary statistics must be those of the
workload. Also pins the harness's rule for excusing a near-tie: the margin
taken is the oracle's at the first decision where two outcomes differ.
"""
import math

import numpy as np
import pytest

from gpu_utils import divergence_margin, load_golden, tree_divergence_margin

CASES = ["verify_B512_K4_V151936_bf16", "step_B64_K5_V128256_bf16", "cache_B32_K7_V128256_bf16",
         "cache_B256_K8_V256000_bf16_tau0.5", "cache_B256_K8_V256000_bf16_tau1.0"]


@pytest.mark.parametrize("name", CASES)
def test_golden_rows_are_the_oracles(name):
    mg, g = load_golden(name)
    cfg, tau, sigma, F, C = mg.case_params(name)
    B, K = cfg.B, cfg.K
    assert g["accepted"].shape == (B,) and g["out_tokens"].shape == (B, K + 1)
    assert g["tokens"].shape == (B, K) and g["row_digest"].shape == (B,)
    assert g["tau"] == np.float32(tau) and g["F"] == (F or [])
    if sigma:
        assert g["cache_tokens"].shape == (B, sum(F))
        assert sum(F) == cfg.n_budget
    assert np.all((g["accepted"] >= 0) & (g["accepted"] <= K))
    for b in sorted({0, B // 2 + 1, B - 1}):
        row = mg.row_outputs(name, b)
        assert row["digest"] == g["row_digest"][b], (name, b)
        for k, v in row.items():
            if k == "digest":
                continue
            stored = g[k][b]
            v = np.asarray(v)
            assert stored.shape == v.shape, (name, b, k)
            same = np.array_equal(stored, v.astype(stored.dtype), equal_nan=stored.dtype.kind == "f")
            assert same, (name, b, k, stored, v)


def test_divergence_margin_takes_the_first_differing_decision():
    ref = {"accepted": np.array([2, 3, -1, 1]),
           "acc_margin": np.array([[0.3, 0.2, 5e-7, np.nan], [0.1, 4e-7, 0.5, 0.2],
                                   [np.nan] * 4, [0.4, 0.6, np.nan, np.nan]]),
           "res_margin": np.array([0.25, 0.01, np.nan, 2e-8])}
    # GPU accepted more than the oracle: the oracle's rejection at 2 is the first difference
    assert divergence_margin(ref, 0, 3, None) == 5e-7
    # GPU accepted fewer: the oracle's acceptance at 1 (a near-tie) is the first difference,
    # not the later, larger margins
    assert divergence_margin(ref, 1, 1, None) == 4e-7
    # same length, different token: the final draw
    assert divergence_margin(ref, 3, 1, None) == 2e-8
    # a near-tie elsewhere in the row must not excuse a different decision
    assert divergence_margin(ref, 1, 0, None) == 0.1
    # a flag on one side only is never a near-tie
    assert divergence_margin(ref, 2, 0, None) is None
    assert divergence_margin(ref, 0, -1, None) is None


def test_tree_divergence_margin_follows_the_walk():
    # root 0 with children 1, 2, 3; node 1 has children 4, 5
    am = np.full(6, np.nan)
    am[1], am[2], am[3], am[4], am[5] = 0.3, 2e-7, 0.4, 0.05, 9e-7
    ref = {"accepted": np.array([1]), "out_nodes": np.array([[0, 2, -1, -1, -1, -1]]),
           "acc_margin": am[None, :], "res_margin": np.array([3e-8])}
    # the GPU kept child 1 where the oracle rejected it: decision at node 1
    assert tree_divergence_margin(ref, 0, 2, np.array([0, 1, 4, -1, -1, -1])) == 0.3
    # the GPU rejected child 2 and kept 3: the first differing test is child 2's
    assert tree_divergence_margin(ref, 0, 1, np.array([0, 3, -1, -1, -1, -1])) == 2e-7
    # the GPU rejected every child: child 2's test again
    assert tree_divergence_margin(ref, 0, 0, np.array([0, -1, -1, -1, -1, -1])) == 2e-7
    # the same path: only the final draw differs
    assert tree_divergence_margin(ref, 0, 1, np.array([0, 2, -1, -1, -1, -1])) == 3e-8
    assert tree_divergence_margin(ref, 0, -1, np.full(6, -1)) is None
    assert not math.isnan(tree_divergence_margin(ref, 0, 1, np.array([0, 2, -1, -1, -1, -1])))

"""GPU parity of token-tree verification (ssd_verify_tree) against the oracle.

Accepted depth, emitted tokens and kept-path nodes must match the oracle
exactly, except rows whose walk took a decision (an accept test or the final
draw) with margin below 1e-6 in probability units; those are counted,
printed and bounded.
"""
import dataclasses

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_utils import EXCUSE, fvec, ivec, log, to_dev, tree_divergence_margin

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import verify_speculation_cache_amd as lib
    lib.lib()
    return lib


def _run(S, d, rows=None, label="", max_excused=1):
    got = S.ssd_verify_tree(to_dev(d["target"], torch), to_dev(d["draft"], torch), d["parent"],
                            ivec(d["tokens"], torch), fvec(d["u_acc"], torch), fvec(d["u_res"], torch),
                            d["tau"])
    torch.cuda.synchronize()
    B = d["tokens"].shape[0]
    sel = list(range(B)) if rows is None else list(rows)
    ref = O.verify_tree(d["target"][sel], d["draft"][sel], d["parent"], d["tokens"][sel], d["u_acc"][sel],
                        d["u_res"][sel], d["tau"])
    acc = got["accepted"].cpu().numpy()
    out = got["out_tokens"].cpu().numpy()
    nodes = got["out_nodes"].cpu().numpy()
    excused = []
    for j, b in enumerate(sel):
        same = (acc[b] == ref["accepted"][j] and np.array_equal(out[b], ref["out_tokens"][j])
                and np.array_equal(nodes[b], ref["out_nodes"][j]))
        if same:
            continue
        m = tree_divergence_margin(ref, j, acc[b], nodes[b])
        assert m is not None and m < EXCUSE, (f"{label} row {b}: accepted {acc[b]} vs {ref['accepted'][j]}, out {out[b]} vs "
                            f"{ref['out_tokens'][j]}, nodes {nodes[b]} vs {ref['out_nodes'][j]}, margin {m}")
        excused.append(b)
    if excused:
        log(f"  {label}: excused rows {excused}")
    assert len(excused) <= max_excused, excused
    return got, ref


def _cfg(B, V, dtype, branching=(2,), tau=0.8, draft_sd=0.7, seed=0):
    return dataclasses.replace(W.TREE_CONFIGS["tree"], B=B, V=V, dtype=dtype, branching=tuple(branching),
                               tau=tau, draft_sd=draft_sd, seed=seed)


def _random_parent(rng, N):
    return [-1] + [int(rng.integers(0, n)) for n in range(1, N)]


TOPOLOGIES = {
    "chain5": [-1, 0, 1, 2, 3, 4],
    "star6": [-1, 0, 0, 0, 0, 0, 0],
    "binary3": W.tree_parent((2, 2, 2)),
    "b4x2x1x1": W.tree_parent((4, 2, 1, 1)),
    "random20": _random_parent(np.random.default_rng(5), 20),
    "root_only": [-1],
    "wide64": [-1] + [0] * 63,
}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("topo", list(TOPOLOGIES))
@pytest.mark.parametrize("V,B", [(20000, 6), (16385, 3), (1000, 8), (8192, 2)])
def test_tree_small(S, dtype, topo, V, B):
    parent = TOPOLOGIES[topo]
    log(f"[gpu] tree {topo} N={len(parent)} V={V} B={B} {dtype}")
    # a large draft noise keeps rejections (and so residual rounds) frequent
    cfg = _cfg(B, V, dtype, tau=0.8, draft_sd=1.5, seed=V + B)
    d = W.make_tree_inputs(cfg, parent=parent)
    _run(S, d, label=f"{topo}/{V}/{dtype}")


def test_tree_many_rejections(S):
    # siblings far from the target: most rows run every round of the topology
    parent = W.tree_parent((6, 3))
    log(f"[gpu] tree many rejections N={len(parent)} rounds={S.ssd_tree_rounds(parent)}")
    cfg = _cfg(24, 12000, "bf16", tau=1.0, draft_sd=4.0, seed=9)
    d = W.make_tree_inputs(cfg, parent=parent)
    got, ref = _run(S, d, label="many-rejections")
    assert np.mean(ref["accepted"] == 0) > 0.3   # the case is what it says


def test_tree_chain_matches_linear_verify(S):
    # a one-chain tree is the single-path verification: same outputs as ssd_verify
    K, B, V = 5, 16, 20000
    parent = [-1] + list(range(K))
    log("[gpu] tree chain vs ssd_verify")
    cfg = _cfg(B, V, "bf16", tau=0.7, draft_sd=1.0, seed=17)
    d = W.make_tree_inputs(cfg, parent=parent)
    got, _ = _run(S, d, label="chain")
    lin = S.ssd_verify(to_dev(d["target"], torch), to_dev(d["draft"][:, :K], torch).contiguous(),
                       ivec(d["tokens"][:, 1:], torch), fvec(d["u_acc"][:, 1:], torch), fvec(d["u_res"], torch),
                       d["tau"])
    torch.cuda.synchronize()
    assert np.array_equal(got["accepted"].cpu().numpy(), lin["accepted"].cpu().numpy())
    assert np.array_equal(got["out_tokens"].cpu().numpy(), lin["out_tokens"].cpu().numpy())


def test_tree_flagged_and_masked(S):
    parent = [-1, 0, 0, 0, 1]
    V, B = 3000, 5
    log("[gpu] tree flagged and masked rows")
    cfg = _cfg(B, V, "f32", seed=23)
    d = W.make_tree_inputs(cfg, parent=parent)
    d["tokens"][1, 4] = V + 3                 # row 1 flagged (token past V)
    d["tokens"][2, 2] = -1                    # row 2 flagged (negative token)
    # row 3: root target = root draft with 2990 masked entries; all three root
    # children hold masked tokens, so each is rejected with an empty
    # residual (p = q) and the draw falls back to p of the root
    row = d["target"][3, 0].copy()
    row[10:] = -np.inf
    d["target"][3, 0] = row
    d["draft"][3, 0] = row
    d["tokens"][3, 1:4] = [100, 2000, 2999]
    # row 4: the root's target row has no mass at all: every child is
    # rejected and the final draw finds nothing (token -1)
    d["target"][4, 0] = -np.inf
    got, ref = _run(S, d, label="flagged/masked", max_excused=0)
    acc = got["accepted"].cpu().numpy()
    assert acc[1] == -1 and acc[2] == -1
    assert np.all(got["out_tokens"].cpu().numpy()[1] == -1)
    assert acc[3] == 0 and 0 <= got["out_tokens"].cpu().numpy()[3, 0] < 10
    assert acc[4] == 0 and got["out_tokens"].cpu().numpy()[4, 0] == -1


def test_tree_workload_full_size(S):
    cfg = W.TREE_CONFIGS["tree"]
    log(f"[gpu] tree workload {cfg.name}")
    d = W.make_tree_inputs(cfg)
    got, ref = _run(S, d, label=cfg.name)
    log(f"  mean accepted depth {np.mean(ref['accepted']):.3f}")
    # repeat: the workspace is reused, outputs are identical
    again = S.ssd_verify_tree(to_dev(d["target"], torch), to_dev(d["draft"], torch), d["parent"],
                              ivec(d["tokens"], torch), fvec(d["u_acc"], torch), fvec(d["u_res"], torch), d["tau"])
    torch.cuda.synchronize()
    for k in ("accepted", "out_tokens", "out_nodes"):
        assert torch.equal(got[k], again[k]), k


def test_tree_first_token_follows_p(S):
    # Losslessness on the GPU: one tiny tree broadcast to many batch rows
    # (batch stride 0), siblings drawn from q on the host, fresh uniforms per
    # row; the first emitted token's histogram must follow p of the root.
    import scipy.stats
    rng = np.random.default_rng(31)
    V, B = 5, 40000
    p0 = rng.dirichlet(np.full(V, 0.7))
    q0 = rng.dirichlet(np.full(V, 0.7))
    leaf = rng.dirichlet(np.full(V, 0.7), size=3)
    parent = [-1, 0, 0, 0]
    with np.errstate(divide="ignore"):
        tgt = np.log(np.vstack([p0, leaf])).astype(np.float32)[None]
        dft = np.log(np.vstack([q0, q0, q0, q0])).astype(np.float32)[None]
    toks = np.zeros((B, 4), dtype=np.int32)
    toks[:, 1:] = rng.choice(V, size=(B, 3), p=q0)
    ua = rng.random((B, 4), dtype=np.float32)
    ur = rng.random(B, dtype=np.float32)
    log("[gpu] tree first-token distribution")
    t = to_dev(tgt, torch).expand(B, 4, V)
    dd = to_dev(dft, torch).expand(B, 4, V)
    got = S.ssd_verify_tree(t, dd, parent, ivec(toks, torch), fvec(ua, torch), fvec(ur, torch), 1.0)
    torch.cuda.synchronize()
    first = got["out_tokens"].cpu().numpy()[:, 0]
    hist = np.bincount(first, minlength=V)
    assert scipy.stats.chisquare(hist, p0 * B).pvalue > 1e-4, (hist / B, p0)


def test_tree_tiny_vocabularies(S):
    # V = 1 (every token 0, everything kept) and V = 2 with ties, 64-node chain
    for V, parent in ((1, W.tree_parent((2, 2))), (2, W.tree_parent((3, 1))), (3, [-1] + list(range(63)))):
        log(f"[gpu] tree tiny V={V} N={len(parent)}")
        cfg = _cfg(5, V, "f32", tau=1.0, draft_sd=0.3, seed=V)
        d = W.make_tree_inputs(cfg, parent=parent)
        got, ref = _run(S, d, label=f"tiny V={V}", max_excused=0)
        if V == 1:
            depth = max(O.tree_depth(parent))
            assert np.all(got["accepted"].cpu().numpy() == depth)

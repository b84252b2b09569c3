"""Helpers for the GPU parity tests: uploads and oracle comparisons."""
import math
import sys

import numpy as np

EXCUSE = 1e-6      # decisions with margin below this may differ (probability units)
P_RTOL = 1e-5      # p, q at drafted tokens
LSE_ATOL = 1e-5    # log-sum-exp of a row
Z_RTOL = 1e-5      # residual mass Z (rows with Z >= 1e-2)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(arr, torch, device="cuda"):
    """numpy logits (uint16 bf16 bits or float32) -> device tensor of the same values."""
    if arr.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(device)


def ivec(a, torch, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def fvec(a, torch, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def divergence_margin(ref, j, a_g, out_g):
    """The oracle's margin at the first decision where a GPU outcome (a_g,
    out_g) of row j departs from the oracle's, or None when the two cannot be
    reconciled by a near-tie (a flagged row on one side only).

    The emitted tokens before position a are the drafted ones on both sides,
    so the first differing decision is the accept test at min(a_ref, a_gpu)
    when the accepted lengths differ, else the final draw."""
    a_r = int(ref["accepted"][j])
    a_g = int(a_g)
    if a_r != a_g:
        if a_r < 0 or a_g < 0:
            return None
        return float(ref["acc_margin"][j][min(a_r, a_g)])
    if a_r < 0:
        return None
    return float(ref["res_margin"][j])


def tree_divergence_margin(ref, j, a_g, nodes_g):
    """The oracle's margin at the first decision where a GPU token-tree walk
    (its kept-path nodes) departs from the oracle's walk of row j, or None
    for a flag mismatch. Both walks test the children of a node in index
    order, so at the first depth where the kept nodes differ, the earliest
    differing decision is the test of the smaller of the two children (a
    walk that stopped there tested, and rejected, every child); with equal
    paths only the final draw can differ."""
    a_r = int(ref["accepted"][j])
    if (a_r < 0) != (int(a_g) < 0):
        return None
    if a_r < 0:
        return None
    nr, ng = ref["out_nodes"][j], nodes_g
    for depth in range(1, len(nr)):
        xr, xg = int(nr[depth]), int(ng[depth])
        if xr == xg:
            if xr < 0:
                break
            continue
        return float(ref["acc_margin"][j][min(x for x in (xr, xg) if x >= 0)])
    return float(ref["res_margin"][j])


def compare_verify(ref, got, K, rows=None, check_lse=True, label=""):
    """Compare GPU verify outputs with the oracle's on the listed batch rows.

    Integer outputs must match exactly unless the oracle's deciding margin at
    the first point of disagreement is below EXCUSE (then the whole row is
    excused). p/q within P_RTOL relative, lse within LSE_ATOL, Z within
    Z_RTOL for Z >= 1e-2. Returns the number of excused rows.
    """
    acc_g = got["accepted"].cpu().numpy()
    out_g = got["out_tokens"].cpu().numpy()
    probs_g = got["probs"].cpu().numpy() if got.get("probs") is not None else None
    mass_g = got["resid_mass"].cpu().numpy() if got.get("resid_mass") is not None else None
    lse_g = got["row_lse"].cpu().numpy() if got.get("row_lse") is not None else None
    B_ref = ref["accepted"].shape[0]
    rows = list(range(B_ref)) if rows is None else list(rows)
    excused = []
    for j, b in enumerate(rows):
        a_r = int(ref["accepted"][j])
        a_g = int(acc_g[b])
        out_r = ref["out_tokens"][j]
        if a_r == a_g and np.array_equal(out_r, out_g[b]):
            pass
        else:
            m = divergence_margin(ref, j, a_g, out_g[b])
            assert m is not None, f"{label} row {b}: flagged mismatch {a_r} vs {a_g}"
            assert m < EXCUSE, (f"{label} row {b}: accepted {a_r} vs {a_g}, out {out_r} vs "
                                f"{out_g[b]}, margin {m}")
            excused.append(b)
            continue
        if a_r < 0:
            continue
        if probs_g is not None:
            pr = ref["probs"][j]
            pg = probs_g[b].astype(np.float64)
            err = np.abs(pg - pr)
            tol = P_RTOL * np.abs(pr) + 1e-35
            assert np.all(err <= tol), f"{label} row {b}: probs {pg} vs {pr}"
        if mass_g is not None:
            Zr = ref["Z"][j]
            if Zr >= 1e-2:
                assert abs(mass_g[b] - Zr) <= Z_RTOL * Zr, f"{label} row {b}: Z {mass_g[b]} vs {Zr}"
        if check_lse and lse_g is not None:
            lr = np.concatenate([ref["lse_t"][j], ref["lse_d"][j]])
            lg = lse_g[b].astype(np.float64)
            fin = np.isfinite(lr)
            assert np.all(np.isfinite(lg) == fin), f"{label} row {b}: lse finiteness"
            assert np.all(np.abs(lg[fin] - lr[fin]) <= LSE_ATOL), f"{label} row {b}: lse {lg} vs {lr}"
    if excused:
        log(f"[{label}] excused rows (margin < {EXCUSE}): {excused}")
    return len(excused)


def compare_cache(cache, ref, F, rows, label):
    """Cache tokens and threshold indices bit-exact; zmax exact; S_top and
    S_rest as masses of the row: each within 1e-5 of the row's total mass
    S_top + S_rest (probability units, the bar of the row log-sum-exp; a
    component many orders below the total, e.g. the tail at a low
    temperature, carries the fp32 exponent error of its far-from-max
    entries and is not held to 1e-5 of itself)."""
    ct = cache["cache_tokens"].cpu().numpy()
    thr = cache["thr"].cpu().numpy()
    st = cache["draft_stats"].cpu().numpy()
    sumF = sum(F)
    for j, b in enumerate(rows):
        assert np.array_equal(ct[b, :sumF], ref["cache_tokens"][j]), f"{label} row {b} cache tokens"
        assert np.array_equal(thr[b, :, 1], ref["thr_idx"][j]), f"{label} row {b} thr"
        for k in range(len(F)):
            zr, tr, rr = ref["stats"][j, k]
            zg, tg, rg = st[b, k]
            tot = abs(tr) + abs(rr)
            assert zg == zr or (np.isinf(zg) and np.isinf(zr)), f"{label} zmax"
            assert abs(tg - tr) <= 1e-5 * tot + 1e-300, f"{label} row {b} k {k} S_top {tg} vs {tr}"
            assert abs(rg - rr) <= 1e-5 * tot + 1e-300, f"{label} row {b} k {k} S_rest {rg} vs {rr}"


def compare_hits(hit_g, slot_g, ref_cache_tokens, F, acc_g, out_g, ref, label):
    """hit/slot of the GPU's own outcome equal the oracle lookup of that
    outcome in the oracle's cache; on rows whose outcome equals the oracle's,
    they equal the oracle's hit/slot."""
    import oracle as O
    h_own, s_own = O.cache_lookup(ref_cache_tokens, F, acc_g, out_g)
    assert np.array_equal(hit_g, h_own), f"{label}: hit of the GPU outcome"
    assert np.array_equal(slot_g.astype(np.int64), s_own), f"{label}: slot of the GPU outcome"
    same = (acc_g == ref["accepted"]) & np.all(out_g == ref["out_tokens"], axis=1)
    if "hit" in ref:
        assert np.array_equal(hit_g[same], ref["hit"][same]), f"{label}: hit"
    return int((~same).sum())


def load_golden(name):
    """Expected outputs stored by tests/golden/make_golden.py (oracle only)."""
    import importlib.util
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "make_golden.py")
    spec = importlib.util.spec_from_file_location("make_golden", path)
    mg = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mg)
    return mg, mg.load(name)


def golden_inputs(name):
    """The golden case's inputs regenerated from the seeded generator, with
    every row's digest checked against the stored one; the drafted tokens are
    the stored ones (drawn by the oracle from q_sigma for cache cases)."""
    import workloads as W
    mg, g = load_golden(name)
    cfg, tau, sigma, F, C = mg.case_params(name)
    d = W.make_inputs(cfg, tau=tau, draw_tokens=not sigma)
    for b in range(cfg.B):
        assert mg.row_digest(d["target"][b], d["draft"][b]) == g["row_digest"][b], f"{name}: input row {b} changed"
    d["tokens"] = np.ascontiguousarray(g["tokens"].astype(np.int32))
    return cfg, d, g

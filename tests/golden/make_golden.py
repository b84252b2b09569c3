"""Expected outputs of the full-size workloads, every batch row, written by the oracle.

Each case below regenerates its inputs row by row from the seeded generator in
workloads/ and runs every batch row through oracle/ (float64 NumPy); nothing
else computes a stored value. The GPU parity tests compare the HIP library
with these arrays on all rows; a CPU test recomputes sampled rows with the
oracle and checks they equal what is stored here.

Cases:
  verify_B512_K4_V151936_bf16        plain verification, drafted tokens from
                                     the workload (softmax drafts)
  step_B64_K5_V128256_bf16           the measured step's shape: cache on
                                     draft rows 0..5 (budget 64, a_p 0.8, r 1,
                                     C 0.5), verification against q_sigma,
                                     lookup; drafts drawn from q_sigma
  cache_B32_K7_V128256_bf16          the same on the B=32 cache workload
  cache_B256_K8_V256000_bf16_tau0.5  the wide cache workload at each of its
  cache_B256_K8_V256000_bf16_tau1.0  two temperatures
Drafts "from q_sigma" are the oracle's inverse-CDF draws
(papernotes.org "Speculative Speculative Decoding", key design 2: the
drafted token comes from the reshaped draft distribution) with the uniforms
of workloads.make_draft_uniforms.

Stored per case (npz, no pickled objects): the drafted tokens and their draw
margins, accepted, out_tokens, the accept and residual margins, p and q at
the drafted tokens, Z, the row log-sum-exps; for cache cases also the cache
tokens, threshold indices, (zmax, S_top, S_rest), hit and slot; a 16-hex
SHA-256 digest of each row's target and draft bytes; F, C and tau.

Usage: python tests/golden/make_golden.py [case ...]    (default: every case)
"""
from __future__ import annotations

import hashlib
import os
import sys
import time
from concurrent.futures import ProcessPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle as O      # noqa: E402
import workloads as W   # noqa: E402

CASES = {
    "verify_B512_K4_V151936_bf16": {"cfg": 4, "tau": None, "sigma": False},
    "step_B64_K5_V128256_bf16": {"cfg": 2, "tau": None, "sigma": True},
    "cache_B32_K7_V128256_bf16": {"cfg": 3, "tau": None, "sigma": True},
    "cache_B256_K8_V256000_bf16_tau0.5": {"cfg": 5, "tau": 0.5, "sigma": True},
    "cache_B256_K8_V256000_bf16_tau1.0": {"cfg": 5, "tau": 1.0, "sigma": True},
}


def golden_path(name: str) -> str:
    return os.path.join(HERE, name + ".npz")


def row_digest(target_row: np.ndarray, draft_row: np.ndarray) -> str:
    h = hashlib.sha256()
    h.update(np.ascontiguousarray(target_row).tobytes())
    h.update(np.ascontiguousarray(draft_row).tobytes())
    return h.hexdigest()[:16]


def case_params(name: str):
    c = CASES[name]
    cfg = W.get_config(c["cfg"])
    tau = float(np.float32(cfg.taus[0] if c["tau"] is None else c["tau"]))
    F = O.fanout(cfg.n_budget, cfg.K, cfg.a_p, cfg.r) if c["sigma"] else None
    C = float(cfg.C) if c["sigma"] else 1.0
    return cfg, tau, c["sigma"], F, C


def row_outputs(name: str, b: int) -> dict:
    """Oracle outputs of batch row b of case `name` (inputs regenerated)."""
    cfg, tau, sigma, F, C = case_params(name)
    K = cfg.K
    d = W.make_inputs(cfg, tau=tau, draw_tokens=not sigma, b_rows=[b])
    tau32 = d["tau"]
    out = {"digest": row_digest(d["target"][0], d["draft"][0])}
    if sigma:
        u_draft = W.make_draft_uniforms(cfg, tau)[b:b + 1]
        toks, dmarg = O.draft_sample(d["draft"][:, :K], tau32, u_draft, F, C)
        toks = toks.astype(np.int32)
        cache = O.build_cache(d["draft"][:, :K + 1], tau32, F, C)
        ref = O.verify(d["target"], d["draft"], toks, d["u_acc"], d["u_res"], tau32, {"F": F, "C": C})
        hit, slot = O.cache_lookup(cache["cache_tokens"], F, ref["accepted"], ref["out_tokens"])
        out.update(cache_tokens=cache["cache_tokens"][0], thr_idx=cache["thr_idx"][0], stats=cache["stats"][0],
                   hit=hit[0], slot=slot[0], draft_margin=dmarg[0])
    else:
        toks = d["tokens"]
        ref = O.verify(d["target"], d["draft"], toks, d["u_acc"], d["u_res"], tau32)
    out.update(tokens=toks[0], accepted=ref["accepted"][0], out_tokens=ref["out_tokens"][0],
               acc_margin=ref["acc_margin"][0], res_margin=ref["res_margin"][0], probs=ref["probs"][0],
               Z=ref["Z"][0], lse_t=ref["lse_t"][0], lse_d=ref["lse_d"][0])
    return out


_DTYPES = {"tokens": np.int32, "accepted": np.int32, "out_tokens": np.int32, "cache_tokens": np.int32,
           "thr_idx": np.int32, "hit": np.uint8, "slot": np.int32}


def _one(args):
    return row_outputs(*args)


def make_case(name: str, workers: int) -> str:
    cfg, tau, sigma, F, C = case_params(name)
    t0 = time.time()
    with ProcessPoolExecutor(max_workers=workers) as ex:
        rows = list(ex.map(_one, [(name, b) for b in range(cfg.B)], chunksize=1))
    arrays = {}
    for k in rows[0]:
        if k == "digest":
            arrays["row_digest"] = np.array([r[k] for r in rows], dtype="U16")
        else:
            arrays[k] = np.stack([np.asarray(r[k]) for r in rows]).astype(_DTYPES.get(k, np.float64))
    arrays["tau"] = np.float32(tau)
    arrays["C"] = np.float64(C)
    arrays["F"] = np.array(F if F is not None else [], dtype=np.int32)
    path = golden_path(name)
    np.savez_compressed(path, **arrays)
    print(f"{name}: {cfg.B} rows in {time.time() - t0:.1f} s -> {os.path.relpath(path, ROOT)} "
          f"({os.path.getsize(path) // 1024} KiB)", flush=True)
    return path


def load(name: str) -> dict:
    with np.load(golden_path(name), allow_pickle=False) as z:
        g = {k: z[k] for k in z.files}
    g["F"] = [int(x) for x in g["F"]]
    g["tau"] = float(g["tau"])
    g["C"] = float(g["C"])
    return g


if __name__ == "__main__":
    names = sys.argv[1:] or list(CASES)
    nw = max(1, min(16, len(os.sched_getaffinity(0))))
    for n in names:
        make_case(n, nw)

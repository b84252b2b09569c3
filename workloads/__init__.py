"""Seeded synthetic inputs for speculative verification and the SAGUARO cache.

This module is shared by the tests, the bench and the smoke check. It draws
logits, drafted tokens and uniforms and holds none of the verification or
cache-build arithmetic: no softmax, no acceptance rule, no residual, no
inverse CDF, no top-F selection, no fan-out.

Workload shapes follow the speculative-decoding setting described on the
source pages: a target and a draft model score K+1 positions over a full
vocabulary (brentwoodlivery.com "Speculative decoding", The Algorithm, steps
1-2), temperatures 0.5-1.0 (papernotes.org "Speculative Speculative
Decoding", ablation table: T=0.7 and T=1.0), acceptance rates in the usual
60-80% band (til.phipham141.dev "Why does speculative decoding exist?",
Where the speedup comes from). No model, dataset or tokenizer is used: the
logits are Gaussian noise plus a Zipf rank bias, the draft is the target plus
Gaussian noise.

Drafted tokens are drawn from softmax(draft/tau) with the Gumbel-max trick
(argmax of logits/tau plus independent Gumbel noise), which yields exact
samples of that softmax without computing it. Drafts from the sigma-reshaped
distribution are not drawn here; statistical tests that need them draw them
with the oracle's own sampler.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np

__all__ = ["Config", "CONFIGS", "get_config", "make_inputs", "make_uniforms", "make_draft_uniforms",
           "f32_to_bf16_bits", "bf16_bits_to_f32", "sha256",
           "TreeConfig", "TREE_CONFIGS", "tree_parent", "make_tree_inputs"]


@dataclasses.dataclass(frozen=True)
class Config:
    """One synthetic workload.

    B batch rows, K draft tokens per row, V vocabulary, dtype of stored
    logits ("bf16" or "f32"), target noise sd, Zipf exponent (0 = none),
    draft noise sd, temperatures, number of stored draft rows K_d (K for
    verify-only workloads, K+1 when the cache build also reads draft row K),
    and the cache parameters (budget n_budget, a_p, r, C) where used.
    """
    name: str
    seed: int
    B: int
    K: int
    V: int
    dtype: str
    target_sd: float
    zipf_s: float
    draft_sd: float
    taus: tuple
    K_d: int
    n_budget: Optional[int] = None
    a_p: Optional[float] = None
    r: Optional[float] = None
    C: Optional[float] = None

    @property
    def has_cache(self) -> bool:
        return self.n_budget is not None

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def target_bytes(self) -> int:
        return self.B * (self.K + 1) * self.V * self.elem_bytes

    def draft_bytes(self, rows: Optional[int] = None) -> int:
        rows = self.K_d if rows is None else rows
        return self.B * rows * self.V * self.elem_bytes


# The five workloads, keyed 1..5. The seeds of the two cache workloads and
# the B=32 one's temperature are readings (seed = key - 1; the B=32 cache
# workload shares the B=64 workload's generator and temperature). The B=64
# workload stores K+1 draft rows so the cache build can be measured on its
# shape (draft rows 0..K) with the B=32 workload's cache parameters.
CONFIGS = {
    1: Config("verify_B1_K4_V32000_f32", 0, 1, 4, 32000, "f32", 3.0, 0.0, 1.0,
              (1.0,), 4),
    2: Config("verify_B64_K5_V128256_bf16", 1, 64, 5, 128256, "bf16", 2.0, 1.1,
              0.5, (0.7,), 6, 64, 0.8, 1.0, 0.5),
    3: Config("cache_B32_K7_V128256_bf16", 2, 32, 7, 128256, "bf16", 2.0,
              1.1, 0.8, (0.7,), 8, 64, 0.8, 1.0, 0.5),
    4: Config("verify_B512_K4_V151936_bf16", 3, 512, 4, 151936, "bf16", 4.0, 1.3,
              1.0, (1.0,), 4),
    5: Config("cache_B256_K8_V256000_bf16", 4, 256, 8, 256000, "bf16", 3.0,
              1.1, 0.6, (0.5, 1.0), 9, 128, 0.7, 0.5, 0.3),
}


def get_config(cid: int, **overrides) -> Config:
    """Return workload `cid`, optionally with fields replaced (e.g. a smaller B)."""
    cfg = CONFIGS[cid]
    if overrides:
        cfg = dataclasses.replace(cfg, **overrides)
    return cfg


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return the bits as uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def _row_streams(seed: int, b: int):
    """Independent generators for batch row b (so any subset of rows can be drawn alone)."""
    kids = np.random.SeedSequence([seed, b]).spawn(4)
    names = ("target", "perm", "draft", "gumbel")
    return {n: np.random.Generator(np.random.PCG64(k)) for n, k in zip(names, kids)}


def _zipf_bias(V: int, s: float) -> np.ndarray:
    # bias = -s * ln(rank), ranks 1..V; the normalising constant is dropped
    return (-s * np.log(np.arange(1, V + 1, dtype=np.float64))).astype(np.float32)


def _gumbel_argmax(x: np.ndarray, g: np.random.Generator) -> np.ndarray:
    """Row-wise argmax of x + Gumbel noise: one exact draw from softmax(x) per row."""
    u = g.random(x.shape)                  # float64 in [0, 1)
    np.maximum(u, np.finfo(np.float64).tiny, out=u)
    np.log(u, out=u)
    np.negative(u, out=u)
    np.log(u, out=u)
    return np.argmax(x - u, axis=-1)


def make_uniforms(cfg: Config, u_seed: Optional[int] = None):
    """Accept uniforms u_acc [B, K] and resample uniforms u_res [B], fp32 in [0, 1).

    u_seed=None gives the workload's own uniforms; an integer gives an
    independent extra draw (for statistical tests over many seeds).
    """
    key = [cfg.seed, 1000003] if u_seed is None else [cfg.seed, 1000003, 7, u_seed]
    kids = np.random.SeedSequence(key).spawn(2)
    ga = np.random.Generator(np.random.PCG64(kids[0]))
    gr = np.random.Generator(np.random.PCG64(kids[1]))
    u_acc = ga.random((cfg.B, cfg.K), dtype=np.float32)
    u_res = gr.random(cfg.B, dtype=np.float32)
    return u_acc, u_res


def make_draft_uniforms(cfg: Config, tau: Optional[float] = None) -> np.ndarray:
    """Uniforms u [B, K] (fp32 in [0, 1)) for drawing the drafted tokens by
    inverse CDF, one stream per (workload, temperature), independent of the
    accept and resample uniforms. Used where the drafts must come from the
    sigma-reshaped draft distribution (the cache workloads); the draw itself
    is the sampler's business, not this module's."""
    tau = float(np.float32(cfg.taus[0] if tau is None else tau))
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, 424242, int(round(tau * 1000))])))
    return g.random((cfg.B, cfg.K), dtype=np.float32)


def make_inputs(cfg: Config, tau: Optional[float] = None, draw_tokens: bool = True,
                b_rows: Optional[range] = None) -> dict:
    """Generate one workload.

    Returns a dict with
      target  [B, K+1, V]  uint16 bf16 bits or float32
      draft   [B, K_d, V]  same dtype; draft = target + N(0, draft_sd^2)
      tokens  [B, K] int32 drafted tokens d_{i+1} ~ softmax(draft row i / tau)
      u_acc   [B, K] float32, u_res [B] float32
      tau     float32 temperature (as the GPU sees it)
    Every batch row has its own seeded streams, so `b_rows` (any iterable of
    batch-row indices) draws exactly those rows of the full workload.
    """
    tau = float(np.float32(cfg.taus[0] if tau is None else tau))
    B, K, V, Kd = cfg.B, cfg.K, cfg.V, cfg.K_d
    rows = list(range(B) if b_rows is None else b_rows)
    nb = len(rows)
    store = np.uint16 if cfg.dtype == "bf16" else np.float32
    target = np.empty((nb, K + 1, V), dtype=store)
    draft = np.empty((nb, Kd, V), dtype=store)
    tokens = np.zeros((nb, K), dtype=np.int32)
    bias = _zipf_bias(V, cfg.zipf_s) if cfg.zipf_s > 0 else None
    nrow_t = max(K + 1, Kd)   # draft row i sits on target row i (i <= K)
    for out_i, b in enumerate(rows):
        st = _row_streams(cfg.seed, b)
        t = st["target"].standard_normal((nrow_t, V), dtype=np.float32)
        t *= np.float32(cfg.target_sd)
        if bias is not None:
            t += st["perm"].permuted(np.broadcast_to(bias, (nrow_t, V)), axis=1)
        d = st["draft"].standard_normal((Kd, V), dtype=np.float32)
        d *= np.float32(cfg.draft_sd)
        d += t[:Kd]
        if cfg.dtype == "bf16":
            target[out_i] = f32_to_bf16_bits(t[:K + 1])
            draft[out_i] = f32_to_bf16_bits(d)
            dvals = bf16_bits_to_f32(draft[out_i])
        else:
            target[out_i], draft[out_i] = t[:K + 1], d
            dvals = d
        if draw_tokens:
            x = dvals[:K].astype(np.float64) / tau
            tokens[out_i] = _gumbel_argmax(x, st["gumbel"])
    u_acc, u_res = make_uniforms(cfg)
    return {
        "cfg": cfg, "tau": tau, "target": target, "draft": draft, "tokens": tokens,
        "rows": np.asarray(rows, dtype=np.int64),
        "u_acc": np.ascontiguousarray(u_acc[rows]), "u_res": np.ascontiguousarray(u_res[rows]),
    }


# ---------------------------------------------------------------------------
# token trees
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class TreeConfig:
    """One synthetic token-tree workload: every node at depth d has
    branching[d] children (node numbering breadth first, so parents come
    first); target and draft rows as in Config, one of each per node."""
    name: str
    seed: int
    B: int
    V: int
    dtype: str
    branching: tuple
    target_sd: float
    zipf_s: float
    draft_sd: float
    tau: float

    @property
    def parent(self) -> list:
        return tree_parent(self.branching)

    @property
    def N(self) -> int:
        return len(self.parent)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4


def tree_parent(branching) -> list:
    """Parent array of the complete tree with the given per-depth branching."""
    parent = [-1]
    level = [0]
    for k in branching:
        nxt = []
        for p in level:
            for _ in range(int(k)):
                parent.append(p)
                nxt.append(len(parent) - 1)
        level = nxt
    return parent


# The tree workload: 32 sequences over a 128256-entry vocabulary (the size of
# the main verification workload), four candidates for the first token, two
# continuations of each, then single chains to depth 4 (29 nodes).
TREE_CONFIGS = {
    "tree": TreeConfig("tree_B32_b4x2x1x1_V128256_bf16", 5, 32, 128256, "bf16", (4, 2, 1, 1),
                       2.0, 1.1, 0.5, 0.7),
}


def make_tree_inputs(cfg: TreeConfig, b_rows: Optional[range] = None, u_seed: Optional[int] = None,
                     parent: Optional[list] = None) -> dict:
    """Generate one tree workload.

    Returns target, draft [B, N, V] (uint16 bf16 bits or float32), tokens
    [B, N] int32 (node n >= 1 drawn from softmax(draft row of its parent /
    tau) with the Gumbel-max trick, siblings independently), u_acc [B, N]
    and u_res [B] float32, parent and tau. `parent` overrides the topology
    (any valid parent array); `u_seed` draws independent extra uniforms.
    """
    parent = cfg.parent if parent is None else list(parent)
    N = len(parent)
    B, V = cfg.B, cfg.V
    rows = list(range(B) if b_rows is None else b_rows)
    store = np.uint16 if cfg.dtype == "bf16" else np.float32
    target = np.empty((len(rows), N, V), dtype=store)
    draft = np.empty((len(rows), N, V), dtype=store)
    tokens = np.zeros((len(rows), N), dtype=np.int32)
    bias = _zipf_bias(V, cfg.zipf_s) if cfg.zipf_s > 0 else None
    tau = float(np.float32(cfg.tau))
    for out_i, b in enumerate(rows):
        st = _row_streams(cfg.seed + 7919, b)
        t = st["target"].standard_normal((N, V), dtype=np.float32)
        t *= np.float32(cfg.target_sd)
        if bias is not None:
            t += st["perm"].permuted(np.broadcast_to(bias, (N, V)), axis=1)
        d = st["draft"].standard_normal((N, V), dtype=np.float32)
        d *= np.float32(cfg.draft_sd)
        d += t
        if cfg.dtype == "bf16":
            target[out_i] = f32_to_bf16_bits(t)
            draft[out_i] = f32_to_bf16_bits(d)
            dvals = bf16_bits_to_f32(draft[out_i])
        else:
            target[out_i], draft[out_i] = t, d
            dvals = d
        if N > 1:
            x = dvals[np.asarray(parent[1:])].astype(np.float64) / tau
            tokens[out_i, 1:] = _gumbel_argmax(x, st["gumbel"])
    key = [cfg.seed, 1000003, 11] + ([] if u_seed is None else [u_seed])
    ga, gr = (np.random.Generator(np.random.PCG64(k)) for k in np.random.SeedSequence(key).spawn(2))
    u_acc = ga.random((B, N), dtype=np.float32)
    u_res = gr.random(B, dtype=np.float32)
    return {"cfg": cfg, "tau": tau, "parent": parent, "target": target, "draft": draft, "tokens": tokens,
            "rows": np.asarray(rows, dtype=np.int64),
            "u_acc": np.ascontiguousarray(u_acc[rows]), "u_res": np.ascontiguousarray(u_res[rows])}

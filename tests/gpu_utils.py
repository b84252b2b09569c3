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
            if a_r != a_g:
                lo = min(a_r, a_g) if a_r >= 0 and a_g >= 0 else -1
                assert lo >= 0, f"{label} row {b}: flagged mismatch {a_r} vs {a_g}"
                m = ref["acc_margin"][j][lo]
            else:
                m = ref["res_margin"][j]
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

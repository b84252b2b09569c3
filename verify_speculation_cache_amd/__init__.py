"""Python binding of libssdv (include/ssd.h): argument marshalling only.

Every call forwards torch tensors' device pointers, strides and the current
HIP stream to the C ABI; all computation runs in the library's gfx950
kernels. Output tensors are allocated here with torch.empty (plumbing), and
workspaces are zero-filled buffers cached per entry point and shape (the
library leaves their counters at zero after every call).
There is no CPU path: a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

__all__ = ["SSD_F32", "SSD_BF16", "SsdError", "lib", "ssd_fanout", "ssd_verify",
           "ssd_residual_sample", "ssd_build_cache", "ssd_cache_lookup", "ssd_draft_sample", "ssd_verify_greedy", "ssd_fanout_uniform",
           "ssd_speedup", "ssd_cache_stats", "Sigma",
           "ssd_verify_workspace_size", "ssd_residual_workspace_size",
           "ssd_build_cache_workspace_size", "ssd_draft_sample_workspace_size",
           "ssd_verify_greedy_workspace_size", "ssd_verify_tree", "ssd_verify_tree_workspace_size",
           "ssd_tree_rounds", "ssd_verify_round", "ssd_verify_round_workspace_size", "ssd_verify_noalloc",
           "ssd_noalloc_scratch_bytes", "EXPORTS",
           "library_path"]

SSD_F32, SSD_BF16 = 0, 1
SSD_MAX_K, SSD_MAX_F, SSD_MAX_TREE = 64, 64, 64
EXPORTS = ("ssd_last_error", "ssd_fanout", "ssd_verify_workspace_size", "ssd_verify",
           "ssd_residual_workspace_size", "ssd_residual_sample",
           "ssd_build_cache_workspace_size", "ssd_build_cache", "ssd_cache_lookup",
           "ssd_draft_sample_workspace_size", "ssd_draft_sample",
           "ssd_verify_greedy_workspace_size", "ssd_verify_greedy", "ssd_fanout_uniform", "ssd_speedup",
           "ssd_cache_stats", "ssd_tree_rounds", "ssd_verify_tree_workspace_size", "ssd_verify_tree",
           "ssd_verify_round_workspace_size", "ssd_verify_round", "ssd_verify_round_marked",
           "ssd_noalloc_scratch_bytes", "ssd_verify_noalloc")

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "libssdv.so")


class SsdError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"ssd status {code}: {msg}")
        self.code = code


class _RowKey(ctypes.Structure):
    _fields_ = [("key", ctypes.c_uint32), ("idx", ctypes.c_int32)]


class _Sigma(ctypes.Structure):
    _fields_ = [("C", ctypes.c_float), ("thr", ctypes.c_void_p), ("draft_stats", ctypes.c_void_p)]


_vp, _i32, _i64, _f32, _f64, _sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                    ctypes.c_float, ctypes.c_double, ctypes.c_size_t)
_SIGS = {
    "ssd_last_error": (ctypes.c_char_p, []),
    "ssd_fanout": (ctypes.c_int, [_i32, _i32, _f64, _f64, _vp]),
    "ssd_verify_workspace_size": (_sz, [_i32, _i32, _i32, ctypes.c_int]),
    "ssd_residual_workspace_size": (_sz, [_i32, _i32, _i32, ctypes.c_int]),
    "ssd_build_cache_workspace_size": (_sz, [_i32, _i32, _i32, ctypes.c_int]),
    "ssd_verify": (ctypes.c_int, [_vp, _i64, _vp, _i64, ctypes.c_int, _i32, _i32, _i32, _f32,
                                  _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "ssd_noalloc_scratch_bytes": (_sz, []),
    "ssd_verify_noalloc": (ctypes.c_int, [_vp, _i64, _vp, _i64, ctypes.c_int, _i32, _i32, _i32, _f32,
                                          _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "ssd_residual_sample": (ctypes.c_int, [_vp, _i64, _vp, _i64, ctypes.c_int, _i32, _i32, _i32,
                                           _f32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "ssd_build_cache": (ctypes.c_int, [_vp, _i64, ctypes.c_int, _i32, _i32, _i32, _f32, _vp,
                                       _vp, _vp, _vp, _vp, _sz, _vp]),
    "ssd_cache_lookup": (ctypes.c_int, [_vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "ssd_draft_sample_workspace_size": (_sz, [_i32, _i32, _i32, ctypes.c_int]),
    "ssd_verify_greedy_workspace_size": (_sz, [_i32, _i32, _i32, ctypes.c_int]),
    "ssd_fanout_uniform": (ctypes.c_int, [_i32, _i32, _vp]),
    "ssd_speedup": (ctypes.c_int, [_f64, _f64, _f64, _f64, _f64, _i32, _vp]),
    "ssd_cache_stats": (ctypes.c_int, [_vp, _vp, _i32, _i32, _vp, _vp]),
    "ssd_verify_greedy": (ctypes.c_int, [_vp, _i64, ctypes.c_int, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz,
                                         _vp]),
    "ssd_draft_sample": (ctypes.c_int, [_vp, _i64, ctypes.c_int, _i32, _i32, _i32, _f32, _vp, _vp, _vp,
                                        _vp, _sz, _vp]),
    "ssd_tree_rounds": (ctypes.c_int, [_vp, _i32]),
    "ssd_verify_round_workspace_size": (_sz, [_i32, _i32, _i32, ctypes.c_int]),
    "ssd_verify_round": (ctypes.c_int, [_vp, _i64, _vp, _i64, ctypes.c_int, _i32, _i32, _i32, _f32, _vp, _f32,
                                        _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "ssd_verify_round_marked": (ctypes.c_int, [_vp, _i64, _vp, _i64, ctypes.c_int, _i32, _i32, _i32, _f32, _vp,
                                               _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                               _vp, _vp]),
    "ssd_verify_tree_workspace_size": (_sz, [_i32, _i32, _i32, ctypes.c_int]),
    "ssd_verify_tree": (ctypes.c_int, [_vp, _i64, _vp, _i64, ctypes.c_int, _i32, _i32, _i32, _f32, _vp,
                                       _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libssdv.so (building it first only if it does not exist)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            from . import _build
            _build.build_library()
        if not os.path.exists(path):
            raise SsdError(-4, f"HIP library {path} is missing and could not be built")
        L = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(code: int):
    if code < 0:
        raise SsdError(code, lib().ssd_last_error().decode(errors="replace"))
    return code


# ---------------------------------------------------------------------------
# torch marshalling helpers
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return SSD_BF16
    if t.dtype == torch.float32:
        return SSD_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def _logits(t, name: str, min_rows: int, V: Optional[int] = None):
    if t.dim() != 3:
        raise ValueError(f"{name} must be [B, rows, V]")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.shape[1] < min_rows:
        raise ValueError(f"{name} needs at least {min_rows} rows per batch element")
    if t.stride(2) != 1 or (t.shape[1] > 1 and t.stride(1) != t.shape[2]):
        raise ValueError(f"{name}: rows must be contiguous and V apart")
    if V is not None and t.shape[2] != V:
        raise ValueError(f"{name}: vocabulary {t.shape[2]} != {V}")
    return t.data_ptr(), int(t.stride(0))


def _dev(t, dtype, shape, name):
    torch = _torch()
    if t.dtype != dtype or not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected contiguous {dtype} device tensor of shape {tuple(shape)},"
                         f" got {t.dtype} {tuple(t.shape)}")
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


_ws_cache = {}


def _workspace(nbytes: int, device, tag: tuple, stream=None):
    """A zero-filled device buffer for one (entry point, shape, dtype, stream).

    The kernels leave their completion counters at zero after each call, so a
    buffer can be reused for the same shape; a different shape uses its own
    buffer (its counters would sit where the other layout keeps data)."""
    torch = _torch()
    key = (tag, str(device), None if stream is None else stream.cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(max(nbytes, 256) + 256, dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    p = buf.data_ptr()
    off = (-p) % 256
    return ctypes.c_void_p(p + off), buf.numel() - off


class Sigma:
    """sigma_{F,C} arguments for ssd_verify / ssd_residual_sample, built by ssd_build_cache."""

    def __init__(self, C: float, thr, draft_stats):
        self.C, self.thr, self.draft_stats = float(C), thr, draft_stats

    def _c(self):
        return _Sigma(self.C, self.thr.data_ptr(), self.draft_stats.data_ptr())


# ---------------------------------------------------------------------------
# the five entry points
# ---------------------------------------------------------------------------
def ssd_verify_workspace_size(B, K, V, dtype) -> int:
    return int(lib().ssd_verify_workspace_size(B, K, V, dtype))


def ssd_residual_workspace_size(B, K, V, dtype) -> int:
    return int(lib().ssd_residual_workspace_size(B, K, V, dtype))


def ssd_build_cache_workspace_size(B, K, V, dtype) -> int:
    return int(lib().ssd_build_cache_workspace_size(B, K, V, dtype))


def ssd_fanout(n_budget: int, K: int, a_p: float, r: float) -> list:
    """Integer geometric fan-out F[0..K] (host call)."""
    arr = (ctypes.c_int32 * (K + 1))()
    _check(lib().ssd_fanout(int(n_budget), int(K), float(a_p), float(r), arr))
    return list(arr)


def ssd_verify(target, draft, draft_tokens, u_acc, u_res, tau: float, sigma: Optional[Sigma] = None,
               *, out: Optional[dict] = None, want_probs: bool = True, want_lse: bool = True,
               stream=None) -> dict:
    """Verify a batch: returns accepted [B], out_tokens [B, K+1], probs [B, K, 2],
    resid_mass [B] and row_lse [B, 2K+1] (device tensors)."""
    torch = _torch()
    B, K = int(draft_tokens.shape[0]), int(draft_tokens.shape[1])
    V = int(target.shape[2])
    dt = _dtype_code(target)
    if _dtype_code(draft) != dt:
        raise TypeError("target and draft dtypes differ")
    tp, tb = _logits(target, "target", K + 1)
    dp, db = _logits(draft, "draft", K, V)
    if target.shape[0] != B or draft.shape[0] != B:
        raise ValueError("target/draft batch size differs from draft_tokens")
    dev = target.device
    tok = _dev(draft_tokens, torch.int32, (B, K), "draft_tokens")
    ua = _dev(u_acc, torch.float32, (B, K), "u_acc")
    ur = _dev(u_res, torch.float32, (B,), "u_res")
    if out is None:
        out = {"accepted": torch.empty(B, dtype=torch.int32, device=dev),
               "out_tokens": torch.empty(B, K + 1, dtype=torch.int32, device=dev),
               "probs": torch.empty(B, K, 2, dtype=torch.float32, device=dev) if want_probs else None,
               "resid_mass": torch.empty(B, dtype=torch.float32, device=dev),
               "row_lse": torch.empty(B, 2 * K + 1, dtype=torch.float32, device=dev) if want_lse else None}
    sig = ctypes.byref(sigma._c()) if sigma is not None else None
    ws, wsz = _workspace(ssd_verify_workspace_size(B, K, V, dt), dev, ("verify", B, K, V, dt), stream)
    ptr = lambda t: None if t is None else t.data_ptr()
    _check(lib().ssd_verify(tp, tb, dp, db, dt, B, K, V, float(tau), tok, ua, ur, sig,
                            ptr(out["accepted"]), ptr(out["out_tokens"]), ptr(out.get("probs")),
                            ptr(out.get("resid_mass")), ptr(out.get("row_lse")),
                            ws, wsz, _stream(stream)))
    return out


def ssd_noalloc_scratch_bytes() -> int:
    return int(lib().ssd_noalloc_scratch_bytes())


def ssd_verify_noalloc(target, draft, draft_tokens, u_acc, u_res, tau: float, sigma: Optional[Sigma] = None,
                       *, out: dict, stream=None) -> dict:
    """ssd_verify through the entry point that allocates nothing (its workspace
    is the library's per-GPU device array). `out` holds caller-allocated
    outputs as for ssd_verify (accepted, out_tokens; probs, resid_mass,
    row_lse may be None); no device memory is allocated here either."""
    torch = _torch()
    B, K = int(draft_tokens.shape[0]), int(draft_tokens.shape[1])
    V = int(target.shape[2])
    dt = _dtype_code(target)
    if _dtype_code(draft) != dt:
        raise TypeError("target and draft dtypes differ")
    tp, tb = _logits(target, "target", K + 1)
    dp, db = _logits(draft, "draft", K, V)
    if target.shape[0] != B or draft.shape[0] != B:
        raise ValueError("target/draft batch size differs from draft_tokens")
    tok = _dev(draft_tokens, torch.int32, (B, K), "draft_tokens")
    ua = _dev(u_acc, torch.float32, (B, K), "u_acc")
    ur = _dev(u_res, torch.float32, (B,), "u_res")
    _dev(out["accepted"], torch.int32, (B,), "accepted")
    _dev(out["out_tokens"], torch.int32, (B, K + 1), "out_tokens")
    sig = ctypes.byref(sigma._c()) if sigma is not None else None
    ptr = lambda t: None if t is None else t.data_ptr()
    _check(lib().ssd_verify_noalloc(tp, tb, dp, db, dt, B, K, V, float(tau), tok, ua, ur, sig,
                                    ptr(out["accepted"]), ptr(out["out_tokens"]), ptr(out.get("probs")),
                                    ptr(out.get("resid_mass")), ptr(out.get("row_lse")), _stream(stream)))
    return out


def ssd_residual_sample(target, draft, row, u, tau: float, sigma: Optional[Sigma] = None,
                        *, stream=None) -> dict:
    """One draw per batch row from position row[b]: residual max(0, p - q) when a
    draft is given and row[b] < K, else p. Returns tokens [B] and mass [B]."""
    torch = _torch()
    B = int(row.shape[0])
    K = int(target.shape[1]) - 1
    V = int(target.shape[2])
    dt = _dtype_code(target)
    tp, tb = _logits(target, "target", 1)
    if target.shape[0] != B:
        raise ValueError("target batch size differs from row")
    if draft is not None:
        if _dtype_code(draft) != dt:
            raise TypeError("target and draft dtypes differ")
        if draft.shape[0] != B:
            raise ValueError("draft batch size differs from row")
        dp, db = _logits(draft, "draft", K, V)
    else:
        dp, db = None, 0
    dev = target.device
    rp = _dev(row, torch.int32, (B,), "row")
    up = _dev(u, torch.float32, (B,), "u")
    tok = torch.empty(B, dtype=torch.int32, device=dev)
    mass = torch.empty(B, dtype=torch.float32, device=dev)
    sig = ctypes.byref(sigma._c()) if sigma is not None else None
    ws, wsz = _workspace(ssd_residual_workspace_size(B, K, V, dt), dev, ("resid", B, K, V, dt), stream)
    _check(lib().ssd_residual_sample(tp, tb, dp, db, dt, B, K, V, float(tau), rp, sig, up,
                                     tok.data_ptr(), mass.data_ptr(), ws, wsz, _stream(stream)))
    return {"tokens": tok, "mass": mass}


def ssd_fanout_uniform(n_budget: int, K: int) -> list:
    """Uniform fan-out F[0..K] (host call)."""
    arr = (ctypes.c_int32 * (K + 1))()
    _check(lib().ssd_fanout_uniform(int(n_budget), int(K), arr))
    return list(arr)


def ssd_speedup(p_hit: float, e_hit: float, e_miss: float, t_p: float, t_b: float, batch: int = 1) -> float:
    """Expected SSD speedup with the batch all-hit probability p_hit**batch (host call)."""
    out = ctypes.c_double()
    _check(lib().ssd_speedup(float(p_hit), float(e_hit), float(e_miss), float(t_p), float(t_b), int(batch),
                             ctypes.byref(out)))
    return out.value


def ssd_cache_stats(accepted, hit, K: int, *, out=None, stream=None):
    """Per-length counts [K+1, 2] (int32 view of uint32): outcomes at length k, hits among them."""
    torch = _torch()
    B = int(accepted.shape[0])
    if out is None:
        out = torch.empty((K + 1, 2), dtype=torch.int32, device=accepted.device)
    _check(lib().ssd_cache_stats(_dev(accepted, torch.int32, (B,), "accepted"),
                                 _dev(hit, torch.uint8, (B,), "hit"), B, int(K),
                                 _dev(out, torch.int32, (K + 1, 2), "out"), _stream(stream)))
    return out


def ssd_verify_greedy_workspace_size(B, K, V, dtype) -> int:
    return int(lib().ssd_verify_greedy_workspace_size(B, K, V, dtype))


def ssd_verify_greedy(target, draft_tokens, *, out: Optional[dict] = None, stream=None) -> dict:
    """Greedy verification: returns accepted [B] and out_tokens [B, K+1]."""
    torch = _torch()
    B, K = int(draft_tokens.shape[0]), int(draft_tokens.shape[1])
    V = int(target.shape[2])
    dt = _dtype_code(target)
    if target.shape[0] != B:
        raise ValueError("target batch size differs from draft_tokens")
    tp, tb = _logits(target, "target", K + 1)
    kp = _dev(draft_tokens, torch.int32, (B, K), "draft_tokens")
    if out is None:
        out = {"accepted": torch.empty(B, dtype=torch.int32, device=target.device),
               "out_tokens": torch.empty((B, K + 1), dtype=torch.int32, device=target.device)}
    ws, wsz = _workspace(ssd_verify_greedy_workspace_size(B, K, V, dt), target.device, ("greedy", B, K, V, dt),
                         stream)
    _check(lib().ssd_verify_greedy(tp, tb, dt, B, K, V, kp, _dev(out["accepted"], torch.int32, (B,), "accepted"),
                                   _dev(out["out_tokens"], torch.int32, (B, K + 1), "out_tokens"), ws, wsz,
                                   _stream(stream)))
    return out


def ssd_draft_sample_workspace_size(B, K, V, dtype) -> int:
    return int(lib().ssd_draft_sample_workspace_size(B, K, V, dtype))


def ssd_draft_sample(draft, u, tau: float, sigma: Optional[Sigma] = None, *, out=None, stream=None):
    """Drafted tokens [B, K] int32: d[b, i] drawn from softmax(draft row i / tau),
    or its sigma form, by inverse CDF with u [B, K]."""
    torch = _torch()
    if u.dim() != 2:
        raise ValueError("u must be [B, K]")
    B, K = int(u.shape[0]), int(u.shape[1])
    V = int(draft.shape[2])
    dt = _dtype_code(draft)
    if draft.shape[0] != B:
        raise ValueError("draft batch size differs from u")
    dp, db = _logits(draft, "draft", K)
    up = _dev(u, torch.float32, (B, K), "u")
    if out is None:
        out = torch.empty((B, K), dtype=torch.int32, device=draft.device)
    _dev(out, torch.int32, (B, K), "out")
    sig = ctypes.byref(sigma._c()) if sigma is not None else None
    ws, wsz = _workspace(ssd_draft_sample_workspace_size(B, K, V, dt), draft.device, ("sample", B, K, V, dt), stream)
    _check(lib().ssd_draft_sample(dp, db, dt, B, K, V, float(tau), sig, up, out.data_ptr(), ws, wsz,
                                  _stream(stream)))
    return out


def ssd_build_cache(draft, tau: float, F: Sequence[int], *, out: Optional[dict] = None,
                    stream=None) -> dict:
    """Top-F_k draft tokens per acceptance length k = 0..K plus sigma statistics.
    Returns cache_tokens [B, sum F] int32, thr [B, K+1, 2] int32 (key bits, index)
    and draft_stats [B, K+1, 3] float64."""
    torch = _torch()
    K = len(F) - 1
    B, V = int(draft.shape[0]), int(draft.shape[2])
    dt = _dtype_code(draft)
    dp, db = _logits(draft, "draft", K + 1)
    dev = draft.device
    sumF = int(sum(F))
    if len(F) < 2:
        raise ValueError("F needs K+1 >= 2 entries")
    if out is None:
        out = {"cache_tokens": torch.empty(B, sumF, dtype=torch.int32, device=dev),
               "thr": torch.empty(B, K + 1, 2, dtype=torch.int32, device=dev),
               "draft_stats": torch.empty(B, K + 1, 3, dtype=torch.float64, device=dev)}
    Fa = (ctypes.c_int32 * (K + 1))(*[int(f) for f in F])
    ws, wsz = _workspace(ssd_build_cache_workspace_size(B, K, V, dt), dev, ("cache", B, K, V, dt), stream)
    _check(lib().ssd_build_cache(
        dp, db, dt, B, K, V, float(tau), Fa,
        _dev(out["cache_tokens"], torch.int32, (B, sumF), "cache_tokens") if sumF > 0 else None,
        _dev(out["thr"], torch.int32, (B, K + 1, 2), "thr"),
        _dev(out["draft_stats"], torch.float64, (B, K + 1, 3), "draft_stats"), ws, wsz, _stream(stream)))
    out["F"] = list(F)
    return out


def ssd_cache_lookup(cache_tokens, F: Sequence[int], accepted, out_tokens, *, out=None,
                     stream=None) -> dict:
    """Hit flag [B] uint8 and slot [B] int32 of the realised outcome (a, t*)."""
    torch = _torch()
    K = len(F) - 1
    B = int(accepted.shape[0])
    dev = accepted.device
    if cache_tokens.dim() != 2 or cache_tokens.shape[0] != B or cache_tokens.shape[1] != sum(F):
        raise ValueError("cache_tokens must be [B, sum F] (row stride sum F)")
    if not cache_tokens.is_contiguous() or cache_tokens.dtype != torch.int32:
        raise ValueError("cache_tokens must be contiguous int32")
    if out is None:
        out = {"hit": torch.empty(B, dtype=torch.uint8, device=dev),
               "slot": torch.empty(B, dtype=torch.int32, device=dev)}
    Fa = (ctypes.c_int32 * (K + 1))(*[int(f) for f in F])
    _check(lib().ssd_cache_lookup(cache_tokens.data_ptr() if sum(F) > 0 else None, Fa, B, K,
                                  _dev(accepted, torch.int32, (B,), "accepted"),
                                  _dev(out_tokens, torch.int32, (B, K + 1), "out_tokens"),
                                  out["hit"].data_ptr(), out["slot"].data_ptr(), _stream(stream)))
    return out


def sigma_from_cache(cache: dict, C: float) -> Sigma:
    return Sigma(C, cache["thr"], cache["draft_stats"])


def _parent_array(parent: Sequence[int]):
    N = len(parent)
    return (ctypes.c_int32 * max(N, 1))(*[int(x) for x in parent]), N


def ssd_tree_rounds(parent: Sequence[int]) -> int:
    """Round kernels ssd_verify_tree launches for this topology."""
    arr, N = _parent_array(parent)
    return _check(lib().ssd_tree_rounds(arr, N))


def ssd_verify_tree_workspace_size(B, N, V, dtype) -> int:
    return int(lib().ssd_verify_tree_workspace_size(B, N, V, dtype))


def ssd_verify_tree(target, draft, parent: Sequence[int], tokens, u_acc, u_res, tau: float, *,
                    out: Optional[dict] = None, stream=None) -> dict:
    """Token-tree verification. target/draft [B, N, V] (one row per node),
    parent: host list of N ints (parent[0] = -1), tokens [B, N] int32,
    u_acc [B, N] and u_res [B] float32. Returns accepted [B], out_tokens
    [B, N] and out_nodes [B, N]."""
    torch = _torch()
    arr, N = _parent_array(parent)
    if tokens.dim() != 2 or tokens.shape[1] != N:
        raise ValueError("tokens must be [B, N] with N = len(parent)")
    B = int(tokens.shape[0])
    V = int(target.shape[2])
    dt = _dtype_code(target)
    if target.shape[0] != B or target.shape[1] != N:
        raise ValueError("target must be [B, N, V]")
    tp, tb = _logits(target, "target", N)
    dp, db = None, 0
    if draft is not None:
        if _dtype_code(draft) != dt:
            raise ValueError("target and draft dtypes differ")
        if draft.shape[0] != B or draft.shape[1] != N:
            raise ValueError("draft must be [B, N, V]")
        dp, db = _logits(draft, "draft", N, V)
    kp = _dev(tokens, torch.int32, (B, N), "tokens")
    ua = _dev(u_acc, torch.float32, (B, N), "u_acc")
    ur = _dev(u_res, torch.float32, (B,), "u_res")
    if out is None:
        out = {"accepted": torch.empty(B, dtype=torch.int32, device=target.device),
               "out_tokens": torch.empty((B, N), dtype=torch.int32, device=target.device),
               "out_nodes": torch.empty((B, N), dtype=torch.int32, device=target.device)}
    nodes = out.get("out_nodes")
    ws, wsz = _workspace(ssd_verify_tree_workspace_size(B, N, V, dt), target.device, ("tree", B, N, V, dt), stream)
    _check(lib().ssd_verify_tree(tp, tb, dp, db, dt, B, N, V, float(tau), arr, kp, ua, ur,
                                 _dev(out["accepted"], torch.int32, (B,), "accepted"),
                                 _dev(out["out_tokens"], torch.int32, (B, N), "out_tokens"),
                                 None if nodes is None else _dev(nodes, torch.int32, (B, N), "out_nodes"),
                                 ws, wsz, _stream(stream)))
    return out


def ssd_verify_round_workspace_size(B, K, V, dtype) -> int:
    return int(lib().ssd_verify_round_workspace_size(B, K, V, dtype))


def ssd_verify_round(target, draft, F: Sequence[int], C: float, draft_tokens, u_acc, u_res, tau: float, *,
                     out: Optional[dict] = None, stream=None, marks=None) -> dict:
    """One verification round with the speculation cache: cache build on
    draft rows 0..K, sigma verification, and the hit of the outcome, in three
    launches. Returns the outputs of ssd_build_cache, ssd_verify and
    ssd_cache_lookup in one dict. marks: optional four torch.cuda.Event
    objects, recorded before the chunk pass and after each launch
    (ssd_verify_round_marked)."""
    torch = _torch()
    B, K = int(draft_tokens.shape[0]), int(draft_tokens.shape[1])
    V = int(target.shape[2])
    dt = _dtype_code(target)
    if _dtype_code(draft) != dt:
        raise ValueError("target and draft dtypes differ")
    if target.shape[0] != B or draft.shape[0] != B:
        raise ValueError("batch sizes differ")
    if len(F) != K + 1:
        raise ValueError("F needs K+1 entries")
    tp, tb = _logits(target, "target", K + 1)
    dp, db = _logits(draft, "draft", K + 1, V)
    Fa = (ctypes.c_int32 * (K + 1))(*[int(f) for f in F])
    sumF = int(sum(F))
    dev = target.device
    if out is None:
        out = {"cache_tokens": torch.empty((B, sumF), dtype=torch.int32, device=dev),
               "thr": torch.empty((B, K + 1, 2), dtype=torch.int32, device=dev),
               "draft_stats": torch.empty((B, K + 1, 3), dtype=torch.float64, device=dev),
               "accepted": torch.empty(B, dtype=torch.int32, device=dev),
               "out_tokens": torch.empty((B, K + 1), dtype=torch.int32, device=dev),
               "hit": torch.empty(B, dtype=torch.uint8, device=dev),
               "slot": torch.empty(B, dtype=torch.int32, device=dev)}
    ws, wsz = _workspace(ssd_verify_round_workspace_size(B, K, V, dt), dev, ("round", B, K, V, dt), stream)
    mk = None
    if marks is not None:
        if len(marks) != 4:
            raise ValueError("marks: four events")
        for ev in marks:
            if ev.cuda_event == 0:   # torch creates an event at its first record
                ev.record(torch.cuda.current_stream() if stream is None else stream)
        mk = (ctypes.c_void_p * 4)(*[ctypes.c_void_p(ev.cuda_event) for ev in marks])
    fn = lib().ssd_verify_round if mk is None else (
        lambda *args: lib().ssd_verify_round_marked(*args, mk))
    _check(fn(
        tp, tb, dp, db, dt, B, K, V, float(tau), Fa, float(C),
        _dev(draft_tokens, torch.int32, (B, K), "draft_tokens"), _dev(u_acc, torch.float32, (B, K), "u_acc"),
        _dev(u_res, torch.float32, (B,), "u_res"),
        _dev(out["cache_tokens"], torch.int32, (B, sumF), "cache_tokens") if sumF > 0 else None,
        _dev(out["thr"], torch.int32, (B, K + 1, 2), "thr"),
        _dev(out["draft_stats"], torch.float64, (B, K + 1, 3), "draft_stats"),
        _dev(out["accepted"], torch.int32, (B,), "accepted"),
        _dev(out["out_tokens"], torch.int32, (B, K + 1), "out_tokens"),
        _dev(out["hit"], torch.uint8, (B,), "hit"),
        _dev(out["slot"], torch.int32, (B,), "slot") if out.get("slot") is not None else None,
        ws, wsz, _stream(stream)))
    return out

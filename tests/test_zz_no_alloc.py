"""ssd_verify_noalloc (the entry point that allocates nothing) against ssd_verify.

Its kernels are ssd_verify's and its workspace is the library's per-GPU
device array, cleared by a fill kernel on every call, so its outputs must
equal ssd_verify's bit for bit, on consecutive calls of different shapes
(the second smaller, laid out over what the first left behind), plain and
with sigma; a shape whose workspace exceeds the array is refused.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_utils import fvec, ivec, log, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import verify_speculation_cache_amd as lib
    lib.lib()
    return lib


def _case(seed, B, K, V, dtype, tau):
    rng = np.random.default_rng(seed)
    t = (rng.standard_normal((B, K + 1, V)) * 2.5).astype(np.float32)
    d = (t + rng.standard_normal((B, K + 1, V)).astype(np.float32) * 0.7).astype(np.float32)
    if dtype == "bf16":
        t, d = W.f32_to_bf16_bits(t), W.f32_to_bf16_bits(d)
    toks = np.array([[O.sample_draft(d[b, i], tau, rng.random()) for i in range(K)] for b in range(B)],
                    dtype=np.int32)
    return {"target": t, "draft": d, "tokens": toks, "u_acc": rng.random((B, K)).astype(np.float32),
            "u_res": rng.random(B).astype(np.float32), "tau": float(np.float32(tau))}


def _outputs(B, K, dev):
    return {"accepted": torch.full((B,), -7, dtype=torch.int32, device=dev),
            "out_tokens": torch.full((B, K + 1), -7, dtype=torch.int32, device=dev),
            "probs": torch.full((B, K, 2), -7.0, dtype=torch.float32, device=dev),
            "resid_mass": torch.full((B,), -7.0, dtype=torch.float32, device=dev),
            "row_lse": torch.full((B, 2 * K + 1), -7.0, dtype=torch.float32, device=dev)}


@pytest.mark.parametrize("sigma", [False, True])
def test_noalloc_equals_verify_on_consecutive_calls(S, sigma):
    assert S.ssd_noalloc_scratch_bytes() == 16 << 20
    dev = torch.device("cuda:0")
    # the second call is smaller; the third returns to the first shape
    for (seed, B, K, V, dtype) in ((11, 48, 6, 70000, "bf16"), (12, 5, 2, 9001, "f32"), (13, 48, 6, 70000, "bf16")):
        log(f"[gpu] noalloc sigma={sigma} B={B} K={K} V={V} {dtype}")
        d = _case(seed, B, K, V, dtype, 0.8)
        tgt, dft = to_dev(d["target"], torch), to_dev(d["draft"], torch)
        toks, ua, ur = ivec(d["tokens"], torch), fvec(d["u_acc"], torch), fvec(d["u_res"], torch)
        sg = None
        if sigma:
            F = [min(f, 64) for f in S.ssd_fanout(40, K, 0.75, 1.0)]
            sg = S.sigma_from_cache(S.ssd_build_cache(dft, d["tau"], F), 0.4)
        want = S.ssd_verify(tgt, dft, toks, ua, ur, d["tau"], sg)
        out = _outputs(B, K, dev)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated(dev)
        S.ssd_verify_noalloc(tgt, dft, toks, ua, ur, d["tau"], sg, out=out)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated(dev) == before
        for k in ("accepted", "out_tokens", "probs", "resid_mass", "row_lse"):
            assert torch.equal(out[k], want[k]), (k, B, K, V)
        assert (out["accepted"] >= 0).all()


def test_noalloc_outputs_optional_and_refuses_oversize(S):
    dev = torch.device("cuda:0")
    d = _case(21, 7, 3, 4000, "bf16", 1.0)
    tgt, dft = to_dev(d["target"], torch), to_dev(d["draft"], torch)
    toks, ua, ur = ivec(d["tokens"], torch), fvec(d["u_acc"], torch), fvec(d["u_res"], torch)
    want = S.ssd_verify(tgt, dft, toks, ua, ur, d["tau"])
    out = {"accepted": torch.empty(7, dtype=torch.int32, device=dev),
           "out_tokens": torch.empty(7, 4, dtype=torch.int32, device=dev)}
    S.ssd_verify_noalloc(tgt, dft, toks, ua, ur, d["tau"], out=out)
    torch.cuda.synchronize()
    assert torch.equal(out["accepted"], want["accepted"]) and torch.equal(out["out_tokens"], want["out_tokens"])
    # a batch whose workspace exceeds the array: refused on the host, nothing launched
    B, K, V = 1 << 15, 64, 1 << 20
    assert S.ssd_verify_workspace_size(B, K, V, S.SSD_BF16) > S.ssd_noalloc_scratch_bytes()
    big_t = tgt[:1].expand(B, -1, -1)
    big_tok = torch.zeros(B, 3, dtype=torch.int32, device=dev)
    with pytest.raises(S.SsdError, match="above its"):
        import ctypes
        rc = S.lib().ssd_verify_noalloc(big_t.data_ptr(), 0, dft.data_ptr(), 0, S.SSD_BF16, B, K, V,
                                        ctypes.c_float(1.0), big_tok.data_ptr(), ua.data_ptr(), ur.data_ptr(), None,
                                        out["accepted"].data_ptr(), out["out_tokens"].data_ptr(), None, None, None,
                                        None)
        S._check(rc)

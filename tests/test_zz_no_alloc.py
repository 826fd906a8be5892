"""The allocation-free flat top-k (tks_topk_flat_static: the workspace is a
static device array of the library) against the workspace entry point
(tks_topk_flat), called directly through the C ABI: two calls in a row,
the second with a smaller input of the other form (fused decode, then a
tiled prefill), must give the same indices and values bit for bit; a call
whose workspace would exceed the static array is refused before any
launch and leaves its outputs untouched."""
import ctypes

import numpy as np
import pytest
import torch

from tks_inputs import fp32_to_bf16_bits, fp32_to_e4m3fn
from top_key_selection_amd import tks

pytestmark = pytest.mark.gpu


def say(msg):
    print("[case] " + msg, flush=True)


def _inputs(seed, batch, n_q, n_k, heads, dim, fp8, floats):
    rng = np.random.default_rng(seed)
    if floats:
        q = rng.standard_normal((batch, n_q, heads, dim)).astype(np.float32)
        w = (rng.standard_normal((batch, n_q, heads)) / 8).astype(np.float32)
        z = rng.standard_normal((batch, n_k, dim)).astype(np.float32)
    else:
        q = rng.integers(-4, 5, (batch, n_q, heads, dim)).astype(np.float32)
        w = rng.integers(-4, 5, (batch, n_q, heads)).astype(np.float32)
        z = rng.integers(-4, 5, (batch, n_k, dim)).astype(np.float32)
    qd = torch.from_numpy(fp32_to_bf16_bits(q).view(np.int16)).view(torch.bfloat16).cuda()
    wd = torch.from_numpy(w).cuda()
    if fp8:
        ks = (np.abs(z).max(axis=2) / 448.0).astype(np.float32) if floats else \
            np.ones((batch, n_k), np.float32)
        kd = torch.from_numpy(fp32_to_e4m3fn(z / ks[..., None])).cuda()
        ksd = torch.from_numpy(ks).cuda()
    else:
        kd = torch.from_numpy(fp32_to_bf16_bits(z).view(np.int16)).view(torch.bfloat16).cuda()
        ksd = None
    return qd, wd, kd, ksd


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _static(S, q, w, k, ks, topk, qc, kt, idx, vals):
    c = S.c()
    return tks.lib().tks_topk_flat_static(ctypes.byref(c), _p(q), _p(w), _p(k), _p(ks), topk, qc, kt,
                                          _p(idx), _p(vals), ctypes.c_void_p(
                                              torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("case", [
    # (batch, n_q, n_k, heads, dim, fp8, floats, topk, q_chunk, k_tile, q_pos0)
    ("decode 64 x 30000 fp8 floats, fused", (64, 1, 30000, 64, 128, True, True, 2048, 0, 0, 29999)),
    ("prefill 2 x 300 bf16 integers, tiled (smaller)", (2, 300, 300, 8, 64, False, False, 40, 128, 96, 0)),
])
def test_static_scratch_equals_workspace_entry_point(case):
    what, (B, NQ, NK, H, D, fp8, floats, K, qc, kt, q0) = case
    say("static scratch: " + what)
    S = tks.Shape(B, NQ, NK, H, D, q_pos0=q0, key_dtype=tks.KEY_FP8_E4M3FN if fp8 else tks.KEY_BF16)
    assert tks.topk_flat_workspace(S, K, qc, kt) <= tks.STATIC_SCRATCH_BYTES
    q, w, k, ks = _inputs(len(what), B, NQ, NK, H, D, fp8, floats)
    ref_i, ref_v = tks.topk_flat(S, q, w, k, ks, K, qc, kt)
    got_i = torch.full_like(ref_i, -7)
    got_v = torch.full_like(ref_v, -7.0)
    assert _static(S, q, w, k, ks, K, qc, kt, got_i, got_v) == tks.OK, tks.last_error()
    torch.cuda.synchronize()
    assert torch.equal(got_i, ref_i)
    assert torch.equal(got_v.view(torch.int32), ref_v.view(torch.int32))


def test_static_scratch_refuses_a_workspace_beyond_it():
    say("static scratch: oversized call refused before launch")
    S = tks.Shape(1, 8192, 8192, 4, 32)
    assert tks.topk_flat_workspace(S, 2048) > tks.STATIC_SCRATCH_BYTES
    q, w, k, ks = _inputs(5, 1, 8192, 8192, 4, 32, False, True)
    idx = torch.full((1, 8192, 2048), -7, dtype=torch.int32, device="cuda")
    assert _static(S, q, w, k, ks, 2048, 0, 0, idx, None) == tks.EWORKSPACE
    assert "static scratch" in tks.last_error()
    torch.cuda.synchronize()
    assert bool((idx == -7).all())

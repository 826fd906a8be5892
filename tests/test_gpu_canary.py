"""Guard bands around everything the library writes: each output, cache
and workspace a call gets is a view into a larger device buffer whose first
and last 256 bytes hold a fixed byte pattern, and after the call the bands
must be unchanged (a kernel that writes past its buffer would change them).
Every entry point is covered, with each form of the flat top-k (fused,
tiled, static scratch) and of the refinement (planned ring, key-segment
ring, per-row block scoring).  A second test runs calls with TKS_DEBUG_SYNC=1
(a synchronisation after every launch) and checks that they succeed with
the same results."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from helpers import host
from tks_inputs import FORCE_FIRST, FORCE_LOCAL, fp32_to_bf16_bits, fp32_to_e4m3fn
from top_key_selection_amd import tks

pytestmark = pytest.mark.gpu

GUARD = 256      # bytes on each side (views stay 256-byte aligned)
PATTERN = 0xA5


def say(msg):
    print("[case] " + msg, flush=True)


class Guarded:
    """A device tensor of the given shape and dtype inside guard bands."""

    def __init__(self, shape, dtype, fill=None):
        self.nbytes = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        self.raw = torch.full((self.nbytes + 2 * GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.t = self.raw[GUARD:GUARD + self.nbytes].view(dtype).view(shape)
        if fill is not None:
            self.t.copy_(fill)

    def intact(self):
        r = self.raw.cpu().numpy()
        return bool((r[:GUARD] == PATTERN).all() and (r[GUARD + self.nbytes:] == PATTERN).all())


def ws_of(nbytes):
    return Guarded((max(int(nbytes), 1),), torch.uint8)


def check(**bufs):
    torch.cuda.synchronize()
    bad = [name for name, g in bufs.items() if g is not None and not g.intact()]
    assert not bad, "guard bands written: " + ", ".join(bad)


def ints(rng, shape, lo=-2, hi=2):
    return rng.integers(lo, hi + 1, shape).astype(np.float32)


def dev(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(a).cuda()


def inputs(seed, batch, n_q, n_k, heads, dim, fp8=False):
    rng = np.random.default_rng(seed)
    q = fp32_to_bf16_bits(ints(rng, (batch, n_q, heads, dim)))
    w = ints(rng, (batch, n_q, heads))
    kv = ints(rng, (batch, n_k, dim))
    if fp8:
        k, ks = fp32_to_e4m3fn(kv), (2.0 ** rng.integers(-3, 2, (batch, n_k))).astype(np.float32)
    else:
        k, ks = fp32_to_bf16_bits(kv), None
    return dev(q), dev(w), dev(k), dev(ks)


@pytest.mark.parametrize("form", ["fused", "tiled", "static"])
def test_flat_topk_writes_inside_its_buffers(form):
    say("guard bands, flat top-k, %s form" % form)
    if form == "tiled":
        S = tks.Shape(1, 300, 3000, 8, 64, q_pos0=2700)
        q, w, k, ks = inputs(1, 1, 300, 3000, 8, 64)
        qc, kt, topk = 100, 1024, 200
    else:
        S = tks.Shape(4, 1, 9000, 64, 128, q_pos0=8999, key_dtype=tks.KEY_FP8_E4M3FN)
        q, w, k, ks = inputs(2, 4, 1, 9000, 64, 128, fp8=True)
        qc, kt, topk = 0, 0, 2048
    rows = S.batch * S.n_q
    idx = Guarded((S.batch, S.n_q, topk), torch.int32)
    vals = Guarded((S.batch, S.n_q, topk), torch.float32)
    if form == "static":
        tks.topk_flat_static(S, q, w, k, ks, topk, qc, kt, idx=idx.t, vals=vals.t)
        check(idx=idx, vals=vals)
    else:
        ws = ws_of(tks.topk_flat_workspace(S, topk, qc, kt))
        tks.topk_flat(S, q, w, k, ks, topk, qc, kt, ws=ws.t, idx=idx.t, vals=vals.t)
        check(idx=idx, vals=vals, ws=ws)
    assert (host(idx.t).reshape(rows, topk)[:, 0] >= 0).all()


def test_scores_topk_pool_and_block_select_write_inside_their_buffers():
    say("guard bands, indexer scores, top-k of scores, pooling, block select")
    S = tks.Shape(2, 40, 1000, 8, 64, q_pos0=960)
    q, w, k, ks = inputs(3, 2, 40, 1000, 8, 64)
    out = Guarded((2, 17, 301), torch.float32)
    tks.indexer_scores(S, q, w, k, ks, 5, 17, 600, 301, out=out.t)
    scores = torch.randn(37, 5000, device="cuda")
    idx = Guarded((37, 300), torch.int32)
    vals = Guarded((37, 300), torch.float32)
    ws = ws_of(tks.topk_scores_workspace(37, 5000, 300))
    tks.topk_scores(scores, 300, ws=ws.t, idx=idx.t, vals=vals.t)
    pooled = Guarded((2, 1000 // 64, 64), torch.bfloat16)
    tks.hisa_pool_keys(S, k, ks, 64, pooled=pooled.t)
    m_total = tks.m_total_of(5, FORCE_FIRST | FORCE_LOCAL)
    blk = Guarded((2, 40, m_total), torch.int32)
    bv = Guarded((2, 40, m_total), torch.float32)
    bws = ws_of(tks.hisa_block_select_workspace(S, 64, 5))
    tks.hisa_block_select(S, q, w, pooled.t, 64, 5, FORCE_FIRST | FORCE_LOCAL, ws=bws.t, blk=blk.t,
                          blk_vals=bv.t)
    check(scores=out, idx=idx, vals=vals, ws=ws, pooled=pooled, blk=blk, blk_vals=bv, block_ws=bws)


@pytest.mark.parametrize("form", ["planned", "segments", "per_row"])
def test_refinement_writes_inside_its_buffers(form):
    say("guard bands, refinement, %s form" % form)
    if form == "planned":      # bf16 keys, D = 128, prefill: plans and the shared ring
        batch, n_q, n_k, heads, dim, block, m = 2, 300, 3000, 64, 128, 64, 6
    elif form == "segments":   # a union too large for a plan: the key-segment ring
        batch, n_q, n_k, heads, dim, block, m = 1, 24, 40000, 16, 128, 32, 148
    else:                      # D = 64: per-row block scoring
        batch, n_q, n_k, heads, dim, block, m = 2, 40, 1000, 8, 64, 64, 5
    S = tks.Shape(batch, n_q, n_k, heads, dim, q_pos0=n_k - n_q)
    q, w, k, ks = inputs(4, batch, n_q, n_k, heads, dim)
    blk = tks.hisa_topk(S, q, w, k, ks, block, m, FORCE_FIRST | FORCE_LOCAL, 64)[2]
    topk = 256
    idx = Guarded((batch, n_q, topk), torch.int32)
    vals = Guarded((batch, n_q, topk), torch.float32)
    ws = ws_of(tks.hisa_refine_workspace(S, block, blk.shape[-1], topk, 0))
    tks.hisa_refine_topk(S, q, w, k, ks, block, blk, topk, ws=ws.t, idx=idx.t, vals=vals.t)
    check(idx=idx, vals=vals, ws=ws)


def test_append_gather_and_attention_write_inside_their_buffers():
    say("guard bands, key append, gather, sparse attention")
    rng = np.random.default_rng(5)
    batch, n_k, dim, ratio, block = 2, 512, 128, 4, 32
    S = tks.Shape(batch, 1, n_k, 8, dim, q_pos0=n_k - 1, causal_ratio=ratio,
                  key_dtype=tks.KEY_FP8_E4M3FN)
    raw = dev(fp32_to_bf16_bits(ints(rng, (batch, n_k * ratio, dim))))
    k = Guarded((batch, n_k, dim), torch.uint8, fill=torch.zeros((batch, n_k, dim), dtype=torch.uint8))
    kscale = Guarded((batch, n_k), torch.float32, fill=torch.zeros((batch, n_k)))
    tail = Guarded((batch, ratio, dim), torch.bfloat16,
                   fill=torch.zeros((batch, ratio, dim), dtype=torch.bfloat16))
    pooled = Guarded((batch, n_k // block, dim), torch.bfloat16,
                     fill=torch.zeros((batch, n_k // block, dim), dtype=torch.bfloat16))
    done = 0
    for n in (7, 1, 300, 1, 1739):   # ragged appends, the last one fills the cache
        tks.kv_append(S, raw[:, done:done + n].contiguous(), done, k.t, kscale.t, tail.t, block,
                      pooled.t)
        done += n
    check(k=k, k_scale=kscale, raw_tail=tail, pooled=pooled)
    kv = dev(fp32_to_bf16_bits(ints(rng, (batch, 700, 576))))
    sel = torch.from_numpy(rng.integers(-1, 700, (batch, 3, 50)).astype(np.int32)).cuda()
    out = Guarded((batch, 3, 50, 576), torch.bfloat16)
    tks.gather_selected(kv, sel, out=out.t)
    qa = dev(fp32_to_bf16_bits(ints(rng, (batch, 3, 16, 128))))
    ka = dev(fp32_to_bf16_bits(ints(rng, (batch, 700, 128))))
    va = dev(fp32_to_bf16_bits(ints(rng, (batch, 700, 128))))
    att = Guarded((batch, 3, 16, 128), torch.float32)
    aws = ws_of(tks.sparse_attention_workspace(batch, 3, 16, 50))
    tks.sparse_attention(qa, ka, va, sel, 0.1, out=att.t, ws=aws.t)
    check(gather_out=out, attention_out=att, attention_ws=aws)


_SYNC_CHILD = r"""
import sys, numpy as np, torch
sys.path.insert(0, %r); sys.path.insert(0, %r)
from top_key_selection_amd import tks
from tks_inputs import FORCE_FIRST, FORCE_LOCAL, fp32_to_bf16_bits
rng = np.random.default_rng(9)
f = lambda s: torch.from_numpy(fp32_to_bf16_bits(rng.integers(-2, 3, s).astype(np.float32)).view(np.int16)).cuda()
q, k = f((2, 300, 64, 128)), f((2, 3000, 128))
w = torch.from_numpy(rng.integers(-2, 3, (2, 300, 64)).astype(np.float32)).cuda()
S = tks.Shape(2, 300, 3000, 64, 128, q_pos0=2700)
fi, fv = tks.topk_flat(S, q, w, k, None, 256)
hi, hv, hb = tks.hisa_topk(S, q, w, k, None, 64, 6, FORCE_FIRST | FORCE_LOCAL, 256)
torch.cuda.synchronize()
out = [t.cpu().numpy() for t in (fi, fv, hi, hv, hb)]
np.savez(sys.argv[1], *out)
print("child ok", flush=True)
"""


def test_debug_sync_mode_gives_the_same_results(tmp_path):
    """TKS_DEBUG_SYNC=1 synchronises after every launch; the calls must
    succeed and give bit-identical outputs (two child processes, one with
    the switch, one without)."""
    say("TKS_DEBUG_SYNC=1 against the default mode (child processes)")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    script = _SYNC_CHILD % (root, os.path.join(root, "tests"))
    res = {}
    for mode in ("0", "1"):
        path = str(tmp_path / ("out_%s.npz" % mode))
        env = dict(os.environ, TKS_DEBUG_SYNC=mode)
        r = subprocess.run([sys.executable, "-c", script, path], env=env, capture_output=True,
                           text=True, timeout=240)
        assert r.returncode == 0 and "child ok" in r.stdout, r.stdout + r.stderr
        res[mode] = np.load(path)
    for key in res["0"].files:
        np.testing.assert_array_equal(res["0"][key].view(np.uint8), res["1"][key].view(np.uint8))

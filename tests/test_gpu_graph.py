"""A decode step captured as a HIP graph and replayed: every replay, with
other work on the GPU in between, must give the eager launches' outputs
bit for bit (flat top-k through the few-long-rows selection, pooling,
block select, refinement)."""
import numpy as np
import pytest
import torch

from test_gpu_small import gpu_inputs, int_case, say
from tks_inputs import FORCE_FIRST, FORCE_LOCAL
from top_key_selection_amd import tks

pytestmark = pytest.mark.gpu


def test_decode_step_graph_replays_match_eager():
    say("HIP graph replay of a decode step, fp8, 8 x 20000 keys")
    n_k, heads, dim, K, B = 20000, 16, 128, 300, 128
    sh, x = int_case(70, batch=8, n_q=1, n_k=n_k, heads=heads, dim=dim, q_pos0=n_k - 1, fp8=True)
    S = tks.Shape(**sh)
    q, w, k, ks = gpu_inputs(x)
    m_scored, force = 20, FORCE_FIRST | FORCE_LOCAL
    mt = m_scored + 2
    f_idx = torch.empty((8, 1, K), dtype=torch.int32, device="cuda")
    f_val = torch.empty((8, 1, K), dtype=torch.float32, device="cuda")
    f_ws = tks.workspace(tks.topk_flat_workspace(S, K))
    pooled = torch.empty((8, n_k // B, dim), dtype=torch.bfloat16, device="cuda")
    blk = torch.empty((8, 1, mt), dtype=torch.int32, device="cuda")
    b_ws = tks.workspace(tks.hisa_block_select_workspace(S, B, m_scored))
    h_idx = torch.empty_like(f_idx)
    h_val = torch.empty_like(f_val)
    r_ws = tks.workspace(tks.hisa_refine_workspace(S, B, mt, K))

    def step():
        tks.topk_flat(S, q, w, k, ks, K, ws=f_ws, idx=f_idx, vals=f_val)
        tks.hisa_pool_keys(S, k, ks, B, pooled=pooled)
        tks.hisa_block_select(S, q, w, pooled, B, m_scored, force, with_vals=False, ws=b_ws, blk=blk)
        tks.hisa_refine_topk(S, q, w, k, ks, B, blk, K, ws=r_ws, idx=h_idx, vals=h_val)

    outs = [f_idx, f_val, pooled, blk, h_idx, h_val]
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()

    # other work between replays: an unrelated top-k on different scores
    other = torch.randn(3, 50000, device="cuda")
    for rep in range(4):
        for t in outs:
            t.fill_(0) if t.dtype == torch.bfloat16 else t.fill_(-7)
        tks.topk_scores(other, 100)
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            if a.dtype == torch.float32:
                a, b = torch.nan_to_num(a, nan=-9.0), torch.nan_to_num(b, nan=-9.0)
            elif a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), "replay %d output %d differs" % (rep, i)
    del g

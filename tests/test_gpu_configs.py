"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times.  The oracle recomputes a deterministic row sample (first /
last rows, rows around topk-1 and block / chunk boundaries, the rest
uniform); float outputs use the tolerance comparator, pooled keys are
compared bit for bit.  HISA is checked in two stages: the block lists
(tolerance on block scores), then the tokens of rows whose block list
matches the oracle's; the refinement is also run on the oracle's block list
so it is compared on every sampled row."""
import numpy as np
import pytest
import torch

import oracle
from helpers import cfg_rows, check_topk_float, dev, host, iou
from tks_inputs import CONFIGS, gen_keys, gen_q, gen_q_rows, gen_w, gen_w_rows, make_inputs, \
    sample_rows
from top_key_selection_amd import tks

pytestmark = pytest.mark.gpu


def say(msg):
    print("[case] " + msg, flush=True)


def upload(cfg):
    k, ks = gen_keys(cfg)
    q = gen_q(cfg)
    w = gen_w(cfg)
    return dict(q=q, w=w, k=k, k_scale=ks), (dev(q), dev(w), dev(k), dev(ks))


def flat_check(cfg, x, gi, gv, rows, what):
    qr, wr = cfg_rows(cfg, x, rows) if x.get("q") is not None else \
        (gen_q_rows(cfg, rows), gen_w_rows(cfg, rows))
    sh = cfg.shape_dict()
    oi, ov = oracle.topk_flat(sh, qr, wr, x["k"], x["k_scale"], cfg.topk, rows)
    rs = oracle.row_scores(sh, qr, wr, x["k"], x["k_scale"], rows)
    rec = check_topk_float(gi[rows], gv[rows], oi, ov, rs, what)
    print("%s: %d rows, recall mean %.5f min %.5f" % (what, len(rows), rec.mean(), rec.min()),
          flush=True)
    return oi


def hisa_check(cfg, x, pooled_g, blk_g, hi_g, hv_g, rows, what, k_dev):
    sh = cfg.shape_dict()
    R = cfg.rows
    qr, wr = cfg_rows(cfg, x, rows)
    pooled_o = oracle.pool(sh, x["k"], x["k_scale"], cfg.block)
    np.testing.assert_array_equal(pooled_g, pooled_o, err_msg=what + " pooled keys")
    blk_o, bv_o = oracle.block_select(sh, qr, wr, pooled_o, cfg.block, cfg.m_scored, cfg.force,
                                      rows)
    # block scores of every block for the sampled rows (the indexer on pooled keys)
    nb = cfg.n_k // cfg.block
    bsh = dict(sh, n_k=nb, key_dtype=0, q_pos0=1 << 30, causal_ratio=1)
    bsc = oracle.row_scores(bsh, qr, wr, pooled_o.reshape(cfg.batch, nb, cfg.dim), None, rows) \
        if cfg.batch == 1 else None
    same = np.all(blk_g[rows] == blk_o, axis=1)
    n_same = int(same.sum())
    for i, r in enumerate(rows):
        if same[i]:
            continue
        # a differing block list is allowed only through a near-tie of block scores
        G, O = set(blk_g[r][blk_g[r] >= 0].tolist()), set(blk_o[i][blk_o[i] >= 0].tolist())
        assert len(G) == len(O), "%s row %d: block count" % (what, r)
        sc = bsc[i] if bsc is not None else oracle.row_scores(
            bsh, qr[i:i + 1], wr[i:i + 1], pooled_o[r // cfg.n_q:r // cfg.n_q + 1], None,
            np.array([0]))[0]
        finite = bv_o[i][np.isfinite(bv_o[i])]
        tau = finite.min() if len(finite) else 0.0
        eps = 1e-3 * max(abs(tau), 1e-3 * float(np.max(np.abs(sc[np.isfinite(sc)]))))
        for b in G - O:
            assert sc[b] >= tau - eps, "%s row %d: extra block %d" % (what, r, b)
        for b in O - G:
            assert sc[b] <= tau + eps, "%s row %d: missed block %d" % (what, r, b)
    print("%s: block lists identical on %d / %d sampled rows" % (what, n_same, len(rows)),
          flush=True)
    # tokens, where the block lists agree
    oi, ov = oracle.refine(sh, qr, wr, x["k"], x["k_scale"], cfg.block, blk_o, cfg.topk, rows)
    rs = oracle.row_scores(sh, qr, wr, x["k"], x["k_scale"], rows)
    sel = np.nonzero(same)[0]
    rec = check_topk_float(hi_g[rows[sel]], hv_g[rows[sel]], oi[sel], ov[sel], rs[sel],
                           what + " tokens")
    print("%s tokens: recall mean %.5f min %.5f" % (what, rec.mean(), rec.min()), flush=True)
    # rows whose block list differs (near-tie swap): the tokens must still be a
    # valid, correctly scored, sorted selection from the GPU's own blocks
    for i in np.nonzero(~same)[0]:
        r = rows[i]
        G = hi_g[r][hi_g[r] >= 0]
        kept = blk_g[r][blk_g[r] >= 0]
        assert np.all(np.isin(G // cfg.block, kept)), "%s row %d: token outside kept blocks" % (what, r)
        assert np.all(np.isfinite(rs[i][G])), "%s row %d: invisible token" % (what, r)
        gv = hv_g[r][:len(G)].astype(np.float64)
        assert np.all(np.abs(gv - rs[i][G]) <= 1e-3 * np.maximum(np.abs(rs[i][G]), 1e-3))
        assert np.all(np.diff(gv) <= 0)
    # the refinement alone, on the oracle's block lists (uploaded as an input)
    blk_in = np.full((R, cfg.m_total), -1, np.int32)
    blk_in[rows] = blk_o
    S = tks.Shape(**sh)
    q, w, k, ks = k_dev
    ri, rv = tks.hisa_refine_topk(S, q, w, k, ks, cfg.block, dev(blk_in).view(
        cfg.batch, cfg.n_q, cfg.m_total), cfg.topk)
    torch.cuda.synchronize()
    ri, rv = host(ri).reshape(R, -1), host(rv).reshape(R, -1)
    rec2 = check_topk_float(ri[rows], rv[rows], oi, ov, rs, what + " refine-on-oracle-blocks")
    print("%s refine on oracle blocks: recall mean %.5f min %.5f" % (what, rec2.mean(),
                                                                      rec2.min()), flush=True)
    return oi


def run_flat(cfg, S, q, w, k, ks, q_chunk=0, k_tile=0):
    idx, vals = tks.topk_flat(S, q, w, k, ks, cfg.topk, q_chunk, k_tile)
    torch.cuda.synchronize()
    return host(idx).reshape(cfg.rows, -1), host(vals).reshape(cfg.rows, -1)


def run_hisa(cfg, S, q, w, k, ks):
    pooled = tks.hisa_pool_keys(S, k, ks, cfg.block)
    blk, _ = tks.hisa_block_select(S, q, w, pooled, cfg.block, cfg.m_scored, cfg.force,
                                   with_vals=False)
    idx, vals = tks.hisa_refine_topk(S, q, w, k, ks, cfg.block, blk, cfg.topk)
    torch.cuda.synchronize()
    return (host(pooled.view(torch.int16)).view(np.uint16), host(blk).reshape(cfg.rows, -1),
            host(idx).reshape(cfg.rows, -1), host(vals).reshape(cfg.rows, -1))


def test_flat_prefill_8k_full_size():
    cfg = CONFIGS[2]
    say("flat prefill L=8192 H=64 D=128 k=2048 (full size, sampled rows)")
    x, (q, w, k, ks) = upload(cfg)
    S = tks.Shape(**cfg.shape_dict())
    gi, gv = run_flat(cfg, S, q, w, k, ks)
    flat_check(cfg, x, gi, gv, sample_rows(cfg, 96), "flat 8k")
    # the chunk / tile plan must not change the result
    gi2, gv2 = run_flat(cfg, S, q, w, k, ks, 1000, 2048)
    np.testing.assert_array_equal(gi2, gi)
    np.testing.assert_array_equal(gv2, gv)


def test_hisa_vs_flat_prefill_32k_full_size():
    cfg = CONFIGS[3]
    say("HISA vs flat prefill L=32768 (full size, sampled rows)")
    x, kd = upload(cfg)
    S = tks.Shape(**cfg.shape_dict())
    gi, gv = run_flat(cfg, S, *kd)
    # 256 rows: first / last, around topk - 1, around the 128-key block
    # boundaries and the 8192-row chunk boundaries, the rest uniform
    rows = sample_rows(cfg, 256, extra=[8191, 8192, 16383, 16384, 24575, 24576])
    flat_check(cfg, x, gi, gv, rows, "flat 32k")
    pooled, blk, hi, hv = run_hisa(cfg, S, *kd)
    hisa_check(cfg, x, pooled, blk, hi, hv, rows, "hisa 32k", kd)
    u = iou(hi, gi)
    print("HISA vs flat token-set IoU over all rows: mean %.4f min %.4f" % (u.mean(), u.min()))
    # queries that see <= 64 blocks keep every block: HISA == flat there
    early = np.arange(0, cfg.m_total * cfg.block)
    np.testing.assert_array_equal(hi[early], gi[early])


def test_decode_64k_fp8_full_size():
    cfg = CONFIGS[4]
    say("decode 64 x 65536 fp8 keys (full size)")
    x, kd = upload(cfg)
    S = tks.Shape(**cfg.shape_dict())
    gi, gv = run_flat(cfg, S, *kd)
    rows = np.arange(cfg.rows)  # every sequence
    flat_check(cfg, x, gi, gv, rows, "flat decode")
    pooled, blk, hi, hv = run_hisa(cfg, S, *kd)
    hisa_check(cfg, x, pooled, blk, hi, hv, rows, "hisa decode", kd)
    u = iou(hi, gi)
    print("HISA vs flat IoU (i.i.d. keys): mean %.4f" % u.mean())


def test_streaming_256k_compressed_full_size():
    cfg = CONFIGS[5]
    say("streaming S=262144 over T=65536 compressed keys, q_chunk 4096, k_tile 8192")
    k, ks = gen_keys(cfg)
    q = gen_q(cfg)
    qd = dev(q)
    del q
    w = gen_w(cfg)
    S = tks.Shape(**cfg.shape_dict())
    wd, kdv = dev(w), dev(k)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    gi, gv = run_flat(cfg, S, qd, wd, kdv, None, cfg.q_chunk, cfg.k_tile)
    outputs = 2 * cfg.rows * cfg.topk * 4
    working = torch.cuda.max_memory_allocated() - base - outputs
    print("working set beyond inputs and outputs: %.1f MiB; a [S,T] fp32 score tensor "
          "would be %.0f GiB" % (working / 2 ** 20,
                                 tks.materialized_score_bytes(1, cfg.n_q, 1, cfg.n_k) / 2 ** 30))
    assert working < 512 * 2 ** 20
    # 256 rows, including the rows around every 8192-key tile boundary (a
    # query at row t sees compressed keys up to floor(t / 4)) and the
    # 4096-row chunk boundaries
    tile_rows = [cfg.causal_ratio * cfg.k_tile * j + d for j in range(1, cfg.n_k // cfg.k_tile)
                 for d in (-1, 0, cfg.causal_ratio - 1, cfg.causal_ratio)]
    rows = sample_rows(cfg, 256, extra=tile_rows)
    flat_check(cfg, dict(q=None, w=None, k=k, k_scale=None), gi, gv, rows, "stream 256k")

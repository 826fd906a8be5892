"""GPU parity on small inputs: exact on integer-valued inputs (fp32 scores are
exact, so indices and values must equal the oracle's), edge cases, chunk /
tile / top-k sweeps (the StreamIndex abstract's three sweep axes; results
must not depend on them), the HISA all-blocks-kept invariant, and the fp8
e4m3fn decode of every code."""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_topk_exact, cfg_rows, check_topk_float, dev, host
from tks_inputs import (CONFIGS, FORCE_FIRST, FORCE_LOCAL, KEY_FP8, Config, fp32_to_bf16_bits,
                        fp32_to_e4m3fn, make_inputs, scaled)
from top_key_selection_amd import tks

pytestmark = pytest.mark.gpu


def say(msg):
    print("[case] " + msg, flush=True)


def int_case(seed, batch=1, n_q=256, n_k=256, heads=4, dim=32, lo=-4, hi=4, q_pos0=0, ratio=1,
             fp8=False):
    rng = np.random.default_rng(seed)
    q = rng.integers(lo, hi + 1, (batch, n_q, heads, dim)).astype(np.float32)
    w = rng.integers(lo, hi + 1, (batch, n_q, heads)).astype(np.float32)
    kv = rng.integers(lo, hi + 1, (batch, n_k, dim)).astype(np.float32)
    x = dict(q=fp32_to_bf16_bits(q), w=w)
    if fp8:
        x["k"] = fp32_to_e4m3fn(kv)                         # small integers are exact codes
        x["k_scale"] = (2.0 ** rng.integers(-3, 2, (batch, n_k))).astype(np.float32)
    else:
        x["k"] = fp32_to_bf16_bits(kv)
        x["k_scale"] = None
    shape = dict(batch=batch, n_q=n_q, n_k=n_k, heads=heads, dim=dim, q_pos0=q_pos0,
                 causal_ratio=ratio, key_dtype=int(fp8))
    return shape, x


def gpu_inputs(x):
    return dev(x["q"]), dev(x["w"]), dev(x["k"]), dev(x["k_scale"])


def oracle_flat(shape, x, topk):
    R = shape["batch"] * shape["n_q"]
    rows = np.arange(R)
    q = x["q"].reshape(R, shape["heads"], shape["dim"])
    w = x["w"].reshape(R, shape["heads"])
    return oracle.topk_flat(shape, q, w, x["k"], x["k_scale"], topk, rows)


def gpu_flat(shape, x, topk, q_chunk=0, k_tile=0):
    q, w, k, ks = gpu_inputs(x)
    idx, vals = tks.topk_flat(tks.Shape(**shape), q, w, k, ks, topk, q_chunk, k_tile)
    torch.cuda.synchronize()
    R = shape["batch"] * shape["n_q"]
    return host(idx).reshape(R, topk), host(vals).reshape(R, topk)


# ------------------------------------------------------------ tiny integer

def test_tiny_integer_workload_flat_exact():
    cfg = CONFIGS[1]
    say("tiny integer flat L=1024 H=4 D=32 k=64")
    x = make_inputs(cfg)
    sh = cfg.shape_dict()
    oi, ov = oracle_flat(sh, x, cfg.topk)
    gi, gv = gpu_flat(sh, x, cfg.topk)
    assert_topk_exact(gi, gv, oi, ov, "tiny flat")


def test_tiny_integer_scores_exact():
    cfg = CONFIGS[1]
    say("tiny integer indexer_scores")
    x = make_inputs(cfg)
    sh = cfg.shape_dict()
    q, w, k, ks = gpu_inputs(x)
    for (q0, qn, k0, kn) in [(0, 1024, 0, 1024), (100, 37, 5, 301), (1000, 24, 990, 34)]:
        got = host(tks.indexer_scores(tks.Shape(**sh), q, w, k, ks, q0, qn, k0, kn))
        ref = oracle.index_scores(sh, x["q"], x["w"], x["k"], None, q0, qn, k0, kn)
        np.testing.assert_array_equal(got.astype(np.float64), ref)


def test_tiny_integer_workload_hisa_exact():
    cfg = CONFIGS[1]
    say("tiny integer HISA B=64 m=4 + local")
    x = make_inputs(cfg)
    sh = cfg.shape_dict()
    R = cfg.rows
    rows = np.arange(R)
    qr, wr = cfg_rows(cfg, x, rows)
    pooled_o = oracle.pool(sh, x["k"], None, cfg.block)
    blk_o, bv_o = oracle.block_select(sh, qr, wr, pooled_o, cfg.block, cfg.m_scored, cfg.force, rows)
    hi_o, hv_o = oracle.refine(sh, qr, wr, x["k"], None, cfg.block, blk_o, cfg.topk, rows)
    q, w, k, ks = gpu_inputs(x)
    S = tks.Shape(**sh)
    pooled = tks.hisa_pool_keys(S, k, ks, cfg.block)
    blk, bv = tks.hisa_block_select(S, q, w, pooled, cfg.block, cfg.m_scored, cfg.force)
    idx, vals = tks.hisa_refine_topk(S, q, w, k, ks, cfg.block, blk, cfg.topk)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(pooled.view(torch.int16)).view(np.uint16), pooled_o)
    np.testing.assert_array_equal(host(blk).reshape(R, -1), blk_o)
    bvg = host(bv).reshape(R, -1).astype(np.float64)
    np.testing.assert_array_equal(np.isnan(bvg), np.isnan(bv_o))
    ok = ~np.isnan(bv_o)
    np.testing.assert_array_equal(bvg[ok], bv_o[ok])
    assert_topk_exact(host(idx).reshape(R, -1), host(vals).reshape(R, -1), hi_o, hv_o, "tiny hisa")


# ------------------------------------------------------------------ sweeps

@pytest.mark.parametrize("q_chunk,k_tile", [(0, 0), (256, 1024), (1000, 512), (37, 32),
                                             (4096, 2048), (3000, 96)])
def test_chunk_and_tile_sweep_is_exact(q_chunk, k_tile):
    say("chunk/tile sweep q_chunk=%d k_tile=%d" % (q_chunk, k_tile))
    sh, x = int_case(20, n_q=3000, n_k=3000, heads=8, dim=64, lo=-3, hi=3)
    oi, ov = _cached_oracle(("sweep",), sh, x, 256)
    gi, gv = gpu_flat(sh, x, 256, q_chunk, k_tile)
    assert_topk_exact(gi, gv, oi, ov, "sweep")


_CACHE = {}


def _cached_oracle(key, sh, x, topk):
    key = key + (topk,)
    if key not in _CACHE:
        _CACHE[key] = oracle_flat(sh, x, topk)
    return _CACHE[key]


@pytest.mark.parametrize("topk", [1, 7, 64, 100, 1024, 2048])
def test_topk_sweep_is_exact(topk):
    say("top-k sweep k=%d" % topk)
    sh, x = int_case(21, n_q=2500, n_k=2500, heads=4, dim=32, lo=-2, hi=2)
    oi, ov = oracle_flat(sh, x, topk)
    for qc, kt in [(0, 0), (700, 640)]:
        gi, gv = gpu_flat(sh, x, topk, qc, kt)
        assert_topk_exact(gi, gv, oi, ov, "topk=%d qc=%d kt=%d" % (topk, qc, kt))


# -------------------------------------------------------------- edge cases

def test_all_equal_scores_take_lowest_indices():
    say("all-equal scores")
    sh, x = int_case(22, n_q=300, n_k=300)
    x["q"] = fp32_to_bf16_bits(np.zeros((1, 300, 4, 32), np.float32))
    gi, gv = gpu_flat(sh, x, 64)
    for t in range(300):
        n = min(64, t + 1)
        np.testing.assert_array_equal(gi[t, :n], np.arange(n))
        assert np.all(gi[t, n:] == -1) and np.all(gv[t, :n] == 0) and not np.signbit(gv[t, :n]).any()


def test_rows_without_visible_keys_are_padding():
    say("negative q_pos0: leading rows see no key")
    sh, x = int_case(23, n_q=64, n_k=64, q_pos0=-5)
    oi, ov = oracle_flat(sh, x, 16)
    gi, gv = gpu_flat(sh, x, 16)
    assert np.all(gi[:5] == -1) and np.all(np.isnan(gv[:5]))
    assert_topk_exact(gi, gv, oi, ov, "neg pos0")


def test_no_keys_at_all():
    say("n_k = 0")
    sh, x = int_case(24, n_q=40, n_k=0)
    x["k"] = np.zeros((1, 0, 32), np.uint16)
    q, w, _, _ = gpu_inputs(x)
    k = torch.zeros((1, 0, 32), dtype=torch.bfloat16, device="cuda")
    idx, vals = tks.topk_flat(tks.Shape(**sh), q, w, k, None, 8)
    torch.cuda.synchronize()
    assert np.all(host(idx) == -1)


@pytest.mark.parametrize("ratio,q_pos0", [(4, 0), (4, -3), (3, 7)])
def test_compressed_causality_exact(ratio, q_pos0):
    say("causal ratio %d q_pos0 %d" % (ratio, q_pos0))
    sh, x = int_case(25, n_q=1200, n_k=300, ratio=ratio, q_pos0=q_pos0)
    oi, ov = oracle_flat(sh, x, 50)
    for qc, kt in [(0, 0), (333, 64)]:
        gi, gv = gpu_flat(sh, x, 50, qc, kt)
        assert_topk_exact(gi, gv, oi, ov, "ratio")


def test_batched_chunked_prefill_continuation():
    say("batch 3, 5 new queries at the end of a 700-key cache")
    sh, x = int_case(26, batch=3, n_q=5, n_k=700, q_pos0=695)
    oi, ov = oracle_flat(sh, x, 100)
    for qc, kt in [(0, 0), (4, 160), (1, 32)]:
        gi, gv = gpu_flat(sh, x, 100, qc, kt)
        assert_topk_exact(gi, gv, oi, ov, "batch")


@pytest.mark.parametrize("heads,dim", [(1, 32), (5, 64), (33, 128), (64, 32), (48, 64), (64, 128)])
def test_head_and_dim_variants_exact(heads, dim):
    say("heads %d dim %d" % (heads, dim))
    sh, x = int_case(27 + heads + dim, n_q=200, n_k=777, heads=heads, dim=dim, q_pos0=577,
                     lo=-2, hi=2)
    oi, ov = oracle_flat(sh, x, 128)
    gi, gv = gpu_flat(sh, x, 128)
    assert_topk_exact(gi, gv, oi, ov, "heads/dim")


@pytest.mark.parametrize("q_chunk,k_tile", [(0, 0), (100, 192), (37, 64), (613, 1024)])
def test_shared_key_prefill_path_exact(q_chunk, k_tile):
    """Prefill with D = 128: blocks of consecutive queries of one sequence
    share staged key tiles.  Ragged sequence lengths, chunks that straddle
    sequence boundaries and tiles of a few stages must still give the oracle's
    exact result."""
    say("shared-key prefill q_chunk=%d k_tile=%d" % (q_chunk, k_tile))
    sh, x = int_case(60, batch=3, n_q=203, n_k=1500, heads=64, dim=128, q_pos0=1297, lo=-2, hi=2)
    oi, ov = _cached_oracle(("shared",), sh, x, 300)
    gi, gv = gpu_flat(sh, x, 300, q_chunk, k_tile)
    assert_topk_exact(gi, gv, oi, ov, "shared prefill")


def test_shared_key_scores_and_ratio_exact():
    """indexer_scores rectangles (masked slots written as -inf) and
    compressed causality through the shared-key scoring path."""
    say("shared-key scores rectangles, ratio 4")
    sh, x = int_case(61, batch=2, n_q=300, n_k=800, heads=64, dim=128, q_pos0=-9, ratio=4,
                     lo=-2, hi=2)
    q, w, k, ks = gpu_inputs(x)
    for (q0, qn, k0, kn) in [(0, 300, 0, 800), (11, 77, 3, 129), (290, 10, 0, 75)]:
        got = host(tks.indexer_scores(tks.Shape(**sh), q, w, k, ks, q0, qn, k0, kn))
        ref = oracle.index_scores(sh, x["q"], x["w"], x["k"], None, q0, qn, k0, kn)
        np.testing.assert_array_equal(got.astype(np.float64), ref)
    oi, ov = oracle_flat(sh, x, 40)
    gi, gv = gpu_flat(sh, x, 40)
    assert_topk_exact(gi, gv, oi, ov, "shared ratio")


def test_shared_key_hisa_prefill_exact():
    """HISA prefill with D = 128: pooled-block scoring runs on the shared-key
    path and refinement on the gathered path; blocks and tokens must equal
    the oracle's."""
    say("HISA prefill D=128 block 64 m 5")
    sh, x = int_case(62, batch=2, n_q=600, n_k=1200, heads=64, dim=128, q_pos0=600, lo=-2, hi=2)
    R = 1200
    rows = np.arange(R)
    qr, wr = x["q"].reshape(R, 64, 128), x["w"].reshape(R, 64)
    blk_o, idx_o, val_o = oracle.hisa(sh, qr, wr, x["k"], None, 64, 5, FORCE_FIRST | FORCE_LOCAL,
                                      256, rows)
    q, w, k, ks = gpu_inputs(x)
    idx, vals, blk = tks.hisa_topk(tks.Shape(**sh), q, w, k, ks, 64, 5, FORCE_FIRST | FORCE_LOCAL,
                                   256)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(blk).reshape(R, -1), blk_o)
    assert_topk_exact(host(idx).reshape(R, -1), host(vals).reshape(R, -1), idx_o, val_o,
                      "shared hisa")


def test_shared_key_refine_ring_refills_exact():
    """HISA prefill long enough that each workgroup's key segment holds more
    ring stages than the ring has slots, so slots are refilled while other
    rows of the workgroup still compute: two sequences, every row keeping a
    different block list, one call over all rows and one whose query chunk
    straddles the sequences.  Sampled rows (wave, chunk and sequence
    boundaries) must equal the oracle's blocks and tokens exactly."""
    say("HISA refine ring refills: 2 x 1024 queries, 32768 keys")
    batch, n_q, n_k, heads = 2, 1024, 32768, 64
    block, m_scored, topk = 64, 16, 512
    flags = FORCE_FIRST | FORCE_LOCAL
    sh, x = int_case(77, batch=batch, n_q=n_q, n_k=n_k, heads=heads, dim=128,
                     q_pos0=n_k - n_q, lo=-2, hi=2)
    R = batch * n_q
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 7, 8, 15, 1023, 1024, 1031, 1535, 1536, 2047],
                                     rng.choice(R, 54, replace=False)]))
    qr = x["q"].reshape(R, heads, 128)[rows]
    wr = x["w"].reshape(R, heads)[rows]
    blk_o, idx_o, val_o = oracle.hisa(sh, qr, wr, x["k"], None, block, m_scored, flags, topk, rows)
    S = tks.Shape(**sh)
    q, w, k, ks = gpu_inputs(x)
    pooled = tks.hisa_pool_keys(S, k, ks, block)
    blk, _ = tks.hisa_block_select(S, q, w, pooled, block, m_scored, flags, with_vals=False)
    for q_chunk in (0, 1536):
        idx, vals = tks.hisa_refine_topk(S, q, w, k, ks, block, blk, topk, q_chunk)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(blk).reshape(R, -1)[rows], blk_o)
        assert_topk_exact(host(idx).reshape(R, -1)[rows], host(vals).reshape(R, -1)[rows], idx_o,
                          val_o, "ring refills q_chunk=%d" % q_chunk)


@pytest.mark.parametrize("block,m_scored,n_k,q_chunk", [(32, 12, 3001, 70), (256, 5, 5000, 0),
                                                         (64, 8, 4100, 33), (128, 3, 700, 0)])
def test_scheduled_refine_block_sizes_exact(block, m_scored, n_k, q_chunk):
    """Prefill refinement with a plan per group of 8 rows (bf16 keys, D = 128):
    32-key blocks put four plan positions in one 128-key ring stage, 256-key
    blocks spread one position over two stages; ragged caches, a query chunk
    that splits sequences and groups, rows with fewer than 8 in their group.
    Blocks and tokens must equal the oracle's."""
    say("scheduled refine B=%d m=%d n_k=%d q_chunk=%d" % (block, m_scored, n_k, q_chunk))
    batch, n_q, heads = 2, 100, 64
    flags = FORCE_FIRST | FORCE_LOCAL
    sh, x = int_case(40 + block, batch=batch, n_q=n_q, n_k=n_k, heads=heads, dim=128,
                     q_pos0=n_k - n_q, lo=-2, hi=2)
    R = batch * n_q
    rows = np.arange(R)
    qr, wr = x["q"].reshape(R, heads, 128), x["w"].reshape(R, heads)
    blk_o, idx_o, val_o = oracle.hisa(sh, qr, wr, x["k"], None, block, m_scored, flags, 300, rows)
    S = tks.Shape(**sh)
    q, w, k, ks = gpu_inputs(x)
    pooled = tks.hisa_pool_keys(S, k, ks, block)
    blk, _ = tks.hisa_block_select(S, q, w, pooled, block, m_scored, flags, with_vals=False)
    idx, vals = tks.hisa_refine_topk(S, q, w, k, ks, block, blk, 300, q_chunk)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(blk).reshape(R, -1), blk_o)
    assert_topk_exact(host(idx).reshape(R, -1), host(vals).reshape(R, -1), idx_o, val_o,
                      "scheduled refine B=%d" % block)


@pytest.mark.parametrize("ratio,q_pos0", [(4, -6), (3, 5)])
def test_scheduled_refine_compressed_causality_exact(ratio, q_pos0):
    """Prefill refinement through the plans with compressed causality: a
    query sees (q_pos0 + t) / ratio + 1 keys, so neighbouring queries of a
    group see the same or almost the same keys, and with q_pos0 < 0 the
    first queries see none (padding rows inside a group).  Blocks and
    tokens must equal the oracle's."""
    say("scheduled refine, causal ratio %d, q_pos0 %d" % (ratio, q_pos0))
    batch, n_q, n_k, heads, block, m_scored, topk = 2, 600, 2000, 64, 64, 6, 150
    flags = FORCE_FIRST | FORCE_LOCAL
    sh, x = int_case(60 + ratio, batch=batch, n_q=n_q, n_k=n_k, heads=heads, dim=128, q_pos0=q_pos0,
                     ratio=ratio, lo=-2, hi=2)
    R = batch * n_q
    rows = np.arange(R)
    qr, wr = x["q"].reshape(R, heads, 128), x["w"].reshape(R, heads)
    blk_o, idx_o, val_o = oracle.hisa(sh, qr, wr, x["k"], None, block, m_scored, flags, topk, rows)
    S = tks.Shape(**sh)
    q, w, k, ks = gpu_inputs(x)
    idx, vals, blk = tks.hisa_topk(S, q, w, k, ks, block, m_scored, flags, topk)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(blk).reshape(R, -1), blk_o)
    assert_topk_exact(host(idx).reshape(R, -1), host(vals).reshape(R, -1), idx_o, val_o,
                      "scheduled refine, compressed causality")


def test_refine_plans_made_chunk_by_chunk_exact():
    """Refinement plans too large to make for every group at once (here
    4096 groups x 1024 positions) are made chunk by chunk; with 1000-row
    chunks, groups of 8 queries straddle chunk boundaries and each chunk
    refines only its own rows of them.  Sampled rows at chunk and group
    boundaries must equal the oracle's blocks and tokens."""
    say("refine, plans per chunk: 32768 queries, 33000 keys, B=32, m_total 128, q_chunk 1000")
    n_q, n_k, heads, block, m_scored, topk = 32768, 33000, 8, 32, 126, 512
    flags = FORCE_FIRST | FORCE_LOCAL
    sh, x = int_case(93, batch=1, n_q=n_q, n_k=n_k, heads=heads, dim=128, q_pos0=n_k - n_q,
                     lo=-2, hi=2)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, 7, 8, 999, 1000, 1001, 1007, 1008, 15999, 16000, 16001,
                                      31999, 32000, 32767], rng.choice(n_q, 34, replace=False)]))
    qr = x["q"].reshape(n_q, heads, 128)[rows]
    wr = x["w"].reshape(n_q, heads)[rows]
    blk_o, idx_o, val_o = oracle.hisa(sh, qr, wr, x["k"], None, block, m_scored, flags, topk, rows)
    S = tks.Shape(**sh)
    q, w, k, ks = gpu_inputs(x)
    pooled = tks.hisa_pool_keys(S, k, ks, block)
    blk, _ = tks.hisa_block_select(S, q, w, pooled, block, m_scored, flags, with_vals=False)
    idx, vals = tks.hisa_refine_topk(S, q, w, k, ks, block, blk, topk, 1000)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(blk).reshape(n_q, -1)[rows], blk_o)
    assert_topk_exact(host(idx).reshape(n_q, -1)[rows], host(vals).reshape(n_q, -1)[rows], idx_o,
                      val_o, "plans per chunk")


def test_refine_lists_too_long_for_a_plan_take_the_segment_ring_exact():
    """A group's union of kept blocks can exceed what one plan holds (here
    8 rows x 150 entries over 1250 blocks of 32 keys): such shapes refine
    through the key-segment ring instead; results must equal the oracle's."""
    say("refine without a plan: B=32, m_total 150, n_k 40000")
    batch, n_q, n_k, heads, block, m_scored = 1, 48, 40000, 64, 32, 148
    flags = FORCE_FIRST | FORCE_LOCAL
    sh, x = int_case(91, batch=batch, n_q=n_q, n_k=n_k, heads=heads, dim=128,
                     q_pos0=n_k - n_q, lo=-2, hi=2)
    R = batch * n_q
    rows = np.arange(R)
    qr, wr = x["q"].reshape(R, heads, 128), x["w"].reshape(R, heads)
    blk_o, idx_o, val_o = oracle.hisa(sh, qr, wr, x["k"], None, block, m_scored, flags, 1024, rows)
    S = tks.Shape(**sh)
    q, w, k, ks = gpu_inputs(x)
    idx, vals, blk = tks.hisa_topk(S, q, w, k, ks, block, m_scored, flags, 1024)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(blk).reshape(R, -1), blk_o)
    assert_topk_exact(host(idx).reshape(R, -1), host(vals).reshape(R, -1), idx_o, val_o,
                      "segment ring refine")


def test_tied_running_list_across_tiles_keeps_lowest_indices():
    """Scores tied at the k-th place across key tiles: the running list of
    earlier tiles carries the tie group, and the later tiles' selection must
    still keep the lowest indices (the running list is not kept sorted
    between tiles)."""
    say("ties across tiles with a running list")
    n_k, K = 9000, 2048
    q = np.zeros((1, 3, 1, 32), np.float32)
    q[..., 0] = 1.0                                    # score = relu(k[s, 0])
    w = np.ones((1, 3, 1), np.float32)
    kv = np.zeros((1, n_k, 32), np.float32)
    hot = np.array([4500, 4501, 5000, 7000, 8999, 6000, 6001, 6002, 4096, 8192])
    kv[0, hot, 0] = 1.0
    kv[0, hot[:3], 0] = 2.0
    x = dict(q=fp32_to_bf16_bits(q), w=w, k=fp32_to_bf16_bits(kv), k_scale=None)
    sh = dict(batch=1, n_q=3, n_k=n_k, heads=1, dim=32, q_pos0=n_k - 3, causal_ratio=1, key_dtype=0)
    oi, ov = oracle_flat(sh, x, K)
    for kt in (0, 4096, 2048, 1024):
        gi, gv = gpu_flat(sh, x, K, 0, kt)
        assert_topk_exact(gi, gv, oi, ov, "ties k_tile=%d" % kt)


def test_fp8_keys_integer_exact():
    say("fp8 keys, integer codes, power-of-two scales")
    sh, x = int_case(28, batch=2, n_q=64, n_k=1100, heads=8, dim=128, q_pos0=1036, fp8=True)
    oi, ov = oracle_flat(sh, x, 200)
    gi, gv = gpu_flat(sh, x, 200)
    assert_topk_exact(gi, gv, oi, ov, "fp8")


@pytest.mark.parametrize("dim,heads", [(128, 64), (64, 8), (32, 33)])
def test_fp8_decode_stream_path_exact(dim, heads):
    """One query per sequence (decode): keys are streamed through the LDS
    ring kernel.  Integer codes with power-of-two scales keep every score
    exact, so flat and HISA must equal the oracle bit for bit."""
    say("fp8 decode stream path dim %d heads %d" % (dim, heads))
    n_k = 5000
    sh, x = int_case(40 + dim, batch=5, n_q=1, n_k=n_k, heads=heads, dim=dim, q_pos0=n_k - 1,
                     fp8=True)
    oi, ov = oracle_flat(sh, x, 300)
    gi, gv = gpu_flat(sh, x, 300)
    assert_topk_exact(gi, gv, oi, ov, "fp8 decode flat")
    R = 5
    rows = np.arange(R)
    qr, wr = x["q"].reshape(R, heads, dim), x["w"].reshape(R, heads)
    blk_o, idx_o, val_o = oracle.hisa(sh, qr, wr, x["k"], x["k_scale"], 128, 6,
                                      FORCE_FIRST | FORCE_LOCAL, 300, rows)
    q, w, k, ks = gpu_inputs(x)
    idx, vals, blk = tks.hisa_topk(tks.Shape(**sh), q, w, k, ks, 128, 6, FORCE_FIRST | FORCE_LOCAL,
                                   300)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(blk).reshape(R, -1), blk_o)
    assert_topk_exact(host(idx).reshape(R, -1), host(vals).reshape(R, -1), idx_o, val_o,
                      "fp8 decode hisa")


@pytest.mark.parametrize("fp8,batch,n_q,n_k", [(True, 2, 64, 1100), (False, 4, 1, 3001)])
def test_hisa_generic_block_paths_exact(fp8, batch, n_q, n_k):
    """HISA through the per-row block-mode scoring: prefill with fp8 keys
    (pooled blocks of dequantised keys) and decode with bf16 keys, 64 heads,
    ragged caches.  Blocks and tokens must equal the oracle's."""
    say("HISA generic block paths fp8=%d batch=%d n_q=%d n_k=%d" % (fp8, batch, n_q, n_k))
    block, m_scored, topk = 64, 6, 200
    flags = FORCE_FIRST | FORCE_LOCAL
    sh, x = int_case(50 + fp8, batch=batch, n_q=n_q, n_k=n_k, heads=64, dim=128, q_pos0=n_k - n_q,
                     lo=-2, hi=2, fp8=fp8)
    R = batch * n_q
    rows = np.arange(R)
    qr, wr = x["q"].reshape(R, 64, 128), x["w"].reshape(R, 64)
    blk_o, idx_o, val_o = oracle.hisa(sh, qr, wr, x["k"], x["k_scale"], block, m_scored, flags, topk,
                                      rows)
    q, w, k, ks = gpu_inputs(x)
    idx, vals, blk = tks.hisa_topk(tks.Shape(**sh), q, w, k, ks, block, m_scored, flags, topk)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(blk).reshape(R, -1), blk_o)
    assert_topk_exact(host(idx).reshape(R, -1), host(vals).reshape(R, -1), idx_o, val_o,
                      "generic block paths")


def test_fp8_every_code_decodes_exactly():
    """One-hot keys: key c holds e4m3fn code c at dim 0, so its score is
    max(0, q0 * value(c)); compared with torch's e4m3fn decode."""
    say("fp8 decode of all 256 codes")
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    n = len(codes)
    k8 = np.zeros((1, n, 32), np.uint8)
    k8[0, :, 0] = codes
    scale = np.ones((1, n), np.float32)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    for sign in (1.0, -1.0):
        q = np.zeros((1, 1, 1, 32), np.float32)
        q[..., 0] = sign
        sh = dict(batch=1, n_q=1, n_k=n, heads=1, dim=32, q_pos0=n - 1, causal_ratio=1,
                  key_dtype=KEY_FP8)
        got = host(tks.indexer_scores(tks.Shape(**sh), dev(fp32_to_bf16_bits(q)),
                                      dev(np.ones((1, 1, 1), np.float32)), dev(k8), dev(scale),
                                      0, 1, 0, n))[0, 0]
        np.testing.assert_array_equal(got.astype(np.float64), np.maximum(sign * ref, 0.0))


def test_fp8_pool_bit_exact():
    say("fp8 pooling vs oracle")
    cfg = scaled(CONFIGS[4], batch=3, n_k=4096 + 77)
    from tks_inputs import gen_keys
    k8, ks = gen_keys(cfg)
    sh = cfg.shape_dict()
    for block in (32, 64, 128, 256):
        ref = oracle.pool(sh, k8, ks, block)
        got = tks.hisa_pool_keys(tks.Shape(**sh), dev(k8), dev(ks), block)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(got.view(torch.int16)).view(np.uint16), ref)


# --------------------------------------------------------------- top-k alone

def brute(scores, n, k):
    idx = np.arange(n)
    order = np.lexsort((idx, -scores[:n].astype(np.float64)))
    out = -np.ones(k, np.int64)
    out[:min(k, n)] = order[:k]
    return out


@pytest.mark.parametrize("n_cols,topk", [(5000, 2048), (70000, 2048), (140000, 2048), (300, 64),
                                         (1, 1)])
def test_topk_scores_matches_full_sort(n_cols, topk):
    say("topk_scores n_cols=%d k=%d" % (n_cols, topk))
    rng = np.random.default_rng(n_cols)
    R = 12
    sc = rng.integers(-20, 20, (R, n_cols)).astype(np.float32)   # heavy ties
    sc[1] = 0.0
    sc[2] = -0.0
    sc[3] = rng.standard_normal(n_cols).astype(np.float32)
    sc[4, ::2] = -np.inf
    # the k best all in one column partition (few long rows are filtered
    # partition by partition into one pool per row)
    sc[5] = np.arange(n_cols, dtype=np.float32)
    sc[6] = -np.arange(n_cols, dtype=np.float32)
    sc[7] = np.where(np.arange(n_cols) % 3 == 0, 5.0, rng.standard_normal(n_cols)).astype(np.float32)
    row_len = rng.integers(0, n_cols + 1, R).astype(np.int32)
    row_len[0] = n_cols
    row_len[5:8] = n_cols
    idx, vals = tks.topk_scores(dev(sc), topk, dev(row_len))
    torch.cuda.synchronize()
    gi, gv = host(idx), host(vals)
    for r in range(R):
        want = brute(sc[r], row_len[r], topk)
        np.testing.assert_array_equal(gi[r], want, err_msg="row %d" % r)
        ok = want >= 0
        np.testing.assert_array_equal(gv[r][ok], sc[r][want[ok]] + np.float32(0.0))


def test_topk_scores_threshold_prefilter_cases():
    """Rows longer than the LDS pool take a sampled threshold; every way the
    sample can mislead (the best scores hidden between sample positions, a
    tie block straddling the threshold, a pool that would overflow) must
    still give the exact result.  Many rows use the narrow workgroups."""
    say("topk_scores prefilter cases")
    rng = np.random.default_rng(77)
    for R, n_cols, topk in [(16, 70000, 2048), (600, 5000, 2048), (600, 20000, 300),
                            (600, 17000, 2048)]:
        sc = rng.standard_normal((R, n_cols)).astype(np.float32)
        pos = (np.arange(2048) * n_cols) // 2048            # the sampled columns
        hidden = np.setdiff1d(np.arange(n_cols), pos)[:topk]
        sc[0] = 0.0
        sc[0, hidden] = 1.0                                  # best keys never sampled
        sc[1] = 0.0
        sc[1, pos[: min(len(pos), topk // 4)]] = 2.0         # a few sampled, rest tied
        sc[2] = rng.integers(0, 3, n_cols).astype(np.float32)  # three huge tie groups
        top = rng.standard_normal(n_cols).astype(np.float32)
        top[: topk // 2] = 50.0 + np.arange(topk // 2, dtype=np.float32)
        top[topk // 2: topk // 2 + 6000 if n_cols > 7000 else n_cols] = 10.0   # tie block at the k-th
        sc[3] = top
        sc[4] = np.sort(rng.standard_normal(n_cols)).astype(np.float32)  # monotone row
        idx, vals = tks.topk_scores(dev(sc), topk)
        torch.cuda.synchronize()
        gi, gv = host(idx), host(vals)
        full = np.full(R, n_cols, np.int32)
        for r in range(R):
            want = brute(sc[r], full[r], topk)
            np.testing.assert_array_equal(gi[r], want, err_msg="R=%d n=%d row %d" % (R, n_cols, r))
            ok = want >= 0
            np.testing.assert_array_equal(gv[r][ok], sc[r][want[ok]] + np.float32(0.0))


@pytest.mark.parametrize("R", [8, 520])
@pytest.mark.parametrize("n_cols", [2049, 4095, 4096, 4097, 8192, 16383, 16384])
def test_topk_scores_route_boundaries(R, n_cols):
    """Row lengths on both sides of every route boundary (gather-and-sort up
    to 2048, histogram below 4096, sampled threshold from 4096 token
    candidates, the few-row and many-row workgroup sizes), integer scores
    with heavy ties and float rows, against a full sort."""
    say("topk_scores route boundaries R=%d n=%d" % (R, n_cols))
    rng = np.random.default_rng(R * 100000 + n_cols)
    sc = rng.integers(-6, 7, (R, n_cols)).astype(np.float32)
    sc[1::3] = rng.standard_normal((len(range(1, R, 3)), n_cols)).astype(np.float32)
    sc[2, :] = 1.0                                           # one tie group
    idx_all = np.broadcast_to(np.arange(n_cols), sc.shape)
    order = np.lexsort((idx_all, -sc.astype(np.float64)), axis=-1)
    for topk in (2048, 700):
        idx, vals = tks.topk_scores(dev(sc), topk)
        torch.cuda.synchronize()
        gi, gv = host(idx), host(vals)
        want = order[:, :topk]
        bad = np.nonzero((gi != want).any(axis=1))[0]
        assert len(bad) == 0, "k=%d: %d rows differ, first %d" % (topk, len(bad), bad[0])
        np.testing.assert_array_equal(gv, np.take_along_axis(sc, want, axis=1) + np.float32(0.0))


def test_tiled_rows_with_prior_list_take_the_prefilter_exactly():
    """Key tiles longer than the LDS pool plus the running list of earlier
    tiles: the sampled threshold covers both, integer scores (many ties)."""
    say("tiled prefilter with running list")
    sh, x = int_case(63, n_q=600, n_k=36000, heads=4, dim=32, q_pos0=35400, lo=-3, hi=3)
    oi, ov = oracle_flat(sh, x, 2048)
    for qc, kt in [(600, 16384), (256, 20000), (600, 4096)]:
        gi, gv = gpu_flat(sh, x, 2048, qc, kt)
        assert_topk_exact(gi, gv, oi, ov, "tiled prefilter qc=%d kt=%d" % (qc, kt))


# ------------------------------------------------------------------- HISA

def test_hisa_all_blocks_kept_equals_flat():
    say("HISA with every block kept == flat")
    sh, x = int_case(29, n_q=1024, n_k=1024, heads=8, dim=64)
    q, w, k, ks = gpu_inputs(x)
    S = tks.Shape(**sh)
    fi, fv = tks.topk_flat(S, q, w, k, ks, 100)
    for block, flags in ((64, FORCE_LOCAL), (32, FORCE_FIRST | FORCE_LOCAL), (128, FORCE_LOCAL)):
        hi, hv, blk = tks.hisa_topk(S, q, w, k, ks, block, 1024 // block, flags, 100)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(hi), host(fi))
        np.testing.assert_array_equal(host(hv), host(fv))


def test_hisa_ragged_cache_exact():
    """n_k not a multiple of the block: the tail block is never pooled or
    scored, but is refined when it is a query's (forced) local block."""
    say("HISA ragged cache, batched decode-style rows")
    sh, x = int_case(30, batch=2, n_q=40, n_k=1000, heads=8, dim=64, q_pos0=960)
    R = 80
    rows = np.arange(R)
    qr = x["q"].reshape(R, 8, 64)
    wr = x["w"].reshape(R, 8)
    for block, m, flags in ((64, 3, FORCE_FIRST | FORCE_LOCAL), (128, 2, FORCE_LOCAL),
                            (32, 0, FORCE_LOCAL), (64, 5, 0)):
        blk_o, idx_o, val_o = oracle.hisa(sh, qr, wr, x["k"], None, block, m, flags, 60, rows)
        q, w, k, ks = gpu_inputs(x)
        idx, vals, blk = tks.hisa_topk(tks.Shape(**sh), q, w, k, ks, block, m, flags, 60)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(blk).reshape(R, -1), blk_o)
        assert_topk_exact(host(idx).reshape(R, -1), host(vals).reshape(R, -1), idx_o, val_o,
                          "ragged hisa B=%d" % block)


@pytest.mark.parametrize("nb,n_q,q_pos0,heads,dim", [
    (300, 40, None, 4, 32), (700, 601, -40, 4, 32), (1500, 37, None, 4, 32), (2600, 30, None, 4, 32),
    (64, 9, -3, 4, 32),
    # D = 128, fewer than 8 rows per sequence (decode-like)
    (512, 1, None, 64, 128), (1000, 5, None, 20, 128), (2048, 3, None, 64, 128), (40, 7, 28, 64, 128),
    (2049, 2, None, 64, 128)])
def test_block_select_rows_exact(nb, n_q, q_pos0, heads, dim):
    """Block selection straight from integer pooled keys in [-2, 2] (block
    scores are integers, so nearly every kept set ends inside a tie): rows
    of up to 512, 1024 and 2048 blocks (a wave per row) and longer rows (the
    workgroup route), with D = 32 and with D = 128 at decode-like row counts;
    queries that see no block, a ragged cache tail, m from 0 to more than a
    row can keep, every force flag combination."""
    block, batch = 32, 2
    n_k = nb * block + 17
    q_pos0 = n_k - n_q if q_pos0 is None else q_pos0
    say("block select nb=%d rows=%d q_pos0=%d heads=%d dim=%d" % (nb, batch * n_q, q_pos0, heads, dim))
    rng = np.random.default_rng(nb + n_q)
    sh = dict(batch=batch, n_q=n_q, n_k=n_k, heads=heads, dim=dim, q_pos0=q_pos0, causal_ratio=1,
              key_dtype=0)
    R = batch * n_q
    q = fp32_to_bf16_bits(rng.integers(-2, 3, (R, heads, dim)).astype(np.float32))
    w = rng.integers(-2, 3, (R, heads)).astype(np.float32)
    pooled = fp32_to_bf16_bits(rng.integers(-2, 3, (batch, nb, dim)).astype(np.float32))
    S = tks.Shape(**sh)
    qd, wd, pd = dev(q.reshape(batch, n_q, heads, dim)), dev(w.reshape(batch, n_q, heads)), dev(pooled)
    for m, flags in ((0, FORCE_LOCAL), (5, FORCE_FIRST | FORCE_LOCAL), (62, FORCE_FIRST),
                     (200, 0), (nb + 3, FORCE_FIRST | FORCE_LOCAL)):
        m = min(m, 510)  # m_total at most 512
        blk_o, bv_o = oracle.block_select(sh, q, w, pooled, block, m, flags, np.arange(R))
        blk, bv = tks.hisa_block_select(S, qd, wd, pd, block, m, flags)
        torch.cuda.synchronize()
        got_b = host(blk).reshape(R, -1)
        got_v = host(bv).reshape(R, -1).astype(np.float64)
        np.testing.assert_array_equal(got_b, blk_o, err_msg="blocks m=%d flags=%d" % (m, flags))
        np.testing.assert_array_equal(got_v, bv_o, err_msg="values m=%d flags=%d" % (m, flags))


def test_small_float_flat_within_tolerance():
    say("float flat L=2048 H=64 D=128 k=512")
    cfg = scaled(CONFIGS[2], n_q=2048, n_k=2048, topk=512)
    x = make_inputs(cfg)
    sh = cfg.shape_dict()
    rows = np.arange(0, 2048, 7)
    qr, wr = cfg_rows(cfg, x, rows)
    oi, ov = oracle.topk_flat(sh, qr, wr, x["k"], None, cfg.topk, rows)
    rs = oracle.row_scores(sh, qr, wr, x["k"], None, rows)
    gi, gv = gpu_flat(sh, x, cfg.topk)
    rec = check_topk_float(gi[rows], gv[rows], oi, ov, rs, "float flat")
    print("recall mean %.5f min %.5f" % (rec.mean(), rec.min()))
    gi2, gv2 = gpu_flat(sh, x, cfg.topk, 300, 512)
    np.testing.assert_array_equal(gi2, gi)     # tiling does not change a float result
    np.testing.assert_array_equal(gv2, gv)

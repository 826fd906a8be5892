"""GPU parity of the fused flat form (one query per sequence, dim 128): the
scoring pass keeps each 4096-key segment's best candidates (with fp8 keys,
each wave's share of the segment) above a threshold of its own, the finish selects the row's top-k from them and
proves it exact, and rows that fail the proof are rescored and selected
exactly.  Integer inputs give exact fp32 scores, so indices and values must
equal the oracle's bit for bit whichever path a row takes; the tests force
the exact rescoring path with tied, equal and clustered scores and check
that it ran (tks_topk_flat_redone).  On float inputs the fused form must
equal the tiled partition-merge bit for bit (same scores, same total
order).  StreamIndex abstract (partition-merge that never materialises the
score tensor) and the threshold-based Indexer-TopK abstract on the same
page (write back only promising candidates, stay exact)."""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_topk_exact, dev, host
from tks_inputs import fp32_to_bf16_bits, fp32_to_e4m3fn
from top_key_selection_amd import tks

pytestmark = pytest.mark.gpu


def say(msg):
    print("[case] " + msg, flush=True)


def decode_case(seed, batch, n_k, heads=64, lo=-4, hi=4, fp8=False, q_pos0=None, ratio=1,
                q_zero=False):
    rng = np.random.default_rng(seed)
    q = rng.integers(lo, hi + 1, (batch, 1, heads, 128)).astype(np.float32)
    if q_zero:
        q[:] = 0.0
    w = rng.integers(lo, hi + 1, (batch, 1, heads)).astype(np.float32)
    kv = rng.integers(lo, hi + 1, (batch, n_k, 128)).astype(np.float32)
    x = dict(q=fp32_to_bf16_bits(q), w=w)
    if fp8:
        x["k"] = fp32_to_e4m3fn(kv)
        x["k_scale"] = (2.0 ** rng.integers(-3, 2, (batch, n_k))).astype(np.float32)
    else:
        x["k"] = fp32_to_bf16_bits(kv)
        x["k_scale"] = None
    sh = dict(batch=batch, n_q=1, n_k=n_k, heads=heads, dim=128,
              q_pos0=n_k - 1 if q_pos0 is None else q_pos0, causal_ratio=ratio,
              key_dtype=int(fp8))
    return sh, x


def run_fused(sh, x, topk, q_chunk=0, k_tile=0):
    S = tks.Shape(**sh)
    q, w, k, ks = dev(x["q"]), dev(x["w"]), dev(x["k"]), dev(x["k_scale"])
    ws = tks.workspace(tks.topk_flat_workspace(S, topk, q_chunk, k_tile), q.device)
    idx, vals = tks.topk_flat(S, q, w, k, ks, topk, q_chunk, k_tile, ws=ws)
    redone = tks.topk_flat_redone(S, topk, ws, q_chunk, k_tile)
    torch.cuda.synchronize()
    R = sh["batch"]
    return host(idx).reshape(R, topk), host(vals).reshape(R, topk), redone


def oracle_rows(sh, x, topk):
    R = sh["batch"]
    rows = np.arange(R)
    return oracle.topk_flat(sh, x["q"].reshape(R, sh["heads"], 128), x["w"].reshape(R, sh["heads"]),
                            x["k"], x["k_scale"], topk, rows)


@pytest.mark.parametrize("fp8", [True, False])
@pytest.mark.parametrize("n_k,topk", [(1, 2048), (700, 2048), (4096, 2048), (4097, 300),
                                      (9000, 2048), (20001, 64), (65536, 2048)])
def test_fused_decode_integer_exact(fp8, n_k, topk):
    """Integer inputs, ragged last segments, fewer keys than k, one key."""
    say("fused decode integer fp8=%d n_k=%d topk=%d" % (fp8, n_k, topk))
    sh, x = decode_case(100 + n_k % 97 + fp8, 6, n_k, fp8=fp8)
    oi, ov = oracle_rows(sh, x, topk)
    gi, gv, redone = run_fused(sh, x, topk)
    print("rows redone by rescoring: %d of %d" % (redone, sh["batch"]), flush=True)
    assert_topk_exact(gi, gv, oi, ov, "fused decode")


@pytest.mark.parametrize("n_k", [262144, 266241])
def test_fused_fp8_long_rows_take_both_filter_forms_exactly(n_k):
    """With fp8 keys every wave of a scoring workgroup filters its own keys as
    a pool segment (four per 4096-key segment) while the finish can take the
    segments (at most 256: rows of up to 262144 keys); longer rows keep one
    filter per 4096-key segment across the workgroup.  Both forms exact on
    integer inputs."""
    say("fused fp8 long rows n_k=%d" % n_k)
    sh, x = decode_case(31 + n_k % 7, 2, n_k, heads=4, fp8=True)
    oi, ov = oracle_rows(sh, x, 2048)
    gi, gv, redone = run_fused(sh, x, 2048)
    print("rows redone by rescoring: %d of %d" % (redone, sh["batch"]), flush=True)
    assert_topk_exact(gi, gv, oi, ov, "fused fp8 n_k=%d" % n_k)


@pytest.mark.parametrize("q_pos0,ratio", [(6500, 1), (40000, 4), (-3, 4), (0, 1)])
def test_fused_decode_partial_visibility_exact(q_pos0, ratio):
    """The query sees only part of the cache (mid-cache position, compressed
    causality, nothing or one key visible)."""
    say("fused decode visibility q_pos0=%d ratio=%d" % (q_pos0, ratio))
    sh, x = decode_case(7 + ratio, 4, 12000, heads=20, fp8=True, q_pos0=q_pos0, ratio=ratio)
    oi, ov = oracle_rows(sh, x, 512)
    gi, gv, _ = run_fused(sh, x, 512)
    assert_topk_exact(gi, gv, oi, ov, "fused visibility")


def test_fused_all_equal_scores_are_redone_and_take_lowest_indices():
    """q = 0: every score is 0, so every segment larger than its survivor cap
    drops all its keys; the finish cannot prove the result and the rows are
    rescored: the answer is keys 0 .. k-1 in order."""
    say("fused all-equal scores (q = 0)")
    sh, x = decode_case(3, 5, 30000, fp8=True, q_zero=True)
    gi, gv, redone = run_fused(sh, x, 2048)
    assert redone == 5
    np.testing.assert_array_equal(gi, np.tile(np.arange(2048, dtype=np.int32), (5, 1)))
    assert np.all(gv == 0.0)


def test_fused_top_keys_clustered_in_one_segment_are_redone_exactly():
    """Keys of one 4096-key segment are made large, so that segment holds
    far more of the row's top-k than its survivor cap: the proof fails and
    the exact rescoring path must give the oracle's answer."""
    say("fused clustered top keys")
    rng = np.random.default_rng(11)
    batch, n_k, heads, topk = 3, 40000, 16, 2048
    q = rng.integers(1, 4, (batch, 1, heads, 128)).astype(np.float32)       # positive
    w = rng.integers(1, 3, (batch, 1, heads)).astype(np.float32)
    kv = rng.integers(-2, 3, (batch, n_k, 128)).astype(np.float32)
    kv[:, 12288:16384] = rng.integers(2, 5, (batch, 4096, 128))             # segment 3
    x = dict(q=fp32_to_bf16_bits(q), w=w, k=fp32_to_bf16_bits(kv), k_scale=None)
    sh = dict(batch=batch, n_q=1, n_k=n_k, heads=heads, dim=128, q_pos0=n_k - 1,
              causal_ratio=1, key_dtype=0)
    oi, ov = oracle_rows(sh, x, topk)
    gi, gv, redone = run_fused(sh, x, topk)
    assert redone == batch
    assert_topk_exact(gi, gv, oi, ov, "fused clustered")
    assert np.all((gi >= 12288) & (gi < 16384))


@pytest.mark.parametrize("fp8", [True, False])
def test_fused_equals_tiled_partition_merge_on_floats(fp8):
    """N(0,1) inputs: the fused form and the tiled partition-merge (explicit
    chunk and tile sizes) see the same fp32 scores, so their outputs are
    identical; no row needs the rescoring path."""
    say("fused vs tiled on floats fp8=%d" % fp8)
    rng = np.random.default_rng(21 + fp8)
    batch, n_k, heads, topk = 8, 30000, 64, 2048
    q = fp32_to_bf16_bits(rng.standard_normal((batch, 1, heads, 128)).astype(np.float32))
    w = (rng.standard_normal((batch, 1, heads)) / 8).astype(np.float32)
    z = rng.standard_normal((batch, n_k, 128)).astype(np.float32)
    if fp8:
        ks = (np.abs(z).max(axis=2) / 448.0).astype(np.float32)
        k = fp32_to_e4m3fn(z / ks[..., None])
    else:
        k, ks = fp32_to_bf16_bits(z), None
    x = dict(q=q, w=w, k=k, k_scale=ks)
    sh = dict(batch=batch, n_q=1, n_k=n_k, heads=heads, dim=128, q_pos0=n_k - 1,
              causal_ratio=1, key_dtype=int(fp8))
    fi, fv, redone = run_fused(sh, x, topk)
    ti, tv, _ = run_fused(sh, x, topk, q_chunk=batch, k_tile=8192)
    assert redone == 0
    np.testing.assert_array_equal(fi, ti)
    np.testing.assert_array_equal(fv.view(np.uint32), tv.view(np.uint32))


def test_fused_many_rows_take_the_wide_grid():
    """More rows than the finish launches wide workgroups for (512): the
    256-thread finish and the persistent repair loop."""
    say("fused 600 sequences")
    sh, x = decode_case(5, 600, 5000, heads=8, lo=-2, hi=2, fp8=True)
    oi, ov = oracle_rows(sh, x, 256)
    gi, gv, redone = run_fused(sh, x, 256)
    print("rows redone by rescoring: %d of %d" % (redone, sh["batch"]), flush=True)
    assert_topk_exact(gi, gv, oi, ov, "fused 600 rows")


def test_wrappers_reject_undersized_tensors_before_launch():
    """The binding checks every tensor's element count against the shape
    before any launch (a short tensor would be read past its end)."""
    say("binding size checks")
    S = tks.Shape(2, 1, 1000, 8, 128, q_pos0=999)
    d = torch.device("cuda")
    q = torch.zeros((2, 1, 8, 128), dtype=torch.bfloat16, device=d)
    w = torch.zeros((2, 1, 8), dtype=torch.float32, device=d)
    k = torch.zeros((2, 1000, 128), dtype=torch.bfloat16, device=d)
    with pytest.raises(ValueError):
        tks.topk_flat(S, q[:1], w, k, None, 16)
    with pytest.raises(ValueError):
        tks.topk_flat(S, q, w[:, :, :4], k, None, 16)
    with pytest.raises(ValueError):
        tks.topk_flat(S, q, w, k[:, :999], None, 16)
    with pytest.raises(ValueError):
        tks.topk_flat(S, q, w, k, None, 16, idx=torch.empty(2 * 15, dtype=torch.int32, device=d))
    with pytest.raises(ValueError):
        tks.topk_flat(S, q, w, k, None, 16, ws=torch.empty(8, dtype=torch.uint8, device=d))
    with pytest.raises(ValueError):
        tks.hisa_pool_keys(S, k, None, 128, pooled=torch.empty((2, 6, 128), dtype=torch.bfloat16,
                                                               device=d))
    blk = torch.zeros((2, 1, 3), dtype=torch.int32, device=d)
    with pytest.raises(ValueError):
        tks.hisa_refine_topk(S, q, w, k, None, 128, blk[:1], 16)
    S8 = tks.Shape(2, 1, 1000, 8, 128, q_pos0=999, key_dtype=tks.KEY_FP8_E4M3FN)
    k8 = torch.zeros((2, 1000, 128), dtype=torch.uint8, device=d)
    with pytest.raises(ValueError):
        tks.topk_flat(S8, q, w, k8, None, 16)
    with pytest.raises(ValueError):
        tks.topk_flat(S8, q, w, k8, torch.ones(1999, device=d), 16)

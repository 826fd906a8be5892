"""C ABI contract, checked on the CPU: the library loads without a GPU, it
exports every function include/tks.h declares, and each malformed or
unsupported argument returns its documented status before any launch (no
call here reaches the GPU)."""
import ctypes
import os
import re

import pytest

from top_key_selection_amd import tks

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

EINVAL, EUNSUP, EWS = tks.EINVAL, tks.EUNSUPPORTED, tks.EWORKSPACE
A = ctypes.c_void_p(4096)        # aligned fake device address (never dereferenced)
MIS = ctypes.c_void_p(4096 + 2)  # misaligned fake address


def header_functions():
    text = open(os.path.join(ROOT, "include", "tks.h")).read()
    return sorted(set(re.findall(r"\b(tks_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = tks.lib()
    names = header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(tks.SYMBOLS)


def test_version_and_empty_error():
    assert tks.version() >= 100


def S(**kw):
    base = dict(batch=1, n_q=16, n_k=16, heads=4, dim=32)
    base.update(kw)
    return tks.Shape(**base).c()


def flat(shape, q=A, w=A, k=A, ks=None, topk=4, qc=0, kt=0, idx=A, vals=None, ws=A, wsb=1 << 30):
    return tks.lib().tks_topk_flat(ctypes.byref(shape), q, w, k, ks, topk, qc, kt, idx, vals, ws,
                                   wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(heads=0), EUNSUP), (dict(heads=65), EUNSUP), (dict(dim=48), EUNSUP),
    (dict(dim=256), EUNSUP), (dict(causal_ratio=0), EINVAL), (dict(n_q=-1), EINVAL),
    (dict(key_dtype=7), EINVAL), (dict(batch=1 << 20, n_q=1 << 12), EUNSUP),
])
def test_flat_rejects_bad_shapes(kw, code):
    assert flat(S(**kw)) == code
    assert tks.last_error()


def test_flat_rejects_bad_arguments():
    s = S()
    assert flat(s, topk=0) == EUNSUP
    assert flat(s, topk=2049) == EUNSUP
    assert flat(s, q=None) == EINVAL
    assert flat(s, w=None) == EINVAL
    assert flat(s, k=None) == EINVAL
    assert flat(s, idx=None) == EINVAL
    assert flat(s, q=MIS) == EINVAL
    assert flat(s, k=MIS) == EINVAL
    assert flat(s, kt=33) == EINVAL
    assert flat(s, qc=-1) == EINVAL
    assert flat(S(key_dtype=1)) == EINVAL          # fp8 keys without scales
    assert flat(s, ws=None) == EWS
    assert flat(s, wsb=0) == EWS
    assert flat(s, ws=MIS) == EINVAL
    assert "workspace" in (flat(s, wsb=1) and tks.last_error())


def test_empty_problem_is_ok_without_launch():
    assert flat(S(n_q=0), q=None, w=None, k=None, idx=None) == tks.OK
    assert flat(S(batch=0), q=None, w=None, k=None, idx=None) == tks.OK


def test_workspace_queries():
    s = tks.Shape(1, 8192, 8192, 64, 128)
    assert tks.topk_flat_workspace(s, 2048) >= 8192 * 4
    # tiled plans carry the running top-k lists
    tiled = tks.topk_flat_workspace(s, 2048, q_chunk=1024, k_tile=2048)
    assert tiled == 1024 * 2048 * 4 + 2 * 1024 * 2048 * 4
    s5 = tks.Shape(1, 262144, 65536, 64, 128, causal_ratio=4)
    ws5 = tks.topk_flat_workspace(s5, 2048, 4096, 8192)
    assert ws5 == 4096 * 8192 * 4 + 2 * 4096 * 2048 * 4   # O(q_chunk * (k_tile + k))
    full = tks.materialized_score_bytes(1, 262144, 64, 65536)
    assert ws5 * 1000 < full
    assert tks.topk_flat_workspace(tks.Shape(1, 8, 8, 0, 32), 4) == 0   # invalid -> 0


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_no_workload_plan_holds_every_score(cid):
    """The automatic flat plan of every workload stays below the fp32
    [batch * n_q, n_k] score tensor (StreamIndex abstract: the chunked
    partition-merge never materialises the full intermediate)."""
    from tks_inputs import CONFIGS
    cfg = CONFIGS[cid]
    s = tks.Shape(**cfg.shape_dict())
    full = cfg.batch * cfg.n_q * cfg.n_k * 4
    for qc, kt in {(0, 0), (cfg.q_chunk, cfg.k_tile)}:
        ws = tks.topk_flat_workspace(s, cfg.topk, qc, kt)
        assert 0 < ws < full, (cid, qc, kt, ws, full)


def test_fused_decode_plan_holds_survivors_not_scores():
    """One query per sequence: the fused plan keeps at most 4096 candidates
    per row (8-byte composites) and a bounded rescoring arena; the decode
    workload's 64 x 65,536 scores (16 MiB) are never held."""
    s = tks.Shape(64, 1, 65536, 64, 128, q_pos0=65535, key_dtype=tks.KEY_FP8_E4M3FN)
    ws = tks.topk_flat_workspace(s, 2048)
    assert ws <= 64 * 4096 * 8 + 64 * (4096 + 2 * 2048) * 4 + 64 * 1024
    assert ws < 64 * 65536 * 4 // 3
    # explicit chunk / tile sizes keep the tiled partition-merge
    assert tks.topk_flat_workspace(s, 2048, 64, 16384) == 64 * 16384 * 4 + 2 * 64 * 2048 * 4


def test_static_scratch_entry_refuses_an_oversized_plan_before_any_gpu_call():
    """tks_topk_flat_static checks its plan against the static scratch
    before touching a device (this runs without a GPU)."""
    s = S(n_q=8192, n_k=8192, heads=4, dim=32)
    assert tks.topk_flat_workspace(tks.Shape(1, 8192, 8192, 4, 32), 2048) > tks.STATIC_SCRATCH_BYTES
    rc = tks.lib().tks_topk_flat_static(ctypes.byref(s), A, A, A, None, 2048, 0, 0, A, None, None)
    assert rc == EWS and "static scratch" in tks.last_error()
    assert tks.lib().tks_topk_flat_static(ctypes.byref(S(dim=48)), A, A, A, None, 4, 0, 0, A, None,
                                          None) == EUNSUP


def test_materialized_score_size_matches_pages():
    # StreamIndex abstract: [B,S,H_I,T] fp32 at S=65,536, H_I=64, T=S/4 is 256 GB
    assert tks.materialized_score_bytes(1, 65536, 64, 65536 // 4) == 2 ** 38


def test_scores_rejects():
    L = tks.lib()
    s = S()
    f = lambda *a: L.tks_indexer_scores(ctypes.byref(s), *a, None)
    assert f(A, A, A, None, 0, 17, 0, 4, A) == EINVAL      # q range past n_q
    assert f(A, A, A, None, 0, 4, 10, 7, A) == EINVAL      # k range past n_k
    assert f(A, A, A, None, 0, 4, 0, 4, None) == EINVAL    # no output
    assert f(A, A, A, None, 0, 0, 0, 4, None) == tks.OK    # empty rectangle


def test_topk_scores_rejects():
    L = tks.lib()
    f = lambda *a: L.tks_topk_scores(*a, None, 0, None)
    assert f(A, 4, 8, 4, None, 2, A, None) == EINVAL       # stride < n_cols
    assert f(A, 4, 8, 8, None, 0, A, None) == EUNSUP
    assert f(None, 4, 8, 8, None, 2, A, None) == EINVAL
    assert f(A, 0, 8, 8, None, 2, None, None) == tks.OK


def test_hisa_rejects():
    L = tks.lib()
    s = S(n_k=256)
    pool = lambda blk, k=A, ks=None, out=A: L.tks_hisa_pool_keys(ctypes.byref(s), k, ks, blk, out, None)
    assert pool(48) == EUNSUP
    assert pool(100) == EUNSUP
    assert pool(64, out=None) == EINVAL
    assert pool(64, k=MIS) == EINVAL
    sel = lambda blk, m, flags, mt, ws=A, wsb=1 << 30: L.tks_hisa_block_select(
        ctypes.byref(s), A, A, A, blk, m, flags, A, None, mt, ws, wsb, None)
    assert sel(64, 4, 2, 4) == EINVAL          # m_total must count the forced block
    assert sel(64, 4, 4, 5) == EINVAL          # unknown flag
    assert sel(64, 600, 0, 600) == EUNSUP      # too many blocks
    assert sel(64, 4, 2, 5, ws=None) == EWS
    ref = lambda blk, mt, topk: L.tks_hisa_refine_topk(ctypes.byref(s), A, A, A, None, blk, A, mt,
                                                       topk, 0, A, None, A, 1 << 30, None)
    assert ref(64, 0, 4) == EUNSUP
    assert ref(64, 4, 0) == EUNSUP
    assert ref(96, 4, 4) == EUNSUP


def test_kv_append_rejects():
    L = tks.lib()

    def app(s, raw=A, n_new=4, raw_len=0, tail=A, k=A, ks=None, blk=0, pooled=None):
        return L.tks_kv_append(ctypes.byref(s), raw, n_new, raw_len, tail, k, ks, blk, pooled, None)

    s4 = S(n_k=16, causal_ratio=4)
    assert app(s4, raw_len=-1) == EINVAL
    assert app(s4, n_new=-1) == EINVAL
    assert app(s4, n_new=68) == EINVAL                      # 68 // 4 > 16 keys
    assert app(s4, raw_len=60, n_new=8) == EINVAL
    assert "overflows" in tks.last_error()
    assert app(s4, blk=48) == EUNSUP
    assert app(s4, blk=64, pooled=None) == EINVAL
    assert app(s4, raw=None) == EINVAL
    assert app(s4, raw=MIS) == EINVAL
    assert app(s4, tail=None) == EINVAL                     # ratio 4 stages raw keys
    assert app(s4, k=None) == EINVAL
    assert app(S(n_k=16, key_dtype=1)) == EINVAL            # fp8 cache without scales
    assert app(s4, n_new=0, raw=None, tail=None, k=None) == tks.OK   # nothing to append
    assert app(S(batch=0, causal_ratio=4), raw=None, tail=None, k=None) == tks.OK


def test_gather_rejects():
    L = tks.lib()
    g = lambda kv=A, b=2, n_kv=10, rb=64, idx=A, n_q=3, k=4, out=A: L.tks_gather_selected(
        kv, b, n_kv, rb, idx, n_q, k, out, None)
    assert g(rb=0) == EUNSUP
    assert g(rb=24) == EUNSUP
    assert g(rb=65552) == EUNSUP
    assert g(idx=None) == EINVAL
    assert g(out=None) == EINVAL
    assert g(out=MIS) == EINVAL
    assert g(kv=MIS) == EINVAL
    assert g(n_q=-1) == EINVAL
    assert g(k=0, idx=None, out=None) == tks.OK


def test_sparse_attention_rejects():
    L = tks.lib()

    def att(q=A, k=A, v=A, b=2, nq=1, h=64, d=128, nkv=100, idx=A, topk=16, scale=0.1, out=A, ws=A,
            wsb=1 << 30):
        return L.tks_sparse_attention(q, k, v, b, nq, h, d, nkv, idx, topk, scale, out, ws, wsb, None)

    assert att(h=8) == EUNSUP
    assert att(h=40) == EUNSUP
    assert att(h=144) == EUNSUP
    assert att(d=64) == EUNSUP
    assert att(topk=0) == EUNSUP
    assert att(topk=2049) == EUNSUP
    assert att(scale=float("nan")) == EINVAL
    assert att(q=MIS) == EINVAL
    assert att(idx=None) == EINVAL
    assert att(out=None) == EINVAL
    assert att(ws=None) == EWS
    assert att(wsb=16) == EWS
    assert att(b=0, q=None, k=None, v=None, idx=None, out=None, ws=None) == tks.OK
    assert tks.sparse_attention_workspace(2, 1, 64, 2048) >= 2 * 8 * 64 * 128 * 4

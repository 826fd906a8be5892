"""Python binding of libtks.so (include/tks.h): argument marshalling only.

Every call goes to the HIP library; there is no fallback.  PyTorch provides
device memory (outputs and workspaces are allocated as torch tensors) and the
current HIP stream.  Function names mirror the C entry points without the
``tks_`` prefix.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# TKS_LIB overrides the library file (the sanitizer check loads a host-only,
# AddressSanitizer-instrumented build of the same sources through it)
LIB_PATH = os.environ.get("TKS_LIB") or os.path.join(_HERE, "libtks.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, -1, -2, -3, -4
KEY_BF16, KEY_FP8_E4M3FN = 0, 1
FORCE_FIRST, FORCE_LOCAL = 1, 2


class TksError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("tks status %d: %s" % (code, msg))
        self.code = code


class CShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "n_q", "n_k", "heads", "dim", "q_pos0", "causal_ratio", "key_dtype")]


@dataclasses.dataclass
class Shape:
    batch: int
    n_q: int
    n_k: int
    heads: int
    dim: int
    q_pos0: int = 0
    causal_ratio: int = 1
    key_dtype: int = KEY_BF16

    def c(self) -> CShape:
        return CShape(self.batch, self.n_q, self.n_k, self.heads, self.dim, self.q_pos0,
                      self.causal_ratio, self.key_dtype)


SYMBOLS = ("tks_version", "tks_last_error", "tks_indexer_scores", "tks_topk_flat_workspace",
           "tks_topk_flat", "tks_topk_flat_static", "tks_topk_flat_redone",
           "tks_topk_scores_workspace", "tks_topk_scores",
           "tks_hisa_pool_keys", "tks_hisa_block_select_workspace", "tks_hisa_block_select",
           "tks_hisa_refine_workspace", "tks_hisa_refine_topk", "tks_kv_append",
           "tks_gather_selected", "tks_sparse_attention_workspace", "tks_sparse_attention",
           "tks_profile_enable", "tks_profile_read")

_lib = None


def lib() -> ctypes.CDLL:
    """Load libtks.so; raises if the HIP library has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libtks.so is not built (run `python -m top_key_selection_amd.build` "
                          "or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, sz, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, \
        ctypes.c_uint32
    SP = ctypes.POINTER(CShape)
    L.tks_version.restype = ctypes.c_int
    L.tks_last_error.restype = ctypes.c_char_p
    L.tks_indexer_scores.argtypes = [SP, P, P, P, P, i32, i32, i32, i32, P, P]
    L.tks_topk_flat_workspace.argtypes = [SP, i32, i32, i32]
    L.tks_topk_flat_workspace.restype = sz
    L.tks_topk_flat.argtypes = [SP, P, P, P, P, i32, i32, i32, P, P, P, sz, P]
    L.tks_topk_flat_redone.argtypes = [SP, i32, i32, i32, P, P, P]
    L.tks_topk_flat_static.argtypes = [SP, P, P, P, P, i32, i32, i32, P, P, P]
    L.tks_topk_scores_workspace.argtypes = [i32, i32, i32]
    L.tks_topk_scores_workspace.restype = sz
    L.tks_topk_scores.argtypes = [P, i32, i32, i64, P, i32, P, P, P, sz, P]
    L.tks_hisa_pool_keys.argtypes = [SP, P, P, i32, P, P]
    L.tks_hisa_block_select_workspace.argtypes = [SP, i32, i32]
    L.tks_hisa_block_select_workspace.restype = sz
    L.tks_hisa_block_select.argtypes = [SP, P, P, P, i32, i32, u32, P, P, i32, P, sz, P]
    L.tks_hisa_refine_workspace.argtypes = [SP, i32, i32, i32, i32]
    L.tks_hisa_refine_workspace.restype = sz
    L.tks_hisa_refine_topk.argtypes = [SP, P, P, P, P, i32, P, i32, i32, i32, P, P, P, sz, P]
    L.tks_kv_append.argtypes = [SP, P, i32, i32, P, P, P, i32, P, P]
    L.tks_gather_selected.argtypes = [P, i32, i32, i32, P, i32, i32, P, P]
    L.tks_sparse_attention_workspace.argtypes = [i32, i32, i32, i32]
    L.tks_sparse_attention_workspace.restype = sz
    L.tks_sparse_attention.argtypes = [P, P, P, i32, i32, i32, i32, i32, P, i32, ctypes.c_float, P, P, sz, P]
    L.tks_profile_enable.argtypes = [ctypes.c_int]
    L.tks_profile_read.argtypes = [ctypes.c_char_p, P, P]
    for s in L.tks_profile_enable, L.tks_profile_read, L.tks_indexer_scores, L.tks_topk_flat, \
            L.tks_topk_flat_redone, L.tks_topk_flat_static, L.tks_topk_scores, L.tks_hisa_pool_keys, \
            L.tks_hisa_block_select, L.tks_hisa_refine_topk, L.tks_kv_append, L.tks_gather_selected, \
            L.tks_sparse_attention:
        s.restype = ctypes.c_int
    _lib = L
    return L


def last_error() -> str:
    return lib().tks_last_error().decode()


def _check(rc: int):
    if rc != OK:
        raise TksError(rc, last_error())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, name, dtypes):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype not in dtypes:
        raise ValueError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _size(t, name, numel):
    """Every buffer must hold exactly the elements its layout needs: a short
    tensor would be read or written past its end by the kernels."""
    if t is not None and t.numel() != numel:
        raise ValueError("%s holds %d elements, the layout needs %d" % (name, t.numel(), numel))
    return t


def _ws(ws, need, dev):
    if ws is None:
        return workspace(need, dev)
    if not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    if ws.numel() * ws.element_size() < need:
        raise ValueError("workspace holds %d bytes, the call needs %d"
                         % (ws.numel() * ws.element_size(), need))
    return ws


def _nbytes(t):
    return t.numel() * t.element_size()


def _qwk(shape: Shape, q, w, k, k_scale):
    """Device, dtype, contiguity and element counts of the indexer inputs."""
    _dev(q, "q", _BF16), _dev(w, "w", (torch.float32,)), _dev(k, "k", _key_dtypes(shape))
    _dev(k_scale, "k_scale", (torch.float32,))
    rows = shape.batch * shape.n_q
    _size(q, "q", rows * shape.heads * shape.dim)
    _size(w, "w", rows * shape.heads)
    _size(k, "k", shape.batch * shape.n_k * shape.dim)
    if shape.key_dtype == KEY_FP8_E4M3FN and k_scale is None and shape.batch * shape.n_k > 0:
        raise ValueError("fp8 keys need k_scale")
    _size(k_scale, "k_scale", shape.batch * shape.n_k)


def _out(t, name, numel, dtype, shape3, dev):
    if t is None:
        return torch.empty(shape3, dtype=dtype, device=dev)
    _dev(t, name, (dtype,))
    return _size(t, name, numel)


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_FP8 = (torch.uint8, torch.float8_e4m3fn)


def _key_dtypes(shape: Shape):
    return _FP8 if shape.key_dtype == KEY_FP8_E4M3FN else _BF16


def workspace(nbytes: int, device=None) -> torch.Tensor:
    """A 256-byte aligned device byte buffer (torch's allocator aligns to 512 B)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device or "cuda")


def version() -> int:
    return lib().tks_version()


def indexer_scores(shape: Shape, q, w, k, k_scale, q_begin, q_count, k_begin, k_count, out=None):
    """fp32 [batch, q_count, k_count] scores, -inf where not visible."""
    _qwk(shape, q, w, k, k_scale)
    out = _out(out, "out", shape.batch * q_count * k_count, torch.float32,
               (shape.batch, q_count, k_count), q.device)
    S = shape.c()
    _check(lib().tks_indexer_scores(ctypes.byref(S), _p(q), _p(w), _p(k), _p(k_scale), q_begin,
                                    q_count, k_begin, k_count, _p(out), _stream()))
    return out


def topk_flat_workspace(shape: Shape, topk, q_chunk=0, k_tile=0) -> int:
    S = shape.c()
    return int(lib().tks_topk_flat_workspace(ctypes.byref(S), topk, q_chunk, k_tile))


def topk_flat(shape: Shape, q, w, k, k_scale, topk, q_chunk=0, k_tile=0, with_vals=True,
              ws=None, idx=None, vals=None):
    """Flat indexer top-k: (idx int32 [batch, n_q, topk], vals fp32 | None)."""
    _qwk(shape, q, w, k, k_scale)
    dev = q.device
    n_out = shape.batch * shape.n_q * topk
    idx = _out(idx, "idx", n_out, torch.int32, (shape.batch, shape.n_q, topk), dev)
    if vals is not None or with_vals:
        vals = _out(vals, "vals", n_out, torch.float32, (shape.batch, shape.n_q, topk), dev)
    ws = _ws(ws, topk_flat_workspace(shape, topk, q_chunk, k_tile), dev)
    S = shape.c()
    _check(lib().tks_topk_flat(ctypes.byref(S), _p(q), _p(w), _p(k), _p(k_scale), topk, q_chunk,
                               k_tile, _p(idx), _p(vals), _p(ws), _nbytes(ws), _stream()))
    return idx, vals


STATIC_SCRATCH_BYTES = 16 << 20  # TKS_STATIC_SCRATCH_BYTES


def topk_flat_static(shape: Shape, q, w, k, k_scale, topk, q_chunk=0, k_tile=0, with_vals=True,
                     idx=None, vals=None):
    """topk_flat with the library's static device scratch instead of a
    workspace (nothing is allocated by the library; outputs are allocated
    here unless given).  Calls that overlap on one GPU must not be issued."""
    _qwk(shape, q, w, k, k_scale)
    dev = q.device
    n_out = shape.batch * shape.n_q * topk
    idx = _out(idx, "idx", n_out, torch.int32, (shape.batch, shape.n_q, topk), dev)
    if vals is not None or with_vals:
        vals = _out(vals, "vals", n_out, torch.float32, (shape.batch, shape.n_q, topk), dev)
    S = shape.c()
    _check(lib().tks_topk_flat_static(ctypes.byref(S), _p(q), _p(w), _p(k), _p(k_scale), topk,
                                      q_chunk, k_tile, _p(idx), _p(vals), _stream()))
    return idx, vals


def topk_flat_redone(shape: Shape, topk, ws, q_chunk=0, k_tile=0) -> int:
    """Rows of the last topk_flat call on workspace `ws` that the fused form
    redid by exact rescoring (0 for the tiled form).  Synchronises."""
    n = ctypes.c_int32()
    S = shape.c()
    _check(lib().tks_topk_flat_redone(ctypes.byref(S), topk, q_chunk, k_tile, _p(ws),
                                      ctypes.byref(n), _stream()))
    return n.value


def topk_scores_workspace(n_rows, n_cols, topk) -> int:
    return int(lib().tks_topk_scores_workspace(n_rows, n_cols, topk))


def topk_scores(scores, topk, row_len=None, with_vals=True, ws=None, idx=None, vals=None):
    """Top-k of each row of an fp32 [n_rows, n_cols] (row-strided) score matrix."""
    _dev(scores, "scores", (torch.float32,)) if scores.is_contiguous() else None
    if scores.dim() != 2 or scores.stride(1) != 1:
        raise ValueError("scores must be 2-D with unit column stride")
    n_rows, n_cols = scores.shape
    _dev(row_len, "row_len", (torch.int32,))
    dev = scores.device
    if idx is None:
        idx = torch.empty((n_rows, topk), dtype=torch.int32, device=dev)
    if vals is None and with_vals:
        vals = torch.empty((n_rows, topk), dtype=torch.float32, device=dev)
    _dev(idx, "idx", (torch.int32,)), _dev(vals, "vals", (torch.float32,))
    for t, name in ((idx, "idx"), (vals, "vals")):
        if t is not None and t.numel() != n_rows * topk:
            raise ValueError("%s must hold n_rows x topk = %d elements" % (name, n_rows * topk))
    _size(row_len, "row_len", n_rows)
    ws = _ws(ws, topk_scores_workspace(n_rows, n_cols, topk), dev)
    _check(lib().tks_topk_scores(_p(scores), n_rows, n_cols, scores.stride(0), _p(row_len), topk,
                                 _p(idx), _p(vals), _p(ws), _nbytes(ws), _stream()))
    return idx, vals


def hisa_pool_keys(shape: Shape, k, k_scale, block, pooled=None):
    """bf16 [batch, n_k // block, dim] pooled keys."""
    _dev(k, "k", _key_dtypes(shape)), _dev(k_scale, "k_scale", (torch.float32,))
    _size(k, "k", shape.batch * shape.n_k * shape.dim)
    _size(k_scale, "k_scale", shape.batch * shape.n_k)
    if block <= 0:
        raise ValueError("block must be positive")
    nb = shape.n_k // block
    if pooled is None:
        pooled = torch.empty((shape.batch, nb, shape.dim), dtype=torch.bfloat16, device=k.device)
    _dev(pooled, "pooled", _BF16)
    _size(pooled, "pooled", shape.batch * nb * shape.dim)
    S = shape.c()
    _check(lib().tks_hisa_pool_keys(ctypes.byref(S), _p(k), _p(k_scale), block, _p(pooled),
                                    _stream()))
    return pooled


def kv_append(shape: Shape, raw, raw_len, k, k_scale=None, raw_tail=None, block=0, pooled=None):
    """Append raw bf16 keys [batch, n_new, dim] to the compressed key cache
    (k, k_scale) whose raw streams hold raw_len keys; with block > 0 the
    completed pooled blocks are written to pooled [batch, n_k // block, dim].
    raw_tail: bf16 [batch, causal_ratio, dim] staging kept between calls."""
    _dev(raw, "raw", _BF16), _dev(k, "k", _key_dtypes(shape))
    _dev(k_scale, "k_scale", (torch.float32,)), _dev(raw_tail, "raw_tail", _BF16)
    _dev(pooled, "pooled", _BF16)
    if raw.dim() != 3 or raw.shape[0] != shape.batch or raw.shape[2] != shape.dim:
        raise ValueError("raw must be [batch, n_new, dim]")
    _size(k, "k", shape.batch * shape.n_k * shape.dim)
    if shape.key_dtype == KEY_FP8_E4M3FN:
        _size(k_scale, "k_scale", shape.batch * shape.n_k)
    if shape.causal_ratio > 1:
        _size(raw_tail, "raw_tail", shape.batch * shape.causal_ratio * shape.dim)
    if block > 0:
        _size(pooled, "pooled", shape.batch * (shape.n_k // block) * shape.dim)
    S = shape.c()
    _check(lib().tks_kv_append(ctypes.byref(S), _p(raw), raw.shape[1], int(raw_len), _p(raw_tail),
                               _p(k), _p(k_scale), int(block), _p(pooled), _stream()))


def gather_selected(kv, idx, out=None):
    """Rows kv[b, idx[b, t, j]] copied to a contiguous [batch, n_q, topk, ...]
    buffer (zeros for -1).  kv: [batch, n_kv, ...] device tensor whose rows are
    a multiple of 16 bytes; idx: int32 [batch, n_q, topk]."""
    if not kv.is_cuda or not kv.is_contiguous() or not idx.is_cuda or not idx.is_contiguous():
        raise ValueError("kv and idx must be contiguous device tensors")
    if idx.dtype != torch.int32 or idx.dim() != 3 or idx.shape[0] != kv.shape[0]:
        raise ValueError("idx must be int32 [batch, n_q, topk]")
    batch, n_kv = kv.shape[0], kv.shape[1]
    row_bytes = kv[0, 0].numel() * kv.element_size() if kv.numel() else 0
    if out is None:
        out = torch.empty((batch, idx.shape[1], idx.shape[2]) + tuple(kv.shape[2:]), dtype=kv.dtype,
                          device=kv.device)
    if not out.is_cuda or not out.is_contiguous() or _nbytes(out) != idx.numel() * row_bytes:
        raise ValueError("out must be a contiguous device tensor of batch x n_q x topk rows")
    _check(lib().tks_gather_selected(_p(kv), batch, n_kv, row_bytes, _p(idx), idx.shape[1], idx.shape[2],
                                     _p(out), _stream()))
    return out


def sparse_attention_workspace(batch, n_q, heads, topk) -> int:
    return int(lib().tks_sparse_attention_workspace(batch, n_q, heads, topk))


def sparse_attention(q, k, v, idx, scale, out=None, ws=None):
    """fp32 [batch, n_q, heads, 128]: attention of q over the keys idx selects.
    q bf16 [batch, n_q, heads, 128]; k, v bf16 [batch, n_kv, 128]; idx int32
    [batch, n_q, topk]."""
    _dev(q, "q", _BF16), _dev(k, "k", _BF16), _dev(v, "v", _BF16), _dev(idx, "idx", (torch.int32,))
    if q.dim() != 4 or k.dim() != 3 or tuple(v.shape) != tuple(k.shape) or idx.dim() != 3:
        raise ValueError("q [batch, n_q, heads, dim], k / v [batch, n_kv, dim], idx [batch, n_q, topk]")
    batch, n_q, heads, dim = q.shape
    if k.shape[0] != batch or k.shape[2] != dim or tuple(idx.shape[:2]) != (batch, n_q):
        raise ValueError("q, k / v and idx disagree on batch, n_q or dim")
    topk = idx.shape[2]
    out = _out(out, "out", batch * n_q * heads * dim, torch.float32, (batch, n_q, heads, dim),
               q.device)
    ws = _ws(ws, sparse_attention_workspace(batch, n_q, heads, topk), q.device)
    _check(lib().tks_sparse_attention(_p(q), _p(k), _p(v), batch, n_q, heads, dim, k.shape[1], _p(idx), topk,
                                      float(scale), _p(out), _p(ws), _nbytes(ws), _stream()))
    return out


def m_total_of(m_scored: int, force_flags: int) -> int:
    return m_scored + bin(force_flags & 3).count("1")


def hisa_block_select_workspace(shape: Shape, block, m_scored) -> int:
    S = shape.c()
    return int(lib().tks_hisa_block_select_workspace(ctypes.byref(S), block, m_scored))


def hisa_block_select(shape: Shape, q, w, pooled, block, m_scored, force_flags, with_vals=True,
                      ws=None, blk=None, blk_vals=None):
    """(blk int32 [batch, n_q, m_total] ascending, blk_vals fp32 | None)."""
    _dev(q, "q", _BF16), _dev(w, "w", (torch.float32,)), _dev(pooled, "pooled", _BF16)
    rows = shape.batch * shape.n_q
    _size(q, "q", rows * shape.heads * shape.dim)
    _size(w, "w", rows * shape.heads)
    if block <= 0:
        raise ValueError("block must be positive")
    _size(pooled, "pooled", shape.batch * (shape.n_k // block) * shape.dim)
    m_total = m_total_of(m_scored, force_flags)
    dev = q.device
    blk = _out(blk, "blk", rows * m_total, torch.int32, (shape.batch, shape.n_q, m_total), dev)
    if blk_vals is not None or with_vals:
        blk_vals = _out(blk_vals, "blk_vals", rows * m_total, torch.float32,
                        (shape.batch, shape.n_q, m_total), dev)
    ws = _ws(ws, hisa_block_select_workspace(shape, block, m_scored), dev)
    S = shape.c()
    _check(lib().tks_hisa_block_select(ctypes.byref(S), _p(q), _p(w), _p(pooled), block, m_scored,
                                       force_flags, _p(blk), _p(blk_vals), m_total, _p(ws),
                                       _nbytes(ws), _stream()))
    return blk, blk_vals


def hisa_refine_workspace(shape: Shape, block, m_total, topk, q_chunk=0) -> int:
    S = shape.c()
    return int(lib().tks_hisa_refine_workspace(ctypes.byref(S), block, m_total, topk, q_chunk))


def hisa_refine_topk(shape: Shape, q, w, k, k_scale, block, blk, topk, q_chunk=0, with_vals=True,
                     ws=None, idx=None, vals=None):
    """(idx int32 [batch, n_q, topk], vals fp32 | None) inside the kept blocks."""
    _qwk(shape, q, w, k, k_scale)
    _dev(blk, "blk", (torch.int32,))
    rows = shape.batch * shape.n_q
    m_total = blk.shape[-1] if blk.dim() > 0 else 0
    _size(blk, "blk", rows * m_total)
    dev = q.device
    idx = _out(idx, "idx", rows * topk, torch.int32, (shape.batch, shape.n_q, topk), dev)
    if vals is not None or with_vals:
        vals = _out(vals, "vals", rows * topk, torch.float32, (shape.batch, shape.n_q, topk), dev)
    ws = _ws(ws, hisa_refine_workspace(shape, block, m_total, topk, q_chunk), dev)
    S = shape.c()
    _check(lib().tks_hisa_refine_topk(ctypes.byref(S), _p(q), _p(w), _p(k), _p(k_scale), block,
                                      _p(blk), m_total, topk, q_chunk, _p(idx), _p(vals), _p(ws),
                                      _nbytes(ws), _stream()))
    return idx, vals


def hisa_topk(shape: Shape, q, w, k, k_scale, block, m_scored, force_flags, topk, pooled=None,
              with_vals=True):
    """Whole HISA indexer: pool (unless `pooled` is given), block select, refine.
    Returns (idx, vals, blk)."""
    if pooled is None:
        pooled = hisa_pool_keys(shape, k, k_scale, block)
    blk, _ = hisa_block_select(shape, q, w, pooled, block, m_scored, force_flags, with_vals=False)
    idx, vals = hisa_refine_topk(shape, q, w, k, k_scale, block, blk, topk, with_vals=with_vals)
    return idx, vals, blk


PROFILE_ROLES = ("score_flat", "score_pooled", "score_refine", "select_flat", "select_pooled",
                 "select_refine", "select_scores", "pool", "append", "gather", "attend")


def profile_enable(on: bool = True):
    """Bracket every library kernel launch with HIP events (see tks.h)."""
    _check(lib().tks_profile_enable(1 if on else 0))


def profile_read(role: str):
    """(total_ms, launches) of one kernel role since profile_enable(True)."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib().tks_profile_read(role.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def materialized_score_bytes(batch: int, seq: int, heads: int, keys: int) -> int:
    """Bytes of the [B, S, H_I, T] fp32 score tensor a materialising indexer
    builds before its top-k (StreamIndex abstract: 256 GB at S = 65,536,
    H_I = 64, T = S / 4).  This library never allocates it."""
    return batch * seq * heads * keys * 4

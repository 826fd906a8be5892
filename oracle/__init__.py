"""ctypes wrapper of the plain CPU oracle (tks_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library or its binding.  It
shares no code with the GPU path; only the seeded input generator
(``tks_inputs``) feeds both.

All functions take numpy arrays in the path's storage formats (bf16 bit
patterns as uint16, e4m3fn codes as uint8) and return numpy arrays; scores
come back as float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tks_oracle.c")
_LIB = os.path.join(_HERE, "libtks_oracle.so")
# TKS_ORACLE_LIB: an oracle built elsewhere (the sanitizer check's build)
_LIB_OVERRIDE = os.environ.get("TKS_ORACLE_LIB")

FORCE_FIRST = 1
FORCE_LOCAL = 2


class _Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "n_q", "n_k", "heads", "dim", "q_pos0", "causal_ratio", "key_fp8")]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP).  Returns the library path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=gnu11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(out_dir: str) -> str:
    """The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
    (ROCm's clang, whose runtime also serves the sanitized library build; no
    OpenMP) into out_dir.  Returns the library path."""
    os.makedirs(out_dir, exist_ok=True)
    out = os.path.join(out_dir, "libtks_oracle.so")
    if not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(_SRC):
        subprocess.check_call(["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-fno-omit-frame-pointer",
                               "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                               "-std=gnu11", "-fPIC", "-shared", "-Wall", "-Wextra", _SRC, "-o",
                               out, "-lm"])
    return out


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, u32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
        SP = ctypes.POINTER(_Shape)
        L.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_double.restype = ctypes.c_double
        L.orc_e4m3fn_to_double.argtypes = [ctypes.c_uint8]
        L.orc_e4m3fn_to_double.restype = ctypes.c_double
        L.orc_double_to_bf16.argtypes = [ctypes.c_double]
        L.orc_double_to_bf16.restype = ctypes.c_uint16
        L.orc_float_to_e4m3fn.argtypes = [ctypes.c_float]
        L.orc_float_to_e4m3fn.restype = ctypes.c_uint8
        L.orc_compress_keys.argtypes = [SP, P, i64, P, P]
        L.orc_n_visible.argtypes = [SP, i64]
        L.orc_n_visible.restype = i64
        L.orc_index_scores.argtypes = [SP, P, P, P, P, i32, i32, i32, i32, P]
        L.orc_topk_flat.argtypes = [SP, P, P, P, P, i32, P, i64, P, P]
        L.orc_row_scores.argtypes = [SP, P, P, P, P, P, i64, P]
        L.orc_pool.argtypes = [SP, P, P, i32, P]
        L.orc_block_select.argtypes = [SP, P, P, P, i32, i32, u32, P, i64, i32, P, P]
        L.orc_refine.argtypes = [SP, P, P, P, P, i32, P, i32, i32, P, i64, P, P]
        L.orc_hisa.argtypes = [SP, P, P, P, P, i32, i32, u32, i32, P, i64, P, P, P]
        L.orc_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _shape(batch, n_q, n_k, heads, dim, q_pos0=0, causal_ratio=1, key_dtype=0):
    return _Shape(batch, n_q, n_k, heads, dim, q_pos0, causal_ratio, int(key_dtype))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return None if a is None else np.ascontiguousarray(a, dtype=dt)


def _keys(k, key_dtype):
    return _c(k, np.uint8 if key_dtype else np.uint16)


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments (rc=%d)" % (what, rc))


def num_threads() -> int:
    return int(lib().orc_num_threads())


def bf16_to_double(bits: int) -> float:
    return lib().orc_bf16_to_double(int(bits))


def e4m3fn_to_double(code: int) -> float:
    return lib().orc_e4m3fn_to_double(int(code))


def double_to_bf16(x: float) -> int:
    return int(lib().orc_double_to_bf16(float(x)))


def float_to_e4m3fn(x: float) -> int:
    return int(lib().orc_float_to_e4m3fn(float(x)))


def n_visible(shape: dict, t: int) -> int:
    S = _shape(**shape)
    return int(lib().orc_n_visible(ctypes.byref(S), int(t)))


def index_scores(shape: dict, q, w, k, k_scale, q_begin, q_count, k_begin, k_count):
    """[batch, q_count, k_count] float64 scores (-inf where not visible).
    q / w: the full [batch, n_q, ...] arrays."""
    S = _shape(**shape)
    q, w, k, ks = _c(q, np.uint16), _c(w, np.float32), _keys(k, S.key_fp8), _c(k_scale, np.float32)
    out = np.empty((S.batch, q_count, k_count), np.float64)
    _check(lib().orc_index_scores(ctypes.byref(S), _ptr(q), _ptr(w), _ptr(k), _ptr(ks),
                                  q_begin, q_count, k_begin, k_count, _ptr(out)), "index_scores")
    return out


def row_scores(shape: dict, q_rows, w_rows, k, k_scale, rows):
    """[n, n_k] float64 scores of every key for the listed rows (-inf where not
    visible).  q_rows / w_rows hold the listed rows only."""
    S = _shape(**shape)
    rows = _c(rows, np.int64)
    out = np.empty((len(rows), S.n_k), np.float64)
    _check(lib().orc_row_scores(ctypes.byref(S), _ptr(_c(q_rows, np.uint16)),
                                _ptr(_c(w_rows, np.float32)), _ptr(_keys(k, S.key_fp8)),
                                _ptr(_c(k_scale, np.float32)), _ptr(rows), len(rows),
                                _ptr(out)), "row_scores")
    return out


def topk_flat(shape: dict, q_rows, w_rows, k, k_scale, topk, rows, with_vals=True):
    """Flat top-k of the listed flat rows (b*n_q+t).  q_rows: [n, H, D] bf16 bits,
    w_rows: [n, H].  Returns (idx int32 [n, topk], vals float64 [n, topk] or None)."""
    S = _shape(**shape)
    rows = _c(rows, np.int64)
    q, w, k, ks = _c(q_rows, np.uint16), _c(w_rows, np.float32), _keys(k, S.key_fp8), \
        _c(k_scale, np.float32)
    n = len(rows)
    idx = np.empty((n, topk), np.int32)
    val = np.empty((n, topk), np.float64) if with_vals else None
    _check(lib().orc_topk_flat(ctypes.byref(S), _ptr(q), _ptr(w), _ptr(k), _ptr(ks), topk,
                               _ptr(rows), n, _ptr(idx), _ptr(val)), "topk_flat")
    return idx, val


def pool(shape: dict, k, k_scale, block):
    """Pooled keys [batch, n_k // block, dim] as bf16 bits."""
    S = _shape(**shape)
    k, ks = _keys(k, S.key_fp8), _c(k_scale, np.float32)
    out = np.empty((S.batch, S.n_k // block, S.dim), np.uint16)
    _check(lib().orc_pool(ctypes.byref(S), _ptr(k), _ptr(ks), block, _ptr(out)), "pool")
    return out


def block_select(shape: dict, q_rows, w_rows, pooled, block, m_scored, flags, rows):
    """(blk int32 [n, m_total], blk_vals float64 [n, m_total])."""
    S = _shape(**shape)
    rows = _c(rows, np.int64)
    m_total = m_scored + bin(flags).count("1")
    blk = np.empty((len(rows), m_total), np.int32)
    bv = np.empty((len(rows), m_total), np.float64)
    _check(lib().orc_block_select(ctypes.byref(S), _ptr(_c(q_rows, np.uint16)),
                                  _ptr(_c(w_rows, np.float32)), _ptr(_c(pooled, np.uint16)),
                                  block, m_scored, flags, _ptr(rows), len(rows), m_total,
                                  _ptr(blk), _ptr(bv)), "block_select")
    return blk, bv


def refine(shape: dict, q_rows, w_rows, k, k_scale, block, blk, topk, rows, with_vals=True):
    """Top-k within the kept blocks blk [n, m_total] of the listed rows."""
    S = _shape(**shape)
    rows = _c(rows, np.int64)
    blk = _c(blk, np.int32)
    n = len(rows)
    idx = np.empty((n, topk), np.int32)
    val = np.empty((n, topk), np.float64) if with_vals else None
    _check(lib().orc_refine(ctypes.byref(S), _ptr(_c(q_rows, np.uint16)),
                            _ptr(_c(w_rows, np.float32)), _ptr(_keys(k, S.key_fp8)),
                            _ptr(_c(k_scale, np.float32)), block, _ptr(blk), blk.shape[1], topk,
                            _ptr(rows), n, _ptr(idx), _ptr(val)), "refine")
    return idx, val


def hisa(shape: dict, q_rows, w_rows, k, k_scale, block, m_scored, flags, topk, rows,
         with_vals=True):
    """Whole HISA indexer: (blk [n, m_total], idx [n, topk], vals [n, topk] | None)."""
    S = _shape(**shape)
    rows = _c(rows, np.int64)
    n = len(rows)
    m_total = m_scored + bin(flags).count("1")
    blk = np.empty((n, m_total), np.int32)
    idx = np.empty((n, topk), np.int32)
    val = np.empty((n, topk), np.float64) if with_vals else None
    _check(lib().orc_hisa(ctypes.byref(S), _ptr(_c(q_rows, np.uint16)),
                          _ptr(_c(w_rows, np.float32)), _ptr(_keys(k, S.key_fp8)),
                          _ptr(_c(k_scale, np.float32)), block, m_scored, flags, topk,
                          _ptr(rows), n, _ptr(blk), _ptr(idx), _ptr(val)), "hisa")
    return blk, idx, val


def compress_keys(raw, ratio: int, key_fp8: bool, n_k: int | None = None):
    """Compressed key cache of raw bf16 keys [batch, n_raw, dim] at ratio m.

    Returns (k, k_scale): k is [batch, n_k, dim] bf16 bits (uint16) or e4m3fn
    codes (uint8), k_scale fp32 [batch, n_k] or None; slots from n_raw // m on
    are zero.  n_k defaults to n_raw // m."""
    raw = _c(raw, np.uint16)
    batch, n_raw, dim = raw.shape
    n_k = n_raw // ratio if n_k is None else n_k
    S = _shape(batch, 1, n_k, 1, dim, 0, ratio, 1 if key_fp8 else 0)
    k = np.zeros((batch, n_k, dim), np.uint8 if key_fp8 else np.uint16)
    ks = np.zeros((batch, n_k), np.float32) if key_fp8 else None
    _check(lib().orc_compress_keys(ctypes.byref(S), _ptr(raw), n_raw, _ptr(k), _ptr(ks)),
           "compress_keys")
    return k, ks


def gather_selected(kv, idx):
    """Re-layout of the selected rows (LongCat Sparse Attention abstract,
    strategy (1): scattered KV entries copied into a contiguous layout):
    out[b, t, j] = kv[b, idx[b, t, j]] when 0 <= idx < n_kv, zeros otherwise.
    kv: [batch, n_kv, ...] numpy array; idx: int [batch, n_q, topk].  Plain
    loops over (b, t, j): for small inputs and sampled rows."""
    kv = np.asarray(kv)
    idx = np.asarray(idx)
    out = np.zeros(idx.shape + kv.shape[2:], kv.dtype)
    for b in range(idx.shape[0]):
        for t in range(idx.shape[1]):
            for j in range(idx.shape[2]):
                s = int(idx[b, t, j])
                if 0 <= s < kv.shape[1]:
                    out[b, t, j] = kv[b, s]
    return out


def sparse_attention(q, k, v, idx, scale):
    """Attention of every query head over its selected keys only (HISA
    abstract: the sparse attention reads only the selected entries; the
    pages give no attention shapes, read here as one shared K / V head):
        p_j = softmax over the valid slots j of scale * q[b, t, h] . k[b, idx_j]
        o[b, t, h] = sum_j p_j v[b, idx_j]
    Slots with idx outside [0, n_kv) (-1 padding) are not keys; a row with
    no valid slot gives zeros.  q: [B, Tq, H, dk], k: [B, n_kv, dk],
    v: [B, n_kv, dv] (float values), idx: int [B, Tq, topk].  fp64, plain
    loops over (b, t)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    idx = np.asarray(idx)
    B, T, H, _ = q.shape
    out = np.zeros((B, T, H, v.shape[2]), np.float64)
    for b in range(B):
        for t in range(T):
            sel = [int(s) for s in idx[b, t] if 0 <= int(s) < k.shape[1]]
            if not sel:
                continue
            kk, vv = k[b, sel], v[b, sel]
            s = scale * (q[b, t] @ kk.T)                 # [H, n_sel]
            s = s - s.max(axis=1, keepdims=True)
            e = np.exp(s)
            out[b, t] = (e / e.sum(axis=1, keepdims=True)) @ vv
    return out

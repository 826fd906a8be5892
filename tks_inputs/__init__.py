"""Seeded synthetic inputs for the indexer + top-k path (shared by the oracle
tests, the GPU parity tests and the benchmark).

This module only draws random numbers and stores them in the input formats
the path consumes (bf16 bit patterns, OCP e4m3fn codes with a per-token fp32
scale, fp32 head weights).  It contains none of the method's arithmetic: no
scoring, pooling or selection.

Workload shapes follow the DeepSeek-V3.2-style indexer described on the HISA
pages (HISA abstract: a lightweight indexer scores every causal key for every
query and keeps a per-query top-k) and the StreamIndex page (abstract: H_I = 64
indexer heads, keys compressed by m = 4, chunk / key-tile sweeps).  No dataset
is used: every tensor is drawn from a counter-addressed PCG64 stream so any
row block can be regenerated on its own.

Streams: tensor ``name`` row-block ``j`` of config seed ``seed`` is drawn from
``PCG64(SeedSequence(entropy=seed, spawn_key=(TENSOR_ID[name], j)))``.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

FORCE_FIRST = 1
FORCE_LOCAL = 2

KEY_BF16 = 0
KEY_FP8 = 1

# Rows of the flattened leading dimension drawn from one PCG64 stream.
ROW_BLOCK = 1024

TENSOR_ID = {"q": 1, "w": 2, "k": 3, "kdrift": 4, "kraw": 5, "append": 6}


@dataclasses.dataclass(frozen=True)
class Config:
    cid: int
    name: str
    batch: int
    n_q: int
    n_k: int
    heads: int
    dim: int
    topk: int
    q_pos0: int = 0
    causal_ratio: int = 1
    key_dtype: int = KEY_BF16
    dist: str = "normal"          # "int" | "normal" | "drift" | "fp8" | "compressed"
    block: int = 128
    m_scored: int = 62
    force: int = FORCE_FIRST | FORCE_LOCAL
    q_chunk: int = 0
    k_tile: int = 0
    seed: int = 0

    @property
    def m_total(self) -> int:
        return self.m_scored + bin(self.force).count("1")

    @property
    def rows(self) -> int:
        return self.batch * self.n_q

    def shape_dict(self) -> dict:
        return dict(batch=self.batch, n_q=self.n_q, n_k=self.n_k, heads=self.heads,
                    dim=self.dim, q_pos0=self.q_pos0, causal_ratio=self.causal_ratio,
                    key_dtype=self.key_dtype)


# The five workloads.  Seeds 1..5 belong to configs 1..5.
CONFIGS = {
    1: Config(1, "tiny_int_1k", batch=1, n_q=1024, n_k=1024, heads=4, dim=32, topk=64,
              dist="int", block=64, m_scored=4, force=FORCE_LOCAL, seed=1),
    2: Config(2, "flat_prefill_8k", batch=1, n_q=8192, n_k=8192, heads=64, dim=128,
              topk=2048, dist="normal", seed=2),
    3: Config(3, "hisa_prefill_32k", batch=1, n_q=32768, n_k=32768, heads=64, dim=128,
              topk=2048, dist="drift", block=128, m_scored=62,
              force=FORCE_FIRST | FORCE_LOCAL, seed=3),
    4: Config(4, "decode_64k_fp8", batch=64, n_q=1, n_k=65536, heads=64, dim=128,
              topk=2048, q_pos0=65535, key_dtype=KEY_FP8, dist="fp8", block=128,
              m_scored=62, force=FORCE_FIRST | FORCE_LOCAL, seed=4),
    5: Config(5, "stream_256k_c4", batch=1, n_q=262144, n_k=65536, heads=64, dim=128,
              topk=2048, causal_ratio=4, dist="compressed", q_chunk=4096, k_tile=8192,
              seed=5),
}


def scaled(cfg: Config, **kw) -> Config:
    """A config with some sizes replaced (for reduced-size parity cases)."""
    return dataclasses.replace(cfg, **kw)


def _rng(seed: int, tensor: str, block: int) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(TENSOR_ID[tensor], block))
    return np.random.Generator(np.random.PCG64(ss))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def fp32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_fp32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _e4m3fn_table() -> np.ndarray:
    """Magnitudes of the 127 non-NaN non-negative OCP e4m3fn codes 0x00..0x7E."""
    codes = np.arange(127)
    e = codes >> 3
    m = codes & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))


_E4M3 = _e4m3fn_table()


def fp32_to_e4m3fn(x: np.ndarray) -> np.ndarray:
    """Encode to OCP e4m3fn codes: nearest, ties to even code, saturating at 448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.clip(np.searchsorted(_E4M3, a, side="left"), 0, 126)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _E4M3[lo]
    dhi = _E4M3[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code |= np.where(np.signbit(x), np.uint8(0x80), np.uint8(0))
    return code


def _row_blocks(n_rows: int):
    return range((n_rows + ROW_BLOCK - 1) // ROW_BLOCK)


def _draw_rows(cfg: Config, tensor: str, width: int, blocks, draw) -> dict:
    """Draw row blocks ``blocks`` of a [rows, width] tensor; returns {block: array}."""
    n_rows = cfg.rows

    def one(j):
        r0 = j * ROW_BLOCK
        r1 = min(n_rows, r0 + ROW_BLOCK)
        return j, draw(_rng(cfg.seed, tensor, j), (r1 - r0, width))

    with ThreadPoolExecutor(_threads()) as ex:
        return dict(ex.map(one, list(blocks)))


def _draw_q(rng, shape, cfg):
    if cfg.dist == "int":
        return fp32_to_bf16_bits(rng.integers(-4, 5, size=shape).astype(np.float32))
    return fp32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def _draw_w(rng, shape, cfg):
    if cfg.dist == "int":
        return rng.integers(-4, 5, size=shape).astype(np.float32)
    return (rng.standard_normal(shape, dtype=np.float32) / np.float32(np.sqrt(cfg.heads))).astype(np.float32)


def gen_q_rows(cfg: Config, rows) -> np.ndarray:
    """bf16 bits of q for the given flat rows (b*n_q + t): [len(rows), H, D]."""
    rows = np.asarray(rows, dtype=np.int64)
    blocks = sorted(set((rows // ROW_BLOCK).tolist()))
    got = _draw_rows(cfg, "q", cfg.heads * cfg.dim, blocks, lambda g, s: _draw_q(g, s, cfg))
    out = np.empty((len(rows), cfg.heads * cfg.dim), dtype=np.uint16)
    for i, r in enumerate(rows):
        out[i] = got[int(r) // ROW_BLOCK][int(r) % ROW_BLOCK]
    return out.reshape(len(rows), cfg.heads, cfg.dim)


def gen_w_rows(cfg: Config, rows) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.int64)
    blocks = sorted(set((rows // ROW_BLOCK).tolist()))
    got = _draw_rows(cfg, "w", cfg.heads, blocks, lambda g, s: _draw_w(g, s, cfg))
    out = np.empty((len(rows), cfg.heads), dtype=np.float32)
    for i, r in enumerate(rows):
        out[i] = got[int(r) // ROW_BLOCK][int(r) % ROW_BLOCK]
    return out


def gen_q(cfg: Config) -> np.ndarray:
    """bf16 bits [batch, n_q, H, D]."""
    got = _draw_rows(cfg, "q", cfg.heads * cfg.dim, _row_blocks(cfg.rows),
                     lambda g, s: _draw_q(g, s, cfg))
    flat = np.concatenate([got[j] for j in sorted(got)], axis=0) if got else \
        np.zeros((0, cfg.heads * cfg.dim), np.uint16)
    return flat.reshape(cfg.batch, cfg.n_q, cfg.heads, cfg.dim)


def gen_w(cfg: Config) -> np.ndarray:
    """fp32 [batch, n_q, H]."""
    got = _draw_rows(cfg, "w", cfg.heads, _row_blocks(cfg.rows), lambda g, s: _draw_w(g, s, cfg))
    flat = np.concatenate([got[j] for j in sorted(got)], axis=0) if got else \
        np.zeros((0, cfg.heads), np.float32)
    return flat.reshape(cfg.batch, cfg.n_q, cfg.heads)


def gen_keys(cfg: Config):
    """Keys as the path consumes them.

    Returns ``(k, k_scale)``: ``k`` is uint16 bf16 bits [batch, n_k, D] (or
    uint8 e4m3fn codes for fp8 keys) and ``k_scale`` is fp32 [batch, n_k] for
    fp8 keys, else None.
    """
    B, T, D = cfg.batch, cfg.n_k, cfg.dim
    if cfg.dist == "int":
        g = _rng(cfg.seed, "k", 0)
        return fp32_to_bf16_bits(g.integers(-4, 5, size=(B, T, D)).astype(np.float32)), None
    if cfg.dist == "normal":
        g = _rng(cfg.seed, "k", 0)
        return fp32_to_bf16_bits(g.standard_normal((B, T, D), dtype=np.float32)), None
    if cfg.dist == "drift":
        # Keys that drift slowly along the sequence so pooled blocks differ:
        # k[s] = z[s] + r[s], r a random walk with N(0, I/T) steps (end-to-end
        # drift has unit standard deviation).
        g = _rng(cfg.seed, "k", 0)
        z = g.standard_normal((B, T, D))
        gd = _rng(cfg.seed, "kdrift", 0)
        r = np.cumsum(gd.standard_normal((B, T, D)) / np.sqrt(T), axis=1)
        return fp32_to_bf16_bits((z + r).astype(np.float32)), None
    if cfg.dist == "fp8":
        # Per-token scale max|z|/448, codes nearest e4m3fn of z/scale.
        k8 = np.empty((B, T, D), np.uint8)
        sc = np.empty((B, T), np.float32)

        def one(b):
            z = _rng(cfg.seed, "k", b).standard_normal((T, D), dtype=np.float32)
            s = (np.abs(z).max(axis=1) / np.float32(448.0)).astype(np.float32)
            safe = np.where(s > 0, s, np.float32(1.0))
            k8[b] = fp32_to_e4m3fn(z / safe[:, None])
            sc[b] = s

        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(B)))
        return k8, sc
    if cfg.dist == "compressed":
        # Raw keys N(0,1) in bf16 at ratio*T positions; each compressed key is
        # the bf16-rounded mean of `ratio` consecutive raw keys (the key
        # compressor sits upstream of the indexer; the path consumes its output).
        m = cfg.causal_ratio
        g = _rng(cfg.seed, "kraw", 0)
        raw = bf16_bits_to_fp32(fp32_to_bf16_bits(
            g.standard_normal((B, T * m, D), dtype=np.float32))).astype(np.float64)
        mean = raw.reshape(B, T, m, D).sum(axis=2) / m
        return fp32_to_bf16_bits(mean.astype(np.float32)), None
    raise ValueError(cfg.dist)


def gen_raw_keys(seed: int, batch: int, n_raw: int, dim: int, seqs=None) -> np.ndarray:
    """Raw keys for the key-cache append: bf16 bits of N(0, 1), [len(seqs), n_raw,
    dim] for the listed sequences (all by default); sequence b comes from its
    own stream, so a sample of sequences can be drawn alone."""
    seqs = list(range(batch)) if seqs is None else [int(b) for b in seqs]
    out = np.empty((len(seqs), n_raw, dim), np.uint16)

    def one(i):
        g = _rng(seed, "append", seqs[i])
        out[i] = fp32_to_bf16_bits(g.standard_normal((n_raw, dim), dtype=np.float32))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(len(seqs))))
    return out


def make_inputs(cfg: Config) -> dict:
    """All inputs of a config as numpy arrays (see gen_q / gen_w / gen_keys)."""
    k, ks = gen_keys(cfg)
    return dict(q=gen_q(cfg), w=gen_w(cfg), k=k, k_scale=ks)


def sample_rows(cfg: Config, n: int, extra=()) -> np.ndarray:
    """A deterministic row sample: first and last rows, rows around topk-1 and
    around block / chunk boundaries, the rest uniform.  Flat row ids, sorted."""
    R = cfg.rows
    if n >= R:
        return np.arange(R, dtype=np.int64)
    pick = set(range(min(16, R)))
    pick.update(range(max(0, R - 16), R))
    for c in (cfg.topk - 2, cfg.topk - 1, cfg.topk):
        if 0 <= c < R:
            pick.add(c)
    for step in {cfg.block, cfg.q_chunk or 0, cfg.k_tile or 0}:
        if step:
            for b in range(step, R, max(step, R // 8)):
                for d in (-1, 0):
                    if 0 <= b + d < R:
                        pick.add(b + d)
    pick.update(int(x) for x in extra if 0 <= x < R)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=cfg.seed, spawn_key=(99,))))
    while len(pick) < n:
        pick.add(int(g.integers(0, R)))
    return np.array(sorted(pick), dtype=np.int64)

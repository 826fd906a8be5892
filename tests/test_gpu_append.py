"""Key-cache append against the oracle (StreamIndex abstract: compressed
keys; HISA abstract, stage (1): pooled block representatives).

Whatever way a raw key stream is split into appends, the key cache, its fp8
scales and the pooled blocks must equal, bit for bit, the oracle's
compression of the whole stream and the oracle's pooling of that cache; the
slots past the completed keys and blocks must stay untouched."""
import numpy as np
import pytest
import torch

import oracle
from helpers import dev, host
from tks_inputs import gen_raw_keys
from top_key_selection_amd import tks

pytestmark = pytest.mark.gpu

K_FILL, S_FILL, P_FILL = 0x55, -3.0, 0x5555


def say(*a):
    print(*a, flush=True)


class Cache:
    def __init__(self, batch, dim, m, fp8, block, n_k):
        self.S = tks.Shape(batch, 1, n_k, 1, dim, causal_ratio=m, key_dtype=1 if fp8 else 0)
        self.fp8, self.block, self.m = fp8, block, m
        if fp8:
            self.k = torch.full((batch, n_k, dim), K_FILL, dtype=torch.uint8, device="cuda")
            self.ks = torch.full((batch, n_k), S_FILL, dtype=torch.float32, device="cuda")
        else:
            self.k = torch.full((batch, n_k, dim), K_FILL * 0x101, dtype=torch.int16, device="cuda")
            self.ks = None
        nb = n_k // block if block else 0
        self.pooled = torch.full((batch, max(nb, 1), dim), P_FILL, dtype=torch.int16,
                                 device="cuda") if block else None
        self.tail = torch.zeros((batch, m, dim), dtype=torch.int16, device="cuda") if m > 1 else None
        self.raw_len = 0

    def append(self, raw_dev):
        tks.kv_append(self.S, raw_dev, self.raw_len, self.k, self.ks, self.tail, self.block,
                      self.pooled)
        self.raw_len += raw_dev.shape[1]

    def check(self, raw_host, seqs=None, what=""):
        """Compare with the oracle on the listed sequences (raw_host holds
        their raw streams, at least raw_len keys)."""
        torch.cuda.synchronize()
        seqs = list(range(self.S.batch)) if seqs is None else list(seqs)
        m, n_k, D = self.m, self.S.n_k, self.S.dim
        g = self.raw_len // m
        ok_k, ok_ks = oracle.compress_keys(raw_host[:, :self.raw_len], m, self.fp8, n_k)
        k = host(self.k)[seqs]
        if not self.fp8:
            k = k.view(np.uint16)
        bad = np.nonzero((k[:, :g] != ok_k[:, :g]).any(axis=2))
        assert len(bad[0]) == 0, "%s: key cache differs at (seq, key) %s" % (
            what, list(zip(bad[0][:5], bad[1][:5])))
        fill = K_FILL if self.fp8 else K_FILL * 0x101
        assert (k[:, g:] == fill).all(), "%s: cache slot past the completed keys written" % what
        if self.fp8:
            ks = host(self.ks)[seqs]
            np.testing.assert_array_equal(ks[:, :g].view(np.uint32), ok_ks[:, :g].view(np.uint32),
                                          err_msg=what + ": scales")
            assert (ks[:, g:] == S_FILL).all()
        if self.block:
            nbg = g // self.block
            shape = dict(batch=len(seqs), n_q=1, n_k=g, heads=1, dim=D, key_dtype=int(self.fp8))
            ok_p = oracle.pool(shape, ok_k[:, :g], ok_ks[:, :g] if self.fp8 else None, self.block)
            p = host(self.pooled)[seqs].view(np.uint16)
            bad = np.nonzero((p[:, :nbg] != ok_p).any(axis=2))
            assert len(bad[0]) == 0, "%s: pooled block differs at (seq, block) %s" % (
                what, list(zip(bad[0][:5], bad[1][:5])))
            assert (p[:, nbg:] == P_FILL).all(), "%s: pooled block past the completed ones written" % what


def split_sizes(rng, total):
    sizes = []
    while sum(sizes) < total:
        r = rng.random()
        n = int(rng.integers(1, 4)) if r < 0.5 else int(rng.integers(4, 40)) if r < 0.9 else \
            int(rng.integers(100, 400))
        sizes.append(min(n, total - sum(sizes)))
    return sizes


@pytest.mark.parametrize("batch,dim,m,fp8,block,n_raw", [
    (3, 128, 4, True, 32, 4 * 300 + 3),
    (2, 64, 4, False, 64, 4 * 300 + 1),
    (2, 32, 3, True, 32, 3 * 200 + 2),
    (2, 128, 1, True, 128, 700),
    (2, 128, 1, False, 32, 333),
    (2, 128, 4, False, 0, 4 * 150 + 2),
    (1, 64, 8, True, 256, 8 * 600 + 7),
])
def test_split_appends_equal_oracle_compression_and_pooling(batch, dim, m, fp8, block, n_raw):
    seed = 1000 + dim + 10 * m + block
    say("append split: batch %d dim %d m %d fp8 %d block %d n_raw %d" % (batch, dim, m, fp8, block, n_raw))
    raw = gen_raw_keys(seed, batch, n_raw, dim)
    rng = np.random.default_rng(seed)
    sizes = split_sizes(rng, n_raw)
    c = Cache(batch, dim, m, fp8, block, n_raw // m + 5)
    rd = dev(raw)
    for i, n in enumerate(sizes):
        c.append(rd[:, c.raw_len:c.raw_len + n].contiguous())
        if i % 7 == 3:
            c.check(raw, what="after %d appends" % (i + 1))
    c.check(raw, what="end")


@pytest.mark.parametrize("m,fp8", [(1, True), (1, False), (4, False), (4, True)])
def test_single_token_appends_cross_block_boundaries(m, fp8):
    batch, dim, block = 2, 128, 32
    n_raw = m * (2 * block + 5)
    say("append decode: m %d fp8 %d, %d single-key appends" % (m, fp8, n_raw))
    raw = gen_raw_keys(77 + m, batch, n_raw, dim)
    c = Cache(batch, dim, m, fp8, block, n_raw // m)
    rd = dev(raw)
    for p in range(n_raw):
        c.append(rd[:, p:p + 1].contiguous())
        if (p + 1) % (m * block) in (0, 1) or p < 3:
            c.check(raw, what="after raw key %d" % p)
    c.check(raw, what="end")


@pytest.mark.parametrize("fp8,m", [(True, 4), (False, 4), (True, 1), (False, 1)])
def test_special_values(fp8, m):
    """All-zero keys (fp8 scale 0), -0 (a mean is a sum from +0: it comes out
    +0), bf16 subnormals, the largest bf16 magnitudes and exact mean ties."""
    batch, dim, block = 2, 64, 32
    n_raw = m * block * 2
    say("append special values fp8 %d m %d" % (fp8, m))
    raw = gen_raw_keys(5, batch, n_raw, dim)
    raw[0, 0:4] = 0                         # all-zero compressed key
    raw[0, 4:8] = 0x8000                    # -0
    raw[1, 8:12] = 0x0001                   # smallest bf16 subnormal
    raw[1, 12:16, :] = 0x7F7F               # largest finite bf16
    raw[1, 16:20, ::2] = 0xFF7F             # and its negative
    raw[0, 20:24] = [[0x3F80], [0x3F80], [0x3F80], [0x3F82]]   # mean 1 + 2^-8: tie
    c = Cache(batch, dim, m, fp8, block, n_raw // m)
    rd = dev(raw)
    c.append(rd[:, :13].contiguous())
    c.append(rd[:, 13:].contiguous())
    c.check(raw, what="special values")


def test_full_size_cache_build_then_decode_appends():
    """The decode 64K fp8 cache (64 sequences x 65,536 keys, B = 128) built by
    one bulk append, then completed by 128 single-key appends that fill the
    last pooled block -- the launch shapes the benchmark times.  Three
    sampled sequences are compared whole."""
    batch, n_raw, dim, block = 64, 65536, 128, 128
    say("append full size: 64 x 65536 fp8, bulk + 128 single-key appends")
    raw = gen_raw_keys(4, batch, n_raw, dim)
    c = Cache(batch, dim, 1, True, block, n_raw)
    rd = dev(raw)
    del raw
    c.append(rd[:, :n_raw - 128].contiguous())
    for p in range(n_raw - 128, n_raw):
        c.append(rd[:, p:p + 1].contiguous())
    seqs = [0, 37, 63]
    c.check(gen_raw_keys(4, batch, n_raw, dim, seqs=seqs), seqs=seqs, what="64K cache")

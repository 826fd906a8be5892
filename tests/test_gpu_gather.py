"""Re-layout of the selected rows against the oracle (LongCat Sparse
Attention abstract, strategy (1): the KV rows the top-k selects copied into
a contiguous layout).  Byte-exact: out[b, t, j] = kv[b, idx[b, t, j]], zeros
for -1 or out-of-range slots."""
import numpy as np
import pytest
import torch

import oracle
from helpers import host
from top_key_selection_amd import tks

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("batch,n_kv,row_bytes,n_q,topk", [
    (3, 500, 1152, 5, 64),
    (2, 97, 16, 4, 33),
    (1, 2048, 256, 7, 2048),
    (2, 300, 4096, 2, 100),
])
def test_gather_matches_oracle(batch, n_kv, row_bytes, n_q, topk):
    say("gather: batch %d n_kv %d row %d B, %d x %d slots" % (batch, n_kv, row_bytes, n_q, topk))
    rng = np.random.default_rng(row_bytes + topk)
    kv = rng.integers(0, 256, (batch, n_kv, row_bytes)).astype(np.uint8)
    idx = rng.integers(0, n_kv, (batch, n_q, topk)).astype(np.int32)
    idx[:, :, ::5] = -1                                     # empty slots
    idx[0, 0, 1] = n_kv                                     # out of range
    idx[-1, -1, -1] = -7
    idx[:, :, 2] = idx[:, :, 3]                             # duplicates
    out = tks.gather_selected(torch.from_numpy(kv).cuda(), torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out), oracle.gather_selected(kv, idx))


def test_gather_decode_latent_rows_full_size():
    """The benchmark's shape: 64 sequences x 65,536 rows of a 576-dim bf16
    latent KV cache (1,152 bytes), 2,048 selected slots per query; three
    sequences compared whole."""
    batch, n_kv, D, topk = 64, 65536, 576, 2048
    say("gather full size: 64 x 65536 x 1152 B, 2048 slots per query")
    g = torch.Generator(device="cuda").manual_seed(5)
    kv = torch.randint(-32768, 32767, (batch, n_kv, D), dtype=torch.int16, device="cuda", generator=g)
    rng = np.random.default_rng(6)
    idx = np.stack([rng.permutation(n_kv)[:topk] for _ in range(batch)]).astype(np.int32)[:, None, :]
    idx[:, :, -3:] = -1
    out = tks.gather_selected(kv, torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    for b in (0, 29, 63):
        ref = oracle.gather_selected(host(kv[b:b + 1]), idx[b:b + 1])
        np.testing.assert_array_equal(host(out[b:b + 1]), ref)

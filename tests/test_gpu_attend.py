"""Sparse attention over the selected keys against the fp64 oracle (HISA
abstract: the sparse attention reads only the entries the indexer keeps).

Tolerance: the weights enter P.V rounded to bf16 (relative error <= 2^-9
each) and are normalised by the sum of those same rounded weights, so an
output moves by at most about 2^-8 * max|v| of the row's selected values;
fp32 scores add far less.  Checked: every element within 2^-8 * max|v| and
the mean error below 2^-12 * max|v| (the rounding errors of the weights
average out; a systematic error would break it)."""
import numpy as np
import pytest
import torch

import oracle
from helpers import dev, host
from tks_inputs import bf16_bits_to_fp32, fp32_to_bf16_bits
from top_key_selection_amd import tks

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def bf16(rng, shape):
    return fp32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def check(o, ref, vmax, what):
    err = np.abs(o - ref)
    tol = 2.0 ** -8 * vmax
    assert err.max() <= tol, "%s: max error %.3g > %.3g" % (what, err.max(), tol)
    assert err.mean() <= 2.0 ** -12 * vmax, "%s: mean error %.3g" % (what, err.mean())


@pytest.mark.parametrize("batch,n_q,heads,n_kv,topk", [
    (2, 3, 16, 300, 100),
    (1, 2, 64, 700, 256),
    (2, 2, 128, 1000, 300),
    (1, 3, 48, 5000, 2048),
    (3, 1, 32, 64, 1),
    (1, 2, 112, 900, 513),
])
def test_attention_matches_oracle(batch, n_q, heads, n_kv, topk):
    say("attend: batch %d n_q %d heads %d n_kv %d topk %d" % (batch, n_q, heads, n_kv, topk))
    rng = np.random.default_rng(heads + topk)
    q, k, v = bf16(rng, (batch, n_q, heads, 128)), bf16(rng, (batch, n_kv, 128)), bf16(rng, (batch, n_kv, 128))
    idx = np.stack([np.stack([rng.permutation(n_kv)[:topk] for _ in range(n_q)]) for _ in range(batch)]).astype(np.int32)
    if topk > 4:
        idx[:, :, ::7] = -1                        # padding inside the list
        idx[0, 0, 1] = n_kv + 3                    # out of range: ignored
    if n_q > 1:
        idx[-1, 1, :] = -1                         # a row with no key
    scale = 1.0 / np.sqrt(128.0)
    out = tks.sparse_attention(dev(q), dev(k), dev(v), dev(idx), scale)
    torch.cuda.synchronize()
    qf, kf, vf = (bf16_bits_to_fp32(x) for x in (q, k, v))
    ref = oracle.sparse_attention(qf, kf, vf, idx, scale)
    check(host(out), ref, np.abs(vf).max(), "attention")
    if n_q > 1:
        assert (host(out)[-1, 1] == 0).all()


def test_attention_large_scores_stay_finite():
    """Scores far from 0 (scale 1, q and k of norm ~ 60) exercise the running
    max: exp2 of the raw scores would overflow fp32."""
    rng = np.random.default_rng(7)
    batch, n_q, heads, n_kv, topk = 1, 2, 16, 400, 300
    q = fp32_to_bf16_bits((rng.standard_normal((batch, n_q, heads, 128)) * 5).astype(np.float32))
    k = fp32_to_bf16_bits((rng.standard_normal((batch, n_kv, 128)) * 5).astype(np.float32))
    v = bf16(rng, (batch, n_kv, 128))
    idx = np.stack([np.stack([rng.permutation(n_kv)[:topk] for _ in range(n_q)])]).astype(np.int32)
    out = tks.sparse_attention(dev(q), dev(k), dev(v), dev(idx), 1.0)
    torch.cuda.synchronize()
    qf, kf, vf = (bf16_bits_to_fp32(x) for x in (q, k, v))
    o = host(out)
    assert np.isfinite(o).all()
    check(o, oracle.sparse_attention(qf, kf, vf, idx, 1.0), np.abs(vf).max(), "large scores")


def test_attention_decode_full_size():
    """The benchmark's shape: 64 sequences, one query of 128 heads each, 2048
    selected keys from 65,536; three rows compared with the oracle."""
    batch, heads, n_kv, topk = 64, 128, 65536, 2048
    say("attend full size: 64 x 128 heads, 2048 of 65536 keys")
    g = torch.Generator(device="cuda").manual_seed(11)
    q = torch.randn((batch, 1, heads, 128), device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn((batch, n_kv, 128), device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn((batch, n_kv, 128), device="cuda", generator=g).to(torch.bfloat16)
    rng = np.random.default_rng(12)
    idx = np.stack([rng.permutation(n_kv)[:topk] for _ in range(batch)]).astype(np.int32)[:, None, :]
    scale = 1.0 / np.sqrt(128.0)
    out = tks.sparse_attention(q, k, v, torch.from_numpy(idx).cuda(), scale)
    torch.cuda.synchronize()
    for b in (0, 31, 63):
        qf = host(q[b:b + 1].float())
        kf = host(k[b:b + 1].float())
        vf = host(v[b:b + 1].float())
        ref = oracle.sparse_attention(qf, kf, vf, idx[b:b + 1], scale)
        check(host(out[b:b + 1]), ref, np.abs(vf[0, idx[b, 0]]).max(), "row %d" % b)


def test_attention_into_a_4_byte_aligned_output():
    """The output need only be 4-byte aligned: a buffer one float past a
    16-byte boundary gives the same values as an aligned one."""
    say("attend into an output offset by one float")
    g = torch.Generator(device="cuda").manual_seed(9)
    B, T, H, n, K = 2, 2, 64, 500, 300
    q = torch.randn((B, T, H, 128), device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn((B, n, 128), device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn((B, n, 128), device="cuda", generator=g).to(torch.bfloat16)
    idx = torch.randint(-1, n, (B, T, K), device="cuda", generator=g, dtype=torch.int32)
    ref = tks.sparse_attention(q, k, v, idx, 0.09)
    buf = torch.full((B * T * H * 128 + 1,), 7.0, device="cuda")
    out = buf[1:].view(B, T, H, 128)
    assert out.data_ptr() % 16 == 4
    tks.sparse_attention(q, k, v, idx, 0.09, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and buf[0].item() == 7.0

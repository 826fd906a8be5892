"""Pins of the CPU oracle against facts fixed independently of it.

Each test pins one part of the oracle to something other than the oracle:
a library routine on a special case (torch's bf16 / e4m3fn casts, numpy
matmul), a closed form, an invariant of the method, or a brute-force full
sort on tiny inputs.  The oracle follows the HISA abstract (indexer scoring,
two-stage block filter + token refinement, per-query top-k interface) and
the StreamIndex abstract (compressed keys, chunked top-k)."""
import numpy as np
import pytest
import torch

import oracle
from tks_inputs import (FORCE_FIRST, FORCE_LOCAL, bf16_bits_to_fp32, fp32_to_bf16_bits,
                        fp32_to_e4m3fn)


def shp(n_q, n_k, heads, dim, batch=1, q_pos0=0, ratio=1, fp8=0):
    return dict(batch=batch, n_q=n_q, n_k=n_k, heads=heads, dim=dim, q_pos0=q_pos0,
                causal_ratio=ratio, key_dtype=fp8)


def rand_int(rng, shape, lo=-4, hi=4):
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


def brute_topk(scores, valid, k):
    """Full lexsort (score desc, index asc) of one row; -1 padded."""
    idx = np.nonzero(valid)[0]
    order = np.lexsort((idx, -scores[idx]))
    top = idx[order][:k]
    out = -np.ones(k, np.int64)
    out[:len(top)] = top
    return out


# ------------------------------------------------------------------ decoders

def test_bf16_decode_matches_torch_for_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.isnan(got[nan]).all()
    np.testing.assert_array_equal(got[~nan], ref[~nan])


def test_e4m3fn_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3fn_to_double(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.isnan(got[nan]).all()
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_bf16_rounding_matches_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(4000).astype(np.float32),
        (rng.standard_normal(1000) * 1e-39).astype(np.float32),      # subnormals
        (rng.standard_normal(1000) * 1e30).astype(np.float32),
        # exact halfway cases: bf16 value + half an ulp (ties to even)
        (bf16_bits_to_fp32(rng.integers(0x3F00, 0x4100, 500).astype(np.uint16)).view(np.uint32)
         + np.uint32(0x8000)).view(np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.double_to_bf16(float(v)) for v in x], np.uint16)
    np.testing.assert_array_equal(got, ref)


def test_generator_bf16_and_e4m3_encoders_match_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(20000).astype(np.float32) * 50
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(fp32_to_bf16_bits(x), ref)
    y = np.clip(x, -448, 448)
    ref8 = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(fp32_to_e4m3fn(y), ref8)


# ------------------------------------------------------------------- scoring

def test_single_head_unit_weight_is_relu_of_matmul():
    """H=1, w=1: I = max(0, q k^T) -- a plain matrix product on integers."""
    rng = np.random.default_rng(2)
    T, D = 48, 32
    q = rand_int(rng, (1, T, 1, D))
    k = rand_int(rng, (1, T, D))
    w = np.ones((1, T, 1), np.float32)
    got = oracle.index_scores(shp(T, T, 1, D), fp32_to_bf16_bits(q), w, fp32_to_bf16_bits(k),
                              None, 0, T, 0, T)[0]
    ref = np.maximum(q[0, :, 0, :].astype(np.float64) @ k[0].T.astype(np.float64), 0.0)
    causal = np.tril(np.ones((T, T), bool))
    np.testing.assert_array_equal(got[causal], ref[causal])
    assert np.all(np.isneginf(got[~causal]))


def _torch_decode_keys(k, fp8, k_scale):
    """Keys as float64 through torch's own casts (independent of the oracle's
    decoders); fp8 keys are scale * e4m3fn."""
    if fp8:
        v = torch.from_numpy(k).view(torch.float8_e4m3fn).double().numpy()
        return v * k_scale.astype(np.float64)[..., None]
    return torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).double().numpy()


def _definition_scores(q_rows, w_rows, kd, rows, n_q, q_pos0, ratio):
    """I[t,s] = sum_h w[t,h] * max(0, q[t,h] . k[s]) from a numpy matmul,
    -inf where s > floor((q_pos0 + t) / ratio) (Python floor division)."""
    qd = torch.from_numpy(q_rows.view(np.int16)).view(torch.bfloat16).double().numpy()
    n_k = kd.shape[1]
    out = np.empty((len(rows), n_k))
    for i, r in enumerate(rows):
        b, t = divmod(int(r), n_q)
        x = qd[i] @ kd[b].T                       # [H, n_k]
        out[i] = w_rows[i].astype(np.float64) @ np.maximum(x, 0.0)
        vis = (q_pos0 + t) // ratio
        out[i, np.arange(n_k) > vis] = -np.inf
    return out


@pytest.mark.parametrize("fp8", [0, 1])
@pytest.mark.parametrize("q_pos0,ratio", [(0, 1), (-3, 4), (5, 4), (-9, 3)])
def test_row_scores_equal_the_definition_on_integer_inputs(fp8, q_pos0, ratio):
    """row_scores (the score every float comparator uses) against the
    definition written with torch's decoders and a numpy matmul: batch 2,
    compressed causality, negative q_pos0, bf16 and fp8 keys.  Integer
    inputs and power-of-two scales keep every score exact in float64, so the
    two must agree bit for bit, -inf included."""
    rng = np.random.default_rng(40 + fp8 + 2 * ratio)
    B, T, NK, H, D = 2, 37, 29, 3, 16
    q = rand_int(rng, (B, T, H, D))
    w = rand_int(rng, (B, T, H))
    kv = rand_int(rng, (B, NK, D))
    if fp8:
        k = fp32_to_e4m3fn(kv)
        ks = (2.0 ** rng.integers(-3, 4, (B, NK))).astype(np.float32)
    else:
        k, ks = fp32_to_bf16_bits(kv), None
    S = shp(T, NK, H, D, batch=B, q_pos0=q_pos0, ratio=ratio, fp8=fp8)
    rows = np.array([0, 1, 5, T - 1, T, T + 7, 2 * T - 1])
    qb = fp32_to_bf16_bits(q).reshape(B * T, H, D)[rows]
    wr = w.reshape(B * T, H)[rows]
    got = oracle.row_scores(S, qb, wr, k, ks, rows)
    ref = _definition_scores(qb, wr, _torch_decode_keys(k, fp8, ks), rows, T, q_pos0, ratio)
    np.testing.assert_array_equal(got, ref)
    # the same scores as the rectangle form, row for row
    rect = oracle.index_scores(S, fp32_to_bf16_bits(q), w, k, ks, 0, T, 0, NK)
    np.testing.assert_array_equal(got, rect.reshape(B * T, NK)[rows])


@pytest.mark.parametrize("fp8", [0, 1])
def test_row_scores_on_float_inputs_match_the_definition_and_the_topk_values(fp8):
    """Float inputs: row_scores within float64 rounding of the torch/numpy
    definition, -inf exactly outside the causal prefix, and equal to the
    values orc_topk_flat reports at the indices it selects."""
    rng = np.random.default_rng(50 + fp8)
    B, T, NK, H, D, K = 2, 64, 300, 8, 32, 40
    q = fp32_to_bf16_bits(rng.standard_normal((B, T, H, D)).astype(np.float32))
    w = (rng.standard_normal((B, T, H)) / np.sqrt(H)).astype(np.float32)
    z = rng.standard_normal((B, NK, D)).astype(np.float32)
    if fp8:
        ks = (np.abs(z).max(axis=2) / 448.0).astype(np.float32)
        k = fp32_to_e4m3fn(z / ks[..., None])
    else:
        k, ks = fp32_to_bf16_bits(z), None
    q_pos0 = NK - T - 10
    S = shp(T, NK, H, D, batch=B, q_pos0=q_pos0, fp8=fp8)
    rows = np.arange(B * T)
    qr, wr = q.reshape(B * T, H, D), w.reshape(B * T, H)
    got = oracle.row_scores(S, qr, wr, k, ks, rows)
    ref = _definition_scores(qr, wr, _torch_decode_keys(k, fp8, ks), rows, T, q_pos0, 1)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got))
    scale = np.abs(ref[fin]).max()
    assert np.max(np.abs(got[fin] - ref[fin])) <= 1e-12 * scale
    idx, val = oracle.topk_flat(S, qr, wr, k, ks, K, rows)
    ok = idx >= 0
    np.testing.assert_array_equal(val[ok], got[np.nonzero(ok)[0], idx[ok]])


def test_basis_keys_pick_one_coordinate_per_head():
    """k[s] = e_{d(s)}: I[t,s] = sum_h w[t,h] * max(0, q[t,h,d(s)])."""
    rng = np.random.default_rng(3)
    T, H, D = 40, 3, 16
    q = rand_int(rng, (1, T, H, D))
    w = rand_int(rng, (1, T, H))
    d_of_s = rng.integers(0, D, T)
    k = np.zeros((1, T, D), np.float32)
    k[0, np.arange(T), d_of_s] = 1.0
    got = oracle.index_scores(shp(T, T, H, D, q_pos0=T), fp32_to_bf16_bits(q), w,
                              fp32_to_bf16_bits(k), None, 0, T, 0, T)[0]
    for t in range(T):
        for s in range(T):
            want = sum(float(w[0, t, h]) * max(0.0, float(q[0, t, h, d_of_s[s]])) for h in range(H))
            assert got[t, s] == want


def test_one_hot_head_weight_selects_that_head():
    rng = np.random.default_rng(4)
    T, H, D = 32, 4, 8
    q = rand_int(rng, (1, T, H, D))
    k = rand_int(rng, (1, T, D))
    for h in range(H):
        w = np.zeros((1, T, H), np.float32)
        w[..., h] = 1.0
        got = oracle.index_scores(shp(T, T, H, D, q_pos0=T), fp32_to_bf16_bits(q), w,
                                  fp32_to_bf16_bits(k), None, 0, T, 0, T)[0]
        ref = np.maximum(q[0, :, h, :].astype(np.float64) @ k[0].T.astype(np.float64), 0)
        np.testing.assert_array_equal(got, ref)


def test_head_permutation_invariance_and_weight_linearity():
    rng = np.random.default_rng(5)
    T, H, D = 24, 5, 8
    q = rand_int(rng, (1, T, H, D))
    k = rand_int(rng, (1, T, D))
    w = rand_int(rng, (1, T, H))
    S = shp(T, T, H, D)
    base = oracle.index_scores(S, fp32_to_bf16_bits(q), w, fp32_to_bf16_bits(k), None, 0, T, 0, T)
    perm = rng.permutation(H)
    p = oracle.index_scores(S, fp32_to_bf16_bits(q[:, :, perm]), w[:, :, perm],
                            fp32_to_bf16_bits(k), None, 0, T, 0, T)
    np.testing.assert_array_equal(base, p)
    two = oracle.index_scores(S, fp32_to_bf16_bits(q), 2 * w, fp32_to_bf16_bits(k), None,
                              0, T, 0, T)
    fin = np.isfinite(base)
    np.testing.assert_array_equal(two[fin], 2 * base[fin])


def test_all_dots_negative_gives_zero_score_even_with_negative_weights():
    T, H, D = 16, 2, 4
    q = np.ones((1, T, H, D), np.float32)
    k = -np.ones((1, T, D), np.float32)
    w = -np.ones((1, T, H), np.float32)
    got = oracle.index_scores(shp(T, T, H, D), fp32_to_bf16_bits(q), w, fp32_to_bf16_bits(k),
                              None, 0, T, 0, T)[0]
    causal = np.tril(np.ones((T, T), bool))
    assert np.all(got[causal] == 0.0) and not np.any(np.signbit(got[causal]))


def test_fp8_keys_equal_bf16_keys_with_same_values():
    """scale * e4m3 values that bf16 holds exactly score like bf16 keys."""
    rng = np.random.default_rng(6)
    T, H, D = 32, 3, 16
    q = rand_int(rng, (1, T, H, D))
    w = rand_int(rng, (1, T, H))
    vals = rand_int(rng, (1, T, D), -8, 8)          # integers are exact in e4m3
    codes = fp32_to_e4m3fn(vals)
    scale = np.full((1, T), 0.25, np.float32)       # power of two keeps it exact
    got = oracle.index_scores(shp(T, T, H, D, fp8=1), fp32_to_bf16_bits(q), w, codes, scale,
                              0, T, 0, T)
    ref = oracle.index_scores(shp(T, T, H, D), fp32_to_bf16_bits(q), w,
                              fp32_to_bf16_bits(vals * 0.25), None, 0, T, 0, T)
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("q_pos0,ratio", [(0, 1), (5, 1), (0, 4), (-3, 4), (-100, 1)])
def test_visibility_counts(q_pos0, ratio):
    S = shp(64, 20, 1, 4, q_pos0=q_pos0, ratio=ratio)
    for t in range(64):
        pos = q_pos0 + t
        vis = pos // ratio                      # python floor division
        want = 0 if vis < 0 else min(vis + 1, 20)
        assert oracle.n_visible(S, t) == want


def test_future_keys_never_selected():
    """Keys after the query are made huge; the causal mask must still skip them."""
    rng = np.random.default_rng(7)
    T, H, D, K = 64, 2, 8, 8
    q = np.abs(rand_int(rng, (1, T, H, D))) + 1
    w = np.ones((1, T, H), np.float32)
    k = rand_int(rng, (1, T, D))
    idx, _ = oracle.topk_flat(shp(T, T, H, D), fp32_to_bf16_bits(q[0]), w[0],
                              fp32_to_bf16_bits(k), None, K, np.arange(T))
    k_big = k.copy()
    for t in range(T):
        kk = k_big.copy()
        kk[0, t + 1:] = 100.0
        i2, _ = oracle.topk_flat(shp(T, T, H, D), fp32_to_bf16_bits(q[0, t:t + 1]),
                                 w[0, t:t + 1], fp32_to_bf16_bits(kk), None, K, [t])
        np.testing.assert_array_equal(i2[0], idx[t])
        assert np.all(i2[0][i2[0] >= 0] <= t)


# --------------------------------------------------------------------- top-k

@pytest.mark.parametrize("seed,k", [(10, 5), (11, 16), (12, 64), (13, 100)])
def test_topk_equals_brute_force_full_sort(seed, k):
    rng = np.random.default_rng(seed)
    T, H, D = 96, 3, 8
    q = rand_int(rng, (1, T, H, D), -2, 2)          # small range: many exact ties
    w = rand_int(rng, (1, T, H), -2, 2)
    kk = rand_int(rng, (1, T, D), -2, 2)
    S = shp(T, T, H, D)
    sc = oracle.index_scores(S, fp32_to_bf16_bits(q), w, fp32_to_bf16_bits(kk), None, 0, T, 0, T)[0]
    idx, val = oracle.topk_flat(S, fp32_to_bf16_bits(q[0]), w[0], fp32_to_bf16_bits(kk), None, k,
                                np.arange(T))
    for t in range(T):
        want = brute_topk(sc[t], np.isfinite(sc[t]), k)
        np.testing.assert_array_equal(idx[t], want)
        ok = want >= 0
        np.testing.assert_array_equal(val[t][ok], sc[t][want[ok]])
        assert np.all(np.isnan(val[t][~ok]))


def test_all_equal_scores_give_lowest_indices():
    T, H, D, K = 200, 2, 4, 64
    q = np.zeros((T, H, D), np.float32)
    w = np.ones((T, H), np.float32)
    k = np.ones((1, T, D), np.float32)
    idx, val = oracle.topk_flat(shp(T, T, H, D), fp32_to_bf16_bits(q), w, fp32_to_bf16_bits(k),
                                None, K, np.arange(T))
    for t in range(T):
        n = min(K, t + 1)
        np.testing.assert_array_equal(idx[t, :n], np.arange(n))
        assert np.all(idx[t, n:] == -1) and np.all(val[t, :n] == 0.0)


def test_planted_maxima_come_first():
    rng = np.random.default_rng(8)
    T, H, D, K = 128, 2, 8, 10
    q = np.ones((1, 1, H, D), np.float32)
    k = rand_int(rng, (1, T, D), -1, 1)
    planted = [3, 77, 100, 127]
    for j, s in enumerate(planted):
        k[0, s] = 4.0 - j * 0.5                      # decreasing planted scores
    w = np.ones((1, 1, H), np.float32)
    idx, _ = oracle.topk_flat(shp(1, T, H, D, q_pos0=T - 1), fp32_to_bf16_bits(q[0]), w[0],
                              fp32_to_bf16_bits(k), None, K, [0])
    np.testing.assert_array_equal(idx[0, :4], planted)


# ----------------------------------------------------------------- pooling

def test_pool_of_integers_is_exact_mean():
    rng = np.random.default_rng(9)
    T, D, B = 256, 16, 64
    k = rand_int(rng, (2, T, D))
    got = oracle.pool(shp(1, T, 1, D, batch=2), fp32_to_bf16_bits(k), None, B)
    ref = k.reshape(2, T // B, B, D).astype(np.float64).mean(axis=2)
    np.testing.assert_array_equal(bf16_bits_to_fp32(got).astype(np.float64), ref)


def _nearest_bf16_ok(bits, exact):
    """bits is a nearest bf16 of `exact` (no other bf16 value is strictly closer)."""
    v = bf16_bits_to_fp32(bits).astype(np.float64)
    up = bf16_bits_to_fp32((bits.astype(np.int32) + 1).astype(np.uint16)).astype(np.float64)
    dn = bf16_bits_to_fp32((bits.astype(np.int32) - 1).astype(np.uint16)).astype(np.float64)
    err = np.abs(v - exact)
    # the neighbour pattern of +0 (0xFFFF) is NaN: no closer value there
    d_up = np.where(np.isnan(up), np.inf, np.abs(up - exact))
    d_dn = np.where(np.isnan(dn), np.inf, np.abs(dn - exact))
    return np.all(err <= d_up) and np.all(err <= d_dn)


def test_pool_of_floats_is_nearest_bf16_of_mean_and_ignores_tail():
    rng = np.random.default_rng(10)
    T, D, B = 1000, 8, 128                           # 7 complete blocks + a 104-key tail
    k = fp32_to_bf16_bits(rng.standard_normal((1, T, D)).astype(np.float32))
    got = oracle.pool(shp(1, T, 1, D), k, None, B)
    assert got.shape == (1, T // B, D)
    kv = bf16_bits_to_fp32(k).astype(np.float64)
    exact = kv[:, :7 * B].reshape(1, 7, B, D).mean(axis=2)
    assert _nearest_bf16_ok(got, exact)
    np.testing.assert_allclose(bf16_bits_to_fp32(got), exact, rtol=2 ** -8)


def test_pool_fp8_uses_dequantised_keys():
    rng = np.random.default_rng(11)
    T, D, B = 256, 8, 64
    codes = rng.integers(0, 256, (1, T, D)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10            # no NaN codes
    scale = (rng.random((1, T)) * 0.01 + 1e-3).astype(np.float32)
    got = oracle.pool(shp(1, T, 1, D, fp8=1), codes, scale, B)
    deq = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy() * \
        scale.astype(np.float64)[..., None]
    exact = deq.reshape(1, T // B, B, D).mean(axis=2)
    assert _nearest_bf16_ok(got, exact)


# --------------------------------------------------------- key compression
# (StreamIndex abstract: the indexer reads keys compressed by a ratio m; the
# compressed key is read as the bf16 mean of m consecutive raw keys, stored
# in an fp8 cache as e4m3fn codes with a per-key scale max|kc| / 448.)

def test_e4m3fn_encoder_matches_torch_on_ties_and_random_values():
    mags = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)   # exact ties
    rng = np.random.default_rng(30)
    x = np.concatenate([
        mags.astype(np.float32), mids,
        np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1000)),
        rng.uniform(-448, 448, 3000).astype(np.float32),
        (rng.standard_normal(3000) * 0.01).astype(np.float32),
    ])
    x = np.concatenate([x, -x])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.float_to_e4m3fn(v) for v in x], np.uint8)
    np.testing.assert_array_equal(got, ref)
    # saturation at the largest finite magnitude, 448
    assert oracle.float_to_e4m3fn(1e6) == 0x7E and oracle.float_to_e4m3fn(-1e6) == 0xFE


def test_compress_ratio_one_is_identity_for_bf16_keys():
    rng = np.random.default_rng(31)
    raw = fp32_to_bf16_bits(rng.standard_normal((2, 50, 16)).astype(np.float32))
    k, ks = oracle.compress_keys(raw, 1, False)
    assert ks is None
    np.testing.assert_array_equal(k, raw)


def test_compress_integer_groups_is_exact_mean_and_drops_the_partial_group():
    rng = np.random.default_rng(32)
    raw = rand_int(rng, (2, 4 * 37 + 3, 8), -16, 16)
    k, _ = oracle.compress_keys(fp32_to_bf16_bits(raw), 4, False)
    assert k.shape == (2, 37, 8)
    # group sums lie in [-64, 64], so every mean is a multiple of 1/4 with at
    # most 7 significant bits: exact in bf16
    ref = raw[:, :4 * 37].reshape(2, 37, 4, 8).astype(np.float64).mean(axis=2)
    np.testing.assert_array_equal(bf16_bits_to_fp32(k).astype(np.float64), ref)


@pytest.mark.parametrize("group,bits", [
    ([1, 1, 1, 1 + 2 ** -6], 0x3F80),               # mean 1 + 2^-8: tie, even is 1
    ([1, 1, 1 + 2 ** -6, 1 + 2 ** -5], 0x3F82),     # mean 1 + 3 * 2^-8: tie, even is 1 + 2^-6
    ([-1, -1, -1, -1 - 2 ** -6], 0xBF80),
    ([1, 1, 2], 0x3FAB),                            # mean 4/3: nearest is 1 + 43/128
])
def test_compress_rounds_the_mean_to_nearest_even_bf16(group, bits):
    raw = fp32_to_bf16_bits(np.array(group, np.float32).reshape(1, len(group), 1))
    k, _ = oracle.compress_keys(raw, len(group), False)
    assert int(k[0, 0, 0]) == bits


def test_compress_random_means_are_nearest_bf16():
    rng = np.random.default_rng(33)
    raw = fp32_to_bf16_bits(rng.standard_normal((3, 4 * 200, 16)).astype(np.float32))
    k, _ = oracle.compress_keys(raw, 4, False)
    exact = bf16_bits_to_fp32(raw).astype(np.float64).reshape(3, 200, 4, 16).mean(axis=2)
    assert _nearest_bf16_ok(k, exact)


def test_fp8_cache_scale_is_max_over_448():
    # keys whose largest magnitude is 7 = 448 * 2^-6: the scale is exactly
    # 2^-6 and every integer coordinate times 64 is an exact e4m3fn value
    rng = np.random.default_rng(35)
    kc = rand_int(rng, (2, 40, 32), -7, 7)
    kc[:, :, 3] = 7.0 * np.where(rng.random((2, 40)) < 0.5, 1, -1)
    kc[1, 5] = 0.0                                  # all-zero key
    raw = fp32_to_bf16_bits(np.repeat(kc, 4, axis=1))   # constant groups: exact means
    k8, ks = oracle.compress_keys(raw, 4, True)
    assert ks[1, 5] == 0.0 and (k8[1, 5] == 0).all()
    mask = np.ones((2, 40), bool)
    mask[1, 5] = False
    assert (ks[mask] == np.float32(2.0 ** -6)).all()
    deq = torch.from_numpy(k8).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(deq[mask] * 2.0 ** -6, kc[mask])


def test_fp8_cache_codes_are_torch_e4m3fn_of_key_over_scale():
    rng = np.random.default_rng(34)
    raw = fp32_to_bf16_bits((rng.standard_normal((2, 4 * 64, 32)) * 3).astype(np.float32))
    kb, _ = oracle.compress_keys(raw, 4, False)
    k8, ks = oracle.compress_keys(raw, 4, True)
    kc = bf16_bits_to_fp32(kb)
    deq = torch.from_numpy(k8).view(torch.float8_e4m3fn).double().numpy()
    # the largest coordinate of every key maps to +-448
    assert (np.abs(deq).max(axis=2) == 448.0).all()
    x = (kc / ks[..., None]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(k8, ref)
    # dequantised keys within half an e4m3fn step (relative 2^-4, absolute
    # 2^-10 * scale on the subnormal grid)
    err = np.abs(deq * ks[..., None] - kc)
    bound = np.maximum(np.abs(kc) * 2.0 ** -4, ks[..., None] * 2.0 ** -10)
    assert (err <= bound * (1 + 1e-6)).all()


# ----------------------------------------------------------- block selection

def _int_case(seed, T=256, H=2, D=8):
    rng = np.random.default_rng(seed)
    q = rand_int(rng, (1, T, H, D))
    w = rand_int(rng, (1, T, H))
    k = rand_int(rng, (1, T, D))
    return fp32_to_bf16_bits(q), w, fp32_to_bf16_bits(k)


def test_hisa_with_every_block_kept_equals_flat():
    """HISA abstract, stage (2): the original indexer on the retained blocks;
    keeping every block must therefore reproduce the flat top-k exactly."""
    T, H, D, B, K = 256, 2, 8, 16, 12
    q, w, k = _int_case(12, T, H, D)
    S = shp(T, T, H, D)
    rows = np.arange(T)
    fi, fv = oracle.topk_flat(S, q[0], w[0], k, None, K, rows)
    for flags in (FORCE_LOCAL, FORCE_FIRST | FORCE_LOCAL):
        blk, hi, hv = oracle.hisa(S, q[0], w[0], k, None, B, T // B, flags, K, rows)
        np.testing.assert_array_equal(hi, fi)
        np.testing.assert_array_equal(hv, fv)


def test_block_size_one_selects_the_flat_top_m_tokens():
    """With B = 1 the pooled keys are the keys; the scored blocks of query t
    are its best m keys among 0..t-1 (flat top-m with one key less visible)."""
    T, H, D, M = 96, 2, 8, 7
    q, w, k = _int_case(13, T, H, D)
    rows = np.arange(T)
    pooled = oracle.pool(shp(T, T, H, D), k, None, 1)
    np.testing.assert_array_equal(pooled, k)
    blk, bv = oracle.block_select(shp(T, T, H, D), q[0], w[0], pooled, 1, M, FORCE_LOCAL, rows)
    fi, fv = oracle.topk_flat(shp(T, T, H, D, q_pos0=-1), q[0], w[0], k, None, M, rows)
    for t in range(T):
        got = blk[t][blk[t] >= 0]
        assert t in got                                   # local block forced
        scored = sorted(set(got.tolist()) - {t})
        want = sorted(x for x in fi[t].tolist() if x >= 0)
        assert scored == want
        np.testing.assert_array_equal(got, np.sort(got))   # ascending
        assert np.all(bv[t][blk[t] == t] == np.inf)


def test_block_select_forced_blocks_and_padding():
    T, H, D, B, M = 512, 2, 8, 32, 3
    q, w, k = _int_case(14, T, H, D)
    rows = np.arange(T)
    pooled = oracle.pool(shp(T, T, H, D), k, None, B)
    blk, bv = oracle.block_select(shp(T, T, H, D), q[0], w[0], pooled, B, M,
                                  FORCE_FIRST | FORCE_LOCAL, rows)
    assert blk.shape == (T, M + 2)
    for t in range(T):
        L = t // B
        got = blk[t][blk[t] >= 0]
        assert L in got and 0 in got
        n_eligible = max(0, L - 1)                         # blocks 1..L-1
        assert len(got) == min(M, n_eligible) + (2 if L > 0 else 1)
        assert np.all(got <= L)
        assert np.all(blk[t][len(got):] == -1)


def test_planted_block_is_selected():
    rng = np.random.default_rng(15)
    T, H, D, B = 1024, 2, 8, 64
    q = np.ones((1, H, D), np.float32)
    w = np.ones((1, H), np.float32)
    k = rand_int(rng, (1, T, D), -1, 1)
    k[0, 5 * B:6 * B] = 3.0
    S = shp(1, T, H, D, q_pos0=T - 1)
    pooled = oracle.pool(S, fp32_to_bf16_bits(k), None, B)
    blk, bv = oracle.block_select(S, fp32_to_bf16_bits(q), w, pooled, B, 1, FORCE_LOCAL, [0])
    assert blk[0].tolist() == [5, 15]


def test_refine_equals_brute_force_on_kept_blocks():
    T, H, D, B, K = 192, 2, 8, 16, 20
    q, w, k = _int_case(16, T, H, D)
    S = shp(T, T, H, D)
    rows = np.arange(T)
    rng = np.random.default_rng(17)
    blk = -np.ones((T, 4), np.int32)
    for t in range(T):
        L = t // B
        chosen = np.sort(rng.choice(L + 1, size=min(4, L + 1), replace=False))
        blk[t, :len(chosen)] = chosen
    idx, val = oracle.refine(S, q[0], w[0], k, None, B, blk, K, rows)
    sc = oracle.index_scores(S, q, w[None, 0] if w.ndim == 2 else w, k, None, 0, T, 0, T)[0]
    for t in range(T):
        keep = np.zeros(T, bool)
        for b in blk[t]:
            if b >= 0:
                keep[b * B:(b + 1) * B] = True
        want = brute_topk(sc[t], keep & np.isfinite(sc[t]), K)
        np.testing.assert_array_equal(idx[t], want)


def test_materialized_score_tensor_size_is_256_gib():
    """StreamIndex abstract: [B, S, H_I, T] fp32 with H_I = 64, m = 4 is 256 GB
    at S = 65,536 (2^16 * 64 * 2^14 * 4 bytes = 2^38 bytes)."""
    S, H, m = 65536, 64, 4
    assert S * H * (S // m) * 4 == 2 ** 38


# ---------------------------------------------------------------- re-layout
# (LongCat Sparse Attention abstract, strategy (1): the selected KV rows
# copied into a contiguous layout.)

def test_gather_equals_numpy_take_and_zero_fills_empty_slots():
    rng = np.random.default_rng(40)
    kv = rng.integers(0, 256, (2, 50, 48)).astype(np.uint8)
    idx = rng.integers(0, 50, (2, 3, 7)).astype(np.int32)
    got = oracle.gather_selected(kv, idx)
    ref = np.take_along_axis(kv[:, None, :, :], idx[..., None].astype(np.int64), axis=2)
    np.testing.assert_array_equal(got, ref)
    idx[0, 1, 2] = -1
    idx[1, 2, 0] = 50                               # outside [0, n_kv)
    got = oracle.gather_selected(kv, idx)
    assert (got[0, 1, 2] == 0).all() and (got[1, 2, 0] == 0).all()
    ar = np.broadcast_to(np.arange(7, dtype=np.int32), (2, 1, 7))
    np.testing.assert_array_equal(oracle.gather_selected(kv, ar)[:, 0], kv[:, :7])


# ------------------------------------------------------ sparse attention
# (HISA abstract: the sparse attention that consumes the selected indices.)

def test_sparse_attention_equals_torch_sdpa_when_every_key_is_selected():
    rng = np.random.default_rng(50)
    B, T, H, n, dk, dv = 2, 3, 4, 40, 16, 8
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, n, dk))
    v = rng.standard_normal((B, n, dv))
    idx = np.broadcast_to(rng.permutation(n).astype(np.int32), (B, T, n)).copy()
    got = oracle.sparse_attention(q, k, v, idx, 0.3)
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)                 # [B, H, T, dk]
    kt = torch.from_numpy(k)[:, None].expand(B, H, n, dk)
    vt = torch.from_numpy(v)[:, None].expand(B, H, n, dv)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.3)
    np.testing.assert_allclose(got, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-12, atol=1e-12)


def test_sparse_attention_closed_forms():
    rng = np.random.default_rng(51)
    B, T, H, n, dk, dv = 1, 2, 3, 30, 8, 5
    k = rng.standard_normal((B, n, dk))
    v = rng.standard_normal((B, n, dv))
    idx = np.full((B, T, 6), -1, np.int32)
    idx[0, 0, :4] = [3, 7, 11, 29]
    idx[0, 1, 2] = 17                                   # one valid slot
    # q = 0: every selected key weighs the same, o is the mean of their v
    got = oracle.sparse_attention(np.zeros((B, T, H, dk)), k, v, idx, 1.0)
    np.testing.assert_allclose(got[0, 0], np.broadcast_to(v[0, [3, 7, 11, 29]].mean(axis=0), (H, dv)))
    np.testing.assert_allclose(got[0, 1], np.broadcast_to(v[0, 17], (H, dv)))
    # slot order and padding do not matter; no valid slot gives zeros
    q = rng.standard_normal((B, T, H, dk))
    a = oracle.sparse_attention(q, k, v, idx, 0.5)
    perm = idx.copy()
    perm[0, 0] = idx[0, 0][::-1]
    np.testing.assert_allclose(oracle.sparse_attention(q, k, v, perm, 0.5), a, rtol=1e-13)
    none = np.full((B, T, 3), -1, np.int32)
    assert (oracle.sparse_attention(q, k, v, none, 0.5) == 0).all()

"""Seeded generator determinism, and the oracle's golden digest / page figures."""
import os

import numpy as np

from tks_inputs import CONFIGS, gen_keys, gen_q, gen_q_rows, gen_w, gen_w_rows, sample_rows, scaled

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_row_regeneration_matches_full_generation():
    cfg = scaled(CONFIGS[2], n_q=2500, n_k=2500)
    q, w = gen_q(cfg), gen_w(cfg)
    rows = np.array([0, 1, 1023, 1024, 2047, 2499])
    np.testing.assert_array_equal(gen_q_rows(cfg, rows), q.reshape(cfg.rows, 64, 128)[rows])
    np.testing.assert_array_equal(gen_w_rows(cfg, rows), w.reshape(cfg.rows, 64)[rows])
    np.testing.assert_array_equal(gen_q(cfg), q)


def test_config_shapes_and_value_ranges():
    c1 = CONFIGS[1]
    q = gen_q(c1)
    assert q.shape == (1, 1024, 4, 32) and q.dtype == np.uint16
    vals = (q.astype(np.uint32) << 16).view(np.float32)
    assert set(np.unique(vals).tolist()) <= set(range(-4, 5))
    k, ks = gen_keys(CONFIGS[4].__class__(**{**CONFIGS[4].__dict__, "batch": 2, "n_k": 4096}))
    assert k.dtype == np.uint8 and ks.shape == (2, 4096)
    assert not np.any((k & 0x7F) == 0x7F)           # no NaN codes
    assert np.all(ks > 0)


def test_sample_rows_cover_edges():
    cfg = CONFIGS[3]
    r = sample_rows(cfg, 256)
    assert len(r) == 256 and r[0] == 0 and r[-1] == cfg.rows - 1
    assert cfg.topk - 1 in r and np.all(np.diff(r) > 0)


def test_oracle_golden_digest_of_tiny_integer_workload():
    import sys
    sys.path.insert(0, GOLDEN)
    from make_golden import digest_cfg1
    want = {}
    for line in open(os.path.join(GOLDEN, "cfg1_oracle_digest.txt")):
        if line.strip() and not line.startswith("#"):
            a, b = line.split()
            want[a] = b
    assert digest_cfg1() == want


def test_page_figures():
    fig = {}
    for line in open(os.path.join(GOLDEN, "pages_numbers.txt")):
        if line.strip() and not line.startswith("#"):
            name, val = line.split()[:2]
            fig[name] = int(val)
    S, H, m = 65536, 64, 4
    assert S * H * (S // m) * 4 == fig["materialized_scores_bytes"]
    assert 1048576 // 32768 == fig["regime_extension"]

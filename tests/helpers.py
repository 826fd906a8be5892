"""Shared test utilities: device upload and the top-k comparators.

Comparators (integer inputs: exact; float inputs: the relative 1e-3
tolerance on scores, with index sets allowed to differ only where the score
gap to the k-th oracle score is within that tolerance)."""
from __future__ import annotations

import numpy as np

RTOL = 1e-3


def dev(a):
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def host(t):
    return t.detach().cpu().numpy()


def cfg_rows(cfg, x, rows):
    """(q_rows [n, H, D] bf16 bits, w_rows [n, H]) of flat rows `rows`."""
    q = x["q"].reshape(cfg.rows, cfg.heads, cfg.dim)
    w = x["w"].reshape(cfg.rows, cfg.heads)
    return q[rows], w[rows]


def assert_topk_exact(g_idx, g_val, o_idx, o_val, what=""):
    g_idx = np.asarray(g_idx).reshape(o_idx.shape)
    bad = np.nonzero((g_idx != o_idx).any(axis=1))[0]
    assert len(bad) == 0, "%s: %d rows differ, first row %d: gpu %s oracle %s" % (
        what, len(bad), bad[0], g_idx[bad[0]][:12], o_idx[bad[0]][:12])
    if g_val is not None:
        g_val = np.asarray(g_val).reshape(o_val.shape)
        ok = o_idx >= 0
        np.testing.assert_array_equal(g_val[ok].astype(np.float64), o_val[ok], err_msg=what)
        assert np.all(np.isnan(g_val[~ok])), what


def check_topk_float(g_idx, g_val, o_idx, o_val, row_scores, what="", rtol=RTOL):
    """Float comparator for one batch of rows.  row_scores: oracle scores of
    every key per row (-inf where not visible).  Returns per-row recall."""
    g_idx = np.asarray(g_idx).reshape(o_idx.shape)
    recall = []
    for i in range(o_idx.shape[0]):
        O = o_idx[i][o_idx[i] >= 0]
        G = g_idx[i][g_idx[i] >= 0]
        assert len(O) == len(G), "%s row %d: %d valid vs oracle %d" % (what, i, len(G), len(O))
        assert np.all(g_idx[i][len(G):] == -1), "%s row %d: padding" % (what, i)
        if len(O) == 0:
            recall.append(1.0)
            continue
        I = row_scores[i]
        assert np.all(np.isfinite(I[G])), "%s row %d: invisible key selected" % (what, i)
        assert len(np.unique(G)) == len(G), "%s row %d: duplicate index" % (what, i)
        tau = o_val[i][len(O) - 1]
        fin = I[np.isfinite(I)]
        eps = rtol * max(abs(tau), 1e-3 * float(np.max(np.abs(fin))))
        if g_val is not None:
            gv = np.asarray(g_val).reshape(o_idx.shape)[i][:len(G)].astype(np.float64)
            err = np.abs(gv - I[G])
            lim = np.maximum(rtol * np.abs(I[G]), eps)
            assert np.all(err <= lim), "%s row %d: score error %g > %g" % (
                what, i, float(np.max(err - lim)), 0.0)
            assert np.all(np.diff(gv) <= 0), "%s row %d: not sorted by score" % (what, i)
        Gs, Os = set(G.tolist()), set(O.tolist())
        for s in Gs - Os:
            assert I[s] >= tau - eps, "%s row %d: extra key %d score %r < tau %r - %r" % (
                what, i, s, I[s], tau, eps)
        for s in Os - Gs:
            assert I[s] <= tau + eps, "%s row %d: missed key %d score %r > tau %r + %r" % (
                what, i, s, I[s], tau, eps)
        recall.append(len(Gs & Os) / len(Os))
    return np.array(recall)


def iou(a, b):
    out = []
    for x, y in zip(a, b):
        X, Y = set(x[x >= 0].tolist()), set(y[y >= 0].tolist())
        out.append(len(X & Y) / max(1, len(X | Y)))
    return np.array(out)

"""Writes tests/golden/cfg1_oracle_digest.txt from the CPU oracle alone.

The digest pins the oracle's full output on the tiny integer workload
(1,024 causal queries, 4 heads, dim 32, top-64; HISA with 64-key blocks,
4 scored blocks plus the local block) so that any later change to the
oracle's arithmetic shows up.  Run:  python tests/golden/make_golden.py
"""
import hashlib
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from tks_inputs import CONFIGS, make_inputs  # noqa: E402


def digest_cfg1():
    cfg = CONFIGS[1]
    x = make_inputs(cfg)
    rows = np.arange(cfg.rows)
    q = x["q"].reshape(cfg.rows, cfg.heads, cfg.dim)
    w = x["w"].reshape(cfg.rows, cfg.heads)
    fi, fv = oracle.topk_flat(cfg.shape_dict(), q, w, x["k"], x["k_scale"], cfg.topk, rows)
    blk, hi, hv = oracle.hisa(cfg.shape_dict(), q, w, x["k"], x["k_scale"], cfg.block,
                              cfg.m_scored, cfg.force, cfg.topk, rows)
    out = {}
    for name, a in (("flat_idx", fi), ("flat_val", np.nan_to_num(fv, nan=-1e300)),
                    ("hisa_blk", blk), ("hisa_idx", hi),
                    ("hisa_val", np.nan_to_num(hv, nan=-1e300))):
        out[name] = hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
    out["inputs"] = hashlib.sha256(x["q"].tobytes() + x["w"].tobytes() + x["k"].tobytes()).hexdigest()
    return out


if __name__ == "__main__":
    d = digest_cfg1()
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "cfg1_oracle_digest.txt")
    with open(path, "w") as f:
        f.write("# sha256 of the CPU oracle's outputs on the tiny integer workload; "
                "written by tests/golden/make_golden.py\n")
        for kk in sorted(d):
            f.write("%s %s\n" % (kk, d[kk]))
    print(open(path).read())

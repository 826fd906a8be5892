#!/usr/bin/env python3
"""Benchmark of the sparse-attention indexer + top-k hot path on one MI355X.

One step is one pass of the whole path over one batch of synthetic inputs
that are already resident in HBM: the flat (DSA-style) indexer top-k, and the
HISA indexer (block selection and token refinement over pooled keys).  The
default workload is the 64K-context decode step (64 sequences x 1 query,
65,536 fp8 e4m3fn keys with per-token scales, 64 heads, dim 128, top-2048;
HISA blocks of 128 keys, first + local block forced, 62 scored).  A decode
step first appends the new token's key to every sequence's cache
(tks_kv_append: fp8 quantisation of the key and the pooled block it
completes), so the pooled keys stay current without re-pooling the cache;
pooling the whole cache is a per-cache cost, timed on its own.  Prefill
steps pool the keys inside the step.

Prints one JSON line.  `value` is the number of query-key indexer scores the
step evaluates per second (flat + HISA block + HISA token scores); the
per-indexer figures (ms per layer, scores/s, HISA speedup over flat) are in
"flat" and "hisa".  "roofline" rates the kernel that takes the most time in
the step, timed with HIP events on its own stream inside the library;
"cpu_baseline" is the plain CPU oracle timed on a bounded row sample.

    python bench.py [--steps K] [--warmup W] [--config N]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer q-k scores/sec and ms/layer at 64K ctx, flat vs HISA, 1 MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PROFILE_DIR = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=4,
                    help="workload id (4 = 64K decode, the headline; 2, 3, 5 = prefill)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-topk-standalone", action="store_true",
                    help="skip the selection-only measurement on a 1 GiB score matrix")
    ap.add_argument("--no-kv-append", action="store_true",
                    help="skip the key-cache append measurement (bulk build + decode appends)")
    ap.add_argument("--no-gather", action="store_true",
                    help="skip the re-layout measurement of the selected latent KV rows")
    ap.add_argument("--no-attention", action="store_true",
                    help="skip the sparse attention measurement over the selected keys")
    ap.add_argument("--eager", action="store_true",
                    help="time the step as eager launches instead of a HIP graph replay")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a device copy of MIB MiB (rocprofv3 counter calibration)")
    return ap.parse_args()


def workload_desc(cfg):
    d = dict(workload=cfg.name, batch=cfg.batch, queries=cfg.n_q, keys=cfg.n_k,
             heads=cfg.heads, dim=cfg.dim, topk=cfg.topk,
             key_dtype="fp8_e4m3fn+fp32 scale" if cfg.key_dtype else "bf16",
             q_pos0=cfg.q_pos0, causal_ratio=cfg.causal_ratio)
    if has_hisa(cfg):
        d.update(hisa_block=cfg.block, hisa_m_scored=cfg.m_scored,
                 hisa_forced="first+local" if cfg.force == 3 else "local")
    if cfg.q_chunk:
        d.update(q_chunk=cfg.q_chunk, k_tile=cfg.k_tile)
    return d


def has_hisa(cfg):
    return cfg.dist in ("int", "drift", "fp8")


def visible_counts(cfg):
    import numpy as np
    t = np.arange(cfg.n_q, dtype=np.int64) + cfg.q_pos0
    vis = np.floor_divide(t, cfg.causal_ratio)
    n = np.where(vis < 0, 0, np.minimum(vis + 1, cfg.n_k))
    return np.tile(n, cfg.batch)


def pmc_traffic(role, workload, src_files):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    when there is none or the kernel source changed since it was taken."""
    path = os.path.join(PROFILE_DIR, "pmc_%s_%s.txt" % (role, workload))
    if not os.path.exists(path):
        return None
    info = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            info[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in src_files:
        h.update(open(os.path.join(ROOT, "top_key_selection_amd", "csrc", f), "rb").read())
    if info.get("source_sha256") != h.hexdigest():
        return None
    try:
        return float(info["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(query rows would shard across GPUs with no exchange between them). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 5}))
        return

    from tks_inputs import CONFIGS, gen_keys, gen_q, gen_w
    from top_key_selection_amd import tks

    cfg = CONFIGS[args.config]
    S = tks.Shape(**cfg.shape_dict())
    dev = torch.device("cuda:0")

    # ---- inputs resident in HBM
    k_np, ks_np = gen_keys(cfg)
    q_np = gen_q(cfg)
    w_np = gen_w(cfg)
    q = torch.from_numpy(q_np.view(np.int16)).view(torch.bfloat16).to(dev)
    del q_np
    w = torch.from_numpy(w_np).to(dev)
    k = (torch.from_numpy(k_np).to(dev) if cfg.key_dtype else
         torch.from_numpy(k_np.view(np.int16)).view(torch.bfloat16).to(dev))
    ks = torch.from_numpy(ks_np).to(dev) if ks_np is not None else None

    # ---- outputs and workspaces, allocated once
    R, K = cfg.rows, cfg.topk
    f_idx = torch.empty((cfg.batch, cfg.n_q, K), dtype=torch.int32, device=dev)
    f_val = torch.empty_like(f_idx, dtype=torch.float32)
    f_ws = tks.workspace(tks.topk_flat_workspace(S, K, cfg.q_chunk, cfg.k_tile), dev)
    hisa = has_hisa(cfg)
    if hisa:
        mt = cfg.m_total
        pooled = torch.empty((cfg.batch, cfg.n_k // cfg.block, cfg.dim), dtype=torch.bfloat16,
                             device=dev)
        blk = torch.empty((cfg.batch, cfg.n_q, mt), dtype=torch.int32, device=dev)
        b_ws = tks.workspace(tks.hisa_block_select_workspace(S, cfg.block, cfg.m_scored), dev)
        h_idx = torch.empty_like(f_idx)
        h_val = torch.empty_like(f_val)
        r_ws = tks.workspace(tks.hisa_refine_workspace(S, cfg.block, mt, K), dev)

    ev = lambda: torch.cuda.Event(enable_timing=True)
    decode = cfg.n_q == 1 and cfg.q_pos0 == cfg.n_k - 1
    pool_once_ms = None
    if hisa and decode:
        # the pooled keys of the resident cache, built once (per-cache cost)
        tks.hisa_pool_keys(S, k, ks, cfg.block, pooled=pooled)
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(5):
            tks.hisa_pool_keys(S, k, ks, cfg.block, pooled=pooled)
        e1.record()
        torch.cuda.synchronize()
        pool_once_ms = e0.elapsed_time(e1) / 5
    if decode:
        # the new token's raw bf16 key of every sequence, appended at the last
        # cache slot each step (the same key each time, so steps repeat
        # exactly); it rewrites that slot's fp8 codes and scale and the
        # pooled block the slot completes
        g_new = torch.Generator(device=dev).manual_seed(4242)
        new_key = torch.randn((cfg.batch, 1, cfg.dim), device=dev, generator=g_new).to(torch.bfloat16)
        a_shape = tks.Shape(cfg.batch, 1, cfg.n_k, 1, cfg.dim, causal_ratio=1,
                            key_dtype=cfg.key_dtype)

    def append():
        tks.kv_append(a_shape, new_key, cfg.n_k - 1, k, ks, None, cfg.block if hisa else 0,
                      pooled if hisa else None)

    def flat():
        tks.topk_flat(S, q, w, k, ks, K, cfg.q_chunk, cfg.k_tile, ws=f_ws, idx=f_idx, vals=f_val)

    def hisa_chain():
        if not decode:
            tks.hisa_pool_keys(S, k, ks, cfg.block, pooled=pooled)
        tks.hisa_block_select(S, q, w, pooled, cfg.block, cfg.m_scored, cfg.force,
                              with_vals=False, ws=b_ws, blk=blk)
        tks.hisa_refine_topk(S, q, w, k, ks, cfg.block, blk, K, ws=r_ws, idx=h_idx, vals=h_val)

    # marks: [0] start, [1] after the append (decode), [2] after flat,
    # [3] after HISA
    def step(marks=None):
        if marks is not None:
            marks[0].record()
        if decode:
            append()
        if marks is not None:
            marks[1].record()
        flat()
        if marks is not None:
            marks[2].record()
        if hisa:
            hisa_chain()
        if marks is not None:
            marks[3].record()

    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # HBM: what the step holds (inputs, outputs, workspaces; the library
    # allocates nothing) against the fp32 score tensors it never builds
    nbytes = lambda *ts: int(sum(t.numel() * t.element_size() for t in ts if t is not None))
    mem = dict(inputs=nbytes(q, w, k, ks), outputs=nbytes(f_idx, f_val),
               workspace=nbytes(f_ws))
    if hisa:
        mem["outputs"] += nbytes(pooled, blk, h_idx, h_val)
        mem["workspace"] += nbytes(b_ws, r_ws)
    mem["peak_allocated"] = int(torch.cuda.max_memory_allocated(dev))
    mem["materialised_scores_fp32"] = cfg.batch * cfg.n_q * cfg.n_k * 4
    mem["flat_workspace"] = nbytes(f_ws)
    mem["flat_form"] = "fused" if (decode and cfg.dim == 128 and not cfg.q_chunk) else "tiled"
    mem["materialises_full_scores"] = nbytes(f_ws) >= mem["materialised_scores_fp32"]
    mem["materialised_head_scores_fp32"] = tks.materialized_score_bytes(cfg.batch, cfg.n_q, cfg.heads,
                                                                         cfg.n_k)

    # ---- timed region: K steps, events between the calls
    marks = [[ev() for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(marks[i])
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    ms_step = wall_s * 1e3 / args.steps
    ms_step_eager = ms_step
    append_ms = float(np.median([m[0].elapsed_time(m[1]) for m in marks])) if decode else None
    flat_ms = float(np.median([m[1].elapsed_time(m[2]) for m in marks]))

    # ---- the same step captured once as a HIP graph and replayed (what a
    # decode loop does): the launches are recorded, the kernels all run
    launch = "eager"
    two_stream_ms = None
    if not args.eager:
        ref = [t.clone() for t in ([f_idx, f_val] + ([blk, h_idx, h_val] if hisa else []))]
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            step()
        outs = [f_idx, f_val] + ([blk, h_idx, h_val] if hisa else [])
        same = True
        for _ in range(3):
            for t in outs:
                t.fill_(-7)
            g.replay()
            torch.cuda.synchronize()
            same = same and all(torch.equal(a, b) if a.dtype != torch.float32 else
                                torch.equal(torch.nan_to_num(a, nan=-9.0), torch.nan_to_num(b, nan=-9.0))
                                for a, b in zip(outs, ref))
        if same:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                g.replay()
            torch.cuda.synchronize()
            ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
            launch = "hip_graph"
        else:
            print("graph replay differs from eager launches: timing eager", file=sys.stderr)
        del g
        # the flat and HISA indexers share no buffer: the same step with HISA
        # forked onto a second stream (default priority) and joined, captured
        # as one graph -- the latency-bound selections of one path overlap the
        # streaming kernels of the other.  Reported beside the sequential step.
        if hisa and same:
            s2 = torch.cuda.Stream()

            def step2():
                cur = torch.cuda.current_stream()
                if decode:
                    append()
                s2.wait_stream(cur)
                with torch.cuda.stream(s2):
                    hisa_chain()
                flat()
                cur.wait_stream(s2)

            g2 = torch.cuda.CUDAGraph()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step2()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            with torch.cuda.graph(g2):
                step2()
            same2 = True
            for _ in range(3):
                for t in outs:
                    t.fill_(-7)
                g2.replay()
                torch.cuda.synchronize()
                same2 = same2 and all(torch.equal(a, b) if a.dtype != torch.float32 else
                                      torch.equal(torch.nan_to_num(a, nan=-9.0), torch.nan_to_num(b, nan=-9.0))
                                      for a, b in zip(outs, ref))
            if same2:
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(args.steps):
                    g2.replay()
                torch.cuda.synchronize()
                two_stream_ms = (time.perf_counter() - t0) * 1e3 / args.steps
            del g2
    if hisa:
        hisa_ms = float(np.median([m[2].elapsed_time(m[3]) for m in marks]))

    # ---- per-kernel times: the same steps again with library event brackets
    tks.profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    roles = {}
    for role in tks.PROFILE_ROLES:
        tot, n = tks.profile_read(role)
        if n:
            roles[role] = (tot, n)
    tks.profile_enable(False)

    # ---- work counts
    nvis = visible_counts(cfg)
    flat_pairs = int(nvis.sum())
    out = {}
    if hisa:
        blk_np = blk.cpu().numpy().reshape(R, -1)
        L = np.where(nvis > 0, (nvis - 1) // cfg.block, -1)
        block_pairs = int(np.maximum(L, 0).sum())           # pooled blocks scored per row
        tok = 0
        for r in range(R):
            kept = blk_np[r][blk_np[r] >= 0]
            tok += int(np.minimum(np.maximum(nvis[r] - kept * cfg.block, 0), cfg.block).sum())
        hisa_pairs = block_pairs + tok
        fi = f_idx.cpu().numpy().reshape(R, -1)
        hi = h_idx.cpu().numpy().reshape(R, -1)
        ious = []
        for r in range(0, R, max(1, R // 256)):
            a, b = set(fi[r][fi[r] >= 0].tolist()), set(hi[r][hi[r] >= 0].tolist())
            ious.append(len(a & b) / max(1, len(a | b)))
        out["hisa"] = dict(
            ms_per_layer=round(hisa_ms, 4),
            pooling="in the step" if not decode else
                    "kept current by the step's key append; full pool timed once per cache",
            full_pool_ms_per_cache=round(pool_once_ms, 4) if pool_once_ms else None,
            qk_scores_scored=hisa_pairs,
            qk_scores_per_s_scored=hisa_pairs / (hisa_ms * 1e-3),
            qk_scores_per_s_flat_equivalent=flat_pairs / (hisa_ms * 1e-3),
            speedup_vs_flat=round(flat_ms / hisa_ms, 3),
            iou_vs_flat_mean=round(float(np.mean(ious)), 4))
    if decode:
        out["append"] = dict(ms=round(append_ms, 4), keys_per_step=cfg.batch,
                             what="one raw bf16 key per sequence: fp8 codes + scale of the "
                                  "last slot and the pooled block it completes")
    else:
        hisa_pairs = block_pairs = tok = 0
    out["flat"] = dict(ms_per_layer=round(flat_ms, 4), qk_scores=flat_pairs,
                       qk_scores_per_s=flat_pairs / (flat_ms * 1e-3))
    total_pairs = flat_pairs + hisa_pairs
    value = total_pairs / (ms_step * 1e-3)

    # ---- roofline of the dominant kernel: algorithmic bytes and flops of
    # one launch (per-unit figures times the units one launch processes)
    kb = cfg.dim * (1 if cfg.key_dtype else 2) + (4 if cfg.key_dtype else 0)  # key + scale
    flops_pair = 2 * cfg.heads * cfg.dim
    qw = cfg.heads * (cfg.dim * 2 + 4)                                          # q row + w row
    nb = cfg.n_k // cfg.block if hisa else 0
    # algorithmic bytes: what the operation must read and write (keys, q /
    # w rows, the output lists); a score tile or survivor pool the design
    # writes and reads back is its own traffic, not counted here
    units = {}  # role -> (bytes, flops) per step
    shared = cfg.n_q > 1  # prefill: key rows are shared by the query rows
    units["score_flat"] = (R * qw + (cfg.batch * cfg.n_k * kb if shared else flat_pairs * kb),
                           flat_pairs * flops_pair)
    units["select_flat"] = (R * K * 8, 0)
    if decode:
        units["append"] = (cfg.batch * (cfg.dim * 2 + kb) +
                           (cfg.batch * (cfg.block * kb + cfg.dim * 2) if hisa else 0), 0)
    if hisa:
        units["pool"] = (cfg.batch * nb * cfg.block * kb + cfg.batch * nb * cfg.dim * 2, 0)
        units["score_pooled"] = (R * qw + cfg.batch * nb * cfg.dim * 2, block_pairs * flops_pair)
        units["select_pooled"] = (R * cfg.m_total * 4, 0)
        units["score_refine"] = (tok * kb + R * qw + R * cfg.m_total * 4, tok * flops_pair)
        units["select_refine"] = (R * cfg.m_total * 4 + R * K * 8, 0)
    dom = max(roles, key=lambda r: roles[r][0])
    tot, n = roles[dom]
    avg_ms = tot / n
    per_launch = n / args.steps
    b, f = units[dom]
    b, f = b / per_launch, f / per_launch
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if f and f / b > ridge:
        ach = f / (avg_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(ach, 2), peak=MFMA_BF16_PEAK_TFLOPS,
                    unit="TFLOP/s", frac=round(ach / MFMA_BF16_PEAK_TFLOPS, 4))
    else:
        ach = b / (avg_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(ach / HBM_PEAK_GBS, 4))
    src = {"pool": ["pool.hip"], "append": ["append.hip"],
           "select_flat": ["fused.hip", "select_impl.hpp"] if mem["flat_form"] == "fused" else
                          ["select.hip", "select_impl.hpp"]}.get(
        dom, ["score.hip", "score_common.hpp"] if dom.startswith("score") else
        ["select.hip", "select_impl.hpp"])
    roof["traffic"] = pmc_traffic(dom, cfg.name, src)
    roof.update(kernel=dom, avg_launch_ms=round(avg_ms, 5),
                algorithmic_bytes_per_launch=int(b), algorithmic_flops_per_launch=int(f))
    kern = {}
    for r, (t, nl) in roles.items():
        rb, rf = units.get(r, (0, 0))
        pl = nl / args.steps
        ms = t / nl
        kern[r] = dict(avg_ms=round(ms, 5), launches_per_step=pl,
                       gb_per_s=round(rb / pl / (ms * 1e-3) / 1e9, 1) if rb else None,
                       tflop_per_s=round(rf / pl / (ms * 1e-3) / 1e12, 2) if rf else None)

    # ---- CPU oracle on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, k_np, ks_np, nvis, args.cpu_seconds)

    # ---- the selection on its own over a materialised 1 GiB fp32 score
    # matrix (4096 rows x 65536 keys): 4 B read per score, 8 B written per
    # output entry (index + value)
    ts = None
    if not args.no_topk_standalone:
        g = torch.Generator(device=dev).manual_seed(12345)
        sc = torch.randn((4096, 65536), device=dev, generator=g)
        t_idx = torch.empty((4096, K), dtype=torch.int32, device=dev)
        t_val = torch.empty((4096, K), dtype=torch.float32, device=dev)
        t_ws = tks.workspace(tks.topk_scores_workspace(4096, 65536, K), dev)
        for _ in range(2):
            tks.topk_scores(sc, K, ws=t_ws, idx=t_idx, vals=t_val)
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(5):
            tks.topk_scores(sc, K, ws=t_ws, idx=t_idx, vals=t_val)
        e1.record()
        torch.cuda.synchronize()
        t_ms = e0.elapsed_time(e1) / 5
        tb = sc.numel() * 4 + 4096 * K * 8
        ts = dict(rows=4096, keys=65536, k=K, ms=round(t_ms, 4),
                  gb_per_s=round(tb / (t_ms * 1e-3) / 1e9, 1),
                  frac_hbm=round(tb / (t_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
        del sc, t_idx, t_val, t_ws

    # ---- key-cache append (compression + fp8 quantisation + pooled blocks in
    # one pass): the workload's cache built from raw keys by one bulk append,
    # then one pooled-block cycle of single-key decode appends
    ka = None
    if not args.no_kv_append:
        ka = kv_append_bench(cfg, S, tks, dev, hisa, k, ks, ev, pool_once_ms)

    # ---- re-layout of the rows the flat top-k selected: a synthetic 576-dim
    # bf16 latent KV cache (512 + 64, the MLA latent of DeepSeek-V3.2-style
    # sparse attention; the pages give no attention shapes), one row per key
    ga = None
    if not args.no_gather:
        ga = gather_bench(cfg, tks, dev, f_idx, ev)

    # ---- the consumer: sparse attention of each query over the keys the flat
    # top-k selected (synthetic shapes: 128 query heads over one shared bf16
    # K / V head of width 128; the pages give none)
    at = None
    if not args.no_attention:
        at = attention_bench(cfg, tks, dev, f_idx, ev)

    line = {
        "metric": METRIC, "value": value, "unit": "q-k scores/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "launch": launch, "ms_per_step_eager": round(ms_step_eager, 4),
        "ms_per_step_two_streams": round(two_stream_ms, 4) if two_stream_ms else None,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": workload_desc(cfg),
        "roofline": roof,
        "cpu_baseline": cpu,
        **out,
        "kernels": kern,
        "hbm_bytes": mem,
        "topk_standalone": ts,
        "kv_append": ka,
        "gather_selected": ga,
        "sparse_attention": at,
    }
    print(json.dumps(line), flush=True)


def kv_append_bench(cfg, S, tks, dev, hisa, k, ks, ev, pool_ms):
    """Times tks_kv_append on the workload's cache shape with its own buffers:
    a bulk build of the whole cache (raw keys read once, codes, scales and
    pooled blocks written once) and a cycle of single-key appends that
    completes one pooled block.  The cycle re-appends the last raw keys, so
    the cache must come out identical to the bulk build."""
    import torch
    m = cfg.causal_ratio
    B = cfg.block if hisa else 0
    n_raw = cfg.n_k * m
    g = torch.Generator(device=dev).manual_seed(777)
    raw = torch.randn((cfg.batch, n_raw, cfg.dim), device=dev, generator=g).to(torch.bfloat16)
    k_a = torch.empty_like(k)
    ks_a = torch.empty_like(ks) if ks is not None else None
    p_a = (torch.empty((cfg.batch, cfg.n_k // B, cfg.dim), dtype=torch.bfloat16, device=dev)
           if B else None)
    tail = torch.zeros((cfg.batch, m, cfg.dim), dtype=torch.bfloat16, device=dev) if m > 1 else None
    sa = tks.Shape(cfg.batch, 1, cfg.n_k, 1, cfg.dim, causal_ratio=m, key_dtype=cfg.key_dtype)
    app = lambda r, pos: tks.kv_append(sa, r, pos, k_a, ks_a, tail, B, p_a)

    for _ in range(2):
        app(raw, 0)
    e0, e1 = ev(), ev()
    reps = 5
    e0.record()
    for _ in range(reps):
        app(raw, 0)
    e1.record()
    torch.cuda.synchronize()
    bulk_ms = e0.elapsed_time(e1) / reps
    nbytes = raw.numel() * 2 + k_a.numel() * k_a.element_size() + \
        (ks_a.numel() * 4 if ks_a is not None else 0) + (p_a.numel() * 2 if p_a is not None else 0)
    ref_k = k_a.clone()
    ref_p = p_a.clone() if p_a is not None else None

    cyc = m * (B or 64)
    r0 = n_raw - cyc
    singles = [raw[:, p:p + 1].contiguous() for p in range(r0, n_raw)]
    for i, r in enumerate(singles):
        app(r, r0 + i)
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    e0.record()
    for i, r in enumerate(singles):
        app(r, r0 + i)
    e1.record()
    torch.cuda.synchronize()
    eager_us = e0.elapsed_time(e1) * 1e3 / cyc
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i, r in enumerate(singles):
            app(r, r0 + i)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    e0.record()
    for _ in range(3):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) * 1e3 / (3 * cyc)
    same = bool(torch.equal(k_a, ref_k) and (p_a is None or torch.equal(p_a, ref_p)))
    del graph
    out = dict(
        ratio=m, block=B, raw_keys_per_seq=n_raw,
        bulk=dict(ms=round(bulk_ms, 4), bytes=int(nbytes),
                  gb_per_s=round(nbytes / (bulk_ms * 1e-3) / 1e9, 1),
                  frac_hbm=round(nbytes / (bulk_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)),
        decode=dict(appends=cyc, us_per_append_eager=round(eager_us, 2),
                    us_per_append_graph=round(graph_us, 2),
                    full_pool_us=round(pool_ms * 1e3, 1) if pool_ms else None),
        cache_identical_to_bulk=same)
    del raw, k_a, ks_a, p_a, tail, singles, ref_k, ref_p
    torch.cuda.empty_cache()
    return out


def gather_bench(cfg, tks, dev, idx, ev, latent_dim=576):
    """tks_gather_selected of the step's flat top-k indices over a latent KV
    cache of the workload's shape: bytes = selected rows read + written once,
    plus the indices."""
    import torch
    g = torch.Generator(device=dev).manual_seed(99)
    kv = torch.randint(-32768, 32767, (cfg.batch, cfg.n_k, latent_dim), dtype=torch.int16, device=dev,
                       generator=g)
    out = torch.empty((cfg.batch, cfg.n_q, cfg.topk, latent_dim), dtype=torch.int16, device=dev)
    for _ in range(2):
        tks.gather_selected(kv, idx, out)
    e0, e1 = ev(), ev()
    reps = 10
    e0.record()
    for _ in range(reps):
        tks.gather_selected(kv, idx, out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = 2 * out.numel() * 2 + idx.numel() * 4
    del kv, out
    torch.cuda.empty_cache()
    return dict(rows=int(idx.numel()), row_bytes=latent_dim * 2, ms=round(ms, 4), bytes=int(nbytes),
                gb_per_s=round(nbytes / (ms * 1e-3) / 1e9, 1),
                frac_hbm=round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))


def attention_bench(cfg, tks, dev, idx, ev, heads=128, dim=128):
    """tks_sparse_attention of the step's queries over the keys the flat top-k
    selected.  Bytes: the selected K and V rows read once, q read and the
    fp32 output written; flops 4 * heads * dim per (query, selected key)."""
    import torch
    g = torch.Generator(device=dev).manual_seed(98)
    q = torch.randn((cfg.batch, cfg.n_q, heads, dim), device=dev, generator=g).to(torch.bfloat16)
    k = torch.randn((cfg.batch, cfg.n_k, dim), device=dev, generator=g).to(torch.bfloat16)
    v = torch.randn((cfg.batch, cfg.n_k, dim), device=dev, generator=g).to(torch.bfloat16)
    out = torch.empty((cfg.batch, cfg.n_q, heads, dim), dtype=torch.float32, device=dev)
    ws = tks.workspace(tks.sparse_attention_workspace(cfg.batch, cfg.n_q, heads, cfg.topk), dev)
    scale = dim ** -0.5
    for _ in range(2):
        tks.sparse_attention(q, k, v, idx, scale, out=out, ws=ws)
    torch.cuda.synchronize()
    tks.profile_enable(True)
    reps = 10
    for _ in range(reps):
        tks.sparse_attention(q, k, v, idx, scale, out=out, ws=ws)
    torch.cuda.synchronize()
    tot, n = tks.profile_read("attend")
    tks.profile_enable(False)
    ms = tot / max(n, 1)
    sel = int((idx >= 0).sum().item())
    nbytes = sel * 2 * dim * 2 + q.numel() * 2 + out.numel() * 4
    flops = 4.0 * heads * dim * sel
    del q, k, v, out, ws
    torch.cuda.empty_cache()
    return dict(heads=heads, dim=dim, selected=sel, ms=round(ms, 4), bytes=int(nbytes),
                gb_per_s=round(nbytes / (ms * 1e-3) / 1e9, 1),
                frac_hbm=round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                tflop_per_s=round(flops / (ms * 1e-3) / 1e12, 2))


def cpu_baseline(cfg, k_np, ks_np, nvis, target_s):
    """The CPU oracle, as it stands, on a sample of the workload's rows: flat
    top-k and (where the workload has it) HISA pooling / selection /
    refinement of those rows.  Rate in q-k scores per second."""
    import numpy as np

    import oracle
    from tks_inputs import gen_q_rows, gen_w_rows

    threads = oracle.num_threads()
    R = cfg.rows
    # pick rows from the end (the longest) and grow the sample until the
    # estimated time reaches the target
    order = np.argsort(-nvis, kind="stable")
    probe = order[:1]
    t0 = time.perf_counter()
    sh = cfg.shape_dict()
    oracle.topk_flat(sh, gen_q_rows(cfg, probe), gen_w_rows(cfg, probe), k_np, ks_np, cfg.topk,
                     probe, with_vals=False)
    per_row = max(time.perf_counter() - t0, 1e-4)
    # rows run in parallel, one per thread; HISA roughly doubles the per-row cost
    n = int(target_s * threads / (per_row * (2 if has_hisa(cfg) else 1)))
    n = max(1, min(R, n))
    rows = np.sort(order[:n])
    qr, wr = gen_q_rows(cfg, rows), gen_w_rows(cfg, rows)
    pairs = int(nvis[rows].sum())
    t0 = time.perf_counter()
    oracle.topk_flat(sh, qr, wr, k_np, ks_np, cfg.topk, rows, with_vals=False)
    if has_hisa(cfg):
        seqs = np.unique(rows // cfg.n_q)
        sub = dict(sh, batch=len(seqs))
        kk = k_np[seqs]
        kks = ks_np[seqs] if ks_np is not None else None
        remap = {int(s): i for i, s in enumerate(seqs)}
        lrows = np.array([remap[int(r) // cfg.n_q] * cfg.n_q + int(r) % cfg.n_q for r in rows])
        blk, _, _ = oracle.hisa(sub, qr, wr, kk, kks, cfg.block, cfg.m_scored, cfg.force,
                                cfg.topk, lrows, with_vals=False)
        L = np.where(nvis[rows] > 0, (nvis[rows] - 1) // cfg.block, -1)
        pairs += int(np.maximum(L, 0).sum())
        for i in range(len(rows)):
            kept = blk[i][blk[i] >= 0]
            pairs += int(np.minimum(np.maximum(nvis[rows[i]] - kept * cfg.block, 0),
                                    cfg.block).sum())
    dt = time.perf_counter() - t0
    what = "flat top-k" + (" + HISA (pooling of the sampled sequences, block select, refine)"
                           if has_hisa(cfg) else "")
    return dict(value=pairs / dt, unit="q-k scores/s", cores=threads, kind="oracle",
                seconds=round(dt, 2),
                sample="%d of %d query rows (the longest), %s, %d q-k scores" % (
                    len(rows), R, what, pairs))


if __name__ == "__main__":
    main()

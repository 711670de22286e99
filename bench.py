#!/usr/bin/env python3
"""Benchmark of the MISA indexer on one MI355X.

Default workload (the headline): hierarchical MISA (MISA†) decode at 128K
context -- 4 sequences x 1 query, L = 131072, H = 64, d = 128, B = 128, h = 8
routed heads, k' = 8192 candidates re-ranked by all 64 heads to k = 2048.

A step is one decode pass of the indexer over the batch: route (top-h heads on
the resident pooled keys) -> routed scoring + top-k' -> dense re-rank -> top-k.
Pooled keys are maintained alongside the key cache in decode, so the step reads
them resident; pooling is timed as its own row, as is the dense DSA indexer on
the same inputs. Inputs sit in HBM before the timed region. Every timed step
uses a different copy of the key cache (rotation over > 512 MiB) so that no step
is served from the 256 MB Infinity Cache.

Prints ONE JSON line (see --help for the other workloads).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "indexer Gtokens scored/s + ms/query at 128K decode; % HBM / MFMA roofline"
ROTATE_BYTES = 600 << 20       # key-cache copies cycled per step (> 2 x 256 MB MALL)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c4", choices=["c1", "c2", "c3", "c4", "c1m"],
                    help="c4 (default): MISA† 128K decode; c1: DeepSeek-V3.2-like decode; "
                         "c3: GLM-5-like decode; c2: causal prefill 16K; c1m: c1 with 4 consecutive "
                         "decode positions per sequence (multi-token prediction)")
    ap.add_argument("--warm-cache", action="store_true", help="no key-cache rotation")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true", help="skip the per-row timings")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of HIP-graph replays of the step")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run 5 plain device-to-device copies of 256 MiB (the reference kernel of known size "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


# HBM traffic of the scoring kernel from rocprofv3 counters (FETCH_SIZE, WRITE_SIZE,
# scaled by a plain copy of known size), recorded in this summary together with a
# hash of the kernel's sources; the figure is reported only while they still match.
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "score_decode_c4.md")
KERNEL_SOURCES = ["score.hip", "misa_score_dev.hpp", "misa_common.hpp", "misa_internal.hpp"]


def kernel_sources_sha256():
    import hashlib
    hsh = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "routed_token_indexer_amd", "csrc", f), "rb") as fh:
            hsh.update(fh.read())
    return hsh.hexdigest()


def recorded_traffic(config_name):
    """Bytes per launch measured for the scoring kernel, or None if not measured for
    this workload or the kernel sources changed since."""
    try:
        with open(TRAFFIC_SUMMARY) as fh:
            kv = dict(line.split(":", 1) for line in fh.read().splitlines()
                      if line.startswith(("kernel_sources_sha256:", "traffic_bytes_per_launch:", "workload_config:")))
    except OSError:
        return None
    if kv.get("workload_config", "").strip() != config_name:
        return None
    if kv.get("kernel_sources_sha256", "").strip() != kernel_sources_sha256():
        return None
    return int(kv["traffic_bytes_per_launch"].strip())


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the indexer runs on one GPU (got --gpus {args.gpus}); it has no multi-GPU mode. "
              f"Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from routed_token_indexer_amd import _lib as M
    from routed_token_indexer_amd.workloads import CONFIGS, make_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        n = 256 << 20
        src = torch.ones(n // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device-to-device copy", "copies": 5, "bytes_read_per_copy": n,
                          "bytes_written_per_copy": n}), flush=True)
        return
    cfg = CONFIGS[args.config]
    t_gen = time.time()
    x = make_inputs(cfg, mode="gauss")
    c = x.cfg
    T, H, d, L, B, h = c.T, c.H, c.d, c.L, c.B, c.h
    hier = c.kc is not None
    prefill = c.phase == "prefill"
    kc = c.kc if hier else 0
    topk = c.topk

    def bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    q = bf16(x.q_bf16).contiguous()
    w = torch.from_numpy(x.w).to(dev)
    q_seq = torch.from_numpy(x.q_seq).to(dev)
    q_len = torch.from_numpy(x.q_len).to(dev)
    k0 = bf16(x.k_bf16).contiguous()
    kbytes = k0.numel() * 2
    ncopy = 1 if args.warm_cache else max(1, -(-ROTATE_BYTES // kbytes))
    ks = [k0] + [k0.clone() for _ in range(ncopy - 1)]
    kbars = [M.pool_keys(kk, B) for kk in ks]
    del x.k_bf16
    t_gen = time.time() - t_gen

    # preallocated outputs and workspaces: nothing is allocated inside the timed loops
    heads = torch.empty((T, h), dtype=torch.int32, device=dev)
    cand = torch.empty((T, kc if hier else topk), dtype=torch.int32, device=dev)
    idx = torch.empty((T, topk), dtype=torch.int32, device=dev)
    sc = torch.empty((T, topk), dtype=torch.float32, device=dev)
    didx = torch.empty((T, topk), dtype=torch.int32, device=dev)
    dsc = torch.empty((T, topk), dtype=torch.float32, device=dev)

    def ws(op, **kw):
        return torch.empty(max(M.workspace_bytes(op, T, H, L, **kw), 256), dtype=torch.uint8, device=dev)

    ws_route = ws(M.OP_ROUTE, B=B)
    ws_score = ws(M.OP_SCORE_TOPK, topk=kc or topk)
    ws_rerank = ws(M.OP_HIER_RERANK, topk=topk, kc=kc) if hier else None
    ws_dense = ws(M.OP_DSA_DENSE, topk=topk)
    kbar_pf = torch.empty_like(kbars[0])

    ws_step = ws(M.OP_HIER_INDEXER if hier else M.OP_INDEXER, B=B, topk=topk, kc=kc)

    def step(i):
        # one call of the whole indexer: route -> routed scoring -> top-k (-> dense re-rank)
        kk = ks[i % ncopy]
        kb = M.pool_keys(kk, B, kbar=kbar_pf) if prefill else kbars[i % ncopy]
        if hier:
            M.hier_indexer(q, w, kk, kb, q_seq, q_len, B, h, kc, topk, heads=heads, cand=cand, idx=idx, score=sc,
                           ws=ws_step)
        else:
            M.indexer(q, w, kk, kb, q_seq, q_len, B, h, topk, heads=heads, idx=idx, score=sc, ws=ws_step)

    def timed(fn, steps, warmup):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    # ---- eager timed region: K steps; the scoring kernel's launches carry HIP events
    # stamped at the kernel's own start and end (on its stream)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    M.timing_begin(M.KERNEL_SCORE, capacity=4 * args.steps + 16)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms_eager = e0.elapsed_time(e1) / args.steps
    score_ms, score_n = M.timing_end()

    # ---- graph timed region: the step (one per key-cache copy) captured once, replayed
    ms_graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            step(0)                      # warm the capture stream
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=cap):
                for i in range(ncopy):
                    step(i)
        torch.cuda.synchronize()
        reps = max(1, -(-args.steps // ncopy))
        for _ in range(max(1, args.warmup // ncopy)):
            graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(reps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        ms_graph = g0.elapsed_time(g1) / (reps * ncopy)
    ms_step = ms_graph if ms_graph is not None else ms_eager
    t_wall = ms_step * args.steps * 1e-3

    tokens = int(x.q_len.astype(np.int64).sum())
    value = tokens / (ms_step * 1e-3) / 1e9

    # ---- roofline of the dominant kernel (token scoring of the routed pass)
    score_launches_per_step = score_n / args.steps
    per_launch_ms = score_ms / max(score_n, 1)
    if prefill:
        flops = 2.0 * h * d * tokens                       # routed q.k MACs of all queries
        achieved = flops / (per_launch_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None}
    else:
        # keys of the visible prefixes read once (per sequence: the longest prefix among
        # its queries) + gathered routed query rows + head weights
        key_tokens = sum(int(x.q_len[x.q_seq == n].max()) for n in np.unique(x.q_seq))
        kernel_bytes = key_tokens * d * 2 + T * h * d * 2 + T * h * 4
        achieved = kernel_bytes / (per_launch_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(c.name),
                "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "algorithmic_bytes_per_launch": int(kernel_bytes)}
    roof["kernel"] = "score_kernel (routed token scoring, MFMA)"
    roof["avg_launch_us"] = round(per_launch_ms * 1e3, 2)
    roof["launches_per_step"] = score_launches_per_step

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "Gtokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "ms_per_query": round(ms_step / T, 6),
        "timing": ("HIP graph replay of the step (captured once per key-cache copy)" if ms_graph is not None
                   else "eager launches"),
        "ms_per_step_eager": round(ms_eager, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": c.description, "name": c.name, "T": T, "L": L, "H": H, "d": d, "B": B, "h": h,
            "topk": topk, "kc": kc or None, "tokens_per_step": tokens,
            "cache": "warm" if args.warm_cache else f"cold (rotating {ncopy} key-cache copies)",
            "step": ("misa_pool_keys + misa_indexer (route, routed scoring, top-k)" if prefill else
                     "misa_hier_indexer (route, routed scoring, top-k', dense re-rank, top-k)" if hier else
                     "misa_indexer (route, routed scoring, top-k)"),
        },
        "roofline": roof,
        "wall_s_timed_region": round(t_wall, 4),
    }
    print(f"[bench] {args.config}: {ms_step * 1e3:.1f} us/step, {value:.2f} Gtok/s "
          f"(inputs generated and uploaded in {t_gen:.0f}s)", file=sys.stderr, flush=True)

    # ---- every row of the path on the same inputs, timed on its own
    if not args.no_rows:
        rows = {}
        n = max(10, args.steps // 2)
        rows["pool_us"] = timed(lambda i: M.pool_keys(ks[i % ncopy], B, kbar=kbar_pf), n, 3) * 1e3
        if not prefill:
            # incremental pooling of a decode step: one token appended to every
            # sequence, each append closing a block (the most work a step can need)
            nseq_k = ks[0].shape[0]
            new_len = torch.full((nseq_k,), (L // B) * B, dtype=torch.int32, device="cuda")
            prev_len = new_len - 1
            rows["pool_update_us"] = timed(lambda i: M.pool_update(ks[i % ncopy], B, prev_len, new_len, 1, kbar_pf),
                                           n, 3) * 1e3
        rows["route_us"] = timed(lambda i: M.route(q, w, ks[i % ncopy], kbars[i % ncopy], q_seq, q_len, B, h,
                                                   heads=heads, ws=ws_route), n, 3) * 1e3
        kk_sel = kc or topk
        rows["score_topk_us"] = timed(lambda i: M.score_topk(q, w, ks[i % ncopy], heads, q_seq, q_len, kk_sel,
                                                             idx=cand, want_score=False, ws=ws_score), n, 3) * 1e3
        if hier:
            rows["hier_rerank_us"] = timed(lambda i: M.hier_rerank(q, w, ks[i % ncopy], cand, q_seq, q_len, topk,
                                                                   idx=idx, score=sc, ws=ws_rerank), n, 3) * 1e3
        rows["dense_dsa_us"] = timed(lambda i: M.dsa_index_dense(q, w, ks[i % ncopy], q_seq, q_len, topk,
                                                                 idx=didx, score=dsc, ws=ws_dense), n, 3) * 1e3
        rows["all_rows_us"] = timed(lambda i: (M.pool_keys(ks[i % ncopy], B, kbar=kbar_pf), step(i),
                                               M.dsa_index_dense(q, w, ks[i % ncopy], q_seq, q_len, topk, idx=didx,
                                                                 score=dsc, ws=ws_dense)), n, 3) * 1e3
        if not prefill:
            # the block filter composed with routing: m complete blocks kept per
            # query (about 4 * topk candidate tokens), routed top-k among them
            m_blk = max(1, min(L // B, (4 * topk) // B))
            bidx = torch.empty_like(idx)
            ws_blk = ws(M.OP_BLOCK_INDEXER, B=B, topk=topk, kc=m_blk)
            rows["block_indexer_us"] = timed(lambda i: M.block_indexer(q, w, ks[i % ncopy], kbars[i % ncopy], q_seq,
                                                                       q_len, B, h, m_blk, topk, idx=bidx,
                                                                       want_score=False, ws=ws_blk), n, 3) * 1e3
        if T > c.nseq:
            # several queries per sequence: the proxy-query shared scan over groups of
            # consecutive queries (one multi-token step per sequence, or 16 prefill positions)
            G_pv = 16 if prefill else T // c.nseq
            kc_pv = min(L, (2 if prefill else 4) * topk)
            pidx = torch.empty_like(idx)
            ws_pv = ws(M.OP_PIVOT_INDEXER, B=G_pv, topk=topk, kc=kc_pv)
            rows["pivot_us"] = timed(lambda i: M.pivot_indexer(q, w, ks[i % ncopy], q_seq, q_len, G_pv, kc_pv, topk,
                                                               idx=pidx, want_score=False, ws=ws_pv),
                                     3 if prefill else n, 1) * 1e3
            out["pivot"] = {"G": G_pv, "kc": kc_pv}
        out["rows"] = {kk: round(v, 2) for kk, v in rows.items()}
        # recall of the routed selections against the dense indexer on the same inputs (no target)
        if not prefill:
            step(0)
            M.dsa_index_dense(q, w, ks[0], q_seq, q_len, topk, idx=didx, score=dsc, ws=ws_dense)
            routed = torch.empty_like(idx)
            M.score_topk(q, w, ks[0], heads, q_seq, q_len, topk, idx=routed, want_score=False, ws=ws_score)
            torch.cuda.synchronize()
            dn, fi, ro = didx.cpu().numpy(), idx.cpu().numpy(), routed.cpu().numpy()
            rec = lambda a: float(np.mean([len(np.intersect1d(a[t], dn[t])) / topk for t in range(T)]))
            out["recall_vs_dense"] = {"misa": round(rec(ro), 4)}
            if hier:
                out["recall_vs_dense"]["misa_hier"] = round(rec(fi), 4)
            M.block_indexer(q, w, ks[0], kbars[0], q_seq, q_len, B, h, m_blk, topk, idx=bidx, want_score=False,
                            ws=ws_blk)
            torch.cuda.synchronize()
            out["recall_vs_dense"][f"block_filter_m{m_blk}"] = round(rec(bidx.cpu().numpy()), 4)
            if T > c.nseq:
                M.pivot_indexer(q, w, ks[0], q_seq, q_len, G_pv, kc_pv, topk, idx=pidx, want_score=False, ws=ws_pv)
                torch.cuda.synchronize()
                out["recall_vs_dense"][f"pivot_G{G_pv}"] = round(rec(pidx.cpu().numpy()), 4)

    # ---- the CPU oracle on the host cores, on a bounded sample of the same workload
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, c, hier, prefill)

    print(json.dumps(out), flush=True)


def cpu_baseline(x, c, hier, prefill):
    from oracle import misa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = None
    if prefill:
        qs = [c.T - 1 - 64 * i for i in range(4)]          # the longest prefixes
    else:
        qs = list(range(c.T))
    tokens = int(sum(int(x.q_len[t]) for t in qs))
    xx = x
    t0 = time.perf_counter()
    runs = 0
    best = float("inf")
    while runs < 3 and (time.perf_counter() - t0) < 30.0:
        t1 = time.perf_counter()
        if hier:
            O.misa_hier_indexer(xx.q, xx.w, xx.k, xx.q_seq, xx.q_len, c.B, c.h, c.kc, c.topk, queries=qs)
        else:
            O.misa_indexer(xx.q, xx.w, xx.k, xx.q_seq, xx.q_len, c.B, c.h, c.topk, queries=qs)
        best = min(best, time.perf_counter() - t1)
        runs += 1
    return {
        "value": round(tokens / best / 1e9, 6), "unit": "Gtokens/s", "cores": threads,
        "kind": "oracle",
        "sample": f"{len(qs)} queries ({tokens} prefix tokens) of the same workload; fp64 NumPy oracle, "
                  f"{'route+score+top-k+re-rank' if hier else 'route+score+top-k'}, best of {runs} runs "
                  f"({best:.2f} s each)",
        "ms_per_query": round(best * 1e3 / len(qs), 2),
    }


if __name__ == "__main__":
    main()

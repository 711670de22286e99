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
is served from the 256 MB Infinity Cache; warm-cache figures (one copy) are
reported beside them.

The same JSON line also carries the other workloads, each timed the same way:
DeepSeek-V3.2-like decode (c1), causal prefill at 16K (c2, MFMA-bound) and
GLM-5-like decode (c3), and the CPU oracle's baseline.

Prints ONE JSON line (see --help for the options).
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
    ap.add_argument("--config", default="c4", choices=["c1", "c2", "c3", "c4", "c1m", "c2_128k"],
                    help="headline workload. c4 (default): MISA† 128K decode; c1: DeepSeek-V3.2-like decode; "
                         "c3: GLM-5-like decode; c2: causal prefill 16K; c1m: c1 with 4 consecutive "
                         "decode positions per sequence (multi-token prediction)")
    ap.add_argument("--no-subconfigs", action="store_true", help="time only the headline workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true", help="skip the per-row timings")
    ap.add_argument("--no-warm", action="store_true", help="skip the warm-cache figures")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of HIP-graph replays of the step")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run 5 plain device-to-device copies of 256 MiB (the reference kernel of known size "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


# HBM traffic of the dominant kernel from rocprofv3 counters (FETCH_SIZE, WRITE_SIZE,
# scaled by a plain copy of known size), recorded in a summary together with a
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
    """Bytes per launch measured for the dominant kernel, or None if not measured for
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


def algorithmic(c, x):
    """What the step must move (decode, bytes) or compute (prefill, flops), and the
    same for its dominant kernel."""
    T, H, d, B, h = c.T, c.H, c.d, c.B, c.h
    q_len = x.q_len.astype(np.int64)
    if c.phase == "prefill":
        routed = 2.0 * h * d * float(q_len.sum())                       # routed q.k multiply-adds
        router = 2.0 * H * d * float(np.sum(-(-q_len // B)))            # q.Kbar over ceil(p / B) blocks
        return {"bound": "mfma", "step": routed + router, "kernel": routed,
                "kernel_label": "score_prefill_kernel (routed token scoring, MFMA)"}
    # keys of the visible prefixes read once per sequence (the longest prefix among its
    # queries), the complete pooled blocks, the query rows and weights, the outputs
    key_tok = sum(int(q_len[x.q_seq == n].max()) for n in np.unique(x.q_seq))
    kbar = sum(int(q_len[x.q_seq == n].max()) // B for n in np.unique(x.q_seq)) * d * 4
    step = key_tok * d * 2 + kbar + T * H * d * 2 + T * H * 4 + T * h * 4 + T * c.topk * 8
    if c.kc:
        # MISA-dagger: the candidates' keys gathered for the dense re-rank, the candidate list
        step += int(np.minimum(q_len, c.kc).sum()) * d * 2 + T * c.kc * 4
    # the dominant kernel, the routed token scoring: every visible key once, the
    # gathered routed query rows and their weights
    kernel = key_tok * d * 2 + T * h * d * 2 + T * h * 4
    return {"bound": "hbm", "step": float(step), "kernel": float(kernel),
            "kernel_label": "score_decode_kernel (routed token scoring, MFMA)"}


class Workload:
    """Device inputs, outputs and workspaces of one workload, and its step."""

    def __init__(self, name, M, dev, warm=False):
        import torch
        from routed_token_indexer_amd.workloads import CONFIGS, make_inputs
        self.t_gen = time.time()
        x = make_inputs(CONFIGS[name], mode="gauss")
        c = x.cfg
        self.x, self.c, self.M = x, c, M
        self.hier = c.kc is not None
        self.prefill = c.phase == "prefill"
        T, H, L, B, h = c.T, c.H, c.L, c.B, c.h
        kc = c.kc if self.hier else 0

        def bf16(bits):
            return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

        self.q = bf16(x.q_bf16).contiguous()
        self.w = torch.from_numpy(x.w).to(dev)
        self.q_seq = torch.from_numpy(x.q_seq).to(dev)
        self.q_len = torch.from_numpy(x.q_len).to(dev)
        k0 = bf16(x.k_bf16).contiguous()
        kbytes = k0.numel() * 2
        # prefill re-reads its 256 MiB of query rows every step (beyond the MALL); its
        # 4 MiB of keys are not rotated
        self.ncopy = 1 if (warm or self.prefill) else max(1, -(-ROTATE_BYTES // kbytes))
        self.ks = [k0] + [k0.clone() for _ in range(self.ncopy - 1)]
        self.kbars = [M.pool_keys(kk, B) for kk in self.ks]
        del x.k_bf16
        self.t_gen = time.time() - self.t_gen

        self.heads = torch.empty((T, h), dtype=torch.int32, device=dev)
        self.cand = torch.empty((T, kc if self.hier else c.topk), dtype=torch.int32, device=dev)
        self.idx = torch.empty((T, c.topk), dtype=torch.int32, device=dev)
        self.sc = torch.empty((T, c.topk), dtype=torch.float32, device=dev)
        self.kbar_pf = torch.empty_like(self.kbars[0])
        self.ws_step = self.ws(M.OP_HIER_INDEXER if self.hier else M.OP_INDEXER, B=B, topk=c.topk, kc=kc)

    def ws(self, op, **kw):
        import torch
        c = self.c
        return torch.empty(max(self.M.workspace_bytes(op, c.T, c.H, c.L, **kw), 256), dtype=torch.uint8,
                           device=self.q.device)

    def step(self, i):
        # one call of the whole indexer: route -> routed scoring -> top-k (-> dense re-rank)
        M, c = self.M, self.c
        kk = self.ks[i % self.ncopy]
        kb = M.pool_keys(kk, c.B, kbar=self.kbar_pf) if self.prefill else self.kbars[i % self.ncopy]
        if self.hier:
            M.hier_indexer(self.q, self.w, kk, kb, self.q_seq, self.q_len, c.B, c.h, c.kc, c.topk, heads=self.heads,
                           cand=self.cand, idx=self.idx, score=self.sc, ws=self.ws_step)
        else:
            M.indexer(self.q, self.w, kk, kb, self.q_seq, self.q_len, c.B, c.h, c.topk, heads=self.heads,
                      idx=self.idx, score=self.sc, ws=self.ws_step)


def timed(fn, steps, warmup):
    import torch
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


def measure(wl, steps, warmup, eager_only=False):
    """Step time (HIP-graph replays and eager launches) and the dominant kernel's
    average launch duration (events stamped at its own start and end, on its stream)."""
    import torch
    M = wl.M
    for i in range(warmup):
        wl.step(i)
    torch.cuda.synchronize()
    M.timing_begin(M.KERNEL_SCORE, capacity=4 * steps + 16)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        wl.step(i)
    e1.record()
    torch.cuda.synchronize()
    ms_eager = e0.elapsed_time(e1) / steps
    k_ms, k_n = M.timing_end()
    ms_graph = None
    if not eager_only:
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            wl.step(0)                      # warm the capture stream
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=cap):
                for i in range(wl.ncopy):
                    wl.step(i)
        torch.cuda.synchronize()
        reps = max(1, -(-steps // wl.ncopy))
        for _ in range(max(1, warmup // wl.ncopy)):
            graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(reps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        ms_graph = g0.elapsed_time(g1) / (reps * wl.ncopy)
        del graph
    return {"ms_graph": ms_graph, "ms_eager": ms_eager, "kernel_ms": k_ms / max(k_n, 1),
            "kernel_launches_per_step": k_n / steps}


def fractions(wl, m):
    """Roofline of the dominant kernel and of the whole step."""
    alg = algorithmic(wl.c, wl.x)
    ms_step = m["ms_graph"] if m["ms_graph"] is not None else m["ms_eager"]
    if alg["bound"] == "mfma":
        unit, peak, scale = "TFLOP/s", MFMA_BF16_PEAK_TFLOPS, 1e12
    else:
        unit, peak, scale = "GB/s", HBM_PEAK_GBS, 1e9
    k_ach = alg["kernel"] / (m["kernel_ms"] * 1e-3) / scale
    s_ach = alg["step"] / (ms_step * 1e-3) / scale
    kernel = {"bound": alg["bound"], "achieved": round(k_ach, 1), "peak": peak, "unit": unit,
              "frac": round(k_ach / peak, 4), "kernel": alg["kernel_label"],
              "avg_launch_us": round(m["kernel_ms"] * 1e3, 2),
              "launches_per_step": m["kernel_launches_per_step"],
              ("algorithmic_flops_per_launch" if alg["bound"] == "mfma" else "algorithmic_bytes_per_launch"):
                  int(alg["kernel"])}
    step = {"bound": alg["bound"], "achieved": round(s_ach, 1), "peak": peak, "unit": unit,
            "frac": round(s_ach / peak, 4),
            ("algorithmic_flops_per_step" if alg["bound"] == "mfma" else "algorithmic_bytes_per_step"): int(alg["step"])}
    return kernel, step, ms_step


def summary(wl, m):
    kernel, step, ms_step = fractions(wl, m)
    tokens = int(wl.x.q_len.astype(np.int64).sum())
    return {"workload": wl.c.description, "us_per_step": round(ms_step * 1e3, 2),
            "us_per_step_eager": round(m["ms_eager"] * 1e3, 2), "gtokens_per_s": round(tokens / ms_step / 1e6, 3),
            "ms_per_query": round(ms_step / wl.c.T, 6), "tokens_per_step": tokens,
            "cache": "warm" if wl.ncopy == 1 and not wl.prefill else
                     ("keys not rotated (the query rows exceed the MALL)" if wl.prefill
                      else f"cold (rotating {wl.ncopy} key-cache copies)"),
            "kernel_frac": kernel["frac"], "kernel_us": kernel["avg_launch_us"], "step_frac": step["frac"],
            "roofline_unit": kernel["unit"]}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the indexer runs on one GPU (got --gpus {args.gpus}); it has no multi-GPU mode. "
              f"Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from routed_token_indexer_amd import _lib as M

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

    if args.config == "c2_128k":
        # the 128K causal prefill alone (the timing record of the default run's configs)
        rec = prefill_128k(M, dev, steps=args.steps, warmup=args.warmup)
        print(json.dumps({"config": "c2_128k", "steps": args.steps, "warmup": args.warmup, **rec}), flush=True)
        return

    wl = Workload(args.config, M, dev)
    c, x = wl.c, wl.x
    T, H, d, L, B, h = c.T, c.H, c.d, c.L, c.B, c.h
    m = measure(wl, args.steps, args.warmup, eager_only=args.eager)
    kernel_roof, step_roof, ms_step = fractions(wl, m)
    kernel_roof["traffic"] = recorded_traffic(c.name)
    kernel_roof["traffic_unit"] = "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    tokens = int(x.q_len.astype(np.int64).sum())
    value = tokens / (ms_step * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "Gtokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "ms_per_query": round(ms_step / T, 6),
        "timing": ("HIP graph replay of the step (captured once per key-cache copy)" if m["ms_graph"] is not None
                   else "eager launches"),
        "ms_per_step_eager": round(m["ms_eager"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": c.description, "name": c.name, "T": T, "L": L, "H": H, "d": d, "B": B, "h": h,
            "topk": c.topk, "kc": c.kc, "tokens_per_step": tokens,
            "cache": "cold (rotating %d key-cache copies)" % wl.ncopy if not wl.prefill else
                     "keys not rotated (the query rows exceed the MALL)",
            "step": ("misa_pool_keys + misa_indexer (route, routed scoring, top-k)" if wl.prefill else
                     "misa_hier_indexer (route, routed scoring, top-k', dense re-rank, top-k)" if wl.hier else
                     "misa_indexer (route, routed scoring, top-k)"),
        },
        "roofline": kernel_roof,
        "step_roofline": step_roof,
        "wall_s_timed_region": round(ms_step * args.steps * 1e-3, 4),
    }
    print(f"[bench] {args.config}: {ms_step * 1e3:.1f} us/step, {value:.2f} Gtok/s, kernel {kernel_roof['frac']:.3f} "
          f"step {step_roof['frac']:.3f} of roofline (inputs generated and uploaded in {wl.t_gen:.0f}s)",
          file=sys.stderr, flush=True)

    # ---- every row of the path on the same inputs, timed on its own
    if not args.no_rows:
        out["rows"], rec = rows_and_recall(wl, args)
        if rec:
            out["recall_vs_dense"] = rec

    # ---- the same step with one key-cache copy (warm: served partly from the MALL)
    if not wl.prefill and not args.no_warm:
        warm = Workload(args.config, M, dev, warm=True)
        mw = measure(warm, args.steps, args.warmup)
        out["warm_cache"] = summary(warm, mw)
        del warm

    # ---- the other workloads, each timed the same way (cold keys)
    if not args.no_subconfigs:
        subs = {}
        for name in ("c1", "c2", "c3", "c4"):
            if name == args.config:
                continue
            del_wl = Workload(name, M, dev)
            ms = measure(del_wl, max(5, args.steps // 2), max(2, args.warmup // 2))
            subs[name] = summary(del_wl, ms)
            print(f"[bench] {name}: {subs[name]['us_per_step']:.1f} us/step, kernel {subs[name]['kernel_frac']:.3f} "
                  f"step {subs[name]['step_frac']:.3f} of roofline", file=sys.stderr, flush=True)
            del del_wl
            torch.cuda.empty_cache()
        # a causal prefill at 128K context (score rows in query slabs)
        try:
            subs["c2_128k"] = prefill_128k(M, dev)
            print(f"[bench] c2_128k: {subs['c2_128k']['us_per_step'] / 1e3:.1f} ms/step, kernel "
                  f"{subs['c2_128k']['kernel_frac']:.3f} step {subs['c2_128k']['step_frac']:.3f} of roofline",
                  file=sys.stderr, flush=True)
        except Exception as e:   # a timing record only: never lose the headline line for it
            subs["c2_128k"] = {"error": f"{type(e).__name__}: {e}"[:300]}
        out["configs"] = subs

    # ---- the CPU oracle on the host cores, on a bounded sample of the same workload
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, c, wl.hier, wl.prefill)

    print(json.dumps(out), flush=True)


def prefill_128k(M, dev, steps=2, warmup=1):
    """A causal prefill at 128K context (every position a query): pooling, routing,
    routed scoring and the row top-k, the c2 step at 8x the length. The score rows
    take consecutive slabs of 2048 queries. Inputs are drawn on the GPU with
    torch's seeded generator: q and k ~ N(0, 1/d) i.i.d., w = softmax of N(0, 1)
    (the workload generator's AR(1) keys would take minutes on the host at this
    size); this is a timing record, not a parity case."""
    import torch
    L = T = 131072
    H, d, B, h, k = 64, 128, 64, 8, 2048
    g = torch.Generator(device=dev)
    g.manual_seed(1302)
    q = (torch.randn(T, H, d, device=dev, generator=g) / d ** 0.5).to(torch.bfloat16)
    keys = (torch.randn(1, L, d, device=dev, generator=g) / d ** 0.5).to(torch.bfloat16)
    w = torch.softmax(torch.randn(T, H, device=dev, generator=g), dim=1).float().contiguous()
    q_seq = torch.zeros(T, dtype=torch.int32, device=dev)
    q_len = torch.arange(1, T + 1, dtype=torch.int32, device=dev)
    kbar = torch.empty((1, L // B, d), dtype=torch.float32, device=dev)
    heads = torch.empty((T, h), dtype=torch.int32, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    sc = torch.empty((T, k), dtype=torch.float32, device=dev)
    wsb = M.workspace_bytes(M.OP_INDEXER, T, H, L, B, k)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

    def step(_):
        M.pool_keys(keys, B, kbar=kbar)
        M.indexer(q, w, keys, kbar, q_seq, q_len, B, h, k, heads=heads, idx=idx, score=sc, ws=ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    M.timing_begin(M.KERNEL_SCORE, capacity=128 * steps + 16)
    ms = timed(step, steps, 0)
    k_ms, k_n = M.timing_end()
    n = (idx >= 0).sum(dim=1)
    valid = bool(n.eq(torch.clamp(q_len, max=k)).all().item())
    p = np.arange(1, T + 1, dtype=np.float64)
    routed = 2.0 * h * d * p.sum()
    router = 2.0 * H * d * np.ceil(p / B).sum()
    tokens = int(p.sum())
    del q, keys, w, ws, idx, sc
    torch.cuda.empty_cache()
    return {"workload": "causal prefill at 128K context: L=131072, every position a query, H=64, d=128, B=64, h=8, "
                        "k=2048 (inputs drawn on the GPU)",
            "us_per_step": round(ms * 1e3, 1), "gtokens_per_s": round(tokens / ms / 1e6, 3),
            "tokens_per_step": tokens, "workspace_bytes": wsb, "score_row_slabs": -(-T // 2048),
            "step_frac": round((routed + router) / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "kernel_frac": round(routed / (k_ms * 1e-3 / max(steps, 1)) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "kernel_us": round(k_ms * 1e3 / max(steps, 1), 1), "kernel_launches_per_step": k_n / max(steps, 1),
            "roofline_unit": "TFLOP/s", "rows_valid": valid, "timing": "eager launches"}


def rows_and_recall(wl, args):
    import torch
    M, c, x = wl.M, wl.c, wl.x
    T, L, B, h, topk = c.T, c.L, c.B, c.h, c.topk
    kc = c.kc or 0
    q, w, q_seq, q_len, ks, kbars, ncopy = wl.q, wl.w, wl.q_seq, wl.q_len, wl.ks, wl.kbars, wl.ncopy
    heads, cand, idx, sc = wl.heads, wl.cand, wl.idx, wl.sc
    didx, dsc = torch.empty_like(idx), torch.empty_like(sc)
    ws_route = wl.ws(M.OP_ROUTE, B=B)
    ws_score = wl.ws(M.OP_SCORE_TOPK, topk=kc or topk)
    ws_rerank = wl.ws(M.OP_HIER_RERANK, topk=topk, kc=kc) if wl.hier else None
    ws_dense = wl.ws(M.OP_DSA_DENSE, topk=topk)
    rows = {}
    n = max(10, args.steps // 2)
    rows["pool_us"] = timed(lambda i: M.pool_keys(ks[i % ncopy], B, kbar=wl.kbar_pf), n, 3) * 1e3
    if not wl.prefill:
        # incremental pooling of a decode step: one token appended to every
        # sequence, each append closing a block (the most work a step can need)
        nseq_k = ks[0].shape[0]
        new_len = torch.full((nseq_k,), (L // B) * B, dtype=torch.int32, device="cuda")
        prev_len = new_len - 1
        rows["pool_update_us"] = timed(lambda i: M.pool_update(ks[i % ncopy], B, prev_len, new_len, 1, wl.kbar_pf),
                                       n, 3) * 1e3
    rows["route_us"] = timed(lambda i: M.route(q, w, ks[i % ncopy], kbars[i % ncopy], q_seq, q_len, B, h,
                                               heads=heads, ws=ws_route), n, 3) * 1e3
    kk_sel = kc or topk
    rows["score_topk_us"] = timed(lambda i: M.score_topk(q, w, ks[i % ncopy], heads, q_seq, q_len, kk_sel,
                                                         idx=cand, want_score=False, ws=ws_score), n, 3) * 1e3
    if wl.hier:
        rows["hier_rerank_us"] = timed(lambda i: M.hier_rerank(q, w, ks[i % ncopy], cand, q_seq, q_len, topk,
                                                               idx=idx, score=sc, ws=ws_rerank), n, 3) * 1e3
    rows["dense_dsa_us"] = timed(lambda i: M.dsa_index_dense(q, w, ks[i % ncopy], q_seq, q_len, topk,
                                                             idx=didx, score=dsc, ws=ws_dense), n, 3) * 1e3
    rows["all_rows_us"] = timed(lambda i: (M.pool_keys(ks[i % ncopy], B, kbar=wl.kbar_pf), wl.step(i),
                                           M.dsa_index_dense(q, w, ks[i % ncopy], q_seq, q_len, topk, idx=didx,
                                                             score=dsc, ws=ws_dense)), n, 3) * 1e3
    m_blk = max(1, min(L // B, (4 * topk) // B))
    bidx = torch.empty_like(idx)
    ws_blk = wl.ws(M.OP_BLOCK_INDEXER, B=B, topk=topk, kc=m_blk)
    if not wl.prefill:
        # the block filter composed with routing: m complete blocks kept per
        # query (about 4 * topk candidate tokens), routed top-k among them
        rows["block_indexer_us"] = timed(lambda i: M.block_indexer(q, w, ks[i % ncopy], kbars[i % ncopy], q_seq,
                                                                   q_len, B, h, m_blk, topk, idx=bidx,
                                                                   want_score=False, ws=ws_blk), n, 3) * 1e3
    pv = None
    if T > c.nseq:
        # several queries per sequence: the proxy-query shared scan over groups of
        # consecutive queries (one multi-token step per sequence, or 16 prefill positions)
        G_pv = 16 if wl.prefill else T // c.nseq
        kc_pv = min(L, (2 if wl.prefill else 4) * topk)
        pidx = torch.empty_like(idx)
        ws_pv = wl.ws(M.OP_PIVOT_INDEXER, B=G_pv, topk=topk, kc=kc_pv)
        rows["pivot_us"] = timed(lambda i: M.pivot_indexer(q, w, ks[i % ncopy], q_seq, q_len, G_pv, kc_pv, topk,
                                                           idx=pidx, want_score=False, ws=ws_pv),
                                 3 if wl.prefill else n, 1) * 1e3
        pv = (G_pv, kc_pv, pidx, ws_pv)
    rows = {kk: round(v, 2) for kk, v in rows.items()}
    rec = None
    # recall of the routed selections against the dense indexer on the same inputs (no target)
    if not wl.prefill:
        wl.step(0)
        M.dsa_index_dense(q, w, ks[0], q_seq, q_len, topk, idx=didx, score=dsc, ws=ws_dense)
        routed = torch.empty_like(idx)
        M.score_topk(q, w, ks[0], heads, q_seq, q_len, topk, idx=routed, want_score=False, ws=ws_score)
        torch.cuda.synchronize()
        dn, fi, ro = didx.cpu().numpy(), idx.cpu().numpy(), routed.cpu().numpy()
        recall = lambda a: float(np.mean([len(np.intersect1d(a[t], dn[t])) / topk for t in range(T)]))
        rec = {"misa": round(recall(ro), 4)}
        if wl.hier:
            rec["misa_hier"] = round(recall(fi), 4)
        M.block_indexer(q, w, ks[0], kbars[0], q_seq, q_len, B, h, m_blk, topk, idx=bidx, want_score=False,
                        ws=ws_blk)
        torch.cuda.synchronize()
        rec[f"block_filter_m{m_blk}"] = round(recall(bidx.cpu().numpy()), 4)
        if pv:
            G_pv, kc_pv, pidx, ws_pv = pv
            M.pivot_indexer(q, w, ks[0], q_seq, q_len, G_pv, kc_pv, topk, idx=pidx, want_score=False, ws=ws_pv)
            torch.cuda.synchronize()
            rec[f"pivot_G{G_pv}"] = round(recall(pidx.cpu().numpy()), 4)
    return rows, rec


def cpu_baseline(x, c, hier, prefill):
    """The fp64 NumPy oracle, as it stands, on the host cores: the headline
    workload on a bounded sample with every core the process may use, and
    1-thread runs of the tiny, DeepSeek-V3.2-like and GLM-5-like decode
    workloads on bounded samples."""
    from oracle import misa_oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits

    from routed_token_indexer_amd.workloads import make_inputs

    cores = len(os.sched_getaffinity(0))
    np.ones((2, 2)) @ np.ones((2, 2))            # load the BLAS library before asking about it
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    blas_info = {"vendor": blas[0].get("internal_api") if blas else None,
                 "version": blas[0].get("version") if blas else None,
                 "threads": max(i.get("num_threads", 1) for i in blas) if blas else None}

    def run(xx, cc, qs, budget_s, max_runs):
        tokens = int(sum(int(xx.q_len[t]) for t in qs))
        t0 = time.perf_counter()
        runs, best = 0, float("inf")
        while runs < max_runs and (runs == 0 or (time.perf_counter() - t0) < budget_s):
            t1 = time.perf_counter()
            if cc.kc:
                O.misa_hier_indexer(xx.q, xx.w, xx.k, xx.q_seq, xx.q_len, cc.B, cc.h, cc.kc, cc.topk, queries=qs)
            else:
                O.misa_indexer(xx.q, xx.w, xx.k, xx.q_seq, xx.q_len, cc.B, cc.h, cc.topk, queries=qs)
            best = min(best, time.perf_counter() - t1)
            runs += 1
        return tokens, best, runs

    qs = [c.T - 1 - 64 * i for i in range(4)] if prefill else list(range(c.T))   # prefill: the longest prefixes
    tokens, best, runs = run(x, c, qs, 30.0, 3)
    res = {
        "value": round(tokens / best / 1e9, 6), "unit": "Gtokens/s", "cores": cores, "kind": "oracle",
        "sample": f"{len(qs)} queries ({tokens} prefix tokens) of the same workload; fp64 NumPy oracle, "
                  f"{'route+score+top-k+re-rank' if hier else 'route+score+top-k'}, best of {runs} runs "
                  f"({best:.2f} s each), BLAS on every core the process may use",
        "ms_per_query": round(best * 1e3 / len(qs), 2),
        "blas": blas_info,
    }
    one = {}
    with threadpool_limits(limits=1, user_api="blas"):
        for name, nq in (("c0", 16), ("c1", 1), ("c3", 1)):
            xx = make_inputs(name, mode="gauss")
            tk, bt, rn = run(xx, xx.cfg, list(range(nq)), 5.0, 3)
            one[name] = {"gtokens_per_s": round(tk / bt / 1e9, 6), "ms_per_query": round(bt * 1e3 / nq, 2),
                         "sample": f"{nq} quer{'y' if nq == 1 else 'ies'}, best of {rn}"}
            del xx
    res["one_thread"] = one
    return res


if __name__ == "__main__":
    main()

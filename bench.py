#!/usr/bin/env python3
"""Benchmark of the DSA lightning indexer + IndexShare + sparse MLA hot path on one MI355X.

One step = one IndexShare group over one batch of synthetic input: the full
layer's indexer score and top-2048, then absorbed sparse MLA for that layer and
its 3 shared layers (4 layers). Default workload: decode, 64 sequences x 131072
cached tokens, one query per sequence (bf16 indexer, bf16 latent cache).

Prints ONE JSON line. `value` is query-tokens/s over the timed steps, inputs
resident in HBM. `roofline` covers the dominant kernel (the indexer score):
algorithmic bytes per launch / its average launch time from HIP events on the
launch stream. `cpu_baseline` times the CPU oracle on a bounded sample.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--workload NAME]
    python bench.py --calibrate-copy     # plain 1 GiB device copy, for counter scaling
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

import long_context_sparse_02_amd as gsa
import workloads as W

METRIC = "query-tokens/s via indexer+top-2048+sparse MLA at 128K/1M; % of roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
SCALE = 1.0 / 16.0           # 1/sqrt(QK dim 256)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def score_bytes(wl, fp8):
    """Algorithmic HBM bytes of one indexer-score launch: every causal key once
    per sequence (queries of a sequence share it) + q + w."""
    key_row = (128 + 4) if fp8 else 256
    q_bytes = wl.n_q * (32 * 128 * (1 if fp8 else 2) + (32 * 4 if fp8 else 0) + 32 * 4)
    return wl.batch * wl.n_ctx * key_row + q_bytes


def mla_bytes(wl):
    """Per layer: gathered rows + indices + q_lat/q_rope + fp32 output (per query)."""
    return wl.n_q * (2048 * 1152 + 2048 * 4 + 64 * 576 * 2 + 64 * 512 * 4)


HERE = os.path.dirname(os.path.abspath(__file__))
SCORE_SOURCES = ("long_context_sparse_02_amd/csrc/indexer_score.hip", "long_context_sparse_02_amd/csrc/device_common.h")


def measured_traffic(wl):
    """HBM bytes per indexer-score launch from the committed counter summary of
    this workload (FETCH_SIZE and WRITE_SIZE passes, copy-calibrated), or None
    when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(HERE, "profiles", f"indexer_score_{wl.name}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    t = re.search(r"^traffic_bytes_per_launch:\s*(\d+)", text, re.M)
    h = re.search(r"^sources_sha256:\s*([0-9a-f]{64})", text, re.M)
    if not t or not h:
        return None
    sha = hashlib.sha256()
    for f in SCORE_SOURCES:
        with open(os.path.join(HERE, f), "rb") as fh:
            sha.update(fh.read())
    return int(t.group(1)) if sha.hexdigest() == h.group(1) else None


def build_inputs(wl, seed, dev):
    t0 = time.time()
    q_seq, q_pos = W.query_layout(wl, dev)
    q_idx, w = W.indexer_queries(wl, seed, 0, dev)
    k_idx = W.indexer_keys(wl, seed, 0, dev)
    fp8 = wl.indexer_dtype == "fp8"
    q_scale = k_scale = None
    if fp8:
        q_idx, q_scale = gsa.quantize_e4m3(q_idx)
        k_idx8, k_scale = gsa.quantize_e4m3(k_idx)
        del k_idx
        k_idx = k_idx8
    layers = []
    if wl.mla:
        for l in range(wl.n_layers):
            q_lat, q_rope = W.mla_queries(wl, seed, l, dev)
            layers.append((q_lat, q_rope, W.mla_cache(wl, seed, l, dev)))
    torch.cuda.synchronize()
    log(f"[bench] inputs for {wl.name} generated in {time.time() - t0:.1f}s")
    return dict(q_seq=q_seq, q_pos=q_pos, q_idx=q_idx, w=w, k_idx=k_idx, q_scale=q_scale,
                k_scale=k_scale, layers=layers, fp8=fp8)


def run_bench(args):
    wl = W.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    inp = build_inputs(wl, args.seed, dev)
    ld = (wl.n_ctx + 3) // 4 * 4
    scores = torch.empty((wl.n_q, ld), dtype=torch.float32, device=dev)
    idx = torch.empty((wl.n_q, 2048), dtype=torch.int32, device=dev)
    ws = torch.empty(max(gsa.group_workspace_bytes(wl.n_q, ld), 16), dtype=torch.uint8, device=dev)
    outs = [(torch.empty((wl.n_q, 64, 512), dtype=torch.float32, device=dev),
             torch.empty((wl.n_q, 64), dtype=torch.float32, device=dev)) for _ in inp["layers"]]

    def step(ev=None):
        # same kernels, order and stream as gsa_indexshare_group; events bracket each call
        if ev is not None:
            ev[0].record()
        gsa.indexer_score(inp["q_idx"], inp["w"], inp["k_idx"], inp["q_seq"], inp["q_pos"],
                          q_scale=inp["q_scale"], k_scale=inp["k_scale"], scores=scores)
        if ev is not None:
            ev[1].record()
        gsa.topk(scores, inp["q_pos"], idx=idx, workspace=ws)
        if ev is not None:
            ev[2].record()
        for (ql, qr, kv), (o, s) in zip(inp["layers"], outs):
            gsa.sparse_mla_attn(ql, qr, kv, inp["q_seq"], idx, SCALE, out=o, lse=s, workspace=ws)
        if ev is not None:
            ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        step(evs[i])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    score_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    topk_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    mla_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs])) if inp["layers"] else 0.0
    value = wl.n_q / (ms_step / 1e3)
    sb = score_bytes(wl, inp["fp8"])
    achieved = sb / (score_ms / 1e3) / 1e9
    log(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step (wall {wall / args.steps * 1e3:.3f}); "
        f"score {score_ms:.3f} ms, top-k {topk_ms:.3f} ms, {len(outs)}x MLA {mla_ms:.3f} ms")
    mla_gbs = (mla_bytes(wl) * len(outs)) / (mla_ms / 1e3) / 1e9 if mla_ms > 0 else None
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if inp["fp8"] else "bf16",
        "data": "synthetic (seeded; integer indexer q/k in [-4,4], w in [1,4]; N(0,1) bf16 latents)",
        "config": {"workload": wl.name, "batch": wl.batch, "context": wl.n_ctx,
                   "queries": wl.n_q, "layers_per_step": len(outs) if wl.mla else 0,
                   "indexer": wl.indexer_dtype, "topk": 2048, "mla_heads": 64, "seed": args.seed},
        "breakdown_ms": {"indexer_score": round(score_ms, 4), "topk": round(topk_ms, 4),
                         "sparse_mla_all_layers": round(mla_ms, 4)},
        "roofline": {"kernel": "indexer_score", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(wl), "traffic_unit": "HBM bytes per launch (rocprofv3 counters)",
                     "bytes_per_launch": sb, "avg_launch_ms": round(score_ms, 4)},
        "mla_achieved_GBs": None if mla_gbs is None else round(mla_gbs, 1),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, inp, args)
    return result


def cpu_baseline(wl, inp, args):
    """The CPU oracle on a bounded sample of the same workload: the full group
    (score over every causal key, top-2048, then 4 layers of sparse MLA) for
    the first `--cpu-queries` queries. Host copies are made before timing."""
    import oracle                                  # test infrastructure: baseline leg only
    n = min(args.cpu_queries, wl.n_q)
    threads = len(os.sched_getaffinity(0))
    torch.set_num_threads(threads)
    qs = inp["q_seq"][:n].cpu().numpy()
    qp = inp["q_pos"][:n].cpu().numpy()
    if inp["fp8"]:
        raise SystemExit("cpu baseline for the fp8 workload is not wired in bench.py")
    q = inp["q_idx"][:n].float().cpu().numpy()
    w = inp["w"][:n].cpu().numpy()
    seqs = sorted(set(int(s) for s in qs))
    remap = {s: i for i, s in enumerate(seqs)}
    keys = np.stack([inp["k_idx"][s].float().cpu().numpy() for s in seqs])
    qs_local = np.array([remap[int(s)] for s in qs])
    t0 = time.perf_counter()
    sc = oracle.indexer_score(q, w, keys, qs_local, qp)
    sel = oracle.topk_select(sc, qp, 2048)
    t_sel = time.perf_counter() - t0
    # the oracle attends over the rows its own indices select; fetch just those rows
    t_mla = 0.0
    for (ql, qr, kv) in inp["layers"]:
        rows = np.zeros((n, 2048, 576), np.float32)
        for i in range(n):
            v = sel[i] >= 0
            rows[i, v] = kv[int(qs[i])][torch.from_numpy(sel[i][v]).to(kv.device).long()].float().cpu().numpy()
        local_idx = np.where(sel >= 0, np.arange(2048)[None, :], -1)
        qln, qrn = ql[:n].float().cpu().numpy(), qr[:n].float().cpu().numpy()
        t1 = time.perf_counter()
        for i in range(n):
            oracle.sparse_mla(qln[i:i + 1], qrn[i:i + 1], rows[i:i + 1], [0], local_idx[i:i + 1], SCALE)
        t_mla += time.perf_counter() - t1
    secs = t_sel + t_mla
    log(f"[bench] oracle: {n} queries in {secs:.2f}s (score+top-k {t_sel:.2f}s, MLA {t_mla:.2f}s) on {threads} threads")
    return {"value": round(n / secs, 3), "unit": "query-tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {wl.n_q} queries of {wl.name}: full group (score over all causal keys, "
                      f"top-2048, {len(inp['layers'])} layers of sparse MLA); host copies untimed",
            "seconds": round(secs, 3)}


def calibrate_copy(args):
    """A plain device copy of known size, run under rocprofv3 --pmc to scale
    FETCH_SIZE / WRITE_SIZE readings to bytes."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(args.steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "launches": args.steps}))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--workload", default="decode_b64_n131072", choices=sorted(W.WORKLOADS))
    ap.add_argument("--cpu-queries", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (this path is measured on a single MI355X); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    gsa.lib()                     # fail loudly if the HIP library is missing
    if args.calibrate_copy:
        calibrate_copy(args)
        return
    res = run_bench(args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the DSA lightning indexer + IndexShare + sparse MLA hot path on one MI355X.

One step = one pass of the measured unit over one batch of synthetic input,
issued as the C-ABI boundary call that runs it:
  group workloads   gsa_indexshare_group: the full layer's indexer score and
                    top-2048, then absorbed sparse MLA for it and its 3 shared
                    layers (4 layers);
  prefill workloads gsa_indexshare_group with no attention layers: the full
                    layer's indexer score and top-2048 (index buffer written);
  stack workloads   gsa_layer_stack: 21 full layers (score + top-2048 each) and
                    78 sparse MLA layers, in layer order.

By default every configuration is measured in turn (tiny group, decode 64 x
128K, prefill 4096 x 128K bf16 and fp8, decode 8 x 1M fp8, the 78-layer stack),
each one's inputs freed before the next. The headline fields of the ONE JSON
line are the decode 64 x 128K group's; `workloads` holds every configuration's
line. Per configuration:
  ms_per_step / value  the boundary call timed whole (HIP events around the
                       timed steps on the launch stream; inputs resident in HBM);
  step_roofline        the step's algorithmic bytes (or the score's matrix work,
                       for prefill) against the HBM (or MFMA) peak;
  roofline             the kernel with the largest share of the step, from a
                       separate pass that issues the same kernels as separate
                       calls with HIP events between them;
  cpu_baseline         the CPU oracle on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload NAME[,NAME...]]
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
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}   # MI355X dense matrix peaks
SCALE = 1.0 / 16.0           # 1/sqrt(QK dim 256)
HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = "long_context_sparse_02_amd/csrc/"
KERNEL_SOURCES = {
    "indexer_score": (CSRC + "indexer_score.hip", CSRC + "device_common.h"),
    "topk": (CSRC + "topk.hip", CSRC + "device_common.h"),
    "sparse_mla": (CSRC + "sparse_mla.hip", CSRC + "device_common.h"),
    "quantize_q": (CSRC + "quantize_e4m3.hip", CSRC + "device_common.h"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def is_stack(wl):
    return wl.mla and wl.n_layers > 4


# ---- algorithmic bytes per launch ---------------------------------------------
def score_bytes(wl, fp8):
    """One indexer-score launch: every causal key once per sequence (the queries
    of a sequence share it) + q + w (+ scales)."""
    key_row = (128 + 4) if fp8 else 256
    q_bytes = wl.n_q * (32 * 128 * (1 if fp8 else 2) + (32 * 4 if fp8 else 0) + 32 * 4)
    return wl.batch * wl.n_ctx * key_row + q_bytes


def topk_bytes(wl):
    """One top-k launch: each query's causal scores read once + its indices written."""
    return causal_pairs(wl) * 4 + wl.n_q * 2048 * 4


def mla_bytes(wl):
    """One sparse-MLA layer: gathered rows (1152 B bf16, 656 B FP8) + indices +
    q_lat/q_rope + fp32 output."""
    row = 656 if wl.kv_dtype == "fp8" else 1152
    return wl.n_q * (2048 * row + 2048 * 4 + 64 * 576 * 2 + 64 * 512 * 4)


def score_flops(wl):
    """One indexer-score launch: 32 heads x 128-dim dot products (2 flops per
    multiply-add) for every causal (query, key) pair; the ReLU and the weighted
    head sum are not matrix work and are left out."""
    return causal_pairs(wl) * 32 * 128 * 2


def causal_pairs(wl):
    first = wl.n_ctx - wl.q_per_seq + 1                     # causal length of the first query
    return wl.batch * sum(first + j for j in range(wl.q_per_seq))


def indexer_topk_bytes(wl, fp8):
    """Score and top-k without a score buffer: the score's inputs + the indices written."""
    return score_bytes(wl, fp8) + wl.n_q * 2048 * 4


def launch_bytes(kind, wl, fp8):
    return {"indexer_score": lambda: score_bytes(wl, fp8), "topk": lambda: topk_bytes(wl),
            "indexer_topk": lambda: indexer_topk_bytes(wl, fp8),
            "sparse_mla": lambda: mla_bytes(wl)}[kind]()


def step_bytes(wl, n_full, n_att):
    """Algorithmic bytes of one step: every full layer's score inputs and index
    write, and every attention layer's gather, queries, indices and output (the
    score buffer between score and top-k is not algorithmic)."""
    fp8 = wl.indexer_dtype in ("fp8", "fp8h")
    return n_full * (score_bytes(wl, fp8) + wl.n_q * 2048 * 4) + n_att * mla_bytes(wl)


def measured_traffic(kind, wl):
    """HBM bytes per launch of `kind` from the committed counter summary of this
    workload (FETCH_SIZE and WRITE_SIZE passes, copy-calibrated), or None when
    there is none or the kernel sources changed since it was taken."""
    path = os.path.join(HERE, "profiles", f"{kind}_{wl.name}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    t = re.search(r"^traffic_bytes_per_launch:\s*(\d+)", text, re.M)
    h = re.search(r"^sources_sha256:\s*([0-9a-f]{64})", text, re.M)
    if not t or not h:
        return None
    sha = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(HERE, f), "rb") as fh:
            sha.update(fh.read())
    return int(t.group(1)) if sha.hexdigest() == h.group(1) else None


# ---- inputs and the step ----------------------------------------------------------
def build_inputs(wl, seed, dev):
    """Device inputs of the workload, drawn by the seeded generators in `workloads`."""
    t0 = time.time()
    q_seq, q_pos = W.query_layout(wl, dev)
    fp8 = wl.indexer_dtype in ("fp8", "fp8h")
    rot = wl.indexer_dtype == "fp8h"           # Hadamard-rotated fp8: the step quantises q
    if is_stack(wl):
        src = gsa.layer_pattern(wl.n_layers)
    else:                                      # one group: layer 0 full, the rest shared
        src = [0] * (wl.n_layers if wl.mla else 1)
    full_layers = [l for l, s in enumerate(src) if s == l]
    indexers = []
    q_src = []                                 # bf16 indexer queries the step quantises (fp8h)
    for f in full_layers:
        q_idx, w = W.indexer_queries(wl, seed, f, dev)
        k_idx = W.indexer_keys(wl, seed, f, dev)
        q_scale = k_scale = None
        q_bf16 = q_idx
        if fp8:
            q_idx, q_scale = gsa.quantize_e4m3(q_idx, hadamard=rot)
            k8, k_scale = gsa.quantize_e4m3(k_idx, hadamard=rot)
            del k_idx
            k_idx = k8
        indexers.append((q_idx, w, k_idx, q_scale, k_scale))
        if rot:
            q_src.append(q_bf16)
    layers = []
    if wl.mla:
        for l in range(wl.n_layers):
            q_lat, q_rope = W.mla_queries(wl, seed, l, dev)
            kv = W.mla_cache(wl, seed, l, dev)
            if wl.kv_dtype == "fp8":                   # the cache is kept quantised
                kv8 = gsa.quantize_latent_fp8(kv)
                del kv
                kv = kv8
            layers.append((q_lat, q_rope, kv))
    torch.cuda.synchronize()
    log(f"[bench] inputs for {wl.name} generated in {time.time() - t0:.1f}s "
        f"({len(full_layers)} full layers, {len(layers)} attention layers)")
    ordinal = {f: j for j, f in enumerate(full_layers)}
    return dict(q_seq=q_seq, q_pos=q_pos, indexers=indexers, full_layers=full_layers,
                src=[ordinal[s] for s in src], layers=layers, fp8=fp8, rot=rot, q_src=q_src)


def make_step(wl, inp, dev, score_buffer=True):
    """The measured unit as the sequence of library calls gsa_indexshare_group /
    gsa_layer_stack make (same kernels, order and stream): per group the full
    layer's score and top-k (score_buffer=False: one gsa_indexer_topk call, the
    selection without a score buffer), then one attention launch over the
    group's layers. Events can be recorded between the calls. Returns (step, buffers, calls):
    step(evs) records evs[i] before call i and evs[-1] after the last; calls is
    [(kind, algorithmic bytes)] per call."""
    ld = (wl.n_ctx + 3) // 4 * 4
    n_full = len(inp["full_layers"])
    n_att = len(inp["layers"])
    # the largest group this step runs decides the workspace (a group of fewer
    # layers may split its queries further and need more attention partials)
    sizes = {sum(1 for l in range(n_att) if inp["src"][l] == j) for j in range(n_full)} or {1}
    ws_bytes = max(gsa.group_workspace_bytes(wl.n_q, ld, max(g, 1)) for g in sizes)
    bufs = dict(
        scores=torch.empty((wl.n_q, ld), dtype=torch.float32, device=dev),
        gmax=torch.empty((wl.n_q, gsa.group_max_ld(ld)), dtype=torch.float32, device=dev),
        idx=torch.empty((n_full, wl.n_q, 2048), dtype=torch.int32, device=dev),
        ws=torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev),
        outs=[(torch.empty((wl.n_q, 64, 512), dtype=torch.float32, device=dev),
               torch.empty((wl.n_q, 64), dtype=torch.float32, device=dev)) for _ in inp["layers"]])
    calls = []                                  # (kind, bytes, fn)
    q_seq, q_pos = inp["q_seq"], inp["q_pos"]

    def score_call(j):
        q, w, k, qs, ks = inp["indexers"][j]
        return lambda: gsa.indexer_score(q, w, k, q_seq, q_pos, q_scale=qs, k_scale=ks,
                                         scores=bufs["scores"], group_max=bufs["gmax"])

    def indexer_topk_call(j):
        q, w, k, qs, ks = inp["indexers"][j]
        return lambda: gsa.indexer_topk(q, w, k, q_seq, q_pos, q_scale=qs, k_scale=ks, idx=bufs["idx"][j],
                                        workspace=bufs["ws"])

    def topk_call(j):
        return lambda: gsa.topk(bufs["scores"], q_pos, idx=bufs["idx"][j], workspace=bufs["ws"],
                                group_max=bufs["gmax"])

    def mla_call(j, layers):
        lay = [inp["layers"][l] for l in layers]
        outs = [bufs["outs"][l] for l in layers]
        return lambda: gsa.sparse_mla_attn_layers(lay, q_seq, bufs["idx"][j], SCALE, outs=outs,
                                                  workspace=bufs["ws"])

    def quant_call(j):
        q, _, _, qs, _ = inp["indexers"][j]
        return lambda: gsa.quantize_e4m3(inp["q_src"][j], hadamard=True, out=(q, qs))

    fp8 = inp["fp8"]
    for j, f in enumerate(inp["full_layers"]):
        if inp["rot"]:                          # rotate + quantise this step's indexer queries
            calls.append(("quantize_q", wl.n_q * 32 * (256 + 128 + 4), quant_call(j)))
        if score_buffer:
            calls.append(("indexer_score", launch_bytes("indexer_score", wl, fp8), score_call(j)))
            calls.append(("topk", launch_bytes("topk", wl, fp8), topk_call(j)))
        else:
            calls.append(("indexer_topk", launch_bytes("indexer_topk", wl, fp8), indexer_topk_call(j)))
        group = [l for l in range(n_att) if inp["src"][l] == j]
        if group:
            calls.append(("sparse_mla", launch_bytes("sparse_mla", wl, fp8) * len(group), mla_call(j, group)))

    def step(evs=None):
        for i, (_, _, fn) in enumerate(calls):
            if evs is not None:
                evs[i].record()
            fn()
        if evs is not None:
            evs[-1].record()

    return step, bufs, [(k, b) for k, b, _ in calls]


def make_boundary_step(wl, inp, bufs, score_buffer=True):
    """The measured unit as the one boundary call that runs it, over the same
    buffers as make_step: gsa_indexshare_group (the group, or for prefill the
    full layer alone) or gsa_layer_stack. The descriptor is marshalled once.
    score_buffer=False: the full layers select without a score buffer."""
    q_seq, q_pos = inp["q_seq"], inp["q_pos"]
    lay = [inp["layers"][l] for l in range(len(inp["layers"]))]
    scores = bufs["scores"] if score_buffer else None
    if is_stack(wl):
        call = gsa.prepare_stack(inp["indexers"], lay, q_seq, q_pos, bufs["idx"], scores=scores,
                                 workspace=bufs["ws"], outs=bufs["outs"], scale=SCALE, score_buffer=score_buffer)
    else:
        q, w, k, qs, ks = inp["indexers"][0]
        call = gsa.prepare_group(lay, q_seq, bufs["idx"][0], q_pos=q_pos, q_idx=q, w=w, k_idx=k, q_scale=qs,
                                 k_scale=ks, scores=scores, workspace=bufs["ws"], outs=bufs["outs"],
                                 scale=SCALE, score_buffer=score_buffer)
    if not inp["rot"]:
        return call
    q, _, _, qs, _ = inp["indexers"][0]

    def step():                      # the rotated fp8 indexer quantises this step's queries first
        gsa.quantize_e4m3(inp["q_src"][0], hadamard=True, out=(q, qs))
        call()
    return step


def time_steps(fn, steps, warmup):
    """ms per call of fn over `steps` calls after `warmup`, from HIP events
    recorded on the current stream (the binding launches there)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    t0.record()
    for _ in range(steps):
        fn()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps, (time.perf_counter() - w0) * 1e3 / steps


def measure(wl, args, cpu_seconds):
    """One configuration: the boundary call timed whole, the per-kernel breakdown
    pass, the rooflines and the CPU oracle's sample. Frees its inputs on return."""
    dev = torch.device("cuda", 0)
    inp = build_inputs(wl, args.seed, dev)
    step_b, bufs, calls = make_step(wl, inp, dev, score_buffer=not args.no_score_buffer)
    whole = make_boundary_step(wl, inp, bufs, score_buffer=not args.no_score_buffer)
    # ---- pass A: the boundary call, timed whole
    ms_step, wall_ms = time_steps(whole, args.steps, args.warmup)
    idx_whole = bufs["idx"].clone()
    # ---- pass B: the same kernels as separate calls, events between them
    for _ in range(args.warmup):
        step_b()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    for i in range(args.steps):
        step_b(evs[i])
    torch.cuda.synchronize()
    same = bool(torch.equal(idx_whole, bufs["idx"]))
    kinds = sorted({k for k, _ in calls}, key=[k for k, _ in calls].index)
    ms_kind = {k: 0.0 for k in kinds}           # per step
    bytes_kind = {k: 0 for k in kinds}          # per step
    launches = {k: 0 for k in kinds}            # per step
    for i, (k, b) in enumerate(calls):
        ms_kind[k] += float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs]))
        bytes_kind[k] += b
        launches[k] += 1
    ms_split = float(np.mean([e[0].elapsed_time(e[-1]) for e in evs]))
    dom = max(ms_kind, key=ms_kind.get)
    fp8 = inp["fp8"]
    n_full, n_att = len(inp["full_layers"]), len(inp["layers"])
    log(f"[bench] {wl.name}: {ms_step:.4f} ms/step as one boundary call (host {wall_ms:.4f} ms/step); "
        f"as separate calls {ms_split:.4f} ms: " +
        ", ".join(f"{k} {launches[k]}x {ms_kind[k] / launches[k] * 1e3:.1f} us" for k in kinds) +
        ("" if same else "  [INDICES DIFFER BETWEEN THE TWO PASSES]"))
    res = {
        "ms_per_step": round(ms_step, 4),
        "value": round(wl.n_q / (ms_step / 1e3), 1),
        "unit": "query-tokens/s",
        "dtype": "fp8" if fp8 else "bf16",
        "config": {"workload": wl.name, "batch": wl.batch, "context": wl.n_ctx, "queries": wl.n_q,
                   "full_layers": n_full, "attention_layers": n_att, "indexer": wl.indexer_dtype,
                   "latent_cache": wl.kv_dtype, "topk": 2048, "mla_heads": 64, "seed": args.seed,
                   "step": "gsa_layer_stack" if is_stack(wl) else "gsa_indexshare_group",
                   "score_buffer": not args.no_score_buffer},
        "step_roofline": step_roofline(wl, fp8, n_full, n_att, ms_step),
        "roofline": roofline(dom, wl, fp8, bytes_kind[dom], ms_kind[dom], launches[dom]),
        "breakdown": {"ms_per_step_separate_calls": round(ms_split, 4),
                      "avg_launch_us": {k: round(ms_kind[k] / launches[k] * 1e3, 2) for k in kinds},
                      "launches_per_step": launches,
                      "achieved_GBs": {k: round(bytes_kind[k] / (ms_kind[k] / 1e3) / 1e9, 1) for k in kinds},
                      "indices_equal_to_boundary_call": same},
    }
    if cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(wl, inp, args, cpu_seconds)
    log(f"[bench] {wl.name}: {res['value']:.1f} q-tok/s; step {res['step_roofline']['frac']:.3f} of "
        f"{res['step_roofline']['bound']}; {dom} {res['roofline']['frac']:.3f} of {res['roofline']['bound']}")
    del inp, bufs, calls, step_b, whole, idx_whole
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def step_roofline(wl, fp8, n_full, n_att, ms):
    """The whole step against its bound: HBM for the decode and stack steps (all
    their algorithmic bytes at the HBM peak), MFMA for prefill (the score's matrix
    work at the peak of its input type; top-k and the index write ride along)."""
    sec = ms / 1e3
    if wl.mla:
        nb = step_bytes(wl, n_full, n_att)
        a = nb / sec / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4), "bytes_per_step": nb,
                "roofline_ms": round(nb / (HBM_PEAK_GBS * 1e9) * 1e3, 4)}
    fl = score_flops(wl) * n_full
    peak = MFMA_PEAK_TFLOPS["fp8" if fp8 else "bf16"]
    a = fl / sec / 1e12
    return {"bound": "mfma", "achieved": round(a, 1), "peak": peak, "unit": "TFLOP/s",
            "frac": round(a / peak, 4), "flops_per_step": fl,
            "roofline_ms": round(fl / (peak * 1e12) * 1e3, 4)}


def roofline(kind, wl, fp8, nbytes, ms, launches):
    """The bound of the dominant kernel: HBM unless its matrix work at the MFMA
    peak of its input type takes longer than its bytes at the HBM peak (the
    indexer score with thousands of queries per sequence)."""
    sec = ms / 1e3
    out = {"kernel": kind}
    flops = score_flops(wl) * launches if kind in ("indexer_score", "indexer_topk") else 0
    peak_tf = MFMA_PEAK_TFLOPS["fp8" if fp8 else "bf16"]
    if flops / (peak_tf * 1e12) > nbytes / (HBM_PEAK_GBS * 1e9):
        achieved = flops / sec / 1e12
        out.update({"bound": "mfma", "achieved": round(achieved, 1), "peak": peak_tf, "unit": "TFLOP/s",
                    "frac": round(achieved / peak_tf, 4), "flops_per_launch": flops // launches})
    else:
        achieved = nbytes / sec / 1e9
        out.update({"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4)})
    out.update({"traffic": measured_traffic(kind, wl),
                "traffic_unit": "HBM bytes per launch (rocprofv3 counters)",
                "bytes_per_launch": nbytes // launches, "avg_launch_ms": round(ms / launches, 4)})
    return out


# ---- the oracle on the host ---------------------------------------------------------
def host_indexer_inputs(wl, inp, j, qi, seed, keys=None):
    """Host copies of full layer j's indexer inputs for query qi: (q [1,32,128],
    w [1,32], keys [N,128]) as the oracle reads them. For the fp8 workload the
    original integer values are redrawn on the device (same generator, same
    values) and the oracle applies its own e4m3 block quantisation. `keys`, a
    dict, keeps each (layer, sequence)'s host keys for later queries."""
    import oracle
    b = int(inp["q_seq"][qi])
    q, w, k, _, _ = inp["indexers"][j]
    kh = None if keys is None else keys.get((j, b))
    if inp["fp8"]:
        f = inp["full_layers"][j]
        quant = oracle.quantize_blocks_hadamard if inp["rot"] else oracle.quantize_blocks
        qv, wv = W.indexer_queries(wl, seed, f, q.device)
        qh = oracle.dequantize_blocks(*quant(qv[qi:qi + 1].float().cpu().numpy()))
        if kh is None:
            kh = W.indexer_keys_seq(wl, seed, f, b, q.device).float().cpu().numpy()
            kh = oracle.dequantize_blocks(*quant(kh))
        wh = wv[qi:qi + 1].cpu().numpy()
    else:
        qh, wh = q[qi:qi + 1].float().cpu().numpy(), w[qi:qi + 1].cpu().numpy()
        if kh is None:
            kh = k[b].float().cpu().numpy()
    if keys is not None:
        keys[(j, b)] = kh
    return qh, wh, kh


def host_rows(kv, b, sel):
    """The latent rows `sel` (valid entries) of sequence b, fetched by torch's
    index_select on the device (FP8 rows dequantised by the oracle), and the
    local indices that address them. For the oracle-side callers only."""
    v = sel >= 0
    rows = np.zeros((len(sel), 576), np.float64)
    got = kv[b].index_select(0, torch.from_numpy(sel[v]).to(kv.device).long()).cpu()
    if kv.dtype == torch.uint8:
        import oracle                                  # test infrastructure: oracle-side helper
        rows[v] = oracle.dequantize_latent(got.numpy())
    else:
        rows[v] = got.float().numpy()
    return rows[None], np.where(v, np.arange(len(sel)), -1)[None]


def cpu_baseline(wl, inp, args, cpu_seconds):
    """The CPU oracle on a bounded sample of the same workload: the first
    `--cpu-queries` queries through the whole measured unit (every full
    layer's score over all causal keys and top-2048, then every attention
    layer over the oracle's own selection). Host copies are made untimed."""
    import oracle                                  # test infrastructure: baseline leg only
    threads = len(os.sched_getaffinity(0))
    torch.set_num_threads(threads)
    secs = 0.0
    n = 0
    keys = {}
    for qi in range(min(args.cpu_queries, wl.n_q)):
        if secs >= cpu_seconds:
            break
        n += 1
        b = int(inp["q_seq"][qi])
        pos = np.array([int(inp["q_pos"][qi])], np.int32)
        sels = []
        for j in range(len(inp["full_layers"])):
            qh, wh, kh = host_indexer_inputs(wl, inp, j, qi, args.seed, keys)
            t0 = time.perf_counter()
            sc = oracle.indexer_score(qh, wh, kh[None], np.zeros(1, np.int32), pos)
            sels.append(oracle.topk_select(sc, pos, 2048)[0])
            secs += time.perf_counter() - t0
        for l, (ql, qr, kv) in enumerate(inp["layers"]):
            rows, local = host_rows(kv, b, sels[inp["src"][l]])
            qln = ql[qi:qi + 1].float().cpu().numpy()
            qrn = qr[qi:qi + 1].float().cpu().numpy()
            t0 = time.perf_counter()
            oracle.sparse_mla(qln, qrn, rows, np.zeros(1, np.int32), local, SCALE)
            secs += time.perf_counter() - t0
    log(f"[bench] oracle: {n} queries in {secs:.2f}s on {threads} threads")
    return {"value": round(n / secs, 3), "unit": "query-tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {wl.n_q} queries of {wl.name} through the whole unit "
                      f"({len(inp['full_layers'])} x score over all causal keys + top-2048, "
                      f"{len(inp['layers'])} x sparse MLA); host copies untimed",
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


DEFAULT_SET = ["group_b1_n4096_q4", "decode_b64_n131072", "prefill_q4096_n131072", "prefill_q4096_n131072_fp8",
               "decode_b8_n1048576_fp8", "stack78_b8_q8_n262144"]
HEADLINE = "decode_b64_n131072"


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--workload", default=",".join(DEFAULT_SET),
                    help="comma-separated workloads (the first one in the list that is the 64 x 128K decode "
                         "group, else the first, gives the headline fields); choices: " + ", ".join(W.WORKLOADS))
    ap.add_argument("--cpu-queries", type=int, default=1 << 30, help="most queries in each CPU sample")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="oracle seconds for the headline workload's CPU sample (it stops at the first query "
                         "that starts past this much oracle time)")
    ap.add_argument("--cpu-seconds-other", type=float, default=3.0,
                    help="the same for every other workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--no-score-buffer", action="store_true",
                    help="full layers select without a score buffer (score + top-k as gsa_indexer_topk)")
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
    names = [n for n in args.workload.split(",") if n]
    for n in names:
        if n not in W.WORKLOADS:
            ap.error(f"unknown workload {n}")
    head = HEADLINE if HEADLINE in names else names[0]
    torch.cuda.set_device(0)
    t0 = time.perf_counter()
    per = {}
    for n in names:
        secs = 0.0 if args.no_cpu_baseline else (args.cpu_seconds if n == head else args.cpu_seconds_other)
        per[n] = measure(W.WORKLOADS[n], args, secs)
        log(f"[bench] {n} done ({time.perf_counter() - t0:.1f}s since start)")
    h = per[head]
    result = {
        "metric": METRIC,
        "value": h["value"],
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": h["dtype"],
        "data": "synthetic (seeded; integer indexer q/k in [-4,4], w in [1,4]; N(0,1) bf16 latents)",
        "config": h["config"],
        "step_roofline": h["step_roofline"],
        "roofline": h["roofline"],
        "breakdown": h["breakdown"],
    }
    if "cpu_baseline" in h:
        result["cpu_baseline"] = h["cpu_baseline"]
    result["workloads"] = per
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

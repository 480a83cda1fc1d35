"""Throughput of routed block-sparse attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload video|nsa|msa|reweight|coarse|h3|reblock]
                    [--no-cpu-baseline]

A step is one pass of the routed block-sparse attention hot path over one
batch of synthetic input already resident in HBM:

  video  (default) tiling tables -> per-block mean pooling -> routing scores ->
         TopK index table -> exact block-sparse attention, on the video-DiT
         workload (115200 tokens = 30x48x80 grid in 4x4x4 blocks, 24 heads,
         D=128, keep 192 of 1920 blocks).
  nsa    NSA selected-branch attention (32768 tokens, 64 query / 4 KV heads,
         blocks of 64, up to 16 selected), query-outer.
  msa    KV-outer schedule + combine (65536 tokens, 64 query / 4 KV heads,
         KV blocks of 128, 16 selected blocks).
  reweight  the video step with Spark-Reweight: block summaries from the mean
         query of each head, and attention over the kept blocks plus one
         virtual token for each of the other 1728 blocks.
  h3     an H3 reference-to-video sequence (text 256, reference video
         8x48x80, audio 500, target video 30x48x80; 146676 tokens, J = 2412):
         multi-region tables -> pooling -> grouped routing (context rows
         dense, video rows keep the prefix + 10 % of each video region) ->
         exact attention over the union.
  reblock the video step on Spark-Reblock layouts: per head the query-side
         second moment, key features and an equal-capacity tree of 64-token
         leaves, then pool/route/TopK and attention over the per-head tables.
  coarse the video step with the coarse pooled-V branch: the routing scores
         are kept, V is pooled, C = softmax(E) V_bar over all 1920 blocks,
         and the attention epilogue adds gate * C to every token.

Prints one JSON line.  ``value`` is the effective attention throughput of the
whole step, 4*h*N*D*k*M / step time (the pages' FLOP count), in TFLOP/s.
``roofline`` describes the dominant kernel, timed with HIP events on the
stream it is launched on.  ``cpu_baseline`` times the float64 oracle on a
bounded sample of the same workload on the host cores.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "block-sparse attn effective TFLOP/s + ms/layer at 1 GPU; % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E (published)


def _profiled_traffic(profile, sources):
    """HBM bytes per launch recorded in a committed profile summary, or None
    when the kernel sources have changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            k_, v_ = line.split(":", 1)
            fields[k_.strip()] = v_.strip()
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "block_sparse_attention_02_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if fields.get("source_sha256") != h.hexdigest() or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def bench_video(args):
    import torch
    import block_sparse_attention_02_amd as bsa
    from workloads import vsa_inputs, workload

    cfg = workload("video")
    dev = torch.device("cuda:0")
    T, H, W = cfg["grid"]
    B, h, D, R = cfg["B"], cfg["h"], cfg["D"], cfg["R"]
    N = T * H * W
    x = vsa_inputs(cfg, device=dev)
    q, k, v = x["q"], x["k"], x["v"]
    J, M = bsa.tile_dims(T, H, W, *cfg["block"])
    perm = torch.empty(J * M, dtype=torch.int32, device=dev)
    block_len = torch.empty(J, dtype=torch.int32, device=dev)
    inv = torch.empty(N, dtype=torch.int32, device=dev)
    q2k_idx = torch.empty((B, h, J, R), dtype=torch.int32, device=dev)
    q2k_num = torch.empty((B, h, J), dtype=torch.int32, device=dev)
    order = torch.empty((B, h, J), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    ws = torch.empty(bsa.route_workspace_bytes(q, J, M, R), dtype=torch.uint8, device=dev)

    L = bsa._lib
    lib = L.load()
    stream = torch.cuda.current_stream(dev)
    s_ptr = bsa.api._stream(dev)

    import ctypes
    def tile():
        L.check(lib.vsa_tile_index(T, H, W, *cfg["block"], bsa.api._ptr(perm), bsa.api._ptr(block_len),
                                   bsa.api._ptr(inv), s_ptr))

    ra = bsa.api._route_args(q, k, perm, block_len, J, M, R, R, 1.0 / D ** 0.5, q2k_idx, q2k_num, None, None, None,
                             order)
    nws = ws.numel()

    def route():
        L.check(lib.vsa_pool_route_topk(ctypes.byref(ra), bsa.api._ptr(ws), nws, s_ptr))

    qa = bsa.api._qouter_args(q, k, v, out, 1.0 / D ** 0.5, L.BSA_SEL_BLOCK, None)
    qa.perm, qa.block_len, qa.J, qa.M = bsa.api._ptr(perm), bsa.api._ptr(block_len), J, M
    qa.q2k_idx, qa.q2k_num, qa.kmax = bsa.api._ptr(q2k_idx), bsa.api._ptr(q2k_num), R
    qa.item_order = bsa.api._ptr(order)

    qws = bsa.qouter_workspace(dev)

    def attend():
        L.check(lib.bsa_forward_qouter(ctypes.byref(qa), bsa.api._ptr(qws), qws.numel(), s_ptr))

    ev = {n: [_events() for _ in range(args.steps)] for n in ("tile", "route", "attn")}

    def step(i=None):
        for name, fn in (("tile", tile), ("route", route), ("attn", attend)):
            if i is not None:
                ev[name][i][0].record(stream)
            fn()
            if i is not None:
                ev[name][i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    ms = {n: sum(a.elapsed_time(b) for a, b in ev[n]) / args.steps for n in ev}

    flops = 4.0 * B * h * N * D * R * M             # nominal, the pages' formula
    pairs = bsa.metrics.vsa_valid_pairs(block_len, q2k_idx, q2k_num)
    valid_flops = 4.0 * D * pairs
    attn_tflops = flops / (ms["attn"] * 1e-3) / 1e12
    # pool/route/TopK algorithmic bytes: read Q and K once, write pooled means and the index table
    route_bytes = 2 * q.numel() * q.element_size() + 2 * B * h * J * D * 4 + B * h * J * (R + 1) * 4
    res = {
        "metric": METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) + per-cell offsets, no dataset or weights)",
        "config": {"workload": "video_dit_vsa", "B": B, "heads": h, "grid": list(cfg["grid"]),
                   "block": list(cfg["block"]), "D": D, "J": J, "M": M, "R": R, "tokens": N},
        "ms": {k_: round(v_, 4) for k_, v_ in ms.items()},
        "attn_tflops_nominal": round(attn_tflops, 2),
        "attn_tflops_valid": round(valid_flops / (ms["attn"] * 1e-3) / 1e12, 2),
        "pct_bf16_peak_attn": round(100 * attn_tflops / PEAK_BF16_TFLOPS, 2),
        "route_gbps": round(route_bytes / (ms["route"] * 1e-3) / 1e9, 1),
        "pct_hbm_route": round(100 * route_bytes / (ms["route"] * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
        "roofline": {"kernel": "vsa4_kernel (bsa_forward_qouter, block mode)", "bound": "mfma",
                     "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": _profiled_traffic("vsa4_kernel_video.md",
                                                  ("attn_vsa.hip", "bsa_device.hpp", "bsa_internal.hpp"))},
    }
    ctx = dict(cfg=cfg, x=x, perm=perm, block_len=block_len, q2k_idx=q2k_idx, q2k_num=q2k_num, J=J, M=M)
    return res, ctx


def bench_reweight(args):
    """Video workload with Spark-Reweight: tiling + pool/route/TopK, block
    summaries, and attention over the kept blocks plus one virtual token per
    other block, under one softmax."""
    import ctypes
    import torch
    import block_sparse_attention_02_amd as bsa
    from workloads import vsa_inputs, workload

    cfg = workload("video")
    dev = torch.device("cuda:0")
    T, H, W = cfg["grid"]
    B, h, D, R = cfg["B"], cfg["h"], cfg["D"], cfg["R"]
    N = T * H * W
    x = vsa_inputs(cfg, device=dev)
    q, k, v = x["q"], x["k"], x["v"]
    J, M = bsa.tile_dims(T, H, W, *cfg["block"])
    perm = torch.empty(J * M, dtype=torch.int32, device=dev)
    block_len = torch.empty(J, dtype=torch.int32, device=dev)
    q2k_idx = torch.empty((B, h, J, R), dtype=torch.int32, device=dev)
    q2k_num = torch.empty((B, h, J), dtype=torch.int32, device=dev)
    order = torch.empty((B, h, J), dtype=torch.int32, device=dev)
    k_sum = torch.empty((B, h, J, D), dtype=torch.bfloat16, device=dev)
    v_sum = torch.empty((B, h, J, D), dtype=torch.bfloat16, device=dev)
    b_sum = torch.empty((B, h, J), dtype=torch.float32, device=dev)
    out = torch.empty_like(q)
    ws = torch.empty(bsa.route_workspace_bytes(q, J, M, R), dtype=torch.uint8, device=dev)
    L = bsa._lib
    lib = L.load()
    stream = torch.cuda.current_stream(dev)
    s_ptr = bsa.api._stream(dev)
    P = bsa.api._ptr

    def tile():
        L.check(lib.vsa_tile_index(T, H, W, *cfg["block"], P(perm), P(block_len), None, s_ptr))

    ra = bsa.api._route_args(q, k, perm, block_len, J, M, R, R, 1.0 / D ** 0.5, q2k_idx, q2k_num, None, None, None,
                             order)

    def route():
        L.check(lib.vsa_pool_route_topk(ctypes.byref(ra), P(ws), ws.numel(), s_ptr))

    sa = L.SummaryArgs(q=P(q), k=P(k), v=P(v), d=bsa.api._desc(k), dt=L.BSA_BF16, perm=P(perm),
                       block_len=P(block_len), J=J, M=M, scale=1.0 / D ** 0.5, anchor=None, anchor_out=None,
                       k_sum=P(k_sum), v_sum=P(v_sum), b_sum=P(b_sum))
    nsw = ctypes.c_size_t(0)
    L.check(lib.spark_summaries_ws(ctypes.byref(sa), ctypes.byref(nsw)))
    sws = torch.empty(max(1, nsw.value), dtype=torch.uint8, device=dev)

    def summarise():
        L.check(lib.spark_summaries(ctypes.byref(sa), P(sws), nsw.value, s_ptr))

    qa = bsa.api._qouter_args(q, k, v, out, 1.0 / D ** 0.5, L.BSA_SEL_BLOCK, None)
    qa.perm, qa.block_len, qa.J, qa.M = P(perm), P(block_len), J, M
    qa.q2k_idx, qa.q2k_num, qa.kmax = P(q2k_idx), P(q2k_num), R
    qa.item_order = P(order)
    qa.k_sum, qa.v_sum, qa.b_sum = P(k_sum), P(v_sum), P(b_sum)

    qws = bsa.qouter_workspace(dev)

    def attend():
        L.check(lib.bsa_forward_qouter(ctypes.byref(qa), bsa.api._ptr(qws), qws.numel(), s_ptr))

    stages = (("tile", tile), ("route", route), ("summaries", summarise), ("attn", attend))
    ev = {n: [_events() for _ in range(args.steps)] for n, _ in stages}

    def step(i=None):
        for name, fn in stages:
            if i is not None:
                ev[name][i][0].record(stream)
            fn()
            if i is not None:
                ev[name][i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ms = {n: sum(a.elapsed_time(b) for a, b in ev[n]) / args.steps for n in ev}
    # nominal work: every query row against R*M exact keys and J - R virtual tokens
    flops = 4.0 * B * h * N * D * (R * M + (J - R))
    attn_tflops = flops / (ms["attn"] * 1e-3) / 1e12
    # summaries: q read for the anchor, k and v read once, summaries written
    sum_bytes = 3 * q.numel() * q.element_size() + 2 * B * h * J * D * 2 + B * h * J * 4
    res = {
        "metric": METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) + per-cell offsets, no dataset or weights)",
        "config": {"workload": "video_dit_vsa_spark_reweight", "B": B, "heads": h, "grid": list(cfg["grid"]),
                   "block": list(cfg["block"]), "D": D, "J": J, "M": M, "R": R, "tokens": N,
                   "virtual_tokens_per_row": J - R},
        "ms": {k_: round(v_, 4) for k_, v_ in ms.items()},
        "summaries_gbps": round(sum_bytes / (ms["summaries"] * 1e-3) / 1e9, 1),
        "pct_hbm_summaries": round(100 * sum_bytes / (ms["summaries"] * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
        "roofline": {"kernel": "vsa4_kernel with summaries (bsa_forward_qouter, block mode)", "bound": "mfma",
                     "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": _profiled_traffic("vsa4_kernel_reweight.md",
                                                  ("attn_vsa.hip", "bsa_device.hpp", "bsa_internal.hpp"))},
    }
    ctx = dict(cfg=cfg, x=x)
    return res, ctx


def cpu_baseline_reweight(ctx, budget_s):
    """Oracle on a bounded sample: head 0's route, anchor and summaries over all
    blocks, and the reweighted attention for as many query blocks as fit."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info

    cfg, x = ctx["cfg"], ctx["x"]
    T, H, W = cfg["grid"]
    D, R = cfg["D"], cfg["R"]
    Q = x["q"][:, :, :1].float().cpu().numpy().astype(np.float64)
    K = x["k"][:, :, :1].float().cpu().numpy().astype(np.float64)
    V = x["v"][:, :, :1].float().cpu().numpy().astype(np.float64)
    t0 = time.perf_counter()
    tab = oracle.tile_index(T, H, W, *cfg["block"])
    J, M = tab["J"], tab["M"]
    qbar = oracle.pool_blocks(Q, tab["perm"], tab["block_len"], M)
    kbar = oracle.pool_blocks(K, tab["perm"], tab["block_len"], M)
    idx, num, _ = oracle.select_topk(oracle.routing_matrix(qbar, kbar), R)
    ks, vs, b, _ = oracle.block_summaries(K, V, tab["perm"], tab["block_len"], M, oracle.anchor_queries(Q))
    t_prep = time.perf_counter() - t0
    done = 0
    t1 = time.perf_counter()
    while done < J and time.perf_counter() - t1 < budget_s:
        items = [(0, 0, i) for i in range(done, min(J, done + 16))]
        oracle.reweight_attention(Q, K, V, tab["perm"], tab["block_len"], M, idx, num, ks, vs, b, items=items)
        done += len(items)
    t_attn = time.perf_counter() - t1
    per_head_s = t_prep + t_attn * J / done
    flops_head = 4.0 * (T * H * W) * D * (R * M + (J - R))
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": round(flops_head / per_head_s / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "head 0 of the video workload: float64 route, anchor and summaries over all %d blocks "
                      "(%.1f s) and reweighted attention for %d of %d query blocks (%.1f s), scaled to one head"
                      % (J, t_prep, done, J, t_attn),
            "ms_per_head": round(per_head_s * 1e3, 1)}


def bench_coarse(args):
    """Video workload with the coarse pooled-V branch: tiling + pool/route/TopK
    (scores kept), V pooling and C = softmax(E) V_bar, and attention with the
    gated C added in its epilogue."""
    import ctypes
    import torch
    import block_sparse_attention_02_amd as bsa
    from workloads import coarse_gate, vsa_inputs, workload

    cfg = workload("video")
    dev = torch.device("cuda:0")
    T, H, W = cfg["grid"]
    B, h, D, R = cfg["B"], cfg["h"], cfg["D"], cfg["R"]
    N = T * H * W
    x = vsa_inputs(cfg, device=dev)
    q, k, v = x["q"], x["k"], x["v"]
    gate = coarse_gate(h, D, seed=cfg["seed"], device=dev)
    J, M = bsa.tile_dims(T, H, W, *cfg["block"])
    perm = torch.empty(J * M, dtype=torch.int32, device=dev)
    block_len = torch.empty(J, dtype=torch.int32, device=dev)
    q2k_idx = torch.empty((B, h, J, R), dtype=torch.int32, device=dev)
    q2k_num = torch.empty((B, h, J), dtype=torch.int32, device=dev)
    order = torch.empty((B, h, J), dtype=torch.int32, device=dev)
    E = torch.empty((B, h, J, J), dtype=torch.float32, device=dev)
    vbar = torch.empty((B, h, J, D), dtype=torch.float32, device=dev)
    C = torch.empty((B, h, J, D), dtype=torch.float32, device=dev)
    out = torch.empty_like(q)
    ws = torch.empty(bsa.route_workspace_bytes(q, J, M, R), dtype=torch.uint8, device=dev)
    L = bsa._lib
    lib = L.load()
    stream = torch.cuda.current_stream(dev)
    s_ptr = bsa.api._stream(dev)
    P = bsa.api._ptr

    def tile():
        L.check(lib.vsa_tile_index(T, H, W, *cfg["block"], P(perm), P(block_len), None, s_ptr))

    ra = bsa.api._route_args(q, k, perm, block_len, J, M, R, R, 1.0 / D ** 0.5, q2k_idx, q2k_num, None, None, E,
                             order)

    def route():
        L.check(lib.vsa_pool_route_topk(ctypes.byref(ra), P(ws), ws.numel(), s_ptr))

    ca = L.CoarseArgs(v=P(v), d=bsa.api._desc(v), dt=L.BSA_BF16, perm=P(perm), block_len=P(block_len), J=J, M=M,
                      E=P(E), vbar=P(vbar), C=P(C))
    n_cws = ctypes.c_size_t()
    L.check(lib.vsa_coarse_ws(ctypes.byref(ca), ctypes.byref(n_cws)))
    cws = torch.empty(n_cws.value, dtype=torch.uint8, device=dev)

    def coarse():
        L.check(lib.vsa_coarse(ctypes.byref(ca), P(cws), cws.numel(), s_ptr))

    qa = bsa.api._qouter_args(q, k, v, out, 1.0 / D ** 0.5, L.BSA_SEL_BLOCK, None)
    qa.perm, qa.block_len, qa.J, qa.M = P(perm), P(block_len), J, M
    qa.q2k_idx, qa.q2k_num, qa.kmax = P(q2k_idx), P(q2k_num), R
    qa.item_order = P(order)
    qa.coarse, qa.gate = P(C), P(gate)

    qws = bsa.qouter_workspace(dev)

    def attend():
        L.check(lib.bsa_forward_qouter(ctypes.byref(qa), bsa.api._ptr(qws), qws.numel(), s_ptr))

    stages = (("tile", tile), ("route", route), ("coarse", coarse), ("attn", attend))
    ev = {n: [_events() for _ in range(args.steps)] for n, _ in stages}

    def step(i=None):
        for name, fn in stages:
            if i is not None:
                ev[name][i][0].record(stream)
            fn()
            if i is not None:
                ev[name][i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ms = {n: sum(a.elapsed_time(b) for a, b in ev[n]) / args.steps for n in ev}
    # nominal work: the sparse attention (the pages' count) plus the coarse
    # product softmax(E) V_bar of every head (2*J*J*D multiply-adds)
    sparse_flops = 4.0 * B * h * N * D * R * M
    coarse_flops = 2.0 * B * h * J * J * D
    attn_tflops = sparse_flops / (ms["attn"] * 1e-3) / 1e12
    # coarse stage: V read and V_bar written by the pooling, then E and V_bar
    # read and C written by the branch
    coarse_bytes = (v.numel() * v.element_size() + B * h * J * D * 4) + (E.numel() * 4 + 2 * B * h * J * D * 4)
    res = {
        "metric": METRIC,
        "value": round((sparse_flops + coarse_flops) / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) + per-cell offsets, seeded N(0, 0.25) gate; no dataset or weights)",
        "config": {"workload": "video_dit_vsa_coarse", "B": B, "heads": h, "grid": list(cfg["grid"]),
                   "block": list(cfg["block"]), "D": D, "J": J, "M": M, "R": R, "tokens": N},
        "ms": {k_: round(v_, 4) for k_, v_ in ms.items()},
        "coarse_gbps": round(coarse_bytes / (ms["coarse"] * 1e-3) / 1e9, 1),
        "pct_hbm_coarse": round(100 * coarse_bytes / (ms["coarse"] * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
        "roofline": {"kernel": "vsa4_kernel with the coarse epilogue (bsa_forward_qouter, block mode)",
                     "bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": _profiled_traffic("coarse_kernel_video.md",
                                                  ("attn_vsa.hip", "bsa_device.hpp", "bsa_internal.hpp"))},
    }
    ctx = dict(cfg=cfg, x=x, gate=gate)
    return res, ctx


def cpu_baseline_coarse(ctx, budget_s):
    """Oracle on a bounded sample: head 0's route and coarse branch over all
    blocks, and the attention plus gated branch for as many query blocks as fit."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info

    cfg, x = ctx["cfg"], ctx["x"]
    T, H, W = cfg["grid"]
    D, R = cfg["D"], cfg["R"]
    Q = x["q"][:, :, :1].float().cpu().numpy().astype(np.float64)
    K = x["k"][:, :, :1].float().cpu().numpy().astype(np.float64)
    V = x["v"][:, :, :1].float().cpu().numpy().astype(np.float64)
    g = ctx["gate"][:1].cpu().numpy().astype(np.float64)
    t0 = time.perf_counter()
    tab = oracle.tile_index(T, H, W, *cfg["block"])
    J, M = tab["J"], tab["M"]
    qbar = oracle.pool_blocks(Q, tab["perm"], tab["block_len"], M)
    kbar = oracle.pool_blocks(K, tab["perm"], tab["block_len"], M)
    E = oracle.routing_matrix(qbar, kbar)
    idx, num, _ = oracle.select_topk(E, R)
    C = oracle.coarse_attention(E, oracle.pool_blocks(V, tab["perm"], tab["block_len"], M))
    t_prep = time.perf_counter() - t0
    done = 0
    t1 = time.perf_counter()
    while done < J and time.perf_counter() - t1 < budget_s:
        items = [(0, 0, i) for i in range(done, min(J, done + 32))]
        O, _ = oracle.vsa_attention(Q, K, V, tab["perm"], tab["block_len"], M, idx, num, items=items)
        oracle.add_coarse(np.nan_to_num(O), C, g, tab["perm"], tab["block_len"], M)
        done += len(items)
    t_attn = time.perf_counter() - t1
    per_head_s = t_prep + t_attn * J / done
    flops_head = 4.0 * (T * H * W) * D * R * M + 2.0 * J * J * D
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": round(flops_head / per_head_s / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "head 0 of the video workload: float64 route, TopK and coarse branch over all %d blocks "
                      "(%.1f s) and attention plus the gated branch for %d of %d query blocks (%.1f s), scaled "
                      "to one head" % (J, t_prep, done, J, t_attn),
            "ms_per_head": round(per_head_s * 1e3, 1)}


def bench_h3(args):
    """H3 multi-region sequence: layout tables, pooling, grouped routing and
    attention over the union of kept blocks."""
    import ctypes
    import torch
    import block_sparse_attention_02_amd as bsa
    from workloads import h3_inputs, workload

    cfg = workload("h3")
    dev = torch.device("cuda:0")
    B, h, D = cfg["B"], cfg["h"], cfg["D"]
    x = h3_inputs(cfg, device=dev)
    q, k, v = x["q"], x["k"], x["v"]
    geom = bsa.H3Geometry(cfg["segments"], cfg["block"], device=dev)
    J, M, N, P = geom.J, geom.M, geom.N, geom.num_prefix
    budgets = geom.budgets(1.0 - cfg["keep"])
    q2k_idx = torch.empty((B, h, J, J), dtype=torch.int32, device=dev)
    q2k_num = torch.empty((B, h, J), dtype=torch.int32, device=dev)
    order = torch.empty((B, h, J), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    L = bsa._lib
    lib = L.load()
    stream = torch.cuda.current_stream(dev)
    s_ptr = bsa.api._stream(dev)
    Pp = bsa.api._ptr
    seg = bsa.api._segments(cfg["segments"])

    def tile():
        L.check(lib.h3_tile_index(seg, len(seg), *cfg["block"], Pp(geom.perm), Pp(geom.block_len), Pp(geom.inv),
                                  s_ptr))

    nr = len(geom.spans)
    spans = (ctypes.c_int32 * (2 * nr))(*[b for sp in geom.spans for b in sp])
    buds = (ctypes.c_int32 * nr)(*budgets)
    ra = L.H3RouteArgs(q=Pp(q), k=Pp(k), d=bsa.api._desc(q), dt=L.BSA_BF16, perm=Pp(geom.perm),
                       block_len=Pp(geom.block_len), J=J, M=M, num_prefix=P, nregions=nr,
                       spans=ctypes.cast(spans, ctypes.c_void_p), budgets=ctypes.cast(buds, ctypes.c_void_p),
                       kmax=J, scale=1.0 / D ** 0.5, q2k_idx=Pp(q2k_idx), q2k_num=Pp(q2k_num), item_order=Pp(order))
    nws = ctypes.c_size_t()
    L.check(lib.h3_pool_route_topk_ws(ctypes.byref(ra), ctypes.byref(nws)))
    ws = torch.empty(nws.value, dtype=torch.uint8, device=dev)

    def route():
        L.check(lib.h3_pool_route_topk(ctypes.byref(ra), Pp(ws), nws.value, s_ptr))

    qa = bsa.api._qouter_args(q, k, v, out, 1.0 / D ** 0.5, L.BSA_SEL_BLOCK, None)
    qa.perm, qa.block_len, qa.J, qa.M = Pp(geom.perm), Pp(geom.block_len), J, M
    qa.q2k_idx, qa.q2k_num, qa.kmax = Pp(q2k_idx), Pp(q2k_num), J
    qa.item_order = Pp(order)

    qws = bsa.qouter_workspace(dev)

    def attend():
        L.check(lib.bsa_forward_qouter(ctypes.byref(qa), bsa.api._ptr(qws), qws.numel(), s_ptr))

    stages = (("tile", tile), ("route", route), ("attn", attend))
    ev = {n: [_events() for _ in range(args.steps)] for n, _ in stages}

    def step(i=None):
        for name, fn in stages:
            if i is not None:
                ev[name][i][0].record(stream)
            fn()
            if i is not None:
                ev[name][i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ms = {n: sum(a.elapsed_time(b) for a, b in ev[n]) / args.steps for n in ev}
    pairs_nominal = float(q2k_num.sum().item())          # kept (query block, key block) pairs
    flops = 4.0 * D * M * M * pairs_nominal              # every pair counted as full blocks
    valid_flops = 4.0 * D * bsa.metrics.vsa_valid_pairs(geom.block_len, q2k_idx, q2k_num)
    attn_tflops = flops / (ms["attn"] * 1e-3) / 1e12
    route_bytes = 2 * q.numel() * q.element_size() + 2 * B * h * J * D * 4 + 4 * float(q2k_num.sum().item())
    res = {
        "metric": METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) + per-cell offsets in the video regions, no dataset or weights)",
        "config": {"workload": "h3_r2v_multi_region", "B": B, "heads": h,
                   "segments": [s_ if isinstance(s_, int) else list(s_) for s_ in cfg["segments"]],
                   "block": list(cfg["block"]), "D": D, "J": J, "M": M, "tokens": N, "prefix_blocks": P,
                   "video_spans": [list(sp) for sp in geom.spans], "budgets": budgets},
        "ms": {k_: round(v_, 4) for k_, v_ in ms.items()},
        "attn_tflops_nominal": round(attn_tflops, 2),
        "attn_tflops_valid": round(valid_flops / (ms["attn"] * 1e-3) / 1e12, 2),
        "route_gbps": round(route_bytes / (ms["route"] * 1e-3) / 1e9, 1),
        "pct_hbm_route": round(100 * route_bytes / (ms["route"] * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
        "roofline": {"kernel": "vsa4_kernel over the grouped index table (bsa_forward_qouter, block mode)",
                     "bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": _profiled_traffic("vsa4_kernel_h3.md",
                                                  ("attn_vsa.hip", "bsa_device.hpp", "bsa_internal.hpp"))},
    }
    ctx = dict(cfg=cfg, x=x, budgets=budgets, pairs_per_head=pairs_nominal / (B * h))
    return res, ctx


def cpu_baseline_h3(ctx, budget_s):
    """Oracle on a bounded sample: head 0's layout, pooling and grouped routing
    over all blocks, and attention for as many query blocks as fit."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info

    cfg, x = ctx["cfg"], ctx["x"]
    D = cfg["D"]
    Q = x["q"][:, :, :1].float().cpu().numpy().astype(np.float64)
    K = x["k"][:, :, :1].float().cpu().numpy().astype(np.float64)
    V = x["v"][:, :, :1].float().cpu().numpy().astype(np.float64)
    t0 = time.perf_counter()
    lay = oracle.h3_layout(cfg["segments"], cfg["block"])
    J, M = lay["J"], lay["M"]
    qbar = oracle.pool_blocks(Q, lay["perm"], lay["block_len"], M)
    kbar = oracle.pool_blocks(K, lay["perm"], lay["block_len"], M)
    idx, num, _ = oracle.h3_route(qbar, kbar, lay["num_prefix"], lay["spans"], ctx["budgets"])
    t_route = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    order = rng.permutation(J)  # a random sample of query blocks of every kind
    done, pairs_done = 0, 0
    t1 = time.perf_counter()
    while done < J and time.perf_counter() - t1 < budget_s:
        blocks = order[done:done + 16]
        oracle.vsa_attention(Q, K, V, lay["perm"], lay["block_len"], M, idx, num,
                             items=[(0, 0, int(i)) for i in blocks])
        pairs_done += int(num[0, 0, blocks].sum())
        done += len(blocks)
    t_attn = time.perf_counter() - t1
    pairs_head = float(num[0, 0].sum())
    per_head_s = t_route + t_attn * pairs_head / max(pairs_done, 1)
    flops_head = 4.0 * D * M * M * pairs_head
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": round(flops_head / per_head_s / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "head 0 of the h3 workload: float64 layout, pooling and grouped routing over all %d blocks "
                      "(%.1f s) and attention for %d random query blocks (%d of %d kept pairs, %.1f s), scaled "
                      "to one head by kept pairs" % (J, t_route, done, pairs_done, int(pairs_head), t_attn),
            "ms_per_head": round(per_head_s * 1e3, 1)}


def bench_reblock(args):
    """Video workload on Spark-Reblock key layouts (reused by the queries)."""
    import ctypes
    import torch
    import block_sparse_attention_02_amd as bsa
    from workloads import vsa_inputs, workload

    cfg = workload("video")
    dev = torch.device("cuda:0")
    T, H, W = cfg["grid"]
    B, h, D, R = cfg["B"], cfg["h"], cfg["D"], cfg["R"]
    N = T * H * W
    M = 64
    x = vsa_inputs(cfg, device=dev)
    q, k, v = x["q"], x["k"], x["v"]
    L = bsa._lib
    lib = L.load()
    Jc, nl = ctypes.c_int(), ctypes.c_int()
    L.check(lib.spark_reblock_dims(N, M, ctypes.byref(Jc), ctypes.byref(nl)))
    J = Jc.value
    perm = torch.empty((B * h, J * M), dtype=torch.int32, device=dev)
    block_len = torch.empty(J, dtype=torch.int32, device=dev)
    q2k_idx = torch.empty((B, h, J, R), dtype=torch.int32, device=dev)
    q2k_num = torch.empty((B, h, J), dtype=torch.int32, device=dev)
    order = torch.empty((B, h, J), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)
    s_ptr = bsa.api._stream(dev)
    P = bsa.api._ptr
    rb = L.ReblockArgs(q=P(q), k=P(k), d=bsa.api._desc(q), dt=L.BSA_BF16, M=M, ridge=1e-4, perm=P(perm),
                       block_len=P(block_len))
    nrb = ctypes.c_size_t()
    L.check(lib.spark_reblock_ws(ctypes.byref(rb), ctypes.byref(nrb)))
    rws = torch.empty(nrb.value, dtype=torch.uint8, device=dev)

    def reblock():
        L.check(lib.spark_reblock(ctypes.byref(rb), P(rws), nrb.value, s_ptr))

    ra = bsa.api._route_args(q, k, perm, block_len, J, M, R, R, 1.0 / D ** 0.5, q2k_idx, q2k_num, None, None, None,
                             order)
    ra.perm_bh_stride = J * M
    ws = torch.empty(bsa.route_workspace_bytes(q, J, M, R), dtype=torch.uint8, device=dev)

    def route():
        L.check(lib.vsa_pool_route_topk(ctypes.byref(ra), P(ws), ws.numel(), s_ptr))

    qa = bsa.api._qouter_args(q, k, v, out, 1.0 / D ** 0.5, L.BSA_SEL_BLOCK, None)
    qa.perm, qa.block_len, qa.J, qa.M = P(perm), P(block_len), J, M
    qa.q2k_idx, qa.q2k_num, qa.kmax = P(q2k_idx), P(q2k_num), R
    qa.item_order = P(order)
    qa.perm_bh_stride = J * M

    qws = bsa.qouter_workspace(dev)

    def attend():
        L.check(lib.bsa_forward_qouter(ctypes.byref(qa), bsa.api._ptr(qws), qws.numel(), s_ptr))

    stages = (("reblock", reblock), ("route", route), ("attn", attend))
    ev = {n: [_events() for _ in range(args.steps)] for n, _ in stages}

    def step(i=None):
        for name, fn in stages:
            if i is not None:
                ev[name][i][0].record(stream)
            fn()
            if i is not None:
                ev[name][i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ms = {n: sum(a.elapsed_time(b) for a, b in ev[n]) / args.steps for n in ev}
    flops = 4.0 * B * h * N * D * R * M
    attn_tflops = flops / (ms["attn"] * 1e-3) / 1e12
    res = {
        "metric": METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) + per-cell offsets, no dataset or weights)",
        "config": {"workload": "video_dit_vsa_spark_reblock", "B": B, "heads": h, "grid": list(cfg["grid"]),
                   "D": D, "J": J, "M": M, "R": R, "tokens": N, "tree_levels": nl.value},
        "ms": {k_: round(v_, 4) for k_, v_ in ms.items()},
        "roofline": {"kernel": "vsa4_kernel over per-head reblocked tables (bsa_forward_qouter, block mode)",
                     "bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": _profiled_traffic("vsa4_kernel_reblock.md",
                                                  ("attn_vsa.hip", "bsa_device.hpp", "bsa_internal.hpp"))},
    }
    return res, dict(cfg=cfg, x=x)


def cpu_baseline_reblock(ctx, budget_s):
    """Oracle on a bounded sample: head 0's moment, features and tree over all
    115200 tokens, then pooling, routing and attention for as many query
    blocks as fit."""
    import numpy as np
    import oracle
    from oracle import reblock as rbo
    from threadpoolctl import threadpool_info

    cfg, x = ctx["cfg"], ctx["x"]
    D, R, M = cfg["D"], cfg["R"], 64
    Q = x["q"][:, :, :1].float().cpu().numpy().astype(np.float64)
    K = x["k"][:, :, :1].float().cpu().numpy().astype(np.float64)
    V = x["v"][:, :, :1].float().cpu().numpy().astype(np.float64)
    N = Q.shape[1]
    t0 = time.perf_counter()
    U = rbo.key_features(K, Q)[0, 0]
    perm, block_len = rbo.reblock_tables(rbo.reblock_orders(U, M)[-1], M)
    J = len(block_len)
    qbar = oracle.pool_blocks(Q, perm, block_len, M)
    kbar = oracle.pool_blocks(K, perm, block_len, M)
    idx, num, _ = oracle.select_topk(oracle.routing_matrix(qbar, kbar), R)
    t_prep = time.perf_counter() - t0
    done = 0
    t1 = time.perf_counter()
    while done < J and time.perf_counter() - t1 < budget_s:
        items = [(0, 0, i) for i in range(done, min(J, done + 32))]
        oracle.vsa_attention(Q, K, V, perm, block_len, M, idx, num, items=items)
        done += len(items)
    t_attn = time.perf_counter() - t1
    per_head_s = t_prep + t_attn * J / done
    flops_head = 4.0 * N * D * R * M
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": round(flops_head / per_head_s / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "head 0 of the video workload: float64 reblock layout, pooling, routing and TopK over all "
                      "%d blocks (%.1f s) and attention for %d of %d query blocks (%.1f s), scaled to one head"
                      % (J, t_prep, done, J, t_attn),
            "ms_per_head": round(per_head_s * 1e3, 1)}


def _time(fn, steps, warmup, stream):
    """Average ms of fn() over `steps` launches, HIP events on `stream`."""
    import torch
    for _ in range(warmup):
        fn()
    evs = [_events() for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return sum(a.elapsed_time(b) for a, b in evs) / steps, wall


def bench_nsa(args):
    """NSA selected branch, query-outer (token mode), 32768 tokens."""
    import torch
    import block_sparse_attention_02_amd as bsa
    from workloads import nsa_inputs, workload

    cfg = workload("nsa")
    dev = torch.device("cuda:0")
    q, k, v, idx, cnt = nsa_inputs(cfg, device=dev)
    G = cfg["HQ"] // cfg["H"]
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)
    ms, wall = _time(lambda: bsa.attention_nsa(q, k, v, idx, cnt, cfg["BS"], out=out), args.steps, args.warmup,
                     stream)
    flops = bsa.metrics.nsa_nominal_flops(cnt, cfg["BS"], G, cfg["D"])
    # algorithmic bytes: q read, o written, k/v read once, index tables
    nbytes = 2 * q.numel() * 2 + 2 * k.numel() * 2 + idx.numel() * 4 + cnt.numel() * 4
    tf = flops / (ms * 1e-3) / 1e12
    return {
        "metric": METRIC, "value": round(tf, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1), random causal selections)",
        "config": {"workload": "nsa_selected_branch", "T": cfg["T"], "HQ": cfg["HQ"], "H": cfg["H"], "D": cfg["D"],
                   "BS": cfg["BS"], "S": cfg["S"], "causal": True},
        "ms": {"attn": round(ms, 4)},
        "roofline": {"kernel": "nsa_attn_kernel (bsa_forward_qouter, token mode)", "bound": "mfma",
                     "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": _profiled_traffic("nsa_attn_kernel_nsa.md",
                                                  ("attn_nsa.hip", "bsa_device.hpp", "bsa_internal.hpp"))},
        "hbm_gbps_algorithmic": round(nbytes / (ms * 1e-3) / 1e9, 1),
    }


def bench_msa(args):
    """KV-outer schedule (reverse index, scheduler, K1) + combine, 65536 positions."""
    import torch
    import block_sparse_attention_02_amd as bsa
    from workloads import msa_inputs, workload

    cfg = workload("msa")
    dev = torch.device("cuda:0")
    q, k, v, q2k = msa_inputs(cfg, device=dev)
    B, N, Hq, D = q.shape
    Hkv, ks, BK = cfg["Hkv"], cfg["k"], cfg["BK"]
    G = Hq // Hkv
    bufs = (torch.empty((B, ks, N, Hq, D), dtype=torch.bfloat16, device=dev),
            torch.empty((B, ks, N, Hq), dtype=torch.float32, device=dev),
            torch.empty((B, N, Hkv), dtype=torch.int32, device=dev))
    out = torch.empty_like(q)
    ws = [None]
    o_buf, lse_buf, nslot = bsa.kvouter(q, k, v, q2k, BK, bufs=bufs)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    def k1():
        bsa.kvouter(q, k, v, q2k, BK, bufs=bufs, workspace=ws[0])

    ws[0] = torch.empty(256 << 20, dtype=torch.uint8, device=dev)   # >= bsa_kvouter_ws for this shape
    ms_k1, _ = _time(k1, args.steps, args.warmup, stream)
    ms_k2, _ = _time(lambda: bsa.combine(o_buf, lse_buf, nslot, Hkv, out=out), args.steps, args.warmup, stream)
    edges = int((q2k >= 0).sum().item())
    flops = bsa.metrics.kvouter_nominal_flops(q2k, BK, G, D)
    # K1 algorithmic bytes (the page's I/O model): K/V once, Q per edge, O_buf + LSE per edge
    k1_bytes = 2 * k.numel() * 2 + edges * G * D * 2 * 2 + edges * G * 4
    k2_bytes = edges * G * (D * 2 + 4) + q.numel() * 2 + nslot.numel() * 4
    ms = ms_k1 + ms_k2
    tf = flops / (ms * 1e-3) / 1e12
    return {
        "metric": METRIC, "value": round(tf, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1), sink + local + Zipf(1.1) selections)",
        "config": {"workload": "msa_kv_outer", "N": N, "Hq": Hq, "Hkv": Hkv, "D": D, "BK": BK, "k": ks,
                   "edges": edges},
        "ms": {"kvouter_k1": round(ms_k1, 4), "combine_k2": round(ms_k2, 4)},
        "k1_tflops": round(flops / (ms_k1 * 1e-3) / 1e12, 2),
        "k1_gbps_algorithmic": round(k1_bytes / (ms_k1 * 1e-3) / 1e9, 1),
        "k2_gbps_algorithmic": round(k2_bytes / (ms_k2 * 1e-3) / 1e9, 1),
        "pct_hbm_k2": round(100 * k2_bytes / (ms_k2 * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
        # the timed call also runs the reverse index (about 2 % of it)
        "roofline": {"kernel": "kv_k1w_kernel (bsa_forward_kvouter)", "bound": "hbm",
                     "achieved": round(k1_bytes / (ms_k1 * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(k1_bytes / (ms_k1 * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                     "traffic": _profiled_traffic("kv_k1w_kernel_msa.md",
                                                  ("kvouter.hip", "bsa_device.hpp", "bsa_internal.hpp"))},
    }


def cpu_baseline_video(ctx, budget_s):
    """Oracle on a bounded sample: pool + route + TopK of one head, and exact
    attention of as many of that head's query blocks as fit the budget."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info

    cfg, J, M = ctx["cfg"], ctx["J"], ctx["M"]
    T, H, W = cfg["grid"]
    D, R = cfg["D"], cfg["R"]
    head = 0
    Q = ctx["x"]["q"][:, :, head:head + 1].float().cpu().numpy().astype(np.float64)
    K = ctx["x"]["k"][:, :, head:head + 1].float().cpu().numpy().astype(np.float64)
    V = ctx["x"]["v"][:, :, head:head + 1].float().cpu().numpy().astype(np.float64)
    t0 = time.perf_counter()
    tab = oracle.tile_index(T, H, W, *cfg["block"])
    qbar = oracle.pool_blocks(Q, tab["perm"], tab["block_len"], M)
    kbar = oracle.pool_blocks(K, tab["perm"], tab["block_len"], M)
    idx, num, _ = oracle.select_topk(oracle.routing_matrix(qbar, kbar), R)
    t_route = time.perf_counter() - t0
    done, t_attn = 0, 0.0
    t1 = time.perf_counter()
    while done < J and time.perf_counter() - t1 < budget_s:
        items = [(0, 0, i) for i in range(done, min(J, done + 32))]
        oracle.vsa_attention(Q, K, V, tab["perm"], tab["block_len"], M, idx, num, items=items)
        done += len(items)
    t_attn = time.perf_counter() - t1
    # per head: route once + J query blocks of attention
    per_head_s = t_route + t_attn * J / done
    flops_head = 4.0 * (T * H * W) * D * R * M
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": round(flops_head / per_head_s / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "head 0 of the video workload: float64 pool+route+TopK over all %d blocks (%.1f s) "
                      "and exact attention for %d of %d query blocks (%.1f s), scaled to one head"
                      % (J, t_route, done, J, t_attn),
            "ms_per_head": round(per_head_s * 1e3, 1)}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="video", choices=["video", "nsa", "msa", "reweight", "coarse", "h3", "reblock"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for hardware byte counters)")
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the routed attention shards by heads with no exchange, "
              "so one MI355X runs one shard's kernels at their real shape; use --gpus 1", file=sys.stderr)
        return 2
    if args.copy_calibration:
        import torch
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel(), "copy_bytes_written": dst.numel(), "launches": 3}))
        return 0
    if args.workload == "nsa":
        res = bench_nsa(args)
    elif args.workload == "msa":
        res = bench_msa(args)
    elif args.workload == "reweight":
        res, ctx = bench_reweight(args)
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = cpu_baseline_reweight(ctx, args.cpu_seconds)
    elif args.workload == "reblock":
        res, ctx = bench_reblock(args)
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = cpu_baseline_reblock(ctx, args.cpu_seconds)
    elif args.workload == "h3":
        res, ctx = bench_h3(args)
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = cpu_baseline_h3(ctx, args.cpu_seconds)
    elif args.workload == "coarse":
        res, ctx = bench_coarse(args)
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = cpu_baseline_coarse(ctx, args.cpu_seconds)
    else:
        res, ctx = bench_video(args)
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = cpu_baseline_video(ctx, args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

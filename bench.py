"""Throughput of routed block-sparse attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload video|nsa|msa|reweight|coarse|h3|reblock]
                    [--schedule qouter|kvouter] [--cold-reps R] [--no-cpu-baseline]

A step is one pass of the routed block-sparse attention hot path over one
batch of synthetic input already resident in HBM:

  video  (default) tiling tables -> per-block mean pooling -> routing scores ->
         TopK index table -> exact block-sparse attention, on the video-DiT
         workload (115200 tokens = 30x48x80 grid in 4x4x4 blocks, 24 heads,
         D=128, keep 192 of 1920 blocks).
  nsa    NSA selected-branch attention (32768 tokens, 64 query / 4 KV heads,
         blocks of 64, up to 16 selected); --schedule qouter (default) runs the
         token-mode query-outer kernel, --schedule kvouter runs the same
         selections through the KV-outer schedule and the combine.
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

Timing.  W untimed warm-up steps, then exactly K steps back to back between
two device synchronisations (wall clock: ``ms_per_step`` and ``value``), with
a HIP event pair around every call on the stream it is launched on (``ms``:
the mean per call over the timed region; ``ms_stats.warm``: its median, min
and 90th percentile).  Then ``--cold-reps`` more runs of every call, each
after 512 MiB of scratch memory has been written so that the L2 caches and
the last-level cache start cold (``ms_stats.cold``: median, min, p90).

Prints one JSON line.  ``value`` is the effective attention throughput of the
whole step, 4*h*N*D*k*M / step time (the pages' FLOP count, every kept block
counted full), in TFLOP/s.  ``roofline`` is the dominant kernel: achieved =
the work that kernel must do per launch (valid query-key pairs for attention,
algorithmic bytes for HBM-bound stages) / its mean event time in the timed
region; ``achieved_nominal`` / ``frac_nominal`` repeat it with the nominal
FLOP count.  ``cpu_baseline`` times the float64 oracle on a bounded sample of
the same workload on the host cores.
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
SCRUB_BYTES = 512 << 20       # written before every cold call: larger than L2 + the last-level cache


# ---------------------------------------------------------------------------- helpers

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


ATTN_SOURCES = ("attn_vsa.hip", "bsa_device.hpp", "bsa_internal.hpp")
# the kernel that serves 64-row blocks without summaries
ATTN_KERNEL = "vsa_pp_kernel"
KV_SOURCES = ("kvouter.hip", "bsa_device.hpp", "bsa_internal.hpp")


def _stats(xs):
    """median, min and 90th percentile (nearest rank) of a list of ms."""
    s = sorted(xs)
    n = len(s)
    if n == 0:
        return None
    med = s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])
    p90 = s[min(n - 1, max(0, -(-9 * n // 10) - 1))]
    return {"median": round(med, 4), "min": round(s[0], 4), "p90": round(p90, 4), "n": n}


def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_stages(stages, args, stream):
    """Run `stages` ((name, fn) in order = one step): warm-up, the timed region
    of args.steps contiguous steps, then args.cold_reps cold runs per call.
    Returns (ms_per_step wall, mean ms per call, {name: {warm, cold}})."""
    import torch
    for _ in range(args.warmup):
        for _, fn in stages:
            fn()
    ev = {n: [_events() for _ in range(args.steps)] for n, _ in stages}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        for n, fn in stages:
            ev[n][i][0].record(stream)
            fn()
            ev[n][i][1].record(stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    warm = {n: [a.elapsed_time(b) for a, b in ev[n]] for n in ev}
    mean = {n: sum(v_) / len(v_) for n, v_ in warm.items()}
    cold = {n: [] for n in ev}
    if args.cold_reps > 0:
        scrub = torch.empty(SCRUB_BYTES, dtype=torch.uint8, device=stream.device)
        cev = {n: [_events() for _ in range(args.cold_reps)] for n in ev}
        for r in range(args.cold_reps):
            for n, fn in stages:
                scrub.fill_(1 + r % 251)
                cev[n][r][0].record(stream)
                fn()
                cev[n][r][1].record(stream)
        torch.cuda.synchronize()
        cold = {n: [a.elapsed_time(b) for a, b in cev[n]] for n in cev}
        del scrub
    stats = {n: {"warm": _stats(warm[n]), "cold": _stats(cold[n])} for n in ev}
    return ms_step, mean, stats


def host_info():
    """CPU model, BLAS library and thread count of the host the oracle runs on."""
    from threadpoolctl import threadpool_info
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max([p.get("num_threads", 1) for p in blas] + [1])
    vendor = ", ".join(sorted({"%s %s" % (p.get("internal_api", "?"), p.get("version", "")) for p in blas})) or "none"
    return {"cpu_model": model, "blas": vendor, "threads": threads,
            "affinity_cores": len(os.sched_getaffinity(0))}


def _baseline(value, unit, sample, extra=None):
    info = host_info()
    res = {"value": value, "unit": unit, "cores": info["threads"], "kind": "oracle", "sample": sample,
           "host": info}
    res.update(extra or {})
    return res


def _line(args, value, ms_step, config, data, ms, stats, roofline, extra=None):
    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": data,
        "config": config,
        "ms": {k_: round(v_, 4) for k_, v_ in ms.items()},
        "ms_stats": stats,
        "roofline": roofline,
    }
    res.update(extra or {})
    return res


def _roofline_mfma(kernel, valid_flops, nominal_flops, ms, traffic):
    tf = valid_flops / (ms * 1e-3) / 1e12
    tfn = nominal_flops / (ms * 1e-3) / 1e12
    return {"kernel": kernel, "bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
            "work": "valid query-key pairs x 4D flops per launch",
            "achieved_nominal": round(tfn, 2), "frac_nominal": round(tfn / PEAK_BF16_TFLOPS, 4),
            "ms_mean": round(ms, 4)}


def _roofline_hbm(kernel, nbytes, ms, traffic):
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": traffic,
            "work": "algorithmic bytes per launch", "bytes": int(nbytes), "ms_mean": round(ms, 4)}


def _gbps(nbytes, ms):
    return round(nbytes / (ms * 1e-3) / 1e9, 1)


def _pct_hbm(nbytes, ms):
    return round(100 * nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2)


def _f64_head(x, head=0):
    import numpy as np
    return {n: x[n][:, :, head:head + 1].float().cpu().numpy().astype(np.float64) for n in ("q", "k", "v")}


# ---------------------------------------------------------------------------- VSA family

class _Vsa:
    """Device buffers and library calls of the video step (shared by the
    video, reweight and coarse workloads)."""

    def __init__(self, with_scores=False):
        import ctypes
        import torch
        import block_sparse_attention_02_amd as bsa
        from workloads import vsa_inputs, workload
        self.ctypes, self.torch, self.bsa = ctypes, torch, bsa
        cfg = self.cfg = workload("video")
        dev = self.dev = torch.device("cuda:0")
        T, H, W = cfg["grid"]
        self.B, self.h, self.D, self.R = cfg["B"], cfg["h"], cfg["D"], cfg["R"]
        self.N = T * H * W
        self.x = vsa_inputs(cfg, device=dev)
        q, k, v = self.x["q"], self.x["k"], self.x["v"]
        J, M = self.J, self.M = bsa.tile_dims(T, H, W, *cfg["block"])
        B, h, D, R = self.B, self.h, self.D, self.R
        self.perm = torch.empty(J * M, dtype=torch.int32, device=dev)
        self.block_len = torch.empty(J, dtype=torch.int32, device=dev)
        self.inv = torch.empty(self.N, dtype=torch.int32, device=dev)
        self.q2k_idx = torch.empty((B, h, J, R), dtype=torch.int32, device=dev)
        self.q2k_num = torch.empty((B, h, J), dtype=torch.int32, device=dev)
        self.order = torch.empty((B, h, J), dtype=torch.int32, device=dev)
        self.E = torch.empty((B, h, J, J), dtype=torch.float32, device=dev) if with_scores else None
        self.out = torch.empty_like(q)
        self.ws = torch.empty(bsa.route_workspace_bytes(q, J, M, R), dtype=torch.uint8, device=dev)
        self.qws = bsa.qouter_workspace(dev)
        self.L = bsa._lib
        self.lib = self.L.load()
        self.stream = torch.cuda.current_stream(dev)
        self.s_ptr = bsa.api._stream(dev)
        P = self.P = bsa.api._ptr
        self.ra = bsa.api._route_args(q, k, self.perm, self.block_len, J, M, R, R, 1.0 / D ** 0.5, self.q2k_idx,
                                      self.q2k_num, None, None, self.E, self.order)
        qa = self.qa = bsa.api._qouter_args(q, k, v, self.out, 1.0 / D ** 0.5, self.L.BSA_SEL_BLOCK, None)
        qa.perm, qa.block_len, qa.J, qa.M = P(self.perm), P(self.block_len), J, M
        qa.q2k_idx, qa.q2k_num, qa.kmax = P(self.q2k_idx), P(self.q2k_num), R
        qa.item_order = P(self.order)

    def tile(self):
        P = self.P
        self.L.check(self.lib.vsa_tile_index(*self.cfg["grid"], *self.cfg["block"], P(self.perm),
                                             P(self.block_len), P(self.inv), self.s_ptr))

    def route(self):
        self.L.check(self.lib.vsa_pool_route_topk(self.ctypes.byref(self.ra), self.P(self.ws), self.ws.numel(),
                                                  self.s_ptr))

    def attend(self):
        self.L.check(self.lib.bsa_forward_qouter(self.ctypes.byref(self.qa), self.P(self.qws), self.qws.numel(),
                                                 self.s_ptr))

    def nominal_flops(self):
        return 4.0 * self.B * self.h * self.N * self.D * self.R * self.M

    def valid_flops(self):
        return 4.0 * self.D * self.bsa.metrics.vsa_valid_pairs(self.block_len, self.q2k_idx, self.q2k_num)

    def route_bytes(self):
        # read Q and K once, write the pooled means and the index table
        q = self.x["q"]
        return (2 * q.numel() * q.element_size() + 2 * self.B * self.h * self.J * self.D * 4
                + self.B * self.h * self.J * (self.R + 1) * 4)

    def config(self, name, **extra):
        c = {"workload": name, "B": self.B, "heads": self.h, "grid": list(self.cfg["grid"]),
             "block": list(self.cfg["block"]), "D": self.D, "J": self.J, "M": self.M, "R": self.R,
             "tokens": self.N}
        c.update(extra)
        return c


DATA_VIDEO = "synthetic (seeded N(0,1) + per-cell offsets, no dataset or weights)"


def bench_video(args):
    w = _Vsa()
    ms_step, ms, stats = time_stages((("tile", w.tile), ("route", w.route), ("attn", w.attend)), args, w.stream)
    rb = w.route_bytes()
    roof = _roofline_mfma(ATTN_KERNEL + " (bsa_forward_qouter, block mode)", w.valid_flops(), w.nominal_flops(),
                          ms["attn"], _profiled_traffic(ATTN_KERNEL + "_video.md", ATTN_SOURCES))
    res = _line(args, w.nominal_flops() / (ms_step * 1e-3) / 1e12, ms_step, w.config("video_dit_vsa"), DATA_VIDEO,
                ms, stats, roof,
                {"pct_bf16_peak_attn_valid": round(100 * roof["frac"], 2),
                 "pct_bf16_peak_attn_nominal": round(100 * roof["frac_nominal"], 2),
                 "route_gbps": _gbps(rb, ms["route"]), "pct_hbm_route": _pct_hbm(rb, ms["route"])})
    return res, w


def cpu_baseline_video(w, budget_s):
    """Oracle on a bounded sample: pool + route + TopK of one head, and exact
    attention of as many of that head's query blocks as fit the budget."""
    import oracle
    cfg, J, M = w.cfg, w.J, w.M
    X = _f64_head(w.x)
    t0 = time.perf_counter()
    tab = oracle.tile_index(*cfg["grid"], *cfg["block"])
    qbar = oracle.pool_blocks(X["q"], tab["perm"], tab["block_len"], M)
    kbar = oracle.pool_blocks(X["k"], tab["perm"], tab["block_len"], M)
    idx, num, _ = oracle.select_topk(oracle.routing_matrix(qbar, kbar), w.R)
    t_route = time.perf_counter() - t0
    done = 0
    t1 = time.perf_counter()
    while done < J and time.perf_counter() - t1 < budget_s:
        items = [(0, 0, i) for i in range(done, min(J, done + 32))]
        oracle.vsa_attention(X["q"], X["k"], X["v"], tab["perm"], tab["block_len"], M, idx, num, items=items)
        done += len(items)
    t_attn = time.perf_counter() - t1
    per_head_s = t_route + t_attn * J / done
    flops_head = 4.0 * w.N * w.D * w.R * M
    return _baseline(round(flops_head / per_head_s / 1e12, 6), "TFLOP/s",
                     "head 0 of the video workload: float64 pool+route+TopK over all %d blocks (%.1f s) and exact "
                     "attention for %d of %d query blocks (%.1f s), scaled to one head" % (J, t_route, done, J, t_attn),
                     {"ms_per_head": round(per_head_s * 1e3, 1)})


def bench_reweight(args):
    """Video workload with Spark-Reweight: tiling + pool/route/TopK, block
    summaries, and attention over the kept blocks plus one virtual token per
    other block, under one softmax."""
    w = _Vsa()
    torch, L, P = w.torch, w.L, w.P
    B, h, J, D = w.B, w.h, w.J, w.D
    k_sum = torch.empty((B, h, J, D), dtype=torch.bfloat16, device=w.dev)
    v_sum = torch.empty((B, h, J, D), dtype=torch.bfloat16, device=w.dev)
    b_sum = torch.empty((B, h, J), dtype=torch.float32, device=w.dev)
    q, k, v = w.x["q"], w.x["k"], w.x["v"]
    sa = L.SummaryArgs(q=P(q), k=P(k), v=P(v), d=w.bsa.api._desc(k), dt=L.BSA_BF16, perm=P(w.perm),
                       block_len=P(w.block_len), J=J, M=w.M, scale=1.0 / D ** 0.5, anchor=None, anchor_out=None,
                       k_sum=P(k_sum), v_sum=P(v_sum), b_sum=P(b_sum))
    nsw = w.ctypes.c_size_t(0)
    L.check(w.lib.spark_summaries_ws(w.ctypes.byref(sa), w.ctypes.byref(nsw)))
    sws = torch.empty(max(1, nsw.value), dtype=torch.uint8, device=w.dev)

    def summarise():
        L.check(w.lib.spark_summaries(w.ctypes.byref(sa), P(sws), nsw.value, w.s_ptr))

    w.qa.k_sum, w.qa.v_sum, w.qa.b_sum = P(k_sum), P(v_sum), P(b_sum)
    ms_step, ms, stats = time_stages((("tile", w.tile), ("route", w.route), ("summaries", summarise),
                                      ("attn", w.attend)), args, w.stream)
    # work: every query row against its exact keys and the J - R virtual tokens
    virt = 4.0 * B * h * w.N * D * (J - w.R)
    nominal = w.nominal_flops() + virt
    valid = w.valid_flops() + virt
    sum_bytes = 3 * q.numel() * q.element_size() + 2 * B * h * J * D * 2 + B * h * J * 4
    roof = _roofline_mfma("vsa4_kernel with summaries (bsa_forward_qouter, block mode)", valid, nominal, ms["attn"],
                          _profiled_traffic("vsa4_kernel_reweight.md", ATTN_SOURCES))
    res = _line(args, nominal / (ms_step * 1e-3) / 1e12, ms_step,
                w.config("video_dit_vsa_spark_reweight", virtual_tokens_per_row=J - w.R), DATA_VIDEO, ms, stats, roof,
                {"summaries_gbps": _gbps(sum_bytes, ms["summaries"]),
                 "pct_hbm_summaries": _pct_hbm(sum_bytes, ms["summaries"])})
    return res, w


def cpu_baseline_reweight(w, budget_s):
    """Oracle on a bounded sample: head 0's route, anchor and summaries over all
    blocks, and the reweighted attention for as many query blocks as fit."""
    import oracle
    cfg = w.cfg
    X = _f64_head(w.x)
    t0 = time.perf_counter()
    tab = oracle.tile_index(*cfg["grid"], *cfg["block"])
    J, M = tab["J"], tab["M"]
    qbar = oracle.pool_blocks(X["q"], tab["perm"], tab["block_len"], M)
    kbar = oracle.pool_blocks(X["k"], tab["perm"], tab["block_len"], M)
    idx, num, _ = oracle.select_topk(oracle.routing_matrix(qbar, kbar), w.R)
    ks, vs, b, _ = oracle.block_summaries(X["k"], X["v"], tab["perm"], tab["block_len"], M,
                                          oracle.anchor_queries(X["q"]))
    t_prep = time.perf_counter() - t0
    done = 0
    t1 = time.perf_counter()
    while done < J and time.perf_counter() - t1 < budget_s:
        items = [(0, 0, i) for i in range(done, min(J, done + 16))]
        oracle.reweight_attention(X["q"], X["k"], X["v"], tab["perm"], tab["block_len"], M, idx, num, ks, vs, b,
                                  items=items)
        done += len(items)
    t_attn = time.perf_counter() - t1
    per_head_s = t_prep + t_attn * J / done
    flops_head = 4.0 * w.N * w.D * (w.R * M + (J - w.R))
    return _baseline(round(flops_head / per_head_s / 1e12, 6), "TFLOP/s",
                     "head 0 of the video workload: float64 route, anchor and summaries over all %d blocks (%.1f s) "
                     "and reweighted attention for %d of %d query blocks (%.1f s), scaled to one head"
                     % (J, t_prep, done, J, t_attn), {"ms_per_head": round(per_head_s * 1e3, 1)})


def bench_coarse(args):
    """Video workload with the coarse pooled-V branch: tiling + pool/route/TopK
    (scores kept), V pooling and C = softmax(E) V_bar, and attention with the
    gated C added in its epilogue."""
    from workloads import coarse_gate
    w = _Vsa(with_scores=True)
    torch, L, P = w.torch, w.L, w.P
    B, h, J, D = w.B, w.h, w.J, w.D
    v = w.x["v"]
    w.gate = coarse_gate(h, D, seed=w.cfg["seed"], device=w.dev)
    vbar = torch.empty((B, h, J, D), dtype=torch.float32, device=w.dev)
    C = torch.empty((B, h, J, D), dtype=torch.float32, device=w.dev)
    ca = L.CoarseArgs(v=P(v), d=w.bsa.api._desc(v), dt=L.BSA_BF16, perm=P(w.perm), block_len=P(w.block_len), J=J,
                      M=w.M, E=P(w.E), vbar=P(vbar), C=P(C))
    n_cws = w.ctypes.c_size_t()
    L.check(w.lib.vsa_coarse_ws(w.ctypes.byref(ca), w.ctypes.byref(n_cws)))
    cws = torch.empty(n_cws.value, dtype=torch.uint8, device=w.dev)

    def coarse():
        L.check(w.lib.vsa_coarse(w.ctypes.byref(ca), P(cws), cws.numel(), w.s_ptr))

    w.qa.coarse, w.qa.gate = P(C), P(w.gate)
    ms_step, ms, stats = time_stages((("tile", w.tile), ("route", w.route), ("coarse", coarse), ("attn", w.attend)),
                                     args, w.stream)
    # the sparse attention (the pages' count) plus the coarse product
    # softmax(E) V_bar of every head (2*J*J*D multiply-adds)
    coarse_flops = 2.0 * B * h * J * J * D
    coarse_bytes = (v.numel() * v.element_size() + B * h * J * D * 4) + (w.E.numel() * 4 + 2 * B * h * J * D * 4)
    roof = _roofline_mfma(ATTN_KERNEL + " with the coarse epilogue (bsa_forward_qouter, block mode)", w.valid_flops(),
                          w.nominal_flops(), ms["attn"], _profiled_traffic("coarse_kernel_video.md", ATTN_SOURCES))
    data = "synthetic (seeded N(0,1) + per-cell offsets, seeded N(0, 0.25) gate; no dataset or weights)"
    res = _line(args, (w.nominal_flops() + coarse_flops) / (ms_step * 1e-3) / 1e12, ms_step,
                w.config("video_dit_vsa_coarse"), data, ms, stats, roof,
                {"coarse_gbps": _gbps(coarse_bytes, ms["coarse"]), "pct_hbm_coarse": _pct_hbm(coarse_bytes,
                                                                                               ms["coarse"])})
    return res, w


def cpu_baseline_coarse(w, budget_s):
    """Oracle on a bounded sample: head 0's route and coarse branch over all
    blocks, and the attention plus gated branch for as many query blocks as fit."""
    import numpy as np
    import oracle
    cfg = w.cfg
    X = _f64_head(w.x)
    g = w.gate[:1].cpu().numpy().astype(np.float64)
    t0 = time.perf_counter()
    tab = oracle.tile_index(*cfg["grid"], *cfg["block"])
    J, M = tab["J"], tab["M"]
    qbar = oracle.pool_blocks(X["q"], tab["perm"], tab["block_len"], M)
    kbar = oracle.pool_blocks(X["k"], tab["perm"], tab["block_len"], M)
    E = oracle.routing_matrix(qbar, kbar)
    idx, num, _ = oracle.select_topk(E, w.R)
    C = oracle.coarse_attention(E, oracle.pool_blocks(X["v"], tab["perm"], tab["block_len"], M))
    t_prep = time.perf_counter() - t0
    done = 0
    t1 = time.perf_counter()
    while done < J and time.perf_counter() - t1 < budget_s:
        items = [(0, 0, i) for i in range(done, min(J, done + 32))]
        O, _ = oracle.vsa_attention(X["q"], X["k"], X["v"], tab["perm"], tab["block_len"], M, idx, num, items=items)
        oracle.add_coarse(np.nan_to_num(O), C, g, tab["perm"], tab["block_len"], M)
        done += len(items)
    t_attn = time.perf_counter() - t1
    per_head_s = t_prep + t_attn * J / done
    flops_head = 4.0 * w.N * w.D * w.R * M + 2.0 * J * J * w.D
    return _baseline(round(flops_head / per_head_s / 1e12, 6), "TFLOP/s",
                     "head 0 of the video workload: float64 route, TopK and coarse branch over all %d blocks (%.1f s) "
                     "and attention plus the gated branch for %d of %d query blocks (%.1f s), scaled to one head"
                     % (J, t_prep, done, J, t_attn), {"ms_per_head": round(per_head_s * 1e3, 1)})


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
                       kmax=J, scale=1.0 / D ** 0.5, q2k_idx=Pp(q2k_idx), q2k_num=Pp(q2k_num), item_order=Pp(order),
                       no_fill=1)   # the attention reads only the first q2k_num entries of a row
    nws = ctypes.c_size_t()
    L.check(lib.h3_pool_route_topk_ws(ctypes.byref(ra), ctypes.byref(nws)))
    ws = torch.empty(nws.value, dtype=torch.uint8, device=dev)

    def route():
        L.check(lib.h3_pool_route_topk(ctypes.byref(ra), Pp(ws), nws.value, s_ptr))

    qa = bsa.api._qouter_args(q, k, v, out, 1.0 / D ** 0.5, L.BSA_SEL_BLOCK, None)
    qa.perm, qa.block_len, qa.J, qa.M = Pp(geom.perm), Pp(geom.block_len), J, M
    qa.q2k_idx, qa.q2k_num, qa.kmax = Pp(q2k_idx), Pp(q2k_num), J
    qa.item_order = Pp(order)
    qa.order_long = P  # the context query blocks (every block kept) start first
    qws = bsa.qouter_workspace(dev)

    def attend():
        L.check(lib.bsa_forward_qouter(ctypes.byref(qa), Pp(qws), qws.numel(), s_ptr))

    ms_step, ms, stats = time_stages((("tile", tile), ("route", route), ("attn", attend)), args, stream)
    pairs_nominal = float(q2k_num.sum().item())          # kept (query block, key block) pairs
    flops = 4.0 * D * M * M * pairs_nominal              # every pair counted as full blocks
    valid_flops = 4.0 * D * bsa.metrics.vsa_valid_pairs(geom.block_len, q2k_idx, q2k_num)
    route_bytes = 2 * q.numel() * q.element_size() + 2 * B * h * J * D * 4 + 4 * pairs_nominal
    roof = _roofline_mfma(ATTN_KERNEL + " over the grouped index table (bsa_forward_qouter, block mode)", valid_flops,
                          flops, ms["attn"], _profiled_traffic(ATTN_KERNEL + "_h3.md", ATTN_SOURCES))
    config = {"workload": "h3_r2v_multi_region", "B": B, "heads": h,
              "segments": [s_ if isinstance(s_, int) else list(s_) for s_ in cfg["segments"]],
              "block": list(cfg["block"]), "D": D, "J": J, "M": M, "tokens": N, "prefix_blocks": P,
              "video_spans": [list(sp) for sp in geom.spans], "budgets": budgets}
    res = _line(args, flops / (ms_step * 1e-3) / 1e12, ms_step, config,
                "synthetic (seeded N(0,1) + per-cell offsets in the video regions, no dataset or weights)", ms, stats,
                roof, {"route_gbps": _gbps(route_bytes, ms["route"]), "pct_hbm_route": _pct_hbm(route_bytes,
                                                                                                ms["route"])})
    return res, dict(cfg=cfg, x=x, budgets=budgets)


def cpu_baseline_h3(ctx, budget_s):
    """Oracle on a bounded sample: head 0's layout, pooling and grouped routing
    over all blocks, and attention for as many query blocks as fit."""
    import numpy as np
    import oracle
    cfg = ctx["cfg"]
    D = cfg["D"]
    X = _f64_head(ctx["x"])
    t0 = time.perf_counter()
    lay = oracle.h3_layout(cfg["segments"], cfg["block"])
    J, M = lay["J"], lay["M"]
    qbar = oracle.pool_blocks(X["q"], lay["perm"], lay["block_len"], M)
    kbar = oracle.pool_blocks(X["k"], lay["perm"], lay["block_len"], M)
    idx, num, _ = oracle.h3_route(qbar, kbar, lay["num_prefix"], lay["spans"], ctx["budgets"])
    t_route = time.perf_counter() - t0
    order = np.random.default_rng(0).permutation(J)  # a random sample of query blocks of every kind
    done, pairs_done = 0, 0
    t1 = time.perf_counter()
    while done < J and time.perf_counter() - t1 < budget_s:
        blocks = order[done:done + 16]
        oracle.vsa_attention(X["q"], X["k"], X["v"], lay["perm"], lay["block_len"], M, idx, num,
                             items=[(0, 0, int(i)) for i in blocks])
        pairs_done += int(num[0, 0, blocks].sum())
        done += len(blocks)
    t_attn = time.perf_counter() - t1
    pairs_head = float(num[0, 0].sum())
    per_head_s = t_route + t_attn * pairs_head / max(pairs_done, 1)
    flops_head = 4.0 * D * M * M * pairs_head
    return _baseline(round(flops_head / per_head_s / 1e12, 6), "TFLOP/s",
                     "head 0 of the h3 workload: float64 layout, pooling and grouped routing over all %d blocks "
                     "(%.1f s) and attention for %d random query blocks (%d of %d kept pairs, %.1f s), scaled to one "
                     "head by kept pairs" % (J, t_route, done, pairs_done, int(pairs_head), t_attn),
                     {"ms_per_head": round(per_head_s * 1e3, 1)})


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
        L.check(lib.bsa_forward_qouter(ctypes.byref(qa), P(qws), qws.numel(), s_ptr))

    ms_step, ms, stats = time_stages((("reblock", reblock), ("route", route), ("attn", attend)), args, stream)
    flops = 4.0 * B * h * N * D * R * M
    valid = 4.0 * D * bsa.metrics.vsa_valid_pairs(block_len, q2k_idx, q2k_num)
    roof = _roofline_mfma(ATTN_KERNEL + " over per-head reblocked tables (bsa_forward_qouter, block mode)", valid, flops,
                          ms["attn"], _profiled_traffic(ATTN_KERNEL + "_reblock.md", ATTN_SOURCES))
    config = {"workload": "video_dit_vsa_spark_reblock", "B": B, "heads": h, "grid": list(cfg["grid"]),
              "D": D, "J": J, "M": M, "R": R, "tokens": N, "tree_levels": nl.value}
    res = _line(args, flops / (ms_step * 1e-3) / 1e12, ms_step, config, DATA_VIDEO, ms, stats, roof)
    return res, dict(cfg=cfg, x=x)


def cpu_baseline_reblock(ctx, budget_s):
    """Oracle on a bounded sample: head 0's moment, features and tree over all
    115200 tokens, then pooling, routing and attention for as many query
    blocks as fit."""
    import oracle
    from oracle import reblock as rbo
    cfg = ctx["cfg"]
    D, R, M = cfg["D"], cfg["R"], 64
    X = _f64_head(ctx["x"])
    N = X["q"].shape[1]
    t0 = time.perf_counter()
    U = rbo.key_features(X["k"], X["q"])[0, 0]
    perm, block_len = rbo.reblock_tables(rbo.reblock_orders(U, M)[-1], M)
    J = len(block_len)
    qbar = oracle.pool_blocks(X["q"], perm, block_len, M)
    kbar = oracle.pool_blocks(X["k"], perm, block_len, M)
    idx, num, _ = oracle.select_topk(oracle.routing_matrix(qbar, kbar), R)
    t_prep = time.perf_counter() - t0
    done = 0
    t1 = time.perf_counter()
    while done < J and time.perf_counter() - t1 < budget_s:
        items = [(0, 0, i) for i in range(done, min(J, done + 32))]
        oracle.vsa_attention(X["q"], X["k"], X["v"], perm, block_len, M, idx, num, items=items)
        done += len(items)
    t_attn = time.perf_counter() - t1
    per_head_s = t_prep + t_attn * J / done
    flops_head = 4.0 * N * D * R * M
    return _baseline(round(flops_head / per_head_s / 1e12, 6), "TFLOP/s",
                     "head 0 of the video workload: float64 reblock layout, pooling, routing and TopK over all %d "
                     "blocks (%.1f s) and attention for %d of %d query blocks (%.1f s), scaled to one head"
                     % (J, t_prep, done, J, t_attn), {"ms_per_head": round(per_head_s * 1e3, 1)})


# ---------------------------------------------------------------------------- NSA / MSA

def _kvouter_stages(bsa, q, k, v, sel, cnt, BK, causal, dev):
    """Stages of the KV-outer schedule + combine for one selection table."""
    import ctypes
    import torch
    B, N, Hq, D = q.shape
    Hkv, ks = k.shape[2], sel.shape[-1]
    bufs = (torch.empty((B, ks, N, Hq, D), dtype=torch.bfloat16, device=dev),
            torch.empty((B, ks, N, Hq), dtype=torch.float32, device=dev),
            torch.empty((B, N, Hkv), dtype=torch.int32, device=dev))
    out = torch.empty_like(q)
    a = bsa.api._kv_args(q, k, v, sel, BK, causal, cnt, 1.0 / D ** 0.5, 0, *bufs)
    n = ctypes.c_size_t()
    L = bsa._lib
    L.check(L.load().bsa_kvouter_ws(ctypes.byref(a), ctypes.byref(n)))
    ws = torch.empty(n.value, dtype=torch.uint8, device=dev)

    def k1():
        bsa.kvouter(q, k, v, sel, BK, causal=causal, q2k_cnt=cnt, bufs=bufs, workspace=ws)

    def k2():
        bsa.combine(*bufs, Hkv, out=out)

    return (("kvouter_k1", k1), ("combine_k2", k2))


def _kv_bytes(q, k, sel, cnt, G):
    """Algorithmic bytes of K1 (the page's I/O model: K/V once, Q per edge,
    O_buf + LSE per edge) and of K2 (partials read once, O written)."""
    import torch
    S = sel.shape[-1]
    live = sel >= 0
    if cnt is not None:
        live &= torch.arange(S, device=sel.device) < cnt[..., None]
    edges = int(live.sum().item())
    D = q.shape[-1]
    k1 = 2 * k.numel() * 2 + edges * G * D * 2 * 2 + edges * G * 4
    k2 = edges * G * (D * 2 + 4) + q.numel() * 2 + sel[..., 0].numel() * 4
    return edges, k1, k2


def bench_nsa(args):
    """NSA selected branch, 32768 tokens: token-mode query-outer attention, or
    the same selections through the KV-outer schedule + combine."""
    import torch
    import block_sparse_attention_02_amd as bsa
    from workloads import nsa_inputs, workload

    cfg = workload("nsa")
    dev = torch.device("cuda:0")
    q, k, v, idx, cnt = nsa_inputs(cfg, device=dev)
    T, BS, D = cfg["T"], cfg["BS"], cfg["D"]
    G = cfg["HQ"] // cfg["H"]
    stream = torch.cuda.current_stream(dev)
    nominal = bsa.metrics.nsa_nominal_flops(cnt, BS, G, D)
    valid = 4.0 * D * bsa.metrics.selection_valid_pairs(idx, cnt, BS, T, G, causal=True)
    config = {"workload": "nsa_selected_branch", "schedule": args.schedule, "T": T, "HQ": cfg["HQ"], "H": cfg["H"],
              "D": D, "BS": BS, "S": cfg["S"], "causal": True}
    data = "synthetic (seeded N(0,1), random causal selections)"
    if args.schedule == "kvouter":
        ms_step, ms, stats = time_stages(_kvouter_stages(bsa, q, k, v, idx, cnt, BS, True, dev), args, stream)
        edges, k1b, k2b = _kv_bytes(q, k, idx, cnt, G)
        t_attn = ms["kvouter_k1"] + ms["combine_k2"]
        roof = _roofline_hbm("kv_k1w_kernel (bsa_forward_kvouter, BK = 64)", k1b, ms["kvouter_k1"],
                             _profiled_traffic("kv_k1w_kernel_nsa.md", KV_SOURCES))
        extra = {"edges": edges, "k1_gbps_algorithmic": _gbps(k1b, ms["kvouter_k1"]),
                 "k2_gbps_algorithmic": _gbps(k2b, ms["combine_k2"]),
                 "k1_tflops_valid": round(valid / (ms["kvouter_k1"] * 1e-3) / 1e12, 2),
                 "pct_bf16_peak_valid": round(100 * valid / (t_attn * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}
    else:
        out = torch.empty_like(q)

        def attend():
            bsa.attention_nsa(q, k, v, idx, cnt, BS, out=out)

        ms_step, ms, stats = time_stages((("attn", attend),), args, stream)
        nbytes = 2 * q.numel() * 2 + 2 * k.numel() * 2 + idx.numel() * 4 + cnt.numel() * 4
        roof = _roofline_mfma("nsa_attn_kernel (bsa_forward_qouter, token mode)", valid, nominal, ms["attn"],
                              _profiled_traffic("nsa_attn_kernel_nsa.md", ("attn_nsa.hip", "bsa_device.hpp",
                                                                           "bsa_internal.hpp")))
        extra = {"hbm_gbps_algorithmic": _gbps(nbytes, ms["attn"])}
    res = _line(args, nominal / (ms_step * 1e-3) / 1e12, ms_step, config, data, ms, stats, roof, extra)
    return res, dict(cfg=cfg, q=q, k=k, v=v, idx=idx, cnt=cnt)


def cpu_baseline_nsa(ctx, budget_s):
    """Oracle on a bounded sample: the float64 NSA definition for as many
    tokens (drawn at random over the sequence, so their selection counts and
    causal spans are representative) as fit the budget."""
    import numpy as np
    import oracle
    cfg = ctx["cfg"]
    T, BS, D = cfg["T"], cfg["BS"], cfg["D"]
    G = cfg["HQ"] // cfg["H"]
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    Q, K, V = f64(ctx["q"]), f64(ctx["k"]), f64(ctx["v"])
    idx, cnt = ctx["idx"].cpu().numpy(), ctx["cnt"].cpu().numpy()
    order = np.random.default_rng(0).permutation(T)
    done, blocks = 0, 0
    t0 = time.perf_counter()
    while done < T and time.perf_counter() - t0 < budget_s:
        toks = order[done:done + 64]
        oracle.nsa_attention(Q, K, V, idx, cnt, BS, causal=True, tokens=[(0, int(t)) for t in toks])
        blocks += int(cnt[0, toks].sum())
        done += len(toks)
    dt = time.perf_counter() - t0
    flops = 4.0 * G * D * BS * blocks
    return _baseline(round(flops / dt / 1e12, 6), "TFLOP/s",
                     "float64 NSA definition for %d random tokens of %d (all 64 query heads, %d selected blocks, "
                     "%.1f s); the GPU line's nominal FLOP count" % (done, T, blocks, dt),
                     {"ms_per_layer_scaled": round(dt * 1e3 * T / done, 1)})


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
    stream = torch.cuda.current_stream(dev)
    ms_step, ms, stats = time_stages(_kvouter_stages(bsa, q, k, v, q2k, None, BK, True, dev), args, stream)
    edges, k1b, k2b = _kv_bytes(q, k, q2k, None, G)
    nominal = bsa.metrics.kvouter_nominal_flops(q2k, BK, G, D)
    valid = 4.0 * D * bsa.metrics.selection_valid_pairs(q2k, None, BK, N, G, causal=True)
    # the timed K1 call also runs the reverse index and the scheduler (about 2 % of it)
    roof = _roofline_hbm("kv_k1w_kernel (bsa_forward_kvouter)", k1b, ms["kvouter_k1"],
                         _profiled_traffic("kv_k1w_kernel_msa.md", KV_SOURCES))
    config = {"workload": "msa_kv_outer", "N": N, "Hq": Hq, "Hkv": Hkv, "D": D, "BK": BK, "k": ks, "edges": edges}
    t_attn = ms["kvouter_k1"] + ms["combine_k2"]
    res = _line(args, nominal / (ms_step * 1e-3) / 1e12, ms_step, config,
                "synthetic (seeded N(0,1), sink + local + Zipf(1.1) selections)", ms, stats, roof,
                {"k1_tflops_nominal": round(nominal / (ms["kvouter_k1"] * 1e-3) / 1e12, 2),
                 "k1_tflops_valid": round(valid / (ms["kvouter_k1"] * 1e-3) / 1e12, 2),
                 "pct_bf16_peak_valid": round(100 * valid / (t_attn * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                 "k1_gbps_algorithmic": _gbps(k1b, ms["kvouter_k1"]),
                 "k2_gbps_algorithmic": _gbps(k2b, ms["combine_k2"]),
                 "pct_hbm_k2": _pct_hbm(k2b, ms["combine_k2"])})
    return res, dict(cfg=cfg, q=q, k=k, v=v, q2k=q2k)


def cpu_baseline_msa(ctx, budget_s):
    """Oracle on a bounded sample: the float64 K1 partials (per selected block,
    the local softmax) and the exact LSE combine for as many positions
    (drawn at random over the sequence) as fit the budget."""
    import numpy as np
    import oracle
    cfg = ctx["cfg"]
    N, BK, D = cfg["N"], cfg["BK"], cfg["D"]
    G = cfg["Hq"] // cfg["Hkv"]
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    Q, K, V = f64(ctx["q"]), f64(ctx["k"]), f64(ctx["v"])
    q2k = ctx["q2k"].cpu().numpy()
    order = np.random.default_rng(0).permutation(N)
    done, edges = 0, 0
    t0 = time.perf_counter()
    while done < N and time.perf_counter() - t0 < budget_s:
        rows = order[done:done + 32]
        O, Lb, ns = oracle.kvouter_partials(Q, K, V, q2k, BK, causal=True, positions=[(0, int(i)) for i in rows])
        # compact rows [P, ks, ...] seen as one batch entry of P positions
        oracle.lse_combine(O.transpose(1, 0, 2, 3)[None], Lb.transpose(1, 0, 2)[None], ns[None], G)
        edges += int((q2k[0, rows] >= 0).sum())
        done += len(rows)
    dt = time.perf_counter() - t0
    flops = 4.0 * G * D * BK * edges
    return _baseline(round(flops / dt / 1e12, 6), "TFLOP/s",
                     "float64 K1 partials + LSE combine for %d random positions of %d (all 64 query heads, %d "
                     "selections, %.1f s); the GPU line's nominal FLOP count" % (done, N, edges, dt),
                     {"ms_per_layer_scaled": round(dt * 1e3 * N / done, 1)})


# ---------------------------------------------------------------------------- main

BENCHES = {
    "video": (bench_video, cpu_baseline_video),
    "reweight": (bench_reweight, cpu_baseline_reweight),
    "coarse": (bench_coarse, cpu_baseline_coarse),
    "h3": (bench_h3, cpu_baseline_h3),
    "reblock": (bench_reblock, cpu_baseline_reblock),
    "nsa": (bench_nsa, cpu_baseline_nsa),
    "msa": (bench_msa, cpu_baseline_msa),
}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="video", choices=sorted(BENCHES))
    ap.add_argument("--schedule", default="qouter", choices=["qouter", "kvouter"],
                    help="nsa only: query-outer token mode, or the KV-outer schedule + combine")
    ap.add_argument("--cold-reps", type=int, default=10,
                    help="runs of every call after a 512 MiB cache scrub (0: none)")
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
    bench, baseline = BENCHES[args.workload]
    res, ctx = bench(args)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = baseline(ctx, args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

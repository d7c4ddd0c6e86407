"""Benchmark of one TSP rank's layer forward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--rank R]
                [--no-cpu-baseline] [--cpu-rows N] [--calib-copy] [--sweep PATH]
                [--gemm-yardstick] [--streamed] [--chunked] [--memory PATH] [--attn-bwd] [--layer-bwd]

A step is one tsp_layer_fwd call: QKV projection of the rank's zigzag shard, causal
attention against the full-sequence K/V, W_O, and the D-shard SwiGLU ring accumulated in
fp32 (TSP summary "Folding Tensor and Sequence Parallelism ...", §2). Inputs are seeded
synthetic tensors already resident in HBM; the peers' K/V rows (what the all-gather
delivers) are filled before timing by the peers' own QKV projections.

Prints ONE JSON line: whole-step throughput in TFLOP/s of algorithmic work (exact
causal pairs) at the median step time (each of the K timed steps has its own pair of HIP
events on the launch stream; min, max and mean are reported beside it), the attention
kernel's roofline, and the CPU oracle timed on a bounded sample of the same workload
(cores = the host CPUs this process may run on). The attention time is the average over
the K timed steps of the library's own phase events, recorded on the launch stream around
the attention launch inside each tsp_layer_fwd call (tsp_timing_start / tsp_timing_read). The
roofline's HBM traffic comes from the committed FETCH_SIZE / WRITE_SIZE counter summary
of the attention kernel, and is reported only while the kernel's sources still hash to
the value recorded there.

--calib-copy runs, before the timed steps, one plain device copy of 256 MiB (fp32
negation: 256 MiB read, 256 MiB written) whose counter readings calibrate FETCH_SIZE and
WRITE_SIZE into bytes.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CUs x 2.4 GHz x 4096 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0
METRIC = "TSP rank-shard layer fwd TFLOP/s (% bf16 MFMA peak), 7B layer, S=16K-128K"
DEFAULT_WORKLOAD = "7b_s128k_d8"
PKG = os.path.join(ROOT, "long_context_transformer_amd")
# What determines the attention kernel's code: its source, the device header it includes
# and its compile flags. The counter summary records their hash.
ATTN_SOURCES = [os.path.join(PKG, "csrc", "tsp_attn.hip"), os.path.join(PKG, "csrc", "tsp_device.h")]
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "attn_fwd_7b_s128k_d8_hbm_traffic.md")
CALIB_MIB = 256


def layer_flops(B, S, D, d, H, hd, F):
    """Algorithmic FLOPs of one rank's layer: QKV + causal attention (C(S+1) exact pairs
    per sequence and head, 2 matmuls) + W_O + SwiGLU over all D shards."""
    C = S // (2 * D)
    M = B * 2 * C
    attn = 4 * B * H * hd * C * (S + 1)
    return 2 * M * d * 3 * d + attn + 2 * M * d * d + 6 * M * d * F, attn


def setup(w, rank):
    import torch
    from long_context_transformer_amd import synth, tsp
    t0 = time.time()
    inp = synth.layer_inputs(w)
    dev = {k: synth.to_torch(v).cuda() for k, v in inp.items()}
    B, S, D, H, hd, d, F = w.B, w.S, w.D, w.n_heads, w.head_dim, w.d_model, w.ffn
    Fs = F // D
    kf = torch.empty((B, S, d), dtype=torch.bfloat16, device="cuda")
    vf = torch.empty_like(kf)
    for peer in range(D):
        if peer != rank:
            idx = torch.from_numpy(tsp.zigzag_index(S, D, peer)).cuda()
            tsp.qkv_fwd(dev["x_full"].index_select(1, idx).contiguous(), dev["w_qkv"], None, kf, vf,
                        B, S, D, peer, H, hd)
    idx = torch.from_numpy(tsp.zigzag_index(S, D, rank)).cuda()
    xs = dev["x_full"].index_select(1, idx).contiguous()
    st = {
        "inputs": inp, "dev": dev, "kf": kf, "vf": vf, "xs": xs,
        "w1": [dev["w1"][j * Fs:(j + 1) * Fs] for j in range(D)],
        "w3": [dev["w3"][j * Fs:(j + 1) * Fs] for j in range(D)],
        "w2": [dev["w2"][:, j * Fs:(j + 1) * Fs].contiguous() for j in range(D)],
        "desc": tsp.make_desc(B, S, D, rank, d, H, hd, F),
        "attn_out": torch.empty((B, S // D, d), dtype=torch.bfloat16, device="cuda"),
        "mlp_out": torch.empty((B, S // D, d), dtype=torch.float32, device="cuda"),
    }
    st["ws"] = torch.empty(tsp.layer_workspace_size(st["desc"]), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    st["setup_s"] = time.time() - t0
    return st


def step(st):
    from long_context_transformer_amd import tsp
    tsp.layer_fwd(st["desc"], st["xs"], st["dev"]["w_qkv"], st["dev"]["w_o"], st["w1"], st["w3"],
                  st["w2"], st["kf"], st["vf"], st["attn_out"], st["mlp_out"], st["ws"])


def time_layer(st, steps, warmup, warmup_s=0.0):
    """Times `steps` steps, each between its own pair of HIP events on the launch stream
    (torch's current stream, which the library launches on). Returns per-step statistics
    (median, min, max, mean, and the whole timed region) in ms, the wall time, and the
    per-phase averages from the library's events recorded inside those same steps.
    Untimed warmup: `warmup` steps, then more until `warmup_s` seconds have passed (the
    GPU's clock takes some tens of ms of work to settle; short steps need more of them)."""
    import statistics
    import torch
    from long_context_transformer_amd import tsp
    for _ in range(warmup):
        step(st)
    torch.cuda.synchronize()
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < warmup_s:
        for _ in range(5):
            step(st)
        torch.cuda.synchronize()
    tsp.timing_start(steps)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    marks = [(ev(), ev()) for _ in range(steps)]
    ev0, ev1 = ev(), ev()
    wall0 = time.perf_counter()
    ev0.record()
    for e0, e1 in marks:
        e0.record()
        step(st)
        e1.record()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per = [e0.elapsed_time(e1) for e0, e1 in marks]
    stats = {"median": statistics.median(per), "min": min(per), "max": max(per),
             "mean": sum(per) / len(per), "region": ev0.elapsed_time(ev1)}
    calls = tsp.timing_read(steps)
    phases = {p: sum(c[p] for c in calls) / len(calls) for p in tsp.PHASES}
    return stats, wall, phases


def calib_copy():
    """One plain copy kernel of known size (CALIB_MIB read, CALIB_MIB written)."""
    import torch
    n = CALIB_MIB * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def attn_sources_hash():
    """sha256 of the attention kernel's source, its device header and its hipcc flags (paths
    relative to the repository, so that the value does not depend on where it is checked out)."""
    from long_context_transformer_amd import build as tsp_build
    h = hashlib.sha256()
    for p in ATTN_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    flags = tsp_build.HIPCC_FLAGS + tsp_build.SOURCE_FLAGS.get("tsp_attn.hip", [])
    h.update("\0".join(f.replace(tsp_build.ROOT, ".") for f in flags).encode())
    return h.hexdigest()


def attn_traffic(workload):
    """HBM bytes per attention launch from the committed counter summary, or None when the
    summary is absent, covers another workload, or the kernel's sources have changed."""
    if workload != DEFAULT_WORKLOAD or not os.path.exists(TRAFFIC_SUMMARY):
        return None
    text = open(TRAFFIC_SUMMARY).read()
    src = re.search(r"^source_sha256:\s*([0-9a-f]{64})", text, re.M)
    val = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not src or not val or src.group(1) != attn_sources_hash():
        return None
    return float(val.group(1))


def arrival_order(D, r):
    """All-gather arrival order of the 2D zigzag chunks: the rank's own two, then the chunk
    pairs of ranks r-1, r-2, ... around the ring."""
    order = [r, 2 * D - 1 - r]
    for t in range(1, D):
        p = (r - t) % D
        order += [p, 2 * D - 1 - p]
    return order


def time_chunked(st, w, rank, reps=3, fused=True):
    """Chunked-arrival attention: tsp_attn_fwd_range per zigzag chunk in arrival order,
    merged into an fp32 accumulator (fused: by the range launch itself; otherwise by a
    tsp_attn_merge launch after each), bf16 O after the last chunk. Times the whole
    pipeline, the range launches and the merges (HIP events on the launch stream), and the
    single-launch attention on the same Q/K/V for comparison."""
    import torch
    from long_context_transformer_amd import tsp
    B, S, D, H, hd, C = w.B, w.S, w.D, w.n_heads, w.head_dim, w.C
    R = S // D
    q = torch.empty((B, R, H * hd), dtype=torch.bfloat16, device="cuda")
    tsp.qkv_fwd(st["xs"], st["dev"]["w_qkv"], q, st["kf"], st["vf"], B, S, D, rank, H, hd)
    acc_o = torch.empty((B, R, H, hd), dtype=torch.float32, device="cuda")
    acc_l = torch.empty((B, H, R), dtype=torch.float32, device="cuda")
    po, pl = torch.empty_like(acc_o), torch.empty_like(acc_l)
    out = torch.empty((B, R, H, hd), dtype=torch.bfloat16, device="cuda")
    bounds = [(c * C, (c + 1) * C) for c in arrival_order(D, rank)]
    ev = lambda: torch.cuda.Event(enable_timing=True)
    t_range = t_merge = t_total = 0.0
    for rep in range(reps + 1):
        acc_o.zero_()
        acc_l.fill_(float("-inf"))
        torch.cuda.synchronize()
        e_all0, e_all1 = ev(), ev()
        marks = []
        e_all0.record()
        for n, (lo, hi) in enumerate(bounds):
            e0, e1, e2 = ev(), ev(), ev()
            last = out if n == len(bounds) - 1 else None
            e0.record()
            if fused:
                tsp.attn_fwd_range(q, st["kf"], st["vf"], acc_o, acc_l, B, S, D, rank, H, hd, lo, hi,
                                   accumulate=True, o_out=last)
                e1.record()
            else:
                tsp.attn_fwd_range(q, st["kf"], st["vf"], po, pl, B, S, D, rank, H, hd, lo, hi)
                e1.record()
                tsp.attn_merge(acc_o, acc_l, po, pl, last, B, S, D, H, hd)
            e2.record()
            marks.append((e0, e1, e2))
        e_all1.record()
        torch.cuda.synchronize()
        if rep == 0:
            continue  # warm-up pass
        t_total += e_all0.elapsed_time(e_all1)
        t_range += sum(a.elapsed_time(b) for a, b, _ in marks)
        t_merge += sum(b.elapsed_time(c) for _, b, c in marks)
    t_total, t_range, t_merge = t_total / reps, t_range / reps, t_merge / reps
    mono = torch.empty_like(out)
    tsp.attn_fwd(q, st["kf"], st["vf"], mono, None, B, S, D, rank, H, hd)
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    e0.record()
    for _ in range(reps):
        tsp.attn_fwd(q, st["kf"], st["vf"], mono, None, B, S, D, rank, H, hd)
    e1.record()
    torch.cuda.synchronize()
    t_mono = e0.elapsed_time(e1) / reps
    diff = float((out.float() - mono.float()).abs().max())
    res = {"chunks": len(bounds), "order": "own chunks, then ring", "fused_merge": fused,
           "ms": round(t_total, 4), "range_launches_ms": round(t_range, 4),
           "single_launch_ms": round(t_mono, 4), "overhead_pct": round(100 * (t_total / t_mono - 1), 2),
           "max_abs_diff_vs_single_launch": diff}
    if not fused:
        # merge traffic per launch: fp32 O read twice and written once, lse read twice and
        # written once; the last merge also writes the bf16 O (counted once)
        n_el = B * R * H * hd
        merge_bytes = len(bounds) * (12 * n_el + 12 * B * H * R) + 2 * n_el
        merge_gbs = merge_bytes / (t_merge * 1e-3) / 1e9
        res["merges_ms"] = round(t_merge, 4)
        res["merge_roofline"] = {"bound": "hbm", "achieved": round(merge_gbs, 1), "peak": PEAK_HBM_GBS,
                                 "unit": "GB/s", "frac": round(merge_gbs / PEAK_HBM_GBS, 4),
                                 "bytes_per_merge": 12 * n_el + 12 * B * H * R}
    return res


def time_streamed(st, w, steps, warmup):
    """Weight-streamed layer (tsp_layer_fwd_streamed): two receive slots per weight kind,
    shard copies on a copy stream, head groups alternating between two attention streams,
    W_O partials on a fourth;
    timed against the same call on one stream (no overlap) and against tsp_layer_fwd with
    every shard resident. Also reports the resident weight bytes of both layouts."""
    import torch
    from long_context_transformer_amd import tsp
    D = w.D
    dev = st["dev"]
    pa = tsp.pack_attn_shards(dev["w_qkv"], dev["w_o"], D)
    pm = tsp.pack_mlp_shards(dev["w1"], dev["w3"], dev["w2"], D)
    ws = torch.empty(tsp.layer_streamed_workspace_size(st["desc"]), dtype=torch.uint8, device="cuda")
    streams = [torch.cuda.Stream() for _ in range(3)]
    a, y = st["attn_out"], st["mlp_out"]
    a_ref, y_ref = a.clone(), y.clone()  # tsp_layer_fwd's outputs from the timed steps

    def run(overlap):
        tsp.layer_fwd_streamed(st["desc"], st["xs"], pa, pm, st["kf"], st["vf"], a, y, ws,
                               streams=streams if overlap else None)

    res = {}
    for name, overlap in (("four_streams", True), ("one_stream", False)):
        for _ in range(warmup):
            run(overlap)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            run(overlap)
        e1.record()
        torch.cuda.synchronize()
        res[name + "_ms"] = round(e0.elapsed_time(e1) / steps, 4)
    da = float((a.float() - a_ref.float()).abs().max() / a_ref.float().abs().max())
    dy = float((y - y_ref).abs().max() / y_ref.abs().max())
    slot_a = pa[0].numel() * 2
    slot_m = pm[0].numel() * 2
    res.update({
        "copied_bytes_per_step": D * (slot_a + slot_m),
        "resident_weight_bytes": 2 * (slot_a + slot_m),
        "resident_weight_bytes_all_shards": sum(dev[k].numel() * 2 for k in ("w_qkv", "w_o", "w1", "w3", "w2")),
        "workspace_bytes": ws.numel(),
        "workspace_bytes_all_shards": st["ws"].numel(),
        "max_rel_diff_vs_resident": {"attn_out": da, "mlp_out": dy},
    })
    return res


def time_attn_bwd(st, w, rank, reps=3):
    """Attention backward (tsp_attn_bwd) on the layer's Q/K/V: the forward with its
    log-sum-exp once, then `reps` timed backward calls (HIP events on the launch stream).
    FLOPs counted the usual way for attention backward: 2.5x the forward's exact causal
    pairs (five products of hd per pair: the recomputed scores, dV, dP, dQ, dK)."""
    import torch
    from long_context_transformer_amd import tsp
    B, S, D, H, hd = w.B, w.S, w.D, w.n_heads, w.head_dim
    R = S // D
    q = torch.empty((B, R, H * hd), dtype=torch.bfloat16, device="cuda")
    tsp.qkv_fwd(st["xs"], st["dev"]["w_qkv"], q, st["kf"], st["vf"], B, S, D, rank, H, hd)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, R), dtype=torch.float32, device="cuda")
    tsp.attn_fwd(q, st["kf"], st["vf"], o, lse, B, S, D, rank, H, hd)
    g = torch.randn((B, R, H * hd), device="cuda", generator=torch.Generator("cuda").manual_seed(5)).to(torch.bfloat16)
    dq = torch.empty((B, R, H * hd), dtype=torch.float32, device="cuda")
    dk = torch.empty((B, S, H * hd), dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    ws = torch.empty(tsp.attn_bwd_workspace_size(B, S, D, H), dtype=torch.uint8, device="cuda")
    run = lambda: tsp.attn_bwd(q, st["kf"], st["vf"], o, lse, g, dq, dk, dv, B, S, D, rank, H, hd, ws)
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    _, attn_fwd_flops = layer_flops(B, S, D, w.d_model, H, hd, w.ffn)
    fl = 2.5 * attn_fwd_flops
    tf = fl / (ms * 1e-3) / 1e12
    del q, o, lse, g, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return {"ms": round(ms, 3), "flops": fl, "tflops": round(tf, 1), "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
            "note": "two launches: dq (query-stationary), dk/dv (key-stationary); fp32 gradients"}


def time_layer_bwd(st, w, rank, reps=3):
    """Backward of the rank's layer: part 1 (MLP ring, W_O, attention) and part 2 (QKV) on
    the layer's own forward activations, timed separately (HIP events on the launch stream).
    The dK/dV exchange between the parts is outside the timing (another GPU's work). FLOPs
    counted as the usual algorithmic backward: twice the forward GEMMs' FLOPs (an input and
    a weight gradient each) plus 2.5x the forward attention; the recomputation of A and of
    the gate pair is extra work not counted."""
    import torch
    from long_context_transformer_amd import tsp
    B, S, D, H, hd, d, F = w.B, w.S, w.D, w.n_heads, w.head_dim, w.d_model, w.ffn
    R, Fs = S // D, F // D
    dev = st["dev"]
    q = torch.empty((B, R, d), dtype=torch.bfloat16, device="cuda")
    tsp.qkv_fwd(st["xs"], dev["w_qkv"], q, st["kf"], st["vf"], B, S, D, rank, H, hd)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, R), dtype=torch.float32, device="cuda")
    tsp.attn_fwd(q, st["kf"], st["vf"], o, lse, B, S, D, rank, H, hd)
    packed = tsp.pack_mlp_shards(dev["w1"], dev["w3"], dev["w2"], D)
    gen = torch.Generator("cuda").manual_seed(7)
    dy = torch.randn((B, R, d), device="cuda", generator=gen) * 1e-2
    dq = torch.empty((B, R, d), device="cuda")
    dk = torch.empty((B, S, d), device="cuda")
    dv = torch.empty_like(dk)
    dwo = torch.empty((d, d), device="cuda")
    dw13 = [torch.empty((2 * Fs, d), device="cuda") for _ in range(D)]
    dw2 = [torch.empty((d, Fs), device="cuda") for _ in range(D)]
    dx = torch.empty((B, R, d), device="cuda")
    dwqkv = torch.empty((3 * d, d), device="cuda")
    desc = st["desc"]
    ws = torch.empty(tsp.layer_bwd_workspace_size(desc), dtype=torch.uint8, device="cuda")
    idx = torch.from_numpy(tsp.zigzag_index(S, D, rank)).cuda()
    part1 = lambda: tsp.layer_bwd_attn_mlp(desc, q, o, lse, st["kf"], st["vf"], dev["w_o"], packed, dy, dq, dk, dv,
                                           dwo, dw13, dw2, ws)
    dk_own = dk.index_select(1, idx).contiguous()
    dv_own = dv.index_select(1, idx).contiguous()
    part2 = lambda: tsp.layer_bwd_qkv(desc, st["xs"], dev["w_qkv"], dq, dk_own, dv_own, dx, dwqkv, ws)
    res = {}
    for name, fn in (("attn_mlp", part1), ("qkv", part2)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name + "_ms"] = round(e0.elapsed_time(e1) / reps, 3)
    fwd, attn = layer_flops(B, S, D, d, H, hd, F)
    fl = 2 * (fwd - attn) + 2.5 * attn
    ms = res["attn_mlp_ms"] + res["qkv_ms"]
    tf = fl / (ms * 1e-3) / 1e12
    res.update({"ms": round(ms, 3), "flops": fl, "tflops": round(tf, 1),
                "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)})
    del q, o, lse, packed, dy, dq, dk, dv, dwo, dw13, dw2, dx, dwqkv, ws, dk_own, dv_own
    torch.cuda.empty_cache()
    return res


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            return int(info[0]["num_threads"]), info[0].get("internal_api", "blas")
    except Exception:
        pass
    return len(os.sched_getaffinity(0)), "unknown"


def cpu_baseline(w, inputs, rank, rows_sample):
    """The fp64 oracle on a bounded sample of the same workload: the rank's last
    `rows_sample` local rows (the end of its mirror chunk, the rows with the longest key
    prefix), through QKV, causal attention, W_O and the SwiGLU, with the K/V projection of
    every position those rows see. Returns TFLOP/s of the work the oracle does for it."""
    import numpy as np
    from long_context_transformer_amd import synth
    from oracle import tsp_oracle as O
    R2 = w.rows
    rows = np.arange(R2 - rows_sample, R2)
    idx = O.zigzag_index(w.S, w.D, rank)
    kmax = int(idx[rows].max()) + 1
    b_sel = slice(0, 1)
    f64 = {k: synth.to_f64(v) for k, v in inputs.items() if k != "x_full"}
    x = synth.to_f64(inputs["x_full"][b_sel, :kmax])
    d, H, hd, F = w.d_model, w.n_heads, w.head_dim, w.ffn
    t0 = time.perf_counter()
    # The prefix [0, kmax) as a one-rank sequence: its local rows are positions, so the
    # sampled positions are evaluated with keys 0..position, exactly as in the full layer.
    O.rank_layer(x, f64["w_qkv"], f64["w_o"], f64["w1"], f64["w3"], f64["w2"], kmax, 1, 0, H,
                 rows=idx[rows])
    dt = time.perf_counter() - t0
    pairs = int((idx[rows] + 1).sum())
    R = len(rows)
    flops = (2 * 2 * kmax * d * d + 2 * R * d * d + 4 * H * hd * pairs + 2 * R * d * d
             + 6 * R * d * F)
    threads, api = blas_threads()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": len(os.sched_getaffinity(0)),
            "blas_threads": threads, "kind": "oracle",
            "sample": (f"{w.name} rank {rank}, batch 0: local rows {R2 - R}..{R2 - 1} (positions "
                       f"{int(idx[rows].min())}..{int(idx[rows].max())}) through QKV, causal "
                       f"attention, W_O and SwiGLU, plus K/V projections of positions 0..{kmax - 1}; "
                       f"{flops / 1e9:.1f} GFLOP in {dt:.1f} s, fp64 numpy ({api})"),
            "wall_s": round(dt, 2)}


def gemm_yardstick(st, w, phases, reps=10, warmup=3):
    """The layer's projections as plain 2-D torch.matmul calls (hipBLASLt on ROCm) on the same
    bf16 operands, each timed alone (median of `reps`, HIP events): QKV x W_qkv^T, W_O, the
    gate/up pair of all D shards as one [2F, d] weight, and the down projection over all F
    columns. They do no zigzag scatter, SwiGLU or fp32 accumulation, so they are a yardstick
    for the matrix work only, not the same computation."""
    import torch
    dev = st["dev"]
    M, d, F = w.B * (w.S // w.D), w.d_model, w.ffn
    x = st["xs"].reshape(M, d)
    a_f = torch.randn((M, F), device="cuda").to(torch.bfloat16)
    w13 = torch.cat([dev["w1"], dev["w3"]], 0).contiguous()
    cases = {"qkv": (x, dev["w_qkv"]), "w_o": (x, dev["w_o"]), "gate_up": (x, w13), "down": (a_f, dev["w2"])}
    res = {}
    for name, (a, b) in cases.items():
        bt = b.t()
        for _ in range(warmup):
            torch.matmul(a, bt)
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            torch.matmul(a, bt)
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = sorted(ts)[len(ts) // 2]
        fl = 2.0 * a.shape[0] * a.shape[1] * b.shape[0]
        res[name] = {"ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 1),
                     "shape_mnk": [a.shape[0], b.shape[0], a.shape[1]]}
    res["library_phases_ms"] = {k: round(phases[k], 4) for k in ("qkv", "w_o", "mlp")}
    res["matmul_mlp_ms"] = round(res["gate_up"]["ms"] + res["down"]["ms"], 4)
    del a_f, w13
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=1024)
    ap.add_argument("--chunked", action="store_true",
                    help="also time chunked-arrival attention (range launches + log-sum-exp merges)")
    ap.add_argument("--streamed", action="store_true",
                    help="also time the weight-streamed layer (two slots, copy stream) against this one")
    ap.add_argument("--memory", default=None,
                    help="also measure one rank's device memory for every workload (weight-streamed layer) "
                    "against the analytic per-layout counts; one JSON line each to this file")
    ap.add_argument("--attn-bwd", action="store_true", help="also time the attention backward (tsp_attn_bwd)")
    ap.add_argument("--layer-bwd", action="store_true", help="also time the layer backward (both parts)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 256 MiB plain copy kernel first (counter calibration)")
    ap.add_argument("--sweep", default=None, help="also time every workload (and every rank of the "
                    "S=32K one) and write one JSON line each to this file")
    ap.add_argument("--gemm-yardstick", action="store_true",
                    help="also time the layer's four projections as plain torch.matmul (hipBLASLt) "
                    "on the same operands, beside this library's phases")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one rank's share on ONE GPU; runs on more than one GPU are not "
              "part of this build (see the sharding design notes).", file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_transformer_amd import synth, tsp
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    tsp.load()

    w = synth.WORKLOADS[args.workload].with_rank(args.rank)
    st = setup(w, args.rank)
    print(f"# setup {st['setup_s']:.1f}s", file=sys.stderr, flush=True)
    if args.calib_copy:
        calib_copy()
    stats, wall, phases = time_layer(st, args.steps, args.warmup)
    ms = stats["median"]
    flops, attn_flops = layer_flops(w.B, w.S, w.D, w.d_model, w.n_heads, w.head_dim, w.ffn)
    tflops = flops / (ms * 1e-3) / 1e12
    attn_ms = phases["attention"]
    attn_tflops = attn_flops / (attn_ms * 1e-3) / 1e12
    print(f"# layer {ms:.3f} ms  {tflops:.1f} TFLOP/s  attention {attn_ms:.3f} ms "
          f"{attn_tflops:.1f} TFLOP/s  phases " + " ".join(f"{k}={v:.3f}" for k, v in phases.items()),
          file=sys.stderr, flush=True)
    traffic = attn_traffic(w.name)
    chunked = None
    if args.chunked:
        chunked = time_chunked(st, w, args.rank, fused=True)
        chunked["with_merge_launches"] = time_chunked(st, w, args.rank, fused=False)
        print("# chunked " + json.dumps(chunked), file=sys.stderr, flush=True)

    streamed = None
    if args.streamed:
        streamed = time_streamed(st, w, max(args.steps // 2, 3), 2)
        streamed["resident_ms"] = round(ms, 4)
        streamed["overhead_pct"] = round(100 * (streamed["four_streams_ms"] / ms - 1), 2)
        print("# streamed " + json.dumps(streamed), file=sys.stderr, flush=True)

    attn_bwd = None
    if args.attn_bwd:
        attn_bwd = time_attn_bwd(st, w, args.rank)
        print("# attention backward " + json.dumps(attn_bwd), file=sys.stderr, flush=True)

    layer_bwd = None
    if args.layer_bwd:
        layer_bwd = time_layer_bwd(st, w, args.rank)
        print("# layer backward " + json.dumps(layer_bwd), file=sys.stderr, flush=True)

    yard = None
    if args.gemm_yardstick:
        yard = gemm_yardstick(st, w, phases)
        print("# gemm yardstick " + json.dumps(yard), file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, st["inputs"], args.rank, args.cpu_rows)
        print(f"# cpu baseline {cpu['value']:.4f} TFLOP/s in {cpu['wall_s']} s", file=sys.stderr,
              flush=True)

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "pct_of_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_median": round(stats["median"], 4),
        "ms_min": round(stats["min"], 4),
        "ms_max": round(stats["max"], 4),
        "ms_mean": round(stats["mean"], 4),
        "ms_timed_region": round(stats["region"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02^2) weights, bf16)",
        "config": {"workload": w.name, "batch": w.B, "seq_len": w.S, "fold": w.D, "rank": args.rank,
                   "d_model": w.d_model, "n_heads": w.n_heads, "head_dim": w.head_dim,
                   "ffn": w.ffn, "flops_per_step": flops},
        "phases_ms": {k: round(v, 4) for k, v in phases.items()},
        "roofline": {"kernel": "attention (attn_fwd_w64)", "bound": "mfma",
                     "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "avg_launch_ms": round(attn_ms, 4),
                     "flops_per_launch": attn_flops},
        "cpu_baseline": cpu,
    }
    if chunked:
        out["chunked_attention"] = chunked
    if streamed:
        out["weight_streamed_layer"] = streamed
    if attn_bwd:
        out["attention_backward"] = attn_bwd
    if layer_bwd:
        out["layer_backward"] = layer_bwd
    if yard:
        out["gemm_yardstick"] = yard
    print(json.dumps(out), flush=True)

    if args.memory:
        from long_context_transformer_amd import memory
        del st
        torch.cuda.empty_cache()
        with open(args.memory, "w") as f:
            for name, base in synth.WORKLOADS.items():
                line = memory.measure_streamed(base.with_rank(0), 0)
                f.write(json.dumps(line) + "\n")
                f.flush()
                print("# memory " + json.dumps(line), file=sys.stderr, flush=True)

    if args.sweep:
        with open(args.sweep, "w") as f:
            for name, base in synth.WORKLOADS.items():
                ranks = range(base.D) if name == "7b_s32k_d8" else [0]
                for r in ranks:
                    ww = base.with_rank(r)
                    s2 = setup(ww, r)
                    st2, _, ph2 = time_layer(s2, 10 if ww.S >= 65536 else 20, 3, warmup_s=0.2)
                    ms2 = st2["median"]
                    fl, afl = layer_flops(ww.B, ww.S, ww.D, ww.d_model, ww.n_heads, ww.head_dim, ww.ffn)
                    ams = ph2["attention"]
                    line = {"workload": name, "rank": r, "ms": round(ms2, 4),
                            "tflops": round(fl / ms2 / 1e9, 2),
                            "pct_peak": round(100 * fl / ms2 / 1e9 / PEAK_BF16_TFLOPS, 2),
                            "attn_ms": round(ams, 4), "attn_tflops": round(afl / ams / 1e9, 2),
                            "phases_ms": {k: round(v, 4) for k, v in ph2.items()}}
                    f.write(json.dumps(line) + "\n")
                    f.flush()
                    print("# sweep " + json.dumps(line), file=sys.stderr, flush=True)
                    del s2
                    torch.cuda.empty_cache()


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of one context-parallel rank's exact GQA attention on one MI355X.

Workload timed per step (``prefill_128k_cp4``): one attention layer of a 128K-token causal
prefill with the per-GPU head share of a 128-query-head / 8-KV-head model under TP8 (16 query
heads, 1 KV head, D_H = 128, bf16), sharded over a CP ring of 4 ranks with load-balanced
chunking. A step plays every rank's ring Pass-KV on this one GPU: the rank's 32K-token Q shard
attends to the 4 KV shards of 32K tokens in ring order (by default each ring step folds its
partial into the running (O, LSE); ``--mode partials`` keeps the 4 partials and merges them).
Inputs are seeded synthetic N(0,1) values rounded to bf16, resident in HBM before timing starts.

value = causal-useful TFLOP/s: 4 * D_H flops per visible (query token, query head, key) triple;
masked and skipped work is not counted. The same JSON line reports the dominant kernel's
roofline (cp_partial_attn's MFMA kernel, per-launch time from HIP events on the launch stream),
secondary measurements (split-KV decode GB/s, persistent-KV Pass-Q TFLOP/s, merge GB/s, and with
--extended the 1M-token varlen rank share), the fp64 oracle timed on host cores for a
bounded sample of the same workload, and (with the secondary legs) the MFMA clock probe: the bf16
MFMA rate and shader clock that MFMA-only code sustains on random and on near-constant operands.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk/CU
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
COUNTERS_MD = os.path.join(ROOT, "profiles", "attn_bf16_prefill_128k_cp4_counters.md")


def parse():
    ap = argparse.ArgumentParser(description="one CP rank's ring attention on one MI355X")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--mode", choices=["running", "partials"], default="running",
                    help="fold each ring step into a running (O, LSE) or keep N partials + merge")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--extended", action="store_true", help="also time the 1M-token varlen rank share")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run a 1 GiB device-to-device copy (calibrates HBM byte counters)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-mfma-probe", action="store_true",
                    help="skip the MFMA clock probe (a separate program) in the device figures")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def visible_pairs(q_segs, kv_segs, causal=True):
    """Visible (query token, key) pairs between two shards given their segment tables."""
    total = 0
    for qs, qp, qn, _ in q_segs:
        p = np.arange(qp, qp + qn, dtype=np.int64)
        for ks, kp, kn, _ in kv_segs:
            if ks != qs:
                continue
            total += int(np.clip(p - kp + 1, 0, kn).sum()) if causal else qn * kn
    return total


def recorded_traffic():
    """HBM bytes per launch of the partial-attention kernel from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None if the kernel sources changed
    since the counters were taken."""
    import hashlib
    try:
        text = open(COUNTERS_MD).read()
    except OSError:
        return None
    line = [l for l in text.splitlines() if l.startswith("traffic_record:")]
    if not line:
        return None
    rec = json.loads(line[-1].split(":", 1)[1])
    h = hashlib.sha256()
    for f in rec["files"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != rec["source_sha256"]:
        return None
    return rec


class Timer:
    """HIP events recorded on torch's current stream, which is the stream the library uses."""

    def __init__(self, torch):
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        self.a.record()
        return self

    def __exit__(self, *exc):
        self.b.record()

    def ms(self):
        self.b.synchronize()
        return self.a.elapsed_time(self.b)


def bf16_tokens(torch, si, seed, tid, tokens, shape):
    return si.to_dtype(si.normal_tokens(seed, tid, tokens, shape), "bf16")[0].cuda()


def time_reps(torch, fn, reps, warm=2):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    t = Timer(torch)
    with t:
        for _ in range(reps):
            fn()
    return t.ms() / reps


# --------------------------------------------------------------------------- secondary workloads
def run_decode(torch, cp, si, seed=0):
    cfg = si.CONFIGS["decode_b32_32k_128k"]
    B, n_h, n_kv, d, S = cfg["batch"], cfg["n_h"], cfg["n_kv"], cfg["d_h"], cfg["n_splits"]
    lens = si.decode_lengths(seed, B, cfg["len_lo"], cfg["len_hi"])
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    total = int(lens.sum())
    toks = np.arange(total)
    kc = bf16_tokens(torch, si, seed, si.TID_K, toks, (n_kv, d))
    vc = bf16_tokens(torch, si, seed, si.TID_V, toks, (n_kv, d))
    q = bf16_tokens(torch, si, seed, si.TID_Q, np.arange(B), (n_h, d))
    ws_o, ws_l = cp.decode_workspace(B, n_h, d, S)
    o = torch.empty(B, n_h, d, device="cuda")
    l = torch.empty(B, n_h, device="cuda")
    offs_d = torch.from_numpy(offs).cuda()
    lens_d = torch.from_numpy(lens).cuda()
    scale = 1.0 / math.sqrt(d)
    fn = lambda: cp.decode_splitkv(q, kc, vc, offs_d, lens_d, S, scale, ws_o, ws_l, o, l)
    ms = time_reps(torch, fn, 20)
    kv_bytes = total * n_kv * d * 2 * 2
    alg_bytes = kv_bytes + B * n_h * d * 2 + B * n_h * (d * 4 + 4)
    ws_bytes = cp.decode_workspace_bytes(B, n_h, d, S)
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    log(f"decode: {ms * 1e3:.1f} us, {gbs:.0f} GB/s ({100 * gbs / PEAK_HBM_GBS:.1f}% of HBM), "
        f"{total} cached keys")
    return {"metric": "decode KV GB/s", "value": round(gbs, 1), "unit": "GB/s",
            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "us_per_call": round(ms * 1e3, 2),
            "algorithmic_bytes": alg_bytes, "workspace_bytes_each_way": ws_bytes,
            "cached_keys": total, "batch": B, "n_splits": S}


def run_decode_step_graph(torch, cp, si, seed=0, L=131072, reps=50):
    """One decode step of one request with a 128K-token cache (the per-token latency case),
    launched eagerly and as a replayed HIP graph (captured through torch)."""
    cfg = si.CONFIGS["decode_b32_32k_128k"]
    n_h, n_kv, d, S = cfg["n_h"], cfg["n_kv"], cfg["d_h"], cfg["n_splits"]
    toks = np.arange(L)
    kc = bf16_tokens(torch, si, seed, si.TID_K, toks, (n_kv, d))
    vc = bf16_tokens(torch, si, seed, si.TID_V, toks, (n_kv, d))
    q = bf16_tokens(torch, si, seed, si.TID_Q, np.arange(1), (n_h, d))
    ws_o, ws_l = cp.decode_workspace(1, n_h, d, S)
    o = torch.empty(1, n_h, d, device="cuda")
    l = torch.empty(1, n_h, device="cuda")
    offs = torch.zeros(1, dtype=torch.int64, device="cuda")
    lens = torch.full((1,), L, dtype=torch.int64, device="cuda")
    scale = 1.0 / math.sqrt(d)
    fn = lambda: cp.decode_splitkv(q, kc, vc, offs, lens, S, scale, ws_o, ws_l, o, l)
    eager_ms = time_reps(torch, fn, reps)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    graph_ms = time_reps(torch, graph.replay, reps)

    def synced(f):  # one step at a time, the host waiting for each (a token-by-token loop)
        f()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            f()
            torch.cuda.synchronize()
        return (time.perf_counter() - t0) / reps * 1e3

    eager_sync_ms, graph_sync_ms = synced(fn), synced(graph.replay)
    alg = L * n_kv * d * 2 * 2 + n_h * d * 2 + n_h * (d * 4 + 4)
    log(f"decode step B=1 L={L}: back to back eager {eager_ms * 1e3:.1f} us, graph "
        f"{graph_ms * 1e3:.1f} us; host-synced eager {eager_sync_ms * 1e3:.1f} us, graph "
        f"{graph_sync_ms * 1e3:.1f} us")
    return {"metric": "decode step latency", "unit": "us", "higher_is_better": False,
            "back_to_back": {"eager_us": round(eager_ms * 1e3, 2), "graph_us": round(graph_ms * 1e3, 2)},
            "host_synced": {"eager_us": round(eager_sync_ms * 1e3, 2),
                            "graph_us": round(graph_sync_ms * 1e3, 2)},
            "eager_GBps": round(alg / (eager_ms * 1e-3) / 1e9, 1), "cached_keys": L, "n_splits": S}


def device_rooflines(torch, probe=True):
    """Peaks derived from the device's reported attributes, next to the published figures, and
    the achievable device-to-device copy bandwidth (1 GiB read + 1 GiB written)."""
    import ctypes
    info = {}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        dev = torch.cuda.current_device()

        def attr(code):  # hipDeviceAttribute values from hip_runtime_api.h
            v = ctypes.c_int(0)
            return v.value if hip.hipDeviceGetAttribute(ctypes.byref(v), code, dev) == 0 else None

        cus, clk_khz, bus_bits, mclk_khz = attr(63), attr(5), attr(59), attr(60)
        info.update({"cus": cus, "peak_clock_mhz": clk_khz and clk_khz / 1e3,
                     "memory_clock_mhz": mclk_khz and mclk_khz / 1e3, "memory_bus_bits": bus_bits})
        if cus and clk_khz:
            info["bf16_peak_tflops_derived"] = round(cus * clk_khz * 1e3 * 4096 / 1e12, 1)
        if bus_bits and mclk_khz:  # HBM3E moves 4 bits per pin per reported memory clock
            info["hbm_peak_gbs_derived_4_per_clock"] = round(4 * mclk_khz * 1e3 * bus_bits / 8 / 1e9, 1)
    except OSError:
        pass
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    ms = time_reps(torch, lambda: dst.copy_(src), 10)
    info["copy_gbs"] = round(2 * src.numel() * 4 / (ms * 1e-3) / 1e9, 1)
    info["published"] = {"bf16_tflops": PEAK_BF16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS}
    del src, dst
    info["mfma_probe"] = run_mfma_probe() if probe else None
    log(f"device: {info}")
    return info


def run_mfma_probe():
    """The MFMA clock probe (a separate program, run as a child process): the bf16 MFMA rate and
    shader clock the chip sustains with random and with near-constant operands. None if the probe
    is not built or fails."""
    import subprocess
    exe = os.path.join(ROOT, "context_ring_attention_amd", "probe_mfma_clock")
    if not os.path.exists(exe):
        log("mfma probe: not built")
        return None
    try:
        res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    except subprocess.TimeoutExpired:
        log("mfma probe: timed out")
        return None
    if res.returncode != 0:
        log(f"mfma probe failed ({res.returncode}): {res.stderr.strip()[-300:]}")
        return None
    info = json.loads(res.stdout.strip().splitlines()[-1])
    log(f"mfma probe: {info}")
    return info


def run_pass_q(torch, cp, si, seed=0):
    cfg = si.CONFIGS["persistent_kv_8k_on_120k"]
    P, T, N, n_h, n_kv, d = cfg["cached"], cfg["new"], cfg["cp"], cfg["n_h"], cfg["n_kv"], cfg["d_h"]
    q_ranges = [(0, P, P + T)]
    kv_ranges = [(0, 0, P), (0, P, P + T)]
    qsh = [cp.shard_map(q_ranges, N, r) for r in range(N)]
    ksh = [cp.shard_map(kv_ranges, N, r) for r in range(N)]
    qs = [bf16_tokens(torch, si, seed, si.TID_Q, t, (n_h, d)) for _, t in qsh]
    ks = [bf16_tokens(torch, si, seed, si.TID_K, t, (n_kv, d)) for _, t in ksh]
    vs = [bf16_tokens(torch, si, seed, si.TID_V, t, (n_kv, d)) for _, t in ksh]
    parts_o = [torch.empty(qs[i // N].shape[0], n_h, d, device="cuda") for i in range(N * N)]
    parts_l = [torch.empty(qs[i // N].shape[0], n_h, device="cuda") for i in range(N * N)]
    o = [torch.empty(x.shape[0], n_h, d, device="cuda") for x in qs]
    l = [torch.empty(x.shape[0], n_h, device="cuda") for x in qs]
    scale = 1.0 / math.sqrt(d)
    fn = lambda: cp.ring_pass_q(qs, [s for s, _ in qsh], ks, vs, [s for s, _ in ksh], True, scale,
                                parts_o, parts_l, o, l)
    ms = time_reps(torch, fn, 5)
    pairs = sum(visible_pairs(qsh[a][0], ksh[b][0]) for a in range(N) for b in range(N))
    flops = 4 * d * n_h * pairs
    tf = flops / (ms * 1e-3) / 1e12
    log(f"pass-q: {ms:.2f} ms, {tf:.1f} useful TFLOP/s")
    return {"metric": "causal-useful TFLOP/s", "value": round(tf, 1), "unit": "TFLOP/s",
            "ms_per_call": round(ms, 3), "useful_tflop": round(flops / 1e12, 3),
            "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


def run_merge(torch, cp, parts_o, parts_l, d):
    rows = parts_o[0].numel() // d
    out = torch.empty(rows, d, device="cuda")
    lse = torch.empty(rows, device="cuda")
    fn = lambda: cp.merge_lse(parts_o, parts_l, out, lse)
    ms = time_reps(torch, fn, 10)
    seen = sum(int(torch.isfinite(x).sum()) for x in parts_l)
    alg = seen * d * 4 + len(parts_l) * rows * 4 + rows * (d * 4 + 4)
    gbs = alg / (ms * 1e-3) / 1e9
    log(f"merge: {ms * 1e3:.1f} us, {gbs:.0f} GB/s")
    return {"metric": "merge GB/s", "value": round(gbs, 1), "unit": "GB/s",
            "us_per_call": round(ms * 1e3, 2), "algorithmic_bytes": alg, "parts": len(parts_l),
            "rows": rows, "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}


def run_prefill_1m(torch, cp, si, seed=0, rank=0):
    cfg = si.CONFIGS["prefill_1m_varlen_cp8"]
    N, n_h, n_kv, d = cfg["cp"], cfg["n_h"], cfg["n_kv"], cfg["d_h"]
    ranges = [(i, 0, L) for i, L in enumerate(cfg["seqs"])]
    shards = [cp.shard_map(ranges, N, r) for r in range(N)]
    ks = [bf16_tokens(torch, si, seed, si.TID_K, t, (n_kv, d)) for _, t in shards]
    vs = [bf16_tokens(torch, si, seed, si.TID_V, t, (n_kv, d)) for _, t in shards]
    q = bf16_tokens(torch, si, seed, si.TID_Q, shards[rank][1], (n_h, d))
    o = torch.empty(q.shape[0], n_h, d, device="cuda")
    l = torch.empty(q.shape[0], n_h, device="cuda")
    scale = 1.0 / math.sqrt(d)
    fn = lambda: cp.ring_pass_kv(q, shards[rank][0], rank, ks, vs, [s for s, _ in shards], True,
                                 scale, o, l, o_acc=o, lse_acc=l)
    ms = time_reps(torch, fn, 3, warm=1)
    pairs = sum(visible_pairs(shards[rank][0], shards[s][0]) for s in range(N))
    flops = 4 * d * n_h * pairs
    tf = flops / (ms * 1e-3) / 1e12
    log(f"prefill 1M varlen CP8 rank {rank}: {ms:.1f} ms, {tf:.1f} useful TFLOP/s")
    return {"metric": "causal-useful TFLOP/s", "value": round(tf, 1), "unit": "TFLOP/s",
            "ms_per_rank": round(ms, 2), "useful_tflop": round(flops / 1e12, 3), "rank": rank,
            "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


def run_cpu_baseline(si, ranges, N, n_h, n_kv, d, seed, budget_s):
    """The fp64 oracle as it stands, on rank 0's Q shard: whole query tokens (all 16 heads),
    spread evenly over the shard, each against its full visible key set (all 4 KV shards)."""
    import oracle
    q_seq, q_pos, q_glob = oracle.shard_tokens(ranges, N, 0)
    ks, vs, kseq, kpos = [], [], [], []
    for s in range(N):
        sq, ps, gl = oracle.shard_tokens(ranges, N, s)
        ks.append(si.to_dtype(si.normal_tokens(seed, si.TID_K, gl, (n_kv, d)), "bf16")[1].numpy())
        vs.append(si.to_dtype(si.normal_tokens(seed, si.TID_V, gl, (n_kv, d)), "bf16")[1].numpy())
        kseq.append(sq)
        kpos.append(ps)
    kf, vf = np.concatenate(ks), np.concatenate(vs)
    kseq, kpos = np.concatenate(kseq), np.concatenate(kpos)
    qf = si.to_dtype(si.normal_tokens(seed, si.TID_Q, q_glob, (n_h, d)), "bf16")[1].numpy()
    order = np.random.default_rng(seed).permutation(len(q_glob))
    done, flops, spent = 0, 0, 0.0
    batch = 8
    while spent < budget_s and done < len(order):
        rows = np.sort(order[done:done + batch])
        t0 = time.perf_counter()
        oracle.attention(qf, kf, vf, n_h, n_kv, q_seq, q_pos, kseq, kpos, True, 1.0 / math.sqrt(d),
                         rows=rows)
        spent += time.perf_counter() - t0
        flops += 4 * d * n_h * int((q_pos[rows] + 1).sum())
        done += len(rows)
    tf = flops / spent / 1e12
    log(f"oracle: {done} query tokens in {spent:.1f}s on {oracle.num_threads()} threads, {tf * 1e3:.2f} GFLOP/s")
    return {"value": round(tf, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{done} random query tokens (x{n_h} heads) of rank 0's 32K-token Q shard of "
                      f"prefill_128k_cp4, each against its full visible key set; {spent:.1f} s of fp64 work",
            "host": {"cpu_model": host_cpu_model(), "logical_cpus": os.cpu_count()}}


def host_cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None where it is not available)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# --------------------------------------------------------------------------- main
def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only: every workload is one CP "
                          "rank's share played out in one GPU's memory; use --gpus 1"}), flush=True)
        sys.exit(2)

    import torch
    import synth_inputs as si
    from context_ring_attention_amd import binding as cp

    cp.load()  # fails loudly if the HIP library is missing: there is no CPU fallback
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    dev = torch.cuda.get_device_properties(0)
    log(f"device {dev.name} {getattr(dev, 'gcnArchName', '')} CUs={dev.multi_processor_count}")

    cfg = si.CONFIGS["prefill_128k_cp4"]
    N, n_h, n_kv, d = cfg["cp"], cfg["n_h"], cfg["n_kv"], cfg["d_h"]
    L = cfg["seqs"][0]
    scale = 1.0 / math.sqrt(d)
    seed = 0
    ranges = [(0, 0, L)]
    shards = [cp.shard_map(ranges, N, r) for r in range(N)]
    t0 = time.time()
    ks = [bf16_tokens(torch, si, seed, si.TID_K, t, (n_kv, d)) for _, t in shards]
    vs = [bf16_tokens(torch, si, seed, si.TID_V, t, (n_kv, d)) for _, t in shards]
    qs = [bf16_tokens(torch, si, seed, si.TID_Q, t, (n_h, d)) for _, t in shards]
    log(f"inputs generated in {time.time() - t0:.1f}s")
    kv_segs = [s for s, _ in shards]
    tq = [q.shape[0] for q in qs]
    o = [torch.empty(t, n_h, d, device="cuda") for t in tq]
    lse = [torch.empty(t, n_h, device="cuda") for t in tq]
    parts = None
    if args.mode == "partials":
        parts = [([torch.empty(t, n_h, d, device="cuda") for _ in range(N)],
                  [torch.empty(t, n_h, device="cuda") for _ in range(N)]) for t in tq]

    pairs = [[visible_pairs(shards[r][0], shards[s][0]) for s in range(N)] for r in range(N)]
    flops_step = sum(4 * d * n_h * sum(row) for row in pairs)

    def step():
        for r in range(N):
            if parts is None:
                cp.ring_pass_kv(qs[r], shards[r][0], r, ks, vs, kv_segs, True, scale, o[r], lse[r],
                                o_acc=o[r], lse_acc=lse[r])
            else:
                cp.ring_pass_kv(qs[r], shards[r][0], r, ks, vs, kv_segs, True, scale, o[r], lse[r],
                                o_parts=parts[r][0], lse_parts=parts[r][1])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_step = elapsed * 1e3 / args.steps
    value = flops_step / (ms_step * 1e-3) / 1e12
    log(f"prefill_128k_cp4: {ms_step:.2f} ms/step (4 ranks), {value:.1f} useful TFLOP/s")

    # ---- dominant kernel: per-launch time of cp_partial_attn (one ring step of one rank) ----
    launch_ms, launch_flops = [], []
    tmr = Timer(torch)
    for _ in range(2):
        for r in range(N):
            for t in range(N):
                s = (r - t) % N
                with tmr:
                    cp.partial_attn(qs[r], ks[s], vs[s], shards[r][0], shards[s][0], True, scale,
                                    o[r], lse[r], accumulate=t > 0)
                launch_ms.append(tmr.ms())
                launch_flops.append(4 * d * n_h * pairs[r][s])
    avg_ms = float(np.mean(launch_ms))
    avg_flops = float(np.mean(launch_flops))
    achieved = avg_flops / (avg_ms * 1e-3) / 1e12
    rec = recorded_traffic()
    traffic = None if rec is None else rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "kernel": "attn_bf16_kernel<128> (cp_partial_attn)",
                "avg_launch_ms": round(avg_ms, 4), "flops_per_launch": avg_flops}
    if rec is not None:
        roofline["traffic_detail"] = {"unit": "bytes per launch", "read": rec["fetch_bytes_per_launch"],
                                      "write": rec["write_bytes_per_launch"],
                                      "source": os.path.relpath(COUNTERS_MD, ROOT)}
    log(f"cp_partial_attn: avg {avg_ms:.3f} ms/launch, {achieved:.1f} TFLOP/s, "
        f"{100 * achieved / PEAK_BF16_TFLOPS:.1f}% of bf16 peak")

    secondary = {}
    if not args.no_secondary:
        # merge of rank 0's four ring partials (the partials mode of the same workload)
        po = [torch.empty(tq[0], n_h, d, device="cuda") for _ in range(N)]
        pl = [torch.empty(tq[0], n_h, device="cuda") for _ in range(N)]
        for t in range(N):
            cp.partial_attn(qs[0], ks[(0 - t) % N], vs[(0 - t) % N], shards[0][0],
                            shards[(0 - t) % N][0], True, scale, po[t], pl[t])
        secondary["merge_4parts_128k_cp4"] = run_merge(torch, cp, po, pl, d)
        del po, pl
        secondary["decode_b32_32k_128k"] = run_decode(torch, cp, si)
        secondary["decode_step_b1_128k_graph"] = run_decode_step_graph(torch, cp, si)
        secondary["persistent_kv_8k_on_120k"] = run_pass_q(torch, cp, si)
        if args.extended:
            secondary["prefill_1m_varlen_cp8"] = run_prefill_1m(torch, cp, si)

    if args.calib_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 1 GiB read, 1 GiB written")

    device_info = device_rooflines(torch, probe=not args.no_mfma_probe) if not args.no_secondary else None
    probe = (device_info or {}).get("mfma_probe")
    if probe and probe.get("random", {}).get("tflops"):
        # the same kernel rate against what MFMA-only code sustains on random operands
        roofline["frac_of_mfma_probe_random"] = round(achieved / probe["random"]["tflops"], 3)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = run_cpu_baseline(si, ranges, N, n_h, n_kv, d, seed, args.cpu_seconds)

    out = {
        "metric": "causal-useful attention TFLOP/s per rank shard",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill_128k_cp4", "seq_len": L, "cp_world": N,
                   "ranks_per_step": N, "q_heads": n_h, "kv_heads": n_kv, "head_dim": d,
                   "causal": True, "ring": "pass_kv", "merge_mode": args.mode,
                   "useful_tflop_per_step": round(flops_step / 1e12, 3)},
        "roofline": roofline,
        "device": device_info,
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

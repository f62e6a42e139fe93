"""Benchmark: paged GDN serving step on one MI355X.

Default workload (one "step"): the mixed hybrid serving step -- 32 prefill
sequences (512..8192 new tokens, page-rounded prefix hits, 4 padded) and 512
decode sequences (2k..64k context, 16 padded), H = Hqk = 32, K = V = 128,
page_size 896, one fp32 pool of 16384 pages (32 GiB).  Slots are derived once
per step (prefill + decode), then 48 GDN layers each run a paged prefill and a
paged decode with the precomputed slots; every layer has its own seeded
inputs, all resident in HBM before timing starts.

Prints ONE JSON line.  ``value`` is prefill tokens per second of the whole step
(each prefill token passes all 48 layers; the decode batch's work is inside
the timed step).  Extra fields give per-call rates measured with HIP events
on the launch stream: per-layer prefill tokens/s and decode state GB/s, each
against its roofline, plus the CPU oracle baseline on a bounded sample.

Other workloads (--workload prefill|decode|long) time the other shapes for
development; they print a line of the same form.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN paged prefill tokens/s + decode state HBM GB/s (frac. of peak), 1×MI355X"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
D = 128
CHUNK = 64
STATE_BYTES = D * D * 4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="hybrid", choices=["hybrid", "prefill", "decode", "long"])
    ap.add_argument("--layers", type=int, default=48)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-side", action="store_true",
                    help="skip the side measurements (bf16-pool decode, long single prompt)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096)
    ap.add_argument("--cpu-sample-decode", type=int, default=128)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB (reference for "
                         "hardware byte counters); reported as copy_GBps")
    return ap.parse_args()


# ----------------------------------------------------------------- measured traffic
COUNTERS_MD = os.path.join(ROOT, "profiles", "hbm_counters__prefill_path_and_decode__hybrid_step.md")


def kernel_sources_digest() -> str:
    """sha256 (first 16 hex digits) of the sources of the measured kernels
    (prefill path and decode) the counters were taken on, with comments and
    whitespace removed (comment edits keep the digest)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_recurrent_state_amd", "csrc")
    for f in [os.path.join(csrc, n) for n in ("gdn_decode.hip", "gdn_internal.h", "gdn_prefill.hip")]:
        with open(f, encoding="utf-8") as fh:
            code = fh.read()
        code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        code = " ".join(code.split())
        h.update(os.path.basename(f).encode() + b"\0" + code.encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE summary
    (copy-calibrated), or None when the kernel sources changed since."""
    try:
        text = open(COUNTERS_MD).read()
    except OSError:
        return None
    m = re.search(r"bench-traffic: sources=([0-9a-f]+) prefill_path_bytes=(\d+) decode_bytes=(\d+)", text)
    if not m or m.group(1) != kernel_sources_digest():
        return None
    return {"prefill": int(m.group(2)), "decode": int(m.group(3))}


# ----------------------------------------------------------------- algorithmic work
def prefill_bytes(T: int, H: int, Hqk: int, n_state_io: int) -> int:
    """q, k (per q/k head), v, o (bf16) and g, beta (fp32) per token, plus the
    fp32 states read and written."""
    return T * (2 * Hqk * D * 2 + 2 * H * D * 2 + 2 * H * 4) + n_state_io * H * STATE_BYTES


def prefill_flops(T: int, H: int) -> int:
    """Chunked form per token and head: K K^T, Q K^T, T.(beta V) and T.(beta gamma K)
    within the chunk (4 x 2*C*d) and W S^T, Q S^T, E^T K across chunks
    (3 x 2*d*d) plus P E (2*C*d)."""
    return T * H * (6 * D * D + 10 * CHUNK * D)


def decode_bytes(B: int, H: int, Hqk: int) -> int:
    return 2 * B * H * STATE_BYTES + B * (2 * Hqk * D * 2 + 2 * H * D * 2 + 2 * H * 4)


# ----------------------------------------------------------------- CPU baseline
def cpu_baseline(pre_cpu, dec_cpu, pool_rows, sample_tokens, sample_decode, layers,
                 step_prefill_tokens, step_decode_seqs):
    """Time the fp64 oracle on a bounded sample of layer 0 and scale to the step."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import gdn as ogdn

    class Rows:
        def __getitem__(self, r):
            return pool_rows[int(r)]

    with threadpool_limits(limits=1):
        # prefill sample: the first `sample_tokens` new tokens of sequence 0
        L0 = int(pre_cpu["new"][0])
        n = min(sample_tokens, L0)
        q, k, v = pre_cpu["q"][:n], pre_cpu["k"][:n], pre_cpu["v"][:n]
        g, beta = pre_cpu["g"][:n], pre_cpu["beta"][:n]
        rd = pre_cpu["read_rows"][0]
        t0 = time.perf_counter()
        ogdn.prefill(q, k, v, g, beta, [0, n], initial_state=Rows(),
                     state_indices=[rd], output_final_state=True, output_state_indices=[rd])
        t_pf = (time.perf_counter() - t0) / n
        # decode sample: the first `sample_decode` sequences
        m = sample_decode
        rows = dec_cpu["read_rows"][:m]
        t0 = time.perf_counter()
        ogdn.decode(dec_cpu["q"][:m], dec_cpu["k"][:m], dec_cpu["v"][:m], dec_cpu["g"][:m],
                    dec_cpu["beta"][:m], initial_state=Rows(), initial_state_indices=rows)
        t_dec = (time.perf_counter() - t0) / m
    step_s = layers * (t_pf * step_prefill_tokens + t_dec * step_decode_seqs)
    return {
        "value": step_prefill_tokens / step_s,
        "unit": "prefill tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"layer 0: {n} new tokens of prefill sequence 0 (all heads) and {m} decode "
                   f"sequences, fp64 NumPy on 1 thread; per-token and per-sequence times "
                   f"scaled to the step's {step_prefill_tokens} prefill tokens and "
                   f"{step_decode_seqs} decode sequences x {layers} layers"),
        "prefill_tokens_per_s_per_layer": 1.0 / t_pf,
        "decode_state_GBps": (2 * STATE_BYTES * pre_cpu["H"]) / t_dec / 1e9,
    }


# ----------------------------------------------------------------- workloads
def _median_ms(torch, run, n, reps=3):
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    E = torch.cuda.Event
    res = []
    for _ in range(reps):
        a, b = E(enable_timing=True), E(enable_timing=True)
        a.record()
        for _ in range(n):
            run()
        b.record()
        torch.cuda.synchronize()
        res.append(a.elapsed_time(b) / n)
    return sorted(res)[len(res) // 2]


def side_measurements(torch, gdn, workloads, pool, dec, ps, H, Hqk, t_dc_ms):
    """Timed beside the step, not part of it: the decode batch on a bf16 copy
    of the pool (the same rows at half the bytes), and the long single prompt
    (one sequence, 32 heads, 32768 tokens in 5 calls) with the
    sequence-parallel recurrence against whole sequences."""
    dev = pool.device
    out = {}
    Bd = int(dec["last_page_len"].shape[0])
    o = torch.empty(Bd, H, D, dtype=torch.bfloat16, device=dev)
    sl = gdn.decode_slots(dec["page_indices"], dec["page_indptr"], dec["last_page_len"])
    pool16 = pool.to(torch.bfloat16)
    ms = _median_ms(torch, lambda: gdn.decode_paged(
        dec["q"], dec["k"], dec["v"], dec["g"], dec["beta"], pool16, dec["page_indices"],
        dec["page_indptr"], ps, dec["last_page_len"], slots=sl, out=o), 20)
    del pool16
    by = decode_bytes(Bd, H, Hqk) - Bd * H * STATE_BYTES  # state rows at 2 bytes an element
    out["bf16_pool_decode"] = {
        "workload": f"the step's decode batch ({Bd} seqs, H={H}) on a bf16 copy of the pool",
        "ms": ms, "state_GBps": by / (ms / 1e3) / 1e9,
        "frac_hbm_peak": by / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS, "fp32_pool_ms": t_dc_ms}
    c = workloads.config3(device=dev)
    # one workspace for the largest call serves every call (sizes only grow)
    t_max = max(int(call["q"].shape[0]) for call in c["calls"])
    ws = torch.empty(gdn.prefill_workspace_size(t_max, 1, c["H"], c["Hqk"]), dtype=torch.uint8,
                     device=dev)

    def run(options=None):
        for call in c["calls"]:
            gdn.prefill(call["q"], call["k"], call["v"], call["g"], call["beta"],
                        call["cu_seqlens"], initial_state=c["pool"],
                        state_indices=call["state_indices"], output_state=c["pool"],
                        output_state_indices=call["output_state_indices"],
                        output_final_state=True, state_checkpoints=c["state_checkpoints"],
                        checkpoint_state_indices=c["checkpoint_state_indices"],
                        checkpoint_cu_starts=call["checkpoint_cu_starts"],
                        prefix_lens=call["prefix_lens"], checkpoint_every_n_tokens=c["every_n"],
                        workspace=ws, options=options)
    T = sum(int(call["q"].shape[0]) for call in c["calls"])
    ms_split = _median_ms(torch, run, 5)
    whole = gdn.Options(prefill_split_chunks=-1)
    ms_whole = _median_ms(torch, lambda: run(whole), 5)
    out["long_prompt"] = {
        "workload": f"one sequence, H=Hqk={c['H']}, {T} tokens in {len(c['calls'])} calls, "
                    f"checkpoints every {c['every_n']}",
        "sequence_parallel_ms": ms_split, "prefill_tokens_per_s": T / (ms_split / 1e3),
        "whole_sequence_ms": ms_whole, "speedup": ms_whole / ms_split}
    return out


def hybrid(args, torch, gdn, workloads):
    dev = "cuda"
    L = args.layers
    c = workloads.config4(device=dev, layers=range(L))
    H, Hqk = c["H"], c["Hqk"]
    ps = c["page_size"]
    pool = c["pool"]
    lay = c["layers"]
    pre0, dec0 = lay[0]["prefill"], lay[0]["decode"]
    T = int(pre0["q"].shape[0])
    Bp = int(pre0["last_page_len"].shape[0])
    Bd = int(dec0["last_page_len"].shape[0])
    ws = torch.empty(gdn.prefill_workspace_size(T, Bp, H, Hqk), dtype=torch.uint8, device=dev)
    o_pre = torch.empty(T, H, D, dtype=torch.bfloat16, device=dev)
    o_dec = torch.empty(Bd, H, D, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    E = torch.cuda.Event

    def step(events=None, slot_events=None):
        if slot_events is not None:
            slot_events[0].record(stream)
        sl_p = gdn.prefill_slots(pre0["cu_seqlens"], pre0["page_indices"], pre0["page_indptr"],
                                 pre0["last_page_len"], ps)
        sl_d = gdn.decode_slots(dec0["page_indices"], dec0["page_indptr"], dec0["last_page_len"])
        if slot_events is not None:
            slot_events[1].record(stream)
        for l in range(L):
            p, d = lay[l]["prefill"], lay[l]["decode"]
            if events is not None:
                events[l][0].record(stream)
            gdn.prefill_paged(p["q"], p["k"], p["v"], p["g"], p["beta"], p["cu_seqlens"], pool,
                              p["page_indices"], p["page_indptr"], ps, p["last_page_len"],
                              slots=sl_p, workspace=ws, out=o_pre)
            if events is not None:
                events[l][1].record(stream)
            gdn.decode_paged(d["q"], d["k"], d["v"], d["g"], d["beta"], pool, d["page_indices"],
                             d["page_indptr"], ps, d["last_page_len"], slots=sl_d, out=o_dec)
            if events is not None:
                events[l][2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[[E(enable_timing=True) for _ in range(3)] for _ in range(L)] for _ in range(args.steps)]
    sevs = [[E(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s], sevs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_pf = [evs[s][l][0].elapsed_time(evs[s][l][1]) for s in range(args.steps) for l in range(L)]
    t_dc = [evs[s][l][1].elapsed_time(evs[s][l][2]) for s in range(args.steps) for l in range(L)]
    t_sl = [sevs[s][0].elapsed_time(sevs[s][1]) for s in range(args.steps)]
    t_pf_ms = sum(t_pf) / len(t_pf)
    t_dc_ms = sum(t_dc) / len(t_dc)

    def pct(xs):
        xs = sorted(xs)
        return [xs[min(len(xs) - 1, int(q * len(xs)))] for q in (0.1, 0.5, 0.9)]
    ms_step = wall * 1000 / args.steps

    n_state_io = sum(1 for r in pre0["read_rows"] if r >= 0)
    n_state_io += sum(1 + (p + n) // ps - p // ps for p, n in zip(pre0["prefix"], pre0["new"]) if n > 0)
    pf_bytes = prefill_bytes(T, H, Hqk, n_state_io)
    dc_bytes = decode_bytes(Bd, H, Hqk)
    pf_tps_layer = T / (t_pf_ms / 1e3)
    pf_roof_tps = T / (pf_bytes / (HBM_PEAK_GBPS * 1e9))
    dc_gbps = dc_bytes / (t_dc_ms / 1e3) / 1e9
    pf_tflops = prefill_flops(T, H) / (t_pf_ms / 1e3) / 1e12

    # The dominant launch of the step: the prefill library call (three kernels
    # on one stream: plan_kernel, wy_kernel, rec_kernel) or the decode call.
    # achieved = algorithmic bytes per call / event-timed call duration.
    traffic = measured_traffic() if L >= 2 else None
    if t_dc_ms >= t_pf_ms:
        roof = {"kernel": "decode_stream_kernel", "bound": "hbm", "achieved": dc_gbps,
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": dc_gbps / HBM_PEAK_GBPS,
                "traffic": traffic and traffic["decode"], "per_launch_bytes": dc_bytes,
                "avg_launch_ms": t_dc_ms}
    else:
        ach = pf_bytes / (t_pf_ms / 1e3) / 1e9
        roof = {"kernel": "prefill path (plan_kernel + wy_kernel + rec_kernel, one call)",
                "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": ach / HBM_PEAK_GBPS, "traffic": traffic and traffic["prefill"],
                "per_launch_bytes": pf_bytes, "avg_launch_ms": t_pf_ms}
    real_prefill = int(c["num_prefill"])
    line = {
        "metric": METRIC,
        "value": T * args.steps / wall,
        "unit": "prefill tokens/s (48-layer hybrid step incl. decode batch)" if L == 48 else
                f"prefill tokens/s ({L}-layer hybrid step incl. decode batch)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16/fp32",
        "data": "synthetic",
        "config": {"workload": "hybrid serving step: 32 (+4 pad) paged prefill seqs with "
                               "page-rounded prefix hits + 512 (+16 pad) paged decode seqs, "
                               f"H=Hqk={H}, K=V=128, page_size {ps}, fp32 pool 16384 pages, "
                               f"{L} GDN layers, slots once per step",
                   "prefill_tokens_per_step": T, "prefill_seqs": real_prefill,
                   "decode_seqs": int(c["num_decode"]), "layers": L},
        "prefill_tokens_per_s_per_layer": pf_tps_layer,
        "prefill_frac_hbm_roofline": pf_tps_layer / pf_roof_tps,
        "prefill_algorithmic_tflops": pf_tflops,
        "prefill_frac_bf16_peak": pf_tflops / BF16_PEAK_TFLOPS,
        "decode_state_GBps": dc_gbps,
        "decode_frac_hbm_peak": dc_gbps / HBM_PEAK_GBPS,
        "prefill_ms_per_layer": t_pf_ms, "decode_ms_per_layer": t_dc_ms,
        "prefill_ms_p10_p50_p90": pct(t_pf), "decode_ms_p10_p50_p90": pct(t_dc),
        "slots_ms_per_step": sum(t_sl) / len(t_sl),
        "roofline": roof,
    }
    if not args.no_side:
        line["side"] = side_measurements(torch, gdn, workloads, pool, dec0, ps, H, Hqk, t_dc_ms)
    cpu_inputs = None
    if not args.no_cpu_baseline:
        pcpu = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in pre0.items()}
        pcpu["H"] = H
        dcpu = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in dec0.items()}
        rows = [pcpu["read_rows"][0]] + list(dcpu["read_rows"][:args.cpu_sample_decode])
        cpu_inputs = (pcpu, dcpu, rows, T, int(c["num_decode"]) + 16)
    return line, cpu_inputs, pool


def single(args, torch, gdn, workloads):
    """Prefill-only (config 1), decode-only (config 2) or long chunked prefill (config 3)."""
    dev = "cuda"
    E = torch.cuda.Event
    stream = torch.cuda.current_stream()
    if args.workload == "prefill":
        c = workloads.config1(device=dev)
        p = c["prefill"]
        H, Hqk = c["H"], c["Hqk"]
        T = int(p["q"].shape[0])
        B = int(p["last_page_len"].shape[0])
        ws = torch.empty(gdn.prefill_workspace_size(T, B, H, Hqk), dtype=torch.uint8, device=dev)
        o = torch.empty(T, H, D, dtype=torch.bfloat16, device=dev)
        sl = gdn.prefill_slots(p["cu_seqlens"], p["page_indices"], p["page_indptr"],
                               p["last_page_len"], 1024)

        def run():
            gdn.prefill_paged(p["q"], p["k"], p["v"], p["g"], p["beta"], p["cu_seqlens"],
                              c["pool"], p["page_indices"], p["page_indptr"], 1024,
                              p["last_page_len"], slots=sl, workspace=ws, out=o)
        n_io = sum(1 for r in p["read_rows"] if r >= 0) + sum(
            1 + (a + n) // 1024 - a // 1024 for a, n in zip(p["prefix"], p["new"]))
        work_bytes = prefill_bytes(T, H, Hqk, n_io)
        desc = "paged prefill B=8, H=Hqk=16, page 1024, shared prefixes"
        unit_val = lambda ms: T / (ms / 1e3)  # noqa: E731
        unit = "prefill tokens/s"
    elif args.workload == "decode":
        c = workloads.config2(device=dev)
        d = c["decode"]
        H, Hqk = c["H"], c["Hqk"]
        B = int(d["last_page_len"].shape[0])
        o = torch.empty(B, H, D, dtype=torch.bfloat16, device=dev)
        # Four page-table variants whose touched pages (the last two of every
        # sequence) are disjoint, used in turn, so that the 256 MB Infinity
        # Cache cannot serve rows the previous call just wrote.
        idx, ip = d["page_indices"], d["page_indptr"]
        n_pages = int(c["pool"].shape[0])
        ends = ip[1:].long()
        pos = torch.cat([ends - 1, (ends - 2)[ends - 2 >= ip[:-1].long()]])
        used = torch.unique(idx[pos].long())
        free_mask = torch.ones(n_pages, dtype=torch.bool, device=dev)
        free_mask[used] = False
        free = torch.nonzero(free_mask).flatten()
        free = free[torch.randperm(free.numel(), generator=torch.Generator().manual_seed(7)).to(dev)]
        tables = [idx]
        for r in range(3):
            lut = torch.arange(n_pages, device=dev)
            lut[used] = free[r * used.numel():(r + 1) * used.numel()]
            t = idx.clone()
            t[pos] = lut[idx[pos].long()].to(idx.dtype)
            tables.append(t)
        slot_sets = [gdn.decode_slots(t, ip, d["last_page_len"]) for t in tables]
        turn = [0]

        def run():
            r = turn[0] % len(tables)
            turn[0] += 1
            gdn.decode_paged(d["q"], d["k"], d["v"], d["g"], d["beta"], c["pool"],
                             tables[r], ip, 1024, d["last_page_len"], slots=slot_sets[r], out=o)
        work_bytes = decode_bytes(B, H, Hqk)
        desc = ("paged decode B=256, Hqk=16, H=32, page 1024, 25% new-page tokens, four page "
                "tables with disjoint touched pages in turn")
        unit_val = lambda ms: work_bytes / (ms / 1e3) / 1e9  # noqa: E731
        unit = "decode state GB/s"
    else:
        c = workloads.config3(device=dev)
        H, Hqk = c["H"], c["Hqk"]
        T = 32768
        calls = c["calls"]
        ws = torch.empty(gdn.prefill_workspace_size(8192, 1, H, Hqk), dtype=torch.uint8,
                         device=dev)

        def run():
            for call in calls:
                gdn.prefill(call["q"], call["k"], call["v"], call["g"], call["beta"],
                            call["cu_seqlens"], initial_state=c["pool"],
                            state_indices=call["state_indices"], output_state=c["pool"],
                            output_state_indices=call["output_state_indices"],
                            output_final_state=True, state_checkpoints=c["state_checkpoints"],
                            checkpoint_state_indices=c["checkpoint_state_indices"],
                            checkpoint_cu_starts=call["checkpoint_cu_starts"],
                            prefix_lens=call["prefix_lens"], checkpoint_every_n_tokens=896,
                            workspace=ws)
        work_bytes = prefill_bytes(T, H, Hqk, 5 + 4 + 18)
        desc = "long chunked prefill B=1, H=32, 32768 tokens in 5 calls, checkpoints every 896"
        unit_val = lambda ms: T / (ms / 1e3)  # noqa: E731
        unit = "prefill tokens/s"
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    evs = [(E(enable_timing=True), E(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
    ach = work_bytes / (ms / 1e3) / 1e9
    line = {
        "metric": METRIC, "value": unit_val(ms), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall * 1000 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16/fp32",
        "data": "synthetic", "config": {"workload": desc},
        "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBPS, "traffic": None,
                     "per_launch_bytes": work_bytes, "avg_launch_ms": ms},
    }
    return line, None, None


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: the path runs on a single GPU and has no multi-GPU mode",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import paged_recurrent_state_amd as gdn
    import workloads

    gdn.load()
    torch.manual_seed(0)
    copy_gbps = None
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        reps = 5
        for _ in range(reps):
            dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        copy_gbps = 2 * n * reps / (a.elapsed_time(b) / 1e3) / 1e9
        del src, dst
    if args.workload == "hybrid":
        line, cpu_inputs, pool = hybrid(args, torch, gdn, workloads)
    else:
        line, cpu_inputs, pool = single(args, torch, gdn, workloads)
    if cpu_inputs is not None:
        pcpu, dcpu, rows, T, ndec = cpu_inputs
        import numpy as np  # noqa: F401
        # The pool rows the sample reads, copied before any timing mutated them?  The
        # timed steps rewrote them; the oracle's speed does not depend on their values.
        pool_rows = {int(r): pool[int(r)].cpu().numpy() for r in rows if int(r) >= 0}
        line["cpu_baseline"] = cpu_baseline(pcpu, dcpu, pool_rows, args.cpu_sample_tokens,
                                            args.cpu_sample_decode, args.layers, T, ndec)
    if copy_gbps is not None:
        line["copy_GBps"] = copy_gbps
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

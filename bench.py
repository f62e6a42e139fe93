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
                    help="skip the other workloads (paged prefill, paged decode, long prompt)")
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


def plain_copy_gbps(torch, mib: int, reps: int = 10, rounds: int = 3, gdn=None) -> float:
    """GB/s (read + written bytes) of a device copy of `mib` MiB, median over
    `rounds` of `reps` back-to-back copies timed with events: the library's
    streaming copy when `gdn` is given, else torch's copy_ (the runtime's
    device-to-device memcpy)."""
    n = mib << 20
    src = torch.empty(n // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    copy = (lambda: gdn.stream_copy(dst, src)) if gdn is not None else (lambda: dst.copy_(src))
    copy()
    torch.cuda.synchronize()
    res = []
    for _ in range(rounds):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            copy()
        b.record()
        torch.cuda.synchronize()
        res.append(2 * n * reps / (a.elapsed_time(b) / 1e3) / 1e9)
    del src, dst
    torch.cuda.empty_cache()
    return sorted(res)[len(res) // 2]


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
# The fp64 oracle timed on the host cores: worker processes (started fresh,
# one oracle thread each) draw seeded inputs of a workload's shapes and
# distributions on the CPU and time only the oracle call on them.  The
# measured per-token (prefill) and per-sequence (decode) times then give each
# workload's time: its sequences dealt longest first to the cores (heads split
# over the cores when one sequence is all there is).

def cpu_cores() -> int:
    """Host cores this process may use, capped at the 16 a one-GPU share has."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _oracle_item(item):
    """One timed oracle run (worker process): item = (kind, n, Hqk, H, seed)."""
    import torch
    from threadpoolctl import threadpool_limits

    import workloads
    from oracle import gdn as ogdn
    kind, n, Hqk, H, seed = item
    with threadpool_limits(limits=1):
        torch.set_num_threads(1)
        gen = workloads.generator(seed)
        t = workloads.token_inputs(n, Hqk, H, D, D, gen)
        s0 = (torch.randn(1, H, D, D, generator=gen, dtype=torch.float64) / math.sqrt(D)).numpy()
        t0 = time.perf_counter()
        if kind == "prefill":
            ogdn.prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], [0, n], initial_state=s0,
                         state_indices=[0], output_final_state=True, shared_pool=False)
        else:  # n sequences of one decode token each
            ogdn.decode(t["q"], t["k"], t["v"], t["g"], t["beta"], initial_state=s0,
                        initial_state_indices=[0] * n, output_state_indices=[-1] * n,
                        shared_pool=False)
        dt = time.perf_counter() - t0
    return os.getpid(), dt


def _lpt(times, cores):
    loads = [0.0] * cores
    for x in sorted(times, reverse=True):
        i = loads.index(min(loads))
        loads[i] += x
    return max(loads)


def cpu_baseline(shapes, layers, n_tok=768, n_dec=96):
    """Oracle rates on the host cores (multi-core and 1 core).

    shapes: per workload, dict(prefill=[new tokens per sequence], H, Hqk,
    decode=number of decode sequences, Hd, Hqkd).  Per (H, Hqk) head layout,
    `cores` workers each time n_tok prefill tokens and n_dec decode sequences
    at once (contended, as the multi-core run would be), and one worker alone
    (the 1-core rate)."""
    import multiprocessing as mp
    C = cpu_cores()
    layouts = sorted({(w["H"], w["Hqk"]) for w in shapes.values() if w.get("prefill")} |
                     {(w["H"] // max(1, C), w["Hqk"] // max(1, C)) for w in shapes.values()
                      if w.get("split_heads")} |
                     {(w["Hd"], w["Hqkd"]) for w in shapes.values() if w.get("decode")})
    layouts = sorted({(max(1, h), max(1, q)) for h, q in layouts})
    per_tok, per_dec = {}, {}
    ctx = mp.get_context("spawn")
    t_start = time.perf_counter()
    with ctx.Pool(C) as pool:
        # start every worker and run each code path once before timing
        pool.map(_oracle_item, [("prefill", 8, 2, 2, 0)] * C + [("decode", 4, 2, 2, 0)] * C,
                 chunksize=1)
        for (H, Hqk) in layouts:
            for kind, n in (("prefill", n_tok), ("decode", n_dec)):
                items = [(kind, n, Hqk, H, 1000 + i) for i in range(C)]
                res = pool.map(_oracle_item, items, chunksize=1)
                multi = max(dt for _, dt in res) / n  # contended, per unit
                single = _oracle_item((kind, n, Hqk, H, 7))[1] / n
                (per_tok if kind == "prefill" else per_dec)[(H, Hqk)] = (multi, single)
    wall = time.perf_counter() - t_start
    out = {}
    for name, w in shapes.items():
        r = {}
        if w.get("prefill"):
            lens = [x for x in w["prefill"] if x > 0]
            T = sum(lens)
            if w.get("split_heads"):  # one sequence: its heads split over the cores
                hh = (max(1, w["H"] // C), max(1, w["Hqk"] // C))
                t_multi = T * per_tok[hh][0] * math.ceil(w["H"] / (hh[0] * C))
            else:
                t_multi = _lpt([x * per_tok[(w["H"], w["Hqk"])][0] for x in lens], C)
            t_single = T * per_tok[(w["H"], w["Hqk"])][1]
            r.update(prefill_tokens_per_s=T / t_multi, prefill_tokens_per_s_1core=T / t_single,
                     prefill_s=t_multi)
        if w.get("decode"):
            Bd, Hd = w["decode"], w["Hd"]
            m, s1 = per_dec[(Hd, w["Hqkd"])]
            t_multi = math.ceil(Bd / C) * m
            gb = 2 * Bd * Hd * STATE_BYTES / 1e9
            r.update(decode_state_GBps=gb / t_multi, decode_state_GBps_1core=gb / (Bd * s1),
                     decode_s=t_multi)
        out[name] = r
    hy = shapes["hybrid"]
    step_multi = layers * (out["hybrid"]["prefill_s"] + out["hybrid"]["decode_s"])
    T_h = sum(hy["prefill"])
    p1 = per_tok[(hy["H"], hy["Hqk"])][1]
    d1 = per_dec[(hy["Hd"], hy["Hqkd"])][1]
    step_single = layers * (T_h * p1 + hy["decode"] * d1)
    return {
        "value": T_h / step_multi,
        "unit": f"prefill tokens/s ({layers}-layer hybrid step incl. decode batch)",
        "cores": C,
        "kind": "oracle",
        "one_core_value": T_h / step_single,
        "sample": (f"fp64 NumPy oracle, one thread per process, {C} processes at once and 1 "
                   f"alone; per head layout each timed {n_tok} prefill tokens and {n_dec} decode "
                   f"sequences of seeded inputs drawn like the workloads; workload times: "
                   f"sequences dealt longest first to the cores (the 32-head single prompt: "
                   f"heads split over the cores), hybrid step = layer 0 x {layers} "
                   f"(extrapolated); {wall:.1f} s wall"),
        "per_workload": out,
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


def _events_ms(torch, run, n, reps=3):
    """Median over `reps` of the mean time of `n` back-to-back runs, HIP events
    on torch's current stream (the one the library launches on), after 3
    warm-up runs; also p10/p50/p90 of single runs."""
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    E = torch.cuda.Event
    stream = torch.cuda.current_stream()
    singles = []
    for _ in range(max(10, n)):
        a, b = E(enable_timing=True), E(enable_timing=True)
        a.record(stream)
        run()
        b.record(stream)
        singles.append((a, b))
    torch.cuda.synchronize()
    xs = sorted(a.elapsed_time(b) for a, b in singles)
    pct = [xs[min(len(xs) - 1, int(q * len(xs)))] for q in (0.1, 0.5, 0.9)]
    return _median_ms(torch, run, n, reps), pct


def _state_rows_prefill(prefix, new, ps):
    """State rows a paged prefill reads and stores: the read page when the
    prefix is not empty, every page boundary crossed, and the final page."""
    n = sum(1 for p, L in zip(prefix, new) if p > 0 and L > 0)
    return n + sum(1 + (p + L) // ps - p // ps for p, L in zip(prefix, new) if L > 0)


def measure_config1(torch, gdn, workloads):
    """Paged prefill with shared prefixes (8 x 16 heads, page 1024), slots
    passed (computed once, as a serving step does) and derived in the call."""
    dev = "cuda"
    c = workloads.config1(device=dev)
    p = c["prefill"]
    H, Hqk = c["H"], c["Hqk"]
    T = int(p["q"].shape[0])
    B = int(p["last_page_len"].shape[0])
    ws = torch.empty(gdn.prefill_workspace_size(T, B, H, Hqk), dtype=torch.uint8, device=dev)
    o = torch.empty(T, H, D, dtype=torch.bfloat16, device=dev)
    sl = gdn.prefill_slots(p["cu_seqlens"], p["page_indices"], p["page_indptr"],
                           p["last_page_len"], 1024)

    def run(slots):
        gdn.prefill_paged(p["q"], p["k"], p["v"], p["g"], p["beta"], p["cu_seqlens"], c["pool"],
                          p["page_indices"], p["page_indptr"], 1024, p["last_page_len"],
                          slots=slots, workspace=ws, out=o)
    by = prefill_bytes(T, H, Hqk, _state_rows_prefill(p["prefix"], p["new"], 1024))
    out = {"workload": "paged prefill, 8 sequences (prefix U[0,8192] not 64-aligned, new "
                       "U[1,4096], half sharing prefix pages), H=Hqk=16, page 1024, 512-page "
                       "fp32 pool", "tokens": T, "algorithmic_bytes": by}
    for _ in range(20):  # both variants warm before either is timed
        run(sl)
        run(None)
    for name, slots in (("slots_passed", sl), ("slots_derived", None)):
        ms, pct = _events_ms(torch, lambda: run(slots), 20, reps=5)
        out[name] = {"ms": ms, "ms_p10_p50_p90": pct, "prefill_tokens_per_s": T / (ms / 1e3),
                     "GBps": by / (ms / 1e3) / 1e9,
                     "frac_hbm_roofline": by / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS}
    whole = gdn.Options(prefill_split_chunks=-1)
    ms_whole, _ = _events_ms(torch, lambda: gdn.prefill_paged(
        p["q"], p["k"], p["v"], p["g"], p["beta"], p["cu_seqlens"], c["pool"], p["page_indices"],
        p["page_indptr"], 1024, p["last_page_len"], slots=sl, workspace=ws, out=o,
        options=whole), 20)
    out["whole_sequences_ms"] = ms_whole
    shape = dict(prefill=list(p["new"]), H=H, Hqk=Hqk)
    del c, ws, o
    return out, shape


def measure_config2(torch, gdn, workloads):
    """Paged decode (256 sequences, 16 q/k heads on 32 v-heads, page 1024),
    four page tables with disjoint touched pages used in turn so the Infinity
    Cache cannot serve rows the previous call wrote; also the same batch on a
    bf16 copy of the pool."""
    dev = "cuda"
    c = workloads.config2(device=dev)
    d = c["decode"]
    H, Hqk = c["H"], c["Hqk"]
    B = int(d["last_page_len"].shape[0])
    o = torch.empty(B, H, D, dtype=torch.bfloat16, device=dev)
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

    def run(pool):
        r = turn[0] % len(tables)
        turn[0] += 1
        gdn.decode_paged(d["q"], d["k"], d["v"], d["g"], d["beta"], pool, tables[r], ip, 1024,
                         d["last_page_len"], slots=slot_sets[r], out=o)
    by = decode_bytes(B, H, Hqk)
    ms, pct = _events_ms(torch, lambda: run(c["pool"]), 40)
    out = {"workload": "paged decode, 256 sequences (context U[1024,32768], 64 opening a new "
                       "page), Hqk=16, H=32, page 1024, 8192-page fp32 pool, four page tables "
                       "with disjoint touched pages in turn",
           "ms": ms, "ms_p10_p50_p90": pct, "state_GBps": by / (ms / 1e3) / 1e9,
           "frac_hbm_peak": by / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS, "algorithmic_bytes": by}
    pool16 = c["pool"].to(torch.bfloat16)
    del c["pool"]
    ms16, _ = _events_ms(torch, lambda: run(pool16), 40)
    by16 = by - B * H * STATE_BYTES  # state rows at 2 bytes an element
    out["bf16_pool"] = {"ms": ms16, "state_GBps": by16 / (ms16 / 1e3) / 1e9,
                        "frac_hbm_peak": by16 / (ms16 / 1e3) / 1e9 / HBM_PEAK_GBPS}
    del pool16
    shape = dict(decode=B, Hd=H, Hqkd=Hqk)
    return out, shape


def measure_config3(torch, gdn, workloads):
    """Long chunked prefill: one sequence, 32 heads, 32768 tokens in 5 calls at
    7001 / 14500 / 20000 / 27777, checkpoints every 896 tokens into a separate
    buffer (every other row -1); per call and in total, with the
    sequence-parallel plan the device picks and as whole sequences."""
    dev = "cuda"
    c = workloads.config3(device=dev)
    H, Hqk = c["H"], c["Hqk"]
    t_max = max(int(call["q"].shape[0]) for call in c["calls"])
    # one workspace for the largest call serves every call (sizes only grow)
    ws = torch.empty(gdn.prefill_workspace_size(t_max, 1, H, Hqk), dtype=torch.uint8, device=dev)

    def one(call, options=None):
        gdn.prefill(call["q"], call["k"], call["v"], call["g"], call["beta"],
                    call["cu_seqlens"], initial_state=c["pool"],
                    state_indices=call["state_indices"], output_state=c["pool"],
                    output_state_indices=call["output_state_indices"],
                    output_final_state=True, state_checkpoints=c["state_checkpoints"],
                    checkpoint_state_indices=c["checkpoint_state_indices"],
                    checkpoint_cu_starts=call["checkpoint_cu_starts"],
                    prefix_lens=call["prefix_lens"], checkpoint_every_n_tokens=c["every_n"],
                    workspace=ws, options=options)
    calls = c["calls"]
    per_call = []
    for call in calls:
        n = int(call["q"].shape[0])
        a, e = int(call["start"]), int(call["end"])
        rows = (1 if a > 0 else 0) + 1 + len([x for x in range(a // 896 + 1, e // 896 + 1)
                                              if (x - 1) % 2 == 0])
        by = prefill_bytes(n, H, Hqk, rows)
        ms, _ = _events_ms(torch, lambda: one(call), 10)
        per_call.append({"tokens": n, "ms": ms, "prefill_tokens_per_s": n / (ms / 1e3),
                         "frac_hbm_roofline": by / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS})
    T = sum(x["tokens"] for x in per_call)
    total_by = prefill_bytes(T, H, Hqk, 4 + 5 + 18)
    ms_total, _ = _events_ms(torch, lambda: [one(call) for call in calls], 5)
    whole = gdn.Options(prefill_split_chunks=-1)
    ms_whole, _ = _events_ms(torch, lambda: [one(call, whole) for call in calls], 5)
    out = {"workload": "one sequence, H=Hqk=32, 32768 tokens in 5 calls (7001/14500/20000/27777), "
                       "checkpoints every 896 into a separate buffer, every other row -1",
           "per_call": per_call, "total_ms": ms_total, "prefill_tokens_per_s": T / (ms_total / 1e3),
           "frac_hbm_roofline": total_by / (ms_total / 1e3) / 1e9 / HBM_PEAK_GBPS,
           "whole_sequence_total_ms": ms_whole, "speedup_vs_whole": ms_whole / ms_total}
    del c, ws
    shape = dict(prefill=[T], H=H, Hqk=Hqk, split_heads=True)
    return out, shape


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
    shapes = {"hybrid": dict(prefill=list(pre0["new"]), H=H, Hqk=Hqk, decode=Bd, Hd=H, Hqkd=Hqk)}
    return line, shapes


def single(args, torch, gdn, workloads):
    """One of the other workloads alone: paged prefill (config 1), paged
    decode (config 2) or the long chunked prefill (config 3)."""
    fn = {"prefill": measure_config1, "decode": measure_config2, "long": measure_config3}
    t0 = time.perf_counter()
    res, _ = fn[args.workload](torch, gdn, workloads)
    wall = time.perf_counter() - t0
    if args.workload == "prefill":
        r = res["slots_passed"]
        val, unit, ms, frac = r["prefill_tokens_per_s"], "prefill tokens/s", r["ms"], r["frac_hbm_roofline"]
    elif args.workload == "decode":
        val, unit, ms, frac = res["state_GBps"], "decode state GB/s", res["ms"], res["frac_hbm_peak"]
    else:
        val, unit, ms, frac = res["prefill_tokens_per_s"], "prefill tokens/s", res["total_ms"], res["frac_hbm_roofline"]
    line = {
        "metric": METRIC, "value": val, "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16/fp32", "data": "synthetic",
        "config": {"workload": res["workload"]},
        "roofline": {"bound": "hbm", "achieved": frac * HBM_PEAK_GBPS, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": frac, "traffic": None, "avg_launch_ms": ms},
        "detail": res, "wall_s": wall,
    }
    return line


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
        copy_gbps = plain_copy_gbps(torch, args.calibrate_copy_mib, reps=5, rounds=1)
    if args.workload != "hybrid":
        print(json.dumps(single(args, torch, gdn, workloads)), flush=True)
        return
    line, shapes = hybrid(args, torch, gdn, workloads)
    torch.cuda.empty_cache()
    if not args.no_side:
        # the other workloads, each alone after the step (their inputs made
        # and freed in turn)
        side = {}
        for name, fn in (("config1_prefill", measure_config1), ("config2_decode", measure_config2),
                         ("config3_long_prefill", measure_config3)):
            side[name], shapes[name] = fn(torch, gdn, workloads)
            torch.cuda.empty_cache()
        # what plain copies of 1 GiB reach on this GPU (1 GiB read + 1 GiB
        # written each): the library's streaming copy, which moves bytes the
        # way the decode does, and the runtime's device-to-device memcpy
        for name, use_lib in (("stream_copy", True), ("hip_memcpy_d2d", False)):
            gbps = plain_copy_gbps(torch, 1024, gdn=gdn if use_lib else None)
            side[name] = {"GBps": gbps, "frac_hbm_peak": gbps / HBM_PEAK_GBPS,
                          "bytes_per_copy": 2 << 30}
        line["side"] = side
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(shapes, args.layers)
    if copy_gbps is not None:
        line["copy_GBps"] = copy_gbps
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""GPU parity on small seeded cases: HIP path vs the fp64 oracle, element by
element, at sizes that span several chunks and ragged tails, plus the edge
cases the pages define (empty, zero-length, -1 rows, page boundaries)."""

import math
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import gdn as ogdn
from oracle import slots as oslots
from tests.gpu_util import (RowView, changed_rows, check_outputs, check_state, cuda,
                            pool_rows_cpu)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def lib():
    import paged_recurrent_state_amd as m
    m.load()
    return m


def opts(**kw):
    """Launch choices of a call (every field not given: the default)."""
    return lib().Options(**kw)


def run_prefill_paged(pre, pool, slots=None, scale=None, options=None):
    m = lib()
    return m.prefill_paged(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"],
                           pre["cu_seqlens"], pool, pre["page_indices"], pre["page_indptr"],
                           pre["page_size"], pre["last_page_len"], slots=slots, scale=scale,
                           options=options)


def state_dtype_of(pool):
    return "bf16" if pool.dtype == torch.bfloat16 else "fp32"


def oracle_prefill_paged(pre, pool_rows, state_dtype="fp32"):
    return ogdn.prefill_paged(pre["q"].cpu(), pre["k"].cpu(), pre["v"].cpu(), pre["g"].cpu(),
                              pre["beta"].cpu(), pre["cu_seqlens"].cpu(), RowView(pool_rows),
                              pre["page_indices"].cpu(), pre["page_indptr"].cpu(),
                              pre["last_page_len"].cpu(), pre["page_size"],
                              state_dtype=state_dtype)


def check_paged_prefill(pre, pool, options=None):
    """Run GPU and oracle on the same inputs; check outputs, written states,
    the write set and every untouched row bit for bit."""
    rows_in = pool_rows_cpu(pool, [r for r in pre["read_rows"]])
    before = pool.clone()
    o = run_prefill_paged(pre, pool, options=options)
    torch.cuda.synchronize()
    o_ref, writes, _ = oracle_prefill_paged(pre, rows_in, state_dtype_of(pool))
    check_outputs(o, o_ref)
    assert changed_rows(before, pool) == sorted(writes), "page-write set differs"
    errs = [check_state(pool[r], s, f"row {r}") for r, s in writes.items()]
    return o, writes, max(errs) if errs else 0.0


def test_slot_rows_config0():
    m = lib()
    c = cuda(workloads.config0())
    pre = c["prefill"]
    sl = m.prefill_slots(pre["cu_seqlens"], pre["page_indices"], pre["page_indptr"],
                         pre["last_page_len"], 128)
    ref = oslots.prefill_slots(pre["cu_seqlens"].tolist(), pre["page_indices"].tolist(),
                               pre["page_indptr"].tolist(), pre["last_page_len"].tolist(), 128)
    for name in sl._fields:
        assert getattr(sl, name).tolist() == ref[name], name
    dec = c["decode"]
    ds = m.decode_slots(dec["page_indices"], dec["page_indptr"], dec["last_page_len"])
    dref = oslots.decode_slots(dec["page_indices"].tolist(), dec["page_indptr"].tolist(),
                               dec["last_page_len"].tolist())
    for name in ds._fields:
        assert getattr(ds, name).tolist() == dref[name], name


def test_config0_prefill_then_decode():
    c = cuda(workloads.config0())
    pool = c["pool"]
    pre = c["prefill"]
    o, writes, err = check_paged_prefill(pre, pool)
    print(f"config0 prefill: worst state rel {err:.2e}")
    assert sorted(writes) == [4, 5, 9, 11, 14]
    # page 2 is allocated to seq1 but unlisted: untouched (checked by the set)
    m = lib()
    dec = c["decode"]
    rows_in = pool_rows_cpu(pool, dec["read_rows"])
    before = pool.clone()
    od = m.decode_paged(dec["q"], dec["k"], dec["v"], dec["g"], dec["beta"], pool,
                        dec["page_indices"], dec["page_indptr"], 128, dec["last_page_len"])
    torch.cuda.synchronize()
    od_ref, dwrites, _ = ogdn.decode_paged(dec["q"].cpu(), dec["k"].cpu(), dec["v"].cpu(),
                                           dec["g"].cpu(), dec["beta"].cpu(), RowView(rows_in),
                                           dec["page_indices"].cpu(), dec["page_indptr"].cpu(),
                                           dec["last_page_len"].cpu())
    check_outputs(od, od_ref)
    assert changed_rows(before, pool) == sorted(dwrites)
    for r, s in dwrites.items():
        check_state(pool[r], s)


def make_case(prefix, new, ps=64, H=2, Hqk=2, seed=0, g_scale=1.0, num_pages=None):
    """Paged prefill batch with given prefixes / new lengths; read rows random,
    all else NaN-poisoned."""
    gen = workloads.generator(seed)
    pages = []
    nxt = 0
    for p, n in zip(prefix, new):
        cnt = (p + n + ps - 1) // ps
        pages.append(list(range(nxt, nxt + cnt)))
        nxt += cnt
    num_pages = num_pages or nxt + 1
    perm = torch.randperm(num_pages, generator=gen).tolist()
    pages = [[perm[x] for x in pg] for pg in pages]
    pre = workloads._prefill_batch(prefix, new, pages, ps, Hqk, H, 128, 128, gen, "cpu", g_scale)
    pool = workloads.nan_pool(num_pages, H, 128, 128)
    workloads.fill_rows(pool, pre["read_rows"], gen, 1 / math.sqrt(128))
    return cuda(pre), pool.to(DEV)


@pytest.mark.parametrize("prefix,new", [
    ([0], [1]), ([0], [63]), ([0], [64]), ([0], [65]), ([0], [200]),
    ([5], [59]), ([5], [60]), ([63], [1]), ([63], [2]), ([64], [64]), ([100], [300]),
    ([0, 37, 128, 1], [130, 1, 64, 250]),
])
def test_prefill_ragged(prefix, new):
    pre, pool = make_case(prefix, new, seed=sum(prefix) + sum(new))
    check_paged_prefill(pre, pool)


def test_prefill_many_sequences():
    """More sequences than one planning tile (1024): the longest-first ranks
    across tiles, each chunk slot found in its tile, zero-length sequences
    (one page, prefix only) among them."""
    rng = np.random.default_rng(21)
    B = 1300
    new = rng.integers(0, 40, size=B)
    new[::7] = 0
    prefix = rng.integers(0, 200, size=B)
    prefix[new == 0] += 1  # every sequence holds at least one token
    pre, pool = make_case(prefix.tolist(), new.tolist(), H=1, Hqk=1, seed=21)
    check_paged_prefill(pre, pool)


def test_prefill_low_decay_gqa():
    # slow decay keeps the prefix state alive across chunks; 4 v-heads on 2 q/k heads
    pre, pool = make_case([70, 0, 300], [400, 333, 129], H=4, Hqk=2, seed=3, g_scale=0.1)
    _, _, err = check_paged_prefill(pre, pool)
    print(f"low decay: worst state rel {err:.2e}")


def test_prefill_no_decay():
    pre, pool = make_case([10, 0], [300, 200], seed=4, g_scale=0.0)
    _, _, err = check_paged_prefill(pre, pool)
    print(f"no decay: worst state rel {err:.2e}")


def test_prefill_zero_length_and_empty():
    m = lib()
    # one zero-length sequence among others: it writes nothing
    pre, pool = make_case([64, 10, 0], [100, 0, 70], seed=5)
    check_paged_prefill(pre, pool)
    # a batch whose every sequence has no new tokens leaves the pool unchanged
    pre, pool = make_case([5, 64], [0, 0], seed=6)
    before = pool.clone()
    o = run_prefill_paged(pre, pool)
    torch.cuda.synchronize()
    assert o.shape[0] == 0
    assert changed_rows(before, pool) == []


def test_prefill_example_2500_tokens():
    # pages [7, 3, 12], page 1024, 452 new tokens: reads page 3, writes page 12 only
    gen = workloads.generator(9)
    pre = workloads._prefill_batch([2048], [452], [[7, 3, 12]], 1024, 2, 2, 128, 128, gen, "cpu")
    pool = workloads.nan_pool(16, 2, 128, 128)
    workloads.fill_rows(pool, [3], gen, 1 / math.sqrt(128))
    pre, pool = cuda(pre), pool.to(DEV)
    _, writes, _ = check_paged_prefill(pre, pool)
    assert sorted(writes) == [12]


def test_prefill_slots_passed_equals_derived():
    m = lib()
    pre, pool = make_case([0, 37, 128, 1], [130, 1, 64, 250], seed=11)
    pool2 = pool.clone()
    o1 = run_prefill_paged(pre, pool)
    sl = m.prefill_slots(pre["cu_seqlens"], pre["page_indices"], pre["page_indptr"],
                         pre["last_page_len"], pre["page_size"])
    o2 = run_prefill_paged(pre, pool2, slots=sl)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert changed_rows(pool, pool2) == []


def test_decode_paths_agree_and_match_oracle():
    m = lib()
    c = cuda(workloads.config2(num_seqs=24, qk_heads=2, v_heads=4, num_pages=24 * 32,
                               new_page_seqs=8))
    dec, pool = c["decode"], c["pool"]
    rows_in = pool_rows_cpu(pool, dec["read_rows"])
    pool2 = pool.clone()
    before = pool.clone()
    o1 = m.decode_paged(dec["q"], dec["k"], dec["v"], dec["g"], dec["beta"], pool,
                        dec["page_indices"], dec["page_indptr"], 1024, dec["last_page_len"])
    sl = m.decode_slots(dec["page_indices"], dec["page_indptr"], dec["last_page_len"])
    o2 = m.decode_paged(dec["q"], dec["k"], dec["v"], dec["g"], dec["beta"], pool2,
                        dec["page_indices"], dec["page_indptr"], 1024, dec["last_page_len"],
                        slots=sl)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert changed_rows(pool, pool2) == []
    o_ref, writes, sref = ogdn.decode_paged(dec["q"].cpu(), dec["k"].cpu(), dec["v"].cpu(),
                                            dec["g"].cpu(), dec["beta"].cpu(), RowView(rows_in),
                                            dec["page_indices"].cpu(), dec["page_indptr"].cpu(),
                                            dec["last_page_len"].cpu())
    assert sl.initial_state_indices.tolist() == sref["initial_state_indices"]
    assert sl.output_state_indices.tolist() == sref["output_state_indices"]
    check_outputs(o1, o_ref)
    assert changed_rows(before, pool) == sorted(writes)
    for r, s in writes.items():
        check_state(pool[r], s)


@pytest.mark.parametrize("waves", ["2", "4", "8", "16", "stream", "stream-grid-5"])
def test_decode_every_workgroup_width(waves):
    """Each decode kernel shape against the oracle, fp32 and bf16 pools, GQA
    and new-page rows: one (sequence, head) per workgroup of 2, 4, 8 or 16
    waves (64 / 32 / 16 / 8 rows a wave), and the streaming walk -- its
    default grid, and a grid of 5 workgroups so each walks ~10 pairs through
    its prefetch pipeline."""
    m = lib()
    o_kw = {"stream": dict(decode_stream_per_cu=6),
            "stream-grid-5": dict(decode_stream_grid=5)}.get(waves, dict(decode_waves=int(waves) if waves.isdigit() else 0))
    options = opts(**o_kw)
    c = cuda(workloads.config2(num_seqs=12, qk_heads=2, v_heads=4, num_pages=12 * 32,
                               new_page_seqs=4, seed=40 + len(waves)))
    dec = c["decode"]
    for pool in (c["pool"], c["pool"].to(torch.bfloat16)):
        rows_in = pool_rows_cpu(pool, dec["read_rows"])
        before = pool.clone()
        o = m.decode_paged(dec["q"], dec["k"], dec["v"], dec["g"], dec["beta"], pool,
                           dec["page_indices"], dec["page_indptr"], 1024, dec["last_page_len"],
                           options=options)
        torch.cuda.synchronize()
        o_ref, writes, _ = ogdn.decode_paged(dec["q"].cpu(), dec["k"].cpu(), dec["v"].cpu(),
                                             dec["g"].cpu(), dec["beta"].cpu(),
                                             RowView(rows_in), dec["page_indices"].cpu(),
                                             dec["page_indptr"].cpu(),
                                             dec["last_page_len"].cpu(),
                                             state_dtype=state_dtype_of(pool))
        check_outputs(o, o_ref)
        assert changed_rows(before, pool) == sorted(writes)
        for r, s in writes.items():
            check_state(pool[r], s)


@pytest.mark.parametrize("idx_dtype", [torch.int32, torch.int64])
def test_general_decode_rows(idx_dtype):
    m = lib()
    gen = workloads.generator(21)
    B, H, Hqk = 5, 4, 2
    t = cuda(workloads.token_inputs(B, Hqk, H, 128, 128, gen))
    init = (torch.randn(6, H, 128, 128, generator=gen) / math.sqrt(128)).to(DEV)
    out = workloads.nan_pool(7, H, 128, 128, device=DEV)
    before = out.clone()
    rd = torch.tensor([0, -1, 3, 5, 2], dtype=idx_dtype, device=DEV)
    wr = torch.tensor([1, 2, -1, 6, 0], dtype=idx_dtype, device=DEV)
    o = m.decode(t["q"], t["k"], t["v"], t["g"], t["beta"], initial_state=init,
                 initial_state_indices=rd, output_state=out, output_state_indices=wr)
    torch.cuda.synchronize()
    res = ogdn.decode(t["q"].cpu(), t["k"].cpu(), t["v"].cpu(), t["g"].cpu(), t["beta"].cpu(),
                      initial_state=init.cpu().numpy(), initial_state_indices=rd.tolist(),
                      output_state_indices=wr.tolist(), shared_pool=False)
    check_outputs(o, res.o)
    assert changed_rows(before, out) == sorted(res.final)
    for r, s in res.final.items():
        check_state(out[r], s)


@pytest.mark.parametrize("idx_dtype,N,g_scale", [(torch.int32, 128, 1.0), (torch.int64, 128, 1.0),
                                                  (torch.int32, 100, 0.1), (torch.int32, 48, 1.0),
                                                  (torch.int64, 17, 0.1), (torch.int32, 1, 0.1)])
def test_general_prefill_checkpoints(idx_dtype, N, g_scale):
    """Slot-argument prefill in pieces with checkpoints every N tokens into a
    separate buffer (-1 rows skipped) and a padded row stride.  N not a
    multiple of 64 puts checkpoints inside chunks (N = 1: after every token)."""
    m = lib()
    H = Hqk = 2
    c = workloads.config3(heads=H, total=1000, splits=(131, 400, 640), every_n=N, num_rows=3,
                          g_scale=g_scale)
    c = cuda(c)
    ckpt = workloads.nan_pool(1000 // N, H, 128, 128, device=DEV, row_stride=H * 128 * 128 + 64)
    slot_pool = c["pool"]
    ck_rows = c["checkpoint_state_indices"].to(idx_dtype)
    ref_slot = np.zeros((3, H, 128, 128))
    ref_ck = {}
    for call in c["calls"]:
        cast = {k: call[k].to(idx_dtype) for k in ("state_indices", "output_state_indices",
                                                   "prefix_lens", "checkpoint_cu_starts")}
        o = m.prefill(call["q"], call["k"], call["v"], call["g"], call["beta"], call["cu_seqlens"],
                      initial_state=slot_pool, state_indices=cast["state_indices"],
                      output_state=slot_pool, output_state_indices=cast["output_state_indices"],
                      output_final_state=True, state_checkpoints=ckpt,
                      checkpoint_state_indices=ck_rows,
                      checkpoint_cu_starts=cast["checkpoint_cu_starts"],
                      prefix_lens=cast["prefix_lens"], checkpoint_every_n_tokens=N)
        torch.cuda.synchronize()
        res = ogdn.prefill(call["q"].cpu(), call["k"].cpu(), call["v"].cpu(), call["g"].cpu(),
                           call["beta"].cpu(), call["cu_seqlens"].cpu(), initial_state=ref_slot,
                           state_indices=call["state_indices"].tolist(),
                           output_final_state=True,
                           output_state_indices=call["output_state_indices"].tolist(),
                           checkpoint_state_indices=c["checkpoint_state_indices"].tolist(),
                           checkpoint_cu_starts=call["checkpoint_cu_starts"].tolist(),
                           prefix_lens=call["prefix_lens"].tolist(), checkpoint_every_n_tokens=N,
                           shared_pool=False)
        check_outputs(o, res.o)
        ref_slot = ogdn.apply_writes(ref_slot, res.final)
        ref_ck.update(res.checkpoints)
        check_state(slot_pool[c["slot"]], ref_slot[c["slot"]], "slot")
    n_ck = 1000 // N
    got = [r for r in range(n_ck) if torch.isfinite(ckpt[r]).all()]
    assert got == sorted(ref_ck) == [r for r in range(n_ck) if r % 2 == 0]
    for r, s in ref_ck.items():
        check_state(ckpt[r], s, f"checkpoint {r}")
    # odd rows kept their NaN bits
    for r in range(n_ck):
        if r % 2:
            assert (ckpt[r].view(torch.int32) == workloads.NAN_BITS).all()


def test_general_prefill_no_state_buffers():
    """No initial state, no final store: outputs only, from the zero state."""
    m = lib()
    gen = workloads.generator(31)
    t = cuda(workloads.token_inputs(300, 2, 2, 128, 128, gen))
    cu = torch.tensor([0, 100, 100, 300], dtype=torch.int32, device=DEV)
    o = m.prefill(t["q"], t["k"], t["v"], None, None, cu)
    torch.cuda.synchronize()
    res = ogdn.prefill(t["q"].cpu(), t["k"].cpu(), t["v"].cpu(), None, None, cu.cpu())
    check_outputs(o, res.o)


def test_split_invariance_on_gpu():
    """Prefill at any split resumes from the written page: GPU split run vs the
    oracle's unsplit run, within tolerance."""
    m = lib()
    ps = 128
    T = 700
    gen = workloads.generator(41)
    t = cuda(workloads.token_inputs(T, 2, 2, 128, 128, gen, g_scale=0.1))
    pages = [9, 2, 7, 4, 0, 6]
    pool = workloads.nan_pool(10, 2, 128, 128, device=DEV)
    o_ref = ogdn.prefill_paged(t["q"].cpu(), t["k"].cpu(), t["v"].cpu(), t["g"].cpu(),
                               t["beta"].cpu(), [0, T], np.zeros((10, 2, 128, 128)),
                               pages, [0, 6], [T - 5 * ps], ps)
    outs = []
    cuts = [0, 77, 128, 129, 450, T]
    for a, b in zip(cuts, cuts[1:]):
        n = (b + ps - 1) // ps
        idx = torch.tensor(pages[:n], dtype=torch.int32, device=DEV)
        ptr = torch.tensor([0, n], dtype=torch.int32, device=DEV)
        lpl = torch.tensor([b - (n - 1) * ps], dtype=torch.int32, device=DEV)
        cu = torch.tensor([0, b - a], dtype=torch.int32, device=DEV)
        outs.append(m.prefill_paged(t["q"][a:b].contiguous(), t["k"][a:b].contiguous(),
                                    t["v"][a:b].contiguous(), t["g"][a:b].contiguous(),
                                    t["beta"][a:b].contiguous(), cu, pool, idx, ptr, ps, lpl))
    torch.cuda.synchronize()
    check_outputs(torch.cat(outs), o_ref[0])
    for r, s in o_ref[1].items():
        check_state(pool[r], s, f"page {r}")


def check_sliced_general(H=2, Hqk=None, N=128, total=1000, splits=(131, 400, 640), g_scale=0.1,
                         options=None, state_dtype=torch.float32, seed=3, idx_dtype=torch.int32,
                         in_place_default=False):
    """A long sequence through the slot-argument call in pieces (state kept in
    one slot row, read and written in place), checkpoints every N tokens into
    a separate NaN-filled buffer with every other row -1; each piece against
    the oracle, then the checkpoint rows.  ``in_place_default`` passes no
    output_state_indices (the write row is then the read row).  Returns the
    worst state error."""
    m = lib()
    sd = "bf16" if state_dtype == torch.bfloat16 else "fp32"
    c = cuda(workloads.config3(heads=H, qk_heads=Hqk, total=total, splits=splits, every_n=N,
                               num_rows=3, g_scale=g_scale, seed=seed))
    slot_pool = c["pool"].to(state_dtype)
    n_ck = total // N
    ckpt = workloads.nan_pool(max(n_ck, 1), H, 128, 128, device=DEV).to(state_dtype)
    ckpt0 = ckpt.clone()
    ck_rows = c["checkpoint_state_indices"].to(idx_dtype)
    ref_slot = np.zeros((3, H, 128, 128))
    ref_ck = {}
    worst = 0.0
    for call in c["calls"]:
        cast = {k: call[k].to(idx_dtype) for k in ("state_indices", "output_state_indices",
                                                   "prefix_lens", "checkpoint_cu_starts")}
        if in_place_default and call["start"] > 0:
            wr = None  # the read row, which is the slot
        else:
            wr = cast["output_state_indices"]
        o = m.prefill(call["q"], call["k"], call["v"], call["g"], call["beta"], call["cu_seqlens"],
                      initial_state=slot_pool, state_indices=cast["state_indices"],
                      output_state=slot_pool, output_state_indices=wr,
                      output_final_state=True, state_checkpoints=ckpt,
                      checkpoint_state_indices=ck_rows,
                      checkpoint_cu_starts=cast["checkpoint_cu_starts"],
                      prefix_lens=cast["prefix_lens"], checkpoint_every_n_tokens=N,
                      options=options)
        torch.cuda.synchronize()
        res = ogdn.prefill(call["q"].cpu(), call["k"].cpu(), call["v"].cpu(), call["g"].cpu(),
                           call["beta"].cpu(), call["cu_seqlens"].cpu(), initial_state=ref_slot,
                           state_indices=call["state_indices"].tolist(), output_final_state=True,
                           output_state_indices=call["output_state_indices"].tolist(),
                           checkpoint_state_indices=c["checkpoint_state_indices"].tolist(),
                           checkpoint_cu_starts=call["checkpoint_cu_starts"].tolist(),
                           prefix_lens=call["prefix_lens"].tolist(), checkpoint_every_n_tokens=N,
                           shared_pool=False, state_dtype=sd)
        check_outputs(o, res.o)
        ref_slot = ogdn.apply_writes(ref_slot, res.final)
        ref_ck.update(res.checkpoints)
        worst = max(worst, check_state(slot_pool[c["slot"]], ref_slot[c["slot"]], "slot"))
    got = [r for r in range(n_ck) if torch.isfinite(ckpt[r].float()).all()]
    assert got == sorted(ref_ck) == [r for r in range(n_ck) if r % 2 == 0]
    for r, st in ref_ck.items():
        worst = max(worst, check_state(ckpt[r], st, f"checkpoint {r}"))
    # odd rows (-1 entries) keep their NaN bits
    assert changed_rows(ckpt0, ckpt) == [r for r in range(n_ck) if r % 2 == 0]
    return worst


@pytest.mark.parametrize("waves", [8, 4, 2, 1])
def test_prefill_every_tile_width(waves):
    """The recurrence kernel in each of its V-tile widths (8, 4, 2 or 1 waves
    per workgroup): ragged sequences, GQA, slow decay, and a general call with
    checkpoints."""
    o = opts(prefill_tile_waves=waves, prefill_split_chunks=-1)
    pre, pool = make_case([0, 37, 128, 1], [130, 1, 64, 250], H=4, Hqk=2, seed=7, g_scale=0.3)
    _, _, err = check_paged_prefill(pre, pool, options=o)
    check_sliced_general(H=2, N=128, total=600, splits=(131, 400), g_scale=1.0, options=o)
    print(f"{waves} waves per workgroup: worst paged state rel {err:.2e}")


@pytest.mark.parametrize("m,waves", [(1, 8), (2, 8), (3, 8), (5, 8), (2, 4)])
def test_prefill_sequence_parallel(m, waves):
    """The sequence-parallel recurrence forced with segments of m chunks:
    the segments' offsets (zero start) and transitions (identity start, v =
    0), the scan of the segment maps and the second pass from the scanned
    starts.  Ragged paged sequences with GQA and slow decay (so start states
    matter across segments), then a sliced long sequence through the general
    call with checkpoints inside and at the ends of chunks."""
    o = opts(prefill_split_chunks=m, prefill_tile_waves=waves)
    pre, pool = make_case([0, 37, 128, 1000], [700, 1, 64, 900], ps=128, H=4, Hqk=2,
                          seed=11 + m, g_scale=0.1)
    _, _, err = check_paged_prefill(pre, pool, options=o)
    for N in (100, 128):
        check_sliced_general(H=2, N=N, options=o)
    print(f"segments of {m} chunks, {waves} waves: worst paged state rel {err:.2e}")


@pytest.mark.parametrize("m", [1, 2])
def test_sequence_parallel_rows_read_and_written(m):
    """Rows the second pass both reads and writes, under forced segments:
    a paged prefix ending inside a page (37 of 128 tokens) whose page a later
    segment checkpoints, next to a page-aligned prefix whose read page is
    outside the call's write set; and the slot-argument call with no
    output_state_indices, which updates each read row in place."""
    o = opts(prefill_split_chunks=m)
    pre, pool = make_case([37, 1, 256, 130], [700, 400, 300, 126], ps=128, H=2, Hqk=1,
                          seed=60 + m, g_scale=0.1)
    _, writes, err = check_paged_prefill(pre, pool, options=o)
    read_rows = [r for r in pre["read_rows"] if r >= 0]
    assert read_rows[0] in writes and read_rows[1] in writes  # read pages re-stored by later segments
    worst = check_sliced_general(H=2, N=100, options=o, in_place_default=True)
    print(f"segments of {m}: worst state rel {err:.2e} / {worst:.2e}")


# ---- v-heads placed on the XCDs in q/k-head groups: H a multiple of 8 H / Hqk

@pytest.mark.parametrize("H,Hqk,split,waves", [(16, 8, -1, 8), (16, 8, 2, 8), (32, 16, -1, 8),
                                               (32, 16, 3, 8), (32, 16, -1, 4), (16, 8, 0, 8)])
def test_prefill_gqa_head_placement(H, Hqk, split, waves):
    """Head layouts where the recurrence and intra-chunk workgroups map block
    indices to v-heads in q/k-head groups (H a multiple of 8 H / Hqk): every
    head against the oracle, whole sequences and forced segments, a tile
    width below whole heads, and the device-planned split (split 0)."""
    o = opts(prefill_split_chunks=split, prefill_tile_waves=waves)
    pre, pool = make_case([0, 37, 1000], [700, 190, 400], ps=128, H=H, Hqk=Hqk,
                          seed=H + Hqk + split, g_scale=0.1)
    _, writes, err = check_paged_prefill(pre, pool, options=o)
    assert len(writes) >= 6
    print(f"H={H} Hqk={Hqk} split {split} waves {waves}: worst state rel {err:.2e}")


@pytest.mark.parametrize("H,Hqk,split,waves", [(32, 8, -1, 8), (32, 8, 2, 4), (64, 8, -1, 8),
                                               (64, 8, 0, 8)])
def test_paged_prefill_wide_groups(H, Hqk, split, waves):
    """Groups of 4 and 8 v-heads per q/k head (32 on 8, 64 on 8), where the
    prefill kernels place eight q/k heads' groups side by side: forced and
    device-planned segments, a 4-wave tile, every head checked."""
    o = opts(prefill_split_chunks=split, prefill_tile_waves=waves)
    pre, pool = make_case([0, 37, 130], [600, 190, 300], ps=128, H=H, Hqk=Hqk,
                          seed=H + Hqk + split + waves, g_scale=0.1)
    _, writes, err = check_paged_prefill(pre, pool, options=o)
    assert len(writes) >= 4
    print(f"H={H} Hqk={Hqk} split {split} waves {waves}: worst state rel {err:.2e}")


@pytest.mark.parametrize("H,Hqk,split", [(16, 8, -1), (32, 16, 2)])
def test_general_prefill_gqa_head_placement(H, Hqk, split):
    """The slot-argument call with interior checkpoints (every 100 tokens) on
    the grouped head placement, int64 rows."""
    err = check_sliced_general(H=H, Hqk=Hqk, N=100, total=700, splits=(131, 400),
                               options=opts(prefill_split_chunks=split), idx_dtype=torch.int64)
    print(f"H={H} Hqk={Hqk} split {split}: worst state rel {err:.2e}")


def test_bf16_pool_gqa_head_placement():
    pre, pool = make_case([0, 37, 1000], [500, 190, 300], ps=128, H=32, Hqk=16, seed=77,
                          g_scale=0.3)
    pool = pool.to(torch.bfloat16)
    _, writes, err = check_paged_prefill(pre, pool)
    print(f"bf16 pool, H=32 Hqk=16: worst state rel {err:.2e}")


# ---- bf16 state pools: states stored rounded to bf16, arithmetic in fp32

@pytest.mark.parametrize("split", [-1, 2])
def test_bf16_pool_prefill(split):
    """Paged prefill on a bf16 pool (whole sequences, and forced segments of
    2 chunks): bf16 read rows, rounded page-boundary and final stores, the
    write set and every untouched row bit for bit."""
    pre, pool = make_case([0, 37, 128, 1000], [700, 1, 64, 900], ps=128, H=4, Hqk=2,
                          seed=31, g_scale=0.3)
    pool = pool.to(torch.bfloat16)
    _, writes, err = check_paged_prefill(pre, pool, options=opts(prefill_split_chunks=split))
    assert len(writes) > 4
    print(f"bf16 pool prefill (split {split}): worst state rel {err:.2e}")


def test_bf16_pool_prefill_then_decode():
    c = cuda(workloads.config0())
    pool = c["pool"].to(torch.bfloat16)
    pre = c["prefill"]
    _, writes, _ = check_paged_prefill(pre, pool)
    assert sorted(writes) == [4, 5, 9, 11, 14]
    m = lib()
    dec = c["decode"]
    rows_in = pool_rows_cpu(pool, dec["read_rows"])
    before = pool.clone()
    od = m.decode_paged(dec["q"], dec["k"], dec["v"], dec["g"], dec["beta"], pool,
                        dec["page_indices"], dec["page_indptr"], 128, dec["last_page_len"])
    torch.cuda.synchronize()
    od_ref, dwrites, _ = ogdn.decode_paged(dec["q"].cpu(), dec["k"].cpu(), dec["v"].cpu(),
                                           dec["g"].cpu(), dec["beta"].cpu(), RowView(rows_in),
                                           dec["page_indices"].cpu(), dec["page_indptr"].cpu(),
                                           dec["last_page_len"].cpu(), state_dtype="bf16")
    check_outputs(od, od_ref)
    assert changed_rows(before, pool) == sorted(dwrites)
    for r, st in dwrites.items():
        check_state(pool[r], st)


def test_bf16_pool_decode_batch():
    """64 sequences (16 opening a new page) on a bf16 pool, GQA 16 -> 32 heads."""
    m = lib()
    c = workloads.config2(device=DEV, num_seqs=64, num_pages=2048, new_page_seqs=16)
    pool = c["pool"].to(torch.bfloat16)
    del c["pool"]
    d = c["decode"]
    rows_in = pool_rows_cpu(pool, d["read_rows"])
    before = pool.clone()
    o = m.decode_paged(d["q"], d["k"], d["v"], d["g"], d["beta"], pool, d["page_indices"],
                       d["page_indptr"], 1024, d["last_page_len"])
    torch.cuda.synchronize()
    o_ref, writes, _ = ogdn.decode_paged(d["q"].cpu(), d["k"].cpu(), d["v"].cpu(), d["g"].cpu(),
                                         d["beta"].cpu(), RowView(rows_in), d["page_indices"].cpu(),
                                         d["page_indptr"].cpu(), d["last_page_len"].cpu(),
                                         state_dtype="bf16")
    check_outputs(o, o_ref)
    assert changed_rows(before, pool) == sorted(writes)
    worst = max(check_state(pool[r], st) for r, st in writes.items())
    print(f"bf16 pool decode batch: worst state rel {worst:.2e}")


def test_bf16_general_prefill_checkpoints():
    """Slot-argument prefill in pieces on bf16 state buffers with checkpoints
    every 100 tokens (inside chunks) into a separate bf16 buffer."""
    err = check_sliced_general(H=2, N=100, state_dtype=torch.bfloat16)
    print(f"bf16 general: worst state rel {err:.2e}")


def test_state_buffers_share_one_dtype():
    m = lib()
    gen = workloads.generator(5)
    t = cuda(workloads.token_inputs(64, 2, 2, 128, 128, gen))
    cu = torch.tensor([0, 64], dtype=torch.int32, device=DEV)
    a = torch.zeros(1, 2, 128, 128, device=DEV)
    with pytest.raises(TypeError):
        m.prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], cu, initial_state=a,
                  output_state=a.to(torch.bfloat16), output_final_state=True)
    with pytest.raises(TypeError):
        m.prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], cu, initial_state=a.half())

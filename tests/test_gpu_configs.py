"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times.  Heads (and sequences) are independent, so where the oracle
would take minutes it computes a sampled subset of them (the ragged paged
prefill is checked on every head); page-write sets and untouched rows are
checked on the whole pool, bit for bit."""

import numpy as np
import pytest
import torch

import workloads
from oracle import gdn as ogdn
from oracle import slots as oslots
from tests.gpu_util import RowView, changed_rows, check_outputs, check_state

pytestmark = pytest.mark.gpu
DEV = "cuda"


def lib():
    import paged_recurrent_state_amd as m
    m.load()
    return m


def head_slice(batch, heads, group):
    """Token inputs restricted to v-heads ``heads`` (q/k mapped per v-head)."""
    qk = [h // group for h in heads]
    return {
        "q": batch["q"][:, qk].cpu(), "k": batch["k"][:, qk].cpu(),
        "v": batch["v"][:, heads].cpu(), "g": batch["g"][:, heads].cpu(),
        "beta": batch["beta"][:, heads].cpu(),
    }


def rows_of(pool, rows, heads):
    return {int(r): pool[int(r)][heads].cpu().numpy() for r in set(rows) if int(r) >= 0}


def seq_slice(batch, seqs):
    """Token rows and page tables of a subset of sequences (for the oracle)."""
    cu = batch["cu_seqlens"].tolist()
    idx = batch["page_indices"].tolist()
    ptr = batch["page_indptr"].tolist()
    lpl = batch["last_page_len"].tolist()
    toks, ncu, nidx, nptr, nlpl = [], [0], [], [0], []
    for b in seqs:
        toks.extend(range(cu[b], cu[b + 1]))
        ncu.append(ncu[-1] + cu[b + 1] - cu[b])
        nidx.extend(idx[ptr[b]:ptr[b + 1]])
        nptr.append(len(nidx))
        nlpl.append(lpl[b])
    return toks, ncu, nidx, nptr, nlpl


def test_config1_prefill_full():
    """Every head of the ragged 8-sequence batch (the oracle takes ~15 s)."""
    m = lib()
    c = workloads.config1(device=DEV)
    pre, pool = c["prefill"], c["pool"]
    H = c["H"]
    heads = list(range(H))
    rows_in = rows_of(pool, pre["read_rows"], heads)
    before = pool.clone()
    o = m.prefill_paged(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], pre["cu_seqlens"],
                        pool, pre["page_indices"], pre["page_indptr"], 1024,
                        pre["last_page_len"])
    torch.cuda.synchronize()
    hs = head_slice(pre, heads, 1)
    o_ref, writes, _ = ogdn.prefill_paged(hs["q"], hs["k"], hs["v"], hs["g"], hs["beta"],
                                          pre["cu_seqlens"].cpu(), RowView(rows_in),
                                          pre["page_indices"].cpu(), pre["page_indptr"].cpu(),
                                          pre["last_page_len"].cpu(), 1024)
    mx, rf = check_outputs(o[:, heads], o_ref)
    assert changed_rows(before, pool) == sorted(writes)
    worst = max(check_state(pool[r][heads], s, f"page {r}") for r, s in writes.items())
    print(f"config1 prefill: o max abs {mx:.2e} rel {rf:.2e}; worst state rel {worst:.2e}")
    assert H == 16


def test_config2_decode_full():
    m = lib()
    c = workloads.config2(device=DEV)
    dec, pool = c["decode"], c["pool"]
    H, Hqk = c["H"], c["Hqk"]
    sl = m.decode_slots(dec["page_indices"], dec["page_indptr"], dec["last_page_len"])
    sref = oslots.decode_slots(dec["page_indices"].tolist(), dec["page_indptr"].tolist(),
                               dec["last_page_len"].tolist())
    assert sl.initial_state_indices.tolist() == sref["initial_state_indices"]
    assert sl.output_state_indices.tolist() == sref["output_state_indices"]
    assert sum(1 for x in dec["last_page_len"].tolist() if x == 1) >= 64
    heads = list(range(H))
    rows_in = {r: pool[r].cpu().numpy() for r in set(sref["initial_state_indices"])}
    before = pool.clone()
    o = m.decode_paged(dec["q"], dec["k"], dec["v"], dec["g"], dec["beta"], pool,
                       dec["page_indices"], dec["page_indptr"], 1024, dec["last_page_len"],
                       slots=sl)
    torch.cuda.synchronize()
    hs = head_slice(dec, heads, H // Hqk)
    o_ref, writes, _ = ogdn.decode_paged(hs["q"], hs["k"], hs["v"], hs["g"], hs["beta"],
                                         RowView(rows_in), dec["page_indices"].cpu(),
                                         dec["page_indptr"].cpu(), dec["last_page_len"].cpu())
    check_outputs(o, o_ref)
    assert changed_rows(before, pool) == sorted(writes)
    worst = max(check_state(pool[r], s, f"page {r}") for r, s in writes.items())
    print(f"config2 decode: worst state rel err {worst:.2e}")


def test_config3_long_prefill_full():
    m = lib()
    c = workloads.config3(device=DEV)
    H = c["H"]
    heads = [3, 30]
    N = c["every_n"]
    slot = c["slot"]
    ref_slot = {}
    ref_ck = {}
    for call in c["calls"]:
        o = m.prefill(call["q"], call["k"], call["v"], call["g"], call["beta"],
                      call["cu_seqlens"], initial_state=c["pool"],
                      state_indices=call["state_indices"], output_state=c["pool"],
                      output_state_indices=call["output_state_indices"],
                      output_final_state=True, state_checkpoints=c["state_checkpoints"],
                      checkpoint_state_indices=c["checkpoint_state_indices"],
                      checkpoint_cu_starts=call["checkpoint_cu_starts"],
                      prefix_lens=call["prefix_lens"], checkpoint_every_n_tokens=N)
        torch.cuda.synchronize()
        hs = head_slice(call, heads, 1)
        res = ogdn.prefill(hs["q"], hs["k"], hs["v"], hs["g"], hs["beta"], [0, call["end"] - call["start"]],
                           initial_state=RowView(ref_slot),
                           state_indices=call["state_indices"].tolist(), output_final_state=True,
                           output_state_indices=call["output_state_indices"].tolist(),
                           checkpoint_state_indices=c["checkpoint_state_indices"].tolist(),
                           checkpoint_cu_starts=call["checkpoint_cu_starts"].tolist(),
                           prefix_lens=call["prefix_lens"].tolist(), checkpoint_every_n_tokens=N,
                           shared_pool=False)
        mx, rf = check_outputs(o[:, heads], res.o, f"call at {call['start']}")
        print(f"config3 call at {call['start']}: o max abs {mx:.2e} rel {rf:.2e}")
        ref_slot.update(res.final)
        ref_ck.update(res.checkpoints)
        check_state(c["pool"][slot][heads], ref_slot[slot], f"slot after {call['end']}")
    assert sorted(ref_ck) == list(range(0, 36, 2))
    ck = c["state_checkpoints"]
    for r in range(36):
        if r in ref_ck:
            check_state(ck[r][heads], ref_ck[r], f"checkpoint {r}")
        else:
            assert (ck[r].view(torch.int32) == workloads.NAN_BITS).all(), f"checkpoint {r} written"


@pytest.mark.parametrize("qk_heads", [32, 16])
def test_config4_hybrid_layer(qk_heads):
    """One layer of the hybrid step with slots derived once: sampled sequences
    and heads against the oracle, write sets on the whole pool.  With 16 q/k
    heads the prefill kernels place the v-heads in q/k-head pairs; the sampled
    heads then cover both v-heads of a pair and both halves of the q/k heads."""
    m = lib()
    c = workloads.config4(device=DEV, layers=(0,), qk_heads=qk_heads)
    group = c["H"] // c["Hqk"]
    pool = c["pool"]
    pre, dec = c["layers"][0]["prefill"], c["layers"][0]["decode"]
    ps = c["page_size"]
    sl_p = m.prefill_slots(pre["cu_seqlens"], pre["page_indices"], pre["page_indptr"],
                           pre["last_page_len"], ps)
    sl_d = m.decode_slots(dec["page_indices"], dec["page_indptr"], dec["last_page_len"])
    ref_p = oslots.prefill_slots(pre["cu_seqlens"].tolist(), pre["page_indices"].tolist(),
                                 pre["page_indptr"].tolist(), pre["last_page_len"].tolist(), ps)
    for name in sl_p._fields:
        assert getattr(sl_p, name).tolist() == ref_p[name], name
    heads = [5, 26] if group == 1 else [5, 10, 19, 26]
    seqs_p = [0, 9, 31, 33]        # includes one padded (zero-length) sequence
    seqs_d = list(range(0, 528, 17))
    rows_in_p = rows_of(pool, [pre["read_rows"][b] for b in seqs_p if pre["new"][b] > 0], heads)
    dslots = oslots.decode_slots(dec["page_indices"].tolist(), dec["page_indptr"].tolist(),
                                 dec["last_page_len"].tolist())
    assert sl_d.initial_state_indices.tolist() == dslots["initial_state_indices"]
    rows_in_d = rows_of(pool, [dslots["initial_state_indices"][b] for b in seqs_d], heads)
    before = pool.clone()
    o_p = m.prefill_paged(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"],
                          pre["cu_seqlens"], pool, pre["page_indices"], pre["page_indptr"], ps,
                          pre["last_page_len"], slots=sl_p)
    o_d = m.decode_paged(dec["q"], dec["k"], dec["v"], dec["g"], dec["beta"], pool,
                         dec["page_indices"], dec["page_indptr"], ps, dec["last_page_len"],
                         slots=sl_d)
    torch.cuda.synchronize()
    # full write set: every prefill page from the first one ending after the
    # prefix, plus every decode write row
    full_p = oslots.prefill_slots(pre["cu_seqlens"].tolist(), pre["page_indices"].tolist(),
                                  pre["page_indptr"].tolist(), pre["last_page_len"].tolist(), ps)
    expect = set(dslots["output_state_indices"])
    ptr = pre["page_indptr"].tolist()
    idx = pre["page_indices"].tolist()
    for b in range(len(pre["new"])):
        if pre["new"][b] == 0:
            continue
        p = full_p["prefix_lens"][b]
        n_pages = ptr[b + 1] - ptr[b]
        for j in range(p // ps, n_pages):
            expect.add(idx[ptr[b] + j])
    assert changed_rows(before, pool) == sorted(expect)
    # prefill oracle on sampled sequences and heads
    toks, ncu, nidx, nptr, nlpl = seq_slice(pre, seqs_p)
    hs = head_slice(pre, heads, group)
    sub = {k: v[toks] for k, v in hs.items()}
    o_ref, writes, _ = ogdn.prefill_paged(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"],
                                          ncu, RowView(rows_in_p), nidx, nptr, nlpl, ps)
    check_outputs(o_p[toks][:, heads], o_ref, "prefill o")
    for r, s in writes.items():
        check_state(pool[r][heads], s, f"prefill page {r}")
    # decode oracle on sampled sequences and heads
    hd = head_slice(dec, heads, group)
    res = ogdn.decode(hd["q"][seqs_d], hd["k"][seqs_d], hd["v"][seqs_d], hd["g"][seqs_d],
                      hd["beta"][seqs_d], initial_state=RowView(rows_in_d),
                      initial_state_indices=[dslots["initial_state_indices"][b] for b in seqs_d],
                      output_state_indices=[dslots["output_state_indices"][b] for b in seqs_d])
    check_outputs(o_d[seqs_d][:, heads], res.o, "decode o")
    for r, s in res.final.items():
        check_state(pool[r][heads], s, f"decode page {r}")

"""GPU parity of the page-table conversions (padded block table <-> CSR)
against the oracle, bit-exact: the drill's printed examples, seeded random
tables with garbage in the padding, batches of more than one scan block, bad
rows, an empty batch, and a converted table driving the slot kernels."""

import json
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import csr as ocsr
from oracle import slots as oslots

pytestmark = pytest.mark.gpu
DEV = "cuda"
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def lib():
    import paged_recurrent_state_amd as m
    m.load()
    return m


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def i32(x):
    return torch.tensor(x, dtype=torch.int32, device=DEV)


def to_csr(table, ctx, ps, bad=None):
    indptr, indices, lpl = lib().block_table_to_csr(table, ctx, ps, bad_rows=bad)
    torch.cuda.synchronize()
    ip = indptr.cpu().tolist()
    return ip, indices[:ip[-1]].cpu().tolist(), lpl.cpu().tolist()


def test_drill_three_sequences_both_directions():
    g = golden("csr_three_sequences.json")
    ps = g["page_size"]
    # the padding cells hold garbage on the page: any value must be ignored
    table = [row[:n] + [777] * (3 - n) for row, n in zip(g["block_table"], g["pages_per_seq"])]
    ip, idx, lpl = to_csr(i32(table), i32(g["lengths"]), ps)
    assert (ip, idx, lpl) == (g["indptr"], g["indices"], g["last_page_len"])
    t, ctx = lib().csr_to_block_table(i32(ip), i32(idx), i32(lpl), ps, 3)
    assert t.cpu().tolist() == g["block_table"]
    assert ctx.cpu().tolist() == g["lengths"]


def test_drill_self_test_1():
    g = golden("csr_self_test.json")
    ps = g["page_size"]
    table = i32([[10 * b + j for j in range(4)] for b in range(len(g["lengths"]))])
    ip, _, lpl = to_csr(table, i32(g["lengths"]), ps)
    assert ip == g["indptr"] and lpl == g["last_page_len"]


@pytest.mark.parametrize("B,max_blocks,ps,seed", [(37, 9, 16, 0), (300, 40, 896, 1),
                                                  (2500, 12, 1024, 2), (5, 2048, 64, 3)])
def test_random_tables_match_oracle_and_round_trip(B, max_blocks, ps, seed):
    rng = np.random.default_rng(seed)
    ctx = rng.integers(1, max_blocks * ps + 1, size=B)
    ctx[: min(B, 3)] = [1, ps, max_blocks * ps][: min(B, 3)]  # one token, a full page, a full row
    stride = max_blocks + 5                                  # padded row stride
    full = rng.integers(0, 1 << 20, size=(B, stride)).astype(np.int32)  # garbage everywhere
    table = torch.from_numpy(full).to(DEV)[:, :max_blocks]
    bad = torch.full((1,), -5, dtype=torch.int32, device=DEV)
    ip, idx, lpl = to_csr(table, i32(ctx.tolist()), ps, bad)
    want = ocsr.block_table_to_csr(full[:, :max_blocks].tolist(), ctx.tolist(), ps)
    assert (ip, idx, lpl) == tuple(want)
    assert bad.item() == 0
    t, c = lib().csr_to_block_table(i32(ip), i32(idx), i32(lpl), ps, max_blocks, bad_rows=bad)
    wt, wc = ocsr.csr_to_block_table(ip, idx, lpl, ps, max_blocks)
    assert t.cpu().tolist() == wt and c.cpu().tolist() == wc == ctx.tolist()
    assert bad.item() == 0


def test_bad_rows_are_counted_and_left_empty():
    ps, mb = 16, 3
    ctx = [5, 0, 49, 48, -3, 16]          # 0, 49 (> 3 pages) and -3 cannot be held
    table = i32([[1, 2, 3], [4, 5, 6], [7, 8, 9], [10, 11, 12], [13, 14, 15], [16, 17, 18]])
    bad = torch.zeros(1, dtype=torch.int32, device=DEV)
    ip, idx, lpl = to_csr(table, i32(ctx), ps, bad)
    assert bad.item() == 3
    assert ip == [0, 1, 1, 1, 4, 4, 5] and idx == [1, 10, 11, 12, 16]
    assert lpl == [5, 0, 0, 16, 0, 16]
    # the other direction: no pages, too many pages, last_page_len 0 or > ps
    indptr = i32([0, 1, 1, 5, 6, 7, 8])
    indices = i32([9, 8, 7, 6, 5, 4, 3, 2])
    lplv = i32([3, 4, 4, 0, 17, 16])
    t, c = lib().csr_to_block_table(indptr, indices, lplv, ps, mb, bad_rows=bad)
    assert bad.item() == 4
    assert t.cpu().tolist() == [[9, 0, 0], [0, 0, 0], [0, 0, 0], [0, 0, 0], [0, 0, 0], [2, 0, 0]]
    assert c.cpu().tolist() == [3, 0, 0, 0, 0, 16]


def test_empty_batch():
    bad = torch.full((1,), 9, dtype=torch.int32, device=DEV)
    ip, idx, lpl = to_csr(torch.empty(0, 4, dtype=torch.int32, device=DEV),
                          torch.empty(0, dtype=torch.int32, device=DEV), 16, bad)
    assert (ip, idx, lpl) == ([0], [], []) and bad.item() == 0
    t, c = lib().csr_to_block_table(i32([0]), torch.empty(0, dtype=torch.int32, device=DEV),
                                    torch.empty(0, dtype=torch.int32, device=DEV), 16, 4, bad_rows=bad)
    assert t.shape == (0, 4) and c.shape == (0,) and bad.item() == 0


def test_converted_table_drives_the_slot_kernels():
    """The hybrid-step page tables (prefill and decode) through the block-table
    form and back give the same CSR, and the slot kernels the same rows."""
    m = lib()
    c = workloads.config4(device=DEV, layers=(0,))
    ps = c["page_size"]
    for part in ("prefill", "decode"):
        d = c["layers"][0][part]
        ip, idx, lpl = d["page_indptr"], d["page_indices"], d["last_page_len"]
        n = (ip[1:] - ip[:-1]).max().item()
        table, ctx = m.csr_to_block_table(ip, idx, lpl, ps, n)
        ip2, idx2, lpl2 = m.block_table_to_csr(table, ctx, ps)
        torch.cuda.synchronize()
        assert torch.equal(ip2, ip) and torch.equal(lpl2, lpl)
        assert torch.equal(idx2[: ip[-1].item()], idx)
        if part == "decode":
            s1 = m.decode_slots(idx, ip, lpl)
            s2 = m.decode_slots(idx2, ip2, lpl2)
            want = oslots.decode_slots(idx.cpu().tolist(), ip.cpu().tolist(), lpl.cpu().tolist())
        else:
            cu = d["cu_seqlens"].to(DEV)
            s1 = m.prefill_slots(cu, idx, ip, lpl, ps)
            s2 = m.prefill_slots(cu, idx2, ip2, lpl2, ps)
            want = oslots.prefill_slots(cu.cpu().tolist(), idx.cpu().tolist(), ip.cpu().tolist(),
                                        lpl.cpu().tolist(), ps)
        torch.cuda.synchronize()
        for a, b in zip(s1, s2):
            assert torch.equal(a, b)
        got = [t.cpu().tolist() for t in s2]
        want = [list(w) for w in (want.values() if isinstance(want, dict) else want)]
        assert got == want, part

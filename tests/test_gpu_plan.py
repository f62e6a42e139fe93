"""The sequence-parallel plan the device builds, read back from the workspace.

White-box: the workspace regions are located as the library lays them out
(per-sequence rows, launch order, zero row, chunk table, intra-chunk records,
then the segment records of both passes -- the first pass's offset runs in the
first half of its room, its transition runs at the same places in the second
half -- the scan records, the counts and the segment states, each region
256-byte aligned).  For forced and device-chosen
segment lengths the records must:
  * cover every sequence's new tokens exactly, in order, in both passes;
  * never read a caller row in the first pass (zero or identity starts) and,
    for a sequence cut in two or more segments, never read one in the second
    pass either (segment 0 reads the scan's copy of the initial state), so no
    launch both reads and writes a caller row;
  * write the caller's final row only from the last segment;
  * use workspace state rows inside the room the size query reserved.
"""

import numpy as np
import pytest
import torch

from tests.test_gpu_small import lib, make_case, opts

pytestmark = pytest.mark.gpu

REC_BYTES = 10240 + 1024  # intra-chunk record per (chunk slot, v-head)


def al(x):
    return (x + 255) // 256 * 256


def plan_regions(T, B, H, split, m_forced=0):
    """Byte offsets of the segment regions (mirrors the workspace layout)."""
    nc = T // 64 + 2 * B + 1
    if m_forced > 0:
        segs = nc // m_forced + B
    else:
        segs = min(nc // 4 + B, 512 // H + B)
    off = al(5 * B * 4) + al(B * 4) + 256 + al(nc * 16) + al(nc * H * 10240) + al(nc * H * 1024)
    seg1 = off
    off += al(2 * segs * 32)
    seg2 = off
    off += al(segs * 32)
    scan = off
    off += al(B * 16)
    counts = off
    return dict(seg1=seg1, seg2=seg2, scan=scan, counts=counts, cap=segs)


def read_i32(ws, off, n):
    return ws[off:off + 4 * n].view(torch.int32).cpu().numpy()


@pytest.mark.parametrize("split", [2, 0])
def test_plan_records(split):
    m = lib()
    # ragged lengths with long sequences, 2 heads: the device plan splits
    prefix = [37, 0, 256, 1000, 5]
    new = [3000, 2500, 60, 4100, 0]
    H = 2
    pre, pool = make_case(prefix, new, ps=128, H=H, Hqk=1, seed=81, g_scale=0.1)
    T, B = sum(new), len(new)
    o = opts(prefill_split_chunks=split)
    ws = torch.zeros(m.prefill_workspace_size(T, B, H, 1, options=o), dtype=torch.uint8,
                     device="cuda")
    sl = m.prefill_slots(pre["cu_seqlens"], pre["page_indices"], pre["page_indptr"],
                         pre["last_page_len"], pre["page_size"])
    m.prefill_paged(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], pre["cu_seqlens"], pool,
                    pre["page_indices"], pre["page_indptr"], pre["page_size"],
                    pre["last_page_len"], slots=sl, workspace=ws, options=o)
    torch.cuda.synchronize()
    reg = plan_regions(T, B, H, split, m_forced=split)
    n1, n2 = read_i32(ws, reg["counts"], 2)  # offset runs (as many transition runs), runs
    cap1 = 2 * reg["cap"]
    rec1_all = read_i32(ws, reg["seg1"], 8 * cap1).reshape(-1, 8)
    off1, map1 = rec1_all[:n1], rec1_all[cap1 // 2:cap1 // 2 + n1]
    rec2 = read_i32(ws, reg["seg2"], 8 * n2).reshape(-1, 8)
    scan = read_i32(ws, reg["scan"], 4 * B).reshape(-1, 4)
    cu = pre["cu_seqlens"].tolist()
    rd = sl.state_indices.tolist()
    wr = sl.output_state_indices.tolist()
    assert n2 <= reg["cap"] and n1 <= reg["cap"]
    assert (off1[:, 7] == 1).all() and (map1[:, 7] == 2).all()  # offset, transition
    assert (off1[:, :4] == map1[:, :4]).all()  # the same segments
    rows = 0
    i1 = i2 = 0
    split_any = False
    for b in range(B):
        G, row0 = int(scan[b][0]), int(scan[b][1])
        L = cu[b + 1] - cu[b]
        if L == 0:
            assert G == 0
            continue
        assert G >= 1
        mine2 = rec2[i2:i2 + G]
        i2 += G
        # second pass covers the tokens in order
        assert mine2[0][0] == cu[b] and sum(int(r[1]) for r in mine2) == L
        for x, y in zip(mine2, mine2[1:]):
            assert y[0] == x[0] + x[1]
        assert [int(r[5]) for r in mine2] == [-1] * (G - 1) + [wr[b]]
        if split == 0 and G > 1:  # balanced: interior segments share one length
            lens = [int(r[1]) for r in mine2[1:-1]]
            assert len(set(lens)) <= 1
        if G == 1:
            assert mine2[0][4] == rd[b]  # a whole sequence reads its own row
            continue
        split_any = True
        assert row0 == rows
        rows += 3 * G - 2
        # every second-pass start is a workspace state: start_g at row0 + g
        assert [int(r[4]) for r in mine2] == [-2 - (row0 + g) for g in range(G)]
        mine1 = np.concatenate([off1[i1:i1 + G - 1], map1[i1:i1 + G - 1]])
        i1 += G - 1
        assert (mine1[:, 4] == -1).all()          # zero / identity starts
        assert (mine1[:, 5] <= -2).all()          # workspace results only
        assert sorted(-2 - mine1[:, 5].astype(int)) == list(range(row0 + G, row0 + 3 * G - 2))
    assert i1 == n1 and i2 == n2
    assert rows <= 3 * reg["cap"]
    assert split_any, "the plan cut no sequence"
    print(f"split {split}: {n1} offset and {n1} transition runs, {n2} second-pass runs; segments per "
          f"sequence {[int(x[0]) for x in scan]}")


@pytest.mark.parametrize("g_scale", [1.0, 0.1])
def test_auto_plan_one_long_head(g_scale):
    """One sequence on one head, 40,000 new tokens after a prefix that ends
    inside a page: the device plan may cut it into hundreds of segments (its
    room is min(chunks / 4 + B, 512 / H + B)); outputs, every page-boundary
    state and the final state against the oracle."""
    from tests.test_gpu_small import check_paged_prefill
    pre, pool = make_case([100], [40000], ps=1024, H=1, Hqk=1, seed=91, g_scale=g_scale)
    _, writes, err = check_paged_prefill(pre, pool, options=opts(prefill_split_chunks=0))
    assert len(writes) == 40
    print(f"g x {g_scale}: {len(writes)} rows written, worst state rel {err:.2e}")


def test_auto_plan_at_the_pair_limit():
    """128 sequences on 2 heads (B * H = 256, the most the device plan takes),
    ragged lengths with a few long ones."""
    from tests.test_gpu_small import check_paged_prefill
    rng = np.random.default_rng(17)
    new = [int(x) for x in rng.integers(1, 200, 128)]
    new[3], new[70], new[101] = 3000, 2200, 1500
    prefix = [int(x) for x in rng.integers(0, 300, 128)]
    pre, pool = make_case(prefix, new, ps=128, H=2, Hqk=1, seed=92, g_scale=0.3)
    _, writes, err = check_paged_prefill(pre, pool, options=opts(prefill_split_chunks=0))
    print(f"{len(writes)} rows written, worst state rel {err:.2e}")


def run_split(m, pre, pool, H, split):
    """A paged prefill with forced segments, its workspace kept for reading."""
    T, B = int(pre["q"].shape[0]), int(pre["last_page_len"].shape[0])
    o = opts(prefill_split_chunks=split)
    ws = torch.zeros(m.prefill_workspace_size(T, B, H, H, options=o), dtype=torch.uint8,
                     device="cuda")
    out = m.prefill_paged(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], pre["cu_seqlens"],
                          pool, pre["page_indices"], pre["page_indptr"], pre["page_size"],
                          pre["last_page_len"], workspace=ws, options=o)
    torch.cuda.synchronize()
    return out, ws


def map_rows(ws, T, B, H, split):
    """The first pass's transition states M_g of sequence 0, as [G - 1, H, V, K]."""
    reg = plan_regions(T, B, H, split, m_forced=split)
    G, row0 = (int(x) for x in read_i32(ws, reg["scan"], 2))
    nc = T // 64 + 2 * B + 1
    # the segment states follow the counts (256 bytes), rows of H * 128 * 128 floats
    states = reg["counts"] + 256
    row = H * 128 * 128 * 4
    first = states + (row0 + 2 * G - 1) * row
    return ws[first:first + (G - 1) * row].view(torch.float32).view(G - 1, H, 128, 128), nc


@pytest.mark.parametrize("g_scale,skipped", [(1.0, True), (0.02, False)])
def test_negligible_transitions(g_scale, skipped):
    """Segments of 8 chunks: with the configs' decay (about 2^-75 a chunk) a
    segment's transition bound is far below 2^-300, so the first pass stores
    zeros for M_g and starts its offset runs late; with decay / 50 it computes
    them.  Either way the outputs and states match the oracle."""
    from tests.test_gpu_small import check_paged_prefill
    m = lib()
    pre, pool = make_case([0], [6000], ps=512, H=2, Hqk=2, seed=93, g_scale=g_scale)
    pool2 = pool.clone()
    check_paged_prefill(pre, pool, options=opts(prefill_split_chunks=8))
    _, ws = run_split(m, pre, pool2, 2, 8)
    M, _ = map_rows(ws, 6000, 1, 2, 8)
    zero = [bool((M[g] == 0).all()) for g in range(M.shape[0])]
    print(f"g x {g_scale}: transitions stored as zeros {zero}")
    assert all(zero) if skipped else not any(zero)


def test_transition_bound_counts_key_norms():
    """Keys with k.k = 2.5 and beta = 1: each token's I - beta k k^T has an
    eigenvalue of -1.5, so the bound adds log2 1.5 a token and the decay alone
    no longer decides; parity against the oracle with forced and planned
    segments."""
    from tests.test_gpu_small import check_paged_prefill
    for split in (8, 0):
        pre, pool = make_case([0, 100], [5000, 3000], ps=512, H=2, Hqk=2, seed=94, g_scale=1.0)
        k = pre["k"].float()
        pre["k"] = (k * (2.5 ** 0.5) / k.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
        pre["beta"] = torch.ones_like(pre["beta"])
        _, writes, err = check_paged_prefill(pre, pool, options=opts(prefill_split_chunks=split))
        print(f"split {split}: {len(writes)} rows written, worst state rel {err:.2e}")

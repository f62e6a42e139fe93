"""Pins for the oracle's page-table and slot logic (CPU only).

Each test checks the oracle against something other than itself: values the
pages print (tests/golden/*.json, each citing its source), brute-force token
walks, or counting identities.
"""

import json
import os
import random

import numpy as np
import pytest

from oracle import csr, gdn, slots

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_csr_self_test_1():
    g = golden("csr_self_test.json")
    indptr, _, lpl = csr.csr_from_lengths(g["lengths"], g["page_size"])
    assert indptr == g["indptr"]
    assert lpl == g["last_page_len"]
    assert [csr.pages_for(n, g["page_size"]) for n in g["lengths"]] == g["pages_per_seq"]


def test_csr_three_sequences_both_directions():
    g = golden("csr_three_sequences.json")
    indptr, indices, lpl = csr.block_table_to_csr(g["block_table"], g["lengths"], g["page_size"])
    assert indptr == g["indptr"] and indices == g["indices"] and lpl == g["last_page_len"]
    table, ctx = csr.csr_to_block_table(indptr, indices, lpl, g["page_size"], 3)
    assert table == g["block_table"]
    assert ctx == g["lengths"]


def test_last_page_len_is_not_ctx_mod_page_size():
    # A full last page has last_page_len == page_size, never 0.
    for ps in (4, 16, 64):
        for ctx in range(1, 5 * ps):
            lpl = csr.last_page_len_for(ctx, ps)
            assert 1 <= lpl <= ps
            assert (csr.pages_for(ctx, ps) - 1) * ps + lpl == ctx


def test_zero_page_sequence_rejected_by_decode():
    g = golden("csr_zero_page_sequence.json")
    indptr = g["indptr"]
    indices = list(range(indptr[-1]))
    with pytest.raises(ValueError):
        slots.decode_slots(indices, indptr, [1, 1, 1])


def test_prefill_2500_token_example():
    g = golden("prefill_2500_tokens.json")
    sl = slots.prefill_slots(g["cu_seqlens"], g["page_indices"], g["page_indptr"],
                             g["last_page_len"], g["page_size"])
    assert sl["prefix_lens"] == [g["prefix"]]
    assert sl["state_indices"] == [g["reads_page"]]
    assert sl["output_state_indices"] == g["writes_pages"]
    assert (g["page_indptr"][1] - 1) * g["page_size"] + g["last_page_len"][0] == \
        g["total_tokens_after_call"]

    # Run the oracle on it (tiny head dims keep it quick): only page 12 is
    # written and pages 7 and 3 keep every bit.
    rng = np.random.default_rng(0)
    H, K, V = 1, 8, 8
    T = 452
    pool = np.full((16, H, V, K), np.nan, dtype=np.float32)
    pool[3] = rng.standard_normal((H, V, K)).astype(np.float32)
    before = pool.copy()
    q = rng.standard_normal((T, H, K))
    k = rng.standard_normal((T, H, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, V))
    gg = -np.log1p(np.exp(rng.standard_normal((T, H))))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, H))))
    o, writes, _ = gdn.prefill_paged(q, k, v, gg, beta, g["cu_seqlens"], pool,
                                     g["page_indices"], g["page_indptr"],
                                     g["last_page_len"], g["page_size"])
    assert sorted(writes) == g["writes_pages"]
    for r in g["unchanged_pages"]:
        assert pool[r].tobytes() == before[r].tobytes()
    assert np.isfinite(o).all()


def _token_walk(pages, p, L, ps):
    """Brute force: walk the new tokens one by one and record which page ends
    at each boundary crossed, then the last page."""
    written = []
    for n in range(1, L + 1):
        pos = p + n
        if pos % ps == 0:
            written.append(pages[pos // ps - 1])
    if L > 0:
        written.append(pages[-1])
    read = -1
    if p > 0:
        # the page whose token range holds token p - 1 (0-based)
        for j, pg in enumerate(pages):
            if j * ps <= p - 1 < (j + 1) * ps:
                read = pg
    return read, written


@pytest.mark.parametrize("ps", [64, 128])
def test_rows_match_token_walk(ps):
    rnd = random.Random(ps)
    for p in range(0, 301):
        for L in range(0, 301, 7 if p % 5 else 1):
            total = p + L
            if total == 0:
                continue
            n = (total + ps - 1) // ps
            pages = rnd.sample(range(1000), n)
            indptr = [0, n]
            lpl = [total - (n - 1) * ps]
            sl = slots.prefill_slots([0, L], pages, indptr, lpl, ps)
            read, written = _token_walk(pages, p, L, ps)
            assert sl["prefix_lens"] == [p]
            assert sl["state_indices"] == [read]
            assert sl["output_state_indices"] == [written[-1] if L else -1]
            # the checkpoint rows the slot arguments select are exactly the
            # boundary pages of the walk
            cnt = (p + L) // ps - p // ps
            ck = [pages[sl["checkpoint_cu_starts"][0] + j] for j in range(cnt)]
            assert ck + ([written[-1]] if L else []) == written
            # never a page that ends at or before the prefix
            for r in written:
                j = pages.index(r)
                assert (j + 1) * ps > p


def test_checkpoint_count_identity():
    for N in (1, 3, 64, 100, 896):
        for p in range(0, 2 * N + 5):
            for L in range(0, 3 * N + 5, max(1, N // 7)):
                assert slots.checkpoint_count(p, L, N) == (p + L) // N - p // N


def test_long_prompt_checkpoint_total():
    # 32768 tokens in calls split at 7001/14500/20000/27777, every 896 tokens:
    # 7 + 9 + 6 + 9 + 5 = 36 = 32768 // 896.
    bounds = [0, 7001, 14500, 20000, 27777, 32768]
    counts = [slots.checkpoint_count(a, b - a, 896) for a, b in zip(bounds, bounds[1:])]
    assert counts == [7, 9, 6, 9, 5]
    assert sum(counts) == 32768 // 896


def test_oracle_checkpoint_writes_sampled():
    """The recurrence oracle stores exactly the walk's pages (tiny heads)."""
    rnd = random.Random(7)
    rng = np.random.default_rng(7)
    for _ in range(60):
        ps = rnd.choice([64, 128])
        p = rnd.randrange(0, 400)
        L = rnd.randrange(0, 400)
        if p + L == 0:
            continue
        n = (p + L + ps - 1) // ps
        pages = rnd.sample(range(64), n)
        pool = np.full((64, 1, 2, 2), np.nan)
        read, written = _token_walk(pages, p, L, ps)
        if read >= 0:
            pool[read] = rng.standard_normal((1, 2, 2))
        q = rng.standard_normal((L, 1, 2))
        k = rng.standard_normal((L, 1, 2))
        v = rng.standard_normal((L, 1, 2))
        g = -rng.random((L, 1))
        beta = rng.random((L, 1))
        o, writes, sl = gdn.prefill_paged(q, k, v, g, beta, [0, L], pool, pages, [0, n],
                                          [p + L - (n - 1) * ps], ps)
        assert sorted(writes) == sorted(set(written))
        assert np.isfinite(o).all()
        for r, s in writes.items():
            assert np.isfinite(s).all()


def test_config0_rows():
    """Rows of the tiny two-sequence case (page table fixed by the workload)."""
    import workloads
    c = workloads.config0()
    pre = c["prefill"]
    sl = slots.prefill_slots(pre["cu_seqlens"].tolist(), pre["page_indices"].tolist(),
                             pre["page_indptr"].tolist(), pre["last_page_len"].tolist(), 128)
    assert pre["page_indptr"].tolist() == [0, 3, 5]
    assert sl["state_indices"] == [-1, 5]
    assert sl["output_state_indices"] == [14, 9]
    assert sl["checkpoint_cu_starts"] == [0, 3]
    assert sl["prefix_lens"] == [0, 64]
    # seq0: 300 tokens from 0 -> 5 chunks; seq1: 130 tokens from 64 -> 3 chunks
    assert sl["chunk_starts"] == [0, 5]
    dec = c["decode"]
    ds = slots.decode_slots(dec["page_indices"].tolist(), dec["page_indptr"].tolist(),
                            dec["last_page_len"].tolist())
    assert dec["last_page_len"].tolist() == [45, 67]
    assert ds["initial_state_indices"] == [14, 9] == ds["output_state_indices"]


def test_decode_rows_new_page():
    # last_page_len == 1: read the previous page, write the new one.
    ds = slots.decode_slots([4, 8, 2, 6, 1], [0, 3, 5], [1, 7])
    assert ds["initial_state_indices"] == [8, 1]
    assert ds["output_state_indices"] == [2, 1]
    with pytest.raises(ValueError):
        slots.decode_slots([4], [0, 1], [1])


def test_chunk_count_left_pad():
    # A prefix that is not a multiple of 64 costs at most one extra chunk.
    for p in range(0, 200):
        for L in range(1, 200):
            c = slots.chunk_count(p, L)
            aligned = (L + 63) // 64
            assert c in (aligned, aligned + 1)
            assert 64 * c >= (p % 64) + L > 64 * (c - 1)

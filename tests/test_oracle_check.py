"""Pins of the batch-validity reference (oracle/slots.check_paged): the
page's examples are valid, each rule broken on its own is caught, and the
touched rows agree with the slot rows and with a token walk."""

import random

from oracle import slots as oslots


def test_page_examples_are_valid():
    # 2500 tokens on pages [7, 3, 12] (page 1024), 452 new: reads 3, writes 12
    assert oslots.check_paged([7, 3, 12], [0, 3], [452], 1024, 16, cu_seqlens=[0, 452]) == 0
    assert oslots.touched_rows([7, 3, 12], 452, 1024, 452) == ({3}, {12})
    # CSR self-test table (page 16, lengths 16, 17, 1, 40) as a decode batch
    assert oslots.check_paged([0, 1, 2, 3, 4, 5, 6], [0, 1, 3, 4, 7], [16, 1, 1, 8], 16, 7) == \
        oslots.CHECK_TOKENS  # the 1-token sequence holds nothing before its decoded token


def test_each_rule():
    ok = dict(page_indices=[4, 1, 6, 2], page_indptr=[0, 2, 4], last_page_len=[10, 64],
              page_size=64, num_pages=8, cu_seqlens=[0, 20, 30])
    assert oslots.check_paged(**ok) == 0
    assert oslots.check_paged(**{**ok, "page_indptr": [1, 2, 4]}) & oslots.CHECK_INDPTR
    assert oslots.check_paged(**{**ok, "page_indptr": [0, 3, 2]}) == oslots.CHECK_INDPTR
    assert oslots.check_paged(**{**ok, "page_indptr": [0, 0, 4]}) == oslots.CHECK_INDPTR
    assert oslots.check_paged(**{**ok, "last_page_len": [0, 64]}) == oslots.CHECK_LAST_PAGE_LEN
    assert oslots.check_paged(**{**ok, "last_page_len": [65, 64]}) == oslots.CHECK_LAST_PAGE_LEN
    assert oslots.check_paged(**{**ok, "cu_seqlens": [0, 75, 80]}) == oslots.CHECK_TOKENS
    assert oslots.check_paged(**{**ok, "cu_seqlens": [1, 20, 30]}) == oslots.CHECK_TOKENS
    assert oslots.check_paged(**{**ok, "num_pages": 6}) == oslots.CHECK_PAGE_ID
    assert oslots.check_paged(**{**ok, "page_indices": [4, 1, 6, -1]}) == oslots.CHECK_PAGE_ID
    # both sequences write their last page: make it one page
    assert oslots.check_paged(**{**ok, "page_indices": [4, 2, 6, 2]}) == oslots.CHECK_SHARED_ROW
    # sequence 1 only reads page 6 (its prefix of 64 ends there); sequence 0,
    # whose prefix of 54 ends inside its first page, writes pages 5 and 6
    shared = dict(page_indices=[5, 6, 6, 2], page_indptr=[0, 2, 4], last_page_len=[10, 10],
                  page_size=64, num_pages=8, cu_seqlens=[0, 20, 30])
    assert oslots.touched_rows([6, 2], 10, 64, 10) == ({6}, {2})
    assert oslots.check_paged(**shared) == oslots.CHECK_SHARED_ROW
    # a shared prefix page that nobody writes is fine
    cold = dict(page_indices=[3, 5, 3, 6], page_indptr=[0, 2, 4], last_page_len=[10, 10],
                page_size=64, num_pages=8, cu_seqlens=[0, 5, 10])
    assert oslots.check_paged(**cold) == 0


def test_touched_rows_against_slots_and_a_token_walk():
    rng = random.Random(3)
    for _ in range(300):
        ps = rng.choice([64, 128])
        p = rng.randint(0, 400)
        L = rng.randint(0, 300)
        total = p + L
        if total == 0:
            continue
        n = (total + ps - 1) // ps
        pages = rng.sample(range(1000), n)
        lpl = total - (n - 1) * ps
        reads, writes = oslots.touched_rows(pages, lpl, ps, L)
        sl = oslots.prefill_slots([0, L], pages, [0, n], [lpl], ps)
        assert reads == ({sl["state_indices"][0]} - {-1})
        # token walk: a page is written when the walk stores a boundary or the end in it
        walk = set()
        for t in range(p + 1, total + 1):
            if t % ps == 0 or t == total:
                walk.add(pages[(t - 1) // ps])
        assert writes == walk

"""Debug validation of paged batches (gdn_check_paged and the paged calls'
check option) against the oracle's validity rules, bit for bit.

Corrupted batches stay memory-safe even where the rules fail: page ids out
of range are still rows of the (larger) pool the test allocates, and only
the standalone check ever sees broken page_indptr, last_page_len or token
counts.  A checked call on a batch with an error must leave the pool and the
output buffer untouched."""

import random

import pytest
import torch

import workloads
from oracle import slots as oslots
from tests.gpu_util import changed_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def lib():
    import paged_recurrent_state_amd as m
    m.load()
    return m


def random_batch(rng, prefill, num_pages):
    B = rng.randint(1, 40)
    ps = rng.choice([64, 128])
    ctx, new = [], []
    for _ in range(B):
        c = rng.randint(2, 600)
        ctx.append(c)
        new.append(rng.randint(0, c) if prefill else 1)
    counts = [(c + ps - 1) // ps for c in ctx]
    ids = rng.sample(range(num_pages), sum(counts))
    ptr = [0]
    for n in counts:
        ptr.append(ptr[-1] + n)
    lpl = [c - (n - 1) * ps for c, n in zip(ctx, counts)]
    cu = [0]
    for L in new:
        cu.append(cu[-1] + L)
    return dict(idx=ids, ptr=ptr, lpl=lpl, cu=cu if prefill else None, ps=ps)


def corrupt(rng, d, kind, num_pages, prefill):
    d = {k: (list(v) if isinstance(v, list) else v) for k, v in d.items()}
    B = len(d["lpl"])
    if kind == "indptr" and B >= 2:
        b = rng.randint(1, B - 1)
        d["ptr"][b] = d["ptr"][b + 1] + 1 if d["ptr"][b + 1] + 1 <= d["ptr"][-1] else d["ptr"][b - 1]
    elif kind == "last_page_len":
        d["lpl"][rng.randrange(B)] = rng.choice([0, d["ps"] + 1])
    elif kind == "tokens":
        if prefill:
            b = rng.randrange(B)
            total = (d["ptr"][b + 1] - d["ptr"][b] - 1) * d["ps"] + d["lpl"][b]
            extra = total + 1 - (d["cu"][b + 1] - d["cu"][b])
            d["cu"] = d["cu"][:b + 1] + [x + extra for x in d["cu"][b + 1:]]
        else:
            b = rng.randrange(B)
            # one page holding a single token: nothing before the decoded one
            n = d["ptr"][b + 1] - d["ptr"][b]
            d["idx"] = d["idx"][:d["ptr"][b]] + d["idx"][d["ptr"][b] + n - 1:]
            d["ptr"] = d["ptr"][:b + 1] + [x - (n - 1) for x in d["ptr"][b + 1:]]
            d["lpl"][b] = 1
    elif kind == "page_id":
        d["idx"][rng.randrange(len(d["idx"]))] = rng.choice([-1, num_pages, num_pages + 5])
    elif kind == "shared" and B >= 2:
        a, b = rng.sample(range(B), 2)
        # a row sequence a writes reappears among the rows sequence b touches
        last_a = d["idx"][d["ptr"][a + 1] - 1]
        d["idx"][d["ptr"][b + 1] - 1] = last_a
    return d


def as_dev(d):
    t = lambda x: torch.tensor(x, dtype=torch.int32, device=DEV)  # noqa: E731
    return t(d["idx"] or [0]), t(d["ptr"]), t(d["lpl"]), (t(d["cu"]) if d["cu"] else None)


@pytest.mark.parametrize("prefill", [True, False])
def test_check_matches_oracle(prefill):
    m = lib()
    rng = random.Random(11 + prefill)
    num_pages = 4000
    kinds = [None, "indptr", "last_page_len", "tokens", "page_id", "shared"]
    seen = set()
    for i in range(120):
        d = random_batch(rng, prefill, num_pages)
        kind = kinds[i % len(kinds)]
        if kind:
            d = corrupt(rng, d, kind, num_pages, prefill)
        idx, ptr, lpl, cu = as_dev(d)
        word = m.check_paged(idx, ptr, lpl, d["ps"], num_pages, cu_seqlens=cu)
        ref = oslots.check_paged(d["idx"], d["ptr"], d["lpl"], d["ps"], num_pages,
                                 cu_seqlens=d["cu"])
        assert int(word.item()) == ref, (i, kind, int(word.item()), ref)
        seen.add(ref)
    assert {0, oslots.CHECK_PAGE_ID, oslots.CHECK_SHARED_ROW, oslots.CHECK_LAST_PAGE_LEN} <= seen


def test_check_skips_the_row_test_beyond_its_size():
    m = lib()
    B, ps = 2100, 64
    ptr = torch.arange(0, 2 * B + 1, 2, dtype=torch.int32, device=DEV)
    idx = torch.arange(2 * B, dtype=torch.int32, device=DEV)
    lpl = torch.full((B,), 5, dtype=torch.int32, device=DEV)
    assert int(m.check_paged(idx, ptr, lpl, ps, 2 * B).item()) == 32  # GDN_CHECK_NOT_CHECKED
    assert int(m.check_paged(idx, ptr, lpl, ps, 2 * B - 1).item()) == oslots.CHECK_PAGE_ID


def paged_prefill_case(seed, shared=False):
    """Four sequences on pages 30.. of a 64-row pool; with `shared`, sequences
    0 and 2 end on one page (both would write it)."""
    gen = workloads.generator(seed)
    prefix, new, ps = [37, 0, 128, 5], [200, 90, 150, 60], 64
    pages, nxt = [], 30
    for p, n in zip(prefix, new):
        cnt = (p + n + ps - 1) // ps
        pages.append(list(range(nxt, nxt + cnt)))
        nxt += cnt
    if shared:
        pages[2][-1] = pages[0][-1]
    pre = workloads._prefill_batch(prefix, new, pages, ps, 2, 2, 128, 128, gen, "cpu", 0.5)
    pool = workloads.nan_pool(64, 2, 128, 128)
    workloads.fill_rows(pool, [r for r in pre["read_rows"] if r >= 0], gen, 0.09)
    pre = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in pre.items()}
    return pre, pool.to(DEV)


def run_prefill(m, pre, pool, options=None, o=None):
    return m.prefill_paged(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], pre["cu_seqlens"],
                           pool, pre["page_indices"], pre["page_indptr"], pre["page_size"],
                           pre["last_page_len"], options=options, out=o)


@pytest.mark.parametrize("split", [0, 2])
def test_checked_prefill(split):
    """A valid batch: word 0, results bit-identical to the unchecked call.  A
    batch whose two sequences write one row, or whose page ids exceed the
    stated pool size: the word says so and neither the pool nor o changes."""
    m = lib()
    word = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    pre, pool = paged_prefill_case(5)
    pool2 = pool.clone()
    o1 = run_prefill(m, pre, pool, options=m.Options(prefill_split_chunks=split))
    o2 = run_prefill(m, pre, pool2, options=m.checked(word, 64, prefill_split_chunks=split))
    torch.cuda.synchronize()
    assert int(word.item()) == 0
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert changed_rows(pool, pool2) == []
    for shared, num_pages, bit in ((True, 64, oslots.CHECK_SHARED_ROW),
                                   (False, 20, oslots.CHECK_PAGE_ID)):
        pre, pool = paged_prefill_case(6, shared=shared)
        before = pool.clone()
        o = torch.full((pre["q"].shape[0], 2, 128), 3.0, dtype=torch.bfloat16, device=DEV)
        run_prefill(m, pre, pool, options=m.checked(word, num_pages, prefill_split_chunks=split),
                    o=o)
        torch.cuda.synchronize()
        assert int(word.item()) == bit
        assert changed_rows(before, pool) == []
        assert bool((o == 3.0).all())


def test_checked_decode():
    m = lib()
    word = torch.zeros(1, dtype=torch.int32, device=DEV)
    c = workloads.config2(device=DEV, num_seqs=24, qk_heads=2, v_heads=4, num_pages=24 * 32,
                          new_page_seqs=6)
    d, pool = c["decode"], c["pool"]
    n_pages = int(pool.shape[0])
    pool2 = pool.clone()
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"])
    o1 = m.decode_paged(*args, pool, d["page_indices"], d["page_indptr"], 1024, d["last_page_len"])
    o2 = m.decode_paged(*args, pool2, d["page_indices"], d["page_indptr"], 1024,
                        d["last_page_len"], options=m.checked(word, n_pages))
    torch.cuda.synchronize()
    assert int(word.item()) == 0
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert changed_rows(pool, pool2) == []
    # two sequences on one last page
    idx = d["page_indices"].clone()
    ptr = d["page_indptr"].tolist()
    idx[ptr[3] - 1] = idx[ptr[8] - 1]
    before = pool.clone()
    o = torch.full_like(o1, 3.0)
    m.decode_paged(*args, pool, idx, d["page_indptr"], 1024, d["last_page_len"], out=o,
                   options=m.checked(word, n_pages, decode_stream_per_cu=6))
    torch.cuda.synchronize()
    assert int(word.item()) == oslots.CHECK_SHARED_ROW
    assert changed_rows(before, pool) == []
    assert bool((o == 3.0).all())

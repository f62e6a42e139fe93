"""gdn_prefill_paged_noalloc (the paged prefill on the library's fixed
per-device scratch) against gdn_prefill_paged with a caller workspace, through
the C ABI: two calls in a row on the same pools, the second smaller, outputs
and every pool row bit for bit; the first also against the oracle."""

import numpy as np
import pytest
import torch

import workloads
from oracle import gdn as ogdn
from tests.gpu_util import RowView, changed_rows, check_outputs, check_state, pool_rows_cpu

pytestmark = pytest.mark.gpu


def lib():
    import paged_recurrent_state_amd as m
    m.load()
    return m


def batch(prefix, new, pages, ps, H, Hqk, seed):
    gen = workloads.generator(seed)
    pre = workloads._prefill_batch(prefix, new, pages, ps, Hqk, H, 128, 128, gen, "cpu", 0.3)
    return {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in pre.items()}


def test_noalloc_matches_workspace_call():
    m = lib()
    ps, H, Hqk = 128, 4, 2
    num_pages = 64
    gen = workloads.generator(90)
    pool = workloads.nan_pool(num_pages, H, 128, 128)
    perm = torch.randperm(num_pages, generator=gen).tolist()
    # call 1: three sequences, 2400 new tokens (the device may plan segments)
    prefix1, new1 = [37, 0, 300], [1500, 600, 300]
    pages1, nxt = [], 0
    for p, n in zip(prefix1, new1):
        cnt = (p + n + ps - 1) // ps
        pages1.append([perm[i] for i in range(nxt, nxt + cnt)])
        nxt += cnt
    pre1 = batch(prefix1, new1, pages1, ps, H, Hqk, 91)
    workloads.fill_rows(pool, [r for r in pre1["read_rows"] if r >= 0], gen, 1 / np.sqrt(128))
    pool_a = pool.to("cuda")
    pool_b = pool_a.clone()
    rows_in = pool_rows_cpu(pool_a, pre1["read_rows"])
    before = pool_a.clone()

    def both(pre):
        args = (pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], pre["cu_seqlens"])
        tab = (pre["page_indices"], pre["page_indptr"], ps, pre["last_page_len"])
        oa = m.prefill_paged(*args, pool_a, *tab)
        ob = m.prefill_paged_noalloc(*args, pool_b, *tab)
        torch.cuda.synchronize()
        return oa, ob

    oa, ob = both(pre1)
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))
    assert changed_rows(pool_a, pool_b) == []
    o_ref, writes, _ = ogdn.prefill_paged(pre1["q"].cpu(), pre1["k"].cpu(), pre1["v"].cpu(),
                                          pre1["g"].cpu(), pre1["beta"].cpu(),
                                          pre1["cu_seqlens"].cpu(), RowView(rows_in),
                                          pre1["page_indices"].cpu(), pre1["page_indptr"].cpu(),
                                          pre1["last_page_len"].cpu(), ps)
    check_outputs(ob, o_ref)
    assert changed_rows(before, pool_b) == sorted(writes)
    for r, s in writes.items():
        check_state(pool_b[r], s, f"row {r}")
    # call 2, smaller: the two sequences continue from call 1's final pages
    prefix2 = [prefix1[0] + new1[0], prefix1[1] + new1[1]]
    new2 = [90, 200]
    pages2 = []
    for b in range(2):
        cnt = (prefix2[b] + new2[b] + ps - 1) // ps
        extra = cnt - len(pages1[b])
        pages2.append(pages1[b] + [perm[i] for i in range(nxt, nxt + extra)])
        nxt += extra
    pre2 = batch(prefix2, new2, pages2, ps, H, Hqk, 92)
    oa, ob = both(pre2)
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))
    assert changed_rows(pool_a, pool_b) == []


def test_noalloc_rejects_calls_beyond_the_scratch():
    """A call whose workspace would not fit fails before any launch."""
    import ctypes as C
    m = lib()
    d = m._lib.Dims(32, 32, 128, 128, 0.0, 0, None)
    fake = C.c_void_p(0x1000)  # never dereferenced: the size check fails first
    rc = m._lib.load().gdn_prefill_paged_noalloc(C.byref(d), fake, fake, fake, None, None, fake,
                                                 1, 10_000_000, fake, 32 * 128 * 128, fake, fake,
                                                 fake, 128, None, fake, None)
    assert rc == -4
    assert b"fixed scratch" in m._lib.load().gdn_last_error()

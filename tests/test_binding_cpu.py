"""The Python binding on the CPU: every entry point refuses host tensors with a
clear error before it reaches the library (the library has no CPU path, and
the binding has no fallback)."""

import pytest
import torch

import paged_recurrent_state_amd as gdn
import workloads


@pytest.fixture(scope="module")
def case():
    c = workloads.config0()
    return c, c["prefill"], c["decode"]


def calls(c, pre, dec):
    ps = pre["page_size"]
    i32 = torch.int32
    yield "prefill_slots", lambda: gdn.prefill_slots(pre["cu_seqlens"], pre["page_indices"],
                                                     pre["page_indptr"], pre["last_page_len"], ps)
    yield "decode_slots", lambda: gdn.decode_slots(dec["page_indices"], dec["page_indptr"],
                                                   dec["last_page_len"])
    yield "prefill_paged", lambda: gdn.prefill_paged(
        pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], pre["cu_seqlens"], c["pool"],
        pre["page_indices"], pre["page_indptr"], ps, pre["last_page_len"])
    yield "prefill_paged_noalloc", lambda: gdn.prefill_paged_noalloc(
        pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], pre["cu_seqlens"], c["pool"],
        pre["page_indices"], pre["page_indptr"], ps, pre["last_page_len"])
    yield "decode_paged", lambda: gdn.decode_paged(
        dec["q"], dec["k"], dec["v"], dec["g"], dec["beta"], c["pool"], dec["page_indices"],
        dec["page_indptr"], ps, dec["last_page_len"])
    yield "prefill", lambda: gdn.prefill(
        pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], pre["cu_seqlens"],
        initial_state=c["pool"], state_indices=torch.zeros(2, dtype=i32),
        output_state=c["pool"], output_state_indices=torch.ones(2, dtype=i32),
        output_final_state=True)
    yield "decode", lambda: gdn.decode(
        dec["q"], dec["k"], dec["v"], dec["g"], dec["beta"], initial_state=c["pool"],
        initial_state_indices=torch.zeros(2, dtype=i32), output_state=c["pool"],
        output_state_indices=torch.ones(2, dtype=i32))
    yield "check_paged", lambda: gdn.check_paged(pre["page_indices"], pre["page_indptr"],
                                                 pre["last_page_len"], ps, c["pool"].shape[0],
                                                 cu_seqlens=pre["cu_seqlens"])
    yield "block_table_to_csr", lambda: gdn.block_table_to_csr(
        torch.zeros(2, 4, dtype=i32), torch.tensor([5, 9], dtype=i32), 4)
    yield "csr_to_block_table", lambda: gdn.csr_to_block_table(
        torch.tensor([0, 1, 3], dtype=i32), torch.tensor([0, 1, 2], dtype=i32),
        torch.tensor([2, 1], dtype=i32), 4, 4)
    yield "stream_copy", lambda: gdn.stream_copy(torch.empty(64, dtype=torch.uint8),
                                                 torch.zeros(64, dtype=torch.uint8))


def test_every_entry_point_refuses_host_tensors(case):
    c, pre, dec = case
    seen = []
    for name, call in calls(c, pre, dec):
        with pytest.raises(ValueError, match="GPU"):
            call()
        seen.append(name)
    exported = {n for n in ("prefill_slots", "decode_slots", "prefill_paged", "prefill_paged_noalloc",
                            "decode_paged", "prefill", "decode", "check_paged", "block_table_to_csr",
                            "csr_to_block_table", "stream_copy")}
    assert set(seen) == exported

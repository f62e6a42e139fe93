"""CSR page tables (test infrastructure only).

Source: FlashInfer CSR paging drill (gpu-kernel-drills, hint F1), sections
1-3 and the self-tests of section 6.  Sequence ``b`` owns the pages
``indices[indptr[b]:indptr[b+1]]``; ``indptr[0] = 0`` and ``indptr[B]`` is the
total page count; ``last_page_len[b]`` is the number of tokens used in the last
page, in ``1..page_size``.  The context length is recovered as
``(pages - 1) * page_size + last_page_len``.

Plain Python integers throughout, one sequence at a time.
"""

from __future__ import annotations

from typing import List, Sequence, Tuple


def pages_for(ctx: int, page_size: int) -> int:
    """Pages a sequence of ``ctx`` tokens needs: ceil(ctx / page_size)."""
    if ctx < 1:
        raise ValueError("a sequence in a CSR page table holds at least one token")
    return (ctx + page_size - 1) // page_size


def last_page_len_for(ctx: int, page_size: int) -> int:
    """Tokens used in the last page.

    The drill stresses that this is ``ctx - (pages - 1) * page_size`` (equal to
    ``(ctx - 1) % page_size + 1``) and NOT ``ctx % page_size``, which gives 0
    for a sequence that fills its last page exactly.
    """
    return ctx - (pages_for(ctx, page_size) - 1) * page_size


def csr_from_lengths(ctx_lens: Sequence[int], page_size: int,
                     page_ids: Sequence[int] | None = None
                     ) -> Tuple[List[int], List[int], List[int]]:
    """Build (indptr, indices, last_page_len) for sequences of ``ctx_lens`` tokens.

    ``page_ids`` lists the physical page ids of all sequences back to back
    (row-major over sequences); when omitted the ids are 0, 1, 2, ...
    """
    indptr = [0]
    lpl = []
    for ctx in ctx_lens:
        indptr.append(indptr[-1] + pages_for(int(ctx), page_size))
        lpl.append(last_page_len_for(int(ctx), page_size))
    total = indptr[-1]
    if page_ids is None:
        indices = list(range(total))
    else:
        indices = [int(x) for x in page_ids]
        if len(indices) != total:
            raise ValueError(f"need {total} page ids, got {len(indices)}")
    return indptr, indices, lpl


def block_table_to_csr(block_table: Sequence[Sequence[int]], ctx_lens: Sequence[int],
                       page_size: int) -> Tuple[List[int], List[int], List[int]]:
    """Padded block table -> CSR (drill section 2): keep the first
    ceil(ctx/page_size) entries of every row, in row-major order."""
    ids = []
    for row, ctx in zip(block_table, ctx_lens):
        ids.extend(int(x) for x in row[:pages_for(int(ctx), page_size)])
    return csr_from_lengths(ctx_lens, page_size, ids)


def csr_to_block_table(indptr: Sequence[int], indices: Sequence[int],
                       last_page_len: Sequence[int], page_size: int, max_blocks: int
                       ) -> Tuple[List[List[int]], List[int]]:
    """CSR -> padded block table plus context lengths (drill section 3).

    Page counts are adjacent differences of ``indptr``; padding entries are 0.
    """
    table = []
    ctx = []
    for b in range(len(indptr) - 1):
        n = indptr[b + 1] - indptr[b]
        row = list(indices[indptr[b]:indptr[b + 1]]) + [0] * (max_blocks - n)
        table.append(row)
        ctx.append((n - 1) * page_size + last_page_len[b])
    return table, ctx

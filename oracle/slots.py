"""Pool rows derived from a paged batch (test infrastructure only).

Source: flashinfer.gdn_paged (docs.flashinfer.ai/api/gdn_paged.html),
section "Page table" and section "Slot arguments of chunk_gated_delta_rule".

A sequence owns ``n`` pages and holds ``(n - 1) * page_size + last_page_len``
tokens AFTER the call; its new tokens are the last ``L`` of them, so its prefix
is ``p = total - L``.  Page ``j`` of a sequence holds the state after the last
token of that page.

Prefill rows (one sequence at a time, plain Python integers):

* read  -- the page holding the last prefix token, i.e. page ``(p-1)//ps`` of
  the sequence, or -1 (zero state) when the prefix is empty.
* write -- the last page, or -1 for a zero-length sequence, which writes
  nothing.
* checkpoints -- the paged call is a thin wrapper over the slot arguments with
  ``checkpoint_every_n_tokens = page_size`` and
  ``checkpoint_state_indices = page_indices``: the ``j``-th checkpoint of the
  call (absolute position ``pos``) goes to page ``pos/ps - 1``, which sits at
  ``page_indices[indptr[b] + p//ps + j]``; so the checkpoint start of the
  sequence is ``indptr[b] + p//ps``.  (Reading of a page that names the slot
  struct's fields only in part.)
* prefix_lens -- ``p``.
* chunk_starts -- exclusive running sum of the 64-token chunk counts;
  chunks sit at absolute positions that are multiples of 64 and the first one
  is padded on the left, so a sequence spans
  ``ceil(((p mod 64) + L) / 64)`` chunks (0 when ``L == 0``).

Decode rows: one new token per sequence.  When that token opens a new page
(``last_page_len == 1``) the call reads the previous page and writes the new
one; otherwise it reads and writes the last page.
"""

from __future__ import annotations

from typing import Dict, List, Sequence

CHUNK = 64


def _seq_pages(page_indices, page_indptr, b):
    return [int(x) for x in page_indices[int(page_indptr[b]):int(page_indptr[b + 1])]]


def prefill_slots(cu_seqlens: Sequence[int], page_indices: Sequence[int],
                  page_indptr: Sequence[int], last_page_len: Sequence[int],
                  page_size: int) -> Dict[str, List[int]]:
    """Rows of a paged prefill batch, one entry per sequence."""
    B = len(cu_seqlens) - 1
    out = {k: [] for k in ("state_indices", "output_state_indices",
                           "checkpoint_cu_starts", "prefix_lens", "chunk_starts")}
    running = 0
    for b in range(B):
        pages = _seq_pages(page_indices, page_indptr, b)
        n = len(pages)
        total = (n - 1) * page_size + int(last_page_len[b])
        L = int(cu_seqlens[b + 1]) - int(cu_seqlens[b])
        p = total - L
        out["state_indices"].append(pages[(p - 1) // page_size] if p > 0 else -1)
        out["output_state_indices"].append(pages[-1] if L > 0 else -1)
        out["checkpoint_cu_starts"].append(int(page_indptr[b]) + p // page_size)
        out["prefix_lens"].append(p)
        out["chunk_starts"].append(running)
        running += chunk_count(p, L)
    return out


def chunk_count(prefix: int, new_len: int) -> int:
    """64-token chunks of a sequence whose chunks sit at absolute multiples of 64."""
    if new_len <= 0:
        return 0
    return ((prefix % CHUNK) + new_len + CHUNK - 1) // CHUNK


def decode_slots(page_indices: Sequence[int], page_indptr: Sequence[int],
                 last_page_len: Sequence[int]) -> Dict[str, List[int]]:
    """Rows of a paged decode batch (T = 1)."""
    B = len(page_indptr) - 1
    rd, wr = [], []
    for b in range(B):
        pages = _seq_pages(page_indices, page_indptr, b)
        if not pages:
            raise ValueError("a decode sequence holds at least one token, so at least one page")
        if int(last_page_len[b]) == 1:
            if len(pages) < 2:
                raise ValueError("a token that opens a new page needs a previous page")
            rd.append(pages[-2])
        else:
            rd.append(pages[-1])
        wr.append(pages[-1])
    return {"initial_state_indices": rd, "output_state_indices": wr}


def checkpoint_count(prefix: int, new_len: int, every_n: int) -> int:
    """Checkpoints a call takes: positions ``prefix + n`` (n = 1..new_len)
    that are multiples of ``every_n``, counted one by one."""
    return sum(1 for n in range(1, new_len + 1) if (prefix + n) % every_n == 0)


# Validity of a paged batch: what the paged calls take on trust (the page
# table holds real page ids, never -1 padding; a row one sequence writes is
# touched by no other sequence of the call), as bits of a mask.  The bit
# values are this library's convention.
CHECK_INDPTR = 1         # indptr[0] != 0, decreasing, or a sequence with no page
CHECK_LAST_PAGE_LEN = 2  # last_page_len outside 1 .. page_size
CHECK_TOKENS = 4         # prefill: cu[0] != 0, negative or too many new tokens;
                         # decode: no token before the decoded one
CHECK_PAGE_ID = 8        # a page id outside 0 .. num_pages - 1
CHECK_SHARED_ROW = 16    # a row one sequence writes is read or written by another


def touched_rows(pages: Sequence[int], last_page_len: int, page_size: int, new_len=None):
    """(rows read, rows written) by one sequence of a paged call: a prefill
    (``new_len`` given) reads the page holding its last prefix token and writes
    every page ending after its prefix; a decode reads the previous page when
    the token opens a new one, else the last page, and writes the last page."""
    n = len(pages)
    total = (n - 1) * page_size + last_page_len
    if new_len is None:
        return ({pages[-2] if last_page_len == 1 else pages[-1]}, {pages[-1]})
    p = total - new_len
    reads = {pages[(p - 1) // page_size]} if p > 0 else set()
    writes = {pages[j] for j in range(p // page_size, n)} if new_len > 0 else set()
    return reads, writes


def check_paged(page_indices, page_indptr, last_page_len, page_size: int, num_pages: int,
                cu_seqlens=None) -> int:
    """Mask of the validity rules a paged batch breaks (0: none).  Structure
    first; page ids and shared rows only once the structure holds, as the
    ranges are unknown otherwise."""
    ptr = [int(x) for x in page_indptr]
    lpl = [int(x) for x in last_page_len]
    B = len(lpl)
    cu = None if cu_seqlens is None else [int(x) for x in cu_seqlens]
    bits = 0
    if ptr[0] != 0:
        bits |= CHECK_INDPTR
    for b in range(B):
        n = ptr[b + 1] - ptr[b]
        if n <= 0:
            bits |= CHECK_INDPTR
            continue
        if not 1 <= lpl[b] <= page_size:
            bits |= CHECK_LAST_PAGE_LEN
        total = (n - 1) * page_size + lpl[b]
        if cu is not None:
            L = cu[b + 1] - cu[b]
            if L < 0 or L > total:
                bits |= CHECK_TOKENS
        elif total < 2:
            bits |= CHECK_TOKENS
    if cu is not None and cu[0] != 0:
        bits |= CHECK_TOKENS
    if bits:
        return bits
    idx = [int(x) for x in page_indices[:ptr[B]]]
    if any(not 0 <= x < num_pages for x in idx):
        return CHECK_PAGE_ID
    touched = []
    for b in range(B):
        pages = idx[ptr[b]:ptr[b + 1]]
        L = None if cu is None else cu[b + 1] - cu[b]
        touched.append(touched_rows(pages, lpl[b], page_size, L))
    for b, (_, wb) in enumerate(touched):
        for c, (rc, wc) in enumerate(touched):
            if c != b and wb & (rc | wc):
                return CHECK_SHARED_ROW
    return 0

"""fp64 token-by-token Gated Delta-Rule over a paged state pool (test infrastructure only).

The recurrence.  The pages name the Gated Delta-Rule (flashinfer.gdn_paged,
opening paragraph) but do not write it out; this oracle uses the standard
gated delta rule with a per-head state ``S`` of shape ``[V, K]``:

    alpha_t = exp(g_t)
    S_t     = alpha_t * S_{t-1} + beta_t * (v_t - alpha_t * S_{t-1} k_t) k_t^T
    o_t     = scale * S_t q_t,            scale = 1 / sqrt(K) unless given

The output uses the state AFTER the token's update.  ``g`` absent means
``g = 0`` and ``beta`` absent means ``beta = 1`` (the page's signature marks
them optional).  With fewer q/k heads than v-heads, v-head ``h`` uses q/k head
``h // (H / Hqk)``.

Row semantics, restated from flashinfer.gdn_paged, section "Slot arguments of
chunk_gated_delta_rule":

* the zero state is used where the read row is -1 (built from literal zeros:
  multiplying a loaded row by 0 would keep a NaN in it);
* where the write row is -1 the final state is not stored; a sequence with no
  new tokens stores nothing at all;
* a sequence's checkpoints are numbered from 0 in the order they occur; the
  j-th of sequence ``i`` is stored in row
  ``checkpoint_state_indices[checkpoint_cu_starts[i] + j]`` (nothing is stored
  where that entry is -1), and one occurs after new token ``n`` whenever
  ``prefix_lens[i] + n`` is divisible by ``checkpoint_every_n_tokens``;
* the three state buffers may alias one pool, and a row that a sequence
  writes must not be touched (read or written) by any other sequence of the
  same call.

No chunking, no padding, no blocking: one token at a time, all heads of the
token at once in fp64.  Inputs are upcast exactly (bf16 and fp32 values are
representable in fp64).

State dtype.  The first page requires only that a pool shared by the prefill
and the decode entry points use an element type that both accept (pool
paragraph of flashinfer.gdn_paged, "Page table").  Reading: every state buffer
of a call has
one element type, fp32 or bf16; the arithmetic is unchanged, and a state is
rounded to the buffer's type only where it is stored (checkpoints and the
final state), to nearest with ties to even.  ``state_dtype="bf16"`` applies
that rounding to the stored states (the fp64 value goes through fp32 first,
both steps to nearest even); ``"fp32"`` keeps the fp64 states unrounded, the
reference the fp32 path is compared against within tolerance.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Optional, Sequence

import numpy as np

from . import slots as _slots


@dataclass
class Result:
    o: np.ndarray                                   # [T, H, V] fp64
    final: Dict[int, np.ndarray] = field(default_factory=dict)        # row -> [H, V, K]
    checkpoints: Dict[int, np.ndarray] = field(default_factory=dict)  # row -> [H, V, K]
    reads: Dict[int, int] = field(default_factory=dict)               # seq -> row read

    def writes(self) -> Dict[int, np.ndarray]:
        """All rows written, for calls whose three buffers are one pool."""
        out = dict(self.checkpoints)
        for r, s in self.final.items():
            if r in out and out[r].tobytes() != s.tobytes():
                raise ValueError(f"row {r} written twice with different states")
            out[r] = s
        return out


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _to_numpy(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor (CPU); bf16 goes through fp32 exactly
        import torch
        t = x.detach().cpu()
        if t.dtype == torch.bfloat16:
            t = t.to(torch.float32)
        return t.numpy()
    return np.asarray(x)


def gdn_token(S: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray,
              g: np.ndarray, beta: np.ndarray, scale: float):
    """One token for every head at once.

    S: [H, V, K]; q, k: [H, K] (already mapped to v-heads); v: [H, V];
    g, beta: [H].  Returns the updated state and the output [H, V].
    """
    alpha = np.exp(g)                                             # [H]
    Sk = np.matmul(S, k[:, :, None])[:, :, 0]                     # S_{t-1} k_t  [H, V]
    delta = beta[:, None] * (v - alpha[:, None] * Sk)             # [H, V]
    S = alpha[:, None, None] * S + delta[:, :, None] * k[:, None, :]
    o = scale * np.matmul(S, q[:, :, None])[:, :, 0]
    return S, o


def round_bf16(x) -> np.ndarray:
    """fp64 values rounded to bfloat16 (via fp32, each step to nearest, ties to
    even), returned as fp64.  bf16 keeps the upper 16 bits of an fp32: add half
    an ulp of the kept part (0x7fff, plus 1 when the kept part is odd) and cut."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    bits = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) << 16
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


def _store(S: np.ndarray, state_dtype: str) -> np.ndarray:
    if state_dtype == "fp32":
        return S.copy()
    if state_dtype == "bf16":
        return round_bf16(S)
    raise ValueError(f"state_dtype must be 'fp32' or 'bf16', got {state_dtype!r}")


def _head_map(H: int, Hqk: int) -> np.ndarray:
    if H % Hqk != 0:
        raise ValueError("v-heads must be a multiple of q/k heads")
    return np.arange(H) // (H // Hqk)


def _check_hazards(reads: Dict[int, int], final_w: Dict[int, set], ckpt_w: Dict[int, set],
                   shared_pool: bool):
    """Rows one sequence writes are read or written by no other sequence.

    With ``shared_pool`` the initial, output and checkpoint buffers are one
    memory (the paged case); otherwise each buffer is checked on its own and
    reads (of the initial buffer) cannot collide with writes."""
    groups = [(final_w, ckpt_w)] if shared_pool else [(final_w,), (ckpt_w,)]
    for grp in groups:
        owner = {}
        for w in grp:
            for b, rows in w.items():
                for r in rows:
                    if r in owner and owner[r] != b:
                        raise ValueError(f"row {r} written by sequences {owner[r]} and {b}")
                    owner[r] = b
        if shared_pool:
            for b, r in reads.items():
                if r in owner and owner[r] != b:
                    raise ValueError(f"row {r} read by sequence {b} but written by {owner[r]}")


def prefill(q, k, v, g, beta, cu_seqlens, *,
            initial_state=None, state_indices=None,
            output_final_state: bool = False, output_state_indices=None,
            checkpoint_state_indices=None, checkpoint_cu_starts=None,
            prefix_lens=None, checkpoint_every_n_tokens: int = 0,
            scale: Optional[float] = None, shared_pool: bool = True,
            state_dtype: str = "fp32") -> Result:
    """General slot-argument prefill over a packed variable-length batch.

    q, k: [T, Hqk, K]; v: [T, H, V]; g, beta: [T, H] or None;
    cu_seqlens: [B + 1]; initial_state: [rows, H, V, K] (anything indexable by
    row) or None.
    Without ``state_indices`` sequence ``b`` reads row ``b`` of
    ``initial_state``; without ``output_state_indices`` it writes back to its
    read row (an in-place slot update).  ``shared_pool`` says whether the
    three state buffers are one memory (for the cross-sequence hazard check).
    ``state_dtype`` is the element type of the state buffers (module docstring).
    """
    _store(np.zeros(1), state_dtype)  # validates the name
    q, k, v = _f64(_to_numpy(q)), _f64(_to_numpy(k)), _f64(_to_numpy(v))
    T, Hqk, K = q.shape
    H, V = v.shape[1], v.shape[2]
    g = np.zeros((T, H)) if g is None else _f64(_to_numpy(g))
    beta = np.ones((T, H)) if beta is None else _f64(_to_numpy(beta))
    cu = [int(x) for x in _to_numpy(cu_seqlens)]
    B = len(cu) - 1
    hmap = _head_map(H, Hqk)
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    init = initial_state  # indexed row by row: ndarray, tensor or any row-indexable object
    sidx = None if state_indices is None else [int(x) for x in _to_numpy(state_indices)]
    oidx = None if output_state_indices is None else [int(x) for x in _to_numpy(output_state_indices)]
    N = int(checkpoint_every_n_tokens)
    cidx = None if checkpoint_state_indices is None else [int(x) for x in _to_numpy(checkpoint_state_indices)]
    cstart = None if checkpoint_cu_starts is None else [int(x) for x in _to_numpy(checkpoint_cu_starts)]
    plen = None if prefix_lens is None else [int(x) for x in _to_numpy(prefix_lens)]
    if cidx is not None and (N <= 0 or plen is None or cstart is None):
        raise ValueError("checkpoint rows need checkpoint_every_n_tokens > 0, prefix_lens "
                         "and checkpoint_cu_starts")
    if oidx is not None and not output_final_state:
        raise ValueError("output_state_indices needs output_final_state")

    res = Result(o=np.zeros((T, H, V)))
    reads, final_w, ckpt_w = {}, {}, {}
    for b in range(B):
        L = cu[b + 1] - cu[b]
        if L == 0:
            continue  # a zero-length sequence writes nothing
        if init is None:
            rd = -1
        else:
            rd = sidx[b] if sidx is not None else b
        if rd == -1:
            S = np.zeros((H, V, K))
        else:
            S = _f64(_to_numpy(init[rd])).copy()
            reads[b] = rd
        res.reads[b] = rd
        p = plen[b] if plen is not None else 0
        for n in range(1, L + 1):
            t = cu[b] + n - 1
            S, res.o[t] = gdn_token(S, q[t, hmap], k[t, hmap], v[t], g[t], beta[t], scale)
            if cidx is not None and (p + n) % N == 0:
                j = (p + n) // N - p // N - 1
                row = cidx[cstart[b] + j]
                if row != -1:
                    res.checkpoints[row] = _store(S, state_dtype)
                    ckpt_w.setdefault(b, set()).add(row)
        if output_final_state:
            if oidx is not None:
                wr = oidx[b]
            else:
                wr = sidx[b] if sidx is not None else b
            if wr != -1:
                res.final[wr] = _store(S, state_dtype)
                final_w.setdefault(b, set()).add(wr)
    _check_hazards(reads, final_w, ckpt_w, shared_pool)
    return res


def decode(q, k, v, g, beta, *, initial_state, initial_state_indices=None,
           output_state_indices=None, scale: Optional[float] = None,
           shared_pool: bool = True, state_dtype: str = "fp32") -> Result:
    """One token per sequence.  q, k: [B, Hqk, K]; v: [B, H, V]; g, beta: [B, H].

    Rows default to ``b``; the write row defaults to the read row.  A read row
    of -1 starts from zero and a write row of -1 skips the store.
    """
    q = _to_numpy(q)
    B = q.shape[0]
    cu = list(range(B + 1))
    ridx = list(range(B)) if initial_state_indices is None else initial_state_indices
    widx = ridx if output_state_indices is None else output_state_indices
    return prefill(q, k, v, g, beta, cu, initial_state=initial_state,
                   state_indices=ridx, output_final_state=True,
                   output_state_indices=widx, scale=scale, shared_pool=shared_pool,
                   state_dtype=state_dtype)


def prefill_paged(q, k, v, g, beta, cu_seqlens, state_pool, page_indices, page_indptr,
                  last_page_len, page_size: int, scale: Optional[float] = None,
                  state_dtype: str = "fp32"):
    """Paged prefill = the slot-argument prefill with all three buffers set to
    the pool, rows from ``slots.prefill_slots``, checkpoints every ``page_size``
    tokens into ``page_indices`` (flashinfer.gdn_paged calls the paged entry
    point a thin wrapper over these arguments).

    Returns (o, writes, slots): ``writes`` maps pool row -> fp64 [H, V, K].
    """
    if page_size <= 0 or page_size % _slots.CHUNK != 0:
        raise ValueError("page_size must be a positive multiple of 64")
    cu = [int(x) for x in _to_numpy(cu_seqlens)]
    pidx = [int(x) for x in _to_numpy(page_indices)]
    ptr = [int(x) for x in _to_numpy(page_indptr)]
    lpl = [int(x) for x in _to_numpy(last_page_len)]
    sl = _slots.prefill_slots(cu, pidx, ptr, lpl, page_size)
    res = prefill(q, k, v, g, beta, cu, initial_state=state_pool,
                  state_indices=sl["state_indices"], output_final_state=True,
                  output_state_indices=sl["output_state_indices"],
                  checkpoint_state_indices=pidx,
                  checkpoint_cu_starts=sl["checkpoint_cu_starts"],
                  prefix_lens=sl["prefix_lens"], checkpoint_every_n_tokens=page_size,
                  scale=scale, state_dtype=state_dtype)
    return res.o, res.writes(), sl


def decode_paged(q, k, v, g, beta, state_pool, page_indices, page_indptr, last_page_len,
                 scale: Optional[float] = None, state_dtype: str = "fp32"):
    """Paged decode (T = 1): rows from ``slots.decode_slots``.

    Returns (o, writes, slots)."""
    pidx = [int(x) for x in _to_numpy(page_indices)]
    ptr = [int(x) for x in _to_numpy(page_indptr)]
    lpl = [int(x) for x in _to_numpy(last_page_len)]
    sl = _slots.decode_slots(pidx, ptr, lpl)
    res = decode(q, k, v, g, beta, initial_state=state_pool,
                 initial_state_indices=sl["initial_state_indices"],
                 output_state_indices=sl["output_state_indices"], scale=scale,
                 state_dtype=state_dtype)
    return res.o, res.writes(), sl


def apply_writes(pool: np.ndarray, writes: Dict[int, np.ndarray]) -> np.ndarray:
    """Return a copy of ``pool`` with ``writes`` stored (no rounding: the copy
    has the dtype of ``pool``, so an fp64 shadow pool stays exact)."""
    out = pool.copy()
    for r, s in writes.items():
        out[r] = s
    return out

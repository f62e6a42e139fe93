"""Helpers for the GPU parity tests: run the HIP path and the oracle on the
same seeded inputs and compare (tolerances below are the acceptance bar)."""

from __future__ import annotations

import numpy as np
import torch

# Acceptance bar: outputs max abs <= 2e-2 and relative Frobenius <= 5e-3;
# final and checkpoint states relative Frobenius <= 1e-3 (fp32 state, bf16
# q/k/v); slot rows, page-write sets and untouched pages bit-exact.
O_MAX_ABS = 2e-2
O_REL_FRO = 5e-3
S_REL_FRO = 1e-3


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def check_outputs(o_gpu: torch.Tensor, o_ref: np.ndarray, what: str = "o"):
    o = o_gpu.detach().float().cpu().numpy().astype(np.float64)
    assert o.shape == o_ref.shape, (o.shape, o_ref.shape)
    assert np.isfinite(o).all(), f"{what}: non-finite values"
    mx = float(np.abs(o - o_ref).max()) if o.size else 0.0
    rf = rel_fro(o, o_ref) if o.size else 0.0
    assert mx <= O_MAX_ABS, f"{what}: max abs err {mx:.3e} > {O_MAX_ABS}"
    assert rf <= O_REL_FRO, f"{what}: rel Frobenius err {rf:.3e} > {O_REL_FRO}"
    return mx, rf


def check_state(s_gpu, s_ref: np.ndarray, what: str = "state"):
    s = s_gpu.detach().float().cpu().numpy().astype(np.float64) if isinstance(s_gpu, torch.Tensor) \
        else np.asarray(s_gpu, dtype=np.float64)
    assert np.isfinite(s).all(), f"{what}: non-finite values"
    rf = rel_fro(s, s_ref)
    assert rf <= S_REL_FRO, f"{what}: rel Frobenius err {rf:.3e} > {S_REL_FRO}"
    return rf


def changed_rows(before: torch.Tensor, after: torch.Tensor, block: int = 512):
    """Rows of a [rows, H, V, K] fp32 or bf16 pool whose bits differ (on device, in blocks)."""
    out = []
    bits = torch.int32 if before.element_size() == 4 else torch.int16
    for r0 in range(0, before.shape[0], block):
        a = before[r0:r0 + block].view(bits).reshape(-1, before[0].numel())
        b = after[r0:r0 + block].view(bits).reshape(-1, after[0].numel())
        out.extend((r0 + torch.nonzero((a != b).any(dim=1)).flatten()).tolist())
    return sorted(out)


def pool_rows_cpu(pool: torch.Tensor, rows):
    """fp32 CPU copy of selected rows (oracle input; bf16 rows convert exactly),
    as a dict-like array."""
    rows = sorted(set(int(r) for r in rows if int(r) >= 0))
    out = {}
    for r in rows:
        out[r] = pool[r].detach().float().cpu().numpy()
    return out


class RowView:
    """Array-like over a dict of rows so the oracle can index pool[row]."""

    def __init__(self, rows):
        self.rows = rows

    def __getitem__(self, r):
        return self.rows[int(r)]


def cuda(d, device="cuda"):
    if isinstance(d, torch.Tensor):
        return d.to(device)
    if isinstance(d, dict):
        return {k: cuda(v, device) for k, v in d.items()}
    if isinstance(d, list):
        return [cuda(v, device) for v in d]
    return d

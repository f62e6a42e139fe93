"""Inputs that stress the precision budget, HIP path against the fp64 oracle.

The configs' inputs (unit-norm q and k, N(0, 1) v, g = -softplus(N(0, 1)),
beta = sigmoid(N(0, 1)), scale 1/sqrt(128)) leave states near 1e-5 and
outputs near 3e-3 relative error.  Here the inputs move to the edges of what
the recurrence meets: weak or no decay over thousands of tokens (the state
then carries every chunk's rounding), values 16x larger, a caller scale of 1,
beta at 1 and near 0, and decay strong enough to reset the state at every
token.  Relative errors are scale-free, so every case checks the relative
bars (outputs 5e-3, states 1e-3); the cases with decay also check the tighter
budget the kernels are built to (states 1e-4, outputs 3.5e-3).  The absolute
output bar (2e-2) is stated for the configs' value ranges and is checked
where those hold."""

import numpy as np
import pytest
import torch

import workloads
from oracle import gdn as ogdn
from tests.gpu_util import RowView, changed_rows, pool_rows_cpu, rel_fro
from tests.test_gpu_small import lib, opts

pytestmark = pytest.mark.gpu
DEV = "cuda"


def paged_case(prefix, new, ps, H, Hqk, seed, shape_inputs):
    gen = workloads.generator(seed)
    pages, nxt = [], 0
    for p, n in zip(prefix, new):
        cnt = (p + n + ps - 1) // ps
        pages.append(list(range(nxt, nxt + cnt)))
        nxt += cnt
    pre = workloads._prefill_batch(prefix, new, pages, ps, Hqk, H, 128, 128, gen, "cpu")
    shape_inputs(pre, gen)
    pool = workloads.nan_pool(nxt + 1, H, 128, 128)
    workloads.fill_rows(pool, [r for r in pre["read_rows"] if r >= 0], gen, 0.09)
    pre = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in pre.items()}
    return pre, pool.to(DEV)


def run_and_compare(pre, pool, scale=None, options=None):
    m = lib()
    rows_in = pool_rows_cpu(pool, pre["read_rows"])
    before = pool.clone()
    o = m.prefill_paged(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], pre["cu_seqlens"],
                        pool, pre["page_indices"], pre["page_indptr"], pre["page_size"],
                        pre["last_page_len"], scale=scale, options=options)
    torch.cuda.synchronize()
    o_ref, writes, _ = ogdn.prefill_paged(pre["q"].cpu(), pre["k"].cpu(), pre["v"].cpu(),
                                          pre["g"].cpu(), pre["beta"].cpu(),
                                          pre["cu_seqlens"].cpu(), RowView(rows_in),
                                          pre["page_indices"].cpu(), pre["page_indptr"].cpu(),
                                          pre["last_page_len"].cpu(), pre["page_size"],
                                          scale=scale)
    og = o.float().cpu().numpy()
    assert np.isfinite(og).all()
    assert changed_rows(before, pool) == sorted(writes)
    o_err = rel_fro(og, o_ref)
    o_abs = float(np.abs(og - o_ref).max())
    s_err = max(rel_fro(pool[r].float().cpu().numpy(), s) for r, s in writes.items())
    return o_err, o_abs, s_err


def scaled(g=None, v=None, beta=None):
    def f(pre, gen):
        if g is not None:
            pre["g"] = g(pre["g"], gen)
        if v is not None:
            pre["v"] = (pre["v"].float() * v).to(torch.bfloat16)
        if beta is not None:
            pre["beta"] = beta(pre["beta"], gen)
    return f


LONG = dict(prefix=[0, 37, 900], new=[2400, 1900, 1300], ps=256, H=4, Hqk=2)


@pytest.mark.parametrize("g_scale,split", [(0.1, 0), (0.1, -1), (0.01, 0), (0.0, -1), (0.0, 0)])
def test_weak_and_no_decay_long(g_scale, split):
    """Decay g / 10, g / 100 and none over ~2k-token sequences (the state
    carries every chunk's rounding; with no decay nothing is forgotten)."""
    pre, pool = paged_case(**LONG, seed=70, shape_inputs=scaled(g=lambda g, _: g * g_scale))
    o_err, o_abs, s_err = run_and_compare(pre, pool, options=opts(prefill_split_chunks=split))
    print(f"g x {g_scale}, split {split}: o {o_err:.2e} (abs {o_abs:.2e}), states {s_err:.2e}")
    assert o_err <= 5e-3 and s_err <= 1e-3 and o_abs <= 2e-2
    if g_scale > 0:
        assert o_err <= 3.5e-3 and s_err <= 1e-4


@pytest.mark.parametrize("case", ["v_x16", "scale_1", "beta_1", "beta_small", "reset"])
def test_value_extremes(case):
    shape = {
        "v_x16": scaled(v=16.0),
        "scale_1": scaled(),
        "beta_1": scaled(beta=lambda b, _: torch.ones_like(b)),
        "beta_small": scaled(beta=lambda b, _: b * 1e-3),
        "reset": scaled(g=lambda g, _: g - 30.0),  # exp(g) < 1e-13: the state restarts each token
    }[case]
    pre, pool = paged_case([0, 37, 900], [700, 500, 300], 128, 4, 2, 71, shape)
    o_err, o_abs, s_err = run_and_compare(pre, pool, scale=1.0 if case == "scale_1" else None)
    print(f"{case}: o {o_err:.2e} (abs {o_abs:.2e}), states {s_err:.2e}")
    assert o_err <= 3.5e-3 and s_err <= 1e-4
    if case not in ("v_x16", "scale_1"):  # outputs in the configs' range
        assert o_abs <= 2e-2


@pytest.mark.parametrize("where", ["g", "beta", "k"])
@pytest.mark.parametrize("split", [8, -1])
def test_nan_input_reaches_later_states(where, split):
    """A NaN in g, beta or k at one token reaches every later output and state
    of the heads it feeds, as in the recurrence, also when the first pass of
    the sequence-parallel plan skips work (8-chunk segments with the configs'
    decay): the token's chunk has a NaN transition bound, so its segment's
    transition is computed in full and carries the NaN into the next
    segment's start, even where the offset run starts after the token.
    Within the token's 64-token chunk the NaN also reaches the rows before it
    (the chunk's triangular products multiply the zeros above the diagonal by
    it), and no further back.  Everything else matches the oracle."""
    def shape(pre, gen):
        if where == "g":
            pre["g"][70, 0] = float("nan")
        elif where == "beta":
            pre["beta"][70, 0] = float("nan")
        else:
            k = pre["k"].clone()
            k[70, 0, 5] = float("nan")
            pre["k"] = k
    pre, pool = paged_case([0], [2048], 256, 2, 1, 91, shape)
    m = lib()
    rows_in = pool_rows_cpu(pool, pre["read_rows"])
    before = pool.clone()
    o = m.prefill_paged(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], pre["cu_seqlens"],
                        pool, pre["page_indices"], pre["page_indptr"], pre["page_size"],
                        pre["last_page_len"], options=opts(prefill_split_chunks=split))
    torch.cuda.synchronize()
    o_ref, writes, _ = ogdn.prefill_paged(pre["q"].cpu(), pre["k"].cpu(), pre["v"].cpu(),
                                          pre["g"].cpu(), pre["beta"].cpu(),
                                          pre["cu_seqlens"].cpu(), RowView(rows_in),
                                          pre["page_indices"].cpu(), pre["page_indptr"].cpu(),
                                          pre["last_page_len"].cpu(), pre["page_size"])
    og = o.float().cpu().numpy()
    nan_heads = [0] if where != "k" else [0, 1]  # k: the q/k head feeds both v-heads
    # outputs: NaN from the token on in the heads it feeds (the oracle), and on
    # the GPU also from the start of its chunk (token 64), nowhere else
    ref_nan = np.isnan(o_ref).any(axis=2)
    got_nan = np.isnan(og).any(axis=2)
    assert ref_nan[70:, nan_heads].all() and not ref_nan[:70].any()
    expect = np.zeros_like(ref_nan)
    expect[64:, nan_heads] = True
    assert (got_nan == expect).all()
    fin = ~got_nan
    assert rel_fro(og[fin], o_ref[fin]) <= 5e-3
    # states: every stored row after the token is NaN in those heads, finite elsewhere
    assert changed_rows(before, pool) == sorted(writes)
    for r, s in writes.items():
        got = pool[r].float().cpu().numpy()
        for h in range(2):
            if np.isnan(s[h]).any():
                assert h in nan_heads and np.isnan(s[h]).all() and np.isnan(got[h]).all(), (r, h)
            else:
                assert np.isfinite(got[h]).all() and rel_fro(got[h], s[h]) <= 1e-3, (r, h)
    print(f"NaN in {where}, split {split}: {len(writes)} rows stored")

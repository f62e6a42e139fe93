"""Seeded random batches against the oracle: paged prefill (batch sizes,
prefixes and new lengths with zeros, page and chunk boundaries, page sizes,
head layouts, decay scales, state types, prefill tile widths and forced
sequence-parallel splits drawn per case), the slot-argument prefill (with and
without drawn launch options), and paged decode over every kernel shape.  The same parity bar as every other GPU test:
outputs and states within tolerance, write sets and untouched rows bit for
bit."""

import os

import numpy as np
import pytest

from tests.test_gpu_small import check_paged_prefill, make_case

pytestmark = pytest.mark.gpu


def seeds(n):
    """The first n seeds, times GDN_RANDOM_SCALE when set (a longer sweep over
    the same draws, e.g. GDN_RANDOM_SCALE=100)."""
    return range(n * max(1, int(os.environ.get("GDN_RANDOM_SCALE", "1"))))


def draw_case(seed):
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 7))
    ps = int(rng.choice([64, 128, 192, 256]))
    H, Hqk = [(1, 1), (2, 1), (2, 2), (4, 2), (4, 4)][int(rng.integers(0, 5))]
    special = [0, 1, 63, 64, 65, ps - 1, ps, ps + 1]
    prefix = [int(rng.choice(special)) if rng.random() < 0.4 else int(rng.integers(0, 600))
              for _ in range(B)]
    new = [int(rng.choice(special)) if rng.random() < 0.4 else int(rng.integers(0, 400))
           for _ in range(B)]
    for b in range(B):
        if prefix[b] + new[b] == 0:
            prefix[b] = 1  # every sequence holds a token (one page)
    g_scale = float(rng.choice([0.0, 0.1, 1.0]))
    bf16 = bool(rng.random() < 0.3)
    waves = int(rng.choice([8, 8, 4, 2]))
    split = int(rng.choice([0, 0, -1, 1, 2, 3]))
    return dict(prefix=prefix, new=new, ps=ps, H=H, Hqk=Hqk, g_scale=g_scale, bf16=bf16,
                waves=waves, split=split)


@pytest.mark.parametrize("seed", seeds(16))
def test_random_paged_prefill(seed):
    import torch

    from tests.test_gpu_small import opts
    c = draw_case(seed)
    pre, pool = make_case(c["prefix"], c["new"], ps=c["ps"], H=c["H"], Hqk=c["Hqk"],
                          seed=seed, g_scale=c["g_scale"])
    if c["bf16"]:
        pool = pool.to(torch.bfloat16)
    o = opts(prefill_tile_waves=c["waves"], prefill_split_chunks=c["split"])
    _, _, err = check_paged_prefill(pre, pool, options=o)
    print(f"case {seed}: {c} worst state rel {err:.2e}")


@pytest.mark.parametrize("seed", seeds(6))
def test_random_paged_prefill_grouped_heads(seed):
    """Random draws on head layouts whose v-heads the prefill kernels place in
    q/k-head groups (16 on 8, 32 on 16), shorter sequences."""
    import torch

    from tests.test_gpu_small import opts
    c = draw_case(100 + seed)
    c["H"], c["Hqk"] = [(16, 8), (32, 16)][seed % 2]
    c["prefix"] = [min(x, 300) for x in c["prefix"]][:4]
    c["new"] = [min(x, 260) for x in c["new"]][:4]
    for b in range(len(c["new"])):
        if c["prefix"][b] + c["new"][b] == 0:
            c["prefix"][b] = 1
    pre, pool = make_case(c["prefix"], c["new"], ps=c["ps"], H=c["H"], Hqk=c["Hqk"],
                          seed=seed, g_scale=c["g_scale"])
    if c["bf16"]:
        pool = pool.to(torch.bfloat16)
    o = opts(prefill_tile_waves=c["waves"], prefill_split_chunks=c["split"])
    _, _, err = check_paged_prefill(pre, pool, options=o)
    print(f"grouped case {seed}: {c} worst state rel {err:.2e}")


def draw_wide(seed):
    """Wider draws: up to 8 sequences of up to 2,500 new tokens, the 896-token
    page of the hybrid step, head groups up to 16 on 8, decay scales from none
    to 3x (gamma underflows to zero inside a chunk), every tile width and
    forced segments of up to 9 chunks (long enough for the first pass to skip
    negligible transitions)."""
    rng = np.random.default_rng(77000 + seed)
    B = int(rng.integers(1, 9))
    ps = int(rng.choice([64, 128, 192, 256, 896]))
    H, Hqk = [(1, 1), (2, 1), (2, 2), (4, 2), (4, 4), (8, 4), (16, 8), (8, 8)][int(rng.integers(0, 8))]
    special = [0, 1, 63, 64, 65, ps - 1, ps, ps + 1]
    maxnew = int(rng.choice([300, 1200, 2500]))
    if H >= 8:
        maxnew = min(maxnew, 1200)
    prefix = [int(rng.choice(special)) if rng.random() < 0.4 else int(rng.integers(0, 2000))
              for _ in range(B)]
    new = [int(rng.choice(special)) if rng.random() < 0.3 else int(rng.integers(0, maxnew))
           for _ in range(B)]
    for b in range(B):
        if prefix[b] + new[b] == 0:
            prefix[b] = 1
    g_scale = float(rng.choice([0.0, 0.02, 0.1, 1.0, 1.0, 3.0]))
    bf16 = bool(rng.random() < 0.25)
    waves = int(rng.choice([8, 8, 8, 4, 2, 1]))
    split = int(rng.choice([0, 0, 0, -1, 1, 2, 3, 4, 5, 7, 9]))
    return dict(prefix=prefix, new=new, ps=ps, H=H, Hqk=Hqk, g_scale=g_scale, bf16=bf16,
                waves=waves, split=split)


@pytest.mark.parametrize("seed", seeds(24))
def test_random_paged_prefill_wide(seed):
    import torch

    from tests.test_gpu_small import opts
    c = draw_wide(seed)
    pre, pool = make_case(c["prefix"], c["new"], ps=c["ps"], H=c["H"], Hqk=c["Hqk"],
                          seed=seed, g_scale=c["g_scale"])
    if c["bf16"]:
        pool = pool.to(torch.bfloat16)
    o = opts(prefill_tile_waves=c["waves"], prefill_split_chunks=c["split"])
    _, _, err = check_paged_prefill(pre, pool, options=o)
    print(f"wide case {seed}: {c} worst state rel {err:.2e}")


def draw_general(seed):
    rng = np.random.default_rng(5000 + seed)
    B = int(rng.integers(1, 6))
    H, Hqk = [(1, 1), (2, 1), (2, 2), (4, 2)][int(rng.integers(0, 4))]
    N = int(rng.choice([1, 17, 48, 64, 100, 128, 200]))
    max_len = 40 if N == 1 else (120 if N < 64 else 300)
    special = [0, 1, 63, 64, 65, N - 1, N, N + 1]
    prefix = [int(rng.choice(special)) if rng.random() < 0.4 else int(rng.integers(0, 500))
              for _ in range(B)]
    new = [min(max_len, int(rng.choice(special)) if rng.random() < 0.4
               else int(rng.integers(0, max_len + 1))) for _ in range(B)]
    return dict(B=B, H=H, Hqk=Hqk, N=N, prefix=[max(0, x) for x in prefix],
                new=[max(0, x) for x in new], g_scale=float(rng.choice([0.1, 1.0])),
                bf16=bool(rng.random() < 0.3), idx64=bool(rng.random() < 0.5),
                scale=None if rng.random() < 0.7 else 0.05, rng=rng)


@pytest.mark.parametrize("seed", seeds(12))
def test_random_general_prefill(seed):
    """The slot-argument call with three separate state buffers, random -1
    rows (zero start, skipped final or checkpoint store), int32 or int64 rows,
    any checkpoint interval and an explicit scale, against the oracle; every
    row no sequence writes keeps its NaN bits."""
    run_general(draw_general(seed), seed)


def draw_general_wide(seed):
    """Longer sequences (up to 2,500 new tokens), head groups up to 16 on 8,
    checkpoint intervals up to the 896-token page, and a drawn tile width and
    sequence-parallel choice (device-planned, whole, or forced segments)."""
    rng = np.random.default_rng(6000 + seed)
    B = int(rng.integers(1, 7))
    H, Hqk = [(1, 1), (2, 1), (4, 2), (8, 4), (16, 8)][int(rng.integers(0, 5))]
    N = int(rng.choice([1, 48, 64, 100, 128, 200, 896]))
    max_len = 200 if N == 1 else (1200 if H >= 8 else 2500)
    special = [0, 1, 63, 64, 65, N - 1, N, N + 1]
    prefix = [int(rng.choice(special)) if rng.random() < 0.4 else int(rng.integers(0, 3000))
              for _ in range(B)]
    new = [min(max_len, int(rng.choice(special)) if rng.random() < 0.3
               else int(rng.integers(0, max_len + 1))) for _ in range(B)]
    return dict(B=B, H=H, Hqk=Hqk, N=N, prefix=[max(0, x) for x in prefix],
                new=[max(0, x) for x in new], g_scale=float(rng.choice([0.0, 0.1, 1.0, 3.0])),
                bf16=bool(rng.random() < 0.25), idx64=bool(rng.random() < 0.5),
                scale=None if rng.random() < 0.7 else 0.05, rng=rng,
                waves=int(rng.choice([8, 8, 4, 2])), split=int(rng.choice([0, 0, -1, 2, 5, 9])))


@pytest.mark.parametrize("seed", seeds(12))
def test_random_general_prefill_wide(seed):
    run_general(draw_general_wide(seed), seed)


def run_general(c, seed):
    import torch

    import workloads
    from oracle import gdn as ogdn
    from tests.gpu_util import RowView, changed_rows, check_outputs, check_state, pool_rows_cpu
    from tests.test_gpu_small import lib, opts

    m = lib()
    rng, B, H, Hqk, N = c["rng"], c["B"], c["H"], c["Hqk"], c["N"]
    dev = "cuda"
    gen = workloads.generator(seed)
    T = sum(c["new"])
    t = {k: v.to(dev) for k, v in workloads.token_inputs(T, Hqk, H, 128, 128, gen,
                                                          g_scale=c["g_scale"]).items()}
    cu = torch.tensor(np.concatenate([[0], np.cumsum(c["new"])]), dtype=torch.int32, device=dev)
    n_ck = [(p + n) // N - p // N for p, n in zip(c["prefix"], c["new"])]
    ck_start = np.concatenate([[0], np.cumsum(n_ck)])[:-1]
    R_in, R_out, R_ck = B + 2, B + 2, max(1, sum(n_ck) + 2)
    sidx = [int(x) if rng.random() < 0.7 else -1 for x in rng.permutation(R_in)[:B]]
    oidx = [int(x) if rng.random() < 0.8 else -1 for x in rng.permutation(R_out)[:B]]
    cidx = [int(x) if rng.random() < 0.7 else -1 for x in rng.permutation(R_ck)[:sum(n_ck)]]
    sd = torch.bfloat16 if c["bf16"] else torch.float32
    init = workloads.nan_pool(R_in, H, 128, 128, device=dev)
    workloads.fill_rows(init, [r for r in sidx if r >= 0], workloads.gen_on(seed + 7, dev), 0.09)
    init = init.to(sd)
    out = workloads.nan_pool(R_out, H, 128, 128, device=dev).to(sd)
    ck = workloads.nan_pool(R_ck, H, 128, 128, device=dev).to(sd)
    it = torch.int64 if c["idx64"] else torch.int32
    mk = lambda x: torch.tensor(np.asarray(x, dtype=np.int64), dtype=it, device=dev)  # noqa: E731
    rows_in = pool_rows_cpu(init, [r for r in sidx if r >= 0])
    out0, ck0 = out.clone(), ck.clone()
    options = (opts(prefill_tile_waves=c["waves"], prefill_split_chunks=c["split"])
               if "split" in c else None)
    o = m.prefill(t["q"], t["k"], t["v"], t["g"], t["beta"], cu, initial_state=init,
                  state_indices=mk(sidx), output_state=out, output_state_indices=mk(oidx),
                  output_final_state=True, state_checkpoints=ck,
                  checkpoint_state_indices=mk(cidx if cidx else [0]),
                  checkpoint_cu_starts=mk(ck_start), prefix_lens=mk(c["prefix"]),
                  checkpoint_every_n_tokens=N, scale=c["scale"], options=options)
    torch.cuda.synchronize()
    res = ogdn.prefill(t["q"].cpu(), t["k"].cpu(), t["v"].cpu(), t["g"].cpu(), t["beta"].cpu(),
                       cu.cpu(), initial_state=RowView(rows_in), state_indices=sidx,
                       output_final_state=True, output_state_indices=oidx,
                       checkpoint_state_indices=cidx if cidx else [0],
                       checkpoint_cu_starts=list(ck_start), prefix_lens=c["prefix"],
                       checkpoint_every_n_tokens=N, scale=c["scale"], shared_pool=False,
                       state_dtype="bf16" if c["bf16"] else "fp32")
    if T:
        check_outputs(o, res.o)
    assert changed_rows(out0, out) == sorted(res.final)
    assert changed_rows(ck0, ck) == sorted(res.checkpoints)
    for r, s in res.final.items():
        check_state(out[r], s, f"final row {r}")
    for r, s in res.checkpoints.items():
        check_state(ck[r], s, f"checkpoint row {r}")
    print(f"general case {seed}: B={B} H={H}/{Hqk} N={N} prefix={c['prefix']} new={c['new']} "
          f"options={(c.get('waves'), c.get('split'))} finals={len(res.final)} "
          f"checkpoints={len(res.checkpoints)}")

DECODE_SHAPES = [dict(), dict(decode_waves=2), dict(decode_waves=4), dict(decode_waves=8),
                 dict(decode_waves=16), dict(decode_stream_per_cu=1), dict(decode_stream_per_cu=6),
                 dict(decode_stream_grid=3), dict(decode_stream_grid=37)]


@pytest.mark.parametrize("seed", seeds(12))
def test_random_paged_decode(seed):
    """Random paged decode batches (1-39 sequences, head layouts up to 16 on 8,
    contexts of 2 to 33,000 tokens, a random share opening a new page, decay
    from none to 3x) with a random kernel shape, slots derived or passed, on
    fp32 and bf16 pools: outputs, states, write set and untouched rows."""
    import torch

    import workloads
    from oracle import gdn as ogdn
    from tests.gpu_util import RowView, changed_rows, check_outputs, check_state, cuda, pool_rows_cpu
    from tests.test_gpu_small import lib, opts, state_dtype_of

    m = lib()
    rng = np.random.default_rng(9000 + seed)
    B = int(rng.integers(1, 40))
    Hqk, H = [(1, 1), (1, 2), (2, 4), (4, 4), (2, 8), (8, 16)][int(rng.integers(0, 6))]
    nps = int(rng.integers(0, B + 1))
    c = cuda(workloads.config2(num_seqs=B, qk_heads=Hqk, v_heads=H, num_pages=B * 34 + 8,
                               new_page_seqs=nps, seed=500 + seed, ctx_lo=2, ctx_hi=33000,
                               g_scale=float(rng.choice([0.0, 0.1, 1.0, 3.0]))))
    dec = c["decode"]
    shape = DECODE_SHAPES[int(rng.integers(0, len(DECODE_SHAPES)))]
    for pool in (c["pool"], c["pool"].to(torch.bfloat16)):
        rows_in = pool_rows_cpu(pool, dec["read_rows"])
        before = pool.clone()
        sl = (m.decode_slots(dec["page_indices"], dec["page_indptr"], dec["last_page_len"])
              if rng.random() < 0.5 else None)
        o = m.decode_paged(dec["q"], dec["k"], dec["v"], dec["g"], dec["beta"], pool,
                           dec["page_indices"], dec["page_indptr"], 1024, dec["last_page_len"],
                           slots=sl, options=opts(**shape))
        torch.cuda.synchronize()
        o_ref, writes, _ = ogdn.decode_paged(dec["q"].cpu(), dec["k"].cpu(), dec["v"].cpu(),
                                             dec["g"].cpu(), dec["beta"].cpu(), RowView(rows_in),
                                             dec["page_indices"].cpu(), dec["page_indptr"].cpu(),
                                             dec["last_page_len"].cpu(),
                                             state_dtype=state_dtype_of(pool))
        check_outputs(o, o_ref)
        assert changed_rows(before, pool) == sorted(writes)
        for r, s in writes.items():
            check_state(pool[r], s)
    print(f"decode case {seed}: B={B} H={H}/{Hqk} new-page={nps} {shape}")

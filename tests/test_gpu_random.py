"""Seeded random paged prefill batches against the oracle: batch sizes,
prefixes and new lengths (zeros, page and chunk boundaries included), page
sizes, head layouts, decay scales, state types, prefill tile widths and forced
sequence-parallel splits drawn per case.  The same parity bar as every other
GPU test: outputs and states within tolerance, page-write set and untouched
rows bit for bit."""

import os

import numpy as np
import pytest

from tests.test_gpu_small import check_paged_prefill, make_case

pytestmark = pytest.mark.gpu


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
    waves = str(int(rng.choice([8, 8, 4, 2])))
    split = rng.choice([None, None, "1", "2", "3"])
    return dict(prefix=prefix, new=new, ps=ps, H=H, Hqk=Hqk, g_scale=g_scale, bf16=bf16,
                waves=waves, split=split)


@pytest.mark.parametrize("seed", range(16))
def test_random_paged_prefill(seed):
    import torch
    c = draw_case(seed)
    env = {"GDN_PREFILL_TILE_WAVES": c["waves"]}
    if c["split"] is not None:
        env["GDN_PREFILL_SPLIT_CHUNKS"] = str(c["split"])
    old = {k: os.environ.get(k) for k in env}
    os.environ.update(env)
    try:
        pre, pool = make_case(c["prefix"], c["new"], ps=c["ps"], H=c["H"], Hqk=c["Hqk"],
                              seed=seed, g_scale=c["g_scale"])
        if c["bf16"]:
            pool = pool.to(torch.bfloat16)
        _, _, err = check_paged_prefill(pre, pool)
        print(f"case {seed}: {c} worst state rel {err:.2e}")
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v

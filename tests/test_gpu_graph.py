"""The calls under HIP graph capture: a hybrid layer (paged prefill and paged
decode on one pool, slots and workspace made beforehand) and the
sequence-parallel prefill are captured once and replayed several times, with
eager work and synchronizations between the replays; every replay must equal
the eager result bit for bit (outputs and the whole pool).  The library
launches kernels only (no memset, allocation or host synchronization inside a
call), which is what makes the calls capturable."""


import pytest
import torch

import workloads
from tests.gpu_util import cuda

pytestmark = pytest.mark.gpu
DEV = "cuda"


def lib():
    import paged_recurrent_state_amd as m
    m.load()
    return m


def bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def replay_and_check(graph, reset, outputs, expected, names, replays=3):
    side = torch.randn(512, 512, device=DEV)
    for i in range(replays):
        reset()
        side = side @ side.T / 512.0  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want, name in zip(outputs, expected, names):
            assert torch.equal(bits(got), bits(want)), f"replay {i}: {name} differs"


def test_graph_hybrid_layer():
    m = lib()
    c = workloads.config4(device=DEV, heads=4, num_prefill=3, prefill_pad=1, num_decode=8,
                          decode_pad=2, page_size=128, num_pages=512, new_lo=64, new_hi=700,
                          hit_hi=1024, ctx_lo=200, ctx_hi=2000)
    ps = c["page_size"]
    pre, dec = c["layers"][0]["prefill"], c["layers"][0]["decode"]
    T, B = pre["q"].shape[0], pre["last_page_len"].shape[0]
    pool0 = c["pool"]
    sl_p = m.prefill_slots(pre["cu_seqlens"], pre["page_indices"], pre["page_indptr"],
                           pre["last_page_len"], ps)
    sl_d = m.decode_slots(dec["page_indices"], dec["page_indptr"], dec["last_page_len"])
    ws = torch.empty(m.prefill_workspace_size(T, B, c["H"], c["Hqk"]), dtype=torch.uint8,
                     device=DEV)

    def layer(pool, o_pre, o_dec):
        m.prefill_paged(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], pre["cu_seqlens"],
                        pool, pre["page_indices"], pre["page_indptr"], ps, pre["last_page_len"],
                        slots=sl_p, workspace=ws, out=o_pre)
        m.decode_paged(dec["q"], dec["k"], dec["v"], dec["g"], dec["beta"], pool,
                       dec["page_indices"], dec["page_indptr"], ps, dec["last_page_len"],
                       slots=sl_d, out=o_dec)

    pool_e = pool0.clone()
    o_pre_e = torch.empty(T, c["H"], 128, dtype=torch.bfloat16, device=DEV)
    o_dec_e = torch.empty(dec["q"].shape[0], c["H"], 128, dtype=torch.bfloat16, device=DEV)
    layer(pool_e, o_pre_e, o_dec_e)
    torch.cuda.synchronize()

    pool_g = pool0.clone()
    o_pre_g, o_dec_g = torch.empty_like(o_pre_e), torch.empty_like(o_dec_e)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer(pool_g, o_pre_g, o_dec_g)
    replay_and_check(g, lambda: pool_g.copy_(pool0), (o_pre_g, o_dec_g, pool_g),
                     (o_pre_e, o_dec_e, pool_e), ("o prefill", "o decode", "pool"))


@pytest.mark.parametrize("split,total,splits", [(3, 1000, (131, 400, 640)),
                                                (0, 3000, (131, 400, 2640))])
def test_graph_sequence_parallel_prefill(split, total, splits):
    """A sequence-parallel prefill captured and replayed: forced segments of 3
    chunks, and the plan the device picks from the lengths (a 2240-token
    middle piece)."""
    m = lib()
    o3 = m.Options(prefill_split_chunks=split)
    c = cuda(workloads.config3(heads=2, total=total, splits=splits, every_n=128,
                               num_rows=3, g_scale=0.1))
    call = c["calls"][2]  # a middle piece: reads and writes the slot, checkpoints inside
    T = call["q"].shape[0]
    ws = torch.empty(m.prefill_workspace_size(T, 1, 2, 2, options=o3), dtype=torch.uint8,
                     device=DEV)
    ckpt0 = workloads.nan_pool(total // 128, 2, 128, 128, device=DEV)
    slot0 = c["pool"]
    slot0.zero_()
    slot0[c["slot"]].normal_(0, 0.05)

    def run(slot, ckpt, o):
        m.prefill(call["q"], call["k"], call["v"], call["g"], call["beta"],
                  call["cu_seqlens"], initial_state=slot,
                  state_indices=call["state_indices"], output_state=slot,
                  output_state_indices=call["output_state_indices"],
                  output_final_state=True, state_checkpoints=ckpt,
                  checkpoint_state_indices=c["checkpoint_state_indices"],
                  checkpoint_cu_starts=call["checkpoint_cu_starts"],
                  prefix_lens=call["prefix_lens"], checkpoint_every_n_tokens=128,
                  workspace=ws, out=o, options=o3)

    slot_e, ckpt_e = slot0.clone(), ckpt0.clone()
    o_e = torch.empty(T, 2, 128, dtype=torch.bfloat16, device=DEV)
    run(slot_e, ckpt_e, o_e)
    torch.cuda.synchronize()

    slot_g, ckpt_g = slot0.clone(), ckpt0.clone()
    o_g = torch.empty_like(o_e)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(slot_g, ckpt_g, o_g)

    def reset():
        slot_g.copy_(slot0)
        ckpt_g.copy_(ckpt0)

    replay_and_check(g, reset, (o_g, ckpt_g, slot_g), (o_e, ckpt_e, slot_e),
                     ("o", "checkpoints", "slot rows"))

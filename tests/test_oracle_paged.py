"""Pins for the oracle's paged prefill/decode semantics (CPU only)."""

import numpy as np
import pytest

from oracle import gdn, slots


def rand_tokens(rng, T, H, K, V, Hqk=None):
    Hqk = Hqk or H
    q = rng.standard_normal((T, Hqk, K))
    k = rng.standard_normal((T, Hqk, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, V))
    g = -np.log1p(np.exp(rng.standard_normal((T, H)))) / 10
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, g, beta


def page_table(total, ps, pages):
    n = (total + ps - 1) // ps
    return pages[:n], [0, n], [total - (n - 1) * ps]


@pytest.mark.parametrize("ps", [64, 128])
def test_split_invariance_bit_exact(ps):
    """Prefill split at any token and resumed from the written page equals
    the unsplit run, bit for bit, on an fp64 shadow pool."""
    rng = np.random.default_rng(ps)
    H, K, V = 2, 4, 4
    T = 300
    q, k, v, g, beta = rand_tokens(rng, T, H, K, V)
    pages = list(rng.permutation(32))
    pool0 = np.full((32, H, V, K), np.nan)
    idx, ptr, lpl = page_table(T, ps, pages)
    o_full, w_full, _ = gdn.prefill_paged(q, k, v, g, beta, [0, T], pool0, idx, ptr, lpl, ps)
    full_pool = gdn.apply_writes(pool0, w_full)
    for cut in list(range(1, 70)) + [127, 128, 129, 191, 250, 299]:
        pool = pool0.copy()
        idx, ptr, lpl = page_table(cut, ps, pages)
        o1, w1, _ = gdn.prefill_paged(q[:cut], k[:cut], v[:cut], g[:cut], beta[:cut],
                                      [0, cut], pool, idx, ptr, lpl, ps)
        pool = gdn.apply_writes(pool, w1)
        idx, ptr, lpl = page_table(T, ps, pages)
        o2, w2, _ = gdn.prefill_paged(q[cut:], k[cut:], v[cut:], g[cut:], beta[cut:],
                                      [0, T - cut], pool, idx, ptr, lpl, ps)
        pool = gdn.apply_writes(pool, w2)
        assert np.array_equal(np.concatenate([o1, o2]), o_full)
        # every page the unsplit run wrote holds the same bits
        for r in w_full:
            assert np.array_equal(pool[r], full_pool[r])


def test_decode_equals_one_token_prefill():
    rng = np.random.default_rng(11)
    H, Hqk, K, V, ps = 4, 2, 4, 4, 64
    ctxs = [65, 64, 130, 2, 129]          # 65 and 129 open a new page
    pages = [[0, 1], [2], [3, 4, 5], [6], [7, 8, 9]]
    idx = sum(pages, [])
    ptr = np.cumsum([0] + [len(p) for p in pages]).tolist()
    lpl = [c - (len(p) - 1) * ps for c, p in zip(ctxs, pages)]
    pool = np.full((10, H, V, K), np.nan)
    for r in slots.decode_slots(idx, ptr, lpl)["initial_state_indices"]:
        pool[r] = rng.standard_normal((H, V, K))
    q, k, v, g, beta = rand_tokens(rng, len(ctxs), H, K, V, Hqk=Hqk)
    o_d, w_d, sl_d = gdn.decode_paged(q, k, v, g, beta, pool, idx, ptr, lpl)
    o_p, w_p, sl_p = gdn.prefill_paged(q, k, v, g, beta, list(range(len(ctxs) + 1)), pool,
                                       idx, ptr, lpl, ps)
    assert sl_d["initial_state_indices"] == sl_p["state_indices"]
    assert sl_d["output_state_indices"] == sl_p["output_state_indices"]
    assert sl_d["initial_state_indices"][0] == 0 and sl_d["output_state_indices"][0] == 1
    assert np.array_equal(o_d, o_p)
    assert sorted(w_d) == sorted(w_p)
    for r in w_d:
        assert np.array_equal(w_d[r], w_p[r])


def test_checkpoint_buffer_with_skipped_rows():
    """Slot-argument prefill: checkpoints at absolute multiples of N into a
    separate buffer, -1 rows skipped; the stored states equal the state
    after that token of the same run."""
    rng = np.random.default_rng(12)
    H, K, V, N = 1, 4, 4, 64
    T = 500
    q, k, v, g, beta = rand_tokens(rng, T, H, K, V)
    bounds = [0, 101, 260, 383, 500]
    n_ck = T // N
    ck_rows = [c if c % 2 == 0 else -1 for c in range(n_ck)]
    slot = np.full((1, H, V, K), np.nan)
    ckpt = {}
    outs = []
    for a, b in zip(bounds, bounds[1:]):
        res = gdn.prefill(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], [0, b - a],
                          initial_state=slot, state_indices=[-1 if a == 0 else 0],
                          output_final_state=True, output_state_indices=[0],
                          checkpoint_state_indices=ck_rows, checkpoint_cu_starts=[a // N],
                          prefix_lens=[a], checkpoint_every_n_tokens=N)
        slot = slot.copy()
        slot[0] = res.final[0]
        ckpt.update(res.checkpoints)
        outs.append(res.o)
    assert sorted(ckpt) == [c for c in range(n_ck) if c % 2 == 0]
    # reference: one unsplit run, state after token (c+1)*N
    S = np.zeros((H, V, K))
    for t in range(T):
        S, _ = gdn.gdn_token(S, q[t], k[t], v[t], g[t], beta[t], 0.5)
        if (t + 1) % N == 0 and ((t + 1) // N - 1) % 2 == 0:
            assert np.array_equal(ckpt[(t + 1) // N - 1], S)
    assert np.array_equal(slot[0], S)


def test_duplicate_final_and_boundary_store_agree():
    # p + L a multiple of the page size: the last boundary page is the last
    # page, and both stores carry the same state.
    rng = np.random.default_rng(13)
    H, K, V, ps = 1, 4, 4, 64
    q, k, v, g, beta = rand_tokens(rng, 100, H, K, V)
    pool = np.full((4, H, V, K), np.nan)
    pool[0] = rng.standard_normal((H, V, K))
    # 128 tokens after the call, 100 new: prefix 28 ends inside page 0, which
    # is read, then written in place at the boundary 64; page 1 ends at 128.
    o, w, sl = gdn.prefill_paged(q, k, v, g, beta, [0, 100], pool, [0, 1], [0, 2], [64], ps)
    assert sl["prefix_lens"] == [28] and sl["state_indices"] == [0]
    assert sorted(w) == [0, 1]
    assert np.isfinite(w[0]).all() and np.isfinite(w[1]).all()
    res = gdn.prefill(q, k, v, g, beta, [0, 100], initial_state=pool, state_indices=[0],
                      output_final_state=True, output_state_indices=[1],
                      checkpoint_state_indices=[0, 1], checkpoint_cu_starts=[0],
                      prefix_lens=[28], checkpoint_every_n_tokens=ps)
    assert res.checkpoints[1].tobytes() == res.final[1].tobytes()


def test_cross_sequence_hazard_rejected():
    rng = np.random.default_rng(14)
    q, k, v, g, beta = rand_tokens(rng, 4, 1, 2, 2)
    pool = np.zeros((4, 1, 2, 2))
    with pytest.raises(ValueError):
        gdn.prefill(q, k, v, g, beta, [0, 2, 4], initial_state=pool, state_indices=[0, 1],
                    output_final_state=True, output_state_indices=[1, 2])


def test_zero_length_prefill_leaves_pool():
    rng = np.random.default_rng(15)
    q, k, v, g, beta = rand_tokens(rng, 0, 1, 2, 2)
    pool = rng.standard_normal((3, 1, 2, 2))
    o, w, sl = gdn.prefill_paged(q, k, v, g, beta, [0, 0], pool, [2], [0, 1], [5], 64)
    assert w == {} and o.shape == (0, 1, 2)
    assert sl["output_state_indices"] == [-1]

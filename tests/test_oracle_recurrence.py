"""Pins for the oracle's recurrence (CPU only).

The oracle applies the gated delta rule one token at a time as a rank-1
update.  These tests pin it to independent facts: the explicit matrix-product
closed form, special cases with exact answers, linearity in the initial state,
split invariance through the pool, and the head mapping checked head by head.
"""

import math

import numpy as np
import pytest

from oracle import gdn


def rand_inputs(rng, T, H, K, V, Hqk=None, low_decay=False):
    Hqk = Hqk or H
    q = rng.standard_normal((T, Hqk, K))
    k = rng.standard_normal((T, Hqk, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, V))
    g = -np.log1p(np.exp(rng.standard_normal((T, H))))
    if low_decay:
        g = g / 10
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, g, beta


def closed_form(S0, q, k, v, g, beta, scale):
    """S_T = S_0 A_1...A_T + sum_t beta_t v_t k_t^T A_{t+1}...A_T with
    A_t = alpha_t (I - beta_t k_t k_t^T); o_t = scale * S_t q_t.  One head."""
    T, K = k.shape
    A = [math.exp(g[t]) * (np.eye(K) - beta[t] * np.outer(k[t], k[t])) for t in range(T)]
    outs = []
    S_t = None
    for t_end in range(1, T + 1):
        prod = np.eye(K)
        for t in range(t_end):
            prod = prod @ A[t]
        S_t = S0 @ prod
        for t in range(t_end):
            tail = np.eye(K)
            for s in range(t + 1, t_end):
                tail = tail @ A[s]
            S_t = S_t + beta[t] * np.outer(v[t], k[t]) @ tail
        outs.append(scale * S_t @ q[t_end - 1])
    return S_t, np.array(outs)


@pytest.mark.parametrize("K,V,T", [(4, 4, 6), (8, 4, 8), (4, 8, 5)])
def test_closed_form_product(K, V, T):
    rng = np.random.default_rng(K * 100 + V * 10 + T)
    q, k, v, g, beta = rand_inputs(rng, T, 1, K, V)
    S0 = rng.standard_normal((1, V, K))
    res = gdn.prefill(q, k, v, g, beta, [0, T], initial_state=S0, state_indices=[0],
                      output_final_state=True, output_state_indices=[0])
    scale = 1 / math.sqrt(K)
    S_ref, o_ref = closed_form(S0[0], q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], scale)
    np.testing.assert_allclose(res.final[0][0], S_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(res.o[:, 0], o_ref, rtol=1e-12, atol=1e-13)


def test_beta0_g0_leaves_state_unchanged():
    rng = np.random.default_rng(1)
    T, H, K, V = 9, 3, 16, 16
    q, k, v, _, _ = rand_inputs(rng, T, H, K, V)
    S0 = rng.standard_normal((1, H, V, K))
    res = gdn.prefill(q, k, v, np.zeros((T, H)), np.zeros((T, H)), [0, T], initial_state=S0,
                      state_indices=[0], output_final_state=True, output_state_indices=[0])
    assert np.array_equal(res.final[0], S0[0])
    # and the output is then the plain read-out of the unchanged state
    np.testing.assert_allclose(res.o[3], np.einsum("hvk,hk->hv", S0[0], q[3]) / math.sqrt(K),
                               rtol=1e-13)


def test_unit_key_writes_value_exactly():
    # g = 0, beta = 1, k = e_i: S k = v after the update (S[:, i] + (v - S[:, i]),
    # so up to one rounding of each term), other columns untouched bit for bit.
    rng = np.random.default_rng(2)
    H, K, V = 2, 8, 8
    S0 = rng.standard_normal((1, H, V, K))
    for i in range(K):
        k = np.zeros((1, H, K))
        k[0, :, i] = 1.0
        q = rng.standard_normal((1, H, K))
        v = rng.standard_normal((1, H, V))
        res = gdn.prefill(q, k, v, np.zeros((1, H)), np.ones((1, H)), [0, 1],
                          initial_state=S0, state_indices=[0], output_final_state=True,
                          output_state_indices=[0])
        bound = 2.0 ** -52 * (np.abs(v[0]) + 2 * np.abs(S0[0][:, :, i]))
        assert (np.abs(res.final[0][:, :, i] - v[0]) <= bound).all()
        # columns other than i keep their values
        others = [j for j in range(K) if j != i]
        assert np.array_equal(res.final[0][:, :, others], S0[0][:, :, others])


def test_beta0_is_pure_decay():
    rng = np.random.default_rng(3)
    T, H, K, V = 20, 2, 8, 8
    q, k, v, g, _ = rand_inputs(rng, T, H, K, V)
    S0 = rng.standard_normal((1, H, V, K))
    res = gdn.prefill(q, k, v, g, np.zeros((T, H)), [0, T], initial_state=S0,
                      state_indices=[0], output_final_state=True, output_state_indices=[0])
    expect = np.exp(g.sum(0))[:, None, None] * S0[0]
    np.testing.assert_allclose(res.final[0], expect, rtol=1e-12)


def test_full_decay_resets_state():
    # g -> -inf: alpha = 0, the state becomes beta v k^T whatever it held.
    rng = np.random.default_rng(4)
    H, K, V = 2, 8, 8
    q, k, v, _, beta = rand_inputs(rng, 1, H, K, V)
    S0 = rng.standard_normal((1, H, V, K)) * 1e3
    res = gdn.prefill(q, k, v, np.full((1, H), -1e4), beta, [0, 1], initial_state=S0,
                      state_indices=[0], output_final_state=True, output_state_indices=[0])
    expect = beta[0][:, None, None] * v[0][:, :, None] * k[0][:, None, :]
    np.testing.assert_allclose(res.final[0], expect, rtol=1e-15, atol=0)


def test_linearity_in_initial_state():
    rng = np.random.default_rng(5)
    T, K, V = 7, 6, 5
    q, k, v, g, beta = rand_inputs(rng, T, 1, K, V)
    S0 = rng.standard_normal((1, 1, V, K))
    zero = np.zeros_like(S0)
    kw = dict(state_indices=[0], output_final_state=True, output_state_indices=[0])
    a = gdn.prefill(q, k, v, g, beta, [0, T], initial_state=S0, **kw).final[0][0]
    b = gdn.prefill(q, k, v, g, beta, [0, T], initial_state=zero, **kw).final[0][0]
    prod = np.eye(K)
    for t in range(T):
        prod = prod @ (math.exp(g[t, 0]) * (np.eye(K) - beta[t, 0] * np.outer(k[t, 0], k[t, 0])))
    np.testing.assert_allclose(a - b, S0[0, 0] @ prod, rtol=1e-11, atol=1e-13)


def test_zero_start_never_reads():
    # read row -1: a NaN-filled initial buffer is never touched
    rng = np.random.default_rng(6)
    T, H, K, V = 5, 2, 4, 4
    q, k, v, g, beta = rand_inputs(rng, T, H, K, V)
    init = np.full((3, H, V, K), np.nan)
    res = gdn.prefill(q, k, v, g, beta, [0, T], initial_state=init, state_indices=[-1],
                      output_final_state=True, output_state_indices=[2])
    ref = gdn.prefill(q, k, v, g, beta, [0, T], output_final_state=True,
                      initial_state=np.zeros((1, H, V, K)), state_indices=[0],
                      output_state_indices=[0])
    assert np.isfinite(res.o).all()
    assert np.array_equal(res.final[2], ref.final[0])


def test_minus_one_write_row_and_zero_length():
    rng = np.random.default_rng(7)
    H, K, V = 1, 4, 4
    q, k, v, g, beta = rand_inputs(rng, 6, H, K, V)
    init = rng.standard_normal((4, H, V, K))
    # seq0 has 0 tokens, seq1 writes -1, seq2 writes row 3
    res = gdn.prefill(q, k, v, g, beta, [0, 0, 3, 6], initial_state=init,
                      state_indices=[0, 1, 2], output_final_state=True,
                      output_state_indices=[0, -1, 3])
    assert sorted(res.final) == [3]
    assert 0 not in res.reads


def test_gqa_head_mapping_head_by_head():
    rng = np.random.default_rng(8)
    T, H, Hqk, K, V = 6, 4, 2, 4, 4
    q, k, v, g, beta = rand_inputs(rng, T, H, K, V, Hqk=Hqk)
    res = gdn.prefill(q, k, v, g, beta, [0, T], output_final_state=True,
                      initial_state=np.zeros((1, H, V, K)), state_indices=[0],
                      output_state_indices=[0])
    for h in range(H):
        hq = h // (H // Hqk)
        one = gdn.prefill(q[:, [hq]], k[:, [hq]], v[:, [h]], g[:, [h]], beta[:, [h]], [0, T],
                          output_final_state=True, initial_state=np.zeros((1, 1, V, K)),
                          state_indices=[0], output_state_indices=[0])
        assert np.array_equal(res.final[0][h], one.final[0][0])
        assert np.array_equal(res.o[:, h], one.o[:, 0])


# ---- bf16 state buffers: stored states rounded to bf16, arithmetic unchanged

def test_round_bf16_matches_torch_and_ties_to_even():
    import torch
    rng = np.random.default_rng(20)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0, -3.5, 65504.0, 1e-40]])
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(gdn.round_bf16(x), want)
    # exact ties between two bf16 values go to the even one (8-bit mantissa)
    u = 2.0 ** -7
    assert gdn.round_bf16(1 + u / 2) == 1.0            # tie: 1.0 (even) not 1 + u
    assert gdn.round_bf16(1 + 3 * u / 2) == 1 + 2 * u  # tie: 1 + 2u (even) not 1 + u
    assert gdn.round_bf16(1 + u / 2 + 2.0 ** -20) == 1 + u  # just above the tie


def test_bf16_states_identity_update_keeps_the_row():
    # g = 0, beta = 0: the state passes through unchanged, so a bf16 row read
    # from the pool is stored back bit for bit
    rng = np.random.default_rng(21)
    T, H, K, V = 5, 2, 16, 16
    q, k, v, _, _ = rand_inputs(rng, T, H, K, V)
    S0 = gdn.round_bf16(rng.standard_normal((1, H, V, K)))
    res = gdn.prefill(q, k, v, np.zeros((T, H)), np.zeros((T, H)), [0, T], initial_state=S0,
                      state_indices=[0], output_final_state=True, output_state_indices=[0],
                      state_dtype="bf16")
    assert np.array_equal(res.final[0], S0[0])


def test_bf16_states_rounded_only_where_stored():
    # one token, g = 0, beta = 1, unit key e_i: column i of the new state is v
    # (delta rule), stored to within half a bf16 ulp; the output uses the
    # unrounded state, so it matches the fp32-buffer run exactly
    rng = np.random.default_rng(22)
    H, K, V = 2, 8, 8
    S0 = gdn.round_bf16(rng.standard_normal((1, H, V, K)))
    k = np.zeros((1, H, K)); k[0, :, 3] = 1.0
    q = rng.standard_normal((1, H, K)); v = rng.standard_normal((1, H, V))
    kw = dict(initial_state=S0, state_indices=[0], output_final_state=True, output_state_indices=[0])
    r16 = gdn.prefill(q, k, v, np.zeros((1, H)), np.ones((1, H)), [0, 1], state_dtype="bf16", **kw)
    r32 = gdn.prefill(q, k, v, np.zeros((1, H)), np.ones((1, H)), [0, 1], **kw)
    assert np.array_equal(r16.o, r32.o)
    col = r16.final[0][:, :, 3]
    assert (np.abs(col - v[0]) <= 2.0 ** -8 * np.abs(v[0]) * (1 + 1e-6)).all()  # half an ulp
    assert np.array_equal(r16.final[0], gdn.round_bf16(r32.final[0]))
    with pytest.raises(ValueError):
        gdn.prefill(q, k, v, None, None, [0, 1], state_dtype="fp16", **kw)

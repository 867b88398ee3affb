"""Pins of the serving-style oracle (CPU): packed variable-length prefill and pooled states.

The packed prefill is, by definition, the mixer run on each sequence alone (continuous batching changes how
prompts are laid out, not what is computed).  Each pin checks a property that a plausible mistake in the
packing breaks: a state leaking from one sequence into the next, offsets read off by one, a conv window
reaching back across a boundary, an empty sequence clobbering its state, a slot indirection applied to the
wrong row, or the states of a padding entry being stored.
"""

import math

import numpy as np
import pytest

import oracle


def _weights(rng, C=6, N=4, R=3, K=4):
    return {
        "conv_w": rng.uniform(-0.5, 0.5, (C, K)),
        "conv_b": rng.normal(0, 0.1, C),
        "x_proj_w": rng.normal(0, 1 / math.sqrt(C), (R + 2 * N, C)),
        "dt_norm_w": rng.uniform(0.5, 1.5, R),
        "b_norm_w": rng.uniform(0.5, 1.5, N),
        "c_norm_w": rng.uniform(0.5, 1.5, N),
        "dt_proj_w": rng.normal(0, 1 / math.sqrt(R), (C, R)),
        "dt_proj_b": np.log(np.expm1(rng.uniform(1e-3, 0.1, C))),
        "A_log": np.log(rng.uniform(0.5, 8.0, (C, N))),
        "D": rng.normal(1.0, 0.3, C),
    }


R_, N_ = 3, 4


def _case(seed, lens, C=6, rows=None):
    rng = np.random.default_rng(seed)
    w = _weights(rng, C)
    T = sum(lens)
    x = rng.normal(0, 1, (T, C))
    z = rng.normal(0, 1, (T, C))
    nrow = len(lens) if rows is None else rows
    cs = rng.normal(0, 1, (nrow, C, 3))
    h0 = rng.normal(0, 0.3, (nrow, C, N_))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(int)
    return w, x, z, cu, cs, h0


def test_equal_lengths_match_the_batched_prefill():
    # packing B sequences of length L back to back is the [B, L] batch of the plain prefill
    B, L = 3, 7
    w, x, z, cu, cs, h0 = _case(1, [L] * B)
    out, c, h = oracle.mixer_prefill_varlen(x, z, cu, w, R_, N_, conv_state=cs, ssm_state=h0)
    ro, rc, rh = oracle.mixer_prefill(x.reshape(B, L, -1), z.reshape(B, L, -1), w, R_, N_, conv_state=cs,
                                      ssm_state=h0)
    np.testing.assert_allclose(out, ro.reshape(B * L, -1), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(h, rh, rtol=1e-13, atol=1e-15)
    assert np.array_equal(c, rc)


def test_sequences_do_not_see_each_other():
    # changing every token of one sequence changes nothing of its neighbours: no state and no conv window
    # crosses a boundary (the conv window of a sequence's first tokens reads its own conv state)
    lens = [5, 2, 9]
    w, x, z, cu, cs, h0 = _case(2, lens)
    a = oracle.mixer_prefill_varlen(x, z, cu, w, R_, N_, conv_state=cs, ssm_state=h0)
    x2, z2 = x.copy(), z.copy()
    x2[cu[1]:cu[2]] += 3.0
    z2[cu[1]:cu[2]] -= 1.0
    b = oracle.mixer_prefill_varlen(x2, z2, cu, w, R_, N_, conv_state=cs, ssm_state=h0)
    for s in (0, 2):
        assert np.array_equal(a[0][cu[s]:cu[s + 1]], b[0][cu[s]:cu[s + 1]])
        assert np.array_equal(a[1][s], b[1][s]) and np.array_equal(a[2][s], b[2][s])
    assert np.abs(a[0][cu[1]:cu[2]] - b[0][cu[1]:cu[2]]).max() > 1e-3
    # and each sequence equals its own prefill
    for s in range(3):
        o, c, h = oracle.mixer_prefill(x[None, cu[s]:cu[s + 1]], z[None, cu[s]:cu[s + 1]], w, R_, N_,
                                       conv_state=cs[s:s + 1], ssm_state=h0[s:s + 1])
        assert np.array_equal(a[0][cu[s]:cu[s + 1]], o[0])
        assert np.array_equal(a[1][s], c[0]) and np.array_equal(a[2][s], h[0])


def test_empty_and_short_sequences_carry_their_states():
    # an empty sequence leaves both states as they were; a 1-token sequence shifts its conv state by one
    # (two old entries and the token, oldest first)
    lens = [4, 0, 1, 0]
    w, x, z, cu, cs, h0 = _case(3, lens)
    out, c, h = oracle.mixer_prefill_varlen(x, z, cu, w, R_, N_, conv_state=cs, ssm_state=h0)
    for s in (1, 3):
        assert np.array_equal(c[s], cs[s]) and np.array_equal(h[s], h0[s])
    assert np.array_equal(c[2], np.concatenate([cs[2][:, 1:], x[cu[2]][:, None]], axis=1))
    assert out.shape == x.shape


def test_state_pool_rows_and_padding_entries():
    # states in a pool: sequence s reads and writes row slots[s]; an entry outside the pool runs from zero
    # states and stores nothing; rows no slot names keep their contents
    lens = [3, 5, 2]
    slots = [4, -1, 1]
    w, x, z, cu, cs, h0 = _case(4, lens, rows=6)
    out, c, h = oracle.mixer_prefill_varlen(x, z, cu, w, R_, N_, conv_state=cs, ssm_state=h0, slots=slots)
    for r in (0, 2, 3, 5):
        assert np.array_equal(c[r], cs[r]) and np.array_equal(h[r], h0[r])
    o0, c0, hh0 = oracle.mixer_prefill(x[None, 0:3], z[None, 0:3], w, R_, N_, conv_state=cs[4:5],
                                       ssm_state=h0[4:5])
    assert np.array_equal(out[0:3], o0[0]) and np.array_equal(c[4], c0[0]) and np.array_equal(h[4], hh0[0])
    o1, _, _ = oracle.mixer_prefill(x[None, 3:8], z[None, 3:8], w, R_, N_)          # zero states
    assert np.array_equal(out[3:8], o1[0])
    o2, _, hh2 = oracle.mixer_prefill(x[None, 8:10], z[None, 8:10], w, R_, N_, conv_state=cs[1:2],
                                      ssm_state=h0[1:2])
    assert np.array_equal(out[8:10], o2[0]) and np.array_equal(h[1], hh2[0])


def test_chunked_prefill_through_the_pool_equals_one_call():
    # a prompt prefilled in two chunks, its states left in a pool row between them, gives the same output
    # and states as one call over the whole prompt (the recurrence composes)
    w, x, z, cu, cs, h0 = _case(5, [11], rows=3)
    full, cf, hf = oracle.mixer_prefill_varlen(x, z, [0, 11], w, R_, N_, conv_state=cs, ssm_state=h0, slots=[2])
    a, c1, h1 = oracle.mixer_prefill_varlen(x[:6], z[:6], [0, 6], w, R_, N_, conv_state=cs, ssm_state=h0,
                                            slots=[2])
    b, c2, h2 = oracle.mixer_prefill_varlen(x[6:], z[6:], [0, 5], w, R_, N_, conv_state=c1, ssm_state=h1,
                                            slots=[2])
    np.testing.assert_allclose(np.concatenate([a, b]), full, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(h2, hf, rtol=1e-12, atol=1e-14)
    assert np.array_equal(c2, cf)


def test_decode_slots_equal_decode_on_gathered_states():
    rng = np.random.default_rng(6)
    w = _weights(rng)
    pool_c = rng.normal(0, 1, (5, 6, 3))
    pool_h = rng.normal(0, 0.3, (5, 6, N_))
    slots = [3, 0, 7]
    x = rng.normal(0, 1, (3, 6))
    z = rng.normal(0, 1, (3, 6))
    out, c, h = oracle.mixer_decode_step_slots(x, z, w, R_, N_, pool_c, pool_h, slots)
    gc = np.stack([pool_c[3], pool_c[0], np.zeros((6, 3))])
    gh = np.stack([pool_h[3], pool_h[0], np.zeros((6, N_))])
    ro, rc, rh = oracle.mixer_decode_step(x, z, w, R_, N_, gc, gh)
    assert np.array_equal(out, ro)
    assert np.array_equal(c[3], rc[0]) and np.array_equal(c[0], rc[1])
    assert np.array_equal(h[3], rh[0]) and np.array_equal(h[0], rh[1])
    for r in (1, 2, 4):
        assert np.array_equal(c[r], pool_c[r]) and np.array_equal(h[r], pool_h[r])


@pytest.mark.parametrize("seed", [7])
def test_layer_varlen_is_the_layer_per_sequence(seed):
    rng = np.random.default_rng(seed)
    w = _weights(rng)
    C, Dm = 6, 5
    lw = {"norm_w": rng.uniform(0.5, 1.5, Dm), "in_proj_w": rng.normal(0, 1 / math.sqrt(Dm), (2 * C, Dm)),
          "out_proj_w": rng.normal(0, 1 / math.sqrt(C), (Dm, C))}
    lens = [4, 0, 6]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = rng.normal(0, 1, (10, Dm))
    out, c, h = oracle.layer_prefill_varlen(x, cu, lw, w, R_, N_)
    for s in (0, 2):
        o, cc, hh = oracle.layer_prefill(x[None, cu[s]:cu[s + 1]], lw, w, R_, N_)
        assert np.array_equal(out[cu[s]:cu[s + 1]], o[0]) and np.array_equal(h[s], hh[0])
    assert np.array_equal(h[1], np.zeros_like(h[1])) and np.array_equal(c[1], np.zeros_like(c[1]))

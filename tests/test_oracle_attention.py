"""Pins for the fp64 attention oracle (CPU only).

Each check ties ``oracle.attention`` to something other than itself: hand
values of the definition, closed forms, invariants of softmax, a library
routine, and the pure-Python brute force.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention, brute

RNG = np.random.default_rng(1234)


def test_hand_example_d1():
    # q = 1, k = (0, ln 2, ln 3): exp scores (1, 2, 3) -> P = (1, 2, 3) / 6;
    # V = (6, 0, 0): O = 1; LSE = ln 6.
    q = np.array([1.0]).reshape(1, 1, 1, 1)
    k = np.array([0.0, math.log(2), math.log(3)]).reshape(1, 3, 1, 1)
    v = np.array([6.0, 0.0, 0.0]).reshape(1, 3, 1, 1)
    o, lse = attention(q, k, v, 1.0)
    assert o[0, 0, 0, 0] == pytest.approx(1.0, abs=1e-15)
    assert lse[0, 0, 0] == pytest.approx(math.log(6.0), abs=1e-15)


def test_hand_example_d2_in_second_head_and_batch():
    # q = (1, 0) only sees the first key coordinate: scores (0, ln 2),
    # P = (1/3, 2/3); V rows (3, 1), (0, 4) -> O = (1, 3); LSE = ln 3.
    # Placed at b=1, h=1 of a random [2, 1, 2, 2] problem so that a swapped
    # axis or a transposed operand moves the answer.
    q = RNG.standard_normal((2, 1, 2, 2))
    k = RNG.standard_normal((2, 2, 2, 2))
    v = RNG.standard_normal((2, 2, 2, 2))
    q[1, 0, 1] = [1.0, 0.0]
    k[1, :, 1] = [[0.0, 5.0], [math.log(2), -3.0]]
    v[1, :, 1] = [[3.0, 1.0], [0.0, 4.0]]
    o, lse = attention(q, k, v, 1.0)
    np.testing.assert_allclose(o[1, 0, 1], [1.0, 3.0], atol=1e-14)
    assert lse[1, 1, 0] == pytest.approx(math.log(3.0), abs=1e-14)


@pytest.mark.parametrize("B,Sq,Skv,H,D", [(1, 1, 1, 1, 1), (2, 3, 5, 2, 4), (1, 4, 7, 3, 3)])
def test_matches_brute_force(B, Sq, Skv, H, D):
    q = RNG.standard_normal((B, Sq, H, D))
    k = RNG.standard_normal((B, Skv, H, D))
    v = RNG.standard_normal((B, Skv, H, D))
    scale = 1.0 / math.sqrt(D)
    o, lse = attention(q, k, v, scale)
    ob, lb = brute.attention(q.tolist(), k.tolist(), v.tolist(), scale)
    np.testing.assert_allclose(o, np.array(ob), atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, np.array(lb), atol=1e-12, rtol=0)


def test_matches_torch_float64_softmax():
    B, Sq, Skv, H, D = 2, 9, 13, 3, 8
    q = RNG.standard_normal((B, Sq, H, D))
    k = RNG.standard_normal((B, Skv, H, D))
    v = RNG.standard_normal((B, Skv, H, D))
    scale = 0.37
    o, lse = attention(q, k, v, scale)
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
    s = scale * tq @ tk.transpose(-1, -2)
    ref_o = (torch.softmax(s, dim=-1) @ tv).permute(0, 2, 1, 3).numpy()
    ref_lse = torch.logsumexp(s, dim=-1).numpy()
    np.testing.assert_allclose(o, ref_o, atol=1e-13, rtol=0)
    np.testing.assert_allclose(lse, ref_lse, atol=1e-13, rtol=0)


def test_q_zero_gives_mean_of_v_and_log_skv():
    B, Sq, Skv, H, D = 1, 4, 37, 2, 16
    q = np.zeros((B, Sq, H, D))
    k = RNG.standard_normal((B, Skv, H, D))
    v = RNG.standard_normal((B, Skv, H, D))
    o, lse = attention(q, k, v, 0.25)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=1, keepdims=True), o.shape), atol=1e-14)
    np.testing.assert_allclose(lse, math.log(Skv), atol=1e-14)


def test_constant_v_is_reproduced():
    q = RNG.standard_normal((1, 5, 2, 8)) * 3
    k = RNG.standard_normal((1, 11, 2, 8))
    v = np.full((1, 11, 2, 8), -2.5)
    o, _ = attention(q, k, v, 0.5)
    np.testing.assert_allclose(o, -2.5, atol=1e-14)


def test_single_key():
    q = RNG.standard_normal((2, 3, 2, 4))
    k = RNG.standard_normal((2, 1, 2, 4))
    v = RNG.standard_normal((2, 1, 2, 4))
    o, lse = attention(q, k, v, 0.7)
    np.testing.assert_allclose(o, np.broadcast_to(v, o.shape), atol=1e-15)
    expect = 0.7 * np.einsum("bihd,bhd->bhi", q, k[:, 0])
    np.testing.assert_allclose(lse, expect, atol=1e-14)


def test_key_shift_invariance():
    # K + 1 c^T: every score of row i moves by scale * q_i . c, so O is
    # unchanged and LSE moves by exactly that amount.
    q = RNG.standard_normal((1, 6, 2, 8))
    k = RNG.standard_normal((1, 9, 2, 8))
    v = RNG.standard_normal((1, 9, 2, 8))
    c = RNG.standard_normal(8)
    o1, l1 = attention(q, k, v, 0.3)
    o2, l2 = attention(q, k + c, v, 0.3)
    np.testing.assert_allclose(o2, o1, atol=1e-13)
    shift = 0.3 * np.einsum("bihd,d->bhi", q, c)
    np.testing.assert_allclose(l2 - l1, shift, atol=1e-13)


def test_joint_key_value_permutation_invariance():
    q = RNG.standard_normal((2, 5, 3, 4))
    k = RNG.standard_normal((2, 10, 3, 4))
    v = RNG.standard_normal((2, 10, 3, 4))
    perm = RNG.permutation(10)
    o1, l1 = attention(q, k, v, 0.5)
    o2, l2 = attention(q, k[:, perm], v[:, perm], 0.5)
    np.testing.assert_allclose(o2, o1, atol=1e-14)
    np.testing.assert_allclose(l2, l1, atol=1e-14)


def test_empty_keys_are_the_merge_identity():
    q = RNG.standard_normal((1, 3, 2, 4))
    k = np.zeros((1, 0, 2, 4))
    o, lse = attention(q, k, k, 1.0)
    assert np.all(o == 0) and np.all(lse == -np.inf)


def test_large_scores_do_not_overflow():
    # scores ~ +-800: a shift-free exp overflows; the oracle must stay finite
    # and agree with the same problem shifted by a constant key offset.
    q = RNG.standard_normal((1, 4, 1, 4)) * 20
    k = RNG.standard_normal((1, 6, 1, 4)) * 20
    v = RNG.standard_normal((1, 6, 1, 4))
    o, lse = attention(q, k, v, 1.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert lse.max() > 300
    # softmax weights are exp(s - LSE): rows must sum to one
    s = np.einsum("bihd,bjhd->bhij", q, k)
    w = np.exp(s - lse[..., None])
    np.testing.assert_allclose(w.sum(-1), 1.0, atol=1e-12)


def test_row_sample_equals_full_rows():
    q = RNG.standard_normal((1, 50, 2, 8))
    k = RNG.standard_normal((1, 70, 2, 8))
    v = RNG.standard_normal((1, 70, 2, 8))
    o, lse = attention(q, k, v, 0.35)
    rows = np.array([49, 0, 17, 17, 3])
    os_, ls = attention(q, k, v, 0.35, rows=rows)
    np.testing.assert_array_equal(os_, o[:, rows])
    np.testing.assert_array_equal(ls, lse[:, :, rows])


def test_row_groups_do_not_change_results():
    q = RNG.standard_normal((1, 33, 1, 8))
    k = RNG.standard_normal((1, 40, 1, 8))
    v = RNG.standard_normal((1, 40, 1, 8))
    o1, l1 = attention(q, k, v, 0.35)
    o2, l2 = attention(q, k, v, 0.35, row_group=5)
    np.testing.assert_allclose(o2, o1, atol=1e-15)
    np.testing.assert_allclose(l2, l1, atol=1e-15)


def test_a_planted_mistake_is_caught():
    # Guard the pins themselves: an attention that forgets the scale must
    # fail the hand example.
    q = np.array([2.0]).reshape(1, 1, 1, 1)
    k = np.array([0.0, math.log(2) / 2, math.log(3) / 2]).reshape(1, 3, 1, 1)
    v = np.array([6.0, 0.0, 0.0]).reshape(1, 3, 1, 1)
    _, lse_right = attention(q, k, v, 1.0)
    _, lse_wrong = attention(q, k, v, 0.5)
    assert lse_right[0, 0, 0] == pytest.approx(math.log(6.0), abs=1e-14)
    assert abs(lse_wrong[0, 0, 0] - math.log(6.0)) > 0.1


# ---- per-batch key lengths (tail-padded keys excluded) ------------------------

def test_kv_len_matches_masked_scores_formulation():
    # the slicing definition against an explicit -inf score mask followed by a
    # softmax over all Skv keys (an independent formulation of the exclusion)
    rng = np.random.default_rng(31)
    B, Sq, Skv, H, D = 3, 5, 9, 2, 4
    q, k, v = (rng.standard_normal(s) for s in ((B, Sq, H, D), (B, Skv, H, D), (B, Skv, H, D)))
    kv_len = [9, 4, 1]
    o, lse = oracle.attention_kv_len(q, k, v, 0.7, kv_len)
    for b in range(B):
        for h in range(H):
            s = 0.7 * q[b, :, h] @ k[b, :, h].T
            s[:, kv_len[b]:] = -np.inf
            p = np.exp(s - s.max(axis=1, keepdims=True))
            ref_o = (p / p.sum(axis=1, keepdims=True)) @ v[b, :, h]
            ref_l = np.log(np.exp(s).sum(axis=1))
            assert np.max(np.abs(o[b, :, h] - ref_o)) <= 1e-12
            assert np.max(np.abs(lse[b, h] - ref_l)) <= 1e-12


def test_kv_len_full_empty_and_chunking():
    rng = np.random.default_rng(32)
    B, Sq, Skv, H, D = 2, 4, 12, 2, 8
    q, k, v = (rng.standard_normal(s) for s in ((B, Sq, H, D), (B, Skv, H, D), (B, Skv, H, D)))
    full = oracle.attention(q, k, v, 0.3)
    o, lse = oracle.attention_kv_len(q, k, v, 0.3, [Skv, 99])   # at and past Skv: all keys
    assert np.max(np.abs(o - full[0])) <= 1e-13 and np.max(np.abs(lse - full[1])) <= 1e-13
    o, lse = oracle.attention_kv_len(q, k, v, 0.3, [0, -3])     # no valid key: merge identity
    assert not np.any(o) and np.all(np.isneginf(lse))
    # a valid prefix split in two and merged equals the prefix at once
    o7, l7 = oracle.attention_kv_len(q, k, v, 0.3, [7, 7])
    a = oracle.attention(q, k[:, :3], v[:, :3], 0.3)
    c = oracle.attention(q, k[:, 3:7], v[:, 3:7], 0.3)
    m = oracle.merge(a[0], a[1], c[0], c[1])
    assert np.max(np.abs(m[0] - o7)) <= 1e-13 and np.max(np.abs(m[1] - l7)) <= 1e-13

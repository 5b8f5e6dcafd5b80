"""Pins for the online-softmax merge and the ring fold (CPU only)."""

import math

import numpy as np
import pytest

from oracle import attention, merge, ring_attention, ring_hop_order

RNG = np.random.default_rng(99)


def _part(B=2, Sq=5, H=3, D=4):
    o = RNG.standard_normal((B, Sq, H, D))
    lse = RNG.standard_normal((B, H, Sq)) * 3
    return o, lse


def test_hand_example():
    # (O=2, L=0) and (O=5, L=ln 2): weights 1/3 and 2/3 -> O = 4, L = ln 3.
    oa = np.full((1, 1, 1, 1), 2.0)
    oc = np.full((1, 1, 1, 1), 5.0)
    o, l = merge(oa, np.zeros((1, 1, 1)), oc, np.full((1, 1, 1), math.log(2)))
    assert o[0, 0, 0, 0] == pytest.approx(4.0, abs=1e-15)
    assert l[0, 0, 0] == pytest.approx(math.log(3), abs=1e-15)


def test_lse_follows_row_layout():
    # LSE is [B, H, Sq] while O is [B, Sq, H, D]: give one (b, h, i) row a
    # dominant partial and check only that row switches.
    oa, la = _part()
    oc, lc = _part()
    lc[:] = -50.0
    lc[1, 2, 3] = 50.0
    o, l = merge(oa, la, oc, lc)
    np.testing.assert_allclose(o[1, 3, 2], oc[1, 3, 2], atol=1e-15)
    mask = np.ones(o.shape[:3], bool)
    mask[1, 3, 2] = False
    np.testing.assert_allclose(o[mask], oa[mask], atol=1e-15)


def test_identity_with_empty_part_is_exact_even_with_garbage():
    oa, la = _part()
    garbage = np.full_like(oa, np.nan)
    o, l = merge(oa, la, garbage, np.full_like(la, -np.inf))
    np.testing.assert_array_equal(o, oa)
    np.testing.assert_array_equal(l, la)
    o, l = merge(garbage, np.full_like(la, -np.inf), oa, la)
    np.testing.assert_array_equal(o, oa)
    np.testing.assert_array_equal(l, la)


def test_both_empty():
    o, l = merge(np.full((1, 2, 1, 3), np.nan), np.full((1, 1, 2), -np.inf),
                 np.full((1, 2, 1, 3), np.inf), np.full((1, 1, 2), -np.inf))
    assert np.all(o == 0) and np.all(l == -np.inf)


def test_commutative_bitwise():
    a, c = _part(), _part()
    o1, l1 = merge(*a, *c)
    o2, l2 = merge(*c, *a)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_associative():
    a, b, c = _part(), _part(), _part()
    left = merge(*merge(*a, *b), *c)
    right = merge(*a, *merge(*b, *c))
    np.testing.assert_allclose(left[0], right[0], atol=1e-13)
    np.testing.assert_allclose(left[1], right[1], atol=1e-13)


@pytest.mark.parametrize("bounds", [
    [0, 40],
    [0, 20, 40],
    [0, 10, 20, 30, 40],
    [0, 3, 3, 29, 40],          # uneven, with an empty chunk
    [0, 0, 40],                 # empty first chunk
    [0, 1, 2, 3, 40],
])
def test_chunked_equals_unchunked(bounds):
    q = RNG.standard_normal((2, 7, 3, 8))
    k = RNG.standard_normal((2, 40, 3, 8))
    v = RNG.standard_normal((2, 40, 3, 8))
    o, l = attention(q, k, v, 0.35)
    R = len(bounds) - 1
    for order in (list(range(R)), ring_hop_order(R, 0), list(reversed(range(R)))):
        oc, lc = ring_attention(q, k, v, 0.35, bounds, order)
        np.testing.assert_allclose(oc, o, atol=1e-13)
        np.testing.assert_allclose(lc, l, atol=1e-13)


def test_single_chunk_is_plain_attention_bitwise():
    q = RNG.standard_normal((1, 4, 2, 4))
    k = RNG.standard_normal((1, 9, 2, 4))
    v = RNG.standard_normal((1, 9, 2, 4))
    o, l = attention(q, k, v, 0.5)
    oc, lc = ring_attention(q, k, v, 0.5, [0, 9])
    np.testing.assert_array_equal(oc, o)
    np.testing.assert_array_equal(lc, l)


def test_hop_order():
    assert ring_hop_order(4, 0) == [0, 3, 2, 1]
    assert ring_hop_order(4, 1) == [1, 0, 3, 2]
    assert ring_hop_order(1, 0) == [0]
    assert sorted(ring_hop_order(5, 3)) == list(range(5))


def test_a_planted_sign_error_is_caught():
    # a merge that weights by exp(m - L) instead of exp(L - m) must break
    # chunked == unchunked
    def bad_merge(oa, la, oc, lc):
        la_ = np.transpose(la, (0, 2, 1))[..., None]
        lc_ = np.transpose(lc, (0, 2, 1))[..., None]
        m = np.maximum(la_, lc_)
        wa, wc = np.exp(m - la_), np.exp(m - lc_)
        return (wa * oa + wc * oc) / (wa + wc), None

    q = RNG.standard_normal((1, 5, 1, 4))
    k = RNG.standard_normal((1, 8, 1, 4)) * 2
    v = RNG.standard_normal((1, 8, 1, 4))
    o, _ = attention(q, k, v, 1.0)
    a = attention(q, k[:, :3], v[:, :3], 1.0)
    c = attention(q, k[:, 3:], v[:, 3:], 1.0)
    good, _ = merge(*a, *c)
    bad, _ = bad_merge(*a, *c)
    np.testing.assert_allclose(good, o, atol=1e-13)
    assert np.abs(bad - o).max() > 1e-3

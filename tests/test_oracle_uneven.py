"""Pins of the oracle's padding-free (uneven) Ulysses maps (CPU only).

Checked against the oracle's padded maps where the two must agree (counts
that divide evenly: no padding, identical buffers), against the global
view (after the exchange, rank r's planes are the full sequence of its head
range), by round trips through both directions, and with ranks that hold no
rows or no heads.
"""

import numpy as np
import pytest

import oracle


def _split(total, U, skew=0):
    base = [total // U + (1 if r < total % U else 0) for r in range(U)]
    if skew and U > 1:           # move `skew` rows from the last rank to the first
        k = min(skew, base[-1])
        base[0] += k
        base[-1] -= k
    return base


def _exchange_s2h(X, B, D, n, sc, hc):
    U = len(sc)
    so = np.concatenate([[0], np.cumsum(sc)])
    sends, sizes = [], []
    for r in range(U):
        shard = [X[pl][:, so[r]:so[r + 1]] for pl in range(n)]
        sends.append(oracle.pack_seq_to_head_uneven(shard, sc, hc, r))
        sizes.append(oracle.uneven_chunk_sizes(B, D, n, sc, hc, r, True)[0])
    return oracle.all_to_all_uneven(sends, sizes)


CASES = [
    # B, S, H, D, n, seq counts, head counts
    (1, 10, 4, 8, 3, _split(10, 3), _split(4, 3)),
    (2, 17, 7, 4, 1, _split(17, 4, skew=2), _split(7, 4)),
    (1, 9, 5, 6, 3, [0, 4, 5], [2, 0, 3]),            # ranks without rows / heads
    (2, 33, 6, 8, 2, [20, 13], [1, 5]),
]


@pytest.mark.parametrize("case", CASES)
def test_global_view_and_round_trip(case):
    B, S, H, D, n, sc, hc = case
    U = len(sc)
    rng = np.random.default_rng(S + H)
    X = [rng.standard_normal((B, S, H, D)) for _ in range(n)]
    recvs = _exchange_s2h(X, B, D, n, sc, hc)
    ho = np.concatenate([[0], np.cumsum(hc)])
    so = np.concatenate([[0], np.cumsum(sc)])
    outs = []
    for r in range(U):
        planes = oracle.unpack_seq_to_head_uneven(recvs[r], B, D, n, sc, hc, r)
        for pl in range(n):
            assert np.array_equal(planes[pl], X[pl][:, :, ho[r]:ho[r + 1]])   # the global view
        outs.append(planes)
    # head-to-sequence back: every rank recovers its own rows of all heads
    sends = [oracle.pack_head_to_seq_uneven(outs[r], sc, hc, r) for r in range(U)]
    sizes = [oracle.uneven_chunk_sizes(B, D, n, sc, hc, r, False)[0] for r in range(U)]
    back = oracle.all_to_all_uneven(sends, sizes)
    for r in range(U):
        planes = oracle.unpack_head_to_seq_uneven(back[r], B, D, n, sc, hc, r)
        for pl in range(n):
            assert np.array_equal(planes[pl], X[pl][:, so[r]:so[r + 1]])


@pytest.mark.parametrize("B,S,H,D,U,n", [(1, 12, 4, 8, 2, 3), (2, 16, 8, 4, 4, 1)])
def test_even_counts_equal_the_padded_maps(B, S, H, D, U, n):
    L = oracle.a2a_layout(B, S, H, D, U, 1, n)
    sc, hc = [S // U] * U, [H // U] * U
    rng = np.random.default_rng(B * S)
    for r in range(U):
        shard = [rng.standard_normal((B, S // U, H, D)) for _ in range(n)]
        assert np.array_equal(oracle.pack_seq_to_head_uneven(shard, sc, hc, r),
                              oracle.pack_seq_to_head(shard, L, r).reshape(-1))
        planes = [rng.standard_normal((B, S, H // U, D)) for _ in range(n)]
        assert np.array_equal(oracle.pack_head_to_seq_uneven(planes, sc, hc, r),
                              oracle.pack_head_to_seq(planes, L, r).reshape(-1))
        buf = rng.standard_normal(L["elems_per_peer"] * U)
        for a, b in zip(oracle.unpack_seq_to_head_uneven(buf, B, D, n, sc, hc, r),
                        oracle.unpack_seq_to_head(buf.reshape(U, n, B, S // U, H // U, D), L, r)):
            assert np.array_equal(a, b)
        for a, b in zip(oracle.unpack_head_to_seq_uneven(buf, B, D, n, sc, hc, r),
                        oracle.unpack_head_to_seq(buf.reshape(U, n, B, S // U, H // U, D), L, r)):
            assert np.array_equal(a, b)


def test_chunk_sizes_balance():
    sc, hc = [5, 0, 7], [2, 3, 1]
    for r in range(3):
        s, rv = oracle.uneven_chunk_sizes(2, 4, 3, sc, hc, r, True)
        assert s[r] == rv[r]              # the chunk a rank keeps for itself
    total_send = sum(sum(oracle.uneven_chunk_sizes(2, 4, 3, sc, hc, r, True)[0]) for r in range(3))
    total_recv = sum(sum(oracle.uneven_chunk_sizes(2, 4, 3, sc, hc, r, True)[1]) for r in range(3))
    assert total_send == total_recv == 3 * 2 * 12 * 6 * 4


@pytest.mark.parametrize("counts,B,H,D,n", [([5, 3, 0, 4], 2, 3, 4, 2), ([7], 1, 2, 8, 1), ([2, 2], 3, 1, 2, 2)])
def test_ring_anything_gather_recovers_the_sequence(counts, B, H, D, n):
    S, S_max = sum(counts), max(counts)
    rng = np.random.default_rng(S * 7 + n)
    X = [rng.standard_normal((B, S, H, D)) for _ in range(n)]
    so = np.concatenate([[0], np.cumsum(counts)])
    padded = []
    for r, c in enumerate(counts):
        buf = oracle.ring_anything_pad([x[:, so[r]:so[r + 1]] for x in X], S_max)
        assert buf.shape == (n, B, S_max, H, D)
        assert not np.any(buf[:, :, c:])                        # pad rows are zeros
        padded.append(buf)
    gathered = np.stack(padded)                                 # the all-gather
    out = oracle.ring_anything_trim(gathered, counts)
    for a, b in zip(out, X):
        assert np.array_equal(a, b)


def test_ring_anything_trim_with_equal_counts_is_a_reshape():
    rng = np.random.default_rng(3)
    U, n, B, S_loc, H, D = 3, 2, 2, 4, 2, 3
    g = rng.standard_normal((U, n, B, S_loc, H, D))
    out = oracle.ring_anything_trim(g, [S_loc] * U)
    want = np.transpose(g, (1, 2, 0, 3, 4, 5)).reshape(n, B, U * S_loc, H, D)
    for i in range(n):
        assert np.array_equal(out[i], want[i])

"""Pins for the Ulysses pack / unpack index maps (CPU only).

The brute-force side states the exchange end to end on the global tensor
(which rows and heads each rank owns before and after) and never uses the
pack / unpack maps, so a wrong index, a swapped axis or a misplaced pad in
the oracle fails here.
"""

import itertools

import numpy as np
import pytest

from oracle import (a2a_layout, all_to_all, brute, pack_head_to_seq, pack_seq_to_head,
                    unpack_head_to_seq, unpack_seq_to_head)

RNG = np.random.default_rng(7)

CASES = [
    # B, S, H, D, U, seq_align, n_planes
    (1, 8, 4, 2, 2, 1, 1),
    (2, 7, 5, 3, 3, 1, 3),      # ragged S and H: pad rows and a pad head
    (1, 10, 6, 2, 4, 1, 3),     # S pad 12, H pad 8
    (2, 9, 3, 2, 2, 4, 1),      # seq_align 4: S_pad = 12
    (1, 5, 2, 1, 5, 1, 1),      # U > H: three pad heads
    (1, 3, 4, 2, 4, 1, 1),      # U > S: one rank holds only pad rows
]


def test_layout_values_for_the_workloads():
    L = a2a_layout(2, 7145, 24, 128, 4, 1, 3)
    assert (L["S_pad"], L["S_loc"], L["H_pad"], L["H_loc"]) == (7148, 1787, 24, 6)
    assert L["elems_per_peer"] * 2 * 4 == 65_875_968
    L = a2a_layout(2, 7145, 24, 128, 5, 1, 3)
    assert (L["S_pad"], L["S_loc"], L["H_pad"], L["H_loc"]) == (7145, 1429, 25, 5)
    assert L["elems_per_peer"] * 2 * 5 == 54_873_600
    L = a2a_layout(2, 7145, 24, 128, 4, 64, 1)
    assert (L["S_pad"], L["S_loc"]) == (7168, 1792)
    L = a2a_layout(1, 4608, 24, 128, 2, 1, 3)
    assert (L["S_loc"], L["H_loc"]) == (2304, 12)
    assert L["elems_per_peer"] * 2 * 2 == 42_467_328
    L = a2a_layout(1, 75600, 40, 128, 8, 1, 1)
    assert (L["S_loc"], L["H_loc"]) == (9450, 5)
    assert L["elems_per_peer"] * 2 * 8 == 96_768_000


def _globals(B, S, H, D, n):
    # distinct labels so a dropped or duplicated element is visible
    return [(np.arange(B * S * H * D, dtype=np.float64).reshape(B, S, H, D) + 1 + 1e6 * pl)
            for pl in range(n)]


@pytest.mark.parametrize("case", CASES)
def test_seq_to_head_composition_matches_brute(case):
    B, S, H, D, U, al, n = case
    L = a2a_layout(B, S, H, D, U, al, n)
    X = _globals(B, S, H, D, n)
    sends = []
    for r in range(U):
        shards = [np.array(brute.local_shard(x.tolist(), r, L["S_loc"])) for x in X]
        # garbage in the pad rows of the input must never be read
        for sh in shards:
            for s in range(L["S_loc"]):
                if r * L["S_loc"] + s >= S:
                    sh[:, s] = -7.0
        sends.append(pack_seq_to_head(shards, L, r))
    recvs = all_to_all(sends)
    for r in range(U):
        got = unpack_seq_to_head(recvs[r], L, r)
        for pl in range(n):
            want = np.array(brute.ulysses_seq_to_head(X[pl].tolist(), U, L["S_loc"], L["H_loc"])[r])
            np.testing.assert_array_equal(got[pl], want)


@pytest.mark.parametrize("case", CASES)
def test_head_to_seq_composition_matches_brute(case):
    B, S, H, D, U, al, n = case
    L = a2a_layout(B, S, H, D, U, al, n)
    O = _globals(B, S, H, D, n)
    sends = []
    for r in range(U):
        heads = [np.array(brute.ulysses_seq_to_head(o.tolist(), U, L["S_loc"], L["H_loc"])[r])
                 for o in O]
        for hh in heads:  # garbage in pad heads must never be read
            for h in range(L["H_loc"]):
                if r * L["H_loc"] + h >= H:
                    hh[:, :, h] = -9.0
        sends.append(pack_head_to_seq(heads, L, r))
    recvs = all_to_all(sends)
    for r in range(U):
        got = unpack_head_to_seq(recvs[r], L, r)
        for pl in range(n):
            want = np.array(brute.ulysses_head_to_seq(O[pl].tolist(), U, L["S_loc"])[r])
            np.testing.assert_array_equal(got[pl], want)


@pytest.mark.parametrize("case", CASES)
def test_round_trip_returns_the_local_shards(case):
    B, S, H, D, U, al, n = case
    L = a2a_layout(B, S, H, D, U, al, n)
    X = _globals(B, S, H, D, n)
    shards = [[np.array(brute.local_shard(x.tolist(), r, L["S_loc"])) for x in X] for r in range(U)]
    recv = all_to_all([pack_seq_to_head(shards[r], L, r) for r in range(U)])
    heads = [unpack_seq_to_head(recv[r], L, r) for r in range(U)]
    back = all_to_all([pack_head_to_seq(heads[r], L, r) for r in range(U)])
    for r in range(U):
        got = unpack_head_to_seq(back[r], L, r)
        for pl in range(n):
            np.testing.assert_array_equal(got[pl], shards[r][pl])


def test_pack_writes_zero_pads_and_moves_every_label_once():
    B, S, H, D, U, al, n = 2, 7, 5, 3, 3, 1, 3
    L = a2a_layout(B, S, H, D, U, al, n)
    X = _globals(B, S, H, D, n)
    labels = []
    for r in range(U):
        shards = [np.array(brute.local_shard(x.tolist(), r, L["S_loc"])) + 0.0 for x in X]
        send = pack_seq_to_head(shards, L, r)
        assert send.shape == (U, n, B, L["S_loc"], L["H_loc"], D)
        for p, pl, b, s, h in itertools.product(range(U), range(n), range(B), range(L["S_loc"]),
                                                range(L["H_loc"])):
            pad = r * L["S_loc"] + s >= S or p * L["H_loc"] + h >= H
            if pad:
                assert np.all(send[p, pl, b, s, h] == 0)
        labels.append(send[send != 0])
    allv = np.sort(np.concatenate(labels))
    want = np.sort(np.concatenate([x.ravel() for x in X]))
    np.testing.assert_array_equal(allv, want)


def test_peer_major_order_hand_case():
    # U=2, one plane, B=1, S=2, H=2, D=1: rank 0 holds row 0 = (a, b) for
    # heads (0, 1); the send buffer is peer-major: peer 0 gets head 0, peer
    # 1 gets head 1; with S_loc = 1 each chunk is a single element.
    L = a2a_layout(1, 2, 2, 1, 2, 1, 1)
    x = np.array([[[[10.0], [20.0]]]])        # [B=1, S_loc=1, H=2, D=1]
    send = pack_seq_to_head([x], L, 0)
    assert send.reshape(-1).tolist() == [10.0, 20.0]
    # receive side of rank 1: chunk from peer 0 (row 0) then peer 1 (row 1)
    recv = np.array([21.0, 22.0]).reshape(2, 1, 1, 1, 1, 1)
    out = unpack_seq_to_head(recv, L, 1)[0]
    assert out.reshape(-1).tolist() == [21.0, 22.0]

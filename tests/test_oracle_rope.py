"""Pins of the oracle's RoPE receive preparation (CPU only).

The rotation of ``oracle.rope`` is checked against an independent
formulation (complex multiplication by exp(i angle) through numpy's complex
arithmetic), against the closed forms of a rotation (identity, quarter turn,
norm preservation, composition of angles) and against the property that
defines rotary embeddings: after rotation, q_m . k_n depends on the
positions only through m - n.  The fused unpack is pinned to the plain
unpack (identity tables, the V plane) and to a round trip.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from sequence_attention_amd import workloads


def _x(B, S, H, D, seed):
    return np.random.default_rng(seed).standard_normal((B, S, H, D))


def _tables(angles):
    return np.cos(angles), np.sin(angles)


def test_matches_complex_multiplication():
    x = _x(2, 7, 3, 8, 1)
    ang = np.random.default_rng(2).uniform(-10, 10, size=(7, 4))
    c, s = _tables(ang)
    y = oracle.rope(x, c, s)
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * ang)[None, :, None, :]
    assert np.max(np.abs(y[..., 0::2] - z.real)) <= 1e-12
    assert np.max(np.abs(y[..., 1::2] - z.imag)) <= 1e-12


def test_identity_quarter_turn_and_norm():
    x = _x(1, 5, 2, 6, 3)
    c, s = np.ones((5, 3)), np.zeros((5, 3))
    assert np.array_equal(oracle.rope(x, c, s), x)
    c, s = _tables(np.full((5, 3), math.pi / 2))
    y = oracle.rope(x, c, s)
    assert np.max(np.abs(y[..., 0::2] + x[..., 1::2])) <= 1e-15
    assert np.max(np.abs(y[..., 1::2] - x[..., 0::2])) <= 1e-15
    c, s = _tables(np.random.default_rng(4).uniform(0, 7, size=(5, 3)))
    y = oracle.rope(x, c, s)
    n_in = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n_out = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.max(np.abs(n_in - n_out)) <= 1e-12


def test_composition_of_angles():
    x = _x(1, 4, 2, 8, 5)
    rng = np.random.default_rng(6)
    a, b = rng.uniform(-3, 3, (4, 4)), rng.uniform(-3, 3, (4, 4))
    y = oracle.rope(oracle.rope(x, *_tables(a)), *_tables(b))
    assert np.max(np.abs(y - oracle.rope(x, *_tables(a + b)))) <= 1e-12


def test_relative_position_property():
    # angle(t, i) = t * w_i: the rotated dot product depends on m - n only
    D, S = 16, 40
    w = 10000.0 ** (-2.0 * np.arange(D // 2) / D)
    c, s = _tables(np.arange(S)[:, None] * w[None, :])
    rng = np.random.default_rng(7)
    qv, kv = rng.standard_normal(D), rng.standard_normal(D)
    q = np.broadcast_to(qv, (1, S, 1, D)).copy()
    k = np.broadcast_to(kv, (1, S, 1, D)).copy()
    rq, rk = oracle.rope(q, c, s)[0, :, 0], oracle.rope(k, c, s)[0, :, 0]
    for delta in (1, 5, 17):
        for m, n in ((3, 9), (10, 2), (0, 0)):
            assert abs(rq[m] @ rk[n] - rq[m + delta] @ rk[n + delta]) <= 1e-10


def test_tables_of_the_input_recipe():
    c, s = workloads.rope_tables(6, 8)
    assert c.dtype == torch.float32 and tuple(c.shape) == (6, 4)
    w = 10000.0 ** (-2.0 * np.arange(4) / 8)
    ang = np.arange(6)[:, None] * w[None, :]
    assert np.max(np.abs(c.double().numpy() - np.cos(ang))) <= 2.0 ** -24
    assert np.max(np.abs(s.double().numpy() - np.sin(ang))) <= 2.0 ** -24


@pytest.mark.parametrize("B,S,H,D,U", [(1, 16, 4, 8, 2), (2, 13, 5, 4, 4), (1, 9, 3, 8, 3)])
def test_fused_unpack_pins(B, S, H, D, U):
    L = oracle.a2a_layout(B, S, H, D, U, 1, 3)
    rng = np.random.default_rng(B * 100 + S)
    glob = [rng.standard_normal((B, S, H, D)) for _ in range(3)]
    shards = []
    for r in range(U):
        rows = [np.zeros((B, L["S_loc"], H, D)) for _ in range(3)]
        lo, hi = r * L["S_loc"], min(S, (r + 1) * L["S_loc"])
        for pl in range(3):
            if hi > lo:
                rows[pl][:, :hi - lo] = glob[pl][:, lo:hi]
        shards.append(rows)
    recv = oracle.all_to_all([oracle.pack_seq_to_head(shards[r], L, r) for r in range(U)])
    ang = np.random.default_rng(9).uniform(-5, 5, size=(S, D // 2))
    c, s = _tables(ang)
    for r in range(U):
        plain = oracle.unpack_seq_to_head(recv[r], L, r)
        fused = oracle.unpack_seq_to_head_rope(recv[r], L, r, c, s)
        # V is the plain unpack; identity tables give the plain unpack
        assert np.array_equal(fused[2], plain[2])
        ident = oracle.unpack_seq_to_head_rope(recv[r], L, r, np.ones_like(c), np.zeros_like(s))
        for pl in range(3):
            assert np.array_equal(ident[pl], plain[pl])
        # rotating back by -angle restores the plain unpack
        for pl in range(2):
            back = oracle.rope(fused[pl], c, -s)
            assert np.max(np.abs(back - plain[pl])) <= 1e-12
        # Q of the head slice: the global tensor's heads, rotated
        h_lo = r * L["H_loc"]
        heads = [h for h in range(h_lo, h_lo + L["H_loc"]) if h < H]
        if heads:
            want = oracle.rope(glob[0][:, :, heads], c, s)
            assert np.max(np.abs(fused[0][:, :, :len(heads)] - want)) <= 1e-12
        # pad heads arrive as zeros and stay zero after the rotation
        assert not np.any(fused[0][:, :, len(heads):])

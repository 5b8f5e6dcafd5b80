"""Pins for the 16-bit conversion inside the packs (CPU only).

``round_to_half`` is written from the two formats' definitions: a ladder of
the values of the non-negative codes, the nearest rung taken, ties to the
even code.  It is pinned to things other than itself:

* hand values the formats fix: ties both ways, the overflow threshold and
  the value just below it, the smallest subnormal and the ties around it,
  signed zero, infinities, NaN;
* numpy's float32 -> float16 conversion and torch's float32 -> bfloat16
  conversion (both IEEE round to nearest, ties to even) on random float32
  bit patterns over every exponent, on every midpoint between adjacent
  codes and on the float32 neighbours of each midpoint;
* the decode of all 65536 codes against numpy's float16 and torch's
  bfloat16.

The converting packs are pinned end to end: every rank's send buffer goes
through the exchange and the oracle's unpack, and the result must equal the
brute-force reshard of the global tensor converted element by element with
the library conversions.
"""

import numpy as np
import pytest
import torch

from oracle import (a2a_layout, all_to_all, brute, half_is_nan, half_value,
                    pack_head_to_seq_convert, pack_seq_to_head_convert, round_to_half,
                    unpack_head_to_seq, unpack_seq_to_head)

RNG = np.random.default_rng(11)

# (value, f16 code, bf16 code); every value is a float32 value
HAND = [
    (0.0, 0x0000, 0x0000),
    (-0.0, 0x8000, 0x8000),
    (1.0, 0x3C00, 0x3F80),
    (-2.0, 0xC000, 0xC000),
    (1 + 2.0 ** -11, 0x3C00, 0x3F80),               # f16 tie -> even (down)
    (1 + 3 * 2.0 ** -11, 0x3C02, 0x3F80),           # f16 tie -> even (up)
    (1 + 2.0 ** -11 + 2.0 ** -20, 0x3C01, 0x3F80),  # just past the f16 tie
    (1 + 2.0 ** -8, 0x3C04, 0x3F80),                # bf16 tie -> even (down)
    (1 + 3 * 2.0 ** -8, 0x3C0C, 0x3F82),            # bf16 tie -> even (up)
    (1 + 2.0 ** -8 + 2.0 ** -20, 0x3C04, 0x3F81),   # just past the bf16 tie
    (65504.0, 0x7BFF, 0x4780),                      # largest finite f16
    (65520.0 - 2.0 ** -8, 0x7BFF, 0x4780),          # f32 just below the f16 overflow midpoint
    (65520.0, 0x7C00, 0x4780),                      # the midpoint rounds to infinity
    (2.0 ** -14, 0x0400, 0x3880),                   # smallest normal f16
    (2.0 ** -24, 0x0001, 0x3380),                   # smallest subnormal f16
    (2.0 ** -25, 0x0000, 0x3300),                   # tie between 0 and 2^-24 -> 0
    (3 * 2.0 ** -25, 0x0002, 0x33C0),               # tie between 1 and 2 ulps -> 2
    (2.0 ** -126, 0x0000, 0x0080),                  # smallest normal bf16 (f32)
    (2.0 ** -133, 0x0000, 0x0001),                  # smallest subnormal bf16
    (2.0 ** -134, 0x0000, 0x0000),                  # tie -> 0
    (3 * 2.0 ** -134, 0x0000, 0x0002),              # tie -> even
    ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7C00, 0x7F7F),     # largest finite bf16
    ((2 - 2.0 ** -8 - 2.0 ** -23) * 2.0 ** 127, 0x7C00, 0x7F7F),
    ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7C00, 0x7F80),     # bf16 overflow midpoint -> inf
    ((2 - 2.0 ** -23) * 2.0 ** 127, 0x7C00, 0x7F80),    # largest float32
    (float("inf"), 0x7C00, 0x7F80),
    (float("-inf"), 0xFC00, 0xFF80),
]


def test_hand_values_are_float32_values():
    v = np.array([h[0] for h in HAND], dtype=np.float64)
    assert np.array_equal(v.astype(np.float32).astype(np.float64), v)


@pytest.mark.parametrize("fmt,col", [("f16", 1), ("bf16", 2)])
def test_hand_table(fmt, col):
    v = np.array([h[0] for h in HAND], dtype=np.float64)
    want = np.array([h[col] for h in HAND], dtype=np.uint16)
    got = round_to_half(v, fmt)
    bad = [(HAND[i][0], hex(got[i]), hex(want[i])) for i in np.nonzero(got != want)[0]]
    assert not bad, bad
    assert np.array_equal(np.signbit(half_value(got, fmt)), np.signbit(v))


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_nan_stays_nan(fmt):
    bits = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0x7FFFFFFF], dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        x = bits.view(np.float32).astype(np.float64)
    assert np.all(half_is_nan(round_to_half(x, fmt), fmt))
    assert not np.any(half_is_nan(round_to_half(np.array([np.inf, -np.inf, 0.0]), fmt), fmt))


def _f16_library(x32):
    with np.errstate(over="ignore"):
        return x32.astype(np.float16).view(np.uint16)


def _bf16_library(x32):
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


LIBRARY = {"f16": _f16_library, "bf16": _bf16_library}


def _check_against_library(x32, fmt):
    with np.errstate(invalid="ignore"):
        got = round_to_half(x32.astype(np.float64), fmt)
    want = LIBRARY[fmt](x32)
    nan = np.isnan(x32)
    assert np.array_equal(half_is_nan(got, fmt), nan)
    assert np.array_equal(half_is_nan(want, fmt), nan)
    mism = np.nonzero((got != want) & ~nan)[0]
    assert mism.size == 0, [(float(x32[i]), hex(got[i]), hex(want[i])) for i in mism[:8]]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_random_float32_bit_patterns(fmt):
    x32 = RNG.integers(0, 2 ** 32, size=300_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    _check_against_library(x32, fmt)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_every_midpoint_and_its_neighbours(fmt):
    inf_code = 0x7C00 if fmt == "f16" else 0x7F80
    v = half_value(np.arange(inf_code), fmt)
    mids = (v[:-1] + v[1:]) / 2
    top = v[-1] + (v[-1] - v[-2]) / 2                 # the overflow midpoint
    mids = np.concatenate([mids, [top]])
    m32 = mids.astype(np.float32)
    assert np.array_equal(m32.astype(np.float64), mids)   # midpoints are float32 values
    near = np.concatenate([m32, np.nextafter(m32, np.float32(np.inf)),
                           np.nextafter(m32, np.float32(0))])
    x32 = np.concatenate([near, -near])
    _check_against_library(x32, fmt)


def test_decode_of_every_code():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    np.testing.assert_array_equal(half_value(codes, "f16"),
                                  codes.view(np.float16).astype(np.float64))
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(half_value(codes, "bf16"), ref)


CASES = [
    # B, S, H, D, U, seq_align, n_planes
    (1, 8, 4, 2, 2, 1, 3),
    (2, 7, 5, 3, 3, 1, 3),      # ragged S and H
    (1, 3, 4, 2, 4, 1, 1),      # a rank holding only pad rows
]


def _special_globals(B, S, H, D, n):
    """float32 planes mixing ordinary values with ties, subnormals, overflow,
    signed zeros, infinities and NaN."""
    pool = np.array([h[0] for h in HAND] + [float("nan")], dtype=np.float32)
    out = []
    for _ in range(n):
        x = RNG.standard_normal((B, S, H, D)).astype(np.float32) * np.float32(300.0)
        pick = RNG.random((B, S, H, D)) < 0.3
        x[pick] = RNG.choice(pool, size=int(pick.sum()))
        out.append(x)
    return out


def _codes_equal(got, want, fmt):
    got = np.asarray(got).astype(np.uint16)
    want = np.asarray(want).astype(np.uint16)
    nan = half_is_nan(want, fmt)
    assert np.array_equal(half_is_nan(got, fmt), nan)
    assert np.array_equal(got[~nan], want[~nan])


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("case", CASES)
def test_seq_to_head_convert_matches_brute(case, fmt):
    B, S, H, D, U, al, n = case
    L = a2a_layout(B, S, H, D, U, al, n)
    X = _special_globals(B, S, H, D, n)
    sends = []
    for r in range(U):
        shards = [np.array(brute.local_shard(x.tolist(), r, L["S_loc"]), dtype=np.float32) for x in X]
        for sh in shards:   # pad rows of the input are never read
            for s in range(L["S_loc"]):
                if r * L["S_loc"] + s >= S:
                    sh[:, s] = np.float32(-7.0)
        send = pack_seq_to_head_convert(shards, L, r, fmt)
        assert send.dtype == np.uint16 and send.shape == (U, n, B, L["S_loc"], L["H_loc"], D)
        sends.append(send)
    recvs = all_to_all(sends)
    for r in range(U):
        got = unpack_seq_to_head(recvs[r], L, r)
        for pl in range(n):
            codes = LIBRARY[fmt](X[pl].reshape(-1)).reshape(X[pl].shape).astype(np.float64)
            want = np.array(brute.ulysses_seq_to_head(codes.tolist(), U, L["S_loc"], L["H_loc"])[r])
            _codes_equal(got[pl], want, fmt)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("case", CASES)
def test_head_to_seq_convert_matches_brute(case, fmt):
    B, S, H, D, U, al, n = case
    L = a2a_layout(B, S, H, D, U, al, n)
    O = _special_globals(B, S, H, D, n)
    sends = []
    for r in range(U):
        heads = [np.array(brute.ulysses_seq_to_head(o.tolist(), U, L["S_loc"], L["H_loc"])[r],
                          dtype=np.float32) for o in O]
        for hh in heads:    # pad heads of the input are never read
            for h in range(L["H_loc"]):
                if r * L["H_loc"] + h >= H:
                    hh[:, :, h] = np.float32(-9.0)
        sends.append(pack_head_to_seq_convert(heads, L, r, fmt))
    recvs = all_to_all(sends)
    for r in range(U):
        got = unpack_head_to_seq(recvs[r], L, r)
        for pl in range(n):
            codes = LIBRARY[fmt](O[pl].reshape(-1)).reshape(O[pl].shape).astype(np.float64)
            want = np.array(brute.ulysses_head_to_seq(codes.tolist(), U, L["S_loc"])[r])
            _codes_equal(got[pl], want, fmt)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_pad_elements_are_positive_zero(fmt):
    L = a2a_layout(1, 7, 5, 4, 3, 1, 3)
    planes = [np.full((1, L["S_loc"], 5, 4), -1.0, dtype=np.float32) for _ in range(3)]
    send = pack_seq_to_head_convert(planes, L, 2, fmt)   # rank 2: one pad row; last peer: a pad head
    one = 0xBC00 if fmt == "f16" else 0xBF80
    assert set(np.unique(send).tolist()) == {0, one}
    # S_loc = 3: rank 2 holds rows 6, 7, 8, of which only row 6 is real; of
    # the 6 padded heads, head 5 is a pad head
    assert np.count_nonzero(send == one) == 1 * 1 * 5 * 4 * 3

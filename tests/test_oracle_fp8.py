"""Pins of the oracle's FP8 Ulysses pieces (CPU only).

E4M3 decoding and round-to-nearest-even encoding are checked against
torch's float8_e4m3fn conversions (an independent library routine) and hand
examples; the block exponent against its definition by search; the round
trip against the E4M3 error bound; and the FP8 exchange layouts against
quantization applied directly to the global tensors (the permutation and
the per-block quantization commute), with K bit-exact.
"""

import numpy as np
import pytest
import torch

import oracle


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_value(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    np.testing.assert_array_equal(got[ok], want[ok])
    np.testing.assert_array_equal(np.signbit(got[ok]), np.signbit(want[ok]))   # -0 at 0x80
    assert oracle.e4m3_value(np.array([0x7E]))[0] == 448.0


def test_encode_hand_examples():
    y = np.array([1.0625, 1.1875, 448.0, -448.0, 2.0 ** -10, 1.5 * 2.0 ** -10, -0.0, -(2.0 ** -11),
                  0.0, 3 * 2.0 ** -10, 2.0 ** -6, 7 * 2.0 ** -9 + 2.0 ** -10])
    want = [0x38, 0x3A, 0x7E, 0xFE, 0x00, 0x01, 0x80, 0x80, 0x00, 0x02, 0x08, 0x08]
    # 1.0625: tie between 1.0 (m=0) and 1.125 (m=1) -> even; 1.1875: tie -> 1.25 (m=2);
    # 2^-10: tie between 0 and the smallest subnormal -> 0; 3*2^-10: tie -> 2*2^-9 (even);
    # 7.5*2^-9: tie between the largest subnormal and 2^-6 -> 2^-6 (code 8, even)
    np.testing.assert_array_equal(oracle.e4m3_encode(y), np.array(want, dtype=np.uint8))


def test_encode_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    # fp32 values across the whole range, plus every midpoint between neighbours
    vals = np.concatenate([
        rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 8, 20000),
    ]).astype(np.float32)
    pos = oracle.e4m3_value(np.arange(0x7F))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    vals = np.concatenate([vals, mids, -mids, pos.astype(np.float32)])
    vals = np.clip(vals, -448, 448)
    want = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.e4m3_encode(vals.astype(np.float64)), want)


def test_scale_exponent_matches_its_definition():
    rng = np.random.default_rng(1)
    amax = np.concatenate([np.abs(rng.standard_normal(3000)) * 2.0 ** rng.integers(-130, 127, 3000),
                           [0.0, 448.0, 448.0 * (1 + 2 ** -20), 1.75, 1.75 * (1 + 2 ** -20), 2.0 ** -140,
                            3.3e38]])
    got = oracle.fp8_scale_exp(amax)
    for a, k in zip(amax, got):
        kk = -300
        while a > 448.0 * 2.0 ** kk:
            kk += 1
        assert k == min(max(kk, -117), 126), (a, k, kk)


def _bf16_values(shape, seed, spread=0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(*shape, generator=g)
    if spread:
        x = x * torch.exp2(torch.randint(-spread, spread + 1, shape[:-1] + (1,), generator=g).float())
    return x.to(torch.bfloat16).view(torch.int16).numpy()


@pytest.mark.parametrize("spread", [0, 20])
def test_block_round_trip_error_bound(spread):
    bits = _bf16_values((64, 4, 128), 2, spread)
    x = oracle.bf16_bits_to_f64(bits)
    codes, sb = oracle.quantize_fp8_blocks(x)
    assert codes.dtype == np.uint8 and sb.shape == (64, 4, 4)
    back = oracle.dequantize_fp8_blocks(codes, sb)
    k = sb.astype(np.int64) - 127
    kk = np.repeat(k, 32, axis=-1)
    bound = np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** (kk - 10.0))
    assert np.all(np.abs(back - x) <= bound)
    assert np.all(np.abs(back) <= 448.0 * 2.0 ** kk)
    # every dequantized value is exactly a bf16 value
    oracle.f64_to_bf16_bits_exact(back)
    # representable values survive unchanged
    again_codes, again_sb = oracle.quantize_fp8_blocks(back)
    np.testing.assert_array_equal(oracle.dequantize_fp8_blocks(again_codes, again_sb), back)


def test_zero_block_and_tiny_blocks():
    # the lowest block scale is 2^-117: its smallest step is 2^-9 * 2^-117 = 2^-126
    x = np.zeros((4, 32))
    x[1] = 2.0 ** -130                        # far below half a step: encodes as zero
    x[2] = 2.0 ** -126                        # exactly one step
    x[3] = 2.0 ** -127                        # half a step: tie, rounds to the even code (zero)
    x[3, 0] = 3 * 2.0 ** -127                 # one and a half steps: tie, rounds to two steps
    codes, sb = oracle.quantize_fp8_blocks(x)
    assert np.all(sb == 127 - 117)
    back = oracle.dequantize_fp8_blocks(codes, sb)
    assert np.all(codes[0] == 0) and np.all(back[0] == 0)
    assert np.all(back[1] == 0)
    assert np.all(back[2] == 2.0 ** -126)
    assert back[3, 0] == 2.0 ** -125 and np.all(back[3, 1:] == 0)


CASES = [
    # B, S, H, D, U, seq_align
    (1, 10, 4, 32, 2, 1),
    (2, 37, 5, 64, 3, 1),      # ragged S and H (pad rows and pad heads)
    (1, 16, 2, 128, 4, 1),     # U > H: ranks with only pad heads
]


def _exchange(sends):
    U = len(sends)
    return [np.stack([sends[p][r] for p in range(U)]) for r in range(U)]


@pytest.mark.parametrize("case", CASES)
def test_fp8_exchange_equals_blockwise_quantization_of_the_global_tensors(case):
    B, S, H, D, U, al = case
    L = oracle.a2a_layout(B, S, H, D, U, al, 3)
    sec, used, stride = oracle.fp8_chunk_sections(L, True)
    Q, K, V = (_bf16_values((B, S, H, D), 10 + i, 8) for i in range(3))
    S_loc = L["S_loc"]

    def shard(x, r):
        out = np.full((B, S_loc, H, D), 0x5555, dtype=np.int16)   # pad rows must never be read
        lo, hi = r * S_loc, min(S, (r + 1) * S_loc)
        if hi > lo:
            out[:, : hi - lo] = x[:, lo:hi]
        return out

    sends = [oracle.pack_seq_to_head_fp8(shard(Q, r), shard(K, r), shard(V, r), L, r) for r in range(U)]
    for s in sends:
        assert s.shape == (U, stride) and not np.any(s[:, used:])   # tail bytes zero
    recvs = _exchange(sends)

    def qdq(x):
        c, sb = oracle.quantize_fp8_blocks(oracle.bf16_bits_to_f64(x))
        return oracle.f64_to_bf16_bits_exact(oracle.dequantize_fp8_blocks(c, sb))

    H_loc = L["H_loc"]
    for r in range(U):
        q, k, v = oracle.unpack_seq_to_head_fp8(recvs[r], L, r)
        lo, hi = r * H_loc, min(H, (r + 1) * H_loc)
        for got, full, quantized in ((q, Q, True), (k, K, False), (v, V, True)):
            want = np.zeros((B, S, H_loc, D), dtype=np.int16)
            if hi > lo:
                want[:, :, : hi - lo] = qdq(full[:, :, lo:hi]) if quantized else full[:, :, lo:hi]
            np.testing.assert_array_equal(got, want)

    # head to sequence: O from every rank's heads, back to sequence shards
    O = _bf16_values((B, S, H, D), 20, 8)
    o_sends = []
    for r in range(U):
        o = np.zeros((B, S, H_loc, D), dtype=np.int16)
        lo, hi = r * H_loc, min(H, (r + 1) * H_loc)
        o[:, :, : max(hi - lo, 0)] = O[:, :, lo:hi]
        if hi - lo < H_loc:
            o[:, :, max(hi - lo, 0):] = 0x5555                       # pad heads must never be read
        o_sends.append(oracle.pack_head_to_seq_fp8(o, L, r))
    o_recvs = _exchange(o_sends)
    for r in range(U):
        got = oracle.unpack_head_to_seq_fp8(o_recvs[r], L, r)
        want = np.zeros((B, S_loc, H, D), dtype=np.int16)
        lo, hi = r * S_loc, min(S, (r + 1) * S_loc)
        if hi > lo:
            want[:, : hi - lo] = qdq(O[:, lo:hi])
        np.testing.assert_array_equal(got, want)


def test_fp8_chunk_is_smaller_than_the_16bit_chunk():
    L = oracle.a2a_layout(1, 4608, 24, 128, 2, 1, 3)
    _, used, stride = oracle.fp8_chunk_sections(L, True)
    E = L["B"] * L["S_loc"] * L["H_loc"] * L["D"]
    assert used == 4 * E + E // 16 and stride % 256 == 0 and stride - used < 256
    assert stride < 6 * E * 0.7                                          # vs 3 bf16 planes
    _, used_o, _ = oracle.fp8_chunk_sections(L, False)
    assert used_o == E + E // 32


# Block membership: which 32 elements share one scale.  A head vector of 64
# elements whose halves differ by 2^20 (and in sign) must give two distinct
# scale bytes, each half encoded against its own scale.  First half:
# x_j = (j + 1) / 8 for j = 0..31, so the block maximum is 4 and the
# exponent is the smallest k with 4 <= 448 * 2^k, i.e. k = -6 (448 * 2^-7 =
# 3.5 is too small), scale byte 121; the scaled values are y_j = 8 (j + 1) =
# 8, 16, ..., 256.  Their E4M3 codes, worked out by hand from
# value = (1 + m/8) * 2^(e - 7): 8 = 2^3 is e = 10, m = 0 (0x50); between 128
# and 256 the spacing is 16, so the odd multiples of 8 there are ties that go
# to the even mantissa (136 -> 128, 152 -> 160, 168 -> 160, 184 -> 192,
# 200 -> 192, 216 -> 224, 232 -> 224, 248 -> 256).  Second half: -x * 2^20,
# exponent 14 (scale byte 141), the same codes with the sign bit set.
HAND_CODES = [
    0x50, 0x58, 0x5C, 0x60, 0x62, 0x64, 0x66, 0x68,
    0x69, 0x6A, 0x6B, 0x6C, 0x6D, 0x6E, 0x6F, 0x70,
    0x70, 0x71, 0x72, 0x72, 0x72, 0x73, 0x74, 0x74,
    0x74, 0x75, 0x76, 0x76, 0x76, 0x77, 0x78, 0x78,
]


def _grouping_pin_holds(quantize) -> bool:
    first = np.arange(1, 33, dtype=np.float64) / 8.0
    x = np.concatenate([first, -first * 2.0 ** 20])[None, None, :]     # one [1, 1, 64] head vector
    codes, sb = quantize(x)
    want_codes = np.array(HAND_CODES + [c | 0x80 for c in HAND_CODES], dtype=np.uint8)
    return (sb.reshape(-1).tolist() == [121, 141]
            and np.array_equal(codes.reshape(-1), want_codes))


def test_block_membership_hand_table():
    assert _grouping_pin_holds(oracle.quantize_fp8_blocks)
    # the hand table is also what torch's E4M3 conversion gives for 8 (j + 1)
    y = torch.arange(8.0, 257.0, 8.0, dtype=torch.float32)
    assert torch.equal(y.to(torch.float8_e4m3fn).view(torch.uint8),
                       torch.tensor(HAND_CODES, dtype=torch.uint8))


def test_block_membership_pin_catches_a_strided_grouping():
    # planted mistake: blocks taken as every other element (a strided
    # reshape) instead of 32 consecutive ones; the pin must reject it
    def strided(x):
        x = np.asarray(x, dtype=np.float64)
        D = x.shape[-1]
        nb = D // oracle.FP8_BLOCK
        blocks = np.swapaxes(x.reshape(x.shape[:-1] + (oracle.FP8_BLOCK, nb)), -1, -2)
        k = oracle.fp8_scale_exp(np.max(np.abs(blocks), axis=-1))
        y = blocks * np.exp2(-k.astype(np.float64))[..., None]
        codes = np.swapaxes(oracle.e4m3_encode(y), -1, -2).reshape(x.shape)
        return codes, (k + 127).astype(np.uint8)

    assert not _grouping_pin_holds(strided)

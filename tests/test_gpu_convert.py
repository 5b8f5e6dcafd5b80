"""GPU parity of the converting packs (float32 planes -> bf16 / f16 send
buffer, round to nearest even), bit-exact against the oracle.

Every rank of each small layout is packed in both directions and both
formats, with inputs that mix ordinary values with rounding ties, values
just past a tie, subnormal results, overflow, signed zeros, infinities and
NaN; regions the map never reads hold a NaN pattern.  NaN outputs are
compared as NaN (their sign and payload are not fixed).  The FLUX and Qwen
shapes are checked at full size on chosen ranks.
"""

import numpy as np
import pytest
import torch

import oracle
import sequence_attention_amd as sa
from tests.gpu_util import DEV, Guarded, log

pytestmark = pytest.mark.gpu

S2H, H2S = sa.DIT_SEQ_TO_HEAD, sa.DIT_HEAD_TO_SEQ
FMT = {"bf16": (torch.bfloat16, sa.DIT_BF16), "f16": (torch.float16, sa.DIT_F16)}
NEVER_READ = np.uint32(0x7FAAAAAA)   # a NaN: any read of it would show

SPECIAL = np.array([
    0.0, -0.0, 1.0, -2.0,
    1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 1 + 2.0 ** -11 + 2.0 ** -20,   # f16 ties and past them
    1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20,      # bf16 ties and past them
    65504.0, 65520.0 - 2.0 ** -8, 65520.0, -65520.0,                   # f16 overflow edge
    2.0 ** -14, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -25, 1e-8,          # f16 subnormals
    2.0 ** -126, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -134, 2.0 ** -149,  # bf16 / f32 subnormals
    (2 - 2.0 ** -7) * 2.0 ** 127, (2 - 2.0 ** -8) * 2.0 ** 127,        # bf16 overflow edge
    (2 - 2.0 ** -23) * 2.0 ** 127, np.inf, -np.inf, np.nan,
], dtype=np.float32)


def _planes(shape, n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        x = (rng.standard_normal(shape) * 40.0).astype(np.float32)
        pick = rng.random(shape) < 0.25
        x[pick] = rng.choice(SPECIAL, size=int(pick.sum()))
        out.append(x)
    return out


def _codes(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _assert_codes(got, want, fmt):
    nan = oracle.half_is_nan(want, fmt)
    np.testing.assert_array_equal(oracle.half_is_nan(got, fmt), nan)
    np.testing.assert_array_equal(got[~nan], want[~nan])


def _device_plane(x, offset_elems=0):
    """x on the device, optionally at an address offset_elems floats past a
    256-byte boundary (to exercise the narrower vector widths)."""
    flat = torch.empty(x.size + offset_elems, dtype=torch.float32, device=DEV)
    t = flat[offset_elems:].view(*x.shape)
    t.copy_(torch.from_numpy(x))
    return t


SMALL = [
    # B, S, H, D, U, seq_align, n_planes, input offset (floats)
    (1, 256, 4, 64, 2, 1, 3, 0),     # 8 elements per thread
    (2, 37, 5, 8, 3, 1, 3, 0),       # ragged S and H
    (1, 10, 6, 12, 4, 1, 1, 0),      # D = 12: 4 per thread
    (2, 9, 3, 16, 2, 4, 3, 0),       # seq_align 4
    (1, 5, 2, 6, 5, 1, 1, 0),        # U > H, D = 6: 2 per thread
    (1, 3, 4, 3, 4, 1, 1, 0),        # a rank with only pad rows, D = 3: 1 per thread
    (1, 40, 4, 128, 2, 1, 3, 1),     # misaligned planes: 1 per thread
    (1, 40, 4, 128, 2, 1, 3, 2),     # 8-byte aligned planes: 2 per thread
    (2, 101, 7, 24, 3, 64, 3, 0),    # lcm(3, 64) alignment
]


def _random_cases(n_cases, seed=4242):
    # seeded sweep: any head size (1 to 8 floats per thread), ragged S and H,
    # U above and below H, every alignment, planes at 0, 4 and 8 bytes past
    # a 16-byte boundary
    r = np.random.default_rng(seed)
    out = []
    for _ in range(n_cases):
        D = int(r.choice([1, 2, 3, 4, 6, 8, 12, 16, 24, 64, 128]))
        out.append((int(r.integers(1, 3)), int(r.integers(1, 200)), int(r.integers(1, 9)), D, int(r.integers(1, 6)),
                    int(r.choice([1, 4, 64])), int(r.choice([1, 3])), int(r.choice([0, 1, 2]))))
    return out


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("case", SMALL + _random_cases(8))
def test_all_ranks_match_oracle(case, fmt):
    B, S, H, D, U, al, n, off = case
    tdt, code = FMT[fmt]
    L = sa.dit_a2a_layout_init(B, S, H, D, U, al, n, code)
    Lo = oracle.a2a_layout(B, S, H, D, U, al, n)
    glob = _planes((B, S, H, D), n, 300 + D)
    for r in range(U):
        log(f"pack_convert {fmt} {case} rank {r}: sequence to head")
        shards = []
        for pl in range(n):
            x = np.full((B, L.S_loc, H, D), NEVER_READ, dtype=np.uint32).view(np.float32)
            lo, hi = r * L.S_loc, min(S, (r + 1) * L.S_loc)
            if hi > lo:
                x[:, : hi - lo] = glob[pl][:, lo:hi]
            shards.append(x)
        send = Guarded((U, n, B, L.S_loc, L.H_loc, D), tdt)
        sa.dit_ulysses_pack_convert(L, S2H, r, [_device_plane(x, off) for x in shards],
                                    send=send.t)
        torch.cuda.synchronize()
        assert send.canary_ok()
        _assert_codes(_codes(send.t), oracle.pack_seq_to_head_convert(shards, Lo, r, fmt), fmt)

        log(f"pack_convert {fmt} {case} rank {r}: head to sequence")
        heads = []
        for pl in range(n):
            x = np.full((B, S, L.H_loc, D), NEVER_READ, dtype=np.uint32).view(np.float32)
            h_hi = min(H, (r + 1) * L.H_loc) - r * L.H_loc
            if h_hi > 0:
                x[:, :, :h_hi] = glob[pl][:, :, r * L.H_loc: r * L.H_loc + h_hi]
            heads.append(x)
        send = Guarded((U, n, B, L.S_loc, L.H_loc, D), tdt)
        sa.dit_ulysses_pack_convert(L, H2S, r, [_device_plane(x, off) for x in heads], send=send.t)
        torch.cuda.synchronize()
        assert send.canary_ok()
        _assert_codes(_codes(send.t), oracle.pack_head_to_seq_convert(heads, Lo, r, fmt), fmt)


FULL = [
    # name, B, S, H, D, U, seq_align, n_planes, ranks, fmt
    ("flux-qkv-bf16", 1, 4608, 24, 128, 2, 1, 3, [0, 1], "bf16"),
    ("flux-qkv-f16", 1, 4608, 24, 128, 2, 1, 3, [1], "f16"),
    ("qwen-u5-qkv-bf16", 2, 7145, 24, 128, 5, 1, 3, [4], "bf16"),   # a pad head, ragged rows
]


@pytest.mark.parametrize("case", FULL, ids=[c[0] for c in FULL])
def test_full_size_ranks_match_oracle(case):
    name, B, S, H, D, U, al, n, ranks, fmt = case
    tdt, code = FMT[fmt]
    L = sa.dit_a2a_layout_init(B, S, H, D, U, al, n, code)
    Lo = oracle.a2a_layout(B, S, H, D, U, al, n)
    for r in ranks:
        log(f"pack_convert full {name} rank {r}: sequence to head")
        shard = _planes((B, L.S_loc, H, D), n, 10 + r)
        send = sa.dit_ulysses_pack_convert(L, S2H, r, [_device_plane(x) for x in shard])
        torch.cuda.synchronize()
        _assert_codes(_codes(send), oracle.pack_seq_to_head_convert(shard, Lo, r, fmt), fmt)
        del send
        log(f"pack_convert full {name} rank {r}: head to sequence")
        heads = _planes((B, S, L.H_loc, D), n, 20 + r)
        send = sa.dit_ulysses_pack_convert(L, H2S, r, [_device_plane(x) for x in heads])
        torch.cuda.synchronize()
        _assert_codes(_codes(send), oracle.pack_head_to_seq_convert(heads, Lo, r, fmt), fmt)


def test_equals_library_conversion_then_plain_pack():
    """The fused pack equals torch's own conversion followed by the plain
    pack of the converted planes (bf16 and f16, finite inputs)."""
    B, S, H, D, U = 1, 300, 6, 64, 3
    for fmt in ("bf16", "f16"):
        tdt, code = FMT[fmt]
        L = sa.dit_a2a_layout_init(B, S, H, D, U, 1, 3, code)
        xs = [torch.randn(B, L.S_loc, H, D, device=DEV) * 100 for _ in range(3)]
        log(f"pack_convert vs torch conversion + pack ({fmt})")
        fused = sa.dit_ulysses_pack_convert(L, S2H, 1, xs)
        plain = sa.dit_ulysses_pack(L, S2H, 1, [x.to(tdt) for x in xs])
        torch.cuda.synchronize()
        assert torch.equal(fused.view(torch.int16), plain.view(torch.int16))


def test_rejects_a_32_bit_send_buffer():
    L = sa.dit_a2a_layout_init(1, 8, 2, 8, 2, 1, 1, sa.DIT_F32)
    x = torch.zeros(1, L.S_loc, 2, 8, device=DEV)
    with pytest.raises(ValueError):
        sa.dit_ulysses_pack_convert(L, S2H, 0, [x])

"""GPU parity of the FP8 Ulysses exchange (bit-exact codes, scale bytes and
decoded values) and of attention on the decoded operands.

Every rank of the group is simulated on the one GPU; each send buffer is
compared byte for byte with the oracle's (codes, scale bytes, K bits, zero
tails), each decoded plane bit for bit.  Inputs span many binades per row so
that the blocks take different exponents, and a targeted case walks every
E4M3 code, rounding ties, subnormal codes, negative zero and the clamped
exponents through the hardware conversions.
"""

import numpy as np
import pytest
import torch

import oracle
import sequence_attention_amd as sa
from tests.gpu_util import DEV, Guarded, bits, f64, log, simulate_all_to_all

pytestmark = pytest.mark.gpu

S2H, H2S = sa.DIT_SEQ_TO_HEAD, sa.DIT_HEAD_TO_SEQ
GARBAGE = -21846  # 0xAAAA in pad rows / heads that must never be read


def _rand(shape, seed, spread=8):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(*shape, generator=g)
    if spread:
        x = x * torch.exp2(torch.randint(-spread, spread + 1, shape[:-1] + (shape[-1] // 32, 1),
                                         generator=g).float()).repeat_interleave(32, -1).reshape(shape)
    return x.to(torch.bfloat16)


def _layouts(B, S, H, D, U, al):
    return (sa.dit_a2a_layout_init(B, S, H, D, U, al, 3), sa.dit_a2a_layout_init(B, S, H, D, U, al, 1),
            oracle.a2a_layout(B, S, H, D, U, al, 3))


CASES = [
    # B, S, H, D, U, seq_align
    (1, 256, 4, 64, 2, 1),
    (2, 37, 5, 64, 3, 1),      # ragged S and H: pad rows and pad heads
    (1, 16, 2, 128, 4, 1),     # U > H: ranks holding only pad heads
    (1, 4608, 24, 128, 2, 1),  # FLUX 1024x1024 shard shape
    (1, 7145, 24, 128, 5, 1),  # Qwen-like, sequence and head padding
    (1, 64, 2, 32, 2, 1),      # D = 32: one scale block per head
]


def _random_cases(n_cases, seed=53):
    # seeded sweep: heads of 1 to 4 scale blocks, ragged S and H, U above
    # and below H, every alignment
    r = np.random.default_rng(seed)
    return [(int(r.integers(1, 3)), int(r.integers(1, 300)), int(r.integers(1, 9)), int(r.choice([32, 64, 96, 128])),
             int(r.integers(1, 6)), int(r.choice([1, 4, 64]))) for _ in range(n_cases)]


@pytest.mark.parametrize("case", CASES + _random_cases(10))
def test_all_ranks_fp8_exchange_matches_oracle(case):
    B, S, H, D, U, al = case
    log(f"fp8 exchange {case}")
    L3, L1, Lo = _layouts(B, S, H, D, U, al)
    S_loc, H_loc = L3.S_loc, L3.H_loc
    stride = sa.dit_a2a_fp8_bytes_per_peer(L3, S2H)
    glob = [_rand((B, S, H, D), 500 + pl) for pl in range(3)]
    sends = []
    for r in range(U):
        shard = []
        for x in glob:
            t = torch.empty((B, S_loc, H, D), dtype=torch.bfloat16)
            t.view(torch.int16).fill_(GARBAGE)
            lo, hi = r * S_loc, min(S, (r + 1) * S_loc)
            if hi > lo:
                t[:, : hi - lo] = x[:, lo:hi]
            shard.append(t)
        send = Guarded((U, stride), torch.uint8, fill_bits=None)
        sa.dit_ulysses_pack_fp8(L3, S2H, r, [t.to(DEV) for t in shard], send=send.t)
        torch.cuda.synchronize()
        assert send.canary_ok()
        want = oracle.pack_seq_to_head_fp8(*[bits(t) for t in shard], Lo, r)
        got = send.t.cpu().numpy()
        np.testing.assert_array_equal(got, want)
        sends.append(send.t)
    recvs = simulate_all_to_all(sends)
    heads = []
    for r in range(U):
        outs = [Guarded((B, S, H_loc, D), torch.bfloat16) for _ in range(3)]
        sa.dit_ulysses_unpack_fp8(L3, S2H, r, recvs[r], out=[o.t for o in outs])
        torch.cuda.synchronize()
        want = oracle.unpack_seq_to_head_fp8(recvs[r].cpu().numpy(), Lo, r)
        for pl in range(3):
            assert outs[pl].canary_ok()
            np.testing.assert_array_equal(bits(outs[pl].t), want[pl])
        heads.append(outs[0].t)                                    # Q stands in for O below
    # head to sequence with O
    Lo1 = dict(Lo, n_planes=1)
    stride1 = sa.dit_a2a_fp8_bytes_per_peer(L1, H2S)
    sends = []
    for r in range(U):
        o = heads[r].clone()
        lo = r * H_loc
        if H - lo < H_loc:                                         # pad heads never read
            o[:, :, max(H - lo, 0):].view(torch.int16).fill_(GARBAGE)
        send = Guarded((U, stride1), torch.uint8)
        sa.dit_ulysses_pack_fp8(L1, H2S, r, [o], send=send.t)
        torch.cuda.synchronize()
        assert send.canary_ok()
        np.testing.assert_array_equal(send.t.cpu().numpy(), oracle.pack_head_to_seq_fp8(bits(o), Lo1, r))
        sends.append(send.t)
    recvs = simulate_all_to_all(sends)
    for r in range(U):
        out = Guarded((B, S_loc, H, D), torch.bfloat16)
        sa.dit_ulysses_unpack_fp8(L1, H2S, r, recvs[r], out=[out.t])
        torch.cuda.synchronize()
        assert out.canary_ok()
        np.testing.assert_array_equal(bits(out.t), oracle.unpack_head_to_seq_fp8(recvs[r].cpu().numpy(), Lo1, r))


def test_every_code_tie_and_exponent_through_the_hardware_conversion():
    """One head of 32-element blocks built to hit every E4M3 magnitude and
    every rounding midpoint, in both signs, under block exponents from the
    lower clamp to large ones, plus zero blocks and negative zeros."""
    log("fp8 code sweep")
    pos = oracle.e4m3_value(np.arange(0x7F))
    mids = (pos[1:] + pos[:-1]) / 2
    vals = np.concatenate([pos, mids, -pos, -mids])
    rows = []
    for k in (-117, -100, -20, -3, 0, 5, 40, 100):
        v = np.concatenate([vals, np.zeros(32 - len(vals) % 32)]) * 2.0 ** k
        blocks = v.reshape(-1, 32)
        blocks[:, 0] = 448.0 * 2.0 ** k                            # pin the block exponent to k
        rows.append(blocks)
    blocks = np.concatenate(rows)
    blocks = np.concatenate([blocks, np.zeros((4, 32)), -np.zeros((4, 32))])
    tiny = np.full((4, 32), 2.0 ** -127)                           # below the lowest clamp's step
    tiny[:, 1] = 3 * 2.0 ** -127
    blocks = np.concatenate([blocks, tiny])
    n_rows = -(-blocks.shape[0] // 4) * 4
    blocks = np.concatenate([blocks, np.ones((n_rows - blocks.shape[0], 32))])
    x = torch.from_numpy(blocks.reshape(-1, 1, 4 * 32).astype(np.float32)).to(torch.bfloat16)
    assert torch.equal(x.double(),
                       torch.from_numpy(blocks.reshape(-1, 1, 128)))  # all values exact in bf16
    S = x.shape[0]
    L = sa.dit_a2a_layout_init(1, S, 1, 128, 1, 1, 1)
    Lo = oracle.a2a_layout(1, S, 1, 128, 1, 1, 1)
    o = x.reshape(1, S, 1, 128).to(DEV)
    send = sa.dit_ulysses_pack_fp8(L, H2S, 0, [o])
    out = sa.dit_ulysses_unpack_fp8(L, H2S, 0, send)[0]
    torch.cuda.synchronize()
    np.testing.assert_array_equal(send.cpu().numpy(), oracle.pack_head_to_seq_fp8(bits(o), Lo, 0))
    np.testing.assert_array_equal(bits(out), oracle.unpack_head_to_seq_fp8(send.cpu().numpy(), Lo, 0))


def _elem_bound(x):
    """Per-element bound of the FP8 round trip: max(2^-4 |x|, 2^(k-10))."""
    _, sb = oracle.quantize_fp8_blocks(x)
    k = np.repeat(sb.astype(np.int64) - 127, 32, axis=-1).reshape(x.shape)
    return np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** (k - 10.0))


def test_fp8_ulysses_step_attention_within_bounds():
    """Pack (FP8) -> exchange -> unpack -> attention on every rank equals the
    oracle's attention on the decoded operands (bf16 tolerance), and the
    decoded operands move the exact result by no more than the bound that
    follows from the per-element FP8 error: with |dq| <= bq elementwise,
    every score moves by at most ds_i = scale * max_j sum_d bq_id |k_jd|, so
    |dLSE_i| <= ds_i and |dO_i| <= (e^(2 ds_i) - 1) max|v'| + max|dv|."""
    B, S, H, D, U = 1, 1024, 4, 128, 2
    log(f"fp8 ulysses step B={B} S={S} H={H} D={D} U={U}")
    L3, L1, Lo = _layouts(B, S, H, D, U, 1)
    q, k, v = (_rand((B, S, H, D), 900 + i, 0) for i in range(3))
    sends = [sa.dit_ulysses_pack_fp8(L3, S2H, r, [t[:, r * L3.S_loc:(r + 1) * L3.S_loc].contiguous().to(DEV)
                                                  for t in (q, k, v)]) for r in range(U)]
    recvs = simulate_all_to_all(sends)
    scale = 1.0 / np.sqrt(D)
    for r in range(U):
        qr, kr, vr = sa.dit_ulysses_unpack_fp8(L3, S2H, r, recvs[r])
        o, lse = sa.dit_attn_fwd(qr, kr, vr)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.attention(f64(qr), f64(kr), f64(vr), scale)
        assert np.max(np.abs(f64(o) - o_ref)) <= 1e-2
        assert np.max(np.abs(lse.double().cpu().numpy() - lse_ref)) <= 1e-3
        hs = slice(r * L3.H_loc, (r + 1) * L3.H_loc)
        q16, k16, v16 = f64(q[:, :, hs]), f64(k[:, :, hs]), f64(v[:, :, hs])
        assert np.array_equal(f64(kr), k16)                                 # K exchanged exactly
        o16, lse16 = oracle.attention(q16, k16, v16, scale)
        bq, bv = _elem_bound(q16), _elem_bound(v16)
        assert np.all(np.abs(f64(qr) - q16) <= bq) and np.all(np.abs(f64(vr) - v16) <= bv)
        # ds[b, i, h] = scale * max_j sum_d bq[b,i,h,d] |k[b,j,h,d]|
        ds = scale * np.einsum("bihd,bjhd->bhij", bq, np.abs(k16)).max(axis=-1)   # [B, H, S]
        assert np.all(np.abs(lse_ref - lse16) <= ds + 1e-12)
        o_bound = (np.expm1(2 * ds) * np.max(np.abs(f64(vr))) + np.max(bv)).transpose(0, 2, 1)[..., None]
        assert np.all(np.abs(o_ref - o16) <= o_bound + 1e-12)

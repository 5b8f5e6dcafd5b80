"""GPU parity of the padding-free (uneven) Ulysses maps and the Ring
Anything pad / trim (bit-exact).

Every rank of the group is simulated on the one GPU: pack on each rank, the
exchange with per-peer split sizes as device slicing, unpack on each rank.
Each buffer is compared with the oracle's on raw bit patterns, each unpacked
plane with the head window (or the row window) of the global tensor, and
the head-to-sequence direction is run back to recover every rank's shard.
Outputs carry a canary band past their end; inputs that must not be read are
not allocated at all (there are no pad rows or heads in these maps).
"""

import numpy as np
import pytest
import torch

import oracle
import sequence_attention_amd as sa
from tests.gpu_util import DEV, Guarded, bits, log

pytestmark = pytest.mark.gpu

S2H, H2S = sa.DIT_SEQ_TO_HEAD, sa.DIT_HEAD_TO_SEQ


def _rand(shape, seed, dtype):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g).to(dtype)


def _split(total, U):
    return [total // U + (1 if r < total % U else 0) for r in range(U)]


def _exchange(sends, sizes):
    """recv_r = concat over p of the part of send_p addressed to r."""
    U = len(sends)
    recvs = []
    for r in range(U):
        parts = []
        for p in range(U):
            off = sum(sizes[p][:r])
            parts.append(sends[p][off:off + sizes[p][r]])
        recvs.append(torch.cat(parts).contiguous())
    return recvs


CASES = [
    # B, S, H, D, U, n_planes, dtype, seq counts, head counts
    (1, 4481, 24, 128, 4, 3, torch.bfloat16, None, None),         # FLUX 1008x1008: S = 512 + 63*63
    (1, 1030, 24, 128, 5, 1, torch.bfloat16, None, None),         # uneven S and uneven heads (24 / 5)
    (2, 37, 5, 8, 3, 3, torch.bfloat16, None, None),              # ragged everything, 16-byte heads
    (1, 9, 5, 6, 3, 3, torch.bfloat16, [0, 4, 5], [2, 0, 3]),     # ranks without rows / heads, 12-byte heads
    (2, 17, 7, 4, 4, 1, torch.float32, [8, 1, 0, 8], None),       # fp32, skewed counts
    (1, 33, 6, 3, 2, 3, torch.float16, [20, 13], [1, 5]),         # fp16, odd D (2-byte vectors)
    (1, 64, 4, 64, 1, 3, torch.bfloat16, None, None),             # U = 1: identity maps
]


def _random_cases(n_cases, seed=91):
    # seeded sweep: random per-rank sequence and head counts (ranks with no
    # rows or no heads included) or the default split, any head size, the
    # three dtypes
    r = np.random.default_rng(seed)
    out = []
    for _ in range(n_cases):
        B, S, H, U = int(r.integers(1, 3)), int(r.integers(1, 200)), int(r.integers(1, 9)), int(r.integers(1, 6))
        D = int(r.choice([1, 2, 3, 4, 8, 16, 24, 64]))
        n = int(r.choice([1, 3]))
        dt = [torch.bfloat16, torch.float16, torch.float32][int(r.integers(0, 3))]
        seq = [int(x) for x in r.multinomial(S, r.dirichlet(np.ones(U)))] if r.random() < 0.6 else None
        heads = [int(x) for x in r.multinomial(H, r.dirichlet(np.ones(U)))] if r.random() < 0.6 else None
        out.append((B, S, H, D, U, n, dt, seq, heads))
    return out


@pytest.mark.parametrize("case", CASES + _random_cases(12))
def test_all_ranks_round_trip_matches_oracle(case):
    B, S, H, D, U, n, dt, sc, hc = case
    log(f"uneven all-ranks {case}")
    L = sa.dit_a2a_uneven_init(B, S, H, D, U, n, dt, sc, hc)
    sc, hc = L.counts()
    so, ho = L.offsets()
    glob = [_rand((B, S, H, D), 300 + pl, dt) for pl in range(n)]

    # sequence-to-head
    sends, sizes = [], []
    for r in range(U):
        shard = [g[:, so[r]:so[r + 1]].contiguous() for g in glob]
        s_cnt, _ = sa.dit_a2a_uneven_sizes(L, S2H, r)
        send = Guarded((sum(s_cnt),), dt)
        sa.dit_ulysses_pack_uneven(L, S2H, r, [x.to(DEV) for x in shard], send=send.t)
        torch.cuda.synchronize()
        assert send.canary_ok()
        want = oracle.pack_seq_to_head_uneven([bits(x) for x in shard], sc, hc, r)
        np.testing.assert_array_equal(bits(send.t), want)
        sends.append(send.t)
        sizes.append(s_cnt)
    recvs = _exchange(sends, sizes)
    heads = []
    for r in range(U):
        outs = [Guarded((B, S, hc[r], D), dt) for _ in range(n)]
        sa.dit_ulysses_unpack_uneven(L, S2H, r, recvs[r], out=[o.t for o in outs])
        torch.cuda.synchronize()
        want = oracle.unpack_seq_to_head_uneven(bits(recvs[r]), B, D, n, sc, hc, r)
        for pl in range(n):
            assert outs[pl].canary_ok()
            np.testing.assert_array_equal(bits(outs[pl].t), want[pl])
            np.testing.assert_array_equal(bits(outs[pl].t), bits(glob[pl][:, :, ho[r]:ho[r + 1]]))
        heads.append([o.t for o in outs])

    # head-to-sequence back to the shards
    sends, sizes = [], []
    for r in range(U):
        s_cnt, _ = sa.dit_a2a_uneven_sizes(L, H2S, r)
        send = Guarded((sum(s_cnt),), dt)
        sa.dit_ulysses_pack_uneven(L, H2S, r, heads[r], send=send.t)
        torch.cuda.synchronize()
        assert send.canary_ok()
        want = oracle.pack_head_to_seq_uneven([bits(x) for x in heads[r]], sc, hc, r)
        np.testing.assert_array_equal(bits(send.t), want)
        sends.append(send.t)
        sizes.append(s_cnt)
    recvs = _exchange(sends, sizes)
    for r in range(U):
        outs = [Guarded((B, sc[r], H, D), dt) for _ in range(n)]
        sa.dit_ulysses_unpack_uneven(L, H2S, r, recvs[r], out=[o.t for o in outs])
        torch.cuda.synchronize()
        want = oracle.unpack_head_to_seq_uneven(bits(recvs[r]), B, D, n, sc, hc, r)
        for pl in range(n):
            assert outs[pl].canary_ok()
            np.testing.assert_array_equal(bits(outs[pl].t), want[pl])
            np.testing.assert_array_equal(bits(outs[pl].t), bits(glob[pl][:, so[r]:so[r + 1]]))


@pytest.mark.parametrize("B,S,H,D,U,n", [(1, 4096, 24, 128, 4, 3), (2, 64, 4, 64, 2, 1)])
def test_even_counts_equal_the_padded_maps(B, S, H, D, U, n):
    """Counts that divide evenly: the padding-free buffers are the padded
    layout's buffers bit for bit (no pad rows or heads exist)."""
    log(f"uneven vs padded B={B} S={S} H={H} D={D} U={U} n={n}")
    dt = torch.bfloat16
    Lu = sa.dit_a2a_uneven_init(B, S, H, D, U, n, dt)
    Lp = sa.dit_a2a_layout_init(B, S, H, D, U, 1, n, dt)
    for r in (0, U - 1):
        shard = [_rand((B, S // U, H, D), 40 + pl, dt).to(DEV) for pl in range(n)]
        a = sa.dit_ulysses_pack_uneven(Lu, S2H, r, shard)
        b = sa.dit_ulysses_pack(Lp, S2H, r, shard)
        planes = [_rand((B, S, H // U, D), 50 + pl, dt).to(DEV) for pl in range(n)]
        c = sa.dit_ulysses_pack_uneven(Lu, H2S, r, planes)
        d = sa.dit_ulysses_pack(Lp, H2S, r, planes)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.reshape(-1).view(torch.int16))
        assert torch.equal(c.view(torch.int16), d.reshape(-1).view(torch.int16))


@pytest.mark.parametrize("case", [
    # B, H, D, n, dtype, per-rank lengths
    (1, 24, 128, 2, torch.bfloat16, [1121, 1120, 1120, 1120]),   # FLUX 1008x1008 K and V over a ring of 4
    (2, 3, 8, 2, torch.bfloat16, [5, 3, 0, 4]),
    (1, 2, 4, 1, torch.float32, [7]),
    (2, 1, 3, 2, torch.float16, [2, 6]),
])
def test_ring_anything_pad_gather_trim(case):
    B, H, D, n, dt, counts = case
    log(f"ring anything {case}")
    U, S = len(counts), sum(counts)
    L = sa.dit_a2a_uneven_init(B, S, H, D, U, n, dt, counts)
    so, _ = L.offsets()
    glob = [_rand((B, S, H, D), 700 + pl, dt) for pl in range(n)]
    padded = []
    for r in range(U):
        shard = [g[:, so[r]:so[r + 1]].contiguous() for g in glob]
        buf = Guarded((n, B, L.S_max, H, D), dt, fill_bits=0x7FAA if dt != torch.float32 else 0x7FAAAAAA)
        sa.dit_ring_anything_pad(L, r, [x.to(DEV) for x in shard], send=buf.t)
        torch.cuda.synchronize()
        assert buf.canary_ok()
        want = oracle.ring_anything_pad([bits(x) for x in shard], L.S_max)
        np.testing.assert_array_equal(bits(buf.t), want)                 # pad rows written as zeros
        padded.append(buf.t)
    gathered = torch.stack(padded).contiguous()                           # the all-gather
    outs = [Guarded((B, S, H, D), dt) for _ in range(n)]
    sa.dit_ring_anything_trim(L, gathered, out=[o.t for o in outs])
    torch.cuda.synchronize()
    want = oracle.ring_anything_trim(bits(gathered), counts)
    for pl in range(n):
        assert outs[pl].canary_ok()
        np.testing.assert_array_equal(bits(outs[pl].t), want[pl])
        np.testing.assert_array_equal(bits(outs[pl].t), bits(glob[pl]))


def test_ring_anything_attention_equals_attention_on_the_sequence():
    """Attention over the trimmed K/V equals attention over the concatenated
    sequence (the trim is exact), and equals the ring over the uneven
    per-rank chunks merged hop by hop within the bf16 tolerance."""
    counts = [1121, 1120, 1120, 1120]
    B, H, D, S = 1, 4, 128, sum(counts)
    log(f"ring anything attention counts={counts}")
    dt = torch.bfloat16
    L = sa.dit_a2a_uneven_init(B, S, H, D, len(counts), 2, dt, counts)
    so, _ = L.offsets()
    q = _rand((B, 256, H, D), 1, dt).to(DEV)
    k, v = _rand((B, S, H, D), 2, dt).to(DEV), _rand((B, S, H, D), 3, dt).to(DEV)
    padded = [sa.dit_ring_anything_pad(L, r, [k[:, so[r]:so[r + 1]].contiguous(),
                                              v[:, so[r]:so[r + 1]].contiguous()])
              for r in range(len(counts))]
    kt, vt = sa.dit_ring_anything_trim(L, torch.stack(padded).contiguous())
    o_full, lse_full = sa.dit_attn_fwd(q, k, v)
    o_trim, lse_trim = sa.dit_attn_fwd(q, kt, vt)
    o_acc = torch.empty_like(o_full)
    lse_acc = torch.full_like(lse_full, float("-inf"))
    for r in range(len(counts)):
        sa.dit_attn_fwd_merge(q, k[:, so[r]:so[r + 1]].contiguous(), v[:, so[r]:so[r + 1]].contiguous(),
                              o_acc, lse_acc)
    torch.cuda.synchronize()
    assert torch.equal(kt, k) and torch.equal(vt, v)
    assert torch.equal(o_trim, o_full) and torch.equal(lse_trim, lse_full)
    assert (o_acc.float() - o_full.float()).abs().max().item() <= 1e-2
    assert (lse_acc - lse_full).abs().max().item() <= 1e-3

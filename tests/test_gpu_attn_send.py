"""GPU parity of dit_attn_fwd_send: attention whose O goes straight into
the head-to-sequence send buffer.

Bit-exact against the unfused pair it replaces (dit_attn_fwd_ws with the
same workspace, then dit_ulysses_pack of O, head to sequence), on every
rank of ragged layouts (pad rows over one or several peers, pad heads, a
rank with only pad heads, U = 1), and within the attention tolerance
against the oracle's attention followed by the oracle's pack
(bf16 O <= 1e-2, LSE <= 1e-3).  V carries nonzero data in pad heads, so
the zeros of the pad heads come from the store, not from the data.  FLUX
and the padded Qwen ranks are checked at full size, bitwise against the
unfused pair and on sampled rows against the oracle.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import sequence_attention_amd as sa
from tests.gpu_util import DEV, Guarded, log

pytestmark = pytest.mark.gpu

H2S = sa.DIT_HEAD_TO_SEQ


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g).to(torch.bfloat16)


def _unfused(q, k, v, L, rank, scale):
    o, lse = sa.dit_attn_fwd(q, k, v, scale=scale)
    send = sa.dit_ulysses_pack(L, H2S, rank, [o])
    return send, lse


def _fused(q, k, v, L, rank, scale):
    send = Guarded((L.U, 1, L.B, L.S_loc, L.H_loc, L.D), torch.bfloat16, fill_bits=0x7FC0)
    lse = Guarded((L.B, L.H_loc, L.S), torch.float32, fill_bits=0x7FC00000)
    sa.dit_attn_fwd_send(q, k, v, L, rank, send=send.t, lse=lse.t, scale=scale)
    torch.cuda.synchronize()
    assert send.canary_ok() and lse.canary_ok(), "write past the end of an output"
    return send.t, lse.t


def _bits(t):
    return t.detach().cpu().view(torch.int16 if t.element_size() == 2 else torch.int32)


CASES = [
    # B, S, H, D, U, seq_align, Skv (None: = S)
    (1, 600, 6, 128, 2, 1, None),     # even split
    (2, 601, 8, 128, 4, 1, None),     # 3 pad rows on the last peer
    (1, 300, 5, 128, 2, 1, None),     # a pad head on rank 1
    (1, 130, 3, 64, 4, 1, None),      # U > H: ranks with only pad heads, D = 64
    (1, 70, 4, 128, 4, 64, None),     # seq_align 64: S_loc 32, pad rows on peers 2 and 3
    (2, 257, 4, 64, 1, 1, None),      # U = 1: the buffer is O itself
    (1, 520, 4, 128, 2, 1, 777),      # more keys than queries (joint attention)
]


def _random_cases(n_cases, seed=67):
    # seeded sweep: ragged S and H, U above and below H, both head sizes,
    # both alignments, key counts other than S
    r = np.random.default_rng(seed)
    out = []
    for _ in range(n_cases):
        S = int(r.integers(1, 700))
        skv = None if r.random() < 0.5 else int(r.integers(1, 900))
        out.append((int(r.integers(1, 3)), S, int(r.integers(1, 9)), int(r.choice([64, 128])), int(r.integers(1, 6)),
                    int(r.choice([1, 64])), skv))
    return out


@pytest.mark.parametrize("case", CASES + _random_cases(8))
def test_all_ranks_bitwise_and_oracle(case):
    B, S, H, D, U, al, Skv = case
    Skv = S if Skv is None else Skv
    L = sa.dit_a2a_layout_init(B, S, H, D, U, al, 1, torch.bfloat16)
    Lo = oracle.a2a_layout(B, S, H, D, U, al, 1)
    scale = 1.0 / math.sqrt(D)
    for r in range(U):
        log(f"attn_fwd_send {case} rank {r}")
        q = _rand((B, S, L.H_loc, D), 10 + r)
        k = _rand((B, Skv, L.H_loc, D), 20 + r)
        v = _rand((B, Skv, L.H_loc, D), 30 + r)
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        send, lse = _fused(qd, kd, vd, L, r, scale)
        ref_send, ref_lse = _unfused(qd, kd, vd, L, r, scale)
        torch.cuda.synchronize()
        assert torch.equal(_bits(send), _bits(ref_send))
        assert torch.equal(_bits(lse), _bits(ref_lse))
        ro, rl = oracle.attention(q.float().numpy(), k.float().numpy(), v.float().numpy(), scale)
        want = oracle.pack_head_to_seq([ro], Lo, r)
        got = send.float().cpu().numpy()
        assert np.abs(got - want).max() <= 1e-2
        assert np.abs(lse.cpu().numpy() - rl).max() <= 1e-3
        # pads are exact zeros: rows past S and heads past H
        zero = np.ones(want.shape, dtype=bool)
        for p in range(U):
            for s in range(L.S_loc):
                if p * L.S_loc + s < S:
                    zero[p, :, :, s, : max(0, min(L.H_loc, H - r * L.H_loc))] = False
        assert np.all(_bits(send).numpy()[zero] == 0)


def test_empty_keys_write_zeros_and_minus_inf():
    B, S, H, D, U = 1, 70, 4, 128, 2
    L = sa.dit_a2a_layout_init(B, S, H, D, U, 1, 1, torch.bfloat16)
    q = _rand((B, S, L.H_loc, D), 1).to(DEV)
    kv = torch.empty((B, 0, L.H_loc, D), dtype=torch.bfloat16, device=DEV)
    log("attn_fwd_send empty keys")
    send, lse = _fused(q, kv, kv, L, 1, 0.1)
    assert torch.count_nonzero(_bits(send)) == 0
    assert torch.all(lse.cpu() == -math.inf)


FULL = [
    # name, B, S, H, D, U, ranks
    ("flux", 1, 4608, 24, 128, 2, [0, 1]),
    ("qwen-u4", 2, 7145, 24, 128, 4, [3]),     # 3 pad rows
    ("qwen-u5", 2, 7145, 24, 128, 5, [4]),     # a pad head
]


@pytest.mark.parametrize("case", FULL, ids=[c[0] for c in FULL])
def test_full_size_bitwise_and_sampled_rows(case):
    name, B, S, H, D, U, ranks = case
    L = sa.dit_a2a_layout_init(B, S, H, D, U, 1, 1, torch.bfloat16)
    Lo = oracle.a2a_layout(B, S, H, D, U, 1, 1)
    scale = 1.0 / math.sqrt(D)
    rows = np.unique(np.concatenate([np.arange(0, S, 997), [S - 1, L.S_loc - 1, L.S_loc]]))
    rows = rows[rows < S]
    for r in ranks:
        log(f"attn_fwd_send full {name} rank {r}")
        q = _rand((B, S, L.H_loc, D), 40 + r)
        k = _rand((B, S, L.H_loc, D), 50 + r)
        v = _rand((B, S, L.H_loc, D), 60 + r)
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        send, lse = _fused(qd, kd, vd, L, r, scale)
        ref_send, ref_lse = _unfused(qd, kd, vd, L, r, scale)
        torch.cuda.synchronize()
        assert torch.equal(_bits(send), _bits(ref_send))
        assert torch.equal(_bits(lse), _bits(ref_lse))
        ro, rl = oracle.attention(q.float().numpy(), k.float().numpy(), v.float().numpy(), scale,
                                  rows=rows)
        got = send.float().cpu().numpy()
        valid_heads = max(0, min(L.H_loc, H - r * L.H_loc))
        for i, t in enumerate(rows):
            p, s = divmod(int(t), L.S_loc)
            g = got[p, 0, :, s]                       # [B, H_loc, D]
            want = ro[:, i].copy()                    # [B, H_loc, D]
            want[:, valid_heads:] = 0.0
            assert np.abs(g - want).max() <= 1e-2
            assert np.abs(lse.cpu().numpy()[:, :, t] - rl[:, :, i]).max() <= 1e-3

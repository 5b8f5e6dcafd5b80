"""GPU parity of dit_attn_fwd_a2a: attention that reads Q, K and V from the
packed sequence-to-head receive buffer and stores O into the
head-to-sequence send buffer.

Bit-exact against the unfused chain it replaces (dit_ulysses_unpack of the
receive buffer, then dit_attn_fwd_send with the same workspace setting), on
every rank of ragged layouts: S_loc not a multiple of the 64-key block (key
blocks that straddle two source peers) and S_loc a multiple of it (the
kernel form without the peer select), pad rows on the last peers, pad
heads, U = 1, seq_align 64; with and without the workspace that splits the
last round.  The receive buffers are random everywhere, pad rows and pad
heads included, so nothing of the pads may leak into O or LSE.  Against the
oracle (its unpack, attention and pack) within the attention tolerance
(bf16 O <= 1e-2, LSE <= 1e-3) on the small layouts; FLUX and the padded
Qwen rank at full size bitwise against the unfused chain.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import sequence_attention_amd as sa
from tests.gpu_util import DEV, Guarded, log

pytestmark = pytest.mark.gpu

S2H = sa.DIT_SEQ_TO_HEAD


def _recv(L, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(L.U * L.elems_per_peer, generator=g).to(torch.bfloat16)


def _bits(t):
    return t.detach().cpu().view(torch.int16 if t.element_size() == 2 else torch.int32)


def _fused(recv, L, rank, workspace):
    n_out = L.U * (L.elems_per_peer // 3)
    send = Guarded((L.U, 1, L.B, L.S_loc, L.H_loc, L.D), torch.bfloat16, fill_bits=0x7FC0)
    lse = Guarded((L.B, L.H_loc, L.S), torch.float32, fill_bits=0x7FC00000)
    assert send.n == n_out
    sa.dit_attn_fwd_a2a(recv, L, rank, send=send.t, lse=lse.t, workspace=workspace)
    torch.cuda.synchronize()
    assert send.canary_ok() and lse.canary_ok(), "write past the end of an output"
    return send.t, lse.t


def _unfused(recv, L, L1, rank, workspace):
    B, S, H, D = L.B, L.S, L.H_loc, L.D
    planes = [torch.empty((B, S, H, D), dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    sa.dit_ulysses_unpack(L, S2H, rank, recv, out=planes)
    return sa.dit_attn_fwd_send(planes[0], planes[1], planes[2], L1, rank, workspace=workspace)


CASES = [
    # B, S, H, D, U, seq_align
    (1, 600, 6, 128, 2, 1),     # S_loc 300: blocks straddle the peer boundary
    (2, 601, 8, 128, 4, 1),     # S_loc 151, 3 pad rows on the last peer
    (1, 300, 5, 128, 2, 1),     # a pad head on rank 1
    (1, 130, 3, 64, 2, 1),      # S_loc 65, D = 64
    (1, 333, 4, 128, 4, 64),    # seq_align 64: S_loc 96, pad rows over two peers
    (2, 257, 4, 64, 1, 1),      # U = 1
    (1, 1000, 4, 64, 3, 1),     # three peers, S_loc 334
    (1, 256, 4, 128, 2, 1),     # S_loc 128: chunks of whole key blocks (no peer select)
    (2, 384, 3, 64, 3, 1),      # S_loc 128, three peers, D = 64
    (1, 500, 5, 128, 4, 64),    # seq_align 64: S_loc 128, pad rows on the last peer
]


def _random_cases(n_cases, seed=61):
    # seeded sweep: chunks of 64 to ~200 rows (whole key blocks or not),
    # pad rows and pad heads, both head sizes, U = 1..4
    r = np.random.default_rng(seed)
    out = []
    for _ in range(n_cases):
        U = int(r.integers(1, 5))
        S = int(r.integers(64 * U, 64 * U + 500))
        out.append((int(r.integers(1, 3)), S, int(r.integers(1, 8)), int(r.choice([64, 128])), U,
                    int(r.choice([1, 64]))))
    return out


@pytest.mark.parametrize("case", CASES + _random_cases(8))
@pytest.mark.parametrize("ws", [True, False], ids=["split", "whole"])
def test_all_ranks_bitwise_and_oracle(case, ws):
    B, S, H, D, U, al = case
    L = sa.dit_a2a_layout_init(B, S, H, D, U, al, 3, torch.bfloat16)
    L1 = sa.dit_a2a_layout_init(B, S, H, D, U, al, 1, torch.bfloat16)
    Lo = oracle.a2a_layout(B, S, H, D, U, al, 3)
    Lo1 = oracle.a2a_layout(B, S, H, D, U, al, 1)
    scale = 1.0 / math.sqrt(D)
    for r in range(U):
        log(f"attn_fwd_a2a {case} rank {r} workspace={ws}")
        recv = _recv(L, 100 + r)
        rd = recv.to(DEV)
        send, lse = _fused(rd, L, r, ws)
        ref_send, ref_lse = _unfused(rd, L, L1, r, ws)
        torch.cuda.synchronize()
        assert torch.equal(_bits(send), _bits(ref_send))
        assert torch.equal(_bits(lse), _bits(ref_lse))
        if ws:
            continue
        q, k, v = oracle.unpack_seq_to_head(recv.float().numpy(), Lo, r)
        ro, rl = oracle.attention(q, k, v, scale)
        want = oracle.pack_head_to_seq([ro], Lo1, r)
        assert np.abs(send.float().cpu().numpy() - want.reshape(send.shape)).max() <= 1e-2
        assert np.abs(lse.cpu().numpy() - rl).max() <= 1e-3


FULL = [
    # name, B, S, H, D, U, ranks
    ("flux", 1, 4608, 24, 128, 2, [0, 1]),
    ("qwen-u4", 2, 7145, 24, 128, 4, [3]),     # S_loc 1787, 3 pad rows
]


@pytest.mark.parametrize("case", FULL, ids=[c[0] for c in FULL])
def test_full_size_bitwise(case):
    name, B, S, H, D, U, ranks = case
    L = sa.dit_a2a_layout_init(B, S, H, D, U, 1, 3, torch.bfloat16)
    L1 = sa.dit_a2a_layout_init(B, S, H, D, U, 1, 1, torch.bfloat16)
    for r in ranks:
        log(f"attn_fwd_a2a full {name} rank {r}")
        rd = _recv(L, 200 + r).to(DEV)
        for ws in (True, False):
            send, lse = _fused(rd, L, r, ws)
            ref_send, ref_lse = _unfused(rd, L, L1, r, ws)
            torch.cuda.synchronize()
            assert torch.equal(_bits(send), _bits(ref_send))
            assert torch.equal(_bits(lse), _bits(ref_lse))

"""GPU parity of dit_ulysses_unpack_rope (receive preparation with RoPE on
Q and K) against the fp64 oracle.

Every rank of a Ulysses group is simulated on the one GPU: the shards are
packed by the library, exchanged by a device chunk transpose, and each
rank's receive buffer is unpacked with RoPE.  Bounds: V bit-exact with the
plain unpack, identity tables bit-exact with the plain unpack, and the
rotated Q/K within one final rounding of the fp64 result computed from the
same inputs and tables:
  |y_gpu - y_ref| <= 2^-8 |y_ref| + 2^-22 (|x_2i| + |x_2i+1|)   (bf16)
with 2^-11 for fp16 and 2^-23 for fp32 in place of 2^-8 (half an ulp of
the stored type) -- the second term covers the fp32 evaluation of the two
products before the final rounding.
"""

import numpy as np
import pytest
import torch

import oracle
import sequence_attention_amd as sa
from sequence_attention_amd import workloads
from tests.gpu_util import DEV, bits, log, simulate_all_to_all

pytestmark = pytest.mark.gpu

HALF_ULP = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11, torch.float32: 2.0 ** -23}
# half the spacing of the subnormals: below the smallest normal the rounding
# error of a correctly rounded result is bounded in absolute terms, not by
# HALF_ULP * |x| (float16 subnormals are 2^-24 apart, below 2^-14)
HALF_SUB = {torch.bfloat16: 2.0 ** -134, torch.float16: 2.0 ** -25, torch.float32: 2.0 ** -150}


def _exchange(B, S, H, D, U, dtype, seed):
    L = sa.dit_a2a_layout_init(B, S, H, D, U, 1, 3, dtype)
    Lo = oracle.a2a_layout(B, S, H, D, U, 1, 3)
    g = torch.Generator().manual_seed(seed)
    glob = [torch.randn(B, S, H, D, generator=g).to(dtype) for _ in range(3)]
    sends = []
    for r in range(U):
        shard = [torch.zeros(B, L.S_loc, H, D, dtype=dtype) for _ in range(3)]
        lo, hi = r * L.S_loc, min(S, (r + 1) * L.S_loc)
        for pl in range(3):
            if hi > lo:
                shard[pl][:, :hi - lo] = glob[pl][:, lo:hi]
        sends.append(sa.dit_ulysses_pack(L, sa.DIT_SEQ_TO_HEAD, r, [x.to(DEV) for x in shard]))
    recvs = simulate_all_to_all(sends)
    torch.cuda.synchronize()
    return L, Lo, recvs


def _check_rotated(got, ref, x_pairs_abs, dtype, what):
    bound = HALF_ULP[dtype] * np.abs(ref) + HALF_SUB[dtype] + 2.0 ** -22 * x_pairs_abs
    excess = np.max(np.abs(got - ref) - bound) if got.size else -1.0
    assert excess <= 0, f"{what}: rotated values off by {excess:.3e} beyond the bound"


def _pair_abs(x):
    a = np.abs(x)
    s = a[..., 0::2] + a[..., 1::2]
    out = np.empty_like(a)
    out[..., 0::2] = s
    out[..., 1::2] = s
    return out


CASES = [
    # B, S, H, D, U, dtype
    (1, 256, 4, 64, 2, torch.bfloat16),      # tiny config
    (1, 4608, 24, 128, 2, torch.bfloat16),   # FLUX U=2
    (2, 7145, 24, 128, 4, torch.bfloat16),   # Qwen U=4: rank 3 holds 3 pad rows
    (2, 7145, 24, 128, 5, torch.bfloat16),   # Qwen U=5: a zero pad head
    (2, 37, 5, 8, 3, torch.bfloat16),        # ragged S and H, D = 8
    (1, 300, 6, 64, 4, torch.float16),
    (1, 129, 4, 32, 2, torch.float32),
]


def _random_cases(n_cases, seed=29):
    # seeded sweep: ragged S and H, U above and below H, head sizes of one
    # to eight 16-byte vectors, the three dtypes
    r = np.random.default_rng(seed)
    out = []
    for _ in range(n_cases):
        dt = [torch.bfloat16, torch.float16, torch.float32][int(r.integers(0, 3))]
        D = int(r.choice([8, 16, 24, 64, 128] if dt != torch.float32 else [4, 8, 12, 64]))
        out.append((int(r.integers(1, 3)), int(r.integers(1, 300)), int(r.integers(1, 9)), D, int(r.integers(1, 6)), dt))
    return out


@pytest.mark.parametrize("case", CASES + _random_cases(10))
def test_all_ranks_match_oracle(case):
    B, S, H, D, U, dt = case
    log(f"rope unpack {case}")
    L, Lo, recvs = _exchange(B, S, H, D, U, dt, seed=S + U)
    cos, sin = workloads.rope_tables(S, D)
    cd, sd = cos.to(DEV), sin.to(DEV)
    ranks = range(U) if S * H <= 200_000 else [0, U - 1]
    for r in ranks:
        got = sa.dit_ulysses_unpack_rope(L, r, recvs[r], cd, sd)
        plain = sa.dit_ulysses_unpack(L, sa.DIT_SEQ_TO_HEAD, r, recvs[r])
        torch.cuda.synchronize()
        rv = recvs[r].float().cpu().numpy()
        ref = oracle.unpack_seq_to_head_rope(rv, Lo, r, cos.numpy(), sin.numpy())
        assert np.array_equal(bits(got[2]), bits(plain[2])), "V differs from the plain unpack"
        for pl in range(2):
            x = plain[pl].float().cpu().numpy().astype(np.float64)
            _check_rotated(got[pl].float().cpu().numpy().astype(np.float64), ref[pl], _pair_abs(x), dt,
                           f"rank {r} plane {pl}")


def test_float16_results_in_the_subnormal_range():
    # inputs of about 1e-5 rotate to float16 results below 2^-14, where one
    # final rounding is bounded by half the subnormal spacing (2^-25)
    B, S, H, D, U = 1, 64, 4, 64, 2
    log("rope unpack float16 subnormal results")
    L = sa.dit_a2a_layout_init(B, S, H, D, U, 1, 3, torch.float16)
    Lo = oracle.a2a_layout(B, S, H, D, U, 1, 3)
    g = torch.Generator().manual_seed(5)
    recv = (torch.randn(U * L.elems_per_peer, generator=g) * 1e-5).to(torch.float16)
    assert (recv.abs() < 2.0 ** -14).float().mean() > 0.9        # mostly subnormal inputs
    cos, sin = workloads.rope_tables(S, D)
    for r in range(U):
        got = sa.dit_ulysses_unpack_rope(L, r, recv.to(DEV), cos.to(DEV), sin.to(DEV))
        torch.cuda.synchronize()
        rv = recv.float().numpy()
        ref = oracle.unpack_seq_to_head_rope(rv, Lo, r, cos.numpy(), sin.numpy())
        x = oracle.unpack_seq_to_head(rv, Lo, r)
        for pl in range(3):
            _check_rotated(got[pl].float().cpu().numpy().astype(np.float64), ref[pl], _pair_abs(x[pl]),
                           torch.float16, f"subnormal rank {r} plane {pl}")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16, torch.float32])
def test_identity_tables_equal_plain_unpack_bitwise(dt):
    B, S, H, D, U = 1, 200, 8, 64, 2
    log(f"rope unpack identity tables {dt}")
    L, _, recvs = _exchange(B, S, H, D, U, dt, seed=3)
    ones = torch.ones(S, D // 2, device=DEV)
    zeros = torch.zeros(S, D // 2, device=DEV)
    for r in range(U):
        got = sa.dit_ulysses_unpack_rope(L, r, recvs[r], ones, zeros)
        plain = sa.dit_ulysses_unpack(L, sa.DIT_SEQ_TO_HEAD, r, recvs[r])
        torch.cuda.synchronize()
        for pl in range(3):
            assert np.array_equal(bits(got[pl]), bits(plain[pl]))


def test_rotation_then_attention_depends_on_relative_position():
    # the attention scores after RoPE are invariant to a common position
    # shift: rotate the same Q/K rows at positions t and t + 64 (one-axis
    # tables) and compare the score matrices of the two
    B, S, H, D, U = 1, 128, 2, 64, 2
    log("rope unpack relative position")
    L, _, recvs = _exchange(B, S, H, D, U, torch.float32, seed=5)
    cos, sin = workloads.rope_tables(S + 64, D)
    a = sa.dit_ulysses_unpack_rope(L, 0, recvs[0], cos[:S].contiguous().to(DEV), sin[:S].contiguous().to(DEV))
    b = sa.dit_ulysses_unpack_rope(L, 0, recvs[0], cos[64:].contiguous().to(DEV), sin[64:].contiguous().to(DEV))
    torch.cuda.synchronize()
    for h in range(L.H_loc):
        sa_ = a[0][0, :, h].double() @ a[1][0, :, h].double().T
        sb_ = b[0][0, :, h].double() @ b[1][0, :, h].double().T
        assert torch.max(torch.abs(sa_ - sb_)).item() <= 1e-3

"""End-to-end parity of one Ulysses x ring step on the Tiny workload, with
every rank of the Ulysses pair simulated on the one GPU: QKV pack ->
exchange -> unpack -> ring chunks + merge -> O pack -> exchange -> unpack,
against the oracle's global attention; then the CFG combine."""

import numpy as np
import pytest
import torch

import oracle
import sequence_attention_amd as sa
from sequence_attention_amd import workloads
from tests.gpu_util import DEV, log, max_abs, simulate_all_to_all

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("S,H,U,R", [(256, 4, 2, 2), (203, 5, 2, 3), (130, 3, 4, 2)])
def test_ulysses_ring_step_matches_global_attention(S, H, U, R):
    log(f"path S={S} H={H} U={U} R={R}")
    B, D = 1, 64
    scale = D ** -0.5
    g = torch.Generator().manual_seed(S)
    X = [torch.randn(B, S, H, D, generator=g).to(torch.bfloat16) for _ in range(3)]   # global Q, K, V
    L = sa.dit_a2a_layout_init(B, S, H, D, U, 1, 3)
    Lo = sa.dit_a2a_layout_init(B, S, H, D, U, 1, 1)
    shards = []
    for r in range(U):
        lo, hi = r * L.S_loc, min(S, (r + 1) * L.S_loc)
        planes = []
        for x in X:
            t = torch.zeros(B, L.S_loc, H, D, dtype=torch.bfloat16)
            if hi > lo:
                t[:, : hi - lo] = x[:, lo:hi]
            planes.append(t.to(DEV))
        shards.append(planes)
    recv = simulate_all_to_all([sa.dit_ulysses_pack(L, sa.DIT_SEQ_TO_HEAD, r, shards[r]) for r in range(U)])
    outs = []
    for r in range(U):
        q, k, v = sa.dit_ulysses_unpack(L, sa.DIT_SEQ_TO_HEAD, r, recv[r])
        bounds = [S * c // R for c in range(R + 1)]
        acc = acc_l = None
        for c in oracle.ring_hop_order(R, 0):
            o, l = sa.dit_attn_fwd(q, k[:, bounds[c]:bounds[c + 1]].contiguous(),
                                   v[:, bounds[c]:bounds[c + 1]].contiguous(), scale=scale)
            if acc is None:
                acc, acc_l = o, l
            else:
                sa.dit_attn_merge(acc, acc_l, o, l)
        outs.append(acc)
    back = simulate_all_to_all([sa.dit_ulysses_pack(Lo, sa.DIT_HEAD_TO_SEQ, r, [outs[r]]) for r in range(U)])
    final = [sa.dit_ulysses_unpack(Lo, sa.DIT_HEAD_TO_SEQ, r, back[r])[0] for r in range(U)]
    torch.cuda.synchronize()
    ref_o, _ = oracle.attention(*(x.float().numpy() for x in X), scale)
    for r in range(U):
        lo, hi = r * L.S_loc, min(S, (r + 1) * L.S_loc)
        got = final[r].float().cpu().numpy()
        assert max_abs(got[:, : max(hi - lo, 0)], ref_o[:, lo:hi]) <= 1e-2
        assert np.all(got[:, max(hi - lo, 0):] == 0)       # pad rows


def test_cfg_after_gather():
    log("path cfg [2,256,256] g=4")
    x = workloads.cfg_inputs((2, 256, 256))
    out = sa.dit_cfg_combine(x[0].contiguous().to(DEV), x[1].contiguous().to(DEV), 4.0)
    torch.cuda.synchronize()
    want = oracle.cfg_combine_f32(x[0].numpy(), x[1].numpy(), 4.0)
    np.testing.assert_array_equal(out.cpu().numpy(), want)

"""GPU parity of per-batch key lengths (dit_attn_fwd_kvlen) and of the joint
text+image ring built from it: the image keys rotate through the ring
(dit_attn_fwd_merge per hop), the replicated, tail-padded text segment is
attended once with its valid lengths and merged into the same accumulator.
Reference: the fp64 oracle on the concatenation of the image keys and the
valid text keys.  Tolerances as for attention (bf16 O 1e-2 / LSE 1e-3,
fp32 1e-5)."""

import numpy as np
import pytest
import torch

import oracle
import sequence_attention_amd as sa
from sequence_attention_amd import workloads
from tests.gpu_util import DEV, log, max_abs

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: (1e-2, 1e-3), torch.float32: (1e-5, 1e-5)}


def _inputs(B, Sq, Skv, H, D, dtype, seed):
    w = workloads.Workload("kvlen", B=B, Sq=Sq, Skv=Skv, H=H, D=D, R=1, S=Skv, H_total=H, U=1)
    return workloads.attention_inputs(w, dtype=dtype, seed=seed) + (w.scale,)


KVLEN = [
    # B, Sq, Skv, H, D, kv_len
    (3, 300, 512, 4, 128, [512, 77, 0]),
    (4, 129, 200, 3, 64, [1, 64, 65, 1000]),     # one value past Skv: clamped
    (1, 256, 4608, 12, 128, [4000]),
]


@pytest.mark.parametrize("case", KVLEN)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_kv_len_vs_oracle(case, dtype):
    B, Sq, Skv, H, D, lens = case
    log(f"kv_len {dtype} {case}")
    q, k, v, scale = _inputs(B, Sq, Skv, H, D, dtype, seed=Sq + Skv)
    kvl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o, lse = sa.dit_attn_fwd_kvlen(q.to(DEV), k.to(DEV), v.to(DEV), kvl, scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_kv_len(q.float().numpy(), k.float().numpy(), v.float().numpy(), scale, lens)
    tol_o, tol_l = TOL[dtype]
    go, gl = o.float().cpu().numpy(), lse.cpu().numpy()
    assert max_abs(go, ro) <= tol_o
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl))
    fin = np.isfinite(rl)
    assert max_abs(gl[fin], rl[fin]) <= tol_l


def test_full_length_equals_plain_attention_bitwise():
    # 216 tiles of 256 rows: on a 256-CU device the plain call takes every tile
    # whole as well, so both paths run the same arithmetic
    q, k, v, scale = _inputs(1, 4608, 700, 12, 128, torch.bfloat16, seed=4)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    kvl = torch.tensor([700], dtype=torch.int32, device=DEV)
    o1, l1 = sa.dit_attn_fwd_kvlen(qd, kd, vd, kvl, scale=scale)
    o2, l2 = sa.dit_attn_fwd(qd, kd, vd, scale=scale)
    torch.cuda.synchronize()
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
    else:
        assert max_abs(o1.float().cpu().numpy(), o2.float().cpu().numpy()) <= 1e-2


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_merge_mode_leaves_empty_batches_untouched(dtype):
    q, k, v, scale = _inputs(2, 100, 64, 2, 64, dtype, seed=6)
    g = torch.Generator().manual_seed(7)
    acc = torch.randn(2, 100, 2, 64, generator=g).to(dtype).to(DEV)
    acc_l = (torch.randn(2, 2, 100, generator=g) * 3).to(DEV)
    acc0, accl0 = acc.clone(), acc_l.clone()
    kvl = torch.tensor([0, 0], dtype=torch.int32, device=DEV)
    sa.dit_attn_fwd_kvlen(q.to(DEV), k.to(DEV), v.to(DEV), kvl, o=acc, lse=acc_l, scale=scale, merge=True)
    torch.cuda.synchronize()
    assert torch.equal(acc, acc0) and torch.equal(acc_l, accl0)


JOINT = [
    # B, S_img (ring-sharded keys), R, T_max (text, replicated), text lengths, H, D, query rows
    (2, 4096, 4, 512, [512, 300], 6, 128, 1024),   # FLUX-like: 4096 image + up to 512 text
    (1, 6889, 3, 256, [201], 4, 128, 700),         # Qwen-like: 83 x 83 image + up to 256 text
]


@pytest.mark.parametrize("case", JOINT)
def test_joint_text_image_ring_vs_oracle(case):
    B, S_img, R, T, tlens, H, D, Sq = case
    log(f"joint text+image ring {case}")
    g = torch.Generator().manual_seed(S_img + T)
    mk = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16)
    q = mk(B, Sq, H, D)
    k_img, v_img = mk(B, S_img, H, D), mk(B, S_img, H, D)
    k_txt, v_txt = mk(B, T, H, D), mk(B, T, H, D)
    scale = D ** -0.5
    qd = q.to(DEV)
    acc = torch.zeros(B, Sq, H, D, dtype=torch.bfloat16, device=DEV)
    acc_l = torch.full((B, H, Sq), -np.inf, device=DEV)
    bounds = [S_img * c // R for c in range(R + 1)]
    for c in oracle.ring_hop_order(R, 0):
        sa.dit_attn_fwd_merge(qd, k_img[:, bounds[c]:bounds[c + 1]].contiguous().to(DEV),
                              v_img[:, bounds[c]:bounds[c + 1]].contiguous().to(DEV), acc, acc_l, scale=scale)
    kvl = torch.tensor(tlens, dtype=torch.int32, device=DEV)
    sa.dit_attn_fwd_kvlen(qd, k_txt.to(DEV), v_txt.to(DEV), kvl, o=acc, lse=acc_l, scale=scale, merge=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, Sq, 37), [Sq - 1]]))
    for b in range(B):
        kk = torch.cat([k_img[b:b + 1], k_txt[b:b + 1, :tlens[b]]], dim=1)
        vv = torch.cat([v_img[b:b + 1], v_txt[b:b + 1, :tlens[b]]], dim=1)
        ro, rl = oracle.attention(q[b:b + 1].float().numpy(), kk.float().numpy(), vv.float().numpy(), scale,
                                  rows=rows)
        go = acc[b:b + 1].float().cpu().numpy()[:, rows]
        gl = acc_l[b:b + 1].cpu().numpy()[:, :, rows]
        assert max_abs(go, ro) <= 1e-2
        assert max_abs(go, ro) / np.max(np.abs(ro)) <= 2e-2
        assert max_abs(gl, rl) <= 1e-3

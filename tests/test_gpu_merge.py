"""GPU parity of dit_attn_merge and of the ring chunk loop (attention per
K/V chunk + merge after each) against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import sequence_attention_amd as sa
from sequence_attention_amd import workloads
from tests.gpu_util import DEV, log, max_abs

pytestmark = pytest.mark.gpu


def _partials(B, Sq, H, D, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    o = torch.randn(B, Sq, H, D, generator=g).to(dtype)
    lse = torch.randn(B, H, Sq, generator=g) * 4
    return o, lse


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(1, 256, 4, 64), (2, 7145, 6, 128), (1, 33, 3, 128), (1, 300, 3, 8),
                                   (2, 37, 2, 16), (1, 70, 2, 32), (1, 45, 2, 256), (1, 21, 2, 512)])
def test_merge_matches_oracle(dtype, shape):
    log(f"merge {dtype} {shape}")
    oa, la = _partials(*shape, dtype, 1)
    op, lp = _partials(*shape, dtype, 2)
    # a few empty rows on either side and on both
    la[0, 0, :3] = -np.inf
    lp[0, 0, 2:5] = -np.inf
    oa_d, la_d = oa.to(DEV), la.to(DEV)
    sa.dit_attn_merge(oa_d, la_d, op.to(DEV), lp.to(DEV))
    torch.cuda.synchronize()
    ro, rl = oracle.merge(oa.float().numpy(), la.numpy(), op.float().numpy(), lp.numpy())
    got = oa_d.float().cpu().numpy()
    # one final rounding of the stored O: half an ulp, 2^-8 relative in bf16
    if dtype == torch.bfloat16:
        assert np.all(np.abs(got - ro) <= 2.0 ** -8 * np.abs(ro) + 1e-6)
    else:
        assert max_abs(got, ro) <= 1e-5
    got_l = la_d.cpu().numpy()
    assert np.array_equal(np.isneginf(got_l), np.isneginf(rl))
    fin = np.isfinite(rl)
    assert max_abs(got_l[fin], rl[fin]) <= 1e-5


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_identity_with_empty_part_is_exact(dtype):
    log(f"merge identity {dtype}")
    oa, la = _partials(1, 300, 4, 128, dtype, 5)
    garbage = torch.full_like(oa, float("nan"))
    oa_d, la_d = oa.to(DEV), la.to(DEV)
    sa.dit_attn_merge(oa_d, la_d, garbage.to(DEV), torch.full_like(la, -np.inf).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(oa_d.cpu(), oa) and torch.equal(la_d.cpu(), la)
    # empty accumulator (holding NaN) absorbs the part exactly
    acc = garbage.to(DEV)
    acc_l = torch.full_like(la, -np.inf).to(DEV)
    sa.dit_attn_merge(acc, acc_l, oa.to(DEV), la.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(acc.cpu(), oa) and torch.equal(acc_l.cpu(), la)


def test_both_empty():
    o = torch.full((1, 10, 2, 64), float("nan")).to(DEV)
    l = torch.full((1, 2, 10), -np.inf).to(DEV)
    sa.dit_attn_merge(o, l, o.clone(), l.clone())
    torch.cuda.synchronize()
    assert torch.count_nonzero(o).item() == 0 and torch.isneginf(l).all().item()


def test_commutative_bitwise():
    oa, la = _partials(1, 512, 4, 128, torch.float32, 11)
    op, lp = _partials(1, 512, 4, 128, torch.float32, 12)
    x, xl = oa.to(DEV), la.to(DEV)
    sa.dit_attn_merge(x, xl, op.to(DEV), lp.to(DEV))
    y, yl = op.to(DEV), lp.to(DEV)
    sa.dit_attn_merge(y, yl, oa.to(DEV), la.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(x, y) and torch.equal(xl, yl)


def test_associative_fp32_within_1e_6():
    # (a + b) + c against a + (b + c) on the fp32 path: the online-softmax
    # merge is associative in exact arithmetic (SGLang "Parallelism
    # Overview", the per-hop merge folds partial results in any grouping),
    # so the two groupings may differ only by fp32 rounding.  O in [-1, 1]
    # keeps an fp32 ulp at or below 2^-23; LSE ~ N(0, 2^2) with a few empty
    # rows on each side.
    log("merge associativity fp32")
    B, Sq, H, D = 1, 700, 6, 128
    g = torch.Generator().manual_seed(21)
    parts = []
    for i in range(3):
        o = torch.rand(B, Sq, H, D, generator=g) * 2 - 1
        lse = torch.randn(B, H, Sq, generator=g) * 2
        lse[0, i, 5 * i:5 * i + 7] = -np.inf
        parts.append((o, lse))
    (oa, la), (ob, lb), (oc, lc) = parts
    left, left_l = oa.to(DEV), la.to(DEV)
    sa.dit_attn_merge(left, left_l, ob.to(DEV), lb.to(DEV))
    sa.dit_attn_merge(left, left_l, oc.to(DEV), lc.to(DEV))
    bc, bc_l = ob.to(DEV), lb.to(DEV)
    sa.dit_attn_merge(bc, bc_l, oc.to(DEV), lc.to(DEV))
    right, right_l = oa.to(DEV), la.to(DEV)
    sa.dit_attn_merge(right, right_l, bc, bc_l)
    torch.cuda.synchronize()
    assert max_abs(left.cpu().numpy(), right.cpu().numpy()) <= 1e-6
    ll, rl = left_l.cpu().numpy(), right_l.cpu().numpy()
    assert np.array_equal(np.isneginf(ll), np.isneginf(rl))
    fin = np.isfinite(ll)
    # LSE compared relative to its magnitude (an fp32 ulp at |L| >= 8 is
    # already 2^-20 ~ 9.5e-7)
    assert np.all(np.abs(ll[fin] - rl[fin]) <= 1e-6 * np.maximum(1.0, np.abs(ll[fin])))
    # and both equal the oracle's fold
    ro, rlo = oracle.merge(*oracle.merge(oa.numpy(), la.numpy(), ob.numpy(), lb.numpy()), oc.numpy(), lc.numpy())
    assert max_abs(left.cpu().numpy(), ro) <= 1e-6


def ring_on_gpu(q, k, v, scale, R, order, acc_dtype):
    """The ring hop loop of one rank run as sequential chunks on one GPU."""
    Skv = k.shape[1]
    bounds = [Skv * c // R for c in range(R + 1)]
    qd = q.to(DEV)
    acc = acc_l = None
    for c in order:
        kc = k[:, bounds[c]:bounds[c + 1]].contiguous().to(DEV)
        vc = v[:, bounds[c]:bounds[c + 1]].contiguous().to(DEV)
        o, l = sa.dit_attn_fwd(qd, kc, vc, scale=scale, o_dtype=acc_dtype)
        if acc is None:
            acc, acc_l = o, l
        else:
            sa.dit_attn_merge(acc, acc_l, o, l)
    torch.cuda.synchronize()
    return acc, acc_l, bounds


@pytest.mark.parametrize("acc_dtype", [torch.bfloat16, torch.float32])
def test_tiny_ring_two_chunks(acc_dtype):
    w = workloads.WORKLOADS["tiny"]
    log(f"ring tiny R=2 acc {acc_dtype}")
    q, k, v = workloads.attention_inputs(w)
    acc, acc_l, bounds = ring_on_gpu(q, k, v, w.scale, 2, oracle.ring_hop_order(2, 0), acc_dtype)
    ro, rl = oracle.ring_attention(q.float().numpy(), k.float().numpy(), v.float().numpy(), w.scale,
                                   bounds, oracle.ring_hop_order(2, 0))
    uo, ul = oracle.attention(q.float().numpy(), k.float().numpy(), v.float().numpy(), w.scale)
    assert max_abs(ro, uo) <= 1e-12           # the oracle's own chunked == unchunked
    assert max_abs(acc.float().cpu().numpy(), ro) <= 1e-2
    assert max_abs(acc_l.cpu().numpy(), rl) <= 1e-3


@pytest.mark.parametrize("order", [[0, 3, 2, 1], [0, 1, 2, 3]])
def test_ring_config_chunked_vs_oracle_and_unchunked(order):
    w = workloads.WORKLOADS["ring"]
    log(f"ring [1,4096,24,128] x 4 chunks order {order}")
    q, k, v = workloads.attention_inputs(w)
    acc, acc_l, bounds = ring_on_gpu(q, k, v, w.scale, 4, order, torch.bfloat16)
    un, un_l = sa.dit_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=w.scale)
    torch.cuda.synchronize()
    rows = np.arange(0, 4096, 61)
    ro, rl = oracle.attention(q.float().numpy(), k.float().numpy(), v.float().numpy(), w.scale, rows=rows)
    go = acc.float().cpu().numpy()[:, rows]
    assert max_abs(go, ro) <= 1e-2
    assert max_abs(go, ro) / np.max(np.abs(ro)) <= 2e-2
    assert max_abs(acc_l.cpu().numpy()[:, :, rows], rl) <= 1e-3
    # chunked vs unchunked on the GPU, whole tensor
    assert max_abs(acc.float().cpu().numpy(), un.float().cpu().numpy()) <= 1e-2
    assert max_abs(acc_l.cpu().numpy(), un_l.cpu().numpy()) <= 1e-3


def test_single_chunk_ring_is_plain_attention_bitwise():
    w = workloads.WORKLOADS["tiny"]
    q, k, v = workloads.attention_inputs(w, seed=4)
    acc, acc_l, _ = ring_on_gpu(q, k, v, w.scale, 1, [0], torch.bfloat16)
    o, l = sa.dit_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(acc, o) and torch.equal(acc_l, l)


# ---- one ring hop per call: attention fused with the merge ------------------

def ring_fused_on_gpu(q, k, v, scale, bounds, order, acc_dtype):
    """The hop loop with dit_attn_fwd_merge: the accumulator starts as the
    merge identity (O = 0, LSE = -inf) and every chunk is folded into it."""
    B, Sq, H, D = q.shape
    qd = q.to(DEV)
    acc = torch.zeros((B, Sq, H, D), dtype=acc_dtype, device=DEV)
    acc_l = torch.full((B, H, Sq), -np.inf, dtype=torch.float32, device=DEV)
    for c in order:
        kc = k[:, bounds[c]:bounds[c + 1]].contiguous().to(DEV)
        vc = v[:, bounds[c]:bounds[c + 1]].contiguous().to(DEV)
        sa.dit_attn_fwd_merge(qd, kc, vc, acc, acc_l, scale=scale)
    torch.cuda.synchronize()
    return acc, acc_l


@pytest.mark.parametrize("acc_dtype", [torch.bfloat16, torch.float32])
def test_fused_tiny_ring_vs_oracle(acc_dtype):
    w = workloads.WORKLOADS["tiny"]
    log(f"fused ring tiny R=2 acc {acc_dtype}")
    q, k, v = workloads.attention_inputs(w)
    bounds = [0, 128, 256]
    order = oracle.ring_hop_order(2, 0)
    acc, acc_l = ring_fused_on_gpu(q, k, v, w.scale, bounds, order, acc_dtype)
    ro, rl = oracle.ring_attention(q.float().numpy(), k.float().numpy(), v.float().numpy(), w.scale,
                                   bounds, order)
    assert max_abs(acc.float().cpu().numpy(), ro) <= 1e-2
    assert max_abs(acc_l.cpu().numpy(), rl) <= 1e-3


@pytest.mark.parametrize("order", [[0, 3, 2, 1], [2, 0, 3, 1]])
def test_fused_ring_config_vs_oracle_and_unfused(order):
    w = workloads.WORKLOADS["ring"]
    log(f"fused ring [1,4096,24,128] x 4 chunks order {order}")
    q, k, v = workloads.attention_inputs(w)
    bounds = [w.Skv * c // 4 for c in range(5)]
    acc, acc_l = ring_fused_on_gpu(q, k, v, w.scale, bounds, order, torch.bfloat16)
    rows = np.arange(0, 4096, 61)
    ro, rl = oracle.attention(q.float().numpy(), k.float().numpy(), v.float().numpy(), w.scale, rows=rows)
    go = acc.float().cpu().numpy()[:, rows]
    assert max_abs(go, ro) <= 1e-2
    assert max_abs(go, ro) / np.max(np.abs(ro)) <= 2e-2
    assert max_abs(acc_l.cpu().numpy()[:, :, rows], rl) <= 1e-3
    # against the unfused hop loop (attention into a temporary + merge)
    un, un_l, _ = ring_on_gpu(q, k, v, w.scale, 4, order, torch.bfloat16)
    assert max_abs(acc.float().cpu().numpy(), un.float().cpu().numpy()) <= 1e-2
    assert max_abs(acc_l.cpu().numpy(), un_l.cpu().numpy()) <= 1e-3


# uneven chunk bounds, ragged rows and head dims, split tiles in the merge path
FUSED_RAGGED = [
    # B, Sq, Skv, H, D, chunk bounds
    (1, 1000, 1000, 8, 128, [0, 300, 301, 1000]),
    (2, 130, 700, 3, 64, [0, 64, 500, 700]),
    (1, 4000, 700, 20, 64, [0, 350, 700]),
]


@pytest.mark.parametrize("case", FUSED_RAGGED)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_fused_ragged_chunks_vs_oracle(case, dtype):
    B, Sq, Skv, H, D, bounds = case
    log(f"fused ring ragged {dtype} {case}")
    wl = workloads.Workload("ragged", B=B, Sq=Sq, Skv=Skv, H=H, D=D, R=len(bounds) - 1, S=Skv,
                            H_total=H, U=1)
    q, k, v = workloads.attention_inputs(wl, dtype=dtype, seed=Sq + Skv)
    order = list(range(len(bounds) - 1))[::-1]
    acc, acc_l = ring_fused_on_gpu(q, k, v, wl.scale, bounds, order, dtype)
    rows = np.unique(np.concatenate([np.arange(0, Sq, max(1, Sq // 97)), [Sq - 1]]))
    ro, rl = oracle.attention(q.float().numpy(), k.float().numpy(), v.float().numpy(), wl.scale, rows=rows)
    tol_o, tol_l = (1e-2, 1e-3) if dtype == torch.bfloat16 else (1e-5, 1e-5)
    assert max_abs(acc.float().cpu().numpy()[:, rows], ro) <= tol_o
    assert max_abs(acc_l.cpu().numpy()[:, :, rows], rl) <= tol_l


def test_fused_empty_chunk_leaves_accumulator_bitwise():
    oa, la = _partials(1, 300, 4, 128, torch.bfloat16, 21)
    acc, acc_l = oa.to(DEV), la.to(DEV)
    q = torch.randn(1, 300, 4, 128).to(torch.bfloat16).to(DEV)
    kv = torch.zeros(1, 0, 4, 128, dtype=torch.bfloat16, device=DEV)
    sa.dit_attn_fwd_merge(q, kv, kv, acc, acc_l)
    torch.cuda.synchronize()
    assert torch.equal(acc.cpu(), oa) and torch.equal(acc_l.cpu(), la)


def test_fused_first_hop_equals_plain_attention():
    # an identity accumulator takes the chunk's result: same O (fp32 path
    # bitwise: the merge weights are exactly 0 and 1) and LSE
    w = workloads.WORKLOADS["tiny"]
    q, k, v = workloads.attention_inputs(w, dtype=torch.float32, seed=8)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o, l = sa.dit_attn_fwd(qd, kd, vd, scale=w.scale)
    acc = torch.zeros_like(o)
    acc_l = torch.full_like(l, -np.inf)
    sa.dit_attn_fwd_merge(qd, kd, vd, acc, acc_l, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(acc, o) and torch.equal(acc_l, l)

"""dit_attn_fwd_noalloc (the entry point for callers that cannot allocate:
its split workspace is the library's static scratch) against
dit_attn_fwd_ws with a caller workspace, through the C ABI, on two calls in
a row, the second with a smaller input (other head dim, fewer tiles), so the
second call runs over scratch the first one left behind."""

import ctypes

import pytest
import torch

import oracle
import sequence_attention_amd as sa
from sequence_attention_amd import _lib, workloads
from tests.gpu_util import DEV, log, max_abs

pytestmark = pytest.mark.gpu

# B, Sq, Skv, H, D: both cut every tile into key chunks on a 256-CU device
CALLS = [(1, 1000, 1000, 8, 128), (1, 520, 900, 3, 64)]


def _noalloc(q, k, v, o, lse, scale):
    B, Sq, H, D = q.shape
    P = ctypes.c_void_p
    st = _lib.lib().dit_attn_fwd_noalloc(
        P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), P(o.data_ptr()), P(lse.data_ptr()),
        B, Sq, k.shape[1], H, D, scale, sa.DIT_BF16, sa.DIT_BF16,
        P(torch.cuda.current_stream().cuda_stream))
    _lib.check(st, "dit_attn_fwd_noalloc")


def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    for i, (B, Sq, Skv, H, D) in enumerate(CALLS):
        log(f"attn noalloc call {i} {(B, Sq, Skv, H, D)}")
        w = workloads.Workload("noalloc", B=B, Sq=Sq, Skv=Skv, H=H, D=D, R=1, S=Skv, H_total=H, U=1)
        q, k, v = workloads.attention_inputs(w, seed=40 + i)
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        need = sa.dit_attn_workspace_size(B, Sq, Skv, H, D)
        assert need > 0          # the call does use scratch
        o = torch.full((B, Sq, H, D), float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full((B, H, Sq), float("nan"), dtype=torch.float32, device=DEV)
        _noalloc(qd, kd, vd, o, lse, w.scale)
        ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
        o_ws, lse_ws = sa.dit_attn_fwd_ws(qd, kd, vd, ws, scale=w.scale)
        torch.cuda.synchronize()
        # the same split plan and kernel: bitwise equal
        assert torch.equal(o, o_ws) and torch.equal(lse, lse_ws)
        ro, rl = oracle.attention(q.float().numpy(), k.float().numpy(), v.float().numpy(), w.scale)
        assert max_abs(o.float().cpu().numpy(), ro) <= 1e-2
        assert max_abs(lse.cpu().numpy(), rl) <= 1e-3

"""GPU parity of dit_cfg_combine against the oracle (bit-exact in fp32)."""

import numpy as np
import pytest
import torch

import oracle
import sequence_attention_amd as sa
from sequence_attention_amd import workloads
from tests.gpu_util import DEV, Guarded, bits, log

pytestmark = pytest.mark.gpu


def _run(u, c, g, out=None):
    out = sa.dit_cfg_combine(u, c, g, out=out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("g", [4.0, 7.5, 0.0, 1.0, -2.25])
def test_tiny_config_fp32_bit_exact(g):
    log(f"cfg fp32 [2,256,256] g={g}")
    x = workloads.cfg_inputs((2, 256, 256))
    u, c = x[0].contiguous(), x[1].contiguous()
    out = Guarded((256, 256), torch.float32)
    _run(u.to(DEV), c.to(DEV), g, out.t)
    assert out.canary_ok()
    got = out.t.cpu().numpy()
    want = oracle.cfg_combine_f32(u.numpy(), c.numpy(), g)
    np.testing.assert_array_equal(got.view(np.int32), want.view(np.int32))
    assert np.max(np.abs(got - oracle.cfg_combine(u.numpy(), c.numpy(), g))) <= 1e-5 * max(1, abs(g))
    if g == 0.0:
        np.testing.assert_array_equal(got, u.numpy())


@pytest.mark.parametrize("n", [1, 3, 4, 5, 1001, 4096 * 4 + 7, 1 << 20])
def test_ragged_sizes_and_in_place(n):
    log(f"cfg fp32 n={n} in place")
    g = torch.Generator().manual_seed(n)
    u = torch.randn(n, generator=g)
    c = torch.randn(n, generator=g)
    want = oracle.cfg_combine_f32(u.numpy(), c.numpy(), 3.3)
    ud = u.to(DEV)
    _run(ud, c.to(DEV), 3.3, out=ud)           # out aliases p_uncond
    np.testing.assert_array_equal(ud.cpu().numpy().view(np.int32), want.view(np.int32))
    cd = c.to(DEV)
    _run(u.to(DEV), cd, 3.3, out=cd)           # out aliases p_cond
    np.testing.assert_array_equal(cd.cpu().numpy().view(np.int32), want.view(np.int32))


@pytest.mark.parametrize("n", [8, 9, 1000, 65536 * 2 + 3])
def test_bf16_rounds_the_fp32_result(n):
    log(f"cfg bf16 n={n}")
    g = torch.Generator().manual_seed(7)
    u = torch.randn(n, generator=g).to(torch.bfloat16)
    c = torch.randn(n, generator=g).to(torch.bfloat16)
    out = Guarded((n,), torch.bfloat16)
    _run(u.to(DEV), c.to(DEV), 4.0, out.t)
    assert out.canary_ok()
    want32 = oracle.cfg_combine_f32(u.float().numpy(), c.float().numpy(), 4.0)
    want = torch.from_numpy(want32).to(torch.bfloat16)       # round to nearest even
    np.testing.assert_array_equal(bits(out.t), bits(want))


def test_random_guidance_scales_and_magnitudes_bit_exact():
    # 60 seeded calls: guidance scales from tiny to hundreds (and 0, +-1),
    # inputs from 1e-30 to 1e30, ragged lengths; every fp32 result equals the
    # oracle's correctly rounded fmaf(g, c - u, u)
    r = np.random.default_rng(777)
    for i in range(60):
        n = int(r.integers(1, 5000))
        g = float(np.float32(r.choice([r.normal() * 5, r.normal() * 100, r.uniform(-1e-3, 1e-3), 0.0, 1.0, -1.0])))
        sc = float(r.choice([1e-30, 1e-3, 1.0, 1e3, 1e30]))
        u = torch.from_numpy(r.standard_normal(n).astype(np.float32)) * sc
        c = torch.from_numpy(r.standard_normal(n).astype(np.float32)) * sc
        out = _run(u.to(DEV), c.to(DEV), g)
        want = oracle.cfg_combine_f32(u.numpy(), c.numpy(), g)
        np.testing.assert_array_equal(out.cpu().numpy().view(np.int32), want.view(np.int32),
                                      err_msg=f"case {i}: n={n} g={g} scale={sc}")


def test_empty_is_a_no_op():
    u = torch.zeros(0, device=DEV)
    out = _run(u, u, 4.0)
    assert out.numel() == 0

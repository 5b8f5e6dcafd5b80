"""Seeded sweep of the attention entry points over random small shapes.

For each of 40 configurations drawn from a fixed seed: B in 1..3, Sq and Skv
anywhere from 1 to a few blocks past a tile (ragged tails on both sides),
H in 1..6, D in {64, 128}, inputs scaled by 0.25..8 (flat to sharp softmax
rows), bf16 or fp32 inputs, and one of the entry points

  * dit_attn_fwd with and without the split workspace, bf16 or fp32 O,
  * dit_attn_fwd_kvlen with random per-batch lengths (0 and past Skv
    included),
  * dit_attn_fwd_merge folding the call into a random accumulator, one of
    whose rows per batch and head is empty (LSE = -inf),

each compared element by element with the fp64 oracle (attention,
attention_kv_len, merge) at the attention tolerances: bf16 O 1e-2 and LSE
1e-3, fp32 1e-5.  Sharp bf16 cases (q and k scaled by 3 or 8: near one-hot
rows, so O takes the size of single V entries) take the stress bound of the
attention tests, 1e-2 plus half a bf16 spacing at each O_ref (the rounding
of P and of the stored O), as the flux-sharp inputs do.  The fp32 bounds scale with
the square of that factor: a score's fp32 rounding error grows with
|q| |k| (a D-term dot product in fp32, about D 2^-24 sum |q_i k_i|), and the
weights, O and LSE inherit it, so fp32 cases take 1e-5 max(1, s^2).  Sizes
keep the whole sweep to a few seconds of oracle time."""

import numpy as np
import pytest
import torch

import oracle
import sequence_attention_amd as sa
from sequence_attention_amd import workloads
from tests.gpu_util import DEV, bf16_half_spacing, log, max_abs

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: (1e-2, 1e-3), torch.float32: (1e-5, 1e-5)}
N_CASES = 40


def _draw(i):
    r = np.random.default_rng(1000 + i)
    B = int(r.integers(1, 4))
    Sq = int(r.integers(1, 600))
    Skv = int(r.integers(1, 800))
    H = int(r.integers(1, 7))
    D = int(r.choice([64, 128]))
    mag = float(r.choice([0.25, 1.0, 3.0, 8.0]))
    dtype = torch.float32 if r.random() < 0.25 else torch.bfloat16
    entry = str(r.choice(["fwd", "fwd_ws", "fwd_f32o", "kvlen", "merge"]))
    lens = [int(x) for x in r.integers(0, Skv + 40, size=B)]
    return B, Sq, Skv, H, D, mag, dtype, entry, lens


def _inputs(B, Sq, Skv, H, D, mag, dtype, seed):
    w = workloads.Workload("sweep", B=B, Sq=Sq, Skv=Skv, H=H, D=D, R=1, S=Skv, H_total=H, U=1)
    q, k, v = workloads.attention_inputs(w, dtype=torch.float32, seed=seed)
    q, k = q * mag, k * mag
    return q.to(dtype), k.to(dtype), v.to(dtype), w.scale


def _compare(go, gl, ro, rl, dtype, what, mag=1.0):
    tol_o, tol_l = TOL[dtype]
    sharp = mag >= 3.0
    if dtype == torch.float32:
        tol_o, tol_l = tol_o * max(1.0, mag * mag), tol_l * max(1.0, mag * mag)
    assert np.all(np.isfinite(go)), f"{what}: non-finite O"
    if sharp and dtype == torch.bfloat16:
        excess = np.max(np.abs(go - ro) - (tol_o + bf16_half_spacing(np.abs(ro) + tol_o)))
        assert excess <= 0, f"{what}: O error exceeds 1e-2 + half a bf16 spacing by {excess:.3e}"
    else:
        assert max_abs(go, ro) <= tol_o, f"{what}: O max-abs {max_abs(go, ro):.3e}"
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl)), f"{what}: empty rows differ"
    fin = np.isfinite(rl)
    if fin.any():
        assert max_abs(gl[fin], rl[fin]) <= tol_l, f"{what}: LSE max-abs {max_abs(gl[fin], rl[fin]):.3e}"


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    B, Sq, Skv, H, D, mag, dtype, entry, lens = _draw(i)
    what = f"case {i}: B={B} Sq={Sq} Skv={Skv} H={H} D={D} x{mag} {dtype} {entry}"
    log(what)
    q, k, v, scale = _inputs(B, Sq, Skv, H, D, mag, dtype, seed=i)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    qn, kn, vn = q.float().numpy(), k.float().numpy(), v.float().numpy()
    if entry in ("fwd", "fwd_ws", "fwd_f32o"):
        if entry == "fwd_f32o":   # fp32 O; the tolerance is the inputs' (bf16 arithmetic stays bf16)
            o, lse = sa.dit_attn_fwd(qd, kd, vd, scale=scale, o_dtype=torch.float32)
        else:
            o, lse = sa.dit_attn_fwd(qd, kd, vd, scale=scale, workspace=entry == "fwd_ws")
        ro, rl = oracle.attention(qn, kn, vn, scale)
    elif entry == "kvlen":
        kvl = torch.tensor(lens, dtype=torch.int32, device=DEV)
        o, lse = sa.dit_attn_fwd_kvlen(qd, kd, vd, kvl, scale=scale)
        ro, rl = oracle.attention_kv_len(qn, kn, vn, scale, lens)
    else:
        r = np.random.default_rng(2000 + i)
        o_acc = torch.from_numpy(r.standard_normal((B, Sq, H, D)).astype(np.float32)).to(dtype)
        l_acc = torch.from_numpy((r.standard_normal((B, H, Sq)) * 3).astype(np.float32))
        l_acc[:, :, 0] = -float("inf")          # an empty accumulator row per (batch, head)
        o_acc[:, 0] = float("nan")              # ... whose O must never be read
        oa, la = o_acc.to(DEV), l_acc.to(DEV)
        sa.dit_attn_fwd_merge(qd, kd, vd, oa, la, scale=scale)
        o, lse = oa, la
        po, pl = oracle.attention(qn, kn, vn, scale)
        ro, rl = oracle.merge(np.nan_to_num(o_acc.float().numpy()), l_acc.numpy(), po, pl)
    torch.cuda.synchronize()
    _compare(o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, dtype, what, mag=mag)

"""The shader-clock probe (a measurement aid): both loads report a clock
between 0.5 and 3.0 GHz on every workgroup, and the MFMA load's cycle count
grows with the loop length."""

import pytest
import torch

import sequence_attention_amd as sa
from tests.gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mfma", [False, True])
def test_clock_in_range(mfma):
    log(f"clock probe mfma={mfma}")
    c = sa.dit_clock_probe(workgroups=64, spin=2000, mfma=mfma)
    assert 0.5 < c["min"] <= c["median"] <= c["max"] < 3.0


def test_cycles_grow_with_the_loop():
    out = torch.empty(2 * 8, dtype=torch.int64, device="cuda")
    cyc = []
    for spin in (1000, 4000):
        log(f"clock probe cycles spin={spin}")
        sa.check(sa.lib().dit_clock_probe(sa._dev(out, "out"), 8, spin, 1, sa._stream(None)),
                 "dit_clock_probe")
        torch.cuda.synchronize()
        cyc.append(int(out.view(-1, 2)[:, 0].min()))
    assert cyc[1] > 3 * cyc[0]

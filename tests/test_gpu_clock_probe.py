"""The shader-clock probe (mxfa_clock_probe), the measurement aid bench.py uses.

One wave counts shader-clock cycles against the 100 MHz real-time counter for
a fixed interval; the test checks the interval it reports and that the clock
lies in the chip's range (it cannot know the exact clock).
"""
from __future__ import annotations

import pytest
import torch

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("tiled_attention_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mx.load_library()


@pytest.mark.parametrize("us", [1, 50, 1000])
def test_probe_interval_and_clock_range(us):
    out = torch.full((2,), -1, dtype=torch.int64, device="cuda:0")
    mx.mxfa_clock_probe(out, us)
    torch.cuda.synchronize()
    cycles, ticks = (int(x) for x in out.cpu())
    print(f"[clock] interval {us} us: {cycles} cycles over {ticks} ticks = {cycles / ticks * 100:.0f} MHz", flush=True)
    # the loop ends on the first counter reading at or past the interval
    assert us * 100 <= ticks <= us * 100 + 2000
    assert 100.0 <= cycles / ticks * 100.0 <= 3000.0


def test_probe_on_a_side_stream_in_stream_order():
    side = torch.cuda.Stream()
    out = torch.zeros(4, dtype=torch.int64, device="cuda:0")
    with torch.cuda.stream(side):
        mx.mxfa_clock_probe(out[:2], 20)
        mx.mxfa_clock_probe(out[2:], 20)
    side.synchronize()
    v = out.cpu().tolist()
    assert v[1] >= 2000 and v[3] >= 2000 and v[0] > 0 and v[2] > 0

"""The clock monitor (a measurement aid that bench.py uses to report the
graphics clock each row runs at): its blocks land on distinct XCDs, they stop
when the stop word is set behind a stretch of work on another stream (well
before their time limit), and the clocks they derive are plausible for an
MI355X (between its idle floor and its 2.4 GHz peak, with margin)."""
import pytest
import torch

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp8_scaled_quantization_reduce_amd")


def _monitor_over(work):
    side = torch.cuda.Stream()
    out = torch.full((3 * fq.CLOCK_BLOCKS + 1,), -1, dtype=torch.int64, device="cuda")
    stop = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    fq.fp8q_clock_monitor(out, stop, stream=side)
    work()
    stop.fill_(1)
    torch.cuda.synchronize()
    return out.cpu().tolist()


def test_clock_monitor_over_work():
    x = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    am = torch.empty(1, device="cuda")

    def work():
        for _ in range(100):
            fq.fp8_amax(x, am)

    s = _monitor_over(work)
    xcds = [s[3 * b] for b in range(fq.CLOCK_BLOCKS)]
    assert all(0 <= v < 8 for v in xcds), xcds
    assert len(set(xcds)) >= 2, xcds
    khz = s[3 * fq.CLOCK_BLOCKS]
    assert khz > 0
    for b in range(fq.CLOCK_BLOCKS):
        ticks = s[3 * b + 2]
        # at least the ~2 ms of work, and stopped by the word, not the limit
        assert khz <= ticks < khz * 1000, (b, ticks)
    mhz = fq.clock_mhz(s)
    assert mhz, s
    assert all(50.0 < f < 3000.0 for f in mhz.values()), mhz


def test_clock_monitor_rejects_bad_arguments():
    stop = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        fq.fp8q_clock_monitor(torch.empty(3, dtype=torch.int64, device="cuda"), stop)
    with pytest.raises(TypeError):
        fq.fp8q_clock_monitor(torch.empty(25, dtype=torch.int64, device="cuda"), torch.zeros(1, device="cuda"))

"""The finishing block's bounded wait, forced from the host.

A reducing launch that ends in a finishing block (fp8_amax, the casts with
amax_out, fp8_quantize_delayed) waits for the other blocks' partials for at
most a bounded number of polling rounds.  fp8q_set_finish_poll_rounds(0)
makes every finishing block give up at once, so the bound's path runs
without any wait that could hang: the call must report the canonical NaN,
every kernel still ends, and the partials that the producing blocks publish
after the finishing block gave up (tagged with that call) must not leak into
the next call, which runs with the default bound and must match the oracle.
Expected values come from the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import f32_bits, host, scalar, to_dev

pytestmark = pytest.mark.gpu

fq = pytest.importorskip("fp8_scaled_quantization_reduce_amd")
E4, E5 = oracle.E4M3FN, oracle.E5M2
CANONICAL_NAN = 0x7FC00000


def _pair(seed):
    rng = np.random.default_rng(seed)
    big = workloads.to_bf16_bits(rng.standard_normal((2048, 4096)) * 100.0)
    small = workloads.to_bf16_bits(rng.standard_normal((384, 256)) * 0.5)
    assert oracle.amax(small) < oracle.amax(big)
    return big, small


class _GiveUpAtOnce:
    def __enter__(self):
        self.prev = fq.fp8q_set_finish_poll_rounds(0)
        return self

    def __exit__(self, *exc):
        fq.fp8q_set_finish_poll_rounds(fq.POLL_ROUNDS_DEFAULT)
        return False


def test_knob_reports_the_bound_in_force():
    prev = fq.fp8q_set_finish_poll_rounds(0)
    try:
        assert fq.fp8q_set_finish_poll_rounds(7) == 0
        assert fq.fp8q_set_finish_poll_rounds(fq.POLL_ROUNDS_DEFAULT) == 7
        assert fq.fp8q_set_finish_poll_rounds(fq.POLL_ROUNDS_DEFAULT) == 1 << 21
    finally:
        fq.fp8q_set_finish_poll_rounds(prev)
    with pytest.raises(ValueError):
        fq.fp8q_set_finish_poll_rounds(-1)


def test_amax_gives_nan_at_the_bound_and_the_next_call_is_exact():
    big, small = _pair(0)
    am = scalar(-1.0)
    with _GiveUpAtOnce():
        fq.fp8_amax(to_dev(big), am)
        torch.cuda.synchronize()
    assert f32_bits(host(am)[0]) == CANONICAL_NAN
    # the big input's partials (published after the finishing block gave up)
    # carry the first call's tag: the second call ignores them
    for x in (small, big, small):
        am = scalar(-1.0)
        fq.fp8_amax(to_dev(x), am)
        assert f32_bits(host(am)[0]) == f32_bits(oracle.amax(x))


def test_cast_with_amax_gives_nan_at_the_bound_and_codes_are_unaffected():
    big, small = _pair(1)
    si = scalar(0.25)
    scale = oracle.reciprocal(np.float32(0.25))
    xd = to_dev(big)
    q = torch.empty(big.size, dtype=torch.uint8, device="cuda")
    am = scalar(-1.0)
    with _GiveUpAtOnce():
        fq.fp8_quantize_tensor(xd, E4, q, scale_inv_in=si, amax_out=am)
        torch.cuda.synchronize()
    assert f32_bits(host(am)[0]) == CANONICAL_NAN
    assert np.array_equal(host(q), oracle.quantize(big, E4, scale).ravel())
    qs = torch.empty(small.size, dtype=torch.uint8, device="cuda")
    am = scalar(-1.0)
    fq.fp8_quantize_tensor(to_dev(small), E4, qs, scale_inv_in=si, amax_out=am)
    assert f32_bits(host(am)[0]) == f32_bits(oracle.amax(small))
    assert np.array_equal(host(qs), oracle.quantize(small, E4, scale).ravel())


def test_tile_and_error_feedback_amax_give_nan_at_the_bound():
    big, small = _pair(2)
    rows, cols = big.shape
    qr = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    qc = torch.empty((cols, rows), dtype=torch.uint8, device="cuda")
    res = torch.zeros(big.size, dtype=torch.float32, device="cuda")
    q = torch.empty(big.size, dtype=torch.uint8, device="cuda")
    am, am2 = scalar(-1.0), scalar(-1.0)
    with _GiveUpAtOnce():
        fq.fp8_quantize_rowwise_colwise(to_dev(big), E4, q_row=qr, q_col=qc, scale_inv_in=scalar(2.0), amax_out=am)
        fq.fp8_quantize_error_feedback(to_dev(big), res, E5, scalar(1.0), q, amax_out=am2)
        torch.cuda.synchronize()
    assert f32_bits(host(am)[0]) == CANONICAL_NAN
    assert f32_bits(host(am2)[0]) == CANONICAL_NAN
    sr, sc = small.shape
    qr2 = torch.empty((sr, sc), dtype=torch.uint8, device="cuda")
    qc2 = torch.empty((sc, sr), dtype=torch.uint8, device="cuda")
    am = scalar(-1.0)
    fq.fp8_quantize_rowwise_colwise(to_dev(small), E4, q_row=qr2, q_col=qc2, scale_inv_in=scalar(2.0), amax_out=am)
    assert f32_bits(host(am)[0]) == f32_bits(oracle.amax(small))


def test_delayed_step_records_nan_at_the_bound_then_recovers_in_the_ring():
    """With the bound hit, the step's amax is NaN and the ring records it (the
    window max then propagates NaN, as the pages' rule does for a NaN amax);
    the next steps, with the default bound, record exact amaxes again."""
    big, small = _pair(3)
    L = 4
    hist = torch.zeros((L, 1), dtype=torch.float32, device="cuda")
    scale, scale_inv = scalar(1.0), scalar(1.0)
    q = torch.empty(big.size, dtype=torch.uint8, device="cuda")
    am = scalar(-1.0)
    with _GiveUpAtOnce():
        fq.fp8_quantize_delayed(to_dev(big), E4, hist, 0, 0, E4, 0, 0, scale, scale_inv, q, amax_out=am)
        torch.cuda.synchronize()
    assert f32_bits(host(am)[0]) == CANONICAL_NAN
    assert np.isnan(host(hist)[0, 0])
    qs = torch.empty(small.size, dtype=torch.uint8, device="cuda")
    for step in range(1, L + 1):
        am = scalar(-1.0)
        fq.fp8_quantize_delayed(to_dev(small), E4, hist, 0, step, E4, 0, 0, scale, scale_inv, qs, amax_out=am)
        assert f32_bits(host(am)[0]) == f32_bits(oracle.amax(small))
    # step L overwrote the NaN slot: the window holds only exact amaxes
    h = host(hist)[:, 0]
    assert not np.isnan(h).any()
    assert all(f32_bits(v) == f32_bits(oracle.amax(small)) for v in h)

"""Host-side checks of bench.py's accounting (no GPU): the algorithmic bytes
it prices each workload at are the sizes the workload recipe fixes, summed
by hand here from the shapes and dtypes:

  per call: Bt L [D (s_x + s_Delta + s_y) + N (s_B + s_C)] + 4 D N (A) + 4 D (D)
            [+ 4 D K + 4 D for the conv weights and bias]

fp32 workload 8 x 2048 x 1536 x 16, fp32 in and out   -> 304.2 MB
conv workload 4 x 8192 x 2560 x 16, bf16 in and out   -> 505.6 MB
long workload 1 x 2^20 x 512 x 16,  bf16 in and out   -> 3288 MB
decode token  256 x 5120 x 16, fp32 state read and written, bf16 x, Delta, y,
              B, C rows, A and D                      -> 176.0 MB
"""
from __future__ import annotations

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import ssm_inputs as SI  # noqa: E402


@pytest.mark.parametrize("name,expected", [
    ("fp32", 8 * 2048 * (1536 * 12 + 16 * 8) + 4 * 1536 * 16 + 4 * 1536),
    ("conv", 4 * 8192 * (2560 * 6 + 16 * 4) + 4 * 2560 * 16 + 4 * 2560 + 4 * 2560 * 4 + 4 * 2560),
    ("long", (1 << 20) * (512 * 6 + 16 * 4) + 4 * 512 * 16 + 4 * 512),
])
def test_scan_bytes(name, expected):
    w = SI.WORKLOADS[name]
    assert bench.algorithmic_bytes(w) == expected


def test_scan_bytes_rounded_sizes():
    mb = lambda n: n / 1e6
    assert round(mb(bench.algorithmic_bytes(SI.WORKLOADS["fp32"])), 1) == 304.2
    assert round(mb(bench.algorithmic_bytes(SI.WORKLOADS["conv"])), 1) == 505.6
    assert round(mb(bench.algorithmic_bytes(SI.WORKLOADS["long"]))) == 3288


def test_state_and_fused_extras():
    w = SI.WORKLOADS["fp32"]
    base = bench.algorithmic_bytes(w)
    assert bench.algorithmic_bytes(w, h0=True, h_last=True) - base == 2 * 4 * 8 * 1536 * 16
    # fused without a conv: the gate stream z and the step-size bias
    assert bench.algorithmic_bytes(w, fused=True) - base == 8 * 2048 * 1536 * 4 + 4 * 1536
    c = SI.WORKLOADS["conv"]
    # with a conv also the fp32 window in and out (K - 1 = 3 inputs per channel)
    assert (bench.algorithmic_bytes(c, fused=True) - bench.algorithmic_bytes(c)
            == 4 * 8192 * 2560 * 2 + 4 * 2560 + 2 * 4 * 4 * 2560 * 3)


def test_scan_slots():
    """VALU issue slots: 5 per element for Delta*B (mul, exp, mul, fma, fma;
    a transcendental issues in one slot), 7 for ZOH, plus 2 per (b, t, d)
    (Delta*u and the skip term); the conv prologue adds 8 per (b, t, d)."""
    w = SI.WORKLOADS["fp32"]
    assert bench.algorithmic_slots(w) == pytest.approx(w.elems * 5 + 8 * 2048 * 1536 * 2)
    long_ = SI.WORKLOADS["long"]
    assert bench.algorithmic_slots(long_) == pytest.approx(long_.elems * 5 + (1 << 20) * 512 * 2)
    conv = SI.WORKLOADS["conv"]
    assert bench.algorithmic_slots(conv) == pytest.approx(conv.elems * 7 + 4 * 8192 * 2560 * 10)


def test_decode_bytes():
    w = SI.WORKLOADS["decode"]
    state = 2 * 4 * 256 * 5120 * 16            # h read and written, fp32
    tokens = 256 * 5120 * 3 * 2                # x, Delta, y in bf16
    rows = 2 * 256 * 16 * 2                    # B, C rows in bf16
    params = 4 * 5120 * 17                     # A and D
    assert bench.decode_bytes(w) == state + tokens + rows + params
    assert round(bench.decode_bytes(w) / 1e6, 1) == 176.0
    extra = 256 * 5120 * 2 + 4 * 5120 * 6 + 2 * 4 * 256 * 5120 * 3
    assert bench.decode_bytes(w, fused=True) - bench.decode_bytes(w) == extra

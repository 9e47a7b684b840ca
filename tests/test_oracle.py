"""The fp64 oracle against what the pages and the mathematics fix (closed
forms, hand expansions, brute force, invariants, special cases)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)


def test_operator_associative():
    oracle_pins.pin_operator_associative()


def test_oracle_rejects_bad_arguments(orc):
    import numpy as np
    # dstate < 1 and a missing A are rejected by the library itself
    n = None
    # (batch, L, dim, dstate, x, delta, delta_bias, softplus, A, B, C, Dskip, z, h0,
    #  conv_w, conv_b, conv_k, conv_state_in, zoh, y, h_last, conv_state_out, threads)
    assert orc.lib.ssm_ref_scan_f64(1, 1, 1, 0, n, n, n, 0, n, n, n, n, n, n, n, n, 0, n, 0,
                                    n, n, n, 1) == -1
    assert orc.lib.ssm_ref_scan_f64(1, 1, 1, 1, n, n, n, 0, n, n, n, n, n, n, n, n, 0, n, 0,
                                    n, n, n, 1) == -1
    # a decode step with a conv of more than one tap needs its conv state
    one = np.ones(4)
    p = orc._ptr(one)
    assert orc.lib.ssm_ref_step_f64(1, 1, 1, p, p, p, n, 0, p, p, p, n, n, p, n, 2, n, 0,
                                    p, 1) == -1
    # empty batch is a no-op
    y, h = orc.scan(np.zeros((0, 4, 3)), np.zeros((0, 4, 3)), -np.ones((3, 2)),
                    np.zeros((0, 4, 2)), np.zeros((0, 4, 2)))
    assert y.shape == (0, 4, 3) and h.shape == (0, 3, 2)

"""The pool K/V criterion of the GPU tests, on the CPU: one bf16 step of the oracle's value
(plus a tiny floor near zero) passes, two steps fail, and the message names the element."""
import numpy as np
import pytest

from gpu_util import KV_FLOOR, assert_kv_close, bf16_ulp
from oracle import dflash_oracle as O


def _bits(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_bf16_ulp_values():
    assert bf16_ulp(np.array([1.0]))[0] == 2.0 ** -7
    assert bf16_ulp(np.array([1.5]))[0] == 2.0 ** -7
    assert bf16_ulp(np.array([-0.75]))[0] == 2.0 ** -8
    assert bf16_ulp(np.array([0.0]))[0] == 0.0


def test_one_step_passes_two_steps_fail():
    rng = np.random.default_rng(0)
    want = O.round_bf16(rng.standard_normal((4, 2, 32)))
    wb = _bits(want)
    assert np.array_equal(O.widen(wb), want)
    assert_kv_close(wb, want, "exact")
    up = wb.copy()
    up[1, 1, 5] += 1                       # one bf16 step up (positive or negative value alike)
    assert_kv_close(up, want, "one step")
    big = np.abs(want) >= 1.0
    idx = tuple(np.argwhere(big)[0])
    two = wb.copy()
    two[idx] += 2
    with pytest.raises(AssertionError, match=f"kv head {idx[1]}, element {idx[2]}") as e:
        assert_kv_close(two, want, "layer 3 V", slots=np.array([10, 11, 12, 13]))
    assert f"slot {10 + idx[0]}" in str(e.value) and "layer 3 V" in str(e.value)


def test_floor_near_zero():
    want = np.zeros((1, 1, 4))
    want[0, 0, 0] = 4.0
    got = want.copy()
    got[0, 0, 1] = 0.9 * KV_FLOOR * 4.0
    assert_kv_close(_bits(got), want, "floor")
    got[0, 0, 1] = 1.1 * KV_FLOOR * 4.0
    with pytest.raises(AssertionError):
        assert_kv_close(_bits(got), want, "floor")

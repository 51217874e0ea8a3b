"""The element-local parity checker itself (CPU, no GPU).

The GPU parity tests bound, besides the whole-tensor normalized L2, the
error of every row, every 32 x 32 block and every 256 x 256 tile of each
output (tests/_util.py, local_errors). Here the checker gets synthetic data
of the 1024 -> 2816, B=8, S=2048 training shapes (Y and dI [16384, 1024],
dWg and dWu [1024, 2816], dWd [2816, 1024]): the reference plus noise at the
bf16 rounding floor measured on the GPU (normalized L2 about 3.6e-3) must
pass, and each planted localized fault must be flagged, including faults the
whole-tensor figure alone lets through.
"""

import numpy as np
import pytest

from tests._util import local_errors, local_ok, nl2

TOL = 1e-2
FLOOR = 3.6e-3


def _pair(shape, seed):
    rng = np.random.default_rng(seed)
    ref = rng.standard_normal(shape)
    got = ref + FLOOR * rng.standard_normal(shape)
    return got, ref


@pytest.mark.parametrize("shape", [(16384, 1024), (1024, 2816), (2816, 1024)])
def test_rounding_floor_passes(shape):
    got, ref = _pair(shape, 1)
    e = local_errors(got, ref)
    assert local_ok(e, TOL), e
    assert 3e-3 < e["whole"] < 4.5e-3


def test_zeroed_row_is_flagged_though_whole_tensor_passes():
    got, ref = _pair((16384, 1024), 2)
    got[5000] = 0.0
    assert nl2(got, ref) <= TOL          # the global figure alone misses it
    e = local_errors(got, ref)
    assert not local_ok(e, TOL)
    assert e["row"] > 0.9 and e["row_at"] == 5000
    assert e["block"] > TOL and e["block_at"][0] == 5000 // 32


def test_wrong_mfma_block_is_flagged_though_whole_tensor_passes():
    # one 32 x 32 block of Y that dropped 1/64 of its K sum: each element off
    # by about 1/8 of its size
    got, ref = _pair((16384, 1024), 3)
    rng = np.random.default_rng(4)
    blk = (slice(32 * 300, 32 * 301), slice(32 * 7, 32 * 8))
    got[blk] = ref[blk] + 0.125 * rng.standard_normal((32, 32))
    assert nl2(got, ref) <= TOL
    e = local_errors(got, ref)
    assert not local_ok(e, TOL)
    assert e["block_at"] == (300, 7) and e["block"] > 0.1


def test_perturbed_block_of_weight_gradient_is_flagged():
    got, ref = _pair((1024, 2816), 5)
    rng = np.random.default_rng(6)
    got[320:352, 640:672] = rng.standard_normal((32, 32))  # a block from the wrong operands
    e = local_errors(got, ref)
    assert not local_ok(e, TOL)
    assert e["block_at"] == (10, 20)


def test_misreduced_split_tile_is_flagged():
    # a 256 x 256 tile of dWd whose split-K reduction lost one of 4 pieces
    got, ref = _pair((2816, 1024), 7)
    rng = np.random.default_rng(8)
    t = (slice(256 * 9, 256 * 10), slice(256 * 2, 256 * 3))
    got[t] = ref[t] + 0.5 * rng.standard_normal((256, 256))
    e = local_errors(got, ref)
    assert not local_ok(e, TOL)
    assert e["tile_at"] == (9, 2)


def test_ragged_edges_and_non_finite_values():
    got, ref = _pair((777, 136), 9)
    assert local_ok(local_errors(got, ref), TOL)
    got[776, 135] = np.nan
    e = local_errors(got, ref)
    assert not local_ok(e, TOL)
    got[776, 135] = ref[776, 135]
    got[0, 0] = np.inf
    assert not local_ok(local_errors(got, ref), TOL)


def test_small_region_is_measured_against_tensor_scale():
    # a region of tiny reference values (e.g. near-cancelling sums) with
    # floor-level absolute error is not a fault
    got, ref = _pair((256, 256), 10)
    ref[:32, :32] *= 1e-6
    got[:32, :32] = ref[:32, :32] + FLOOR * np.random.default_rng(11).standard_normal((32, 32))
    assert local_ok(local_errors(got, ref), TOL)

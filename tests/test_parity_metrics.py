"""CPU tests of the error measures the GPU parity tests use: each measure
catches the failure it is there for (a wrong tile, a corner of one, a single
wrong element), where the whole-matrix relative error would not."""
import numpy as np
import pytest

from parity_metrics import bucket_errors, matrix_errors, summary


def _pair(seed=0, shape=(1024, 2816), noise=1e-3):
    rng = np.random.default_rng(seed)
    r = rng.standard_normal(shape) / np.sqrt(shape[1])
    o = r + noise * np.abs(r).mean() * rng.standard_normal(shape)
    return o, r


def test_exact_and_noise_floor():
    o, r = _pair(noise=0.0)
    e = matrix_errors(o, r)
    assert e["rel"] == 0.0 and e["block_rel"] == 0.0 and e["elem_max"] == 0.0 and e["cos"] == pytest.approx(1.0)
    o, r = _pair(noise=1e-3)
    e = matrix_errors(o, r)
    # uniform noise: every block sees about the matrix's relative error
    assert e["block_rel"] == pytest.approx(e["rel"], rel=0.1)


@pytest.mark.parametrize("part", [1.0, 0.25, 1 / 16])
def test_wrong_tile_is_caught_by_the_block_measure(part):
    """Zero out (part of) one 256 x 256 tile of a 2048 x 4096 matrix (128
    tiles): for a sixteenth of a tile the whole-matrix error stays below the
    3e-2 bar (on the 7B bucket's 688 tiles even a whole tile moves it by only
    1/sqrt(688) = 3.8%), the block measure does not."""
    o, r = _pair(shape=(2048, 4096), noise=1e-3)
    h = int(256 * np.sqrt(part))
    o[512:512 + h, 768:768 + h] = 0.0
    e = matrix_errors(o, r)
    assert e["block_rel"] >= 0.2
    if part <= 1 / 16:
        assert e["rel"] < 3e-2


def test_single_wrong_element_is_caught_by_the_element_measure():
    o, r = _pair(noise=1e-3)
    rms = np.sqrt(np.mean(r * r))
    o[700, 2000] += 10 * rms
    e = matrix_errors(o, r)
    assert e["elem_max"] >= 9.9
    assert e["rel"] < 1e-2 and e["block_rel"] < 0.1


def test_ragged_edge_block_uses_its_own_elements():
    o, r = _pair(shape=(300, 1000), noise=0.0)
    o[290:, 990:] = 0.0  # the 10 x 10 corner of the last (ragged) block
    e = matrix_errors(o, r)
    assert e["block_rel"] > 0.05


def test_bucket_and_summary():
    o1, r1 = _pair(0)
    o2, r2 = _pair(1, noise=2e-3)
    errs = bucket_errors(np.stack([o1, o2]), np.stack([r1, r2]))
    s = summary(errs)
    assert s["n"] == 2 and s["rel_max"] == max(e["rel"] for e in errs)
    assert s["cos_min"] == min(e["cos"] for e in errs)
    assert summary([]) == {"n": 0}

"""The parity bars themselves (host logic, no GPU): at the full-width output
scale (RMS 0.025, about the size of the 2e-2 element bar) they must reject
the mistakes the element bar alone lets through -- a uniform 10% error, one
head scaled 3% off, one wrong row -- and accept bf16-sized rounding noise."""
import numpy as np
import pytest

import datagen as dg
from gpu_util import assert_parity, assert_tensor_close

ROWS, H, DV = 64, 96, 128


def _ref(seed=0):
    return np.random.default_rng(seed).standard_normal((ROWS, H * DV)) * 0.025


def _noise(ref, rel, seed=1):
    return ref * (1 + rel * np.random.default_rng(seed).standard_normal(ref.shape))


def test_rounding_noise_passes():
    ref = _ref()
    assert_parity(_noise(ref, 2.0 ** -8), ref, dg.BF16, "noise", block=DV)


@pytest.mark.parametrize("mistake", ["uniform 10%", "head 3%", "one row", "one head block"])
def test_mistakes_the_element_bar_misses_are_rejected(mistake):
    ref = _ref()
    got = _noise(ref, 2.0 ** -8)
    if mistake == "uniform 10%":
        got = got * 1.10
    elif mistake == "head 3%":
        got.reshape(ROWS, H, DV)[:, 17] *= 1.03
    elif mistake == "one row":
        got[5] *= 1.05
    else:
        got.reshape(ROWS, H, DV)[7, 40] *= 0.9
    assert np.abs(got - ref).max() <= 2e-2, "the element bar alone would pass this"
    with pytest.raises(AssertionError):
        assert_parity(got, ref, dg.BF16, mistake, block=DV)


def test_gradient_slices():
    rng = np.random.default_rng(3)
    ref = rng.standard_normal((2, 50, 8, 64))
    ok = ref * (1 + 2.0 ** -8 * rng.standard_normal(ref.shape))
    slices = [("row", (100, 8 * 64), (0,)), ("head", (100, 8, 64), (1,))]
    assert_tensor_close(ok, ref, "noise", slices)
    bad = ok.copy()
    bad[1, 3] *= 1.03               # one row 3% off, invisible in the whole tensor
    with pytest.raises(AssertionError):
        assert_tensor_close(bad, ref, "one slice", [("row", (100, 8 * 64), (0,))])
    bad = ok.copy()
    bad[:, :, 2] *= 1.03            # one head 3% off everywhere
    with pytest.raises(AssertionError):
        assert_tensor_close(bad, ref, "one head", [("head", (100, 8, 64), (1,))])
    # a slice that is exactly zero is held to an absolute bar
    z = ref.copy()
    z[0, 0] = 0.0
    g = ok.copy()
    g[0, 0] = 1e-3 * np.sqrt(np.mean(ref * ref))
    assert_tensor_close(g, z, "near-zero slice, small noise", slices)
    g[0, 0] = 0.05 * np.sqrt(np.mean(ref * ref))
    with pytest.raises(AssertionError):
        assert_tensor_close(g, z, "near-zero slice, large noise", slices)

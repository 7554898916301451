"""The gradient parity check itself (tests/tolerances.py): it accepts rounding-sized deviations
and rejects the plausible mistakes a kernel could make (a dropped term, a wrong sign, a scale
factor, a transposed operand), on a seeded stand-in for a gradient tensor."""
import numpy as np

from tolerances import GRAD_ATOL_RMS, grad_excess


def _ref():
    rng = np.random.default_rng(7)
    return rng.standard_normal((4, 33, 2, 64)) * rng.uniform(0.1, 3.0, (1, 33, 1, 1))


def test_accepts_rounding_noise():
    ref = _ref()
    rms = np.sqrt(np.mean(ref * ref))
    noise = np.random.default_rng(8).standard_normal(ref.shape) * 2 * 2.0 ** -9 * rms
    assert grad_excess(ref + noise, ref) <= 1.0
    assert grad_excess(ref * (1 + 2.0 ** -8), ref) <= 1.0


def test_rejects_mistakes():
    ref = _ref()
    assert grad_excess(ref * 1.05, ref) > 1.0                      # a 5% scale error
    assert grad_excess(-ref, ref) > 1.0                            # a sign
    bad = ref.copy()
    bad[1, 7, 0] = 0.0                                            # one row dropped
    assert grad_excess(bad, ref) > 1.0
    assert grad_excess(ref[:, :, ::-1].copy(), ref) > 1.0         # heads swapped
    assert grad_excess(np.swapaxes(ref[:, :32, :, :32], 1, 3).copy(), ref[:, :32, :, :32]) > 1.0
    # a small element's error is judged against the tensor's scale, not its largest value
    small = ref.copy()
    k = np.unravel_index(np.argmin(np.abs(ref)), ref.shape)
    small[k] += 2 * GRAD_ATOL_RMS * np.sqrt(np.mean(ref * ref))
    assert grad_excess(small, ref) > 1.0


def test_zero_gradient_floor():
    z = np.zeros((3, 5))
    assert grad_excess(z + 5e-5, z) <= 1.0
    assert grad_excess(z + 2e-4, z) > 1.0

"""The worst-row error measure the full-size parity tests gate on (CPU)."""
import numpy as np

from parity_metrics import rel, row_err


def test_single_wrong_row_is_caught_where_whole_tensor_error_is_not():
    """One replaced row among 131072 (the global-mask workload's 16 heads x
    8192 rows): the whole-tensor error stays under the bf16 gate, the
    worst-row error does not."""
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((16, 8192, 128))
    x = ref * (1 + 2e-3 * rng.standard_normal(ref.shape))
    assert rel(x, ref) < 2e-2 and row_err(x, ref) < 2e-2
    x[3, 100] = rng.standard_normal(128)
    assert rel(x, ref) < 2e-2
    assert row_err(x, ref) > 0.5


def test_rows_small_by_cancellation_are_measured_against_the_typical_row():
    """A row whose reference is tiny is measured against the RMS row norm,
    so that its rounding-sized error does not read as a relative blow-up."""
    ref = np.ones((4, 8))
    ref[2] = 1e-9
    x = ref.copy()
    x[2] += 1e-4
    assert abs(row_err(x, ref) - 1e-4 * np.sqrt(8) / np.sqrt(np.mean(np.sum(ref * ref, axis=1)))) < 1e-12


def test_scalar_rows():
    ref = np.array([1.0, 2.0, 4.0])
    x = np.array([1.0, 2.0, 4.4])
    assert abs(row_err(x, ref) - 0.1) < 1e-12
    assert row_err(ref, ref) == 0.0

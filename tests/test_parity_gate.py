"""The GPU parity gate's own logic, on the CPU: the per-row check catches an
error confined to small-magnitude rows that the per-tensor max-norm lets
through, and treats exactly-zero reference rows and all-zero tensors as the
per-tensor check does."""
import numpy as np
import pytest

from tests.gpu_util import TOL_BF16, assert_close, elementwise_err, row_errs


def _grad_like(seed=0, rows=256, d=64):
    """Rows whose magnitude decays like the late keys of a causal dK / dV."""
    rng = np.random.default_rng(seed)
    scale = 1.0 / (1.0 + np.arange(rows))[:, None]
    return rng.standard_normal((rows, d)) * scale


def test_localised_error_in_small_rows_is_caught():
    ref = _grad_like()
    bad = ref.copy()
    bad[-10:] *= 1.5                     # 50% wrong, but in rows ~1/250 of the largest
    assert assert_close("t", bad, ref, TOL_BF16) <= TOL_BF16     # the per-tensor gate passes it
    with pytest.raises(AssertionError, match="row"):
        assert_close("t", bad, ref, TOL_BF16, row_len=ref.shape[1])


def test_rounding_sized_errors_pass_the_row_gate():
    ref = _grad_like(1)
    x = ref * (1 + 2.0**-8 * np.sign(np.random.default_rng(2).standard_normal(ref.shape)))
    assert assert_close("t", x, ref, TOL_BF16, row_len=ref.shape[1]) < 5e-3
    assert elementwise_err(x, ref) < 5e-3


def test_zero_rows_and_zero_tensors():
    ref = _grad_like(3)
    ref[0] = 0.0                         # e.g. the first query of a causal head: dQ = 0 exactly
    x = ref.copy()
    x[0] = 1e-4                          # rounding noise there: no relative error, per-tensor covers it
    assert row_errs(x, ref, ref.shape[1])[0] == 0.0
    assert_close("t", x, ref, TOL_BF16, row_len=ref.shape[1])
    z = np.zeros((4, 8))
    assert np.allclose(row_errs(z + 1e-3, z, 8), 1e-3)     # all-zero reference: absolute
    with pytest.raises(AssertionError):
        assert_close("t", z + 0.5, z, TOL_BF16, row_len=8)

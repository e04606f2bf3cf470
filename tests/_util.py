"""Helpers shared by the tests: the error metric and small conveniences."""
import numpy as np


def norm_err(got, ref) -> float:
    """max |got - ref| / max |ref| over one tensor; absolute max error if ref is all zero."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    scale = float(np.max(np.abs(ref)))
    err = float(np.max(np.abs(got - ref)))
    return err / scale if scale > 0 else err


SCAN_OUTPUTS = ("d_u", "d_delta", "d_A_log", "d_B", "d_C", "d_D", "d_z")

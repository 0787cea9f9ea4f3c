"""Error metrics used by the parity tests (test infrastructure only).

max_abs   = max |O - O*|
rel_l2    = ||O - O*||_F / ||O*||_F over the whole tensor
lse_max   = max |L - L*|

These are the tolerance metrics of the parity gate (maximum absolute error,
relative L2 error over the whole tensor, largest logsumexp error).  Pinned by
hand-computed cases and planted mistakes in tests/test_compare_pins.py.
"""

import numpy as np


def errors(o, o_ref, lse=None, lse_ref=None):
    o = np.asarray(o, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    diff = o - o_ref
    out = {
        "max_abs": float(np.max(np.abs(diff))) if diff.size else 0.0,
        "rel_l2": float(np.linalg.norm(diff) / max(np.linalg.norm(o_ref), 1e-300)) if diff.size else 0.0,
    }
    if lse is not None:
        dl = np.asarray(lse, dtype=np.float64) - np.asarray(lse_ref, dtype=np.float64)
        out["lse_max"] = float(np.max(np.abs(dl))) if dl.size else 0.0
    return out

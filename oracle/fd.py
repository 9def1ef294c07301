"""Central finite differences of the scalar  <dy, y(inputs)>  -- TEST INFRASTRUCTURE."""
from __future__ import annotations

import numpy as np


def central_diff(fwd, inputs: dict, name: str, index, dy, eps: float = 1e-6) -> float:
    """d<dy, y>/d inputs[name][index] by a central difference with step eps."""
    plus = {k: np.array(v, dtype=np.float64, copy=True) for k, v in inputs.items()}
    minus = {k: np.array(v, dtype=np.float64, copy=True) for k, v in inputs.items()}
    plus[name][index] += eps
    minus[name][index] -= eps
    fp = float(np.sum(fwd(**plus) * dy))
    fm = float(np.sum(fwd(**minus) * dy))
    return (fp - fm) / (2.0 * eps)

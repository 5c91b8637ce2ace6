"""Central finite differences, float64 (test infrastructure only).

The Rust course checks its tiled gradients by finite-differencing every Q, K, V
coordinate with step 1e-6 and absolute tolerance 4e-6 (intale.github.io ch. 19,
"Compare derivatives, then the same restored model").  This helper does the
same for any scalar function of a list of arrays.
"""

import numpy as np


def gradient(fn, arrays, step=1e-6):
    """d fn / d a for every coordinate of every array in ``arrays``.

    fn(arrays) -> float; the arrays are perturbed in place and restored.
    """
    grads = []
    for a in arrays:
        g = np.zeros_like(a, dtype=np.float64)
        flat = a.reshape(-1)
        gflat = g.reshape(-1)
        for k in range(flat.size):
            x0 = flat[k]
            flat[k] = x0 + step
            fp = fn(arrays)
            flat[k] = x0 - step
            fm = fn(arrays)
            flat[k] = x0
            gflat[k] = (fp - fm) / (2.0 * step)
        grads.append(g)
    return grads

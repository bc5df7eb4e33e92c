"""Tolerance bars derived from the arithmetic (test-only)."""

import numpy as np


def grad_w_extra(gz, y):
    """Extra absolute bar for grad_W[i, j] = sum over every (token, channel)
    pair of t = gz[., i, .] * y[., j, .]. fp32 accumulation of such a sum
    errs by about u * sqrt(chain length) * sqrt(sum t^2); 1e-5 * sqrt(sum t^2)
    is about 170 units of rounding at that scale, which covers any chain the
    kernels use while a dropped or mis-paired term (of size |t|) still shows."""
    H, D = gz.shape[-2], gz.shape[-1]
    g = np.asarray(gz).reshape(-1, H, D)
    v = np.asarray(y).reshape(-1, H, D)
    acc = np.zeros((H, H))
    for s in range(0, g.shape[0], 2048):
        gb = g[s:s + 2048].astype(np.float64)
        vb = v[s:s + 2048].astype(np.float64)
        acc += (gb * gb).transpose(1, 0, 2).reshape(H, -1) @ (vb * vb).transpose(1, 0, 2).reshape(H, -1).T
    return 1e-5 * np.sqrt(acc)

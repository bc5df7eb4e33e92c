"""Tolerance bars derived from the arithmetic (test-only)."""

import numpy as np

# A float32 sum of n products t_k, accumulated in any order or blocking, errs by
# about u * sqrt(n) * sqrt(sum t_k^2) (u = 2^-24 per rounding, errors of random
# sign); with n up to 65,536 that is at most 256 u = 1.5e-5 of sqrt(sum t^2), and
# the mixer kernels' accumulators (4 products per MFMA step, partial sums per K
# tile and per split) keep each chain far shorter. RMS_TERM = 1e-5 is about 170
# units of rounding of sqrt(sum t^2) -- above what any of those chains makes,
# while a dropped or mis-paired term, of size |t| (about sqrt(sum t^2 / n)),
# still shows for every n up to 10^9.
RMS_TERM = 1e-5


def _sq(a):
    a = np.asarray(a, np.float64)
    return a * a


def mix_forward_extra(y, W):
    """Extra absolute bar of z[m, o] = sum_k W[o, k] y[m, k]: RMS_TERM times
    sqrt(sum_k (W[o, k] y[m, k])^2), shaped like y."""
    F = W.shape[0]
    Y = np.asarray(y).reshape(-1, F)
    return (RMS_TERM * np.sqrt(_sq(Y) @ _sq(W).T)).reshape(np.shape(y))


def mix_grad_y_extra(gz, W):
    """Extra bar of grad_y[m, k] = sum_o gz[m, o] W[o, k]."""
    F = W.shape[0]
    G = np.asarray(gz).reshape(-1, F)
    return (RMS_TERM * np.sqrt(_sq(G) @ _sq(W))).reshape(np.shape(gz))


def mix_grad_w_extra(gz, y):
    """Extra bar of grad_W[o, k] = sum_m gz[m, o] y[m, k] (sum over every token)."""
    F = np.shape(y)[-2] * np.shape(y)[-1]
    G = np.asarray(gz).reshape(-1, F)
    Y = np.asarray(y).reshape(-1, F)
    acc = np.zeros((F, F))
    for s in range(0, G.shape[0], 4096):
        acc += _sq(G[s:s + 4096]).T @ _sq(Y[s:s + 4096])
    return RMS_TERM * np.sqrt(acc)

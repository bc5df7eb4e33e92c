"""Pins of the oracle's MIMO head mixer (CPU).

The mixer (index.html lab 02 "MIMO MIXER": a fully connected mixer across the
SSM heads, identity at initialisation) is read as one H x H matrix shared by
every token and channel: z[m, i, d] = sum_j W[i, j] y[m, j, d]. These tests tie
the oracle's loops to facts fixed independently of them:
  * the pages' initial state of the mixer, the identity, leaves y unchanged;
  * a permutation matrix permutes the heads, and a single off-diagonal link
    copies one head into another (what one "cross-head link" means);
  * a hand-worked 2-head example;
  * numpy's matmul over the head axis (a library routine, not the oracle's
    loops);
  * the gradients: exact central differences of the oracle's own forward
    (the map is linear, so a difference quotient with small-integer inputs is
    exact), and the adjoint identity <gz, W y> = <W^T gz, y>.
A mutation test plants plausible mistakes (a transposed weight, a swapped
head index, a truncated sum) in copies of the oracle source and checks that
the pins catch each one.
"""

import os
import shutil
import tempfile

import numpy as np
import pytest

import oracle


def _ints(rng, shape, lo=-4, hi=5):
    return rng.integers(lo, hi, size=shape).astype(np.float32)


def pin_identity(lib):
    rng = np.random.default_rng(0)
    y = rng.standard_normal((3, 5, 16, 64)).astype(np.float32)
    z = oracle.head_mix(y, np.eye(16, dtype=np.float32), lib=lib)
    assert np.array_equal(z, y.astype(np.float64))


def pin_permutation(lib):
    rng = np.random.default_rng(1)
    H = 7
    y = rng.standard_normal((4, H, 9)).astype(np.float32)
    perm = rng.permutation(H)
    W = np.zeros((H, H), np.float32)
    W[np.arange(H), perm] = 1.0
    z = oracle.head_mix(y, W, lib=lib)
    assert np.array_equal(z, y[:, perm, :].astype(np.float64))


def pin_single_link(lib):
    rng = np.random.default_rng(2)
    H = 16
    y = rng.standard_normal((2, 3, H, 8)).astype(np.float32)
    W = np.zeros((H, H), np.float32)
    W[3, 11] = 1.0
    z = oracle.head_mix(y, W, lib=lib)
    expect = np.zeros_like(z)
    expect[..., 3, :] = y[..., 11, :]
    assert np.array_equal(z, expect)


def pin_hand_worked(lib):
    # W = [[1, 2], [3, 4]], one token, D = 2 with head rows (5, 6) and (7, 8):
    # head 0 = 1*(5, 6) + 2*(7, 8) = (19, 22); head 1 = 3*(5, 6) + 4*(7, 8) = (43, 50)
    y = np.array([[[5, 6], [7, 8]]], np.float32)
    W = np.array([[1, 2], [3, 4]], np.float32)
    z = oracle.head_mix(y, W, lib=lib)
    assert np.array_equal(z, np.array([[[19, 22], [43, 50]]], np.float64))


def pin_numpy_matmul(lib):
    rng = np.random.default_rng(3)
    y = rng.standard_normal((2, 6, 12, 10)).astype(np.float32)
    W = rng.standard_normal((12, 12)).astype(np.float32)
    z = oracle.head_mix(y, W, lib=lib)
    ref = np.matmul(W.astype(np.float64), y.astype(np.float64))
    assert np.abs(z - ref).max() < 1e-12 * (1 + np.abs(ref).max())


def pin_difference_quotients(lib, H, D):
    rng = np.random.default_rng(H * 10 + D)
    M = 3
    y = _ints(rng, (M, H, D))
    W = _ints(rng, (H, H))
    gz = _ints(rng, (M, H, D))
    gy, gW = oracle.head_mix_backward(y, W, gz, lib=lib)
    gzd = gz.astype(np.float64)
    loss = lambda yy, WW: float((gzd * oracle.head_mix(yy, WW, lib=lib)).sum())
    step = 1.0  # the loss is linear in y and in W: exact with integer data
    for idx in np.ndindex(W.shape):
        Wp, Wm = W.copy(), W.copy()
        Wp[idx] += step
        Wm[idx] -= step
        assert (loss(y, Wp) - loss(y, Wm)) / (2 * step) == gW[idx], ("W", idx)
    for idx in list(np.ndindex(y.shape))[:: max(1, y.size // 40)]:
        yp, ym = y.copy(), y.copy()
        yp[idx] += step
        ym[idx] -= step
        assert (loss(yp, W) - loss(ym, W)) / (2 * step) == gy[idx], ("y", idx)


def pin_adjoint(lib):
    rng = np.random.default_rng(7)
    y = rng.standard_normal((5, 16, 64)).astype(np.float32)
    W = rng.standard_normal((16, 16)).astype(np.float32)
    gz = rng.standard_normal((5, 16, 64)).astype(np.float32)
    gy, gW = oracle.head_mix_backward(y, W, gz, lib=lib)
    z = oracle.head_mix(y, W, lib=lib)
    lhs = (gz.astype(np.float64) * z).sum()
    scale = np.abs(gz).sum() * np.abs(z).max()
    assert abs(lhs - (gy * y).sum()) < 1e-9 * scale
    # W enters linearly: <gW, W> is the same loss again
    assert abs(lhs - (gW * W).sum()) < 1e-9 * scale


def pin_zero_tokens(lib):
    y = np.zeros((0, 4, 8), np.float32)
    W = np.eye(4, dtype=np.float32)
    assert oracle.head_mix(y, W, lib=lib).shape == (0, 4, 8)
    gy, gW = oracle.head_mix_backward(y, W, y, lib=lib)
    assert gy.shape == (0, 4, 8) and np.array_equal(gW, np.zeros((4, 4)))


PINS = {
    "identity": pin_identity,
    "permutation": pin_permutation,
    "single_link": pin_single_link,
    "hand_worked": pin_hand_worked,
    "numpy_matmul": pin_numpy_matmul,
    "fd_2x3": lambda lib: pin_difference_quotients(lib, 2, 3),
    "fd_5x4": lambda lib: pin_difference_quotients(lib, 5, 4),
    "fd_16x2": lambda lib: pin_difference_quotients(lib, 16, 2),
    "adjoint": pin_adjoint,
    "zero_tokens": pin_zero_tokens,
}


@pytest.mark.parametrize("name", sorted(PINS))
def test_mixer_pin(name):
    PINS[name](oracle.load())


# --------------------------------------------------------------- planted bugs

_MIX_PLANTS = {
    "forward_W_transposed": ("acc += (double)W[i * H + j] * (double)y[(m * H + j) * D + d];",
                             "acc += (double)W[j * H + i] * (double)y[(m * H + j) * D + d];"),
    "forward_output_head_read": ("acc += (double)W[i * H + j] * (double)y[(m * H + j) * D + d];",
                                 "acc += (double)W[i * H + j] * (double)y[(m * H + i) * D + d];"),
    "grad_y_W_not_transposed": ("acc += (double)W[i * H + j] * (double)gz[(m * H + i) * D + d];",
                                "acc += (double)W[j * H + i] * (double)gz[(m * H + i) * D + d];"),
    "grad_W_heads_swapped": (
        "acc += (double)gz[(m * H + i) * D + d] * (double)y[(m * H + j) * D + d];",
        "acc += (double)gz[(m * H + j) * D + d] * (double)y[(m * H + i) * D + d];"),
    "grad_W_first_token_only": (
        "for (int64_t m = 0; m < M; ++m)\n                    for (int64_t d = 0; d < D; ++d)\n"
        "                        acc += (double)gz",
        "for (int64_t m = 0; m < 1; ++m)\n                    for (int64_t d = 0; d < D; ++d)\n"
        "                        acc += (double)gz"),
    "grad_W_channels_misaligned": (
        "acc += (double)gz[(m * H + i) * D + d] * (double)y[(m * H + j) * D + d];",
        "acc += (double)gz[(m * H + i) * D + d] * (double)y[(m * H + j) * D + (D - 1 - d)];"),
}


@pytest.fixture(scope="module")
def plant_dir():
    d = tempfile.mkdtemp(prefix="oracle_mix_plants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("plant", sorted(_MIX_PLANTS))
def test_planted_mixer_mistake_is_caught(plant, plant_dir):
    src = open(oracle.SOURCE).read()
    old, new = _MIX_PLANTS[plant]
    assert src.count(old) == 1, "plant anchor must be unique: %s" % plant
    path = os.path.join(plant_dir, plant + ".c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.load(oracle.build(os.path.join(plant_dir, plant + ".so"), source=path))
    caught = []
    for name, pin in PINS.items():
        try:
            pin(lib)
        except AssertionError:
            caught.append(name)
    assert caught, "planted mistake %s went unnoticed" % plant

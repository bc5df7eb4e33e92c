"""Pins of the oracle's MIMO head mixer (CPU).

The mixer is a dense real map of a token's flattened heads: with F = H * D
and k = h * D + d, z[m, o] = sum_k W[o, k] y[m, k] for an (F, F) matrix W
(index.html lab 02 "MIMO MIXER": 1024 -> 1024 as 16 heads of 64, identity at
initialisation, 240 off-diagonal head links = the 16 * 15 off-diagonal D x D
blocks; the parameter count of the "Extending" guide's documentation rule,
433,662,400, holds only with a dense 1024 x 1024 matrix per layer). These tests
tie the oracle's loops to facts fixed independently of them:
  * the pages' initial state, the identity, leaves y unchanged;
  * a block permutation (P kron I_D) permutes whole heads, and one
    off-diagonal block feeds one head from another through that block (what a
    "cross-head link" is);
  * a Kronecker-structured W = W_h kron I_D mixes heads channel by channel
    (the special case where every link is a multiple of the identity);
  * a hand-worked 4 x 4 example that mixes channels inside a head;
  * numpy's float64 matmul (a library routine, not the oracle's loops), for
    the forward and both gradients;
  * the gradients: exact central differences of the oracle's own forward
    (the loss is linear in y and in W, so a difference quotient with
    small-integer inputs is exact), and the adjoint identity.
A mutation test plants plausible mistakes in copies of the oracle source (a
transposed weight, links shared across channels, a channel-major flattening,
a truncated sum, swapped gradient operands) and checks that the pins catch each.
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
    z = oracle.head_mix(y, np.eye(16 * 64, dtype=np.float32), lib=lib)
    assert np.array_equal(z, y.astype(np.float64))


def pin_head_permutation(lib):
    rng = np.random.default_rng(1)
    H, D = 7, 5
    y = rng.standard_normal((4, H, D)).astype(np.float32)
    perm = rng.permutation(H)
    P = np.zeros((H, H), np.float32)
    P[np.arange(H), perm] = 1.0
    z = oracle.head_mix(y, np.kron(P, np.eye(D, dtype=np.float32)), lib=lib)
    assert np.array_equal(z, y[:, perm, :].astype(np.float64))


def pin_single_block_link(lib):
    rng = np.random.default_rng(2)
    H, D = 16, 8
    y = _ints(rng, (2, 3, H, D))
    K = _ints(rng, (D, D))
    W = np.zeros((H * D, H * D), np.float32)
    W[3 * D:4 * D, 11 * D:12 * D] = K  # head 11 -> head 3 through K
    z = oracle.head_mix(y, W, lib=lib)
    expect = np.zeros(z.shape)
    for m in np.ndindex(y.shape[:2]):
        for i in range(D):
            expect[m + (3, i)] = sum(float(K[i, j]) * float(y[m + (11, j)]) for j in range(D))
    assert np.array_equal(z, expect)


def pin_kronecker_heads(lib):
    rng = np.random.default_rng(4)
    H, D = 5, 6
    y = _ints(rng, (3, H, D))
    Wh = _ints(rng, (H, H))
    z = oracle.head_mix(y, np.kron(Wh, np.eye(D, dtype=np.float32)), lib=lib)
    expect = np.zeros(z.shape)
    for m in range(3):
        for i in range(H):
            for d in range(D):
                expect[m, i, d] = sum(float(Wh[i, j]) * float(y[m, j, d]) for j in range(H))
    assert np.array_equal(z, expect)


def pin_hand_worked(lib):
    # H = 2 heads of D = 2 channels, y = (5, 6 | 7, 8) flattened head-major and
    #   W = [[1, 2, 0, 0],     z0 = 1*5 + 2*6         = 17
    #        [0, 1, 0, 0],     z1 = 6                 = 6
    #        [0, 0, 1, 0],     z2 = 7                 = 7
    #        [3, 0, 0, 1]]     z3 = 3*5 + 8           = 23
    y = np.array([[[5, 6], [7, 8]]], np.float32)
    W = np.array([[1, 2, 0, 0], [0, 1, 0, 0], [0, 0, 1, 0], [3, 0, 0, 1]], np.float32)
    z = oracle.head_mix(y, W, lib=lib)
    assert np.array_equal(z, np.array([[[17, 6], [7, 23]]], np.float64))
    # gradients with grad_z = (1, 0, 0, 1): grad_y = W^T grad_z = (4, 2, 0, 1) and
    # grad_W = grad_z (outer) y: rows 0 and 3 equal y, rows 1 and 2 zero
    gz = np.array([[[1, 0], [0, 1]]], np.float32)
    gy, gW = oracle.head_mix_backward(y, W, gz, lib=lib)
    assert np.array_equal(gy, np.array([[[4, 2], [0, 1]]], np.float64))
    expect = np.zeros((4, 4))
    expect[0] = expect[3] = (5, 6, 7, 8)
    assert np.array_equal(gW, expect)


def pin_numpy_matmul(lib):
    rng = np.random.default_rng(3)
    H, D = 6, 10
    y = rng.standard_normal((2, 7, H, D)).astype(np.float32)
    W = rng.standard_normal((H * D, H * D)).astype(np.float32)
    gz = rng.standard_normal(y.shape).astype(np.float32)
    z = oracle.head_mix(y, W, lib=lib)
    Y = y.astype(np.float64).reshape(-1, H * D)
    G = gz.astype(np.float64).reshape(-1, H * D)
    W64 = W.astype(np.float64)
    ref = (Y @ W64.T).reshape(y.shape)
    assert np.abs(z - ref).max() < 1e-12 * (1 + np.abs(ref).max())
    gy, gW = oracle.head_mix_backward(y, W, gz, lib=lib)
    ref_gy = (G @ W64).reshape(y.shape)
    ref_gW = G.T @ Y
    assert np.abs(gy - ref_gy).max() < 1e-12 * (1 + np.abs(ref_gy).max())
    assert np.abs(gW - ref_gW).max() < 1e-12 * (1 + np.abs(ref_gW).max())


def pin_difference_quotients(lib, H, D):
    rng = np.random.default_rng(H * 10 + D)
    M = 3
    F = H * D
    y = _ints(rng, (M, H, D))
    W = _ints(rng, (F, F))
    gz = _ints(rng, (M, H, D))
    gy, gW = oracle.head_mix_backward(y, W, gz, lib=lib)
    gzd = gz.astype(np.float64)
    loss = lambda yy, WW: float((gzd * oracle.head_mix(yy, WW, lib=lib)).sum())
    step = 1.0  # the loss is linear in y and in W: exact with integer data
    for idx in list(np.ndindex(W.shape))[:: max(1, W.size // 60)]:
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
    H, D = 4, 16
    y = rng.standard_normal((5, H, D)).astype(np.float32)
    W = rng.standard_normal((H * D, H * D)).astype(np.float32)
    gz = rng.standard_normal((5, H, D)).astype(np.float32)
    gy, gW = oracle.head_mix_backward(y, W, gz, lib=lib)
    z = oracle.head_mix(y, W, lib=lib)
    lhs = (gz.astype(np.float64) * z).sum()
    scale = np.abs(gz).sum() * np.abs(z).max()
    assert abs(lhs - (gy * y).sum()) < 1e-9 * scale
    # W enters linearly: <gW, W> is the same loss again
    assert abs(lhs - (gW * W).sum()) < 1e-9 * scale


def pin_zero_tokens(lib):
    y = np.zeros((0, 4, 8), np.float32)
    W = np.eye(32, dtype=np.float32)
    assert oracle.head_mix(y, W, lib=lib).shape == (0, 4, 8)
    gy, gW = oracle.head_mix_backward(y, W, y, lib=lib)
    assert gy.shape == (0, 4, 8) and np.array_equal(gW, np.zeros((32, 32)))


PINS = {
    "identity": pin_identity,
    "head_permutation": pin_head_permutation,
    "single_block_link": pin_single_block_link,
    "kronecker_heads": pin_kronecker_heads,
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


def test_the_parameter_count_needs_a_dense_mixer():
    """The model size the pages fix (433,662,400) from the layer shapes they
    give: tied embedding 50,257 x 1024; per layer in_proj 1024 x 16(64 + 4*64
    + 1), the mixer, out_proj 1024 x 1024, a SwiGLU of 3 * 1024 * 2048, two
    RMSNorm weights and A (16 complex entries); 28 layers and a final norm.
    Only the dense (H*D)^2 mixer makes it add up; one H x H matrix gives the
    figure the pages rule out (404M)."""
    hidden, H, D, N, layers, vocab, ffn = 1024, 16, 64, 64, 28, 50257, 2048

    def total(mixer):
        per_layer = (hidden * H * (D + 4 * N + 1) + mixer + hidden * hidden
                     + 3 * hidden * ffn + 2 * hidden + H)
        return vocab * hidden + layers * per_layer + hidden

    assert total((H * D) ** 2) == 433_662_400
    assert total(H * H) == 404_309_440


# --------------------------------------------------------------- planted bugs

_MIX_PLANTS = {
    "forward_W_transposed": [(
        "acc += (double)W[o * F + k] * (double)y[m * F + k];",
        "acc += (double)W[k * F + o] * (double)y[m * F + k];")],
    "forward_links_shared_across_channels": [(
        "acc += (double)W[o * F + k] * (double)y[m * F + k];",
        "acc += (k % D == o % D) ? (double)W[o * F + k] * (double)y[m * F + k] : 0.0;")],
    "forward_channel_major_flattening": [(
        "acc += (double)W[o * F + k] * (double)y[m * F + k];",
        "acc += (double)W[o * F + k] * (double)y[m * F + (k % D) * H + k / D];")],
    "forward_last_input_dropped": [(
        "for (int64_t k = 0; k < F; ++k)\n                acc += (double)W",
        "for (int64_t k = 0; k < F - 1; ++k)\n                acc += (double)W")],
    "grad_y_W_not_transposed": [(
        "row[k] += g * (double)W[o * F + k];",
        "row[k] += g * (double)W[k * F + o];")],
    "grad_y_first_output_dropped": [(
        "for (int64_t o = 0; o < F; ++o) {\n                const double g = (double)gz[m * F + o];",
        "for (int64_t o = 1; o < F; ++o) {\n                const double g = (double)gz[m * F + o];")],
    "grad_W_operands_swapped": [
        ("const double g = (double)gz[m * F + o];\n                    double *row = gW",
         "const double g = (double)y[m * F + o];\n                    double *row = gW"),
        ("row[k] += g * (double)y[m * F + k];", "row[k] += g * (double)gz[m * F + k];")],
    "grad_W_first_token_only": [(
        "for (int64_t m = 0; m < M; ++m)\n                for (int64_t o = o0;",
        "for (int64_t m = 0; m < 1; ++m)\n                for (int64_t o = o0;")],
}


@pytest.fixture(scope="module")
def plant_dir():
    d = tempfile.mkdtemp(prefix="oracle_mix_plants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("plant", sorted(_MIX_PLANTS))
def test_planted_mixer_mistake_is_caught(plant, plant_dir):
    src = open(oracle.SOURCE).read()
    for old, new in _MIX_PLANTS[plant]:
        assert src.count(old) == 1, "plant anchor must be unique: %s" % plant
        src = src.replace(old, new)
    path = os.path.join(plant_dir, plant + ".c")
    with open(path, "w") as f:
        f.write(src)
    lib = oracle.load(oracle.build(os.path.join(plant_dir, plant + ".so"), source=path))
    caught = []
    for name, pin in PINS.items():
        try:
            pin(lib)
        except AssertionError:
            caught.append(name)
    assert caught, "planted mistake %s went unnoticed" % plant

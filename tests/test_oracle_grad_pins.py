"""Pins for the oracle's gradients (runs without a GPU).

The backward oracle (oracle_scan_backward: reverse-mode through the plain
recurrence) is fixed against things other than itself:
  * central finite differences of the forward oracle's loss, for every real
    component of every input, on small shapes;
  * torch's autograd through a plain complex128 loop of the recurrence (this
    pins the gradient convention for complex inputs: dl/dRe + i dl/dIm);
  * the chunkwise re-association of the gradients (tests/chunkwise_ref.py),
    which is the algebra the GPU backward uses, for many chunk sizes;
  * exact special cases: a step with nothing before it has zero decay
    gradient, batch rows add up in the gradient of A;
and a mutation test plants plausible mistakes in copies of the oracle source
and checks that the finite-difference pin catches each one.
"""

import os
import shutil
import tempfile

import numpy as np
import pytest

import oracle
import ssd_inputs
from chunkwise_ref import chunkwise_scan_backward


def _rand_complex(rng, shape, scale=1.0):
    return ((rng.standard_normal(shape) + 1j * rng.standard_normal(shape)) * scale)


def _problem(shape, seed, with_final=True, with_init=True, dt_scale=1.0):
    Bsz, T, H, N, D = shape
    inp = ssd_inputs.random_case(Bsz, T, H, N, D, seed, dt_scale=dt_scale)
    rng = np.random.default_rng(seed + 1000)
    arrays = {
        "x": inp.x.numpy().copy(), "A": inp.A.numpy().copy(), "B_t": inp.B_t.numpy().copy(),
        "C_t": inp.C_t.numpy().copy(), "dt": inp.dt.numpy().copy(),
    }
    gy = rng.standard_normal((Bsz, T, H, D)).astype(np.float32)
    gf = _rand_complex(rng, (Bsz, H, N, D)).astype(np.complex64) if with_final else None
    init = _rand_complex(rng, (Bsz, H, N, D), 0.5) if with_init else None
    return arrays, gy, gf, init


def _loss(arrays, gy, gf, init, lib=None):
    y, fs = oracle.scan(arrays["x"], arrays["A"], arrays["B_t"], arrays["C_t"], arrays["dt"],
                        initial_state=init, threads=1, lib=lib)
    val = float((gy.astype(np.float64) * y.real).sum())
    if gf is not None:
        val += float((np.conj(gf.astype(np.complex128)) * fs).real.sum())
    return val


def _fd_component(arrays, name, idx, part, gy, gf, init, h, lib=None):
    """Central difference of the loss along one real component, with the
    perturbed values rounded to float32 and the exact step they imply."""
    base = arrays[name]
    orig = base[idx]
    vals = []
    steps = []
    for sgn in (1.0, -1.0):
        if np.iscomplexobj(base):
            v = complex(orig) + (sgn * h if part == 0 else 1j * sgn * h)
            base[idx] = np.complex64(v)
            steps.append(float(base[idx].real if part == 0 else base[idx].imag))
        else:
            base[idx] = np.float32(float(orig) + sgn * h)
            steps.append(float(base[idx]))
        vals.append(_loss(arrays, gy, gf, init, lib))
    base[idx] = orig
    return (vals[0] - vals[1]) / (steps[0] - steps[1])


def _fd_init_component(arrays, idx, part, gy, gf, init, h, lib=None):
    vals = []
    for sgn in (1.0, -1.0):
        i2 = init.copy()
        i2[idx] += sgn * h if part == 0 else 1j * sgn * h
        vals.append(_loss(arrays, gy, gf, i2, lib))
    return (vals[0] - vals[1]) / (2 * h)


def _check_fd(arrays, gy, gf, init, lib=None, max_per_input=None, rng=None):
    g = oracle.scan_backward(arrays["x"], arrays["A"], arrays["B_t"], arrays["C_t"],
                             arrays["dt"], gy, gf, init, threads=1, lib=lib)
    grads = {"x": g.x, "A": g.A, "B_t": g.B_t, "C_t": g.C_t, "dt": g.dt}
    for name, grad in grads.items():
        arr = arrays[name]
        idxs = list(np.ndindex(arr.shape))
        if max_per_input is not None and len(idxs) > max_per_input:
            pick = rng.choice(len(idxs), max_per_input, replace=False)
            idxs = [idxs[i] for i in pick]
        # x, B_t and C_t enter the loss linearly: the central difference is
        # exact up to rounding. dt and A enter through exp(softplus(dt) A).
        linear = name in ("x", "B_t", "C_t")
        h = 1e-2 if linear else 2e-3
        tol = 1e-9 if linear else 2e-5
        for idx in idxs:
            parts = (0, 1) if np.iscomplexobj(arr) else (0,)
            for part in parts:
                fd = _fd_component(arrays, name, idx, part, gy, gf, init, h, lib)
                an = grad[idx].real if part == 0 else (grad[idx].imag if np.iscomplexobj(arr) else 0)
                if not np.iscomplexobj(arr):
                    an = grad[idx]
                assert abs(fd - an) <= tol * (1.0 + abs(fd)), (name, idx, part, fd, an)
    if init is not None:
        for idx in list(np.ndindex(init.shape))[: (max_per_input or init.size)]:
            for part in (0, 1):
                fd = _fd_init_component(arrays, idx, part, gy, gf, init, 1e-2, lib)
                an = g.initial_state[idx].real if part == 0 else g.initial_state[idx].imag
                assert abs(fd - an) <= 1e-9 * (1.0 + abs(fd)), ("init", idx, part, fd, an)
    return g


@pytest.mark.parametrize("shape,seed,final,init", [
    ((2, 6, 2, 4, 3), 0, True, True),
    ((1, 9, 1, 2, 2), 1, False, False),
    ((1, 5, 3, 2, 3), 2, True, False),
    ((2, 4, 1, 6, 2), 3, False, True),
])
def test_gradients_match_finite_differences(shape, seed, final, init):
    arrays, gy, gf, i0 = _problem(shape, seed, final, init)
    _check_fd(arrays, gy, gf, i0)


def test_gradients_match_finite_differences_strong_dt():
    """Larger steps: the softplus and exp factors far from their linear range."""
    arrays, gy, gf, init = _problem((1, 7, 2, 2, 2), 7, True, True, dt_scale=3.0)
    _check_fd(arrays, gy, gf, init)


def test_gradients_match_torch_autograd():
    """A plain complex128 loop of the recurrence under torch.autograd; complex
    leaves receive dl/dRe + i dl/dIm, the convention the oracle follows."""
    import torch
    arrays, gy, gf, init = _problem((2, 8, 2, 4, 3), 11, True, True)
    t = {k: torch.tensor(v.astype(np.complex128 if np.iscomplexobj(v) else np.float64),
                         requires_grad=True) for k, v in arrays.items()}
    s0 = torch.tensor(init, dtype=torch.complex128, requires_grad=True)
    Bsz, T, H, D = arrays["x"].shape
    loss = 0
    finals = []
    for b in range(Bsz):
        for h in range(H):
            s = s0[b, h]
            for k in range(T):
                abar = torch.exp(torch.nn.functional.softplus(t["dt"][b, k, h]) * t["A"][h])
                s = abar * s + t["B_t"][b, k, h][:, None] * t["x"][b, k, h][None, :]
                y = (t["C_t"][b, k, h][:, None] * s).sum(0)
                loss = loss + (torch.tensor(gy[b, k, h], dtype=torch.float64) * y.real).sum()
            finals.append(s)
    fs = torch.stack(finals).reshape(Bsz, H, *finals[0].shape)
    loss = loss + (torch.conj(torch.tensor(gf, dtype=torch.complex128)) * fs).real.sum()
    loss.backward()
    g = oracle.scan_backward(arrays["x"], arrays["A"], arrays["B_t"], arrays["C_t"],
                             arrays["dt"], gy, gf, init)
    for name, mine in (("x", g.x), ("A", g.A), ("B_t", g.B_t), ("C_t", g.C_t), ("dt", g.dt)):
        ref = t[name].grad.numpy()
        assert np.abs(mine - ref).max() <= 1e-11 * (1 + np.abs(ref).max()), name
    assert np.abs(g.initial_state - s0.grad.numpy()).max() <= 1e-11 * (1 + np.abs(s0.grad.numpy()).max())


@pytest.mark.parametrize("chunk", [1, 2, 3, 5, 8, 16, 31, 32, 64])
def test_chunkwise_gradients_equal_the_oracle(chunk):
    arrays, gy, gf, init = _problem((2, 45, 2, 6, 5), 20 + chunk, True, True)
    g = oracle.scan_backward(arrays["x"], arrays["A"], arrays["B_t"], arrays["C_t"],
                             arrays["dt"], gy, gf, init)
    ref = chunkwise_scan_backward(arrays["x"], arrays["A"], arrays["B_t"], arrays["C_t"],
                                  arrays["dt"], gy, chunk, gf, init)
    for name, a, r in zip(g._fields, g, ref):
        assert np.abs(a - r).max() <= 1e-12 * (1 + np.abs(a).max()), name


def test_first_step_decay_gradient_is_zero_without_initial_state():
    """With a zero initial state nothing precedes token 0, so its decay factor
    multiplies zero: its dt gradient is exactly zero."""
    arrays, gy, gf, _ = _problem((2, 10, 3, 4, 4), 31, True, False)
    g = oracle.scan_backward(arrays["x"], arrays["A"], arrays["B_t"], arrays["C_t"],
                             arrays["dt"], gy, gf, None)
    assert np.all(g.dt[:, 0, :] == 0.0)


def test_gradient_of_A_adds_over_batch_rows():
    arrays, gy, gf, init = _problem((3, 12, 2, 4, 3), 41, True, True)
    g = oracle.scan_backward(arrays["x"], arrays["A"], arrays["B_t"], arrays["C_t"],
                             arrays["dt"], gy, gf, init)
    acc = 0
    for b in range(3):
        sub = {k: (v[b:b + 1] if k != "A" else v) for k, v in arrays.items()}
        gb = oracle.scan_backward(sub["x"], sub["A"], sub["B_t"], sub["C_t"], sub["dt"],
                                  gy[b:b + 1], gf[b:b + 1], init[b:b + 1])
        acc = acc + gb.A
        assert np.array_equal(gb.x[0], g.x[b])
    assert np.abs(acc - g.A).max() <= 1e-13 * (1 + np.abs(g.A).max())


def test_no_upstream_gradient_gives_zero():
    arrays, _, _, init = _problem((1, 6, 2, 2, 2), 51, False, True)
    gy = np.zeros((1, 6, 2, 2), np.float32)
    g = oracle.scan_backward(arrays["x"], arrays["A"], arrays["B_t"], arrays["C_t"],
                             arrays["dt"], gy, None, init)
    for v in g:
        assert np.all(v == 0)


def test_zero_length_passes_the_final_gradient_through():
    rng = np.random.default_rng(3)
    Bsz, H, N, D = 2, 2, 4, 3
    x = np.zeros((Bsz, 0, H, D), np.complex64)
    Bm = np.zeros((Bsz, 0, H, N), np.complex64)
    dt = np.zeros((Bsz, 0, H), np.float32)
    A = _rand_complex(rng, H).astype(np.complex64)
    gf = _rand_complex(rng, (Bsz, H, N, D)).astype(np.complex64)
    g = oracle.scan_backward(x, A, Bm, Bm, dt, np.zeros((Bsz, 0, H, D), np.float32), gf)
    assert np.array_equal(g.initial_state, gf.astype(np.complex128))
    assert np.all(g.A == 0)


# --------------------------------------------------------------- planted bugs

_GRAD_PLANTS = {
    "adjoint_C_not_conjugated": ("cplx cn = conj(load_c(Ct, row * N + n));",
                                 "cplx cn = load_c(Ct, row * N + n);"),
    "gB_x_not_conjugated": ("acc_b += lam[n * D + d] * conj(load_c(x, row * D + d));",
                            "acc_b += lam[n * D + d] * load_c(x, row * D + d);"),
    "gx_B_not_conjugated": ("acc += conj(load_c(Bt, row * N + n)) * lam[n * D + d];",
                            "acc += load_c(Bt, row * N + n) * lam[n * D + d];"),
    "gC_from_previous_state": ("const cplx *s_t = states + (t + 1) * ND;",
                               "const cplx *s_t = states + t * ND;"),
    "decay_grad_from_current_state": ("const cplx *s_prev = states + t * ND;",
                                      "const cplx *s_prev = states + (t + 1) * ND;"),
    "decay_grad_abar_not_conjugated": ("cplx ga = conj(Abar) * g_abar;", "cplx ga = Abar * g_abar;"),
    "dt_grad_no_sigmoid": ("* sigmoid((double)dt[row]);", ";"),
    "dt_grad_A_not_conjugated": ("gdt[row] = creal(conj(Ah) * ga)", "gdt[row] = creal(Ah * ga)"),
    "A_grad_no_softplus": ("gA_acc += sp * ga;", "gA_acc += ga;"),
    "adjoint_decay_not_conjugated": ("lam[i] = conj(Abar) * lam[i];", "lam[i] = Abar * lam[i];"),
    "final_gradient_ignored": ("lam[i] = grad_final ?", "lam[i] = 0 ?"),
    "sigmoid_wrong_sign": ("return 1.0 / (1.0 + exp(-v));", "return 1.0 / (1.0 + exp(v));"),
}


def _grad_battery(lib):
    failed = []
    rng = np.random.default_rng(5)
    for shape, seed in (((2, 6, 2, 4, 3), 60), ((1, 5, 1, 2, 2), 61)):
        arrays, gy, gf, init = _problem(shape, seed, True, True)
        try:
            _check_fd(arrays, gy, gf, init, lib=lib, max_per_input=12, rng=rng)
        except (AssertionError, RuntimeError):
            failed.append(shape)
    return failed


@pytest.fixture(scope="module")
def plant_dir():
    d = tempfile.mkdtemp(prefix="oracle_grad_plants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def test_grad_battery_passes_on_the_real_oracle():
    assert _grad_battery(oracle.load()) == []


@pytest.mark.parametrize("plant", sorted(_GRAD_PLANTS))
def test_planted_gradient_mistake_is_caught(plant, plant_dir):
    src = open(oracle.SOURCE).read()
    old, new = _GRAD_PLANTS[plant]
    assert src.count(old) == 1, "plant anchor must be unique: %s" % plant
    path = os.path.join(plant_dir, plant + ".c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.load(oracle.build(os.path.join(plant_dir, plant + ".so"), source=path))
    assert _grad_battery(lib), "planted mistake %s went unnoticed" % plant

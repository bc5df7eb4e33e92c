"""Pins for the CPU oracle (runs without a GPU).

Each test fixes part of the oracle against something other than itself:
brute-force sums, closed forms, library routines and invariants that follow
from the recurrence defined on the Mamba-3-Lite pages ("Extending" guide,
Path A Step 1; index.html lab 03). A mutation test at the end plants plausible
mistakes in a copy of the oracle source and checks that these pins catch them.
"""

import cmath
import math
import os
import shutil
import subprocess
import sys
import tempfile

import numpy as np
import pytest

import oracle
import ssd_inputs
from chunkwise_ref import chunkwise_scan

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")


def _np(inp):
    return (inp.x.numpy().astype(np.complex128), inp.A.numpy().astype(np.complex128),
            inp.B_t.numpy().astype(np.complex128), inp.C_t.numpy().astype(np.complex128),
            inp.dt.numpy().astype(np.float64))


def _run(inp, lib=None, **kw):
    return oracle.scan(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt, lib=lib, **kw)


def _close(a, b, rel=1e-12):
    a = np.asarray(a)
    b = np.asarray(b)
    scale = 1.0 + max(np.abs(a).max(initial=0.0), np.abs(b).max(initial=0.0))
    return np.abs(a - b).max(initial=0.0) <= rel * scale


# ----------------------------------------------------------------- brute force

def _brute_force(x, A, Bm, Cm, dt):
    """Dual (unrolled) form, pure Python: y_t = sum_{k<=t} (C_t . B_k) prod_{k<j<=t} Abar_j x_k."""
    Bsz, T, H, D = x.shape
    N = Bm.shape[-1]
    y = np.zeros((Bsz, T, H, D), np.complex128)
    fs = np.zeros((Bsz, H, N, D), np.complex128)
    for b in range(Bsz):
        for h in range(H):
            abar = [cmath.exp(math.log(1.0 + math.exp(float(dt[b, j, h]))) * complex(A[h]))
                    for j in range(T)]
            for t in range(T):
                for d in range(D):
                    acc = 0j
                    for k in range(t + 1):
                        w = 0j
                        for n in range(N):
                            w += complex(Cm[b, t, h, n]) * complex(Bm[b, k, h, n])
                        p = 1 + 0j
                        for j in range(k + 1, t + 1):
                            p *= abar[j]
                        acc += w * p * complex(x[b, k, h, d])
                    y[b, t, h, d] = acc
            for n in range(N):
                for d in range(D):
                    acc = 0j
                    for k in range(T):
                        p = 1 + 0j
                        for j in range(k + 1, T):
                            p *= abar[j]
                        acc += complex(Bm[b, k, h, n]) * p * complex(x[b, k, h, d])
                    fs[b, h, n, d] = acc
    return y, fs


@pytest.mark.parametrize("shape,seed", [((2, 9, 2, 4, 3), 0), ((1, 12, 3, 1, 2), 1),
                                        ((2, 7, 1, 3, 1), 2), ((1, 1, 2, 2, 2), 3)])
def test_brute_force_dual_form(shape, seed):
    B, T, H, N, D = shape
    inp = ssd_inputs.random_case(B, T, H, N, D, seed, dt_scale=1.5)
    y, fs = _run(inp)
    yb, fb = _brute_force(*_np(inp))
    assert _close(y, yb), np.abs(y - yb).max()
    assert _close(fs, fb), np.abs(fs - fb).max()


def test_brute_force_tiny_recipe():
    """The Skills-page tiny recipe (seed 0), both dt variants, checked by brute force."""
    for tv in (False, True):
        inp = ssd_inputs.tiny_case(tv)
        y, fs = _run(inp)
        yb, fb = _brute_force(*_np(inp))
        assert _close(y, yb), np.abs(y - yb).max()
        assert _close(fs, fb)


# ------------------------------------------------------- discretisation pins

def test_discretise_matches_library_softplus():
    inp = ssd_inputs.random_case(2, 23, 3, 2, 2, 5, dt_scale=8.0)
    abar, lam = oracle.discretise(inp.dt, inp.A, chunk=5)
    x, A, _, _, dt = _np(inp)
    a = np.logaddexp(0.0, dt) * A[None, None, :]
    assert _close(abar, np.exp(a), 1e-14)
    nc = lam.shape[2]
    assert lam.shape == (2, 3, 5, 5)
    for c in range(nc):
        seg = a[:, c * 5:min(c * 5 + 5, 23), :]
        cs = np.cumsum(seg, axis=1).transpose(0, 2, 1)
        k = cs.shape[-1]
        assert _close(lam[:, :, c, :k], cs, 1e-14)
        # positions past T carry the last real running sum
        for j in range(k, 5):
            assert _close(lam[:, :, c, j], cs[..., -1], 1e-14)


def test_discretise_softplus_special_values():
    """softplus(0) = ln 2 (Abar = 2^A); softplus(ln(e-1)) = 1 (Abar = e^A); large dt -> dt."""
    A = np.array([-0.7 + 0.3j, 0.2 - 1.1j], np.complex64)
    dt = np.array([[[0.0, 0.0], [math.log(math.e - 1.0)] * 2, [40.0, 40.0]]], np.float32)
    abar, _ = oracle.discretise(dt, A)
    A64 = A.astype(np.complex128)
    assert _close(abar[0, 0], 2.0 ** A64, 1e-14)
    # dt is rounded to float32 at the boundary, so softplus is 1 within ~1e-7
    assert _close(abar[0, 1], np.exp(A64), 1e-6)
    assert _close(abar[0, 2], np.exp(40.0 * A64), 1e-12)


# ---------------------------------------------------------------- closed forms

def test_dt_zero_closed_form():
    """dt = 0: Abar = 2^A, s_t = sum_{k<=t} Abar^(t-k) B_k x_k^T."""
    inp = ssd_inputs.random_case(2, 11, 2, 3, 4, 11, dt_scale=0.0)
    y, fs = _run(inp)
    x, A, Bm, Cm, _ = _np(inp)
    T = x.shape[1]
    for b in range(2):
        for h in range(2):
            ab = 2.0 ** A[h]
            for t in range(T):
                s = sum((ab ** (t - k)) * np.outer(Bm[b, k, h], x[b, k, h]) for k in range(t + 1))
                assert _close(y[b, t, h], Cm[b, t, h] @ s)
                if t == T - 1:
                    assert _close(fs[b, h], s)


def _scalar_inputs(T, A, dt=0.0):
    one = np.ones((1, T, 1, 1), np.complex64)
    return (one, np.array([A], np.complex64), one, one, np.full((1, T, 1), dt, np.float32))


def test_scalar_worked_example_golden():
    """N=D=H=B=1, A=-1, dt=0, x=B=C=1: Abar = 1/2 and y_t = 2 - 2^-t (geometric series)."""
    rows = []
    with open(os.path.join(GOLDEN, "scalar_halving.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([float(v) for v in line.split()])
    T = len(rows)
    y, fs = oracle.scan(*_scalar_inputs(T, -1.0))
    for t, yt in rows:
        assert abs(y[0, int(t), 0, 0] - yt) <= 1e-15 * 2
        assert abs(y[0, int(t), 0, 0].imag) == 0.0
    assert abs(fs[0, 0, 0, 0] - rows[-1][1]) <= 1e-15 * 2


def test_pure_rotation_geometric_series():
    """A = i*omega, dt = 0: Abar = e^{i theta}, theta = omega ln 2; y_t = (1 - e^{i theta (t+1)}) / (1 - e^{i theta})."""
    omega = float(np.float32(1.3))  # A reaches the oracle as complex64
    T = 40
    y, _ = oracle.scan(*_scalar_inputs(T, 1j * omega))
    th = omega * math.log(2.0)
    for t in range(T):
        want = (1 - cmath.exp(1j * th * (t + 1))) / (1 - cmath.exp(1j * th))
        assert abs(y[0, t, 0, 0] - want) <= 1e-12


def test_single_step_ignores_decay():
    """T = 1: y_0 = (C_0 . B_0) x_0 whatever A and dt are."""
    inp = ssd_inputs.random_case(3, 1, 2, 4, 5, 21, dt_scale=3.0)
    y, fs = _run(inp)
    x, A, Bm, Cm, _ = _np(inp)
    want = np.einsum("bthn,bthn->bth", Cm, Bm)[..., None] * x
    assert _close(y, want)
    assert _close(fs, np.einsum("bhn,bhd->bhnd", Bm[:, 0], x[:, 0]))


def test_memoryless_limit():
    """Re A = -1e4: Abar underflows to 0 and y_t = (C_t . B_t) x_t."""
    inp = ssd_inputs.random_case(2, 9, 2, 3, 2, 4)
    inp.A = (inp.A * 0 + (-1e4 + 0.5j)).to(inp.A.dtype)
    y, _ = _run(inp)
    x, A, Bm, Cm, _ = _np(inp)
    want = np.einsum("bthn,bthn->bth", Cm, Bm)[..., None] * x
    assert _close(y, want)


# ------------------------------------------------------------------ invariants

def test_conjugation_symmetry():
    inp = ssd_inputs.random_case(2, 13, 2, 4, 3, 8)
    y, fs = _run(inp)
    c = ssd_inputs.ScanInputs(inp.x.conj().resolve_conj(), inp.A.conj().resolve_conj(),
                              inp.B_t.conj().resolve_conj(), inp.C_t.conj().resolve_conj(), inp.dt)
    yc, fc = _run(c)
    assert _close(yc, np.conj(y))
    assert _close(fc, np.conj(fs))


@pytest.mark.parametrize("which", ["x", "B_t", "C_t"])
def test_linearity(which):
    import torch
    i1 = ssd_inputs.random_case(1, 10, 2, 4, 3, 9)
    i2 = ssd_inputs.random_case(1, 10, 2, 4, 3, 10)
    al, be = 0.75 - 0.5j, -1.25 + 0.25j
    mix = ssd_inputs.ScanInputs(i1.x, i1.A, i1.B_t, i1.C_t, i1.dt)
    other = ssd_inputs.ScanInputs(i1.x, i1.A, i1.B_t, i1.C_t, i1.dt)
    v1, v2 = getattr(i1, which), getattr(i2, which)
    setattr(mix, which, (al * v1.to(torch.complex128) + be * v2.to(torch.complex128)))
    setattr(other, which, v2)
    ym, _ = _run(mix)
    y1, _ = _run(i1)
    y2, _ = _run(other)
    # inputs are rounded to complex64 at the boundary; compare in that precision
    assert _close(ym, al * y1 + be * y2, 1e-6)


def test_causality_bit_exact():
    inp = ssd_inputs.random_case(1, 20, 2, 4, 3, 12)
    y, _ = _run(inp)
    t0 = 11
    inp.x[:, t0] += 3.0
    inp.B_t[:, t0 + 2] -= 1.0
    inp.dt[:, t0] += 2.0
    y2, _ = _run(inp)
    assert np.array_equal(y[:, :t0], y2[:, :t0])
    assert not np.allclose(y[:, t0:], y2[:, t0:])


def test_head_and_batch_independence():
    inp = ssd_inputs.random_case(3, 8, 4, 2, 3, 13)
    y, fs = _run(inp)
    perm = [2, 0, 3, 1]
    bperm = [1, 2, 0]
    p = ssd_inputs.ScanInputs(inp.x[bperm][:, :, perm], inp.A[perm], inp.B_t[bperm][:, :, perm],
                              inp.C_t[bperm][:, :, perm], inp.dt[bperm][:, :, perm])
    yp, fp = _run(p)
    assert np.array_equal(yp, y[bperm][:, :, perm])
    assert np.array_equal(fp, fs[bperm][:, perm])


def test_initial_state_composes_segments():
    """run(T1) then run(T2 | final_state) equals run(T1 + T2)."""
    inp = ssd_inputs.random_case(2, 30, 2, 4, 3, 14)
    y, fs = _run(inp)
    a = ssd_inputs.ScanInputs(inp.x[:, :17], inp.A, inp.B_t[:, :17], inp.C_t[:, :17], inp.dt[:, :17])
    b = ssd_inputs.ScanInputs(inp.x[:, 17:].contiguous(), inp.A, inp.B_t[:, 17:].contiguous(),
                              inp.C_t[:, 17:].contiguous(), inp.dt[:, 17:].contiguous())
    ya, fa = _run(a)
    yb, fb = _run(b, initial_state=fa)
    assert _close(np.concatenate([ya, yb], axis=1), y)
    assert _close(fb, fs)


# ------------------------------------------------------ chunkwise re-association

@pytest.mark.parametrize("chunk", [1, 2, 3, 4, 5, 8, 16, 29, 64])
def test_chunkwise_equals_naive(chunk):
    """The chunkwise algebra (per-chunk cumsum, L, Y_diag, chunk states,
    inter-chunk passing, state-to-output) reproduces the oracle for every chunk
    size, dividing T or not, with time-varying dt and several N."""
    for N in (2, 4, 6, 8):
        inp = ssd_inputs.random_case(2, 29, 2, N, 3, 100 + N, dt_scale=1.0, dt_mean=0.5)
        y, fs = _run(inp)
        yc, fc = chunkwise_scan(*_np(inp), chunk)
        assert _close(y, yc), (chunk, N, np.abs(y - yc).max())
        assert _close(fs, fc)


def test_chunkwise_with_initial_state():
    inp = ssd_inputs.random_case(1, 19, 2, 4, 3, 31)
    rng = np.random.default_rng(0)
    init = rng.standard_normal((1, 2, 4, 3)) + 1j * rng.standard_normal((1, 2, 4, 3))
    y, fs = _run(inp, initial_state=init)
    yc, fc = chunkwise_scan(*_np(inp), 4, initial_state=init)
    assert _close(y, yc) and _close(fs, fc)


def test_tiny_recipe_golden():
    """Regression pin: the tiny recipe's real output, stored by tests/golden/make_golden.py."""
    for tv, name in ((False, "tiny_dt_zero.txt"), (True, "tiny_dt_varying.txt")):
        inp = ssd_inputs.tiny_case(tv)
        y, _ = _run(inp)
        want = np.loadtxt(os.path.join(GOLDEN, name)).reshape(y.shape)
        assert np.abs(y.real - want).max() <= 1e-12


def test_threads_do_not_change_results():
    inp = ssd_inputs.random_case(3, 25, 3, 4, 5, 41)
    y1, f1 = _run(inp, threads=1)
    y4, f4 = _run(inp, threads=4)
    assert np.array_equal(y1, y4) and np.array_equal(f1, f4)


# --------------------------------------------------------------- planted bugs

_PLANTS = {
    "conjugated_B": ("bn * load_c(x, row * D + d)", "conj(bn) * load_c(x, row * D + d)"),
    "conjugated_C": ("acc += load_c(Ct, row * N + n) * s[n * D + d]",
                     "acc += conj(load_c(Ct, row * N + n)) * s[n * D + d]"),
    "no_softplus": ("cplx Abar = cexp(softplus((double)dt[row]) * Ah)",
                    "cplx Abar = cexp(((double)dt[row]) * Ah)"),
    "softplus_dropped_term": ("return fmax(v, 0.0) + log1p(exp(-fabs(v)));",
                              "return log1p(exp(-fabs(v)));"),
    "decay_after_input": ("s[n * D + d] = Abar * s[n * D + d] + bn * load_c(x, row * D + d)",
                          "s[n * D + d] = Abar * (s[n * D + d] + bn * load_c(x, row * D + d))"),
    "conjugated_A": ("cplx Ah = load_c(A, h);\n        for (int64_t t = 0; t < T; ++t)",
                     "cplx Ah = conj(load_c(A, h));\n        for (int64_t t = 0; t < T; ++t)"),
    "reversed_d": ("bn * load_c(x, row * D + d)", "bn * load_c(x, row * D + (D - 1 - d))"),
    "dt_off_by_one": ("softplus((double)dt[row])",
                      "softplus((double)dt[(b * T + (t > 0 ? t - 1 : 0)) * H + h])"),
    "initial_state_ignored": ("s[i] = init_state ?", "s[i] = 0 ?"),
    "output_from_old_state": ("/* y_t = sum_n C_t[n] * s[n, :] */",
                              "/* y_t = sum_n C_t[n] * s[n, :] */ if (0)"),
    "lambda_not_reset": ("run = 0.0;\n                    run += a;", "run += 0.0;\n                    run += a;"),
    "head_swapped_A": ("cplx Ah = load_c(A, h);\n        for", "cplx Ah = load_c(A, (h + 1) % H);\n        for"),
}


def _pin_battery(lib):
    """Run the pins above against an alternative oracle library; return failures."""
    failed = []

    def check(name, fn):
        try:
            fn()
        except (AssertionError, RuntimeError, ValueError):
            failed.append(name)

    def brute():
        for shape, seed in (((2, 9, 2, 4, 3), 0), ((1, 6, 3, 2, 2), 1)):
            inp = ssd_inputs.random_case(*shape, seed, dt_scale=1.5)
            y, fs = _run(inp, lib=lib)
            yb, fb = _brute_force(*_np(inp))
            assert _close(y.real, yb.real) and _close(fs, fb)

    def disc():
        inp = ssd_inputs.random_case(2, 23, 3, 2, 2, 5, dt_scale=8.0)
        abar, lam = oracle.discretise(inp.dt, inp.A, chunk=5, lib=lib)
        _, A, _, _, dt = _np(inp)
        a = np.logaddexp(0.0, dt) * A[None, None, :]
        assert _close(abar, np.exp(a), 1e-14)
        assert _close(lam[:, :, 1, :], np.cumsum(a[:, 5:10], axis=1).transpose(0, 2, 1), 1e-14)

    def scalar():
        y, _ = oracle.scan(*_scalar_inputs(12, -1.0), lib=lib)
        assert np.allclose(y[0, :, 0, 0].real, [2 - 2.0 ** -t for t in range(12)], atol=1e-14)

    def compose():
        inp = ssd_inputs.random_case(2, 30, 2, 4, 3, 14)
        y, fs = _run(inp, lib=lib)
        a = ssd_inputs.ScanInputs(inp.x[:, :17], inp.A, inp.B_t[:, :17], inp.C_t[:, :17], inp.dt[:, :17])
        b = ssd_inputs.ScanInputs(inp.x[:, 17:].contiguous(), inp.A, inp.B_t[:, 17:].contiguous(),
                                  inp.C_t[:, 17:].contiguous(), inp.dt[:, 17:].contiguous())
        ya, fa = _run(a, lib=lib)
        yb, fb = _run(b, lib=lib, initial_state=fa)
        assert _close(np.concatenate([ya, yb], axis=1), y) and _close(fb, fs)

    def heads():
        inp = ssd_inputs.random_case(1, 8, 4, 2, 3, 13)
        y, _ = _run(inp, lib=lib)
        ys = [_run(inp.select(0, h), lib=lib)[0] for h in range(4)]
        assert _close(np.concatenate(ys, axis=2), y)

    for name, fn in (("brute", brute), ("discretise", disc), ("scalar", scalar),
                     ("compose", compose), ("heads", heads)):
        check(name, fn)
    return failed


@pytest.fixture(scope="module")
def plant_dir():
    d = tempfile.mkdtemp(prefix="oracle_plants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def test_battery_passes_on_the_real_oracle():
    assert _pin_battery(oracle.load()) == []


@pytest.mark.parametrize("plant", sorted(_PLANTS))
def test_planted_mistake_is_caught(plant, plant_dir):
    src = open(oracle.SOURCE).read()
    old, new = _PLANTS[plant]
    assert src.count(old) >= 1, "plant anchor not found: %s" % plant
    mutated = src.replace(old, new, 1)
    path = os.path.join(plant_dir, plant + ".c")
    with open(path, "w") as f:
        f.write(mutated)
    so = oracle.build(os.path.join(plant_dir, plant + ".so"), source=path)
    lib = oracle.load(so)
    assert _pin_battery(lib), "planted mistake %s went unnoticed" % plant

"""CPU oracle for the complex SSD scan (TEST INFRASTRUCTURE ONLY).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The product library never loads it, and the two share no
code: the oracle is the plain sequential recurrence written in C
(``ssd_oracle.c``), evaluated in double precision.

Functions
---------
build(out_path=None, extra_cflags=(), source=None) -> path of the shared object
build_timing(out_path) -> path of a float (complex64) build at -O3 -march=native,
    used only to time the plain recurrence as the CPU baseline
scan(x, A, B_t, C_t, dt, initial_state=None, threads=0, lib=None)
    -> (y complex128 (B,T,H,D), final_state complex128 (B,H,N,D))
discretise(dt, A, chunk=0, lib=None)
    -> (A_bar complex128 (B,T,H), Lambda complex128 (B,H,nc,chunk) or None)
scan_backward(x, A, B_t, C_t, dt, grad_y, grad_final_state=None,
              initial_state=None, threads=0, lib=None)
    -> Grads(x, A, B_t, C_t, dt, initial_state): the gradients of
       sum(grad_y * y.real) + sum(Re(conj(grad_final_state) * final_state)),
       complex ones as dl/dRe + i dl/dIm (torch's convention), in float64
head_mix(y, W, lib=None) -> z float64, same shape as y (..., H, D):
    with F = H * D and each token's heads flattened head-major (k = h*D + d),
    z[..., o] = sum_k W[o, k] y[..., k] for a dense (F, F) W (the MIMO mixer)
head_mix_backward(y, W, grad_z, lib=None) -> (grad_y, grad_W) float64
"""

from __future__ import annotations

import collections
import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "ssd_oracle.c")
LIBPATH = os.path.join(_HERE, "liboracle.so")

_lock = threading.Lock()
_lib = None


def build(out_path: str | None = None, extra_cflags=(), source: str | None = None) -> str:
    """Compile the oracle with gcc (plain -O2, IEEE semantics, OpenMP)."""
    out_path = out_path or LIBPATH
    source = source or SOURCE
    tmp = out_path + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           *extra_cflags, source, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


def build_timing(out_path: str) -> str:
    """The same source with the recurrence in float (the pages' complex64),
    -O3 -march=native for the host it runs on: the timed CPU baseline. The
    outputs are still returned as float64 arrays; no parity check uses it."""
    return build(out_path, extra_cflags=("-O3", "-march=native", "-DORACLE_REAL=float"))


def _bind(lib):
    i64 = ctypes.c_int64
    p = ctypes.c_void_p
    lib.oracle_scan.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, p, p, p, ctypes.c_int]
    lib.oracle_scan.restype = ctypes.c_int
    lib.oracle_discretise.argtypes = [p, p, i64, i64, i64, i64, p, p]
    lib.oracle_discretise.restype = ctypes.c_int
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_scan_backward.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, p, p, p,
                                         p, p, p, p, p, p, ctypes.c_int]
    lib.oracle_scan_backward.restype = ctypes.c_int
    lib.oracle_head_mix.argtypes = [p, p, i64, i64, i64, p]
    lib.oracle_head_mix.restype = ctypes.c_int
    lib.oracle_head_mix_backward.argtypes = [p, p, p, i64, i64, i64, p, p]
    lib.oracle_head_mix_backward.restype = ctypes.c_int
    return lib


def load(path: str | None = None):
    """Load (building first if absent) the oracle shared object."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(LIBPATH) or os.path.getmtime(LIBPATH) < os.path.getmtime(SOURCE):
                build()
            _lib = _bind(ctypes.CDLL(LIBPATH))
    return _lib


def _as_f32(a, complex_=False) -> np.ndarray:
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu()
            if complex_:
                a = torch.view_as_real(a.to(torch.complex64).resolve_conj()).contiguous()
            a = a.numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.asarray(a)
    if complex_ and np.iscomplexobj(a):
        a = np.stack([a.real, a.imag], axis=-1)
    return np.ascontiguousarray(a, dtype=np.float32)


def max_threads(lib=None) -> int:
    return (lib or load()).oracle_max_threads()


def scan(x, A, B_t, C_t, dt, initial_state=None, threads: int = 0, lib=None):
    lib = lib or load()
    xf = _as_f32(x, True)
    Af = _as_f32(A, True)
    Bf = _as_f32(B_t, True)
    Cf = _as_f32(C_t, True)
    dtf = _as_f32(dt)
    Bsz, T, H, D = xf.shape[:4]
    N = Bf.shape[3]
    assert Af.shape == (H, 2) and Bf.shape == (Bsz, T, H, N, 2) and Cf.shape == Bf.shape
    assert dtf.shape == (Bsz, T, H)
    y = np.zeros((Bsz, T, H, D, 2), np.float64)
    fs = np.zeros((Bsz, H, N, D, 2), np.float64)
    init_p = None
    if initial_state is not None:
        init = np.asarray(initial_state)
        if np.iscomplexobj(init):
            init = np.stack([init.real, init.imag], -1)
        init = np.ascontiguousarray(init, np.float64)
        assert init.shape == (Bsz, H, N, D, 2)
        init_p = init.ctypes.data
    rc = lib.oracle_scan(xf.ctypes.data, Af.ctypes.data, Bf.ctypes.data, Cf.ctypes.data,
                         dtf.ctypes.data, Bsz, T, H, N, D, init_p, y.ctypes.data, fs.ctypes.data,
                         int(threads))
    if rc != 0:
        raise RuntimeError("oracle_scan failed with %d" % rc)
    return y[..., 0] + 1j * y[..., 1], fs[..., 0] + 1j * fs[..., 1]


def discretise(dt, A, chunk: int = 0, lib=None):
    lib = lib or load()
    dtf = _as_f32(dt)
    Af = _as_f32(A, True)
    Bsz, T, H = dtf.shape
    abar = np.zeros((Bsz, T, H, 2), np.float64)
    lam = None
    lam_p = None
    if chunk > 0:
        nc = (T + chunk - 1) // chunk
        lam = np.zeros((Bsz, H, nc, chunk, 2), np.float64)
        lam_p = lam.ctypes.data
    rc = lib.oracle_discretise(dtf.ctypes.data, Af.ctypes.data, Bsz, T, H, int(chunk),
                               abar.ctypes.data, lam_p)
    if rc != 0:
        raise RuntimeError("oracle_discretise failed with %d" % rc)
    abar_c = abar[..., 0] + 1j * abar[..., 1]
    lam_c = None if lam is None else lam[..., 0] + 1j * lam[..., 1]
    return abar_c, lam_c


Grads = collections.namedtuple("Grads", "x A B_t C_t dt initial_state")


def _as_f64_complex(a, shape):
    a = np.asarray(a.detach().cpu().numpy() if hasattr(a, "detach") else a)
    if np.iscomplexobj(a):
        a = np.stack([a.real, a.imag], -1)
    a = np.ascontiguousarray(a, np.float64)
    assert a.shape == shape + (2,), (a.shape, shape)
    return a


def scan_backward(x, A, B_t, C_t, dt, grad_y, grad_final_state=None, initial_state=None,
                  threads: int = 0, lib=None):
    lib = lib or load()
    xf = _as_f32(x, True)
    Af = _as_f32(A, True)
    Bf = _as_f32(B_t, True)
    Cf = _as_f32(C_t, True)
    dtf = _as_f32(dt)
    gyf = _as_f32(grad_y)
    Bsz, T, H, D = xf.shape[:4]
    N = Bf.shape[3]
    assert gyf.shape == (Bsz, T, H, D)
    gff = None
    if grad_final_state is not None:
        gff = _as_f32(grad_final_state, True)
        assert gff.shape == (Bsz, H, N, D, 2)
    init = None
    if initial_state is not None:
        init = _as_f64_complex(initial_state, (Bsz, H, N, D))
    gx = np.zeros((Bsz, T, H, D, 2))
    gA = np.zeros((H, 2))
    gB = np.zeros((Bsz, T, H, N, 2))
    gC = np.zeros((Bsz, T, H, N, 2))
    gdt = np.zeros((Bsz, T, H))
    gi = np.zeros((Bsz, H, N, D, 2))
    rc = lib.oracle_scan_backward(
        xf.ctypes.data, Af.ctypes.data, Bf.ctypes.data, Cf.ctypes.data, dtf.ctypes.data,
        Bsz, T, H, N, D, None if init is None else init.ctypes.data, gyf.ctypes.data,
        None if gff is None else gff.ctypes.data, gx.ctypes.data, gA.ctypes.data,
        gB.ctypes.data, gC.ctypes.data, gdt.ctypes.data, gi.ctypes.data, int(threads))
    if rc != 0:
        raise RuntimeError("oracle_scan_backward failed with %d" % rc)
    c = lambda v: v[..., 0] + 1j * v[..., 1]
    return Grads(c(gx), c(gA), c(gB), c(gC), gdt, c(gi))


def _mix_operands(y, W):
    yf = _as_f32(y)
    Wf = _as_f32(W)
    if yf.ndim < 2:
        raise ValueError("y must be (..., H, D)")
    H, D = yf.shape[-2:]
    F = H * D
    if Wf.shape != (F, F):
        raise ValueError("W must be (H*D, H*D) = (%d, %d)" % (F, F))
    M = int(np.prod(yf.shape[:-2], dtype=np.int64))
    return yf, Wf, M, H, D


def head_mix(y, W, lib=None):
    """z[..., o] = sum_k W[o, k] y[..., k] over the flattened heads (k = h*D + d),
    in double, from float32 inputs."""
    lib = lib or load()
    yf, Wf, M, H, D = _mix_operands(y, W)
    z = np.zeros(yf.shape, np.float64)
    rc = lib.oracle_head_mix(yf.ctypes.data, Wf.ctypes.data, M, H, D, z.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle_head_mix failed with %d" % rc)
    return z


def head_mix_backward(y, W, grad_z, lib=None):
    """Gradients of sum(grad_z * head_mix(y, W)) for y and W, in double."""
    lib = lib or load()
    yf, Wf, M, H, D = _mix_operands(y, W)
    gzf = _as_f32(grad_z)
    if gzf.shape != yf.shape:
        raise ValueError("grad_z must have the shape of y")
    gy = np.zeros(yf.shape, np.float64)
    gW = np.zeros((H * D, H * D), np.float64)
    rc = lib.oracle_head_mix_backward(yf.ctypes.data, Wf.ctypes.data, gzf.ctypes.data, M, H, D,
                                      gy.ctypes.data, gW.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle_head_mix_backward failed with %d" % rc)
    return gy, gW

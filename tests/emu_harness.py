"""Host emulation of the scan library (TEST INFRASTRUCTURE).

Builds the unchanged C-ABI and kernel sources against tests/emu/ssd_device.h,
which runs each GPU thread as a fiber and evaluates wave64 MFMA tiles,
shuffles and workgroup barriers on the CPU. The resulting shared object
exports the same ssd_* functions; pointers are host pointers.
"""

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
EMU = os.path.join(HERE, "emu")
CSRC = os.path.join(ROOT, "complex_chunkwise_ssd_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
CLANG = "/opt/rocm/llvm/bin/clang++"

_lock = threading.Lock()
_lib = None


def _sources():
    srcs = [os.path.join(EMU, f) for f in os.listdir(EMU)]
    srcs += [os.path.join(CSRC, f) for f in os.listdir(CSRC)]
    srcs += [os.path.join(INCLUDE, "ssd.h")]
    return srcs


def _flags():
    return ["-x", "c++", "-std=c++17", "-I" + EMU, "-I" + CSRC, "-I" + INCLUDE]


def build_lib(out_dir):
    out = os.path.join(out_dir, "libssd_emu.so")
    cmd = [CLANG, *_flags(), "-O1", "-g", "-fPIC", "-shared", os.path.join(EMU, "emu_lib.cpp"),
           "-o", out]
    subprocess.run(cmd, check=True)
    return out


def build_asan_exe(out_dir):
    out = os.path.join(out_dir, "ssd_emu_asan")
    cmd = [CLANG, *_flags(), "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer",
           os.path.join(EMU, "emu_asan_main.cpp"), "-o", out]
    subprocess.run(cmd, check=True)
    return out


def build_tsan_exe(out_dir):
    """The bounds-check driver built under ThreadSanitizer (host code only): the
    emulator turns every GPU thread into a sanitizer fiber whose only ordering is
    the GPU's (barriers, a wave's collectives, launches), so a shared-memory
    access pair that no barrier orders is reported."""
    out = os.path.join(out_dir, "ssd_emu_tsan")
    cmd = [CLANG, *_flags(), "-O1", "-g", "-fsanitize=thread",
           os.path.join(EMU, "emu_asan_main.cpp"), "-o", out]
    subprocess.run(cmd, check=True)
    return out


def load(out_dir):
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build_lib(out_dir))
            p = ctypes.c_void_p
            i64 = ctypes.c_int64
            lib.ssd_chunk_forward.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, i64, p, p, p,
                                              p, ctypes.c_size_t, p]
            lib.ssd_chunk_forward.restype = ctypes.c_int
            lib.ssd_chunk_forward_workspace_bytes.argtypes = [i64] * 6
            lib.ssd_chunk_forward_workspace_bytes.restype = ctypes.c_size_t
            lib.ssd_chunk_forward_noalloc.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64,
                                                      i64, p, p, p, p]
            lib.ssd_chunk_forward_noalloc.restype = ctypes.c_int
            lib.ssd_discretise.argtypes = [p, p, i64, i64, i64, i64, p, p, p]
            lib.ssd_discretise.restype = ctypes.c_int
            lib.ssd_chunk_backward.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, i64, p, p,
                                               p, p, p, p, p, p, p, p, ctypes.c_size_t, p]
            lib.ssd_chunk_backward.restype = ctypes.c_int
            lib.ssd_chunk_backward_proj.argtypes = [p, i64, p, i64, i64, i64, i64, i64, i64, p, p,
                                                    p, p, p, p, p, ctypes.c_size_t, p]
            lib.ssd_chunk_backward_proj.restype = ctypes.c_int
            lib.ssd_chunk_backward_proj_bf16.argtypes = lib.ssd_chunk_backward_proj.argtypes
            lib.ssd_chunk_backward_proj_bf16.restype = ctypes.c_int
            lib.ssd_chunk_backward_workspace_bytes.argtypes = [i64] * 6
            lib.ssd_chunk_backward_workspace_bytes.restype = ctypes.c_size_t
            lib.ssd_chunk_forward_proj.argtypes = [p, i64, p, i64, i64, i64, i64, i64, i64, p, p, p,
                                                   p, ctypes.c_size_t, p]
            lib.ssd_chunk_forward_proj.restype = ctypes.c_int
            lib.ssd_chunk_forward_proj_bf16.argtypes = lib.ssd_chunk_forward_proj.argtypes
            lib.ssd_chunk_forward_proj_bf16.restype = ctypes.c_int
            lib.ssd_head_mix.argtypes = [p, p, i64, i64, i64, p, p]
            lib.ssd_head_mix.restype = ctypes.c_int
            lib.ssd_head_mix_backward_workspace_bytes.argtypes = [i64] * 3
            lib.ssd_head_mix_backward_workspace_bytes.restype = ctypes.c_size_t
            lib.ssd_head_mix_backward.argtypes = [p, p, p, i64, i64, i64, p, p, p, ctypes.c_size_t,
                                                  p]
            lib.ssd_head_mix_backward.restype = ctypes.c_int
            lib.emu_mfma_count.restype = ctypes.c_long
            lib.emu_set_shuffle_seed.argtypes = [ctypes.c_ulonglong]
            lib.emu_set_shuffle_seed.restype = None
            lib.emu_sincos.argtypes = [p, p, p, ctypes.c_long]
            lib.emu_sincos.restype = None
            _lib = lib
    return _lib


def _c64(t):
    a = np.asarray(t.detach().cpu().numpy() if hasattr(t, "detach") else t)
    return np.ascontiguousarray(a.astype(np.complex64))


def chunk_forward(lib, inp, chunk, initial_state=None, want_final=True):
    x, A, Bm, Cm = (_c64(v) for v in (inp.x, inp.A, inp.B_t, inp.C_t))
    dt = np.ascontiguousarray(inp.dt.numpy().astype(np.float32))
    Bsz, T, H, D = x.shape
    N = Bm.shape[-1]
    y = np.full((Bsz, T, H, D), np.nan, np.float32)
    fs = np.full((Bsz, H, N, D), np.nan + 0j, np.complex64) if want_final else None
    init = None if initial_state is None else np.ascontiguousarray(initial_state, np.complex64)
    ws_n = lib.ssd_chunk_forward_workspace_bytes(Bsz, T, H, N, D, chunk)
    ws = np.full(ws_n // 4 + 64, np.nan, np.float32)
    ws_p = ws.ctypes.data
    ws_p = ws_p + (-ws_p) % 256
    st = lib.ssd_chunk_forward(x.ctypes.data, A.ctypes.data, Bm.ctypes.data, Cm.ctypes.data,
                               dt.ctypes.data, Bsz, T, H, N, D, chunk,
                               None if init is None else init.ctypes.data, y.ctypes.data,
                               None if fs is None else fs.ctypes.data,
                               ws_p if ws_n else None, ws_n, None)
    return st, y, fs


def chunk_backward(lib, inp, chunk, grad_y, grad_final=None, initial_state=None, want_init=True):
    """Returns (status, gx, gA, gB, gC, gdt, ginit) from the emulated library."""
    x, A, Bm, Cm = (_c64(v) for v in (inp.x, inp.A, inp.B_t, inp.C_t))
    dt = np.ascontiguousarray(inp.dt.numpy().astype(np.float32))
    Bsz, T, H, D = x.shape
    N = Bm.shape[-1]
    gy = np.ascontiguousarray(grad_y, np.float32)
    gf = None if grad_final is None else np.ascontiguousarray(grad_final, np.complex64)
    init = None if initial_state is None else np.ascontiguousarray(initial_state, np.complex64)
    nan = np.nan + 1j * np.nan
    gx = np.full(x.shape, nan, np.complex64)
    gA = np.full((H,), nan, np.complex64)
    gB = np.full(Bm.shape, nan, np.complex64)
    gC = np.full(Bm.shape, nan, np.complex64)
    gdt = np.full(dt.shape, np.nan, np.float32)
    gi = np.full((Bsz, H, N, D), nan, np.complex64) if want_init else None
    ws_n = lib.ssd_chunk_backward_workspace_bytes(Bsz, T, H, N, D, chunk)
    ws = np.full(ws_n // 4 + 64, np.nan, np.float32)
    ws_p = ws.ctypes.data
    ws_p = ws_p + (-ws_p) % 256
    ptr = lambda a: None if a is None else a.ctypes.data
    st = lib.ssd_chunk_backward(ptr(x), ptr(A), ptr(Bm), ptr(Cm), ptr(dt), Bsz, T, H, N, D, chunk,
                                ptr(init), ptr(gy), ptr(gf), ptr(gx), ptr(gA), ptr(gB), ptr(gC),
                                ptr(gdt), ptr(gi), ws_p if ws_n else None, ws_n, None)
    return st, gx, gA, gB, gC, gdt, gi


def chunk_forward_proj(lib, proj, A, H, N, D, chunk, initial_state=None):
    """proj (B, T, S) float32 or bfloat16 (torch) in the in_proj layout; returns
    (status, y, final_state)."""
    import torch
    bf16 = hasattr(proj, "dtype") and proj.dtype == torch.bfloat16
    if bf16:
        pr = np.ascontiguousarray(proj.contiguous().view(torch.int16).numpy())
    else:
        pr = np.ascontiguousarray(proj.numpy() if hasattr(proj, "numpy") else proj, np.float32)
    Av = _c64(A)
    Bsz, T, S = pr.shape
    y = np.full((Bsz, T, H, D), np.nan, np.float32)
    fs = np.full((Bsz, H, N, D), np.nan + 0j, np.complex64)
    init = None if initial_state is None else np.ascontiguousarray(initial_state, np.complex64)
    ws_n = lib.ssd_chunk_forward_workspace_bytes(Bsz, T, H, N, D, chunk)
    ws = np.full(ws_n // 4 + 64, np.nan, np.float32)
    ws_p = ws.ctypes.data
    ws_p = ws_p + (-ws_p) % 256
    fn = lib.ssd_chunk_forward_proj_bf16 if bf16 else lib.ssd_chunk_forward_proj
    st = fn(pr.ctypes.data, S, Av.ctypes.data, Bsz, T, H, N, D, chunk,
                                    None if init is None else init.ctypes.data, y.ctypes.data,
                                    fs.ctypes.data, ws_p if ws_n else None, ws_n, None)
    return st, y, fs


def chunk_backward_proj(lib, proj, A, H, N, D, chunk, grad_y, grad_final=None):
    """Returns (status, grad_proj rows (B, T, S) with NaN past the blocks,
    grad_A, grad_initial_state). proj float32 numpy/torch, or a bfloat16 torch
    tensor; bfloat16 gradient rows come back widened to float32."""
    import torch
    bf16 = hasattr(proj, "dtype") and proj.dtype == torch.bfloat16
    if bf16:
        pr = np.ascontiguousarray(proj.contiguous().view(torch.int16).numpy())
    else:
        pr = np.ascontiguousarray(proj.numpy() if hasattr(proj, "numpy") else proj, np.float32)
    Av = _c64(A)
    Bsz, T, S = pr.shape
    gy = np.ascontiguousarray(grad_y, np.float32)
    gf = None if grad_final is None else np.ascontiguousarray(grad_final, np.complex64)
    # NaN (as bfloat16 bits 0x7fc0 or float32) past the blocks
    grows = np.full((Bsz, T, S), 0x7fc0, np.uint16) if bf16 else np.full((Bsz, T, S), np.nan,
                                                                          np.float32)
    W = H * (D + 4 * N + 1)
    gA = np.full((H,), np.nan + 0j, np.complex64)
    gi = np.full((Bsz, H, N, D), np.nan + 0j, np.complex64)
    ws_n = lib.ssd_chunk_backward_workspace_bytes(Bsz, T, H, N, D, chunk)
    ws = np.full(ws_n // 4 + 64, np.nan, np.float32)
    ws_p = ws.ctypes.data
    ws_p = ws_p + (-ws_p) % 256
    ptr = lambda a: None if a is None else a.ctypes.data
    fn = lib.ssd_chunk_backward_proj_bf16 if bf16 else lib.ssd_chunk_backward_proj
    st = fn(ptr(pr), S, ptr(Av), Bsz, T, H, N, D, chunk, None, ptr(gy), ptr(gf), ptr(grows),
            ptr(gA), ptr(gi), ws_p if ws_n else None, ws_n, None)
    if bf16:
        grows = (grows.astype(np.uint32) << 16).view(np.float32)
    return st, grows, gA, gi, W


def head_mix(lib, y, W, offset=0):
    """y (..., H, D) float32 numpy, W (H*D, H*D); returns (status, z). `offset`
    floats shift y and z off 16-byte alignment (the scalar path)."""
    y = np.asarray(y, np.float32)
    H, D = y.shape[-2:]
    M = int(np.prod(y.shape[:-2], dtype=np.int64))
    yb = np.zeros(y.size + 8, np.float32)
    zb = np.full(y.size + 8, np.nan, np.float32)
    yb[offset:offset + y.size] = y.ravel()
    Wv = np.ascontiguousarray(W, np.float32)
    st = lib.ssd_head_mix(yb.ctypes.data + 4 * offset, Wv.ctypes.data, M, H, D,
                          zb.ctypes.data + 4 * offset, None)
    return st, zb[offset:offset + y.size].reshape(y.shape)


def head_mix_backward(lib, y, W, gz):
    """Returns (status, grad_y, grad_W) from the emulated library."""
    y = np.ascontiguousarray(y, np.float32)
    gz = np.ascontiguousarray(gz, np.float32)
    H, D = y.shape[-2:]
    M = int(np.prod(y.shape[:-2], dtype=np.int64))
    Wv = np.ascontiguousarray(W, np.float32)
    gy = np.full(y.shape, np.nan, np.float32)
    gW = np.full((H * D, H * D), np.nan, np.float32)
    ws_n = lib.ssd_head_mix_backward_workspace_bytes(M, H, D)
    ws = np.full(ws_n // 4 + 64, np.nan, np.float32)
    ws_p = ws.ctypes.data
    ws_p = ws_p + (-ws_p) % 256
    st = lib.ssd_head_mix_backward(y.ctypes.data, Wv.ctypes.data, gz.ctypes.data, M, H, D,
                                   gy.ctypes.data, gW.ctypes.data, ws_p if ws_n else None, ws_n,
                                   None)
    return st, gy, gW

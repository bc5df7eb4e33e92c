"""Python binding of the MI355X complex chunkwise SSD scan library.

Argument marshalling only: every step of the scan runs in the HIP kernels of
``libssd.so`` (C ABI in include/ssd.h). PyTorch supplies device memory and the
current stream. Importing works without a GPU; calling needs the built library
and a visible GPU, and fails loudly otherwise (there is no fallback path).

    y, final_state = chunk_forward(x, A, B_t, C_t, dt, chunk_size=64)
    y, final_state = chunk_forward_noalloc(x, A, B_t, C_t, dt)   # no device allocation
    y, final_state = chunk_forward_proj(proj, A, H, N, D, chunk_size=64)
    grads = chunk_backward(x, A, B_t, C_t, dt, grad_y, grad_final_state=None)
    A_bar, log_decay_cumsum = discretise(dt, A, chunk_size=64)
    z = head_mix(y, W)                       # MIMO head mixer after the scan (W: (H*D, H*D))
    grad_y, grad_W = head_mix_backward(y, W, grad_z)
"""

from __future__ import annotations

import collections
import ctypes
import os
import re
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBPATH = os.path.join(_PKG, "libssd.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "ssd.h")

SSD_OK = 0
SSD_ERR_NULL = -1
SSD_ERR_SHAPE = -2
SSD_ERR_ODD_N = -3
SSD_ERR_BLOCK_DIMS = -4
SSD_ERR_WORKSPACE = -5
SSD_ERR_ALIGN = -6
SSD_ERR_HIP = -7
SSD_ERR_UNSUPPORTED = -8
SSD_ERR_ALIAS = -9
SSD_NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024  # include/ssd.h

_lock = threading.Lock()
_lib = None


class SSDError(ValueError):
    """A call was rejected by the library (status < 0)."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_string(status), status))


def load_library(path: str | None = None):
    """Load libssd.so (raises OSError if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIBPATH
        if not os.path.exists(p):
            raise OSError("libssd.so not found at %s; build it with "
                          "`python -m complex_chunkwise_ssd_amd.build`" % p)
        lib = ctypes.CDLL(p)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        lib.ssd_discretise.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp, vp]
        lib.ssd_discretise.restype = ctypes.c_int
        lib.ssd_chunk_forward_workspace_bytes.argtypes = [i64] * 6
        lib.ssd_chunk_forward_workspace_bytes.restype = ctypes.c_size_t
        lib.ssd_chunk_forward.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, vp, vp,
                                          vp, vp, ctypes.c_size_t, vp]
        lib.ssd_chunk_forward.restype = ctypes.c_int
        lib.ssd_chunk_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                                  vp, vp, vp, vp]
        lib.ssd_chunk_forward_noalloc.restype = ctypes.c_int
        lib.ssd_chunk_forward_proj.argtypes = [vp, i64, vp, i64, i64, i64, i64, i64, i64, vp, vp,
                                               vp, vp, ctypes.c_size_t, vp]
        lib.ssd_chunk_forward_proj.restype = ctypes.c_int
        lib.ssd_chunk_forward_proj_bf16.argtypes = lib.ssd_chunk_forward_proj.argtypes
        lib.ssd_chunk_forward_proj_bf16.restype = ctypes.c_int
        lib.ssd_chunk_backward_workspace_bytes.argtypes = [i64] * 6
        lib.ssd_chunk_backward_workspace_bytes.restype = ctypes.c_size_t
        lib.ssd_chunk_backward.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, vp, vp,
                                           vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.ssd_chunk_backward.restype = ctypes.c_int
        lib.ssd_chunk_backward_proj.argtypes = [vp, i64, vp, i64, i64, i64, i64, i64, i64, vp, vp,
                                                vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.ssd_chunk_backward_proj.restype = ctypes.c_int
        lib.ssd_chunk_backward_proj_bf16.argtypes = lib.ssd_chunk_backward_proj.argtypes
        lib.ssd_chunk_backward_proj_bf16.restype = ctypes.c_int
        lib.ssd_head_mix.argtypes = [vp, vp, i64, i64, i64, vp, vp]
        lib.ssd_head_mix.restype = ctypes.c_int
        lib.ssd_head_mix_backward_workspace_bytes.argtypes = [i64] * 3
        lib.ssd_head_mix_backward_workspace_bytes.restype = ctypes.c_size_t
        lib.ssd_head_mix_backward.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, vp,
                                              ctypes.c_size_t, vp]
        lib.ssd_head_mix_backward.restype = ctypes.c_int
        lib.ssd_status_string.argtypes = [ctypes.c_int]
        lib.ssd_status_string.restype = ctypes.c_char_p
        lib.ssd_version.restype = ctypes.c_int
        if path is None:
            _lib = lib
        return lib


def header_functions(header: str = HEADER):
    """Names of the functions declared in include/ssd.h."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(ssd_\w+)\s*\(", text, flags=re.M)


def status_string(status: int) -> str:
    return load_library().ssd_status_string(int(status)).decode()


def workspace_bytes(batch, T, H, N, D, chunk_size) -> int:
    return int(load_library().ssd_chunk_forward_workspace_bytes(batch, T, H, N, D, chunk_size))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.device != device:
        raise ValueError("%s must be on %s, got %s" % (name, device, t.device))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous() or t.is_conj():
        raise ValueError("%s must be contiguous and not a lazy conjugate view" % name)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def chunk_forward(x, A, B_t, C_t, dt, chunk_size: int = 64, initial_state=None,
                  want_final_state: bool = True, y=None, final_state=None, workspace=None):
    """Chunkwise complex SSD scan forward on the current stream.

    x (B,T,H,D) complex64; A (H,) complex64; B_t, C_t (B,T,H,N) complex64;
    dt (B,T,H) float32; optional initial_state (B,H,N,D) complex64.
    Returns (y (B,T,H,D) float32 = real part, final_state (B,H,N,D) complex64 or None).
    Outputs and the workspace may be passed in preallocated.
    """
    lib = load_library()
    if not isinstance(x, torch.Tensor) or x.dim() != 4:
        raise ValueError("x must be a (B, T, H, D) tensor")
    Bsz, T, H, D = x.shape
    if not isinstance(B_t, torch.Tensor) or B_t.dim() != 4:
        raise ValueError("B_t must be a (B, T, H, N) tensor")
    N = B_t.shape[-1]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device, got %s" % dev)
    _check(x, "x", torch.complex64, (Bsz, T, H, D), dev)
    _check(A, "A", torch.complex64, (H,), dev)
    _check(B_t, "B_t", torch.complex64, (Bsz, T, H, N), dev)
    _check(C_t, "C_t", torch.complex64, (Bsz, T, H, N), dev)
    _check(dt, "dt", torch.float32, (Bsz, T, H), dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", torch.complex64, (Bsz, H, N, D), dev)
    if y is None:
        y = torch.empty((Bsz, T, H, D), dtype=torch.float32, device=dev)
    _check(y, "y", torch.float32, (Bsz, T, H, D), dev)
    if want_final_state and final_state is None:
        final_state = torch.empty((Bsz, H, N, D), dtype=torch.complex64, device=dev)
    if final_state is not None:
        _check(final_state, "final_state", torch.complex64, (Bsz, H, N, D), dev)
    ws_n = int(lib.ssd_chunk_forward_workspace_bytes(Bsz, T, H, N, D, chunk_size))
    if ws_n and workspace is None:
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    ws_size = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.ssd_chunk_forward(_ptr(x), _ptr(A), _ptr(B_t), _ptr(C_t), _ptr(dt), Bsz, T, H, N, D,
                               int(chunk_size), _ptr(initial_state), _ptr(y), _ptr(final_state),
                               _ptr(workspace), ws_size, _stream(dev))
    if st != SSD_OK:
        raise SSDError(st, "ssd_chunk_forward")
    return y, final_state


def chunk_forward_noalloc(x, A, B_t, C_t, dt, chunk_size: int = 64, initial_state=None,
                          want_final_state: bool = True, y=None, final_state=None):
    """chunk_forward through ssd_chunk_forward_noalloc: the library takes its
    workspace from a static per-GPU device array (SSD_NOALLOC_SCRATCH_BYTES)
    and allocates nothing. Pass y and final_state to allocate nothing here
    either. Calls that overlap on one GPU race on that array."""
    lib = load_library()
    if not isinstance(x, torch.Tensor) or x.dim() != 4 or not isinstance(B_t, torch.Tensor) \
            or B_t.dim() != 4:
        raise ValueError("x must be (B, T, H, D) and B_t (B, T, H, N) tensors")
    Bsz, T, H, D = x.shape
    N = B_t.shape[-1]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device, got %s" % dev)
    _check(x, "x", torch.complex64, (Bsz, T, H, D), dev)
    _check(A, "A", torch.complex64, (H,), dev)
    _check(B_t, "B_t", torch.complex64, (Bsz, T, H, N), dev)
    _check(C_t, "C_t", torch.complex64, (Bsz, T, H, N), dev)
    _check(dt, "dt", torch.float32, (Bsz, T, H), dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", torch.complex64, (Bsz, H, N, D), dev)
    if y is None:
        y = torch.empty((Bsz, T, H, D), dtype=torch.float32, device=dev)
    _check(y, "y", torch.float32, (Bsz, T, H, D), dev)
    if want_final_state and final_state is None:
        final_state = torch.empty((Bsz, H, N, D), dtype=torch.complex64, device=dev)
    if final_state is not None:
        _check(final_state, "final_state", torch.complex64, (Bsz, H, N, D), dev)
    st = lib.ssd_chunk_forward_noalloc(_ptr(x), _ptr(A), _ptr(B_t), _ptr(C_t), _ptr(dt), Bsz, T,
                                       H, N, D, int(chunk_size), _ptr(initial_state), _ptr(y),
                                       _ptr(final_state), _stream(dev))
    if st != SSD_OK:
        raise SSDError(st, "ssd_chunk_forward_noalloc")
    return y, final_state


def proj_width(H: int, N: int, D: int) -> int:
    """Floats of one token's in_proj row that the scan reads: x, the four N-blocks, dt."""
    return H * (D + 4 * N + 1)


def chunk_forward_proj(proj, A, H: int, N: int, D: int, chunk_size: int = 64,
                       initial_state=None, want_final_state: bool = True, y=None,
                       final_state=None, workspace=None):
    """The scan read from in_proj output rows: proj (B, T, S) float32 or bfloat16,
    contiguous, each token row [x (H*D) | Re B | Im B | Re C | Im C (H*N each) |
    dt (H) | ...] with S >= H*(D + 4N + 1); bfloat16 rows are widened to float32
    as they are loaded. Returns (y (B,T,H,D) float32, final_state or None)."""
    lib = load_library()
    if not isinstance(proj, torch.Tensor) or proj.dim() != 3:
        raise ValueError("proj must be a (B, T, S) tensor")
    Bsz, T, S = proj.shape
    dev = proj.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device, got %s" % dev)
    bf16 = proj.dtype == torch.bfloat16
    _check(proj, "proj", torch.bfloat16 if bf16 else torch.float32, (Bsz, T, S), dev)
    _check(A, "A", torch.complex64, (H,), dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", torch.complex64, (Bsz, H, N, D), dev)
    if y is None:
        y = torch.empty((Bsz, T, H, D), dtype=torch.float32, device=dev)
    _check(y, "y", torch.float32, (Bsz, T, H, D), dev)
    if want_final_state and final_state is None:
        final_state = torch.empty((Bsz, H, N, D), dtype=torch.complex64, device=dev)
    if final_state is not None:
        _check(final_state, "final_state", torch.complex64, (Bsz, H, N, D), dev)
    ws_n = int(lib.ssd_chunk_forward_workspace_bytes(Bsz, T, H, N, D, chunk_size))
    if ws_n and workspace is None:
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    ws_size = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fn = lib.ssd_chunk_forward_proj_bf16 if bf16 else lib.ssd_chunk_forward_proj
    st = fn(_ptr(proj), S, _ptr(A), Bsz, T, H, N, D, int(chunk_size), _ptr(initial_state), _ptr(y),
            _ptr(final_state), _ptr(workspace), ws_size, _stream(dev))
    if st != SSD_OK:
        raise SSDError(st, "ssd_chunk_forward_proj" + ("_bf16" if bf16 else ""))
    return y, final_state


Grads = collections.namedtuple("Grads", "x A B_t C_t dt initial_state")


def backward_workspace_bytes(batch, T, H, N, D, chunk_size) -> int:
    return int(load_library().ssd_chunk_backward_workspace_bytes(batch, T, H, N, D, chunk_size))


def chunk_backward(x, A, B_t, C_t, dt, grad_y, grad_final_state=None, chunk_size: int = 64,
                   initial_state=None, want_initial_state_grad: bool = True, out=None,
                   workspace=None):
    """Gradients of sum(grad_y * y) + sum(Re(conj(grad_final_state) * final_state))
    for the forward call with the same inputs, on the current stream.

    grad_y (B,T,H,D) float32; grad_final_state (B,H,N,D) complex64 or None.
    Returns Grads(x, A, B_t, C_t, dt, initial_state): complex64 gradients as
    dl/dRe + i dl/dIm (torch's convention), dt's float32; initial_state's is
    None unless requested. `out` may supply preallocated Grads.
    """
    lib = load_library()
    if not isinstance(x, torch.Tensor) or x.dim() != 4:
        raise ValueError("x must be a (B, T, H, D) tensor")
    Bsz, T, H, D = x.shape
    if not isinstance(B_t, torch.Tensor) or B_t.dim() != 4:
        raise ValueError("B_t must be a (B, T, H, N) tensor")
    N = B_t.shape[-1]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device, got %s" % dev)
    _check(x, "x", torch.complex64, (Bsz, T, H, D), dev)
    _check(A, "A", torch.complex64, (H,), dev)
    _check(B_t, "B_t", torch.complex64, (Bsz, T, H, N), dev)
    _check(C_t, "C_t", torch.complex64, (Bsz, T, H, N), dev)
    _check(dt, "dt", torch.float32, (Bsz, T, H), dev)
    _check(grad_y, "grad_y", torch.float32, (Bsz, T, H, D), dev)
    if grad_final_state is not None:
        _check(grad_final_state, "grad_final_state", torch.complex64, (Bsz, H, N, D), dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", torch.complex64, (Bsz, H, N, D), dev)
    if out is None:
        c64 = dict(dtype=torch.complex64, device=dev)
        out = Grads(torch.empty((Bsz, T, H, D), **c64), torch.empty((H,), **c64),
                    torch.empty((Bsz, T, H, N), **c64), torch.empty((Bsz, T, H, N), **c64),
                    torch.empty((Bsz, T, H), dtype=torch.float32, device=dev),
                    torch.empty((Bsz, H, N, D), **c64) if want_initial_state_grad else None)
    _check(out.x, "grad x", torch.complex64, (Bsz, T, H, D), dev)
    _check(out.A, "grad A", torch.complex64, (H,), dev)
    _check(out.B_t, "grad B_t", torch.complex64, (Bsz, T, H, N), dev)
    _check(out.C_t, "grad C_t", torch.complex64, (Bsz, T, H, N), dev)
    _check(out.dt, "grad dt", torch.float32, (Bsz, T, H), dev)
    if out.initial_state is not None:
        _check(out.initial_state, "grad initial_state", torch.complex64, (Bsz, H, N, D), dev)
    ws_n = int(lib.ssd_chunk_backward_workspace_bytes(Bsz, T, H, N, D, chunk_size))
    if ws_n and workspace is None:
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    ws_size = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.ssd_chunk_backward(_ptr(x), _ptr(A), _ptr(B_t), _ptr(C_t), _ptr(dt), Bsz, T, H, N, D,
                                int(chunk_size), _ptr(initial_state), _ptr(grad_y),
                                _ptr(grad_final_state), _ptr(out.x), _ptr(out.A), _ptr(out.B_t),
                                _ptr(out.C_t), _ptr(out.dt), _ptr(out.initial_state),
                                _ptr(workspace), ws_size, _stream(dev))
    if st != SSD_OK:
        raise SSDError(st, "ssd_chunk_backward")
    return out


def chunk_backward_proj(proj, A, H: int, N: int, D: int, grad_y, grad_final_state=None,
                        chunk_size: int = 64, initial_state=None, grad_proj=None,
                        want_initial_state_grad: bool = True, workspace=None):
    """Gradients of the scan read from in_proj rows (chunk_forward_proj), as
    gradient rows of the same layout and dtype (float32, or bfloat16 rounded
    from float32 results): returns (grad_proj (B, T, S), grad_A (H,) complex64,
    grad_initial_state or None). The x block gets dl/dx (x is real), the B and
    C blocks the real and imaginary parts of their gradients, the dt block
    dl/ddt; elements past the blocks are left as they are (zero in a freshly
    allocated grad_proj)."""
    lib = load_library()
    if not isinstance(proj, torch.Tensor) or proj.dim() != 3:
        raise ValueError("proj must be a (B, T, S) tensor")
    Bsz, T, S = proj.shape
    dev = proj.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device, got %s" % dev)
    bf16 = proj.dtype == torch.bfloat16
    rdt = torch.bfloat16 if bf16 else torch.float32
    _check(proj, "proj", rdt, (Bsz, T, S), dev)
    _check(A, "A", torch.complex64, (H,), dev)
    _check(grad_y, "grad_y", torch.float32, (Bsz, T, H, D), dev)
    if grad_final_state is not None:
        _check(grad_final_state, "grad_final_state", torch.complex64, (Bsz, H, N, D), dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", torch.complex64, (Bsz, H, N, D), dev)
    if grad_proj is None:
        grad_proj = torch.zeros((Bsz, T, S), dtype=rdt, device=dev)
    _check(grad_proj, "grad_proj", rdt, (Bsz, T, S), dev)
    gA = torch.empty((H,), dtype=torch.complex64, device=dev)
    gi = None
    if want_initial_state_grad:
        gi = torch.empty((Bsz, H, N, D), dtype=torch.complex64, device=dev)
    ws_n = int(lib.ssd_chunk_backward_workspace_bytes(Bsz, T, H, N, D, chunk_size))
    if ws_n and workspace is None:
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    ws_size = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fn = lib.ssd_chunk_backward_proj_bf16 if bf16 else lib.ssd_chunk_backward_proj
    st = fn(_ptr(proj), S, _ptr(A), Bsz, T, H, N, D, int(chunk_size), _ptr(initial_state),
            _ptr(grad_y), _ptr(grad_final_state), _ptr(grad_proj), _ptr(gA), _ptr(gi),
            _ptr(workspace), ws_size, _stream(dev))
    if st != SSD_OK:
        raise SSDError(st, "ssd_chunk_backward_proj" + ("_bf16" if bf16 else ""))
    return grad_proj, gA, gi


def discretise(dt, A, chunk_size: int = 0, want_abar: bool = True):
    """A_bar = exp(softplus(dt) A) (B,T,H) and, if chunk_size > 0, the per-chunk
    running sums of softplus(dt) A (B,H,nc,chunk_size), both complex64."""
    lib = load_library()
    if not isinstance(dt, torch.Tensor) or dt.dim() != 3:
        raise ValueError("dt must be a (B, T, H) tensor")
    Bsz, T, H = dt.shape
    dev = dt.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device, got %s" % dev)
    _check(dt, "dt", torch.float32, (Bsz, T, H), dev)
    _check(A, "A", torch.complex64, (H,), dev)
    abar = torch.empty((Bsz, T, H), dtype=torch.complex64, device=dev) if want_abar else None
    lam = None
    if chunk_size > 0:
        nc = (T + chunk_size - 1) // chunk_size
        lam = torch.empty((Bsz, H, nc, chunk_size), dtype=torch.complex64, device=dev)
    st = lib.ssd_discretise(_ptr(dt), _ptr(A), Bsz, T, H, int(chunk_size), _ptr(abar), _ptr(lam),
                            _stream(dev))
    if st != SSD_OK:
        raise SSDError(st, "ssd_discretise")
    return abar, lam


def algorithmic_flops_per_token_head(N: int, D: int, Q: int) -> float:
    """Real flops the chunkwise method must do per (token, head): the causal
    C B^T (8N per pair), Re((C B^T o L) X) (4D per pair), the chunk state
    B^T X (8ND), the state-to-output term Re(C H) (4ND) and the state passing
    (8ND/Q). Transcendentals are not counted."""
    return 8 * N * (Q + 1) / 2 + 4 * D * (Q + 1) / 2 + 12 * N * D + 8 * N * D / Q


def proj_algorithmic_flops_per_token_head(N: int, D: int, Q: int) -> float:
    """As algorithmic_flops_per_token_head with real x: Re((C B^T o L) X) costs
    2D per pair and the chunk state B^T X 4ND."""
    return 8 * N * (Q + 1) / 2 + 2 * D * (Q + 1) / 2 + 8 * N * D + 8 * N * D / Q


def proj_algorithmic_bytes_per_token_head(N: int, D: int, T: int, elem: int = 4) -> float:
    """x (real), the four N-blocks and dt read (elem bytes each: 4 for float32
    rows, 2 for bfloat16), y written (float32), final state amortised."""
    return elem * (D + 4 * N + 1) + 4 * D + 8 * N * D / T


def algorithmic_bytes_per_token_head(N: int, D: int, T: int) -> float:
    """Bytes the scan must move per (token, head): x, B_t, C_t (complex64),
    dt, y (float32) and the final state amortised over T."""
    return 8 * D + 16 * N + 4 + 4 * D + 8 * N * D / T


def block_rows(chunk_size: int) -> int:
    """Tokens the forward evaluates per chunk: chunk_size up to 64; a longer chunk
    runs as 64-token sub-chunks with the state passed between them."""
    return min(int(chunk_size), 64)


def backward_block_rows(chunk_size: int) -> int:
    """Tokens the backward evaluates per chunk (the state spacing it stores)."""
    return min(int(chunk_size), 32)


def backward_algorithmic_flops_per_token_head(N: int, D: int, Q: int) -> float:
    """Real flops the chunkwise gradients need per (token, head) at chunk Q:
    the forward chunk states B^T X (8ND) and the adjoint's C'^T gy (4ND), each
    passed between chunks (8ND/Q each); the causal Gram C B^T and its two uses
    V^T C and V B (8N per pair each); gy x^T and M^T gy (4D per pair each);
    and the edge terms B G (8ND), x G^T (8ND) and gy H^T (4ND)."""
    pairs = (Q + 1) / 2
    return 32 * N * D + 16 * N * D / Q + 24 * N * pairs + 8 * D * pairs


def proj_backward_algorithmic_flops_per_token_head(N: int, D: int, Q: int) -> float:
    """As backward_algorithmic_flops_per_token_head with real x (in_proj rows):
    the chunk states B^T x take 4ND, gy x^T and the real part of M^T gy 2D per
    pair each, and of the edge terms only Re(B G) (4ND), x G^T (4ND) and gy H^T
    (4ND) remain."""
    pairs = (Q + 1) / 2
    return 20 * N * D + 16 * N * D / Q + 24 * N * pairs + 4 * D * pairs


def backward_algorithmic_bytes_per_token_head(N: int, D: int, T: int) -> float:
    """Bytes the gradients must move per (token, head): x, B_t, C_t, dt, grad_y
    in; grad_x, grad_B_t, grad_C_t, grad_dt out; the state gradients amortised."""
    return (8 * D + 16 * N + 4 + 4 * D) + (8 * D + 16 * N + 4) + 16 * N * D / T


def _mix_shape(y, W):
    if not isinstance(y, torch.Tensor) or y.dim() < 2:
        raise ValueError("y must be a (..., H, D) tensor")
    H, D = y.shape[-2], y.shape[-1]
    F = H * D
    dev = y.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device, got %s" % dev)
    _check(y, "y", torch.float32, tuple(y.shape), dev)
    _check(W, "W", torch.float32, (F, F), dev)
    tokens = 1
    for n in y.shape[:-2]:
        tokens *= int(n)
    return tokens, H, D, dev


def head_mix(y, W, z=None):
    """MIMO head mixer after the scan: with each token's heads flattened
    head-major (k = h * D + d, F = H * D), z[..., o] = sum_k W[o, k] y[..., k].
    y (..., H, D) float32 (e.g. the scan's (B, T, H, D) output), W (F, F)
    float32 (row o = weights of output o); z, if passed, must not overlap y."""
    lib = load_library()
    tokens, H, D, dev = _mix_shape(y, W)
    if z is None:
        z = torch.empty_like(y)
    _check(z, "z", torch.float32, tuple(y.shape), dev)
    st = lib.ssd_head_mix(_ptr(y), _ptr(W), tokens, H, D, _ptr(z), _stream(dev))
    if st != SSD_OK:
        raise SSDError(st, "ssd_head_mix")
    return z


def head_mix_workspace_bytes(tokens: int, H: int, D: int) -> int:
    return int(load_library().ssd_head_mix_backward_workspace_bytes(tokens, H, D))


def head_mix_backward(y, W, grad_z, grad_y=None, grad_W=None, workspace=None):
    """Gradients of sum(grad_z * head_mix(y, W)): returns (grad_y, grad_W),
    grad_y = grad_z W per token and grad_W = sum over tokens of
    grad_z (outer) y."""
    lib = load_library()
    tokens, H, D, dev = _mix_shape(y, W)
    F = H * D
    _check(grad_z, "grad_z", torch.float32, tuple(y.shape), dev)
    if grad_y is None:
        grad_y = torch.empty_like(y)
    _check(grad_y, "grad_y", torch.float32, tuple(y.shape), dev)
    if grad_W is None:
        grad_W = torch.empty((F, F), dtype=torch.float32, device=dev)
    _check(grad_W, "grad_W", torch.float32, (F, F), dev)
    ws_n = int(lib.ssd_head_mix_backward_workspace_bytes(tokens, H, D))
    if ws_n and workspace is None:
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    ws_size = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.ssd_head_mix_backward(_ptr(y), _ptr(W), _ptr(grad_z), tokens, H, D, _ptr(grad_y),
                                   _ptr(grad_W), _ptr(workspace), ws_size, _stream(dev))
    if st != SSD_OK:
        raise SSDError(st, "ssd_head_mix_backward")
    return grad_y, grad_W


def mix_algorithmic_flops(tokens: int, H: int, D: int) -> float:
    """Real flops of one mixer product (forward, grad_y or grad_W): 2 M F^2."""
    F = H * D
    return 2.0 * tokens * F * F


def mix_algorithmic_bytes(tokens: int, H: int, D: int, backward: bool = False) -> float:
    """Bytes the mixer must move: forward y in, z out, W in (8 M F + 4 F^2);
    backward y, grad_z in, grad_y out, W in, grad_W out (12 M F + 8 F^2)."""
    F = H * D
    if backward:
        return 12.0 * tokens * F + 8.0 * F * F
    return 8.0 * tokens * F + 4.0 * F * F

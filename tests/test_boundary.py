"""The C ABI boundary on the CPU: the library loads, exports what include/ssd.h
declares, and rejects invalid arguments before launching anything (these calls
never reach the HIP runtime, so no GPU is needed)."""

import ctypes
import os
import subprocess

import pytest

import complex_chunkwise_ssd_amd as ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssd.LIBPATH):
        from complex_chunkwise_ssd_amd import build
        build.build()
    return ssd.load_library()


def test_header_declares_the_boundary():
    names = set(ssd.header_functions())
    assert {"ssd_discretise", "ssd_chunk_forward", "ssd_chunk_forward_workspace_bytes",
            "ssd_chunk_backward", "ssd_chunk_backward_workspace_bytes",
            "ssd_status_string", "ssd_version"} <= names


def test_library_exports_every_declared_symbol(lib):
    for name in ssd.header_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", ssd.LIBPATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(ssd.header_functions()) <= exported


def test_library_is_built_for_gfx950():
    # the fat binary of our own build names its offload target
    data = open(ssd.LIBPATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in data


def test_status_strings(lib):
    for st in range(-9, 1):
        s = ssd.status_string(st)
        assert s and s != "unknown status"
    assert ssd.status_string(-99) == "unknown status"
    assert lib.ssd_version() >= 100


def _fwd(lib, B=1, T=16, H=2, N=4, D=4, Q=4, ptrs=True, ws=None, ws_n=0, align=0):
    p = ctypes.c_void_p(0x100000 + align) if ptrs else None
    p16 = ctypes.c_void_p(0x100000 + (align if align % 16 else 0)) if ptrs else None
    return lib.ssd_chunk_forward(p, p, p16, p16, p, B, T, H, N, D, Q, None, p, None, ws, ws_n, None)


def test_shape_errors(lib):
    assert _fwd(lib, B=-1) == ssd.SSD_ERR_SHAPE
    assert _fwd(lib, T=-1) == ssd.SSD_ERR_SHAPE
    assert _fwd(lib, H=-1) == ssd.SSD_ERR_SHAPE
    assert _fwd(lib, N=0) == ssd.SSD_ERR_SHAPE
    assert _fwd(lib, D=0) == ssd.SSD_ERR_SHAPE
    assert _fwd(lib, Q=0) == ssd.SSD_ERR_SHAPE


def test_odd_n_rejected(lib):
    for n in (1, 3, 63):
        assert _fwd(lib, N=n) == ssd.SSD_ERR_ODD_N


def test_block_dims_cap(lib):
    assert _fwd(lib, N=258) == ssd.SSD_ERR_BLOCK_DIMS
    assert _fwd(lib, D=257) == ssd.SSD_ERR_BLOCK_DIMS
    assert _fwd(lib, Q=257) == ssd.SSD_ERR_BLOCK_DIMS


def test_null_and_alignment(lib):
    assert _fwd(lib, ptrs=False) == ssd.SSD_ERR_NULL
    assert _fwd(lib, align=4) == ssd.SSD_ERR_ALIGN      # complex arrays need 8 bytes
    # 8-byte complex arrays pass the alignment check (this call then needs a workspace)
    assert _fwd(lib, align=8) == ssd.SSD_ERR_WORKSPACE


def test_workspace_checks(lib):
    need = lib.ssd_chunk_forward_workspace_bytes(1, 2048, 16, 64, 64, 64)
    assert need > 0
    args = dict(B=1, T=2048, H=16, N=64, D=64, Q=64)
    assert _fwd(lib, ws=None, ws_n=need, **args) == ssd.SSD_ERR_WORKSPACE
    assert _fwd(lib, ws=ctypes.c_void_p(0x200000), ws_n=need - 1, **args) == ssd.SSD_ERR_WORKSPACE
    assert _fwd(lib, ws=ctypes.c_void_p(0x200010), ws_n=need, **args) == ssd.SSD_ERR_ALIGN


def test_state_sizes_above_64(lib):
    # the forward takes N up to 256 in 64-row slices; their partial outputs need
    # workspace, so a call without one is refused
    need = lib.ssd_chunk_forward_workspace_bytes(1, 16, 2, 66, 4, 4)
    assert need >= 2 * 1 * 16 * 2 * 4 * 4
    assert _fwd(lib, N=66, D=4) == ssd.SSD_ERR_WORKSPACE
    assert _fwd(lib, N=256, D=4) == ssd.SSD_ERR_WORKSPACE
    assert _fwd(lib, N=258, D=4) == ssd.SSD_ERR_BLOCK_DIMS
    assert _fwd(lib, N=64, Q=256) != ssd.SSD_ERR_UNSUPPORTED


def test_workspace_sizes(lib):
    f = lib.ssd_chunk_forward_workspace_bytes
    # 512 sequences fill the GPU: no segments, no workspace
    assert f(32, 2048, 16, 64, 64, 64) == 0
    # fewer sequences: segments whose end states need N*D complex each
    n = f(8, 2048, 16, 64, 64, 64)
    assert n >= 8 * 16 * 64 * 64 * 8
    assert f(-1, 16, 2, 4, 4, 4) == 0 and f(1, 16, 2, 3, 4, 4) == 0
    assert f(0, 16, 2, 4, 4, 4) == 0 and f(1, 0, 2, 4, 4, 4) == 0
    # N = 128 at the network shape: two slices' partial outputs, no segments
    assert f(32, 2048, 16, 128, 64, 64) >= 2 * 32 * 2048 * 16 * 64 * 4


def test_empty_batch_is_a_noop(lib):
    assert lib.ssd_chunk_forward(None, None, None, None, None, 0, 16, 2, 4, 4, 4, None, None, None,
                                 None, 0, None) == ssd.SSD_OK
    assert lib.ssd_chunk_forward(None, None, None, None, None, 2, 16, 0, 4, 4, 4, None, None, None,
                                 None, 0, None) == ssd.SSD_OK
    assert lib.ssd_chunk_forward(None, None, None, None, None, 2, 0, 2, 4, 4, 4, None, None, None,
                                 None, 0, None) == ssd.SSD_OK


def test_discretise_argument_checks(lib):
    p = ctypes.c_void_p(0x100000)
    assert lib.ssd_discretise(p, p, -1, 4, 2, 0, p, None, None) == ssd.SSD_ERR_SHAPE
    assert lib.ssd_discretise(p, p, 1, 4, 2, 0, p, p, None) == ssd.SSD_ERR_SHAPE
    assert lib.ssd_discretise(p, p, 1, 4, 2, 300, None, p, None) == ssd.SSD_ERR_BLOCK_DIMS
    assert lib.ssd_discretise(None, p, 1, 4, 2, 4, None, p, None) == ssd.SSD_ERR_NULL
    assert lib.ssd_discretise(p, ctypes.c_void_p(0x100004), 1, 4, 2, 4, None, p, None) == \
        ssd.SSD_ERR_ALIGN
    assert lib.ssd_discretise(p, p, 0, 4, 2, 4, None, p, None) == ssd.SSD_OK


def test_python_layer_rejects_bad_tensors():
    import torch
    x = torch.zeros(1, 4, 2, 4, dtype=torch.complex64)
    A = torch.zeros(2, dtype=torch.complex64)
    B = torch.zeros(1, 4, 2, 4, dtype=torch.complex64)
    dt = torch.zeros(1, 4, 2)
    with pytest.raises(ValueError):
        ssd.chunk_forward(x, A, B, B, dt)                # CPU tensors
    with pytest.raises(ValueError):
        ssd.discretise(dt, A, 4)


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(OSError):
        ssd.load_library(str(tmp_path / "libssd.so"))


def _bwd(lib, B=1, T=16, H=2, N=4, D=4, Q=4, ptrs=True, ws=None, ws_n=0, align=0, gA=True):
    p = ctypes.c_void_p(0x100000 + align) if ptrs else None
    a = ctypes.c_void_p(0x100000) if gA else None
    return lib.ssd_chunk_backward(p, p, p, p, p, B, T, H, N, D, Q, None, p, None, p, a, p, p, p,
                                  None, ws, ws_n, None)


def test_backward_argument_checks(lib):
    need = lib.ssd_chunk_backward_workspace_bytes(1, 16, 2, 4, 4, 4)
    ws = ctypes.c_void_p(0x200000)
    assert _bwd(lib, B=-1) == ssd.SSD_ERR_SHAPE
    assert _bwd(lib, Q=0) == ssd.SSD_ERR_SHAPE
    assert _bwd(lib, N=3) == ssd.SSD_ERR_ODD_N
    assert _bwd(lib, D=257) == ssd.SSD_ERR_BLOCK_DIMS
    # N and D up to 256 are covered (64 x 64 state blocks): a valid N = 66 or D = 65
    # passes the size checks and stops at the missing workspace
    assert _bwd(lib, N=66) == ssd.SSD_ERR_WORKSPACE
    assert _bwd(lib, D=65) == ssd.SSD_ERR_WORKSPACE
    assert _bwd(lib, gA=False) == ssd.SSD_ERR_NULL
    assert _bwd(lib, ptrs=False) == ssd.SSD_ERR_NULL
    assert _bwd(lib, align=4, ws=ws, ws_n=need) == ssd.SSD_ERR_ALIGN
    assert _bwd(lib, ws=None, ws_n=need) == ssd.SSD_ERR_WORKSPACE
    assert _bwd(lib, ws=ws, ws_n=need - 1) == ssd.SSD_ERR_WORKSPACE
    assert _bwd(lib, ws=ctypes.c_void_p(0x200010), ws_n=need) == ssd.SSD_ERR_ALIGN
    assert lib.ssd_chunk_backward(None, None, None, None, None, 0, 16, 2, 4, 4, 4, None, None, None,
                                  None, None, None, None, None, None, None, 0, None) == ssd.SSD_OK


def test_backward_workspace_sizes(lib):
    f = lib.ssd_chunk_backward_workspace_bytes
    # two (B, H, chunks, 64, 64) complex state arrays + per-chunk gA shares
    assert f(32, 2048, 16, 64, 64, 64) >= 2 * 32 * 16 * 64 * 64 * 64 * 8
    assert f(1, 100, 2, 4, 4, 8) >= 2 * 2 * 13 * 64 * 64 * 8
    assert f(1, 16, 2, 4, 257, 4) == 0 and f(0, 16, 2, 4, 4, 4) == 0 and f(1, 0, 2, 4, 4, 4) == 0
    # N = 130, D = 70: 3 x 2 state blocks and the per-slice partial gradients
    blocks = 2 * 1 * 2 * 6 * 4 * 64 * 64 * 8   # states + adjoints, 4 chunks of 4 tokens
    parts = 8 * 16 * 2 * (3 * 70 + 2 * 2 * 130) + 4 * 16 * 2 * 6
    assert f(1, 16, 2, 130, 70, 4) >= blocks + parts
    assert ssd.backward_workspace_bytes(1, 100, 2, 4, 4, 8) == f(1, 100, 2, 4, 4, 8)
    # the chunk pass indexes (virtual sequence, chunk) pairs in 32 bits: 2^20 sequences of
    # 2^11 32-token chunks are 2^31 pairs, one too many
    assert f(1 << 20, 1 << 16, 1, 2, 2, 32) == 0
    assert f(1 << 20, (1 << 16) - 32, 1, 2, 2, 32) > 0


def test_backward_chunk_count_limit(lib):
    args = dict(B=1 << 20, T=1 << 16, H=1, N=2, D=2, Q=32)
    assert _bwd(lib, **args) == ssd.SSD_ERR_UNSUPPORTED


def test_python_backward_rejects_bad_tensors():
    import torch
    x = torch.zeros(1, 4, 2, 4, dtype=torch.complex64)
    A = torch.zeros(2, dtype=torch.complex64)
    B = torch.zeros(1, 4, 2, 4, dtype=torch.complex64)
    dt = torch.zeros(1, 4, 2)
    with pytest.raises(ValueError):
        ssd.chunk_backward(x, A, B, B, dt, torch.zeros(1, 4, 2, 4))  # CPU tensors


def _proj(lib, B=1, T=16, H=2, N=4, D=4, Q=4, S=None, ptrs=True, align=0, ws=None, ws_n=0):
    S = H * (D + 4 * N + 1) if S is None else S
    p = ctypes.c_void_p(0x100000 + align) if ptrs else None
    a = ctypes.c_void_p(0x100000) if ptrs else None
    return lib.ssd_chunk_forward_proj(p, S, a, B, T, H, N, D, Q, None, a, None, ws, ws_n, None)


def test_proj_argument_checks(lib):
    assert _proj(lib, S=2 * (4 + 16 + 1) - 2) == ssd.SSD_ERR_SHAPE   # row shorter than its blocks
    assert _proj(lib, N=3) == ssd.SSD_ERR_ODD_N
    assert _proj(lib, N=66, D=4) == ssd.SSD_ERR_WORKSPACE      # N slices need workspace
    assert _proj(lib, S=1 << 23) == ssd.SSD_ERR_UNSUPPORTED
    assert _proj(lib, ptrs=False) == ssd.SSD_ERR_NULL
    assert _proj(lib, align=4) == ssd.SSD_ERR_ALIGN                  # proj needs 8 bytes
    assert _proj(lib, S=2 * (4 + 16 + 1) + 1) == ssd.SSD_ERR_ALIGN    # odd row length
    assert _proj(lib, H=1, D=3, S=(3 + 16 + 1) + 1) == ssd.SSD_ERR_ALIGN  # H*D odd
    need = lib.ssd_chunk_forward_workspace_bytes(1, 2048, 16, 64, 64, 64)
    assert _proj(lib, B=1, T=2048, H=16, N=64, D=64, Q=64, ws=None, ws_n=need) == \
        ssd.SSD_ERR_WORKSPACE
    assert lib.ssd_chunk_forward_proj(None, 42, None, 0, 16, 2, 4, 4, 4, None, None, None, None,
                                      0, None) == ssd.SSD_OK



def test_backward_proj_argument_checks(lib):
    p = ctypes.c_void_p(0x100000)
    S = 2 * (4 + 16 + 1)
    need = lib.ssd_chunk_backward_workspace_bytes(1, 16, 2, 4, 4, 4)
    f = lib.ssd_chunk_backward_proj
    assert f(p, S - 1, p, 1, 16, 2, 4, 4, 4, None, p, None, p, p, None, p, need, None) == \
        ssd.SSD_ERR_SHAPE
    assert f(p, 1000, p, 1, 16, 2, 4, 65, 4, None, p, None, p, p, None, p, need, None) == \
        ssd.SSD_ERR_WORKSPACE  # D = 65 is covered; its workspace is larger
    assert f(p, S, p, 1, 16, 2, 4, 4, 4, None, p, None, None, p, None, p, need, None) == \
        ssd.SSD_ERR_NULL
    assert f(p, S, p, 1, 16, 2, 4, 4, 4, None, p, None, p, None, None, p, need, None) == \
        ssd.SSD_ERR_NULL
    assert f(ctypes.c_void_p(0x100002), S, p, 1, 16, 2, 4, 4, 4, None, p, None, p, p, None, p,
             need, None) == ssd.SSD_ERR_ALIGN
    assert f(p, S, p, 1, 16, 2, 4, 4, 4, None, p, None, p, p, None, None, need, None) == \
        ssd.SSD_ERR_WORKSPACE


def test_noalloc_argument_checks(lib):
    p = ctypes.c_void_p(0x100000)
    f = lib.ssd_chunk_forward_noalloc
    # sizes whose workspace exceeds the static scratch are refused before anything runs
    assert lib.ssd_chunk_forward_workspace_bytes(1, 2048, 16, 256, 256, 64) > \
        ssd.SSD_NOALLOC_SCRATCH_BYTES
    assert f(p, p, p, p, p, 1, 2048, 16, 256, 256, 64, None, p, None, None) == \
        ssd.SSD_ERR_WORKSPACE
    assert f(p, p, p, p, p, 1, 16, 2, 3, 4, 4, None, p, None, None) == ssd.SSD_ERR_ODD_N
    assert f(None, p, p, p, p, 32, 16, 16, 4, 4, 4, None, p, None, None) == ssd.SSD_ERR_NULL
    assert f(p, p, p, p, p, 0, 16, 2, 4, 4, 4, None, p, None, None) == ssd.SSD_OK


def test_head_mix_argument_checks(lib):
    # distinct fake device addresses, far enough apart not to overlap
    y, W, z = (ctypes.c_void_p(a) for a in (0x10000000, 0x20000000, 0x30000000))
    f = lib.ssd_head_mix
    assert f(None, W, 4, 16, 64, z, None) == ssd.SSD_ERR_NULL
    assert f(y, None, 4, 16, 64, z, None) == ssd.SSD_ERR_NULL
    assert f(y, W, 4, 16, 64, None, None) == ssd.SSD_ERR_NULL
    assert f(y, W, -1, 16, 64, z, None) == ssd.SSD_ERR_SHAPE
    assert f(y, W, 4, 0, 64, z, None) == ssd.SSD_ERR_SHAPE
    assert f(y, W, 4, 16, 0, z, None) == ssd.SSD_ERR_SHAPE
    assert f(y, W, 4, 16, 257, z, None) == ssd.SSD_ERR_BLOCK_DIMS
    assert f(y, W, 4, 257, 64, z, None) == ssd.SSD_ERR_UNSUPPORTED  # H * D above 16384
    assert f(ctypes.c_void_p(0x10000002), W, 4, 16, 64, z, None) == ssd.SSD_ERR_ALIGN
    assert f(y, W, 4, 16, 64, y, None) == ssd.SSD_ERR_ALIAS  # in place is not a GEMM
    # z's 4 * 1024 floats reach into W only when W starts inside them
    assert f(y, ctypes.c_void_p(0x30000000 + 4 * 4095), 4, 16, 64, z, None) == ssd.SSD_ERR_ALIAS
    assert f(y, W, 0, 16, 64, z, None) == ssd.SSD_OK  # no tokens: nothing launched


def test_head_mix_workspace_sizes(lib):
    ws = lib.ssd_head_mix_backward_workspace_bytes
    # the network layer: 65,536 tokens of 1024 -> 16 token splits of (1024, 1024) floats
    assert ws(65536, 16, 64) == 16 * 1024 * 1024 * 4
    assert ws(5, 16, 64) == 0           # one split: written straight to grad_W
    assert ws(0, 16, 64) == 0
    assert ws(4, 257, 64) == 0          # invalid
    assert ws(2100, 2, 4) == 768        # three splits of an 8 x 8 gradient, rounded to 256


def test_head_mix_backward_argument_checks(lib):
    y, W, gz, gy, gW, w = (ctypes.c_void_p(a) for a in (0x10000000, 0x20000000, 0x30000000,
                                                         0x40000000, 0x50000000, 0x60000000))
    f = lib.ssd_head_mix_backward
    need = lib.ssd_head_mix_backward_workspace_bytes(65536, 16, 64)
    assert f(y, W, gz, 8, 16, 64, gy, None, w, need, None) == ssd.SSD_ERR_NULL
    assert f(y, W, None, 8, 16, 64, gy, gW, w, need, None) == ssd.SSD_ERR_NULL
    assert f(y, W, gz, 8, 257, 64, gy, gW, w, need, None) == ssd.SSD_ERR_UNSUPPORTED
    assert f(y, W, gz, 65536, 16, 64, gy, gW, None, need, None) == ssd.SSD_ERR_WORKSPACE
    assert f(y, W, gz, 65536, 16, 64, gy, gW, w, 16, None) == ssd.SSD_ERR_WORKSPACE
    assert f(y, W, gz, 65536, 16, 64, gy, gW, ctypes.c_void_p(0x60000010), need, None) == \
        ssd.SSD_ERR_ALIGN                # the workspace must be 256-byte aligned
    assert f(y, W, gz, 8, 16, 64, ctypes.c_void_p(0x40000001), gW, w, need, None) == \
        ssd.SSD_ERR_ALIGN
    assert f(y, W, gz, 8, 16, 64, gz, gW, w, need, None) == ssd.SSD_ERR_ALIAS
    assert f(y, W, gz, 8, 16, 64, gy, W, w, need, None) == ssd.SSD_ERR_ALIAS
    assert f(y, W, gz, 65536, 16, 64, gy, gW, y, need, None) == ssd.SSD_ERR_ALIAS


def test_python_head_mix_rejects_bad_tensors():
    import torch
    y = torch.zeros(2, 3, 4, 8)
    with pytest.raises(ValueError):
        ssd.head_mix(y, torch.eye(32))  # CPU tensors
    with pytest.raises(ValueError):
        ssd.head_mix_backward(y, torch.eye(32), y)


def test_backward_proj_bf16_argument_checks(lib):
    p = ctypes.c_void_p(0x100000)
    S = 2 * (4 + 16 + 1)
    need = lib.ssd_chunk_backward_workspace_bytes(1, 16, 2, 4, 4, 4)
    f = lib.ssd_chunk_backward_proj_bf16
    assert f(p, S - 1, p, 1, 16, 2, 4, 4, 4, None, p, None, p, p, None, p, need, None) == \
        ssd.SSD_ERR_SHAPE
    assert f(p, S, p, 1, 16, 2, 4, 4, 4, None, p, None, None, p, None, p, need, None) == \
        ssd.SSD_ERR_NULL
    assert f(ctypes.c_void_p(0x100001), S, p, 1, 16, 2, 4, 4, 4, None, p, None, p, p, None, p,
             need, None) == ssd.SSD_ERR_ALIGN     # bfloat16 rows need 2 bytes
    assert f(p, S, p, 1, 16, 2, 4, 4, 4, None, p, None, p, p, None, None, need, None) == \
        ssd.SSD_ERR_WORKSPACE

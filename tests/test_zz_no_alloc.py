"""ssd_chunk_forward_noalloc (workspace in a static per-GPU device array) against
ssd_chunk_forward (caller-supplied workspace), both called through the C ABI
with ctypes: the same kernels on the same inputs, so the outputs must be
bit-identical. Two calls in a row, the second smaller than the first (the
scratch keeps the first call's contents), then a size past the scratch."""

import ctypes

import numpy as np
import pytest
import torch

import complex_chunkwise_ssd_amd as ssd
import ssd_inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _run(lib, g, Q, init, noalloc):
    Bsz, T, H, D = g.x.shape
    N = g.B_t.shape[-1]
    y = torch.full((Bsz, T, H, D), float("nan"), device=DEV)
    fs = torch.full((Bsz, H, N, D), float("nan"), dtype=torch.complex64, device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    args = [_ptr(g.x), _ptr(g.A), _ptr(g.B_t), _ptr(g.C_t), _ptr(g.dt), Bsz, T, H, N, D, Q,
            _ptr(init), _ptr(y), _ptr(fs)]
    if noalloc:
        st = lib.ssd_chunk_forward_noalloc(*args, stream)
    else:
        n = int(lib.ssd_chunk_forward_workspace_bytes(Bsz, T, H, N, D, Q))
        ws = torch.full((max(n, 1),), 255, dtype=torch.uint8, device=DEV)
        st = lib.ssd_chunk_forward(*args, _ptr(ws) if n else None, n, stream)
    assert st == ssd.SSD_OK, ssd.status_string(st)
    torch.cuda.synchronize()
    return y.cpu(), fs.cpu()


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_the_workspace_entry_point(order):
    lib = ssd.load_library()
    cases = [
        # B=1, T=2048, H=16, N=D=64, chunk 64: 16 segments per sequence (8 MiB of scratch)
        (ssd_inputs.layer_case(1, 2048, 16, 64, 64, seed=1, device=DEV), 64, None),
        # smaller, with an initial state and a ragged chunk: the scratch holds the
        # first call's larger contents
        (ssd_inputs.random_case(2, 300, 4, 64, 64, seed=5).to(DEV), 32,
         (torch.randn(2, 4, 64, 64, generator=torch.Generator().manual_seed(6)) * 0.3).to(
             torch.complex64).to(DEV)),
    ]
    for g, Q, init in cases:
        Bsz, T, H, D = g.x.shape
        N = g.B_t.shape[-1]
        assert 0 < lib.ssd_chunk_forward_workspace_bytes(Bsz, T, H, N, D, Q) <= \
            ssd.SSD_NOALLOC_SCRATCH_BYTES
        print("noalloc case B=%d T=%d H=%d N=%d D=%d Q=%d" % (Bsz, T, H, N, D, Q), flush=True)
        ya, fa = _run(lib, g, Q, init, noalloc=True)
        yb, fb = _run(lib, g, Q, init, noalloc=False)
        assert torch.isfinite(ya).all() and torch.equal(ya, yb) and torch.equal(fa, fb)


def test_noalloc_rejects_sizes_past_the_scratch():
    lib = ssd.load_library()
    p = ctypes.c_void_p(0x100000)
    # N = D = 256 on 16 sequences: 128 MiB of partial outputs, more than the scratch
    assert lib.ssd_chunk_forward_workspace_bytes(1, 2048, 16, 256, 256, 64) > \
        ssd.SSD_NOALLOC_SCRATCH_BYTES
    st = lib.ssd_chunk_forward_noalloc(p, p, p, p, p, 1, 2048, 16, 256, 256, 64, None, p, None,
                                       None)
    assert st == ssd.SSD_ERR_WORKSPACE

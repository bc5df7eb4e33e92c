"""The entry points under HIP graph capture (torch.cuda.CUDAGraph), for callers
that capture their step once and replay it: each call launches its kernels on
the caller's stream and nothing else (no allocation, no memset, no host
synchronisation), so a captured call replays the same work.

Every buffer is allocated before capture and passed in; one eager call per
entry point comes first (the no-allocation entry point resolves its static
scratch array on its first call). Each graph is replayed three times with new
inputs copied into its input tensors, eager calls and synchronisations in
between, and every replay must equal the eager call on the same inputs bit for
bit. The shapes take the segmented forward (prefix and fix-up passes), the
fused backward and the mixer's split weight gradient.
"""

import pytest
import torch

import complex_chunkwise_ssd_amd as ssd
import ssd_inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _capture(fn):
    """Eager warm-up on a side stream, then capture fn() into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _load(dst, src):
    for d, s in zip(dst, src):
        d.copy_(s)


@pytest.mark.parametrize("noalloc", [False, True])
def test_forward_replays_equal_eager_calls(noalloc):
    # 8 sequences of 600 tokens: cut into segments, so the prefix and fix-up run too
    Bsz, T, H, N, D, Q = 2, 600, 4, 64, 64, 64
    first = ssd_inputs.random_case(Bsz, T, H, N, D, seed=81).to(DEV)
    xs, As, Bs, Cs, ds = (t.clone() for t in (first.x, first.A, first.B_t, first.C_t, first.dt))
    y = torch.empty((Bsz, T, H, D), device=DEV)
    fs = torch.empty((Bsz, H, N, D), dtype=torch.complex64, device=DEV)
    n = ssd.workspace_bytes(Bsz, T, H, N, D, Q)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)

    def call(y_out, f_out, wsp):
        if noalloc:
            ssd.chunk_forward_noalloc(xs, As, Bs, Cs, ds, chunk_size=Q, y=y_out, final_state=f_out)
        else:
            ssd.chunk_forward(xs, As, Bs, Cs, ds, chunk_size=Q, y=y_out, final_state=f_out,
                              workspace=wsp)

    g = _capture(lambda: call(y, fs, ws))
    ye, fe = torch.empty_like(y), torch.empty_like(fs)
    we = torch.empty_like(ws)
    for rep in range(3):
        inp = ssd_inputs.random_case(Bsz, T, H, N, D, seed=90 + rep).to(DEV)
        _load((xs, As, Bs, Cs, ds), (inp.x, inp.A, inp.B_t, inp.C_t, inp.dt))
        call(ye, fe, we)  # eager, same inputs, other buffers
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ye) and torch.equal(fs, fe), "replay %d" % rep


def test_backward_replays_equal_eager_calls():
    # 256 sequences: the fused adjoint walk
    Bsz, T, H, N, D, Q = 16, 80, 16, 64, 64, 64
    first = ssd_inputs.random_case(Bsz, T, H, N, D, seed=83).to(DEV)
    ins = [t.clone() for t in (first.x, first.A, first.B_t, first.C_t, first.dt)]
    gy0, gf0 = ssd_inputs.upstream_grads(Bsz, T, H, N, D, seed=84)
    gy, gf = gy0.to(DEV), gf0.to(DEV)
    n = ssd.backward_workspace_bytes(Bsz, T, H, N, D, Q)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
    we = torch.empty_like(ws)

    def grads():
        c64 = dict(dtype=torch.complex64, device=DEV)
        return ssd.Grads(torch.empty((Bsz, T, H, D), **c64), torch.empty((H,), **c64),
                         torch.empty((Bsz, T, H, N), **c64), torch.empty((Bsz, T, H, N), **c64),
                         torch.empty((Bsz, T, H), device=DEV), torch.empty((Bsz, H, N, D), **c64))

    out, ref = grads(), grads()

    def call(o, wsp):
        ssd.chunk_backward(*ins, gy, gf, chunk_size=Q, out=o, workspace=wsp)

    g = _capture(lambda: call(out, ws))
    for rep in range(3):
        inp = ssd_inputs.random_case(Bsz, T, H, N, D, seed=95 + rep).to(DEV)
        _load(ins, (inp.x, inp.A, inp.B_t, inp.C_t, inp.dt))
        u, f = ssd_inputs.upstream_grads(Bsz, T, H, N, D, seed=98 + rep)
        _load((gy, gf), (u, f))
        call(ref, we)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(out, ref):
            assert torch.equal(a, b), "replay %d" % rep


def test_mixer_replays_equal_eager_calls():
    # 2100 tokens: grad_W in three token splits and their fixed-order sum
    lead, H, D = (2100,), 4, 16
    y0, W0, gz0 = ssd_inputs.mix_case(lead + (H, D), seed=85)
    y, W, gz = y0.to(DEV), W0.to(DEV), gz0.to(DEV)
    F = H * D
    z, gyo, gWo = torch.empty_like(y), torch.empty_like(y), torch.empty((F, F), device=DEV)
    ze, gye, gWe = torch.empty_like(z), torch.empty_like(gyo), torch.empty_like(gWo)
    n = ssd.head_mix_workspace_bytes(lead[0], H, D)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
    we = torch.empty_like(ws)

    def call(zz, gyy, gww, wsp):
        ssd.head_mix(y, W, z=zz)
        ssd.head_mix_backward(y, W, gz, grad_y=gyy, grad_W=gww, workspace=wsp)

    g = _capture(lambda: call(z, gyo, gWo, ws))
    for rep in range(3):
        a, b, c = ssd_inputs.mix_case(lead + (H, D), seed=86 + rep)
        _load((y, W, gz), (a, b, c))
        call(ze, gye, gWe, we)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(z, ze) and torch.equal(gyo, gye) and torch.equal(gWo, gWe), \
            "replay %d" % rep

"""GPU parity of the MIMO head mixer (ssd_head_mix, ssd_head_mix_backward)
against the oracle, through the C ABI.

Bars: z and grad_y are sums of H products: |d| <= 1e-4 + 1e-4 |ref|
elementwise. grad_W sums every (token, channel) pair: |d| <= 1e-4 (1 + |ref|)
plus 1e-5 * sqrt(sum of squared terms) (tests/tolerances.py). The network
layer's shape (32 x 2048 tokens, 16 heads of 64) is compared in full.
"""

import numpy as np
import pytest
import torch

import complex_chunkwise_ssd_amd as ssd
import oracle
import ssd_inputs
import tolerances

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

CASES = [
    # leading (token) shape, H, D
    ((5,), 16, 64),
    ((2, 3), 7, 10),
    ((9,), 20, 8),
    ((1,), 1, 1),
    ((3,), 32, 12),
    ((2, 300), 16, 64),
    ((4, 33), 5, 36),
    ((1, 2048), 16, 64),      # one sequence of the single-layer shape
    ((3, 7), 16, 100),        # the fused backward over two channel blocks
    ((9,), 12, 132),          # fewer heads than a block, three channel blocks
    ((2, 5), 20, 64),         # more than 16 heads: the two-pass backward
]


def _fwd_check(z, ref, what):
    assert np.isfinite(z).all(), what
    e = np.abs(z - ref)
    assert (e <= 1e-4 + 1e-4 * np.abs(ref)).all(), "%s max %.3e" % (what, e.max())


def _bwd_check(gy, gW, ry, rW, gz, y, what):
    assert np.isfinite(gy).all() and np.isfinite(gW).all(), what
    e = np.abs(gy - ry)
    assert (e <= 1e-4 + 1e-4 * np.abs(ry)).all(), "%s grad_y max %.3e" % (what, e.max())
    tol = 1e-4 * (1 + np.abs(rW)) + tolerances.grad_w_extra(gz, y)
    eW = np.abs(gW - rW)
    assert (eW <= tol).all(), "%s grad_W max %.3e (bar %.3e)" % (what, eW.max(), tol.min())


@pytest.mark.parametrize("case", CASES)
def test_head_mix_matches_oracle(case):
    lead, H, D = case
    y, W, gz = ssd_inputs.mix_case(lead + (H, D), seed=H * 1000 + D)
    z = ssd.head_mix(y.to(DEV), W.to(DEV))
    gy, gW = ssd.head_mix_backward(y.to(DEV), W.to(DEV), gz.to(DEV))
    torch.cuda.synchronize()
    _fwd_check(z.cpu().numpy(), oracle.head_mix(y, W), str(case))
    ry, rW = oracle.head_mix_backward(y, W, gz)
    _bwd_check(gy.cpu().numpy(), gW.cpu().numpy(), ry, rW, gz.numpy(), y.numpy(), str(case))


def test_head_mix_network_layer_shape():
    """One layer of the network load, B=32, T=2048, H=16, D=64, compared in full."""
    y, W, gz = ssd_inputs.mix_case((32, 2048, 16, 64), seed=5)
    yd, Wd, gzd = y.to(DEV), W.to(DEV), gz.to(DEV)
    z = ssd.head_mix(yd, Wd)
    gy, gW = ssd.head_mix_backward(yd, Wd, gzd)
    torch.cuda.synchronize()
    _fwd_check(z.cpu().numpy(), oracle.head_mix(y, W), "network layer")
    ry, rW = oracle.head_mix_backward(y, W, gz)
    _bwd_check(gy.cpu().numpy(), gW.cpu().numpy(), ry, rW, gz.numpy(), y.numpy(), "network layer")


def test_head_mix_misaligned_rows_take_the_scalar_path():
    y, W, gz = ssd_inputs.mix_case((7, 16, 64), seed=11)
    buf = torch.zeros(y.numel() + 1, device=DEV)
    buf[1:] = y.to(DEV).reshape(-1)
    yv = buf[1:].view(7, 16, 64)           # 4 bytes past 16-byte alignment
    out = torch.zeros(y.numel() + 1, device=DEV)
    zv = out[1:].view(7, 16, 64)
    ssd.head_mix(yv, W.to(DEV), z=zv)
    torch.cuda.synchronize()
    _fwd_check(zv.cpu().numpy(), oracle.head_mix(y, W), "misaligned")


def test_head_mix_in_place_and_identity():
    y, W, gz = ssd_inputs.mix_case((3, 40, 16, 64), seed=12)
    yd = y.to(DEV)
    z = ssd.head_mix(yd, torch.eye(16, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(z.cpu(), y)               # the identity mixer is exact
    ssd.head_mix(yd, W.to(DEV), z=yd)            # in place
    torch.cuda.synchronize()
    _fwd_check(yd.cpu().numpy(), oracle.head_mix(y, W), "in place")


def test_head_mix_after_the_scan():
    """The pipeline order scan -> mixer: the mixer applied to the scan's y
    equals the oracle mixer applied to the oracle scan's y within the sum of
    both bars."""
    inp = ssd_inputs.layer_case(2, 256, 16, 64, 64, seed=3, device="cpu")
    g = inp.to(DEV)
    y, _ = ssd.chunk_forward(g.x, g.A, g.B_t, g.C_t, g.dt, chunk_size=64)
    _, W, _ = ssd_inputs.mix_case((1, 16, 64), seed=4)
    z = ssd.head_mix(y, W.to(DEV))
    torch.cuda.synchronize()
    yo, _ = oracle.scan(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt)
    zo = np.matmul(W.numpy().astype(np.float64), yo.real)
    bar = np.abs(W.numpy()).astype(np.float64) @ (1e-4 + 1e-4 * np.abs(yo.real))
    e = np.abs(z.cpu().numpy() - zo)
    assert (e <= bar + 1e-4 + 1e-4 * np.abs(zo)).all(), e.max()


def test_head_mix_backward_is_deterministic_and_repeatable():
    y, W, gz = ssd_inputs.mix_case((4, 1000, 16, 64), seed=13)
    yd, Wd, gzd = y.to(DEV), W.to(DEV), gz.to(DEV)
    a = ssd.head_mix_backward(yd, Wd, gzd)
    b = ssd.head_mix_backward(yd, Wd, gzd)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_head_mix_zero_tokens():
    y = torch.zeros(0, 16, 64, device=DEV)
    W = torch.eye(16, device=DEV)
    z = ssd.head_mix(y, W)
    gy, gW = ssd.head_mix_backward(y, W, y)
    torch.cuda.synchronize()
    assert z.shape == (0, 16, 64) and torch.equal(gW.cpu(), torch.zeros(16, 16))


def test_head_mix_backward_in_place():
    """grad_y may be grad_z itself: each token's grad_z is read before its grad_y
    is written."""
    y, W, gz = ssd_inputs.mix_case((6, 50, 16, 64), seed=14)
    yd, Wd = y.to(DEV), W.to(DEV)
    g = gz.to(DEV).clone()
    ref_y, ref_W = ssd.head_mix_backward(yd, Wd, gz.to(DEV))
    gy, gW = ssd.head_mix_backward(yd, Wd, g, grad_y=g)
    torch.cuda.synchronize()
    assert torch.equal(gy, ref_y) and torch.equal(gW, ref_W)

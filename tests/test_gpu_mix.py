"""GPU parity of the MIMO head mixer (ssd_head_mix, ssd_head_mix_backward)
against the oracle, through the C ABI.

The mixer is the dense map z[m, o] = sum_k W[o, k] y[m, k] over each token's
flattened heads (F = H * D), with gradients grad_y = grad_z W and
grad_W = grad_z^T y. Bars: every output is a float32 sum of products t, so
|d| <= 1e-4 + 1e-4 |ref| + 1e-5 * sqrt(sum t^2) elementwise
(tests/tolerances.py derives the last term). The network layer's shape
(32 x 2048 tokens, 16 heads of 64, a dense 1024 x 1024 W) is compared in full.
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
    ((5,), 16, 64),           # F = 1024, four column tiles
    ((2, 3), 7, 10),          # F = 70: scalar loads
    ((1,), 1, 1),
    ((300,), 4, 80),          # ragged row and column tiles
    ((2, 300), 16, 64),       # three row tiles, the last ragged
    ((4, 33), 5, 36),
    ((1, 2048), 16, 64),      # one sequence of the single-layer shape
    ((3, 7), 16, 100),        # F = 1600: seven column tiles, the last ragged
    ((2100,), 2, 4),          # the token sum of grad_W cut into three splits
    ((9,), 12, 132),
]


def _fwd_check(z, ref, y, W, what):
    assert np.isfinite(z).all(), what
    e = np.abs(z - ref)
    tol = 1e-4 + 1e-4 * np.abs(ref) + tolerances.mix_forward_extra(y, W)
    assert (e <= tol).all(), "%s max %.3e" % (what, e.max())


def _bwd_check(gy, gW, ry, rW, gz, y, W, what):
    assert np.isfinite(gy).all() and np.isfinite(gW).all(), what
    e = np.abs(gy - ry)
    ty = 1e-4 + 1e-4 * np.abs(ry) + tolerances.mix_grad_y_extra(gz, W)
    assert (e <= ty).all(), "%s grad_y max %.3e" % (what, e.max())
    tw = 1e-4 * (1 + np.abs(rW)) + tolerances.mix_grad_w_extra(gz, y)
    eW = np.abs(gW - rW)
    assert (eW <= tw).all(), "%s grad_W max %.3e (bar %.3e)" % (what, eW.max(), tw.min())


@pytest.mark.parametrize("case", CASES)
def test_head_mix_matches_oracle(case):
    lead, H, D = case
    print("head_mix case", case, flush=True)
    y, W, gz = ssd_inputs.mix_case(lead + (H, D), seed=H * 1000 + D)
    z = ssd.head_mix(y.to(DEV), W.to(DEV))
    gy, gW = ssd.head_mix_backward(y.to(DEV), W.to(DEV), gz.to(DEV))
    torch.cuda.synchronize()
    _fwd_check(z.cpu().numpy(), oracle.head_mix(y, W), y.numpy(), W.numpy(), str(case))
    ry, rW = oracle.head_mix_backward(y, W, gz)
    _bwd_check(gy.cpu().numpy(), gW.cpu().numpy(), ry, rW, gz.numpy(), y.numpy(), W.numpy(),
               str(case))


def test_head_mix_network_layer_shape():
    """One layer of the network load, B=32, T=2048, H=16, D=64 (65,536 tokens
    through a dense 1024 x 1024 W), every output and weight gradient compared."""
    y, W, gz = ssd_inputs.mix_case((32, 2048, 16, 64), seed=5)
    yd, Wd, gzd = y.to(DEV), W.to(DEV), gz.to(DEV)
    z = ssd.head_mix(yd, Wd)
    gy, gW = ssd.head_mix_backward(yd, Wd, gzd)
    torch.cuda.synchronize()
    yn, Wn, gzn = y.numpy(), W.numpy(), gz.numpy()
    _fwd_check(z.cpu().numpy(), oracle.head_mix(y, W), yn, Wn, "network layer")
    del z
    ry, rW = oracle.head_mix_backward(y, W, gz)
    _bwd_check(gy.cpu().numpy(), gW.cpu().numpy(), ry, rW, gzn, yn, Wn, "network layer")


def test_head_mix_misaligned_rows_take_the_scalar_loads():
    y, W, gz = ssd_inputs.mix_case((7, 16, 64), seed=11)
    buf = torch.zeros(y.numel() + 1, device=DEV)
    buf[1:] = y.to(DEV).reshape(-1)
    yv = buf[1:].view(7, 16, 64)           # 4 bytes past 16-byte alignment
    out = torch.zeros(y.numel() + 1, device=DEV)
    zv = out[1:].view(7, 16, 64)
    ssd.head_mix(yv, W.to(DEV), z=zv)
    gbuf = torch.zeros(y.numel() + 1, device=DEV)
    gbuf[1:] = gz.to(DEV).reshape(-1)
    gyv = torch.zeros(y.numel() + 1, device=DEV)[1:].view(7, 16, 64)
    _, gW = ssd.head_mix_backward(yv, W.to(DEV), gbuf[1:].view(7, 16, 64), grad_y=gyv)
    torch.cuda.synchronize()
    _fwd_check(zv.cpu().numpy(), oracle.head_mix(y, W), y.numpy(), W.numpy(), "misaligned")
    ry, rW = oracle.head_mix_backward(y, W, gz)
    _bwd_check(gyv.cpu().numpy(), gW.cpu().numpy(), ry, rW, gz.numpy(), y.numpy(), W.numpy(),
               "misaligned")


def test_head_mix_identity_and_head_permutation_are_exact():
    """The pages' initial mixer (the identity) and a block permutation of the
    heads (P kron I_D) add only exact zeros to one product each: bit-exact."""
    y, _, _ = ssd_inputs.mix_case((3, 40, 16, 64), seed=12)
    yd = y.to(DEV)
    z = ssd.head_mix(yd, torch.eye(1024, device=DEV))
    perm = torch.randperm(16, generator=torch.Generator().manual_seed(3))
    P = torch.zeros(16, 16)
    P[torch.arange(16), perm] = 1.0
    zp = ssd.head_mix(yd, torch.kron(P, torch.eye(64)).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(z.cpu(), y)
    assert torch.equal(zp.cpu(), y[:, :, perm, :])


def test_head_mix_after_the_scan():
    """The pipeline order scan -> mixer: the mixer applied to the scan's y
    equals the oracle mixer applied to the oracle scan's y within the scan's
    bar carried through |W| plus the mixer's own bar."""
    inp = ssd_inputs.layer_case(2, 256, 16, 64, 64, seed=3, device="cpu")
    g = inp.to(DEV)
    y, _ = ssd.chunk_forward(g.x, g.A, g.B_t, g.C_t, g.dt, chunk_size=64)
    _, W, _ = ssd_inputs.mix_case((1, 16, 64), seed=4)
    z = ssd.head_mix(y, W.to(DEV))
    torch.cuda.synchronize()
    yo, _ = oracle.scan(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt)
    Yo = yo.real.reshape(-1, 1024)
    W64 = W.numpy().astype(np.float64)
    zo = (Yo @ W64.T).reshape(yo.shape)
    bar = ((1e-4 + 1e-4 * np.abs(Yo)) @ np.abs(W64).T).reshape(yo.shape)
    bar += 1e-4 + 1e-4 * np.abs(zo) + tolerances.mix_forward_extra(yo.real, W.numpy())
    e = np.abs(z.cpu().numpy() - zo)
    assert (e <= bar).all(), e.max()


def test_head_mix_backward_is_deterministic_and_repeatable():
    y, W, gz = ssd_inputs.mix_case((4, 1000, 16, 64), seed=13)
    yd, Wd, gzd = y.to(DEV), W.to(DEV), gz.to(DEV)
    a = ssd.head_mix_backward(yd, Wd, gzd)
    b = ssd.head_mix_backward(yd, Wd, gzd)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_head_mix_zero_tokens():
    y = torch.zeros(0, 16, 64, device=DEV)
    W = torch.eye(1024, device=DEV)
    z = ssd.head_mix(y, W)
    gW = torch.full((1024, 1024), float("nan"), device=DEV)
    gy, gW = ssd.head_mix_backward(y, W, y, grad_W=gW)
    torch.cuda.synchronize()
    assert z.shape == (0, 16, 64) and torch.equal(gW.cpu(), torch.zeros(1024, 1024))


def test_head_mix_rejects_overlapping_output():
    y, W, gz = ssd_inputs.mix_case((4, 16, 64), seed=15)
    yd, Wd = y.to(DEV), W.to(DEV)
    with pytest.raises(ValueError):
        ssd.head_mix(yd, Wd, z=yd)
    with pytest.raises(ValueError):
        g = gz.to(DEV)
        ssd.head_mix_backward(yd, Wd, g, grad_y=g)

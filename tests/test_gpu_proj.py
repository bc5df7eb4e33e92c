"""GPU parity of the scan read straight from in_proj output rows
(ssd_chunk_forward_proj) against the oracle on the complex inputs the rows
stand for (x = x_real + 0i, B_t = Re B + i Im B, C_t likewise).

Bar (elementwise, as for ssd_chunk_forward): |dy| <= 1e-4 + 1e-4 |y|, and the
same per complex component of final_state. Unused floats at the end of each
row are NaN, so any read outside the row's blocks would show in the output.
"""

import numpy as np
import pytest
import torch

import complex_chunkwise_ssd_amd as ssd
import oracle
import ssd_inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _check(y, fs, yo, fo, what):
    assert np.isfinite(y).all(), what
    e = np.abs(y - yo.real)
    bad = e > 1e-4 + 1e-4 * np.abs(yo.real)
    assert not bad.any(), "%s: %d violations, max |dy| %.3e" % (what, int(bad.sum()), e.max())
    if fs is not None:
        for comp in (np.real, np.imag):
            d = np.abs(comp(fs) - comp(fo))
            assert (d <= 1e-4 + 1e-4 * np.abs(comp(fo))).all(), "%s state %.3e" % (what, d.max())


CASES = [
    # B, T, H, N, D, Q, extra floats per row (row length even)
    (2, 16, 2, 4, 4, 4, 0),
    (1, 64, 1, 64, 64, 64, 1),
    (2, 150, 3, 64, 64, 64, 5),
    (1, 97, 2, 8, 8, 32, 2),
    (2, 50, 2, 6, 10, 16, 4),
    (1, 45, 1, 10, 70, 32, 1),
    (1, 23, 2, 4, 6, 1, 0),
    (3, 7, 1, 2, 2, 64, 1),
    (2, 300, 4, 32, 64, 48, 0),
    (1, 260, 2, 64, 64, 256, 6),
    (2, 90, 2, 128, 32, 32, 2),    # two N slices from in_proj rows
]


@pytest.mark.parametrize("case", CASES)
def test_proj_small_shapes(case):
    B, T, H, N, D, Q, extra = case
    proj, A = ssd_inputs.proj_case(B, T, H, N, D, seed=sum(case), dt_mean=0.3, extra=extra)
    y, fs = ssd.chunk_forward_proj(proj.to(DEV), A.to(DEV), H, N, D, chunk_size=Q)
    torch.cuda.synchronize()
    inp = ssd_inputs.unpack_proj(proj, A, H, N, D)
    yo, fo = oracle.scan(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt)
    _check(y.cpu().numpy(), fs.cpu().numpy(), yo, fo, str(case))


# The decay extremes of the complex-layout tests, read from float32 and bfloat16 in_proj
# rows (B=2, T=300 with a ragged last chunk, H=4, N=D=64, chunk 64): the memoryless
# limit (Re A = -1e4), pure rotation (Re A = 0, dt = 0), very strong decay
# (dt ~ N(4, 1)), and slow growth (Re A = +0.02, dt = 0) with the float32-attainable
# bar of a growing state: 5e-5 times the running maximum of |y| is added.
PROJ_EXTREMES = ["memoryless", "rotation", "strong", "growth"]


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("regime", PROJ_EXTREMES)
def test_proj_extreme_decay_regimes(regime, bf16):
    H, N, D = 4, 64, 64
    seed = 31 + PROJ_EXTREMES.index(regime)
    proj, A = ssd_inputs.proj_case(2, 300, H, N, D, seed=seed,
                                   dt_mean=4.0 if regime == "strong" else 0.0)
    if regime != "strong":
        re = {"memoryless": -1e4, "rotation": 0.0, "growth": 0.02}[regime]
        A = torch.complex(torch.full_like(A.real, re), A.imag)
    if regime in ("rotation", "growth"):
        proj[..., H * (D + 4 * N):H * (D + 4 * N + 1)] = 0.0
    if bf16:
        proj = proj.to(torch.bfloat16)
    y, fs = ssd.chunk_forward_proj(proj.to(DEV), A.to(DEV), H, N, D, chunk_size=64)
    torch.cuda.synchronize()
    inp = ssd_inputs.unpack_proj(proj, A, H, N, D)
    yo, fo = oracle.scan(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt)
    y, fs = y.cpu().numpy(), fs.cpu().numpy()
    what = "%s bf16=%s" % (regime, bf16)
    if regime != "growth":
        _check(y, fs, yo, fo, what)
        return
    yr = yo.real
    scale = np.maximum.accumulate(np.abs(yr).max(axis=3, keepdims=True), axis=1)
    e = np.abs(y - yr)
    assert np.isfinite(y).all() and (e <= 1e-4 + 1e-4 * np.abs(yr) + 5e-5 * scale).all(), what
    for comp in (np.real, np.imag):
        ref = comp(fo)
        top = np.abs(ref).max(axis=(2, 3), keepdims=True)
        assert (np.abs(comp(fs) - ref) <= 1e-4 + 1e-4 * np.abs(ref) + 5e-5 * top).all(), what


def test_proj_layer_b1_full():
    """One Mamba-3-Lite layer (B=1, T=2048, H=16, N=D=64, chunk 64) in the in_proj layout."""
    proj, A = ssd_inputs.proj_case(1, 2048, 16, 64, 64, seed=1, extra=2)
    y, fs = ssd.chunk_forward_proj(proj.to(DEV), A.to(DEV), 16, 64, 64, chunk_size=64)
    torch.cuda.synchronize()
    inp = ssd_inputs.unpack_proj(proj, A, 16, 64, 64)
    yo, fo = oracle.scan(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt)
    _check(y.cpu().numpy(), fs.cpu().numpy(), yo, fo, "proj layer_b1")


def test_proj_network_layer_sampled_and_complex_path():
    """The network layer shape (B=32): sampled sequences against the oracle, and
    every output against the complex-layout entry point on the unpacked inputs."""
    proj, A = ssd_inputs.proj_case(32, 2048, 16, 64, 64, seed=0, device=DEV)
    y, fs = ssd.chunk_forward_proj(proj, A, 16, 64, 64, chunk_size=64)
    inp = ssd_inputs.unpack_proj(proj, A, 16, 64, 64)
    y2, fs2 = ssd.chunk_forward(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt, chunk_size=64)
    torch.cuda.synchronize()
    a, r = y.cpu().numpy(), y2.cpu().numpy()
    assert (np.abs(a - r) <= 2e-4 + 2e-4 * np.abs(r)).all()
    pairs = [(0, 0), (31, 15), (17, 6)]
    host = inp.to("cpu")
    for b, h in pairs:
        one = host.select(b, h)
        yo, fo = oracle.scan(one.x, one.A, one.B_t, one.C_t, one.dt)
        _check(a[b:b + 1, :, h:h + 1], fs.cpu().numpy()[b:b + 1, h:h + 1], yo, fo,
               "proj network (%d, %d)" % (b, h))


def test_proj_initial_state_and_zero_length():
    B, T, H, N, D = 2, 130, 2, 16, 16
    proj, A = ssd_inputs.proj_case(B, T, H, N, D, seed=5, extra=0)
    rng = np.random.default_rng(4)
    init = ((rng.standard_normal((B, H, N, D)) + 1j * rng.standard_normal((B, H, N, D))) * 0.5
            ).astype(np.complex64)
    y, fs = ssd.chunk_forward_proj(proj.to(DEV), A.to(DEV), H, N, D, chunk_size=32,
                                   initial_state=torch.as_tensor(init).to(DEV))
    torch.cuda.synchronize()
    inp = ssd_inputs.unpack_proj(proj, A, H, N, D)
    yo, fo = oracle.scan(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt, initial_state=init)
    _check(y.cpu().numpy(), fs.cpu().numpy(), yo, fo, "proj initial state")
    empty = torch.zeros((B, 0, H * (D + 4 * N + 1)), device=DEV)
    y0, f0 = ssd.chunk_forward_proj(empty, A.to(DEV), H, N, D, chunk_size=32,
                                    initial_state=torch.as_tensor(init).to(DEV))
    torch.cuda.synchronize()
    assert y0.numel() == 0 and np.array_equal(f0.cpu().numpy(), init)


# bfloat16 rows (ssd_chunk_forward_proj_bf16): the oracle runs on the same rows
# widened to float32, so the float32 bar applies unchanged.

@pytest.mark.parametrize("case", CASES[:6])
def test_proj_bf16_small_shapes(case):
    B, T, H, N, D, Q, extra = case
    proj, A = ssd_inputs.proj_case(B, T, H, N, D, seed=sum(case) + 50, dt_mean=0.3, extra=extra,
                                   dtype=torch.bfloat16)
    y, fs = ssd.chunk_forward_proj(proj.to(DEV), A.to(DEV), H, N, D, chunk_size=Q)
    torch.cuda.synchronize()
    inp = ssd_inputs.unpack_proj(proj, A, H, N, D)
    yo, fo = oracle.scan(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt)
    _check(y.cpu().numpy(), fs.cpu().numpy(), yo, fo, "bf16 " + str(case))


def test_proj_bf16_network_layer_matches_float32_rows():
    """The network layer shape (B=32) from bfloat16 rows equals the float32 entry
    point on the widened rows (same arithmetic), and sampled sequences the oracle."""
    proj, A = ssd_inputs.proj_case(32, 2048, 16, 64, 64, seed=0, device=DEV, dtype=torch.bfloat16)
    y, fs = ssd.chunk_forward_proj(proj, A, 16, 64, 64, chunk_size=64)
    y32, fs32 = ssd.chunk_forward_proj(proj.float(), A, 16, 64, 64, chunk_size=64)
    torch.cuda.synchronize()
    a = y.cpu().numpy()
    assert np.array_equal(a, y32.cpu().numpy())
    assert np.array_equal(fs.cpu().numpy(), fs32.cpu().numpy())
    host = ssd_inputs.unpack_proj(proj.cpu(), A.cpu(), 16, 64, 64)
    for b, h in [(3, 2), (30, 13)]:
        one = host.select(b, h)
        yo, fo = oracle.scan(one.x, one.A, one.B_t, one.C_t, one.dt)
        _check(a[b:b + 1, :, h:h + 1], fs.cpu().numpy()[b:b + 1, h:h + 1], yo, fo,
               "bf16 network (%d, %d)" % (b, h))


# Gradients from in_proj rows (ssd_chunk_backward_proj): every block of the
# gradient rows against the oracle's gradients of the complex inputs the rows
# stand for, with the gradient bar (grad_A's absolute term grows 1e-6 per
# token summed); floats past the blocks stay untouched.

# bfloat16 gradient rows: the float32 result is rounded to nearest bfloat16
# (8 significant bits), which adds at most 2^-8 of the value to the float32 bar.
BF16_REL = 1e-4 + 2.0 ** -8


def _check_grad_rows(rows, gA, gi, ref, S, W, what, tokens, rel=1e-4):
    want = ssd_inputs.pack_proj_grads(ref.x, ref.B_t, ref.C_t, ref.dt, S)
    got = rows[..., :W]
    assert np.isfinite(got).all(), what
    err = np.abs(got - want[..., :W])
    bad = err > 1e-4 + rel * np.abs(want[..., :W])
    assert not bad.any(), "%s: %d violations, max %.3e" % (what, int(bad.sum()), err.max())
    assert (rows[..., W:] == 0).all(), what
    for comp in (np.real, np.imag):
        assert (np.abs(comp(gA) - comp(ref.A)) <= 1e-4 + 1e-6 * tokens
                + 1e-4 * np.abs(comp(ref.A))).all(), what
        d = np.abs(comp(gi) - comp(ref.initial_state))
        assert (d <= 1e-4 + 1e-4 * np.abs(comp(ref.initial_state))).all(), what


@pytest.mark.parametrize("case", CASES[:8] + [CASES[10]])
def test_backward_proj_small_shapes(case):
    """Includes D = 70 (two d-slices) and N = 128 (two n-slices): partial
    gradients of the state blocks summed into the gradient rows."""
    B, T, H, N, D, Q, extra = case
    proj, A = ssd_inputs.proj_case(B, T, H, N, D, seed=sum(case) + 70, dt_mean=0.3, extra=extra)
    gy, gf = ssd_inputs.upstream_grads(B, T, H, N, D, seed=sum(case))
    rows, gA, gi = ssd.chunk_backward_proj(proj.to(DEV), A.to(DEV), H, N, D, gy.to(DEV),
                                           gf.to(DEV), chunk_size=Q)
    torch.cuda.synchronize()
    inp = ssd_inputs.unpack_proj(proj, A, H, N, D)
    ref = oracle.scan_backward(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt, gy, gf)
    _check_grad_rows(rows.cpu().numpy(), gA.cpu().numpy(), gi.cpu().numpy(), ref, proj.shape[-1],
                     H * (D + 4 * N + 1), "bwd proj " + str(case), B * T)


def test_backward_proj_network_layer_sampled():
    """Network layer shape (B=32): sampled sequences' gradient rows, and the x,
    B and C blocks against the complex-layout backward on the unpacked inputs."""
    H, N, D = 16, 64, 64
    proj, A = ssd_inputs.proj_case(32, 2048, H, N, D, seed=0, device=DEV)
    gy, gf = ssd_inputs.upstream_grads(32, 2048, H, N, D, seed=0, device=DEV)
    rows, gA, gi = ssd.chunk_backward_proj(proj, A, H, N, D, gy, gf, chunk_size=64)
    inp = ssd_inputs.unpack_proj(proj, A, H, N, D)
    g = ssd.chunk_backward(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt, gy, gf, chunk_size=64)
    torch.cuda.synchronize()
    want = ssd_inputs.pack_proj_grads(g.x.cpu().numpy(), g.B_t.cpu().numpy(), g.C_t.cpu().numpy(),
                                      g.dt.cpu().numpy(), proj.shape[-1])
    r = rows.cpu().numpy()
    assert (np.abs(r - want) <= 2e-4 + 2e-4 * np.abs(want)).all()
    host, hgy, hgf = inp.to("cpu"), gy.cpu(), gf.cpu()
    for b, h in [(2, 5), (29, 14)]:
        one = host.select(b, h)
        ref = oracle.scan_backward(one.x, one.A, one.B_t, one.C_t, one.dt,
                                   hgy[b:b + 1, :, h:h + 1], hgf[b:b + 1, h:h + 1])
        want1 = ssd_inputs.pack_proj_grads(ref.x, ref.B_t, ref.C_t, ref.dt, 1 * (D + 4 * N + 1))
        got1 = np.concatenate([
            r[b, :, h * D:(h + 1) * D],
            r[b, :, H * D + h * N:H * D + (h + 1) * N],
            r[b, :, H * D + H * N + h * N:H * D + H * N + (h + 1) * N],
            r[b, :, H * D + 2 * H * N + h * N:H * D + 2 * H * N + (h + 1) * N],
            r[b, :, H * D + 3 * H * N + h * N:H * D + 3 * H * N + (h + 1) * N],
            r[b, :, H * D + 4 * H * N + h:H * D + 4 * H * N + h + 1]], axis=-1)[None]
        e = np.abs(got1 - want1)
        assert (e <= 1e-4 + 1e-4 * np.abs(want1)).all(), ((b, h), e.max())


@pytest.mark.parametrize("case", [CASES[0], CASES[1], CASES[2], CASES[5], CASES[6], CASES[7]])
def test_backward_proj_bf16_small_shapes(case):
    """bfloat16 rows in, bfloat16 gradient rows out: against the oracle run on
    the rows widened to float32, with the bfloat16 bar."""
    B, T, H, N, D, Q, extra = case
    proj, A = ssd_inputs.proj_case(B, T, H, N, D, seed=sum(case) + 90, dt_mean=0.3, extra=extra,
                                   dtype=torch.bfloat16)
    gy, gf = ssd_inputs.upstream_grads(B, T, H, N, D, seed=sum(case) + 1)
    rows, gA, gi = ssd.chunk_backward_proj(proj.to(DEV), A.to(DEV), H, N, D, gy.to(DEV),
                                           gf.to(DEV), chunk_size=Q)
    torch.cuda.synchronize()
    assert rows.dtype == torch.bfloat16
    inp = ssd_inputs.unpack_proj(proj, A, H, N, D)
    ref = oracle.scan_backward(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt, gy, gf)
    _check_grad_rows(rows.float().cpu().numpy(), gA.cpu().numpy(), gi.cpu().numpy(), ref,
                     proj.shape[-1], H * (D + 4 * N + 1), "bwd proj bf16 " + str(case), B * T,
                     rel=BF16_REL)


def test_backward_proj_bf16_network_layer_rounds_the_float32_rows():
    """Network layer shape: the bfloat16 gradient rows are the float32 path's
    gradient rows (same widened inputs) rounded to nearest bfloat16, to within
    one bfloat16 step where the two float32 results straddle a rounding boundary."""
    H, N, D = 16, 64, 64
    proj, A = ssd_inputs.proj_case(32, 2048, H, N, D, seed=0, device=DEV, dtype=torch.bfloat16)
    gy, gf = ssd_inputs.upstream_grads(32, 2048, H, N, D, seed=0, device=DEV)
    rows16, gA16, gi16 = ssd.chunk_backward_proj(proj, A, H, N, D, gy, gf, chunk_size=64)
    rows32, gA32, gi32 = ssd.chunk_backward_proj(proj.float(), A, H, N, D, gy, gf, chunk_size=64)
    torch.cuda.synchronize()
    W = H * (D + 4 * N + 1)
    a = rows16.float()[..., :W]
    r = rows32[..., :W].to(torch.bfloat16).float()
    step = torch.abs(r) * 2.0 ** -7 + 1e-30
    assert bool((torch.abs(a - r) <= step).all())
    assert float((a != r).float().mean()) < 0.01  # nearly all identical
    assert torch.equal(gA16, gA32) and torch.equal(gi16, gi32)

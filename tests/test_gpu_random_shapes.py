"""Seeded random shapes through the forward and the backward against the oracle,
at the plain bars of the other parity tests: batch, length, heads, state rows N
(even, up to 160, so one to three 64-row slices), D (up to 150), chunk sizes on
and off the tile grid (1 to 256), with and without an initial state and a
final-state gradient, from complex64 tensors and from in_proj rows (float32 and
bfloat16 rows forward, float32 rows backward, spare floats at the row end; H * D
and the token stride even, as those entry points require). Each draw is a shape that no hand-picked case names; a failure prints the shape,
which then belongs among the fixed cases.

Bars, elementwise: |y - Re y_oracle| <= 1e-4 + 1e-4 |Re y_oracle| (final state per
complex component likewise); every gradient the same per component, grad A with
1e-6 per token summed added to its absolute term. The head mixer's random shapes
(tokens, H, D) keep its own bars: 1e-4 + 1e-4 |ref| + 1e-5 sqrt(sum of squared
products) (tests/tolerances.py).
"""

import numpy as np
import pytest
import torch

import complex_chunkwise_ssd_amd as ssd
import oracle
import ssd_inputs
import tolerances

pytestmark = pytest.mark.gpu

ATOL = 1e-4
RTOL = 1e-4
DEV = torch.device("cuda:0")
CHUNKS = (1, 3, 8, 16, 17, 31, 32, 48, 64, 100, 128, 256)


def _draw(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B = int(rng.integers(1, 4))
        T = int(rng.integers(1, 301))
        H = int(rng.integers(1, 5))
        N = 2 * int(rng.integers(1, 81))
        D = int(rng.integers(1, 151))
        Q = int(rng.choice(CHUNKS))
        edges = bool(rng.integers(0, 2))
        out.append((B, T, H, N, D, Q, edges))
    return out


FORWARD = _draw(48, 2026)
BACKWARD = _draw(32, 1203)


def _proj_draw(n, seed):
    """As _draw, within the in_proj entry points' layout rules: H * D even (the
    N-blocks are read as float pairs) and an even token stride."""
    out = []
    for B, T, H, N, D, Q, flag in _draw(n, seed):
        if (H * D) % 2:
            D += 1
        out.append((B, T, H, N, D, Q, flag))
    return out


def _spare(case):
    """Unused floats at the end of each row (0 to 3), keeping the stride even."""
    B, T, H, N, D = case[:5]
    s0 = H * (D + 4 * N + 1)
    return s0 % 2 + 2 * ((B + T) % 2)


PROJ_FORWARD = _proj_draw(24, 77)
PROJ_BACKWARD = _proj_draw(16, 78)


def _close(name, got, ref, atol=ATOL):
    got = np.asarray(got)
    assert np.isfinite(got).all(), name
    comps = (np.real, np.imag) if np.iscomplexobj(ref) else (lambda v: v,)
    for comp in comps:
        e = np.abs(comp(got) - comp(ref))
        bad = e > atol + RTOL * np.abs(comp(ref))
        assert not bad.any(), "%s: %d violations, max err %.3e at %s" % (
            name, int(bad.sum()), e.max(), np.argwhere(bad)[:3].tolist())


def _edge_arrays(B, H, N, D, seed):
    rng = np.random.default_rng(seed)
    gf = (rng.standard_normal((B, H, N, D)) + 1j * rng.standard_normal((B, H, N, D))).astype(np.complex64)
    init = ((rng.standard_normal((B, H, N, D)) + 1j * rng.standard_normal((B, H, N, D))) * 0.5).astype(
        np.complex64)
    return gf, init


@pytest.mark.parametrize("case", FORWARD)
def test_random_shape_forward(case):
    B, T, H, N, D, Q, edges = case
    inp = ssd_inputs.random_case(B, T, H, N, D, seed=sum(case[:6]) + 7, dt_mean=0.3)
    _, init = _edge_arrays(B, H, N, D, sum(case[:6])) if edges else (None, None)
    g = inp.to(DEV)
    it = None if init is None else torch.as_tensor(init).to(DEV)
    y, fs = ssd.chunk_forward(g.x, g.A, g.B_t, g.C_t, g.dt, chunk_size=Q, initial_state=it)
    torch.cuda.synchronize()
    yo, fo = oracle.scan(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt, initial_state=init, threads=0)
    _close("%s y" % (case,), y.cpu().numpy(), yo.real)
    _close("%s final state" % (case,), fs.cpu().numpy(), fo)


@pytest.mark.parametrize("case", BACKWARD)
def test_random_shape_backward(case):
    B, T, H, N, D, Q, edges = case
    inp = ssd_inputs.random_case(B, T, H, N, D, seed=sum(case[:6]) + 9, dt_mean=0.3)
    gy, _ = ssd_inputs.upstream_grads(B, T, H, N, D, seed=sum(case[:6]), with_final=False)
    gf, init = _edge_arrays(B, H, N, D, sum(case[:6]) + 1) if edges else (None, None)
    g = inp.to(DEV)
    t = lambda a, dt: None if a is None else torch.as_tensor(a, dtype=dt).to(DEV)
    out = ssd.chunk_backward(g.x, g.A, g.B_t, g.C_t, g.dt, t(gy, torch.float32),
                             t(gf, torch.complex64), chunk_size=Q,
                             initial_state=t(init, torch.complex64))
    torch.cuda.synchronize()
    got = [None if v is None else v.cpu().numpy() for v in out]
    ref = oracle.scan_backward(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt, gy, gf, init)
    for name, a, r in zip(ref._fields, got, ref):
        if a is None:
            continue
        _close("%s grad %s" % (case, name), a, r, atol=ATOL + (1e-6 * B * T if name == "A" else 0.0))


@pytest.mark.parametrize("case", PROJ_FORWARD)
def test_random_shape_forward_from_proj_rows(case):
    B, T, H, N, D, Q, bf16 = case  # the draw's last flag picks bfloat16 rows here
    extra = _spare(case)
    proj, A = ssd_inputs.proj_case(B, T, H, N, D, seed=sum(case[:6]) + 11, dt_mean=0.3, extra=extra,
                                   dtype=torch.bfloat16 if bf16 else None)
    y, fs = ssd.chunk_forward_proj(proj.to(DEV), A.to(DEV), H, N, D, chunk_size=Q)
    torch.cuda.synchronize()
    inp = ssd_inputs.unpack_proj(proj, A, H, N, D)
    yo, fo = oracle.scan(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt, threads=0)
    _close("%s proj y" % (case,), y.cpu().numpy(), yo.real)
    _close("%s proj final state" % (case,), fs.cpu().numpy(), fo)


@pytest.mark.parametrize("case", PROJ_BACKWARD)
def test_random_shape_backward_from_proj_rows(case):
    B, T, H, N, D, Q, _ = case
    extra = _spare(case)
    proj, A = ssd_inputs.proj_case(B, T, H, N, D, seed=sum(case[:6]) + 13, dt_mean=0.3, extra=extra)
    gy, gf = ssd_inputs.upstream_grads(B, T, H, N, D, seed=sum(case[:6]) + 2)
    rows, gA, gi = ssd.chunk_backward_proj(proj.to(DEV), A.to(DEV), H, N, D, gy.to(DEV), gf.to(DEV),
                                           chunk_size=Q)
    torch.cuda.synchronize()
    inp = ssd_inputs.unpack_proj(proj, A, H, N, D)
    ref = oracle.scan_backward(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt, gy, gf)
    W = H * (D + 4 * N + 1)
    want = ssd_inputs.pack_proj_grads(ref.x, ref.B_t, ref.C_t, ref.dt, proj.shape[-1])
    r = rows.cpu().numpy()
    _close("%s proj grad rows" % (case,), r[..., :W], want[..., :W])
    assert (r[..., W:] == 0).all(), "%s: spare floats written" % (case,)
    _close("%s proj grad A" % (case,), gA.cpu().numpy(), ref.A, atol=ATOL + 1e-6 * B * T)
    _close("%s proj grad initial state" % (case,), gi.cpu().numpy(), ref.initial_state)


def _mix_draw(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        H = int(rng.integers(1, 17))
        D = int(rng.integers(1, 129))
        M = int(rng.integers(0, 3001))
        out.append((M, H, D))
    return out


@pytest.mark.parametrize("case", _mix_draw(16, 79))
def test_random_shape_head_mix(case):
    M, H, D = case
    y, W, gz = ssd_inputs.mix_case((M, H, D), seed=M + 7 * H + 13 * D)
    z = ssd.head_mix(y.to(DEV), W.to(DEV))
    gy, gW = ssd.head_mix_backward(y.to(DEV), W.to(DEV), gz.to(DEV))
    torch.cuda.synchronize()
    yn, Wn, gzn = y.numpy(), W.numpy(), gz.numpy()
    zo = oracle.head_mix(y, W)
    ry, rW = oracle.head_mix_backward(y, W, gz)
    for name, got, ref, extra in (("z", z, zo, tolerances.mix_forward_extra(yn, Wn)),
                                  ("grad_y", gy, ry, tolerances.mix_grad_y_extra(gzn, Wn)),
                                  ("grad_W", gW, rW, tolerances.mix_grad_w_extra(gzn, yn))):
        g = got.cpu().numpy()
        assert np.isfinite(g).all(), (case, name)
        e = np.abs(g - ref)
        assert (e <= 1e-4 + 1e-4 * np.abs(ref) + extra).all(), "%s %s max %.3e" % (case, name, e.max())

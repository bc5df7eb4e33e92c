"""Seeded synthetic inputs for the complex chunkwise SSD scan.

This module only draws random numbers. It holds none of the scan's
arithmetic, so both the HIP path and the CPU oracle can be fed from it.

Shapes and distributions follow the Mamba-3-Lite pages:
  * "Skills Reference", Skill 2 (the tiny equivalence recipe): torch seed 0,
    draw x, A (= randn - 1), B_t, C_t in that order, all complex64, dt zero.
  * "index.html", lab 01 (eigen-spectrum explorer): decay range
    alpha in [-3.0, -0.05], rotation |omega| in [0.35, 2.20].
  * "index.html", stat card: one layer is ctx 2048, chunk 64, 16 heads x 64,
    state N = 64 complex64; 28 layers.

Conventions (readings where the pages are silent):
  * "complex N(0, s^2)" means torch's complex randn (re and im each carry
    half the variance) times s.
  * Im A is a magnitude uniform in [0.35, 2.20] with an independent fair sign.
  * Draw order for the layer recipe: A (re, |im|, sign), dt, x, B_t, C_t.

Every tensor is produced by ``torch.randn``/``torch.rand`` with an explicit
``torch.Generator`` on the requested device, so a given (seed, device) pair is
reproducible. The CUDA generator's stream differs from the CPU one; parity
tests that compare against the oracle copy the very same tensors to the host.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass
class ScanInputs:
    x: torch.Tensor     # (B, T, H, D) complex64
    A: torch.Tensor     # (H,) complex64
    B_t: torch.Tensor   # (B, T, H, N) complex64
    C_t: torch.Tensor   # (B, T, H, N) complex64
    dt: torch.Tensor    # (B, T, H) float32

    @property
    def shape(self):
        b, t, h, d = self.x.shape
        return b, t, h, self.B_t.shape[-1], d

    def to(self, device) -> "ScanInputs":
        return ScanInputs(*(v.to(device) for v in (self.x, self.A, self.B_t, self.C_t, self.dt)))

    def select(self, b: int, h: int) -> "ScanInputs":
        """One (batch row, head) sequence as a B=1, H=1 problem (views copied)."""
        return ScanInputs(
            self.x[b:b + 1, :, h:h + 1].contiguous(),
            self.A[h:h + 1].contiguous(),
            self.B_t[b:b + 1, :, h:h + 1].contiguous(),
            self.C_t[b:b + 1, :, h:h + 1].contiguous(),
            self.dt[b:b + 1, :, h:h + 1].contiguous(),
        )


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def tiny_case(time_varying_dt: bool, device="cpu") -> ScanInputs:
    """B=2, T=16, H=2, D=N=4 recipe of the Skills page (seed 0).

    x, A, B_t, C_t are drawn exactly in the page's order. dt is zeros, or
    (time_varying_dt) the next randn(B, T, H) draw of the same stream.
    """
    B, T, H, D, N = 2, 16, 2, 4, 4
    g = _gen(0, "cpu")
    x = torch.randn(B, T, H, D, dtype=torch.complex64, generator=g)
    A = torch.randn(H, dtype=torch.complex64, generator=g) - 1.0
    B_t = torch.randn(B, T, H, N, dtype=torch.complex64, generator=g)
    C_t = torch.randn(B, T, H, N, dtype=torch.complex64, generator=g)
    if time_varying_dt:
        dt = torch.randn(B, T, H, generator=g)
    else:
        dt = torch.zeros(B, T, H)
    return ScanInputs(x, A, B_t, C_t, dt).to(device)


def layer_case(batch: int, T: int, H: int, N: int, D: int, seed: int,
               dt_mean: float = 0.0, device="cpu") -> ScanInputs:
    """One Mamba-3-Lite-shaped layer of scan inputs.

    A: Re ~ U[-3.0, -0.05], Im = +-U[0.35, 2.20]; dt ~ N(dt_mean, 1);
    x ~ complex N(0, 1); B_t, C_t ~ complex N(0, 1/N).
    """
    g = _gen(seed, device)
    a_re = -3.0 + 2.95 * torch.rand(H, generator=g, device=device)
    a_im = 0.35 + 1.85 * torch.rand(H, generator=g, device=device)
    sign = torch.where(torch.rand(H, generator=g, device=device) < 0.5, -1.0, 1.0)
    A = torch.complex(a_re, a_im * sign).to(torch.complex64)
    dt = torch.randn(batch, T, H, generator=g, device=device) + dt_mean
    x = torch.randn(batch, T, H, D, dtype=torch.complex64, generator=g, device=device)
    s = 1.0 / math.sqrt(N)
    B_t = torch.randn(batch, T, H, N, dtype=torch.complex64, generator=g, device=device) * s
    C_t = torch.randn(batch, T, H, N, dtype=torch.complex64, generator=g, device=device) * s
    return ScanInputs(x, A, B_t, C_t, dt)


# Named workloads. Each entry: (batch, T, H, N, D, chunk sizes, seed, dt_mean).
WORKLOADS = {
    # single Mamba-3-Lite layer, one sequence per head
    "layer_b1_t2048": dict(batch=1, T=2048, H=16, N=64, D=64, chunks=(64,), seed=1, dt_mean=0.0),
    # training-batch slice
    "layer_b8_t2048": dict(batch=8, T=2048, H=16, N=64, D=64, chunks=(64,), seed=1, dt_mean=0.0),
    # long-context chunk-size sweep; one input set shared by all four chunk sizes
    "sweep_b4_t8192": dict(batch=4, T=8192, H=16, N=64, D=64, chunks=(32, 64, 128, 256), seed=3,
                           dt_mean=0.5),
    # full 28-layer network scan load; layer l uses seed l
    "network_28x_b32_t2048": dict(batch=32, T=2048, H=16, N=64, D=64, chunks=(64,), seed=None,
                                  dt_mean=0.0, layers=28),
}


def random_case(batch, T, H, N, D, seed, device="cpu", dt_scale=1.0, dt_mean=0.0,
                a_re_range=(-3.0, -0.05)) -> ScanInputs:
    """Small irregular shapes for edge-case tests (same families as layer_case)."""
    g = _gen(seed, device)
    lo, hi = a_re_range
    a_re = lo + (hi - lo) * torch.rand(H, generator=g, device=device)
    a_im = 0.35 + 1.85 * torch.rand(H, generator=g, device=device)
    sign = torch.where(torch.rand(H, generator=g, device=device) < 0.5, -1.0, 1.0)
    A = torch.complex(a_re, a_im * sign).to(torch.complex64)
    dt = torch.randn(batch, T, H, generator=g, device=device) * dt_scale + dt_mean
    x = torch.randn(batch, T, H, D, dtype=torch.complex64, generator=g, device=device)
    s = 1.0 / math.sqrt(max(N, 1))
    B_t = torch.randn(batch, T, H, N, dtype=torch.complex64, generator=g, device=device) * s
    C_t = torch.randn(batch, T, H, N, dtype=torch.complex64, generator=g, device=device) * s
    return ScanInputs(x, A, B_t, C_t, dt)


def upstream_grads(batch, T, H, N, D, seed, device="cpu", with_final=True):
    """Seeded upstream gradients for the backward: grad_y ~ N(0, 1) (B,T,H,D)
    float32 and grad_final_state ~ complex N(0, 1) (B,H,N,D) complex64 (or None)."""
    g = _gen(seed + 7919, device)
    gy = torch.randn((batch, T, H, D), generator=g, device=device, dtype=torch.float32)
    gf = None
    if with_final:
        gf = torch.randn((batch, H, N, D), generator=g, device=device, dtype=torch.complex64)
    return gy, gf


def proj_case(batch, T, H, N, D, seed, device="cpu", dt_mean=0.0, extra=0, dtype=None):
    """One layer's scan inputs in the in_proj layout: (proj, A) with proj of shape
    (batch, T, H*(D + 4N + 1) + extra) float32, each token row
    [x | Re B | Im B | Re C | Im C | dt | extra], x ~ N(0, 1) real, every B and C
    part ~ N(0, 1/(2N)) (complex variance 1/N as in layer_case), dt ~ N(dt_mean, 1),
    A as in layer_case; the `extra` floats per row are NaN (they must never be read).
    dtype=torch.bfloat16 rounds the finished rows to bfloat16."""
    g = _gen(seed, device)
    a_re = -3.0 + 2.95 * torch.rand(H, generator=g, device=device)
    a_mag = 0.35 + 1.85 * torch.rand(H, generator=g, device=device)
    a_sgn = torch.where(torch.rand(H, generator=g, device=device) < 0.5, -1.0, 1.0)
    A = torch.complex(a_re, a_mag * a_sgn).to(torch.complex64)
    W = H * (D + 4 * N + 1)
    proj = torch.empty((batch, T, W + extra), dtype=torch.float32, device=device)
    proj[..., :H * D] = torch.randn((batch, T, H * D), generator=g, device=device)
    proj[..., H * D:H * (D + 4 * N)] = torch.randn((batch, T, 4 * H * N), generator=g,
                                                   device=device) * (0.5 / N) ** 0.5
    proj[..., H * (D + 4 * N):W] = dt_mean + torch.randn((batch, T, H), generator=g, device=device)
    if extra:
        proj[..., W:] = float("nan")
    if dtype is not None:
        proj = proj.to(dtype)
    return proj, A


def unpack_proj(proj, A, H, N, D):
    """The complex-layout ScanInputs that the in_proj rows stand for (layout
    marshalling only: x = x_real + 0i, B_t = Re B + i Im B, C_t likewise)."""
    Bsz, T = proj.shape[:2]
    proj = proj.float()  # bfloat16 rows widen exactly
    HD, HN = H * D, H * N
    x = torch.complex(proj[..., :HD], torch.zeros_like(proj[..., :HD])).reshape(Bsz, T, H, D)
    blk = lambda k: proj[..., HD + k * HN:HD + (k + 1) * HN].reshape(Bsz, T, H, N)
    B_t = torch.complex(blk(0), blk(1))
    C_t = torch.complex(blk(2), blk(3))
    dt = proj[..., HD + 4 * HN:HD + 4 * HN + H]
    return ScanInputs(x.contiguous(), A, B_t.contiguous(), C_t.contiguous(), dt.contiguous())


def pack_proj_grads(gx, gB, gC, gdt, S):
    """Gradient rows in the in_proj layout from the complex-layout gradients of the
    inputs the rows stand for (layout marshalling only): the x block takes the
    real part of x's gradient (x is real), the B and C blocks the real and
    imaginary parts, the dt block dt's gradient; floats past the blocks are 0."""
    import numpy as np
    gx, gB, gC, gdt = (np.asarray(v) for v in (gx, gB, gC, gdt))
    Bsz, T, H, D = gx.shape
    N = gB.shape[-1]
    HD, HN = H * D, H * N
    rows = np.zeros((Bsz, T, S), np.float64)
    rows[..., :HD] = gx.real.reshape(Bsz, T, HD)
    rows[..., HD:HD + HN] = gB.real.reshape(Bsz, T, HN)
    rows[..., HD + HN:HD + 2 * HN] = gB.imag.reshape(Bsz, T, HN)
    rows[..., HD + 2 * HN:HD + 3 * HN] = gC.real.reshape(Bsz, T, HN)
    rows[..., HD + 3 * HN:HD + 4 * HN] = gC.imag.reshape(Bsz, T, HN)
    rows[..., HD + 4 * HN:HD + 4 * HN + H] = gdt.reshape(Bsz, T, H)
    return rows


def mix_case(shape, seed, device="cpu", spread=0.02):
    """Inputs of the MIMO head mixer: y and the upstream gradient gz of the
    given (..., H, D) shape, standard normal float32, and the dense (F, F)
    weight W = identity + spread * N(0, 1) per entry, F = H * D (the pages start
    the mixer at the identity and let training grow the cross-head links; the
    perturbation stands in for a trained mixer). Draw order: W noise, y, gz."""
    g = _gen(seed, device)
    F = shape[-2] * shape[-1]
    W = torch.eye(F, device=device) + spread * torch.randn(F, F, generator=g, device=device)
    y = torch.randn(*shape, generator=g, device=device)
    gz = torch.randn(*shape, generator=g, device=device)
    return y, W.contiguous(), gz

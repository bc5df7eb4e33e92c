"""GPU parity of the gradients: ssd_chunk_backward, called through the C ABI,
against the oracle's reverse-mode gradients (oracle_scan_backward).

Bar (written here, applied elementwise to every gradient, per complex
component): |g_gpu - g_oracle| <= 1e-4 + 1e-4 |g_oracle| -- the forward's bar,
since each gradient is, like y, a sum of decayed products of the inputs. The
gradient of A is a sum over every token of the batch; its bar scales with the
number of tokens summed: |dgA| <= 1e-4 (1 + |gA|) + 1e-6 * B*T.
"""

import numpy as np
import pytest
import torch

import complex_chunkwise_ssd_amd as ssd
import oracle
import ssd_inputs

pytestmark = pytest.mark.gpu

ATOL = 1e-4
RTOL = 1e-4
DEV = torch.device("cuda:0")


def _close(name, got, ref, atol=ATOL):
    got = np.asarray(got)
    assert np.isfinite(got).all(), name
    comps = (np.real, np.imag) if np.iscomplexobj(ref) else (lambda v: v,)
    for comp in comps:
        e = np.abs(comp(got) - comp(ref))
        bad = e > atol + RTOL * np.abs(comp(ref))
        assert not bad.any(), "%s: %d violations, max err %.3e (max |ref| %.3e) at %s" % (
            name, int(bad.sum()), e.max(), np.abs(ref).max(), np.argwhere(bad)[:3].tolist())


def _gpu_grads(inp, Q, gy, gf=None, init=None):
    g = inp.to(DEV)
    t = lambda a, dt: None if a is None else torch.as_tensor(a, dtype=dt).to(DEV)
    out = ssd.chunk_backward(g.x, g.A, g.B_t, g.C_t, g.dt, t(gy, torch.float32),
                             t(gf, torch.complex64), chunk_size=Q,
                             initial_state=t(init, torch.complex64))
    torch.cuda.synchronize()
    return [None if v is None else v.cpu().numpy() for v in out]


def _oracle_grads(inp, gy, gf=None, init=None):
    return oracle.scan_backward(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt, gy, gf, init)


def _check_all(got, ref, what, tokens):
    for name, a, r in zip(ref._fields, got, ref):
        if name == "A":
            _close("%s grad A" % what, a, r, atol=ATOL + 1e-6 * tokens)
        elif a is not None:
            _close("%s grad %s" % (what, name), a, r)


def _edges(B, H, N, D, seed):
    rng = np.random.default_rng(seed)
    gf = (rng.standard_normal((B, H, N, D)) + 1j * rng.standard_normal((B, H, N, D))).astype(np.complex64)
    init = ((rng.standard_normal((B, H, N, D)) + 1j * rng.standard_normal((B, H, N, D))) * 0.5).astype(np.complex64)
    return gf, init


@pytest.mark.parametrize("tv", [False, True])
def test_tiny_recipe_gradients(tv):
    inp = ssd_inputs.tiny_case(tv)
    gy, _ = ssd_inputs.upstream_grads(2, 16, 2, 4, 4, seed=0, with_final=False)
    gf, init = _edges(2, 2, 4, 4, 1)
    got = _gpu_grads(inp, 4, gy, gf, init)
    _check_all(got, _oracle_grads(inp, gy, gf, init), "tiny", 32)


SMALL = [
    # B, T, H, N, D, Q
    (2, 16, 2, 4, 4, 4),
    (1, 64, 1, 64, 64, 64),
    (2, 150, 3, 64, 64, 64),
    (1, 97, 2, 8, 8, 32),
    (2, 50, 2, 6, 10, 16),
    (1, 45, 1, 10, 40, 32),
    (1, 33, 1, 2, 3, 33),
    (1, 23, 2, 4, 5, 1),
    (1, 12, 1, 4, 4, 12),
    (3, 7, 1, 2, 2, 64),
    (2, 300, 4, 32, 64, 48),
    (1, 260, 2, 64, 64, 256),
]


@pytest.mark.parametrize("edges", [False, True])
@pytest.mark.parametrize("case", SMALL)
def test_small_shapes_gradients(case, edges):
    B, T, H, N, D, Q = case
    inp = ssd_inputs.random_case(B, T, H, N, D, seed=sum(case) + 5, dt_mean=0.3)
    gy, _ = ssd_inputs.upstream_grads(B, T, H, N, D, seed=sum(case), with_final=False)
    gf, init = _edges(B, H, N, D, sum(case)) if edges else (None, None)
    got = _gpu_grads(inp, Q, gy, gf, init)
    _check_all(got, _oracle_grads(inp, gy, gf, init), str(case), B * T)


# Decay extremes (B=2, T=300 with a ragged last chunk, H=4, N=D=64, chunk 64, upstream
# gradients for y and the final state, an initial state): the memoryless limit
# (Re A = -1e4, every decay underflows), pure rotation (Re A = 0, dt = 0: nothing decays,
# so every adjoint sums the whole rest of the sequence) and very strong decay
# (dt ~ N(4, 2)). Strong decay and the memoryless limit keep the bar above; in the
# memoryless limit every decay between two tokens is an exact zero, so grad dt must be
# zero to the bit (the kernel keeps each token's pair with itself out of the decay
# gradients' row sums). One derived bar:
# * rotation: undecayed sums over ~300 tokens cancel to values far below the sequence's
#   largest, where float32 rounding of that largest value remains (a plain float32
#   reverse walk misses the plain bar here: tests/test_float32_walk_bars.py), so 5e-5
#   times the largest magnitude of that gradient over its (b, h) sequence is added.
def _close_scaled(name, got, ref, scale):
    comps = (np.real, np.imag) if np.iscomplexobj(ref) else (lambda v: v,)
    assert np.isfinite(got).all(), name
    for comp in comps:
        e = np.abs(comp(got) - comp(ref))
        bad = e > ATOL + RTOL * np.abs(comp(ref)) + scale
        assert not bad.any(), "%s: %d violations, max err %.3e" % (name, int(bad.sum()), e.max())


@pytest.mark.parametrize("regime", ["memoryless", "rotation", "strong"])
def test_backward_extreme_decay_regimes(regime):
    B, T, H, N, D = 2, 300, 4, 64, 64
    kw = dict(dt_mean=4.0, dt_scale=2.0) if regime == "strong" else {}
    inp = ssd_inputs.random_case(B, T, H, N, D, seed=51 + len(regime), **kw)
    A, dt = inp.A, inp.dt
    if regime != "strong":
        re = -1e4 if regime == "memoryless" else 0.0
        A = torch.complex(torch.full_like(A.real, re), A.imag)
    if regime == "rotation":
        dt = torch.zeros_like(dt)
    inp = ssd_inputs.ScanInputs(inp.x, A, inp.B_t, inp.C_t, dt)
    gy, _ = ssd_inputs.upstream_grads(B, T, H, N, D, seed=5, with_final=False)
    gf, init = _edges(B, H, N, D, 6)
    got = _gpu_grads(inp, 64, gy, gf, init)
    ref = _oracle_grads(inp, gy, gf, init)
    if regime == "strong":
        _check_all(got, ref, regime, B * T)
        return
    for name, a, r in zip(ref._fields, got, ref):
        if a is None:
            continue
        what = "%s grad %s" % (regime, name)
        if name == "A":
            _close(what, a, r, atol=ATOL + 1e-6 * B * T)
        elif regime == "memoryless":
            _close_scaled(what, a, r, 0.0)
            if name == "dt":
                assert np.abs(r).max() < 1e-30 and np.array_equal(a, np.zeros_like(a)), what
        else:
            seq_axes = (1,) + tuple(range(3, r.ndim)) if r.ndim >= 3 and name != "initial_state" \
                else tuple(range(2, r.ndim))
            top = np.abs(r).max(axis=seq_axes, keepdims=True)
            _close_scaled(what, a, r, 5e-5 * top)


def test_backward_long_sequence():
    """One sequence of 65,536 tokens (B=1, H=1, N=D=64): the state and adjoint passes
    walk 2,048 chunks in order and grad A adds 2,048 per-chunk shares; every gradient
    compared."""
    B, T, H, N, D = 1, 65536, 1, 64, 64
    inp = ssd_inputs.random_case(B, T, H, N, D, seed=79)
    gy, _ = ssd_inputs.upstream_grads(B, T, H, N, D, seed=80, with_final=False)
    rng = np.random.default_rng(81)
    gf = (rng.standard_normal((B, H, N, D)) + 1j * rng.standard_normal((B, H, N, D))).astype(np.complex64)
    got = _gpu_grads(inp, 64, gy, gf)
    _check_all(got, _oracle_grads(inp, gy, gf), "T=65536", B * T)


def test_layer_b1_gradients_full():
    """Single layer B=1, T=2048, H=16, N=D=64: every gradient compared."""
    w = ssd_inputs.WORKLOADS["layer_b1_t2048"]
    inp = ssd_inputs.layer_case(w["batch"], w["T"], 16, 64, 64, seed=w["seed"])
    gy, gf = ssd_inputs.upstream_grads(1, 2048, 16, 64, 64, seed=w["seed"])
    got = _gpu_grads(inp, 64, gy, gf)
    _check_all(got, _oracle_grads(inp, gy, gf), "layer_b1", 2048)


# State blocks: N or D above 64 cut the state into 64 x 64 blocks whose partial
# gradients are summed (N = 128 and D = 128 singly and together, N = 256 with a
# D sliver, ragged chunks, an initial state and a final-state gradient).
SLICED = [
    (2, 150, 3, 128, 64, 32),
    (2, 150, 3, 64, 128, 64),
    (1, 200, 2, 128, 128, 16),
    (1, 97, 2, 256, 70, 32),
]


@pytest.mark.parametrize("case", SLICED)
def test_state_blocks_above_64(case):
    B, T, H, N, D, Q = case
    print("sliced backward case", case, flush=True)
    inp = ssd_inputs.random_case(B, T, H, N, D, seed=sum(case), dt_mean=0.3)
    gy, _ = ssd_inputs.upstream_grads(B, T, H, N, D, seed=sum(case), with_final=False)
    gf, init = _edges(B, H, N, D, sum(case) + 1)
    got = _gpu_grads(inp, Q, gy.numpy(), gf, init)
    _check_all(got, _oracle_grads(inp, gy.numpy(), gf, init), "N=%d D=%d" % (N, D), B * T)


def test_state_blocks_network_shape_n128():
    """One network-shaped layer with N = 128 (B=2, T=2048, H=16): every gradient."""
    g = ssd_inputs.layer_case(2, 2048, 16, 128, 64, seed=23, device=DEV)
    gy, gf = ssd_inputs.upstream_grads(2, 2048, 16, 128, 64, seed=23, device=DEV)
    _full_grads(g, gy, gf, 64, "network shape N=128")


def _full_grads(g, gy, gf, Q, what):
    """Gradients of the device inputs g at chunk Q against the oracle on the same
    inputs (copied to the host): every component of every gradient."""
    out = ssd.chunk_backward(g.x, g.A, g.B_t, g.C_t, g.dt, gy, gf, chunk_size=Q)
    torch.cuda.synchronize()
    got = [v.cpu().numpy() for v in out]
    del out
    inp = g.to("cpu")
    ref = _oracle_grads(inp, gy.cpu().numpy(), gf.cpu().numpy())
    _check_all(got, ref, what, g.x.shape[0] * g.x.shape[1])


def test_layer_b8_gradients_full():
    """Training-batch slice B=8, T=2048, H=16, N=D=64 (seed 1): all 128 sequences."""
    w = ssd_inputs.WORKLOADS["layer_b8_t2048"]
    g = ssd_inputs.layer_case(w["batch"], w["T"], 16, 64, 64, seed=w["seed"], device=DEV)
    gy, gf = ssd_inputs.upstream_grads(8, 2048, 16, 64, 64, seed=w["seed"], device=DEV)
    _full_grads(g, gy, gf, 64, "layer_b8")


def test_network_layer_gradients_full():
    """One layer of the full-network load (B=32, T=2048, H=16, N=D=64, seed 0):
    all 512 sequences, every gradient."""
    g = ssd_inputs.layer_case(32, 2048, 16, 64, 64, seed=0, device=DEV)
    gy, gf = ssd_inputs.upstream_grads(32, 2048, 16, 64, 64, seed=0, device=DEV)
    _full_grads(g, gy, gf, 64, "network layer 0")


@pytest.mark.parametrize("Q", [16, 64])
def test_sweep_b4_t8192_gradients(Q):
    """Long context B=4, T=8192, dt ~ N(0.5, 1), evaluated in 16- and 32-token
    chunks: all 64 sequences, every gradient."""
    w = ssd_inputs.WORKLOADS["sweep_b4_t8192"]
    g = ssd_inputs.layer_case(w["batch"], w["T"], 16, 64, 64, seed=w["seed"], dt_mean=w["dt_mean"],
                              device=DEV)
    gy, gf = ssd_inputs.upstream_grads(4, 8192, 16, 64, 64, seed=w["seed"], device=DEV)
    _full_grads(g, gy, gf, Q, "sweep Q=%d" % Q)


@pytest.mark.parametrize("Q", [64, 16])
def test_fused_adjoint_walk_matches_the_three_passes(Q):
    """B=16, H=16 (256 sequences) takes the fused chunk pass, which walks the
    adjoint in shared memory; the same batch in two calls of 128 sequences takes
    the stored-adjoint passes. Same arithmetic in the same order: the per-token
    and initial-state gradients are bit-identical, grad A agrees to rounding."""
    B, T, H, N, D = 16, 300, 16, 64, 64
    inp = ssd_inputs.random_case(B, T, H, N, D, seed=95 + Q, dt_mean=0.3)
    gy, _ = ssd_inputs.upstream_grads(B, T, H, N, D, seed=96, with_final=False)
    gf, init = _edges(B, H, N, D, 97)
    whole = _gpu_grads(inp, Q, gy.numpy(), gf, init)
    halves = []
    for sl in (slice(0, 8), slice(8, 16)):
        part = ssd_inputs.ScanInputs(inp.x[sl].contiguous(), inp.A, inp.B_t[sl].contiguous(),
                                     inp.C_t[sl].contiguous(), inp.dt[sl].contiguous())
        halves.append(_gpu_grads(part, Q, gy.numpy()[sl], gf[sl], init[sl]))
    for k in (0, 2, 3, 4, 5):
        assert np.array_equal(whole[k], np.concatenate([halves[0][k], halves[1][k]], axis=0)), k
    _close("fused grad A", whole[1], halves[0][1] + halves[1][1], atol=ATOL + 1e-6 * B * T)


def test_backward_determinism_bitwise():
    inp = ssd_inputs.random_case(2, 300, 4, 64, 64, seed=77)
    gy, gf = ssd_inputs.upstream_grads(2, 300, 4, 64, 64, seed=77)
    a = _gpu_grads(inp, 64, gy.numpy(), gf.numpy())
    b = _gpu_grads(inp, 64, gy.numpy(), gf.numpy())
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_backward_chunk_size_invariance():
    inp = ssd_inputs.random_case(2, 333, 2, 64, 64, seed=81, dt_mean=0.5)
    gy, gf = ssd_inputs.upstream_grads(2, 333, 2, 64, 64, seed=81)
    ref = _gpu_grads(inp, 64, gy.numpy(), gf.numpy())
    for Q in (7, 16, 20):
        got = _gpu_grads(inp, Q, gy.numpy(), gf.numpy())
        for name, a, r in zip(ssd.Grads._fields, got, ref):
            tol = 2 * (ATOL + RTOL * np.abs(r)) + (1e-6 * 666 if name == "A" else 0)
            assert (np.abs(a - r) <= tol).all(), (Q, name)


def test_backward_zero_length():
    inp = ssd_inputs.random_case(2, 0, 3, 4, 4, seed=80)
    gf = (np.arange(2 * 3 * 4 * 4, dtype=np.float32).reshape(2, 3, 4, 4) * (1 - 0.5j)).astype(np.complex64)
    got = _gpu_grads(inp, 4, np.zeros((2, 0, 3, 4), np.float32), gf)
    assert got[0].size == 0 and np.array_equal(got[5], gf) and np.all(got[1] == 0)


def test_backward_through_initial_state_composes():
    """Gradients of run(T1) -> run(T2 | final state) chained by hand equal the
    gradients of run(T1 + T2): the second run's initial-state gradient is the
    first run's final-state gradient."""
    inp = ssd_inputs.random_case(2, 190, 2, 64, 32, seed=79)
    gy, gf = ssd_inputs.upstream_grads(2, 190, 2, 64, 32, seed=79)
    gy, gf = gy.numpy(), gf.numpy()
    whole = _gpu_grads(inp, 64, gy, gf)
    cut = 77
    a = ssd_inputs.ScanInputs(inp.x[:, :cut].contiguous(), inp.A, inp.B_t[:, :cut].contiguous(),
                              inp.C_t[:, :cut].contiguous(), inp.dt[:, :cut].contiguous())
    b = ssd_inputs.ScanInputs(inp.x[:, cut:].contiguous(), inp.A, inp.B_t[:, cut:].contiguous(),
                              inp.C_t[:, cut:].contiguous(), inp.dt[:, cut:].contiguous())
    ga_dev = a.to(DEV)
    _, fa = ssd.chunk_forward(ga_dev.x, ga_dev.A, ga_dev.B_t, ga_dev.C_t, ga_dev.dt, chunk_size=64)
    gb = _gpu_grads(b, 64, gy[:, cut:], gf, init=fa.cpu().numpy())
    ga = _gpu_grads(a, 64, gy[:, :cut], gb[5])
    _close("composed gx", np.concatenate([ga[0], gb[0]], axis=1), whole[0])
    _close("composed gdt", np.concatenate([ga[4], gb[4]], axis=1), whole[4])
    _close("composed gA", ga[1] + gb[1], whole[1], atol=ATOL + 1e-6 * 380)


@pytest.mark.parametrize("Q", [64, 10])
def test_many_sequences_full(Q):
    """256 sequences of T=300 (chunks of 32 and 10 tokens): every gradient
    compared, with a final-state gradient and an initial state."""
    B, T, H, N, D = 16, 300, 16, 64, 64
    inp = ssd_inputs.random_case(B, T, H, N, D, seed=90 + Q, dt_mean=0.3)
    gy, _ = ssd_inputs.upstream_grads(B, T, H, N, D, seed=90, with_final=False)
    gf, init = _edges(B, H, N, D, 91)
    got = _gpu_grads(inp, Q, gy.numpy(), gf, init)
    _check_all(got, _oracle_grads(inp, gy.numpy(), gf, init), "256 sequences Q=%d" % Q, B * T)

"""The unchanged kernel and C-ABI sources, run on the CPU under the host wave
emulator (tests/emu), against the oracle. This checks the kernels' lane
layouts, tiling, padding and segment logic without a GPU; the same cases run
on the GPU in test_gpu_parity.py. An AddressSanitizer build checks every
global and shared-memory access for bounds."""

import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch
import pytest

import emu_harness
import oracle
import ssd_inputs
import tolerances


@pytest.fixture(scope="module")
def emu(tmp_path_factory):
    return emu_harness.load(str(tmp_path_factory.mktemp("emu")))


def _check(y, fs, yo, fo):
    yr = yo.real
    err = np.abs(y - yr)
    assert np.isfinite(y).all()
    bad = err > 1e-4 + 1e-4 * np.abs(yr)
    assert not bad.any(), "max err %.3e at %s" % (err.max(), np.argwhere(bad)[:3])
    if fs is not None:
        ferr = np.abs(fs - fo)
        assert (ferr <= 1e-4 + 1e-4 * np.abs(fo)).all(), ferr.max()


CASES = [
    # B, T, H, N, D, Q
    (2, 16, 2, 4, 4, 4),       # the pages' tiny shape
    (1, 64, 1, 64, 64, 64),    # one full chunk
    (1, 150, 2, 64, 64, 64),   # ragged last chunk, several segments
    (1, 97, 1, 8, 8, 32),
    (2, 50, 2, 6, 10, 16),
    (1, 45, 1, 10, 70, 32),    # two D slices
    (1, 33, 1, 2, 3, 33),      # Q not a tile multiple
    (1, 23, 2, 4, 5, 1),       # Q = 1
    (1, 12, 1, 4, 4, 12),      # T == Q
    (3, 7, 1, 2, 2, 64),       # T < Q
    (1, 300, 1, 8, 8, 128),    # chunk longer than the 64-row block
    (1, 200, 1, 4, 4, 256),
    (1, 130, 1, 64, 256, 256),  # the largest D and chunk_size
    (1, 5, 1, 2, 1, 1),         # the smallest N and D
    (1, 70, 2, 66, 10, 16),     # N above 64: two slices, the second 2 rows
    (2, 37, 1, 130, 70, 32),    # three N slices and two D slices
    (1, 45, 1, 256, 8, 64),     # the largest N
    (16, 40, 16, 4, 6, 16),     # 256 sequences: each workgroup walks several chunks
    (16, 150, 16, 4, 6, 64),    # the same with 64-row blocks and a partial last chunk
]


@pytest.mark.parametrize("case", CASES)
def test_emulated_matches_oracle(emu, case):
    B, T, H, N, D, Q = case
    inp = ssd_inputs.random_case(B, T, H, N, D, seed=sum(case), dt_scale=1.0, dt_mean=0.3)
    st, y, fs = emu_harness.chunk_forward(emu, inp, Q)
    assert st == 0
    yo, fo = oracle.scan(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt)
    _check(y, fs, yo, fo)


@pytest.mark.parametrize("tv", [False, True])
def test_emulated_tiny_recipe(emu, tv):
    inp = ssd_inputs.tiny_case(tv)
    st, y, fs = emu_harness.chunk_forward(emu, inp, 4)
    assert st == 0
    yo, fo = oracle.scan(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt)
    _check(y, fs, yo, fo)


def test_emulated_initial_state(emu):
    inp = ssd_inputs.random_case(2, 70, 2, 8, 6, seed=5)
    rng = np.random.default_rng(1)
    init = (rng.standard_normal((2, 2, 8, 6)) + 1j * rng.standard_normal((2, 2, 8, 6))) * 0.5
    st, y, fs = emu_harness.chunk_forward(emu, inp, 16, initial_state=init)
    assert st == 0
    yo, fo = oracle.scan(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt,
                         initial_state=init.astype(np.complex64))
    _check(y, fs, yo, fo)


def test_emulated_zero_length(emu):
    inp = ssd_inputs.random_case(2, 0, 2, 4, 4, seed=6)
    init = np.arange(2 * 2 * 4 * 4, dtype=np.float32).reshape(2, 2, 4, 4).astype(np.complex64)
    st, y, fs = emu_harness.chunk_forward(emu, inp, 4, initial_state=init)
    assert st == 0 and y.size == 0
    assert np.array_equal(fs, init)


def test_emulated_chunk_size_invariance(emu):
    inp = ssd_inputs.random_case(1, 100, 1, 8, 8, seed=7, dt_mean=0.5)
    outs = [emu_harness.chunk_forward(emu, inp, q)[1] for q in (5, 16, 40, 64)]
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 1e-4 * (1 + np.abs(outs[0]).max())


def _build_planted_tsan(root):
    """A copy of the kernels without the barrier between phase 2 (each wave leaves
    its partial y in shared memory) and the y stores (which read the partner
    wave's part), driven by one small forward call, under ThreadSanitizer."""
    src = root / "csrc"
    shutil.copytree(emu_harness.CSRC, src)
    text = (src / "ssd_kernels.h").read_text()
    anchor = "        block_sync();\n\n        // ---- store y."
    assert text.count(anchor) == 1
    (src / "ssd_kernels.h").write_text(text.replace(anchor, "\n        // ---- store y."))
    main = root / "tsan_planted.cpp"
    main.write_text('#include "%s"\n'
                    'int main() {\n'
                    '  const int B = 1, T = 40, H = 1, N = 4, D = 6, Q = 16;\n'
                    '  static float x[B * T * H * D * 2], A[2] = {-0.5f, 1.f}, Bt[B * T * H * N * 2],\n'
                    '      Ct[B * T * H * N * 2], dt[B * T * H], y[B * T * H * D];\n'
                    '  for (int i = 0; i < B * T * H * D * 2; ++i) x[i] = 0.01f * (i %% 7);\n'
                    '  for (int i = 0; i < B * T * H * N * 2; ++i) Bt[i] = Ct[i] = 0.02f * (i %% 5);\n'
                    '  size_t ws = ssd_chunk_forward_workspace_bytes(B, T, H, N, D, Q);\n'
                    '  void *w = ws ? aligned_alloc(256, ws) : nullptr;\n'
                    '  return ssd_chunk_forward((ssd_c64 *)x, (ssd_c64 *)A, (ssd_c64 *)Bt, (ssd_c64 *)Ct, dt,\n'
                    '                           B, T, H, N, D, Q, nullptr, y, nullptr, w, ws, nullptr);\n'
                    '}\n' % (src / "ssd_api.hip"))
    exe = root / "tsan_planted"
    subprocess.run([emu_harness.CLANG, "-x", "c++", "-std=c++17", "-I" + emu_harness.EMU,
                    "-I" + str(src), "-I" + emu_harness.INCLUDE, "-O1", "-g", "-fsanitize=thread",
                    str(main), "-o", str(exe)], check=True)
    return str(exe)


def _asan_job(root):
    exe = emu_harness.build_asan_exe(str(root))
    # the case list in four parts, run side by side
    procs = [subprocess.Popen([exe, "part=%d/4" % i], stdout=subprocess.PIPE,
                              stderr=subprocess.PIPE, text=True) for i in range(4)]
    results = []
    for p in procs:
        out, err = p.communicate(timeout=900)
        results.append((p.returncode, out, err))
    return results


def _tsan_job(root):
    exe = emu_harness.build_tsan_exe(str(root))
    res = subprocess.run([exe, "races"], capture_output=True, text=True, timeout=1200)
    return res.returncode, res.stdout, res.stderr


def _planted_job(root):
    res = subprocess.run([_build_planted_tsan(root)], capture_output=True, text=True, timeout=600)
    return res.returncode, res.stdout, res.stderr


# test -> (job name, job): each job builds a sanitizer executable and runs it
SANITIZER_JOBS = {
    "test_asan_bounds": ("asan", _asan_job),
    "test_tsan_finds_no_unordered_shared_memory_access": ("tsan", _tsan_job),
    "test_tsan_reports_a_missing_barrier": ("planted", _planted_job),
}


@pytest.fixture(scope="module", autouse=True)
def sanitizer_run(request, tmp_path_factory):
    """The sanitizer jobs that this session's tests need, started side by side when
    the module's first test starts (each build and run is a process of its own,
    beside the other tests); returns job name -> its result, waiting for that job."""
    wanted = {SANITIZER_JOBS[i.name] for i in request.session.items if i.name in SANITIZER_JOBS}
    root = tmp_path_factory.mktemp("sanitizers")
    pool = ThreadPoolExecutor(max_workers=max(len(wanted), 1))
    futures = {}
    for name, job in wanted:
        (root / name).mkdir()
        futures[name] = pool.submit(job, root / name)
    yield lambda name: futures[name].result()
    pool.shutdown(wait=True)


def test_asan_bounds(sanitizer_run):
    """Every case of the bounds-check driver under AddressSanitizer (host build):
    every global and shared-memory access of the kernels and the ABI layer."""
    for rc, out, err in sanitizer_run("asan"):
        assert rc == 0, out + err
        assert "OK" in out


def test_kernel_sincos_accuracy(emu):
    """The kernels' sin/cos (Cody-Waite reduction + Taylor) against double
    precision, over the phases a scan can produce (|Im A| * softplus(dt) summed
    over a 16-token tile stays far below 2000) and beyond."""
    rng = np.random.default_rng(11)
    x = np.concatenate([
        np.linspace(-8.0, 8.0, 20001),
        rng.uniform(-2000.0, 2000.0, 200000),
        np.array([0.0, -0.0, np.pi / 4, np.pi / 2, np.pi, 1e-30, -1e-30]),
        (np.arange(-1000, 1001) * (np.pi / 2)),  # near the reduction boundaries
    ]).astype(np.float32)
    s = np.empty_like(x)
    c = np.empty_like(x)
    emu.emu_sincos(x.ctypes.data, s.ctypes.data, c.ctypes.data, x.size)
    xd = x.astype(np.float64)
    assert np.abs(s - np.sin(xd)).max() < 1.5e-7
    assert np.abs(c - np.cos(xd)).max() < 1.5e-7
    small = np.abs(xd) < 1e-3  # sin keeps its relative accuracy near zero
    assert (np.abs(s[small] - xd[small]) <= 1e-7 * np.abs(xd[small])).all()


BWD_CASES = [
    # B, T, H, N, D, Q
    (2, 16, 2, 4, 4, 4),       # the pages' tiny shape
    (1, 32, 1, 64, 64, 32),    # one full 32-row chunk
    (1, 97, 1, 64, 64, 64),    # chunks of 32 with a ragged last one
    (2, 50, 2, 6, 10, 16),
    (1, 45, 2, 10, 40, 8),
    (1, 23, 2, 4, 5, 1),       # Q = 1
    (3, 7, 1, 2, 2, 64),       # T < Q
    (1, 130, 1, 8, 8, 256),
    (2, 600, 2, 4, 4, 4),      # 600 chunks: each workgroup of the chunk pass takes several
    (16, 40, 16, 4, 6, 8),     # 256 sequences, 1280 chunks over 256 workgroups
    (32, 70, 8, 8, 4, 32),     # the same with 32-row chunks and a ragged last one
    (1, 40, 1, 130, 70, 16),   # N, D above 64: 3 x 2 state blocks, partial gradients summed
    (2, 37, 2, 66, 130, 32),   # 2 x 3 blocks with two-row and two-column slivers
]


def _check_grads(got, ref):
    for name, a, r in zip(ref._fields, got, ref):
        a = np.asarray(a)
        assert np.isfinite(a).all(), name
        err = np.abs(a - r)
        bad = err > 1e-4 + 1e-4 * np.abs(r)
        assert not bad.any(), "%s: max err %.3e at %s" % (name, err.max(), np.argwhere(bad)[:3])


@pytest.mark.parametrize("case", BWD_CASES)
@pytest.mark.parametrize("edges", ["none", "both"])
def test_emulated_backward_matches_oracle(emu, case, edges):
    B, T, H, N, D, Q = case
    inp = ssd_inputs.random_case(B, T, H, N, D, seed=sum(case) + 1, dt_scale=1.0, dt_mean=0.3)
    rng = np.random.default_rng(sum(case))
    gy = rng.standard_normal((B, T, H, D)).astype(np.float32)
    gf = init = None
    if edges == "both":
        gf = (rng.standard_normal((B, H, N, D)) + 1j * rng.standard_normal((B, H, N, D))).astype(np.complex64)
        init = ((rng.standard_normal((B, H, N, D)) + 1j * rng.standard_normal((B, H, N, D))) * 0.5).astype(np.complex64)
    st, *got = emu_harness.chunk_backward(emu, inp, Q, gy, gf, init)
    assert st == 0
    ref = oracle.scan_backward(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt, gy, gf, init)
    _check_grads(got, ref)


def _run_all_kernels(emu):
    """Outputs of a forward walking several chunks per workgroup, a segmented
    forward (prefix and fix-up passes), a backward whose chunk pass takes several
    chunks per workgroup, and the mixer's three products."""
    out = []
    for B, T, H, N, D, Q, seed in ((16, 40, 16, 4, 6, 16, 1), (1, 130, 1, 8, 8, 16, 2)):
        inp = ssd_inputs.random_case(B, T, H, N, D, seed=seed + 60)
        st, y, fs = emu_harness.chunk_forward(emu, inp, Q)
        assert st == 0
        out += [y, fs]
    inp = ssd_inputs.random_case(2, 600, 2, 4, 4, seed=63)
    gy = np.random.default_rng(63).standard_normal((2, 600, 2, 4)).astype(np.float32)
    st, *g = emu_harness.chunk_backward(emu, inp, 4, gy)
    assert st == 0
    out += g
    # 256 sequences: the fused chunk pass walks the adjoint in shared memory
    inp = ssd_inputs.random_case(16, 40, 16, 4, 6, seed=65)
    rng = np.random.default_rng(65)
    gy = rng.standard_normal((16, 40, 16, 6)).astype(np.float32)
    gf = (rng.standard_normal((16, 16, 4, 6)) + 1j * rng.standard_normal((16, 16, 4, 6))).astype(
        np.complex64)
    st, *g = emu_harness.chunk_backward(emu, inp, 16, gy, gf)
    assert st == 0
    out += g
    y, W, gz = ssd_inputs.mix_case((300, 4, 80), seed=64)
    st, z = emu_harness.head_mix(emu, y.numpy(), W.numpy())
    st2, gyy, gW = emu_harness.head_mix_backward(emu, y.numpy(), W.numpy(), gz.numpy())
    assert st == 0 and st2 == 0
    return out + [z, gyy, gW]


def test_emulated_results_do_not_depend_on_thread_order(emu):
    """Race check: the threads between sync points run in shuffled orders (two
    seeds); without a missing barrier every output stays bit-identical."""
    base = _run_all_kernels(emu)
    try:
        for seed in (0x9E3779B97F4A7C15, 12345):
            emu.emu_set_shuffle_seed(seed)
            got = _run_all_kernels(emu)
            for k, (a, b) in enumerate(zip(base, got)):
                assert np.array_equal(a, b, equal_nan=True), "output %d differs under seed %d" % (
                    k, seed)
    finally:
        emu.emu_set_shuffle_seed(0)


def test_shuffled_order_catches_a_missing_barrier(tmp_path):
    """The race check itself: a copy of the scan kernel without the barrier
    between phase 2 (each wave leaves its partial y for its partner in shared
    memory) and the y stores (which read the partner's part) gives different
    results under different thread orders."""
    import ctypes
    import shutil
    src = tmp_path / "csrc"
    shutil.copytree(emu_harness.CSRC, src)
    text = (src / "ssd_kernels.h").read_text()
    anchor = "        block_sync();\n\n        // ---- store y."
    assert text.count(anchor) == 1
    (src / "ssd_kernels.h").write_text(text.replace(anchor, "\n        // ---- store y."))
    main = tmp_path / "emu_planted.cpp"
    main.write_text('#include "%s"\n'
                    'extern "C" void emu_set_shuffle_seed(unsigned long long s) { emu::g_shuffle = s; }\n'
                    % (src / "ssd_api.hip"))
    so = tmp_path / "libplanted.so"
    subprocess.run([emu_harness.CLANG, "-x", "c++", "-std=c++17", "-I" + emu_harness.EMU,
                    "-I" + str(src), "-I" + emu_harness.INCLUDE, "-O1", "-fPIC", "-shared",
                    str(main), "-o", str(so)], check=True)
    lib = ctypes.CDLL(str(so))
    lib.emu_set_shuffle_seed.argtypes = [ctypes.c_ulonglong]
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.ssd_chunk_forward.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, i64, p, p, p, p,
                                      ctypes.c_size_t, p]
    lib.ssd_chunk_forward_workspace_bytes.argtypes = [i64] * 6
    lib.ssd_chunk_forward_workspace_bytes.restype = ctypes.c_size_t
    inp = ssd_inputs.random_case(16, 40, 16, 4, 6, seed=61)
    outs = []
    for seed in (0, 0x9E3779B97F4A7C15, 12345):
        lib.emu_set_shuffle_seed(seed)
        st, y, _ = emu_harness.chunk_forward(lib, inp, 16)
        assert st == 0
        outs.append(y)
    assert not (np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])), \
        "the shuffled order did not expose the missing barrier"


def test_tsan_finds_no_unordered_shared_memory_access(sanitizer_run):
    """The kernels under ThreadSanitizer (host build): every GPU thread is a
    sanitizer fiber, ordered only by barriers, its wave's collectives and the
    launches, so any pair of accesses to one word of shared or global memory by
    two threads with no barrier between them, one a write, is reported. Cases:
    workgroups that stage the next chunk behind the current one, segments with
    their prefix and fix-up passes, N and D slices, the fused adjoint walk (its
    deferred decay gradients and two-slot per-chunk values), the three-pass
    backward, state blocks, and the mixer's two-stage GEMM."""
    rc, stdout, stderr = sanitizer_run("tsan")
    out = stdout + stderr
    assert "WARNING: ThreadSanitizer" not in out, out[:6000]
    assert rc == 0 and "OK" in stdout, out[-3000:]


def test_tsan_reports_a_missing_barrier(sanitizer_run):
    """The check itself: a copy of the scan kernel without the barrier between
    phase 2 and the y stores is reported as a race."""
    rc, stdout, stderr = sanitizer_run("planted")
    out = stdout + stderr
    assert "WARNING: ThreadSanitizer: data race" in out, out[-3000:]
    assert "scan_kernel" in out, out[-3000:]


def test_emulated_noalloc_matches_workspace_call(emu):
    """ssd_chunk_forward_noalloc takes its workspace from the static scratch
    array: two calls (segments, then a smaller case) equal ssd_chunk_forward."""
    for B, T, H, N, D, Q, seed in ((1, 130, 1, 8, 8, 16, 1), (1, 45, 2, 6, 10, 8, 2)):
        inp = ssd_inputs.random_case(B, T, H, N, D, seed=seed + 40)
        assert emu.ssd_chunk_forward_workspace_bytes(B, T, H, N, D, Q) > 0
        x, A, Bm, Cm = (np.ascontiguousarray(v.numpy()) for v in (inp.x, inp.A, inp.B_t, inp.C_t))
        dt = np.ascontiguousarray(inp.dt.numpy())
        y = np.full((B, T, H, D), np.nan, np.float32)
        fs = np.full((B, H, N, D), np.nan, np.complex64)
        st = emu.ssd_chunk_forward_noalloc(x.ctypes.data, A.ctypes.data, Bm.ctypes.data,
                                           Cm.ctypes.data, dt.ctypes.data, B, T, H, N, D, Q, None,
                                           y.ctypes.data, fs.ctypes.data, None)
        assert st == 0
        st, y2, fs2 = emu_harness.chunk_forward(emu, inp, Q)
        assert st == 0 and np.array_equal(y, y2) and np.array_equal(fs, fs2)


@pytest.mark.parametrize("Q", [8, 32])
def test_emulated_fused_adjoint_walk_matches_the_three_passes(emu, Q):
    """256 sequences take the fused chunk pass (the adjoint walked in shared
    memory); the same batch split into two calls of 128 sequences takes the
    stored-adjoint passes. Same arithmetic in the same order: every per-token
    and initial-state gradient is bit-identical; grad A (summed over the batch)
    agrees to rounding."""
    B, T, H, N, D = 16, 45, 16, 4, 6
    inp = ssd_inputs.random_case(B, T, H, N, D, seed=71 + Q, dt_mean=0.3)
    rng = np.random.default_rng(72)
    gy = rng.standard_normal((B, T, H, D)).astype(np.float32)
    gf = (rng.standard_normal((B, H, N, D)) + 1j * rng.standard_normal((B, H, N, D))).astype(np.complex64)
    st, *whole = emu_harness.chunk_backward(emu, inp, Q, gy, gf)
    assert st == 0
    halves = []
    for sl in (slice(0, 8), slice(8, 16)):
        part = ssd_inputs.ScanInputs(inp.x[sl].contiguous(), inp.A, inp.B_t[sl].contiguous(),
                                     inp.C_t[sl].contiguous(), inp.dt[sl].contiguous())
        st, *g = emu_harness.chunk_backward(emu, part, Q, gy[sl], gf[sl])
        assert st == 0
        halves.append(g)
    for k in (0, 2, 3, 4, 5):  # gx, gB, gC, gdt, g_init
        assert np.array_equal(whole[k], np.concatenate([halves[0][k], halves[1][k]], axis=0)), k
    assert np.allclose(whole[1], halves[0][1] + halves[1][1], rtol=1e-5, atol=1e-4)


def test_emulated_backward_memoryless_limit_is_exact(emu):
    """Re A = -1e4: every decay between two tokens underflows to zero, so dF/da
    is a sum of exact zeros and grad dt must be zero to the bit (grad dt scales
    dF/da by |A| = 1e4, so any leftover of a token's pair with itself would show).
    The other gradients keep the plain bar."""
    B, T, H, N, D, Q = 1, 70, 2, 64, 64, 64
    inp = ssd_inputs.random_case(B, T, H, N, D, seed=91)
    A = torch.complex(torch.full_like(inp.A.real, -1e4), inp.A.imag)
    inp = ssd_inputs.ScanInputs(inp.x, A, inp.B_t, inp.C_t, inp.dt)
    rng = np.random.default_rng(92)
    gy = rng.standard_normal((B, T, H, D)).astype(np.float32)
    st, *got = emu_harness.chunk_backward(emu, inp, Q, gy)
    assert st == 0
    ref = oracle.scan_backward(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt, gy)
    assert np.abs(ref.dt).max() < 1e-30
    assert np.array_equal(got[4], np.zeros_like(got[4]))
    _check_grads(got, ref)


def test_emulated_backward_zero_length(emu):
    inp = ssd_inputs.random_case(2, 0, 2, 4, 4, seed=6)
    rng = np.random.default_rng(2)
    gf = (rng.standard_normal((2, 2, 4, 4)) + 1j * rng.standard_normal((2, 2, 4, 4))).astype(np.complex64)
    st, gx, gA, gB, gC, gdt, gi = emu_harness.chunk_backward(
        emu, inp, 4, np.zeros((2, 0, 2, 4), np.float32), gf)
    assert st == 0 and gx.size == 0
    assert np.array_equal(gi, gf) and np.all(gA == 0)


PROJ_CASES = [
    # B, T, H, N, D, Q, extra floats per row (NaN: must never be read; the row
    # length must be even)
    (1, 60, 2, 128, 8, 16, 2),     # two N slices from in_proj rows
    (2, 16, 2, 4, 4, 4, 0),
    (1, 97, 2, 8, 6, 32, 6),
    (1, 150, 1, 64, 64, 64, 1),    # several segments
    (2, 45, 2, 10, 70, 16, 4),     # two D slices
    (1, 300, 1, 8, 8, 128, 1),
    (16, 150, 16, 4, 6, 64, 2),    # 256 sequences, several chunks per workgroup
]


@pytest.mark.parametrize("case", PROJ_CASES)
def test_emulated_proj_layout_matches_oracle(emu, case):
    B, T, H, N, D, Q, extra = case
    proj, A = ssd_inputs.proj_case(B, T, H, N, D, seed=sum(case), dt_mean=0.3, extra=extra)
    st, y, fs = emu_harness.chunk_forward_proj(emu, proj, A, H, N, D, Q)
    assert st == 0
    inp = ssd_inputs.unpack_proj(proj, A, H, N, D)
    yo, fo = oracle.scan(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt)
    _check(y, fs, yo, fo)


@pytest.mark.parametrize("case", PROJ_CASES[:3])
def test_emulated_proj_bf16_matches_oracle(emu, case):
    """bfloat16 rows: the oracle runs on the same rows widened to float32."""
    import torch
    B, T, H, N, D, Q, extra = case
    proj, A = ssd_inputs.proj_case(B, T, H, N, D, seed=sum(case) + 3, dt_mean=0.3, extra=extra,
                                   dtype=torch.bfloat16)
    st, y, fs = emu_harness.chunk_forward_proj(emu, proj, A, H, N, D, Q)
    assert st == 0
    inp = ssd_inputs.unpack_proj(proj, A, H, N, D)
    yo, fo = oracle.scan(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt)
    _check(y, fs, yo, fo)


@pytest.mark.parametrize("case", [(2, 16, 2, 4, 4, 4, 0), (1, 97, 2, 8, 6, 32, 6),
                                  (2, 50, 2, 6, 10, 16, 4), (1, 40, 2, 130, 70, 16, 2),
                                  (16, 37, 16, 4, 6, 32, 1)])  # 256 sequences: the fused walk
def test_emulated_backward_proj_matches_oracle(emu, case):
    """Gradient rows of the in_proj layout: every block against the oracle's
    gradients of the complex inputs the rows stand for; floats past the blocks
    are not written."""
    B, T, H, N, D, Q, extra = case
    proj, A = ssd_inputs.proj_case(B, T, H, N, D, seed=sum(case) + 9, dt_mean=0.3, extra=extra)
    rng = np.random.default_rng(sum(case))
    gy = rng.standard_normal((B, T, H, D)).astype(np.float32)
    gf = (rng.standard_normal((B, H, N, D)) + 1j * rng.standard_normal((B, H, N, D))).astype(np.complex64)
    st, rows, gA, gi, W = emu_harness.chunk_backward_proj(emu, proj, A, H, N, D, Q, gy, gf)
    assert st == 0
    inp = ssd_inputs.unpack_proj(proj, A, H, N, D)
    ref = oracle.scan_backward(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt, gy, gf)
    want = ssd_inputs.pack_proj_grads(ref.x, ref.B_t, ref.C_t, ref.dt, proj.shape[-1])
    got = rows[..., :W]
    assert np.isfinite(got).all()
    err = np.abs(got - want[..., :W])
    assert (err <= 1e-4 + 1e-4 * np.abs(want[..., :W])).all(), err.max()
    assert np.isnan(rows[..., W:]).all()
    assert (np.abs(gA - ref.A) <= 1e-4 + 1e-6 * B * T + 1e-4 * np.abs(ref.A)).all()
    assert (np.abs(gi - ref.initial_state) <= 1e-4 + 1e-4 * np.abs(ref.initial_state)).all()


MIX_CASES = [
    # tokens shape, H, D, float offset (1 = off 16-byte alignment)
    ((5,), 16, 64, 0),      # the pages' 16 heads of 64: F = 1024, four column tiles
    ((2, 3), 7, 10, 0),     # F = 70, not a multiple of 4: scalar loads
    ((300,), 4, 80, 0),     # two row and two column tiles, both ragged
    ((1,), 1, 1, 0),
    ((4,), 4, 16, 1),       # misaligned rows take the scalar loads
]


@pytest.mark.parametrize("case", MIX_CASES)
def test_emulated_head_mix_matches_oracle(emu, case):
    lead, H, D, off = case
    y, W, gz = ssd_inputs.mix_case(lead + (H, D), seed=H * 100 + D)
    st, z = emu_harness.head_mix(emu, y.numpy(), W.numpy(), offset=off)
    assert st == 0
    ref = oracle.head_mix(y, W)
    assert np.isfinite(z).all()
    err = np.abs(z - ref)
    tol = 1e-4 + 1e-4 * np.abs(ref) + tolerances.mix_forward_extra(y.numpy(), W.numpy())
    assert (err <= tol).all(), err.max()


@pytest.mark.parametrize("case", MIX_CASES[1:3] + [((2100,), 2, 4, 0), ((40,), 8, 34, 0)])
def test_emulated_head_mix_backward_matches_oracle(emu, case):
    """(2100,) x 8 channels cuts the token sum into three splits; (40,) x 272
    channels has ragged row and column tiles in both products."""
    lead, H, D, _ = case
    y, W, gz = ssd_inputs.mix_case(lead + (H, D), seed=H * 100 + D + 1)
    st, gy, gW = emu_harness.head_mix_backward(emu, y.numpy(), W.numpy(), gz.numpy())
    assert st == 0
    ry, rW = oracle.head_mix_backward(y, W, gz)
    assert np.isfinite(gy).all() and np.isfinite(gW).all()
    ty = 1e-4 + 1e-4 * np.abs(ry) + tolerances.mix_grad_y_extra(gz.numpy(), W.numpy())
    assert (np.abs(gy - ry) <= ty).all()
    tw = 1e-4 * (1 + np.abs(rW)) + tolerances.mix_grad_w_extra(gz.numpy(), y.numpy())
    assert (np.abs(gW - rW) <= tw).all(), np.abs(gW - rW).max()


def test_emulated_head_mix_zero_tokens(emu):
    y = np.zeros((0, 4, 8), np.float32)
    W = np.eye(32, dtype=np.float32)
    st, z = emu_harness.head_mix(emu, y, W)
    assert st == 0 and z.shape == (0, 4, 8)
    st, gy, gW = emu_harness.head_mix_backward(emu, y, W, y)
    assert st == 0 and np.array_equal(gW, np.zeros((32, 32), np.float32))


@pytest.mark.parametrize("case", [(2, 16, 2, 4, 4, 4, 0), (1, 97, 2, 8, 6, 32, 6)])
def test_emulated_backward_proj_bf16_matches_oracle(emu, case):
    """bfloat16 rows and gradient rows: the oracle runs on the widened rows; the
    bar adds the bfloat16 rounding of the result (2^-8 of it)."""
    import torch
    B, T, H, N, D, Q, extra = case
    proj, A = ssd_inputs.proj_case(B, T, H, N, D, seed=sum(case) + 19, dt_mean=0.3, extra=extra,
                                   dtype=torch.bfloat16)
    rng = np.random.default_rng(sum(case) + 1)
    gy = rng.standard_normal((B, T, H, D)).astype(np.float32)
    gf = (rng.standard_normal((B, H, N, D)) + 1j * rng.standard_normal((B, H, N, D))).astype(np.complex64)
    st, rows, gA, gi, W = emu_harness.chunk_backward_proj(emu, proj, A, H, N, D, Q, gy, gf)
    assert st == 0
    inp = ssd_inputs.unpack_proj(proj, A, H, N, D)
    ref = oracle.scan_backward(inp.x, inp.A, inp.B_t, inp.C_t, inp.dt, gy, gf)
    want = ssd_inputs.pack_proj_grads(ref.x, ref.B_t, ref.C_t, ref.dt, proj.shape[-1])
    got = rows[..., :W]
    assert np.isfinite(got).all()
    err = np.abs(got - want[..., :W])
    assert (err <= 1e-4 + (1e-4 + 2.0 ** -8) * np.abs(want[..., :W])).all(), err.max()
    assert np.isnan(rows[..., W:]).all()
    assert (np.abs(gA - ref.A) <= 1e-4 + 1e-6 * B * T + 1e-4 * np.abs(ref.A)).all()

// ssd_device.h (host emulation) -- TEST INFRASTRUCTURE.
//
// Provides the same primitives as the gfx950 header of the same name, but for
// a plain x86-64 host build, so that the unchanged kernel and C-ABI sources can
// run on the CPU. Each GPU thread is a fiber; a wave64's lanes meet at every
// MFMA and shuffle, all threads of a workgroup meet at every barrier, and the
// collective is evaluated once every participant has arrived. Workgroups run
// one after another. A sync point that not every participant reaches (a
// divergent MFMA, shuffle or barrier) is reported as a deadlock and aborts.
//
// Race check: by default the threads between two sync points run in index
// order. With a nonzero shuffle seed (emu_set_shuffle_seed) every scheduling
// round runs them in a fresh pseudo-random order instead. Each thread's own
// arithmetic does not depend on that order, so a kernel whose waves only meet
// in shared memory across barriers gives bit-identical results under every
// seed; a missing barrier (one wave reading or overwriting shared memory that
// another wave writes or reads in the same interval) makes the result depend
// on the order and shows as a difference between seeds.
//
// Under ThreadSanitizer (a -fsanitize=thread host build) every wave is one
// sanitizer fiber (its lanes run in lockstep on the GPU, so their accesses are
// in program order), switched to without implied ordering, and the only
// happens-before edges between waves are the GPU's own: a workgroup barrier
// orders every access of the workgroup before it against every access after it,
// and launches and workgroups are ordered one after another. Two accesses to the
// same word of shared (or global) memory by different waves with no barrier
// between them, one of them a write, are reported as a race, whatever order the
// fibers happened to run in. Each ordering token alternates between two slots by
// generation, so that a wave resuming late cannot pick up releases that faster
// waves made after the point it is synchronising on.
//
// MFMA 16x16x4 fp32 data layout emulated here (one wave64):
//   lane L supplies A[L % 16][L / 16] and B[L / 16][L % 16];
//   component r of lane L's accumulator is D[4 * (L / 16) + r][L % 16].
#pragma once

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <functional>

#if defined(__has_feature)
#if __has_feature(address_sanitizer)
#define EMU_ASAN 1
#endif
#endif
#ifdef EMU_ASAN
#include <sanitizer/common_interface_defs.h>
#endif
#if defined(__has_feature)
#if __has_feature(thread_sanitizer)
#define EMU_TSAN 1
#endif
#elif defined(__SANITIZE_THREAD__)
#define EMU_TSAN 1
#endif
#ifdef EMU_TSAN
#include <sanitizer/tsan_interface.h>
extern "C" void AnnotateBenignRaceSized(const char *file, int line, const volatile void *mem,
                                        size_t size, const char *desc);
#define EMU_TSAN_BENIGN(p, n) AnnotateBenignRaceSized(__FILE__, __LINE__, (p), (n), "emulator state")
#endif

typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

#define SSD_DEVICE static inline
#define SSD_KERNEL(threads)
#define SSD_KERNEL_WAVES(threads, waves)
#define SSD_LDS static __attribute__((aligned(16)))

// Base-2 exponential and logarithm (the gfx950 header uses v_exp_f32 / v_log_f32).
SSD_DEVICE float hw_exp2(float x) { return exp2f(x); }
SSD_DEVICE float hw_log2(float x) { return log2f(x); }

// ---------------------------------------------------------------- HIP host API
typedef void *hipStream_t;
typedef int hipError_t;
#define hipSuccess 0
struct dim3 {
    unsigned x, y, z;
    dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {}
};

namespace emu {

enum { RUN = 0, AT_MFMA, AT_BARRIER, AT_SHFL, DONE };
enum { SH_SHR = 0, SH_SHL, SH_READ, SH_IDX };

struct Fiber {
    void *sp;
    char *stack;
    int state;
    // MFMA operands / result
    float a, b;
    v4f c, d;
    // shuffle operands / result
    int mode, arg;
    float sv, sr;
    long sync_count;  // number of collectives this thread has joined
#ifdef EMU_TSAN
    int bars;         // workgroup barriers passed in this workgroup
#endif
};

static const size_t kStack = 256 * 1024;
static Fiber *g_f = nullptr;
static int g_cap = 0;
static int g_n = 0;
static int g_cur = -1;
static int64_t g_block = 0;
static int64_t g_grid = 0;
static void *g_sched_sp = nullptr;
static std::function<void()> *g_fn = nullptr;
static long g_mfma_count = 0;
static unsigned long long g_shuffle = 0;  // 0: index order; else the state of a xorshift64
static int *g_order = nullptr;
static int g_order_cap = 0;
static int g_error = 0;
#ifdef EMU_TSAN
static void *g_sched_tsan = nullptr;
static void *g_wave_tsan[16];  // this workgroup's waves
static char g_tok_block[2];    // workgroup k releases slot k % 2 and acquires the other
static char g_tok_bar[2];      // barrier generation g: slot g % 2
#endif
#ifdef EMU_ASAN
static void *g_fake_stack = nullptr;
static const void *g_sched_bottom = nullptr;
static size_t g_sched_size = 0;
#endif

extern "C" void emu_swap(void **save_sp, void *load_sp);
__asm__(".text\n"
        ".globl emu_swap\n"
        ".type emu_swap,@function\n"
        "emu_swap:\n"
        "  pushq %rbp\n  pushq %rbx\n  pushq %r12\n  pushq %r13\n  pushq %r14\n  pushq %r15\n"
        "  movq %rsp, (%rdi)\n"
        "  movq %rsi, %rsp\n"
        "  popq %r15\n  popq %r14\n  popq %r13\n  popq %r12\n  popq %rbx\n  popq %rbp\n"
        "  ret\n");

static void to_scheduler()
{
    Fiber &f = g_f[g_cur];
#ifdef EMU_TSAN
    __tsan_switch_to_fiber(g_sched_tsan, __tsan_switch_to_fiber_no_sync);
#endif
#ifdef EMU_ASAN
    void *fake = nullptr;
    __sanitizer_start_switch_fiber(f.state == DONE ? nullptr : &fake, g_sched_bottom, g_sched_size);
#endif
    emu_swap(&f.sp, g_sched_sp);
#ifdef EMU_ASAN
    __sanitizer_finish_switch_fiber(fake, nullptr, nullptr);
#endif
}

static void trampoline()
{
#ifdef EMU_ASAN
    __sanitizer_finish_switch_fiber(nullptr, &g_sched_bottom, &g_sched_size);
#endif
#ifdef EMU_TSAN
    __tsan_acquire(&g_tok_block[(g_block & 1) ^ 1]);
#endif
    (*g_fn)();
#ifdef EMU_TSAN
    __tsan_release(&g_tok_block[g_block & 1]);
#endif
    g_f[g_cur].state = DONE;
    to_scheduler();
    abort();  // never resumed
}

static void run_fiber(int i)
{
    g_cur = i;
#ifdef EMU_TSAN
    __tsan_switch_to_fiber(g_wave_tsan[i >> 6], __tsan_switch_to_fiber_no_sync);
#endif
#ifdef EMU_ASAN
    __sanitizer_start_switch_fiber(&g_fake_stack, g_f[i].stack, kStack);
#endif
    emu_swap(&g_sched_sp, g_f[i].sp);
#ifdef EMU_ASAN
    __sanitizer_finish_switch_fiber(g_fake_stack, &g_sched_bottom, &g_sched_size);
#endif
}

static void init_fiber(int i)
{
    Fiber &f = g_f[i];
    uintptr_t top = ((uintptr_t)f.stack + kStack) & ~(uintptr_t)15;
    uint64_t *sp = (uint64_t *)top;
    *--sp = 0;                          // fake return address of the trampoline
    *--sp = (uint64_t)(void *)&trampoline;
    for (int k = 0; k < 6; ++k)
        *--sp = 0;                      // rbp rbx r12 r13 r14 r15
    f.sp = sp;
    f.state = RUN;
    f.sync_count = 0;
#ifdef EMU_TSAN
    f.bars = 0;
    if ((i & 63) == 0)
        g_wave_tsan[i >> 6] = __tsan_create_fiber(0);
#endif
}

static void resolve_wave(int w, bool &progress)
{
    const int lo = 64 * w;
    if (lo + 64 > g_n)
        return;
    const int st = g_f[lo].state;
    if (st != AT_MFMA && st != AT_SHFL)
        return;
    for (int l = 0; l < 64; ++l)
        if (g_f[lo + l].state != st)
            return;
    if (st == AT_MFMA) {
        for (int i = 0; i < 16; ++i)
            for (int j = 0; j < 16; ++j) {
                Fiber &out = g_f[lo + j + 16 * (i / 4)];
                float acc = out.c[i % 4];
                for (int k = 0; k < 4; ++k)
                    acc += g_f[lo + i + 16 * k].a * g_f[lo + j + 16 * k].b;
                out.d[i % 4] = acc;
            }
        ++g_mfma_count;
    } else {
        const int mode = g_f[lo].mode;
        for (int l = 0; l < 64; ++l)
            if (g_f[lo + l].mode != mode) {
                fprintf(stderr, "emu: mixed shuffle kinds in wave %d\n", w);
                abort();
            }
        for (int l = 0; l < 64; ++l) {
            Fiber &f = g_f[lo + l];
            int src = l;
            bool zero = false;
            if (mode == SH_SHR) {
                zero = (l & 15) < f.arg;
                src = l - f.arg;
            } else if (mode == SH_SHL) {
                zero = (l & 15) + f.arg >= 16;
                src = l + f.arg;
            } else if (mode == SH_IDX) {
                src = f.arg & 63;
            } else {
                if (f.arg != g_f[lo].arg) {
                    fprintf(stderr, "emu: lane_read with a non-uniform source lane\n");
                    abort();
                }
                src = f.arg & 63;
            }
            f.sr = zero ? 0.f : g_f[lo + src].sv;
        }
    }
    for (int l = 0; l < 64; ++l)
        g_f[lo + l].state = RUN;
    progress = true;
}

static void launch(dim3 grid, dim3 block, std::function<void()> fn)
{
    const int n = (int)(block.x * block.y * block.z);
    if (n > g_cap) {
        for (int i = 0; i < g_cap; ++i)
            free(g_f[i].stack);
        free(g_f);
        g_f = (Fiber *)calloc((size_t)n, sizeof(Fiber));
        for (int i = 0; i < n; ++i)
            g_f[i].stack = (char *)aligned_alloc(64, kStack);
        g_cap = n;
#ifdef EMU_TSAN
        EMU_TSAN_BENIGN(g_f, (size_t)n * sizeof(Fiber));
#endif
    }
#ifdef EMU_TSAN
    // the scheduler's bookkeeping, read by every thread (thread and block ids)
    EMU_TSAN_BENIGN(&g_cur, sizeof(g_cur));
    EMU_TSAN_BENIGN(&g_block, sizeof(g_block));
    EMU_TSAN_BENIGN(&g_grid, sizeof(g_grid));
    EMU_TSAN_BENIGN(&g_fn, sizeof(g_fn));
    EMU_TSAN_BENIGN(&g_f, sizeof(g_f));
    EMU_TSAN_BENIGN(&g_sched_tsan, sizeof(g_sched_tsan));
    g_sched_tsan = __tsan_get_current_fiber();
    __tsan_release(&g_tok_block[1]);  // the host's writes before the launch, for workgroup 0
#endif
    g_n = n;
    g_fn = &fn;
    const int64_t blocks = (int64_t)grid.x * grid.y * grid.z;
    g_grid = blocks;
    for (int64_t blk = 0; blk < blocks; ++blk) {
        g_block = blk;
        for (int i = 0; i < n; ++i)
            init_fiber(i);
        if (n > g_order_cap) {
            free(g_order);
            g_order = (int *)malloc(sizeof(int) * (size_t)n);
            g_order_cap = n;
        }
        for (int i = 0; i < n; ++i)
            g_order[i] = i;
        for (;;) {
            if (g_shuffle) {  // Fisher-Yates with xorshift64
                for (int i = n - 1; i > 0; --i) {
                    g_shuffle ^= g_shuffle << 13;
                    g_shuffle ^= g_shuffle >> 7;
                    g_shuffle ^= g_shuffle << 17;
                    const int j = (int)(g_shuffle % (unsigned long long)(i + 1));
                    const int t = g_order[i];
                    g_order[i] = g_order[j];
                    g_order[j] = t;
                }
            }
            bool progress = false;
            for (int k = 0; k < n; ++k) {
                const int i = g_order[k];
                if (g_f[i].state == RUN) {
                    run_fiber(i);
                    progress = true;
                }
            }
            int done = 0, at_bar = 0;
            for (int i = 0; i < n; ++i) {
                done += g_f[i].state == DONE;
                at_bar += g_f[i].state == AT_BARRIER;
            }
            if (done == n)
                break;
            for (int w = 0; w * 64 < n; ++w)
                resolve_wave(w, progress);
            if (at_bar == n) {
                for (int i = 0; i < n; ++i)
                    g_f[i].state = RUN;
                progress = true;
            } else if (at_bar > 0 && done > 0) {
                fprintf(stderr, "emu: barrier reached while %d threads already exited (block %lld)\n",
                        done, (long long)blk);
                abort();
            }
            if (!progress) {
                fprintf(stderr, "emu: deadlock in block %lld:", (long long)blk);
                for (int i = 0; i < n; i += 64)
                    fprintf(stderr, " w%d=%d", i / 64, g_f[i].state);
                fprintf(stderr, "\n");
                abort();
            }
        }
#ifdef EMU_TSAN
        for (int w = 0; w * 64 < n; ++w)
            __tsan_destroy_fiber(g_wave_tsan[w]);
#endif
    }
#ifdef EMU_TSAN
    __tsan_acquire(&g_tok_block[0]);  // the host reads what the launch wrote
    __tsan_acquire(&g_tok_block[1]);
#endif
    g_fn = nullptr;
}

}  // namespace emu

#define hipLaunchKernelGGL(K, G, B, S, ST, ...) \
    (::emu::launch(dim3(G), dim3(B), [&]() { K(__VA_ARGS__); }))

static inline hipError_t hipGetLastError() { return emu::g_error; }

// Static device arrays are plain host arrays here; their "device address" is
// their host address, and there is one emulated device.
#define __device__
#define __align__(n) __attribute__((aligned(n)))
#define HIP_SYMBOL(x) ((const void *)&(x))
static inline hipError_t hipGetDevice(int *dev)
{
    *dev = 0;
    return hipSuccess;
}
static inline hipError_t hipGetSymbolAddress(void **ptr, const void *symbol)
{
    *ptr = (void *)symbol;
    return hipSuccess;
}

// ------------------------------------------------------------ device primitives
SSD_DEVICE int thread_id() { return emu::g_cur; }
SSD_DEVICE int64_t block_id() { return emu::g_block; }
SSD_DEVICE int64_t grid_blocks() { return emu::g_grid; }
SSD_DEVICE int wave_id() { return emu::g_cur >> 6; }

SSD_DEVICE v4f mfma_16x16x4(float a, float b, v4f c)
{
    emu::Fiber &f = emu::g_f[emu::g_cur];
    f.a = a;
    f.b = b;
    f.c = c;
    f.state = emu::AT_MFMA;
    ++f.sync_count;
    emu::to_scheduler();
    return emu::g_f[emu::g_cur].d;
}

SSD_DEVICE float emu_shfl(float v, int mode, int arg)
{
    emu::Fiber &f = emu::g_f[emu::g_cur];
    f.sv = v;
    f.mode = mode;
    f.arg = arg;
    f.state = emu::AT_SHFL;
    ++f.sync_count;
    emu::to_scheduler();
    return emu::g_f[emu::g_cur].sr;
}

template <int n>
SSD_DEVICE float row_shr(float v) { return emu_shfl(v, emu::SH_SHR, n); }
template <int n>
SSD_DEVICE float row_shl(float v) { return emu_shfl(v, emu::SH_SHL, n); }
SSD_DEVICE float lane_read(float v, int src) { return emu_shfl(v, emu::SH_READ, src); }
template <int n>
SSD_DEVICE int row_shr_i(int v)
{
    return __builtin_bit_cast(int, emu_shfl(__builtin_bit_cast(float, v), emu::SH_SHR, n));
}
template <int n>
SSD_DEVICE int row_shl_i(int v)
{
    return __builtin_bit_cast(int, emu_shfl(__builtin_bit_cast(float, v), emu::SH_SHL, n));
}
SSD_DEVICE int lane_read_i(int v, int src)
{
    return __builtin_bit_cast(int, emu_shfl(__builtin_bit_cast(float, v), emu::SH_READ, src));
}
SSD_DEVICE float lane_fetch(float v, int src) { return emu_shfl(v, emu::SH_IDX, src); }
SSD_DEVICE float uniform(float v) { return v; }
SSD_DEVICE int uniform_i(int v) { return v; }
SSD_DEVICE v2f ld_c_uniform(const float *p, int64_t i) { return v2f{p[2 * i], p[2 * i + 1]}; }
// A wave-level meeting point: every lane of the wave arrives before any goes on.
SSD_DEVICE void wave_lds_sync() { (void)emu_shfl(0.f, emu::SH_READ, 0); }

// Buffer resources: an access must lie wholly inside [0, bytes) or wholly
// outside it (outside reads zero, outside stores are dropped); a straddling
// access is a layout error and aborts.
struct buf_t {
    const char *base;
    uint32_t n;
};
SSD_DEVICE buf_t make_buf(const void *base, uint32_t bytes) { return buf_t{(const char *)base, bytes}; }
SSD_DEVICE bool emu_buf_in(buf_t r, uint32_t off, uint32_t sz)
{
    if ((uint64_t)off + sz <= r.n)
        return true;
    if (off < r.n) {
        fprintf(stderr, "emu: buffer access straddles the end (off %u size %u bytes %u)\n", off, sz, r.n);
        abort();
    }
    return false;
}
SSD_DEVICE v4f buf_load4(buf_t r, uint32_t off)
{
    v4f v = {0.f, 0.f, 0.f, 0.f};
    if (emu_buf_in(r, off, 16))
        memcpy(&v, r.base + off, 16);
    return v;
}
SSD_DEVICE v2f buf_load2(buf_t r, uint32_t off)
{
    v2f v = {0.f, 0.f};
    if (emu_buf_in(r, off, 8))
        memcpy(&v, r.base + off, 8);
    return v;
}
SSD_DEVICE float buf_load1(buf_t r, uint32_t off)
{
    float v = 0.f;
    if (emu_buf_in(r, off, 4))
        memcpy(&v, r.base + off, 4);
    return v;
}
SSD_DEVICE uint32_t buf_load_u32(buf_t r, uint32_t off)
{
    uint32_t v = 0;
    if (emu_buf_in(r, off, 4))
        memcpy(&v, r.base + off, 4);
    return v;
}
SSD_DEVICE uint32_t buf_load_u16(buf_t r, uint32_t off)
{
    uint16_t v = 0;
    if (emu_buf_in(r, off, 2))
        memcpy(&v, r.base + off, 2);
    return v;
}
SSD_DEVICE void buf_store1(buf_t r, uint32_t off, float v)
{
    if (emu_buf_in(r, off, 4))
        memcpy((char *)r.base + off, &v, 4);
}
SSD_DEVICE void buf_store2(buf_t r, uint32_t off, v2f v)
{
    if (emu_buf_in(r, off, 8))
        memcpy((char *)r.base + off, &v, 8);
}
SSD_DEVICE void lds_add(float *p, float v) { *p += v; }
SSD_DEVICE void sched_fence() {}

SSD_DEVICE void block_sync()
{
#ifdef EMU_TSAN
    const int slot = emu::g_f[emu::g_cur].bars++ & 1;
    __tsan_release(&emu::g_tok_bar[slot]);
#endif
    emu::g_f[emu::g_cur].state = emu::AT_BARRIER;
    emu::to_scheduler();
#ifdef EMU_TSAN
    __tsan_acquire(&emu::g_tok_bar[slot]);
#endif
}

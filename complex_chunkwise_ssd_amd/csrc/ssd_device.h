// ssd_device.h -- the small set of gfx950 device primitives the scan kernels
// are written against: vector types, the fp32 MFMA tile, wave shuffles, the
// workgroup barrier and the thread/block indices.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

#define SSD_DEVICE __device__ __forceinline__
#define SSD_KERNEL(threads) __global__ __launch_bounds__(threads)
// ... with at least `waves` waves per SIMD (a register budget of 512 / waves)
#define SSD_KERNEL_WAVES(threads, waves) __global__ __launch_bounds__(threads, waves)
#define SSD_LDS __shared__ __attribute__((aligned(16)))

// D(16x16) += A(16x4) * B(4x16), fp32, one wave64. Lane L supplies
// A[L % 16][L / 16] and B[L / 16][L % 16]; it receives D[4 * (L / 16) + r][L % 16]
// in component r of the result.
SSD_DEVICE v4f mfma_16x16x4(float a, float b, v4f c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

SSD_DEVICE void block_sync() { __syncthreads(); }

// The hardware's base-2 exponential and logarithm (v_exp_f32, v_log_f32; about
// 1 ulp, results below the normal range flushed to zero).
SSD_DEVICE float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
SSD_DEVICE float hw_log2(float x) { return __builtin_amdgcn_logf(x); }

// Orders one wave's shared-memory accesses around this point: the wave's LDS
// instructions complete in the order they issue, so its earlier writes are
// seen by its later reads; this only keeps the compiler from moving memory
// accesses across the point.
SSD_DEVICE void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Buffer resources: 32-bit byte offsets from a wave-uniform base. An access
// at or past `bytes` reads zero and a store there is dropped, which is how the
// kernels mask padded rows and columns.
typedef __amdgpu_buffer_rsrc_t buf_t;
SSD_DEVICE buf_t make_buf(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)bytes, 0x00020000);
}
SSD_DEVICE v4f buf_load4(buf_t r, uint32_t off)
{
    return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
SSD_DEVICE v2f buf_load2(buf_t r, uint32_t off)
{
    return __builtin_bit_cast(v2f, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
SSD_DEVICE float buf_load1(buf_t r, uint32_t off)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
SSD_DEVICE uint32_t buf_load_u32(buf_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
SSD_DEVICE uint32_t buf_load_u16(buf_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
SSD_DEVICE void buf_store1(buf_t r, uint32_t off, float v)
{
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, (int)off, 0, 0);
}
SSD_DEVICE void buf_store2(buf_t r, uint32_t off, v2f v)
{
    typedef unsigned u2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, v), r, (int)off, 0, 0);
}

// Keeps the instruction scheduler from moving anything across this point (used to
// hold a software pipeline's loads ahead of the MFMAs that consume older ones).
SSD_DEVICE void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Shared-memory float accumulate (ds_add_f32).
SSD_DEVICE void lds_add(float *p, float v) { atomicAdd(p, v); }
SSD_DEVICE int thread_id() { return (int)threadIdx.x; }
SSD_DEVICE int64_t block_id() { return (int64_t)blockIdx.x; }
SSD_DEVICE int64_t grid_blocks() { return (int64_t)gridDim.x; }
// Wave index as a wave-uniform (scalar) value.
SSD_DEVICE int wave_id() { return __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6); }

// Row shifts inside aligned groups of 16 lanes (DPP row_shr / row_shl): lane i
// of a row receives lane i - n (shr) or i + n (shl) of the same row, or 0 when
// that lane is outside the row.
template <int n>
SSD_DEVICE float row_shr(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 0x110 + n, 0xf, 0xf, true));
}
template <int n>
SSD_DEVICE float row_shl(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 0x100 + n, 0xf, 0xf, true));
}
template <int n>
SSD_DEVICE int row_shr_i(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, 0x110 + n, 0xf, 0xf, true);
}
template <int n>
SSD_DEVICE int row_shl_i(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, 0x100 + n, 0xf, 0xf, true);
}
SSD_DEVICE int lane_read_i(int v, int src) { return __builtin_amdgcn_readlane(v, src); }
// Value of lane `src` (wave-uniform) for every lane.
SSD_DEVICE float lane_read(float v, int src)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src));
}
// v from lane src (any lane of the wave, chosen per lane).
SSD_DEVICE float lane_fetch(float v, int src)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, v)));
}
// A wave-uniform value kept in scalar registers.
SSD_DEVICE float uniform(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}
SSD_DEVICE int uniform_i(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Complex element i (interleaved float pairs) of an array that no kernel writes,
// at a wave-uniform index: read through the constant address space, a scalar
// load, so no vector-memory wait counter covers it.
SSD_DEVICE v2f ld_c_uniform(const float *p, int64_t i)
{
    using cv2f = __attribute__((address_space(4))) const v2f;
    return ((cv2f *)p)[i];
}

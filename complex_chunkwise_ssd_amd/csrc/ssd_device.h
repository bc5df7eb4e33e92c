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
#define SSD_LDS __shared__ __attribute__((aligned(16)))

// D(16x16) += A(16x4) * B(4x16), fp32, one wave64. Lane L supplies
// A[L % 16][L / 16] and B[L / 16][L % 16]; it receives D[4 * (L / 16) + r][L % 16]
// in component r of the result.
SSD_DEVICE v4f mfma_16x16x4(float a, float b, v4f c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

SSD_DEVICE void block_sync() { __syncthreads(); }
SSD_DEVICE int thread_id() { return (int)threadIdx.x; }
SSD_DEVICE int64_t block_id() { return (int64_t)blockIdx.x; }
// Wave index as a wave-uniform (scalar) value.
SSD_DEVICE int wave_id() { return __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6); }

// Shuffles inside aligned groups of 16 lanes; a lane whose source falls
// outside its group keeps its own value.
SSD_DEVICE float shfl_up16(float v, int d) { return __shfl_up(v, (unsigned)d, 16); }
SSD_DEVICE float shfl_down16(float v, int d) { return __shfl_down(v, (unsigned)d, 16); }
// Value of lane `src` (0..63) of the wave.
SSD_DEVICE float shfl_idx(float v, int src) { return __shfl(v, src, 64); }

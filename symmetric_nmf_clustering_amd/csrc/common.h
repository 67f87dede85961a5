// Device-side helpers shared by the libsymnmf kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float floatx4 __attribute__((ext_vector_type(4)));

namespace symnmf {

constexpr int kWave = 64;

// v_mfma_f32_16x16x4_f32: D(16x16) = A(16x4) B(4x16) + C. Lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16]; it receives
// D[4 (l / 16) + r][l % 16] in element r of the result.
__device__ __forceinline__ floatx4 mfma16x16x4(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Orders a wave's LDS accesses across its lanes: what lanes wrote before it is
// seen by the reads of other lanes after it (the wave's LDS operations run in
// order; this keeps the compiler from moving them across).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): output c+1 of the
// sequence whose state starts at `key`.
__host__ __device__ __forceinline__ uint64_t splitmix64(uint64_t key, uint64_t c) {
    uint64_t z = key + (c + 1ull) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Top 24 bits of the SplitMix64 output as a float in [0, 1). Exact in fp32.
__host__ __device__ __forceinline__ float uniform24(uint64_t key, uint64_t c) {
    return (float)(splitmix64(key, c) >> 40) * (1.0f / 16777216.0f);
}

constexpr uint64_t kSamplerKeyXor = 0x5851F42D4C957F2Dull;

// Fixed-order wave reduction (butterfly over lane xor masks; every lane ends
// with the same total, and the order of additions does not depend on timing).
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

// Block-wide fixed-order sum for blockDim.x == 256 (4 waves). `red` needs 4
// slots of shared memory. Result valid in every thread.
__device__ __forceinline__ double block_sum256(double v, double* red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    double s = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return s;
}

// sum_{s < count} p[s * stride] added in index order. Eight loads are issued
// before their additions, so a long sum waits for count/8 memory round trips
// instead of count; the order of the additions, and so the result, is the
// same as the plain loop's.
__device__ __forceinline__ float ordered_strided_sum(const float* __restrict__ p, int count,
                                                     int64_t stride) {
    float s = 0.f;
    int sp = 0;
    for (; sp + 8 <= count; sp += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = p[(int64_t)(sp + u) * stride];
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; sp < count; ++sp) s += p[(int64_t)sp * stride];
    return s;
}

}  // namespace symnmf

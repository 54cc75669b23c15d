// Diagnostic ceilings: an MFMA-only loop and a streaming read, used to put the
// fused kernel's measured rates next to what the device sustains.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swk {

__global__ __launch_bounds__(256) void probe_mfma_kernel(float* sink, int iters) {
    typedef __bf16 v8 __attribute__((ext_vector_type(8)));
    typedef float v16 __attribute__((ext_vector_type(16)));
    const int tid = threadIdx.x;
    v8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(1.0f + 0.001f * (float)((tid + e) & 7));
        b[e] = (__bf16)(0.5f - 0.001f * (float)((tid * 3 + e) & 7));
    }
    v16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[i][r];
    sink[(size_t)blockIdx.x * blockDim.x + tid] = s;
}

__global__ __launch_bounds__(256) void probe_read_kernel(const uint4* __restrict__ src, long long n16,
                                                         uint32_t* sink) {
    const long long stride = (long long)gridDim.x * blockDim.x;
    uint32_t x = 0;
    long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
        x ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w;
        x ^= v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^ v3.w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = src[i];
        x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

}  // namespace swk

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

// Streaming read with non-temporal loads (each byte is read once, as the
// decode kernels' weights are), four 16-byte loads in flight per lane.
__global__ __launch_bounds__(256) void probe_read_kernel(const uint4* __restrict__ src4, long long n16,
                                                         uint32_t* sink) {
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    const v4u* src = reinterpret_cast<const v4u*>(src4);
    const long long stride = (long long)gridDim.x * blockDim.x;
    v4u x = {0u, 0u, 0u, 0u};
    long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const v4u v0 = __builtin_nontemporal_load(src + i);
        const v4u v1 = __builtin_nontemporal_load(src + i + stride);
        const v4u v2 = __builtin_nontemporal_load(src + i + 2 * stride);
        const v4u v3 = __builtin_nontemporal_load(src + i + 3 * stride);
        x ^= v0 ^ v1 ^ v2 ^ v3;
    }
    for (; i < n16; i += stride) x ^= __builtin_nontemporal_load(src + i);
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

}  // namespace swk

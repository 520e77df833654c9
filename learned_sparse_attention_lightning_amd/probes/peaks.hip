// peaks.hip -- what this device actually sustains, for the roofline
// fractions reported beside the vendor peaks:
//   probe_stream_read   coalesced 16-byte nontemporal reads of a buffer, four or
//                       eight loads in flight per thread (the access pattern of
//                       the decode key stream), one word written per workgroup;
//   probe_mfma_bf16     back-to-back v_mfma_f32_32x32x16_bf16 on register
//                       operands, four independent accumulators per wave;
//   probe_mfma_fp8      the same with the fp8 e4m3 32x32x64 scaled form.
// Each returns the launch status; the caller times the launch with events on
// `stream`.  Measurement only: nothing here is part of the forward path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define PROBE_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kReadThreads = 256;

template <int InFlight>
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4 *__restrict__ p,
                                                                   size_t n16,
                                                                   uint32_t *__restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * kReadThreads;
    uint32_t acc = 0u;
    size_t j = (size_t)blockIdx.x * kReadThreads + threadIdx.x;
    for (; j + (InFlight - 1) * stride < n16; j += InFlight * stride) {
        u32x4 v[InFlight];
#pragma unroll
        for (int u = 0; u < InFlight; ++u) v[u] = __builtin_nontemporal_load(p + j + u * stride);
#pragma unroll
        for (int u = 0; u < InFlight; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; j < n16; j += stride) {
        const u32x4 v = __builtin_nontemporal_load(p + j);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    // one word per workgroup keeps the loads alive
    for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
    if ((threadIdx.x & 63) == 0) atomicXor(&sink[blockIdx.x], acc);
}

template <bool Fp8>
__global__ __launch_bounds__(256) void mfma_loop_kernel(float *__restrict__ sink, int iters) {
    const int lane = threadIdx.x & 63;
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    if constexpr (Fp8) {
        i32x8 a, b;
        for (int e = 0; e < 8; ++e) {
            a[e] = 0x38383838 + lane + e;  // small fp8 values
            b[e] = 0x30303030 + lane - e;
        }
        for (int it = 0; it < iters; ++it) {
            c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 127, 0, 127);
            c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c1, 0, 0, 0, 127, 0, 127);
            c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c2, 0, 0, 0, 127, 0, 127);
            c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, b, c3, 0, 0, 0, 127, 0, 127);
        }
    } else {
        bf16x8 a, b;
        for (int e = 0; e < 8; ++e) {
            a[e] = (__bf16)(0.001f * (lane + e));
            b[e] = (__bf16)(0.002f * (lane - e));
        }
        for (int it = 0; it < iters; ++it) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
        }
    }
    float s = 0.0f;
    for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
    if (threadIdx.x == 0) sink[blockIdx.x] = s;
}

}  // namespace

// Reads `bytes` (a multiple of 16) from `buf` once, `inflight` (4 or 8)
// 16-byte loads in flight per thread; sink holds `blocks` words.
PROBE_EXPORT int probe_stream_read(const void *buf, size_t bytes, uint32_t *sink, int blocks,
                                   int inflight, void *stream) {
    if (inflight == 8)
        hipLaunchKernelGGL(stream_read_kernel<8>, dim3(blocks), dim3(kReadThreads), 0,
                           (hipStream_t)stream, static_cast<const u32x4 *>(buf), bytes / 16, sink);
    else
        hipLaunchKernelGGL(stream_read_kernel<4>, dim3(blocks), dim3(kReadThreads), 0,
                           (hipStream_t)stream, static_cast<const u32x4 *>(buf), bytes / 16, sink);
    return (int)hipGetLastError();
}

// blocks x 4 waves x iters x 4 products; 32x32x16 bf16 = 32768 flop a product.
PROBE_EXPORT int probe_mfma_bf16(float *sink, int iters, int blocks, void *stream) {
    hipLaunchKernelGGL(mfma_loop_kernel<false>, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       sink, iters);
    return (int)hipGetLastError();
}

// 32x32x64 fp8 = 131072 flop a product.
PROBE_EXPORT int probe_mfma_fp8(float *sink, int iters, int blocks, void *stream) {
    hipLaunchKernelGGL(mfma_loop_kernel<true>, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       sink, iters);
    return (int)hipGetLastError();
}

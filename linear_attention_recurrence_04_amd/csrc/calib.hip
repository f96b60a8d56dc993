// calib.hip -- calibration kernels: what this GPU sustains for a streaming
// copy (HBM bytes) and for dense bf16 matrix-core work (flops).  The roofline
// fractions of the gated-delta-rule kernels are stated against these as well
// as against the published peaks.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn.h"
#include "gdn_calib.h"

namespace gdn {
namespace calib {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kCopyThreads = 256;

// One tile of kCopyThreads * U 16-byte elements per workgroup, one pass over
// the grid: every thread issues its U loads before its first store.
template <int U, bool NT>
__global__ __launch_bounds__(kCopyThreads) void copy_kernel(const u32x4* __restrict__ src,
                                                            u32x4* __restrict__ dst, size_t n16) {
    const size_t tile = (size_t)blockIdx.x * (kCopyThreads * U);
    const u32x4* s = src + tile + threadIdx.x;
    u32x4* d = dst + tile + threadIdx.x;
    u32x4 r[U];
    if (tile + kCopyThreads * U <= n16) {   // whole tile: no per-element checks
#pragma unroll
        for (int u = 0; u < U; ++u) r[u] = NT ? __builtin_nontemporal_load(s + u * kCopyThreads) : s[u * kCopyThreads];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (NT) __builtin_nontemporal_store(r[u], d + u * kCopyThreads);
            else d[u * kCopyThreads] = r[u];
        }
        return;
    }
    const int left = (int)(n16 - tile);     // last, partial tile
#pragma unroll
    for (int u = 0; u < U; ++u)
        if ((int)threadIdx.x + u * kCopyThreads < left) d[u * kCopyThreads] = s[u * kCopyThreads];
}

template <int U, bool NT>
static hipError_t launch_copy(const void* src, void* dst, size_t n16, hipStream_t stream) {
    const size_t per = (size_t)kCopyThreads * U;
    const size_t blocks = (n16 + per - 1) / per;
    hipLaunchKernelGGL((copy_kernel<U, NT>), dim3((unsigned)blocks), dim3(kCopyThreads), 0, stream,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
    return hipGetLastError();
}

constexpr int kChains = 8;

// Eight matrix-core instructions per wave and iteration on register operands:
// one accumulator chain for 16x16x32 (VARIANT 0; several 4-register chains
// make the compiler rotate accumulators with register moves that then bound
// the loop), eight independent chains for 32x32x16 (VARIANT 1).  The wave's
// accumulators are summed and stored once so the work stays live.
template <int VARIANT>
__global__ __launch_bounds__(256) void mfma_loop_kernel(float* __restrict__ out, int iters) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (__bf16)(0.001f * (float)((lane + j) & 7));
        b[j] = (__bf16)(0.001f * (float)((lane * 3 + j) & 7));
    }
    float total = 0.f;
    if constexpr (VARIANT == 0) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int c = 0; c < kChains; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
        }
        total = acc[0] + acc[1] + acc[2] + acc[3];
    } else {
        f32x16 acc[kChains];
#pragma unroll
        for (int c = 0; c < kChains; ++c)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int c = 0; c < kChains; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < kChains; ++c)
#pragma unroll
            for (int e = 0; e < 16; ++e) total += acc[c][e];
    }
    if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = total;
}

}  // namespace calib
}  // namespace gdn

using namespace gdn::calib;

extern "C" gdn_status gdn_calib_copy(const void* src, void* dst, size_t bytes, int32_t variant,
                                     void* hip_stream) {
    if (variant < 0 || variant > 2) return GDN_ERR_UNSUPPORTED;
    if (bytes % 16 != 0) return GDN_ERR_BAD_SHAPE;
    if (bytes == 0) return GDN_OK;
    if (!src || !dst) return GDN_ERR_NULL_POINTER;
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 != 0)
        return GDN_ERR_MISALIGNED;
    const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
    if (s < d + bytes && d < s + bytes) return GDN_ERR_BAD_SHAPE;
    const size_t n16 = bytes / 16;
    if (n16 / kCopyThreads + 1 > 0x7fffffffu) return GDN_ERR_BAD_SHAPE;   // grid size
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    hipError_t err;
    switch (variant) {
        case 0: err = launch_copy<1, false>(src, dst, n16, stream); break;
        case 1: err = launch_copy<4, false>(src, dst, n16, stream); break;
        default: err = launch_copy<2, true>(src, dst, n16, stream); break;
    }
    return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

extern "C" gdn_status gdn_calib_mfma_loop(float* out, int32_t workgroups, int32_t iters,
                                          int32_t variant, void* hip_stream) {
    if (variant < 0 || variant > 1) return GDN_ERR_UNSUPPORTED;
    if (!out) return GDN_ERR_NULL_POINTER;
    if (reinterpret_cast<uintptr_t>(out) % 16 != 0) return GDN_ERR_MISALIGNED;
    if (workgroups < 1 || iters < 1) return GDN_ERR_BAD_SHAPE;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (variant == 0)
        hipLaunchKernelGGL((mfma_loop_kernel<0>), dim3(workgroups), dim3(256), 0, stream, out, iters);
    else
        hipLaunchKernelGGL((mfma_loop_kernel<1>), dim3(workgroups), dim3(256), 0, stream, out, iters);
    return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

// gdn_device.h -- small device helpers shared by the gated-delta-rule kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// bfloat16 is handled as its raw 16-bit pattern.
typedef uint16_t bf16_t;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Round-to-nearest-even conversion, NaN kept quiet.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>(0x7fc0);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<bf16_t>(u >> 16);
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return f32_to_bf16(x); }

// Butterfly sum over `width` consecutive lanes (width a power of two <= 64);
// every lane of the group receives the total, in the same order on all lanes.
template <int width>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int m = width / 2; m >= 1; m /= 2) x += __shfl_xor(x, m, 64);
    return x;
}

// Qwen gates from the raw per-token projections a, b of a value head with
// parameters A_log, dt_bias: log g = -exp(A_log) softplus(a + dt_bias) (never
// positive) and beta = sigmoid(b).  softplus(x) = log(1 + e^x), taken as x
// itself above 20 where the two agree in fp32.
__device__ __forceinline__ float raw_log_decay(float a, float A_log, float dt_bias) {
    const float x = a + dt_bias;
    const float sp = x > 20.f ? x : log1pf(expf(x));
    return -expf(A_log) * sp;
}
__device__ __forceinline__ float raw_beta(float b) { return 1.0f / (1.0f + expf(-b)); }

// A token's log decay as the chunked kernels use it.  They exponentiate
// differences of in-chunk prefix sums of log g, and a token with g = 0
// (log g = -inf) would make such a difference -inf - (-inf) = NaN.  Below -87,
// g = exp(log g) is already under the smallest normal fp32 (about 1.2e-38), so
// holding log g at -87 there changes a result only far below fp32 rounding.
// Written as a comparison so that a NaN passes through unchanged.
__device__ __forceinline__ float chunk_log_decay(float lg) { return lg < -87.f ? -87.f : lg; }

// Tokens of sequence b on the token axis: [first, first + count).  Without
// cu_seqlens sequence b is tokens [b T, b T + T).  With them (packed
// variable-length batch) the bounds are clamped into [0, total] and the count
// to T, the longest sequence the launch was sized for, so any cu_seqlens
// content keeps every access in bounds.
__device__ __forceinline__ void seq_span(const int* cu, int b, int T, long long total,
                                         size_t& first, int& count) {
    if (!cu) {
        first = (size_t)b * T;
        count = T;
        return;
    }
    const long long s0 = min(max((long long)cu[b], 0LL), total);
    const long long s1 = min(max((long long)cu[b + 1], s0), total);
    first = (size_t)s0;
    count = (int)min(s1 - s0, (long long)T);
}

// 1 / max(sqrt(ss), 1e-6): the L2-normalisation factor used by every kernel.
__device__ __forceinline__ float inv_l2(float ss) {
    return 1.0f / fmaxf(sqrtf(ss), 1e-6f);
}

}  // namespace gdn

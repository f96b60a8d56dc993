// conv_norm.hip -- the operations around the recurrence: causal depthwise
// conv1d over the channels of the q, k, v projections with the convolution
// state carried between calls, and the gated RMS norm of the output ("Qwen3.5
// Gated Delta Net NKI Kernel for AWS Neuron", section "How It Works", names
// them; "Add Qwen3.6-27B hybrid DeltaNet/GQA contrib model and vLLM serving
// path", section "Summary", checkpoints the convolution state).
//
// Both are streaming passes (a few flops per byte), bound by HBM:
//  * conv: a thread owns 16 bytes of channels (8 bf16 or 4 fp32) over a
//    tile of CONV_TT = 64 consecutive tokens, keeps CONV_RING row loads in
//    flight and slides a window of K inputs in registers; a wave covers 1 KiB
//    of one token row.  (Tiles of 4, 8, 16, 32, 64, 128 tokens measured on
//    MI355X at the 27B layer's shape: 344, 254, 200, 162, 160, 167 us; the
//    per-thread weights and the K-1 halo rows amortise over the tile.)  The
//    ring runs in whole blocks of CONV_RING tokens with no branch and a
//    scheduling barrier after each token, so the compiler neither drains the
//    loads at every block (a conditional store leaves the count of stores in
//    flight unknown to it) nor sinks them next to their use; the last
//    partial block follows.  y is written with non-temporal stores: nothing
//    here reads it again, and bypassing the caches gained ~7% (155 -> 145
//    us).  The K-1 tokens before the tile come from the previous tile's rows
//    (mostly cache hits) or, before the first token, from the carried state.
//    The new state (one thread per 16 bytes of channels reads every old value
//    it needs before writing, so it may overwrite the old one, also when
//    T < K-1) is written by the conv kernel itself when a call is one tile per
//    sequence (decode, short calls: 15.7 -> 13.2 us per call back to back at
//    B=64, T=1 over the 27B channels), else by a second small kernel launched
//    after it on the same stream, since then tile 0 reads the old state while
//    the last tile ends.
//  * gated RMS norm: a group of D/VEC lanes per row (two rows per group),
//    the sum of squares reduced by shuffles in a fixed order; each lane reads
//    its x and z before writing y, so y may be x.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int CONV_TT = kConvTileTokens;   // tokens per thread
constexpr int CONV_RING = 8;               // loads in flight per thread
constexpr int CONV_THREADS = 256;

template <typename TIn>
struct Vec16 {                   // 16 bytes of one token row
    static constexpr int N = 16 / sizeof(TIn);
    TIn v[N];
};

template <typename TIn>
__device__ __forceinline__ void load16(const TIn* p, float (&out)[16 / sizeof(TIn)]) {
    const uint4 raw = *reinterpret_cast<const uint4*>(p);
    const Vec16<TIn> x = __builtin_bit_cast(Vec16<TIn>, raw);
#pragma unroll
    for (int i = 0; i < Vec16<TIn>::N; ++i) out[i] = to_f32(x.v[i]);
}

template <typename TIn>
__device__ __forceinline__ void store16(TIn* p, const float (&in)[16 / sizeof(TIn)]) {
    Vec16<TIn> x;
#pragma unroll
    for (int i = 0; i < Vec16<TIn>::N; ++i) x.v[i] = from_f32<TIn>(in[i]);
    *reinterpret_cast<uint4*>(p) = __builtin_bit_cast(uint4, x);
}

// the same, as one non-temporal 16-byte store (a streaming output)
template <typename TIn>
__device__ __forceinline__ void store16_nt(TIn* p, const float (&in)[16 / sizeof(TIn)]) {
    Vec16<TIn> x;
#pragma unroll
    for (int i = 0; i < Vec16<TIn>::N; ++i) x.v[i] = from_f32<TIn>(in[i]);
    const uint4 u = __builtin_bit_cast(uint4, x);
    uint4* d = reinterpret_cast<uint4*>(p);
    __builtin_nontemporal_store(u.x, &d->x);
    __builtin_nontemporal_store(u.y, &d->y);
    __builtin_nontemporal_store(u.z, &d->z);
    __builtin_nontemporal_store(u.w, &d->w);
}

// x / (1 + e^-x) with the hardware exponential and reciprocal (about 1 ulp
// each, far below the rounding of the stored output); 0 * x for x -> -inf
__device__ __forceinline__ float silu(float x) {
    return x * __builtin_amdgcn_rcpf(1.f + __expf(-x));
}

// new state [B, P, C] of sequence b at channels c0 .. c0 + 15 bytes: the last
// P entries of concat(old state, x), copied bit for bit; every value is read
// before any is written, so state_out may be state_in
template <typename TIn, int K>
__device__ __forceinline__ void carry_state(const TIn* x, const TIn* state_in, TIn* state_out, int T, int C,
                                            int b, int c0) {
    constexpr int P = K - 1;
    uint4 keep[P > 0 ? P : 1];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int s = T - P + i;   // position in the sequence; < 0: from the old state
        if (s >= 0)
            keep[i] = *reinterpret_cast<const uint4*>(x + ((size_t)b * T + s) * C + c0);
        else if (state_in)
            keep[i] = *reinterpret_cast<const uint4*>(state_in + ((size_t)b * P + (P + s)) * C + c0);
        else
            keep[i] = uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < P; ++i)
        *reinterpret_cast<uint4*>(state_out + ((size_t)b * P + i) * C + c0) = keep[i];
}

// grid: x = channel groups (C / N) in blocks of CONV_THREADS, y = token tiles,
// z = sequences.  CARRY (one tile per sequence only): the thread also writes
// the new state of its channels, which no other thread reads.
template <typename TIn, int K, bool CARRY>
__global__ __launch_bounds__(CONV_THREADS) void conv1d_kernel(
    const TIn* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias,
    const TIn* state_in, TIn* __restrict__ y, TIn* state_out, int T, int C, int silu_on) {
    constexpr int N = Vec16<TIn>::N;
    constexpr int P = K - 1;
    const int cg = blockIdx.x * CONV_THREADS + threadIdx.x;
    if (cg * N >= C) return;
    const int c0 = cg * N;
    const int t0 = blockIdx.y * CONV_TT;
    const int b = blockIdx.z;
    const TIn* xb = x + (size_t)b * T * C + c0;
    TIn* yb = y + (size_t)b * T * C + c0;

    float wk[K][N], bs[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
#pragma unroll
        for (int j = 0; j < K; ++j) wk[j][i] = w[(size_t)(c0 + i) * K + j];
        bs[i] = bias ? bias[c0 + i] : 0.f;
    }
    // window: u[t0 - P .. t0 - 1]
    float win[K][N];
#pragma unroll
    for (int j = 0; j < P; ++j) {
        const int s = t0 - P + j;
        if (s >= 0) {
            load16(xb + (size_t)s * C, win[j]);
        } else if (state_in) {
            load16(state_in + ((size_t)b * P + (P + s)) * C + c0, win[j]);
        } else {
#pragma unroll
            for (int i = 0; i < N; ++i) win[j][i] = 0.f;
        }
    }
    // token tt of the tile from its row's 16 bytes: y, then the window slides
    auto step = [&](const uint4 raw, int tt) __attribute__((always_inline)) {
        const Vec16<TIn> v = __builtin_bit_cast(Vec16<TIn>, raw);
#pragma unroll
        for (int i = 0; i < N; ++i) win[P][i] = to_f32(v.v[i]);
        float out[N];
#pragma unroll
        for (int i = 0; i < N; ++i) {
            float acc = bs[i];
#pragma unroll
            for (int j = 0; j < K; ++j) acc += wk[j][i] * win[j][i];
            out[i] = silu_on ? silu(acc) : acc;
        }
        store16_nt(yb + (size_t)(t0 + tt) * C, out);
#pragma unroll
        for (int j = 0; j < P; ++j)
#pragma unroll
            for (int i = 0; i < N; ++i) win[j][i] = win[j + 1][i];
    };
    // the tile's tokens through a ring of CONV_RING loads in flight; a load
    // past the last token re-reads the last row (in bounds, never used)
    const int tn = min(CONV_TT, T - t0);
    const TIn* xt = xb + (size_t)t0 * C;
    const int last = tn - 1;
    uint4 ring[CONV_RING];
#pragma unroll
    for (int r = 0; r < CONV_RING; ++r)
        ring[r] = *reinterpret_cast<const uint4*>(xt + (size_t)min(r, last) * C);
    int base = 0;
    for (; base + CONV_RING <= tn; base += CONV_RING) {
#pragma unroll
        for (int r = 0; r < CONV_RING; ++r) {
            const uint4 raw = ring[r];
            ring[r] = *reinterpret_cast<const uint4*>(xt + (size_t)min(base + r + CONV_RING, last) * C);
            step(raw, base + r);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int r = 0; r < CONV_RING - 1; ++r)
        if (base + r < tn) step(ring[r], base + r);
    if constexpr (CARRY) carry_state<TIn, K>(x, state_in, state_out, T, C, b, c0);
}

// new state [B, P, C] of every sequence (calls of more than one tile): one
// thread per 16 bytes of channels, all reads before any write
template <typename TIn, int K>
__global__ __launch_bounds__(CONV_THREADS) void conv_state_kernel(
    const TIn* __restrict__ x, const TIn* state_in, TIn* state_out, int T, int C) {
    constexpr int N = Vec16<TIn>::N;
    const int cg = blockIdx.x * CONV_THREADS + threadIdx.x;
    if (cg * N >= C) return;
    carry_state<TIn, K>(x, state_in, state_out, T, C, blockIdx.y, cg * N);
}

template <typename TIn, int K>
hipError_t launch_conv_k(const ConvArgs& a, hipStream_t stream) {
    constexpr int N = Vec16<TIn>::N;
    const int groups = a.C / N;
    const TIn* x = static_cast<const TIn*>(a.x);
    const TIn* st_in = static_cast<const TIn*>(a.state_in);
    TIn* st_out = static_cast<TIn*>(a.state_out);
    // one tile per sequence (decode, short calls): the conv kernel carries the
    // state itself, one launch instead of two
    const bool carry = st_out && K > 1 && a.T > 0 && a.T <= CONV_TT;
    if (a.B > 0 && a.T > 0) {
        const dim3 grid((groups + CONV_THREADS - 1) / CONV_THREADS, (a.T + CONV_TT - 1) / CONV_TT, a.B);
        const auto kern = carry ? conv1d_kernel<TIn, K, true> : conv1d_kernel<TIn, K, false>;
        hipLaunchKernelGGL(kern, grid, dim3(CONV_THREADS), 0, stream, x, a.w, a.bias, st_in,
                           static_cast<TIn*>(a.y), st_out, a.T, a.C, a.silu);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess || carry) return err;
    }
    if (a.state_out && a.B > 0 && K > 1) {
        const dim3 grid((groups + CONV_THREADS - 1) / CONV_THREADS, a.B);
        hipLaunchKernelGGL((conv_state_kernel<TIn, K>), grid, dim3(CONV_THREADS), 0, stream, x,
                           static_cast<const TIn*>(a.state_in), static_cast<TIn*>(a.state_out), a.T,
                           a.C);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <typename TIn>
hipError_t launch_conv_t(const ConvArgs& a, hipStream_t stream) {
    switch (a.K) {
        case 1: return launch_conv_k<TIn, 1>(a, stream);
        case 2: return launch_conv_k<TIn, 2>(a, stream);
        case 3: return launch_conv_k<TIn, 3>(a, stream);
        default: return launch_conv_k<TIn, 4>(a, stream);
    }
}

constexpr int NORM_THREADS = 256;

// G lanes per row (D = G * N), 64 / G rows per wave
constexpr int NORM_ROWS = 2;   // rows per lane group

typedef __attribute__((ext_vector_type(4))) unsigned int u32v4;

// G lanes per row (D = G * N), NORM_ROWS rows per lane group.  Every load (x
// and z of all its rows, then w) is issued before any arithmetic or store:
// written in that order the compiler keeps it (y may be x, so it may not move
// a later row's loads above an earlier row's store), and the loads are in
// flight together.  The rows go through buffer resources on the block's rows,
// sized to the rows that exist: a lane past the last row loads zeros and its
// store is dropped by the hardware, so no branch guards a store (a guarded
// store let the compiler sink the z loads into the branch, after the
// reduction over x).  Rows are read and written with non-temporal accesses.
// On the 27B output shape (786,432 rows of 128 bf16, gated), against one row
// per group with plain accesses: 103 -> 91 us per call back to back, 112 ->
// 101 us timed one call at a time.
template <typename TIn, int G, bool GATED>
__global__ __launch_bounds__(NORM_THREADS) void gated_rmsnorm_kernel(
    const TIn* x, const TIn* __restrict__ z, const float* __restrict__ w, float eps, TIn* y,
    long long rows) {
    constexpr int N = Vec16<TIn>::N;
    constexpr int D = G * N;
    constexpr int RPB = NORM_THREADS / G;   // rows of one block step
    constexpr int BR = NORM_ROWS * RPB;     // rows of the block
    const int part = threadIdx.x % G;
    const long long row0 = (long long)blockIdx.x * BR;
    const long long left = rows - row0;   // > 0: the grid covers the rows exactly
    const int nrows = left < BR ? (int)left : BR;
    const int nbytes = nrows * D * (int)sizeof(TIn);
    const size_t base = (size_t)row0 * D;
    const auto xs = __builtin_amdgcn_make_buffer_rsrc(const_cast<TIn*>(x) + base, (short)0, nbytes, 0x00020000);
    const auto zs = __builtin_amdgcn_make_buffer_rsrc(const_cast<TIn*>(GATED ? z : x) + base, (short)0, nbytes,
                                                      0x00020000);
    const auto ys = __builtin_amdgcn_make_buffer_rsrc(y + base, (short)0, nbytes, 0x00020000);
    int voff[NORM_ROWS];   // bytes from the block's first row
#pragma unroll
    for (int j = 0; j < NORM_ROWS; ++j)
        voff[j] = ((j * RPB + (int)threadIdx.x / G) * D + part * N) * (int)sizeof(TIn);
    Vec16<TIn> xr[NORM_ROWS], zr[NORM_ROWS];
#pragma unroll
    for (int j = 0; j < NORM_ROWS; ++j) {
        xr[j] = __builtin_bit_cast(Vec16<TIn>, __builtin_amdgcn_raw_buffer_load_b128(xs, voff[j], 0, 2));
        if constexpr (GATED)
            zr[j] = __builtin_bit_cast(Vec16<TIn>, __builtin_amdgcn_raw_buffer_load_b128(zs, voff[j], 0, 2));
    }
    float wv[N];
#pragma unroll
    for (int i = 0; i < N; ++i) wv[i] = w[part * N + i];
#pragma unroll
    for (int j = 0; j < NORM_ROWS; ++j) {
        float xv[N];
#pragma unroll
        for (int i = 0; i < N; ++i) xv[i] = to_f32(xr[j].v[i]);
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < N; ++i) ss += xv[i] * xv[i];
#pragma unroll
        for (int m = 1; m < G; m *= 2) ss += __shfl_xor(ss, m, 64);
        const float inv = 1.f / sqrtf(ss / (float)D + eps);
        Vec16<TIn> o;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const float g = GATED ? silu(to_f32(zr[j].v[i])) : 1.f;
            o.v[i] = from_f32<TIn>(xv[i] * inv * wv[i] * g);
        }
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32v4, o), ys, voff[j], 0, 2);
    }
}

template <typename TIn, int G>
hipError_t launch_norm_g(const NormArgs& a, hipStream_t stream) {
    const long long groups = (a.rows + NORM_THREADS / G - 1) / (NORM_THREADS / G);
    const long long blocks = (groups + NORM_ROWS - 1) / NORM_ROWS;
    const auto kern = a.z ? gated_rmsnorm_kernel<TIn, G, true> : gated_rmsnorm_kernel<TIn, G, false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(NORM_THREADS), 0, stream,
                       static_cast<const TIn*>(a.x), static_cast<const TIn*>(a.z), a.w, a.eps,
                       static_cast<TIn*>(a.y), a.rows);
    return hipGetLastError();
}

template <typename TIn>
hipError_t launch_norm_t(const NormArgs& a, hipStream_t stream) {
    constexpr int N = Vec16<TIn>::N;
    switch (a.D / N) {
        case 2: return launch_norm_g<TIn, 2>(a, stream);
        case 4: return launch_norm_g<TIn, 4>(a, stream);
        case 8: return launch_norm_g<TIn, 8>(a, stream);
        case 16: return launch_norm_g<TIn, 16>(a, stream);
        case 32: return launch_norm_g<TIn, 32>(a, stream);
        default: return launch_norm_g<TIn, 64>(a, stream);
    }
}

}  // namespace

bool conv_norm_dim_supported(int D, bool bf16) {
    const int n = bf16 ? 8 : 4;
    if (D % n != 0) return false;
    const int g = D / n;
    return g >= 2 && g <= 64 && (g & (g - 1)) == 0;
}

hipError_t launch_causal_conv1d(const ConvArgs& a, hipStream_t stream) {
    return a.bf16 ? launch_conv_t<bf16_t>(a, stream) : launch_conv_t<float>(a, stream);
}

hipError_t launch_gated_rmsnorm(const NormArgs& a, hipStream_t stream) {
    if (a.rows == 0) return hipSuccess;
    return a.bf16 ? launch_norm_t<bf16_t>(a, stream) : launch_norm_t<float>(a, stream);
}

}  // namespace gdn

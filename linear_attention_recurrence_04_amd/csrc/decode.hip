// decode.hip -- single-token gated-delta-rule step with the state updated in place.
//
// Per (batch b, value head h) the five steps of "Qwen3.5 Gated Delta Net NKI
// Kernel for AWS Neuron", section "How It Works", are fused into ONE pass over
// the fp32 state:
//     a = S^T k_hat,  c = S^T q_hat          (both from the old state)
//     delta = beta (v - g a)                  (the read of the decayed state)
//     o = q_scale (g c + delta (k_hat . q_hat))   (= (g S + k delta^T)^T q_hat)
//     S <- g S + k_hat delta^T                (stored to the same addresses)
// so each step reads and writes every state element exactly once.  That is
// the whole cost: the state is 4*dk*dv bytes per head against ~7*dk*dv flops,
// so the kernel is bound by HBM bandwidth.
//
// T > 1 tokens per call (multi-token decode, speculative verification) run
// the same pass once per token with the state kept in registers: it is read
// once and written once per call, and optionally also stored after every
// token (the per-token states a verifier rolls back to).
//
// Mapping: one workgroup of NT threads per (b, h).  A thread owns a float4
// column strip of D/RG rows (RG = row groups), held in VGPRs between the read
// and the write; rows are interleaved so each wave load covers whole 512-byte
// rows (fully coalesced 16-byte accesses).  Column reductions over the rows
// combine per-thread partials in LDS in a fixed order (deterministic).
// NT is 256 for several tokens per call and for head dim 64; a single step
// at head dim 128 uses 512 threads (8 rows per thread), or 1024 (4 rows) once
// the whole state no longer fits the 256 MB Infinity Cache and streams from
// HBM (measured on the 27B head shape: 64 sequences, 201 MB of state, 512
// threads -2% against 256, 1024 threads +27%; 128 sequences, 403 MB, 1024
// threads -7%).
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <int D, typename TIn, bool MULTI, int NTHR>
__global__ __launch_bounds__(NTHR) void decode_step_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const float* __restrict__ log_g, const float* __restrict__ beta,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias,
    float* __restrict__ state, TIn* __restrict__ o, float* __restrict__ states,
    int T, int Hk, int Hv, int l2norm, float q_scale) {
    constexpr int NT = NTHR;
    constexpr int CG = D / 4;     // float4 column groups per row
    constexpr int RG = NT / CG;   // row groups
    constexpr int RPT = D / RG;   // rows per thread
    static_assert(RPT * RG == D && CG * RG == NT, "decode tiling");

    const int bh = blockIdx.x;    // b * Hv + h
    const int b = bh / Hv;
    const int h = bh - b * Hv;
    const int hk = h / (Hv / Hk);
    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int rg = tid / CG;

    __shared__ float kh[D];
    __shared__ float qh[D];
    __shared__ float red[2][RG][D];
    __shared__ float wsum[NT / 64][3];
    __shared__ float dl[D];

    float* S = state + (size_t)bh * D * D;

    // 1. stream this head's state into registers (all loads in flight at once)
    float4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        s[i] = *reinterpret_cast<const float4*>(S + (size_t)(rg + RG * i) * D + 4 * cg);

    const int NTOK = MULTI ? T : 1;   // a single step compiles to straight-line code
    for (int t = 0; t < NTOK; ++t) {
        if (t > 0) __syncthreads();   // the previous token is done with kh, qh, dl
        const size_t bt_idx = (size_t)b * T + t;   // (sequence, token)
        const size_t row = bt_idx * Hv + h;        // (sequence, token, value head)

        // 2. q, k of the key head, normalised in fp32
        float kv = 0.f, qv = 0.f;
        if (tid < D) {
            const size_t off = (bt_idx * Hk + hk) * D + tid;
            kv = to_f32(k[off]);
            qv = to_f32(q[off]);
        }
        float ssk = group_sum<64>(kv * kv);
        float ssq = group_sum<64>(qv * qv);
        if ((tid & 63) == 0) {
            wsum[tid >> 6][0] = ssk;
            wsum[tid >> 6][1] = ssq;
        }
        __syncthreads();
        float rk = 1.f, rq = 1.f;
        if (l2norm) {
            float tk = 0.f, tq = 0.f;
    #pragma unroll
            for (int w = 0; w < (D + 63) / 64; ++w) {
                tk += wsum[w][0];
                tq += wsum[w][1];
            }
            rk = inv_l2(tk);
            rq = inv_l2(tq);
        }
        if (tid < D) {
            kh[tid] = kv * rk;
            qh[tid] = qv * rq;
        }
        __syncthreads();
        // k_hat . q_hat (needed by the fused output identity)
        float kq_part = (tid < D) ? kh[tid] * qh[tid] : 0.f;
        kq_part = group_sum<64>(kq_part);
        if ((tid & 63) == 0) wsum[tid >> 6][2] = kq_part;

        // 3. per-thread partial reads a = S^T k, c = S^T q over its rows
        float pa[4] = {0.f, 0.f, 0.f, 0.f}, pc[4] = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const float kr = kh[rg + RG * i];
            const float qr = qh[rg + RG * i];
            pa[0] += s[i].x * kr; pa[1] += s[i].y * kr; pa[2] += s[i].z * kr; pa[3] += s[i].w * kr;
            pc[0] += s[i].x * qr; pc[1] += s[i].y * qr; pc[2] += s[i].z * qr; pc[3] += s[i].w * qr;
        }
    #pragma unroll
        for (int c = 0; c < 4; ++c) {
            red[0][rg][4 * cg + c] = pa[c];
            red[1][rg][4 * cg + c] = pc[c];
        }
        __syncthreads();

        // 4. column totals, delta and the output (one thread per column)
        float lgv = log_g[row], bt = beta[row];
        if (A_log) {   // raw projections a, b
            const int h = bh % Hv;
            lgv = raw_log_decay(lgv, A_log[h], dt_bias[h]);
            bt = raw_beta(bt);
        }
        const float g = expf(lgv);
        if (tid < D) {
            float a = 0.f, c = 0.f;
    #pragma unroll
            for (int r = 0; r < RG; ++r) {
                a += red[0][r][tid];
                c += red[1][r][tid];
            }
            float kq = 0.f;
    #pragma unroll
            for (int w = 0; w < (D + 63) / 64; ++w) kq += wsum[w][2];
            const float vj = to_f32(v[row * D + tid]);
            const float delta = bt * (vj - g * a);
            dl[tid] = delta;
            o[row * D + tid] = from_f32<TIn>(q_scale * (g * c + delta * kq));
        }
        __syncthreads();

        // 5. S <- g S + k delta^T (and the per-token state when asked for)
        const float4 d4 = *reinterpret_cast<const float4*>(&dl[4 * cg]);
    #pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const float kr = kh[rg + RG * i];
            float4 n;
            n.x = g * s[i].x + kr * d4.x;
            n.y = g * s[i].y + kr * d4.y;
            n.z = g * s[i].z + kr * d4.z;
            n.w = g * s[i].w + kr * d4.w;
            if (MULTI)
                s[i] = n;
            else   // a single step writes back over the same addresses at once
                *reinterpret_cast<float4*>(S + (size_t)(rg + RG * i) * D + 4 * cg) = n;
        }
        if (MULTI && states) {
            float* St = states + row * D * D;
    #pragma unroll
            for (int i = 0; i < RPT; ++i)
                *reinterpret_cast<float4*>(St + (size_t)(rg + RG * i) * D + 4 * cg) = s[i];
        }
    }   // tokens

    if (MULTI) {   // the state back over the same addresses
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            *reinterpret_cast<float4*>(S + (size_t)(rg + RG * i) * D + 4 * cg) = s[i];
    }
}

template <int D, typename TIn, int NTHR>
static void launch_single(const DecodeArgs& a, int blocks, hipStream_t stream) {
    hipLaunchKernelGGL((decode_step_kernel<D, TIn, false, NTHR>), dim3(blocks), dim3(NTHR), 0, stream,
                       static_cast<const TIn*>(a.q), static_cast<const TIn*>(a.k),
                       static_cast<const TIn*>(a.v), a.log_g, a.beta, a.A_log, a.dt_bias,
                       a.state, static_cast<TIn*>(a.o), nullptr, 1, a.Hk, a.Hv, a.l2norm, a.q_scale);
}

// bytes of decode state beyond which a single step streams it from HBM
constexpr size_t kInfinityCacheBytes = size_t(256) << 20;

template <int D, typename TIn>
static hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    const int blocks = a.B * a.Hv;
    if (blocks == 0 || a.T == 0) return hipSuccess;
    if (a.T == 1 && !a.states) {
        if constexpr (D == 128) {
            const size_t state_bytes = (size_t)blocks * D * D * sizeof(float);
            if (state_bytes > kInfinityCacheBytes) launch_single<D, TIn, 1024>(a, blocks, stream);
            else launch_single<D, TIn, 512>(a, blocks, stream);
        } else {
            launch_single<D, TIn, 256>(a, blocks, stream);
        }
    } else
        hipLaunchKernelGGL((decode_step_kernel<D, TIn, true, 256>), dim3(blocks), dim3(256), 0, stream,
                           static_cast<const TIn*>(a.q), static_cast<const TIn*>(a.k),
                           static_cast<const TIn*>(a.v), a.log_g, a.beta, a.A_log, a.dt_bias,
                           a.state, static_cast<TIn*>(a.o), a.states, a.T, a.Hk, a.Hv, a.l2norm,
                           a.q_scale);
    return hipGetLastError();
}

hipError_t launch_decode_step(const DecodeArgs& a, hipStream_t stream) {
    if (a.D == 128)
        return a.bf16 ? launch_decode<128, bf16_t>(a, stream) : launch_decode<128, float>(a, stream);
    return a.bf16 ? launch_decode<64, bf16_t>(a, stream) : launch_decode<64, float>(a, stream);
}

}  // namespace gdn

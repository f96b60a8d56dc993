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
// Mapping: a workgroup of NT threads per column block of CB state columns
// of one (b, h) at a time (CB = D: the whole head).  Columns are independent (every
// reduction runs over rows), so a block needs no other workgroup.  A thread
// owns a float4 column strip of D/RG rows (RG = row groups), held in VGPRs
// between the read and the write; rows are interleaved so each wave load
// covers whole rows of the block (coalesced 16-byte accesses).  Column sums
// over the rows combine per-thread partials in LDS in two fixed-order stages
// (deterministic): every thread adds 4 row groups of one column, then one
// thread per column adds the RG/4 parts.
//
// A single step at head dim 128 runs 1024 threads per head (4 rows per
// thread, at most 64 VGPRs: two workgroups per CU) with non-temporal state
// loads and stores through a buffer resource on the head.  The workgroups are
// persistent: as many as fit at once, each walking heads blockIdx.x,
// + gridDim.x, ...  The state is streamed: in a model the other layers'
// states pass through the caches between two steps of one layer.  Measured on
// MI355X, B=128 and B=64 with the state cycled over four buffers (both past
// the 256 MB Infinity Cache): 133 and 68 us per step, 6.08 and 5.97 TB/s.
// One workgroup per head (6144 of them at B=128) took 139 and 71 us: a
// memory-only kernel of the same shape loses the same ~9 us to starting 12
// workgroups per slot.  Prefetching the next head while storing this one,
// one workgroup per CU, 256 to 512 threads per block of 32 to 128 columns
// (partial rows scatter the accesses) and plain accesses were all slower.
// Plain accesses keep a state that fits the Infinity Cache resident from step
// to step (6.5 TB/s at B=64 on one buffer), which a model never sees.
// Several tokens per call use 256 threads (non-temporal state at head dim
// 128); a single step at head dim 64 uses 256 threads and plain accesses.
#include <algorithm>

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

typedef __attribute__((ext_vector_type(4))) float f32v4;

// 16-byte state access; NTS bit 0: non-temporal loads, bit 1: non-temporal
// stores (streaming: no reuse expected)
template <int NTS>
__device__ __forceinline__ float4 load_state(const float* p) {
    if constexpr ((NTS & 1) != 0) {
        const f32v4 x = __builtin_nontemporal_load(reinterpret_cast<const f32v4*>(p));
        return make_float4(x[0], x[1], x[2], x[3]);
    } else {
        return *reinterpret_cast<const float4*>(p);
    }
}

template <int NTS>
__device__ __forceinline__ void store_state(float* p, const float4& v) {
    if constexpr ((NTS & 2) != 0) {
        const f32v4 x = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(x, reinterpret_cast<f32v4*>(p));
    } else {
        *reinterpret_cast<float4*>(p) = v;
    }
}

template <int D, typename TIn, bool MULTI, int NTHR, int CB, int NTS>
__global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(MULTI ? 1 : 8))) void decode_step_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const float* __restrict__ log_g, const float* __restrict__ beta,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias,
    float* __restrict__ state, TIn* __restrict__ o, float* __restrict__ states,
    int T, int Hk, int Hv, int l2norm, float q_scale, int units) {
    constexpr int NT = NTHR;
    constexpr int NCB = D / CB;   // column blocks per (b, h): one workgroup each
    constexpr int CG = CB / 4;    // float4 column groups per row of the block
    constexpr int RG = NT / CG;   // row groups
    constexpr int RPT = D / RG;   // rows per thread
    static_assert(RPT * RG == D && CG * RG == NT && NCB * CB == D, "decode tiling");
    static_assert(NT >= D, "one thread per element of q and k");
    static_assert(!MULTI || NCB == 1, "several tokens per call keep the whole head");

    __shared__ __align__(16) float kh[D];
    __shared__ __align__(16) float qh[D];
    constexpr int NP = RG / 4;   // column sums in two stages: NP parts of 4 row groups
    static_assert(NP * 4 == RG && NP * CB == NT, "two-stage column sum");
    __shared__ __align__(16) float red[2][RG][CB];
    __shared__ __align__(16) float red2[2][NP][CB];
    __shared__ __align__(16) float wsum[NT / 64][3];
    __shared__ __align__(16) float dl[CB];   // read as float4

    // A single step's workgroup walks units (b, h, column block) blockIdx.x,
    // + gridDim.x, ... (the grid never exceeds the units); several tokens per
    // call take one unit per workgroup, and the loop folds away.  No barrier
    // is needed between two units: every shared array is written in a unit
    // only after a barrier that follows its last read in the previous unit,
    // or (wsum[][0..1]) long after it.
    int unit = blockIdx.x;
    do {
        // a single step passes the thread index through an empty asm in every
        // unit, so the addresses derived from it are not hoisted out of the
        // loop and kept live across it (VGPR spills at the 64-register cap)
        int tid = threadIdx.x;
        if constexpr (!MULTI) asm volatile("" : "+v"(tid));
        const int cg = tid % CG;
        const int rg = tid / CG;
        const int bh = unit / NCB;   // b * Hv + h
        const int c0 = (unit - bh * NCB) * CB;   // first state column of the block
        const int b = bh / Hv;
        const int h = bh - b * Hv;
        const int hk = h / (Hv / Hk);
        float* S = state + (size_t)bh * D * D + c0;

        // A single step issues its small loads (q, k, v, the gates) before the
        // state: memory waits complete in issue order, so the norms below can
        // then run while the state is still in flight.  Every lane loads (the
        // indices are clamped), so no branch splits the waits.
        TIn k0 = TIn(), q0 = TIn(), v0 = TIn();
        float lg0 = 0.f, bt0 = 0.f;
        if constexpr (!MULTI) {
            const size_t off = ((size_t)b * Hk + hk) * D + (tid < D ? tid : D - 1);
            k0 = k[off];
            q0 = q[off];
            v0 = v[(size_t)bh * D + c0 + (tid < CB ? tid : CB - 1)];
            lg0 = log_g[bh];
            bt0 = beta[bh];
        }

        // 1. stream this block of the state into registers (all loads in flight at
        //    once).  A single step addresses it through a buffer resource on the
        //    block: one VGPR offset per thread, the row step in a scalar offset.
        float4 s[RPT];
        __amdgpu_buffer_rsrc_t srs;
        const int voff = ((rg * D) + 4 * cg) * 4;   // bytes
        if constexpr (!MULTI) {
            srs = __builtin_amdgcn_make_buffer_rsrc(S, (short)0, (D * D - c0) * 4, 0x00020000);
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const f32v4 x = __builtin_amdgcn_raw_buffer_load_b128(srs, voff, i * RG * D * 4,
                                                                      (NTS & 1) ? 2 : 0);
                s[i] = make_float4(x[0], x[1], x[2], x[3]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < RPT; ++i) s[i] = load_state<NTS>(S + (size_t)(rg + RG * i) * D + 4 * cg);
        }

        const int NTOK = MULTI ? T : 1;   // a single step compiles to straight-line code
        for (int t = 0; t < NTOK; ++t) {
            if (t > 0) __syncthreads();   // the previous token is done with kh, qh, dl
            const size_t bt_idx = (size_t)b * T + t;   // (sequence, token)
            const size_t row = bt_idx * Hv + h;        // (sequence, token, value head)

            // 2. q, k of the key head, normalised in fp32
            float kv = 0.f, qv = 0.f;
            if constexpr (!MULTI) {
                kv = tid < D ? to_f32(k0) : 0.f;
                qv = tid < D ? to_f32(q0) : 0.f;
            } else if (tid < D) {
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
            {   // every thread: one column's sum over 4 row groups
                const int col = tid % CB, part = tid / CB;
                float a4 = 0.f, c4 = 0.f;
        #pragma unroll
                for (int r = 0; r < 4; ++r) {
                    a4 += red[0][4 * part + r][col];
                    c4 += red[1][4 * part + r][col];
                }
                red2[0][part][col] = a4;
                red2[1][part][col] = c4;
            }
            __syncthreads();

            // 4. column totals, delta and the output (one thread per column)
            float lgv = MULTI ? log_g[row] : lg0, bt = MULTI ? beta[row] : bt0;
            if (A_log) {   // raw projections a, b
                lgv = raw_log_decay(lgv, A_log[h], dt_bias[h]);
                bt = raw_beta(bt);
            }
            const float g = expf(lgv);
            if (tid < CB) {
                float a = 0.f, c = 0.f;
        #pragma unroll
                for (int r = 0; r < NP; ++r) {
                    a += red2[0][r][tid];
                    c += red2[1][r][tid];
                }
                float kq = 0.f;
        #pragma unroll
                for (int w = 0; w < (D + 63) / 64; ++w) kq += wsum[w][2];
                const float vj = MULTI ? to_f32(v[row * D + c0 + tid]) : to_f32(v0);
                const float delta = bt * (vj - g * a);
                dl[tid] = delta;
                o[row * D + c0 + tid] = from_f32<TIn>(q_scale * (g * c + delta * kq));
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
                if (MULTI) {
                    s[i] = n;
                } else {   // a single step writes back over the same addresses at once
                    const f32v4 x = {n.x, n.y, n.z, n.w};
                    __builtin_amdgcn_raw_buffer_store_b128(x, srs, voff, i * RG * D * 4, (NTS & 2) ? 2 : 0);
                }
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
            for (int i = 0; i < RPT; ++i) store_state<NTS>(S + (size_t)(rg + RG * i) * D + 4 * cg, s[i]);
        }
    } while (!MULTI && (unit += gridDim.x) < units);
}

// A single step runs persistent workgroups, as many as fit on the device at
// once, each walking its share of the units: one workgroup per unit spent
// ~9 us of a 403 MB step (B=128) on starting 6144 workgroups, 12 per slot.
template <int D, typename TIn, int NTHR, int CB, int NTS>
static hipError_t launch_single(const DecodeArgs& a, hipStream_t stream) {
    const auto kern = decode_step_kernel<D, TIn, false, NTHR, CB, NTS>;
    static const int per_cu = [&] {
        int n = 0;
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, NTHR, 0) == hipSuccess && n > 0 ? n : 1;
    }();
    int dev = 0, cus = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    const long long units = (long long)a.B * a.Hv * (D / CB);
    const int blocks = (int)std::min<long long>(units, (long long)per_cu * std::max(cus, 1));
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(NTHR), 0, stream, static_cast<const TIn*>(a.q),
                       static_cast<const TIn*>(a.k), static_cast<const TIn*>(a.v), a.log_g, a.beta,
                       a.A_log, a.dt_bias, a.state, static_cast<TIn*>(a.o), nullptr, 1, a.Hk, a.Hv,
                       a.l2norm, a.q_scale, (int)units);
    return hipGetLastError();
}

template <int D, typename TIn>
static hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    const int heads = a.B * a.Hv;
    if (heads == 0 || a.T == 0) return hipSuccess;
    if (a.T == 1 && !a.states) {
        if constexpr (D == 128)
            return launch_single<D, TIn, 1024, D, 3>(a, stream);   // non-temporal state loads and stores
        else
            return launch_single<D, TIn, 256, D, 0>(a, stream);
    }
    // several tokens per call: 256 threads per head (1024 threads, the single
    // step's form, ran twice as long: the per-token barriers and reductions
    // dominate), non-temporal state at head dim 128 (2-4% faster)
    hipLaunchKernelGGL((decode_step_kernel<D, TIn, true, 256, D, D == 128 ? 3 : 0>), dim3(heads), dim3(256), 0, stream,
                       static_cast<const TIn*>(a.q), static_cast<const TIn*>(a.k),
                       static_cast<const TIn*>(a.v), a.log_g, a.beta, a.A_log, a.dt_bias, a.state,
                       static_cast<TIn*>(a.o), a.states, a.T, a.Hk, a.Hv, a.l2norm, a.q_scale, heads);
    return hipGetLastError();
}

hipError_t launch_decode_step(const DecodeArgs& a, hipStream_t stream) {
    if (a.D == 128)
        return a.bf16 ? launch_decode<128, bf16_t>(a, stream) : launch_decode<128, float>(a, stream);
    return a.bf16 ? launch_decode<64, bf16_t>(a, stream) : launch_decode<64, float>(a, stream);
}

}  // namespace gdn

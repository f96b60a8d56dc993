// prefill_generic.hip -- chunked gated-delta-rule prefill, fp32 arithmetic.
//
// The portable kernel: every supported head dim (64, 128), chunk (16, 32, 64)
// and storage dtype, computing in fp32 throughout.  It serves fp32 inputs
// (where fp32 products are needed to meet a 1e-4 max-abs bar) and is the
// fallback for shapes the MFMA kernel does not cover.
//
// Chunk form (per value head, chunk of L <= C tokens starting from state S;
// gamma_r = sum_{s<=r} log g_s inside the chunk, Gamma_r = exp(gamma_r)):
//   A_rs  = beta_r exp(gamma_r - gamma_s) (k_r . k_s)      s <  r   (decay-masked beta K K^T)
//   M_rs  = exp(gamma_r - gamma_s) (q_r . k_s)             s <= r
//   X_r   = beta_r (v_r - Gamma_r S^T k_r)
//   (I + A) Delta = X      solved directly by forward substitution
//   o_r   = Gamma_r S^T q_r + sum_{s<=r} M_rs Delta_s
//   S'    = Gamma_L S + sum_s exp(gamma_L - gamma_s) k_s Delta_s^T
// This is the token recurrence of "Qwen3.5 Gated Delta Net NKI Kernel for AWS
// Neuron" ("How It Works") unrolled over a chunk; the direct solve (not the
// Neumann power series) follows "Qwen3.6: Fused DeltaNet Direct-Solve
// Follow-Up" ("Why This Exists", "Implementation Details").  Only decay
// differences gamma_r - gamma_s with s <= r are exponentiated, so nothing
// overflows for log g <= 0.
//
// Mapping: one workgroup per (b, value head, 32-column block of the state);
// columns of the state evolve independently, so the blocks never communicate.
// Everything of a chunk lives in LDS; the state block stays in LDS across all
// chunks and touches HBM only at the start (h0), the end (hT) and at the
// optional checkpoints.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <int D, int C, int BV, typename TIn>
__global__ __launch_bounds__(256) void prefill_generic_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const float* __restrict__ log_g, const float* __restrict__ beta,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias,
    const float* h0, float* hT, TIn* __restrict__ o,
    int T, int Hk, int Hv, int l2norm, float q_scale,
    float* __restrict__ ckpt, int ckpt_every, int nck, const int* __restrict__ cu, long long total) {
    constexpr int NT = 256;
    constexpr int TPR = NT / C;   // threads per chunk row (normalisation)
    constexpr int P = NT / BV;    // partial-sum lanes per column (solve)
    static_assert(C <= 64 && NT % C == 0 && NT % BV == 0 && P <= 64, "generic tiling");

    __shared__ float Ks[C][D];
    __shared__ float Qs[C][D];
    __shared__ float Ss[D][BV];
    __shared__ float Xs[C][BV];
    __shared__ float Am[C][C];
    __shared__ float Mm[C][C];
    __shared__ float lgs[C], bts[C], gam[C], Gm[C], Wd[C];

    const int tid = threadIdx.x;
    const int bh = blockIdx.x;
    const int b = bh / Hv;
    const int h = bh - b * Hv;
    const int hk = h / (Hv / Hk);
    const int j0 = blockIdx.y * BV;
    const size_t state_base = (size_t)bh * D * D;
    size_t tb0;   // first token of sequence b
    int Tb;       // its length (T for equal-length batches)
    seq_span(cu, b, T, total, tb0, Tb);

    for (int e = tid; e < D * BV; e += NT) {
        const int i = e / BV, j = e % BV;
        Ss[i][j] = h0 ? h0[state_base + (size_t)i * D + j0 + j] : 0.f;
    }

    for (int t0 = 0; t0 < Tb; t0 += C) {
        const int L = min(C, Tb - t0);
        __syncthreads();  // previous chunk fully consumed
        for (int e = tid; e < C * D; e += NT) {
            const int r = e / D, i = e % D;
            float kv = 0.f, qv = 0.f;
            if (r < L) {
                const size_t off = ((tb0 + t0 + r) * Hk + hk) * D + i;
                kv = to_f32(k[off]);
                qv = to_f32(q[off]);
            }
            Ks[r][i] = kv;
            Qs[r][i] = qv;
        }
        for (int e = tid; e < C * BV; e += NT) {
            const int r = e / BV, j = e % BV;
            Xs[r][j] = (r < L) ? to_f32(v[((tb0 + t0 + r) * Hv + h) * D + j0 + j]) : 0.f;
        }
        if (tid < C) {
            const bool in = tid < L;
            const size_t gi = (tb0 + t0 + tid) * Hv + h;
            float lgv = in ? log_g[gi] : 0.f, btv = in ? beta[gi] : 0.f;
            if (A_log && in) {   // raw projections a, b
                lgv = raw_log_decay(lgv, A_log[h], dt_bias[h]);
                btv = raw_beta(btv);
            }
            lgs[tid] = chunk_log_decay(lgv);   // padding rows: g = 1, beta = 0, k = q = 0
            bts[tid] = btv;
        }
        __syncthreads();

        if (l2norm) {
            const int r = tid / TPR, p = tid % TPR;
            float sk = 0.f, sq = 0.f;
            for (int i = p; i < D; i += TPR) {
                sk += Ks[r][i] * Ks[r][i];
                sq += Qs[r][i] * Qs[r][i];
            }
            sk = group_sum<TPR>(sk);
            sq = group_sum<TPR>(sq);
            const float rk = inv_l2(sk), rq = inv_l2(sq);
            for (int i = p; i < D; i += TPR) {
                Ks[r][i] *= rk;
                Qs[r][i] *= rq;
            }
        }
        if (tid < 64) {  // inclusive scan of the log-decays
            float x = (tid < C) ? lgs[tid] : 0.f;
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) {
                const float y = __shfl_up(x, m, 64);
                if (tid >= m) x += y;
            }
            if (tid < C) gam[tid] = x;
        }
        __syncthreads();
        if (tid < C) {
            Gm[tid] = expf(gam[tid]);
            Wd[tid] = expf(gam[C - 1] - gam[tid]);
        }

        // decay-masked Gram matrices
        for (int e = tid; e < C * C; e += NT) {
            const int r = e / C, s = e % C;
            float a = 0.f, m = 0.f;
            if (s <= r) {
                float dkk = 0.f, dqk = 0.f;
                for (int i = 0; i < D; ++i) {
                    const float ks = Ks[s][i];
                    dkk += Ks[r][i] * ks;
                    dqk += Qs[r][i] * ks;
                }
                const float dec = expf(gam[r] - gam[s]);
                if (s < r) a = bts[r] * dec * dkk;
                m = dec * dqk;
            }
            Am[r][s] = a;
            Mm[r][s] = m;
        }
        __syncthreads();
        // right-hand side X = beta (V - Gamma K S)
        for (int e = tid; e < C * BV; e += NT) {
            const int r = e / BV, j = e % BV;
            float acc = 0.f;
            for (int i = 0; i < D; ++i) acc += Ks[r][i] * Ss[i][j];
            Xs[r][j] = bts[r] * (Xs[r][j] - Gm[r] * acc);
        }
        __syncthreads();
        // direct forward substitution (I + A) Delta = X, in place
        {
            const int j = tid / P, p = tid % P;
            for (int r = 1; r < L; ++r) {
                float part = 0.f;
                for (int s = p; s < r; s += P) part += Am[r][s] * Xs[s][j];
                part = group_sum<P>(part);
                if (p == 0) Xs[r][j] -= part;   // rows < r are only read this pass
                __syncthreads();
            }
        }
        // outputs (from the state entering the chunk)
        for (int e = tid; e < C * BV; e += NT) {
            const int r = e / BV, j = e % BV;
            if (r < L) {
                float acc = 0.f;
                for (int i = 0; i < D; ++i) acc += Qs[r][i] * Ss[i][j];
                acc *= Gm[r];
                for (int s = 0; s <= r; ++s) acc += Mm[r][s] * Xs[s][j];
                o[((tb0 + t0 + r) * Hv + h) * D + j0 + j] = from_f32<TIn>(q_scale * acc);
            }
        }
        __syncthreads();
        // state hand-off; a checkpoint slot receives the state after every
        // ckpt_every tokens and after the last token
        const float GL = Gm[C - 1];
        const int done = t0 + L;
        float* ck = nullptr;
        if (ckpt && (done % ckpt_every == 0 || done == Tb))
            ck = ckpt + (((size_t)b * nck + (done + ckpt_every - 1) / ckpt_every - 1) * Hv + h) * D * D;
        for (int e = tid; e < D * BV; e += NT) {
            const int i = e / BV, j = e % BV;
            float acc = GL * Ss[i][j];
            for (int s = 0; s < L; ++s) acc += Wd[s] * Ks[s][i] * Xs[s][j];
            Ss[i][j] = acc;
            if (ck) ck[(size_t)i * D + j0 + j] = acc;
        }
    }
    __syncthreads();
    if (hT) {
        for (int e = tid; e < D * BV; e += NT) {
            const int i = e / BV, j = e % BV;
            hT[state_base + (size_t)i * D + j0 + j] = Ss[i][j];
        }
    }
}

template <int D, int C, typename TIn>
static hipError_t launch_generic(const PrefillArgs& a, hipStream_t stream) {
    constexpr int BV = 32;
    dim3 grid(a.B * a.Hv, D / BV);
    hipLaunchKernelGGL((prefill_generic_kernel<D, C, BV, TIn>), grid, dim3(256), 0, stream,
                       static_cast<const TIn*>(a.q), static_cast<const TIn*>(a.k),
                       static_cast<const TIn*>(a.v), a.log_g, a.beta, a.A_log, a.dt_bias, a.h0, a.hT,
                       static_cast<TIn*>(a.o), a.T, a.Hk, a.Hv, a.l2norm, a.q_scale,
                       a.ckpt, a.ckpt_every, a.nck, a.cu, a.total);
    return hipGetLastError();
}

template <int D, typename TIn>
static hipError_t launch_generic_c(const PrefillArgs& a, hipStream_t stream) {
    switch (a.C) {
        case 16: return launch_generic<D, 16, TIn>(a, stream);
        case 32: return launch_generic<D, 32, TIn>(a, stream);
        default: return launch_generic<D, 64, TIn>(a, stream);
    }
}

hipError_t launch_prefill_generic(const PrefillArgs& a, hipStream_t stream) {
    if (a.B * a.Hv == 0) return hipSuccess;
    if (a.D == 128)
        return a.bf16 ? launch_generic_c<128, bf16_t>(a, stream) : launch_generic_c<128, float>(a, stream);
    return a.bf16 ? launch_generic_c<64, bf16_t>(a, stream) : launch_generic_c<64, float>(a, stream);
}

// ---------------------------------------------------------------------------

__global__ void state_copy_kernel(const float* __restrict__ src, float* __restrict__ dst, size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src ? src[i] : 0.f;
}

hipError_t launch_state_copy(const float* h0, float* hT, size_t n, hipStream_t stream) {
    if (!hT || n == 0 || h0 == hT) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, h0, hT, n);
    return hipGetLastError();
}

}  // namespace gdn

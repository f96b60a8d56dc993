// prefill_mfma.hip -- chunked gated-delta-rule prefill on bf16 MFMA (gfx950).
//
// Shape: head dim 128, chunk 64, bf16 q/k/v/o, fp32 gates and state.
//
// Per value head and chunk of C = 64 tokens starting from state S (128 x dv):
//   gamma_r = sum_{s<=r} log g_s (in-chunk), Gamma_r = exp(gamma_r),
//   rk_r, rq_r = 1 / max(|k_r|, 1e-6), 1 / max(|q_r|, 1e-6) (L2 normalisation),
//   A_rs = beta_r exp(gamma_r - gamma_s) rk_r rk_s (k_r . k_s)   s <  r   decay-masked beta K K^T
//   P_rs = exp(gamma_r - gamma_s) rq_r rk_s (q_r . k_s)           s <= r
//   X    = diag(beta) (V - diag(Gamma rk) K S)                   right-hand side
//   (I + A) Delta = X                                             direct solve
//   O    = diag(Gamma rq) Q S + P Delta
//   S'   = Gamma_C S + K^T diag(exp(gamma_C - gamma) rk) Delta
// This is the token recurrence of "Qwen3.5 Gated Delta Net NKI Kernel for AWS
// Neuron" ("How It Works") unrolled over a chunk.  The unit lower-triangular
// system is solved directly -- forward substitution inside 16x16 diagonal
// blocks, then block forward substitution with MFMA -- never with the Neumann
// power series ("Qwen3.6: Fused DeltaNet Direct-Solve Follow-Up", "Why This
// Exists", "Implementation Details").  Only exp(gamma_r - gamma_s) with s <= r
// is formed, so nothing overflows for log g <= 0.
//
// Mapping: one workgroup (4 waves) per (b, value head, 32-column block of the
// state).  Columns of the state are independent, so blocks never communicate.
// The fp32 state block lives in MFMA accumulator layout in registers for the
// whole sequence (wave w owns rows 32w..32w+31); it is read from h0 once and
// written to hT once.  Chunk data is staged in LDS with padded rows so that the
// 16-byte operand reads of 16 lanes hit distinct banks.  Raw bf16 q and k are
// the MFMA operands (exact); the normalisation scales are applied in fp32 to
// products, so the only bf16 roundings are of S, X, Delta, A, P and the 16x16
// inverses used as operands.  Workgroups sharing a key head are placed on one
// XCD so their repeated q/k chunk reads hit the same L2.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace mfma_prefill {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int D = 128;   // head dim (dk = dv)
constexpr int C = 64;    // chunk
constexpr int BV = 32;   // state columns per workgroup
constexpr int NT = 256;  // threads
constexpr int SK = D + 8;   // padded row stride (elements) of [C][D] bf16 arrays
constexpr int SC = C + 8;   // padded row stride of [*][C] bf16 arrays
constexpr int ST = 20;      // row stride of the 16x16 bf16 inverses

struct Smem {
    uint16_t Kr[C][SK];      // raw k rows of the chunk (bf16)
    uint16_t Qr[C][SK];      // raw q rows
    uint16_t Kt[D][SC];      // k transposed: [i][s]
    uint16_t Vt[BV][SC];     // v block transposed: [j][s]
    uint16_t Sbt[BV][SK];    // state block transposed, bf16: [j][i]
    uint16_t An[C][SC];      // -A (bf16) [r][s]
    uint16_t Pb[C][SC];      // P (bf16) [r][s]
    uint16_t Dt[BV][SC];     // Delta^T (bf16) [j][s]
    uint16_t Dw[BV][SC];     // (exp(gamma_C - gamma) rk Delta)^T (bf16) [j][s]
    uint16_t Tb[4][16][ST];  // (I + A_ii)^-1 (bf16), diagonal blocks
    float Af[4][16][17];     // A_ii (fp32), diagonal blocks
    float rk[C], rq[C], bt[C], gam[C], Gm[C], Wd[C];
    float lgn[2][C], btn[2][C];  // gates of the current / next chunk
};

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ short bfbits(float f) {
    return __builtin_bit_cast(short, static_cast<__bf16>(f));
}
__device__ __forceinline__ s16x4 pack4(f32x4 v) {
    s16x4 r;
    r[0] = bfbits(v[0]); r[1] = bfbits(v[1]); r[2] = bfbits(v[2]); r[3] = bfbits(v[3]);
    return r;
}
__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ s16x4 ld4(const uint16_t* p) {
    return *reinterpret_cast<const s16x4*>(p);
}
__device__ __forceinline__ void st4(uint16_t* p, s16x4 v) {
    *reinterpret_cast<s16x4*>(p) = v;
}

// x if keep, else zero (component-wise, no control flow)
__device__ __forceinline__ uint4 mask4(uint4 x, bool keep) {
    const uint32_t m = keep ? 0xffffffffu : 0u;
    return make_uint4(x.x & m, x.y & m, x.z & m, x.w & m);
}

// Lower-triangular 16x16 tiles of a 64x64 matrix, in an order the waves split.
__device__ __forceinline__ void tile_of(int idx, int& a, int& b) {
    // (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3)
    a = (idx >= 1) + (idx >= 3) + (idx >= 6);
    b = idx - (a * (a + 1)) / 2;
}

__global__ __launch_bounds__(NT) void prefill_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float* __restrict__ log_g, const float* __restrict__ beta,
    const float* h0, float* hT, bf16_t* __restrict__ o,
    int T, int Hk, int Hv, int l2norm, float q_scale, int xcd_remap) {
    __shared__ Smem sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int g = lane >> 4;    // lane group (0..3)
    const int n = lane & 15;    // lane column in a 16-wide tile

    int lid = blockIdx.x;
    if (xcd_remap) {  // consecutive logical ids on one XCD (dispatch is round-robin over 8)
        const int per = gridDim.x >> 3;
        lid = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    }
    const int bh = lid >> 2;
    const int j0 = (lid & 3) * BV;
    const int b = bh / Hv;
    const int h = bh - b * Hv;
    const int hk = h / (Hv / Hk);
    const size_t state_base = (size_t)bh * D * D;

    // ---- state block in accumulator layout: tile (a, c) holds rows
    //      32w + 16a + 4g + t and columns j0 + 16c + n
    f32x4 S[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                S[a][c][t] = h0 ? h0[state_base + (size_t)(32 * w + 16 * a + 4 * g + t) * D + j0 + 16 * c + n]
                                : 0.f;

    // ---- prefetch registers for one chunk
    uint4 pk[4], pq[4], pv;
    float plg = 0.f, pbt = 0.f;
    // Loads are branch-free (rows past the end read a clamped valid row and are
    // zeroed when staged), so no wait is forced right after issuing them.
    auto prefetch = [&](int t0) {
        const int last = min(C, T - t0) - 1;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int seg = tid + NT * u;       // 0..1023: (row, 8-element column group)
            const int r = min(seg >> 4, last);
            const int c8 = (seg & 15) * 8;
            const size_t off = (((size_t)b * T + t0 + r) * Hk + hk) * D + c8;
            pk[u] = *reinterpret_cast<const uint4*>(k + off);
            pq[u] = *reinterpret_cast<const uint4*>(q + off);
        }
        {
            const int r = min(tid >> 2, last);
            const int c8 = (tid & 3) * 8;
            pv = *reinterpret_cast<const uint4*>(v + (((size_t)b * T + t0 + r) * Hv + h) * D + j0 + c8);
        }
        {
            const size_t gi = ((size_t)b * T + t0 + min(lane, last)) * Hv + h;
            plg = log_g[gi];
            pbt = beta[gi];
        }
    };

    if (T > 0) {
        prefetch(0);
        if (w == 0) {
            sm.lgn[0][lane] = plg;
            sm.btn[0][lane] = pbt;
        }
    }

    for (int t0 = 0; t0 < T; t0 += C) {
        const int L = min(C, T - t0);
        __syncthreads();  // (A) every reader of the previous chunk's LDS is done

        // ---- stage the chunk in LDS (rows >= L are zero: g = 1, beta = 0, q = k = v = 0)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int seg = tid + NT * u;
            const int r = seg >> 4;
            const int c8 = (seg & 15) * 8;
            *reinterpret_cast<uint4*>(&sm.Kr[r][c8]) = mask4(pk[u], r < L);
            *reinterpret_cast<uint4*>(&sm.Qr[r][c8]) = mask4(pq[u], r < L);
        }
        {
            const int r = tid >> 2;
            const int c8 = (tid & 3) * 8;
            const uint4 vv = mask4(pv, r < L);
            const uint32_t words[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
            for (int x = 0; x < 8; ++x)
                sm.Vt[c8 + x][r] = static_cast<uint16_t>(words[x >> 1] >> (16 * (x & 1)));
        }
        const int par = (t0 / C) & 1;
        const float lg_mine = (lane < L) ? sm.lgn[par][lane] : 0.f;
        const float bt_mine = (lane < L) ? sm.btn[par][lane] : 0.f;
        __syncthreads();  // (B)

        // next chunk's loads overlap everything below
        if (t0 + C < T) prefetch(t0 + C);

        // ---- row norms (4 threads per row) and the in-chunk decay scan (wave 0)
        {
            const int r = tid >> 2;
            const int p = tid & 3;
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const uint4 kk = *reinterpret_cast<const uint4*>(&sm.Kr[r][32 * p + 8 * x]);
                const uint4 qq = *reinterpret_cast<const uint4*>(&sm.Qr[r][32 * p + 8 * x]);
                const uint32_t kw[4] = {kk.x, kk.y, kk.z, kk.w};
                const uint32_t qw[4] = {qq.x, qq.y, qq.z, qq.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float k0 = __uint_as_float(kw[e] << 16), k1 = __uint_as_float(kw[e] & 0xffff0000u);
                    const float q0 = __uint_as_float(qw[e] << 16), q1 = __uint_as_float(qw[e] & 0xffff0000u);
                    sk += k0 * k0 + k1 * k1;
                    sq += q0 * q0 + q1 * q1;
                }
            }
            sk = group_sum<4>(sk);
            sq = group_sum<4>(sq);
            if (p == 0) {
                sm.rk[r] = l2norm ? inv_l2(sk) : 1.f;
                sm.rq[r] = l2norm ? inv_l2(sq) : 1.f;
            }
        }
        if (w == 0) {
            float x = lg_mine;
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) {
                const float y = __shfl_up(x, m, 64);
                if (lane >= m) x += y;
            }
            const float total = __shfl(x, 63, 64);
            sm.gam[lane] = x;
            sm.Gm[lane] = expf(x);
            sm.Wd[lane] = expf(total - x);
            sm.bt[lane] = bt_mine;
        }
        __syncthreads();  // (C)

        // ---- Gram tiles: 10 lower tiles of K K^T (-> -A) and 10 of Q K^T (-> P).
        //      Computed transposed (s on the M side) so each lane ends up with
        //      four consecutive s of one row r: 8-byte row-major writes.
#pragma unroll 1
        for (int task = w; task < 20; task += 4) {
            const bool is_qk = task >= 10;
            int a, bb;
            tile_of(is_qk ? task - 10 : task, a, bb);   // r-block a >= s-block bb
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const uint16_t* rowsB = is_qk ? &sm.Qr[16 * a + n][0] : &sm.Kr[16 * a + n][0];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 av = ld8(&sm.Kr[16 * bb + n][32 * ks + 8 * g]);   // rows s
                const bf16x8 bv = ld8(rowsB + 32 * ks + 8 * g);               // rows r
                acc = mfma32(av, bv, acc);
            }
            const int r = 16 * a + n;
            const float gr = sm.gam[r];
            const float sr = is_qk ? sm.rq[r] : sm.rk[r] * sm.bt[r];
            float val[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int s = 16 * bb + 4 * g + t;
                const bool keep = is_qk ? (s <= r) : (s < r);
                val[t] = keep ? expf(gr - sm.gam[s]) * sr * sm.rk[s] * acc[t] : 0.f;
            }
            const int s0 = 16 * bb + 4 * g;
            if (is_qk) {
                f32x4 pv4 = {val[0], val[1], val[2], val[3]};
                st4(&sm.Pb[r][s0], pack4(pv4));
                if (a == bb && (a == 0 || a == 2)) {  // upper neighbour read by P Delta: zero it
                    s16x4 z = {0, 0, 0, 0};
                    st4(&sm.Pb[r][s0 + 16], z);
                }
            } else {
                f32x4 nv = {-val[0], -val[1], -val[2], -val[3]};
                st4(&sm.An[r][s0], pack4(nv));
                if (a == bb) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) sm.Af[a][n][4 * g + t] = val[t];
                }
            }
        }

        // ---- k transposed ([i][s], operand of the state update), read from the
        //      staged rows: 8 two-byte reads of one column, one 16-byte write
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int task = tid + NT * u;
            const int i = task & (D - 1);
            const int s8 = (task >> 7) * 8;
            uint32_t wd[4];
#pragma unroll
            for (int x = 0; x < 4; ++x)
                wd[x] = static_cast<uint32_t>(sm.Kr[s8 + 2 * x][i]) |
                        (static_cast<uint32_t>(sm.Kr[s8 + 2 * x + 1][i]) << 16);
            *reinterpret_cast<uint4*>(&sm.Kt[i][s8]) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
        }

        // ---- state block -> bf16, transposed (operand of K S and Q S)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int c = 0; c < 2; ++c)
                st4(&sm.Sbt[16 * c + n][32 * w + 16 * a + 4 * g], pack4(S[a][c]));
        __syncthreads();  // (D)

        // ---- (I + A_ww)^-1 of diagonal block w by forward substitution; lane n = column
        if (lane < 16) {
            float tc[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == n) ? 1.f : 0.f;
#pragma unroll
                for (int s = 0; s < r; ++s) acc -= sm.Af[w][r][s] * tc[s];
                tc[r] = acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.Tb[w][r][n] = static_cast<uint16_t>(bfbits(tc[r]));
        }
        if (w == 0 && t0 + C < T) {  // gates of the next chunk (loaded by the prefetch)
            sm.lgn[par ^ 1][lane] = plg;
            sm.btn[par ^ 1][lane] = pbt;
        }
        __syncthreads();  // (E)

        // ---- waves 0,1: X = beta (V - Gamma rk K S), direct block solve -> Delta
        //      waves 2,3: Gamma rq Q S (first half of the output)
        const int ct = w & 1;                 // column tile of this wave
        f32x4 acc4[4];
        {
            const uint16_t* Abase = (w < 2) ? &sm.Kr[0][0] : &sm.Qr[0][0];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                acc4[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const bf16x8 av = ld8(Abase + (16 * a + n) * SK + 32 * ks + 8 * g);
                    const bf16x8 bv = ld8(&sm.Sbt[16 * ct + n][32 * ks + 8 * g]);
                    acc4[a] = mfma32(av, bv, acc4[a]);
                }
            }
        }
        if (w < 2) {
            f32x4 dl[4];
            s16x4 dlb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // right-hand side rows 16i + 4g + t, column 16ct + n
                const s16x4 vv = ld4(&sm.Vt[16 * ct + n][16 * i + 4 * g]);
                f32x4 rhs;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int s = 16 * i + 4 * g + t;
                    const float vf = __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(vv[t])) << 16);
                    rhs[t] = sm.bt[s] * (vf - sm.Gm[s] * sm.rk[s] * acc4[i][t]);
                }
                // subtract the solved blocks: rhs += (-A_ij) Delta_j
#pragma unroll
                for (int jb = 0; jb < i; ++jb)
                    rhs = mfma16(ld4(&sm.An[16 * i + n][16 * jb + 4 * g]), dlb[jb], rhs);
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                dl[i] = mfma16(ld4(&sm.Tb[i][n][4 * g]), pack4(rhs), zero);
                dlb[i] = pack4(dl[i]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                st4(&sm.Dt[16 * ct + n][16 * i + 4 * g], dlb[i]);
                f32x4 sc;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int s = 16 * i + 4 * g + t;
                    sc[t] = sm.Wd[s] * sm.rk[s] * dl[i][t];
                }
                st4(&sm.Dw[16 * ct + n][16 * i + 4 * g], pack4(sc));
            }
        } else {
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int r = 16 * a + 4 * g + t;
                    acc4[a][t] *= sm.Gm[r] * sm.rq[r];
                }
        }
        __syncthreads();  // (F)

        // ---- state update S <- Gamma_C S + K^T Dw (all waves, own rows)
        {
            const float GC = sm.Gm[C - 1];
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    f32x4 s4 = S[a][c] * GC;
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        s4 = mfma32(ld8(&sm.Kt[32 * w + 16 * a + n][32 * ks + 8 * g]),
                                    ld8(&sm.Dw[16 * c + n][32 * ks + 8 * g]), s4);
                    S[a][c] = s4;
                }
        }
        // ---- waves 2,3: O = Gamma rq Q S + P Delta, stored as bf16
        if (w >= 2) {
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                f32x4 o4 = acc4[a];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    if (ks == 1 && a < 2) continue;   // P is zero there
                    o4 = mfma32(ld8(&sm.Pb[16 * a + n][32 * ks + 8 * g]),
                                ld8(&sm.Dt[16 * ct + n][32 * ks + 8 * g]), o4);
                }
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int r = 16 * a + 4 * g + t;
                    if (r < L)
                        o[(((size_t)b * T + t0 + r) * Hv + h) * D + j0 + 16 * ct + n] =
                            static_cast<uint16_t>(bfbits(q_scale * o4[t]));
                }
            }
        }
    }

    if (hT) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    hT[state_base + (size_t)(32 * w + 16 * a + 4 * g + t) * D + j0 + 16 * c + n] = S[a][c][t];
    }
}

}  // namespace mfma_prefill

bool prefill_mfma_supported(const PrefillArgs& a) {
    return a.bf16 && a.D == 128 && a.C == 64;
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t stream) {
    const int blocks = a.B * a.Hv * (128 / mfma_prefill::BV);
    if (blocks == 0) return hipSuccess;
    const int remap = (blocks % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL(mfma_prefill::prefill_mfma_kernel, dim3(blocks), dim3(mfma_prefill::NT), 0, stream,
                       static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k),
                       static_cast<const bf16_t*>(a.v), a.log_g, a.beta, a.h0, a.hT,
                       static_cast<bf16_t*>(a.o), a.T, a.Hk, a.Hv, a.l2norm, a.q_scale, remap);
    return hipGetLastError();
}

}  // namespace gdn

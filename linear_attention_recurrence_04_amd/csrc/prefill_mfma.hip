// prefill_mfma.hip -- chunked gated-delta-rule prefill on bf16 MFMA (gfx950).
//
// Shape: head dim 128, chunk C = 64, bf16 q/k/v/o, fp32 gates and state.
//
// Per value head and chunk (gamma_r = sum_{s<=r} log g_s inside the chunk,
// Gamma_r = exp(gamma_r), rk/rq = 1 / max(|k|, 1e-6) / 1 / max(|q|, 1e-6)):
//   A_rs  = beta_r exp(gamma_r - gamma_s) rk_r rk_s (k_r . k_s)   s <  r   decay-masked beta K K^T
//   P_rs  = exp(gamma_r - gamma_s) rq_r rk_s (q_r . k_s)           s <= r
//   T     = (I + A)^-1                                             direct triangular solve
//   X     = diag(beta) (V - diag(Gamma rk) K S)
//   Delta = T X
//   O     = diag(Gamma rq) Q S + P Delta
//   S'    = Gamma_C S + K^T diag(exp(gamma_C - gamma) rk) Delta
// which is the token recurrence of "Qwen3.5 Gated Delta Net NKI Kernel for
// AWS Neuron" ("How It Works") unrolled over a chunk.  T is obtained by
// forward substitution -- inside the 16x16 diagonal blocks in fp32, then block
// by block with MFMA -- never by the Neumann power series ("Qwen3.6: Fused
// DeltaNet Direct-Solve Follow-Up", "Why This Exists", "Implementation
// Details").  Only exp(gamma_r - gamma_s) with s <= r is formed, so nothing
// overflows for log g <= 0.
//
// Two kernels:
//  * chunk_prep_kernel -- everything that does not depend on the state, for
//    all chunks and heads at once (one workgroup per (b, key head, chunk)):
//    row norms and the two Gram products (MFMA) once per key head; gates,
//    A, the triangular inverse T and P for each value head of the group.  T, P
//    and the gate vectors go to the caller's workspace, T and P already in
//    MFMA operand order.
//  * chunk_scan_kernel -- the serial chain over chunks.  One workgroup per
//    (b, value head, 32 state columns).  Each of its two state waves owns a
//    16-column strip of the fp32 state for all 128 rows, in MFMA accumulator
//    layout, for the whole sequence, and per chunk computes K S, X,
//    Delta = T X and the state update in its own registers: a pair of
//    accumulator tiles is, element for element, a valid operand of the next
//    product once the contraction index of the other operand is stored in the
//    matching order (kperm below).  The k^T operands of the update are read
//    from the k rows in LDS with transposed LDS loads.  Two output waves, one
//    chunk behind, form Q S + P Delta from the bf16 state and Delta operands
//    the state waves leave in LDS, so the chain from chunk to chunk carries
//    only K S, Delta and the update; they also store the output.  Four loader
//    waves stream the inputs into double-buffered LDS with direct
//    global -> LDS loads.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace mfma_prefill {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

constexpr int D = 128;      // head dim (dk = dv)
constexpr int C = 64;       // chunk
constexpr int NT = 256;     // threads per workgroup (both kernels)
constexpr int SK = D + 8;   // padded row stride (elements) of [64][128] bf16 tiles
constexpr int SC = C + 8;   // padded row stride of [*][64] bf16 tiles

// Workspace record per (b, value head, chunk): T and P (64x64 bf16 in
// operand order, compact images: see imgc) and the gate vectors (fp32):
// grk, wrk, beta, Gamma_C (read with k) and grq (read with q).
constexpr int IMG_BYTES = (32 * 32 + 32 * 64) * 2;   // 6144
constexpr int WS_T = 0;
constexpr int WS_P = IMG_BYTES;
constexpr int WS_G = 2 * IMG_BYTES;
constexpr int WS_GQ = WS_G + 4 * C * 4;
constexpr int WS_REC = WS_GQ + C * 4;               // 13568 bytes

// Contraction-index order inside each 32-wide k step.  A pair of accumulator
// tiles (rows 32ks.., 32ks+16..) gives lane (g, n) the rows {4g..4g+3} and
// {16+4g..16+4g+3}; a 16x16x32 operand gives lane (g, n) the logical
// k = 8g..8g+7.  Storing the other operand's physical 4-group q
// (k = 4q..4q+3) at logical offset kperm(q) makes the two agree.
__host__ __device__ constexpr int kperm(int q) { return 8 * (q & 3) + 4 * (q >> 2); }
// logical position of physical index p
__device__ __forceinline__ int lpos(int p) { return (p & ~31) + kperm((p >> 2) & 7) + (p & 3); }

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
// operand from an accumulator tile pair (lo = rows 4g.., hi = rows 16+4g..)
__device__ __forceinline__ bf16x8 pack8(f32x4 lo, f32x4 hi) {
    bf16x8 r;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        r[t] = static_cast<__bf16>(lo[t]);
        r[4 + t] = static_cast<__bf16>(hi[t]);
    }
    return r;
}
__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ s16x4 ld4(const uint16_t* p) { return *reinterpret_cast<const s16x4*>(p); }
__device__ __forceinline__ uint4 mask4(uint4 x, bool keep) {
    const uint32_t m = keep ? 0xffffffffu : 0u;
    return make_uint4(x.x & m, x.y & m, x.z & m, x.w & m);
}
// Sum over each row of 16 lanes with DPP moves: swap neighbours, swap pairs,
// mirror within 8 lanes, mirror within 16 lanes.  Every lane of the row ends
// with the row's sum.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_mov<0xB1>(x);    // quad_perm [1, 0, 3, 2]
    x += dpp_mov<0x4E>(x);    // quad_perm [2, 3, 0, 1]
    x += dpp_mov<0x141>(x);   // row_half_mirror
    x += dpp_mov<0x140>(x);   // row_mirror
    return x;
}
// exp(x) through the hardware base-2 exponential (arguments here are <= 0)
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// Lower-triangular 16x16 tiles of a 64x64 matrix: (0,0) (1,0) (1,1) (2,0) ...
__device__ __forceinline__ void tile_of(int idx, int& a, int& b) {
    a = (idx >= 1) + (idx >= 3) + (idx >= 6);
    b = idx - (a * (a + 1)) / 2;
}
__host__ __device__ constexpr int tile_a(int idx) { return (idx >= 1) + (idx >= 3) + (idx >= 6); }
__host__ __device__ constexpr int tile_b(int idx) { return idx - (tile_a(idx) * (tile_a(idx) + 1)) / 2; }

// T and P are read by the scan as 16-byte MFMA operands: rows 0..31 only at
// logical columns 0..31 (their first k step; the rest is zero), rows 32..63
// at all 64.  The image keeps just those: rows 0..31 as 64-byte rows, rows
// 32..63 as 128-byte rows after them.  Chunk c (logical columns 8c..8c+7) of
// row r sits at chunk c ^ 2((r >> 2) & 1) in the short rows and at
// c ^ ((r >> 1) & 7) in the long ones, so that the 16 rows an operand read
// touches fall in distinct LDS banks.  Element position of logical column L
// in row r (L < 32 when r < 32):
__host__ __device__ constexpr int imgc(int r, int L) {
    return r < 32 ? r * 32 + 8 * ((L >> 3) ^ (((r >> 2) & 1) << 1)) + (L & 7)
                  : 1024 + (r - 32) * 64 + 8 * ((L >> 3) ^ ((r >> 1) & 7)) + (L & 7);
}
// the same position in 16-byte units for logical chunk c
__host__ __device__ constexpr int imgq(int r, int c) {
    return r < 32 ? r * 4 + (c ^ (((r >> 2) & 1) << 1)) : 128 + (r - 32) * 8 + (c ^ ((r >> 1) & 7));
}

// ===========================================================================
// prep: one workgroup per (b, key head, chunk).  k, q, their norms and the
// two Gram products are formed once for the Hv / Hk value heads that share
// the key head; the gates, A, T and P once per value head.
// ===========================================================================

constexpr int GH = 4;   // value heads prepared together (one per wave for the gates,
                        // one per 16-lane group in the diagonal solve)

// Lower-triangular 16x16 blocks of a 64x64 matrix, stored compactly:
// diagonal and below (i >= j) at tl_idx, strictly below (i > k) at ab_idx.
__host__ __device__ constexpr int tl_idx(int i, int j) { return i * (i + 1) / 2 + j; }
__host__ __device__ constexpr int ab_idx(int i, int k) { return i * (i - 1) / 2 + k; }

// k and q rows are needed only up to the Gram products; the triangular
// factors of the group's value heads reuse their space.
struct PrepSmem {
    union {
        struct {
            uint16_t Kr[C][SK];       // raw k rows (bf16)
            uint16_t Qr[C][SK];       // raw q rows
        } in;
        struct {
            float AfT[GH][4][16][16];      // A diagonal blocks (fp32), transposed: [head][block][s][r]
            uint16_t Ab[GH][6][16][16];    // A blocks below the diagonal (bf16)
            uint16_t Tl[GH][10][16][16];   // T blocks on and below the diagonal (bf16)
        } tri;
    };
    float rk[C], rq[C];
    float gam[GH][C], bt[GH][C];
};

// Gating of one wave's five Gram tiles (tasks W, W + 4, .., W + 16: tasks
// 0..9 are K K^T tiles, 10..19 Q K^T tiles) for the nh value heads of a
// group, with the tile geometry known at compile time so that every LDS
// read of a head is issued before its arithmetic.  Lane (g, n) holds
// s = 16bb + 4g + t, r = 16a + n.  A goes to LDS (diagonal blocks fp32,
// others bf16); P goes to the record of each head (rec0 + hh * rec_stride).
template <int W>
__device__ __forceinline__ void gate_tiles(PrepSmem& sm, const f32x4 (&gram)[5], int nh, int g, int n,
                                           unsigned char* rec0, size_t rec_stride) {
    f32x4 ks[4];
    float rkr[4], rqr[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        ks[x] = *reinterpret_cast<const f32x4*>(&sm.rk[16 * x + 4 * g]);
        rkr[x] = sm.rk[16 * x + n];
        rqr[x] = sm.rq[16 * x + n];
    }
#pragma unroll 1
    for (int hh = 0; hh < nh; ++hh) {
        float gr[4], btr[4];
        f32x4 gs[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            gr[x] = sm.gam[hh][16 * x + n];
            btr[x] = sm.bt[hh][16 * x + n];
            gs[x] = *reinterpret_cast<const f32x4*>(&sm.gam[hh][16 * x + 4 * g]);
        }
        uint16_t* Pg = reinterpret_cast<uint16_t*>(rec0 + hh * rec_stride + WS_P);
#pragma unroll
        for (int u = 0; u < 5; ++u) {
            const int task = W + 4 * u;
            const bool is_qk = task >= 10;
            const int a = tile_a(is_qk ? task - 10 : task);
            const int bb = tile_b(is_qk ? task - 10 : task);
            const int r = 16 * a + n;
            const float sr = is_qk ? rqr[a] : rkr[a] * btr[a];
            f32x4 val;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int s2 = 16 * bb + 4 * g + t;
                const bool keep = is_qk ? (s2 <= r) : (s2 < r);
                const float x = exp_hw(gr[a] - gs[bb][t]) * sr * ks[bb][t] * gram[u][t];
                val[t] = keep ? x : 0.f;
            }
            if (is_qk) {
                const int q4 = 4 * bb + g;   // physical 4-group of s
                *reinterpret_cast<s16x4*>(Pg + imgc(r, 32 * (q4 >> 3) + kperm(q4 & 7))) = pack4(val);
                if (a == bb && (a == 0 || a == 2)) {  // upper neighbour read by the scan: zero
                    const int qz = q4 + 4;
                    const s16x4 z = {0, 0, 0, 0};
                    *reinterpret_cast<s16x4*>(Pg + imgc(r, 32 * (qz >> 3) + kperm(qz & 7))) = z;
                }
            } else if (a == bb) {
#pragma unroll
                for (int t = 0; t < 4; ++t) sm.tri.AfT[hh][a][4 * g + t][n] = val[t];
            } else {
                *reinterpret_cast<s16x4*>(&sm.tri.Ab[hh][ab_idx(a, bb)][n][4 * g]) = pack4(val);
            }
        }
    }
}

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(3))) void chunk_prep_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
    const float* __restrict__ log_g, const float* __restrict__ beta,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias,
    unsigned char* __restrict__ ws, int T, int NTc, int Hk, int Hv, int l2norm) {
    __shared__ PrepSmem sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int g = lane >> 4;
    const int n = lane & 15;

    const int chunk = blockIdx.x % NTc;
    const int bk = blockIdx.x / NTc;
    const int b = bk / Hk;
    const int hk = bk - b * Hk;
    const int rr = Hv / Hk;
    const int t0 = chunk * C;
    const int L = min(C, T - t0);

    // gate inputs of value head hk * rr + jg + w for t0 + lane (clamped row;
    // padding rows get g = 1, beta = 0 below), fetched one group ahead
    auto gate_in = [&](int jg, float& lgr, float& btr) __attribute__((always_inline)) {
        const int j = min(jg + w, rr - 1);
        const size_t gi = ((size_t)b * T + t0 + min(lane, L - 1)) * Hv + hk * rr + j;
        lgr = log_g[gi];
        btr = beta[gi];
        if (A_log) {   // raw projections a, b
            lgr = raw_log_decay(lgr, A_log[hk * rr + j], dt_bias[hk * rr + j]);
            btr = raw_beta(btr);
        }
    };
    float lg_next, bt_next;
    gate_in(0, lg_next, bt_next);

    // ---- stage raw q, k rows (rows >= L are zero) and their inverse norms
    //      (16 lanes per row); all eight loads are issued first
    u32x4 kv[4], qv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int r = (tid + NT * u) >> 4;
        const int c8 = (tid & 15) * 8;
        const size_t off = (((size_t)b * T + t0 + min(r, L - 1)) * Hk + hk) * D + c8;
        kv[u] = *reinterpret_cast<const u32x4*>(k + off);
        qv[u] = *reinterpret_cast<const u32x4*>(q + off);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int r = (tid + NT * u) >> 4;
        const int c8 = (tid & 15) * 8;
        const uint32_t m = (r < L) ? 0xffffffffu : 0u;
        const u32x4 kx = kv[u] & m, qx = qv[u] & m;
        *reinterpret_cast<u32x4*>(&sm.in.Kr[r][c8]) = kx;
        *reinterpret_cast<u32x4*>(&sm.in.Qr[r][c8]) = qx;
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float k0 = __uint_as_float(kx[e] << 16), k1 = __uint_as_float(kx[e] & 0xffff0000u);
            const float q0 = __uint_as_float(qx[e] << 16), q1 = __uint_as_float(qx[e] & 0xffff0000u);
            sk += k0 * k0 + k1 * k1;
            sq += q0 * q0 + q1 * q1;
        }
        sk = row16_sum(sk);
        sq = row16_sum(sq);
        if ((lane & 15) == 0) {
            sm.rk[r] = l2norm ? inv_l2(sk) : 1.f;
            sm.rq[r] = l2norm ? inv_l2(sq) : 1.f;
        }
    }
    __syncthreads();

    // ---- raw Gram tiles, computed transposed (s on the M side), kept in
    //      registers: 10 of K K^T, 10 of Q K^T; wave w owns tasks w + 4u.
    //      Lane (g, n) holds s = 16bb + 4g + t, r = 16a + n.
    f32x4 gram[5];
#pragma unroll
    for (int u = 0; u < 5; ++u) {
        const int task = w + 4 * u;
        const bool is_qk = task >= 10;
        int a, bb;
        tile_of(is_qk ? task - 10 : task, a, bb);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const uint16_t* rowsB = is_qk ? &sm.in.Qr[16 * a + n][0] : &sm.in.Kr[16 * a + n][0];
        bf16x8 opa[4], opb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            opa[ks] = ld8(&sm.in.Kr[16 * bb + n][32 * ks + 8 * g]);
            opb[ks] = ld8(rowsB + 32 * ks + 8 * g);
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mfma32(opa[ks], opb[ks], acc);
        gram[u] = acc;
    }

    for (int jg = 0; jg < rr; jg += GH) {
        const int nh = min(GH, rr - jg);   // value heads in this group
        // ---- gates of value heads jg .. jg + GH - 1 (wave w: head jg + w):
        //      decay scan, then Gamma rk, exp(gamma_C - gamma) rk, Gamma rq,
        //      beta, Gamma_C to the record.  Padding rows: g = 1, beta = 0.
        const float lgr = lg_next, btr = bt_next;
        if (jg + GH < rr) gate_in(jg + GH, lg_next, bt_next);
        if (w < nh) {
            const int h = hk * rr + jg + w;
            float x = (lane < L) ? lgr : 0.f;
            const float btv = (lane < L) ? btr : 0.f;
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) {
                const float y = __shfl_up(x, m, 64);
                if (lane >= m) x += y;
            }
            sm.gam[w][lane] = x;
            sm.bt[w][lane] = btv;
            const float total = __shfl(x, 63, 64);
            const float Gm = exp_hw(x);
            const float rkv = sm.rk[lane];
            float* gp = reinterpret_cast<float*>(ws + (((size_t)b * Hv + h) * NTc + chunk) * WS_REC + WS_G);
            gp[0 * C + lane] = Gm * rkv;
            gp[1 * C + lane] = exp_hw(total - x) * rkv;
            gp[2 * C + lane] = btv;
            gp[3 * C + lane] = exp_hw(total);
            gp[4 * C + lane] = Gm * sm.rq[lane];
        }
        __syncthreads();   // k and q rows are dead from here: their space holds A and T

        // ---- gate the Gram tiles for every head of the group: A (diagonal
        //      blocks fp32, others bf16) to LDS, P straight to the record
        {
            unsigned char* rec0 = ws + (((size_t)b * Hv + hk * rr + jg) * NTc + chunk) * WS_REC;
            const size_t rec_stride = (size_t)NTc * WS_REC;
            switch (w) {
                case 0: gate_tiles<0>(sm, gram, nh, g, n, rec0, rec_stride); break;
                case 1: gate_tiles<1>(sm, gram, nh, g, n, rec0, rec_stride); break;
                case 2: gate_tiles<2>(sm, gram, nh, g, n, rec0, rec_stride); break;
                default: gate_tiles<3>(sm, gram, nh, g, n, rec0, rec_stride); break;
            }
        }
        __syncthreads();

        // ---- diagonal blocks: T_ww = (I + A_ww)^-1 by forward substitution.
        //      Wave w solves block w for every head at once: lane (g, n) is
        //      column n of head g.  Once row s of the column is final, its
        //      multiples are removed from the rows below it.
        {
            const int hh = g;
            float tc[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) tc[r] = (r == n) ? 1.f : 0.f;
#pragma unroll
            for (int s2 = 0; s2 < 15; ++s2) {
                float col[16];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const f32x4 c4 = *reinterpret_cast<const f32x4*>(&sm.tri.AfT[hh][w][s2][4 * x]);
                    col[4 * x] = c4[0]; col[4 * x + 1] = c4[1]; col[4 * x + 2] = c4[2]; col[4 * x + 3] = c4[3];
                }
#pragma unroll
                for (int r = s2 + 1; r < 16; ++r) tc[r] -= col[r] * tc[s2];
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.tri.Tl[hh][tl_idx(w, w)][r][n] = static_cast<uint16_t>(bfbits(tc[r]));
        }
        __syncthreads();

        // ---- blocks below the diagonal in column block j = w, every head:
        //      (I + A_ii) T_ij + sum_{k=j}^{i-1} A_ik T_kj = 0  =>  T_ij = -T_ii sum_k A_ik T_kj
        {
            const int j = w;
            s16x4 tk[GH][4];   // T_kj as operand (accumulator layout), k = j..3
#pragma unroll
            for (int hh = 0; hh < GH; ++hh) {
                s16x4 d;
#pragma unroll
                for (int t = 0; t < 4; ++t) d[t] = static_cast<short>(sm.tri.Tl[hh][tl_idx(j, j)][4 * g + t][n]);
                tk[hh][0] = d;
            }
#pragma unroll
            for (int di = 1; di < 4; ++di) {
                const int i = j + di;
                if (i < 4) {
#pragma unroll
                    for (int hh = 0; hh < GH; ++hh) {
                        if (hh < nh) {
                            f32x4 R = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int dk = 0; dk < di; ++dk)
                                R = mfma16(ld4(&sm.tri.Ab[hh][ab_idx(i, j + dk)][n][4 * g]), tk[hh][dk], R);
                            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                            const f32x4 Tij = mfma16(ld4(&sm.tri.Tl[hh][tl_idx(i, i)][n][4 * g]), pack4(-R), zero);
                            tk[hh][di] = pack4(Tij);
#pragma unroll
                            for (int t = 0; t < 4; ++t)
                                sm.tri.Tl[hh][tl_idx(i, j)][4 * g + t][n] = static_cast<uint16_t>(tk[hh][di][t]);
                        }
                    }
                }
            }
        }
        __syncthreads();

        // ---- T of every head to its record in operand order (8-byte groups,
        //      permuted per 32); blocks above the diagonal are zero.  The next
        //      group rewrites A first and T only after its next barrier.
        for (int hh = 0; hh < nh; ++hh) {
            const int h = hk * rr + jg + hh;
            uint16_t* Tg = reinterpret_cast<uint16_t*>(ws + (((size_t)b * Hv + h) * NTc + chunk) * WS_REC + WS_T);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = tid + NT * u;        // 1024 groups: row r, physical group Qg (16 per row)
                const int r = e >> 4;
                const int Qg = e & 15;
                const int bi = r >> 4, bj = Qg >> 2;
                if (r < 32 && Qg >= 8) continue;   // not in the image (zero)
                uint2 val = make_uint2(0u, 0u);
                if (bj <= bi) val = *reinterpret_cast<const uint2*>(&sm.tri.Tl[hh][tl_idx(bi, bj)][r & 15][4 * (Qg & 3)]);
                *reinterpret_cast<uint2*>(Tg + imgc(r, 32 * (Qg >> 3) + kperm(Qg & 7))) = val;
            }
        }
    }
}

// ===========================================================================
// scan: one workgroup per (b, value head h, 32 state columns), in three roles:
//  * two state waves (one per 16-column strip): K S, X, Delta = T X and the
//    state update, the chain that carries the state from chunk to chunk;
//  * two output waves (one per strip), one chunk behind: Q S and P Delta from
//    the bf16 state and Delta operands the state waves leave in LDS, and the
//    output stores;
//  * four loader waves: direct global -> LDS loads of the next chunk's inputs
//    into double-buffered LDS, and cache-line touches of a chunk further
//    ahead.
// All eight meet at one barrier per chunk.
// ===========================================================================

constexpr int SW = 16;            // state columns per strip
constexpr int NSTRIP = 2;         // strips per workgroup
constexpr int LWAVES = 4;         // loader waves
constexpr int SNT = 64 * (2 * NSTRIP + LWAVES);   // threads per workgroup
constexpr int BVS = SW * NSTRIP;  // state columns per workgroup
constexpr int OS = BVS + 8;       // row stride (elements) of the output staging tile

// 16-byte chunk c of a 256-byte k or q row r is stored at c ^ swz(r).  Row
// operand reads (16 rows, one chunk) and transposed reads (4 rows x 4 chunks
// per 16 lanes) both hit 16 distinct chunk positions.
__host__ __device__ constexpr int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

struct KSet {              // state-wave inputs of one chunk
    uint4 K[C * 16];       // k rows, swizzled
    uint4 T[IMG_BYTES / 16];   // T image
    uint4 V[C * 4];        // v rows of the 32 columns: chunk c of row s at c ^ ((s >> 2) & 3)
    float gate[4 * C];     // grk, wrk, beta, Gamma_C
};
struct QSet {              // output-wave inputs of one chunk
    uint4 Q[C * 16];       // q rows, swizzled
    uint4 P[IMG_BYTES / 16];   // P image
    float gate[C];         // grq
};
struct ScanSmem {
    KSet ks[3];                    // k side: chunk c in ks[c % 3], loaded two chunks ahead
    QSet qs[2];                    // q side: chunk c in qs[c % 2], loaded one chunk ahead
    bf16x8 Sx[2][NSTRIP][4][64];   // bf16 state operands (per strip, k step, lane)
    bf16x8 Dx[2][NSTRIP][2][64];   // Delta operands
    uint16_t Os[C][OS];            // output tile, transposed to rows for 16-byte stores
    uint32_t sink[LWAVES][64];     // landing area of the cache-line touches
};

// direct 16-byte load of one lane into LDS at base + 16 * lane (base wave-uniform)
__device__ __forceinline__ void lds_load16(const void* g, void* lds_base) {
    __builtin_amdgcn_global_load_lds(g, lds_base, 16, 0, 0);
}
// 4-byte direct load: used to touch cache lines ahead of their use
__device__ __forceinline__ void lds_load4(const void* g, void* lds_base) {
    __builtin_amdgcn_global_load_lds(g, lds_base, 4, 0, 0);
}
// s_waitcnt immediate that waits until at most n vector memory operations are
// outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and
// lgkmcnt fields at their maximum, i.e. not waited for)
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// transposed 4 x 16-bit read: within each 16 lanes, lane i receives element
// i & 3 of the 8-byte pieces addressed by lanes (i >> 2) + 4j, j = 0..3
__device__ __forceinline__ s16x4 ld_tr4(const void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

__global__ __launch_bounds__(SNT) void chunk_scan_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const unsigned char* __restrict__ ws, const float* h0, float* hT, bf16_t* __restrict__ o,
    int T, int NTc, int Hk, int Hv, float q_scale, int xcd_remap,
    float* __restrict__ ckpt, int ckpt_every, int nck) {
    __shared__ ScanSmem sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int g = lane >> 4;
    const int n = lane & 15;

    int lid = blockIdx.x;
    if (xcd_remap) {  // consecutive logical ids on one XCD (dispatch is round-robin over 8)
        const int per = gridDim.x >> 3;
        lid = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    }
    constexpr int NB = D / BVS;          // column blocks per head
    const int bh = lid / NB;
    const int j0 = (lid % NB) * BVS;
    const int b = bh / Hv;
    const int h = bh - b * Hv;
    const int hk = h / (Hv / Hk);
    const size_t state_base = (size_t)bh * D * D;
    const unsigned char* rec0 = ws + (size_t)bh * NTc * WS_REC;
    const bf16_t* kbase = k + ((size_t)b * T * Hk + hk) * D;
    const bf16_t* qbase = q + ((size_t)b * T * Hk + hk) * D;
    const bf16_t* vbase = v + ((size_t)b * T * Hv + h) * D + j0;
    bf16_t* obase = o + ((size_t)b * T * Hv + h) * D + j0;
    const int rowk = Hk * D;             // element stride between tokens of q and k
    const int rowv = Hv * D;             // element stride between tokens of v and o

    // ======================= loader waves =======================
    // Rows past the end read a clamped valid row: their beta is zero and their
    // rows of T and P are those of the identity and zero, so they add nothing.
    if (w >= 2 * NSTRIP) {
        const int lw = w - 2 * NSTRIP;
        // per-lane byte offsets inside a chunk (rows clamped to `last`), so
        // that each k, q or v load is a uniform base plus a 32-bit lane offset;
        // the k side and the q side switch to the last chunk's rows separately
        constexpr int NKB = 16 / LWAVES, NVB = 4 / LWAVES, NRB = (IMG_BYTES / 1024 + LWAVES - 1) / LWAVES;
        uint32_t offk[NKB], offq[NKB], offv[NVB];
        auto kq_offsets = [&](uint32_t (&off)[NKB], int last) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < NKB; ++u) {            // k / q: 16 blocks of 4 rows
                const int r = 4 * (lw + LWAVES * u) + (lane >> 4);
                off[u] = 2u * (uint32_t)(min(r, last) * rowk + 8 * ((lane & 15) ^ swz(r)));
            }
        };
        auto v_offsets = [&](int last) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < NVB; ++u) {            // v: 4 blocks of 16 rows
                const int s2 = 16 * (lw + LWAVES * u) + (lane >> 2);
                offv[u] = 2u * (uint32_t)(min(s2, last) * rowv + 8 * ((lane & 3) ^ ((s2 >> 2) & 3)));
            }
        };
        const int last_rows = T - (NTc - 1) * C - 1;   // last row of the last chunk
        kq_offsets(offk, C - 1);
        kq_offsets(offq, C - 1);
        v_offsets(C - 1);

        // The k side of a chunk is 7 direct loads per loader wave (k 4, T 2
        // or 1, v 1, gates 1 on one wave; the fourth wave repeats its last k
        // block), so that one wait count fits every wave.
        constexpr int NKLOADS = 7;
        auto load_k = [&](int chunk, int slot) __attribute__((always_inline)) {
            if (chunk == NTc - 1) {   // the last chunk: clamp its rows
                kq_offsets(offk, last_rows);
                v_offsets(last_rows);
            }
            KSet& B = sm.ks[slot];
            const int t0 = chunk * C;
            const unsigned char* kc = reinterpret_cast<const unsigned char*>(kbase + (size_t)t0 * rowk);
            const unsigned char* vc = reinterpret_cast<const unsigned char*>(vbase + (size_t)t0 * rowv);
            const unsigned char* rec = rec0 + (size_t)chunk * WS_REC;
#pragma unroll
            for (int u = 0; u < NKB; ++u) lds_load16(kc + offk[u], &B.K[64 * (lw + LWAVES * u)]);
#pragma unroll
            for (int u = 0; u < NRB; ++u) {            // 6 blocks of 1 KiB
                const int blk = lw + LWAVES * u;
                if (blk < IMG_BYTES / 1024) lds_load16(rec + WS_T + 1024 * blk + 16 * lane, &B.T[64 * blk]);
            }
#pragma unroll
            for (int u = 0; u < NVB; ++u) lds_load16(vc + offv[u], &B.V[64 * (lw + LWAVES * u)]);
            if (lw == 2) lds_load16(rec + WS_G + 16 * lane, B.gate);   // 1 KiB
            if (lw == 3) lds_load16(kc + offk[NKB - 1], &B.K[64 * (lw + LWAVES * (NKB - 1))]);   // count filler
        };
        auto load_q = [&](int chunk, int slot) __attribute__((always_inline)) {
            if (chunk == NTc - 1) kq_offsets(offq, last_rows);
            QSet& B = sm.qs[slot];
            const int t0 = chunk * C;
            const unsigned char* qc = reinterpret_cast<const unsigned char*>(qbase + (size_t)t0 * rowk);
            const unsigned char* rec = rec0 + (size_t)chunk * WS_REC;
#pragma unroll
            for (int u = 0; u < NKB; ++u) lds_load16(qc + offq[u], &B.Q[64 * (lw + LWAVES * u)]);
#pragma unroll
            for (int u = 0; u < NRB; ++u) {
                const int blk = lw + LWAVES * u;
                if (blk < IMG_BYTES / 1024) lds_load16(rec + WS_P + 1024 * blk + 16 * lane, &B.P[64 * blk]);
            }
            if (lw == 3 && lane < 16) lds_load16(rec + WS_GQ + 16 * lane, B.gate);   // 256 bytes
        };
        // Cache-line touches (4-byte loads into a scratch row of LDS) of the
        // chunk TOUCH_AHEAD chunks ahead, so that its direct loads find the
        // lines in L2 instead of waiting on HBM.  Each line is touched by one
        // workgroup of those that share it: k and q lines by the first column
        // block of the key head's first value head, the T, P and gate record
        // by the head's first column block, v lines (128 bytes = two column
        // blocks) by the even column blocks.  A wave touches two sets of
        // lines or none.
        constexpr int TOUCH_AHEAD = 3;
        const bool first_block = (j0 == 0);
        bool toucher;
        if (lw == 0) toucher = first_block;
        else if (lw == 1) toucher = (j0 % 64) == 0;
        else toucher = first_block && (h % (Hv / Hk)) == 0;
        auto touch = [&](int chunk) __attribute__((always_inline)) {
            const int t0 = chunk * C;
            const int row = t0 + min(lane, T - t0 - 1);
            uint32_t* sink = sm.sink[lw];
            const unsigned char* rec = rec0 + (size_t)chunk * WS_REC;   // 106 lines of 128 bytes
            if (lw == 0) {
                lds_load4(rec + 128 * lane, sink);
                lds_load4(rec + 128 * min(64 + lane, WS_REC / 128 - 1), sink);
            } else if (lw == 1) {
                lds_load4(vbase + (size_t)row * rowv, sink);
                lds_load4(vbase + (size_t)row * rowv + 32, sink);   // same line: keeps two per toucher
            } else {
                const bf16_t* base = (lw == 2) ? kbase : qbase;
                lds_load4(base + (size_t)row * rowk, sink);
                lds_load4(base + (size_t)row * rowk + 64, sink);
            }
        };
        constexpr int NTOUCH = 2;
        // iteration c: the state waves work on chunk c and the output waves on
        // chunk c - 1; load the q side of chunk c, then the k side of chunk
        // c + 2, then the touches.  Operations complete in issue order, so
        // waiting until only the k loads and touches of this iteration are
        // outstanding covers the q side of chunk c and the k side of chunk
        // c + 1 (issued an iteration ago): what the next iteration reads.
        if (toucher)
            for (int c = 1; c <= TOUCH_AHEAD && c < NTc; ++c) touch(c);
        load_k(0, 0);
        if (NTc > 1) load_k(1, 1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        for (int c = 0; c <= NTc; ++c) {
            if (c < NTc) load_q(c, c & 1);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            const bool kload = c + 2 < NTc;
            if (kload) load_k(c + 2, (c + 2) % 3);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            const bool tload = toucher && c + TOUCH_AHEAD < NTc;
            if (tload) touch(c + TOUCH_AHEAD);
            if (kload && tload) __builtin_amdgcn_s_waitcnt(waitcnt_vm(NKLOADS + NTOUCH));
            else if (kload) __builtin_amdgcn_s_waitcnt(waitcnt_vm(NKLOADS));
            else if (tload) __builtin_amdgcn_s_waitcnt(waitcnt_vm(NTOUCH));
            else __builtin_amdgcn_s_waitcnt(0);
            // a plain barrier: a fenced one would also wait for the loads
            // and touches still in flight
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
        return;
    }
    __syncthreads();

    const int strip = (w < NSTRIP) ? w : w - NSTRIP;
    const int jw = j0 + SW * strip;      // first state column of the strip
    const int sn = swz(n);               // swizzle of rows 16i + n

    // ======================= state waves =======================
    if (w < NSTRIP) {
        // State strip in accumulator layout.  Tile a, lane (g, n), element t holds
        // state row lpos(16a + 4g + t) = 32(a >> 1) + 8g + 4(a & 1) + t, column jw + n:
        // with rows in this order a tile pair is the K S operand with k in natural order.
        f32x4 S[8];
        if (h0) {
            const float* hp = h0 + state_base + jw + n;
#pragma unroll
            for (int a = 0; a < 8; ++a)
#pragma unroll
                for (int t = 0; t < 4; ++t) S[a][t] = hp[(32 * (a >> 1) + 8 * g + 4 * (a & 1) + t) * D];
        } else {
#pragma unroll
            for (int a = 0; a < 8; ++a) S[a] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        for (int c = 0; c <= NTc; ++c) {
            if (c < NTc) {
                const KSet& B = sm.ks[c % 3];
                // ---- K operands of the first k step, then the bf16 state
                //      operands (also left in LDS for the output wave)
                bf16x8 ak[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) ak[i] = __builtin_bit_cast(bf16x8, B.K[(16 * i + n) * 16 + (g ^ sn)]);
                bf16x8 SB[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    SB[ks] = pack8(S[2 * ks], S[2 * ks + 1]);
                    sm.Sx[c & 1][strip][ks][lane] = SB[ks];   // for the output wave
                }
                // ---- K S: k step outer, 4 independent accumulators inner.  The
                //      v values, Gamma rk, beta and the T operands, needed only
                //      after it, are read behind the operands of the later k steps.
                f32x4 KS[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) KS[i] = f32x4{0.f, 0.f, 0.f, 0.f};
                s16x4 vt[4];
                f32x4 btv[4], grk[4];
                bf16x8 at0[4], at1[2];   // T operands
                const unsigned char* Vb = reinterpret_cast<const unsigned char*>(B.V);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    bf16x8 nk[4];
                    if (ks < 3) {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            nk[i] = __builtin_bit_cast(bf16x8, B.K[(16 * i + n) * 16 + ((4 * (ks + 1) + g) ^ sn)]);
                    }
                    if (ks == 1) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            // transposed read: lane (g, n) receives v rows 16i + 4g + j,
                            // j = 0..3, at column 16 strip + n; it addresses row
                            // 16i + 4g + (n >> 2), columns 16 strip + 4 (n & 3) .. + 3
                            const int sr = 16 * i + 4 * g + (n >> 2);
                            vt[i] = ld_tr4(Vb + sr * 64 + 16 * ((2 * strip + ((n >> 1) & 1)) ^ g) + 8 * (n & 1));
                            grk[i] = *reinterpret_cast<const f32x4*>(&B.gate[0 * C + 16 * i + 4 * g]);
                        }
                    }
                    if (ks == 2) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            btv[i] = *reinterpret_cast<const f32x4*>(&B.gate[2 * C + 16 * i + 4 * g]);
                            at0[i] = __builtin_bit_cast(bf16x8, B.T[imgq(16 * i + n, g)]);
                        }
                    }
                    if (ks == 3) {
                        at1[0] = __builtin_bit_cast(bf16x8, B.T[imgq(32 + n, 4 + g)]);
                        at1[1] = __builtin_bit_cast(bf16x8, B.T[imgq(48 + n, 4 + g)]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) KS[i] = mfma32(ak[i], SB[ks], KS[i]);
                    __builtin_amdgcn_sched_barrier(0);
                    if (ks < 3) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) ak[i] = nk[i];
                    }
                }
                // ---- X = beta (V - Gamma rk K S)
                f32x4 X[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        X[i][t] = btv[i][t] * (__uint_as_float((uint32_t)(uint16_t)vt[i][t] << 16) - grk[i][t] * KS[i][t]);
                const bf16x8 XB0 = pack8(X[0], X[1]);
                const bf16x8 XB1 = pack8(X[2], X[3]);
                // ---- k^T operands of the state update, read transposed from the
                //      k rows: tile a, k step kk; lane (g, n) gets k column
                //      lpos(16a + n) at tokens 32kk + 4g + j and 32kk + 16 + 4g + j
                const unsigned char* Kb = reinterpret_cast<const unsigned char*>(B.K);
                bf16x8 akt[8][2];
#pragma unroll
                for (int a = 0; a < 8; ++a)
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        const int r0 = 32 * kk + 4 * g + (n >> 2);
                        const int ch = 4 * (a >> 1) + (n & 3);
                        const int sz = ((n >> 2) << 2) | g;     // swz(r0) = swz(r0 + 16)
                        const s16x4 lo = ld_tr4(Kb + r0 * 256 + 16 * (ch ^ sz) + 8 * (a & 1));
                        const s16x4 hi = ld_tr4(Kb + (r0 + 16) * 256 + 16 * (ch ^ sz) + 8 * (a & 1));
                        akt[a][kk] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    }
                const f32x4 wlo0 = *reinterpret_cast<const f32x4*>(&B.gate[C + 4 * g]);
                const f32x4 whi0 = *reinterpret_cast<const f32x4*>(&B.gate[C + 16 + 4 * g]);
                const f32x4 wlo1 = *reinterpret_cast<const f32x4*>(&B.gate[C + 32 + 4 * g]);
                const f32x4 whi1 = *reinterpret_cast<const f32x4*>(&B.gate[C + 48 + 4 * g]);
                const float GC = B.gate[3 * C];
                __builtin_amdgcn_sched_barrier(0);
                // ---- Delta = T X (T lower triangular: row tile i needs k steps <= i/2)
                f32x4 Dl[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) Dl[i] = mfma32(at0[i], XB0, f32x4{0.f, 0.f, 0.f, 0.f});
                Dl[2] = mfma32(at1[0], XB1, Dl[2]);
                Dl[3] = mfma32(at1[1], XB1, Dl[3]);
                // ---- Delta operands: plain (to the output wave) and scaled (state update)
                sm.Dx[c & 1][strip][0][lane] = pack8(Dl[0], Dl[1]);
                sm.Dx[c & 1][strip][1][lane] = pack8(Dl[2], Dl[3]);
                const bf16x8 DWB0 = pack8(Dl[0] * wlo0, Dl[1] * whi0);
                const bf16x8 DWB1 = pack8(Dl[2] * wlo1, Dl[3] * whi1);
                // ---- state update S <- Gamma_C S + K^T (wrk Delta), 8 independent tiles
#pragma unroll
                for (int a = 0; a < 8; ++a) S[a] = mfma32(akt[a][0], DWB0, S[a] * GC);
#pragma unroll
                for (int a = 0; a < 8; ++a) S[a] = mfma32(akt[a][1], DWB1, S[a]);
                // ---- checkpoint slot: the state after every ckpt_every tokens
                //      and after the last token
                if (ckpt) {
                    const int done = min((c + 1) * C, T);
                    if (done % ckpt_every == 0 || c == NTc - 1) {
                        const int slot = (done + ckpt_every - 1) / ckpt_every - 1;
                        float* cp = ckpt + (((size_t)b * nck + slot) * Hv + h) * D * D + jw + n;
#pragma unroll
                        for (int a = 0; a < 8; ++a)
#pragma unroll
                            for (int t = 0; t < 4; ++t) cp[(32 * (a >> 1) + 8 * g + 4 * (a & 1) + t) * D] = S[a][t];
                    }
                }
            }
            __syncthreads();
        }
        if (hT) {
            float* hp = hT + state_base + jw + n;
#pragma unroll
            for (int a = 0; a < 8; ++a)
#pragma unroll
                for (int t = 0; t < 4; ++t) hp[(32 * (a >> 1) + 8 * g + 4 * (a & 1) + t) * D] = S[a][t];
        }
        return;
    }

    // ======================= output waves =======================
    for (int c = 0; c <= NTc; ++c) {
        if (c >= 1) {
            const int cc = c - 1;
            const QSet& B = sm.qs[cc & 1];
            // ---- operands: state and Delta from the state wave, q rows, P, gates
            bf16x8 SB[4], aq[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) SB[ks] = sm.Sx[cc & 1][strip][ks][lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) aq[i] = __builtin_bit_cast(bf16x8, B.Q[(16 * i + n) * 16 + (g ^ sn)]);
            f32x4 QS[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) QS[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            // ---- Q S
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                bf16x8 nq[4];
                if (ks < 3) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        nq[i] = __builtin_bit_cast(bf16x8, B.Q[(16 * i + n) * 16 + ((4 * (ks + 1) + g) ^ sn)]);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < 4; ++i) QS[i] = mfma32(aq[i], SB[ks], QS[i]);
                __builtin_amdgcn_sched_barrier(0);
                if (ks < 3) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) aq[i] = nq[i];
                }
            }
            bf16x8 ap0[4], ap1[2];
#pragma unroll
            for (int i = 0; i < 4; ++i) ap0[i] = __builtin_bit_cast(bf16x8, B.P[imgq(16 * i + n, g)]);
            ap1[0] = __builtin_bit_cast(bf16x8, B.P[imgq(32 + n, 4 + g)]);
            ap1[1] = __builtin_bit_cast(bf16x8, B.P[imgq(48 + n, 4 + g)]);
            const bf16x8 DB0 = sm.Dx[cc & 1][strip][0][lane];
            const bf16x8 DB1 = sm.Dx[cc & 1][strip][1][lane];
            f32x4 grq[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) grq[i] = *reinterpret_cast<const f32x4*>(&B.gate[16 * i + 4 * g]);
            // ---- O = Gamma rq Q S + P Delta
            f32x4 O4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) O4[i] = mfma32(ap0[i], DB0, grq[i] * QS[i]);
            O4[2] = mfma32(ap1[0], DB1, O4[2]);
            O4[3] = mfma32(ap1[1], DB1, O4[3]);
            uint16_t (*Ot)[OS] = sm.Os;   // each output wave reads back only its own columns
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    Ot[16 * i + 4 * g + t][SW * strip + n] = static_cast<uint16_t>(bfbits(q_scale * O4[i][t]));
            // ---- the strip's 64 rows x 32 bytes back from LDS (this wave's own
            //      writes, so no barrier) and to HBM in 16-byte pieces
            const int t0 = cc * C;
            const int L = min(C, T - t0);
            bf16_t* oc = obase + (size_t)t0 * rowv + SW * strip;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int r = (lane >> 1) + 32 * u;
                const int c8 = 8 * (lane & 1);
                if (r < L)
                    *reinterpret_cast<uint4*>(oc + r * rowv + c8) =
                        *reinterpret_cast<const uint4*>(&Ot[r][SW * strip + c8]);
            }
        }
        __syncthreads();
    }
}

}  // namespace mfma_prefill

bool prefill_mfma_supported(const PrefillArgs& a) {
    return a.bf16 && a.D == 128 && a.C == 64;
}

size_t prefill_mfma_workspace_bytes(int B, int T, int Hk, int Hv) {
    const size_t NTc = (size_t)(T + mfma_prefill::C - 1) / mfma_prefill::C;
    (void)Hk;
    return (size_t)B * Hv * NTc * mfma_prefill::WS_REC;
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t stream) {
    using namespace mfma_prefill;
    const int NTc = (a.T + C - 1) / C;
    const int prep_blocks = a.B * a.Hk * NTc;
    if (prep_blocks == 0) return hipSuccess;
    unsigned char* ws = static_cast<unsigned char*>(a.ws);
    hipLaunchKernelGGL(chunk_prep_kernel, dim3(prep_blocks), dim3(NT), 0, stream,
                       static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k), a.log_g, a.beta,
                       a.A_log, a.dt_bias, ws, a.T, NTc, a.Hk, a.Hv, a.l2norm);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int scan_blocks = a.B * a.Hv * (D / BVS);
    const int remap = (scan_blocks % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL(chunk_scan_kernel, dim3(scan_blocks), dim3(SNT), 0, stream,
                       static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k),
                       static_cast<const bf16_t*>(a.v), ws, a.h0, a.hT,
                       static_cast<bf16_t*>(a.o), a.T, NTc, a.Hk, a.Hv, a.q_scale, remap,
                       a.ckpt, a.ckpt_every, a.nck);
    return hipGetLastError();
}

}  // namespace gdn

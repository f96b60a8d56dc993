// prefill_fused.hip -- single-pass chunked gated-delta-rule prefill on bf16
// MFMA (gfx950): every per-chunk intermediate stays in LDS or registers.
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
// forward substitution -- inside the 16x16 diagonal blocks in fp32, then
// block by block with MFMA -- never by the Neumann power series ("Qwen3.6:
// Fused DeltaNet Direct-Solve Follow-Up", "Why This Exists", "Implementation
// Details", whose context-encoding kernel is likewise one fused chunked
// forward).  Only exp(gamma_r - gamma_s) with s <= r is formed, so nothing
// overflows for log g <= 0.
//
// One workgroup per (sequence, value head, 32 state columns); columns of the
// state evolve independently, so workgroups never talk.  Eight waves in five
// roles run a software pipeline over the chunks, one workgroup barrier per
// iteration; in iteration `it`:
//  * state waves (2, one per 16-column strip): chunk it.  K S, X,
//    Delta = T X and the state update, with the fp32 state in MFMA
//    accumulator layout for the whole sequence.  They leave the bf16 Delta
//    and the next state's bf16 operands in LDS for the output waves.
//  * output waves (2, one per pair of 16-row tiles): Q K^T of chunk it
//    (gated into P in registers), Q S of chunk it, and P Delta of chunk
//    it - 1 with the output store.  Q goes from memory straight to their
//    registers.  The output is formed transposed (O^T = S^T Q^T + Delta^T
//    P^T), so that each lane holds one token: the q norm and the decay of
//    a row are then per-lane scalars.
//  * Gram waves (2): chunk it + 2.  K K^T (MFMA), the k norms from its
//    diagonal, the in-chunk decay scan, the gate vectors, and A (diagonal
//    blocks fp32, others bf16) for the solve wave.
//  * solve wave (1): chunk it + 1.  T = (I + A)^-1 into LDS in MFMA operand
//    order.
//  * loader wave (1): direct global -> LDS loads of k and the gates of chunk
//    it + 4 and of v of chunk it + 2, and cache-line touches further ahead.
#include "prefill_mfma_common.h"

#include <type_traits>

namespace gdn {
namespace fused_prefill {

using namespace mfma_prefill;

constexpr int SW = 16;                 // state columns per strip
constexpr int NSTRIP = 2;              // strips per workgroup
constexpr int BVS = SW * NSTRIP;       // state columns per workgroup
constexpr int FNT = 512;               // threads per workgroup (8 waves)
constexpr int KBUF = 5;                // k chunks in LDS
constexpr int VBUF = 3;                // v chunks in LDS
constexpr int GBUF = 3;                // raw gate chunks in LDS
constexpr int GVBUF = 3;               // gate-vector sets in LDS
constexpr int K_AHEAD = 4;             // k and gates of chunk c are loaded in iteration c - K_AHEAD
constexpr int V_AHEAD = 2;             // v of chunk c in iteration c - V_AHEAD
constexpr int TOUCH_AHEAD = 6;         // cache lines of chunk c are touched in iteration c - TOUCH_AHEAD
constexpr int IT_FIRST = -K_AHEAD;     // first pipeline iteration

// wave roles
// (waves are dealt to the four SIMDs of a compute unit in turn, wave w to
// SIMD w % 4: the two state waves share their SIMDs with the light solve and
// loader waves, the output waves with the Gram waves)
constexpr int W_STATE = 0;    // waves 0, 1
constexpr int W_OUT = 2;      // waves 2, 3
constexpr int W_SOLVE = 4;
constexpr int W_LOAD = 5;
constexpr int W_GRAM = 6;     // waves 6, 7

// Gate vectors of a chunk, written by the Gram waves.
constexpr int GV_GRK = 0;     // Gamma_r rk_r        (state waves: row scale of K S)
constexpr int GV_WRK = 1;     // exp(gamma_C - gamma_s) rk_s  (state update)
constexpr int GV_BETA = 2;    // beta (0 on padding rows)
constexpr int GV_GC = 3;      // Gamma_C in entry 0
constexpr int GV_GAM = 4;     // gamma (output waves)
constexpr int GV_RK = 5;      // rk    (output waves)
constexpr int GV_U = 6;       // exp(gamma_e - gamma_s) rk_s, e = last row of s's 16-row block
constexpr int NGV = 7;

// 16-byte chunk c of a 256-byte k row r is stored at c ^ swz(r).  The LDS has
// 64 banks of 4 bytes; a 16-byte read is served 16 lanes at a time, in the
// lane groups {0-3, 12-15, 20-27} and {4-11, 16-19, 28-31} (and the same plus
// 32), an 8-byte read 32 lanes at a time.  Operand reads (lane 16g + n reads
// chunk 4ks + g of row 16i + n) are conflict-free: swz maps rows {0-3, 12-15}
// onto chunk positions closed under xor 1, and the partner lanes of a group
// differ in g by that bit.  Transposed reads (half wave: rows 4g + j x chunks
// 4A..4A+3, one 8-byte half) reach 16 bank pairs with 32 lanes; two-way is
// their floor, which they meet since swz(r) >> 2 takes each value twice over
// every 8 consecutive rows.
__host__ __device__ constexpr int swz(int r) { return (r & 1) | ((r & 8) >> 2) | ((r & 6) << 1); }
// 16-byte chunk c of a 64-byte v row s is stored at c ^ vswz(s): a transposed
// read of a strip's chunk pair takes rows 4g + j of both g of a half wave, and
// vswz sends odd g to the other strip's pair, so the 32 lanes hit distinct banks.
__host__ __device__ constexpr int vswz(int s) { return ((s >> 3) & 1) | ((s >> 1) & 2); }

struct GramScratch {          // private to one Gram wave
    float gam[C], bt[C], rk[C], u[C];
};

struct FusedSmem {
    uint4 K[KBUF][C * 16];                    // k rows, swizzled
    uint4 V[VBUF][C * 4];                     // v rows of the 32 columns: chunk c of row s at c ^ vswz(s)
    float graw[GBUF][2][C];                   // log g (or a) and beta (or b) as loaded
    float gv[GVBUF][NGV][C];                  // gate vectors (GV_*)
    struct {
        float d[4][16][16];                   // diagonal blocks, fp32, transposed: [block][s][r]
        uint16_t o[6][16][16];                // blocks below the diagonal, bf16: [ab_idx][r][s]
    } A[2];
    uint16_t Tc[4][16][16];                   // diagonal blocks of T, bf16, by column: [block][col][row]
    uint4 Timg[2][IMG_BYTES / 16];            // T in MFMA operand order (imgc)
    bf16x8 Sx[2][NSTRIP][4][64];              // bf16 state operands (per strip, k step, lane)
    bf16x8 Dx[2][NSTRIP][2][64];              // Delta operands
    GramScratch gs[2];
    uint32_t sink[64];                        // landing area of the cache-line touches
};

// direct 16-byte load of one lane into LDS at base + 16 * lane (base wave-uniform)
__device__ __forceinline__ void lds_load16(const void* g, void* lds_base) {
    __builtin_amdgcn_global_load_lds(g, lds_base, 16, 0, 0);
}
// direct 4-byte load of one lane into LDS at base + 4 * lane
__device__ __forceinline__ void lds_load4(const void* g, void* lds_base) {
    __builtin_amdgcn_global_load_lds(g, lds_base, 4, 0, 0);
}
// s_waitcnt immediate (gfx9 encoding): at most n vector memory operations
// outstanding; expcnt and lgkmcnt not waited for
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// s_waitcnt immediate: LDS operations complete; vmcnt and expcnt not waited for
constexpr int WAIT_LGKM0 = 0xF | (3 << 14) | (7 << 4);

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// transposed 4 x 16-bit read: within each 16 lanes, lane i receives element
// i & 3 of the 8-byte pieces addressed by lanes (i >> 2) + 4j, j = 0..3
__device__ __forceinline__ s16x4 ld_tr4(const void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// Workgroup barrier after this wave's LDS writes have completed.  Vector
// memory operations (loads into registers, output stores) stay in flight.
__device__ __forceinline__ void barrier_lds() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
// Order this wave's LDS writes before its later LDS reads of other lanes' data.
__device__ __forceinline__ void wave_lds_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
}

// Inclusive prefix sum over the 64 lanes with DPP: row shifts inside each
// 16-lane row, then the row totals broadcast into the later rows.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xf, false));
}
__device__ __forceinline__ float wave_scan(float x) {
    x = dpp_add<0x111, 0xf>(x);   // row_shr:1
    x = dpp_add<0x112, 0xf>(x);   // row_shr:2
    x = dpp_add<0x114, 0xf>(x);   // row_shr:4
    x = dpp_add<0x118, 0xf>(x);   // row_shr:8
    x = dpp_add<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
    x = dpp_add<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
    return x;
}
__device__ __forceinline__ float lane_of(float x, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
// 1 / max(sqrt(ss), 1e-6) with the hardware reciprocal square root (about
// one ulp; the bf16 operands these factors scale carry far larger rounding)
__device__ __forceinline__ float inv_l2_fast(float ss) {
    return ss > 1e-12f ? __builtin_amdgcn_rsqf(ss) : 1e6f;
}

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
// fp32 -> bf16 (round to nearest even) two values per conversion
__device__ __forceinline__ s16x4 cvt4(f32x4 v) {
    return __builtin_bit_cast(s16x4, __builtin_convertvector(v, bf16x4));
}
__device__ __forceinline__ bf16x8 cvt8(f32x4 lo, f32x4 hi) {
    const bf16x4 a = __builtin_convertvector(lo, bf16x4), b = __builtin_convertvector(hi, bf16x4);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
// sum of squares of the 8 bf16 values of an operand
__device__ __forceinline__ float sumsq8(bf16x8 x) {
    const u32x4 u = __builtin_bit_cast(u32x4, x);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) s += bf_lo(u[e]) * bf_lo(u[e]) + bf_hi(u[e]) * bf_hi(u[e]);
    return s;
}

// Gram wave tiles: K K^T tile (a, bb) is computed with s (block bb) on the M
// side and r (block a) on the N side: lane (g, n) element t holds
// k_s . k_r, s = 16 bb + 4g + t, r = 16 a + n.  Each Gram wave gates five
// tiles into A; it also forms the two diagonal tiles of the other wave, so
// that it has the norms of all 64 rows without waiting for it.
template <int HALF> struct GramTiles;
template <> struct GramTiles<0> {
    static constexpr int n = 7;
    static constexpr int a[7] = {0, 3, 3, 3, 3, 1, 2};
    static constexpr int b[7] = {0, 0, 1, 2, 3, 1, 2};
    static constexpr int own = 5;             // tiles gated into A
    static constexpr int diag[4] = {0, 5, 6, 4};   // tile index holding diagonal block x
};
template <> struct GramTiles<1> {
    static constexpr int n = 7;
    static constexpr int a[7] = {1, 1, 2, 2, 2, 0, 3};
    static constexpr int b[7] = {0, 1, 0, 1, 2, 0, 3};
    static constexpr int own = 5;
    static constexpr int diag[4] = {5, 1, 4, 6};
};

// Output-wave row tiles: wave OS forms rows of tiles ta[OS][0] and ta[OS][1]
// of the chunk.  Q K^T tiles (a, bb) with bb <= a are needed; P of tile x at
// k step m pairs the tiles bb = 2m, 2m + 1 (zero above the diagonal).
__host__ __device__ constexpr int out_tile(int os, int x) { return os == 0 ? (x == 0 ? 0 : 3) : (x == 0 ? 1 : 2); }

template <bool RAW>
__global__ __launch_bounds__(FNT) void chunk_fused_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float* __restrict__ log_g, const float* __restrict__ beta,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias,
    const float* h0, float* hT, bf16_t* __restrict__ o,
    int T, int Hk, int Hv, int l2norm, float q_scale, int xcd_remap,
    float* __restrict__ ckpt, int ckpt_every, int nck, const int* __restrict__ cu, long long total) {
    __shared__ FusedSmem sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int g = lane >> 4;
    const int n = lane & 15;
    const int sn = swz(n);               // swizzle of rows 16i + n

    constexpr int NB = D / BVS;          // column blocks per head
    int lid = blockIdx.x;
    if (xcd_remap) {
        // Workgroups are dispatched round-robin over the 8 XCDs (blockIdx & 7).
        // The G = (Hv / Hk) * NB workgroups of one (sequence, key head) read
        // the same k and q lines, so they go to one XCD and share its L2;
        // groups are dealt to the XCDs in turn and each XCD runs its groups in
        // order, so every XCD starts with the first sequences.  Needs the
        // number of groups B * Hk to be a multiple of 8.
        const int G = (Hv / Hk) * NB;
        const int kk = blockIdx.x >> 3;
        lid = ((kk / G) * 8 + (blockIdx.x & 7)) * G + kk % G;
    }
    const int bh = lid / NB;
    const int j0 = (lid % NB) * BVS;
    const int b = bh / Hv;
    const int h = bh - b * Hv;
    const int rr = Hv / Hk;
    const int hk = h / rr;
    size_t tb0;   // first token of sequence b
    int Tb;       // its length
    seq_span(cu, b, T, total, tb0, Tb);
    const int NTb = (Tb + C - 1) / C;
    const int Llast = Tb - (NTb - 1) * C;   // rows of the last chunk
    const size_t state_base = (size_t)bh * D * D;
    const bf16_t* kbase = k + (tb0 * Hk + hk) * D;
    const bf16_t* qbase = q + (tb0 * Hk + hk) * D;
    const bf16_t* vbase = v + (tb0 * Hv + h) * D + j0;
    bf16_t* obase = o + (tb0 * Hv + h) * D + j0;
    const int rowk = Hk * D;             // element stride between tokens of q and k
    const int rowv = Hv * D;             // element stride between tokens of v and o
    auto rows_of = [&](int c) __attribute__((always_inline)) { return c == NTb - 1 ? Llast : C; };

    // ======================= loader wave =======================
    // Every iteration issues the same number of loads (chunk indices clamped
    // into the sequence; a load for a chunk past the end fills a buffer no
    // role reads), so one wait-count immediate covers them: at the end of
    // iteration it, only the loads of iteration it may be outstanding.
    if (w == W_LOAD) {
        const int jb = j0 / BVS;                 // column block
        const int hh = h % rr;                   // value head within the key head's group
        // cache-line touches of chunk it + TOUCH_AHEAD, dealt out over the
        // workgroups that share the lines
        const bool t_k = (jb == 0 && hh == 0);
        const bool t_q = (jb == 0 && hh == min(1, rr - 1));
        const bool t_v = (jb == 1 || jb == 3);
        const bool t_g = (jb == 2 && hh == 0);
        const int ntouch = (t_k ? 2 : 0) + (t_q ? 2 : 0) + (t_v ? 1 : 0) + (t_g ? 2 : 0);
        const bf16_t* vline = vbase - (j0 & 63);   // the 128-byte v line holding the columns
        for (int it = IT_FIRST; it <= NTb; ++it) {
            if (NTb > 0) {
                {   // touches
                    const int ct = min(max(it + TOUCH_AHEAD, 0), NTb - 1);
                    const size_t row = (size_t)ct * C + min(lane, rows_of(ct) - 1);
                    if (t_k) {
                        lds_load4(kbase + row * rowk, sm.sink);
                        lds_load4(kbase + row * rowk + 64, sm.sink);
                    }
                    if (t_q) {
                        lds_load4(qbase + row * rowk, sm.sink);
                        lds_load4(qbase + row * rowk + 64, sm.sink);
                    }
                    if (t_v) lds_load4(vline + row * rowv, sm.sink);
                    if (t_g) {
                        lds_load4(log_g + (tb0 + row) * Hv + h, sm.sink);
                        lds_load4(beta + (tb0 + row) * Hv + h, sm.sink);
                    }
                }
                {   // k rows and gates of chunk it + K_AHEAD
                    const int cl = it + K_AHEAD;         // >= 0
                    const int cc = min(cl, NTb - 1);
                    const int last = rows_of(cc) - 1;
                    uint4* Kb = sm.K[cl % KBUF];
                    const unsigned char* kc = reinterpret_cast<const unsigned char*>(kbase + (size_t)cc * C * rowk);
#pragma unroll
                    for (int u = 0; u < 16; ++u) {       // 4 rows per load
                        const int r = 4 * u + (lane >> 4);
                        const uint32_t off = 2u * (uint32_t)(min(r, last) * rowk + 8 * ((lane & 15) ^ swz(r)));
                        lds_load16(kc + off, &Kb[64 * u]);
                    }
                    const size_t gi = (tb0 + (size_t)cc * C + min(lane, last)) * Hv + h;
                    lds_load4(log_g + gi, sm.graw[cl % GBUF][0]);
                    lds_load4(beta + gi, sm.graw[cl % GBUF][1]);
                }
                {   // v rows of chunk it + V_AHEAD
                    const int cl = it + V_AHEAD;
                    const int cc = min(max(cl, 0), NTb - 1);
                    const int last = rows_of(cc) - 1;
                    uint4* Vb = sm.V[(cl + 2 * VBUF) % VBUF];
                    const unsigned char* vc = reinterpret_cast<const unsigned char*>(vbase + (size_t)cc * C * rowv);
#pragma unroll
                    for (int u = 0; u < 4; ++u) {        // 16 rows per load
                        const int s2 = 16 * u + (lane >> 2);
                        const uint32_t off = 2u * (uint32_t)(min(s2, last) * rowv + 8 * ((lane & 3) ^ vswz(s2)));
                        lds_load16(vc + off, &Vb[64 * u]);
                    }
                }
                constexpr int NLOAD = 16 + 2 + 4;
                switch (ntouch) {   // wait for the previous iteration's loads
                    case 0: __builtin_amdgcn_s_waitcnt(waitcnt_vm(NLOAD)); break;
                    case 1: __builtin_amdgcn_s_waitcnt(waitcnt_vm(NLOAD + 1)); break;
                    case 2: __builtin_amdgcn_s_waitcnt(waitcnt_vm(NLOAD + 2)); break;
                    case 3: __builtin_amdgcn_s_waitcnt(waitcnt_vm(NLOAD + 3)); break;
                    case 4: __builtin_amdgcn_s_waitcnt(waitcnt_vm(NLOAD + 4)); break;
                    case 5: __builtin_amdgcn_s_waitcnt(waitcnt_vm(NLOAD + 5)); break;
                    case 6: __builtin_amdgcn_s_waitcnt(waitcnt_vm(NLOAD + 6)); break;
                    default: __builtin_amdgcn_s_waitcnt(waitcnt_vm(0)); break;
                }
            } else {
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            }
            // a plain barrier: a fenced one would also wait for this
            // iteration's loads
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        return;
    }

    // ======================= Gram waves =======================
    if (w == W_GRAM || w == W_GRAM + 1) {
        const int half = w - W_GRAM;
        float alog = 0.f, dtb = 0.f;
        if (RAW) {
            alog = A_log[h];
            dtb = dt_bias[h];
        }
        auto body = [&](auto HC) __attribute__((always_inline)) {
            constexpr int HALF = decltype(HC)::value;
            using TL = GramTiles<HALF>;
            GramScratch& gsc = sm.gs[HALF];
            for (int it = IT_FIRST; it <= NTb; ++it) {
                const int c = it + 2;
                if (c >= 0 && c < NTb) {
                    const uint4* Kc = sm.K[c % KBUF];
                    const int L = rows_of(c);
                    // ---- K operands of all four row blocks, natural k order
                    bf16x8 kop[4][4];
#pragma unroll
                    for (int blk = 0; blk < 4; ++blk)
#pragma unroll
                        for (int ks = 0; ks < 4; ++ks)
                            kop[blk][ks] = __builtin_bit_cast(bf16x8, Kc[(16 * blk + n) * 16 + ((4 * ks + g) ^ sn)]);
                    // ---- gates of the chunk: padding rows get log g = 0, beta = 0
                    float lg = sm.graw[c % GBUF][0][lane];
                    float bt = sm.graw[c % GBUF][1][lane];
                    if (RAW) {
                        lg = raw_log_decay(lg, alog, dtb);
                        bt = raw_beta(bt);
                    }
                    lg = chunk_log_decay(lg);
                    float x = (lane < L) ? lg : 0.f;
                    const float btv = (lane < L) ? bt : 0.f;
                    // ---- Gram tiles
                    f32x4 G[TL::n];
#pragma unroll
                    for (int i = 0; i < TL::n; ++i) {
                        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < 4; ++ks) acc = mfma32(kop[TL::b[i]][ks], kop[TL::a[i]][ks], acc);
                        G[i] = acc;
                    }
                    // ---- in-chunk inclusive scan of log g
                    x = wave_scan(x);
                    gsc.gam[lane] = x;
                    gsc.bt[lane] = btv;
                    // ---- inverse k norms from the diagonal of K K^T: lane
                    //      (g, n) with g = n >> 2 holds |k_r|^2 of r = 16 blk + n
                    //      in element n & 3
#pragma unroll
                    for (int blk = 0; blk < 4; ++blk) {
                        const f32x4 d4 = G[TL::diag[blk]];
                        const int t = n & 3;
                        const float ss = t == 0 ? d4[0] : t == 1 ? d4[1] : t == 2 ? d4[2] : d4[3];
                        if (g == (n >> 2)) gsc.rk[16 * blk + n] = l2norm ? inv_l2_fast(ss) : 1.f;
                    }
                    wave_lds_sync();
                    const float total_g = lane_of(x, 63);
                    // u_s = exp(gamma_e - gamma_s) rk_s with e the last row of
                    // s's 16-row block: below the diagonal blocks the decay
                    // exp(gamma_r - gamma_s) = exp(gamma_r - gamma_e) u_s / rk_s
                    // with both exponents <= 0
                    const float rkl = gsc.rk[lane];
                    const float g15 = lane_of(x, 15), g31 = lane_of(x, 31), g47 = lane_of(x, 47);
                    const float ge = lane < 16 ? g15 : lane < 32 ? g31 : lane < 48 ? g47 : total_g;
                    const float ul = exp_hw(ge - x) * rkl;
                    gsc.u[lane] = ul;
                    float* gvc = &sm.gv[c % GVBUF][0][0];
                    if (HALF == 0) {
                        gvc[GV_GRK * C + lane] = exp_hw(x) * rkl;
                        gvc[GV_WRK * C + lane] = exp_hw(total_g - x) * rkl;
                        gvc[GV_BETA * C + lane] = btv;
                        gvc[GV_GC * C + lane] = exp_hw(total_g);
                    } else {
                        gvc[GV_GAM * C + lane] = x;
                        gvc[GV_RK * C + lane] = rkl;
                        gvc[GV_U * C + lane] = ul;
                    }
                    wave_lds_sync();
                    // ---- gate the wave's own tiles into A
                    auto& Ab = sm.A[c & 1];
#pragma unroll
                    for (int i = 0; i < TL::own; ++i) {
                        const int a = TL::a[i], bb = TL::b[i];
                        const int r = 16 * a + n;
                        const float sr = gsc.bt[r] * gsc.rk[r];
                        const float gr = gsc.gam[r];
                        f32x4 val;
                        if (a == bb) {   // diagonal block: s < r, one exp per element
                            const f32x4 gs4 = *reinterpret_cast<const f32x4*>(&gsc.gam[16 * bb + 4 * g]);
                            const f32x4 ks4 = *reinterpret_cast<const f32x4*>(&gsc.rk[16 * bb + 4 * g]);
#pragma unroll
                            for (int t = 0; t < 4; ++t) {
                                const int s2 = 16 * bb + 4 * g + t;
                                const float xv = exp_hw(gr - gs4[t]) * sr * ks4[t] * G[i][t];
                                val[t] = (s2 < r) ? xv : 0.f;
                            }
#pragma unroll
                            for (int t = 0; t < 4; ++t) Ab.d[a][4 * g + t][n] = val[t];
                        } else {         // below the diagonal: every s < r
                            const f32x4 u4 = *reinterpret_cast<const f32x4*>(&gsc.u[16 * bb + 4 * g]);
                            const float f = sr * exp_hw(gr - gsc.gam[16 * bb + 15]);
#pragma unroll
                            for (int t = 0; t < 4; ++t) val[t] = G[i][t] * u4[t] * f;
                            *reinterpret_cast<s16x4*>(&Ab.o[ab_idx(a, bb)][n][4 * g]) = cvt4(val);
                        }
                    }
                }
                barrier_lds();
            }
        };
        if (half == 0) body(std::integral_constant<int, 0>{});
        else body(std::integral_constant<int, 1>{});
        return;
    }

    // ======================= solve wave =======================
    if (w == W_SOLVE) {
        // Image position (16-byte units of bf16 pairs -> element index) of the
        // 8-byte piece holding row R at physical columns 4q .. 4q + 3: the
        // 4-group q sits at logical offset kperm(q & 7) of its 32-column half.
        auto piece = [](int R, int q) __attribute__((always_inline)) {
            return imgc(R, 32 * (q >> 3) + kperm(q & 7));
        };
        // Blocks above the diagonal that the image stores are zero: block
        // (0, 1) and block (2, 3).  The solve never writes them.
#pragma unroll
        for (int bufi = 0; bufi < 2; ++bufi) {
            uint16_t* Tg = reinterpret_cast<uint16_t*>(sm.Timg[bufi]);
            *reinterpret_cast<uint2*>(Tg + piece(n, 4 + g)) = make_uint2(0u, 0u);
            *reinterpret_cast<uint2*>(Tg + piece(32 + n, 12 + g)) = make_uint2(0u, 0u);
        }
        float idc[16];   // column n of the identity
#pragma unroll
        for (int r = 0; r < 16; ++r) idc[r] = (r == n) ? 1.f : 0.f;
        for (int it = IT_FIRST; it <= NTb; ++it) {
            const int c = it + 1;
            if (c >= 0 && c < NTb) {
                auto& Ab = sm.A[c & 1];
                uint16_t* Tg = reinterpret_cast<uint16_t*>(sm.Timg[c & 1]);
                // ---- diagonal blocks: T_ii = (I + A_ii)^-1 by forward
                //      substitution; lane (g, n) is column n of block g.  Once
                //      row s of the column is final, its multiples are removed
                //      from the rows below it.
                {
                    // the block's columns below the diagonal, all read up front
                    f32x4 acol[15][4];
#pragma unroll
                    for (int s2 = 0; s2 < 15; ++s2)
#pragma unroll
                        for (int x4 = s2 / 4; x4 < 4; ++x4)
                            acol[s2][x4] = *reinterpret_cast<const f32x4*>(&Ab.d[g][s2][4 * x4]);
                    float tc[16];
#pragma unroll
                    for (int r = 0; r < 16; ++r) tc[r] = idc[r];
#pragma unroll
                    for (int s2 = 0; s2 < 15; ++s2)
#pragma unroll
                        for (int r = s2 + 1; r < 16; ++r) tc[r] -= acol[s2][r >> 2][r & 3] * tc[s2];
                    // column n of T_gg, 16 bf16, to Tc[g][n]
                    u32x4 lo, hi;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        lo[e] = cvt2(tc[2 * e], tc[2 * e + 1]);
                        hi[e] = cvt2(tc[8 + 2 * e], tc[8 + 2 * e + 1]);
                    }
                    *reinterpret_cast<u32x4*>(&sm.Tc[g][n][0]) = lo;
                    *reinterpret_cast<u32x4*>(&sm.Tc[g][n][8]) = hi;
                }
                wave_lds_sync();
                // ---- each diagonal block as row pieces (lane (g, n): T_bb[n][4g .. 4g + 3],
                //      by a transposed read of the column storage) into the
                //      image, and as column pieces (T_bb[4g .. 4g + 3][n])
                s16x4 rowT[4], colT[4];
#pragma unroll
                for (int bk = 0; bk < 4; ++bk) {
                    rowT[bk] = ld_tr4(&sm.Tc[bk][4 * g + (n >> 2)][4 * (n & 3)]);
                    colT[bk] = ld4(&sm.Tc[bk][n][4 * g]);
                    *reinterpret_cast<s16x4*>(Tg + piece(16 * bk + n, 4 * bk + g)) = rowT[bk];
                }
                // ---- blocks below the diagonal, from T (I + A) = I:
                //      T_ij = -(sum_{k=j+1}^{i} T_ik A_kj) T_jj, row block by
                //      row block from the diagonal leftwards (three independent
                //      chains), computed transposed so that each lane ends with
                //      row pieces T_ij[n][4g .. 4g + 3]:
                //      U^T = sum_k A_kj^T T_ik^T,  T_ij^T = -T_jj^T U^T.
                //      A_kj^T comes from the row-major A blocks by transposed reads.
                {
                    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                    s16x4 Tr[4][4];   // Tr[i][k]: row pieces of T_ik
#pragma unroll
                    for (int i = 1; i < 4; ++i) Tr[i][i] = rowT[i];
#pragma unroll
                    for (int d = 1; d < 4; ++d) {          // distance from the diagonal
#pragma unroll
                        for (int i = d; i < 4; ++i) {
                            const int j = i - d;
                            f32x4 U = zero;
#pragma unroll
                            for (int kb = j + 1; kb <= i; ++kb)
                                U = mfma16(ld_tr4(&Ab.o[ab_idx(kb, j)][4 * g + (n >> 2)][4 * (n & 3)]), Tr[i][kb], U);
                            const f32x4 Tij = mfma16(colT[j], cvt4(-U), zero);
                            Tr[i][j] = cvt4(Tij);
                            *reinterpret_cast<s16x4*>(Tg + piece(16 * i + n, 4 * j + g)) = Tr[i][j];
                        }
                    }
                }
            }
            barrier_lds();
        }
        return;
    }

    // ======================= state waves =======================
    if (w < W_OUT) {
        const int strip = w;
        const int jw = j0 + SW * strip;      // first state column of the strip
        // Per-lane LDS byte offsets inside a chunk's buffers, formed once; each
        // chunk adds its buffers' (wave-uniform) bases, and the parts that do
        // not depend on the lane are immediate offsets of the reads.
        // K operands (k step ks, row tile i at + 4096 i): row 16 i + n, 16-byte
        // chunk (4 ks + g) ^ swz(n)
        uint32_t koff[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) koff[ks] = n * 256 + 16 * ((4 * ks + g) ^ sn);
        // k^T operands of the update, read transposed from the k rows: tile a,
        // k step kk; lane (g, n) gets k column lpos(16a + n) at tokens
        // 32kk + 4g + j and 32kk + 16 + 4g + j.  It addresses row
        // 32kk + 4g + (n >> 2) (+ 16), chunk (4 (a >> 1) + (n & 3)) ^ swz(row),
        // half a & 1: offset toff[a >> 1] + 8192 kk + 8 (a & 1) (+ 4096)
        // swz(4g + j) = 4 tx + ty, split so that chunk 4 ah + m lands at 4 (ah ^ tx) + (m ^ ty)
        const int tx = ((n >> 3) & 1) | ((g & 1) << 1), ty = ((n >> 2) & 1) | (g & 2);
        uint32_t toff[4];
#pragma unroll
        for (int ah = 0; ah < 4; ++ah)
            toff[ah] = (4 * g + (n >> 2)) * 256 + 16 * (4 * (ah ^ tx) + ((n & 3) ^ ty));
        // v, transposed read: lane (g, n) receives v rows 16i + 4g + j, j = 0..3,
        // at column 16 strip + n; it addresses row 16i + 4g + (n >> 2),
        // columns 16 strip + 4 (n & 3) .. + 3 (+ 1024 i)
        const uint32_t voff = (4 * g + (n >> 2)) * 64 + 16 * ((2 * strip + ((n >> 1) & 1)) ^ vswz(4 * g)) + 8 * (n & 1);
        // T operands: rows 16i + n (i < 2: + 1024 i; i >= 2: + 2048 (i - 2)) at
        // chunk g, and rows 32 + n (+ 2048 for 48 + n) at chunk 4 + g (imgq)
        const uint32_t tof0 = 16 * imgq(n, g);
        const uint32_t tof1 = 16 * imgq(32 + n, g);
        const uint32_t tof2 = 16 * imgq(32 + n, 4 + g);
        const uint32_t goff = 16 * g;       // gate vector entries 16 i + 4 g .. + 3
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
        for (int it = IT_FIRST; it <= NTb; ++it) {
            const int c = it;
            if (c >= 0 && c < NTb) {
                const unsigned char* Kb = reinterpret_cast<const unsigned char*>(sm.K[c % KBUF]);
                const unsigned char* Tb8 = reinterpret_cast<const unsigned char*>(sm.Timg[c & 1]);
                const unsigned char* Vb = reinterpret_cast<const unsigned char*>(sm.V[c % VBUF]);
                const unsigned char* Gb = reinterpret_cast<const unsigned char*>(&sm.gv[c % GVBUF][0][0]) + goff;
                auto kop = [&](int i, int ks) __attribute__((always_inline)) {
                    return *reinterpret_cast<const bf16x8*>(Kb + koff[ks] + 4096 * i);
                };
                auto ldkt = [&](int a, int kk) __attribute__((always_inline)) {
                    const unsigned char* p = Kb + toff[a >> 1] + 8192 * kk + 8 * (a & 1);
                    const s16x4 lo = ld_tr4(p);
                    const s16x4 hi = ld_tr4(p + 4096);
                    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                };
                auto gvec = [&](int v, int i) __attribute__((always_inline)) {
                    return *reinterpret_cast<const f32x4*>(Gb + v * (C * 4) + 64 * i);
                };
                // ---- every K operand of the chunk, issued together
                bf16x8 kq[4][4];   // [k step][row tile]
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                    for (int i = 0; i < 4; ++i) kq[ks][i] = kop(i, ks);
                // ---- bf16 state operands (natural k order, see lpos), also
                //      left in LDS for the output waves (they use them in the
                //      next iteration)
                bf16x8 SB[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    SB[ks] = cvt8(S[2 * ks], S[2 * ks + 1]);
                    sm.Sx[c & 1][strip][ks][lane] = SB[ks];
                }
                bf16x8 at0[4], at1[2];   // T operands
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    at0[i] = *reinterpret_cast<const bf16x8*>(Tb8 + (i < 2 ? tof0 + 1024 * i : tof1 + 2048 * (i - 2)));
                at1[0] = *reinterpret_cast<const bf16x8*>(Tb8 + tof2);
                at1[1] = *reinterpret_cast<const bf16x8*>(Tb8 + tof2 + 2048);
                __builtin_amdgcn_sched_barrier(0);
                // ---- K S as eight independent chains (k steps 0, 1 and 2, 3
                //      into separate accumulators, added afterwards)
                f32x4 KA[4], KB[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) KA[i] = mfma32(kq[0][i], SB[0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int i = 0; i < 4; ++i) KB[i] = mfma32(kq[2][i], SB[2], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int i = 0; i < 4; ++i) KA[i] = mfma32(kq[1][i], SB[1], KA[i]);
#pragma unroll
                for (int i = 0; i < 4; ++i) KB[i] = mfma32(kq[3][i], SB[3], KB[i]);
                __builtin_amdgcn_sched_barrier(0);
                // ---- what X, the update and its gates need, read behind K S
                s16x4 vt[4];
                f32x4 btv[4], grk[4];
                f32x4 wg[4];             // exp(gamma_C - gamma) rk of the four row tiles
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    vt[i] = ld_tr4(Vb + voff + 1024 * i);
                    grk[i] = gvec(GV_GRK, i);
                    btv[i] = gvec(GV_BETA, i);
                }
                bf16x8 akt[8][2];
#pragma unroll
                for (int a = 0; a < 8; ++a) akt[a][0] = ldkt(a, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) wg[i] = gvec(GV_WRK, i);
                const float GC = *reinterpret_cast<const float*>(Gb - goff + GV_GC * (C * 4));
#pragma unroll
                for (int a = 0; a < 8; ++a) akt[a][1] = ldkt(a, 1);
                f32x4 KS[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) KS[i] = KA[i] + KB[i];
                // ---- X = beta (V - Gamma rk K S)
                f32x4 X[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        X[i][t] = btv[i][t] * (__uint_as_float((uint32_t)(uint16_t)vt[i][t] << 16) - grk[i][t] * KS[i][t]);
                const bf16x8 XB0 = cvt8(X[0], X[1]);
                const bf16x8 XB1 = cvt8(X[2], X[3]);
                __builtin_amdgcn_sched_barrier(0);
                // ---- Delta = T X (T lower triangular: row tile i needs k steps <= i/2)
                f32x4 Dl[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) Dl[i] = mfma32(at0[i], XB0, f32x4{0.f, 0.f, 0.f, 0.f});
                Dl[2] = mfma32(at1[0], XB1, Dl[2]);
                Dl[3] = mfma32(at1[1], XB1, Dl[3]);
                __builtin_amdgcn_sched_barrier(0);
                // ---- Delta operands: plain (to the output waves) and scaled (state update)
                sm.Dx[c & 1][strip][0][lane] = cvt8(Dl[0], Dl[1]);
                sm.Dx[c & 1][strip][1][lane] = cvt8(Dl[2], Dl[3]);
                const bf16x8 DWB0 = cvt8(Dl[0] * wg[0], Dl[1] * wg[1]);
                const bf16x8 DWB1 = cvt8(Dl[2] * wg[2], Dl[3] * wg[3]);
                // ---- state update S <- Gamma_C S + K^T (wrk Delta), 8 independent tiles
#pragma unroll
                for (int a = 0; a < 8; ++a) S[a] = mfma32(akt[a][0], DWB0, S[a] * GC);
#pragma unroll
                for (int a = 0; a < 8; ++a) S[a] = mfma32(akt[a][1], DWB1, S[a]);
                // ---- checkpoint slot: the state after every ckpt_every tokens
                //      and after the last token
                if (ckpt) {
                    const int done = min((c + 1) * C, Tb);
                    if (done % ckpt_every == 0 || done == Tb) {
                        const int slot = (done + ckpt_every - 1) / ckpt_every - 1;
                        float* cp = ckpt + (((size_t)b * nck + slot) * Hv + h) * D * D + jw + n;
#pragma unroll
                        for (int a = 0; a < 8; ++a)
#pragma unroll
                            for (int t = 0; t < 4; ++t) cp[(32 * (a >> 1) + 8 * g + 4 * (a & 1) + t) * D] = S[a][t];
                    }
                }
            }
            barrier_lds();
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
    // Wave OS forms the output rows of tiles out_tile(OS, 0) and out_tile(OS, 1)
    // of each chunk, transposed: lane (g, n) element t of a tile holds token
    // 16 a + n at state column 16 strip + 4g + t.
    auto out_body = [&](auto OSC) __attribute__((always_inline)) {
        constexpr int OS = decltype(OSC)::value;
        constexpr int A0 = out_tile(OS, 0), A1 = out_tile(OS, 1);
        // q operands (rows 16 a + n, natural k order) of chunk c (clamped into
        // the sequence), loaded into registers one iteration ahead
        auto load_q = [&](int c, bf16x8 (&qd)[2][4]) __attribute__((always_inline)) {
            c = min(c, NTb - 1);
            const int last = rows_of(c) - 1;
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int r = min(16 * (x == 0 ? A0 : A1) + n, last);
                const bf16_t* qr = qbase + ((size_t)c * C + r) * rowk + 8 * g;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) qd[x][ks] = *reinterpret_cast<const bf16x8*>(qr + 32 * ks);
            }
        };
        // One step per iteration: gate chunk c (its q rows in qc) and finish
        // chunk c - 1 (its q rows in qp, its P operands and Gamma rq from the
        // previous step), interleaved so that the latencies of one half hide
        // behind the work of the other.
        bf16x8 pop[3];             // P operands of chunk c - 1: (x0, m0), (x1, m0), (x1, m1)
        float grq[2];              // q_scale Gamma_r rq_r of chunk c - 1's rows
        auto step = [&](int c, const bf16x8 (&qc)[2][4], const bf16x8 (&qp)[2][4]) __attribute__((always_inline)) {
            const bool gate_c = c < NTb;     // chunk c exists
            const bool fin = c >= 1;         // chunk c - 1 exists
            f32x4 qq[2], PT[2][4];
            const uint4* Kc = sm.K[c % KBUF];
            // ---- chunk c, first half: Q Q^T diagonal tiles and the Q K^T
            //      tiles (s = 16 bb + 4g + t on the M side, r on the N side)
            if (gate_c) {
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    qq[x] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) qq[x] = mfma32(qc[x][ks], qc[x][ks], qq[x]);
                }
#pragma unroll
                for (int x = 0; x < 2; ++x)
#pragma unroll
                    for (int bb = 0; bb < 4; ++bb) PT[x][bb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    if (bb > A1) continue;
                    bf16x8 kb[4];
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        kb[ks] = __builtin_bit_cast(bf16x8, Kc[(16 * bb + n) * 16 + ((4 * ks + g) ^ sn)]);
#pragma unroll
                    for (int x = 0; x < 2; ++x) {
                        if (bb > (x == 0 ? A0 : A1)) continue;
#pragma unroll
                        for (int ks = 0; ks < 4; ++ks) PT[x][bb] = mfma32(kb[ks], qc[x][ks], PT[x][bb]);
                    }
                }
            }
            // ---- chunk c - 1: O^T = Gamma rq (S^T Q^T) + Delta^T P^T, store.
            //      S of chunk c - 1 was left in LDS by the state waves at the
            //      start of the previous iteration.
            if (fin) {
                const int cp = c - 1;
                const int L = rows_of(cp);
                bf16_t* oc = obase + (size_t)cp * C * rowv;
#pragma unroll
                for (int st = 0; st < NSTRIP; ++st) {
                    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const bf16x8 sb = sm.Sx[cp & 1][st][ks][lane];
                        a0 = mfma32(sb, qp[0][ks], a0);
                        a1 = mfma32(sb, qp[1][ks], a1);
                    }
                    const bf16x8 D0 = sm.Dx[cp & 1][st][0][lane];
                    const bf16x8 D1 = sm.Dx[cp & 1][st][1][lane];
                    f32x4 O0 = mfma32(D0, pop[0], a0 * grq[0]);
                    f32x4 O1 = mfma32(D0, pop[1], a1 * grq[1]);
                    O1 = mfma32(D1, pop[2], O1);
                    const int r0 = 16 * A0 + n, r1 = 16 * A1 + n;
                    if (r0 < L) *reinterpret_cast<s16x4*>(oc + (size_t)r0 * rowv + SW * st + 4 * g) = cvt4(O0);
                    if (r1 < L) *reinterpret_cast<s16x4*>(oc + (size_t)r1 * rowv + SW * st + 4 * g) = cvt4(O1);
                }
            }
            // ---- chunk c, second half: inverse q norms of the lane's rows
            //      from the Q Q^T diagonal (lane (g, n) with g = n >> 2 holds
            //      |q_r|^2 of r = 16 a + n in element n & 3; q_scale folded
            //      in: it scales both terms of the output), then the gating of
            //      P by exp(gamma_r - gamma_s) rq_r rk_s for s <= r: one exp
            //      per element on the diagonal blocks, exp(gamma_r - gamma_e)
            //      u_s below them
            if (gate_c) {
                const float* gate = &sm.gv[c % GVBUF][0][0];
                float rq[2], gr[2];
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const int t = n & 3;
                    float ss = t == 0 ? qq[x][0] : t == 1 ? qq[x][1] : t == 2 ? qq[x][2] : qq[x][3];
                    ss = __shfl(ss, 16 * (n >> 2) + n, 64);
                    rq[x] = q_scale * (l2norm ? inv_l2_fast(ss) : 1.f);
                    gr[x] = gate[GV_GAM * C + 16 * (x == 0 ? A0 : A1) + n];
                }
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
#pragma unroll
                    for (int x = 0; x < 2; ++x) {
                        const int a = x == 0 ? A0 : A1;
                        if (bb > a) continue;
                        if (bb == a) {
                            const f32x4 gs4 = *reinterpret_cast<const f32x4*>(&gate[GV_GAM * C + 16 * bb + 4 * g]);
                            const f32x4 rk4 = *reinterpret_cast<const f32x4*>(&gate[GV_RK * C + 16 * bb + 4 * g]);
#pragma unroll
                            for (int t = 0; t < 4; ++t) {
                                const float xv = exp_hw(gr[x] - gs4[t]) * rq[x] * rk4[t] * PT[x][bb][t];
                                PT[x][bb][t] = (4 * g + t <= n) ? xv : 0.f;
                            }
                        } else {
                            const f32x4 u4 = *reinterpret_cast<const f32x4*>(&gate[GV_U * C + 16 * bb + 4 * g]);
                            const float f = rq[x] * exp_hw(gr[x] - gate[GV_GAM * C + 16 * bb + 15]);
#pragma unroll
                            for (int t = 0; t < 4; ++t) PT[x][bb][t] = PT[x][bb][t] * u4[t] * f;
                        }
                    }
                }
                pop[0] = cvt8(PT[0][0], PT[0][1]);
                pop[1] = cvt8(PT[1][0], PT[1][1]);
                pop[2] = cvt8(PT[1][2], PT[1][3]);
                grq[0] = exp_hw(gr[0]) * rq[0];
                grq[1] = exp_hw(gr[1]) * rq[1];
            }
            barrier_lds();
        };
        // The pipeline's first iterations carry nothing for these waves; then
        // one step per chunk and a last step that only finishes.  The q rows
        // of chunks c - 1, c and c + 1 (loaded one iteration ahead) rotate
        // through three register sets; every steady-state step issues the
        // same memory operations (q rows past the end are loaded clamped),
        // which keeps the compiler's wait counts exact across the sets.
        for (int it = IT_FIRST; it < 0; ++it) barrier_lds();
        if (NTb > 0) {
            bf16x8 q0[2][4], q1[2][4], q2[2][4];
            load_q(0, q0);
            load_q(1, q1);
            step(0, q0, q2);
            int c = 1;
            for (; c + 2 < NTb; c += 3) {
                load_q(c + 1, q2);
                step(c, q1, q0);
                load_q(c + 2, q0);
                step(c + 1, q2, q1);
                load_q(c + 3, q1);
                step(c + 2, q0, q2);
            }
            // at most two chunks left; chunk c's q rows are in q1, c - 1's in q0
            if (c < NTb) {
                load_q(c + 1, q2);
                step(c, q1, q0);
                ++c;
                if (c < NTb) {
                    step(c, q2, q1);
                    ++c;
                    step(c, q0, q2);   // finishes chunk c - 1 only
                } else {
                    step(c, q0, q1);   // finishes chunk c - 1 only
                }
            } else {
                step(c, q2, q0);       // finishes chunk c - 1 only
            }
        } else {
            barrier_lds();
        }
    };
    if (w == W_OUT) out_body(std::integral_constant<int, 0>{});
    else out_body(std::integral_constant<int, 1>{});
}

}  // namespace fused_prefill

hipError_t launch_prefill_fused(const PrefillArgs& a, hipStream_t stream) {
    using namespace fused_prefill;
    const int blocks = a.B * a.Hv * (D / BVS);
    if (blocks == 0 || a.T == 0) return hipSuccess;
    const int remap = ((a.B * a.Hk) % 8 == 0) ? 1 : 0;
    auto kernel = a.A_log ? chunk_fused_kernel<true> : chunk_fused_kernel<false>;
    hipLaunchKernelGGL(kernel, dim3(blocks), dim3(FNT), 0, stream,
                       static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k),
                       static_cast<const bf16_t*>(a.v), a.log_g, a.beta, a.A_log, a.dt_bias,
                       a.h0, a.hT, static_cast<bf16_t*>(a.o), a.T, a.Hk, a.Hv, a.l2norm, a.q_scale,
                       remap, a.ckpt, a.ckpt_every, a.nck, a.cu, a.total);
    return hipGetLastError();
}

}  // namespace gdn

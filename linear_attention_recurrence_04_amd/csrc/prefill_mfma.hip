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
#include "prefill_mfma_common.h"
#include <type_traits>

namespace gdn {
namespace mfma_prefill {

// The prep kernel with the gates given; the same body with raw gate
// projections is compiled in prefill_prep_raw.hip.
#define PREP_KERNEL chunk_prep_kernel
#define PREP_RAW false
#include "prefill_prep.inc"
#undef PREP_KERNEL
#undef PREP_RAW

// ===========================================================================
// scan: one workgroup per (b, value head h, 32 state columns), in three roles:
//  * two state waves (one per 16-column strip): K S, X, Delta = T X and the
//    state update, the chain that carries the state from chunk to chunk;
//  * two output waves (one per half of the chunk's 64 rows, both strips), one
//    chunk behind: Q S and P Delta from the bf16 state and Delta operands the
//    state waves leave in LDS, and the output stores.  Splitting by rows
//    rather than by strips lets each read only half of the q rows and of P;
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

// 16-byte chunk c of a 256-byte k or q row r is stored at c ^ swz(r).  The
// LDS has 64 banks of 4 bytes, so a chunk's banks follow from its position in
// the row.  A 16-byte read is served 16 lanes at a time, in the lane groups
// {0-3, 12-15, 20-27} and {4-11, 16-19, 28-31} (and the same plus 32); an
// 8-byte read, transposed or not, 32 lanes at a time (each half wave).
// Row operand reads (lane 16g + n reads chunk 4ks + g of row 16i + n) are
// conflict-free: swz maps rows {0-3, 12-15} onto chunk positions closed under
// xor 1, and the partner lanes of a group differ in g by exactly that bit.
// Transposed reads (half wave: rows 4g + j, j < 4, g < 2, x chunks 4A..4A+3,
// one 8-byte half) reach only 16 bank pairs with 32 lanes, so two-way is their
// floor; they meet it because swz(r) >> 2 takes each value twice over every
// 8 consecutive rows.
__host__ __device__ constexpr int swz(int r) { return (r & 1) | ((r & 8) >> 2) | ((r & 6) << 1); }
// 16-byte chunk c of a 64-byte v row s (32 columns) is stored at c ^ vswz(s).
// A transposed read of a strip's two chunks takes rows 4g + j of both g of a
// half wave; vswz sends the rows of odd g to the other strip's chunk pair, so
// that the 32 lanes reach 32 distinct bank pairs.
__host__ __device__ constexpr int vswz(int s) { return ((s >> 3) & 1) | ((s >> 1) & 2); }

struct KSet {              // state-wave inputs of one chunk
    uint4 K[C * 16];       // k rows, swizzled
    uint4 T[IMG_BYTES / 16];   // T image
    uint4 V[C * 4];        // v rows of the 32 columns: chunk c of row s at c ^ vswz(s)
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
    int T, int NRc, int Hk, int Hv, float q_scale, int xcd_remap,
    float* __restrict__ ckpt, int ckpt_every, int nck, const int* __restrict__ cu, long long total,
    int c_first, int n_chunks) {
    __shared__ ScanSmem sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int g = lane >> 4;
    const int n = lane & 15;

    constexpr int NB = D / BVS;          // column blocks per head
    int lid = blockIdx.x;
    if (xcd_remap) {
        // Workgroups are dispatched round-robin over the 8 XCDs (blockIdx & 7).
        // The G = (Hv / Hk) * NB workgroups of one (sequence, key head) read
        // the same k and q lines, so they go to one XCD and share its L2;
        // groups are dealt to the XCDs in turn and each XCD runs its groups in
        // order, so every XCD starts with the first sequences (a batch sorted
        // by decreasing length starts its longest chains first everywhere).
        // Needs the number of groups B * Hk to be a multiple of 8.
        const int G = (Hv / Hk) * NB;
        const int kk = blockIdx.x >> 3;
        lid = ((kk / G) * 8 + (blockIdx.x & 7)) * G + kk % G;
    }
    const int bh = lid / NB;
    const int j0 = (lid % NB) * BVS;
    const int b = bh / Hv;
    const int h = bh - b * Hv;
    const int hk = h / (Hv / Hk);
    size_t tb0;   // first token of sequence b
    int Tb;       // its length (T for equal-length batches)
    seq_span(cu, b, T, total, tb0, Tb);
    // The launch runs chunks [c_first, c_first + n_chunks) of each sequence,
    // from the state h0 holds before chunk c_first.
    const int Tseq = Tb;                 // the whole sequence (checkpoint slots)
    const int skip = min(c_first * C, Tb);
    tb0 += skip;
    Tb = min(Tb - skip, n_chunks * C);
    const int NTb = (Tb + C - 1) / C;    // chunks to run: records 0 .. NTb - 1 of the NRc per head
    const size_t state_base = (size_t)bh * D * D;
    const unsigned char* rec0 = ws + (size_t)bh * NRc * WS_REC;
    const bf16_t* kbase = k + (tb0 * Hk + hk) * D;
    const bf16_t* qbase = q + (tb0 * Hk + hk) * D;
    const bf16_t* vbase = v + (tb0 * Hv + h) * D + j0;
    bf16_t* obase = o + (tb0 * Hv + h) * D + j0;
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
                offv[u] = 2u * (uint32_t)(min(s2, last) * rowv + 8 * ((lane & 3) ^ vswz(s2)));
            }
        };
        const int last_rows = Tb - (NTb - 1) * C - 1;   // last row of the last chunk
        kq_offsets(offk, C - 1);
        kq_offsets(offq, C - 1);
        v_offsets(C - 1);

        // The k side of a chunk is 27 direct loads of 1 KiB: k 16, T 6, v 4,
        // gates 1; seven on loader waves 0..2 (the gates on wave 2) and six
        // on wave 3, which also issues the workgroup's cache-line touches.
        constexpr int NKLOADS = 7;
        constexpr int NKLOADS3 = 6;
        auto load_k = [&](int chunk, int slot) __attribute__((always_inline)) {
            if (chunk == NTb - 1) {   // the last chunk: clamp its rows
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
        };
        auto load_q = [&](int chunk, int slot) __attribute__((always_inline)) {
            if (chunk == NTb - 1) kq_offsets(offq, last_rows);
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
        // workgroup of those that share it, and the sets are dealt out so that
        // no workgroup of a key head's group touches more than one (k and q
        // both only when a key head has a single value head): the T, P and
        // gate record by the head's column block 0, the v lines of columns
        // 0..63 and 64..127 (128 bytes each) by column blocks 1 and 3, the k
        // lines by column block 2 of the group's first value head, the q
        // lines by column block 2 of its second.  Loader wave 3 issues them,
        // two lines per lane per set.
        constexpr int TOUCH_AHEAD = 3;
        const int jb = j0 / BVS;               // column block
        const int hh = h % (Hv / Hk);          // value head within the key head's group
        const bool t_rec = (jb == 0);
        const bool t_v = (jb == 1 || jb == 3);
        const bool t_k = (jb == 2 && hh == 0);
        const bool t_q = (jb == 2 && hh == min(1, Hv / Hk - 1));
        const bool toucher = (lw == 3) && (t_rec || t_v || t_k || t_q);
        const bool two_sets = t_k && t_q;      // a key head with a single value head
        const bf16_t* vline = vbase - (j0 & 63);   // the 128-byte v line holding the columns
        auto touch = [&](int chunk) __attribute__((always_inline)) {
            const int t0 = chunk * C;
            const int row = t0 + min(lane, Tb - t0 - 1);
            uint32_t* sink = sm.sink[lw];
            const unsigned char* rec = rec0 + (size_t)chunk * WS_REC;   // 106 lines of 128 bytes
            if (t_rec) {
                lds_load4(rec + 128 * lane, sink);
                lds_load4(rec + 128 * min(64 + lane, WS_REC / 128 - 1), sink);
            } else if (t_v) {
                lds_load4(vline + (size_t)row * rowv, sink);
                lds_load4(vline + (size_t)row * rowv + 32, sink);   // same line: keeps two per set
            } else {
                if (t_k) {
                    lds_load4(kbase + (size_t)row * rowk, sink);
                    lds_load4(kbase + (size_t)row * rowk + 64, sink);
                }
                if (t_q) {
                    lds_load4(qbase + (size_t)row * rowk, sink);
                    lds_load4(qbase + (size_t)row * rowk + 64, sink);
                }
            }
        };
        // iteration c: the state waves work on chunk c and the output waves on
        // chunk c - 1; load the q side of chunk c, then the k side of chunk
        // c + 2, then the touches.  Operations complete in issue order, so
        // waiting until only the k loads and touches of this iteration are
        // outstanding covers the q side of chunk c and the k side of chunk
        // c + 1 (issued an iteration ago): what the next iteration reads.
        if (toucher)
            for (int c = 1; c <= TOUCH_AHEAD && c < NTb; ++c) touch(c);
        if (NTb > 0) load_k(0, 0);
        if (NTb > 1) load_k(1, 1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        for (int c = 0; c <= NTb; ++c) {
            if (c < NTb) load_q(c, c & 1);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            const bool kload = c + 2 < NTb;
            if (kload) load_k(c + 2, (c + 2) % 3);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            const bool tload = toucher && c + TOUCH_AHEAD < NTb;
            if (tload) touch(c + TOUCH_AHEAD);
            if (lw != 3) {
                if (kload) __builtin_amdgcn_s_waitcnt(waitcnt_vm(NKLOADS));
                else __builtin_amdgcn_s_waitcnt(0);
            } else if (kload && tload) {
                if (two_sets) __builtin_amdgcn_s_waitcnt(waitcnt_vm(NKLOADS3 + 4));
                else __builtin_amdgcn_s_waitcnt(waitcnt_vm(NKLOADS3 + 2));
            } else if (kload) {
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(NKLOADS3));
            } else if (tload) {
                if (two_sets) __builtin_amdgcn_s_waitcnt(waitcnt_vm(4));
                else __builtin_amdgcn_s_waitcnt(waitcnt_vm(2));
            } else {
                __builtin_amdgcn_s_waitcnt(0);
            }
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
        // one chunk; the buffer indices (c % 3, c % 2) are compile-time
        // constants, so that every LDS address is a fixed lane offset plus
        // an immediate
        auto chunk_step = [&](auto kbuf, auto xbuf, int c) __attribute__((always_inline)) {
            constexpr int KB = decltype(kbuf)::value;
            constexpr int XB = decltype(xbuf)::value;
            if (c < NTb) {
                const KSet& B = sm.ks[KB];
                // ---- K operands of the first k step, then the bf16 state
                //      operands (also left in LDS for the output wave)
                bf16x8 ak[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) ak[i] = __builtin_bit_cast(bf16x8, B.K[(16 * i + n) * 16 + (g ^ sn)]);
                bf16x8 SB[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    SB[ks] = pack8(S[2 * ks], S[2 * ks + 1]);
                    sm.Sx[XB][strip][ks][lane] = SB[ks];   // for the output wave
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
                f32x4 wg[4];             // exp(gamma_C - gamma) rk of the four row tiles
                float GC;                // Gamma_C
                // k^T operands of the state update, read transposed from the k
                // rows: tile a, k step kk; lane (g, n) gets k column lpos(16a + n)
                // at tokens 32kk + 4g + j and 32kk + 16 + 4g + j
                const unsigned char* Kb = reinterpret_cast<const unsigned char*>(B.K);
                auto ldkt = [&](int a, int kk) __attribute__((always_inline)) {
                    const int r0 = 32 * kk + 4 * g + (n >> 2);
                    const int ch = 4 * (a >> 1) + (n & 3);
                    const int sz = swz(4 * g + (n >> 2));   // = swz(r0) = swz(r0 + 16)
                    const s16x4 lo = ld_tr4(Kb + r0 * 256 + 16 * (ch ^ sz) + 8 * (a & 1));
                    const s16x4 hi = ld_tr4(Kb + (r0 + 16) * 256 + 16 * (ch ^ sz) + 8 * (a & 1));
                    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                };
                bf16x8 akt[8][2];
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
                            vt[i] = ld_tr4(Vb + sr * 64 + 16 * ((2 * strip + ((n >> 1) & 1)) ^ vswz(sr)) + 8 * (n & 1));
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
                        wg[0] = *reinterpret_cast<const f32x4*>(&B.gate[C + 4 * g]);
                        wg[1] = *reinterpret_cast<const f32x4*>(&B.gate[C + 16 + 4 * g]);
                        wg[2] = *reinterpret_cast<const f32x4*>(&B.gate[C + 32 + 4 * g]);
                        wg[3] = *reinterpret_cast<const f32x4*>(&B.gate[C + 48 + 4 * g]);
                        GC = B.gate[3 * C];
                    }
                    if (ks == 3) {
#pragma unroll
                        for (int a = 0; a < 8; ++a) akt[a][0] = ldkt(a, 0);
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
                __builtin_amdgcn_sched_barrier(0);
                // ---- Delta = T X (T lower triangular: row tile i needs k steps <= i/2)
                f32x4 Dl[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) Dl[i] = mfma32(at0[i], XB0, f32x4{0.f, 0.f, 0.f, 0.f});
                Dl[2] = mfma32(at1[0], XB1, Dl[2]);
                Dl[3] = mfma32(at1[1], XB1, Dl[3]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int a = 0; a < 8; ++a) akt[a][1] = ldkt(a, 1);
                __builtin_amdgcn_sched_barrier(0);
                // ---- Delta operands: plain (to the output wave) and scaled (state update)
                sm.Dx[XB][strip][0][lane] = pack8(Dl[0], Dl[1]);
                sm.Dx[XB][strip][1][lane] = pack8(Dl[2], Dl[3]);
                const bf16x8 DWB0 = pack8(Dl[0] * wg[0], Dl[1] * wg[1]);
                const bf16x8 DWB1 = pack8(Dl[2] * wg[2], Dl[3] * wg[3]);
                // ---- state update S <- Gamma_C S + K^T (wrk Delta), 8 independent tiles
#pragma unroll
                for (int a = 0; a < 8; ++a) S[a] = mfma32(akt[a][0], DWB0, S[a] * GC);
#pragma unroll
                for (int a = 0; a < 8; ++a) S[a] = mfma32(akt[a][1], DWB1, S[a]);
                // ---- checkpoint slot: the state after every ckpt_every tokens
                //      and after the last token
                if (ckpt) {
                    const int done = skip + min((c + 1) * C, Tb);   // tokens of the sequence
                    if (done % ckpt_every == 0 || done == Tseq) {
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
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        for (int c = 0; c <= NTb; c += 6) {
            chunk_step(I0{}, I0{}, c);
            if (c + 1 <= NTb) chunk_step(I1{}, I1{}, c + 1);
            if (c + 2 <= NTb) chunk_step(I2{}, I0{}, c + 2);
            if (c + 3 <= NTb) chunk_step(I0{}, I1{}, c + 3);
            if (c + 4 <= NTb) chunk_step(I1{}, I0{}, c + 4);
            if (c + 5 <= NTb) chunk_step(I2{}, I1{}, c + 5);
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
    // Output wave `half` forms rows 32 half .. 32 half + 31 of the chunk's
    // output for both strips, so each reads half of the q rows and of P.
    // Rows 0..31 of P are zero past column 31, so the first half needs only
    // the first k step of P Delta.
    const int half = strip;
    for (int c = 0; c <= NTb; ++c) {
        if (c >= 1) {
            const int cc = c - 1;
            const QSet& B = sm.qs[cc & 1];
            bf16x8 SB[NSTRIP][4], aq[2];
#pragma unroll
            for (int ii = 0; ii < 2; ++ii)
                aq[ii] = __builtin_bit_cast(bf16x8, B.Q[(16 * (2 * half + ii) + n) * 16 + (g ^ sn)]);
#pragma unroll
            for (int st = 0; st < NSTRIP; ++st)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) SB[st][ks] = sm.Sx[cc & 1][st][ks][lane];
            f32x4 QS[NSTRIP][2];
#pragma unroll
            for (int st = 0; st < NSTRIP; ++st)
#pragma unroll
                for (int ii = 0; ii < 2; ++ii) QS[st][ii] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                bf16x8 nq[2];
                if (ks < 3) {
#pragma unroll
                    for (int ii = 0; ii < 2; ++ii)
                        nq[ii] = __builtin_bit_cast(bf16x8, B.Q[(16 * (2 * half + ii) + n) * 16 + ((4 * (ks + 1) + g) ^ sn)]);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int st = 0; st < NSTRIP; ++st)
#pragma unroll
                    for (int ii = 0; ii < 2; ++ii) QS[st][ii] = mfma32(aq[ii], SB[st][ks], QS[st][ii]);
                __builtin_amdgcn_sched_barrier(0);
                if (ks < 3) {
#pragma unroll
                    for (int ii = 0; ii < 2; ++ii) aq[ii] = nq[ii];
                }
            }
            bf16x8 ap0[2], ap1[2];
#pragma unroll
            for (int ii = 0; ii < 2; ++ii) {
                ap0[ii] = __builtin_bit_cast(bf16x8, B.P[imgq(16 * (2 * half + ii) + n, g)]);
                if (half) ap1[ii] = __builtin_bit_cast(bf16x8, B.P[imgq(32 + 16 * ii + n, 4 + g)]);
            }
            f32x4 grq[2];
#pragma unroll
            for (int ii = 0; ii < 2; ++ii)
                grq[ii] = *reinterpret_cast<const f32x4*>(&B.gate[16 * (2 * half + ii) + 4 * g]);
            uint16_t (*Ot)[OS] = sm.Os;   // each output wave reads back only its own rows
#pragma unroll
            for (int st = 0; st < NSTRIP; ++st) {
                const bf16x8 DB0 = sm.Dx[cc & 1][st][0][lane];
                f32x4 O4[2];
#pragma unroll
                for (int ii = 0; ii < 2; ++ii) O4[ii] = mfma32(ap0[ii], DB0, grq[ii] * QS[st][ii]);
                if (half) {
                    const bf16x8 DB1 = sm.Dx[cc & 1][st][1][lane];
#pragma unroll
                    for (int ii = 0; ii < 2; ++ii) O4[ii] = mfma32(ap1[ii], DB1, O4[ii]);
                }
                // lane pairs (n, n ^ 1) trade two of their four rows, so each
                // lane writes two rows of two adjacent columns as 4-byte words
#pragma unroll
                for (int ii = 0; ii < 2; ++ii) {
                    const uint32_t lo = (uint32_t)(uint16_t)bfbits(q_scale * O4[ii][0]) |
                                        ((uint32_t)(uint16_t)bfbits(q_scale * O4[ii][1]) << 16);
                    const uint32_t hi = (uint32_t)(uint16_t)bfbits(q_scale * O4[ii][2]) |
                                        ((uint32_t)(uint16_t)bfbits(q_scale * O4[ii][3]) << 16);
                    const bool odd = (n & 1) != 0;
                    const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)(odd ? lo : hi), 0xB1, 0xF, 0xF, false);
                    const uint32_t pa = odd ? recv : lo;   // column n & ~1
                    const uint32_t pb = odd ? hi : recv;   // column n | 1
                    const int r0 = 16 * (2 * half + ii) + 4 * g + (odd ? 2 : 0);
                    const int c0 = SW * st + (n & ~1);
                    *reinterpret_cast<uint32_t*>(&Ot[r0][c0]) = (pa & 0xffffu) | (pb << 16);
                    *reinterpret_cast<uint32_t*>(&Ot[r0 + 1][c0]) = (pa >> 16) | (pb & 0xffff0000u);
                }
            }
            // ---- the wave's 32 rows x 64 bytes back from LDS (its own writes,
            //      so no barrier) and to HBM in 16-byte pieces
            const int t0 = cc * C;
            const int L = min(C, Tb - t0);
            bf16_t* oc = obase + (size_t)t0 * rowv;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int r = 32 * half + (lane >> 2) + 16 * u;
                const int c8 = 8 * (lane & 3);
                if (r < L)
                    *reinterpret_cast<uint4*>(oc + r * rowv + c8) = *reinterpret_cast<const uint4*>(&Ot[r][c8]);
            }
        }
        __syncthreads();
    }
}

}  // namespace mfma_prefill

bool prefill_mfma_supported(const PrefillArgs& a) {
    return a.bf16 && a.D == 128 && a.C == 64;
}

namespace {

using namespace mfma_prefill;

// A call runs in pieces of at most kPieceChunks chunks (or as many as the
// workspace holds), each a prep launch then a scan launch on the caller's
// stream; the records of one piece are reused by the next, and the state
// passes from piece to piece through hT (or a slot after the records when
// the caller wants no final state).  Every chunk computes the same whatever
// the pieces, so the results are bitwise those of one piece.
constexpr int kPieceChunks = 256;

size_t records_bytes(int B, int Hv, int chunks) {
    return (size_t)B * Hv * (size_t)chunks * WS_REC;
}
size_t carry_bytes(int B, int Hv) { return (size_t)B * Hv * D * D * sizeof(float); }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
// workspace for pieces of `piece` chunks out of NTc
size_t workspace_for(int B, int Hv, int NTc, int piece) {
    const int pc = piece < NTc ? piece : NTc;
    return pc < NTc ? align256(records_bytes(B, Hv, pc)) + carry_bytes(B, Hv) : records_bytes(B, Hv, pc);
}

hipError_t launch_prep(const PrefillArgs& a, int NRc, unsigned char* ws, int c_first,
                       int n_chunks, hipStream_t stream) {
    if (a.A_log) return launch_prep_raw(a, NRc, ws, c_first, n_chunks, stream);
    hipLaunchKernelGGL(chunk_prep_kernel, dim3(a.B * a.Hk * n_chunks), dim3(NT), 0, stream,
                       static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k), a.log_g,
                       a.beta, nullptr, nullptr, ws, a.T, NRc, a.Hk, a.Hv, a.l2norm, a.cu,
                       a.total, c_first, n_chunks);
    return hipGetLastError();
}

hipError_t launch_scan(const PrefillArgs& a, int NRc, const unsigned char* ws, const float* h0,
                       float* hT, int c_first, int n_chunks, hipStream_t stream) {
    const int scan_blocks = a.B * a.Hv * (D / BVS);
    const int remap = ((a.B * a.Hk) % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL(chunk_scan_kernel, dim3(scan_blocks), dim3(SNT), 0, stream,
                       static_cast<const bf16_t*>(a.q), static_cast<const bf16_t*>(a.k),
                       static_cast<const bf16_t*>(a.v), ws, h0, hT,
                       static_cast<bf16_t*>(a.o), a.T, NRc, a.Hk, a.Hv, a.q_scale, remap,
                       a.ckpt, a.ckpt_every, a.nck, a.cu, a.total, c_first, n_chunks);
    return hipGetLastError();
}

}  // namespace

size_t prefill_mfma_workspace_bytes(int B, int T, int Hk, int Hv) {
    (void)Hk;
    return workspace_for(B, Hv, (T + C - 1) / C, kPieceChunks);
}

size_t prefill_mfma_min_workspace_bytes(int B, int T, int Hk, int Hv) {
    (void)Hk;
    return workspace_for(B, Hv, (T + C - 1) / C, 1);
}

// Piece by piece: the prep of the piece's chunks, then the serial pass over
// them, on the caller's stream.  a.ws_bytes (at least the minimum above)
// sets the piece length.
hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t stream) {
    const int NTc = (a.T + C - 1) / C;
    if (a.B * a.Hk * NTc == 0) return hipSuccess;
    unsigned char* ws = static_cast<unsigned char*>(a.ws);
    int piece = NTc;
    if (records_bytes(a.B, a.Hv, NTc) > a.ws_bytes) {
        const size_t per = records_bytes(a.B, a.Hv, 1);
        const size_t room = a.ws_bytes > carry_bytes(a.B, a.Hv) ? a.ws_bytes - carry_bytes(a.B, a.Hv) : 0;
        size_t p = room / per < (size_t)NTc ? room / per : (size_t)NTc;
        while (p > 0 && align256(records_bytes(a.B, a.Hv, (int)p)) > room) --p;
        if (p < 1) return hipErrorInvalidValue;   // below the minimum the caller checked
        piece = (int)p;
    }
    float* carry = a.hT ? a.hT : reinterpret_cast<float*>(ws + align256(records_bytes(a.B, a.Hv, piece)));
    const float* h_in = a.h0;
    for (int c0 = 0; c0 < NTc; c0 += piece) {
        const int n = NTc - c0 < piece ? NTc - c0 : piece;
        float* h_out = (c0 + n >= NTc) ? a.hT : carry;
        hipError_t err = launch_prep(a, piece, ws, c0, n, stream);
        if (err != hipSuccess) return err;
        err = launch_scan(a, piece, ws, h_in, h_out, c0, n, stream);
        if (err != hipSuccess) return err;
        h_in = carry;
    }
    return hipSuccess;
}

}  // namespace gdn

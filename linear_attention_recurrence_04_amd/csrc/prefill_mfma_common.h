// prefill_mfma_common.h -- definitions shared by the two translation units
// of the bf16 MFMA chunked prefill (prefill_mfma.hip: the prep kernel with
// given gates, the scan kernel and the launcher; prefill_prep_raw.hip: the
// prep kernel with raw gate projections): vector types, the workspace record
// layout, operand-order helpers and the prep kernel's shared-memory layout.
// The method itself is described at the top of prefill_mfma.hip.
#pragma once

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
constexpr int SK = D + 16;  // row stride (elements) of the staged k / q rows: 288 bytes, so the
                            // Gram operand reads (16 rows at a time) hit distinct LDS banks
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
            // per head, padded by 32 bytes so that the heads' blocks start on
            // different LDS banks (lanes of different heads read them together)
            struct { float v[4][16][16]; float pad[8]; } AfT[GH];         // A diagonal blocks (fp32), transposed: [block][s][r]
            struct { uint16_t v[6][16][16]; uint16_t pad[16]; } Ab[GH];   // A blocks below the diagonal (bf16)
            struct { uint16_t v[10][16][16]; uint16_t pad[16]; } Tl[GH];  // T blocks on and below the diagonal (bf16)
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
                for (int t = 0; t < 4; ++t) sm.tri.AfT[hh].v[a][4 * g + t][n] = val[t];
            } else {
                *reinterpret_cast<s16x4*>(&sm.tri.Ab[hh].v[ab_idx(a, bb)][n][4 * g]) = pack4(val);
            }
        }
    }
}

// The prep kernel reading raw gate projections (prefill_prep_raw.hip): its
// own translation unit, because with both prep kernels in one unit the
// register allocator spilled in both.
hipError_t launch_prep_raw(const PrefillArgs& a, int NRc, unsigned char* ws, int c_first,
                          int n_chunks, hipStream_t stream);

}  // namespace mfma_prefill
}  // namespace gdn

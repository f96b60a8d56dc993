// gdn_api.cpp -- the C ABI (include/gdn.h): argument checks and kernel dispatch.
//
// Every check runs on the host before anything is enqueued, so a rejected call
// leaves the stream untouched.  The checks turn the forward-time assertions of
// "Qwen3.5 Gated Delta Net NKI Kernel for AWS Neuron" ("Correctness Contract":
// head dims equal and supported) into status codes.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "gdn.h"
#include "gdn_launch.h"

namespace {

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, size_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + bytes};
}

bool overlaps(Range a, Range b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared checks of the problem description.  `decode` selects the decode rules
// (T == 1, chunk ignored); `multi` the multi-token decode rules (any T >= 0,
// chunk ignored).
gdn_status check_problem(const gdn_problem* p, bool decode, bool multi = false) {
    if (!p) return GDN_ERR_NULL_POINTER;
    if (p->B < 0 || p->T < 0 || p->Hk < 1 || p->Hv < 1) return GDN_ERR_BAD_SHAPE;
    if (p->Hv % p->Hk != 0) return GDN_ERR_BAD_SHAPE;
    if (decode && !multi && p->T != 1) return GDN_ERR_BAD_SHAPE;
    if (p->dk != p->dv) return GDN_ERR_UNSUPPORTED;
    if (p->dk != 64 && p->dk != 128) return GDN_ERR_UNSUPPORTED;
    if (p->dtype != GDN_DTYPE_F32 && p->dtype != GDN_DTYPE_BF16) return GDN_ERR_UNSUPPORTED;
    if (p->qk_l2norm != 0 && p->qk_l2norm != 1) return GDN_ERR_UNSUPPORTED;
    if (!decode && p->chunk != 0 && p->chunk != 16 && p->chunk != 32 && p->chunk != 64)
        return GDN_ERR_UNSUPPORTED;
    // grid limits: one workgroup row per (b, h); sizes must fit the index math
    const long long bh = (long long)p->B * p->Hv;
    if (bh > 0x7fffffffLL) return GDN_ERR_BAD_SHAPE;
    const long long elems = (long long)p->B * p->T * p->Hv * p->dv;
    if (elems > (1LL << 46)) return GDN_ERR_BAD_SHAPE;
    return GDN_OK;
}

size_t dsize(const gdn_problem* p) { return p->dtype == GDN_DTYPE_BF16 ? 2 : 4; }

gdn::PrefillArgs prefill_args(const gdn_problem* p) {
    gdn::PrefillArgs a = {};
    a.B = p->B; a.T = p->T; a.Hk = p->Hk; a.Hv = p->Hv; a.D = p->dk;
    a.C = p->chunk ? p->chunk : 64;
    a.bf16 = p->dtype == GDN_DTYPE_BF16;
    a.l2norm = p->qk_l2norm;
    a.q_scale = p->q_scale;
    return a;
}

// GDN_FORCE_GENERIC=1 in the environment routes every prefill to the fp32
// kernel (A/B comparisons between the two kernels on the same problem).
bool force_generic() {
    const char* e = getenv("GDN_FORCE_GENERIC");
    return e && e[0] == '1';
}

bool use_mfma(const gdn::PrefillArgs& a) { return !force_generic() && gdn::prefill_mfma_supported(a); }

size_t mfma_workspace_bytes(const gdn::PrefillArgs& a) {
    return gdn::prefill_mfma_workspace_bytes(a.B, a.T, a.Hk, a.Hv);
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_string(gdn_status s) {
    switch (s) {
        case GDN_OK: return "ok";
        case GDN_ERR_NULL_POINTER: return "a required pointer is NULL";
        case GDN_ERR_BAD_SHAPE: return "invalid sizes (negative, Hv not a multiple of Hk, decode T != 1, or too large)";
        case GDN_ERR_UNSUPPORTED: return "unsupported head dim, chunk, dtype or flag (dk == dv in {64,128}; chunk in {0,16,32,64})";
        case GDN_ERR_MISALIGNED: return "a pointer is not 16-byte aligned";
        case GDN_ERR_WORKSPACE: return "workspace missing or too small";
        case GDN_ERR_HIP: return "the HIP runtime rejected a kernel launch";
        case GDN_ERR_ALIAS: return "an output buffer overlaps an input";
        default: break;
    }
    return "unknown gdn_status";
}

const char* gdn_chunk_prefill_variant(const gdn_problem* p) {
    if (check_problem(p, false) != GDN_OK) return "invalid";
    return use_mfma(prefill_args(p)) ? "mfma_bf16" : "generic_f32";
}

size_t gdn_chunk_prefill_workspace_bytes(const gdn_problem* p) {
    if (check_problem(p, false) != GDN_OK) return 0;
    const gdn::PrefillArgs a = prefill_args(p);
    if (use_mfma(a)) return mfma_workspace_bytes(a);
    return 0;  // the fp32 kernel keeps every intermediate on chip
}

}  // extern "C"

namespace {

// gdn_chunk_prefill with optional checkpoints (h_ckpt == NULL and
// ckpt_every == 0 for none; the caller has checked ckpt_every) and optional
// raw gates (A_log, dt_bias non-null: log_g, beta hold the projections a, b).
// Packed variable-length batches pass cu (device [B + 1]) and the length
// `total` of the token axis; otherwise cu is NULL and total = B * T.
// any_piece: accept any workspace that holds one chunk's records and the
// carried state (the call then runs in pieces that fit), instead of the
// size gdn_chunk_prefill_workspace_bytes documents.
gdn_status prefill_impl(const gdn_problem* p, const void* q, const void* k, const void* v,
                        const float* log_g, const float* beta, const float* A_log,
                        const float* dt_bias, const float* h0, float* hT, void* o,
                        float* h_ckpt, int ckpt_every, void* workspace,
                        size_t workspace_bytes, void* hip_stream,
                        const int32_t* cu = nullptr, long long total = -1, bool onchip = false,
                        bool any_piece = false) {
    const size_t es = dsize(p);
    if (total < 0) total = (long long)p->B * p->T;
    const size_t BT = (size_t)total;
    const size_t qk_bytes = BT * p->Hk * p->dk * es;
    const size_t v_bytes = BT * p->Hv * p->dv * es;
    const size_t g_bytes = BT * p->Hv * sizeof(float);
    const size_t s_bytes = (size_t)p->B * p->Hv * p->dk * p->dv * sizeof(float);
    const int nck = ckpt_every > 0 ? (p->T + ckpt_every - 1) / ckpt_every : 0;
    const size_t ck_bytes = s_bytes * (size_t)nck;

    if (BT > 0 && (!q || !k || !v || !log_g || !beta || !o)) return GDN_ERR_NULL_POINTER;
    if (ck_bytes > 0 && !h_ckpt) return GDN_ERR_NULL_POINTER;
    const void* ptrs[] = {q, k, v, log_g, beta, h0, hT, o, workspace, h_ckpt, A_log, dt_bias, cu};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return GDN_ERR_MISALIGNED;

    size_t need_ws = onchip ? 0 : gdn_chunk_prefill_workspace_bytes(p);
    if (any_piece && need_ws > 0) need_ws = gdn::prefill_mfma_min_workspace_bytes(p->B, p->T, p->Hk, p->Hv);
    if (need_ws > 0 && (!workspace || workspace_bytes < need_ws)) return GDN_ERR_WORKSPACE;

    // outputs against inputs: hT may be exactly h0, nothing else may overlap
    const size_t par_bytes = (size_t)p->Hv * sizeof(float);
    const Range ins[] = {range_of(q, BT ? qk_bytes : 0), range_of(k, BT ? qk_bytes : 0),
                         range_of(v, BT ? v_bytes : 0), range_of(log_g, BT ? g_bytes : 0),
                         range_of(beta, BT ? g_bytes : 0), range_of(A_log, A_log ? par_bytes : 0),
                         range_of(dt_bias, dt_bias ? par_bytes : 0),
                         range_of(cu, cu ? ((size_t)p->B + 1) * sizeof(int32_t) : 0)};
    const Range r_o = range_of(o, BT ? v_bytes : 0);
    const Range r_hT = range_of(hT, hT ? s_bytes : 0);
    const Range r_h0 = range_of(h0, h0 ? s_bytes : 0);
    const Range r_ws = range_of(workspace, workspace ? need_ws : 0);
    const Range r_ck = range_of(h_ckpt, h_ckpt ? ck_bytes : 0);
    for (const Range& in : ins) {
        if (overlaps(in, r_o) || overlaps(in, r_hT) || overlaps(in, r_ws) || overlaps(in, r_ck))
            return GDN_ERR_ALIAS;
    }
    if (overlaps(r_o, r_hT) || overlaps(r_o, r_h0) || overlaps(r_o, r_ws)) return GDN_ERR_ALIAS;
    if (overlaps(r_hT, r_ws) || overlaps(r_h0, r_ws)) return GDN_ERR_ALIAS;
    if (hT && h0 && hT != h0 && overlaps(r_hT, r_h0)) return GDN_ERR_ALIAS;
    if (overlaps(r_ck, r_o) || overlaps(r_ck, r_hT) || overlaps(r_ck, r_h0) || overlaps(r_ck, r_ws))
        return GDN_ERR_ALIAS;

    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (p->B == 0 || p->Hv == 0) return GDN_OK;
    hipError_t err;
    if (p->T == 0 || BT == 0) {   // every sequence is empty
        err = gdn::launch_state_copy(h0, hT, s_bytes / sizeof(float), stream);
        return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
    }
    gdn::PrefillArgs a = prefill_args(p);
    a.cu = cu;
    a.total = total;
    a.q = q; a.k = k; a.v = v; a.log_g = log_g; a.beta = beta;
    a.A_log = A_log; a.dt_bias = dt_bias;
    a.h0 = h0; a.hT = hT; a.o = o; a.ws = workspace; a.ws_bytes = workspace_bytes;
    a.ckpt = nck > 0 ? h_ckpt : nullptr;
    a.ckpt_every = nck > 0 ? ckpt_every : 0;
    a.nck = nck;
    if (!use_mfma(a)) err = gdn::launch_prefill_generic(a, stream);
    else err = onchip ? gdn::launch_prefill_fused(a, stream) : gdn::launch_prefill_mfma(a, stream);
    return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // namespace

int gdn::prefill_checked(const void* problem, const void* q, const void* k, const void* v,
                         const float* log_g, const float* beta, const float* h0, float* hT,
                         void* o, void* workspace, size_t workspace_bytes, void* hip_stream) {
    const gdn_problem* p = static_cast<const gdn_problem*>(problem);
    const gdn_status st = check_problem(p, false);
    if (st != GDN_OK) return st;
    return prefill_impl(p, q, k, v, log_g, beta, nullptr, nullptr, h0, hT, o, nullptr, 0,
                        workspace, workspace_bytes, hip_stream, nullptr, -1, false, true);
}

extern "C" {

gdn_status gdn_chunk_prefill(const gdn_problem* p, const void* q, const void* k, const void* v,
                             const float* log_g, const float* beta, const float* h0, float* hT,
                             void* o, void* workspace, size_t workspace_bytes, void* hip_stream) {
    const gdn_status st = check_problem(p, false);
    if (st != GDN_OK) return st;
    return prefill_impl(p, q, k, v, log_g, beta, nullptr, nullptr, h0, hT, o, nullptr, 0,
                        workspace, workspace_bytes, hip_stream);
}

gdn_status gdn_chunk_prefill_ckpt(const gdn_problem* p, const void* q, const void* k,
                                  const void* v, const float* log_g, const float* beta,
                                  const float* h0, float* hT, void* o, float* h_ckpt,
                                  int32_t ckpt_every, void* workspace, size_t workspace_bytes,
                                  void* hip_stream) {
    const gdn_status st = check_problem(p, false);
    if (st != GDN_OK) return st;
    const int C = p->chunk ? p->chunk : 64;
    if (ckpt_every <= 0 || ckpt_every % C != 0) return GDN_ERR_BAD_SHAPE;
    return prefill_impl(p, q, k, v, log_g, beta, nullptr, nullptr, h0, hT, o, h_ckpt,
                        ckpt_every, workspace, workspace_bytes, hip_stream);
}

gdn_status gdn_chunk_prefill_gated(const gdn_problem* p, const void* q, const void* k,
                                   const void* v, const float* a, const float* b,
                                   const float* A_log, const float* dt_bias, const float* h0,
                                   float* hT, void* o, float* h_ckpt, int32_t ckpt_every,
                                   void* workspace, size_t workspace_bytes, void* hip_stream) {
    const gdn_status st = check_problem(p, false);
    if (st != GDN_OK) return st;
    if (!A_log || !dt_bias) return GDN_ERR_NULL_POINTER;
    const int C = p->chunk ? p->chunk : 64;
    if (ckpt_every < 0 || ckpt_every % C != 0) return GDN_ERR_BAD_SHAPE;
    if (ckpt_every == 0 && h_ckpt) return GDN_ERR_BAD_SHAPE;
    return prefill_impl(p, q, k, v, a, b, A_log, dt_bias, h0, hT, o, h_ckpt, ckpt_every,
                        workspace, workspace_bytes, hip_stream);
}

gdn_status gdn_chunk_prefill_varlen(const gdn_problem* p, const int32_t* cu_seqlens,
                                    int64_t total_tokens, const void* q, const void* k,
                                    const void* v, const float* log_g, const float* beta,
                                    const float* h0, float* hT, void* o, void* workspace,
                                    size_t workspace_bytes, void* hip_stream) {
    const gdn_status st = check_problem(p, false);
    if (st != GDN_OK) return st;
    if (total_tokens < 0) return GDN_ERR_BAD_SHAPE;
    const long long elems = (long long)total_tokens * p->Hv * p->dv;
    if (total_tokens > 0x7fffffffLL || elems > (1LL << 46)) return GDN_ERR_BAD_SHAPE;
    if (p->B > 0 && !cu_seqlens) return GDN_ERR_NULL_POINTER;
    return prefill_impl(p, q, k, v, log_g, beta, nullptr, nullptr, h0, hT, o, nullptr, 0,
                        workspace, workspace_bytes, hip_stream, cu_seqlens, total_tokens);
}

gdn_status gdn_chunk_prefill_onchip(const gdn_problem* p, const void* q, const void* k,
                                    const void* v, const float* log_g, const float* beta,
                                    const float* h0, float* hT, void* o, float* h_ckpt,
                                    int32_t ckpt_every, void* hip_stream) {
    const gdn_status st = check_problem(p, false);
    if (st != GDN_OK) return st;
    const int C = p->chunk ? p->chunk : 64;
    if (ckpt_every < 0 || ckpt_every % C != 0) return GDN_ERR_BAD_SHAPE;
    if (ckpt_every == 0 && h_ckpt) return GDN_ERR_BAD_SHAPE;
    return prefill_impl(p, q, k, v, log_g, beta, nullptr, nullptr, h0, hT, o, h_ckpt, ckpt_every,
                        nullptr, 0, hip_stream, nullptr, -1, true);
}

}  // extern "C"

namespace {

// T tokens per sequence (1 for gdn_decode_step); `states` optional.
gdn_status decode_impl(const gdn_problem* p, const void* q, const void* k, const void* v,
                       const float* log_g, const float* beta, const float* A_log,
                       const float* dt_bias, float* state, void* o, float* states,
                       void* hip_stream) {
    const size_t BT = (size_t)p->B * p->T;
    if (p->B > 0 && !state) return GDN_ERR_NULL_POINTER;
    if (BT > 0 && (!q || !k || !v || !log_g || !beta || !o)) return GDN_ERR_NULL_POINTER;
    const void* ptrs[] = {q, k, v, log_g, beta, state, o, A_log, dt_bias, states};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return GDN_ERR_MISALIGNED;
    const size_t es = dsize(p);
    const size_t par_bytes = (size_t)p->Hv * sizeof(float);
    const size_t s_bytes = (size_t)p->B * p->Hv * p->dk * p->dv * sizeof(float);
    const Range r_state = range_of(state, s_bytes);
    const Range r_o = range_of(o, BT * p->Hv * p->dv * es);
    const Range r_sts = range_of(states, states ? s_bytes * p->T : 0);
    const Range ins[] = {range_of(q, BT * p->Hk * p->dk * es), range_of(k, BT * p->Hk * p->dk * es),
                         range_of(v, BT * p->Hv * p->dv * es), range_of(log_g, BT * p->Hv * 4),
                         range_of(beta, BT * p->Hv * 4), range_of(A_log, A_log ? par_bytes : 0),
                         range_of(dt_bias, dt_bias ? par_bytes : 0)};
    for (const Range& in : ins)
        if (overlaps(in, r_state) || overlaps(in, r_o) || overlaps(in, r_sts)) return GDN_ERR_ALIAS;
    if (overlaps(r_state, r_o) || overlaps(r_sts, r_state) || overlaps(r_sts, r_o))
        return GDN_ERR_ALIAS;
    if (BT == 0) return GDN_OK;

    gdn::DecodeArgs a;
    a.B = p->B; a.T = p->T; a.Hk = p->Hk; a.Hv = p->Hv; a.D = p->dk;
    a.bf16 = p->dtype == GDN_DTYPE_BF16;
    a.l2norm = p->qk_l2norm;
    a.q_scale = p->q_scale;
    a.q = q; a.k = k; a.v = v; a.log_g = log_g; a.beta = beta;
    a.A_log = A_log; a.dt_bias = dt_bias;
    a.state = state; a.o = o; a.states = states;
    const hipError_t err = gdn::launch_decode_step(a, static_cast<hipStream_t>(hip_stream));
    return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // namespace

extern "C" {

gdn_status gdn_decode_step(const gdn_problem* p, const void* q, const void* k, const void* v,
                           const float* log_g, const float* beta, float* state, void* o,
                           void* hip_stream) {
    const gdn_status st = check_problem(p, true);
    if (st != GDN_OK) return st;
    return decode_impl(p, q, k, v, log_g, beta, nullptr, nullptr, state, o, nullptr, hip_stream);
}

gdn_status gdn_decode_multi(const gdn_problem* p, const void* q, const void* k, const void* v,
                            const float* log_g, const float* beta, const float* A_log,
                            const float* dt_bias, float* state, void* o, float* states,
                            void* hip_stream) {
    const gdn_status st = check_problem(p, true, true);
    if (st != GDN_OK) return st;
    if ((A_log == nullptr) != (dt_bias == nullptr)) return GDN_ERR_NULL_POINTER;
    return decode_impl(p, q, k, v, log_g, beta, A_log, dt_bias, state, o, states, hip_stream);
}

gdn_status gdn_decode_step_gated(const gdn_problem* p, const void* q, const void* k,
                                 const void* v, const float* a, const float* b,
                                 const float* A_log, const float* dt_bias, float* state,
                                 void* o, void* hip_stream) {
    const gdn_status st = check_problem(p, true);
    if (st != GDN_OK) return st;
    if (!A_log || !dt_bias) return GDN_ERR_NULL_POINTER;
    return decode_impl(p, q, k, v, a, b, A_log, dt_bias, state, o, nullptr, hip_stream);
}

}  // extern "C"

extern "C" {

gdn_status gdn_causal_conv1d(int32_t B, int32_t T, int32_t C, int32_t K, int32_t dtype,
                             const void* x, const float* weight, const float* bias,
                             const void* state_in, void* state_out, void* y, int32_t silu,
                             void* hip_stream) {
    if (dtype != GDN_DTYPE_F32 && dtype != GDN_DTYPE_BF16) return GDN_ERR_UNSUPPORTED;
    if (K < 1 || K > 4) return GDN_ERR_UNSUPPORTED;
    if (B < 0 || T < 0 || C <= 0) return GDN_ERR_BAD_SHAPE;
    const size_t es = dtype == GDN_DTYPE_BF16 ? 2 : 4;
    if ((C * es) % 16 != 0) return GDN_ERR_UNSUPPORTED;
    if ((T + gdn::kConvTileTokens - 1) / gdn::kConvTileTokens > 65535 || B > 65535)
        return GDN_ERR_BAD_SHAPE;   // grid limits: token tiles (y), sequences (z)
    const size_t xy_bytes = (size_t)B * T * C * es;
    const size_t st_bytes = (size_t)B * (K - 1) * C * es;
    if (!weight) return GDN_ERR_NULL_POINTER;
    if (xy_bytes > 0 && (!x || !y)) return GDN_ERR_NULL_POINTER;
    const void* ptrs[] = {x, weight, bias, state_in, state_out, y};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return GDN_ERR_MISALIGNED;
    const Range r_x = range_of(x, xy_bytes), r_y = range_of(y, xy_bytes);
    const Range r_w = range_of(weight, (size_t)C * K * 4), r_b = range_of(bias, bias ? (size_t)C * 4 : 0);
    const Range r_si = range_of(state_in, state_in ? st_bytes : 0);
    const Range r_so = range_of(state_out, state_out ? st_bytes : 0);
    const Range ins[] = {r_x, r_w, r_b, r_si};
    for (const Range& in : ins)
        if (overlaps(in, r_y)) return GDN_ERR_ALIAS;
    if (overlaps(r_so, r_y) || overlaps(r_so, r_x) || overlaps(r_so, r_w) || overlaps(r_so, r_b))
        return GDN_ERR_ALIAS;
    if (state_in && state_out && state_in != state_out && overlaps(r_si, r_so)) return GDN_ERR_ALIAS;
    gdn::ConvArgs a{B, T, C, K, dtype == GDN_DTYPE_BF16, x, weight, bias, state_in, state_out, y,
                    silu ? 1 : 0};
    const hipError_t err = gdn::launch_causal_conv1d(a, static_cast<hipStream_t>(hip_stream));
    return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

gdn_status gdn_gated_rmsnorm(int64_t rows, int32_t D, int32_t dtype, const void* x, const void* z,
                             const float* weight, float eps, void* y, void* hip_stream) {
    if (dtype != GDN_DTYPE_F32 && dtype != GDN_DTYPE_BF16) return GDN_ERR_UNSUPPORTED;
    if (rows < 0 || D <= 0 || !(eps >= 0.f)) return GDN_ERR_BAD_SHAPE;
    if (!gdn::conv_norm_dim_supported(D, dtype == GDN_DTYPE_BF16)) return GDN_ERR_UNSUPPORTED;
    if (rows >= ((int64_t)1 << 32)) return GDN_ERR_BAD_SHAPE;   // grid limit (blocks of 256 lanes)
    if (!weight) return GDN_ERR_NULL_POINTER;
    const size_t es = dtype == GDN_DTYPE_BF16 ? 2 : 4;
    const size_t bytes = (size_t)rows * D * es;
    if (bytes > 0 && (!x || !y)) return GDN_ERR_NULL_POINTER;
    const void* ptrs[] = {x, z, weight, y};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return GDN_ERR_MISALIGNED;
    const Range r_x = range_of(x, bytes), r_y = range_of(y, bytes);
    const Range r_z = range_of(z, z ? bytes : 0), r_w = range_of(weight, (size_t)D * 4);
    if (overlaps(r_z, r_y) || overlaps(r_w, r_y)) return GDN_ERR_ALIAS;
    if (x != y && overlaps(r_x, r_y)) return GDN_ERR_ALIAS;
    gdn::NormArgs a{rows, D, dtype == GDN_DTYPE_BF16, x, z, weight, eps, y};
    const hipError_t err = gdn::launch_gated_rmsnorm(a, static_cast<hipStream_t>(hip_stream));
    return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // extern "C"

// gdn_launch.h -- internal launch interface between the C ABI and the kernels.
// Arguments here are already validated by the ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace gdn {

struct DecodeArgs {
    int B, T, Hk, Hv, D;   // T tokens per sequence (1 for a plain decode step)
    bool bf16;
    int l2norm;
    float q_scale;
    const void *q, *k, *v;
    const float *log_g, *beta;   // or the raw projections a, b when A_log is set
    const float *A_log, *dt_bias;  // [Hv] gate parameters, or null
    float* state;
    void* o;
    float* states;   // [B, T, Hv, D, D] state after every token, or null
};

struct PrefillArgs {
    int B, T, Hk, Hv, D, C;
    bool bf16;
    int l2norm;
    float q_scale;
    const void *q, *k, *v;
    const float *log_g, *beta;   // or the raw projections a, b when A_log is set
    const float *A_log, *dt_bias;  // [Hv] gate parameters, or null
    const float* h0;   // may be null (zeros)
    float* hT;         // may be null; may equal h0
    void* o;
    void* ws;          // workspace (validated size)
    size_t ws_bytes;
    float* ckpt;       // [B, nck, Hv, D, D] state checkpoints, or null
    int ckpt_every;    // tokens between checkpoints (a multiple of C), 0 if none
    int nck;           // ceil(T / ckpt_every), 0 if none
    const int* cu;     // device [B + 1] sequence starts on a packed token axis, or null
    long long total;   // tokens on the token axis (B * T without cu)
};

hipError_t launch_decode_step(const DecodeArgs& a, hipStream_t stream);

// Portable path: any supported (D, C, dtype); fp32 arithmetic throughout.
hipError_t launch_prefill_generic(const PrefillArgs& a, hipStream_t stream);

// bf16 MFMA path: bf16 inputs, head dim 128, chunk 64.  Two kernels (a
// parallel per-chunk prep writing T, P and gates to the workspace, then the
// serial scan over chunks), launched for pieces of at most 256 chunks (more
// if a.ws_bytes holds them) one after the other.
bool prefill_mfma_supported(const PrefillArgs& a);
size_t prefill_mfma_workspace_bytes(int B, int T, int Hk, int Hv);
// the least workspace the bf16 MFMA prefill runs with (pieces of one chunk)
size_t prefill_mfma_min_workspace_bytes(int B, int T, int Hk, int Hv);
hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t stream);

// The same bf16 MFMA path (same supported shapes) in one kernel: every
// per-chunk intermediate stays on chip (no workspace).
hipError_t launch_prefill_fused(const PrefillArgs& a, hipStream_t stream);

// hT = h0 (or zeros) without touching anything else (T == 0).
hipError_t launch_state_copy(const float* h0, float* hT, size_t n, hipStream_t stream);

// Causal depthwise conv1d over [B, T, C] with the last K-1 inputs carried
// (C a multiple of 16 bytes of the dtype, 1 <= K <= 4).  Grid: x channel
// groups, y tiles of kConvTileTokens tokens (at most 65535), z sequences.
constexpr int kConvTileTokens = 64;
struct ConvArgs {
    int B, T, C, K;
    bool bf16;
    const void* x;          // [B, T, C]
    const float* w;         // [C, K]
    const float* bias;      // [C] or null
    const void* state_in;   // [B, K-1, C] or null (zeros)
    void* state_out;        // [B, K-1, C] or null; may be state_in
    void* y;                // [B, T, C]
    int silu;
};
hipError_t launch_causal_conv1d(const ConvArgs& a, hipStream_t stream);

// y = x / sqrt(mean(x^2) + eps) * w * silu(z) per row of D values.
struct NormArgs {
    long long rows;
    int D;
    bool bf16;
    const void* x;          // [rows, D]
    const void* z;          // [rows, D] or null (no gate)
    const float* w;         // [D]
    float eps;
    void* y;                // [rows, D]; may be x
};
bool conv_norm_dim_supported(int D, bool bf16);
hipError_t launch_gated_rmsnorm(const NormArgs& a, hipStream_t stream);

// gdn_chunk_prefill's checks and dispatch with the workspace given by the
// caller of this function (gdn_api.cpp), which may be as small as one
// chunk's records and the carried state (the call then runs in pieces that
// fit); returns a gdn_status value.
int prefill_checked(const void* problem, const void* q, const void* k, const void* v,
                    const float* log_g, const float* beta, const float* h0, float* hT, void* o,
                    void* workspace, size_t workspace_bytes, void* hip_stream);

}  // namespace gdn

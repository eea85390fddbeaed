// Internal interface between the C-ABI layer (atma_api.cpp) and the kernel files.
// Every launcher assumes its arguments were validated by the ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace atma {

struct GdnFwdArgs {
    const void *q, *k, *v;
    const float *alpha, *beta, *init_state;
    void* o;
    float* final_state;
    int B, T, H, Dk, Dv;
    bool bf16_io;
    void* workspace;
    // packed batch (bf16 path): B sequences with row offsets cu[0..B] (device), T = the longest
    const int* cu = nullptr;
    int total = 0;
};
size_t gdn_fwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, bool bf16_io);
hipError_t launch_gdn_fwd(const GdnFwdArgs& a, hipStream_t stream);
// bf16-input fast path (fp16-staged operands), used by launch_gdn_fwd
size_t gdn_bf16_workspace_bytes(int B, int T, int H, int Dk, int Dv);
hipError_t launch_gdn_bf16(const GdnFwdArgs& a, hipStream_t stream);

// Backward of the chunked memory prefill (fixed-length batches), fp32 arithmetic.
struct GdnBwdArgs {
    const void *q, *k, *v, *dO;
    const float *alpha, *beta, *init_state, *dS_final;
    void *dq, *dk, *dv;
    float *dalpha, *dbeta, *d_init;
    int B, T, H, Dk, Dv;
    bool bf16_io;
    void* workspace;
};
size_t gdn_bwd_workspace_bytes(int B, int T, int H, int Dk, int Dv);
hipError_t launch_gdn_bwd(const GdnBwdArgs& a, hipStream_t stream);

struct GdnDecodeArgs {
    const void *q, *k, *v;
    const float *alpha, *beta;
    float* state;
    void* o;
    int B, H, Dk, Dv;
    bool bf16_io;
};
hipError_t launch_gdn_decode(const GdnDecodeArgs& a, hipStream_t stream);

struct PolarParamsDev {
    const float *temp_raw, *null_slope_raw, *null_bias, *mag_beta, *v_null;
    float eps;
};

struct PolarFwdArgs {
    const void *q, *k, *v;
    PolarParamsDev p;
    void* o;
    float *mu_out, *meff_out;
    int B, T, Hq, Hkv, D;
    // packed batch: B sequences with row offsets cu[0..B] (device), T = the longest, total rows
    const int* cu = nullptr;
    int total = 0;
    // plain causal softmax attention (the NoPE / RoPE control core): no temperature, no null,
    // output sum_j w_j v_j; p, mu_out and meff_out unused
    bool softmax = false;
    // training outputs (Polar only, NULL when not wanted): per row {lse2, real mass, squared
    // mass, normaliser} [B, Hq, T, 4] and the direction c [B, T, Hq, D], both fp32
    float* stats = nullptr;
    float* dir = nullptr;
};
hipError_t launch_polar_fwd(const PolarFwdArgs& a, hipStream_t stream);

// Backward of causal Polar attention (fixed-length batches), from the forward's training outputs.
struct PolarBwdArgs {
    const void *q, *k, *v, *dO;
    PolarParamsDev p;
    const float *mu, *stats, *dir;
    void *dq, *dk, *dv;
    float *d_temp_raw, *d_null_slope_raw, *d_null_bias, *d_mag_beta, *d_v_null;
    int B, T, Hq, Hkv, D;
    void* workspace;
};
size_t polar_bwd_workspace_bytes(int B, int T, int Hq, int D);
hipError_t launch_polar_bwd(const PolarBwdArgs& a, hipStream_t stream);

// Rotary embedding of x [B, T, H, D] (bf16) into y: row t at position pos0 + t.
struct RopeArgs {
    const void* x;
    void* y;
    int B, T, H, D, pos0;
    double theta;
};
hipError_t launch_rope(const RopeArgs& a, hipStream_t stream);

// Canon prologue: depthwise causal convolution of x [B, T, C] (bf16) with w [K, C] (fp32),
// optional residual and unit norm per head (heads > 0), state [B, K-1, C] in and out.
struct CanonArgs {
    const void* x;
    const float* w;
    const void* state_in;
    void* state_out;
    void* y;
    int B, T, C, K, residual, heads;
    float eps;
};
hipError_t launch_canon(const CanonArgs& a, hipStream_t stream);

struct PolarDecodeArgs {
    const void *q, *k_cache, *v_cache;
    PolarParamsDev p;
    void* o;
    float* mu_out;
    int cache_len, Lmax, B, Hq, Hkv, D;
    void* workspace;
    // per-sequence cache lengths on the device (NULL: every sequence has cache_len); with them,
    // cache_len is the upper bound that sizes the split grid
    const int* lens = nullptr;
    // decode row of the NoPE / RoPE control core (p and mu_out unused); rope_theta > 0 rotates
    // the query to position cache_len - 1 (cached keys already rotated)
    bool softmax = false;
    double rope_theta = 0.0;
};
size_t polar_decode_workspace_bytes(int B, int Hq, int cache_len, int D);
// Head layouts the decode kernels have code for: D in {64, 128}, Hkv in {1,2,4,8,16,32} with
// Hkv * D <= 2048, Hq/Hkv in {1,2,4,8}.
bool polar_decode_supported(int Hq, int Hkv, int D);
hipError_t launch_polar_decode(const PolarDecodeArgs& a, hipStream_t stream);
// The same launches with the split records in the library's fixed per-device array
// (a.workspace ignored); fails when they need more than polar_decode_scratch_bytes().
size_t polar_decode_scratch_bytes();
hipError_t launch_polar_decode_noalloc(PolarDecodeArgs a, hipStream_t stream);

// Sets the dynamic-LDS limit of a kernel once per process.
template <typename K>
inline hipError_t ensure_lds_limit(K kernel, size_t bytes) {
    return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace atma

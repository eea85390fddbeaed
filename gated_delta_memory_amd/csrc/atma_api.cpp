// C-ABI layer of libatma: host-side validation, then kernel launches on the caller's
// stream.  Every check happens before the first HIP call, so a rejected call has no side
// effect on the device.  No allocation, no synchronisation, no exceptions cross the ABI.
#include "atma.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "launch.hpp"

namespace {

constexpr int64_t kMaxElems = (int64_t(1) << 31) - 1;

bool pos(int x) { return x >= 1; }
bool head_width_ok(int d) { return d == 64 || d == 128; }
bool fits(int64_t a, int64_t b, int64_t c, int64_t d) {
    const int64_t ab = a * b;
    if (ab > kMaxElems) return false;
    const int64_t abc = ab * c;
    if (abc > kMaxElems) return false;
    return abc * d <= kMaxElems;
}
int launched(hipError_t e) { return e == hipSuccess ? ATMA_OK : ATMA_ERR_LAUNCH; }

int check_params(const atma_polar_params* p) {
    if (!p || !p->temp_raw || !p->null_slope_raw || !p->null_bias || !p->mag_beta || !p->v_null)
        return ATMA_ERR_NULL;
    if (!(p->eps >= 0.0f) || !std::isfinite(p->eps)) return ATMA_ERR_SHAPE;
    return ATMA_OK;
}

atma::PolarParamsDev dev_params(const atma_polar_params* p) {
    return {p->temp_raw, p->null_slope_raw, p->null_bias, p->mag_beta, p->v_null, p->eps};
}

}  // namespace

extern "C" {

const char* atma_status_string(int status) {
    switch (status) {
        case ATMA_OK: return "ok";
        case ATMA_ERR_NULL: return "a required pointer is NULL";
        case ATMA_ERR_SHAPE: return "invalid or inconsistent size";
        case ATMA_ERR_UNSUPPORTED: return "unsupported head width, chunk or dtype";
        case ATMA_ERR_WORKSPACE: return "workspace missing or too small";
        case ATMA_ERR_LAUNCH: return "HIP launch error";
        default: return "unknown status";
    }
}

int atma_version(void) { return 100; }

size_t atma_gdn_fwd_workspace_bytes_dtype(int B, int T, int H, int Dk, int Dv, int chunk, atma_dtype dt) {
    if (!pos(B) || !pos(T) || !pos(H) || !head_width_ok(Dk) || !head_width_ok(Dv) || chunk != 64) return 0;
    if (dt != ATMA_BF16 && dt != ATMA_F32) return 0;
    return atma::gdn_fwd_workspace_bytes(B, T, H, Dk, Dv, dt == ATMA_BF16);
}

size_t atma_gdn_fwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int chunk) {
    const size_t a = atma_gdn_fwd_workspace_bytes_dtype(B, T, H, Dk, Dv, chunk, ATMA_BF16);
    const size_t b = atma_gdn_fwd_workspace_bytes_dtype(B, T, H, Dk, Dv, chunk, ATMA_F32);
    return a > b ? a : b;
}

int atma_gdn_fwd(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                 const float* init_state, void* o, float* final_state, int B, int T, int H, int Dk, int Dv,
                 int chunk, atma_dtype dt, void* workspace, size_t ws_bytes, void* stream) {
    if (!q || !k || !v || !alpha || !beta || !o) return ATMA_ERR_NULL;
    if (!pos(B) || !pos(T) || !pos(H) || !pos(Dk) || !pos(Dv) || !pos(chunk)) return ATMA_ERR_SHAPE;
    if (!head_width_ok(Dk) || !head_width_ok(Dv) || chunk != 64) return ATMA_ERR_UNSUPPORTED;
    if (dt != ATMA_BF16 && dt != ATMA_F32) return ATMA_ERR_UNSUPPORTED;
    if (!fits(B, T, H, Dk > Dv ? Dk : Dv) || !fits(B, H, Dv, Dk)) return ATMA_ERR_SHAPE;
    if (H > 65535 || B > 65535) return ATMA_ERR_SHAPE;
    const size_t need = atma::gdn_fwd_workspace_bytes(B, T, H, Dk, Dv, dt == ATMA_BF16);
    if (!workspace || ws_bytes < need) return ATMA_ERR_WORKSPACE;
    atma::GdnFwdArgs a{q, k, v, alpha, beta, init_state, o, final_state, B, T, H, Dk, Dv, dt == ATMA_BF16,
                       workspace};
    return launched(atma::launch_gdn_fwd(a, (hipStream_t)stream));
}

int atma_gdn_fwd_varlen(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                        const int* cu_seqlens, int nseq, int max_seqlen, const float* init_state, void* o,
                        float* final_state, int total_T, int H, int Dk, int Dv, int chunk, atma_dtype dt,
                        void* workspace, size_t ws_bytes, void* stream) {
    if (!q || !k || !v || !alpha || !beta || !cu_seqlens || !o) return ATMA_ERR_NULL;
    if (!pos(nseq) || !pos(max_seqlen) || !pos(total_T) || !pos(H) || !pos(Dk) || !pos(Dv) || !pos(chunk))
        return ATMA_ERR_SHAPE;
    if (max_seqlen > total_T) return ATMA_ERR_SHAPE;
    if (!head_width_ok(Dk) || !head_width_ok(Dv) || chunk != 64 || dt != ATMA_BF16) return ATMA_ERR_UNSUPPORTED;
    if (!fits(1, total_T, H, Dk > Dv ? Dk : Dv) || !fits(nseq, max_seqlen, H, 1) || !fits(nseq, H, Dv, Dk))
        return ATMA_ERR_SHAPE;
    if (H > 65535 || nseq > 65535) return ATMA_ERR_SHAPE;
    const size_t need = atma::gdn_fwd_workspace_bytes(nseq, max_seqlen, H, Dk, Dv, true);
    if (!workspace || ws_bytes < need) return ATMA_ERR_WORKSPACE;
    atma::GdnFwdArgs a{q, k, v, alpha, beta, init_state, o, final_state, nseq, max_seqlen, H, Dk, Dv, true,
                       workspace, cu_seqlens, total_T};
    return launched(atma::launch_gdn_fwd(a, (hipStream_t)stream));
}

int atma_gdn_decode_step(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                         float* state, void* o, int B, int H, int Dk, int Dv, atma_dtype dt, void* stream) {
    if (!q || !k || !v || !alpha || !beta || !state || !o) return ATMA_ERR_NULL;
    if (!pos(B) || !pos(H) || !pos(Dk) || !pos(Dv)) return ATMA_ERR_SHAPE;
    if (!head_width_ok(Dk) || !head_width_ok(Dv)) return ATMA_ERR_UNSUPPORTED;
    if (dt != ATMA_BF16 && dt != ATMA_F32) return ATMA_ERR_UNSUPPORTED;
    if (!fits(B, H, Dv, Dk)) return ATMA_ERR_SHAPE;
    if (H > 65535 || B > 65535) return ATMA_ERR_SHAPE;
    atma::GdnDecodeArgs a{q, k, v, alpha, beta, state, o, B, H, Dk, Dv, dt == ATMA_BF16};
    return launched(atma::launch_gdn_decode(a, (hipStream_t)stream));
}

size_t atma_polar_attn_workspace_bytes(int B, int T, int Hq, int D) {
    (void)B; (void)T; (void)Hq; (void)D;
    return 0;
}

int atma_polar_attn_fwd(const void* q, const void* k, const void* v, const atma_polar_params* p, void* o,
                        float* mu_out, float* meff_out, int B, int T, int Hq, int Hkv, int D, atma_dtype dt,
                        void* workspace, size_t ws_bytes, void* stream) {
    (void)workspace; (void)ws_bytes;
    if (!q || !k || !v || !o) return ATMA_ERR_NULL;
    const int pc = check_params(p);
    if (pc != ATMA_OK) return pc;
    if (!pos(B) || !pos(T) || !pos(Hq) || !pos(Hkv) || !pos(D)) return ATMA_ERR_SHAPE;
    if (Hq % Hkv != 0) return ATMA_ERR_SHAPE;
    if ((D != 64 && D != 128) || dt != ATMA_BF16) return ATMA_ERR_UNSUPPORTED;
    if (!fits(B, T, Hq, D) || Hq > 65535 || B > 65535) return ATMA_ERR_SHAPE;
    atma::PolarFwdArgs a{q, k, v, dev_params(p), o, mu_out, meff_out, B, T, Hq, Hkv, D};
    return launched(atma::launch_polar_fwd(a, (hipStream_t)stream));
}

size_t atma_gdn_bwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int chunk, atma_dtype dt) {
    if (!pos(B) || !pos(T) || !pos(H) || !head_width_ok(Dk) || !head_width_ok(Dv) || chunk != 64) return 0;
    if (dt != ATMA_BF16 && dt != ATMA_F32) return 0;
    return atma::gdn_bwd_workspace_bytes(B, T, H, Dk, Dv);
}

int atma_gdn_bwd(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                 const float* init_state, const void* dO, const float* dS_final, void* dq, void* dk, void* dv,
                 float* dalpha, float* dbeta, float* d_init, int B, int T, int H, int Dk, int Dv, int chunk,
                 atma_dtype dt, void* workspace, size_t ws_bytes, void* stream) {
    if (!q || !k || !v || !alpha || !beta || !dO || !dq || !dk || !dv || !dalpha || !dbeta) return ATMA_ERR_NULL;
    if (!pos(B) || !pos(T) || !pos(H) || !pos(Dk) || !pos(Dv)) return ATMA_ERR_SHAPE;
    if (!head_width_ok(Dk) || !head_width_ok(Dv) || chunk != 64) return ATMA_ERR_UNSUPPORTED;
    if (dt != ATMA_BF16 && dt != ATMA_F32) return ATMA_ERR_UNSUPPORTED;
    if (!fits(B, T, H, Dk > Dv ? Dk : Dv) || H > 65535 || B > 65535) return ATMA_ERR_SHAPE;
    if (!workspace || ws_bytes < atma::gdn_bwd_workspace_bytes(B, T, H, Dk, Dv)) return ATMA_ERR_WORKSPACE;
    atma::GdnBwdArgs a{q, k, v, dO, alpha, beta, init_state, dS_final, dq, dk, dv, dalpha, dbeta, d_init,
                       B, T, H, Dk, Dv, dt == ATMA_BF16, workspace};
    return launched(atma::launch_gdn_bwd(a, (hipStream_t)stream));
}

int atma_polar_attn_fwd_train(const void* q, const void* k, const void* v, const atma_polar_params* p, void* o,
                              float* mu_out, float* stats, float* dir, int B, int T, int Hq, int Hkv, int D,
                              atma_dtype dt, void* stream) {
    if (!q || !k || !v || !o || !mu_out || !stats || !dir) return ATMA_ERR_NULL;
    const int pc = check_params(p);
    if (pc != ATMA_OK) return pc;
    if (!(p->eps > 0.0f)) return ATMA_ERR_SHAPE;
    if (!pos(B) || !pos(T) || !pos(Hq) || !pos(Hkv) || !pos(D)) return ATMA_ERR_SHAPE;
    if (Hq % Hkv != 0) return ATMA_ERR_SHAPE;
    if ((D != 64 && D != 128) || dt != ATMA_BF16) return ATMA_ERR_UNSUPPORTED;
    if (!fits(B, T, Hq, D) || Hq > 65535 || B > 65535) return ATMA_ERR_SHAPE;
    atma::PolarFwdArgs a{q, k, v, dev_params(p), o, mu_out, nullptr, B, T, Hq, Hkv, D};
    a.stats = stats;
    a.dir = dir;
    return launched(atma::launch_polar_fwd(a, (hipStream_t)stream));
}

size_t atma_polar_attn_bwd_workspace_bytes(int B, int T, int Hq, int Hkv, int D) {
    if (!pos(B) || !pos(T) || !pos(Hq) || !pos(Hkv) || !head_width_ok(D) || !fits(B, T, Hq, D)) return 0;
    return atma::polar_bwd_workspace_bytes(B, T, Hq, D);
}

int atma_polar_attn_bwd(const void* q, const void* k, const void* v, const atma_polar_params* p, const float* mu,
                        const float* stats, const float* dir, const void* dO, void* dq, void* dk, void* dv,
                        const atma_polar_param_grads* dp, int B, int T, int Hq, int Hkv, int D, atma_dtype dt,
                        void* workspace, size_t ws_bytes, void* stream) {
    if (!q || !k || !v || !mu || !stats || !dir || !dO || !dq || !dk || !dv || !dp) return ATMA_ERR_NULL;
    if (!dp->temp_raw || !dp->null_slope_raw || !dp->null_bias || !dp->mag_beta || !dp->v_null) return ATMA_ERR_NULL;
    const int pc = check_params(p);
    if (pc != ATMA_OK) return pc;
    if (!(p->eps > 0.0f)) return ATMA_ERR_SHAPE;
    if (!pos(B) || !pos(T) || !pos(Hq) || !pos(Hkv) || !pos(D)) return ATMA_ERR_SHAPE;
    if (Hq % Hkv != 0) return ATMA_ERR_SHAPE;
    if ((D != 64 && D != 128) || dt != ATMA_BF16) return ATMA_ERR_UNSUPPORTED;
    if (!fits(B, T, Hq, D) || Hq > 65535 || B > 65535) return ATMA_ERR_SHAPE;
    if (!workspace || ws_bytes < atma::polar_bwd_workspace_bytes(B, T, Hq, D)) return ATMA_ERR_WORKSPACE;
    atma::PolarBwdArgs a{q, k, v, dO, dev_params(p), mu, stats, dir, dq, dk, dv, dp->temp_raw, dp->null_slope_raw,
                         dp->null_bias, dp->mag_beta, dp->v_null, B, T, Hq, Hkv, D, workspace};
    return launched(atma::launch_polar_bwd(a, (hipStream_t)stream));
}

int atma_polar_attn_fwd_varlen(const void* q, const void* k, const void* v, const int* cu_seqlens, int nseq,
                               int max_seqlen, const atma_polar_params* p, void* o, float* mu_out, float* meff_out,
                               int total_T, int Hq, int Hkv, int D, atma_dtype dt, void* stream) {
    if (!q || !k || !v || !cu_seqlens || !o) return ATMA_ERR_NULL;
    const int pc = check_params(p);
    if (pc != ATMA_OK) return pc;
    if (!pos(nseq) || !pos(max_seqlen) || !pos(total_T) || !pos(Hq) || !pos(Hkv) || !pos(D)) return ATMA_ERR_SHAPE;
    if (Hq % Hkv != 0 || max_seqlen > total_T) return ATMA_ERR_SHAPE;
    if ((D != 64 && D != 128) || dt != ATMA_BF16) return ATMA_ERR_UNSUPPORTED;
    if (!fits(1, total_T, Hq, D) || !fits(nseq, max_seqlen, 1, 1) || Hq > 65535 || nseq > 65535)
        return ATMA_ERR_SHAPE;
    atma::PolarFwdArgs a{q, k, v, dev_params(p), o, mu_out, meff_out, nseq, max_seqlen, Hq, Hkv, D, cu_seqlens,
                         total_T};
    return launched(atma::launch_polar_fwd(a, (hipStream_t)stream));
}

size_t atma_polar_attn_decode_workspace_bytes(int B, int Hq, int cache_len, int D) {
    if (!pos(B) || !pos(Hq) || !pos(cache_len) || (D != 64 && D != 128)) return 0;
    return atma::polar_decode_workspace_bytes(B, Hq, cache_len, D);
}

int atma_polar_attn_decode(const void* q, const void* k_cache, const void* v_cache, int cache_len, int Lmax,
                           const atma_polar_params* p, void* o, float* mu_out, int B, int Hq, int Hkv, int D,
                           atma_dtype dt, void* workspace, size_t ws_bytes, void* stream) {
    if (!q || !k_cache || !v_cache || !o) return ATMA_ERR_NULL;
    const int pc = check_params(p);
    if (pc != ATMA_OK) return pc;
    if (!pos(B) || !pos(Hq) || !pos(Hkv) || !pos(D) || !pos(cache_len) || !pos(Lmax)) return ATMA_ERR_SHAPE;
    if (cache_len > Lmax || Hq % Hkv != 0) return ATMA_ERR_SHAPE;
    if (dt != ATMA_BF16 || !atma::polar_decode_supported(Hq, Hkv, D)) return ATMA_ERR_UNSUPPORTED;
    // the cache may exceed 2^31 elements in total (offsets are 64-bit); one sequence may not
    if (!fits(Lmax, Hkv, D, 1) || !fits(B, Hq, D, 1) || Hq > 65535 || B > 65535) return ATMA_ERR_SHAPE;
    const size_t need = atma::polar_decode_workspace_bytes(B, Hq, cache_len, D);
    if (!workspace || ws_bytes < need) return ATMA_ERR_WORKSPACE;
    atma::PolarDecodeArgs a{q, k_cache, v_cache, dev_params(p), o, mu_out, cache_len, Lmax, B, Hq, Hkv, D,
                            workspace};
    return launched(atma::launch_polar_decode(a, (hipStream_t)stream));
}

int atma_polar_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, int cache_len, int Lmax,
                                   const atma_polar_params* p, void* o, float* mu_out, int B, int Hq, int Hkv, int D,
                                   atma_dtype dt, void* stream) {
    if (!q || !k_cache || !v_cache || !o) return ATMA_ERR_NULL;
    const int pc = check_params(p);
    if (pc != ATMA_OK) return pc;
    if (!pos(B) || !pos(Hq) || !pos(Hkv) || !pos(D) || !pos(cache_len) || !pos(Lmax)) return ATMA_ERR_SHAPE;
    if (cache_len > Lmax || Hq % Hkv != 0) return ATMA_ERR_SHAPE;
    if (dt != ATMA_BF16 || !atma::polar_decode_supported(Hq, Hkv, D)) return ATMA_ERR_UNSUPPORTED;
    if (!fits(Lmax, Hkv, D, 1) || !fits(B, Hq, D, 1) || Hq > 65535 || B > 65535) return ATMA_ERR_SHAPE;
    if (atma::polar_decode_workspace_bytes(B, Hq, cache_len, D) > atma::polar_decode_scratch_bytes())
        return ATMA_ERR_WORKSPACE;
    atma::PolarDecodeArgs a{q, k_cache, v_cache, dev_params(p), o, mu_out, cache_len, Lmax, B, Hq, Hkv, D, nullptr};
    return launched(atma::launch_polar_decode_noalloc(a, (hipStream_t)stream));
}

int atma_polar_attn_decode_varlen(const void* q, const void* k_cache, const void* v_cache, const int* cache_lens,
                                  int max_cache_len, int Lmax, const atma_polar_params* p, void* o, float* mu_out,
                                  int B, int Hq, int Hkv, int D, atma_dtype dt, void* workspace, size_t ws_bytes,
                                  void* stream) {
    if (!q || !k_cache || !v_cache || !cache_lens || !o) return ATMA_ERR_NULL;
    const int pc = check_params(p);
    if (pc != ATMA_OK) return pc;
    if (!pos(B) || !pos(Hq) || !pos(Hkv) || !pos(D) || !pos(max_cache_len) || !pos(Lmax)) return ATMA_ERR_SHAPE;
    if (max_cache_len > Lmax || Hq % Hkv != 0) return ATMA_ERR_SHAPE;
    if (dt != ATMA_BF16 || !atma::polar_decode_supported(Hq, Hkv, D)) return ATMA_ERR_UNSUPPORTED;
    if (!fits(Lmax, Hkv, D, 1) || !fits(B, Hq, D, 1) || Hq > 65535 || B > 65535) return ATMA_ERR_SHAPE;
    const size_t need = atma::polar_decode_workspace_bytes(B, Hq, max_cache_len, D);
    if (!workspace || ws_bytes < need) return ATMA_ERR_WORKSPACE;
    atma::PolarDecodeArgs a{q, k_cache, v_cache, dev_params(p), o, mu_out, max_cache_len, Lmax, B, Hq, Hkv, D,
                            workspace, cache_lens};
    return launched(atma::launch_polar_decode(a, (hipStream_t)stream));
}

int atma_rope(const void* x, void* y, int B, int T, int H, int D, int pos0, float theta, atma_dtype dt,
              void* stream) {
    if (!x || !y) return ATMA_ERR_NULL;
    if (!pos(B) || !pos(T) || !pos(H) || !pos(D) || pos0 < 0 || !(theta > 0.0f)) return ATMA_ERR_SHAPE;
    if (D % 2 != 0 || dt != ATMA_BF16) return ATMA_ERR_UNSUPPORTED;
    if (!fits(B, T, H, D) || (int64_t)pos0 + T > 0x7fffffffLL) return ATMA_ERR_SHAPE;
    atma::RopeArgs a{x, y, B, T, H, D, pos0, (double)theta};
    return launched(atma::launch_rope(a, (hipStream_t)stream));
}

size_t atma_softmax_attn_workspace_bytes(int B, int T, int Hq, int Hkv, int D, float rope_theta) {
    if (!pos(B) || !pos(T) || !pos(Hq) || !pos(Hkv) || !pos(D) || !fits(B, T, Hq + Hkv, D)) return 0;
    return rope_theta > 0.0f ? (size_t)B * T * (Hq + Hkv) * D * 2 : 0;
}

int atma_softmax_attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int T, int Hq, int Hkv, int D,
                          float rope_theta, atma_dtype dt, void* workspace, size_t ws_bytes, void* stream) {
    if (!q || !k || !v || !o) return ATMA_ERR_NULL;
    if (!pos(B) || !pos(T) || !pos(Hq) || !pos(Hkv) || !pos(D) || !(rope_theta >= 0.0f)) return ATMA_ERR_SHAPE;
    if (Hq % Hkv != 0) return ATMA_ERR_SHAPE;
    if ((D != 64 && D != 128) || dt != ATMA_BF16) return ATMA_ERR_UNSUPPORTED;
    if (!fits(B, T, Hq + Hkv, D) || Hq > 65535 || B > 65535) return ATMA_ERR_SHAPE;
    const size_t need = atma_softmax_attn_workspace_bytes(B, T, Hq, Hkv, D, rope_theta);
    if (need && (!workspace || ws_bytes < need)) return ATMA_ERR_WORKSPACE;
    const hipStream_t st = (hipStream_t)stream;
    if (rope_theta > 0.0f) {  // rotated copies of q and k in the workspace
        char* qr = (char*)workspace;
        char* kr = qr + (size_t)B * T * Hq * D * 2;
        atma::RopeArgs rq{q, qr, B, T, Hq, D, 0, (double)rope_theta}, rk{k, kr, B, T, Hkv, D, 0, (double)rope_theta};
        const int s1 = launched(atma::launch_rope(rq, st));
        if (s1 != ATMA_OK) return s1;
        const int s2 = launched(atma::launch_rope(rk, st));
        if (s2 != ATMA_OK) return s2;
        q = qr;
        k = kr;
    }
    atma::PolarFwdArgs a{q, k, v, atma::PolarParamsDev{}, o, nullptr, nullptr, B, T, Hq, Hkv, D};
    a.softmax = true;
    return launched(atma::launch_polar_fwd(a, st));
}

int atma_softmax_attn_decode(const void* q, const void* k_cache, const void* v_cache, int cache_len, int Lmax,
                             float rope_theta, void* o, int B, int Hq, int Hkv, int D, atma_dtype dt,
                             void* workspace, size_t ws_bytes, void* stream) {
    if (!q || !k_cache || !v_cache || !o) return ATMA_ERR_NULL;
    if (!pos(B) || !pos(Hq) || !pos(Hkv) || !pos(D) || !pos(cache_len) || !pos(Lmax) || !(rope_theta >= 0.0f))
        return ATMA_ERR_SHAPE;
    if (cache_len > Lmax || Hq % Hkv != 0) return ATMA_ERR_SHAPE;
    if (dt != ATMA_BF16 || !atma::polar_decode_supported(Hq, Hkv, D)) return ATMA_ERR_UNSUPPORTED;
    if (!fits(Lmax, Hkv, D, 1) || !fits(B, Hq, D, 1) || Hq > 65535 || B > 65535) return ATMA_ERR_SHAPE;
    const size_t need = atma::polar_decode_workspace_bytes(B, Hq, cache_len, D);
    if (!workspace || ws_bytes < need) return ATMA_ERR_WORKSPACE;
    atma::PolarDecodeArgs a{q, k_cache, v_cache, atma::PolarParamsDev{}, o, nullptr, cache_len, Lmax, B, Hq, Hkv, D,
                            workspace};
    a.softmax = true;
    a.rope_theta = rope_theta;
    return launched(atma::launch_polar_decode(a, (hipStream_t)stream));
}

int atma_canon(const void* x, const float* w, const void* state_in, void* state_out, void* y, int B, int T, int C,
               int K, int residual, int heads, float eps, atma_dtype dt, void* stream) {
    if (!x || !w || !y) return ATMA_ERR_NULL;
    if (!pos(B) || !pos(T) || !pos(C) || K < 1 || K > 8 || heads < 0 || !(eps > 0.0f)) return ATMA_ERR_SHAPE;
    if (x == y) return ATMA_ERR_SHAPE;  // out of place (a token's inputs are read by later tokens)
    if (dt != ATMA_BF16 || C % 8 != 0) return ATMA_ERR_UNSUPPORTED;
    if (heads > 0) {
        if (C % heads != 0) return ATMA_ERR_SHAPE;
        const int D = C / heads;
        if (D % 8 != 0 || D > 512 || (D & (D - 1)) != 0) return ATMA_ERR_UNSUPPORTED;  // D / 8 lanes, a power of 2
    }
    if (!fits(B, T, C, 1) || !fits(B, K, C, 1)) return ATMA_ERR_SHAPE;
    atma::CanonArgs a{x, w, state_in, state_out, y, B, T, C, K, residual ? 1 : 0, heads, eps};
    return launched(atma::launch_canon(a, (hipStream_t)stream));
}

}  // extern "C"

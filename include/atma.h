/*
 * atma.h - C ABI of libatma, the MI355X (gfx950) hot path of the ATMA hybrid global
 * layer: gated-delta compression memory and causal Polar attention, prefill and decode.
 *
 * Source of every definition: "ATMA: Long-Context Language Modeling via Polar Attention
 * and Gated-Delta Compression Memory" (arXiv 2606.25156).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensor arguments are DEVICE pointers owned by the caller; the library never
 *    allocates, frees or retains them.  Arrays are dense and row-major with the last
 *    index fastest.  `stream` is a hipStream_t (NULL = the default stream).
 *  - Every tensor and workspace pointer is 16-byte aligned (any hipMalloc or torch
 *    allocation is): the kernels move rows in 8- and 16-byte pieces.  Not checked.
 *  - Calls are asynchronous on `stream`: the library performs no host synchronisation,
 *    no allocation and keeps no state between calls (thread-safe; concurrent calls on
 *    different streams must use different workspaces).
 *  - Every argument is validated on the host BEFORE anything is launched; a call that
 *    returns an error has launched nothing.  After the launches a failed
 *    hipGetLastError() returns ATMA_ERR_LAUNCH.  No C++ exception crosses the ABI.
 *  - Supported shapes: memory head widths Dk, Dv in {64, 128} (fp32 or bf16); Polar and
 *    control-core head width D in {64, 128} (bf16); chunk = 64; Hq a multiple of Hkv; every
 *    size >= 1; B * T * H * D below 2^31 for every prefill tensor; a decode KV cache may
 *    exceed 2^31 elements in total but Lmax * Hkv * D must stay below 2^31.
 *  - Preconditions that are documented but not checked (they live on the device):
 *    memory q and k rows have unit L2 norm (Appendix A.2 premise); alpha in (0, 1];
 *    beta in [0, 1]; mag_beta >= 0.  Violating them gives defined but meaningless
 *    numbers, never out-of-bounds accesses.
 *  - Numerics: bf16 operands with fp32 accumulation and fp32 statistics; the memory
 *    state is fp32 in HBM and in registers.  Outputs are written in the input dtype.
 *    Exception: the bf16 memory prefill stages its chunk operands in fp16 (11-bit mantissa,
 *    range below 2^15; see atma_gdn_fwd).
 *    The memory backward computes in fp32 throughout; the Polar backward contracts on
 *    bf16 MFMA like the forward.  Parameter and gate gradients are fp32.
 */
#ifndef ATMA_H
#define ATMA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATMA_OK = 0,
    ATMA_ERR_NULL = -1,        /* a required pointer is NULL                                  */
    ATMA_ERR_SHAPE = -2,       /* a size is < 1, inconsistent, or too large                   */
    ATMA_ERR_UNSUPPORTED = -3, /* a head width, chunk or dtype the library has no kernel for  */
    ATMA_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than the matching *_workspace_bytes */
    ATMA_ERR_LAUNCH = -5       /* the HIP runtime reported an error after launch              */
} atma_status;

typedef enum { ATMA_F32 = 0, ATMA_BF16 = 1 } atma_dtype;

/* Per-head Polar parameters (host struct holding DEVICE pointers, all fp32).
 *   temp_raw[Hq]       : alpha of Section 3.2; temperature t_i = 1 + softplus(temp_raw) ln n_i
 *   null_slope_raw[Hq] : gamma of Section 3.2; null floor nu_i = null_bias + softplus(gamma) sqrt(ln(n_i + 1))
 *   null_bias[Hq]      : b of Section 3.2 (Appendix A.1 assumes b >= 0; not required)
 *   mag_beta[Hq]       : beta of Appendix A.2; magnitude mu_i = tanh(mag_beta ln(1 + m_eff,i))
 *   v_null[Hq * D]     : value of the virtual null sink (Appendix C.3: it joins the direction numerator with the null weight)
 *   eps                : clamp of the direction normaliser max(||s_i||, eps) (Appendix A.2)
 * n_i is the number of real keys query i may see (i + 1 in prefill, cache_len in decode). */
typedef struct {
    const float* temp_raw;
    const float* null_slope_raw;
    const float* null_bias;
    const float* mag_beta;
    const float* v_null;
    float eps;
} atma_polar_params;

/* ---------------------------------------------------------------------------------
 * Gated-delta memory, chunked prefill (Section 3.3 equation):
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t
 * with the paper's gamma_t written alpha_t, M_t written S_t and r_t written o_t.
 * Evaluated exactly (up to rounding) in chunks of `chunk` tokens.
 *
 *   q, k        [B, T, H, Dk]  dtype `dt`  (unit-norm rows; no 1/sqrt(D) is applied)
 *   v           [B, T, H, Dv]  dtype `dt`
 *   alpha, beta [B, T, H]      fp32
 *   init_state  [B, H, Dv, Dk] fp32, or NULL for a zero initial state
 *   o           [B, T, H, Dv]  dtype `dt`  (output)
 *   final_state [B, H, Dv, Dk] fp32 (output), or NULL; may alias init_state
 *   Dk, Dv in {64, 128}; chunk == 64; dt == ATMA_BF16 or ATMA_F32.
 *   workspace   device buffer of at least atma_gdn_fwd_workspace_bytes(...) bytes (or the
 *               smaller atma_gdn_fwd_workspace_bytes_dtype(..., dt)), contents ignored on entry
 *               and undefined on exit.
 * Range (bf16 inputs): the bf16 path stages its chunk operands (the UT-transformed keys and
 * values, the entering state and the chunk's state correction) as fp16 MFMA operands, which hold
 * magnitudes below 2^15 = 32768.  Values |v| and state entries must stay below that (inputs of
 * unit-norm keys and queries with |v| ~ 1 use about 2^-15 of the range); beyond it the fp16
 * staging overflows and o and final_state hold inf or NaN.  Not checked (the values live on the
 * device).  The fp32 path has no such limit.
 * ------------------------------------------------------------------------------- */
int atma_gdn_fwd(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                 const float* init_state, void* o, float* final_state, int B, int T, int H, int Dk,
                 int Dv, int chunk, atma_dtype dt, void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes atma_gdn_fwd needs for either input dtype (the larger of the two). */
size_t atma_gdn_fwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int chunk);

/* Workspace bytes atma_gdn_fwd needs for inputs of dtype `dt` (0 for unsupported arguments). */
size_t atma_gdn_fwd_workspace_bytes_dtype(int B, int T, int H, int Dk, int Dv, int chunk, atma_dtype dt);

/* ---------------------------------------------------------------------------------
 * Gated-delta memory, chunked prefill of a packed batch: nseq sequences of different
 * lengths concatenated along the token axis (no padding); each sequence runs the recurrence
 * of atma_gdn_fwd on its own rows, from its own initial state.
 *   q, k, v      [total_T, H, Dk|Dk|Dv] bf16;  alpha, beta [total_T, H] fp32;  o [total_T, H, Dv]
 *   cu_seqlens   [nseq + 1] int32 in device memory: sequence s holds rows
 *                cu_seqlens[s] .. cu_seqlens[s+1]-1 (0 = cu_seqlens[0] <= ... <= total_T)
 *   max_seqlen   host-side bound on every sequence length (sizes grids and workspace),
 *                <= total_T
 *   init_state   [nseq, H, Dv, Dk] fp32 or NULL (zeros);  final_state [nseq, H, Dv, Dk] or NULL
 *   chunk == 64, dt == ATMA_BF16, Dk and Dv in {64, 128}.
 *   workspace at least atma_gdn_fwd_workspace_bytes_dtype(nseq, max_seqlen, H, Dk, Dv, chunk,
 *   ATMA_BF16) bytes.  The fp16 staging range of atma_gdn_fwd applies.  The offsets are read on
 *   the device: a sequence whose bounds are not inside [0, total_T], decrease, or exceed
 *   max_seqlen is skipped (its rows of o and its final state are left unwritten); no access
 *   leaves the buffers.
 * ------------------------------------------------------------------------------- */
int atma_gdn_fwd_varlen(const void* q, const void* k, const void* v, const float* alpha,
                        const float* beta, const int* cu_seqlens, int nseq, int max_seqlen,
                        const float* init_state, void* o, float* final_state, int total_T, int H,
                        int Dk, int Dv, int chunk, atma_dtype dt, void* workspace, size_t ws_bytes,
                        void* stream);

/* ---------------------------------------------------------------------------------
 * Gated-delta memory, backward of the chunked prefill: gradients of a loss L through
 * o = atma_gdn_fwd(...) (and its final state), given dO = dL/do and optionally dS_final =
 * dL/dS_T.  The chain rule on the Section 3.3 recurrence, taken on its exact chunk form: the
 * forward is recomputed chunk by chunk (states kept per chunk), the state gradient is carried
 * backwards (per chunk an affine map, the transpose of the forward's), then every chunk's
 * input gradients are formed in parallel.  fp32 arithmetic throughout.
 *   q, k, v, alpha, beta, init_state   the forward's inputs (init_state may be NULL = zero)
 *   dO        [B, T, H, Dv] dtype `dt`;  dS_final [B, H, Dv, Dk] fp32 or NULL (zero)
 *   dq, dk    [B, T, H, Dk] dtype `dt`;  dv [B, T, H, Dv] dtype `dt`
 *   dalpha, dbeta [B, T, H] fp32;  d_init [B, H, Dv, Dk] fp32 or NULL (the gradient on the
 *             initial state)
 *   Dk, Dv in {64, 128}; chunk == 64; dt == ATMA_BF16 or ATMA_F32.  All outputs are written,
 *   not accumulated.  alpha must be > 0 (the gradient divides by it).
 *   workspace at least atma_gdn_bwd_workspace_bytes(...) bytes (per chunk: the recomputed
 *   chunk operands, the chunk's input state and its gradient; about 520 KB per chunk at
 *   Dk = Dv = 128).
 * ------------------------------------------------------------------------------- */
int atma_gdn_bwd(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                 const float* init_state, const void* dO, const float* dS_final, void* dq, void* dk,
                 void* dv, float* dalpha, float* dbeta, float* d_init, int B, int T, int H, int Dk,
                 int Dv, int chunk, atma_dtype dt, void* workspace, size_t ws_bytes, void* stream);

size_t atma_gdn_bwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int chunk, atma_dtype dt);

/* ---------------------------------------------------------------------------------
 * Gated-delta memory, one decode step (the same equation for a single token):
 *     S <- alpha (S - beta (S k) k^T) + beta v k^T ;  o = S q
 *   q, k   [B, H, Dk] dtype `dt`;  v [B, H, Dv] dtype `dt`;  alpha, beta [B, H] fp32
 *   state  [B, H, Dv, Dk] fp32, updated in place;  o [B, H, Dv] dtype `dt` (output)
 * No workspace.  The recurrent state has a fixed size, so decode cost does not depend
 * on the context length (Appendix H.1).
 * ------------------------------------------------------------------------------- */
int atma_gdn_decode_step(const void* q, const void* k, const void* v, const float* alpha,
                         const float* beta, float* state, void* o, int B, int H, int Dk, int Dv,
                         atma_dtype dt, void* stream);

/* ---------------------------------------------------------------------------------
 * Causal Polar attention, prefill (Section 3.2 equation; Appendix A.2 channels;
 * Appendix C.2 single softmax over real logits plus one virtual null logit; streamed
 * with the running statistics of Appendix C.3, Table 6).  For query i (0-based) of
 * head h, with kv head h / (Hq / Hkv), n = i + 1:
 *     t = 1 + softplus(temp_raw) ln n,   nu = null_bias + softplus(null_slope_raw) sqrt(ln(n+1))
 *     real logits  l_j = t (q_i . k_j) / sqrt(D), j = 0..i;   null logit  l_0 = t nu
 *     w = softmax over {l_j} U {l_0};  R = sum_j w_j;  n_eff = R^2 / sum_j w_j^2
 *     m_eff = n_eff R;  mu = tanh(mag_beta ln(1 + m_eff))
 *     s = sum_j w_j v_j + w_0 v_null;  c = s / max(||s||, eps);  o_i = mu c
 *   q        [B, T, Hq, D]  dtype `dt`;  k, v [B, T, Hkv, D] dtype `dt`
 *   o        [B, T, Hq, D]  dtype `dt` (output)
 *   mu_out   [B, Hq, T] fp32 (output) or NULL;  meff_out [B, Hq, T] fp32 or NULL
 *   D in {64, 128} and dt == ATMA_BF16; workspace may be NULL when
 *   atma_polar_attn_workspace_bytes returns 0 (it does in this version).
 * ------------------------------------------------------------------------------- */
int atma_polar_attn_fwd(const void* q, const void* k, const void* v, const atma_polar_params* p,
                        void* o, float* mu_out, float* meff_out, int B, int T, int Hq, int Hkv, int D,
                        atma_dtype dt, void* workspace, size_t ws_bytes, void* stream);

size_t atma_polar_attn_workspace_bytes(int B, int T, int Hq, int D);

/* ---------------------------------------------------------------------------------
 * Causal Polar attention, training forward: the operation of atma_polar_attn_fwd, also writing
 * what atma_polar_attn_bwd reads (the layer is trained end to end; the backward recomputes
 * the weights from these instead of storing the T x T matrix, as the streaming form of
 * Appendix C.3 does for the forward).
 *   q, k, v, o as atma_polar_attn_fwd;  mu_out [B, Hq, T] fp32 (required)
 *   stats    [B, Hq, T, 4] fp32: per row {lse2, R, Q2, den}: lse2 = log2 of the softmax
 *            partition (real keys and null) in units where weight_j = exp2(t log2(e) q.k_j /
 *            sqrt(D) - lse2); R = real mass; Q2 = sum_j w_j^2; den = ||s|| when ||s|| > eps,
 *            else -eps (the clamp was taken)
 *   dir      [B, T, Hq, D] fp32: the direction c = s / max(||s||, eps)
 *   D in {64, 128}, dt == ATMA_BF16, eps > 0.  No workspace.
 * ------------------------------------------------------------------------------- */
int atma_polar_attn_fwd_train(const void* q, const void* k, const void* v, const atma_polar_params* p,
                              void* o, float* mu_out, float* stats, float* dir, int B, int T, int Hq,
                              int Hkv, int D, atma_dtype dt, void* stream);

/* Gradients of the per-head Polar parameters (DEVICE pointers, fp32, written, not accumulated):
 * temp_raw, null_slope_raw, null_bias, mag_beta [Hq]; v_null [Hq * D]. */
typedef struct {
    float* temp_raw;
    float* null_slope_raw;
    float* null_bias;
    float* mag_beta;
    float* v_null;
} atma_polar_param_grads;

/* ---------------------------------------------------------------------------------
 * Causal Polar attention, backward: gradients of a loss L through o = atma_polar_attn_fwd(...),
 * given dO = dL/do.  The chain rule on the definitions above (Section 3.2 equation, Appendix
 * C.2 single softmax, Appendix A.2 channels): with w the weights of row i, R, Q2, m_eff = R^3 / Q2,
 * mu, s, c and den as in the forward,
 *   dmu = dO . c;  ds = mu (dO - [||s|| > eps] dmu c) / den;  dm_eff = dmu (1 - mu^2) beta / (1 + m_eff)
 *   dl_j = w_j (ds . v_j + dR + 2 w_j dQ2 - Sigma) with dR = 3 dm_eff m_eff / R,
 *   dQ2 = -dm_eff m_eff / Q2, Sigma = dR R + 2 dQ2 Q2 + ds . s;  the null logit likewise;
 *   dq = t / sqrt(D) sum_j dl_j k_j;  dk_j, dv_j summed over every query (and query head) that
 *   sees key j;  the parameter gradients summed over every row of the batch.
 *   q, k, v   the forward's inputs;  mu, stats, dir  the outputs of atma_polar_attn_fwd_train
 *   dO        [B, T, Hq, D] bf16
 *   dq        [B, T, Hq, D] bf16;  dk, dv [B, T, Hkv, D] bf16 (written, not accumulated)
 *   dp        parameter gradients (written)
 *   workspace at least atma_polar_attn_bwd_workspace_bytes(B, T, Hq, Hkv, D) bytes.
 *   D in {64, 128}, dt == ATMA_BF16, eps > 0.  The result is deterministic (no atomics).
 * ------------------------------------------------------------------------------- */
int atma_polar_attn_bwd(const void* q, const void* k, const void* v, const atma_polar_params* p,
                        const float* mu, const float* stats, const float* dir, const void* dO, void* dq,
                        void* dk, void* dv, const atma_polar_param_grads* dp, int B, int T, int Hq,
                        int Hkv, int D, atma_dtype dt, void* workspace, size_t ws_bytes, void* stream);

size_t atma_polar_attn_bwd_workspace_bytes(int B, int T, int Hq, int Hkv, int D);

/* ---------------------------------------------------------------------------------
 * Causal Polar attention, prefill of a packed batch: nseq sequences of different lengths
 * concatenated along the token axis (no padding).  Same operation as atma_polar_attn_fwd
 * within each sequence (n = i + 1 for the sequence's own query i; no attention across
 * sequences).
 *   q            [total_T, Hq, D] dtype `dt`;  k, v [total_T, Hkv, D];  o [total_T, Hq, D]
 *   cu_seqlens   [nseq + 1] int32 in device memory: sequence s holds rows
 *                cu_seqlens[s] .. cu_seqlens[s+1]-1 (0 = cu_seqlens[0] <= ... <= total_T)
 *   max_seqlen   host-side bound on every sequence length (sizes the grid), <= total_T
 *   mu_out, meff_out  [Hq, total_T] fp32 or NULL
 *   D in {64, 128} and dt == ATMA_BF16.  No workspace.  The offsets are read on the device: a
 *   sequence whose bounds are not inside [0, total_T], decrease, or exceed max_seqlen is
 *   skipped (its rows of o are left unwritten); no access leaves the buffers.
 * ------------------------------------------------------------------------------- */
int atma_polar_attn_fwd_varlen(const void* q, const void* k, const void* v, const int* cu_seqlens,
                               int nseq, int max_seqlen, const atma_polar_params* p, void* o,
                               float* mu_out, float* meff_out, int total_T, int Hq, int Hkv, int D,
                               atma_dtype dt, void* stream);

/* ---------------------------------------------------------------------------------
 * Polar attention, one decode step: the last causal row for a KV cache.
 *   q        [B, Hq, D] dtype `dt`
 *   k_cache, v_cache [B, Lmax, Hkv, D] dtype `dt`; slots 0..cache_len-1 are valid and the
 *            caller has already written the new token's k, v into slot cache_len-1.
 *   n = cache_len in the formulas above (1 <= cache_len <= Lmax).
 *   D in {64, 128}, dt == ATMA_BF16, Hkv in {1, 2, 4, 8, 16, 32} with Hkv * D <= 2048, and
 *   Hq / Hkv in {1, 2, 4, 8} (so the real-model layout, 8 query / 2 kv heads at D = 128, works).
 *   o        [B, Hq, D] dtype `dt` (output);  mu_out [B, Hq] fp32 or NULL
 *   workspace at least atma_polar_attn_decode_workspace_bytes(B, Hq, cache_len, D) bytes
 *            (per split of the cache: running max, real mass, squared mass and value sum).
 * ------------------------------------------------------------------------------- */
int atma_polar_attn_decode(const void* q, const void* k_cache, const void* v_cache, int cache_len,
                           int Lmax, const atma_polar_params* p, void* o, float* mu_out, int B, int Hq,
                           int Hkv, int D, atma_dtype dt, void* workspace, size_t ws_bytes,
                           void* stream);

size_t atma_polar_attn_decode_workspace_bytes(int B, int Hq, int cache_len, int D);

/* ---------------------------------------------------------------------------------
 * Polar attention, one decode step that allocates nothing and takes no workspace: for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same operation, arguments and results as
 * atma_polar_attn_decode (bitwise: the same kernels and split grid), with the split records in
 * a fixed array of device memory inside the library: 16 MiB, one copy per GPU the library runs
 * on, held until the process ends.
 *   Limit: atma_polar_attn_decode_workspace_bytes(B, Hq, cache_len, D) <= 16 MiB (for example
 *   B * Hq * (D + 4) * 4 * splits with at most 512 splits in all; every B up to 512 fits at
 *   Hq * (D + 4) <= 8192); larger calls return ATMA_ERR_WORKSPACE without launching.
 *   The stream must belong to the current device.  Every call on one GPU shares that GPU's array
 *   (each call overwrites what it reads, nothing is carried between calls), so calls that overlap
 *   on one GPU -- on different streams or from different threads -- race and must be ordered by
 *   the caller.  The first call on a device looks the array up (no allocation).
 * ------------------------------------------------------------------------------- */
int atma_polar_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, int cache_len,
                                   int Lmax, const atma_polar_params* p, void* o, float* mu_out, int B, int Hq,
                                   int Hkv, int D, atma_dtype dt, void* stream);

/* ---------------------------------------------------------------------------------
 * Polar attention, one decode step for a batch of sequences with different cache lengths
 * (heterogeneous serving batches).  Same operation as atma_polar_attn_decode with
 * n = cache_lens[b] for sequence b.
 *   cache_lens    [B] int32 in device memory: valid slots 0..cache_lens[b]-1 of sequence b
 *                 (the new token's k, v already written at slot cache_lens[b]-1)
 *   max_cache_len host-side bound, 1 <= cache_lens[b] <= max_cache_len <= Lmax; it sizes
 *                 the split grid and the workspace:
 *                 atma_polar_attn_decode_workspace_bytes(B, Hq, max_cache_len, D) bytes.
 *   Other arguments as for atma_polar_attn_decode.  The lengths are read on the device, so
 *   the host cannot check them: a sequence whose length lies outside [1, max_cache_len] gets
 *   NaN in o (and mu_out); the other sequences are unaffected.
 * ------------------------------------------------------------------------------- */
int atma_polar_attn_decode_varlen(const void* q, const void* k_cache, const void* v_cache,
                                  const int* cache_lens, int max_cache_len, int Lmax,
                                  const atma_polar_params* p, void* o, float* mu_out, int B, int Hq,
                                  int Hkv, int D, atma_dtype dt, void* workspace, size_t ws_bytes,
                                  void* stream);

/* ---------------------------------------------------------------------------------
 * Control cores: the NoPE and RoPE attention the ATMA paper matches Polar against
 * (Section 3.1: only the attention core changes among NoPE, RoPE and Polar).  Causal
 * softmax attention with logits q_i . k_j / sqrt(D) and output o_i = sum_j w_ij v_j (no
 * temperature, no null, no channels); for RoPE every adjacent pair (x[2p], x[2p+1]) of q and
 * k at position m is first turned by the angle m * theta^(-2p/D) (rotary position embedding,
 * theta = 10000 in the usual setting).  Same prefill and decode kernels as Polar.
 * ------------------------------------------------------------------------------- */

/* Rotary embedding: y = x with row t of every sequence turned to position pos0 + t.
 *   x, y [B, T, H, D] bf16 (y may alias x), D even, theta > 0, pos0 >= 0.
 *   The angle is formed in fp64.  Use it to fill a RoPE KV cache with rotated keys. */
int atma_rope(const void* x, void* y, int B, int T, int H, int D, int pos0, float theta, atma_dtype dt,
              void* stream);

/* Prefill: q [B, T, Hq, D], k, v [B, T, Hkv, D], o [B, T, Hq, D]; D in {64, 128}, bf16.
 *   rope_theta == 0: NoPE;  rope_theta > 0: RoPE with that base (positions 0..T-1).
 *   workspace: atma_softmax_attn_workspace_bytes(...) bytes (the rotated q and k; 0 for NoPE). */
int atma_softmax_attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int T, int Hq,
                          int Hkv, int D, float rope_theta, atma_dtype dt, void* workspace,
                          size_t ws_bytes, void* stream);

size_t atma_softmax_attn_workspace_bytes(int B, int T, int Hq, int Hkv, int D, float rope_theta);

/* Decode: the query (position cache_len - 1) against cache slots 0..cache_len-1.  For RoPE
 *   (rope_theta > 0) the cache holds keys already rotated to their slot positions (atma_rope);
 *   the query is rotated inside.  Shapes, head layouts and workspace as for
 *   atma_polar_attn_decode (atma_polar_attn_decode_workspace_bytes). */
int atma_softmax_attn_decode(const void* q, const void* k_cache, const void* v_cache, int cache_len,
                             int Lmax, float rope_theta, void* o, int B, int Hq, int Hkv, int D,
                             atma_dtype dt, void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * Canon prologue (Section 3.1: Canon depthwise causal convolutions on q, k and v before
 * attention; the pages fix neither width, bias nor residual): per channel c,
 *     y_t[c] = sum_{j<K} w[j][c] x_{t-j}[c]  (+ x_t[c] when residual != 0),
 * inputs before the first token taken from state_in (the K-1 previous inputs, oldest first;
 * zeros when NULL); then, when heads > 0, each head's D = C / heads channels are scaled to
 * unit L2 norm, y / max(||y||, eps) (the memory path's unit-norm queries and keys).
 *   x, y      [B, T, C] bf16 (y must not alias x);  w [K, C] fp32;  1 <= K <= 8;  C % 8 == 0
 *   heads     0, or a divisor of C with D = C / heads a power of two in [8, 512]
 *   state_in  [B, K-1, C] bf16 or NULL;  state_out [B, K-1, C] bf16 or NULL: receives the last
 *             K-1 inputs (from state_in where T < K-1); it may alias state_in (decode: T = 1).
 * ------------------------------------------------------------------------------- */
int atma_canon(const void* x, const float* w, const void* state_in, void* state_out, void* y, int B, int T,
               int C, int K, int residual, int heads, float eps, atma_dtype dt, void* stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* atma_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int atma_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATMA_H */

// Gated-delta memory, chunked backward, for gfx950.
//
// Gradients of o_t = S_t q_t through S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
// (ATMA paper, Section 3.3 equation), taken on the exact chunk form of the forward (derivation in
// gdn_fwd.hip): for a chunk of C = 64 tokens with state S_in,
//     Delta = U - W S_in^T,   O = QG S_in^T + P Delta,   S_out = e^{g_last} S_in + Delta^T KD,
//     W = Tinv diag(beta e^g) K,  U = Tinv diag(beta) V,  Tinv = (I + A)^{-1},
//     A = strict_lower(diag(beta) (K K^T) o E),  P = lower_incl((Q K^T) o E),  E_rs = e^{g_r - g_s},
//     QG = diag(e^g) Q,  KD = diag(e^{g_last - g}) K.
// Reverse mode, per chunk, given dO and the gradient dS_out on its output state:
//     dDelta = P^T dO + KD dS_out^T
//     dS_in  = e^{g_last} dS_out + dO^T QG - dDelta^T W          (the carry: affine in dS_out)
//     dU = dDelta, dW = -dDelta S_in, dQG = dO S_in, dP = lower_incl(dO Delta^T), dKD = Delta dS_out
//     dTinv = dU (diag(beta) V)^T + dW (diag(beta e^g) K)^T,  dA = -strict_lower(Tinv^T dTinv Tinv^T)
//     dv = beta o (Tinv^T dU),  dq = e^g o dQG + (dP o E) K,
//     dk = beta e^g o (Tinv^T dW) + e^{g_last - g} o dKD + (dP o E)^T Q + M K + M^T K,  M = dA o beta E
//     dbeta_r = sum_s dA_rs E_rs k_r.k_s + (Tinv^T dU)_r . v_r + e^{g_r} (Tinv^T dW)_r . k_r
//     dg_r = rowsum_r(dA o A) - colsum_r(dA o A) + rowsum_r(dP o P) - colsum_r(dP o P)
//            + beta_r e^{g_r} (Tinv^T dW)_r . k_r + e^{g_r} dQG_r . q_r - dKD_r . KD_r
//            (+ sum_r dKD_r . KD_r + e^{g_last} <dS_out, S_in> on the last row of the chunk)
//     d ln(alpha_s) = sum_{r >= s} dg_r within the chunk;  dalpha = d ln(alpha) / alpha.
// Five kernels, all fp32 arithmetic (inputs bf16 or fp32, converted on load):
//   prep   (parallel over chunks)  g, A, Tinv (forward substitution), W, U, KD; raw K K^T
//   walk   (sequential over chunks, one workgroup per 32 state rows)  S_in and Delta per chunk
//   pre    (parallel over chunks)  P^T dO and dO^T QG; raw Q K^T
//   walk   (sequential, reverse)   dS_out and dDelta per chunk, the gradient on the initial state
//   post   (parallel over chunks)  every gradient above
// Matrix products use one LDS-staged fp32 routine on v_mfma_f32_16x16x4_f32 (K in slices of 16).  Rows past the end of a ragged last chunk are zero (k = q = v = 0,
// beta = 0, alpha = 1), which keeps every formula exact for the real rows.
#include "atma_device.hpp"
#include "launch.hpp"

namespace atma {
namespace {

constexpr int NT = 256;
constexpr int C = 64;
constexpr int KS = 16;   // k-slice of the tiled product
constexpr int LD64 = C + 1;

// C[M][N] = sum_k A(i, k) B(k, j), delivered element by element to epi(i, j, value).  A and B
// come from run functors (global memory or LDS) that return four consecutive elements along the
// operand's contiguous direction: la(i, k) = A(i, k..k+3) if AK, else A(i..i+3, k); lb(k, j) =
// B(k, j..j+3) if BJ, else B(k..k+3, j) -- one 16-byte (fp32) or 8-byte (bf16) load where the
// source is a row-major array.  K slices of KS are staged in LDS as sA [KS][M + 16] and sB
// [KS][N + 16] (the padding of 16 puts the four k rows one fp32 MFMA reads on four different
// 16-bank groups).  The product runs on v_mfma_f32_16x16x4_f32: lane l supplies
// A[i0 + l % 16][k + l / 16] and B[k + l / 16][j0 + l % 16] and holds C[i0 + 4 (l / 16) + v][j0 + l % 16]
// in accumulator v.  Each wave owns a band of 16-row tiles (all column tiles), or for M = 16 a
// quarter of the column tiles.  AK: A's contiguous index in memory is k (else i); BJ: B's is j
// (else k) -- chooses the staging order so that consecutive threads read consecutive addresses.
// tgemm_blk hands the finished accumulators to blk(acc, rt0, ct0): acc[x][y][v] is element
// (16 (rt0 + x) + 4 (lane / 16) + v, 16 (ct0 + y) + lane % 16); tgemm applies epi to each.
template <int M, int N, int K, bool AK, bool BJ, class LA, class LB, class BLK>
__device__ __forceinline__ void tgemm_blk(float* stage, LA la, LB lb, BLK blk) {
    static_assert(M % 16 == 0 && N % 16 == 0 && K % KS == 0, "tile shape");
    constexpr int MT = M / 16, NTL = N / 16;
    static_assert(MT % 4 == 0 || (MT == 1 && NTL % 4 == 0), "wave split");
    constexpr int RT = MT >= 4 ? MT / 4 : 1, CT = MT >= 4 ? NTL : NTL / 4;
    constexpr int LDA = M + 16, LDB = N + 16;
    float* sA = stage;
    float* sB = stage + KS * LDA;
    const int tid = (int)threadIdx.x, lane = tid & 63, w = tid >> 6, G = lane >> 4, c16 = lane & 15;
    const int rt0 = MT >= 4 ? w * RT : 0, ct0 = MT >= 4 ? 0 : w * CT;
    __syncthreads();  // what earlier epilogues wrote (LDS or global) is visible to the staging below
    f32x4 acc[RT][CT];
#pragma unroll
    for (int x = 0; x < RT; ++x)
#pragma unroll
        for (int y = 0; y < CT; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
    // software pipeline: the next K slice is fetched into registers while the current one is
    // multiplied, so the latency of the operand loads overlaps the MFMAs.  Each thread moves runs
    // of four elements along the operand's contiguous direction (consecutive LDS slots where the
    // slice row is contiguous)
    constexpr int PA = M * KS / NT / 4, PB = N * KS / NT / 4, NS = K / KS;
    static_assert(M * KS % (NT * 4) == 0 && N * KS % (NT * 4) == 0, "staging split");
    // two slices in flight: slice s + 2 is requested while slice s is multiplied (the slice loop
    // is unrolled so the register buffers are indexed statically)
    f32x4 ra[2][PA], rb[2][PB];
    auto a_pos = [&](int m, int& i, int& kk) {  // first element of run m of this thread
        const int q = tid + m * NT;
        if (AK) { i = q / (KS / 4); kk = (q % (KS / 4)) * 4; }
        else { kk = q / (M / 4); i = (q % (M / 4)) * 4; }
    };
    auto b_pos = [&](int m, int& j, int& kk) {
        const int q = tid + m * NT;
        if (BJ) { kk = q / (N / 4); j = (q % (N / 4)) * 4; }
        else { j = q / (KS / 4); kk = (q % (KS / 4)) * 4; }
    };
    auto fetch = [&](int buf, int k0) {
#pragma unroll
        for (int m = 0; m < PA; ++m) {
            int i, kk;
            a_pos(m, i, kk);
            ra[buf][m] = la(i, k0 + kk);
        }
#pragma unroll
        for (int m = 0; m < PB; ++m) {
            int j, kk;
            b_pos(m, j, kk);
            rb[buf][m] = lb(k0 + kk, j);
        }
    };
    fetch(0, 0);
    if (NS > 1) fetch(1, KS);
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
        const int buf = sl & 1;
#pragma unroll
        for (int m = 0; m < PA; ++m) {
            int i, kk;
            a_pos(m, i, kk);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (AK) sA[(kk + u) * LDA + i] = ra[buf][m][u];
                else sA[kk * LDA + i + u] = ra[buf][m][u];
            }
        }
#pragma unroll
        for (int m = 0; m < PB; ++m) {
            int j, kk;
            b_pos(m, j, kk);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (BJ) sB[kk * LDB + j + u] = rb[buf][m][u];
                else sB[(kk + u) * LDB + j] = rb[buf][m][u];
            }
        }
        __syncthreads();
        if (sl + 2 < NS) fetch(buf, (sl + 2) * KS);
#pragma unroll
        for (int kk = 0; kk < KS; kk += 4) {
            float a[RT], b[CT];
#pragma unroll
            for (int x = 0; x < RT; ++x) a[x] = sA[(kk + G) * LDA + (rt0 + x) * 16 + c16];
#pragma unroll
            for (int y = 0; y < CT; ++y) b[y] = sB[(kk + G) * LDB + (ct0 + y) * 16 + c16];
#pragma unroll
            for (int x = 0; x < RT; ++x)
#pragma unroll
                for (int y = 0; y < CT; ++y) acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[x], b[y], acc[x][y], 0, 0, 0);
        }
        __syncthreads();
    }
    blk(acc, rt0, ct0);
}

template <class ACC, class EPI>
__device__ __forceinline__ void each_elem(const ACC& acc, int rt0, int ct0, EPI epi) {
    constexpr int RT = sizeof(ACC) / sizeof(acc[0]), CT = sizeof(acc[0]) / sizeof(f32x4);
    const int lane = (int)threadIdx.x & 63, G = lane >> 4, c16 = lane & 15;
#pragma unroll
    for (int x = 0; x < RT; ++x)
#pragma unroll
        for (int y = 0; y < CT; ++y)
#pragma unroll
            for (int v = 0; v < 4; ++v) epi((rt0 + x) * 16 + 4 * G + v, (ct0 + y) * 16 + c16, acc[x][y][v]);
}

template <int M, int N, int K, bool AK, bool BJ, class LA, class LB, class EPI>
__device__ __forceinline__ void tgemm(float* stage, LA la, LB lb, EPI epi) {
    tgemm_blk<M, N, K, AK, BJ>(stage, la, lb, [&](const auto& acc, int rt0, int ct0) { each_elem(acc, rt0, ct0, epi); });
}

// For a product with one 16-row tile per wave (M = 64): rowdot(acc, rt0, f) returns, in every lane,
// the four sums over the product's columns j of C[i][j] f(i, j) for the lane's rows
// i = 16 rt0 + 4 (lane / 16) + v (the 16 lanes of a row group hold its columns).
template <int CT, class F>
__device__ __forceinline__ f32x4 rowdot(const f32x4 (&acc)[1][CT], int rt0, F f) {
    const int lane = (int)threadIdx.x & 63, G = lane >> 4, c16 = lane & 15;
    f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int y = 0; y < CT; ++y)
#pragma unroll
        for (int v = 0; v < 4; ++v) part[v] = fmaf(acc[0][y][v], f(16 * rt0 + 4 * G + v, 16 * y + c16), part[v]);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1)
#pragma unroll
        for (int v = 0; v < 4; ++v) part[v] += __shfl_xor(part[v], o, 16);
    return part;
}

// The values f(r, c) that rowdot or an epilogue pairs with this lane's accumulator elements of a
// product with one 16-row tile per wave (M = 64, so wave w owns row tile w), requested before the
// product so that their trip to memory overlaps its MFMAs: pre[y][v] = f(16 w + 4 (lane / 16) + v,
// 16 y + lane % 16).
template <int CT, class F>
__device__ __forceinline__ void prefetch_rows(f32x4 (&pre)[CT], F f) {
    const int lane = (int)threadIdx.x & 63, G = lane >> 4, c16 = lane & 15, rt0 = (int)threadIdx.x >> 6;
#pragma unroll
    for (int y = 0; y < CT; ++y)
#pragma unroll
        for (int v = 0; v < 4; ++v) pre[y][v] = f(16 * rt0 + 4 * G + v, 16 * y + c16);
}
// rowdot with the factors already in registers (the same sums in the same order).
template <int CT>
__device__ __forceinline__ f32x4 rowdot_pre(const f32x4 (&acc)[1][CT], const f32x4 (&pre)[CT]) {
    f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int y = 0; y < CT; ++y)
#pragma unroll
        for (int v = 0; v < 4; ++v) part[v] = fmaf(acc[0][y][v], pre[y][v], part[v]);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1)
#pragma unroll
        for (int v = 0; v < 4; ++v) part[v] += __shfl_xor(part[v], o, 16);
    return part;
}

constexpr size_t STAGE_FLOATS = (size_t)KS * (128 + 16) * 2;  // sA + sB for the largest shapes (M, N <= 128)

// Per-chunk fp32 workspace arrays, chunk id cid = (b H + h) NC + c.
template <int DK, int DV>
struct WsLay {
    static constexpr size_t W = 0, U = W + (size_t)C * DK, KD = U + (size_t)C * DV, TI = KD + (size_t)C * DK,
                            G = TI + (size_t)C * C, EGL = G + C, SIN = EGL + 4, DL = SIN + (size_t)DV * DK,
                            E = DL + (size_t)C * DV, F = E + (size_t)C * DV, DDL = F + (size_t)DV * DK,
                            DSO = DDL + (size_t)C * DV, X1 = DSO + (size_t)DV * DK,
                            X2 = X1 + (size_t)C * DK, X4 = X2 + (size_t)C * DK,
                            NQK = X4 + (size_t)C * DK, NKK = NQK + C * C,
                            DSS = NKK + C * C,  // DSS: <dS_out, S_in> per row slice of the walk
                            PER = DSS + 4;                       // floats per chunk
};

// Four consecutive elements p[0..3] as fp32: one 16-byte (fp32) or 8-byte (bf16) load.  Every run
// the products request starts at a multiple of four elements of a row whose length is a multiple
// of 64, so with 16-byte-aligned base pointers the loads are naturally aligned.
__device__ __forceinline__ f32x4 ld4(const float* p) { return *(const f32x4*)p; }
__device__ __forceinline__ f32x4 ld4(const bf16* p) {
    const bf16x4 x = *(const bf16x4*)p;
    return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}
// Four elements read one by one (a run that is strided in its source).
template <class F>
__device__ __forceinline__ f32x4 gather4(F f) { return f32x4{f(0), f(1), f(2), f(3)}; }
constexpr f32x4 kZero4 = {0.f, 0.f, 0.f, 0.f};

// Token layout helpers: row r of chunk c of (b, h) is token t0 + r; rows >= n read as zero.
struct ChunkPos {
    int b, h, c, n, t0;
    size_t cid;
};
__device__ __forceinline__ ChunkPos chunk_pos(int Tlen, int H, int NC) {
    ChunkPos p;
    p.c = (int)blockIdx.x; p.h = (int)blockIdx.y; p.b = (int)blockIdx.z;
    p.t0 = p.c * C;
    p.n = min(C, Tlen - p.t0);
    p.cid = ((size_t)p.b * H + p.h) * NC + p.c;
    return p;
}

// ---------------------------------------------------------------------------------------------
// prep: g, A, Tinv, W, U, KD per chunk
// ---------------------------------------------------------------------------------------------
template <typename T, int DK, int DV>
__global__ __launch_bounds__(NT, 2) void gdn_bwd_prep(const T* __restrict__ k, const T* __restrict__ v,
                                                      const float* __restrict__ alpha, const float* __restrict__ beta,
                                                      float* __restrict__ ws, int Tlen, int H, int NC) {
    using L = WsLay<DK, DV>;
    // The chunk's K and V rows are read once, with 16-byte loads issued before anything else, and
    // every product takes them from LDS (rows padded by 16 bytes); A lives in the products' staging
    // buffer between its product and the inverse.
    constexpr int EK = 16 / (int)sizeof(T), LDK = DK + EK, LDV = DV + EK;
    constexpr int NKL = C * DK / EK / NT, NVL = C * DV / EK / NT;
    static_assert(NKL * EK * NT == C * DK && NVL * EK * NT == C * DV, "tile copy split");
    constexpr int LT = C + 4;  // row stride of A and Tinv (16-byte rows)
    static_assert((size_t)C * LT <= STAGE_FLOATS, "A in the staging buffer");
    __shared__ __align__(16) float stage[STAGE_FLOATS];
    __shared__ __align__(16) T Kt[C * LDK];
    __shared__ __align__(16) T Vt[C * LDV];
    __shared__ __align__(16) float Tm[C * LT];
    __shared__ float gs[C], bs[C], g2[C], bsg[C], ekd[C];
    float* Am = stage;
    const ChunkPos P = chunk_pos(Tlen, H, NC);
    float* rec = ws + P.cid * L::PER;
    const size_t tok0 = ((size_t)P.b * Tlen + P.t0) * H + P.h;
    const int tid = (int)threadIdx.x, n = P.n;
    const size_t ks = (size_t)H * DK, vs = (size_t)H * DV;
    const T* kc = k + tok0 * DK;
    const T* vc = v + tok0 * DV;
    f32x4 kr[NKL], vr[NVL];  // 16-byte carriers (raw bits of EK elements)
#pragma unroll
    for (int m = 0; m < NKL; ++m) {
        const int i = (tid + m * NT) * EK, r = i / DK, d = i % DK;
        kr[m] = kZero4;
        if (r < n) __builtin_memcpy(&kr[m], kc + (size_t)r * ks + d, 16);
    }
#pragma unroll
    for (int m = 0; m < NVL; ++m) {
        const int i = (tid + m * NT) * EK, r = i / DV, d = i % DV;
        vr[m] = kZero4;
        if (r < n) __builtin_memcpy(&vr[m], vc + (size_t)r * vs + d, 16);
    }
    if (tid < 64) {
        const bool ok = tid < n;
        float la = ok ? logf(alpha[tok0 + (size_t)tid * H]) : 0.0f;
        bs[tid] = ok ? beta[tok0 + (size_t)tid * H] : 0.0f;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_up(la, o, 64);
            if (tid >= o) la += y;
        }
        gs[tid] = la;
        rec[L::G + tid] = la;
        // exponentials of the gates once per row (base 2 on the hardware unit)
        const float l2 = la * kLog2e, gl2 = __shfl(la, n - 1, 64) * kLog2e;
        g2[tid] = l2;
        bsg[tid] = bs[tid] * fast_exp2(l2);
        ekd[tid] = fast_exp2(gl2 - l2);
    }
#pragma unroll
    for (int m = 0; m < NKL; ++m) {
        const int i = (tid + m * NT) * EK;
        __builtin_memcpy(Kt + (i / DK) * LDK + i % DK, &kr[m], 16);
    }
#pragma unroll
    for (int m = 0; m < NVL; ++m) {
        const int i = (tid + m * NT) * EK;
        __builtin_memcpy(Vt + (i / DV) * LDV + i % DV, &vr[m], 16);
    }
    __syncthreads();
    auto krow4 = [&](int r, int d) { return ld4(Kt + r * LDK + d); };
    // A = strict_lower(diag(beta) (K K^T) o E); the raw K K^T also goes to the workspace for post
    tgemm<C, C, DK, true, false>(stage, krow4, [&](int d, int s) { return krow4(s, d); },
                                 [&](int r, int s, float x) {
                                     Am[r * LT + s] = s < r ? bs[r] * fast_exp2(g2[r] - g2[s]) * x : 0.0f;
                                     rec[L::NKK + r * C + s] = x;
                                 });
    __syncthreads();
    // Tinv = (I + A)^{-1} (unit lower triangular) in 16 x 16 blocks.  Diagonal blocks: forward
    // substitution in registers, one lane per (block, column) of wave 0, while the other waves clear
    // the upper blocks.  Off-diagonal blocks by distance d = i - j = 1, 2, 3 (one wave each):
    //     T_ij = -T_ii sum_{m = j}^{i - 1} A_im T_mj
    // on fp32 MFMA; in step e the lanes of group G supply k slot 4 G + e of both operands, and the
    // second product takes the first one's accumulator as its B operand in the same slot order.
    {
        const int lane = tid & 63, w = tid >> 6, G = lane >> 4, l16 = lane & 15;
        if (w == 0) {
            const int o = 16 * G, col = l16;
            float a[16][16];
#pragma unroll
            for (int r = 1; r < 16; ++r)
#pragma unroll
                for (int s4 = 0; s4 < 16; s4 += 4)
                    if (s4 < r) {
                        const f32x4 x = *(const f32x4*)&Am[(o + r) * LT + o + s4];
#pragma unroll
                        for (int u = 0; u < 4; ++u) a[r][s4 + u] = x[u];
                    }
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = r == col ? 1.0f : 0.0f;
#pragma unroll
                for (int s2 = 0; s2 < r; ++s2) acc = fmaf(-a[r][s2], x[s2], acc);
                x[r] = acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) Tm[(o + r) * LT + o + col] = x[r];
        } else {
            for (int i = tid - 64; i < 6 * 256; i += NT - 64) {
                const int u = i >> 8, e = i & 255;
                const int bi = u < 3 ? 0 : u < 5 ? 1 : 2, bj = u < 3 ? u + 1 : u < 5 ? u - 1 : 3;
                Tm[(16 * bi + (e >> 4)) * LT + 16 * bj + (e & 15)] = 0.0f;
            }
        }
        __syncthreads();
        for (int d = 1; d < 4; ++d) {
            if (w < 4 - d) {
                const int j = w, i = w + d;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                for (int m = j; m < i; ++m)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Am[(16 * i + l16) * LT + 16 * m + 4 * G + e],
                                                                   Tm[(16 * m + 4 * G + e) * LT + 16 * j + l16], acc, 0, 0, 0);
                f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    y = __builtin_amdgcn_mfma_f32_16x16x4f32(Tm[(16 * i + l16) * LT + 16 * i + 4 * G + e], acc[e], y, 0, 0, 0);
#pragma unroll
                for (int x = 0; x < 4; ++x) Tm[(16 * i + 4 * G + x) * LT + 16 * j + l16] = -y[x];
            }
            __syncthreads();
        }
    }
    for (int i = 4 * tid; i < C * C; i += 4 * NT) *(f32x4*)(rec + L::TI + i) = *(const f32x4*)&Tm[(i / C) * LT + i % C];
    // W = Tinv diag(beta e^g) K,  U = Tinv diag(beta) V
    auto trow4 = [&](int r, int s) { return *(const f32x4*)&Tm[r * LT + s]; };
    tgemm<C, DK, C, true, true>(stage, trow4, [&](int s, int d) { return bsg[s] * krow4(s, d); },
                                [&](int r, int d, float x) { rec[L::W + (size_t)r * DK + d] = x; });
    tgemm<C, DV, C, true, true>(stage, trow4, [&](int s, int d) { return bs[s] * ld4(Vt + s * LDV + d); },
                                [&](int r, int d, float x) { rec[L::U + (size_t)r * DV + d] = x; });
    for (int i = 4 * tid; i < C * DK; i += 4 * NT) {
        const int r = i / DK, d = i % DK;
        *(f32x4*)(rec + L::KD + i) = ekd[r] * krow4(r, d);
    }
    if (tid == 0) rec[L::EGL] = expf(gs[n - 1]);
}

// ---------------------------------------------------------------------------------------------
// walk: the two sequential state walks, one kernel.  A workgroup owns RW = 32 state rows of a
// (batch, head) and visits the chunks in order (forward) or in reverse (backward):
//   forward:   S_in stored;  Delta = U[:, rows] - W S^T;           S = e^{g_last} S + Delta^T KD
//   backward:  dS_out stored; dDelta = E[:, rows] + KD dS^T;       dS = e^{g_last} dS + F[rows, :] - dDelta^T W
// (S^T and Delta written for the per-chunk kernels; the backward walk also leaves each slice's share
// of <dS_out, S_in> for the chunk's decay gradient).  The chunk's two 64 x Dk operands (W and KD,
// in the order the walk uses them) sit whole in LDS; the next chunk's operands are loaded into
// registers while the current chunk multiplies, so the walk waits on memory only once.  Products
// on v_mfma_f32_16x16x4_f32 straight from LDS: rows padded by 4 floats where a lane reads along
// the row (A operand), by 16 where the lanes of a group read along a column (B operand), so the
// 64 lanes of a read hit 64 different banks.
// ---------------------------------------------------------------------------------------------
constexpr int RW = 32;
constexpr int NTW = 512, NWW = NTW / 64;  // threads and waves of a walk workgroup (two waves per SIMD)

template <int DK, int DV, bool BACK>
__global__ __launch_bounds__(NTW) __attribute__((amdgpu_waves_per_eu(2, 2))) void gdn_bwd_walk(const float* __restrict__ s0, float* __restrict__ sfinal,
                                                   float* __restrict__ ws, int H, int NC) {
    using L = WsLay<DK, DV>;
    constexpr int LA = DK + 4, LB = DK + 16, LS = DK + 4, LX = RW + 16;
    constexpr size_t OFF_A = BACK ? L::KD : L::W;   // A operand of the first product
    constexpr size_t OFF_B = BACK ? L::W : L::KD;   // B operand of the second product
    constexpr size_t OFF_X = BACK ? L::E : L::U;    // added to the first product
    constexpr size_t OFF_XO = BACK ? L::DDL : L::DL;
    constexpr size_t OFF_SO = BACK ? L::DSO : L::SIN;
    constexpr float SG1 = BACK ? 1.0f : -1.0f, SG2 = BACK ? -1.0f : 1.0f;
    constexpr int NA = C * DK / 4 / NTW, NX = C * RW / 4 / NTW, NF = RW * DK / 4 / NTW;
    static_assert(NA >= 1 && NX >= 1 && NF >= 1, "split");
    __shared__ __align__(16) float As[C * LA];
    __shared__ __align__(16) float Bs[C * LB];
    __shared__ __align__(16) float St[RW * LS];
    __shared__ __align__(16) float Xs[C * LX];
    // Flat grid of (b H + h) * (DV / RW) + slice items.  Workgroup i is dispatched to XCD i % 8;
    // the items are renumbered so that every XCD takes a contiguous range of them, which puts the
    // row slices of one (batch, head) on one XCD and lets them share each chunk's W and KD in its L2.
    const int nwg = (int)gridDim.x, wg = (int)blockIdx.x, per = nwg >> 3, extra = nwg & 7, xcd = wg & 7;
    const int item = xcd * per + min(xcd, extra) + (wg >> 3);
    const int row0 = (item % (DV / RW)) * RW, tid = (int)threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, G = lane >> 4, c16 = lane & 15;
    const size_t bh = (size_t)(item / (DV / RW));
    // state rows in, zero when absent
    for (int q = tid; q < RW * DK / 4; q += NTW) {
        const int i = q / (DK / 4), d4 = (q % (DK / 4)) * 4;
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (s0) x = *(const f32x4*)(s0 + (bh * DV + row0 + i) * DK + d4);
        *(f32x4*)(St + i * LS + d4) = x;
    }
    f32x4 ra[NA], rb[NA], rx[NX], rf[NF], rs[NF];
    float regl;
    __shared__ float wred[NWW];
    // part p of NP of a chunk's operands (part 0 also takes the small ones): the parts are issued
    // between the k ranges of the first product, so the loads drain while the MFMAs run instead
    // of stalling the waves at issue
    constexpr int NP = NA >= 4 ? 4 : NA;
    static_assert(NA % NP == 0 && NP >= 2 && DK % (4 * NP) == 0, "fetch split");
    auto fetch_part = [&](int c, int p) {
        const float* rec = ws + (bh * NC + c) * L::PER;
#pragma unroll
        for (int m = p * (NA / NP); m < (p + 1) * (NA / NP); ++m) {
            const int q = tid + m * NTW, r = q / (DK / 4), d4 = (q % (DK / 4)) * 4;
            ra[m] = *(const f32x4*)(rec + OFF_A + (size_t)r * DK + d4);
            rb[m] = *(const f32x4*)(rec + OFF_B + (size_t)r * DK + d4);
        }
        if constexpr (BACK) {
            if (p == 1)
#pragma unroll
                for (int m = 0; m < NF; ++m) {
                    const int q = tid + m * NTW, i = q / (DK / 4), d4 = (q % (DK / 4)) * 4;
                    rs[m] = *(const f32x4*)(rec + L::SIN + (size_t)(row0 + i) * DK + d4);
                }
        }
        if (p != 0) return;
#pragma unroll
        for (int m = 0; m < NX; ++m) {
            const int q = tid + m * NTW, r = q / (RW / 4), c4 = (q % (RW / 4)) * 4;
            rx[m] = *(const f32x4*)(rec + OFF_X + (size_t)r * DV + row0 + c4);
        }
        if constexpr (BACK) {
#pragma unroll
            for (int m = 0; m < NF; ++m) {
                const int q = tid + m * NTW, i = q / (DK / 4), d4 = (q % (DK / 4)) * 4;
                rf[m] = *(const f32x4*)(rec + L::F + (size_t)(row0 + i) * DK + d4);
            }
        }
        regl = rec[L::EGL];
    };
#pragma unroll
    for (int p = 0; p < NP; ++p) fetch_part(BACK ? NC - 1 : 0, p);
    for (int it = 0; it < NC; ++it) {
        const int c = BACK ? NC - 1 - it : it;
        float* rec = ws + (bh * NC + c) * L::PER;
        const float egl = regl;
        f32x4 fcur[NF];
#pragma unroll
        for (int m = 0; m < NF; ++m) fcur[m] = rf[m];
        __syncthreads();  // the previous chunk is done with As, Bs, Xs and St
        // operands of this chunk into LDS; the state (S_in or dS_out) out to the workspace
#pragma unroll
        for (int m = 0; m < NA; ++m) {
            const int q = tid + m * NTW, r = q / (DK / 4), d4 = (q % (DK / 4)) * 4;
            *(f32x4*)(As + r * LA + d4) = ra[m];
            *(f32x4*)(Bs + r * LB + d4) = rb[m];
        }
#pragma unroll
        for (int m = 0; m < NX; ++m) {
            const int q = tid + m * NTW, r = q / (RW / 4), c4 = (q % (RW / 4)) * 4;
            *(f32x4*)(Xs + r * LX + c4) = rx[m];
        }
        if constexpr (BACK) {  // dS_out out, and this slice's share of <dS_out, S_in>
            float dot = 0.f;
#pragma unroll
            for (int m = 0; m < NF; ++m) {
                const int q = tid + m * NTW, i = q / (DK / 4), d4 = (q % (DK / 4)) * 4;
                const f32x4 x = *(const f32x4*)(St + i * LS + d4);
                *(f32x4*)(rec + OFF_SO + (size_t)(row0 + i) * DK + d4) = x;
                dot = fmaf(x[0], rs[m][0], fmaf(x[1], rs[m][1], fmaf(x[2], rs[m][2], fmaf(x[3], rs[m][3], dot))));
            }
            dot = wave_sum(dot);
            if (lane == 0) wred[w] = dot;
        } else {
            for (int q = tid; q < RW * DK / 4; q += NTW) {
                const int i = q / (DK / 4), d4 = (q % (DK / 4)) * 4;
                *(f32x4*)(rec + OFF_SO + (size_t)(row0 + i) * DK + d4) = *(const f32x4*)(St + i * LS + d4);
            }
        }
        __syncthreads();
        if (BACK && tid == 0) {
            float dss = 0.f;
#pragma unroll
            for (int i = 0; i < NWW; ++i) dss += wred[i];
            rec[L::DSS + row0 / RW] = dss;
        }
        // X[r][i] += SG1 * sum_d A[r][d] St[i][d]: wave w owns the 16 x 16 tile (rows 16 (w % 4),
        // columns 16 (w / 4)); the next chunk's operands are requested a part at a time between the
        // k ranges.  Lane group G takes the quarter d in [G DK / 4, (G + 1) DK / 4) (MFMA step t
        // sums d = G DK / 4 + t over the four groups), so every lane reads its A row and its S^T
        // column as runs of four (16-byte LDS reads), and four accumulators (steps t mod 4) split
        // the chain of dependent MFMAs.
        static_assert(C / 16 * (RW / 16) == NWW, "one tile per wave");
        {
            const int rt = w % (C / 16), yt = w / (C / 16);
            constexpr int KQ = DK / 4;
            static_assert(KQ % (4 * NP) == 0, "steps per part");
            f32x4 acc4[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) acc4[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            const float* arow = As + (16 * rt + c16) * LA + G * KQ;
            const float* srow = St + (16 * yt + c16) * LS + G * KQ;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                if (it + 1 < NC) fetch_part(BACK ? c - 1 : c + 1, p);
#pragma unroll
                for (int t = p * (KQ / NP); t < (p + 1) * (KQ / NP); t += 4) {
                    const f32x4 a4 = *(const f32x4*)(arow + t), s4 = *(const f32x4*)(srow + t);
#pragma unroll
                    for (int u = 0; u < 4; ++u) acc4[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[u], s4[u], acc4[u], 0, 0, 0);
                }
            }
            f32x4 acc;
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[v] = (acc4[0][v] + acc4[1][v]) + (acc4[2][v] + acc4[3][v]);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = 16 * rt + 4 * G + v, i = 16 * yt + c16;
                const float x = Xs[r * LX + i] + SG1 * acc[v];
                Xs[r * LX + i] = x;
                rec[OFF_XO + (size_t)r * DV + row0 + i] = x;
            }
        }
        __syncthreads();
        // St = e^{g_last} St (+ F rows)
#pragma unroll
        for (int m = 0; m < NF; ++m) {
            const int q = tid + m * NTW, i = q / (DK / 4), d4 = (q % (DK / 4)) * 4;
            f32x4 x = *(const f32x4*)(St + i * LS + d4);
#pragma unroll
            for (int u = 0; u < 4; ++u) x[u] = BACK ? fmaf(egl, x[u], fcur[m][u]) : egl * x[u];
            *(f32x4*)(St + i * LS + d4) = x;
        }
        __syncthreads();
        // St[i][d] += SG2 * sum_r X[r][i] B[r][d]: wave w owns column tiles of one row tile
        {
            constexpr int DT = DK / 16 / (NWW / (RW / 16));  // column tiles per wave
            const int yt = w % (RW / 16), d0 = (w / (RW / 16)) * DT;
            // the two halves of the chunk accumulate separately (twice the independent MFMA chains)
            f32x4 acc[2][DT];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int x = 0; x < DT; ++x) acc[hf][x] = f32x4{0.f, 0.f, 0.f, 0.f};
            // operands of four k steps are read before their MFMAs (one LDS round trip per group)
#pragma unroll
            for (int k0 = 0; k0 < C / 2; k0 += 16) {
                float a[2][4], b[2][4][DT];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int kk = k0 + 4 * j + hf * (C / 2);
                        a[hf][j] = Xs[(kk + G) * LX + 16 * yt + c16];
#pragma unroll
                        for (int x = 0; x < DT; ++x) b[hf][j][x] = Bs[(kk + G) * LB + 16 * (d0 + x) + c16];
                    }
                __builtin_amdgcn_sched_barrier(0);  // keep the group's reads ahead of its MFMAs
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                        for (int x = 0; x < DT; ++x)
                            acc[hf][x] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[hf][j], b[hf][j][x], acc[hf][x], 0, 0, 0);
            }
#pragma unroll
            for (int x = 0; x < DT; ++x)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int i = 16 * yt + 4 * G + v, d = 16 * (d0 + x) + c16;
                    St[i * LS + d] += SG2 * (acc[0][x][v] + acc[1][x][v]);
                }
        }
    }
    __syncthreads();
    if (sfinal)
        for (int q = tid; q < RW * DK / 4; q += NTW) {
            const int i = q / (DK / 4), d4 = (q % (DK / 4)) * 4;
            *(f32x4*)(sfinal + (bh * DV + row0 + i) * DK + d4) = *(const f32x4*)(St + i * LS + d4);
        }
}

// ---------------------------------------------------------------------------------------------
// pre: E = P^T dO and F = dO^T QG per chunk
// ---------------------------------------------------------------------------------------------
template <typename T, int DK, int DV>
__global__ __launch_bounds__(NT) void gdn_bwd_pre(const T* __restrict__ q, const T* __restrict__ k,
                                                  const T* __restrict__ dO, float* __restrict__ ws, int Tlen, int H,
                                                  int NC) {
    using L = WsLay<DK, DV>;
    __shared__ float stage[STAGE_FLOATS];
    __shared__ float Pm[C * LD64];
    __shared__ float g2[C], eg[C];
    const ChunkPos P = chunk_pos(Tlen, H, NC);
    float* rec = ws + P.cid * L::PER;
    const int tid = (int)threadIdx.x, n = P.n;
    if (tid < C) {
        g2[tid] = rec[L::G + tid] * kLog2e;
        eg[tid] = fast_exp2(g2[tid]);
    }
    __syncthreads();
    const size_t tok0 = ((size_t)P.b * Tlen + P.t0) * H + P.h, ks = (size_t)H * DK, vs = (size_t)H * DV;
    const T *qc = q + tok0 * DK, *kc = k + tok0 * DK, *oc = dO + tok0 * DV;
    // rows past n read row n - 1 and are zeroed after the load: no branch around the load, so the
    // loads of a product's K slice are all in flight together
    auto qrow4 = [&](int r, int d) { const f32x4 x = ld4(qc + (size_t)min(r, n - 1) * ks + d); return r < n ? x : kZero4; };
    auto orow4 = [&](int r, int j) { const f32x4 x = ld4(oc + (size_t)min(r, n - 1) * vs + j); return r < n ? x : kZero4; };
    tgemm<C, C, DK, true, false>(stage, qrow4,
                                 [&](int d, int s) { const f32x4 x = ld4(kc + (size_t)min(s, n - 1) * ks + d); return s < n ? x : kZero4; },
                                 [&](int r, int s, float x) {
                                     Pm[r * LD64 + s] = s <= r ? x * fast_exp2(g2[r] - g2[s]) : 0.0f;
                                     rec[L::NQK + r * C + s] = x;  // raw Q K^T, for post
                                 });
    __syncthreads();
    tgemm<C, DV, C, false, true>(stage,
                                 [&](int s, int r) { return gather4([&](int u) { return Pm[r * LD64 + s + u]; }); },
                                 orow4, [&](int s, int j, float x) { rec[L::E + (size_t)s * DV + j] = x; });
    tgemm<DV, DK, C, false, true>(stage, [&](int i, int r) { return orow4(r, i); },
                                  [&](int r, int d) { return eg[r] * qrow4(r, d); },
                                  [&](int i, int d, float x) { rec[L::F + (size_t)i * DK + d] = x; });
}

// ---------------------------------------------------------------------------------------------
// post: every input gradient of a chunk
// ---------------------------------------------------------------------------------------------
template <typename T, int DK, int DV>
__global__ __launch_bounds__(NT, 2) void gdn_bwd_post(const T* __restrict__ q, const T* __restrict__ k,
                                                   const T* __restrict__ v, const float* __restrict__ alpha,
                                                   const float* __restrict__ beta, const T* __restrict__ dO,
                                                   T* __restrict__ dq, T* __restrict__ dk, T* __restrict__ dv,
                                                   float* __restrict__ dalpha, float* __restrict__ dbeta,
                                                   float* __restrict__ ws, int Tlen, int H, int NC) {
    using L = WsLay<DK, DV>;
    __shared__ float stage[STAGE_FLOATS];
    __shared__ float gs[C], bs[C], rowv[6][C], red[NT], g2[C], eg[C], bsg[C], ekd[C];
    const ChunkPos P = chunk_pos(Tlen, H, NC);
    float* rec = ws + P.cid * L::PER;
    constexpr int LD64 = C;  // row stride of the workspace 64 x 64 arrays
    const float* Tm = rec + L::TI;
    float *QK = rec + L::NQK, *KK = rec + L::NKK;
    // dP, dTinv (later dA) and Z (later M) are read and rewritten several times each: they stay in LDS
    // (rows of C + 4 floats), the rest of the chunk's intermediates go through the workspace.
    constexpr int LN = C + 4;
    __shared__ __align__(16) float dP[C * LN], dT[C * LN], Zm[C * LN];
    const int tid = (int)threadIdx.x, n = P.n;
    if (tid < C) {
        gs[tid] = rec[L::G + tid];
        bs[tid] = tid < n ? beta[((size_t)P.b * Tlen + P.t0 + tid) * H + P.h] : 0.0f;
        // exponentials of the gates once per row (base 2 on the hardware unit)
        g2[tid] = gs[tid] * kLog2e;
        eg[tid] = fast_exp2(g2[tid]);
        bsg[tid] = bs[tid] * eg[tid];
        ekd[tid] = fast_exp2(rec[L::G + n - 1] * kLog2e - g2[tid]);
    }
    __syncthreads();
    const size_t tok0 = ((size_t)P.b * Tlen + P.t0) * H + P.h, ks = (size_t)H * DK, vs = (size_t)H * DV;
    const T *qc = q + tok0 * DK, *kc = k + tok0 * DK, *vc = v + tok0 * DV, *oc = dO + tok0 * DV;
    // rows past n read row n - 1 and are zeroed after the load: no branch around the load, so the
    // loads of a product's K slice (and of a prefetch) are all in flight together
    auto qrow4 = [&](int r, int d) { const f32x4 x = ld4(qc + (size_t)min(r, n - 1) * ks + d); return r < n ? x : kZero4; };
    auto krow4 = [&](int r, int d) { const f32x4 x = ld4(kc + (size_t)min(r, n - 1) * ks + d); return r < n ? x : kZero4; };
    auto vrow4 = [&](int r, int j) { const f32x4 x = ld4(vc + (size_t)min(r, n - 1) * vs + j); return r < n ? x : kZero4; };
    auto orow4 = [&](int r, int j) { const f32x4 x = ld4(oc + (size_t)min(r, n - 1) * vs + j); return r < n ? x : kZero4; };
    const float* Sin = rec + L::SIN;
    const float* dSo = rec + L::DSO;
    // element loaders for the per-row dot products (rows past n read as zero)
    auto qel = [&](int r, int d) { const float x = to_f32(qc[(size_t)min(r, n - 1) * ks + d]); return r < n ? x : 0.0f; };
    auto kel = [&](int r, int d) { const float x = to_f32(kc[(size_t)min(r, n - 1) * ks + d]); return r < n ? x : 0.0f; };
    auto vel = [&](int r, int j) { const float x = to_f32(vc[(size_t)min(r, n - 1) * vs + j]); return r < n ? x : 0.0f; };
    // Per-row sums, each formed in the epilogue of the product that makes its left factor (so no
    // product is read back for them): rowv[0] = dq_r . q_r, [1] = colsum over the n x n terms,
    // [2] = sum_s dA_rs E_rs k_r . k_s, [3] = X3_r . v_r, [4] = X4_r . k_r, [5] = X2_r . k_r.
    const int c16 = tid & 15, G4 = ((tid & 63) >> 4) * 4;
    auto put_rows = [&](int slot, int rt0, f32x4 part) {
        if (c16 == 0)
#pragma unroll
            for (int v = 0; v < 4; ++v) rowv[slot][16 * rt0 + G4 + v] = part[v];
    };
    // the k elements of X2_r . k_r and X4_r . k_r, in flight during the first products
    f32x4 kpre[DK / 16];
    prefetch_rows(kpre, kel);
    // X1 = dW = -dDelta S_in
    tgemm<C, DK, DV, true, true>(stage, [&](int r, int i) { return ld4(rec + L::DDL + (size_t)r * DV + i); },
                                 [&](int i, int d) { return ld4(Sin + (size_t)i * DK + d); },
                                 [&](int r, int d, float x) { rec[L::X1 + (size_t)r * DK + d] = -x; });
    // X2 = dKD = Delta dS_out (kept for dk), and X2_r . k_r
    tgemm_blk<C, DK, DV, true, true>(stage, [&](int r, int i) { return ld4(rec + L::DL + (size_t)r * DV + i); },
                                     [&](int i, int d) { return ld4(dSo + (size_t)i * DK + d); },
                                     [&](const auto& acc, int rt0, int ct0) {
                                         each_elem(acc, rt0, ct0, [&](int r, int d, float x) {
                                             rec[L::X2 + (size_t)r * DK + d] = x;
                                         });
                                         put_rows(5, rt0, rowdot_pre(acc, kpre));
                                     });
    // dP = lower_incl(dO Delta^T) (the raw Q K^T and K K^T are in the workspace, from pre and prep)
    tgemm<C, C, DV, true, false>(stage, orow4, [&](int j, int s) { return ld4(rec + L::DL + (size_t)s * DV + j); },
                                 [&](int r, int s, float x) { dP[r * LN + s] = s <= r ? x : 0.0f; });
    // the v elements of X3_r . v_r, in flight during dTinv
    f32x4 vpre[DV / 16];
    prefetch_rows(vpre, vel);
    // dTinv = dDelta (diag(beta) V)^T + dW (diag(beta e^g) K)^T
    tgemm<C, C, DV + DK, true, false>(
        stage,
        [&](int r, int j) {
            return j < DV ? ld4(rec + L::DDL + (size_t)r * DV + j) : ld4(rec + L::X1 + (size_t)r * DK + j - DV);
        },
        [&](int j, int s) { return j < DV ? bs[s] * vrow4(s, j) : bsg[s] * krow4(s, j - DV); },
        [&](int r, int s, float x) { dT[r * LN + s] = x; });
    // X3 = Tinv^T dDelta: dv = beta o X3, and X3_r . v_r
    tgemm_blk<C, DV, C, false, true>(stage, [&](int r, int s) { return ld4(Tm + s * LD64 + r); },
                                     [&](int s, int j) { return ld4(rec + L::DDL + (size_t)s * DV + j); },
                                     [&](const auto& acc, int rt0, int ct0) {
                                         each_elem(acc, rt0, ct0, [&](int r, int j, float x) {
                                             if (r < n) dv[(size_t)r * vs + j + tok0 * DV] = from_f32<T>(bs[r] * x);
                                         });
                                         put_rows(3, rt0, rowdot_pre(acc, vpre));
                                     });
    // X4 = Tinv^T dW (kept for dk), and X4_r . k_r
    tgemm_blk<C, DK, C, false, true>(stage, [&](int r, int s) { return ld4(Tm + s * LD64 + r); },
                                     [&](int s, int d) { return ld4(rec + L::X1 + (size_t)s * DK + d); },
                                     [&](const auto& acc, int rt0, int ct0) {
                                         each_elem(acc, rt0, ct0, [&](int r, int d, float x) {
                                             rec[L::X4 + (size_t)r * DK + d] = x;
                                         });
                                         put_rows(4, rt0, rowdot_pre(acc, kpre));
                                     });
    // the q elements of dq_r . q_r, in flight from here to the dq product
    f32x4 qpre[DK / 16];
    prefetch_rows(qpre, qel);
    // Z = dTinv Tinv^T, then dA = -strict_lower(Tinv^T Z) (into dT)
    tgemm<C, C, C, true, false>(stage, [&](int r, int s) { return ld4(dT + r * LN + s); },
                                [&](int s, int c2) { return ld4(Tm + c2 * LD64 + s); },
                                [&](int r, int c2, float x) { Zm[r * LN + c2] = x; });
    tgemm<C, C, C, false, true>(stage, [&](int r, int s) { return ld4(Tm + s * LD64 + r); },
                                [&](int s, int c2) { return ld4(Zm + s * LN + c2); },
                                [&](int r, int c2, float x) { dT[r * LN + c2] = c2 < r ? -x : 0.0f; });
    __syncthreads();
    // column sums over the n x n terms, rowv[1] = colsum(dA o A + dP o P), and
    // rowv[2] = sum_s dA_rs E_rs k_r.k_s (so rowsum(dA o A) = beta_r rowv[2]; rowsum(dP o P) is part
    // of dq_r . q_r).  Thread t visits (r = t / 64 + 4 m, s = t % 64), m = 0..15: every visit reads
    // whole rows of the workspace arrays (coalesced); a wave covers one row per visit, so row sums are
    // wave reductions, and column sums stay in the thread (fixed s) until four partials meet in LDS.
    {
        const int sc = tid & (C - 1), w0 = tid >> 6;
        float col = 0.f;
        float kkv[C / 4], qkv[C / 4];  // every workspace value of the loop, requested before it starts
#pragma unroll
        for (int m = 0; m < C / 4; ++m) {
            kkv[m] = KK[(w0 + 4 * m) * LD64 + sc];
            qkv[m] = QK[(w0 + 4 * m) * LD64 + sc];
        }
#pragma unroll 4
        for (int m = 0; m < C / 4; ++m) {
            const int r = w0 + 4 * m;
            const float e = sc <= r ? fast_exp2(g2[r] - g2[sc]) : 0.0f;  // never exp of the upper triangle
            const float dA = dT[r * LN + sc], kk = kkv[m];
            const float pP = sc <= r ? qkv[m] * e : 0.0f;
            const float dae = dA * e * kk;
            col += fmaf(dae, bs[r], dP[r * LN + sc] * pP);
            const float r2 = wave_sum(dae);
            if (sc == 0) rowv[2][r] = r2;
        }
        red[tid] = col;
        __syncthreads();
        if (tid < C) rowv[1][tid] = (red[tid] + red[tid + C]) + (red[tid + 2 * C] + red[tid + 3 * C]);
    }
    __syncthreads();
    // dP o E into dP, M = dA o beta E into Zm
#pragma unroll
    for (int i = tid; i < C * C; i += NT) {
        const int r = i / C, s = i % C;
        const float e = s <= r ? fast_exp2(g2[r] - g2[s]) : 0.0f;
        dP[r * LN + s] *= e;
        Zm[r * LN + s] = dT[r * LN + s] * bs[r] * e;
    }
    __syncthreads();
    // X4 and dKD for dk's epilogue (the elements this lane itself stored: the same row and column
    // tiles), in flight during the dq product
    f32x4 x4pre[DK / 16], x2pre[DK / 16];
    prefetch_rows(x4pre, [&](int r, int d) { return rec[L::X4 + (size_t)r * DK + d]; });
    prefetch_rows(x2pre, [&](int r, int d) { return rec[L::X2 + (size_t)r * DK + d]; });
    // dq = e^g o dQG + (dP o E) K = [diag(e^g) dO | dP o E] [S_in; K]  (dQG = dO S_in), and dq_r . q_r
    tgemm_blk<C, DK, DV + C, true, true>(
        stage, [&](int r, int kk) { return kk < DV ? eg[r] * orow4(r, kk) : ld4(dP + r * LN + kk - DV); },
        [&](int kk, int d) { return kk < DV ? ld4(Sin + (size_t)kk * DK + d) : krow4(kk - DV, d); },
        [&](const auto& acc, int rt0, int ct0) {
            each_elem(acc, rt0, ct0, [&](int r, int d, float x) {
                if (r < n) dq[tok0 * DK + (size_t)r * ks + d] = from_f32<T>(x);
            });
            put_rows(0, rt0, rowdot_pre(acc, qpre));
        });
    // dk = beta e^g o X4 + e^{g_last - g} o dKD + [(dP o E)^T | M | M^T] [Q; K; K]
    const float glast = gs[n - 1];
    tgemm_blk<C, DK, 3 * C, false, true>(stage,
        [&](int r, int kk) {
            return kk < C       ? ld4(dP + kk * LN + r)
                   : kk < 2 * C ? gather4([&](int u) { return Zm[(r + u) * LN + kk - C]; })
                                : ld4(Zm + (kk - 2 * C) * LN + r);
        },
        [&](int kk, int d) { return kk < C ? qrow4(kk, d) : krow4(kk % C, d); },
        [&](const auto& acc, int rt0, int ct0) {
            constexpr int CTK = DK / 16;
#pragma unroll
            for (int y = 0; y < CTK; ++y)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int r = 16 * rt0 + G4 + v, d = 16 * (ct0 + y) + c16;
                    if (r < n) {
                        const float val = bsg[r] * x4pre[y][v] + ekd[r] * x2pre[y][v] + acc[0][y][v];
                        dk[tok0 * DK + (size_t)r * ks + d] = from_f32<T>(val);
                    }
                }
        });
    __syncthreads();  // every row sum is in place
    // dbeta_r = sum_s dA_rs E_rs k_r.k_s + X3_r . v_r + e^{g_r} X4_r . k_r
    // dg_r = rowsum(dA o A) - colsum(dA o A + dP o P) + dq_r . q_r + beta_r e^{g_r} X4_r . k_r - dKD_r . KD_r
    //        (dq_r . q_r = e^{g_r} dQG_r . q_r + rowsum(dP o P); the last row also takes the chunk terms)
    if (tid < C) {
        const int r = tid;
        const float er = eg[r], tw = rowv[4][r], kd = ekd[r] * rowv[5][r];
        red[r] = rowv[2][r] + rowv[3][r] + er * tw;
        red[C + r] = bs[r] * rowv[2][r] - rowv[1][r] + rowv[0][r] + bs[r] * er * tw - kd;
        red[2 * C + r] = kd;
    }
    __syncthreads();
    if (tid < C) {  // wave 0, lane = row
        const int r = tid;
        const float kdsum = wave_sum(red[2 * C + r]);
        const float dss = wave_sum(r < DV / RW ? rec[L::DSS + r] : 0.0f);  // <dS_out, S_in> by row slice (reverse walk)
        float x = r < n ? red[C + r] : 0.0f;
        if (r == n - 1) x += kdsum + expf(glast) * dss;
        // d ln(alpha_s) = sum_{r >= s} dg_r over the real rows: a suffix scan across the wave
#pragma unroll
        for (int o = 1; o < C; o <<= 1) {
            const float y = __shfl_down(x, o, 64);
            if (r + o < C) x += y;
        }
        if (r < n) {
            const size_t t = ((size_t)P.b * Tlen + P.t0 + r) * H + P.h;
            dalpha[t] = x / alpha[t];
            dbeta[t] = red[r];
        }
    }
}

}  // namespace

size_t gdn_bwd_workspace_bytes(int B, int T, int H, int Dk, int Dv) {
    const size_t NC = (size_t)(T + C - 1) / C;
    size_t per;
    if (Dk == 64 && Dv == 64) per = WsLay<64, 64>::PER;
    else if (Dk == 64 && Dv == 128) per = WsLay<64, 128>::PER;
    else if (Dk == 128 && Dv == 64) per = WsLay<128, 64>::PER;
    else per = WsLay<128, 128>::PER;
    return (size_t)B * H * NC * per * sizeof(float);
}

template <typename T, int DK, int DV>
static void launch_bwd_typed(const GdnBwdArgs& a, hipStream_t s) {
    const int NC = (a.T + C - 1) / C;
    float* ws = (float*)a.workspace;
    const dim3 gc(NC, a.H, a.B), gr((unsigned)(DV / RW) * a.H * a.B);
    hipLaunchKernelGGL((gdn_bwd_prep<T, DK, DV>), gc, dim3(NT), 0, s, (const T*)a.k, (const T*)a.v, a.alpha, a.beta,
                       ws, a.T, a.H, NC);
    hipLaunchKernelGGL((gdn_bwd_walk<DK, DV, false>), gr, dim3(NTW), 0, s, a.init_state, nullptr, ws, a.H, NC);
    hipLaunchKernelGGL((gdn_bwd_pre<T, DK, DV>), gc, dim3(NT), 0, s, (const T*)a.q, (const T*)a.k, (const T*)a.dO, ws,
                       a.T, a.H, NC);
    hipLaunchKernelGGL((gdn_bwd_walk<DK, DV, true>), gr, dim3(NTW), 0, s, a.dS_final, a.d_init, ws, a.H, NC);
    hipLaunchKernelGGL((gdn_bwd_post<T, DK, DV>), gc, dim3(NT), 0, s, (const T*)a.q, (const T*)a.k, (const T*)a.v,
                       a.alpha, a.beta, (const T*)a.dO, (T*)a.dq, (T*)a.dk, (T*)a.dv, a.dalpha, a.dbeta, ws, a.T,
                       a.H, NC);
}

template <typename T>
static hipError_t launch_bwd_dims(const GdnBwdArgs& a, hipStream_t s) {
    if (a.Dk == 64 && a.Dv == 64) launch_bwd_typed<T, 64, 64>(a, s);
    else if (a.Dk == 64 && a.Dv == 128) launch_bwd_typed<T, 64, 128>(a, s);
    else if (a.Dk == 128 && a.Dv == 64) launch_bwd_typed<T, 128, 64>(a, s);
    else if (a.Dk == 128 && a.Dv == 128) launch_bwd_typed<T, 128, 128>(a, s);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_gdn_bwd(const GdnBwdArgs& a, hipStream_t stream) {
    return a.bf16_io ? launch_bwd_dims<bf16>(a, stream) : launch_bwd_dims<float>(a, stream);
}

}  // namespace atma

// Gated-delta memory, chunked prefill, for gfx950.
//
// Recurrence (ATMA paper, Section 3.3 equation; the paper's gamma_t is alpha_t here):
//     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t.
// Writing S_t = alpha_t S_{t-1} + delta_t k_t^T with delta_t = beta_t (v_t - alpha_t S_{t-1} k_t)
// and unrolling over a chunk of C tokens that enters with state S_in
// (g_r = sum_{s<=r} ln alpha_s inside the chunk) gives the exact chunk step
//     A     = strict_lower(diag(beta) (K K^T) o E),   E[r][s] = exp(g_r - g_s)
//     Tinv  = (I + A)^{-1}                                   (unit lower triangular)
//     W     = Tinv diag(beta e^g) K,   U = Tinv diag(beta) V
//     Delta = U - W S_in^T
//     O     = diag(e^g) Q S_in^T + lower_incl((Q K^T) o E) Delta
//     S_out = e^{g_last} S_in + (diag(e^{g_last - g}) K)^T Delta       (S^T form below)
// This file holds the derivation above and the exact (fp32-input) path; the bf16-input
// fast path lives in gdn_fwd_bf16.hip.  fp32 path, two kernels:
//   gdn_prep_f32  - one workgroup per (chunk, head, batch), all chunks in parallel: K K^T
//                   and Q K^T on fp32 MFMA, the blocked triangular inverse (substitution on
//                   the 16x16 diagonal blocks, fp32 MFMA for the off-diagonal blocks), W and
//                   U; writes W, U, P and g per chunk to the workspace.
//   gdn_carry_f32 - one workgroup per (64 state rows of Dv, head, batch); its four waves
//                   each own 16 state rows and walk the chunks in order, keeping S^T in
//                   fp32 MFMA accumulators; the next chunk's tiles are prefetched into
//                   registers while the current one is computed.
// Used where 1e-4 agreement with the fp64 recurrence is required.
#include "gdn_common.hpp"
#include "launch.hpp"

namespace atma {
namespace {

using gdn::C;
using gdn::NT;
using gdn::TileRegs;

template <typename T> struct Pad;
template <> struct Pad<bf16> { static constexpr int v = 8; };   // keeps 16-byte row alignment
template <> struct Pad<float> { static constexpr int v = 4; };

// Per-chunk workspace record: W [C][DK], U [C][DV], P [C][C] (element type T), g [C] fp32.
template <typename T, int DK, int DV> struct Rec {
    static constexpr size_t W = 0;
    static constexpr size_t U = W + (size_t)C * DK * sizeof(T);
    static constexpr size_t P = U + (size_t)C * DV * sizeof(T);
    static constexpr size_t G = P + (size_t)C * C * sizeof(T);
    static constexpr size_t BYTES = G + C * sizeof(float);
};

// ------------------------------------------------------------------------------------
// chunk preparation
// ------------------------------------------------------------------------------------
template <typename T, int DK, int DV>
struct PrepSmem {
    static constexpr int LDK = DK + Pad<T>::v, LDV = DV + Pad<T>::v, LDA = C + 1;
    T Ks[C * LDK];
    T Qs[C * LDK];
    T Vs[C * LDV];
    float Am[C * LDA];
    float Tm[C * LDA];
    float Gs[C];
    float Bs[C];
};

template <typename T, int DK, int DV>
__global__ __launch_bounds__(NT) void gdn_prep_f32(const T* __restrict__ q, const T* __restrict__ k,
                                                     const T* __restrict__ v, const float* __restrict__ alpha,
                                                     const float* __restrict__ beta, char* __restrict__ ws,
                                                     int Tlen, int H) {
    using S = PrepSmem<T, DK, DV>;
    using R = Rec<T, DK, DV>;
    constexpr int LDK = S::LDK, LDV = S::LDV, LDA = S::LDA;
    extern __shared__ __align__(16) char smem_raw[];
    S& sm = *reinterpret_cast<S*>(smem_raw);

    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int NC = gridDim.x;
    const int t0 = c * C;
    const int n = min(C, Tlen - t0);
    const int lane = lane_id(), w = wave_id(), G = lane >> 4, l16 = lane & 15;
    const size_t tok0 = ((size_t)b * Tlen + t0) * H + h;
    char* rec = ws + (((size_t)b * H + h) * NC + c) * R::BYTES;

    // ---- load the chunk ---------------------------------------------------------
    {
        TileRegs<T, C, DK> kr, qr;
        TileRegs<T, C, DV> vr;
        kr.load(k + tok0 * DK, (size_t)H * DK, n);
        qr.load(q + tok0 * DK, (size_t)H * DK, n);
        vr.load(v + tok0 * DV, (size_t)H * DV, n);
        kr.template store<LDK>(sm.Ks);
        qr.template store<LDK>(sm.Qs);
        vr.template store<LDV>(sm.Vs);
    }
    if (w == 0) {
        const bool ok = lane < n;
        float la = ok ? __logf(alpha[tok0 + (size_t)lane * H]) : 0.0f;
        const float be = ok ? beta[tok0 + (size_t)lane * H] : 0.0f;
        // inclusive prefix sum of ln(alpha) over the chunk
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_up(la, o, 64);
            if (lane >= o) la += y;
        }
        sm.Gs[lane] = la;
        sm.Bs[lane] = be;
        ((float*)(rec + R::G))[lane] = la;
    }
    __syncthreads();

    // ---- K K^T and Q K^T tiles: A (strict lower, fp32, LDS) and P (lower incl., workspace)
    T* Pg = (T*)(rec + R::P);
    for (int ti = w; ti < 16; ti += 4) {
        // lower tiles first (0..9), then the six upper tiles that are all zero
        int i, j;
        if (ti < 10) {
            i = (ti >= 6) ? 3 : (ti >= 3) ? 2 : (ti >= 1) ? 1 : 0;
            j = ti - i * (i + 1) / 2;
        } else {
            const int u = ti - 10;  // (0,1),(0,2),(0,3),(1,2),(1,3),(2,3)
            i = (u < 3) ? 0 : (u < 5) ? 1 : 2;
            j = (u < 3) ? u + 1 : (u < 5) ? u - 1 : 3;
        }
        f32x4 kk = {0, 0, 0, 0}, qk = {0, 0, 0, 0};
        if (ti < 10) {
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                Frag<T> a, bq, bk;
                load_frag_rows(bk, sm.Ks, LDK, 16 * j + l16, 32 * kb);
                load_frag_rows(a, sm.Ks, LDK, 16 * i + l16, 32 * kb);
                load_frag_rows(bq, sm.Qs, LDK, 16 * i + l16, 32 * kb);
                mma(kk, a, bk);
                mma(qk, bq, bk);
            }
        }
        const int s = 16 * j + l16;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int r = 16 * i + 4 * G + x;
            const float e = (s <= r) ? __expf(sm.Gs[r] - sm.Gs[s]) : 0.0f;
            sm.Am[r * LDA + s] = (s < r) ? sm.Bs[r] * e * kk[x] : 0.0f;
            Pg[r * C + s] = from_f32<T>(e * qk[x]);
        }
    }
    __syncthreads();

    // ---- Tinv = (I + A)^{-1}: 16x16 diagonal blocks by forward substitution -------
    if (w == 0) {
        const int blk = lane >> 4, col = l16, o = 16 * blk;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == col) ? 1.0f : 0.0f;
#pragma unroll
            for (int s2 = 0; s2 < r; ++s2) acc -= sm.Am[(o + r) * LDA + o + s2] * x[s2];
            x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.Tm[(o + r) * LDA + o + col] = x[r];
    } else {
        // zero the strictly upper blocks
        for (int i = threadIdx.x - 64; i < 6 * 256; i += NT - 64) {
            const int u = i >> 8, e = i & 255;
            const int bi = (u < 3) ? 0 : (u < 5) ? 1 : 2;
            const int bj = (u < 3) ? u + 1 : (u < 5) ? u - 1 : 3;
            sm.Tm[(16 * bi + (e >> 4)) * LDA + 16 * bj + (e & 15)] = 0.0f;
        }
    }
    __syncthreads();
    // off-diagonal blocks by block distance d: Tinv_ij = -Tinv_ii sum_{m=j}^{i-1} A_im Tinv_mj
    for (int d = 1; d < 4; ++d) {
        if (w < 4 - d) {
            const int j = w, i = w + d;
            f32x4 acc = {0, 0, 0, 0};
            for (int m = j; m < i; ++m) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float a = sm.Am[(16 * i + l16) * LDA + 16 * m + 4 * G + e];
                    const float bb = sm.Tm[(16 * m + 4 * G + e) * LDA + 16 * j + l16];
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bb, acc, 0, 0, 0);
                }
            }
            f32x4 y = {0, 0, 0, 0};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = sm.Tm[(16 * i + l16) * LDA + 16 * i + 4 * G + e];
                y = __builtin_amdgcn_mfma_f32_16x16x4f32(a, acc[e], y, 0, 0, 0);
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) sm.Tm[(16 * i + 4 * G + x) * LDA + 16 * j + l16] = -y[x];
        }
        __syncthreads();
    }

    // ---- W = Tinv diag(beta e^g) K  and  U = Tinv diag(beta) V ----------------------
    {
        const int i = w;  // row tile
        const int nkb = (i < 2) ? 1 : 2;
        Frag<T> aw[2], au[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int s = 32 * kb + kmap(G, e);
                const float t = sm.Tm[(16 * i + l16) * LDA + s];
                const float bs = sm.Bs[s];
                aw[kb].set(e, t * bs * __expf(sm.Gs[s]));
                au[kb].set(e, t * bs);
            }
        }
        T* Wg = (T*)(rec + R::W);
        T* Ug = (T*)(rec + R::U);
#pragma unroll
        for (int ct = 0; ct < DK / 16; ++ct) {
            f32x4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (kb < nkb) {
                    Frag<T> bk;
                    load_frag_cols(bk, sm.Ks, LDK, 16 * ct + l16, 32 * kb);
                    mma(acc, aw[kb], bk);
                }
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) Wg[(16 * i + 4 * G + x) * DK + 16 * ct + l16] = from_f32<T>(acc[x]);
        }
#pragma unroll
        for (int ct = 0; ct < DV / 16; ++ct) {
            f32x4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (kb < nkb) {
                    Frag<T> bv;
                    load_frag_cols(bv, sm.Vs, LDV, 16 * ct + l16, 32 * kb);
                    mma(acc, au[kb], bv);
                }
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) Ug[(16 * i + 4 * G + x) * DV + 16 * ct + l16] = from_f32<T>(acc[x]);
        }
    }
}

// ------------------------------------------------------------------------------------
// sequential carry over chunks
// ------------------------------------------------------------------------------------
constexpr int SLICE = 64;  // state rows (of Dv) per workgroup; 16 per wave

template <typename T, int DK>
struct CarrySmem {
    static constexpr int LDK = DK + Pad<T>::v, LDKT = C + Pad<T>::v, LDP = C + Pad<T>::v,
                         LDU = SLICE + Pad<T>::v;
    T Ws[C * LDK];
    T Qs[C * LDK];
    T Kt[DK * LDKT];
    T Ps[C * LDP];
    T Us[C * LDU];
    float Gs[C];
};

template <typename T, int DK, int DV>
__global__ __launch_bounds__(NT) void gdn_carry_f32(const T* __restrict__ q, const T* __restrict__ k,
                                                      const char* __restrict__ ws,
                                                      const float* init_state, T* __restrict__ o,
                                                      float* final_state, int Tlen, int H) {
    using S = CarrySmem<T, DK>;
    using R = Rec<T, DK, DV>;
    constexpr int LDK = S::LDK, LDKT = S::LDKT, LDP = S::LDP, LDU = S::LDU;
    constexpr int NKT = DK / 16;  // accumulator tiles of S^T per wave
    extern __shared__ __align__(16) char smem_raw[];
    S& sm = *reinterpret_cast<S*>(smem_raw);

    const int h = blockIdx.y, b = blockIdx.z;
    const int lane = lane_id(), w = wave_id(), G = lane >> 4, l16 = lane & 15;
    const int col0 = blockIdx.x * SLICE;       // first state row (Dv index) of this workgroup
    const int row = col0 + 16 * w + l16;      // state row this lane's accumulators hold
    const int NC = (Tlen + C - 1) / C;
    const char* rec0 = ws + ((size_t)b * H + h) * NC * R::BYTES;

    // S^T tiles: st[t][x] = S[row][16 t + 4 G + x]
    f32x4 st[NKT];
    const size_t srow = (((size_t)b * H + h) * DV + row) * DK;
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
        if (init_state) st[t] = *(const f32x4*)(init_state + srow + 16 * t + 4 * G);
        else st[t] = f32x4{0, 0, 0, 0};
    }

    TileRegs<T, C, DK> wr, qr, kr;
    TileRegs<T, C, C> pr;
    TileRegs<T, C, SLICE> ur;
    float gr = 0.0f;
    auto prefetch = [&](int c) {
        const char* rec = rec0 + (size_t)c * R::BYTES;
        const int t0 = c * C, n = min(C, Tlen - t0);
        const size_t tok0 = ((size_t)b * Tlen + t0) * H + h;
        wr.load((const T*)(rec + R::W), DK, C);
        pr.load((const T*)(rec + R::P), C, C);
        ur.load((const T*)(rec + R::U) + col0, DV, C);
        qr.load(q + tok0 * DK, (size_t)H * DK, n);
        kr.load(k + tok0 * DK, (size_t)H * DK, n);
        if (threadIdx.x < C) gr = ((const float*)(rec + R::G))[threadIdx.x];
    };
    prefetch(0);

    for (int c = 0; c < NC; ++c) {
        __syncthreads();  // previous chunk's readers are done
        wr.template store<LDK>(sm.Ws);
        qr.template store<LDK>(sm.Qs);
        kr.template store_t<LDKT>(sm.Kt);
        pr.template store<LDP>(sm.Ps);
        ur.template store<LDU>(sm.Us);
        if (threadIdx.x < C) sm.Gs[threadIdx.x] = gr;
        __syncthreads();
        if (c + 1 < NC) prefetch(c + 1);

        const int t0 = c * C, n = min(C, Tlen - t0);
        // S_in^T as B fragments (reduction over Dk)
        Frag<T> sf[DK / 32];
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) acc_to_frag(sf[kb], st[2 * kb], st[2 * kb + 1]);

        // Delta = U - W S_in^T  (rows = chunk positions, cols = this wave's 16 state rows)
        f32x4 dl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                Frag<T> a;
                load_frag_rows(a, sm.Ws, LDK, 16 * i + l16, 32 * kb);
                mma(acc, a, sf[kb]);
            }
#pragma unroll
            for (int x = 0; x < 4; ++x)
                dl[i][x] = to_f32(sm.Us[(16 * i + 4 * G + x) * LDU + 16 * w + l16]) - acc[x];
        }
        // O = diag(e^g) Q S_in^T + P Delta
        Frag<T> df[2];
        acc_to_frag(df[0], dl[0], dl[1]);
        acc_to_frag(df[1], dl[2], dl[3]);
        const float glast = sm.Gs[C - 1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                Frag<T> a;
                load_frag_rows(a, sm.Qs, LDK, 16 * i + l16, 32 * kb);
                mma(acc, a, sf[kb]);
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) acc[x] *= __expf(sm.Gs[16 * i + 4 * G + x]);
#pragma unroll
            for (int kb = 0; kb < (i < 2 ? 1 : 2); ++kb) {
                Frag<T> a;
                load_frag_rows(a, sm.Ps, LDP, 16 * i + l16, 32 * kb);
                mma(acc, a, df[kb]);
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int r = 16 * i + 4 * G + x;
                if (r < n) o[(((size_t)b * Tlen + t0 + r) * H + h) * DV + row] = from_f32<T>(acc[x]);
            }
        }
        // S_out^T = e^{g_last} S_in^T + K^T diag(e^{g_last - g}) Delta
        Frag<T> ddf[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const float d0 = dl[2 * kb][x] * __expf(glast - sm.Gs[32 * kb + 4 * G + x]);
                const float d1 = dl[2 * kb + 1][x] * __expf(glast - sm.Gs[32 * kb + 16 + 4 * G + x]);
                ddf[kb].set(x, d0);
                ddf[kb].set(x + 4, d1);
            }
        }
        const float eg = __expf(glast);
#pragma unroll
        for (int t = 0; t < NKT; ++t) {
            st[t] *= eg;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                Frag<T> a;
                load_frag_rows(a, sm.Kt, LDKT, 16 * t + l16, 32 * kb);
                mma(st[t], a, ddf[kb]);
            }
        }
    }
    if (final_state) {
#pragma unroll
        for (int t = 0; t < NKT; ++t) *(f32x4*)(final_state + srow + 16 * t + 4 * G) = st[t];
    }
}

template <int DK, int DV>
hipError_t launch_f32(const GdnFwdArgs& a, hipStream_t stream) {
    const int NC = (a.T + C - 1) / C;
    const size_t prep_smem = sizeof(PrepSmem<float, DK, DV>);
    const size_t carry_smem = sizeof(CarrySmem<float, DK>);
    static const hipError_t attr = [&] {
        hipError_t e = ensure_lds_limit(gdn_prep_f32<float, DK, DV>, prep_smem);
        return e != hipSuccess ? e : ensure_lds_limit(gdn_carry_f32<float, DK, DV>, carry_smem);
    }();
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((gdn_prep_f32<float, DK, DV>), dim3(NC, a.H, a.B), dim3(NT), prep_smem, stream,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, a.alpha, a.beta, (char*)a.workspace,
                       a.T, a.H);
    hipLaunchKernelGGL((gdn_carry_f32<float, DK, DV>), dim3(DV / SLICE, a.H, a.B), dim3(NT), carry_smem, stream,
                       (const float*)a.q, (const float*)a.k, (const char*)a.workspace, a.init_state, (float*)a.o,
                       a.final_state, a.T, a.H);
    return hipGetLastError();
}

}  // namespace

size_t gdn_fwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, bool bf16_io) {
    if (bf16_io) return gdn_bf16_workspace_bytes(B, T, H, Dk, Dv);
    const size_t nc = (size_t)((T + C - 1) / C);
    return (size_t)B * H * nc * ((size_t)C * Dk * 4 + (size_t)C * Dv * 4 + (size_t)C * C * 4 + C * sizeof(float));
}

hipError_t launch_gdn_fwd(const GdnFwdArgs& a, hipStream_t stream) {
    if (a.bf16_io) return launch_gdn_bf16(a, stream);
#define ATMA_GDN_CASE(DKK, DVV) \
    if (a.Dk == DKK && a.Dv == DVV) return launch_f32<DKK, DVV>(a, stream);
    ATMA_GDN_CASE(64, 64) ATMA_GDN_CASE(64, 128) ATMA_GDN_CASE(128, 64) ATMA_GDN_CASE(128, 128)
#undef ATMA_GDN_CASE
    return hipErrorInvalidValue;
}

}  // namespace atma

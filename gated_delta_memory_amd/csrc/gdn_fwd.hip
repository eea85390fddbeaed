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
// Each path has two kernels:
//   prep  - one workgroup per (chunk, head, batch), all chunks in parallel: K K^T and Q K^T
//           on MFMA, the blocked triangular inverse in fp32 (substitution on the 16x16
//           diagonal blocks, fp32 MFMA for the off-diagonal blocks), W and U on MFMA.
//   carry - walks the chunks of one (batch, head) in order; the state is held transposed in
//           fp32 MFMA accumulators for the whole sequence, 16 state rows per wave.
// bf16 inputs (fast path): prep writes, per chunk, one record of fp16 MFMA operands already
//   laid out in the carry kernel's swizzled LDS order -- W, diag(e^g) Q, the decayed K
//   transposed, P and U -- with W and U formed from an fp32-accurate hi/lo bf16 split of
//   Tinv.  The carry kernel streams each record into a double-buffered LDS stage with
//   direct global->LDS copies while the previous chunk is computed, so its sequential loop
//   holds only MFMAs, the fp32 state update and the output store.  fp16 operands (11-bit
//   mantissa) keep the chunked result within a few 1e-3 of the fp64 recurrence; they need
//   |v| and the state entries below 2^15.
// fp32 inputs (exact path): the same algebra with fp32 operands on fp32 MFMA, used where
//   1e-4 agreement with the fp64 recurrence is required.
#include "atma_device.hpp"
#include "launch.hpp"

namespace atma {
namespace {

constexpr int C = 64;  // chunk length
constexpr int NT = 256;

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

// Copies a ROWS x COLS tile (row stride `ld` elements in global memory) through
// registers into LDS (row stride LDS_LD).  Rows >= nrows read as zero.
template <typename T, int ROWS, int COLS>
struct TileRegs {
    static constexpr int VEC = 16 / sizeof(T);
    static constexpr int NVEC = ROWS * COLS / VEC;
    static constexpr int PER = (NVEC + NT - 1) / NT;
    u32x4 r[PER];
    __device__ __forceinline__ void load(const T* g, size_t ld, int nrows) {
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int i = threadIdx.x + m * NT;
            const int row = i / (COLS / VEC), cv = i % (COLS / VEC);
            u32x4 x = {0u, 0u, 0u, 0u};
            if (i < NVEC && row < nrows) x = *(const u32x4*)(g + (size_t)row * ld + cv * VEC);
            r[m] = x;
        }
    }
    template <int LDS_LD>
    __device__ __forceinline__ void store(T* s) const {
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int i = threadIdx.x + m * NT;
            if (i < NVEC) {
                const int row = i / (COLS / VEC), cv = i % (COLS / VEC);
                *(u32x4*)(s + row * LDS_LD + cv * VEC) = r[m];
            }
        }
    }
    // Transposed store: element (row, col) goes to s[col * LDS_LD + row].
    template <int LDS_LD>
    __device__ __forceinline__ void store_t(T* s) const {
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int i = threadIdx.x + m * NT;
            if (i < NVEC) {
                const int row = i / (COLS / VEC), cv = i % (COLS / VEC);
                const T* e = (const T*)&r[m];
#pragma unroll
                for (int x = 0; x < VEC; ++x) s[(cv * VEC + x) * LDS_LD + row] = e[x];
            }
        }
    }
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

// ====================================================================================
// bf16 inputs: fp16-staged records
// ====================================================================================
// Record of one chunk (fp16, every tile row-major with XOR-swizzled 16-byte chunks):
//   W  [C][DK]   Tinv diag(beta e^g) K
//   QG [C][DK]   diag(e^g) Q
//   KDT[DK][C]   (diag(e^{g_last - g}) K)^T
//   P  [C][C]    lower_incl((Q K^T) o E)
//   U  DV/64 slices of [C][64]   Tinv diag(beta) V
// The carry workgroup that owns state rows [64 s, 64 s + 64) copies W..P plus U slice s.
template <int DK, int DV> struct RecH {
    static constexpr int RBK = DK * 2;  // bytes per W / QG row
    static constexpr size_t W = 0;
    static constexpr size_t QG = W + (size_t)C * DK * 2;
    static constexpr size_t KDT = QG + (size_t)C * DK * 2;
    static constexpr size_t P = KDT + (size_t)DK * C * 2;
    static constexpr size_t U = P + (size_t)C * C * 2;
    static constexpr size_t USLICE = (size_t)C * 64 * 2;
    static constexpr size_t BYTES = U + (size_t)(DV / 64) * USLICE;
    static constexpr size_t STAGE = U + USLICE;  // bytes one carry workgroup streams per chunk
};

template <int DK, int DV>
struct PrepSmemH {
    static constexpr int LDK = DK + 8, LDV = DV + 8, LDA = C + 1;
    bf16 Ks[C * LDK];
    bf16 Qs[C * LDK];  // later: W staging (fp16, record layout)
    bf16 Vs[C * LDV];
    float Am[C * LDA];  // later: U staging (fp16, record layout)
    float Tm[C * LDA];  // first: P staging (fp16, record layout)
    float Gs[C];
    float Bs[C];
};

// Copies `bytes` (multiple of 16) from LDS to global memory with 16-byte stores.
__device__ __forceinline__ void copy_out(char* __restrict__ dst, const char* src, int bytes) {
    for (int i = threadIdx.x * 16; i < bytes; i += NT * 16) *(u32x4*)(dst + i) = *(const u32x4*)(src + i);
}

template <int DK, int DV>
__global__ __launch_bounds__(NT) void gdn_prep_h(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                 const bf16* __restrict__ v, const float* __restrict__ alpha,
                                                 const float* __restrict__ beta, char* __restrict__ ws,
                                                 float* __restrict__ egl_out, int Tlen, int H) {
    using S = PrepSmemH<DK, DV>;
    using R = RecH<DK, DV>;
    constexpr int LDK = S::LDK, LDV = S::LDV, LDA = S::LDA, RBK = R::RBK;
    extern __shared__ __align__(16) char smem_raw[];
    S& sm = *reinterpret_cast<S*>(smem_raw);

    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int NC = gridDim.x;
    const int t0 = c * C;
    const int n = min(C, Tlen - t0);
    const int lane = lane_id(), w = wave_id(), G = lane >> 4, l16 = lane & 15;
    const size_t tok0 = ((size_t)b * Tlen + t0) * H + h;
    const size_t chunk_id = ((size_t)b * H + h) * NC + c;
    char* rec = ws + chunk_id * R::BYTES;

    // ---- A: load the chunk, cumulative log decay ------------------------------------
    {
        TileRegs<bf16, C, DK> kr, qr;
        TileRegs<bf16, C, DV> vr;
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
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_up(la, o, 64);
            if (lane >= o) la += y;
        }
        sm.Gs[lane] = la;
        sm.Bs[lane] = be;
        if (lane == C - 1) egl_out[chunk_id] = __expf(la);
    }
    __syncthreads();

    // ---- B: A (strict lower, fp32) and P (lower incl., fp16 staged in Tm) ----------------
    char* pstage = (char*)sm.Tm;
    for (int ti = w; ti < 16; ti += 4) {
        int i, j;
        if (ti < 10) {
            i = (ti >= 6) ? 3 : (ti >= 3) ? 2 : (ti >= 1) ? 1 : 0;
            j = ti - i * (i + 1) / 2;
        } else {
            const int u = ti - 10;
            i = (u < 3) ? 0 : (u < 5) ? 1 : 2;
            j = (u < 3) ? u + 1 : (u < 5) ? u - 1 : 3;
        }
        f32x4 kk = {0, 0, 0, 0}, qk = {0, 0, 0, 0};
        if (ti < 10) {
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                Frag<bf16> a, bq, bk;
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
            *(half*)(pstage + swz16<128>(r, s)) = (half)(e * qk[x]);
        }
    }
    __syncthreads();
    copy_out(rec + R::P, pstage, C * C * 2);

    // ---- C: diag(e^g) Q and the decayed K^T, straight to the record ----------------------
    for (int id = threadIdx.x; id < C * DK / 8; id += NT) {
        const int r = id / (DK / 8), cc = id % (DK / 8);
        const float e = __expf(sm.Gs[r]);
        const bf16x8 x = *(const bf16x8*)&sm.Qs[r * LDK + 8 * cc];
        f16x8 y;
#pragma unroll
        for (int t = 0; t < 8; ++t) y[t] = (half)((float)x[t] * e);
        *(f16x8*)(rec + R::QG + swz16<RBK>(r, 8 * cc)) = y;
    }
    {
        // lane i of 16-lane group g gets K[pc .. pc + 7][16 cg + i] with two transpose reads
        const float glast = sm.Gs[C - 1];
        for (int combo = w * 4 + G; combo < (DK / 16) * (C / 8); combo += 16) {
            const int cg = combo % (DK / 16), pc = 8 * (combo / (DK / 16));
            const char* kb_ = (const char*)sm.Ks;
            const int col = 16 * cg + 4 * (l16 & 3);
            const s16x4 r0 = tr_read_b16(kb_ + ((pc + (l16 >> 2)) * LDK + col) * 2);
            const s16x4 r1 = tr_read_b16(kb_ + ((pc + 4 + (l16 >> 2)) * LDK + col) * 2);
            const bf16x4 k0 = __builtin_bit_cast(bf16x4, r0), k1 = __builtin_bit_cast(bf16x4, r1);
            f16x8 y;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                y[t] = (half)((float)k0[t] * __expf(glast - sm.Gs[pc + t]));
                y[t + 4] = (half)((float)k1[t] * __expf(glast - sm.Gs[pc + 4 + t]));
            }
            *(f16x8*)(rec + R::KDT + swz16<128>(16 * cg + l16, pc)) = y;
        }
    }
    __syncthreads();  // P staging (Tm) fully copied before Tinv overwrites it

    // ---- D: Tinv = (I + A)^{-1} ---------------------------------------------------------
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
        for (int i = threadIdx.x - 64; i < 6 * 256; i += NT - 64) {
            const int u = i >> 8, e = i & 255;
            const int bi = (u < 3) ? 0 : (u < 5) ? 1 : 2;
            const int bj = (u < 3) ? u + 1 : (u < 5) ? u - 1 : 3;
            sm.Tm[(16 * bi + (e >> 4)) * LDA + 16 * bj + (e & 15)] = 0.0f;
        }
    }
    __syncthreads();
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

    // ---- E: W and U with an fp32-accurate hi/lo bf16 split of the scaled Tinv rows -------
    {
        const int i = w;
        const int nkb = (i < 2) ? 1 : 2;
        Frag<bf16> wh[2], wl[2], uh[2], ul[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int s = 32 * kb + kmap(G, e);
                const float t = sm.Tm[(16 * i + l16) * LDA + s];
                const float tw = t * sm.Bs[s] * __expf(sm.Gs[s]);
                const float tu = t * sm.Bs[s];
                const bf16 hw = (bf16)tw, hu = (bf16)tu;
                wh[kb].set_raw(e, hw);
                wl[kb].set(e, tw - (float)hw);
                uh[kb].set_raw(e, hu);
                ul[kb].set(e, tu - (float)hu);
            }
        }
        char* wstage = (char*)sm.Qs;
        char* ustage = (char*)sm.Am;
        // B fragments of K / V (rows = chunk positions) by transpose reads
        auto bfrag = [&](const bf16* tile, int ld, int ct, int kb) {
            const char* base = (const char*)tile;
            const int col = 16 * ct + 4 * (l16 & 3);
            const s16x4 r0 = tr_read_b16(base + ((32 * kb + 4 * G + (l16 >> 2)) * ld + col) * 2);
            const s16x4 r1 = tr_read_b16(base + ((32 * kb + 16 + 4 * G + (l16 >> 2)) * ld + col) * 2);
            Frag<bf16> f;
            f.v = __builtin_shufflevector(__builtin_bit_cast(bf16x4, r0), __builtin_bit_cast(bf16x4, r1), 0, 1, 2, 3,
                                          4, 5, 6, 7);
            return f;
        };
        __syncthreads();  // Qs and Am are free: every wave is past phase C and D
#pragma unroll
        for (int ct = 0; ct < DK / 16; ++ct) {
            f32x4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (kb < nkb) {
                    const Frag<bf16> bk = bfrag(sm.Ks, LDK, ct, kb);
                    mma(acc, wh[kb], bk);
                    mma(acc, wl[kb], bk);
                }
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) *(half*)(wstage + swz16<RBK>(16 * i + 4 * G + x, 16 * ct + l16)) = (half)acc[x];
        }
#pragma unroll
        for (int ct = 0; ct < DV / 16; ++ct) {
            f32x4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (kb < nkb) {
                    const Frag<bf16> bv = bfrag(sm.Vs, LDV, ct, kb);
                    mma(acc, uh[kb], bv);
                    mma(acc, ul[kb], bv);
                }
            }
            const int sl = (16 * ct) / 64, cl = (16 * ct) % 64 + l16;
#pragma unroll
            for (int x = 0; x < 4; ++x)
                *(half*)(ustage + sl * R::USLICE + swz16<128>(16 * i + 4 * G + x, cl)) = (half)acc[x];
        }
        __syncthreads();
        copy_out(rec + R::W, wstage, C * DK * 2);
        copy_out(rec + R::U, ustage, C * DV * 2);
    }
}

// ------------------------------------------------------------------------------------
// Separate LDS objects per stage: the compiler's wait-count analysis can then tell the
// stage being read from the stage the asynchronous copy is filling, so reads of the current
// chunk do not wait for the copy of the next one.
constexpr int kStageMax = 65536;
__shared__ __align__(16) char g_stage0[kStageMax];
__shared__ __align__(16) char g_stage1[kStageMax];
__shared__ __align__(16) char g_ostage0[C * 72 * 2];
__shared__ __align__(16) char g_ostage1[C * 72 * 2];

template <int DK, int DV>
struct CarryH {
    using R = RecH<DK, DV>;
    static constexpr int RBK = R::RBK, NKT = DK / 16, NCH = (int)R::STAGE / 16;
    static_assert(R::STAGE <= kStageMax, "stage too large");
    static_assert(NCH % NT == 0, "stage must be a whole number of 16-byte rounds");

    const char* rec0;
    const float* egl;
    bf16* o;
    int Tlen, H, NC, b, h, sl, col0;

    __device__ __forceinline__ void issue(int c, char* dst) const {
        const int w = wave_id();
        const char* src = rec0 + (size_t)c * R::BYTES;
#pragma unroll
        for (int m = 0; m < NCH / NT; ++m) {
            const int ch = m * NT + threadIdx.x;
            const size_t off =
                (size_t)ch * 16 < R::U ? (size_t)ch * 16 : R::U + sl * R::USLICE + ((size_t)ch * 16 - R::U);
            __builtin_amdgcn_global_load_lds((const void*)(src + off), (void*)(dst + (m * NT + w * 64) * 16), 16, 0, 0);
        }
    }
    __device__ __forceinline__ void flush(int c, const char* src) const {
        const int t0 = c * C, n = min(C, Tlen - t0);
        for (int id = threadIdx.x; id < C * 8; id += NT) {
            const int r = id >> 3, cc = id & 7;
            if (r < n)
                *(u32x4*)(o + (((size_t)b * Tlen + t0 + r) * H + h) * DV + col0 + 8 * cc) =
                    *(const u32x4*)(src + (r * 72 + 8 * cc) * 2);
        }
    }
    // one chunk: consume stage `sW`, write the output tile to `os`
    __device__ __forceinline__ void step(int c, const char* sW, char* os, f32x4* st) const {
        const int lane = lane_id(), w = wave_id(), G = lane >> 4, l16 = lane & 15;
        const char* sQ = sW + R::QG;
        const char* sK = sW + R::KDT;
        const char* sP = sW + R::P;
        const char* sU = sW + R::U;
        const float eg = egl[c];
        Frag<half> sf[DK / 32];
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) acc_to_frag(sf[kb], st[2 * kb], st[2 * kb + 1]);
        // Delta = U - W S_in^T
        f32x4 dl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                Frag<half> a;
                a.v = frag_swz_f16<RBK>(sW, 16 * i + l16, 32 * kb);
                mma(acc, a, sf[kb]);
            }
            const s16x4 ur = tr_read_b16(sU + swz16<128>(16 * i + 4 * G + (l16 >> 2), 16 * w + 4 * (l16 & 3)));
            const f16x4 u = __builtin_bit_cast(f16x4, ur);
#pragma unroll
            for (int x = 0; x < 4; ++x) dl[i][x] = (float)u[x] - acc[x];
        }
        Frag<half> df[2];
        acc_to_frag(df[0], dl[0], dl[1]);
        acc_to_frag(df[1], dl[2], dl[3]);
        // S_out^T = e^{g_last} S_in^T + KD^T Delta
#pragma unroll
        for (int t = 0; t < NKT; ++t) {
            st[t] *= eg;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                Frag<half> a;
                a.v = frag_swz_f16<128>(sK, 16 * t + l16, 32 * kb);
                mma(st[t], a, df[kb]);
            }
        }
        // O = QG S_in^T + P Delta -> bf16 staging tile
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                Frag<half> a;
                a.v = frag_swz_f16<RBK>(sQ, 16 * i + l16, 32 * kb);
                mma(acc, a, sf[kb]);
            }
#pragma unroll
            for (int kb = 0; kb < (i < 2 ? 1 : 2); ++kb) {
                Frag<half> a;
                a.v = frag_swz_f16<128>(sP, 16 * i + l16, 32 * kb);
                mma(acc, a, df[kb]);
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) *(bf16*)(os + ((16 * i + 4 * G + x) * 72 + 16 * w + l16) * 2) = (bf16)acc[x];
        }
    }
};

// vmcnt(0), other counters untouched (gfx9 s_waitcnt encoding)
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int DK, int DV>
__global__ __launch_bounds__(NT, 1) void gdn_carry_h(const char* __restrict__ ws, const float* __restrict__ egl_arr,
                                                     const float* init_state, bf16* __restrict__ o,
                                                     float* final_state, int Tlen, int H) {
    using R = RecH<DK, DV>;
    constexpr int NKT = DK / 16;
    const int sl = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = lane_id(), w = wave_id(), G = lane >> 4, l16 = lane & 15;
    const int NC = (Tlen + C - 1) / C;
    const size_t bh = (size_t)b * H + h;
    const CarryH<DK, DV> k{ws + bh * NC * R::BYTES, egl_arr + bh * NC, o, Tlen, H, NC, b, h, sl, sl * 64};
    const int row = k.col0 + 16 * w + l16;  // state row held by this lane's accumulators

    f32x4 st[NKT];  // st[t][x] = S[row][16 t + 4 G + x]
    const size_t srow = (bh * DV + row) * DK;
#pragma unroll
    for (int t = 0; t < NKT; ++t)
        st[t] = init_state ? *(const f32x4*)(init_state + srow + 16 * t + 4 * G) : f32x4{0, 0, 0, 0};

    k.issue(0, g_stage0);
    for (int c = 0; c < NC; c += 2) {
        // even chunk: read stage0 / ostage0, fill stage1
        wait_vmem_all();
        __syncthreads();
        if (c + 1 < NC) k.issue(c + 1, g_stage1);
        if (c > 0) k.flush(c - 1, g_ostage1);
        k.step(c, g_stage0, g_ostage0, st);
        if (c + 1 >= NC) break;
        // odd chunk: read stage1 / ostage1, fill stage0
        wait_vmem_all();
        __syncthreads();
        if (c + 2 < NC) k.issue(c + 2, g_stage0);
        k.flush(c, g_ostage0);
        k.step(c + 1, g_stage1, g_ostage1, st);
    }
    __syncthreads();
    k.flush(NC - 1, (NC - 1) & 1 ? g_ostage1 : g_ostage0);
    if (final_state) {
#pragma unroll
        for (int t = 0; t < NKT; ++t) *(f32x4*)(final_state + srow + 16 * t + 4 * G) = st[t];
    }
}

template <int DK, int DV>
hipError_t launch_h(const GdnFwdArgs& a, hipStream_t stream) {
    using R = RecH<DK, DV>;
    const int NC = (a.T + C - 1) / C;
    const size_t prep_smem = sizeof(PrepSmemH<DK, DV>);
    static const hipError_t attr = ensure_lds_limit(gdn_prep_h<DK, DV>, prep_smem);
    if (attr != hipSuccess) return attr;
    char* ws = (char*)a.workspace;
    float* egl = (float*)(ws + (size_t)a.B * a.H * NC * R::BYTES);
    hipLaunchKernelGGL((gdn_prep_h<DK, DV>), dim3(NC, a.H, a.B), dim3(NT), prep_smem, stream, (const bf16*)a.q,
                       (const bf16*)a.k, (const bf16*)a.v, a.alpha, a.beta, ws, egl, a.T, a.H);
    hipLaunchKernelGGL((gdn_carry_h<DK, DV>), dim3(DV / 64, a.H, a.B), dim3(NT), 0, stream,
                       (const char*)ws, (const float*)egl, a.init_state, (bf16*)a.o, a.final_state, a.T, a.H);
    return hipGetLastError();
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
    const size_t nc = (size_t)((T + C - 1) / C);
    if (!bf16_io)
        return (size_t)B * H * nc *
               ((size_t)C * Dk * 4 + (size_t)C * Dv * 4 + (size_t)C * C * 4 + C * sizeof(float));
    const size_t rec = (size_t)C * Dk * 2 * 3 + (size_t)C * C * 2 + (size_t)C * Dv * 2;
    return (size_t)B * H * nc * (rec + sizeof(float));
}

hipError_t launch_gdn_fwd(const GdnFwdArgs& a, hipStream_t stream) {
#define ATMA_GDN_CASE(FN, DKK, DVV) \
    if (a.Dk == DKK && a.Dv == DVV) return FN<DKK, DVV>(a, stream);
    if (a.bf16_io) {
        ATMA_GDN_CASE(launch_h, 64, 64) ATMA_GDN_CASE(launch_h, 64, 128) ATMA_GDN_CASE(launch_h, 128, 64)
        ATMA_GDN_CASE(launch_h, 128, 128)
    } else {
        ATMA_GDN_CASE(launch_f32, 64, 64) ATMA_GDN_CASE(launch_f32, 64, 128) ATMA_GDN_CASE(launch_f32, 128, 64)
        ATMA_GDN_CASE(launch_f32, 128, 128)
    }
#undef ATMA_GDN_CASE
    return hipErrorInvalidValue;
}

}  // namespace atma

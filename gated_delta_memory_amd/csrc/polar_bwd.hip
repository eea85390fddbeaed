// Causal Polar attention, backward, for gfx950 (bf16 in/out, head width 64 or 128).
//
// Gradients of o_i = mu_i c_i (ATMA paper: Section 3.2 equation for t_i and nu_i, Appendix C.2
// single softmax over the real logits and the null logit, Appendix A.2 channels) by the chain
// rule, given dO.  With w_j the softmax weights of row i, w_0 the null weight, R = sum_j w_j,
// Q2 = sum_j w_j^2, m_eff = R^3 / Q2, s = sum_j w_j v_j + w_0 v_null, den = max(||s||, eps),
// c = s / den:
//   dmu = dO . c;  ds = mu (dO - [||s|| > eps] dmu c) / den
//   dm_eff = dmu (1 - mu^2) beta / (1 + m_eff);  dR = 3 dm_eff m_eff / R;  dQ2 = -dm_eff m_eff / Q2
//   Sigma = dR R + 2 dQ2 Q2 + ds . s;  a = dR - Sigma;  b = 2 dQ2
//   real logit l_ij = t_i q_i.k_j / sqrt(D):  dl_ij = w_ij (ds_i . v_j + a_i + b_i w_ij)
//   dq_i = (t_i / sqrt(D)) sum_j dl_ij k_j;  dk_j = sum_i (t_i / sqrt(D)) dl_ij q_i;  dv_j = sum_i w_ij ds_i
//   null logit t_i nu_i:  dl_0 = w_0 (ds . v_null - Sigma);  dnu = dl_0 t;  dt = q.dq / t + dl_0 nu
//   parameters: dtemp_raw = sum_i dt_i ln(n_i) sigmoid(temp_raw), dnull_slope_raw =
//   sum_i dnu_i sqrt(ln(n_i + 1)) sigmoid(null_slope_raw), dnull_bias = sum_i dnu_i,
//   dmag_beta = sum_i dmu_i (1 - mu_i^2) ln(1 + m_eff,i), dv_null = sum_i w_0,i ds_i.
// The weights are recomputed, so no T x T matrix is stored: w_ij = exp2(cq_i (q_i . k_j) - lse2_i)
// with cq_i = t_i log2(e) / sqrt(D).  The row sums the backward needs come from the training
// forward: its real mass R and squared mass Q2 are sums of the fp32 weights exp2(cq_i (q_i . k_j)
// - M) it forms from the same bf16 operands on the same MFMA (origin M, rescaled to lse2 at the
// end), i.e. of the weights recomputed here up to fp32 rounding, and the value sum is s = den c
// from its direction.  So Sigma = dR R + 2 dQ2 Q2 + ds . s is formed per row before any pass over
// the keys.  The logit gradients of a row then sum to sum_j dl_ij + dl_0 = ds . (s' - s), s' the
// value sum of the recomputed fp32 weights, where the forward's s took its weights rounded to
// bf16: a residue of about u |ds| |v| / sqrt(n_eff) per row (u = 2^-8, the bf16 unit roundoff),
// the size of the other bf16 roundings.  (Masses summed from the bf16-rounded weights would add (dR - Sigma)(R' - R), which
// the large mass terms dR, growing with m_eff, would carry into dq_i = sum_j dl_ij k_j, a sum that
// largely cancels.)
//
// Kernels (one call = five launches):
//   prep    ds one row per D/8 lanes, then one row per lane: ds (bf16) and the row scalars {cq, lse2, t a / sqrt(D),
//           t b / sqrt(D), t / sqrt(D)} laid out [B, Hq, 5, Tp] (Tp = T rounded up to 64; padding
//           rows get a log partition of +inf so their weights are exactly zero), and the per-row
//           parameter partials;
//   dq      a workgroup per 128-query tile (4 waves x 32 queries) streams 64-key blocks of K and V
//           through two LDS stages, as the forward does: S^T = K Q^T and dP^T = V dS^T on
//           v_mfma_f32_32x32x16_bf16 (a lane holds 16 keys of one query column, so every row
//           scalar is a per-lane constant), then dQ^T += K^T dL^T with K^T read transposed;
//   dkv     a workgroup per 128-key tile (4 waves x 32 keys, K and V fragments held in registers)
//           streams 64-query blocks of Q, dS and the row scalars of every query head that reads
//           this kv head: S = Q K^T and dP = dS V^T (a lane holds 16 queries of one key column,
//           so the row scalars are read from LDS, four queries per read), then dV^T += dS^T P and
//           dK^T += Q^T dL with dS^T and Q^T read transposed;
//   params  64 workgroups per head sum ranges of rows, a second kernel sums their partials.
// Every tile is read both row-wise (16-byte fragment reads, rows 0..15 per bank cycle) and
// transposed (ds_read_b64_tr_b16, four consecutive rows and 32 bytes per 16-lane group), so one
// swizzle serves both: chunk c of row r sits at c ^ s(r) with, for 128-byte rows,
// s(r) = 4 ((r >> 1) & 1) + ((r >> 2) & 3) (rows of each bank half get distinct chunks; rows r and
// r + 2 differ by 4, so four consecutive rows' 32-byte pieces never share banks), and for 256-byte
// rows s(r) = 4 (r & 3) + ((r >> 2) & 3) (a bijection on 16 rows whose top two bits differ across
// four consecutive rows).
#include "atma_device.hpp"
#include "launch.hpp"

namespace atma {
namespace {

constexpr int NT = 256;
constexpr int BQ = 128;  // queries per dq workgroup
constexpr int BKT = 128; // keys per dkv workgroup
constexpr int BB = 64;   // rows per streamed block
constexpr int NREC = 5;  // row scalars: cq, lse2, a', b', tq

template <int D>
struct BShape {
    static constexpr int NKS = D / 16;          // k-steps of a D-deep MFMA chain
    static constexpr int NDT = D / 32;          // 32-row tiles along D
    static constexpr int ROWB = D * 2;          // bytes per row
    static constexpr int CPR = D / 8;           // 16-byte chunks per row
    static constexpr int TILE = BB * ROWB;      // bytes of one 64-row tile
    static constexpr int CPT = BB * CPR / NT;   // chunks each thread copies per tile
    static constexpr int RPP = NT / CPR;        // rows per pass of the copy
    static constexpr float kInvSqrtD = D == 64 ? 0.125f : 0.08838834764831845f;
};

__device__ __forceinline__ float softplus(float x) { return x > 0.0f ? x + log1pf(expf(-x)) : log1pf(expf(x)); }
__device__ __forceinline__ float sigmoidf(float x) { return 1.0f / (1.0f + expf(-x)); }

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D>
__device__ __forceinline__ int swz(int r, int c) {
    const int s = D == 64 ? (((r & 2) << 1) | ((r >> 2) & 3)) : (((r & 3) << 2) | ((r >> 2) & 3));
    return r * (2 * D) + ((c ^ s) << 4);
}

__device__ __forceinline__ bf16x4 tr_read(const char* lds_base, int byte_off) {
    s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_base + byte_off));
    return __builtin_bit_cast(bf16x4, r);
}

// Wave priority by the share of the largest workload a workgroup still has to stream (rem of maxw
// blocks): a SIMD serves its co-resident waves unevenly, and letting the waves with more work to
// go issue first makes co-resident workgroups finish together.
__device__ __forceinline__ void prio_by_work(int rem, int maxw) {
    const int l = 4 * rem / (maxw + 1);
    if (l >= 3) __builtin_amdgcn_s_setprio(3);
    else if (l == 2) __builtin_amdgcn_s_setprio(2);
    else if (l == 1) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
}

__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Per-lane fragment offsets shared by the two main kernels.  Row reads (A operand, lane row l32,
// d = 16 ks + 8 G2 .. + 7): koff[ks].  Transposed reads of a 64-row tile (A operand of a
// contraction over rows, rows 16 st' + 4 G2 + i16 / 4 (+ 8 for the upper half) of the 16-row
// group, columns 32 dt + 16 (g16 & 1) + 4 (i16 & 3) .. + 3): tlo[dt], thi[dt].
template <int D>
struct Offsets {
    int koff[BShape<D>::NKS], tlo[BShape<D>::NDT], thi[BShape<D>::NDT];
    __device__ __forceinline__ Offsets(int lane) {
        const int l32 = lane & 31, G2 = lane >> 5, g16 = lane >> 4, i16 = lane & 15;
#pragma unroll
        for (int ks = 0; ks < BShape<D>::NKS; ++ks) koff[ks] = swz<D>(l32, 2 * ks + G2);
#pragma unroll
        for (int dt = 0; dt < BShape<D>::NDT; ++dt) {
            const int dcol = 32 * dt + 16 * (g16 & 1) + 4 * (i16 & 3);
            tlo[dt] = swz<D>(4 * G2 + (i16 >> 2), dcol >> 3) + ((dcol & 7) << 1);
            thi[dt] = swz<D>(8 + 4 * G2 + (i16 >> 2), dcol >> 3) + ((dcol & 7) << 1);
        }
    }
};

// ---------------------------------------------------------------------------------------------
// prep: ds of one row (b, h, i) per CH = D / 8 lanes, 8 elements per lane, then the row scalars of
// one row per lane; rows i of [T, Tp) are the padding rows of the streamed query blocks.  Writes
// ds (bf16) and the row scalars the gradient
// kernels read, {cq, lse2, t a / sqrt(D), t b / sqrt(D), t / sqrt(D)} in [B, Hq, 5, Tp], from the
// training forward's statistics: its real mass R and squared mass Q2 are sums of the same fp32
// weights the gradient kernels recompute from the same operands, and its direction gives the value
// sum s = den c, so Sigma = dR R + 2 dQ2 Q2 + ds . s needs no pass over the keys.
// ---------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(NT) void polar_bwd_prep(const bf16* __restrict__ dO, const float* __restrict__ dir,
                                                     const float* __restrict__ stats, const float* __restrict__ mu_in,
                                                     PolarParamsDev prm, bf16* __restrict__ dsg, float* __restrict__ rec,
                                                     float* __restrict__ part, int B, int T, int Tp, int Hq) {
    using SH = BShape<D>;
    constexpr int CH = D / 8, NG = 64 / CH;
    // A wave takes 64 consecutive positions of one (batch, head) (Tp is a multiple of 64): in step
    // `it` each group of CH lanes forms ds for position i0 + NG it + g, and lane ci == it keeps
    // that row's three sums; afterwards every lane finishes the row scalars of its own position
    // i0 + NG ci + g, so the scalar tail runs on all 64 lanes instead of one lane per row, and the
    // scalars of the wave's 64 positions are read and written as whole runs.
    const size_t gw = ((size_t)blockIdx.x * NT + threadIdx.x) >> 6;
    const size_t rid0 = gw * 64;
    const size_t bh = rid0 / Tp;
    if (bh >= (size_t)B * Hq) return;
    const int i0 = (int)(rid0 - bh * Tp);
    const int h = (int)(bh % Hq);
    const int b = (int)(bh / Hq);
    const int lane = lane_id(), g = lane / CH, ci = lane % CH;
    const f32x4 vn0 = *(const f32x4*)(prm.v_null + (size_t)h * D + ci * 8);
    const f32x4 vn1 = *(const f32x4*)(prm.v_null + (size_t)h * D + ci * 8 + 4);
    float kdmu = 0.f, kdsv = 0.f, kdsc = 0.f;  // the sums of row i0 + NG ci + g
#pragma unroll
    for (int it = 0; it < CH; ++it) {
        const int i = i0 + NG * it + g;
        const int ic = min(i, T - 1);  // padding rows re-read the last row; nothing of theirs is stored
        const size_t e0 = (((size_t)b * T + ic) * Hq + h) * D + ci * 8;
        const bf16x8 gb = *(const bf16x8*)(dO + e0);
        const f32x4 c0 = *(const f32x4*)(dir + e0), c1 = *(const f32x4*)(dir + e0 + 4);
        const float dens = stats[(bh * T + ic) * 4 + 3];
        const float mu = mu_in[bh * T + ic];
        float gg[8], c[8], vn[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            gg[e] = (float)gb[e]; gg[e + 4] = (float)gb[e + 4];
            c[e] = c0[e]; c[e + 4] = c1[e];
            vn[e] = vn0[e]; vn[e + 4] = vn1[e];
        }
        const bool clamped = dens < 0.0f;
        const float den = fabsf(dens);
        float dmu = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) dmu += gg[e] * c[e];
#pragma unroll
        for (int o = CH / 2; o >= 1; o >>= 1) dmu += __shfl_xor(dmu, o, CH);
        // ds is rounded to bf16 once and every later use (dP on MFMA, ds . v_null and ds . c here)
        // takes the rounded value
        float dsv = 0.f, dsc = 0.f;
        const float sc = mu / den, pr = clamped ? 0.0f : dmu;
        bf16x8 dsb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            dsb[e] = (bf16)(sc * (gg[e] - pr * c[e]));
            dsv += (float)dsb[e] * vn[e];
            dsc += (float)dsb[e] * c[e];
        }
#pragma unroll
        for (int o = CH / 2; o >= 1; o >>= 1) {
            dsv += __shfl_xor(dsv, o, CH);
            dsc += __shfl_xor(dsc, o, CH);
        }
        if (i < T) *(bf16x8*)(dsg + e0) = dsb;
        if (ci == it) {
            kdmu = dmu;
            kdsv = dsv;
            kdsc = dsc;
        }
    }
    const int i = i0 + NG * ci + g;
    float* rr = rec + bh * NREC * Tp + i;
    if (i >= T) {  // padding row: zero weight (log partition +inf), zero gradient
        rr[0] = 1.0f;
        rr[(size_t)Tp] = INFINITY;
        rr[(size_t)2 * Tp] = 0.0f;
        rr[(size_t)3 * Tp] = 0.0f;
        rr[(size_t)4 * Tp] = 0.0f;
        return;
    }
    const f32x4 st = *(const f32x4*)(stats + (bh * T + i) * 4);
    const float lse2 = st[0], R = st[1], Q2 = st[2], den = fabsf(st[3]);
    const float mu = mu_in[bh * T + i];
    const float dmu = kdmu, dsv = kdsv, dsc = kdsc;
    // t and nu exactly as the forward forms them (cq below is its cq; its null logit t nu).  The
    // masses stay IEEE divisions: on null-dominated rows R^3 underflows and Q2 can be subnormal,
    // where a hardware reciprocal (subnormals flushed) would turn 0 / Q2 into 0 * inf.
    const float n = (float)(i + 1);
    const float t = 1.0f + softplus(prm.temp_raw[h]) * logf(n);
    const float nu = prm.null_bias[h] + softplus(prm.null_slope_raw[h]) * __builtin_sqrtf(__logf(n + 1.0f));
    const float me = R * R * R / Q2;
    const float om = 1.0f - mu * mu;
    const float dme = dmu * om * prm.mag_beta[h] / (1.0f + me);
    const float dR = 3.0f * dme * me / R, dQ2 = -dme * me / Q2;
    const float wn = 1.0f - R;  // the null weight
    const float Sig = dR * R + 2.0f * dQ2 * Q2 + den * dsc;
    const float tqr = t * SH::kInvSqrtD;
    rr[0] = t * kLog2e * SH::kInvSqrtD;  // cq, as the forward forms it
    rr[(size_t)Tp] = lse2;
    rr[(size_t)2 * Tp] = tqr * (dR - Sig);
    rr[(size_t)3 * Tp] = tqr * (2.0f * dQ2);
    rr[(size_t)4 * Tp] = tqr;
    const float dl0 = wn * (dsv - Sig);
    const f32x4 pp = {dl0 * nu, dl0 * t, dmu * om * log1pf(me), wn};
    *(f32x4*)(part + (bh * T + i) * 4) = pp;
}

// ---------------------------------------------------------------------------------------------
// dq: 128 queries per workgroup, key blocks of 64 through two LDS stages
// ---------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(NT, 2) void polar_bwd_dq(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                      const bf16* __restrict__ v, const bf16* __restrict__ dsg,
                                                      const float* __restrict__ rec, bf16* __restrict__ dq,
                                                      float* __restrict__ dtr, int T, int Tp, int Hq, int Hkv) {
    using SH = BShape<D>;
    constexpr int NKS = SH::NKS, NDT = SH::NDT, ROWB = SH::ROWB;
    __shared__ __align__(16) char g_kv0[2 * SH::TILE];
    __shared__ __align__(16) char g_kv1[2 * SH::TILE];
    const int nqt = (T + BQ - 1) / BQ;
    const int nwg = (int)gridDim.x, wg = (int)blockIdx.x, per = nwg >> 3, extra = nwg & 7, xcd = wg & 7;
    const int item = xcd * per + min(xcd, extra) + (wg >> 3);
    const int bh = item / nqt;
    const int qt = nqt - 1 - (item - bh * nqt);  // heaviest tiles first
    const int h = bh % Hq, b = bh / Hq;
    const int hk = h / (Hq / Hkv);
    const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(wave_id());
    const int l32 = lane & 31, G2 = lane >> 5;
    const size_t qstride = (size_t)Hq * D, kvstride = (size_t)Hkv * D;
    const unsigned rowbytes = (unsigned)(kvstride * 2);
    const bf16* kbase = k + (size_t)b * T * kvstride + (size_t)hk * D;
    const bf16* vbase = v + (size_t)b * T * kvstride + (size_t)hk * D;
    const int r0 = (int)threadIdx.x / SH::CPR, pc = (int)threadIdx.x % SH::CPR;
    const unsigned off0 = (unsigned)(swz<D>(r0, pc) - r0 * ROWB);
    auto issue = [&](int kb, const char* stage) {
        const size_t blk = (size_t)kb * BB * kvstride;
        const unsigned lds = lds_addr(stage) + (unsigned)(w * 64 * 16);
        const bool ragged = kb * BB + BB > T;
#pragma unroll
        for (int m = 0; m < SH::CPT; ++m) {
            const int r = ragged ? min(r0 + SH::RPP * m, T - 1 - kb * BB) : r0 + SH::RPP * m;
            lds_dma16(kbase + blk, r * rowbytes + off0, lds + m * NT * 16);
            lds_dma16(vbase + blk, r * rowbytes + off0, lds + SH::TILE + m * NT * 16);
        }
    };
    const Offsets<D> of(lane);

    const int q0 = qt * BQ, qw0 = q0 + w * 32, qi = qw0 + l32, qc = min(qi, T - 1);
    const float* rr = rec + (size_t)bh * NREC * Tp + qc;
    const float cq = rr[0], lse2 = rr[(size_t)Tp], ap = rr[(size_t)2 * Tp], bp = rr[(size_t)3 * Tp],
                tq = rr[(size_t)4 * Tp];
    bf16x8 qf[NKS], sf[NKS];
    {
        const size_t e0 = ((size_t)b * T + qc) * qstride + (size_t)h * D + 8 * G2;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            qf[ks] = *(const bf16x8*)(q + e0 + 16 * ks);
            sf[ks] = *(const bf16x8*)(dsg + e0 + 16 * ks);
        }
    }
    f32x16 acc[NDT];  // dQ^T[d = 32 dt + 8 (x / 4) + 4 G2 + x % 4][qi]
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x16{};
    const int nkb = (min(T, q0 + BQ) + BB - 1) / BB;

    auto block = [&](int kb, const char* Ks) {
        const char* Vs = Ks + SH::TILE;
        const int key0 = kb * BB;
        if (key0 > qw0 + 31) return;  // whole block in this wave's future
        const bool edge = (key0 + BB - 1 > qw0) || (key0 + BB > T);
        f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                s[kt] = mfma32(*(const bf16x8*)(Ks + of.koff[ks] + kt * 32 * ROWB), qf[ks], s[kt]);
                dp[kt] = mfma32(*(const bf16x8*)(Vs + of.koff[ks] + kt * 32 * ROWB), sf[ks], dp[kt]);
            }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                bf16x8 lf;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int x = 8 * st + e;
                    float p = fast_exp2(fmaf(s[kt][x], cq, -lse2));
                    if (edge) {
                        const int key = key0 + 32 * kt + 8 * (x >> 2) + 4 * G2 + (x & 3);
                        p = (key > qi || key >= T) ? 0.0f : p;
                    }
                    lf[e] = (bf16)(p * fmaf(tq, dp[kt][x], fmaf(bp, p, ap)));
                }
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const int base = (32 * kt + 16 * st) * ROWB;
                    const bf16x4 lo = tr_read(Ks, base + of.tlo[dt]);
                    const bf16x4 hi = tr_read(Ks, base + of.thi[dt]);
                    acc[dt] = mfma32(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), lf, acc[dt]);
                }
            }
    };

    const int maxw = (T + BB - 1) / BB;  // key blocks of the heaviest query tile
    issue(0, g_kv0);
    for (int kb = 0; kb < nkb; kb += 2) {
        wait_vmcnt<0>();
        lds_barrier();
        prio_by_work(nkb - kb, maxw);
        if (kb + 1 < nkb) issue(kb + 1, g_kv1);
        block(kb, g_kv0);
        if (kb + 1 >= nkb) break;
        wait_vmcnt<0>();
        lds_barrier();
        if (kb + 2 < nkb) issue(kb + 2, g_kv0);
        block(kb + 1, g_kv1);
    }

    // dq row, and the temperature's share of this row: q . dq / t (dq already carries t / sqrt(D))
    if (qi < T) {
        const size_t e0 = ((size_t)b * T + qi) * qstride + (size_t)h * D;
        float qd = 0.f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * dt + 8 * g + 4 * G2;
                const bf16x4 qv = *(const bf16x4*)(q + e0 + d);
                bf16x4 y;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    y[x] = (bf16)acc[dt][4 * g + x];
                    qd += (float)qv[x] * acc[dt][4 * g + x];
                }
                *(bf16x4*)(dq + e0 + d) = y;
            }
        qd = pair_sum(qd);  // lanes l and l ^ 32 share a query, so both take this branch
        if (G2 == 0) dtr[(size_t)bh * T + qi] = qd / (tq * (1.0f / SH::kInvSqrtD));
    }
}

// ---------------------------------------------------------------------------------------------
// dkv: 128 keys per workgroup, query blocks of 64 (every head of the group) through two stages.
// MODE 0 forms dK and dV together.  At head width 128 their accumulators and fragments need more
// than half a SIMD's registers (one wave per SIMD, and one workgroup per CU at the usual grid
// sizes), so one launch runs a dV role (MODE 1: S and dV) in its first half of workgroups and a
// dK role (MODE 2: S, dP and dK) in its second half: each fits two waves per SIMD, and a CU holds
// one workgroup of each.  Every product is the same in all modes, so the results are bitwise equal.
// ---------------------------------------------------------------------------------------------
template <int D>
constexpr int dkv_stage_bytes() { return 2 * BShape<D>::TILE + NREC * BB * 4; }  // Q tile | dS tile | row scalars [5][64]

// Workgroup wg of nwg runs on XCD wg % 8; renumber so that every XCD receives a contiguous range
// of work items (the tiles of one (batch, kv head) then share an XCD's L2).
__device__ __forceinline__ int xcd_item(int wg, int nwg) {
    const int per = nwg >> 3, extra = nwg & 7, xcd = wg & 7;
    return xcd * per + min(xcd, extra) + (wg >> 3);
}

template <int D, int MODE>
__device__ __forceinline__ void dkv_body(int item, char* g_st0, char* g_st1, const bf16* __restrict__ q,
                                         const bf16* __restrict__ k, const bf16* __restrict__ v,
                                         const bf16* __restrict__ dsg, const float* __restrict__ rec,
                                         bf16* __restrict__ dk, bf16* __restrict__ dv, int T, int Tp, int Hq, int Hkv) {
    using SH = BShape<D>;
    constexpr int NKS = SH::NKS, NDT = SH::NDT, ROWB = SH::ROWB;
    const int nkt = (T + BKT - 1) / BKT;
    const int bk = item / nkt;
    const int j = item - bk * nkt;  // key tile; tile 0 streams the most query blocks and goes first
    const int hk = bk % Hkv, b = bk / Hkv;
    const int G = Hq / Hkv;
    const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(wave_id());
    const int l32 = lane & 31, G2 = lane >> 5;
    const size_t qstride = (size_t)Hq * D, kvstride = (size_t)Hkv * D;
    const unsigned rowbytes = (unsigned)(qstride * 2);
    const int kw0 = j * BKT + w * 32, key = kw0 + l32, kc = min(key, T - 1);
    bf16x8 kf[NKS], vf[NKS];
    {
        const size_t e0 = ((size_t)b * T + kc) * kvstride + (size_t)hk * D + 8 * G2;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            kf[ks] = *(const bf16x8*)(k + e0 + 16 * ks);
            if constexpr (MODE != 1) vf[ks] = *(const bf16x8*)(v + e0 + 16 * ks);
        }
    }
    const int r0 = (int)threadIdx.x / SH::CPR, pc = (int)threadIdx.x % SH::CPR;
    const unsigned off0 = (unsigned)(swz<D>(r0, pc) - r0 * ROWB);
    const int qb0 = (j * BKT) / BB, nqb = (T + BB - 1) / BB, nb = nqb - qb0;
    const int nit = G * nb;
    auto issue = [&](int it, const char* stage) {
        const int h = hk * G + it / nb, qb = qb0 + it % nb;
        const size_t rowoff = ((size_t)b * T + (size_t)qb * BB) * qstride + (size_t)h * D;
        const unsigned lds = lds_addr(stage) + (unsigned)(w * 64 * 16);
        const bool ragged = qb * BB + BB > T;
#pragma unroll
        for (int m = 0; m < SH::CPT; ++m) {
            const int r = ragged ? min(r0 + SH::RPP * m, T - 1 - qb * BB) : r0 + SH::RPP * m;
            lds_dma16(q + rowoff, r * rowbytes + off0, lds + m * NT * 16);
            lds_dma16(dsg + rowoff, r * rowbytes + off0, lds + SH::TILE + m * NT * 16);
        }
        // row scalars: five runs of 64 floats (16 chunks each), threads 0..79
        if (w < 2) {
            const int t = (int)threadIdx.x;
            if (t < NREC * 16) {
                const float* src = rec + ((size_t)(b * Hq + h) * NREC) * Tp + (size_t)qb * BB;
                lds_dma16(src, (unsigned)(((t >> 4) * Tp + (t & 15) * 4) * 4),
                          lds_addr(stage) + 2 * SH::TILE + (unsigned)(w * 64 * 16));
            }
        }
    };
    const Offsets<D> of(lane);
    f32x16 dka[NDT], dva[NDT];  // dK^T, dV^T [d = 32 dt + 8 (x / 4) + 4 G2 + x % 4][key]
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) dka[dt] = dva[dt] = f32x16{};

    auto block = [&](int it, const char* Qs) {
        const char* Ss = Qs + SH::TILE;
        const float* Rs = (const float*)(Qs + 2 * SH::TILE);
        const int q0 = (qb0 + it % nb) * BB;
        if (q0 + BB - 1 < kw0 || kw0 >= T) return;  // every query of the block precedes every key
        const bool edge = q0 < kw0 + 32;
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                s = mfma32(*(const bf16x8*)(Qs + of.koff[ks] + qt * 32 * ROWB), kf[ks], s);
                if constexpr (MODE != 1) dp = mfma32(*(const bf16x8*)(Ss + of.koff[ks] + qt * 32 * ROWB), vf[ks], dp);
            }
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const int ql = 32 * qt + 16 * st + 4 * G2;  // queries ql + (e & 3) + 8 (e >> 2)
                // the transposed dS and Q fragments of this step are requested before the weights
                // are formed, so their LDS latency overlaps the exponentials
                bf16x8 sfr[NDT], qfr[NDT];
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const int base = (32 * qt + 16 * st) * ROWB;
                    if constexpr (MODE != 2) {
                        const bf16x4 slo = tr_read(Ss, base + of.tlo[dt]), shi = tr_read(Ss, base + of.thi[dt]);
                        sfr[dt] = __builtin_shufflevector(slo, shi, 0, 1, 2, 3, 4, 5, 6, 7);
                    }
                    if constexpr (MODE != 1) {
                        const bf16x4 qlo = tr_read(Qs, base + of.tlo[dt]), qhi = tr_read(Qs, base + of.thi[dt]);
                        qfr[dt] = __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7);
                    }
                }
                f32x4 rc[2], rl[2], ra[2], rb[2], rt[2];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    rc[hf] = *(const f32x4*)(Rs + 0 * BB + ql + 8 * hf);
                    rl[hf] = *(const f32x4*)(Rs + 1 * BB + ql + 8 * hf);
                    ra[hf] = *(const f32x4*)(Rs + 2 * BB + ql + 8 * hf);
                    rb[hf] = *(const f32x4*)(Rs + 3 * BB + ql + 8 * hf);
                    rt[hf] = *(const f32x4*)(Rs + 4 * BB + ql + 8 * hf);
                }
                bf16x8 pf, lf;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int x = 8 * st + e, hf = e >> 2, z = e & 3;
                    float p = fast_exp2(fmaf(s[x], rc[hf][z], -rl[hf][z]));
                    if (edge) p = (q0 + ql + 8 * hf + z < key) ? 0.0f : p;
                    pf[e] = (bf16)p;
                    if constexpr (MODE != 1) lf[e] = (bf16)(p * fmaf(rt[hf][z], dp[x], fmaf(rb[hf][z], p, ra[hf][z])));
                }
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    if constexpr (MODE != 2) dva[dt] = mfma32(sfr[dt], pf, dva[dt]);
                    if constexpr (MODE != 1) dka[dt] = mfma32(qfr[dt], lf, dka[dt]);
                }
            }
        }
    };

    issue(0, g_st0);
    for (int it = 0; it < nit; it += 2) {
        wait_vmcnt<0>();
        lds_barrier();
        prio_by_work(nit - it, G * nqb);  // the heaviest key tile streams G nqb query blocks
        if (it + 1 < nit) issue(it + 1, g_st1);
        block(it, g_st0);
        if (it + 1 >= nit) break;
        wait_vmcnt<0>();
        lds_barrier();
        if (it + 2 < nit) issue(it + 2, g_st0);
        block(it + 1, g_st1);
    }

    if (key < T) {
        const size_t e0 = ((size_t)b * T + key) * kvstride + (size_t)hk * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 yk, yv;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    yk[x] = (bf16)dka[dt][4 * g + x];
                    yv[x] = (bf16)dva[dt][4 * g + x];
                }
                if constexpr (MODE != 1) *(bf16x4*)(dk + e0 + 32 * dt + 8 * g + 4 * G2) = yk;
                if constexpr (MODE != 2) *(bf16x4*)(dv + e0 + 32 * dt + 8 * g + 4 * G2) = yv;
            }
    }
}

template <int D>
__global__ __launch_bounds__(NT, D == 64 ? 2 : 1) void polar_bwd_dkv(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                       const bf16* __restrict__ v, const bf16* __restrict__ dsg,
                                                       const float* __restrict__ rec, bf16* __restrict__ dk,
                                                       bf16* __restrict__ dv, int T, int Tp, int Hq, int Hkv) {
    __shared__ __align__(16) char g_st0[dkv_stage_bytes<D>()];
    __shared__ __align__(16) char g_st1[dkv_stage_bytes<D>()];
    dkv_body<D, 0>(xcd_item((int)blockIdx.x, (int)gridDim.x), g_st0, g_st1, q, k, v, dsg, rec, dk, dv, T, Tp, Hq,
                   Hkv);
}

// grid 2 nk: work item 2 j is the dV role of key tile j and item 2 j + 1 its dK role, so the
// two roles of a tile (which stream the same query blocks) sit side by side on one XCD
template <int D>
__global__ __launch_bounds__(NT, 2) void polar_bwd_dkv_split(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                             const bf16* __restrict__ v, const bf16* __restrict__ dsg,
                                                             const float* __restrict__ rec, bf16* __restrict__ dk,
                                                             bf16* __restrict__ dv, int T, int Tp, int Hq, int Hkv) {
    __shared__ __align__(16) char g_st0[dkv_stage_bytes<D>()];
    __shared__ __align__(16) char g_st1[dkv_stage_bytes<D>()];
    const int it = xcd_item((int)blockIdx.x, (int)gridDim.x);
    if ((it & 1) == 0) dkv_body<D, 1>(it >> 1, g_st0, g_st1, q, k, v, dsg, rec, dk, dv, T, Tp, Hq, Hkv);
    else dkv_body<D, 2>(it >> 1, g_st0, g_st1, q, k, v, dsg, rec, dk, dv, T, Tp, Hq, Hkv);
}

// ---------------------------------------------------------------------------------------------
// params: per head, PCH workgroups each sum a contiguous range of rows (D / 8 lanes per row, 8
// elements of ds each); a second kernel sums the PCH partials.  Fixed order: deterministic.
// ---------------------------------------------------------------------------------------------
constexpr int PCH = 64;

template <int D>
__global__ __launch_bounds__(NT) void polar_bwd_params_partial(const bf16* __restrict__ dsg,
                                                               const float* __restrict__ part,
                                                               const float* __restrict__ dtr,
                                                               float* __restrict__ ppart, int B, int T, int Hq) {
    constexpr int CH = D / 8, RL = NT / CH, U = 4;
    __shared__ float red[4][NT];
    __shared__ float vred[RL][D];
    const int h = (int)blockIdx.x / PCH, c = (int)blockIdx.x % PCH, tid = (int)threadIdx.x;
    const int ci = tid % CH, rl = tid / CH;
    const long rows = (long)B * T, r0 = rows * c / PCH, r1 = rows * (c + 1) / PCH;
    if (r1 <= r0) {  // fewer rows than workgroups: an empty range contributes zeros
        float* out = ppart + ((size_t)h * PCH + c) * (4 + D);
        if (tid < 4 + D) out[tid] = 0.0f;
        return;
    }
    auto row_index = [&](long r) {  // row r of this head's B*T rows in the [B, Hq, T] layouts
        const int b = (int)(r / T), i = (int)(r - (long)b * T);
        return ((size_t)b * Hq + h) * T + i;
    };
    // the scalar parameters: one row per thread, U rows requested together (rows past the range
    // re-read its first row and are skipped)
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    for (long rb = r0 + tid; rb < r1; rb += (long)U * NT) {
        f32x4 p[U];
        float dt[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const long r = rb + (long)u * NT;
            const size_t ri = row_index(r < r1 ? r : r0);
            p[u] = *(const f32x4*)(part + ri * 4);
            dt[u] = dtr[ri];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const long r = rb + (long)u * NT;
            if (r < r1) {
                const int i = (int)(r % T);
                const float n = (float)(i + 1);
                s0 += (dt[u] + p[u][0]) * logf(n);
                s1 += p[u][1] * sqrtf(logf(n + 1.0f));
                s2 += p[u][1];
                s3 += p[u][2];
            }
        }
    }
    // v_null: CH lanes per row (8 value columns each), U rows requested together
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (long rb = r0 + rl; rb < r1; rb += (long)U * RL) {
        bf16x8 d8[U];
        float wn[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const long r = rb + (long)u * RL;
            const long rc = r < r1 ? r : r0;
            const int b = (int)(rc / T), i = (int)(rc - (long)b * T);
            const float x = part[row_index(rc) * 4 + 3];
            wn[u] = r < r1 ? x : 0.0f;
            d8[u] = *(const bf16x8*)(dsg + (((size_t)b * T + i) * Hq + h) * D + ci * 8);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = fmaf(wn[u], (float)d8[u][e], acc[e]);
    }
    red[0][tid] = s0; red[1][tid] = s1; red[2][tid] = s2; red[3][tid] = s3;
#pragma unroll
    for (int e = 0; e < 8; ++e) vred[rl][ci * 8 + e] = acc[e];
    __syncthreads();
    for (int o = NT / 2; o >= 1; o >>= 1) {
        if (tid < o)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[e][tid] += red[e][tid + o];
        __syncthreads();
    }
    float* out = ppart + ((size_t)h * PCH + c) * (4 + D);
    if (tid < 4) out[tid] = red[tid][0];
    if (tid < D) {
        float sum = 0.f;
        for (int r = 0; r < RL; ++r) sum += vred[r][tid];
        out[4 + tid] = sum;
    }
}

template <int D>
__global__ __launch_bounds__(NT) void polar_bwd_params_final(const float* __restrict__ ppart, PolarParamsDev prm,
                                                             float* __restrict__ d_temp_raw, float* __restrict__ d_slope,
                                                             float* __restrict__ d_bias, float* __restrict__ d_beta,
                                                             float* __restrict__ d_vnull) {
    const int h = (int)blockIdx.x, tid = (int)threadIdx.x;
    if (tid >= 4 + D) return;
    float sum = 0.f;
#pragma unroll 16
    for (int c = 0; c < PCH; ++c) sum += ppart[((size_t)h * PCH + c) * (4 + D) + tid];
    if (tid == 0) d_temp_raw[h] = sum * sigmoidf(prm.temp_raw[h]);
    else if (tid == 1) d_slope[h] = sum * sigmoidf(prm.null_slope_raw[h]);
    else if (tid == 2) d_bias[h] = sum;
    else if (tid == 3) d_beta[h] = sum;
    else d_vnull[(size_t)h * D + tid - 4] = sum;
}

struct BwdWs {
    bf16* dsg;
    float *rec, *part, *dtr, *ppart;
};
BwdWs carve(void* ws, int B, int T, int Hq, int D) {
    const size_t Tp = (size_t)(T + BB - 1) / BB * BB;
    char* p = (char*)ws;
    BwdWs w;
    w.dsg = (bf16*)p;
    p += ((size_t)B * T * Hq * D * 2 + 255) / 256 * 256;
    w.rec = (float*)p;
    p += ((size_t)B * Hq * NREC * Tp * 4 + 255) / 256 * 256;
    w.part = (float*)p;
    p += ((size_t)B * Hq * T * 16 + 255) / 256 * 256;
    w.dtr = (float*)p;
    p += ((size_t)B * Hq * T * 4 + 255) / 256 * 256;
    w.ppart = (float*)p;
    return w;
}

}  // namespace

size_t polar_bwd_workspace_bytes(int B, int T, int Hq, int D) {
    const size_t Tp = (size_t)(T + BB - 1) / BB * BB;
    return ((size_t)B * T * Hq * D * 2 + 255) / 256 * 256 + ((size_t)B * Hq * NREC * Tp * 4 + 255) / 256 * 256 +
           ((size_t)B * Hq * T * 16 + 255) / 256 * 256 + ((size_t)B * Hq * T * 4 + 255) / 256 * 256 +
           (size_t)Hq * PCH * (4 + D) * 4;
}

hipError_t launch_polar_bwd(const PolarBwdArgs& a, hipStream_t stream) {
    const BwdWs w = carve(a.workspace, a.B, a.T, a.Hq, a.D);
    const int Tp = (a.T + BB - 1) / BB * BB;
    const long long nq = (long long)((a.T + BQ - 1) / BQ) * a.Hq * a.B;
    const long long nk = (long long)((a.T + BKT - 1) / BKT) * a.Hkv * a.B;
    const long long prep_threads = (long long)a.B * Tp * a.Hq;  // one lane per row (64 rows per wave)
    if (nq > 0x7fffffffLL || 2 * nk > 0x7fffffffLL || prep_threads / NT > 0x7fffffffLL) return hipErrorInvalidConfiguration;
#define ATMA_PB_LAUNCH(DD)                                                                                        \
    do {                                                                                                          \
        hipLaunchKernelGGL(polar_bwd_prep<DD>, dim3((unsigned)((prep_threads + NT - 1) / NT)), dim3(NT), 0,       \
                           stream, (const bf16*)a.dO, a.dir, a.stats, a.mu, a.p, w.dsg, w.rec, w.part, a.B, a.T,   \
                           Tp, a.Hq);                                                                              \
        hipLaunchKernelGGL(polar_bwd_dq<DD>, dim3((unsigned)nq), dim3(NT), 0, stream, (const bf16*)a.q,           \
                           (const bf16*)a.k, (const bf16*)a.v, (const bf16*)w.dsg, (const float*)w.rec,            \
                           (bf16*)a.dq, w.dtr, a.T, Tp, a.Hq, a.Hkv);                                              \
        if (DD == 64)                                                                                             \
            hipLaunchKernelGGL(polar_bwd_dkv<DD>, dim3((unsigned)nk), dim3(NT), 0, stream, (const bf16*)a.q,      \
                               (const bf16*)a.k, (const bf16*)a.v, (const bf16*)w.dsg, (const float*)w.rec,        \
                               (bf16*)a.dk, (bf16*)a.dv, a.T, Tp, a.Hq, a.Hkv);                                    \
        else                                                                                                      \
            hipLaunchKernelGGL(polar_bwd_dkv_split<DD>, dim3((unsigned)(2 * nk)), dim3(NT), 0, stream,            \
                               (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)w.dsg,          \
                               (const float*)w.rec, (bf16*)a.dk, (bf16*)a.dv, a.T, Tp, a.Hq, a.Hkv);               \
        hipLaunchKernelGGL(polar_bwd_params_partial<DD>, dim3(a.Hq * PCH), dim3(NT), 0, stream,                   \
                           (const bf16*)w.dsg, (const float*)w.part, (const float*)w.dtr, w.ppart, a.B, a.T, a.Hq); \
        hipLaunchKernelGGL(polar_bwd_params_final<DD>, dim3(a.Hq), dim3(NT), 0, stream, (const float*)w.ppart,    \
                           a.p, a.d_temp_raw, a.d_null_slope_raw, a.d_null_bias, a.d_mag_beta, a.d_v_null);        \
    } while (0)
    if (a.D == 64) ATMA_PB_LAUNCH(64);
    else if (a.D == 128) ATMA_PB_LAUNCH(128);
    else return hipErrorInvalidValue;
#undef ATMA_PB_LAUNCH
    return hipGetLastError();
}

}  // namespace atma

// Causal Polar attention, prefill, for gfx950 (bf16 in/out, head width 64).
//
// Definitions (ATMA paper): temperature t_i = 1 + softplus(alpha) ln n_i and null floor
// nu_i = b + softplus(gamma) sqrt(ln(n_i + 1)) (Section 3.2 equation), with n_i = i + 1 real
// keys visible to query i; one softmax over the real logits t_i q_i.k_j / sqrt(D) and the
// virtual null logit t_i nu_i (Appendix C.2); direction c_i = s_i / max(||s_i||, eps) and
// magnitude mu_i = tanh(beta ln(1 + m_eff)) (Appendix A.2); o_i = mu_i c_i.
// Streaming form (Appendix C.3, Table 6): per query row keep an origin M for the real
// logits, L = sum p, Q2 = sum p^2 and Sv = sum p v with p = exp(logit - M); moving the
// origin by delta scales the three sums by exp(-delta), exp(-2 delta) and exp(-delta).  The
// null enters once, at the end, with the common origin M* = max(M, null logit):
//     p_null = e^{l_null - M*},  L* = L e^{M - M*},  Z = L* + p_null,  n_eff = L^2 / Q2,
//     m_eff = n_eff L* / Z,  s = (Sv e^{M - M*} + p_null v_null) / Z.
// Every formula is invariant to the choice of origin, so M is moved only when a block's
// maximum exceeds it by more than 8 (base-2 units): p <= 2^8 keeps every sum far from
// overflow and most blocks skip the rescale.  Exponentials are base 2 on logits scaled
// by log2(e).
//
// Kernel layout (one workgroup of 4 waves per pair of 128-query tiles of one head and batch;
// within a tile each wave owns 32 consecutive queries):
//   * keys stream in blocks of 64 through two LDS stages (K and V row-major, 16-byte chunks
//     XOR-swizzled by key so fragment reads are bank-conflict free), filled by asynchronous
//     global->LDS copies one block ahead, one barrier per block;
//   * scores are formed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16: a lane holds
//     16 keys of one query column, so row statistics are per-lane partial sums (the two
//     lanes that share a query are combined with v_permlane32_swap);
//   * the same registers, cast to bf16, are the B operand of O^T = V^T P^T; the V^T
//     fragments come straight from the row-major V tile with ds_read_b64_tr_b16;
//   * L and Q2 are accumulated from the fp32 weights (before their rounding to bf16 for the value
//     product), which are exactly the weights the backward recomputes from the same operands, so
//     the backward can take its row statistics from this pass (the control cores, which have no
//     backward, sum the bf16 weights with v_dot2_f32_bf16);
//   * a workgroup computes two query tiles of one (batch, head), the k-th heaviest and the
//     k-th lightest, so all workgroups stream the same number of key blocks (causal balance);
//     the tiles of one (batch, head) go to one XCD so their K/V stream is shared in its L2.
// Packed batches (sequences of different lengths concatenated, offsets cu[0..B] on the device)
// use the same kernel: the grid is sized for the longest sequence and each workgroup reads its
// sequence's bounds, skipping tiles past its end.  Offsets that are not a valid partition of
// the packed rows (or a sequence longer than the declared maximum) skip that sequence, so a
// malformed offset array can never address memory outside the buffers.
// With POLAR false the same kernel is the plain causal softmax attention of the NoPE / RoPE
// control cores (ATMA paper, Section 3.1): logits q.k / sqrt(D) (no temperature), no null,
// output sum_j w_j v_j = Sv / L (no direction / magnitude channels).
#include "atma_device.hpp"
#include "launch.hpp"

namespace atma {
namespace {

constexpr int NT = 256;
constexpr int BQ = 128;  // queries per workgroup
constexpr int QW = 32;   // queries per wave
constexpr int BK = 64;   // keys per block
constexpr float kLazy = 8.0f;

// Head-width dependent shapes (D = 64 or 128).
template <int D>
struct Shape {
    static constexpr int NKS = D / 16;          // k-steps of the score MFMA
    static constexpr int NDT = D / 32;          // 32-row tiles of O^T
    static constexpr int ROWB = D * 2;          // bytes per key row
    static constexpr int CPR = D / 8;           // 16-byte chunks per row
    static constexpr int TILE = BK * ROWB;      // bytes of one K (or V) tile
    static constexpr int CPT = BK * CPR / NT;   // chunks each thread copies per tile
    static constexpr int RPP = NT / CPR;        // rows per pass of the copy
    static constexpr int OCC = D == 64 ? 4 : 2; // waves per SIMD (two 2-stage LDS buffers of 64 KB at D=128)
    static constexpr float kInvSqrtD = D == 64 ? 0.125f : 0.08838834764831845f;
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ float softplus(float x) { return x > 0.0f ? x + log1pf(expf(-x)) : log1pf(expf(x)); }

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Byte offset of 16-byte chunk c of key row `key` in a 64 x D bf16 tile.  The LDS has 64
// four-byte banks (256 bytes).  K tiles are read 16 bytes per lane with rows 0..15 in one bank
// cycle.  D = 64 (128-byte rows): rows r and r + 1 use disjoint bank halves, so XOR-ing the
// chunk with (r >> 1) & 7 gives the rows of each parity eight distinct chunks.  D = 128
// (256-byte rows, every row on all banks): XOR with r & 15 gives the sixteen rows sixteen
// distinct chunks.  V tiles are read by ds_read_b64_tr_b16, which takes four consecutive rows and
// two adjacent chunks per 16-lane group: XOR-ing with 2 (r & 3) puts the four rows' pieces on
// four different 32-byte bank groups at either width.
template <int D>
__device__ __forceinline__ int swz_k(int key, int c) {
    return key * (2 * D) + ((c ^ (D == 64 ? ((key >> 1) & 7) : (key & 15))) << 4);
}
template <int D>
__device__ __forceinline__ int swz_v(int key, int c) { return key * (2 * D) + ((c ^ ((key & 3) << 1)) << 4); }

// partner-lane (l ^ 32) combine via v_permlane32_swap
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x4 tr_read(const char* lds_base, int byte_off) {
    s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_base + byte_off));
    return __builtin_bit_cast(bf16x4, r);
}

template <int D, bool POLAR>
__global__ __launch_bounds__(NT, Shape<D>::OCC) void polar_fwd_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                          const bf16* __restrict__ v, PolarParamsDev prm,
                                                          bf16* __restrict__ o, float* __restrict__ mu_out,
                                                          float* __restrict__ meff_out, float* __restrict__ stats,
                                                          float* __restrict__ dir, int Tmax, int Hq, int Hkv,
                                                          int paired, const int* __restrict__ cu, int total) {
    // Work items.  With `paired` set (few tiles in all), a workgroup computes two query tiles
    // of one (batch, head), tile nqt - 1 - p and tile p: every pair streams the same number of
    // key blocks (causal balance) and the per-tile start-up and finalisation are spread over
    // twice the work.  Otherwise a workgroup computes one tile, heaviest (last) tiles first.
    // Workgroup i is dispatched to XCD i % 8; the flat grid is renumbered so that every XCD
    // receives a contiguous range of items and the tiles of one (batch, head) share that
    // XCD's L2 for their K/V stream.
    using SH = Shape<D>;
    constexpr int NKS = SH::NKS, NDT = SH::NDT, ROWB = SH::ROWB;
    // Two K/V stages, one LDS object each (the copy into one stage overlaps the reads of the other).
    __shared__ __align__(16) char g_kv0[2 * SH::TILE];
    __shared__ __align__(16) char g_kv1[2 * SH::TILE];
    // per-head constants of the finalisation: v_null[0..D), softplus(null slope), null bias,
    // magnitude beta.  Read from LDS when a tile finalises: global loads there would expose a
    // round trip to memory per tile (the loop leaves nothing to overlap them with).
    __shared__ __align__(16) float g_par[D + 4];
    const int nqt_grid = (Tmax + BQ - 1) / BQ;
    const int per_bh = paired ? (nqt_grid + 1) / 2 : nqt_grid;
    const int nwg = (int)gridDim.x, wg = (int)blockIdx.x, per = nwg >> 3, extra = nwg & 7, xcd = wg & 7;
    const int item = xcd * per + min(xcd, extra) + (wg >> 3);
    const int bh = item / per_bh;
    const int pr = item - bh * per_bh;
    const int h = bh % Hq, b = bh / Hq;
    const int hk = h / (Hq / Hkv);
    // this sequence: first packed row seq0 and length T
    size_t seq0;
    int T;
    if (cu) {
        const int s0 = __builtin_amdgcn_readfirstlane(cu[b]), s1 = __builtin_amdgcn_readfirstlane(cu[b + 1]);
        if (s0 < 0 || s1 < s0 || s1 > total || s1 - s0 > Tmax) return;  // malformed offsets
        seq0 = (size_t)s0;
        T = s1 - s0;
    } else {
        seq0 = (size_t)b * Tmax;
        T = Tmax;
    }
    const int nqt = (T + BQ - 1) / BQ;
    if (pr >= (paired ? (nqt + 1) / 2 : nqt)) return;  // past the end of this sequence
    const size_t mu_base = cu ? (size_t)h * total + seq0 : ((size_t)b * Hq + h) * Tmax;
    const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(wave_id());  // wave-uniform
    const int l32 = lane & 31, G2 = lane >> 5, g16 = lane >> 4, i16 = lane & 15;
    const float a_t = POLAR ? softplus(prm.temp_raw[h]) : 0.0f;
    const size_t qstride = (size_t)Hq * D;
    const size_t kvstride = (size_t)Hkv * D;
    const unsigned rowbytes = (unsigned)(kvstride * 2);
    const bf16* kbase = k + seq0 * kvstride + (size_t)hk * D;
    const bf16* vbase = v + seq0 * kvstride + (size_t)hk * D;

    // Asynchronous copy of key block kb into a stage [K tile | V tile]: 16-byte chunk ch of a
    // tile lands at LDS slot ch (row ch / CPR, position ch % CPR); the source chunk is chosen so
    // the tile comes out swizzled.  Thread t moves chunks t + 256 m (m < CPT) of each tile:
    // rows r0 + RPP m at position pc, all with the same swizzle.
    const int r0 = (int)threadIdx.x / SH::CPR, pc = (int)threadIdx.x % SH::CPR;
    const unsigned koff0 = (unsigned)(swz_k<D>(r0, pc) - r0 * ROWB);
    const unsigned voff0 = (unsigned)(swz_v<D>(r0, pc) - r0 * ROWB);
    auto issue = [&](int kb, const char* stage) {
        const size_t blk = (size_t)kb * BK * kvstride;
        const unsigned lds = lds_addr(stage) + (unsigned)(w * 64 * 16);
        const bool ragged = kb * BK + BK > T;  // last block of a ragged sequence: rows past T repeat row T - 1
#pragma unroll
        for (int m = 0; m < SH::CPT; ++m) {
            const int r = ragged ? min(r0 + SH::RPP * m, T - 1 - kb * BK) : r0 + SH::RPP * m;
            lds_dma16(kbase + blk, r * rowbytes + koff0, lds + m * NT * 16);
            lds_dma16(vbase + blk, r * rowbytes + voff0, lds + SH::TILE + m * NT * 16);
        }
    };

    // Lane-constant fragment offsets inside a stage.  K (A operand of S^T = K Q^T): lane reads
    // key 32 kt + l32, d = 16 ks + 8 G2 .. + 7.  V^T (A operand of O^T = V^T P^T) via transposed
    // reads: for weight slot group (kt, st) the 16-lane group g16 reads keys
    // 32 kt + 16 st + 4 G2 + (i16 / 4) (+ 8 for the upper half of the fragment), columns
    // 32 dt + 16 (g16 & 1) + 4 (i16 & 3) .. + 3.
    int koff[NKS], voff[NDT];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) koff[ks] = swz_k<D>(l32, 2 * ks + G2);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
        const int dcol = 32 * dt + 16 * (g16 & 1) + 4 * (i16 & 3);
        voff[dt] = swz_v<D>(4 * G2 + (i16 >> 2), dcol >> 3) + ((dcol & 7) << 1);
    }

  // `after`: key blocks this workgroup streams after this tile (its second tile, when paired);
  // `first`: the workgroup's first tile (it fills g_par)
  auto tile = [&](int qt, int after, bool first) {
    const int q0 = qt * BQ;
    const int qw0 = q0 + w * QW;
    const int qi = qw0 + l32;  // this lane's query
    const float cq = POLAR ? (1.0f + a_t * logf((float)(qi + 1))) * kLog2e * SH::kInvSqrtD  // t_i log2(e) / sqrt(D)
                           : kLog2e * SH::kInvSqrtD;

    // the finalisation constants are requested with the tile's first loads (stored after them)
    float pv = 0.0f;
    const int tp = (int)threadIdx.x;
    if (POLAR && first && tp < D + 3)
        pv = tp < D ? prm.v_null[h * D + tp] : tp == D ? prm.null_slope_raw[h] : tp == D + 1 ? prm.null_bias[h] : prm.mag_beta[h];
    // Q^T fragments (B operand): lane supplies Q[qi][16 ks + 8 G2 + e]
    bf16x8 qf[NKS];
    {
        const int qc = min(qi, T - 1);
        const bf16* qrow = q + (seq0 + qc) * qstride + (size_t)h * D + 8 * G2;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qf[ks] = *(const bf16x8*)(qrow + 16 * ks);
    }

    f32x16 oacc[NDT];  // O^T[d = 32 dt + 8(x/4) + 4 G2 + x%4][qi]
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16{};
    float m_used = -INFINITY;
    float lsum[4] = {0.f, 0.f, 0.f, 0.f}, q2sum[4] = {0.f, 0.f, 0.f, 0.f};  // split to shorten dependency chains

    const int kend = min(T, q0 + BQ);
    const int nkb = (kend + BK - 1) / BK;

    auto block = [&](int kb, const char* Ks) {
        const char* Vs = Ks + SH::TILE;
        const int key0 = kb * BK;
        if (key0 > qw0 + QW - 1) return;  // whole block in this wave's future
        const bool edge = (key0 + BK - 1 > qw0) || (key0 + BK > T);


        // S^T = K Q^T : two 32-key sub-tiles, chains interleaved
        f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) s[kt] = mfma32(*(const bf16x8*)(Ks + koff[ks] + kt * 32 * ROWB), qf[ks], s[kt]);

        // causal / length mask on edge blocks (raw scores; cq > 0 scales them later)
        if (edge) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    const int key = key0 + 32 * kt + 8 * (x >> 2) + 4 * G2 + (x & 3);
                    s[kt][x] = (key > qi || key >= T) ? -INFINITY : s[kt][x];
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int x = 0; x < 16; ++x) mx = fmaxf(mx, s[kt][x]);
        mx = pair_max(mx) * cq;
        // lazy origin move (wave-uniform branch)
        const bool move = mx > m_used + kLazy;
        if (__builtin_amdgcn_ballot_w64(move) != 0) {
            const float mnew = move ? mx : m_used;
            const float rho = fast_exp2(m_used - mnew);
            m_used = mnew;
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                lsum[a4] *= rho;
                q2sum[a4] *= rho * rho;
            }
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= rho;
        }
        // weights, their sums, and O^T += V^T P^T
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                bf16x8 pf;
                float& ls = lsum[2 * kt + st];
                float& qs = q2sum[2 * kt + st];
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const float p0 = fast_exp2(fmaf(s[kt][8 * st + e], cq, -m_used));
                    const float p1 = fast_exp2(fmaf(s[kt][8 * st + e + 1], cq, -m_used));
                    const bf16x2 pp = {(bf16)p0, (bf16)p1};
                    if constexpr (POLAR) {  // the fp32 weights, as the backward recomputes them
                        ls += p0;
                        ls += p1;
                        qs = fmaf(p0, p0, qs);
                        qs = fmaf(p1, p1, qs);
                    } else {
                        ls = __builtin_amdgcn_fdot2_f32_bf16(pp, bf16x2{(bf16)1.0f, (bf16)1.0f}, ls, false);
                    }
                    pf[e] = pp[0];
                    pf[e + 1] = pp[1];
                }
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const int base = voff[dt] + (32 * kt + 16 * st) * ROWB;
                    const bf16x4 lo = tr_read(Vs, base);
                    const bf16x4 hi = tr_read(Vs, base + 8 * ROWB);
                    oacc[dt] = mfma32(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pf, oacc[dt]);
                }
            }
        }
    };

    // two-stage pipeline: the copy of block kb + 1 overlaps the computation of block kb.  The
    // loop is unrolled by two so each stage is a fixed LDS address and every fragment read
    // takes its offset as an immediate.
    // Wave priority by the share of the heaviest workgroup's work this workgroup has left: a SIMD
    // serves its co-resident waves unevenly, so equal work does not end at equal times; letting the
    // waves with more blocks to go issue first makes the workgroups of a CU finish together (at the
    // 2K layer ~7% sooner, at 16K ~3%).
    auto prio = [&](int kb) {
        const int rem = nkb - kb + after;
        const int maxw = paired ? 2 * nqt + 2 : 2 * nqt;  // key blocks of the heaviest workgroup
        const int l = 4 * rem / (maxw + 1);
        if (l >= 3) __builtin_amdgcn_s_setprio(3);
        else if (l == 2) __builtin_amdgcn_s_setprio(2);
        else if (l == 1) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
    };
    issue(0, g_kv0);
    if (POLAR && first) {  // visible to every wave after the loop's first barrier
        __builtin_amdgcn_sched_barrier(0);
        if (tp < D + 3) g_par[tp] = tp == D ? softplus(pv) : pv;
    }
    for (int kb = 0; kb < nkb; kb += 2) {
        wait_vmcnt<0>();
        lds_barrier();
        prio(kb);
        if (kb + 1 < nkb) issue(kb + 1, g_kv1);
        block(kb, g_kv0);
        if (kb + 1 >= nkb) break;
        wait_vmcnt<0>();
        lds_barrier();
        if (kb + 2 < nkb) issue(kb + 2, g_kv0);
        block(kb + 1, g_kv1);
    }

    // ---- finalise: null merge, channels, output ------------------------------------------------
    const float L = pair_sum((lsum[0] + lsum[1]) + (lsum[2] + lsum[3]));
    if constexpr (!POLAR) {  // plain softmax: o = Sv / L
        const float invL = 1.0f / L;
        if (qi < T) {
            bf16* orow = o + (seq0 + qi) * qstride + (size_t)h * D;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    bf16x4 y;
#pragma unroll
                    for (int x = 0; x < 4; ++x) y[x] = (bf16)(oacc[dt][4 * g + x] * invL);
                    *(bf16x4*)(orow + 32 * dt + 8 * g + 4 * G2) = y;
                }
        }
        return;
    }
    const float Q2 = pair_sum((q2sum[0] + q2sum[1]) + (q2sum[2] + q2sum[3]));
    // the row scalars with the hardware's log, exp, square root and reciprocal (errors of a few
    // fp32 ulps, far below the bf16 output's rounding; the IEEE library forms cost ~3% at 2K)
    const float s_nu = g_par[D], nbias = g_par[D + 1], mbeta = g_par[D + 2];
    const float n = (float)(qi + 1);
    const float t = 1.0f + a_t * __logf(n);
    const float nu = nbias + s_nu * __builtin_sqrtf(__logf(n + 1.0f));
    const float lnull = t * nu * kLog2e;
    const float Ms = fmaxf(m_used, lnull);
    const float pn = fast_exp2(lnull - Ms);
    const float f = fast_exp2(m_used - Ms);
    const float Ls = L * f;
    const float Z = Ls + pn;
    const float invZ = __builtin_amdgcn_rcpf(Z);
    const float neff = L * L * __builtin_amdgcn_rcpf(Q2);
    const float meff = neff * (Ls * invZ);
    const float xarg = mbeta * __logf(1.0f + meff);
    const float em = __expf(-2.0f * xarg);
    const float mu = (1.0f - em) * __builtin_amdgcn_rcpf(1.0f + em);
    float nrm2 = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 vn = *(const f32x4*)&g_par[32 * dt + 8 * g + 4 * G2];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const float sv = (oacc[dt][4 * g + x] * f + pn * vn[x]) * invZ;
                oacc[dt][4 * g + x] = sv;
                nrm2 += sv * sv;
            }
        }
    nrm2 = pair_sum(nrm2);
    const float scale = mu * __builtin_amdgcn_rcpf(fmaxf(__builtin_sqrtf(nrm2), prm.eps));
    if (qi < T) {
        bf16* orow = o + (seq0 + qi) * qstride + (size_t)h * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 y;
#pragma unroll
                for (int x = 0; x < 4; ++x) y[x] = (bf16)(oacc[dt][4 * g + x] * scale);
                *(bf16x4*)(orow + 32 * dt + 8 * g + 4 * G2) = y;
            }
        if (G2 == 0) {
            const size_t si = mu_base + qi;
            if (mu_out) mu_out[si] = mu;
            if (meff_out) meff_out[si] = meff;
        }
        if (stats) {  // training: what the backward pass reads instead of recomputing the row
            const float nrm = sqrtf(nrm2);
            if (G2 == 0) {
                // base-2 log partition in the scaled logit units (weight = exp2(cq q.k - lse2)), real
                // mass, squared mass of the normalised weights, and the normaliser (negative when
                // the eps clamp was taken)
                const f32x4 st = {Ms + fast_log2(Z), Ls * invZ, Q2 * f * f * invZ * invZ, nrm > prm.eps ? nrm : -prm.eps};
                *(f32x4*)(stats + (mu_base + qi) * 4) = st;
            }
            const float invden = 1.0f / fmaxf(nrm, prm.eps);
            float* drow = dir + (seq0 + qi) * qstride + (size_t)h * D;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    f32x4 y;
#pragma unroll
                    for (int x = 0; x < 4; ++x) y[x] = oacc[dt][4 * g + x] * invden;
                    *(f32x4*)(drow + 32 * dt + 8 * g + 4 * G2) = y;
                }
        }
    }
  };

    const int second = (paired && pr != nqt - 1 - pr) ? (min(T, pr * BQ + BQ) + BK - 1) / BK : 0;
    tile(nqt - 1 - pr, second, true);
    if (second) {
        lds_barrier();  // every wave is done with the stages before they are refilled
        tile(pr, 0, false);
    }
}

}  // namespace

hipError_t launch_polar_fwd(const PolarFwdArgs& a, hipStream_t stream) {
    const int nqt = (a.T + BQ - 1) / BQ;
    const long long ntiles = (long long)nqt * a.Hq * a.B;
    if (ntiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    // pair tiles when there are at most about two rounds of workgroups (4 per CU on 256 CUs)
    const int paired = ntiles <= 2048 * 2 ? 1 : 0;
    const int per_bh = paired ? (nqt + 1) / 2 : nqt;
#define ATMA_PF_LAUNCH(DD, POL)                                                                            \
    hipLaunchKernelGGL((polar_fwd_kernel<DD, POL>), dim3(per_bh * a.Hq * a.B), dim3(NT), 0, stream,        \
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.p, (bf16*)a.o,               \
                       POL ? a.mu_out : nullptr, POL ? a.meff_out : nullptr, POL ? a.stats : nullptr,         \
                       POL ? a.dir : nullptr, a.T, a.Hq, a.Hkv, paired, a.cu, a.total)
    if (a.D == 64) {
        if (a.softmax) ATMA_PF_LAUNCH(64, false);
        else ATMA_PF_LAUNCH(64, true);
    } else if (a.D == 128) {
        if (a.softmax) ATMA_PF_LAUNCH(128, false);
        else ATMA_PF_LAUNCH(128, true);
    } else {
        return hipErrorInvalidValue;
    }
#undef ATMA_PF_LAUNCH
    return hipGetLastError();
}

}  // namespace atma

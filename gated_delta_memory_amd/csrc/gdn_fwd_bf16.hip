// Gated-delta memory, chunked prefill, bf16 inputs, for gfx950.
//
// Chunk algebra (exact rewrite of the ATMA paper's Section 3.3 recurrence, derivation in
// gdn_fwd.hip): for a chunk of C = 64 tokens entering with state S_in,
//     Delta = U - W S_in^T,  S_out^T = e^{g_last} S_in^T + KD^T Delta,
//     O     = QG S_in^T + P Delta,
// with W = Tinv diag(beta e^g) K, U = Tinv diag(beta) V, Tinv = (I + A)^{-1},
// QG = diag(e^g) Q, KD = diag(e^{g_last - g}) K and P = lower_incl((Q K^T) o E).
//
// Three kernels; only the middle one is sequential along the sequence:
//   gdn_prep_h  (parallel over chunks) - A, Tinv (fp32), W and U from an fp32-accurate
//               hi/lo bf16 split of Tinv, and KD^T; writes them as fp16 tiles already in
//               the carry's MFMA-fragment order, plus the chunk's g for the output kernel.
//               A and Tinv share one 64 x 64 tile (A transposed above the diagonal, Tinv
//               below), so its LDS fits four workgroups per CU.  When the carry forms the
//               output, prep also writes P and QG as fp16 fragments.
//   gdn_carry_h (one workgroup per 64 state rows of a (batch, head), walks the chunks)
//               keeps S^T in fp32 MFMA accumulators; per chunk it only forms Delta and the
//               state update (32 MFMAs per wave), streaming W, KD^T and its U slice through
//               three LDS stages with direct global->LDS copies issued two chunks ahead.
//               It writes the fp16 operands it built anyway -- S_in^T and Delta, in MFMA
//               fragment order -- for the output kernel; or, in its two-wave form (grids
//               too small to fill the GPU), hands them through LDS to two output waves of
//               the same workgroup, which form O = QG S_in^T + P Delta for its 32 columns
//               while the carry goes on (no output kernel, no S_in^T / Delta records).
//   gdn_out_h   (parallel over chunks, after the four-wave carry) - QG and P from the bf16
//               Q and K tiles, then O = QG S_in^T + P Delta, coalesced bf16 stores.
// Long sequences with few (batch, head) pairs leave most of the GPU idle during the carry, so
// the sequence is cut into segments.  Per chunk the state map is affine in S,
//     S_out = S_in A_c + B_c,  A_c = e^{g_last} I - W^T KD,  B_c = U^T KD,
// and so is a whole segment: S_end = S_start A_seg + B_seg.  A summary pass (the carry
// kernel in summary mode, all segments in parallel) runs the segment from S_start = 0 for the
// Dv real state rows (giving B_seg) and from S_start = I with U = 0 for Dk extra rows (giving
// A_seg); gdn_seg_scan then walks the segments in order, S_start(s+1) = S_start(s) A_seg(s) +
// B_seg(s) in fp32, and the carry proper runs every segment in parallel from its S_start.
// fp16 staging (11-bit mantissa) keeps the result within a few 1e-3 of the fp64
// recurrence; it needs |v| and the state entries below 2^15.
#include "gdn_common.hpp"
#include "launch.hpp"

namespace atma {
namespace {

using gdn::C;
using gdn::NT;
using gdn::TileRegs;
using gdn::copy_out;

// ---- workspace layout ------------------------------------------------------------------
// Per chunk, in separate arrays indexed by chunk id = (b H + h) NC + c:
//   RA : W [C][DK] | KDT [DK][C] | U slices [DV/64] x 8 KB      (read by the carry kernel)
//   RB : g [C] (fp32 cumulative log decay)                       (read by the output kernel)
// (W and KDT fragment-major, U slices in the carry's accumulator order; see below)
//   SF : S_in^T fragments [DV/64][DK/32][4 waves][64 lanes] x 16 B
//   DF : Delta fragments  [DV/64][2][4 waves][64 lanes] x 16 B
//   EGL: e^{g_last} (fp32)
// When the carry forms the output itself (see gdn_carry_h), SF and DF are not needed; instead
//   RP : P fragments [4][2][64 lanes] x 16 B | QG fragments [4][DK/32][64 lanes] x 16 B
//        (fragment-major fp16 A operands of O = QG S_in^T + P Delta, written by the prep kernel)
template <int DK, int DV> struct Lay {
    static constexpr int RBK = DK * 2;  // bytes per W / QG row
    static constexpr size_t A_W = 0;
    static constexpr size_t A_KDT = A_W + (size_t)C * DK * 2;
    static constexpr size_t A_U = A_KDT + (size_t)DK * C * 2;
    static constexpr size_t USLICE = (size_t)C * 64 * 2;
    static constexpr size_t RA = A_U + (size_t)(DV / 64) * USLICE;
    static constexpr size_t RB = (size_t)C * sizeof(float);  // g_r of the chunk (for the output kernel)
    static constexpr size_t SF = (size_t)DV * DK * 2;
    static constexpr size_t DF = (size_t)C * DV * 2;
    static constexpr size_t STAGE = A_U + USLICE;  // bytes one carry workgroup streams per chunk
    static constexpr size_t P_OFF = 0, QG_OFF = (size_t)4 * 2 * 1024;
    static constexpr size_t RP = QG_OFF + (size_t)4 * (DK / 32) * 1024;
    static size_t total(size_t nchunks, bool fused) {  // + seg_bytes
        return nchunks * (RA + RB + (fused ? RP : SF + DF) + sizeof(float));
    }
};

struct Regions {
    char *ra, *rb, *sf, *df, *rp;  // sf, df without the fused output; rp with it
    float* egl;
    float* seg;  // segment summaries [B H][nseg][Dv + Dk rows][Dk]: B_seg rows, then A_seg rows
    float* sst;  // segment start states [B H][nseg][Dv][Dk]
};
template <int DK, int DV>
Regions regions(void* ws, size_t nchunks, size_t nbh, int nseg, bool fused) {
    using L = Lay<DK, DV>;
    char* p = (char*)ws;
    Regions r;
    r.ra = p;
    r.rb = r.ra + nchunks * L::RA;
    char* e = r.rb + nchunks * L::RB;
    if (fused) {
        r.sf = r.df = nullptr;
        r.rp = e;
        e += nchunks * L::RP;
    } else {
        r.rp = nullptr;
        r.sf = e;
        r.df = r.sf + nchunks * L::SF;
        e = r.df + nchunks * L::DF;
    }
    r.egl = (float*)e;
    char* q = (char*)(r.egl + nchunks);
    q += (256 - (size_t)q % 256) % 256;
    r.seg = nseg > 1 ? (float*)q : nullptr;
    r.sst = nseg > 1 ? r.seg + nbh * nseg * (size_t)(DV + DK) * DK : nullptr;
    return r;
}
template <int DK, int DV>
size_t seg_bytes(size_t nbh, int nseg) {
    return nseg > 1 ? 256 + nbh * nseg * ((size_t)(DV + DK) * DK + (size_t)DV * DK) * sizeof(float) : 0;
}

// Number of segments: a cost model over the carry's per-chunk step (about 1.3 us) and the
// scan's per-segment step (about 1.5 us), with one carry workgroup per CU on 256 CUs.
int choose_nseg(int B, int T, int H, int Dk, int Dv) {
    const int NC = (T + C - 1) / C;
    const double bh = (double)B * H, tc = 1.3, ts = 1.5;
    auto rounds = [](double wgs) { return wgs <= 256.0 ? 1.0 : (double)(long long)((wgs + 255.0) / 256.0); };
    int best = 1;
    double best_cost = rounds(bh * Dv / 64) * NC * tc;
    for (int g = 2; g <= 64 && 4 * g <= NC; g *= 2) {
        const int len = (NC + g - 1) / g;
        const double cost = (rounds(bh * g * (Dv + Dk) / 64) + rounds(bh * g * Dv / 64)) * len * tc + g * ts;
        if (cost < best_cost) {
            best = g;
            best_cost = cost;
        }
    }
    const int len = (NC + best - 1) / best;
    return (NC + len - 1) / len;  // every segment non-empty
}

// Two-wave carry workgroups (32 state rows each) when four-wave ones would leave more than half
// of the 256 CUs idle; those carry workgroups also form the output (a third wave), so the S_in^T
// and Delta records never go through memory and there is no output kernel.
bool small_carry(int B, int H, int nseg, int Dv) { return (long long)H * nseg * B * (Dv / 64) * 2 <= 256; }

// ---- fragment-major tiles -----------------------------------------------------------------
// An R x K fp16 MFMA A-operand tile is stored as its fragments, [R/16][K/32][64 lanes][8]:
// element (r, k) sits in fragment (r/16, k/32), lane (r mod 16) + 16 G, slot e, where
// k mod 32 = kmap(G, e).  A consumer wave then loads each fragment with one 16-byte LDS read
// per lane (a contiguous, conflict-free 1 KB), with no swizzle arithmetic or repacking.
template <int K>
__device__ __forceinline__ constexpr int fm_off(int r, int k) {  // byte offset of element (r, k)
    const int kk = k & 31;
    const int G = (kk & 15) >> 2;
    const int e = (kk & 3) + ((kk >> 4) << 2);
    return ((((r >> 4) * (K / 32) + (k >> 5)) * 64 + (r & 15) + 16 * G) * 8 + e) * 2;
}
template <int K>
__device__ __forceinline__ f16x8 fm_frag(const char* tile, int rt, int kb) {
    return *(const f16x8*)(tile + ((rt * (K / 32) + kb) * 64 + lane_id()) * 16);
}
// U slice for the carry kernel: [4 waves][4 row tiles][64 lanes] x 4 fp16, lane (l16 + 16 G)
// of wave w holding U[16 i + 4 G + x][16 w + l16], x = 0..3 (its accumulator layout).
__device__ __forceinline__ constexpr int u_off(int w, int i, int lane) { return ((w * 4 + i) * 64 + lane) * 8; }

// =========================================================================================
// prep
// =========================================================================================
template <int DK, int DV>
struct PrepSmem {
    static constexpr int LDK = (DK > DV ? DK : DV) + 8, LDX = LDK, LDA = C + 4;
    bf16 Ks[C * LDK];   // K, then V once W is formed
    // AT[r][c]: Tinv[r][c] for c <= r (its diagonal blocks in full, zeros above the diagonal
    // included) and A[c][r] for c < r outside the diagonal blocks (A is strictly lower, so its
    // transpose fits above the diagonal; A's diagonal blocks are read once, by the inverse of
    // those blocks, before Tinv's overwrite them).  Later the W staging tile, then the U
    // staging tile.
    float AT[C * LDA];
    float Gs[C];  // g_r = sum_{s <= r} ln alpha_s
    float Bs[C];  // beta_r
    float Es[C];  // beta_r e^{g_r}
};
static_assert(sizeof(float) * 64 * 68 >= 64 * 128 * 2, "the staging tiles fit the A / Tinv tile");

// B fragment (kmap order over the chunk positions) of a row-major bf16 LDS tile, columns
// 16 ct .. 16 ct + 15, by two transpose reads.
__device__ __forceinline__ Frag<bf16> bfrag_tr(const bf16* tile, int ld, int ct, int kb) {
    const int G = lane_id() >> 4, l16 = lane_id() & 15;
    const char* base = (const char*)tile;
    const int col = 16 * ct + 4 * (l16 & 3);
    const s16x4 r0 = tr_read_b16(base + ((32 * kb + 4 * G + (l16 >> 2)) * ld + col) * 2);
    const s16x4 r1 = tr_read_b16(base + ((32 * kb + 16 + 4 * G + (l16 >> 2)) * ld + col) * 2);
    Frag<bf16> f;
    f.v = __builtin_shufflevector(__builtin_bit_cast(bf16x4, r0), __builtin_bit_cast(bf16x4, r1), 0, 1, 2, 3, 4, 5,
                                  6, 7);
    return f;
}

template <int DK, int DV>
__global__ __launch_bounds__(NT, 4) void gdn_prep_h(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                    const bf16* __restrict__ v, const float* __restrict__ alpha,
                                                    const float* __restrict__ beta, Regions rg, int Tmax, int H,
                                                    const int* __restrict__ cu, int total) {
    using S = PrepSmem<DK, DV>;
    using L = Lay<DK, DV>;
    constexpr int LDK = S::LDK, LDX = S::LDX, LDA = S::LDA, RBK = L::RBK;
    extern __shared__ __align__(16) char smem_raw[];
    S& sm = *reinterpret_cast<S*>(smem_raw);

    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int NC = gridDim.x;  // chunk-record stride: chunks of the longest sequence
    size_t seq0;
    int Tlen;
    if (!gdn::seq_bounds(cu, b, Tmax, total, seq0, Tlen) || c * C >= Tlen) return;
    const int t0 = c * C;
    const int n = min(C, Tlen - t0);
    const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(wave_id()), G = lane >> 4, l16 = lane & 15;
    const size_t tok0 = (seq0 + t0) * H + h;
    const size_t cid = ((size_t)b * H + h) * NC + c;
    char* ra = rg.ra + cid * L::RA;
    char* rb = rg.rb + cid * L::RB;

    // ---- A: K into LDS, cumulative log decay ------------------------------------------------
    // (the gates are requested right behind the tile, so that they share one trip to memory)
    float a_in = 1.0f, b_in = 0.0f;
    {
        TileRegs<bf16, C, DK> kr;
        kr.load(k + tok0 * DK, (size_t)H * DK, n);
        if (w == 0) {
            const size_t gi = tok0 + (size_t)min(lane, n - 1) * H;  // rows past n re-read row n-1, then discarded
            a_in = alpha[gi];
            b_in = beta[gi];
        }
        kr.template store<LDK>(sm.Ks);
    }
    if (w == 0) {
        const bool ok = lane < n;
        float la = ok ? __logf(a_in) : 0.0f;
        const float be = ok ? b_in : 0.0f;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_up(la, o, 64);
            if (lane >= o) la += y;
        }
        sm.Gs[lane] = la;
        sm.Bs[lane] = be;
        sm.Es[lane] = be * __expf(la);
        ((float*)rb)[lane] = la;
        if (lane == C - 1) rg.egl[cid] = __expf(la);
    }
    __syncthreads();

    // ---- B: A = strict_lower(diag(beta) (K K^T) o E) in fp32, stored transposed --------------
    // (the ten tiles on or below the diagonal; lane (G, l16) holds rows r = 16 i + 4 G + x of
    // column s = 16 j + l16, which are consecutive in A^T)
    for (int ti = w; ti < 10; ti += 4) {
        const int i = (ti >= 6) ? 3 : (ti >= 3) ? 2 : (ti >= 1) ? 1 : 0;
        const int j = ti - i * (i + 1) / 2;
        const f32x4 gr = *(const f32x4*)&sm.Gs[16 * i + 4 * G];
        const f32x4 br = *(const f32x4*)&sm.Bs[16 * i + 4 * G];
        const float gs = sm.Gs[16 * j + l16];
        f32x4 kk = {0, 0, 0, 0};
        {
            // every fragment of the tile is requested before the first MFMA waits on one
            Frag<bf16> a[DK / 32], bk[DK / 32];
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                load_frag_rows(bk[kb], sm.Ks, LDK, 16 * j + l16, 32 * kb);
                load_frag_rows(a[kb], sm.Ks, LDK, 16 * i + l16, 32 * kb);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) mma(kk, a[kb], bk[kb]);
        }
        const int s = 16 * j + l16;
        f32x4 y;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int r = 16 * i + 4 * G + x;
            // g_r - g_s <= 0 wherever the mask keeps the entry (s < r)
            const float e = __expf(fminf(gr[x] - gs, 0.0f));
            y[x] = (s < r) ? br[x] * e * kk[x] : 0.0f;
        }
        *(f32x4*)&sm.AT[s * LDA + 16 * i + 4 * G] = y;
    }
    // V's load starts here (after the A tiles' fragments are dead) and lands after W is formed
    TileRegs<bf16, C, DV> vr;
    vr.template load<true>(v + tok0 * DV, (size_t)H * DV, n);

    // ---- C: KD^T, straight to the records ----------------------------------------------------
    {
        const float glast = sm.Gs[C - 1];
#pragma unroll
        for (int combo = w * 4 + G; combo < (DK / 16) * (C / 8); combo += 16) {
            const int cg = combo % (DK / 16), pc = 8 * (combo / (DK / 16));
            const f32x4 g0 = *(const f32x4*)&sm.Gs[pc], g1 = *(const f32x4*)&sm.Gs[pc + 4];
            const char* kbase = (const char*)sm.Ks;
            const int col = 16 * cg + 4 * (l16 & 3);
            const s16x4 r0 = tr_read_b16(kbase + ((pc + (l16 >> 2)) * LDK + col) * 2);
            const s16x4 r1 = tr_read_b16(kbase + ((pc + 4 + (l16 >> 2)) * LDK + col) * 2);
            const bf16x4 k0 = __builtin_bit_cast(bf16x4, r0), k1 = __builtin_bit_cast(bf16x4, r1);
            f16x8 y;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                y[t] = (half)((float)k0[t] * __expf(glast - g0[t]));
                y[t + 4] = (half)((float)k1[t] * __expf(glast - g1[t]));
            }
            *(f16x4*)(ra + L::A_KDT + fm_off<C>(16 * cg + l16, pc)) = __builtin_shufflevector(y, y, 0, 1, 2, 3);
            *(f16x4*)(ra + L::A_KDT + fm_off<C>(16 * cg + l16, pc + 4)) = __builtin_shufflevector(y, y, 4, 5, 6, 7);
        }
    }
    __syncthreads();  // A complete

    // ---- P and QG for a carry that forms the output (waves 1-3, while wave 0 solves the
    // diagonal blocks below) -----------------------------------------------------------------
    // (plain stores, like W, KD^T and U: at the 2K layer the records of a call fit the last-level
    // cache, from which the carry reads them back; streaming stores made the call 11% slower)
    // QG = diag(e^g) Q and P = lower_incl((Q K^T) o E) as fragment-major fp16 A operands.  P is
    // formed transposed, P^T = K Q^T, so that the accumulator of tile (jt, it) -- lane (l16, G)
    // holding P[16 it + l16][16 jt + 4 G + x] -- is already half of the A fragment (it, jt / 2).
    if (w != 0 && rg.rp) {
        char* rp = rg.rp + cid * L::RP;
        auto pq = [&](int it) {
            const int r = 16 * it + l16;
            const bf16* qrow = q + (tok0 + (size_t)min(r, n - 1) * H) * DK + 4 * G;  // rows past n: row n - 1
            Frag<bf16> qf[DK / 32];
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                const bf16x4 lo = *(const bf16x4*)(qrow + 32 * kb), hi = *(const bf16x4*)(qrow + 32 * kb + 16);
                qf[kb].v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
            const float gr = sm.Gs[r];
            const float eg = __expf(gr);
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                f16x8 y;
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = (half)((float)qf[kb].v[e] * eg);
                *(f16x8*)(rp + L::QG_OFF + ((it * (DK / 32) + kb) * 64 + lane) * 16) = y;
            }
            for (int jt = 0; jt <= it; ++jt) {
                Frag<bf16> kf[DK / 32];
#pragma unroll
                for (int kb = 0; kb < DK / 32; ++kb) load_frag_rows(kf[kb], sm.Ks, LDK, 16 * jt + l16, 32 * kb);
                f32x4 pt = {0, 0, 0, 0};
#pragma unroll
                for (int kb = 0; kb < DK / 32; ++kb) mma(pt, kf[kb], qf[kb]);
                const f32x4 gs = *(const f32x4*)&sm.Gs[16 * jt + 4 * G];
                f16x4 y;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int s2 = 16 * jt + 4 * G + x;
                    const float e = __expf(fminf(gr - gs[x], 0.0f));  // g_r - g_s <= 0 where s <= r
                    y[x] = (half)((s2 <= r) ? e * pt[x] : 0.0f);
                }
                *(f16x4*)(rp + L::P_OFF + ((it * 2 + (jt >> 1)) * 64 + lane) * 16 + (jt & 1) * 8) = y;
            }
            if ((it & 1) == 0)  // tile it + 1 of the same fragment lies above the diagonal
                *(f16x4*)(rp + L::P_OFF + ((it * 2 + (it >> 1)) * 64 + lane) * 16 + 8) = f16x4{0, 0, 0, 0};
        };
        pq(w);
        if (w == 3) pq(0);
    }

    // ---- D: Tinv = (I + A)^{-1} -----------------------------------------------------------
    if (w == 0) {
        // 16x16 diagonal blocks: lane (blk, col) solves column `col` of block `blk` by forward
        // substitution, a column of A at a time (a row of A^T: x[r] -= A[r][s] x[s], r > s, for
        // s = 0, 1, ..., so every x[r] takes its terms in the order of s)
        const int blk = lane >> 4, col = l16, o = 16 * blk;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == col) ? 1.0f : 0.0f;
#pragma unroll
        for (int s2 = 0; s2 < 15; ++s2) {
            float acol[16];
#pragma unroll
            for (int r4 = 0; r4 < 16; r4 += 4) {
                if (r4 + 3 > s2) {
                    const f32x4 v4 = *(const f32x4*)&sm.AT[(o + s2) * LDA + o + r4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) acol[r4 + u] = v4[u];
                }
            }
#pragma unroll
            for (int r = s2 + 1; r < 16; ++r) x[r] -= acol[r] * x[s2];
        }
        // the whole block, zeros above its diagonal included (after every read of the block)
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.AT[(o + r) * LDA + o + col] = x[r];
    }
    __syncthreads();
    for (int d = 1; d < 4; ++d) {
        if (w < 4 - d) {
            const int j = w, i = w + d;
            f32x4 acc = {0, 0, 0, 0};
            for (int m = j; m < i; ++m) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float av = sm.AT[(16 * m + 4 * G + e) * LDA + 16 * i + l16];  // A[16 i + l16][16 m + 4 G + e]
                    const float bv = sm.AT[(16 * m + 4 * G + e) * LDA + 16 * j + l16];  // Tinv, block (m, j), m >= j
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc, 0, 0, 0);
                }
            }
            f32x4 y = {0, 0, 0, 0};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float av = sm.AT[(16 * i + l16) * LDA + 16 * i + 4 * G + e];
                y = __builtin_amdgcn_mfma_f32_16x16x4f32(av, acc[e], y, 0, 0, 0);
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) sm.AT[(16 * i + 4 * G + x) * LDA + 16 * j + l16] = -y[x];
        }
        __syncthreads();
    }

    // ---- E: W = Tinv diag(beta e^g) K and U = Tinv diag(beta) V, hi/lo split of Tinv -------
    {
        const int i = w;  // row tile
        const int nkb = (i < 2) ? 1 : 2;
        Frag<bf16> wh[2], wl[2], uh[2], ul[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            // slots e < 4 hold chunk positions 32 kb + 4 G + e, slots e >= 4 hold 32 kb + 16 + 4 G + e - 4
            f32x4 tv[2], bv[2], ev[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int s0 = 32 * kb + 16 * hh + 4 * G;
                // blocks above the diagonal hold A: Tinv is zero there
                tv[hh] = 2 * kb + hh > i ? f32x4{0, 0, 0, 0} : *(const f32x4*)&sm.AT[(16 * i + l16) * LDA + s0];
                bv[hh] = *(const f32x4*)&sm.Bs[s0];
                ev[hh] = *(const f32x4*)&sm.Es[s0];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float t = tv[e >> 2][e & 3];
                const float tw = t * ev[e >> 2][e & 3];
                const float tu = t * bv[e >> 2][e & 3];
                const bf16 hw = (bf16)tw, hu = (bf16)tu;
                wh[kb].set_raw(e, hw);
                wl[kb].set(e, tw - (float)hw);
                uh[kb].set_raw(e, hu);
                ul[kb].set(e, tu - (float)hu);
            }
        }
        __syncthreads();  // Tinv consumed: AT becomes the W staging tile, then the U staging tile
        char* wstage = (char*)sm.AT;
        char* ustage = (char*)sm.AT;
        // B fragments are requested a group of column tiles at a time before their MFMAs (one
        // LDS round trip per group): two tiles for W, while V's tile is in flight in registers,
        // four for U
        Frag<bf16> bx[4][2];
        constexpr int GW = 2;
#pragma unroll
        for (int c0 = 0; c0 < DK / 16; c0 += GW) {
#pragma unroll
            for (int ct = 0; ct < GW; ++ct)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    if (kb < nkb) bx[ct][kb] = bfrag_tr(sm.Ks, LDK, c0 + ct, kb);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ct = 0; ct < GW; ++ct) {
                f32x4 acc = {0, 0, 0, 0};
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    if (kb < nkb) {
                        mma(acc, wh[kb], bx[ct][kb]);
                        mma(acc, wl[kb], bx[ct][kb]);
                    }
                }
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    *(half*)(wstage + fm_off<DK>(16 * i + 4 * G + x, 16 * (c0 + ct) + l16)) = (half)acc[x];
            }
        }
        __syncthreads();  // W staged, every wave is done with K: W goes out and V takes K's place
        copy_out(ra + L::A_W, wstage, C * DK * 2);
        vr.template store<LDX>(sm.Ks);
        __syncthreads();  // W has left the staging tile
#pragma unroll
        for (int c0 = 0; c0 < DV / 16; c0 += 4) {
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    if (kb < nkb) bx[ct][kb] = bfrag_tr(sm.Ks, LDX, c0 + ct, kb);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                f32x4 acc = {0, 0, 0, 0};
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    if (kb < nkb) {
                        mma(acc, uh[kb], bx[ct][kb]);
                        mma(acc, ul[kb], bx[ct][kb]);
                    }
                }
                f16x4 y;
#pragma unroll
                for (int x = 0; x < 4; ++x) y[x] = (half)acc[x];
                *(f16x4*)(ustage + ((c0 + ct) >> 2) * L::USLICE + u_off((c0 + ct) & 3, i, lane)) = y;
            }
        }
        __syncthreads();
        copy_out(ra + L::A_U, ustage, C * DV * 2);
    }
}

// =========================================================================================
// carry (sequential)
// =========================================================================================
// One LDS object per stage, so the compiler's wait-count analysis can tell the stage being
// read from the stages the asynchronous copies are filling.
constexpr int kStageMax = 40960 + 1024;  // tiles + e^{g_last} (one word per lane)
__shared__ __align__(16) char g_stage0[kStageMax];
__shared__ __align__(16) char g_stage1[kStageMax];
__shared__ __align__(16) char g_stage2[kStageMax];
// Fused output (two carry waves and two output waves): each carry wave's S_in^T and Delta
// fragments of a chunk, double-buffered, [2][2 waves][DK/32 + 2][64 lanes] x 16 B, and the output
// waves' staging tile of 64 rows x 32 columns (bf16, rows padded to 40; 32 rows per output wave).
constexpr int kHandMax = 2 * 2 * (128 / 32 + 2) * 1024;
constexpr int kOLD = 40;
__shared__ __align__(16) char g_hand[kHandMax];
__shared__ __align__(16) bf16 g_ostage[C * kOLD];

// byte offset of fragment `slot` of carry wave `wv` in hand-off buffer `buf` (this lane's 16 bytes)
template <int DK>
__device__ __forceinline__ int hand_off(int buf, int wv, int slot) {
    return ((buf * 2 + wv) * (DK / 32 + 2) + slot) * 1024 + lane_id() * 16;
}

// NW waves per workgroup (4, or 2 for grids too small to fill the GPU: 16 NW state rows per
// workgroup either way one 16-row band per wave); wave w of the workgroup is wave wq of the
// 64-row record slice sl (U slices, S_in^T and Delta fragments are laid out per 64 rows).
template <int DK, int DV, bool STORE, int NW, bool FUSE>
struct Carry {
    using L = Lay<DK, DV>;
    static constexpr int RBK = L::RBK, NKT = DK / 16, NTC = 64 * NW;
    static constexpr int NCH = (int)L::STAGE / 16;  // 16-byte copies per chunk
    static constexpr int TPT = NCH / NTC;            // tile copies per thread per chunk
    static constexpr int DPT = TPT + 1;              // all copies per thread per chunk (+ e^{g_last})
    static constexpr int SPT = STORE && !FUSE ? DK / 32 + 2 : 0;  // fragment stores per thread per chunk
    static_assert(!FUSE || (STORE && NW == 2 && DK <= 128), "the fused output serves the two-wave carry");
    static_assert(L::STAGE + 1024 <= kStageMax, "stage too large");
    static_assert(NCH % NTC == 0, "stage must be a whole number of copy rounds");
    static_assert(DPT + SPT < 64, "vmcnt range");

    const char* ra0;   // this (batch, head)'s first chunk record
    char* sf0;
    char* df0;
    const float* egl;
    int sl;       // U slice copied with each chunk
    float ukeep;  // 1 for real state rows, 0 for the identity rows of a segment summary
    int wq;       // this wave within the 64-row slice

    // Starts the copy of chunk c into `dst`.  The chunk's e^{g_last} is copied into the
    // stage too (every lane copies the same word, so all threads issue the same operations)
    // and read back from LDS: a plain global load carried across the loop would make the
    // compiler wait for every copy in flight.
    // The copies take a wave-uniform source base and LDS address (scalar registers) and a
    // per-lane 32-bit offset, so issuing one costs a handful of scalar instructions.
    __device__ __forceinline__ void issue(int c, char* dst) const {
        const int w = __builtin_amdgcn_readfirstlane(wave_id());
        const char* src = ra0 + (size_t)c * L::RA;
        const unsigned lds = gdn::lds_addr(dst) + (unsigned)(w * 64 * 16);
        gdn::lds_dma4((const void*)(egl + c), 0u, gdn::lds_addr(dst) + (unsigned)(L::STAGE + w * 256));
#pragma unroll
        for (int m = 0; m < TPT; ++m) {
            const unsigned ch = (unsigned)(m * NTC) + threadIdx.x;
            const unsigned off = ch * 16 < (unsigned)L::A_U
                                     ? ch * 16
                                     : (unsigned)(L::A_U + sl * L::USLICE) + (ch * 16 - (unsigned)L::A_U);
            gdn::lds_dma16((const void*)src, off, lds + (unsigned)(m * NTC * 16));
        }
    }

    __device__ __forceinline__ void step(int c, const char* sW, f32x4* st) const {
        const int lane = lane_id(), w = wq;
        const char* sK = sW + L::A_KDT;
        const char* sU = sW + L::A_U;
        // All LDS operands of the chunk are requested in two batches ahead of their MFMAs
        // (with one wave per SIMD nothing else hides LDS latency); the scheduling barriers
        // keep the compiler from sinking the reads next to their uses.
        f16x8 wf[4][DK / 32];
        f16x4 u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) wf[i][kb] = fm_frag<DK>(sW, i, kb);
            u[i] = *(const f16x4*)(sU + u_off(w, i, lane));
        }
        const float eg = *(const float*)(sW + L::STAGE);
        __builtin_amdgcn_sched_barrier(0);
        // S_in^T as fp16 B fragments; also kept for the output kernel
        Frag<half> sf[DK / 32];
        char* sfo = sf0 + (size_t)c * L::SF + (size_t)sl * (DK / 32) * 4096;
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
            acc_to_frag(sf[kb], st[2 * kb], st[2 * kb + 1]);
            if constexpr (FUSE) *(f16x8*)(g_hand + hand_off<DK>(c & 1, wave_id(), kb)) = sf[kb].v;
            else if constexpr (STORE) __builtin_nontemporal_store(sf[kb].v, (f16x8*)(sfo + ((kb * 4 + w) * 64 + lane) * 16));
        }
        f16x8 kf[NKT][2];
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) kf[t][kb] = fm_frag<C>(sK, t, kb);
        __builtin_amdgcn_sched_barrier(0);
        // Delta = U - W S_in^T
        f32x4 dl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) dl[i] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Frag<half> a;
                a.v = wf[i][kb];
                mma(dl[i], a, sf[kb]);
            }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int x = 0; x < 4; ++x) dl[i][x] = ukeep * (float)u[i][x] - dl[i][x];
        Frag<half> df[2];
        char* dfo = df0 + (size_t)c * L::DF + (size_t)sl * 2 * 4096;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            acc_to_frag(df[kb], dl[2 * kb], dl[2 * kb + 1]);
            if constexpr (FUSE) *(f16x8*)(g_hand + hand_off<DK>(c & 1, wave_id(), DK / 32 + kb)) = df[kb].v;
            else if constexpr (STORE) __builtin_nontemporal_store(df[kb].v, (f16x8*)(dfo + ((kb * 4 + w) * 64 + lane) * 16));
        }
        // S_out^T = e^{g_last} S_in^T + KD^T Delta
#pragma unroll
        for (int t = 0; t < NKT; ++t) st[t] *= eg;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int t = 0; t < NKT; ++t) {
                Frag<half> a;
                a.v = kf[t][kb];
                mma(st[t], a, df[kb]);
            }
    }
};

// Pipeline: the copy of chunk c + 2 is issued while chunk c is computed, always (a chunk
// past the end re-copies the last one into a stage that is never read again), so every
// iteration issues the same operations: DPT copies (tiles and e^{g_last})
// and SPT fragment stores per thread.  Before chunk c >= 1 is read, the operations issued
// after its copy are at least the stores of chunk c - 1 and the copy of chunk c + 1; with
// in-order retirement, waiting until no more than DPT + SPT are outstanding is sufficient.
// Chunk 0 waits until only the copy of chunk 1 may be outstanding.
// One workgroup per CU (the three stages fill the LDS): let the scheduler use the whole
// register file to keep more LDS reads in flight.
//
// Grid (slices, H nseg, B); the workgroup walks the chunks of segment s of (b, h).
// STORE (the carry proper): Dv / 64 slices of real state rows, starting from the segment's
// start state (the initial state when there is one segment); writes the S_in^T and Delta
// fragments for the output kernel and, in the last segment, the final state.
// !STORE (segment summary): (Dv + Dk) / 64 slices; real rows start from zero, the Dk extra
// rows start from the identity with U ignored; the end state goes to the summary region.
//
// FUSE (two carry waves): two more waves form the output, rows 32 cw .. 32 cw + 31 each (cw = 0,
// 1).  In the interval after the barrier that opens carry step c, output wave cw forms its rows of
// chunk c - 1 from that chunk's S_in^T and Delta fragments, which the carry waves left in the LDS
// hand-off buffer (c - 1) & 1 during step c - 1 and overwrite only in step c + 1, and from the P
// and QG fragments prep wrote, requested three intervals ahead (three register sets, by chunk
// index mod 3; plain loads, so the four workgroups of a (batch, head) share them in the L2); the carry waves pass one more barrier after their last step, so both sides pass
// the same number.
template <int DK, int DV, int CW>
struct OutFrags {
    static constexpr int NKB = DK / 32, NP = CW == 0 ? 2 : 4;  // P fragments (it, kb), kb < (it < 2 ? 1 : 2)
    f16x8 pf[NP], qg[2][NKB];
    __device__ __forceinline__ void request(const char* r) {
        using L = Lay<DK, DV>;
        const int lane = lane_id();
#pragma unroll
        for (int f = 0; f < NP; ++f) {
            const int it = CW == 0 ? f : 2 + (f >> 1), kb = CW == 0 ? 0 : (f & 1);
            pf[f] = *(const f16x8*)(r + L::P_OFF + ((it * 2 + kb) * 64 + lane) * 16);
        }
#pragma unroll
        for (int il = 0; il < 2; ++il)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
                qg[il][kb] = *(const f16x8*)(r + L::QG_OFF + (((2 * CW + il) * NKB + kb) * 64 + lane) * 16);
    }
};

template <int DK, int DV, int CW>
__device__ __forceinline__ void carry_output_chunk(const OutFrags<DK, DV, CW>& fr, int cc, bf16* __restrict__ o,
                                                   size_t seq0, int tfirst, int Tlen, int H, int h, int col0) {
    constexpr int NKB = DK / 32;
    const int lane = lane_id(), G = lane >> 4, l16 = lane & 15, buf = cc & 1;
#pragma unroll
    for (int j = 0; j < 2; ++j) {  // the two carry waves' 16 state rows = 16 output columns each
        Frag<half> sf[NKB], df[2];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) sf[kb].v = *(const f16x8*)(g_hand + hand_off<DK>(buf, j, kb));
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) df[kb].v = *(const f16x8*)(g_hand + hand_off<DK>(buf, j, NKB + kb));
#pragma unroll
        for (int il = 0; il < 2; ++il) {
            const int i = 2 * CW + il;
            f32x4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                Frag<half> a;
                a.v = fr.qg[il][kb];
                mma(acc, a, sf[kb]);
            }
#pragma unroll
            for (int kb = 0; kb < (CW == 0 ? 1 : 2); ++kb) {
                Frag<half> a;
                a.v = fr.pf[CW == 0 ? il : 2 * il + kb];
                mma(acc, a, df[kb]);
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) g_ostage[(16 * i + 4 * G + x) * kOLD + 16 * j + l16] = (bf16)acc[x];
        }
    }
    // this wave's 32 rows of 32 columns (64 bytes each) out
    const int t0 = tfirst + cc * C, nrow = min(C, Tlen - t0);
#pragma unroll
    for (int m = 2 * CW; m < 2 * CW + 2; ++m) {
        const int r = (lane >> 2) + 16 * m, qd = lane & 3;
        const u32x4 y = *(const u32x4*)&g_ostage[r * kOLD + 8 * qd];
        if (r < nrow) __builtin_nontemporal_store(y, (u32x4*)(o + ((seq0 + t0 + r) * H + h) * DV + col0 + 8 * qd));
    }
}

template <int DK, int DV, int CW>
__device__ __forceinline__ void carry_output(const char* rp0, bf16* __restrict__ o, size_t seq0, int tfirst, int Tlen,
                                             int H, int h, int col0, int n) {
    using L = Lay<DK, DV>;
    OutFrags<DK, DV, CW> f0, f1, f2;  // chunks of index 0, 1, 2 mod 3
    f0.request(rp0);
    if (1 < n) f1.request(rp0 + L::RP);
    for (int c = 0; c <= n; c += 3) {
        gdn::lds_barrier();  // opens carry step c (or follows the last one)
        if (c > 0) carry_output_chunk<DK, DV, CW>(f2, c - 1, o, seq0, tfirst, Tlen, H, h, col0);
        if (c + 2 < n) f2.request(rp0 + (size_t)(c + 2) * L::RP);
        if (c + 1 > n) break;
        gdn::lds_barrier();
        carry_output_chunk<DK, DV, CW>(f0, c, o, seq0, tfirst, Tlen, H, h, col0);
        if (c + 3 < n) f0.request(rp0 + (size_t)(c + 3) * L::RP);
        if (c + 2 > n) break;
        gdn::lds_barrier();
        carry_output_chunk<DK, DV, CW>(f1, c + 1, o, seq0, tfirst, Tlen, H, h, col0);
        if (c + 4 < n) f1.request(rp0 + (size_t)(c + 4) * L::RP);
    }
}

template <int DK, int DV, bool STORE, int NW, bool FUSE>
__global__ __launch_bounds__(64 * (NW + (FUSE ? 2 : 0)), 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void gdn_carry_h(
    Regions rg, const float* init_state, float* final_state, int Tmax, int H, int nseg, int seglen,
    const int* __restrict__ cu, int total, bf16* __restrict__ o) {
    using L = Lay<DK, DV>;
    using K = Carry<DK, DV, STORE, NW, FUSE>;
    constexpr int NKT = DK / 16;
    // slices of one (b, h, segment) on one XCD (workgroup i runs on XCD i % 8)
    const int nsl = (int)gridDim.x, nwg = nsl * (int)gridDim.y * (int)gridDim.z;
    const int wgi = (int)(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
    const int per = nwg >> 3, extra = nwg & 7, xcd = wgi & 7;
    const int item = xcd * per + min(xcd, extra) + (wgi >> 3);
    const int sl = item % nsl, yy = (item / nsl) % (int)gridDim.y, b = item / (nsl * (int)gridDim.y);
    const int h = yy / nseg, sg = yy % nseg;
    const int lane = lane_id(), G = lane >> 4, l16 = lane & 15;
    const int wq = (sl % (4 / NW)) * NW + wave_id();  // wave within the 64-row slice
    const int sl64 = sl / (4 / NW);                     // 64-row slice
    size_t seq0;
    int Tlen;
    if (!gdn::seq_bounds(cu, b, Tmax, total, seq0, Tlen)) return;
    const int NC = (Tlen + C - 1) / C;         // this sequence's chunks
    const int NCs = (Tmax + C - 1) / C;        // chunk-record stride
    const int cb = sg * seglen, n = min(NC - cb, seglen);  // this segment's chunks (<= 0: none)
    const size_t bh = (size_t)b * H + h;
    const size_t c0 = bh * NCs + cb;
    if constexpr (FUSE) {
        if (wave_id() >= NW) {  // the output waves (uniform branches: whole waves)
            if (n > 0) {
                if (wave_id() == NW) carry_output<DK, DV, 0>(rg.rp + c0 * L::RP, o, seq0, cb * C, Tlen, H, h, 32 * sl, n);
                else carry_output<DK, DV, 1>(rg.rp + c0 * L::RP, o, seq0, cb * C, Tlen, H, h, 32 * sl, n);
            }
            return;
        }
    }
    const bool real = sl64 < DV / 64;
    const K k{rg.ra + c0 * L::RA, rg.sf + c0 * L::SF, rg.df + c0 * L::DF, rg.egl + c0, real ? sl64 : 0,
              real ? 1.0f : 0.0f, wq};
    const int row = sl64 * 64 + 16 * wq + l16;  // state row held by this lane's accumulators

    f32x4 st[NKT];  // st[t][x] = S[row][16 t + 4 G + x]
    if constexpr (STORE) {
        const float* src = nseg > 1 ? rg.sst + (bh * nseg + sg) * DV * DK : init_state ? init_state + bh * DV * DK
                                                                                      : nullptr;
#pragma unroll
        for (int t = 0; t < NKT; ++t)
            st[t] = src ? *(const f32x4*)(src + (size_t)row * DK + 16 * t + 4 * G) : f32x4{0, 0, 0, 0};
    } else {
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
            for (int x = 0; x < 4; ++x) st[t][x] = (!real && 16 * t + 4 * G + x == row - DV) ? 1.0f : 0.0f;
    }

    gdn::wait_vmcnt<0>();  // initial state in registers before the untracked copies start
    // the end state: final state (last segment) or segment summary
    auto finish = [&]() {
        if constexpr (STORE) {
            if (final_state && sg == nseg - 1) {
#pragma unroll
                for (int t = 0; t < NKT; ++t)
                    *(f32x4*)(final_state + (bh * DV + row) * DK + 16 * t + 4 * G) = st[t];
            }
        } else {
            float* dst = rg.seg + ((bh * nseg + sg) * (DV + DK) + row) * DK;
#pragma unroll
            for (int t = 0; t < NKT; ++t) *(f32x4*)(dst + 16 * t + 4 * G) = st[t];
        }
    };
    // A segment past the end of a (packed) sequence has no chunks: its map is the identity, so
    // it only passes its start state on.
    if (n <= 0) {
        finish();
        return;
    }
    const int last = n - 1;
    const int NC_seg = n;
    k.issue(0, g_stage0);
    k.issue(min(1, last), g_stage1);
    gdn::wait_vmcnt<K::DPT>();
    gdn::lds_barrier();
    k.issue(min(2, last), g_stage2);
    k.step(0, g_stage0, st);
    for (int c = 1; c < NC_seg; c += 3) {
        gdn::wait_vmcnt<K::DPT + K::SPT>();
        gdn::lds_barrier();
        k.issue(min(c + 2, last), g_stage0);
        k.step(c, g_stage1, st);
        if (c + 1 >= NC_seg) break;
        gdn::wait_vmcnt<K::DPT + K::SPT>();
        gdn::lds_barrier();
        k.issue(min(c + 3, last), g_stage1);
        k.step(c + 1, g_stage2, st);
        if (c + 2 >= NC_seg) break;
        gdn::wait_vmcnt<K::DPT + K::SPT>();
        gdn::lds_barrier();
        k.issue(min(c + 4, last), g_stage2);
        k.step(c + 2, g_stage0, st);
    }
    if constexpr (FUSE) gdn::lds_barrier();  // the output waves read the last chunk's hand-off after it
    finish();
}

// =========================================================================================
// segment scan (sequential over segments, parallel over 16-row blocks of the state)
// =========================================================================================
// Grid (Dv / 16, H, B), 4 waves.  The workgroup owns state rows 16 rt .. 16 rt + 15 of (b, h)
// (rows of S evolve independently): S_start(0) = initial state (or 0), S_start(s + 1) =
// S_start(s) A_seg(s) + B_seg(s), exact fp32 products on v_mfma_f32_16x16x4_f32.  Wave w
// computes output column tiles w, w + 4, ...
template <int DK, int DV>
struct ScanSmem {
    static constexpr int LDS_S = DK + 4, LDS_A = DK + 16;  // strides with conflict-free operand reads
    float S[16 * LDS_S];
    float A[DK * LDS_A];
};
template <int DK, int DV>
__global__ __launch_bounds__(NT) void gdn_seg_scan(Regions rg, const float* init_state, int H, int nseg) {
    using S = ScanSmem<DK, DV>;
    constexpr int LDS_S = S::LDS_S, LDS_A = S::LDS_A;
    extern __shared__ __align__(16) char smem_raw[];
    S& sm = *reinterpret_cast<S*>(smem_raw);
    const int rt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = lane_id(), w = wave_id(), G = lane >> 4, l16 = lane & 15;
    const size_t bh = (size_t)b * H + h;
    // start state rows into LDS and out as S_start(0)
    for (int i = threadIdx.x; i < 16 * DK / 4; i += NT) {
        const int r = i / (DK / 4), c4 = i % (DK / 4);
        const size_t gi = (bh * DV + 16 * rt + r) * DK + 4 * c4;
        const f32x4 x = init_state ? *(const f32x4*)(init_state + gi) : f32x4{0, 0, 0, 0};
        *(f32x4*)&sm.S[r * LDS_S + 4 * c4] = x;
        *(f32x4*)(rg.sst + bh * nseg * DV * DK + (size_t)(16 * rt + r) * DK + 4 * c4) = x;
    }
    // A_seg(sg) travels through registers one step ahead (its loads overlap the MFMAs of the
    // previous step), B_seg(sg) rows go straight into the accumulators.
    constexpr int AR = DK * DK / 4 / NT;
    f32x4 areg[AR];
    f32x4 breg[DK / 64];
    auto load_ab = [&](int sg) {
        const float* sum = rg.seg + (bh * nseg + sg) * (DV + DK) * DK;
#pragma unroll
        for (int m = 0; m < AR; ++m) {
            const int i = threadIdx.x + m * NT, r = i / (DK / 4), c4 = i % (DK / 4);
            areg[m] = *(const f32x4*)(sum + (size_t)(DV + r) * DK + 4 * c4);
        }
#pragma unroll
        for (int j = 0; j < DK / 64; ++j)
#pragma unroll
            for (int x = 0; x < 4; ++x) breg[j][x] = sum[(size_t)(16 * rt + 4 * G + x) * DK + 16 * (w + 4 * j) + l16];
    };
    auto store_a = [&]() {
#pragma unroll
        for (int m = 0; m < AR; ++m) {
            const int i = threadIdx.x + m * NT, r = i / (DK / 4), c4 = i % (DK / 4);
            *(f32x4*)&sm.A[r * LDS_A + 4 * c4] = areg[m];
        }
    };
    if (nseg > 1) {
        load_ab(0);
        store_a();
    }
    __syncthreads();
    for (int sg = 0; sg + 1 < nseg; ++sg) {
        f32x4 acc[DK / 64];
#pragma unroll
        for (int j = 0; j < DK / 64; ++j) acc[j] = breg[j];
        if (sg + 2 < nseg) load_ab(sg + 1);
#pragma unroll
        for (int j = 0; j < DK / 64; ++j) {
            const int ct = w + 4 * j;
#pragma unroll 8
            for (int kk = 0; kk < DK / 4; ++kk)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.S[l16 * LDS_S + 4 * kk + G],
                                                              sm.A[(4 * kk + G) * LDS_A + 16 * ct + l16], acc[j],
                                                              0, 0, 0);
        }
        __syncthreads();  // every wave is done reading S and A
        float* nxt = rg.sst + (bh * nseg + sg + 1) * DV * DK;
#pragma unroll
        for (int j = 0; j < DK / 64; ++j) {
            const int ct = w + 4 * j;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                sm.S[(4 * G + x) * LDS_S + 16 * ct + l16] = acc[j][x];
                nxt[(size_t)(16 * rt + 4 * G + x) * DK + 16 * ct + l16] = acc[j][x];
            }
        }
        if (sg + 2 < nseg) store_a();
        __syncthreads();
    }
}

// =========================================================================================
// output
// =========================================================================================
// The output kernel forms P = lower_incl((Q K^T) o E) and QG = diag(e^{g}) Q itself from the
// bf16 inputs (its MFMA operands in fp16, fragment-major in LDS), then
// O = QG S_in^T + P Delta with the S_in^T and Delta fragments the carry wrote.  The K tile's
// space takes QG once P is built, and the Q tile's space takes the output staging once QG is
// built, so three workgroups fit a CU.
template <int DK, int DV>
struct OutSmem {
    static constexpr int LDQ = DK + 8, LDO = DV + 8;
    static constexpr int A_BYTES = C * LDQ * 2 > C * LDO * 2 ? C * LDQ * 2 : C * LDO * 2;
    static constexpr int B_BYTES = C * LDQ * 2 > C * DK * 2 ? C * LDQ * 2 : C * DK * 2;
    __align__(16) char ra[A_BYTES];  // Q tile (bf16, row stride LDQ), then the output staging (LDO)
    __align__(16) char rb[B_BYTES];  // K tile (bf16, row stride LDQ), then QG (fragment-major fp16)
    __align__(16) char pm[C * C * 2];  // P, fragment-major fp16
    float Gs[C];
};

template <int DK, int DV>
__global__ __launch_bounds__(NT, 3) void gdn_out_h(const bf16* __restrict__ q, const bf16* __restrict__ k, Regions rg,
                                                   bf16* __restrict__ o, int Tmax, int H, const int* __restrict__ cu,
                                                   int total) {
    using L = Lay<DK, DV>;
    using S = OutSmem<DK, DV>;
    constexpr int LDQ = S::LDQ, LDO = S::LDO;
    extern __shared__ __align__(16) char smem_raw[];
    S& sm = *reinterpret_cast<S*>(smem_raw);
    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int NC = gridDim.x;  // chunk-record stride
    size_t seq0;
    int Tlen;
    if (!gdn::seq_bounds(cu, b, Tmax, total, seq0, Tlen) || c * C >= Tlen) return;
    const int t0 = c * C, n = min(C, Tlen - t0);
    const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(wave_id()), G = lane >> 4, l16 = lane & 15;
    const size_t cid = ((size_t)b * H + h) * NC + c;
    const size_t tok0 = (seq0 + t0) * H + h;
    // this wave's S_in^T and Delta fragments (n-tiles nt = w + 4 m of 16 state rows: carry slice
    // nt / 4, wave nt % 4), requested with the tiles so their trip to memory overlaps P and QG
    constexpr int NTW = DV / 64;
    Frag<half> sf[NTW][DK / 32], df[NTW][2];
    {
        const char* sfc = rg.sf + cid * L::SF;
        const char* dfc = rg.df + cid * L::DF;
#pragma unroll
        for (int m = 0; m < NTW; ++m) {
            const int sl = m, wp = w;
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb)
                sf[m][kb].v = __builtin_nontemporal_load(
                    (const f16x8*)(sfc + (size_t)sl * (DK / 32) * 4096 + ((kb * 4 + wp) * 64 + lane) * 16));
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                df[m][kb].v = __builtin_nontemporal_load(
                    (const f16x8*)(dfc + (size_t)sl * 2 * 4096 + ((kb * 4 + wp) * 64 + lane) * 16));
        }
    }
    {
        TileRegs<bf16, C, DK> qr, kr;
        qr.template load<true>(q + tok0 * DK, (size_t)H * DK, n);
        kr.load(k + tok0 * DK, (size_t)H * DK, n);
        if (threadIdx.x < C) sm.Gs[threadIdx.x] = ((const float*)(rg.rb + cid * L::RB))[threadIdx.x];
        qr.template store<LDQ>((bf16*)sm.ra);
        kr.template store<LDQ>((bf16*)sm.rb);
    }
    __syncthreads();
    const bf16* Qs = (const bf16*)sm.ra;
    const bf16* Ks = (const bf16*)sm.rb;
    // P tiles (i, j): the ten on or below the diagonal from Q K^T, the six above it zero
    for (int ti = w; ti < 16; ti += 4) {
        int i, j;
        if (ti < 10) {
            i = (ti >= 6) ? 3 : (ti >= 3) ? 2 : (ti >= 1) ? 1 : 0;
            j = ti - i * (i + 1) / 2;
        } else {
            const int uu = ti - 10;
            i = (uu < 3) ? 0 : (uu < 5) ? 1 : 2;
            j = (uu < 3) ? uu + 1 : (uu < 5) ? uu - 1 : 3;
        }
        const f32x4 gr = *(const f32x4*)&sm.Gs[16 * i + 4 * G];
        const float gs = sm.Gs[16 * j + l16];
        f32x4 qk = {0, 0, 0, 0};
        if (ti < 10) {
            Frag<bf16> a[DK / 32], bk[DK / 32];
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                load_frag_rows(bk[kb], Ks, LDQ, 16 * j + l16, 32 * kb);
                load_frag_rows(a[kb], Qs, LDQ, 16 * i + l16, 32 * kb);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) mma(qk, a[kb], bk[kb]);
        }
        const int s2 = 16 * j + l16;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int r = 16 * i + 4 * G + x;
            const float e = __expf(fminf(gr[x] - gs, 0.0f));  // g_r - g_s <= 0 where s <= r
            *(half*)(sm.pm + fm_off<C>(r, s2)) = (half)((s2 <= r) ? e * qk[x] : 0.0f);
        }
    }
    __syncthreads();  // P ready; the K tile is dead and QG takes its place
    // QG = diag(e^g) Q
#pragma unroll
    for (int id = threadIdx.x; id < C * DK / 8; id += NT) {
        const int r = id / (DK / 8), cc = id % (DK / 8);
        const float e = __expf(sm.Gs[r]);
        const bf16x8 x = *(const bf16x8*)&Qs[r * LDQ + 8 * cc];
        f16x8 y;
#pragma unroll
        for (int t = 0; t < 8; ++t) y[t] = (half)((float)x[t] * e);
        *(f16x4*)(sm.rb + fm_off<DK>(r, 8 * cc)) = __builtin_shufflevector(y, y, 0, 1, 2, 3);
        *(f16x4*)(sm.rb + fm_off<DK>(r, 8 * cc + 4)) = __builtin_shufflevector(y, y, 4, 5, 6, 7);
    }
    __syncthreads();  // QG ready; the Q tile is dead and the output staging takes its place
    const char* sQ = sm.rb;
    const char* sP = sm.pm;
#pragma unroll
    for (int m = 0; m < NTW; ++m) {
        const int nt = 4 * m + w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 acc = {0, 0, 0, 0};
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                Frag<half> a;
                a.v = fm_frag<DK>(sQ, i, kb);
                mma(acc, a, sf[m][kb]);
            }
#pragma unroll
            for (int kb = 0; kb < (i < 2 ? 1 : 2); ++kb) {
                Frag<half> a;
                a.v = fm_frag<C>(sP, i, kb);
                mma(acc, a, df[m][kb]);
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) ((bf16*)sm.ra)[(16 * i + 4 * G + x) * LDO + 16 * nt + l16] = (bf16)acc[x];
        }
    }
    __syncthreads();
    for (int id = threadIdx.x; id < C * (DV / 8); id += NT) {
        const int r = id / (DV / 8), cc = id % (DV / 8);
        if (r < n)
            __builtin_nontemporal_store(*(const u32x4*)((const bf16*)sm.ra + r * LDO + 8 * cc),
                                        (u32x4*)(o + ((seq0 + t0 + r) * H + h) * DV + 8 * cc));
    }
}

template <int DK, int DV>
hipError_t launch(const GdnFwdArgs& a, hipStream_t stream) {
    const int NC = (a.T + C - 1) / C;
    const size_t nbh = (size_t)a.B * a.H;
    const int nseg = choose_nseg(a.B, a.T, a.H, DK, DV);
    const int seglen = (NC + nseg - 1) / nseg;
    const bool fused = small_carry(a.B, a.H, nseg, DV);
    const Regions rg = regions<DK, DV>(a.workspace, nbh * NC, nbh, nseg, fused);
    const size_t prep_smem = sizeof(PrepSmem<DK, DV>), out_smem = sizeof(OutSmem<DK, DV>);
    const size_t scan_smem = sizeof(ScanSmem<DK, DV>);
    static const hipError_t attr = [&] {
        hipError_t e = ensure_lds_limit(gdn_prep_h<DK, DV>, prep_smem);
        if (e == hipSuccess) e = ensure_lds_limit(gdn_out_h<DK, DV>, out_smem);
        if (e == hipSuccess) e = ensure_lds_limit(gdn_seg_scan<DK, DV>, scan_smem);
        return e;
    }();
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((gdn_prep_h<DK, DV>), dim3(NC, a.H, a.B), dim3(NT), prep_smem, stream, (const bf16*)a.q,
                       (const bf16*)a.k, (const bf16*)a.v, a.alpha, a.beta, rg, a.T, a.H, a.cu, a.total);
    // Carry workgroups hold 64 state rows with four waves, or 32 rows with two when four-wave
    // workgroups would leave more than half of the 256 CUs idle (one workgroup per CU: the LDS
    // stages fill it), so that the carry's LDS reads are spread over twice the CUs.  The two-wave
    // carry also forms the output (a third wave); after the four-wave carry the output kernel does.
    const long long units = (long long)a.H * nseg * a.B;
    if (nseg > 1) {
        if (units * ((DV + DK) / 64) * 2 <= 256)
            hipLaunchKernelGGL((gdn_carry_h<DK, DV, false, 2, false>), dim3((DV + DK) / 32, a.H * nseg, a.B), dim3(128),
                               0, stream, rg, a.init_state, a.final_state, a.T, a.H, nseg, seglen, a.cu, a.total,
                               nullptr);
        else
            hipLaunchKernelGGL((gdn_carry_h<DK, DV, false, 4, false>), dim3((DV + DK) / 64, a.H * nseg, a.B), dim3(NT),
                               0, stream, rg, a.init_state, a.final_state, a.T, a.H, nseg, seglen, a.cu, a.total,
                               nullptr);
        hipLaunchKernelGGL((gdn_seg_scan<DK, DV>), dim3(DV / 16, a.H, a.B), dim3(NT), scan_smem, stream, rg,
                           a.init_state, a.H, nseg);
    }
    if (fused) {
        hipLaunchKernelGGL((gdn_carry_h<DK, DV, true, 2, true>), dim3(DV / 32, a.H * nseg, a.B), dim3(256), 0, stream,
                           rg, a.init_state, a.final_state, a.T, a.H, nseg, seglen, a.cu, a.total, (bf16*)a.o);
    } else {
        hipLaunchKernelGGL((gdn_carry_h<DK, DV, true, 4, false>), dim3(DV / 64, a.H * nseg, a.B), dim3(NT), 0, stream,
                           rg, a.init_state, a.final_state, a.T, a.H, nseg, seglen, a.cu, a.total, nullptr);
        hipLaunchKernelGGL((gdn_out_h<DK, DV>), dim3(NC, a.H, a.B), dim3(NT), out_smem, stream, (const bf16*)a.q,
                           (const bf16*)a.k, rg, (bf16*)a.o, a.T, a.H, a.cu, a.total);
    }
    return hipGetLastError();
}

}  // namespace

size_t gdn_bf16_workspace_bytes(int B, int T, int H, int Dk, int Dv) {
    const size_t nbh = (size_t)B * H, nchunks = nbh * ((T + C - 1) / C);
    const int nseg = choose_nseg(B, T, H, Dk, Dv);
    const bool fused = small_carry(B, H, nseg, Dv);
    if (Dk == 64 && Dv == 64) return Lay<64, 64>::total(nchunks, fused) + seg_bytes<64, 64>(nbh, nseg);
    if (Dk == 64 && Dv == 128) return Lay<64, 128>::total(nchunks, fused) + seg_bytes<64, 128>(nbh, nseg);
    if (Dk == 128 && Dv == 64) return Lay<128, 64>::total(nchunks, fused) + seg_bytes<128, 64>(nbh, nseg);
    if (Dk == 128 && Dv == 128) return Lay<128, 128>::total(nchunks, fused) + seg_bytes<128, 128>(nbh, nseg);
    return 0;
}

hipError_t launch_gdn_bf16(const GdnFwdArgs& a, hipStream_t stream) {
    if (a.Dk == 64 && a.Dv == 64) return launch<64, 64>(a, stream);
    if (a.Dk == 64 && a.Dv == 128) return launch<64, 128>(a, stream);
    if (a.Dk == 128 && a.Dv == 64) return launch<128, 64>(a, stream);
    if (a.Dk == 128 && a.Dv == 128) return launch<128, 128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace atma

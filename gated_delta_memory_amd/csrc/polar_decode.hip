// Polar attention, one decode step, for gfx950 (bf16 KV cache, head width 64).
//
// The decode query is the last causal row: n = cache_len real keys, temperature
// t = 1 + softplus(alpha) ln n and null floor nu = b + softplus(gamma) sqrt(ln(n + 1))
// (ATMA paper, Section 3.2 equation), one softmax over the real logits t q.k_j / sqrt(D) and
// the null logit t nu (Appendix C.2), channels of Appendix A.2.
//
// Split-KV: the cache is cut into contiguous token ranges.  polar_decode_partial streams one
// range for all heads of one sequence (each token's K and V rows for all kv heads are one
// contiguous 2*Hkv*D-byte run, read with 16-byte non-temporal loads: the cache is read once
// per step, so it should not displace anything in the caches) and keeps, per query head, the
// streaming statistics of Appendix C.3 / Table 6: running maximum M of the real logits,
// L = sum p, Q2 = sum p^2 and Sv = sum p v.  Those four statistics of two disjoint key
// ranges combine exactly:  M = max(M_a, M_b), r_x = e^{M_x - M},
//     L = r_a L_a + r_b L_b,  Q2 = r_a^2 Q2_a + r_b^2 Q2_b,  Sv = r_a Sv_a + r_b Sv_b,
// so polar_decode_combine merges the ranges per (sequence, head) and finalises with the
// null sink exactly as the prefill kernel does.  Exponentials are base 2 on logits scaled
// by log2(e).
// Heterogeneous batches pass one cache length per sequence (device array): the split grid is
// sized by the longest, and each sequence cuts its own length into the same number of ranges.
// A length outside [1, bound] is an error the host cannot see; that sequence's outputs are NaN.
// With SOFTMAX set the kernels are the decode row of the NoPE / RoPE control cores: logits
// q.k / sqrt(D), no temperature, no null, output Sv / L; for RoPE the query is rotated to
// position cache_len - 1 (angle in fp64) and the cached keys are expected already rotated.
#include <atomic>
#include <mutex>

#include "atma_device.hpp"
#include "launch.hpp"

namespace atma {
namespace {

constexpr int NT = 256;
constexpr int UNROLL = 4;   // tokens in flight per thread
// floats per partial record: M, L, Q2, pad, Sv[D]
__host__ __device__ constexpr int rec_floats(int D) { return 4 + D; }

__device__ __forceinline__ float softplus(float x) { return x > 0.0f ? x + log1pf(expf(-x)) : log1pf(expf(x)); }

int num_splits(int B, int cache_len) {
    const int by_len = (cache_len + 127) / 128;
    const int target = 512 / B > 0 ? 512 / B : 1;  // about two workgroups per CU
    int n = by_len < target ? by_len : target;
    return n < 1 ? 1 : n;
}

__device__ __forceinline__ void unpack8(const u32x4& r, float* f) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        f[2 * x] = __uint_as_float(r[x] << 16);
        f[2 * x + 1] = __uint_as_float(r[x] & 0xffff0000u);
    }
}

// grid (nsplit, B); block 256.  Thread = (token slot, kv head, 8-wide dim chunk).
template <int D, int GQ, bool SOFTMAX>
__global__ __launch_bounds__(NT) void polar_decode_partial(const bf16* __restrict__ q, const bf16* __restrict__ kc,
                                                           const bf16* __restrict__ vc, PolarParamsDev prm,
                                                           float* __restrict__ ws, int max_len, int Lmax,
                                                           int Hkv, const int* __restrict__ lens, double log2_theta) {
    const int split = blockIdx.x, nsplit = gridDim.x, b = blockIdx.y;
    constexpr int CH = D / 8;                 // 8-wide dimension chunks (threads) per head
    constexpr int REC = rec_floats(D);
    const int Hq = Hkv * GQ;
    const int tpt = Hkv * CH;                // threads per token
    const int slots = NT / tpt;              // tokens per pass
    const int slot = threadIdx.x / tpt;
    const int hk = (threadIdx.x % tpt) / CH, chunk = threadIdx.x % CH;
    int cache_len = lens ? __builtin_amdgcn_readfirstlane(lens[b]) : max_len;
    if (cache_len < 1 || cache_len > max_len) cache_len = 0;  // invalid: no keys (the combine writes NaN)
    const int t_begin = (int)((long)cache_len * split / nsplit);
    const int t_end = (int)((long)cache_len * (split + 1) / nsplit);

    const float lnn = logf((float)cache_len);
    // RoPE (control core): the rotation of this thread's four pairs at position cache_len - 1
    float rc[4] = {1.f, 1.f, 1.f, 1.f}, rs[4] = {0.f, 0.f, 0.f, 0.f};
    if (SOFTMAX && log2_theta > 0.0) {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int p = chunk * 4 + x;
            double ang = (double)(cache_len - 1) * exp2(-2.0 * p / D * log2_theta);
            ang -= 6.283185307179586 * floor(ang * 0.15915494309189535);
            sincosf((float)ang, &rs[x], &rc[x]);
        }
    }
    float qv[GQ][8], cq[GQ], m[GQ], L[GQ], Q2[GQ], sv[GQ][8];
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
        const int h = hk * GQ + g;
        const float t = SOFTMAX ? 1.0f : 1.0f + softplus(prm.temp_raw[h]) * lnn;
        cq[g] = t * kLog2e * (D == 64 ? 0.125f : 0.08838834764831845f);  // t log2(e) / sqrt(D)
        const u32x4 r = *(const u32x4*)(q + ((size_t)b * Hq + h) * D + chunk * 8);
        unpack8(r, qv[g]);
        if (SOFTMAX) {
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const float a0 = qv[g][2 * x], a1 = qv[g][2 * x + 1];
                qv[g][2 * x] = a0 * rc[x] - a1 * rs[x];
                qv[g][2 * x + 1] = a0 * rs[x] + a1 * rc[x];
            }
        }
        m[g] = -INFINITY; L[g] = 0.f; Q2[g] = 0.f;
#pragma unroll
        for (int x = 0; x < 8; ++x) sv[g][x] = 0.f;
    }
    const size_t tstride = (size_t)Hkv * D;
    const bf16* kb = kc + (size_t)b * Lmax * tstride + (size_t)hk * D + chunk * 8;
    const bf16* vb = vc + (size_t)b * Lmax * tstride + (size_t)hk * D + chunk * 8;

    for (int t0 = t_begin + slot; t0 < t_end; t0 += slots * UNROLL) {
        u32x4 kr[UNROLL], vr[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int t = t0 + u * slots;
            if (t < t_end) {
                kr[u] = __builtin_nontemporal_load((const u32x4*)(kb + (size_t)t * tstride));
                vr[u] = __builtin_nontemporal_load((const u32x4*)(vb + (size_t)t * tstride));
            } else {
                kr[u] = u32x4{0u, 0u, 0u, 0u};
                vr[u] = u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int g = 0; g < GQ; ++g) {
            float lg[UNROLL];
            float bmax = -INFINITY;
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                float kf[8];
                unpack8(kr[u], kf);
                float d = 0.f;
#pragma unroll
                for (int x = 0; x < 8; ++x) d += qv[g][x] * kf[x];
#pragma unroll
                for (int o = CH / 2; o >= 1; o >>= 1) d += __shfl_xor(d, o, CH);
                lg[u] = (t0 + u * slots < t_end) ? d * cq[g] : -INFINITY;
                bmax = fmaxf(bmax, lg[u]);
            }
            const float mnew = fmaxf(m[g], bmax);
            const float rho = fast_exp2(m[g] - mnew);
            m[g] = mnew;
            L[g] *= rho;
            Q2[g] *= rho * rho;
#pragma unroll
            for (int x = 0; x < 8; ++x) sv[g][x] *= rho;
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const float p = fast_exp2(lg[u] - mnew);
                L[g] += p;
                Q2[g] += p * p;
                float vf[8];
                unpack8(vr[u], vf);
#pragma unroll
                for (int x = 0; x < 8; ++x) sv[g][x] += p * vf[x];
            }
        }
    }

    // merge the token slots of this workgroup through LDS, then write one record per head
    __shared__ float part[NT / CH][3];  // per (slot, kv head): M, L, Q2 (written by chunk 0)
    __shared__ float psv[NT][8];
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
        if (chunk == 0) {
            part[threadIdx.x / CH][0] = m[g];
            part[threadIdx.x / CH][1] = L[g];
            part[threadIdx.x / CH][2] = Q2[g];
        }
#pragma unroll
        for (int x = 0; x < 8; ++x) psv[threadIdx.x][x] = sv[g][x];
        __syncthreads();
        if (slot == 0) {
            float M = -INFINITY;
            for (int s = 0; s < slots; ++s) M = fmaxf(M, part[(s * tpt + threadIdx.x) / CH][0]);
            float LL = 0.f, QQ = 0.f, acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            for (int s = 0; s < slots; ++s) {
                const float* ps = part[(s * tpt + threadIdx.x) / CH];
                const float r = (ps[0] == -INFINITY) ? 0.0f : fast_exp2(ps[0] - M);
                LL += r * ps[1];
                QQ += r * r * ps[2];
#pragma unroll
                for (int x = 0; x < 8; ++x) acc[x] += r * psv[s * tpt + threadIdx.x][x];
            }
            const int h = hk * GQ + g;
            float* rec = ws + (((size_t)b * Hq + h) * nsplit + split) * REC;
            if (chunk == 0) *(f32x4*)rec = f32x4{M, LL, QQ, 0.f};
            *(f32x4*)(rec + 4 + chunk * 8) = f32x4{acc[0], acc[1], acc[2], acc[3]};
            *(f32x4*)(rec + 8 + chunk * 8) = f32x4{acc[4], acc[5], acc[6], acc[7]};
        }
        __syncthreads();
    }
}

// grid (Hq, B); block 1024.  Wave j merges R ranges at a time (R = 64 at D = 64, 32 at D = 128):
// ranges s = R j .. R j + R - 1 (then + 16 R, ...), in one round of loads: lane i reads the header
// (M, L, Q2) of range R j + i and every lane reads its value dimensions (d, and d + 64 at D = 128)
// of all R ranges, so all loads are in flight together.  The wave's merge weights
// e_i = exp(M_i - max M) are formed per lane and broadcast with v_readlane for the value sums;
// the sixteen wave merges are combined through LDS.
constexpr int CNW = 16;        // waves per combine workgroup
constexpr int CNT = 64 * CNW;  // threads per combine workgroup
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}
template <int D, bool SOFTMAX>
__global__ __launch_bounds__(CNT) void polar_decode_combine(const float* __restrict__ ws, PolarParamsDev prm,
                                                            bf16* __restrict__ o, float* __restrict__ mu_out,
                                                            int nsplit, int max_len, const int* __restrict__ lens) {
    constexpr int NV = D / 64;            // value dimensions per lane
    constexpr int R = 64 / NV;            // ranges per wave and round
    constexpr int REC = rec_floats(D);
    const int h = blockIdx.x, Hq = gridDim.x, b = blockIdx.y;
    const int cache_len = lens ? __builtin_amdgcn_readfirstlane(lens[b]) : max_len;
    if (cache_len < 1 || cache_len > max_len) {  // invalid length: NaN outputs for this sequence
        if (threadIdx.x < D) o[((size_t)b * Hq + h) * D + threadIdx.x] = (bf16)__builtin_nanf("");
        if (threadIdx.x == 0 && mu_out) mu_out[(size_t)b * Hq + h] = __builtin_nanf("");
        return;
    }
    const int d = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const float* base = ws + ((size_t)b * Hq + h) * nsplit * REC;  // records of (b, h), split-major
    float M = -INFINITY, L = 0.f, Q2 = 0.f, Sv[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) Sv[j] = 0.f;
    for (int s0 = R * wv; s0 < nsplit; s0 += R * CNW) {
        const int cnt = min(R, nsplit - s0);
        const float* r0 = base + (size_t)s0 * REC;
        const f32x4 hd = d < cnt ? *(const f32x4*)(r0 + d * REC) : f32x4{-INFINITY, 0.f, 0.f, 0.f};
        float rs[NV][R];
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int j = 0; j < NV; ++j) rs[j][i] = i < cnt ? r0[i * REC + 4 + 64 * j + d] : 0.f;
        const float bm = fmaxf(M, wave_max(hd[0]));
        if (bm == -INFINITY) continue;  // nothing seen yet (empty ranges)
        const float e0 = fast_exp2(M - bm);  // 0 when M = -inf
        const float e = (hd[0] == -INFINITY) ? 0.0f : fast_exp2(hd[0] - bm);
        L = L * e0 + wave_sum(e * hd[1]);
        Q2 = Q2 * e0 * e0 + wave_sum(e * e * hd[2]);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            float acc = Sv[j] * e0;
#pragma unroll
            for (int i = 0; i < R; ++i)
                acc = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(e), i)), rs[j][i], acc);
            Sv[j] = acc;
        }
        M = bm;
    }
    __shared__ float part[CNW][3];
    __shared__ float psv[CNW][D];
    if (d == 0) {
        part[wv][0] = M;
        part[wv][1] = L;
        part[wv][2] = Q2;
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) psv[wv][64 * j + d] = Sv[j];
    __syncthreads();
    if (wv != 0) return;
    M = -INFINITY;
#pragma unroll
    for (int w = 0; w < CNW; ++w) M = fmaxf(M, part[w][0]);
    L = Q2 = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) Sv[j] = 0.f;
#pragma unroll
    for (int w = 0; w < CNW; ++w) {
        const float e = (part[w][0] == -INFINITY) ? 0.0f : fast_exp2(part[w][0] - M);
        L += e * part[w][1];
        Q2 += e * e * part[w][2];
#pragma unroll
        for (int j = 0; j < NV; ++j) Sv[j] += e * psv[w][64 * j + d];
    }
    bf16* orow = o + ((size_t)b * Hq + h) * D;
    if constexpr (SOFTMAX) {  // control core: o = Sv / L
#pragma unroll
        for (int j = 0; j < NV; ++j) orow[64 * j + d] = (bf16)(Sv[j] / L);
        return;
    }
    const float n = (float)cache_len;
    const float t = 1.0f + softplus(prm.temp_raw[h]) * logf(n);
    const float nu = prm.null_bias[h] + softplus(prm.null_slope_raw[h]) * sqrtf(logf(n + 1.0f));
    const float lnull = t * nu * kLog2e;
    const float Ms = fmaxf(M, lnull);
    const float pn = fast_exp2(lnull - Ms);
    const float f = fast_exp2(M - Ms);
    const float Ls = L * f;
    const float Z = Ls + pn;
    const float neff = L * L / Q2;
    const float meff = neff * (Ls / Z);
    const float xarg = prm.mag_beta[h] * log1pf(meff);
    const float em = expf(-2.0f * xarg);
    const float mu = (1.0f - em) / (1.0f + em);
    float sv[NV], ss = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        sv[j] = (Sv[j] * f + pn * prm.v_null[h * D + 64 * j + d]) / Z;
        ss += sv[j] * sv[j];
    }
    const float sc = mu / fmaxf(sqrtf(wave_sum(ss)), prm.eps);
#pragma unroll
    for (int j = 0; j < NV; ++j) orow[64 * j + d] = (bf16)(sv[j] * sc);
    if (d == 0 && mu_out) mu_out[(size_t)b * Hq + h] = mu;
}

}  // namespace

size_t polar_decode_workspace_bytes(int B, int Hq, int cache_len, int Dh) {
    return (size_t)B * num_splits(B, cache_len) * Hq * rec_floats(Dh) * sizeof(float);
}

hipError_t launch_polar_decode(const PolarDecodeArgs& a, hipStream_t stream) {
    const int nsplit = num_splits(a.B, a.cache_len);
    const int gq = a.Hq / a.Hkv;
    float* ws = (float*)a.workspace;
    const double l2t = a.rope_theta > 0.0 ? log2(a.rope_theta) : 0.0;
#define ATMA_PD_CASE(DD, G, S)                                                                             \
    if (a.D == DD && gq == G && a.softmax == S) {                                                          \
        hipLaunchKernelGGL((polar_decode_partial<DD, G, S>), dim3(nsplit, a.B), dim3(NT), 0, stream,       \
                           (const bf16*)a.q, (const bf16*)a.k_cache, (const bf16*)a.v_cache, a.p, ws,      \
                           a.cache_len, a.Lmax, a.Hkv, a.lens, l2t);                                       \
        hipLaunchKernelGGL((polar_decode_combine<DD, S>), dim3(a.Hq, a.B), dim3(CNT), 0, stream,           \
                           (const float*)ws, a.p, (bf16*)a.o, S ? nullptr : a.mu_out, nsplit, a.cache_len, \
                           a.lens);                                                                        \
    } else
#define ATMA_PD_GQ(DD, S) ATMA_PD_CASE(DD, 1, S) ATMA_PD_CASE(DD, 2, S) ATMA_PD_CASE(DD, 4, S) ATMA_PD_CASE(DD, 8, S)
    ATMA_PD_GQ(64, false) ATMA_PD_GQ(64, true) ATMA_PD_GQ(128, false) ATMA_PD_GQ(128, true) {
        return hipErrorInvalidValue;
    }
#undef ATMA_PD_GQ
#undef ATMA_PD_CASE
    return hipGetLastError();
}

// ---- allocation-free decode ---------------------------------------------------------------
// Callers that cannot allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation) get the split records in a fixed array of device memory instead of a
// workspace: 16 MiB, one copy per GPU the library runs on, held until the process ends.  The
// partial kernel writes every record the combine kernel reads, so nothing needs clearing between
// calls; calls that overlap on one GPU (different streams) share the array and race.
namespace {
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, looked up once per device.  In host code the
// array's name is only a stand-in for the symbol; the kernels receive this address instead.
hipError_t scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* addr = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!addr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        addr = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!addr) {
            e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            g_scratch_addr[dev].store(addr, std::memory_order_release);
        }
    }
    *out = addr;
    return hipSuccess;
}
}  // namespace

size_t polar_decode_scratch_bytes() { return kScratchBytes; }

hipError_t launch_polar_decode_noalloc(PolarDecodeArgs a, hipStream_t stream) {
    if (polar_decode_workspace_bytes(a.B, a.Hq, a.cache_len, a.D) > kScratchBytes) return hipErrorInvalidValue;
    void* addr = nullptr;
    const hipError_t e = scratch_address(&addr);
    if (e != hipSuccess) return e;
    a.workspace = addr;
    return launch_polar_decode(a, stream);
}

bool polar_decode_supported(int Hq, int Hkv, int D) {
    const int gq = Hq / Hkv;
    const bool g_ok = gq == 1 || gq == 2 || gq == 4 || gq == 8;
    // a token's K row for all kv heads is read by Hkv * D / 8 threads of one 256-thread workgroup
    const bool h_ok = (Hkv == 1 || Hkv == 2 || Hkv == 4 || Hkv == 8 || Hkv == 16 || Hkv == 32) && Hkv * D / 8 <= NT;
    return (D == 64 || D == 128) && g_ok && h_ok;
}

}  // namespace atma

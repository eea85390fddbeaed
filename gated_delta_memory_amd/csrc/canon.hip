// Canon prologue (ATMA paper, Section 3.1: depthwise causal convolutions on q, k and v before
// attention): per channel c, y_t = sum_{j<K} w[j][c] x_{t-j} (+ x_t with `residual`), inputs
// before the first token taken from the carried state (the K-1 previous inputs); then,
// optionally, each head's D = C / heads channels scaled to unit L2 norm (the memory path's
// unit-norm queries and keys).  One thread per (run of TR = 8 tokens, 8-channel chunk): it slides
// down its run with the K-1 previous inputs in registers, so every input row is read once (plus
// a K-1 row halo per run), with 16-byte loads along the channel axis; fp32 weights and
// accumulation, bf16 output.  The run's rows are loaded and y is stored non-temporally (each is
// touched once), so the L2 keeps the K-1 halo rows the next run re-reads.  The chunks of a run are consecutive lanes, so a head's norm is a
// reduction over D / 8 adjacent lanes, all at the same token.
// A second kernel then writes the new state (the last K-1 inputs); one thread owns all K-1
// slots of its channels, so the state may be updated in place.
#include "atma_device.hpp"
#include "launch.hpp"

namespace atma {
namespace {

constexpr int NT = 256;

__device__ __forceinline__ void load8(const bf16* p, float* f) {
    const u32x4 r = *(const u32x4*)p;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        f[2 * x] = __uint_as_float(r[x] << 16);
        f[2 * x + 1] = __uint_as_float(r[x] & 0xffff0000u);
    }
}

constexpr int TR = 8;  // tokens per run

template <int K>
__global__ __launch_bounds__(NT) void canon_kernel(const bf16* __restrict__ x, const float* __restrict__ w,
                                                   const bf16* __restrict__ state, bf16* __restrict__ y, int B, int T,
                                                   int C, int residual, int dch, float eps) {
    const int nch = C / 8, nr = (T + TR - 1) / TR;
    const long long id = (long long)blockIdx.x * NT + threadIdx.x;
    if (id >= (long long)B * nr * nch) return;  // whole runs, so whole head groups, leave together
    const long long run = id / nch;
    const int ch = (int)(id - run * nch), b = (int)(run / nr), t0 = (int)(run % nr) * TR;
    float wk[K][8], win[K][8];  // taps; win[j] = x_{t-j} at token t
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const f32x4 w0 = *(const f32x4*)(w + (size_t)j * C + 8 * ch);
        const f32x4 w1 = *(const f32x4*)(w + (size_t)j * C + 8 * ch + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            wk[j][e] = w0[e];
            wk[j][e + 4] = w1[e];
        }
    }
#pragma unroll
    for (int j = 1; j < K; ++j) {  // the K-1 inputs before the run: earlier tokens, the state, or zero
        const int s = t0 - j;
#pragma unroll
        for (int e = 0; e < 8; ++e) win[j][e] = 0.f;
        if (s >= 0) load8(x + ((size_t)b * T + s) * C + 8 * ch, win[j]);
        else if (state && K - 1 + s >= 0) load8(state + ((size_t)b * (K - 1) + (K - 1 + s)) * C + 8 * ch, win[j]);
    }
    // the run's rows, all requested before the first is used (TR loads in flight per thread)
    u32x4 raw[TR];
#pragma unroll
    for (int i = 0; i < TR; ++i) {
        raw[i] = u32x4{0u, 0u, 0u, 0u};
        if (t0 + i < T) raw[i] = __builtin_nontemporal_load((const u32x4*)(x + ((size_t)b * T + t0 + i) * C + 8 * ch));
    }
#pragma unroll
    for (int i = 0; i < TR; ++i) {
        const int t = t0 + i;
        if (t < T) {  // the same for every lane of a run
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                win[0][2 * q] = __uint_as_float(raw[i][q] << 16);
                win[0][2 * q + 1] = __uint_as_float(raw[i][q] & 0xffff0000u);
            }
            float acc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float a = residual ? win[0][e] : 0.f;
#pragma unroll
                for (int j = 0; j < K; ++j) a = fmaf(wk[j][e], win[j][e], a);
                acc[e] = a;
            }
            if (dch > 0) {  // unit L2 norm per head: the dch = D / 8 lanes of a head reduce together
                float n2 = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) n2 = fmaf(acc[e], acc[e], n2);
                for (int o = dch / 2; o >= 1; o >>= 1) n2 += __shfl_xor(n2, o, dch);
                const float inv = 1.0f / fmaxf(sqrtf(n2), eps);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] *= inv;
            }
            u32x4 out;
#pragma unroll
            for (int x2 = 0; x2 < 4; ++x2) {
                const bf16x2 pr = {(bf16)acc[2 * x2], (bf16)acc[2 * x2 + 1]};
                out[x2] = __builtin_bit_cast(unsigned, pr);
            }
            __builtin_nontemporal_store(out, (u32x4*)(y + ((size_t)b * T + t) * C + 8 * ch));
        }
#pragma unroll
        for (int j = K - 1; j >= 1; --j)
#pragma unroll
            for (int e = 0; e < 8; ++e) win[j][e] = win[j - 1][e];
    }
}

// new state: slot r (0 = oldest) of the last K-1 inputs = input T - (K-1) + r, which lies in the
// old state when negative (zeros without one).  K <= 8.
__global__ __launch_bounds__(NT) void canon_state_kernel(const bf16* __restrict__ x, const bf16* state_in,
                                                         bf16* state_out, int B, int T, int C, int K) {
    const int nch = C / 8;
    const long long id = (long long)blockIdx.x * NT + threadIdx.x;
    if (id >= (long long)B * nch) return;
    const long long b = id / nch;
    const int ch = (int)(id - b * nch);
    u32x4 v[7];
#pragma unroll
    for (int r = 0; r < 7; ++r) {
        v[r] = u32x4{0u, 0u, 0u, 0u};
        if (r >= K - 1) continue;
        const int s = T - (K - 1) + r;
        if (s >= 0) v[r] = *(const u32x4*)(x + ((size_t)b * T + s) * C + 8 * ch);
        else if (state_in) v[r] = *(const u32x4*)(state_in + ((size_t)b * (K - 1) + (K - 1 + s)) * C + 8 * ch);
    }
#pragma unroll
    for (int r = 0; r < 7; ++r)
        if (r < K - 1) *(u32x4*)(state_out + ((size_t)b * (K - 1) + r) * C + 8 * ch) = v[r];
}

}  // namespace

hipError_t launch_canon(const CanonArgs& a, hipStream_t stream) {
    const long long runs = (long long)a.B * ((a.T + TR - 1) / TR);
    const long long n = runs * (a.C / 8);
    const long long blocks = (n + NT - 1) / NT;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const int dch = a.heads > 0 ? a.C / a.heads / 8 : 0;
#define CANON_K(KK)                                                                                                 \
    case KK:                                                                                                      \
        hipLaunchKernelGGL(canon_kernel<KK>, dim3((unsigned)blocks), dim3(NT), 0, stream, (const bf16*)a.x, a.w,   \
                           (const bf16*)a.state_in, (bf16*)a.y, a.B, a.T, a.C, a.residual, dch, a.eps);          \
        break;
    switch (a.K) {
        CANON_K(1) CANON_K(2) CANON_K(3) CANON_K(4) CANON_K(5) CANON_K(6) CANON_K(7) CANON_K(8)
        default: return hipErrorInvalidValue;
    }
#undef CANON_K
    if (a.state_out && a.K > 1) {
        const long long ns = (long long)a.B * (a.C / 8);
        hipLaunchKernelGGL(canon_state_kernel, dim3((unsigned)((ns + NT - 1) / NT)), dim3(NT), 0, stream,
                           (const bf16*)a.x, (const bf16*)a.state_in, (bf16*)a.state_out, a.B, a.T, a.C, a.K);
    }
    return hipGetLastError();
}

}  // namespace atma

// Canon prologue (ATMA paper, Section 3.1: depthwise causal convolutions on q, k and v before
// attention): per channel c, y_t = sum_{j<K} w[j][c] x_{t-j} (+ x_t with `residual`), inputs
// before the first token taken from the carried state (the K-1 previous inputs); then,
// optionally, each head's D = C / heads channels scaled to unit L2 norm (the memory path's
// unit-norm queries and keys).  One thread per (token, 8-channel chunk): 16-byte loads along
// the channel axis, fp32 weights and accumulation, bf16 output.  A token's chunks are
// consecutive lanes, so a head's norm is a reduction over D / 8 adjacent lanes.
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

__global__ __launch_bounds__(NT) void canon_kernel(const bf16* __restrict__ x, const float* __restrict__ w,
                                                   const bf16* __restrict__ state, bf16* __restrict__ y, long long ntok,
                                                   int T, int C, int K, int residual, int dch, float eps) {
    const int nch = C / 8;
    const long long id = (long long)blockIdx.x * NT + threadIdx.x;
    const bool live = id < ntok * nch;
    const long long tok = live ? id / nch : 0;
    const int ch = live ? (int)(id - tok * nch) : 0;
    const long long b = tok / T;
    const int t = (int)(tok - b * T);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (live) {
        float xv[8];
        for (int j = 0; j < K; ++j) {
            const int s = t - j;
            if (s >= 0) load8(x + ((size_t)b * T + s) * C + 8 * ch, xv);
            else if (state && K - 1 + s >= 0) load8(state + ((size_t)b * (K - 1) + (K - 1 + s)) * C + 8 * ch, xv);
            else continue;
            const f32x4 w0 = *(const f32x4*)(w + (size_t)j * C + 8 * ch);
            const f32x4 w1 = *(const f32x4*)(w + (size_t)j * C + 8 * ch + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[e] = fmaf(w0[e], xv[e], acc[e]);
                acc[e + 4] = fmaf(w1[e], xv[e + 4], acc[e + 4]);
            }
        }
        if (residual) {
            load8(x + (size_t)tok * C + 8 * ch, xv);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += xv[e];
        }
    }
    if (dch > 0) {  // unit L2 norm per head: the dch = D / 8 lanes of a head reduce together
        float n2 = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) n2 += acc[e] * acc[e];
        for (int o = dch / 2; o >= 1; o >>= 1) n2 += __shfl_xor(n2, o, dch);
        const float inv = 1.0f / fmaxf(sqrtf(n2), eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= inv;
    }
    if (live) {
        u32x4 out;
#pragma unroll
        for (int x2 = 0; x2 < 4; ++x2) {
            const bf16x2 p = {(bf16)acc[2 * x2], (bf16)acc[2 * x2 + 1]};
            out[x2] = __builtin_bit_cast(unsigned, p);
        }
        *(u32x4*)(y + (size_t)tok * C + 8 * ch) = out;
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
    const long long ntok = (long long)a.B * a.T;
    const long long n = ntok * (a.C / 8);
    const long long blocks = (n + NT - 1) / NT;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(canon_kernel, dim3((unsigned)blocks), dim3(NT), 0, stream, (const bf16*)a.x, a.w,
                       (const bf16*)a.state_in, (bf16*)a.y, ntok, a.T, a.C, a.K, a.residual,
                       a.heads > 0 ? a.C / a.heads / 8 : 0, a.eps);
    if (a.state_out && a.K > 1) {
        const long long ns = (long long)a.B * (a.C / 8);
        hipLaunchKernelGGL(canon_state_kernel, dim3((unsigned)((ns + NT - 1) / NT)), dim3(NT), 0, stream,
                           (const bf16*)a.x, (const bf16*)a.state_in, (bf16*)a.state_out, a.B, a.T, a.C, a.K);
    }
    return hipGetLastError();
}

}  // namespace atma

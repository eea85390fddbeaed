// Rotary position embedding for the RoPE control core (rotary embedding of Su et al.; the
// ATMA paper's matched RoPE models, Section 3.1, differ from NoPE only by it): every adjacent
// pair (x[2p], x[2p+1]) of a head row at position m is turned by the angle m * theta^(-2p/D).
// One thread per (token, pair) computes the angle once and rotates that pair in every head.
// The angle is formed and reduced modulo 2 pi in fp64: positions reach 2^18, where an fp32
// product would already be off by ~1e-2 rad; the rotation itself is fp32 on bf16 data.
#include "atma_device.hpp"
#include "launch.hpp"

namespace atma {
namespace {

constexpr int NT = 256;

__global__ __launch_bounds__(NT) void rope_kernel(const bf16* __restrict__ x, bf16* __restrict__ y, long long ntok,
                                                  int T, int H, int D, int pos0, double log2_theta) {
    const int npair = D / 2;
    const long long id = (long long)blockIdx.x * NT + threadIdx.x;
    if (id >= ntok * npair) return;
    const long long tok = id / npair;
    const int p = (int)(id - tok * npair);
    const int t = (int)(tok % T);
    const double inv_freq = exp2(-2.0 * p / D * log2_theta);
    double ang = (double)(pos0 + t) * inv_freq;
    ang -= 6.283185307179586 * floor(ang * 0.15915494309189535);  // [0, 2 pi)
    float s, c;
    sincosf((float)ang, &s, &c);
    const size_t row = (size_t)tok * H * D + 2 * p;
    for (int h = 0; h < H; ++h) {
        const bf16x2 v = *(const bf16x2*)(x + row + (size_t)h * D);
        const float a = (float)v[0], b = (float)v[1];
        *(bf16x2*)(y + row + (size_t)h * D) = bf16x2{(bf16)(a * c - b * s), (bf16)(a * s + b * c)};
    }
}

}  // namespace

hipError_t launch_rope(const RopeArgs& a, hipStream_t stream) {
    const long long ntok = (long long)a.B * a.T;
    const long long n = ntok * (a.D / 2);
    const long long blocks = (n + NT - 1) / NT;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(rope_kernel, dim3((unsigned)blocks), dim3(NT), 0, stream, (const bf16*)a.x, (bf16*)a.y, ntok,
                       a.T, a.H, a.D, a.pos0, log2(a.theta));
    return hipGetLastError();
}

}  // namespace atma

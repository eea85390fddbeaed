// Gated-delta memory, one decode step, for gfx950 (ATMA paper, Section 3.3 equation
// applied to a single token; the recurrent state has a fixed size, Appendix H.1):
//     u = S k;   S <- alpha (S - beta u k^T) + beta v k^T;   o = S q.
// Rows of S are independent given (q, k, v, alpha, beta): a 32-lane group owns one row at
// a time (Dk = 128: 4 floats per lane; Dk = 64: 2 floats per lane), reads it once, forms
// u_r and o_r with group reductions and writes the row back.  The kernel is HBM-bound:
// every state byte is read once and written once.
#include "atma_device.hpp"
#include "launch.hpp"

namespace atma {
namespace {

constexpr int NT = 256;
constexpr int ROWS_PER_BLOCK = 32;  // 8 lane groups x 4 rows

template <int N> struct FVec;
template <> struct FVec<4> { typedef f32x4 type; };
template <> struct FVec<2> { typedef f32x2 type; };

template <typename T, int DK, int DV>
__global__ __launch_bounds__(NT) void gdn_decode_step_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                             const T* __restrict__ v,
                                                             const float* __restrict__ alpha,
                                                             const float* __restrict__ beta,
                                                             float* __restrict__ state, T* __restrict__ o, int H) {
    constexpr int PER = DK / 32;  // state columns per lane
    typedef typename FVec<PER>::type vec;
    const int h = blockIdx.y, b = blockIdx.z;
    const int bh = b * H + h;
    const int sub = threadIdx.x & 31, grp = threadIdx.x >> 5;  // 8 groups of 32 lanes
    const float a = alpha[bh], be = beta[bh];
    float kk[PER], qq[PER];
#pragma unroll
    for (int x = 0; x < PER; ++x) {
        kk[x] = to_f32(k[(size_t)bh * DK + sub * PER + x]);
        qq[x] = to_f32(q[(size_t)bh * DK + sub * PER + x]);
    }
#pragma unroll
    for (int it = 0; it < ROWS_PER_BLOCK / 8; ++it) {
        const int r = blockIdx.x * ROWS_PER_BLOCK + it * 8 + grp;
        float* srow = state + ((size_t)bh * DV + r) * DK + sub * PER;
        vec s = *(vec*)srow;
        float u = 0.0f;
#pragma unroll
        for (int x = 0; x < PER; ++x) u += s[x] * kk[x];
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) u += __shfl_xor(u, off, 32);
        const float vr = to_f32(v[(size_t)bh * DV + r]);
        float y = 0.0f;
#pragma unroll
        for (int x = 0; x < PER; ++x) {
            s[x] = a * (s[x] - be * u * kk[x]) + be * vr * kk[x];
            y += s[x] * qq[x];
        }
        *(vec*)srow = s;
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) y += __shfl_xor(y, off, 32);
        if (sub == 0) o[(size_t)bh * DV + r] = from_f32<T>(y);
    }
}

template <typename T, int DK, int DV>
hipError_t launch_typed(const GdnDecodeArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((gdn_decode_step_kernel<T, DK, DV>), dim3(DV / ROWS_PER_BLOCK, a.H, a.B), dim3(NT), 0,
                       stream, (const T*)a.q, (const T*)a.k, (const T*)a.v, a.alpha, a.beta, a.state, (T*)a.o,
                       a.H);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gdn_decode(const GdnDecodeArgs& a, hipStream_t stream) {
#define ATMA_DEC_CASE(TT, DKK, DVV) \
    if (a.Dk == DKK && a.Dv == DVV) return launch_typed<TT, DKK, DVV>(a, stream);
    if (a.bf16_io) {
        ATMA_DEC_CASE(bf16, 64, 64) ATMA_DEC_CASE(bf16, 64, 128) ATMA_DEC_CASE(bf16, 128, 64)
        ATMA_DEC_CASE(bf16, 128, 128)
    } else {
        ATMA_DEC_CASE(float, 64, 64) ATMA_DEC_CASE(float, 64, 128) ATMA_DEC_CASE(float, 128, 64)
        ATMA_DEC_CASE(float, 128, 128)
    }
#undef ATMA_DEC_CASE
    return hipErrorInvalidValue;
}

}  // namespace atma

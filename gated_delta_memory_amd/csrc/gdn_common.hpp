// Pieces shared by the two gated-delta prefill paths (fp32 and bf16 inputs).
#pragma once
#include "atma_device.hpp"

namespace atma {
namespace gdn {

constexpr int C = 64;    // chunk length
constexpr int NT = 256;  // threads per workgroup (4 waves)

// Copies a ROWS x COLS tile (row stride `ld` elements in global memory) through registers
// into LDS (row stride LDS_LD elements).  Rows >= nrows read as zero.
template <typename T, int ROWS, int COLS>
struct TileRegs {
    static constexpr int VEC = 16 / sizeof(T);
    static constexpr int NVEC = ROWS * COLS / VEC;
    static constexpr int PER = (NVEC + NT - 1) / NT;
    u32x4 r[PER];
    int nr;  // rows < nr are real; the rest are stored as zero
    // STREAM: non-temporal loads, for data no later kernel reads.  Every load is issued without a
    // branch (rows at and past nrows >= 1 re-read row nrows - 1) and nothing reads the registers
    // until the stores, which write those rows as zero: all the loads are in flight together.
    template <bool STREAM = false>
    __device__ __forceinline__ void load(const T* g, size_t ld, int nrows) {
        nr = nrows;
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int i = threadIdx.x + m * NT;
            const int row = i / (COLS / VEC), cv = i % (COLS / VEC);
            const u32x4* src = (const u32x4*)(g + (size_t)min(row, nrows - 1) * ld + cv * VEC);
            if constexpr (NVEC % NT == 0) {  // every thread has PER pieces: no branch at all
                if constexpr (STREAM) r[m] = __builtin_nontemporal_load(src);
                else r[m] = *src;
            } else {
                r[m] = u32x4{0u, 0u, 0u, 0u};
                if (i < NVEC) {
                    if constexpr (STREAM) r[m] = __builtin_nontemporal_load(src);
                    else r[m] = *src;
                }
            }
        }
    }
    template <int LDS_LD>
    __device__ __forceinline__ void store(T* s) const {
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int i = threadIdx.x + m * NT;
            if (i < NVEC) {
                const int row = i / (COLS / VEC), cv = i % (COLS / VEC);
                *(u32x4*)(s + row * LDS_LD + cv * VEC) = row < nr ? r[m] : u32x4{0u, 0u, 0u, 0u};
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
                const u32x4 v = row < nr ? r[m] : u32x4{0u, 0u, 0u, 0u};
                const T* e = (const T*)&v;
#pragma unroll
                for (int x = 0; x < VEC; ++x) s[(cv * VEC + x) * LDS_LD + row] = e[x];
            }
        }
    }
};

// Copies `bytes` (multiple of 16) from LDS to global memory with 16-byte stores; streaming
// (non-temporal) stores for data no kernel reads back soon, so it does not displace what does.
template <bool STREAM = false>
__device__ __forceinline__ void copy_out(char* __restrict__ dst, const char* src, int bytes) {
    for (int i = threadIdx.x * 16; i < bytes; i += NT * 16) {
        const u32x4 x = *(const u32x4*)(src + i);
        if constexpr (STREAM) __builtin_nontemporal_store(x, (u32x4*)(dst + i));
        else *(u32x4*)(dst + i) = x;
    }
}

// Packed rows [seq0, seq0 + T) of sequence b.  Without offsets every sequence has Tmax rows;
// with offsets cu[0..B] (device memory) the bounds are read and checked: a sequence whose
// offsets leave [0, total], decrease, or span more than Tmax rows is reported invalid, and
// every kernel skips it, so malformed offsets never address memory outside the buffers.
__device__ __forceinline__ bool seq_bounds(const int* cu, int b, int Tmax, int total, size_t& seq0, int& T) {
    if (!cu) {
        seq0 = (size_t)b * Tmax;
        T = Tmax;
        return true;
    }
    // b is uniform across the workgroup; readfirstlane keeps the bounds (and everything derived
    // from them, such as chunk counts and copy addresses) in scalar registers
    const int s0 = __builtin_amdgcn_readfirstlane(cu[b]), s1 = __builtin_amdgcn_readfirstlane(cu[b + 1]);
    if (s0 < 0 || s1 < s0 || s1 > total || s1 - s0 > Tmax) return false;
    seq0 = (size_t)s0;
    T = s1 - s0;
    return true;
}

using atma::wait_vmcnt;
using atma::lds_dma16;
using atma::lds_dma4;
using atma::lds_barrier;
using atma::lds_addr;

}  // namespace gdn
}  // namespace atma

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

// Copies `bytes` (multiple of 16) from LDS to global memory with 16-byte stores.
__device__ __forceinline__ void copy_out(char* __restrict__ dst, const char* src, int bytes) {
    for (int i = threadIdx.x * 16; i < bytes; i += NT * 16) *(u32x4*)(dst + i) = *(const u32x4*)(src + i);
}

// s_waitcnt vmcnt(N) leaving the other counters untouched (gfx9 encoding: vmcnt bits [3:0]
// and [15:14], expcnt [6:4], lgkmcnt [11:8]).  Vector memory operations, loads, LDS-DMA
// copies and stores alike, retire in issue order on this architecture.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Asynchronous global->LDS copy of 16 bytes per lane: lane l writes LDS bytes
// [lds_base + 16 l, lds_base + 16 l + 16).  Issued from inline assembly so the compiler
// does not track it: callers retire it with an explicit wait_vmcnt before a barrier and
// only then read the destination.  (Tracked copies make the compiler's conservative
// wait-count analysis stall on every LDS read while any copy is in flight.)
__device__ __forceinline__ void lds_dma16(const void* gaddr, const void* lds_wave_base) {
    typedef __attribute__((address_space(3))) const char* lds_ptr;
    const unsigned base = __builtin_amdgcn_readfirstlane((unsigned)(size_t)(lds_ptr)lds_wave_base);
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(gaddr), "s"(base)
        : "memory", "m0");
}
// Same, 4 bytes per lane (lane l writes [lds_base + 4 l, lds_base + 4 l + 4)).
__device__ __forceinline__ void lds_dma4(const void* gaddr, const void* lds_wave_base) {
    typedef __attribute__((address_space(3))) const char* lds_ptr;
    const unsigned base = __builtin_amdgcn_readfirstlane((unsigned)(size_t)(lds_ptr)lds_wave_base);
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %0, off"
        :
        : "v"(gaddr), "s"(base)
        : "memory", "m0");
}

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS operations, then
// s_barrier, without the release/acquire fences of __syncthreads() (those would also wait
// for every global store and asynchronous copy in flight).  The empty asm statements keep
// the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt untouched
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace gdn
}  // namespace atma

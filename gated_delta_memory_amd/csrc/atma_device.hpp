// Device-side building blocks shared by the libatma kernels (gfx950 only).
//
// MFMA tiles used here are 16x16 outputs.  For one 16x16 tile the accumulator (C/D
// operand, 4 fp32 per lane) holds element (row 4*G + v, col l % 16) in register v of
// lane l, where G = l / 16 is the lane group.  An A or B operand "fragment" covers a
// 32-wide slice of the reduction index: lane l supplies 8 values for row (A) or column
// (B) l % 16 at reduction offsets kmap(G, e), e = 0..7:
//     kmap(G, e) = 4G + e            for e < 4
//                = 16 + 4G + (e - 4) for e >= 4
// The hardware pairs lane-group/slot positions of A and B, so any bijection works as
// long as both operands use it; this one makes two vertically stacked accumulator tiles
// (rows 0-15 and 16-31 of a 32-row block) directly usable as a B fragment without any
// data movement.
//   bf16: one v_mfma_f32_16x16x32_bf16 consumes the 8 values (slot 8G + e <-> kmap(G, e)).
//   fp32: eight v_mfma_f32_16x16x4_f32, the e-th consuming value e of every lane group.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace atma {

typedef __bf16 bf16;
typedef _Float16 half;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ constexpr int kmap(int G, int e) { return e < 4 ? 4 * G + e : 12 + 4 * G + e; }

// ---- conversions ---------------------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

// exp2 / log2 on the hardware transcendental unit (ulp-level accurate for normal inputs).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---- fragments -------------------------------------------------------------------
template <typename T> struct Frag;
template <> struct Frag<bf16> {
    bf16x8 v;
    __device__ __forceinline__ void set(int e, float x) { v[e] = (bf16)x; }
    __device__ __forceinline__ void set_raw(int e, bf16 x) { v[e] = x; }
};
template <> struct Frag<half> {
    f16x8 v;
    __device__ __forceinline__ void set(int e, float x) { v[e] = (half)x; }
    __device__ __forceinline__ void set_raw(int e, half x) { v[e] = x; }
};
template <> struct Frag<float> {
    float v[8];
    __device__ __forceinline__ void set(int e, float x) { v[e] = x; }
    __device__ __forceinline__ void set_raw(int e, float x) { v[e] = x; }
};

__device__ __forceinline__ void mma(f32x4& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const Frag<half>& a, const Frag<half>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

// Fragment of a row-major matrix M (leading dimension ld, in elements) whose row for
// this lane is `row` and whose 32-wide reduction block starts at column k0: the lane
// reads M[row][k0 + kmap(G, e)] as two contiguous runs of 4.
__device__ __forceinline__ void load_frag_rows(Frag<bf16>& f, const bf16* M, int ld, int row, int k0) {
    const int G = lane_id() >> 4;
    const bf16* p = M + (size_t)row * ld + k0 + 4 * G;
    bf16x4 lo = *(const bf16x4*)p;
    bf16x4 hi = *(const bf16x4*)(p + 16);
    f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void load_frag_rows(Frag<float>& f, const float* M, int ld, int row, int k0) {
    const int G = lane_id() >> 4;
    const float* p = M + (size_t)row * ld + k0 + 4 * G;
    f32x4 lo = *(const f32x4*)p;
    f32x4 hi = *(const f32x4*)(p + 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) { f.v[e] = lo[e]; f.v[e + 4] = hi[e]; }
}
// Fragment read down a column: the lane reads M[k0 + kmap(G, e)][col].
template <typename T>
__device__ __forceinline__ void load_frag_cols(Frag<T>& f, const T* M, int ld, int col, int k0) {
    const int G = lane_id() >> 4;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.set_raw(e, M[(size_t)(k0 + kmap(G, e)) * ld + col]);
}

// Two vertically stacked accumulator tiles (reduction rows 0-15 and 16-31) as a B fragment.
template <typename T>
__device__ __forceinline__ void acc_to_frag(Frag<T>& f, const f32x4& top, const f32x4& bottom) {
#pragma unroll
    for (int e = 0; e < 4; ++e) { f.set(e, top[e]); f.set(e + 4, bottom[e]); }
}

// ---- LDS transpose reads and swizzled 16-bit tiles ------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ds_read_b64_tr_b16: within each 16-lane group, lane j supplies the address of a 4-element
// (8-byte) row r_j; lane i receives element (i mod 4) of rows r_{4e + i/4}, e = 0..3.  With
// lane j pointing at M[r0 + j/4][c0 + 4 (j mod 4)], lane i receives M[r0 + e][c0 + i].
__device__ __forceinline__ s16x4 tr_read_b16(const char* lds_byte_addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)lds_byte_addr);
}

// Byte offset of 16-bit element (r, c) in a row-major tile with RB-byte rows whose
// 16-byte chunks are XOR-swizzled by the row index (conflict-free column-slice reads).
template <int RB>
__device__ __host__ __forceinline__ constexpr int swz16(int r, int c) {
    return r * RB + ((((c >> 3) ^ (r & ((RB >> 4) - 1 > 15 ? 15 : (RB >> 4) - 1)))) << 4) + ((c & 7) << 1);
}

// A or B fragment (kmap order) from a swizzled 16-bit tile: row `row`, reduction columns
// k0 + kmap(G, e) -- two 8-byte reads.
template <int RB>
__device__ __forceinline__ f16x8 frag_swz_f16(const char* tile, int row, int k0) {
    const int G = lane_id() >> 4;
    const f16x4 lo = *(const f16x4*)(tile + swz16<RB>(row, k0 + 4 * G));
    const f16x4 hi = *(const f16x4*)(tile + swz16<RB>(row, k0 + 16 + 4 * G));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
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
// LDS byte address of a __shared__ object (a constant for a named array).
__device__ __forceinline__ unsigned lds_addr(const void* p) {
    typedef __attribute__((address_space(3))) const char* lds_ptr;
    return (unsigned)(size_t)(lds_ptr)p;
}
// A wave-uniform 64-bit pointer, in scalar registers even where the compiler cannot prove it
// uniform (free when it already is).
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const unsigned long long x = (unsigned long long)p;
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)x);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(x >> 32));
    return (const void*)(((unsigned long long)hi << 32) | lo);
}

// Same copy with the global address split into a wave-uniform 64-bit base and a per-lane
// 32-bit byte offset, and the LDS destination given as a wave-uniform byte address.
__device__ __forceinline__ void lds_dma16(const void* sbase, unsigned voff, unsigned lds_wave_addr) {
    const unsigned m0v = __builtin_amdgcn_readfirstlane(lds_wave_addr);
    sbase = uniform_ptr(sbase);
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(sbase), "s"(m0v)
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

// Same with a wave-uniform 64-bit base, a per-lane 32-bit byte offset and a wave-uniform LDS
// byte address, 4 bytes per lane.
__device__ __forceinline__ void lds_dma4(const void* sbase, unsigned voff, unsigned lds_wave_addr) {
    const unsigned m0v = __builtin_amdgcn_readfirstlane(lds_wave_addr);
    sbase = uniform_ptr(sbase);
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %0, %1"
        :
        : "v"(voff), "s"(sbase), "s"(m0v)
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

// ---- wave reductions ---------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

}  // namespace atma

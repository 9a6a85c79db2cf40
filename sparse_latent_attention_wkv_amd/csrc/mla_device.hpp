// Device-side helpers shared by the gfx950 kernels: vector types, bf16 packing, MFMA wrappers
// and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kHidden = 7168;
constexpr int kLora = 512;
constexpr int kRope = 64;
constexpr int kKvAOut = 576;
constexpr int kHeads = 128;
constexpr int kNope = 128;
constexpr int kQkHead = 192;
constexpr int kVHead = 128;
constexpr int kKvBOut = 32768;
constexpr int kQRank = 1536;     // q_lora_rank (not on the pages; the library's fixed reading)

// bf16 storage <-> fp32 (exact widening).
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round two fp32 values to bf16 (nearest, ties to even; the gfx950 conversion instruction) and
// pack them, `lo` in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// 32x32x16 bf16 MFMA, fp32 accumulate. Operand layout (wave64): lane l supplies row/column
// (l % 32) and eight consecutive reduction indices selected by (l / 32); the 16 results of
// lane l are D[8*(r/4) + 4*(l/32) + (r%4)][l % 32], r = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

template <typename T>
__device__ __forceinline__ T ldg(const T* p) { return *p; }

// Non-temporal-free plain 16-byte global load / store.
__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void store16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x2 load8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ void store8(void* p, const u32x2& v) { *reinterpret_cast<u32x2*>(p) = v; }

// ---- Direct global->LDS loads issued from inline assembly.
// dma16(sbase, voff, lds): lane l's 16 bytes at sbase + voff land at LDS address lds + 16 l
// (global_load_lds_dwordx4, scalar-base form: sbase and the LDS address wave-uniform, voff a
// 32-bit byte offset per lane; M0 takes the LDS address, one wait state before the load reads
// it). Issued from assembly so that the compiler's wait bookkeeping does not see it: while such
// a load may be in flight, the compiler otherwise treats every LDS read as unordered with it and
// drains all outstanding LDS reads before each use. Every read of a destination therefore waits
// explicitly (vmcnt of the issuing waves, then a barrier); loads the compiler does not see only
// make its own vmcnt waits stricter.
__device__ __forceinline__ uint32_t uniform32(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const uint64_t x = (uint64_t)(size_t)p;
    return (const void*)(size_t)(((uint64_t)uniform32((uint32_t)(x >> 32)) << 32) | uniform32((uint32_t)x));
}
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, void* lds) {
    const uint32_t l = uniform32((uint32_t)(size_t)(__attribute__((address_space(3))) void*)lds);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(uniform_ptr(sbase)), "s"(l)
                 : "memory", "m0");
}
// The same load with the LDS destination given as a 32-bit LDS byte address (wave-uniform), so
// no generic-to-LDS pointer conversion (and its null check) is needed per load.
__device__ __forceinline__ void dma16_lds(const void* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(uniform_ptr(sbase)), "s"(uniform32(lds))
                 : "memory", "m0");
}
// 4-byte form: lane l's 4 bytes at sbase + voff land at LDS address lds + 4 l
// (global_load_lds_dword).
__device__ __forceinline__ void dma4_lds(const void* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :
                 : "v"(voff), "s"(uniform_ptr(sbase)), "s"(uniform32(lds))
                 : "memory", "m0");
}
// 32-bit LDS byte address of an LDS object.
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(T* p) {
    return (uint32_t)(size_t)(__attribute__((address_space(3))) T*)p;
}
// s_waitcnt immediate for vmcnt(n), n < 64 (bits 3:0 and 15:14), other counters unconstrained.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
// Workgroup barrier without the release fence of __syncthreads(), whose vmcnt(0) would drain
// loads still meant to be in flight. This thread's LDS reads complete first, so no later load
// into a buffer can overtake a read of it; loads that must have landed are waited for with vmcnt
// before the barrier.
__device__ __forceinline__ void barrier_keep_loads() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Sum over the 64 lanes of a wave; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

}  // namespace mla

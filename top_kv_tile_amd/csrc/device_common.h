// Device helpers shared by the attention kernels (gfx950): vector types, buffer
// resources, and the explicitly scheduled loads the multi-stage kernels use.
//
// The compiler cannot tell which LDS stage a buffer-to-LDS DMA writes. After a
// DMA issued through the builtin it therefore waits for every outstanding load
// before the next transposing LDS read (ds_read_b64_tr_b16), and
// __syncthreads() also waits for all loads. Kernels that keep tiles in flight
// across such reads and barriers issue their DMA with the instruction itself
// (it has no register result, so nothing the compiler tracks is left in
// flight), wait with explicit vmcnt counts and synchronise with a bare
// s_barrier. Such a kernel issues no DMA through the builtin, because the
// compiler assumes it owns M0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) short4_t lds_s4;
typedef const __attribute__((address_space(4))) int32_t cint32;

// s_waitcnt immediates (gfx9 encoding): vmcnt(n) with expcnt and lgkmcnt at their maximum.
constexpr int kVmcnt0 = 0x0F70;
// lgkmcnt(0) with vmcnt and expcnt at their maximum.
constexpr int kLgkmcnt0 = 0xC07F;
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0F70; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer resource over `bytes` bytes at p (stride 0, no swizzle): loads
// at offsets past `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}
// The same resource as four scalar words, for the DMA instructions below.
__device__ __forceinline__ u32x4 rsrc_words(const void* p, uint32_t bytes) {
    const uint64_t x = (uint64_t)p;
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((uint32_t)x);
    r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32) & 0xFFFFu);
    r[2] = __builtin_amdgcn_readfirstlane(bytes);
    r[3] = 0x00020000u;
    return r;
}
// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p);
}
// Buffer-to-LDS DMA: 16 bytes per lane from byte offset voff to LDS address lds + 16 * lane.
__device__ __forceinline__ void dma16(u32x4 rs, uint32_t lds, int voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rs) : "memory");
}
// Buffer-to-LDS DMA: 4 bytes per lane from byte offset voff to LDS address lds + 4 * lane.
__device__ __forceinline__ void dma4(u32x4 rs, uint32_t lds, int voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rs) : "memory");
}
// Workgroup barrier that, unlike __syncthreads(), does not wait for vector
// memory loads (tiles in flight stay in flight; the caller waits for the ones
// it needs with vmcnt first). It does wait for this wave's LDS operations
// (lgkmcnt(0)): a transposing or row read of a stage still queued at the
// barrier could otherwise be overtaken by another wave's DMA into that stage
// issued right after it.
__device__ __forceinline__ void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kLgkmcnt0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
// Uniform load through the constant address space: a scalar load (counted by
// lgkmcnt) when the index is wave-uniform. Only for data no kernel of the
// launch writes.
__device__ __forceinline__ int ld_scalar(const int32_t* p, int64_t i) { return ((cint32*)p)[i]; }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace nsa

// Device primitives for gfx950 (CDNA4): vector types, MFMA wrappers,
// conversions and lane exchanges used by the attention kernels.
//
// MFMA register layouts relied on (wave64, 32x32 output tiles):
//  * v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//      A: lane l holds 8 bf16 of row (l % 32); B: lane l holds 8 bf16 of
//      column (l % 32).  Element i of lane l in A multiplies element i of lane
//      (l' with the same l / 32) in B: the contraction index is a function of
//      (l / 32, i) that is the same for A and B, so any consistent assignment
//      of K-indices to (l / 32, i) gives the same product.
//      D: lane l, register r holds row 8*(r/4) + 4*(l/32) + (r%4), column l%32.
//  * v_mfma_i32_32x32x32_i8 and v_mfma_scale_f32_32x32x64_f8f6f4 (fp8) use
//    the same row/column/output layout with 16 and 32 8-bit values per lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_bf16: A lane l holds 8 bf16 of row l%16, B of column
// l%16 (contraction index a function of (l/16, element), the same for A and
// B); D lane l, register r holds row 4*(l/16) + r, column l%16.
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ i32x16 mfma_i8_32x32x32(i32x4 a, i32x4 b, i32x16 c)
{
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// FP8 (E4M3, format code 0 for both operands) with unit block scales
// (E8M0 exponent 127 == 2^0).
__device__ __forceinline__ f32x16 mfma_fp8_32x32x64(i32x8 a, i32x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

// Round-to-nearest-even fp32 -> bf16, two values packed low/high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// acc + lo + hi of a packed bf16 pair (one v_dot2c_f32_bf16 against (1, 1)):
// the sum of exactly the rounded values that enter a bf16 MFMA.
__device__ __forceinline__ float add_bf16x2(uint32_t u, float acc)
{
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u), ones, acc, false);
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// v_exp_f32: 2^x (exp2(-inf) == 0).
// max of three signed ints (the compiler forms v_max3_i32).  Written in C,
// not as inline asm: the compiler cannot see the operands of an asm
// instruction, so it would not insert the wait states a VALU read of a
// matrix-core result needs when the max directly follows the MFMA.
__device__ __forceinline__ int vmax3_i32(int a, int b, int c) { return max(max(a, b), c); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value held by the lane 32 positions away (lanes l and l ^ 32 exchange).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// v_permlane32_swap on two copies of x: one result holds the lower-half
// lanes' values in both halves, the other the upper-half lanes' values, so a
// symmetric combination of the two is the combination of lanes l and l ^ 32.
__device__ __forceinline__ float max_xor32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [I0, N).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Row m of a 32-row MFMA block is taken from index perm32(m): lane half g
// then holds indices 16g .. 16g+15 in accumulator registers 0..15.
__device__ __forceinline__ int perm32(int m) { return ((m >> 2) & 1) * 16 + (m >> 3) * 4 + (m & 3); }

// LDS byte address of a __shared__ pointer.
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// LDS reads issued as inline asm.  Kernels that fill LDS with direct
// global->LDS loads use them because the compiler cannot tell these reads
// from the in-flight direct loads of another stage and would otherwise wait
// for those loads; completion is awaited explicitly with lgkm_wait.
template <int OFF>
__device__ __forceinline__ u32x4 lds_read_b128(uint32_t addr)
{
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF) : "memory");
    return r;
}
template <int OFF>
__device__ __forceinline__ u32x2 lds_read_tr16_b64(uint32_t addr)
{
    u32x2 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF) : "memory");
    return r;
}

// Wait until at most N LDS operations are outstanding; the operand is tied
// to the wait so that its consumer cannot be scheduled above it.
template <int N, typename T>
__device__ __forceinline__ void lgkm_wait(T &v)
{
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "n"(N));
}

// Direct 16-byte global->LDS load: lane l's 16 bytes land at lds + 16*l.
__device__ __forceinline__ void dma16(const void *gsrc, void *lds)
{
    __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void *)lds, 16, 0,
                                     0);
}

// The same with the non-temporal cache policy, for data read exactly once
// (streamed K/V caches): on gfx950 such loads stream from HBM about 12% faster
// than loads with the default policy (measured 6.9 against 6.2 TB/s).
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ void dma16_nt(const void *gsrc, void *lds)
{
    __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void *)lds, 16, 0,
                                     kCachePolicyNT);
}

// Buffer resource for raw byte-addressed loads from [base, base + nbytes):
// loads at offsets >= nbytes return zero without touching memory.  base and
// nbytes must be wave-uniform (the resource lives in scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void *base, uint32_t nbytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)nbytes,
                                             0x00020000);
}

// 16-byte direct load through a buffer resource into LDS: lane l's bytes
// [voff, voff + 16) land at lds + 16 * l (lds wave-uniform).
__device__ __forceinline__ void dma16_rsrc(__amdgpu_buffer_rsrc_t r, uint32_t voff, void *lds)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16,
                                             voff, 0, 0, 0);
}

// The same with a wave-uniform byte offset soff added to voff (a scalar
// operand, so that loads at different soff share one voff register).
__device__ __forceinline__ void dma16_rsrc_so(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                              void *lds)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16,
                                             voff, soff, 0, 0);
}

// 4-byte direct load through a buffer resource into LDS: lane l's bytes
// [voff, voff + 4) land at lds + 4 * l (lds wave-uniform).
__device__ __forceinline__ void dma4_rsrc(__amdgpu_buffer_rsrc_t r, uint32_t voff, void *lds)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 4,
                                             voff, 0, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void vm_wait_n()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void vm_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Global loads/stores of 16 bytes.
__device__ __forceinline__ u32x4 ld16(const void *p) { return *(const u32x4 *)p; }
// a 16-byte load with the non-temporal cache policy (see dma16_nt)
__device__ __forceinline__ u32x4 ld16_nt(const void *p)
{
    return __builtin_nontemporal_load((const u32x4 *)p);
}
__device__ __forceinline__ void st16(void *p, u32x4 v) { *(u32x4 *)p = v; }

}  // namespace attn

// Device-side helpers shared by the MoE kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest even (gfx950's v_cvt_pk_bf16_f32);
// NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16). Lane l supplies row l%16
// of A and column l%16 of B, eight consecutive k each at k-offset 8*(l/16);
// it receives D rows 4*(l/16)+0..3 of column l%16.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Unconditional 16-byte load. Callers pass an address that is always valid
// (clamped) and zero the value afterwards with sel() when it lies outside the
// operand, so the compiler never wraps loads in branches and can keep several
// of them in flight.
__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *(const u32x4*)p; }
__device__ __forceinline__ u32x4 sel(bool keep, u32x4 v) {
    return u32x4{keep ? v[0] : 0u, keep ? v[1] : 0u, keep ? v[2] : 0u, keep ? v[3] : 0u};
}

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16). Lane l supplies row
// l%32 of A and column l%32 of B, eight k each at k-offset 8*(l/32); it
// receives D[8*(i/4) + 4*(l/32) + i%4][l%32] in element i (checked on the
// device).
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

typedef __attribute__((address_space(3))) void lds_void;

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's 16 bytes land at lds_base + 16*l. lds_base must be wave-uniform.
// The compiler does not order later LDS reads after these copies: callers
// wait with vm_wait() and a barrier.
__device__ __forceinline__ void lds_dma16(const void* g, void* lds_base) {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_base, 16, 0, 0);
}

// s_waitcnt vmcnt(N) (gfx9 encoding; expcnt and lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS only: waits for this wave's LDS accesses, then
// s_barrier; the fences (LDS address space, workgroup scope) keep the
// compiler from moving LDS accesses across it without waiting on global loads.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Index of element (r, c) of a bf16 matrix with `cols` columns (a multiple
// of 32) stored as MFMA fragment blocks, the layout of moe_pack_weights and
// of act: 16-row x 32-column blocks of 512 elements, row-band major, column
// block minor; inside a block lane l = 16*((c%32)/8) + r%16 holds columns
// 8*((c%32)/8) .. +7 of row r, so one 16-byte lane load is one lane of an
// MFMA operand fragment.
__device__ __forceinline__ int64_t frag_index(int64_t r, int c, int cols) {
    return ((r >> 4) * (cols >> 5) + (c >> 5)) * 512 + ((((c & 31) >> 3) << 4) + (r & 15)) * 8 + (c & 7);
}

// One element of the down projection's output: fp16 (round to nearest even)
// when Y16, else fp32.
template <bool Y16>
__device__ __forceinline__ void store_y(void* y, int64_t idx, float v) {
    if constexpr (Y16)
        ((_Float16*)y)[idx] = (_Float16)v;
    else
        ((float*)y)[idx] = v;
}

// f(std::integral_constant<int, I>{}) for I = B .. E-1, unrolled at compile
// time (for counts that must be template arguments, such as vm_wait's).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// SiLU z * sigmoid(z) with the hardware reciprocal (about 1 ulp, far below
// the bf16 rounding that follows): exp(-z) overflowing to inf gives -0.
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

template <typename T>
__device__ __forceinline__ T wave_shfl_xor(T v, int mask) {
    return __shfl_xor(v, mask, kWave);
}

}  // namespace moe

// Device-side helpers shared by the gfx950 kernels of libtpshard.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace tpk {

// Compile-time loop: f(std::integral_constant<int, 0>{}), ..., up to N - 1.
// Register-resident arrays indexed through it see constant indices from the
// start, so they are never demoted to scratch memory.
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// bf16 is handled as raw 16-bit patterns in memory.
typedef uint16_t bf16_t;

// MFMA operand / accumulator vector types (gfx950 builtins).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// 16-byte loads with the non-temporal hint (data read exactly once: keep it
// from displacing reusable lines in L2).
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
}
__device__ __forceinline__ float4 ld_nt16f(const void* p) {
    return __builtin_bit_cast(float4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
}

// Buffer resources: a scalar base and extent in bytes (a read past the
// extent returns zeros), addressed by 32-bit lane offsets plus an immediate
// or scalar offset, so an operand read this way stays below kMaxBufferBytes
// (kernels.h). Word 3 of an untyped buffer resource: 32-bit data format, no
// swizzle, no index stride.
constexpr int kRawBufferWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_source(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(uint32_t)bytes, kRawBufferWord3);
}
__device__ __forceinline__ uint4 buffer_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

// fp32 -> bf16, round to nearest, ties to even. NaN stays NaN (quieted);
// overflow past the largest finite bf16 rounds to infinity; subnormals round
// on the same grid as normals (bf16 and fp32 share the exponent field).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x0040u) & 0xffffu;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Workgroup barrier for data exchanged through LDS only. It waits for this
// wave's LDS accesses but not for its outstanding global loads; a plain
// __syncthreads() is a release of all memory and, since global loads and
// stores share one counter on this GPU, waits for every load in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// SiLU of [P1 3.2]'s SwiGLU MLP: g / (1 + e^-g). For very negative g, e^-g
// overflows to +inf and the quotient is -0, the limit; for large positive g
// it is g. Shared by the SwiGLU kernel and the fused GEMM epilogue so both
// give the same bits.
__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

// Pack two fp32 values as bf16 into one 32-bit word (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// Unpack the 8 bf16 values of a 16-byte vector to fp32.
__device__ __forceinline__ void unpack_bf16x8(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
}

__device__ __forceinline__ uint4 pack_bf16x8(const float* f) {
    uint4 v;
    v.x = pack_bf16x2(f[0], f[1]);
    v.y = pack_bf16x2(f[2], f[3]);
    v.z = pack_bf16x2(f[4], f[5]);
    v.w = pack_bf16x2(f[6], f[7]);
    return v;
}

}  // namespace tpk

// tq_device.h -- small device helpers shared by the library's HIP kernels.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace tq {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct f32_tag {};
struct bf16_tag {};
struct f16_tag {};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
    _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
    return (float)h;
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
    _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    return (float)h;
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// 8 consecutive elements starting at element `off` (16-byte aligned for 16-bit types,
// 32-byte aligned for fp32), converted to fp32.
__device__ __forceinline__ void load8(const void *base, int64_t off, float (&o)[8], f32_tag) {
    const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(base) + off);
    float4 a = p[0], b = p[1];
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
__device__ __forceinline__ void load8(const void *base, int64_t off, float (&o)[8], bf16_tag) {
    uint4 a = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + off);
    o[0] = bf16_lo(a.x); o[1] = bf16_hi(a.x); o[2] = bf16_lo(a.y); o[3] = bf16_hi(a.y);
    o[4] = bf16_lo(a.z); o[5] = bf16_hi(a.z); o[6] = bf16_lo(a.w); o[7] = bf16_hi(a.w);
}
__device__ __forceinline__ void load8(const void *base, int64_t off, float (&o)[8], f16_tag) {
    uint4 a = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + off);
    o[0] = f16_lo(a.x); o[1] = f16_hi(a.x); o[2] = f16_lo(a.y); o[3] = f16_hi(a.y);
    o[4] = f16_lo(a.z); o[5] = f16_hi(a.z); o[6] = f16_lo(a.w); o[7] = f16_hi(a.w);
}

__device__ __forceinline__ float load1(const void *base, int64_t off, f32_tag) {
    return static_cast<const float *>(base)[off];
}
__device__ __forceinline__ float load1(const void *base, int64_t off, bf16_tag) {
    return __uint_as_float((uint32_t)static_cast<const uint16_t *>(base)[off] << 16);
}
__device__ __forceinline__ float load1(const void *base, int64_t off, f16_tag) {
    return (float)__builtin_bit_cast(_Float16, static_cast<const uint16_t *>(base)[off]);
}

// flip the sign of x when bit is 1
__device__ __forceinline__ float flip_sign(float x, uint32_t bit) {
    return __uint_as_float(__float_as_uint(x) ^ (bit << 31));
}

}  // namespace tq

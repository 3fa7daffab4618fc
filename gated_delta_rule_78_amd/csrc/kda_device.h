// Device-side helpers for the gfx950 KDA kernels: element conversion, MFMA operand policies,
// wave-local LDS ordering. Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

typedef uint16_t bf16_t;  // raw bfloat16 bits in memory

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Scalar element load / store as float for the two storage types.
__device__ __forceinline__ float ld_f(const bf16_t* p) { return bf16_bits_to_f32(*p); }
__device__ __forceinline__ float ld_f(const float* p) { return *p; }
__device__ __forceinline__ void st_f(bf16_t* p, float x) { *p = f32_to_bf16_bits(x); }
__device__ __forceinline__ void st_f(float* p, float x) { *p = x; }

// Unpack 16 bytes of storage into floats.
__device__ __forceinline__ void unpack16(uint4 u, const bf16_t*, float* out) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(w[i] << 16);
        out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void unpack16(uint4 u, const float*, float* out) {
    out[0] = __uint_as_float(u.x); out[1] = __uint_as_float(u.y);
    out[2] = __uint_as_float(u.z); out[3] = __uint_as_float(u.w);
}
template <typename T> struct ElemsPer16 { static constexpr int value = 16 / sizeof(T); };

// Store 4 consecutive floats as storage type T (8 bytes for bf16, 16 bytes for fp32).
__device__ __forceinline__ void store4(bf16_t* p, float a, float b, float c, float d) {
    uint2 u;
    u.x = (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
    u.y = (uint32_t)f32_to_bf16_bits(c) | ((uint32_t)f32_to_bf16_bits(d) << 16);
    *reinterpret_cast<uint2*>(p) = u;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// Order this wave's LDS writes before its later LDS reads (all lanes of the wave).
__device__ __forceinline__ void wave_lds_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------------------------------------
// MFMA operand policies. Fragment convention for a 16x16 output tile (lane l in 0..63):
//   A operand: row m = l % 16, a run of consecutive k starting at kw * (l / 16)
//   B operand: col n = l % 16, the same run of k
//   D (4 floats): rows 4 * (l / 16) + r (r = 0..3), col l % 16
// K32 fragments hold 8 consecutive k, K16 fragments 4. Because A and B use the same k
// placement, any k permutation the hardware applies cancels in the product.
// ---------------------------------------------------------------------------------------------
struct OpBF16 {
    typedef bf16_t elem;
    typedef bf16x8 frag32;
    typedef i16x4 frag16;
    __device__ static __forceinline__ frag32 load32(const elem* p) { return *reinterpret_cast<const bf16x8*>(p); }
    __device__ static __forceinline__ frag16 load16(const elem* p) { return *reinterpret_cast<const i16x4*>(p); }
    __device__ static __forceinline__ f32x4 mma32(frag32 a, frag32 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ f32x4 mma16(frag16 a, frag16 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ elem cvt(float x) { return f32_to_bf16_bits(x); }
};

struct OpF32 {
    typedef float elem;
    struct frag32 { f32x4 lo, hi; };
    typedef f32x4 frag16;
    __device__ static __forceinline__ frag32 load32(const elem* p) {
        frag32 f;
        f.lo = *reinterpret_cast<const f32x4*>(p);
        f.hi = *reinterpret_cast<const f32x4*>(p + 4);
        return f;
    }
    __device__ static __forceinline__ frag16 load16(const elem* p) { return *reinterpret_cast<const f32x4*>(p); }
    __device__ static __forceinline__ f32x4 mma16(frag16 a, frag16 b, f32x4 c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
        return c;
    }
    __device__ static __forceinline__ f32x4 mma32(frag32 a, frag32 b, f32x4 c) {
        c = mma16(a.lo, b.lo, c);
        return mma16(a.hi, b.hi, c);
    }
    __device__ static __forceinline__ elem cvt(float x) { return x; }
};

}  // namespace kda

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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats to two bfloat16 (round to nearest even) in one 32-bit word, low half = a.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Store 4 consecutive floats as storage type T (8 bytes for bf16, 16 bytes for fp32).
__device__ __forceinline__ void store4(bf16_t* p, float a, float b, float c, float d) {
    uint2 u;
    u.x = pack_bf16x2(a, b);
    u.y = pack_bf16x2(c, d);
    *reinterpret_cast<uint2*>(p) = u;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// Store 8 consecutive floats (16 bytes for bf16, 32 bytes for fp32).
__device__ __forceinline__ void store8(bf16_t* p, const float* x) {
    uint4 u;
    u.x = pack_bf16x2(x[0], x[1]); u.y = pack_bf16x2(x[2], x[3]);
    u.z = pack_bf16x2(x[4], x[5]); u.w = pack_bf16x2(x[6], x[7]);
    *reinterpret_cast<uint4*>(p) = u;
}
__device__ __forceinline__ void store8(float* p, const float* x) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}

// Lane shuffle within a wave via DPP; lanes whose source is outside the pattern read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, true));
}

// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele inside each 16-lane row
// (row_shr 1, 2, 4, 8), then row 0's total into rows 1 and 3 (row_bcast:15) and lane 31's
// total into rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ float wave_prefix_sum(float x) {
    x += dpp_f32<0x111, 0xf>(x);
    x += dpp_f32<0x112, 0xf>(x);
    x += dpp_f32<0x114, 0xf>(x);
    x += dpp_f32<0x118, 0xf>(x);
    x += dpp_f32<0x142, 0xa>(x);
    x += dpp_f32<0x143, 0xc>(x);
    return x;
}

__device__ __forceinline__ float lane_value(float x, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// Order this wave's LDS writes before its later LDS reads (all lanes of the wave).
// The lane's index in its wave, computed where it is used: a volatile asm is neither hoisted out
// of a loop nor merged with another, so the addresses a phase derives from it are rebuilt (a few
// ALU operations) instead of being held in registers across a long loop, where the register
// allocator would spill them and reload them behind waits on the memory queue.
__device__ __forceinline__ int fresh_lane() {
    int x;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(x));
    return x;
}

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

// Workgroup barrier that orders LDS accesses only. __syncthreads() also waits for every
// outstanding global load and store of the wave; this one lets a prefetch stay in flight across
// it. For kernels whose workgroups never read back, through global memory, what they wrote there.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace kda

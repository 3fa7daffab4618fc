// gfx950 MFMA fragment helpers, LDS transposed reads and raw buffer access shared by the bf16
// prefill kernels. Internal to the library.
//
// Fragment convention for one 16x16 output tile, lane l (l16 = l % 16, lq = l / 16):
//   A operand (16 x K): row l16, a run of k values held in register order e = 0..7 (K32) or
//                       e = 0..3 (K16)
//   B operand (K x 16): column l16, the same run of k
//   D (4 floats):       rows 4*lq + r (r = 0..3), column l16
// A and B share the k placement, so any permutation of k cancels in the product. The kernels
// use, for a K32 fragment over a 32-wide k window, k(e) = 16*(e/4) + 4*lq + e%4: with it, the
// D registers of two vertically adjacent 16x16 tiles are exactly one K32 B (or A^T) operand,
// so accumulators feed the next product without leaving registers.
#pragma once

#include "kda_device.h"

namespace kda {

typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// ds_read_b64_tr_b16. Within each 16-lane group, lane i receives as element k (k = 0..3) the
// (i % 4)-th 16-bit value of the 8-byte chunk addressed by lane 4k + i/4 of the same group.
// From a row-major bf16 matrix X (row stride ld elements), the address
//   &X[(r0 + 4*lq + l16/4) * ld + m0 + 4*(l16 % 4)]
// yields element e = X[r0 + 4*lq + e][m0 + l16]: a K16 operand whose k runs down the rows.
__device__ __forceinline__ i16x4 tr_read(const bf16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}
__device__ __forceinline__ i16x4 read8(const void* p) { return *reinterpret_cast<const i16x4*>(p); }
__device__ __forceinline__ bf16x8 read16(const void* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16x8 cat(i16x4 a, i16x4 b) {
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}
__device__ __forceinline__ i16x4 lo4(bf16x8 v) {
    return __builtin_shufflevector(__builtin_bit_cast(i16x8, v), __builtin_bit_cast(i16x8, v), 0, 1, 2, 3);
}
__device__ __forceinline__ i16x4 hi4(bf16x8 v) {
    return __builtin_shufflevector(__builtin_bit_cast(i16x8, v), __builtin_bit_cast(i16x8, v), 4, 5, 6, 7);
}
// Four floats to four bf16 (round to nearest even), packed as a K16 fragment.
__device__ __forceinline__ i16x4 cvt4(f32x4 x) {
    uint2 u;
    u.x = pack_bf16x2(x[0], x[1]);
    u.y = pack_bf16x2(x[2], x[3]);
    return __builtin_bit_cast(i16x4, u);
}
__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(i16x4 a, i16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 unpack4f(i16x4 v) {
    const uint2 u = __builtin_bit_cast(uint2, v);
    f32x4 f;
    f[0] = __uint_as_float(u.x << 16); f[1] = __uint_as_float(u.x & 0xffff0000u);
    f[2] = __uint_as_float(u.y << 16); f[3] = __uint_as_float(u.y & 0xffff0000u);
    return f;
}
constexpr f32x4 kZero4 = {0.f, 0.f, 0.f, 0.f};

// A value the compiler may hold per lane but that is the same in every lane (e.g. a 64-bit
// quotient of block indices), moved to scalar registers so that addresses built from it stay
// scalar (buffer descriptors in particular).
__device__ __forceinline__ int64_t uniform64(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// True when every window flag [0, nseg - 1) of a lane is set: the entry states of all its
// segments came from the window launch of a sequence split, so its pass 1 and scan are skipped.
__device__ __forceinline__ bool window_split_exact(const int32_t* flag, int nseg) {
    int all = 1;
    for (int s = 0; s + 1 < nseg; ++s) all &= flag[s];
    return all != 0;
}

// Broadcast lane 15 of each 16-lane row to the whole row (DPP row_newbcast:15).
__device__ __forceinline__ float row_bcast15(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x15F, 0xf, 0xf, false));
}

// Raw buffer access (gfx9 descriptor): an offset at or beyond num_records reads zeros and drops
// stores, so rows past the end of a sequence need neither clamping nor branches. The address is
// base + voffset (per lane) + soffset (uniform), but only voffset is range-checked against
// num_records: an offset that must read as zero past the end belongs in voffset.
constexpr int32_t kBufFlags = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufFlags);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, (int)soff, 0));
}
__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
// Store four floats at byte offset `off` as bf16 (8 bytes) or fp32 (16 bytes).
__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, bf16_t*, f32x4 x) {
    uint2 u;
    u.x = pack_bf16x2(x[0], x[1]);
    u.y = pack_bf16x2(x[2], x[3]);
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, u), r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, float*, f32x4 x) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, x), r, (int)off, 0, 0);
}

}  // namespace kda

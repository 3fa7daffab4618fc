// The state step of the chunk form and the record copy that feeds it, shared by the state pass
// (kda_inter.hip) and the fused single-pass kernel (kda_fused.hip). Kimi K3 reading notes,
// liuzhao09.github.io/papers/kimi-k3.html, section 2.2 chunk equations: for the chunk's record
// (kda_record.h) and entry state S,
//   V~ = U - W S,   O = Q~ S + A_qk V~,   S <- Diag(gamma_C) S + K-^T V~.
// Internal to the library.
#pragma once

#include "kda_internal.h"
#include "kda_mfma.h"
#include "kda_record.h"

namespace kda {

// Where a lane's rows, records and checkpoints are (SeqMap): its first row in the row-major
// tensors, its length, its first record slot, and the index of its first checkpoint and the
// stride between its checkpoints (ChunkLaunch::ckpt). Packed lengths are clamped into the rows
// and to max_len, so malformed lengths give wrong numbers but no access outside the tensors.
struct LaneSpan {
    int64_t row_base, len, slot0, ck_base, ck_stride;
};
__device__ __forceinline__ LaneSpan lane_span(const ChunkLaunch& p, int64_t lane) {
    LaneSpan r{0, 0, 0, 0, 1};
    if (p.map.cu) {
        const int64_t s = uniform64(lane / p.map.H), h = uniform64(lane % p.map.H);
        const int64_t rows = p.map.rows;
        int64_t c0 = p.map.cu[s], c1 = p.map.cu[s + 1];
        c0 = c0 < 0 ? 0 : (c0 > rows ? rows : c0);
        c1 = c1 < c0 ? c0 : (c1 > rows ? rows : c1);
        r.len = c1 - c0 < p.map.max_len ? c1 - c0 : p.map.max_len;
        r.row_base = h * rows + c0;
        r.slot0 = h * p.map.slots + (c0 >> 6) + s;
        if (p.ckpt) { r.ck_base = (int64_t)p.ck_off[s] * p.map.H + h; r.ck_stride = p.map.H; }
    } else {
        r.len = p.T;
        r.row_base = lane * p.T;
        r.slot0 = lane * p.nchunks;
        if (p.ckpt) {   // sequence s = lane / H has its checkpoints at rows s * ck_per_lane + j - 1
            const int64_t s = uniform64(lane / p.map.H), h = uniform64(lane % p.map.H);
            r.ck_base = s * p.ck_per_lane * p.map.H + h;
            r.ck_stride = p.map.H;
        }
    }
    r.row_base = uniform64(r.row_base); r.len = uniform64(r.len); r.slot0 = uniform64(r.slot0);
    r.ck_base = uniform64(r.ck_base); r.ck_stride = uniform64(r.ck_stride);
    return r;
}

// The segments that hold a lane's nch chunks: [0, live), live >= 1. A packed batch plans its
// segments for its longest sequence, so a shorter lane ends in an earlier segment, which then
// finishes the lane (S_T); the boundaries past it have no window and count as exact. (Equal
// lengths: live = nseg.)
__device__ __forceinline__ int live_segments(const ChunkLaunch& p, int64_t nch) {
    const int64_t n = (nch + p.chunks_per_seg - 1) / p.chunks_per_seg;
    return (int)uniform64(n < 1 ? 1 : (n > p.nseg ? p.nseg : n));
}

// Four output values in storage form (bf16: 8 bytes; fp32: 16 bytes) and their buffer store.
__device__ __forceinline__ void store_out(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 x, bf16_t*) {
    typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
    const u32x2 u = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    __builtin_amdgcn_raw_buffer_store_b64(u, r, (int)off, 0, 0);
}
__device__ __forceinline__ void store_out(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 x, float*) {
    typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, (int)off, 0, 0);
}

// Store two 16-column output tiles of one token row (accumulator layout: lane (lq, l16) holds
// columns 4 lq .. 4 lq + 3 of each tile for token l16). One permlane16 swap per register trades
// rows 1 <-> 0 and 3 <-> 2 between the tiles, after which lane lq holds the 8 consecutive columns
// starting at 16 (lq & 1) + 8 (lq >> 1): a 16-byte store per lane, and every token row written in
// whole 64-byte pieces (two 8-byte stores per lane wrote 32-byte pieces).
__device__ __forceinline__ void swap_pair(f32x4 x, f32x4 y, f32x4& a, f32x4& b) {
    typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u32x2 sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[i]), __float_as_uint(y[i]), false, false);
        a[i] = __uint_as_float(sw[0]);
        b[i] = __uint_as_float(sw[1]);
    }
}
// first of the lane's 8 consecutive columns within a pair of tiles, after swap_pair
__device__ __forceinline__ uint32_t pair_col(int lq) { return 16u * (uint32_t)(lq & 1) + 8u * (uint32_t)(lq >> 1); }
__device__ __forceinline__ void store_bf16x8(__amdgpu_buffer_rsrc_t r, uint32_t elem_off, f32x4 a, f32x4 b) {
    typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
    const u32x4 u = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
    __builtin_amdgcn_raw_buffer_store_b128(u, r, (int)(elem_off * 2u), 0, 0);
}


// Fused epilogue of one output tile: y = sigmoid(gate) * w * o * rstd for 4 columns of a token.
__device__ __forceinline__ f32x4 gated_norm(f32x4 o, uint2 g, f32x4 w, float rstd) {
    const float gv[4] = {__uint_as_float(g.x << 16), __uint_as_float(g.x & 0xffff0000u),
                         __uint_as_float(g.y << 16), __uint_as_float(g.y & 0xffff0000u)};
    f32x4 y;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        y[r] = o[r] * rstd * w[r] * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-gv[r] * kLog2e));
    return y;
}

// Copy this wave's share (blocks w, w + 4, ...) of the blocks of one chunk record that a role
// reads (FINISH: all; SUMMARY: all but Q~ and A_qk) into an LDS buffer: one direct-to-LDS buffer
// load per 1 KiB block; the descriptor covers the chunk's record, offsets stay scalar. Every wave
// issues the same count: indices past the end repeat the last block (the same bytes to the same
// place), which keeps the copy free of branches.
template <int DK, int DV, bool FIN>
struct CopyPlan {
    typedef RecordLayout<DK, DV> R;
    static constexpr int NSKIP = 4 * R::NKS;
    static constexpr int NLOAD = FIN ? R::BLOCKS : R::BLOCKS - NSKIP - 6;
    static constexpr int ITERS = (NLOAD + 3) / 4;                 // loads per wave
    static constexpr int PART = (ITERS + R::NKS - 1) / R::NKS;   // loads per k step of a chunk
};

// Loads I0 .. I1 - 1 of this wave's share (all of them by default).
template <int DK, int DV, bool FIN, int I0 = 0, int I1 = CopyPlan<DK, DV, FIN>::ITERS>
__device__ __forceinline__ void copy_record(__amdgpu_buffer_rsrc_t rsrc, uint32_t chunk_off, unsigned char* dst, int w, int l) {
    typedef RecordLayout<DK, DV> R;
    constexpr int NSKIP = CopyPlan<DK, DV, FIN>::NSKIP;
    constexpr int NLOAD = CopyPlan<DK, DV, FIN>::NLOAD;
    constexpr int IEND = I1 < (NLOAD + 3) / 4 ? I1 : (NLOAD + 3) / 4;
#pragma unroll
    for (int i = I0; i < IEND; ++i) {
        const int b = w + 4 * i < NLOAD ? w + 4 * i : NLOAD - 1;
        const int blk = FIN ? b : (b < R::Q ? b : (b < R::Q + 2 * R::NM ? b + NSKIP : b + NSKIP + 6));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + blk * 1024), 16, (unsigned)(l * 16),
                                                 chunk_off + (uint32_t)(blk * 1024), 0, 0);
    }
}

// One chunk for state tiles G0 .. G0 + NTG - 1 of this wave. Tile nt < nu is value-column tile
// col0 / 16 + nt (U added); the tiles from nu on are columns of M (U = 0; SUMMARY and WINDOW).
// The next chunk's record copy (when `copy`) is issued in parts, one after each k step of the
// first products: issued in one piece before them, its stalls (the copies queue behind the
// record stream) kept the wave from starting the products for about a microsecond per chunk.
// With `ureg`, the U tiles come from registers (ureg[nt][I]: the record's bf16 U values of tile
// G0 + nt, rows 16I + 4lq + r) instead of the record.
template <typename TOut, int DK, int DV, int NT, int G0, int NTG, bool FIN>
__device__ __forceinline__ void chunk_step(const unsigned char* rbuf, f32x4 (&S)[NT][DK / 16], int col0, int nu,
                                           f32x4 (&Opend)[NT][4], bool copy, __amdgpu_buffer_rsrc_t crs,
                                           unsigned char* cdst, int w, const i16x4 (*ureg)[4] = nullptr) {
    typedef CopyPlan<DK, DV, FIN> CP;
    typedef RecordLayout<DK, DV> R;
    constexpr int NKS = R::NKS, NM = R::NM;
    const int l = threadIdx.x & 63;
    const int lq = l >> 4;
    const unsigned char* rb = rbuf + l * 16;
#define KDA_FRAG(b) read16(rb + (b) * 1024)

    // V~ = U + (-W) S (rows = tokens 16I + 4lq + r; U = 0 on SUMMARY's M columns) and, for
    // FINISH, O^T = S^T Q~^T. k steps outer: each step converts its slice of S once and issues
    // 4 NTG (+ 4 NTG) independent MFMAs.
    f32x4 Vt[NTG][4], Ot[NTG][4];
#pragma unroll
    for (int nt = 0; nt < NTG; ++nt) {
        const int n = col0 / 16 + G0 + nt;
        if (ureg) {
#pragma unroll
            for (int I = 0; I < 4; ++I) Vt[nt][I] = unpack4f(ureg[G0 + nt][I]);
        } else if (FIN || G0 + nt < nu) {
            const bf16x8 u0 = KDA_FRAG(R::u(n, 0));
            const bf16x8 u1 = KDA_FRAG(R::u(n, 1));
            Vt[nt][0] = unpack4f(lo4(u0)); Vt[nt][1] = unpack4f(hi4(u0));
            Vt[nt][2] = unpack4f(lo4(u1)); Vt[nt][3] = unpack4f(hi4(u1));
        } else {
#pragma unroll
            for (int I = 0; I < 4; ++I) Vt[nt][I] = kZero4;
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) Ot[nt][I] = kZero4;
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        bf16x8 sk[NTG];
#pragma unroll
        for (int nt = 0; nt < NTG; ++nt) sk[nt] = cat(cvt4(S[G0 + nt][2 * ks]), cvt4(S[G0 + nt][2 * ks + 1]));
        bf16x8 wa[4], qb[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            wa[I] = KDA_FRAG(R::w(I, ks));
            if (FIN) qb[I] = KDA_FRAG(R::q(I, ks));
        }
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int nt = 0; nt < NTG; ++nt) Vt[nt][I] = mma32(wa[I], sk[nt], Vt[nt][I]);
        if (FIN) {
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int nt = 0; nt < NTG; ++nt) Ot[nt][I] = mma32(sk[nt], qb[I], Ot[nt][I]);
        }
        if (copy) {
            if (ks == 0) copy_record<DK, DV, FIN, 0, CP::PART>(crs, 0u, cdst, w, l);
            if (ks == 1) copy_record<DK, DV, FIN, CP::PART, 2 * CP::PART>(crs, 0u, cdst, w, l);
            if (ks == 2) copy_record<DK, DV, FIN, 2 * CP::PART, 3 * CP::PART>(crs, 0u, cdst, w, l);
            if (ks == 3) copy_record<DK, DV, FIN, 3 * CP::PART, 4 * CP::PART>(crs, 0u, cdst, w, l);
        }
    }
    // V~ as K32 B operands over tokens 0..31 (v01) and 32..63 (v23)
    bf16x8 v01[NTG], v23[NTG];
#pragma unroll
    for (int nt = 0; nt < NTG; ++nt) {
        v01[nt] = cat(cvt4(Vt[nt][0]), cvt4(Vt[nt][1]));
        v23[nt] = cat(cvt4(Vt[nt][2]), cvt4(Vt[nt][3]));
    }
    if (FIN) {
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            const bf16x8 a0 = KDA_FRAG(R::a(I, 0));
#pragma unroll
            for (int nt = 0; nt < NTG; ++nt) Ot[nt][I] = mma32(v01[nt], a0, Ot[nt][I]);
            if (I >= 2) {
                const bf16x8 a1 = KDA_FRAG(R::a(I, 1));
#pragma unroll
                for (int nt = 0; nt < NTG; ++nt) Ot[nt][I] = mma32(v23[nt], a1, Ot[nt][I]);
            }
            // O^T tile: rows = columns 4lq + r, column = token 16I + l16 (stored next iteration)
#pragma unroll
            for (int nt = 0; nt < NTG; ++nt) Opend[G0 + nt][I] = Ot[nt][I];
        }
    }
    // S <- Diag(gamma_C) S + K-^T V~, in two sweeps of independent MFMAs
    const float* gam = reinterpret_cast<const float*>(rbuf + R::G * 1024);
#pragma unroll
    for (int M = 0; M < NM; ++M) {
        const f32x4 g4 = *reinterpret_cast<const f32x4*>(&gam[16 * M + 4 * lq]);
        const bf16x8 k0 = KDA_FRAG(R::k(M, 0));
#pragma unroll
        for (int nt = 0; nt < NTG; ++nt) S[G0 + nt][M] = mma32(k0, v01[nt], g4 * S[G0 + nt][M]);
    }
#pragma unroll
    for (int M = 0; M < NM; ++M) {
        const bf16x8 k1 = KDA_FRAG(R::k(M, 1));
#pragma unroll
        for (int nt = 0; nt < NTG; ++nt) S[G0 + nt][M] = mma32(k1, v23[nt], S[G0 + nt][M]);
    }
#undef KDA_FRAG
}

}  // namespace kda

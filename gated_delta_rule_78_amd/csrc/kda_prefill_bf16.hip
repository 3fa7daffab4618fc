// KDA chunkwise prefill for gfx950, bf16 inputs: register-resident state path.
//
// Mathematics as in kda_chunk.hip (Kimi K3 reading notes, liuzhao09.github.io/papers/kimi-k3.html,
// section 2.2 chunk equations, section 2.5 affine pair). For a 64-row chunk with entry state S,
// G = cumsum(log alpha) per key channel, Gamma = exp(G), gamma_C = Gamma_C:
//   Q~ = Q*Gamma, K~ = K*Gamma, K^ = K/Gamma
//   A_kk = Diag(beta) StrictTril(K~ K^^T),  A_qk = Tril(Q~ K^^T)
//   V~ = (I + A_kk)^{-1} Diag(beta) (V - K~ S)
//   O  = Q~ S + A_qk V~
//   S' = Diag(gamma_C) (S + K^^T V~)          (= Diag(gamma_C) S + (K*gamma_C/Gamma)^T V~)
//
// gfx950 mapping. A workgroup of NW waves owns (lane, segment, NW*16 state columns); wave w owns
// 16 columns. Everything that depends on the state stays in registers:
//  * MFMA operand placement: a 16x16x32 bf16 fragment holds 8 k-values per lane; A and B share
//    the placement, so any k permutation cancels. This kernel uses k = 16*b(e/4) + 4*(l/16) + e%4
//    for fragment element e: then the 4 accumulator rows a lane holds for two 16-row tiles are
//    exactly its 8 fragment values. The fp32 state tiles, V~ and X tiles feed MFMAs straight
//    from registers (converted to bf16), with no LDS round trip.
//  * Operands needed transposed relative to their row-major LDS tile (K^^T for the state update,
//    g^T for the prefix sum, V in accumulator layout) are read with ds_read_b64_tr_b16.
//  * The cumulative decay over the 64 rows is an MFMA: G^T = g^T U with U[s][t] = (s <= t).
// Per chunk: phase A (wave-local: raw rows to LDS, prefix-sum MFMA, exponentials, Q~/K~/K^ written
// back in place), barrier, phase B (the 20 Gram tiles spread over all waves), barrier, phase D
// (per wave: K~S and S^T Q~^T from the register state while the wave inverts the four 16x16
// diagonal blocks of I + A_kk into its own LDS stage; blocked forward substitution; output via
// buffer stores; state update), barrier. Inputs arrive through buffer loads one chunk ahead.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kC = 64;
typedef short i16x8 __attribute__((ext_vector_type(8)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ i16x4 tr_read(const bf16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}
__device__ __forceinline__ i16x4 read8(const bf16_t* p) { return *reinterpret_cast<const i16x4*>(p); }
__device__ __forceinline__ bf16x8 cat(i16x4 a, i16x4 b) {
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}
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
__device__ __forceinline__ void unpack4(i16x4 v, float* f) {
    const uint2 u = __builtin_bit_cast(uint2, v);
    f[0] = __uint_as_float(u.x << 16); f[1] = __uint_as_float(u.x & 0xffff0000u);
    f[2] = __uint_as_float(u.y << 16); f[3] = __uint_as_float(u.y & 0xffff0000u);
}
// Raw buffer access (gfx9 descriptor): an offset at or beyond num_records reads zeros and drops
// stores, so rows past the end of a sequence need neither clamping nor branches.
constexpr int32_t kBufFlags = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufFlags);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, bf16_t*, f32x4 x) {
    uint2 u;
    u.x = pack_bf16x2(x[0], x[1]);
    u.y = pack_bf16x2(x[2], x[3]);
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, u), r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, float*, f32x4 x) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, x), r, (int)off, 0, 0);
}
__device__ __forceinline__ void write8(bf16_t* p, float a, float b, float c, float d) { store4(p, a, b, c, d); }

// Constant operand of the prefix-sum MFMA: U[s][t] = (s <= t) in the permuted k placement, for
// token tile I (t = 16 I + l16) and k step ks (s = 32 ks + 16 (e/4) + 4 lq + e%4).
__device__ __forceinline__ bf16x8 ufrag(int I, int ks, int lq, int l16) {
    i16x8 u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int s = 32 * ks + 16 * (e >> 2) + 4 * lq + (e & 3);
        u[e] = (s <= 16 * I + l16) ? (short)0x3F80 : (short)0;
    }
    return __builtin_bit_cast(bf16x8, u);
}

template <int DK, int NW, int NT>
struct __align__(16) PrefillSmem {
    static constexpr int W = NW * NT * 16;    // state columns of the workgroup
    static constexpr int LDK = DK + 8;        // [64][DK] tiles, 16-byte row padding
    static constexpr int LDV = W + 8;         // [64][W] value tile
    static constexpr int LDC = kC + 8;        // [64][64] tiles
    static constexpr int LDT = 16 + 8;        // inverted diagonal blocks
    static constexpr int LDB = 16 * 16 + 4;   // fp32 diagonal blocks (block stride, floats)
    bf16_t q[kC * LDK];     // raw q, then Q~
    bf16_t k[kC * LDK];     // raw k, then K~
    bf16_t kh[kC * LDK];    // raw log_alpha, then K^
    bf16_t v[kC * LDV];     // raw v (this workgroup's columns)
    bf16_t aqk[kC * LDC];   // A_qk (lower 16x16 blocks)
    bf16_t l[kC * LDC];     // A_kk (off-diagonal 16x16 blocks)
    bf16_t tw[NW][4 * 16 * LDT];  // per wave: its copy of (I + L_II)^{-1}, I = 0..3
    float ld[4 * LDB];      // diagonal blocks of A_kk, fp32
    float gam[DK];
    float beta[kC];
};

// One Gram tile: rows 16*I.. of A (K~ or Q~) against rows 16*J.. of K^, contraction over DK.
template <int DK, int LDK>
__device__ __forceinline__ f32x4 gram_tile(const bf16x8* fa, const bf16_t* kh, int J, int l16, int lq) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks)
        acc = mma32(fa[ks], *reinterpret_cast<const bf16x8*>(&kh[(16 * J + l16) * LDK + 32 * ks + 8 * lq]), acc);
    return acc;
}

template <typename TOut, int DK, int NW, int NT>
__global__ __launch_bounds__(NW * 64) void prefill_bf16_kernel(ChunkLaunch p) {
    typedef PrefillSmem<DK, NW, NT> Sm;
    constexpr int LDK = Sm::LDK, LDV = Sm::LDV, LDC = Sm::LDC, LDT = Sm::LDT, LDB = Sm::LDB;
    constexpr int W = Sm::W;
    constexpr int CPW = DK / NW;      // key channels prepared per wave
    constexpr int NVK = CPW / 8;      // 16-byte vectors per row per key-side tensor
    constexpr int NVV = 2 * NT;       // 16-byte vectors per row of the wave's value columns
    constexpr int NM = DK / 16;       // 16-row tiles of the state
    constexpr int NKS = DK / 32;      // 32-wide k steps over the key dimension
    static_assert(CPW % 16 == 0, "each wave prepares whole 16-channel tiles");
    __shared__ Sm sm;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int l16 = l & 15;
    const int lq = l >> 4;
    const int64_t DV = p.dv;

    int64_t bid = blockIdx.x;
    const int64_t nblk = gridDim.x;
    if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);  // siblings share an XCD
    const int ncb_fin = (int)(DV / W);
    const int ncb_sum = (int)((DV + DK) / W);
    const int64_t n_fin = p.lanes * p.fin_nseg * ncb_fin;
    bool summary;
    int cb, seg;
    int64_t lane;
    if (bid < n_fin) {
        summary = false;
        cb = (int)(bid % ncb_fin);
        const int64_t r = bid / ncb_fin;
        seg = p.fin_seg_lo + (int)(r % p.fin_nseg);
        lane = r / p.fin_nseg;
    } else {
        summary = true;
        const int64_t b2 = bid - n_fin;
        cb = (int)(b2 % ncb_sum);
        const int64_t r = b2 / ncb_sum;
        seg = p.sum_seg_lo + (int)(r % p.sum_nseg);
        lane = r / p.sum_nseg;
    }
    const int64_t T = p.T;
    const int64_t nchunks = (T + kC - 1) / kC;
    const int64_t c_begin = (int64_t)seg * p.chunks_per_seg;
    const int64_t c_end = c_begin + p.chunks_per_seg < nchunks ? c_begin + p.chunks_per_seg : nchunks;

    const int colw = 16 * NT * w;            // this wave's first column inside the workgroup tile
    const int col0 = cb * W + colw;          // ... in the (augmented) column space
    const bool m_cols = summary && col0 >= DV;   // whole wave on M columns (DV is a multiple of 16*NT)
    const int ch0 = w * CPW;

    const bf16_t* qg = (const bf16_t*)p.q + lane * T * DK;
    const bf16_t* kg = (const bf16_t*)p.k + lane * T * DK;
    const bf16_t* gg = (const bf16_t*)p.la + lane * T * DK;
    const bf16_t* vg = (const bf16_t*)p.v + lane * T * DV;
    const bf16_t* bg = (const bf16_t*)p.beta + lane * T;

    // ---- entry state (fp32 accumulators: rows c = 16M + 4lq + r, column 16nt + l16) -------
    f32x4 S[NT][NM];
    {
        const float* entry = nullptr;
        if (!summary) {
            if (seg > 0) entry = p.ws_entry + ((lane * p.nseg + seg) * DK) * DV;
            else if (p.S0) entry = p.S0 + lane * DK * DV;
        }
        if (entry) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const float* e = entry + col0 + 16 * nt + l16;
#pragma unroll
                for (int M = 0; M < NM; ++M)
#pragma unroll
                    for (int r = 0; r < 4; ++r) S[nt][M][r] = e[(int64_t)(16 * M + 4 * lq + r) * DV];
            }
        } else {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int diag = m_cols ? col0 + 16 * nt - (int)DV + l16 : -1;
#pragma unroll
                for (int M = 0; M < NM; ++M)
#pragma unroll
                    for (int r = 0; r < 4; ++r) S[nt][M][r] = (16 * M + 4 * lq + r == diag) ? 1.f : 0.f;
            }
        }
    }

    // ---- one-chunk-ahead prefetch: lane = row l of the chunk ------------------------------
    // Buffer loads: rows past T read zeros (so does the value tile of a summary's M columns:
    // its descriptor has no records), which is exactly the padding of a ragged last chunk.
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qg, (uint32_t)(T * DK * 2));
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg, (uint32_t)(T * DK * 2));
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(gg, (uint32_t)(T * DK * 2));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg, m_cols ? 0u : (uint32_t)(T * DV * 2));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(bg, (uint32_t)(T * 2));
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc(summary ? nullptr : (const TOut*)p.o + lane * T * DV, summary ? 0u : (uint32_t)(T * DV * sizeof(TOut)));
    const int vcol = m_cols ? 0 : col0;
    uint4 pq[NVK], pk[NVK], pg[NVK], pv[NVV];
    uint32_t pb = 0;
#define KDA_LOAD_CHUNK(cidx)                                                                    \
    do {                                                                                        \
        const uint32_t row_ = (uint32_t)((cidx) * kC + l);                                      \
        _Pragma("unroll") for (int i_ = 0; i_ < NVK; ++i_) {                                    \
            const uint32_t off_ = (row_ * DK + ch0 + 8 * i_) * 2;                               \
            pq[i_] = buf_load16(rq, off_);                                                      \
            pk[i_] = buf_load16(rk, off_);                                                      \
            pg[i_] = buf_load16(rg, off_);                                                      \
        }                                                                                       \
        _Pragma("unroll") for (int i_ = 0; i_ < NVV; ++i_)                                      \
            pv[i_] = buf_load16(rv, (uint32_t)(row_ * DV + vcol + 8 * i_) * 2);                  \
        pb = buf_load2(rb, row_ * 2);                                                           \
    } while (0)
    if (c_begin < c_end) KDA_LOAD_CHUNK(c_begin);

    for (int64_t c = c_begin; c < c_end; ++c) {
        // ================= phase A: key-side preparation (wave-local channels) =============
        {
#pragma unroll
            for (int i = 0; i < NVK; ++i) {
                *reinterpret_cast<uint4*>(&sm.q[l * LDK + ch0 + 8 * i]) = pq[i];
                *reinterpret_cast<uint4*>(&sm.k[l * LDK + ch0 + 8 * i]) = pk[i];
                *reinterpret_cast<uint4*>(&sm.kh[l * LDK + ch0 + 8 * i]) = pg[i];
            }
#pragma unroll
            for (int i = 0; i < NVV; ++i) *reinterpret_cast<uint4*>(&sm.v[l * LDV + colw + 8 * i]) = pv[i];
            if (w == 0) sm.beta[l] = __uint_as_float(pb << 16);
            if (c + 1 < c_end) KDA_LOAD_CHUNK(c + 1);
            wave_lds_sync();
#pragma unroll
            for (int t16 = 0; t16 < CPW / 16; ++t16) {
                const int cc = ch0 + 16 * t16;  // 16-channel tile
                // G^T[c][t] = sum_s g[s][c] (s <= t): A = g^T via transposed reads
                bf16x8 ga[2];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const bf16_t* b0 = &sm.kh[(32 * ks + 4 * lq + (l16 >> 2)) * LDK + cc + 4 * (l16 & 3)];
                    ga[ks] = cat(tr_read(b0), tr_read(b0 + 16 * LDK));
                }
                f32x4 G[4];
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    G[I] = f32x4{0.f, 0.f, 0.f, 0.f};
                    G[I] = mma32(ga[0], ufrag(I, 0, lq, l16), G[I]);
                    if (I >= 2) G[I] = mma32(ga[1], ufrag(I, 1, lq, l16), G[I]);
                }
                // lane holds channels cc + 4lq + r for token 16I + l16
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    const int t = 16 * I + l16;
                    float qf[4], kf[4], oq[4], ok_[4], okh[4];
                    unpack4(read8(&sm.q[t * LDK + cc + 4 * lq]), qf);
                    unpack4(read8(&sm.k[t * LDK + cc + 4 * lq]), kf);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float g2 = G[I][r] * kLog2e;
                        const float gam = __builtin_amdgcn_exp2f(g2);
                        const float igam = __builtin_amdgcn_exp2f(-g2);
                        oq[r] = qf[r] * gam;
                        ok_[r] = kf[r] * gam;
                        okh[r] = kf[r] * igam;
                        if (I == 3) G[3][r] = gam;
                    }
                    write8(&sm.q[t * LDK + cc + 4 * lq], oq[0], oq[1], oq[2], oq[3]);
                    write8(&sm.k[t * LDK + cc + 4 * lq], ok_[0], ok_[1], ok_[2], ok_[3]);
                    write8(&sm.kh[t * LDK + cc + 4 * lq], okh[0], okh[1], okh[2], okh[3]);
                }
                if (l16 == 15) *reinterpret_cast<float4*>(&sm.gam[cc + 4 * lq]) = make_float4(G[3][0], G[3][1], G[3][2], G[3][3]);
            }
        }
        __syncthreads();

        // ================= phase B: Gram tiles ==============================================
        // A_kk (diagonal blocks in fp32 for the inverses, off-diagonal blocks in bf16) and A_qk
        // (FINISH only). With 4 waves, wave w takes the row blocks {0,3} (w even) or {1,2}
        // (w odd) of A_kk (w < 2) or A_qk (w >= 2), so each wave loads a row block's operand once.
        {
            auto emit = [&](int kind, int I, int J, f32x4 acc) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int il = 4 * lq + r;
                    const int i = 16 * I + il;
                    const int j = 16 * J + l16;
                    if (kind == 0) {
                        if (I == J) sm.ld[I * LDB + il * 16 + l16] = (l16 < il) ? sm.beta[i] * acc[r] : 0.f;
                        else sm.l[i * LDC + j] = f32_to_bf16_bits(sm.beta[i] * acc[r]);
                    } else {
                        sm.aqk[i * LDC + j] = f32_to_bf16_bits(j <= i ? acc[r] : 0.f);
                    }
                }
            };
            if constexpr (NW == 4) {
                const int kind = w >> 1;
                if (!(summary && kind == 1)) {
                    const bf16_t* A = kind ? sm.q : sm.k;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int I = (w & 1) ? 1 + h : 3 * h;
                        bf16x8 fa[NKS];
#pragma unroll
                        for (int ks = 0; ks < NKS; ++ks)
                            fa[ks] = *reinterpret_cast<const bf16x8*>(&A[(16 * I + l16) * LDK + 32 * ks + 8 * lq]);
                        for (int J = 0; J <= I; ++J) emit(kind, I, J, gram_tile<DK, LDK>(fa, sm.kh, J, l16, lq));
                    }
                }
            } else {
                const int ntiles = summary ? 10 : 20;
                for (int idx = w; idx < ntiles; idx += NW) {
                    int I, J, kind;
                    if (idx < 10) {
                        kind = 0;
                        I = idx < 1 ? 0 : (idx < 3 ? 1 : (idx < 6 ? 2 : 3));
                        J = idx - (I * (I + 1)) / 2;
                    } else {
                        const int t = idx - 10;
                        kind = 1;
                        I = t < 1 ? 0 : (t < 3 ? 1 : (t < 6 ? 2 : 3));
                        J = t - (I * (I + 1)) / 2;
                    }
                    const bf16_t* A = kind ? sm.q : sm.k;
                    bf16x8 fa[NKS];
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
                        fa[ks] = *reinterpret_cast<const bf16x8*>(&A[(16 * I + l16) * LDK + 32 * ks + 8 * lq]);
                    emit(kind, I, J, gram_tile<DK, LDK>(fa, sm.kh, J, l16, lq));
                }
            }
        }
        __syncthreads();

        // ================= phase D: per wave, no further workgroup barrier ===================
        // K~S and S^T Q~^T from the register state (each key-side fragment feeds NT MFMAs), while
        // this wave inverts the four diagonal blocks of I + A_kk into its own stage: lane
        // (I = l/16, j = l%16) solves column j of (I + L_II)^{-1} by forward substitution (fp32).
        bf16x8 sf[NT][NKS];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) sf[nt][ks] = cat(cvt4(S[nt][2 * ks]), cvt4(S[nt][2 * ks + 1]));
        f32x4 Y[NT][4], Ot[NT][4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) Y[nt][I] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int i = 16 * I + l16;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8 a = cat(read8(&sm.k[i * LDK + 32 * ks + 4 * lq]), read8(&sm.k[i * LDK + 32 * ks + 16 + 4 * lq]));
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) Y[nt][I] = mma32(a, sf[nt][ks], Y[nt][I]);
            }
        }
        if (!summary) {
#pragma unroll
            for (int I = 0; I < 4; ++I) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) Ot[nt][I] = f32x4{0.f, 0.f, 0.f, 0.f};
                const int i = 16 * I + l16;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const bf16x8 b = cat(read8(&sm.q[i * LDK + 32 * ks + 4 * lq]), read8(&sm.q[i * LDK + 32 * ks + 16 + 4 * lq]));
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) Ot[nt][I] = mma32(sf[nt][ks], b, Ot[nt][I]);
                }
            }
        }
        bf16_t* tw = &sm.tw[w][0];
        {
            const float* Lb = &sm.ld[lq * LDB];
            float tc[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) tc[i] = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float s = 0.f;
#pragma unroll
                for (int mb = 0; mb < (i + 3) / 4; ++mb) {
                    const float4 L4 = *reinterpret_cast<const float4*>(&Lb[i * 16 + 4 * mb]);
                    s += L4.x * tc[4 * mb] + L4.y * tc[4 * mb + 1] + L4.z * tc[4 * mb + 2] + L4.w * tc[4 * mb + 3];
                }
                tc[i] = (i == l16) ? 1.f : ((i < l16) ? 0.f : -s);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) tw[(lq * 16 + i) * LDT + l16] = f32_to_bf16_bits(tc[i]);
            wave_lds_sync();
        }
        f32x4 Vt[NT][4];   // V~ tiles: rows = tokens 16I + 4lq + r, column 16nt + l16
        {
            f32x4 R[NT][4];
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const float4 b4 = *reinterpret_cast<const float4*>(&sm.beta[16 * I + 4 * lq]);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    float vv[4];
                    unpack4(tr_read(&sm.v[(16 * I + 4 * lq + (l16 >> 2)) * LDV + colw + 16 * nt + 4 * (l16 & 3)]), vv);
                    R[nt][I][0] = b4.x * (vv[0] - Y[nt][I][0]);
                    R[nt][I][1] = b4.y * (vv[1] - Y[nt][I][1]);
                    R[nt][I][2] = b4.z * (vv[2] - Y[nt][I][2]);
                    R[nt][I][3] = b4.w * (vv[3] - Y[nt][I][3]);
                }
            }
            // (I + A_kk) V~ = R, one 16-row block at a time; X and V~ stay in registers
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const int rowL = (16 * I + l16) * LDC;
                i16x4 l0, l2;
                bf16x8 l01;
                if (I == 1) l0 = read8(&sm.l[rowL + 4 * lq]);
                if (I >= 2) l01 = cat(read8(&sm.l[rowL + 4 * lq]), read8(&sm.l[rowL + 16 + 4 * lq]));
                if (I == 3) l2 = read8(&sm.l[rowL + 32 + 4 * lq]);
                const i16x4 tI = read8(&tw[(16 * I + l16) * LDT + 4 * lq]);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    f32x4 X = R[nt][I];
                    if (I == 1) {
                        X = X - mma16(l0, cvt4(Vt[nt][0]), zero);
                    } else if (I >= 2) {
                        X = X - mma32(l01, cat(cvt4(Vt[nt][0]), cvt4(Vt[nt][1])), zero);
                        if (I == 3) X = X - mma16(l2, cvt4(Vt[nt][2]), zero);
                    }
                    Vt[nt][I] = mma16(tI, cvt4(X), zero);
                }
            }
        }
        bf16x8 v01[NT], v23[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            v01[nt] = cat(cvt4(Vt[nt][0]), cvt4(Vt[nt][1]));
            v23[nt] = cat(cvt4(Vt[nt][2]), cvt4(Vt[nt][3]));
        }
        if (!summary) {
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const int i = 16 * I + l16;
                i16x4 q0, q2;
                bf16x8 q01, q23;
                if (I == 0) q0 = read8(&sm.aqk[i * LDC + 4 * lq]);
                else q01 = cat(read8(&sm.aqk[i * LDC + 4 * lq]), read8(&sm.aqk[i * LDC + 16 + 4 * lq]));
                if (I == 2) q2 = read8(&sm.aqk[i * LDC + 32 + 4 * lq]);
                if (I == 3) q23 = cat(read8(&sm.aqk[i * LDC + 32 + 4 * lq]), read8(&sm.aqk[i * LDC + 48 + 4 * lq]));
                const uint32_t row = (uint32_t)(c * kC + i);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    f32x4 o16 = {0.f, 0.f, 0.f, 0.f};
                    if (I == 0) {
                        o16 = mma16(cvt4(Vt[nt][0]), q0, o16);
                    } else {
                        Ot[nt][I] = mma32(v01[nt], q01, Ot[nt][I]);
                        if (I == 2) o16 = mma16(cvt4(Vt[nt][2]), q2, o16);
                        if (I == 3) Ot[nt][I] = mma32(v23[nt], q23, Ot[nt][I]);
                    }
                    buf_store4(ro, (row * (uint32_t)DV + col0 + 16 * nt + 4 * lq) * (uint32_t)sizeof(TOut), (TOut*)nullptr,
                               Ot[nt][I] + o16);
                }
            }
        }
        // S <- Diag(gamma_C) (S + K^^T V~); K^^T comes from transposed reads of the K^ tile
#pragma unroll
        for (int M = 0; M < NM; ++M) {
            const bf16_t* kb = &sm.kh[(4 * lq + (l16 >> 2)) * LDK + 16 * M + 4 * (l16 & 3)];
            const bf16x8 a01 = cat(tr_read(kb), tr_read(kb + 16 * LDK));
            const bf16x8 a23 = cat(tr_read(kb + 32 * LDK), tr_read(kb + 48 * LDK));
            const float4 g4 = *reinterpret_cast<const float4*>(&sm.gam[16 * M + 4 * lq]);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                f32x4 acc = mma32(a01, v01[nt], S[nt][M]);
                acc = mma32(a23, v23[nt], acc);
                S[nt][M][0] = acc[0] * g4.x; S[nt][M][1] = acc[1] * g4.y; S[nt][M][2] = acc[2] * g4.z; S[nt][M][3] = acc[3] * g4.w;
            }
        }
        __syncthreads();
    }
#undef KDA_LOAD_CHUNK

    // ---- exit state --------------------------------------------------------------------------
    float* dst = nullptr;
    int64_t ld_dst = DV;
    if (summary) {
        dst = p.ws_pair + (lane * p.nseg + seg) * DK * (DV + DK);
        ld_dst = DV + DK;
    } else if (seg == p.nseg - 1) {
        dst = p.S_T ? p.S_T + lane * DK * DV : nullptr;
    } else if (seg == 0) {
        dst = p.ws_entry + ((lane * p.nseg + 1) * DK) * DV;
    }
    if (dst) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int M = 0; M < NM; ++M)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dst[(int64_t)(16 * M + 4 * lq + r) * ld_dst + col0 + 16 * nt + l16] = S[nt][M][r];
    }
}

template <typename TOut, int DK, int NW, int NT>
hipError_t launch_t(const ChunkLaunch& a, hipStream_t st) {
    const int W = NW * NT * 16;
    const int64_t blocks = a.lanes * ((int64_t)a.fin_nseg * (a.dv / W) + (int64_t)a.sum_nseg * ((a.dv + DK) / W));
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL((prefill_bf16_kernel<TOut, DK, NW, NT>), dim3((unsigned)blocks), dim3(NW * 64), 0, st, a);
    return hipGetLastError();
}

template <typename TOut>
hipError_t launch_o(const ChunkLaunch& a, hipStream_t st) {
    if (a.dk == 128) {
        if (a.nw == 8) return launch_t<TOut, 128, 8, 1>(a, st);
        if (a.nt == 2) return launch_t<TOut, 128, 4, 2>(a, st);   // 4 waves x 32 columns
        return launch_t<TOut, 128, 4, 1>(a, st);
    }
    return launch_t<TOut, 64, 4, 1>(a, st);
}

}  // namespace

hipError_t launch_prefill_bf16(const ChunkLaunch& a, hipStream_t st) {
    return a.out_bf16 ? launch_o<bf16_t>(a, st) : launch_o<float>(a, st);
}

}  // namespace kda

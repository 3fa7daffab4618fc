// KDA intra-chunk kernel for gfx950, bf16 inputs: everything of a 64-token chunk that does not
// depend on the recurrent state (Kimi K3 reading notes, liuzhao09.github.io/papers/kimi-k3.html,
// section 2.2: cumulative decay Gamma, the decay-weighted Gram tiles and the UT transform).
//
// Every chunk of every lane is independent. A persistent grid of two workgroups (4 waves each) per
// compute unit walks the (lane, chunk) pairs, loading the next chunk's raw rows into registers
// while it works on the current one, so the kernel is bound by HBM traffic, not by latency. Input
// loads are row-contiguous (64 bytes per row per wave). Output: the chunk's record
// (kda_record.h) in the workspace. Steps, with G = cumsum(log alpha) over the chunk's rows:
//   1. per wave, 32 key channels: G^T = g^T U (U[s][t] = (s <= t)) on the MFMA, Gamma = exp(G);
//      Q~ = Q Gamma, K~ = K Gamma, K^ = K / Gamma, K- = K gamma_C / Gamma, all from fp32 factors
//      rounded once to bf16. Q~ and K- go straight to the record; Q~, K~, K^ go to LDS as
//      fragment blocks.
//   2. Gram tiles from the LDS blocks: the diagonal blocks of A_kk = Diag(beta) StrictTril(K~K^^T)
//      in fp32 (wave 0, which then inverts I + A_kk's four 16x16 diagonal blocks by substitution),
//      its off-diagonal blocks in bf16 (wave 1) and A_qk = Tril(Q~K^^T) into the record (waves 2-3).
//   3. blocked forward substitution (I + A_kk) [W | U] = Diag(beta) [K~ | V] on the MFMA, 16
//      columns per tile, right-hand sides and results in registers; U goes to the record, -W is
//      transposed through LDS into fragment order.
#include "kda_internal.h"
#include "kda_mfma.h"
#include "kda_record.h"

namespace kda {
namespace {

constexpr int kC = 64;

// Constant operand of the prefix-sum MFMA: U[s][t] = (s <= t) in the K32 placement, for token
// tile I (t = 16 I + l16) and k window ks (s = 32 ks + 16 (e/4) + 4 lq + e%4).
__device__ __forceinline__ bf16x8 ufrag(int I, int ks, int lq, int l16) {
    i16x8 u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int s = 32 * ks + 16 * (e >> 2) + 4 * lq + (e & 3);
        u[e] = (s <= 16 * I + l16) ? (short)0x3F80 : (short)0;
    }
    return __builtin_bit_cast(bf16x8, u);
}

// Operands of the blocked substitution for one chunk: A_kk's off-diagonal blocks as A fragments,
// the inverted diagonal blocks T_I = (I + A_kk,II)^{-1} and beta of the lane's accumulator rows.
struct SolveOps {
    i16x4 a10, a32, t0, t1, t2, t3;
    bf16x8 a2, a3;      // (2,0|2,1) and (3,0|3,1) as K32 fragments
    f32x4 b0, b1, b2, b3;
};

// (I + A_kk) X = Diag(beta) R for one 16-column tile; R and X in accumulator layout (rows
// 16I + 4lq + r). X_I = T_I (beta R_I - sum_{J<I} A_IJ X_J). Products of different MFMA shapes
// go to separate accumulators and are combined on the VALU.
__device__ __forceinline__ void ut_solve(const SolveOps& o, i16x4 r0, i16x4 r1, i16x4 r2, i16x4 r3,
                                         f32x4& X0, f32x4& X1, f32x4& X2, f32x4& X3) {
    X0 = mma16(o.t0, cvt4(o.b0 * unpack4f(r0)), kZero4);
    const i16x4 x0 = cvt4(X0);
    const f32x4 y1 = o.b1 * unpack4f(r1) - mma16(o.a10, x0, kZero4);
    X1 = mma16(o.t1, cvt4(y1), kZero4);
    const bf16x8 x01 = cat(x0, cvt4(X1));
    const f32x4 y2 = o.b2 * unpack4f(r2) - mma32(o.a2, x01, kZero4);
    X2 = mma16(o.t2, cvt4(y2), kZero4);
    const f32x4 y3 = o.b3 * unpack4f(r3) - mma32(o.a3, x01, kZero4) - mma16(o.a32, cvt4(X2), kZero4);
    X3 = mma16(o.t3, cvt4(y3), kZero4);
}

template <int DK, int DV>
struct IntraCfg {
    static constexpr int NKS = DK / 32;                    // waves 0..NKS-1 own 32 key channels each
    static constexpr int VPW = (DV == 128 || DK == 64) ? 2 : 1;   // value tiles per wave
    // First value tile of wave w, and whether wave w has value tiles at all.
    __device__ static constexpr int vt0(int w) { return (DK == 64 && DV == 64) ? 2 * (w - 2) : VPW * w; }
    __device__ static constexpr bool has_v(int w) { return !(DK == 64 && DV == 64) || w >= 2; }
    static constexpr int LDG = 40;             // g stage / K- stage row: 32 channels + pad
    static constexpr int LDVS = 16 * VPW + 8;  // v stage row
    static constexpr int LDW = 72;             // W^T stage row: 64 tokens + pad
    static constexpr int STAGE_A = kC * LDG * 2;     // g, then K- (token-major)
    static constexpr int STAGE_B = 12 * 1024;        // v, then this wave's Q~/K~/K^ blocks
    static constexpr int REGION = STAGE_A + STAGE_B; // after the Gram: W^T stage
    static_assert(kC * LDVS * 2 <= STAGE_B, "v stage fits");
    static_assert(32 * LDW * 2 <= REGION, "W^T stage fits");
};

template <int DK, int DV>
struct __align__(16) IntraSmem {
    typedef IntraCfg<DK, DV> Cfg;
    unsigned char region[4][Cfg::REGION];
    float ld[4][16 * 16];       // beta-scaled strictly lower diagonal blocks of A_kk, column-major
    bf16_t akk[6][256];         // off-diagonal blocks (I, J), I > J, as K16 A fragments
    bf16_t tinv[4][16 * 24];    // (I + A_kk,II)^{-1}, row-major, 24-element rows
    float beta[kC];
};

template <int DK, int DV>
__global__ __launch_bounds__(256, 2) void intra_kernel(IntraArgs p) {
    typedef IntraCfg<DK, DV> Cfg;
    typedef RecordLayout<DK, DV> R;
    constexpr int NKS = Cfg::NKS, VPW = Cfg::VPW, LDG = Cfg::LDG, LDVS = Cfg::LDVS, LDW = Cfg::LDW;
    __shared__ IntraSmem<DK, DV> sm;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int l16 = l & 15;
    const int lq = l >> 4;

    const int64_t T = p.T;
    const int64_t total = p.lanes * p.nchunks;
    unsigned char* reg = sm.region[w];
    bf16_t* stA = reinterpret_cast<bf16_t*>(reg);                    // g, then K- (token-major)
    unsigned char* stB = reg + Cfg::STAGE_A;                         // v, then blocks
    auto lblk = [&](int ks, int X, int I) -> unsigned char* {        // LDS block of tensor X (0 Q~, 1 K~, 2 K^)
        return sm.region[ks] + Cfg::STAGE_A + (X * 4 + I) * 1024;
    };

    const bool kw = w < NKS;          // this wave prepares key channels 32w .. 32w + 31
    const bool vw = Cfg::has_v(w);    // this wave solves value tiles vt0 .. vt0 + VPW - 1
    const int vc0 = 16 * Cfg::vt0(w);
    constexpr int LPR = 2 * VPW;      // lanes per row of the value stage load
    // Lane's 16-byte slice of a q/k row: rows (lq = 0, 1) and (2, 3) then trade halves with one
    // permlane16 swap per dword pair, which leaves each lane its fragment channels
    // 32w + 16h + 4lq .. +3 for h = 0, 1.
    const int qk_off = 8 * (((lq & 1) << 1) | (lq >> 1));

    // Raw inputs of one chunk, loaded one chunk ahead. Rows at or past T read as zeros.
    uint4 pq[4], pk[4], pg[4], pv[LPR];
    uint32_t pb = 0;
#define KDA_INTRA_LOAD(tt)                                                                          \
    do {                                                                                            \
        const int64_t c_ = uniform64((tt) % p.nchunks);                                             \
        const int64_t lane_ = uniform64((tt) / p.nchunks);                                          \
        const uint32_t r0_ = (uint32_t)(c_ * kC);                                                   \
        if (kw) {                                                                                   \
            const __amdgpu_buffer_rsrc_t rq_ = make_rsrc((const bf16_t*)p.q + lane_ * T * DK, (uint32_t)(T * DK * 2)); \
            const __amdgpu_buffer_rsrc_t rk_ = make_rsrc((const bf16_t*)p.k + lane_ * T * DK, (uint32_t)(T * DK * 2)); \
            const __amdgpu_buffer_rsrc_t rg_ = make_rsrc((const bf16_t*)p.la + lane_ * T * DK, (uint32_t)(T * DK * 2)); \
            _Pragma("unroll") for (int I_ = 0; I_ < 4; ++I_) {                                      \
                const uint32_t o_ = ((r0_ + 16 * I_ + l16) * DK + 32 * w + qk_off) * 2;               \
                pq[I_] = buf_load16(rq_, o_);                                                       \
                pk[I_] = buf_load16(rk_, o_);                                                       \
                pg[I_] = buf_load16(rg_, ((r0_ + 16 * I_ + (l >> 2)) * DK + 32 * w + 8 * (l & 3)) * 2); \
            }                                                                                       \
        }                                                                                           \
        if (vw) {                                                                                   \
            const __amdgpu_buffer_rsrc_t rv_ = make_rsrc((const bf16_t*)p.v + lane_ * T * DV, (uint32_t)(T * DV * 2)); \
            _Pragma("unroll") for (int i_ = 0; i_ < LPR; ++i_)                                      \
                pv[i_] = buf_load16(rv_, ((r0_ + i_ * (64 / LPR) + l / LPR) * DV + vc0 + 8 * (l % LPR)) * 2); \
        }                                                                                           \
        if (w == 0) {                                                                               \
            const __amdgpu_buffer_rsrc_t rb_ = make_rsrc((const bf16_t*)p.beta + lane_ * T, (uint32_t)(T * 2)); \
            pb = buf_load2(rb_, (r0_ + l) * 2);                                                     \
        }                                                                                           \
    } while (0)

    // Persistent: workgroup b takes chunks b, b + gridDim.x, ... of the flattened (lane, chunk)
    // index, so the loads of the next chunk overlap the Gram tiles and solve of this one.
    int64_t t = blockIdx.x;
    if (t < total) KDA_INTRA_LOAD(t);
    for (; t < total; t += gridDim.x) {
    const int64_t c = uniform64(t % p.nchunks);
    const int64_t lane = uniform64(t / p.nchunks);
    unsigned char* rec = p.rec + (lane * p.nchunks + c) * (int64_t)R::BYTES;
    auto blk = [&](int b) -> unsigned char* { return rec + b * 1024 + l * 16; };

    // ================= phase 1: decay and scaled operands (wave-local) =========================
    i16x4 vacc[VPW][4];     // V rows 16I + 4lq + e, column vc0 + 16j + l16 (accumulator layout)
    i16x4 kacc[2][4];       // K~ rows 16I + 4lq + e, channel 32w + 16h + l16
    {
        uint2 qv[2][4], kv[2][4];
        bf16_t* vst = reinterpret_cast<bf16_t*>(stB);
        if (kw) {
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                *reinterpret_cast<uint4*>(&stA[(16 * I + (l >> 2)) * LDG + 8 * (l & 3)]) = pg[I];
                typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
                const u32x2 sq0 = __builtin_amdgcn_permlane16_swap(pq[I].x, pq[I].z, false, false);
                const u32x2 sq1 = __builtin_amdgcn_permlane16_swap(pq[I].y, pq[I].w, false, false);
                const u32x2 sk0 = __builtin_amdgcn_permlane16_swap(pk[I].x, pk[I].z, false, false);
                const u32x2 sk1 = __builtin_amdgcn_permlane16_swap(pk[I].y, pk[I].w, false, false);
                qv[0][I] = make_uint2(sq0[0], sq1[0]); qv[1][I] = make_uint2(sq0[1], sq1[1]);
                kv[0][I] = make_uint2(sk0[0], sk1[0]); kv[1][I] = make_uint2(sk0[1], sk1[1]);
            }
        }
        if (vw) {
#pragma unroll
            for (int i = 0; i < LPR; ++i) *reinterpret_cast<uint4*>(&vst[(i * (64 / LPR) + l / LPR) * LDVS + 8 * (l % LPR)]) = pv[i];
        }
        if (w == 0) sm.beta[l] = __uint_as_float(pb << 16);
        if (t + gridDim.x < total) KDA_INTRA_LOAD(t + gridDim.x);
        wave_lds_sync();
        if (vw) {
#pragma unroll
            for (int j = 0; j < VPW; ++j)
#pragma unroll
                for (int I = 0; I < 4; ++I)
                    vacc[j][I] = tr_read(&vst[(16 * I + 4 * lq + (l16 >> 2)) * LDVS + 16 * j + 4 * (l16 & 3)]);
        }
        if (kw) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                bf16x8 ga[2];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const bf16_t* b0 = &stA[(32 * s + 4 * lq + (l16 >> 2)) * LDG + 16 * h + 4 * (l16 & 3)];
                    ga[s] = cat(tr_read(b0), tr_read(b0 + 16 * LDG));
                }
                // D[r] = G for channel 32w + 16h + 4lq + r at token 16I + l16
                f32x4 G[4];
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    G[I] = mma32(ga[0], ufrag(I, 0, lq, l16), kZero4);
                    if (I >= 2) G[I] = mma32(ga[1], ufrag(I, 1, lq, l16), G[I]);
                }
                f32x4 gC;   // gamma_C of the lane's four channels (lane 15 of the row holds token 63)
#pragma unroll
                for (int r = 0; r < 4; ++r) gC[r] = row_bcast15(__builtin_amdgcn_exp2f(G[3][r] * kLog2e));
                if (l16 == 15)
                    *reinterpret_cast<f32x4*>(rec + R::G * 1024 + (32 * w + 16 * h + 4 * lq) * 4) = gC;
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    const f32x4 qf = unpack4f(__builtin_bit_cast(i16x4, qv[h][I]));
                    const f32x4 kf = unpack4f(__builtin_bit_cast(i16x4, kv[h][I]));
                    f32x4 oq, ok, oh, ob;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float g2 = G[I][r] * kLog2e;
                        const float gam = __builtin_amdgcn_exp2f(g2);
                        const float igam = __builtin_amdgcn_exp2f(-g2);
                        oq[r] = qf[r] * gam;
                        ok[r] = kf[r] * gam;
                        oh[r] = kf[r] * igam;
                        ob[r] = oh[r] * gC[r];
                    }
                    // fragment blocks (I, ks = w): register elements e < 4 come from h = 0, e >= 4
                    // from h = 1, i.e. bytes 8h .. 8h + 7 of the lane's 16
                    const i16x4 bq = cvt4(oq);
                    *reinterpret_cast<i16x4*>(lblk(w, 0, I) + l * 16 + 8 * h) = bq;
                    *reinterpret_cast<i16x4*>(lblk(w, 1, I) + l * 16 + 8 * h) = cvt4(ok);
                    *reinterpret_cast<i16x4*>(lblk(w, 2, I) + l * 16 + 8 * h) = cvt4(oh);
                    *reinterpret_cast<i16x4*>(blk(R::q(I, w)) + 8 * h) = bq;
                    // K- token-major into the g stage columns 16h.. (already consumed above)
                    *reinterpret_cast<uint2*>(&stA[(16 * I + l16) * LDG + 16 * h + 4 * lq]) =
                        __builtin_bit_cast(uint2, cvt4(ob));
                }
            }
            wave_lds_sync();
            // K- blocks (M = 2w + h, half): K-[32 half + k(e)][16M + l16]
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const bf16_t* b0 = &stA[(32 * half + 4 * lq + (l16 >> 2)) * LDG + 16 * h + 4 * (l16 & 3)];
                    *reinterpret_cast<bf16x8*>(blk(R::k(2 * w + h, half))) = cat(tr_read(b0), tr_read(b0 + 16 * LDG));
                }
            // K~ in accumulator layout from its own blocks: the 8-byte chunk addressed by lane
            // (lq, l16) is K~[16I + 4lq + l16/4][32w + 16h + 4(l16%4) ..], i.e. block lane
            // (l16 % 4, 4lq + l16/4), half h.
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int I = 0; I < 4; ++I)
                    kacc[h][I] = tr_read(reinterpret_cast<const bf16_t*>(
                        lblk(w, 1, I) + ((l16 & 3) * 16 + 4 * lq + (l16 >> 2)) * 16 + 8 * h));
        }
    }
    __syncthreads();

    // ================= phase 2: Gram tiles ====================================================
    if (w == 0) {
        // diagonal blocks, rows i = 16I + 4lq + r, column m = 16I + l16; wave 0 then inverts them
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            f32x4 acc = kZero4;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                acc = mma32(read16(lblk(ks, 1, I) + l * 16), read16(lblk(ks, 2, I) + l * 16), acc);
            const float4 b4 = *reinterpret_cast<const float4*>(&sm.beta[16 * I + 4 * lq]);
            f32x4 o;
            o[0] = (l16 < 4 * lq + 0) ? b4.x * acc[0] : 0.f;
            o[1] = (l16 < 4 * lq + 1) ? b4.y * acc[1] : 0.f;
            o[2] = (l16 < 4 * lq + 2) ? b4.z * acc[2] : 0.f;
            o[3] = (l16 < 4 * lq + 3) ? b4.w * acc[3] : 0.f;
            *reinterpret_cast<f32x4*>(&sm.ld[I][l16 * 16 + 4 * lq]) = o;   // column m = l16
        }
        wave_lds_sync();
        // Lane (block lq, row i = l16): row i of T = (I + L)^{-1} from T (I + L) = I, i.e.
        // t[m] = -sum_{n > m} t[n] L[n][m] for m < i, t[i] = 1, t[m > i] = 0.
        const float* Lc = sm.ld[lq];
        const int i = l16;
        float t[16];
#pragma unroll
        for (int n = 0; n < 16; ++n) t[n] = (n == i) ? 1.f : 0.f;
#pragma unroll
        for (int m = 14; m >= 0; --m) {
            float s = 0.f;
#pragma unroll
            for (int nb = (m + 1) / 4; nb < 4; ++nb) {
                const float4 L4 = *reinterpret_cast<const float4*>(&Lc[m * 16 + 4 * nb]);
                s += L4.x * t[4 * nb] + L4.y * t[4 * nb + 1] + L4.z * t[4 * nb + 2] + L4.w * t[4 * nb + 3];
            }
            if (m < i) t[m] = -s;
        }
        uint4 r0, r1;
        r0.x = pack_bf16x2(t[0], t[1]);   r0.y = pack_bf16x2(t[2], t[3]);
        r0.z = pack_bf16x2(t[4], t[5]);   r0.w = pack_bf16x2(t[6], t[7]);
        r1.x = pack_bf16x2(t[8], t[9]);   r1.y = pack_bf16x2(t[10], t[11]);
        r1.z = pack_bf16x2(t[12], t[13]); r1.w = pack_bf16x2(t[14], t[15]);
        *reinterpret_cast<uint4*>(&sm.tinv[lq][i * 24]) = r0;
        *reinterpret_cast<uint4*>(&sm.tinv[lq][i * 24 + 8]) = r1;
    } else if (w == 1) {
        // off-diagonal blocks transposed: lane holds A_kk[16I + l16][16J + 4lq + r]
#pragma unroll
        for (int I = 1; I < 4; ++I)
#pragma unroll
            for (int J = 0; J < I; ++J) {
                f32x4 acc = kZero4;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    acc = mma32(read16(lblk(ks, 2, J) + l * 16), read16(lblk(ks, 1, I) + l * 16), acc);
                const float b = sm.beta[16 * I + l16];
                *reinterpret_cast<i16x4*>(&sm.akk[I * (I - 1) / 2 + J][l * 4]) = cvt4(acc * b);
            }
    } else {
        // A_qk transposed, lane holds A_qk[16I + l16][16J + 4lq + r] (j <= i kept); wave 2 writes
        // the record blocks (0,0), (1,0), (2,0), wave 3 (2,1), (3,0), (3,1)
        auto qk = [&](int I, int J) -> i16x4 {
            f32x4 acc = kZero4;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                acc = mma32(read16(lblk(ks, 2, J) + l * 16), read16(lblk(ks, 0, I) + l * 16), acc);
            if (J == I) {
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = (4 * lq + r <= l16) ? acc[r] : 0.f;
            }
            return cvt4(acc);
        };
        const i16x4 z = {0, 0, 0, 0};
        if (w == 2) {
            *reinterpret_cast<bf16x8*>(blk(R::a(0, 0))) = cat(qk(0, 0), z);
            *reinterpret_cast<bf16x8*>(blk(R::a(1, 0))) = cat(qk(1, 0), qk(1, 1));
            *reinterpret_cast<bf16x8*>(blk(R::a(2, 0))) = cat(qk(2, 0), qk(2, 1));
        } else {
            *reinterpret_cast<bf16x8*>(blk(R::a(2, 1))) = cat(qk(2, 2), z);
            *reinterpret_cast<bf16x8*>(blk(R::a(3, 0))) = cat(qk(3, 0), qk(3, 1));
            *reinterpret_cast<bf16x8*>(blk(R::a(3, 1))) = cat(qk(3, 2), qk(3, 3));
        }
    }
    __syncthreads();

    // ================= phase 3: (I + A_kk) [W | U] = Diag(beta) [K~ | V] =========================
    {
        SolveOps ops;
        ops.a10 = read8(&sm.akk[0][l * 4]);
        ops.a2 = cat(read8(&sm.akk[1][l * 4]), read8(&sm.akk[2][l * 4]));
        ops.a3 = cat(read8(&sm.akk[3][l * 4]), read8(&sm.akk[4][l * 4]));
        ops.a32 = read8(&sm.akk[5][l * 4]);
        ops.t0 = read8(&sm.tinv[0][l16 * 24 + 4 * lq]);
        ops.t1 = read8(&sm.tinv[1][l16 * 24 + 4 * lq]);
        ops.t2 = read8(&sm.tinv[2][l16 * 24 + 4 * lq]);
        ops.t3 = read8(&sm.tinv[3][l16 * 24 + 4 * lq]);
        ops.b0 = *reinterpret_cast<const f32x4*>(&sm.beta[0 + 4 * lq]);
        ops.b1 = *reinterpret_cast<const f32x4*>(&sm.beta[16 + 4 * lq]);
        ops.b2 = *reinterpret_cast<const f32x4*>(&sm.beta[32 + 4 * lq]);
        ops.b3 = *reinterpret_cast<const f32x4*>(&sm.beta[48 + 4 * lq]);
        if (vw) {
#pragma unroll
            for (int j = 0; j < VPW; ++j) {
                f32x4 X[4];
                ut_solve(ops, vacc[j][0], vacc[j][1], vacc[j][2], vacc[j][3], X[0], X[1], X[2], X[3]);
                const int n = vc0 / 16 + j;
                *reinterpret_cast<bf16x8*>(blk(R::u(n, 0))) = cat(cvt4(X[0]), cvt4(X[1]));
                *reinterpret_cast<bf16x8*>(blk(R::u(n, 1))) = cat(cvt4(X[2]), cvt4(X[3]));
            }
        }
        if (kw) {
            bf16_t* wt = reinterpret_cast<bf16_t*>(reg);   // W^T [32 channels][64 tokens]
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f32x4 X[4];
                ut_solve(ops, kacc[h][0], kacc[h][1], kacc[h][2], kacc[h][3], X[0], X[1], X[2], X[3]);
#pragma unroll
                for (int I = 0; I < 4; ++I)   // the record holds -W
                    *reinterpret_cast<i16x4*>(&wt[(16 * h + l16) * LDW + 16 * I + 4 * lq]) = cvt4(-X[I]);
            }
            wave_lds_sync();
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const bf16_t* b0 = &wt[(4 * lq + (l16 >> 2)) * LDW + 16 * I + 4 * (l16 & 3)];
                *reinterpret_cast<bf16x8*>(blk(R::w(I, w))) = cat(tr_read(b0), tr_read(b0 + 16 * LDW));
            }
        }
    }
    __syncthreads();   // the next chunk rewrites the stages, beta and the A_kk blocks
    }
#undef KDA_INTRA_LOAD
}

// Resident workgroups for the persistent grid: two per compute unit (the LDS budget).
int resident_workgroups() {
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 512;
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        cached[dev] = 2 * cus;
    }
    return cached[dev];
}

template <int DK, int DV>
hipError_t launch_dd(const IntraArgs& a, hipStream_t st) {
    int64_t blocks = a.lanes * a.nchunks;
    if (blocks <= 0) return hipSuccess;
    if (blocks > resident_workgroups()) blocks = resident_workgroups();
    hipLaunchKernelGGL((intra_kernel<DK, DV>), dim3((unsigned)blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_intra(const IntraArgs& a, hipStream_t st) {
    if (a.dk == 128) return a.dv == 128 ? launch_dd<128, 128>(a, st) : launch_dd<128, 64>(a, st);
    return a.dv == 128 ? launch_dd<64, 128>(a, st) : launch_dd<64, 64>(a, st);
}

}  // namespace kda

// One wave's share of the intra-chunk work on one 64-token chunk (Kimi K3 reading notes,
// liuzhao09.github.io/papers/kimi-k3.html, section 2.2: cumulative decay Gamma, the decay-weighted
// Gram tiles and the UT transform), shared by the intra-chunk kernel (kda_intra.hip), which writes
// each chunk's record to the workspace, and the fused kernel (kda_fused.hip), which builds it in
// LDS for its state step. Four waves work on a chunk; the steps are those listed in kda_intra.hip.
// The caller places a workgroup barrier between decay() and gram() and between gram() and solve(),
// and after solve() before the next chunk's decay(). Internal to the library.
#pragma once

#include "kda_internal.h"
#include "kda_mfma.h"
#include "kda_record.h"

namespace kda {
namespace intra {

constexpr int kC = 64;

// Constant operand of the prefix-sum MFMA: U[s][t] = (s <= t) in the K32 placement, for token
// tile I (t = 16 I + l16) and k window ks (s = 32 ks + 16 (e/4) + 4 lq + e%4). Its six fragments
// hold a single lane-dependent 4-element pattern, P[e] = (4 lq + e <= l16); every other half is
// all ones or all zeros: (I, ks) = (0, 0) and (2, 1) are [P | 0], (1, 0) and (3, 1) are [1 | P],
// (2, 0) and (3, 0) are [1 | 1].
struct UFrags {
    bf16x8 p0, onep, ones;   // [P | 0], [1 | P], [1 | 1]
    __device__ __forceinline__ bf16x8 get(int I, int ks) const {
        return ks == 0 ? (I == 0 ? p0 : (I == 1 ? onep : ones)) : (I == 2 ? p0 : onep);
    }
};
__device__ __forceinline__ UFrags ufrags(int lq, int l16) {
    i16x4 pv, one, zero;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        pv[e] = (4 * lq + e <= l16) ? (short)0x3F80 : (short)0;
        one[e] = (short)0x3F80;
        zero[e] = 0;
    }
    return UFrags{cat(pv, zero), cat(one, pv), cat(one, one)};
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
__device__ __forceinline__ void ut_solve(const SolveOps& o, f32x4 r0, f32x4 r1, f32x4 r2, f32x4 r3,
                                         f32x4& X0, f32x4& X1, f32x4& X2, f32x4& X3) {
    X0 = mma16(o.t0, cvt4(o.b0 * r0), kZero4);
    const i16x4 x0 = cvt4(X0);
    const f32x4 y1 = o.b1 * r1 - mma16(o.a10, x0, kZero4);
    X1 = mma16(o.t1, cvt4(y1), kZero4);
    const bf16x8 x01 = cat(x0, cvt4(X1));
    const f32x4 y2 = o.b2 * r2 - mma32(o.a2, x01, kZero4);
    X2 = mma16(o.t2, cvt4(y2), kZero4);
    const f32x4 y3 = o.b3 * r3 - mma32(o.a3, x01, kZero4) - mma16(o.a32, cvt4(X2), kZero4);
    X3 = mma16(o.t3, cvt4(y3), kZero4);
}

// Make a loaded value "used" at this point: the wait for its load is placed here, not at its
// real use. vmcnt counts loads and stores in issue order, so waiting for a prefetch at the top of
// the next chunk would also wait for every record store issued after it.
__device__ __forceinline__ void pin(uint4& v) { asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w)); }
__device__ __forceinline__ void pin(uint32_t& v) { asm volatile("" : "+v"(v)); }

// Pair index of an off-diagonal block (I > J): (1,0) (2,0) (2,1) (3,0) (3,1) (3,2).
__host__ __device__ constexpr int pair_index(int I, int J) { return I * (I - 1) / 2 + J; }

// A K32 operand fragment of K^ (block J) scaled channel-wise by f_IJ (channels of the fragment:
// 32ks + 16(e/4) + 4lq + e%4), re-rounded to bf16: the reference point moves from block J's start
// to block I's start, and every factor stays <= 1.
__device__ __forceinline__ bf16x8 scale_frag(bf16x8 a, const bf16_t* f, int ks, int lq) {
    const f32x4 f0 = unpack4f(read8(f + 32 * ks + 4 * lq));
    const f32x4 f1 = unpack4f(read8(f + 32 * ks + 16 + 4 * lq));
    return cat(cvt4(unpack4f(lo4(a)) * f0), cvt4(unpack4f(hi4(a)) * f1));
}

// Fused decay prologue on 8 packed bf16 pre-activations z: g = g_min * sigmoid(eA * z) with
// eA = exp(A_h), in fp32, rounded back to bf16 (the form a bf16 log_alpha input has).
__device__ __forceinline__ uint4 decay_from_z(uint4 zr, float eA, float g_min) {
    const uint32_t w[4] = {zr.x, zr.y, zr.z, zr.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float z0 = __uint_as_float(w[i] << 16), z1 = __uint_as_float(w[i] & 0xffff0000u);
        const float s0 = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-eA * z0 * kLog2e));
        const float s1 = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-eA * z1 * kLog2e));
        o[i] = pack_bf16x2(g_min * s0, g_min * s1);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
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
    static_assert(LDG * 2 >= 64 + 16 && kC >= 24, "the decay's P table fits the g stage padding");
};

template <int DK, int DV>
struct __align__(16) IntraSmem {
    typedef IntraCfg<DK, DV> Cfg;
    unsigned char region[4][Cfg::REGION];
    float ld[4][16 * 16];       // beta-scaled strictly lower diagonal blocks of A_kk, row-major
    bf16_t akk[6][256];         // off-diagonal blocks (I, J), I > J, as K16 A fragments
    bf16_t tinv[4][16 * 24];    // (I + A_kk,II)^{-1}, row-major, 24-element rows
    float beta[kC];
    bf16_t fij[6][DK];          // exp(G_ref(I) - G_ref(J)) per channel for the pairs I > J
};

// LDS fragment block of tensor X (0 Q~, 1 K~, 2 K^), token block I, of the wave owning key
// channels 32ks .. 32ks + 31 (block-relative factors; see ChunkWave::decay).
template <int DK, int DV>
__device__ __forceinline__ unsigned char* lds_block(IntraSmem<DK, DV>& sm, int ks, int X, int I) {
    return sm.region[ks] + IntraCfg<DK, DV>::STAGE_A + (X * 4 + I) * 1024;
}

// Diagonal block I of A_kk = Diag(beta) StrictTril(K~ K^^T), rows i = 16I + 4lq + r and column
// m = 16I + l16, in fp32 into sm.ld[I] (row-major).
template <int DK, int DV>
__device__ __forceinline__ void diag_akk_block(IntraSmem<DK, DV>& sm, int I, int l) {
    const int l16 = l & 15, lq = l >> 4;
    f32x4 acc = kZero4;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks)
        acc = mma32(read16(lds_block(sm, ks, 1, I) + l * 16), read16(lds_block(sm, ks, 2, I) + l * 16), acc);
    const float4 b4 = *reinterpret_cast<const float4*>(&sm.beta[16 * I + 4 * lq]);
    const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.ld[I][(4 * lq + r) * 16 + l16] = (l16 < 4 * lq + r) ? bb[r] * acc[r] : 0.f;
}

// Row i of T = (I + L)^{-1} for the strictly lower block L = sm.ld[b], from T (I + L) = I:
// t[m] = -sum_{n > m} t[n] L[n][m] for m < i, t[i] = 1, t[m > i] = 0; stored to sm.tinv[b] as bf16
// when `store`. Right-looking: once t[n] is final, every partial sum of a column m < n takes its
// term at once, so the dependent chain is one multiply-add per row (16) rather than one per term.
template <int DK, int DV>
__device__ __forceinline__ void invert_row(IntraSmem<DK, DV>& sm, int b, int i, bool store) {
    const float* L = sm.ld[b];
    float t[16], s[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) s[m] = 0.f;
#pragma unroll
    for (int n = 15; n >= 0; --n) {
        t[n] = n == i ? 1.f : (n < i ? -s[n] : 0.f);
        // row n's address depends (in form only) on t[n + 4]: its loads go out at most four rows
        // ahead, instead of all 36 at the top, which would hold about 140 registers
        int off = n * 16;
        if (n + 4 <= 15) asm volatile("" : "+v"(off) : "v"(t[n + 4]));
#pragma unroll
        for (int mb = 0; 4 * mb < n; ++mb) {
            const float4 L4 = *reinterpret_cast<const float4*>(&L[off + 4 * mb]);   // L[n][4mb ..]
            if (4 * mb + 0 < n) s[4 * mb + 0] += L4.x * t[n];
            if (4 * mb + 1 < n) s[4 * mb + 1] += L4.y * t[n];
            if (4 * mb + 2 < n) s[4 * mb + 2] += L4.z * t[n];
            if (4 * mb + 3 < n) s[4 * mb + 3] += L4.w * t[n];
        }
    }
    uint4 r0, r1;
    r0.x = pack_bf16x2(t[0], t[1]);   r0.y = pack_bf16x2(t[2], t[3]);
    r0.z = pack_bf16x2(t[4], t[5]);   r0.w = pack_bf16x2(t[6], t[7]);
    r1.x = pack_bf16x2(t[8], t[9]);   r1.y = pack_bf16x2(t[10], t[11]);
    r1.z = pack_bf16x2(t[12], t[13]); r1.w = pack_bf16x2(t[14], t[15]);
    if (store) {
        *reinterpret_cast<uint4*>(&sm.tinv[b][i * 24]) = r0;
        *reinterpret_cast<uint4*>(&sm.tinv[b][i * 24 + 8]) = r1;
    }
}

// Off-diagonal block pair (I > J): K^_J rescaled once by f_IJ and used for both the A_kk block
// (bf16, beta-scaled, to sm.akk) and the A_qk block (to the record). Transposed: the lane holds
// X[16I + l16][16J + 4lq + r], so the A_kk blocks are K16 A operands as computed and the A_qk
// blocks are record halves (record block A(I, h) holds J = 2h in bytes 0..7 and J = 2h + 1 in
// bytes 8..15 of each lane's 16).
template <int DK, int DV>
__device__ __forceinline__ void gram_pair(IntraSmem<DK, DV>& sm, unsigned char* rec, int I, int J, int l) {
    typedef RecordLayout<DK, DV> R;
    const int l16 = l & 15, lq = l >> 4;
    const bf16_t* f = sm.fij[pair_index(I, J)];
    f32x4 akk = kZero4, aqk = kZero4;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
        const bf16x8 a = scale_frag(read16(lds_block(sm, ks, 2, J) + l * 16), f, ks, lq);
        akk = mma32(a, read16(lds_block(sm, ks, 1, I) + l * 16), akk);
        aqk = mma32(a, read16(lds_block(sm, ks, 0, I) + l * 16), aqk);
    }
    *reinterpret_cast<i16x4*>(&sm.akk[pair_index(I, J)][l * 4]) = cvt4(akk * sm.beta[16 * I + l16]);
    *reinterpret_cast<i16x4*>(rec + R::a(I, J >> 1) * 1024 + l * 16 + 8 * (J & 1)) = cvt4(aqk);
}

// Diagonal A_qk block I (j <= i kept) to the record; for I = 0 (I = 2) also the zero J = 1 (J = 3)
// half of record block A(0,0) (A(2,1)).
template <int DK, int DV>
__device__ __forceinline__ void diag_aqk_block(IntraSmem<DK, DV>& sm, unsigned char* rec, int I, int l) {
    typedef RecordLayout<DK, DV> R;
    const int l16 = l & 15, lq = l >> 4;
    f32x4 acc = kZero4;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks)
        acc = mma32(read16(lds_block(sm, ks, 2, I) + l * 16), read16(lds_block(sm, ks, 0, I) + l * 16), acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = (4 * lq + r <= l16) ? acc[r] : 0.f;
    unsigned char* b = rec + R::a(I, I >> 1) * 1024 + l * 16;
    *reinterpret_cast<i16x4*>(b + 8 * (I & 1)) = cvt4(acc);
    if ((I & 1) == 0) *reinterpret_cast<uint2*>(b + 8) = make_uint2(0u, 0u);
}

// Operands of the blocked substitution, from the Gram phase's LDS results.
template <int DK, int DV>
__device__ __forceinline__ SolveOps solve_ops(const IntraSmem<DK, DV>& sm, int l) {
    const int l16 = l & 15, lq = l >> 4;
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
    return ops;
}

// The wave's part of one chunk. `rec` (global or LDS memory) receives the chunk's record
// (kda_record.h). With DEFER, decay() keeps the record pieces it forms (Q~, K-, gamma) in
// registers and in the wave's LDS stage, and publish() writes them: the fused kernel's consumer
// waves may still be reading the previous chunk's record while decay() runs.
// With SPLIT (the fused kernel's producer) the value side and the diagonal blocks of A_kk belong
// to other waves (ValueWave): decay() loads and stages no V, gram() spreads the off-diagonal pairs
// and the diagonal A_qk blocks over all four waves, and solve() solves the W tiles only.
template <int DK, int DV, bool ZPRO, bool SPLIT = false>
struct ChunkWave {
    typedef IntraCfg<DK, DV> Cfg;
    typedef RecordLayout<DK, DV> R;
    static constexpr int NKS = Cfg::NKS, VPW = Cfg::VPW, LDG = Cfg::LDG, LDVS = Cfg::LDVS, LDW = Cfg::LDW;
    static constexpr int LPR = 2 * VPW;   // lanes per row of the value stage load

    IntraSmem<DK, DV>& sm;
    int w, l, l16, lq;
    bool kw, vw;       // this wave prepares key channels 32w .. 32w + 31 / solves value tiles
    int vc0;           // first value column of this wave
    uint32_t qk_voff, g_voff, v_voff;
    // Raw inputs of the chunk being loaded (one chunk ahead).
    uint4 pq[4], pk[4], pg[4], pv[LPR];
    uint32_t pb;
    // decay() -> solve(): V rows 16I + 4lq + e at column vc0 + 16j + l16, and K~ (chunk-relative)
    // rows 16I + 4lq + e at channel 32w + 16h + l16 (accumulator layout)
    i16x4 vacc[VPW][4];
    i16x4 kacc[2][4];
    // DEFER: the Q~ record blocks (I, w) and gamma of channels 32w + 16h + 4lq .. (lanes l16 = 15)
    bf16x8 qblk[4];
    f32x4 gam[2];

    __device__ __forceinline__ explicit ChunkWave(IntraSmem<DK, DV>& s) : sm(s) {
        const int tid = threadIdx.x;
        w = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);
        l = tid & 63;
        l16 = l & 15;
        lq = l >> 4;
        kw = NKS == 4 || w < NKS;
        vw = !SPLIT && Cfg::has_v(w);
        vc0 = 16 * Cfg::vt0(w);
        // Lane's 16-byte slice of a q/k row: rows (lq = 0, 1) and (2, 3) then trade halves with one
        // permlane16 swap per dword pair, which leaves each lane its fragment channels
        // 32w + 16h + 4lq .. +3 for h = 0, 1.
        const int qk_off = 8 * (((lq & 1) << 1) | (lq >> 1));
        qk_voff = (l16 * DK + 32 * w + qk_off) * 2;
        g_voff = ((l >> 2) * DK + 32 * w + 8 * (l & 3)) * 2;
        v_voff = ((l / LPR) * DV + vc0 + 8 * (l % LPR)) * 2;
    }
    __device__ __forceinline__ unsigned char* region() const { return sm.region[w]; }
    // LDS block of tensor X (0 Q~, 1 K~, 2 K^), token block I, of the wave owning channels 32ks..
    __device__ __forceinline__ unsigned char* lblk(int ks, int X, int I) const { return lds_block(sm, ks, X, I); }

    // Issue the loads of one chunk: rows row0 .. row0 + n - 1 of the bf16 row-major inputs q, k,
    // g (the decay rows: log_alpha, or the pre-activation z of the fused prologue), v and beta
    // (n <= 64; rows from n on read as zeros: every descriptor starts at the chunk's first row and
    // covers its valid rows only; n = 0 moves no data).
    __device__ __forceinline__ void load(const void* q, const void* k, const void* g, const void* v, const void* beta,
                                         int64_t row0, uint32_t n) {
        if (kw) {
            const uint32_t nk = n * (DK * 2);
            const __amdgpu_buffer_rsrc_t rq = make_rsrc((const bf16_t*)q + row0 * DK, nk);
            const __amdgpu_buffer_rsrc_t rk = make_rsrc((const bf16_t*)k + row0 * DK, nk);
            const __amdgpu_buffer_rsrc_t rg = make_rsrc((const bf16_t*)g + row0 * DK, nk);
            // Row offsets stay in the vector offset, the part of the address the buffer range
            // check sees; the empty asm stops the compiler from hoisting one register per row group.
            uint32_t qo = qk_voff, go = g_voff;
            asm volatile("" : "+v"(qo), "+v"(go));
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                pq[I] = buf_load16(rq, qo + 16 * I * DK * 2);
                pk[I] = buf_load16(rk, qo + 16 * I * DK * 2);
                pg[I] = buf_load16(rg, go + 16 * I * DK * 2);
            }
        }
        if (vw) {
            const __amdgpu_buffer_rsrc_t rv = make_rsrc((const bf16_t*)v + row0 * DV, n * (DV * 2));
            uint32_t vo = v_voff;
            asm volatile("" : "+v"(vo));
#pragma unroll
            for (int i = 0; i < LPR; ++i) pv[i] = buf_load16(rv, vo + i * (64 / LPR) * DV * 2);
        }
        if (w == 0) {
            const __amdgpu_buffer_rsrc_t rb = make_rsrc((const bf16_t*)beta + row0, n * 2);
            pb = buf_load2(rb, l * 2);
        }
    }
    // Wait for the loaded rows here: vmcnt counts loads and stores in issue order, so a wait left
    // to their first use would also wait for every store issued after them.
    __device__ __forceinline__ void pin_inputs() {
#pragma unroll
        for (int i = 0; i < 4; ++i) { pin(pq[i]); pin(pk[i]); pin(pg[i]); }
#pragma unroll
        for (int i = 0; i < LPR; ++i) pin(pv[i]);
        pin(pb);
    }

    // Phase 1 (wave-local): decay and scaled operands of the loaded chunk. eA = exp(A_h), g_min and
    // the chunk's valid rows feed the fused decay prologue only (padded rows must not decay there).
    template <bool DEFER>
    __device__ __forceinline__ void decay(unsigned char* rec, float eA, float g_min, uint32_t nrows) {
        if constexpr (DK < 128) {
            // dk = 64: the lane's offsets rebuilt for this phase (the compiler otherwise holds a
            // dozen LDS addresses across the chunk loop and spills them, each reload waiting for
            // the prefetch)
            const int sl = l, sl16 = l16, slq = lq;
            l = fresh_lane(); l16 = l & 15; lq = l >> 4;
            decay_body<DEFER>(rec, eA, g_min, nrows);
            l = sl; l16 = sl16; lq = slq;
        } else {
            decay_body<DEFER>(rec, eA, g_min, nrows);
        }
    }
    template <bool DEFER>
    __device__ __forceinline__ void decay_body(unsigned char* rec, float eA, float g_min, uint32_t nrows) {
        unsigned char* reg = region();
        bf16_t* stA = reinterpret_cast<bf16_t*>(reg);                    // g, then K- (token-major)
        unsigned char* stB = reg + Cfg::STAGE_A;                         // v, then blocks
        auto blk = [&](int b) -> unsigned char* { return rec + b * 1024 + l * 16; };
        uint2 qv[2][4], kv[2][4];
        bf16_t* vst = reinterpret_cast<bf16_t*>(stB);
        if (kw) {
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                *reinterpret_cast<uint4*>(&stA[(16 * I + (l >> 2)) * LDG + 8 * (l & 3)]) =
                    !ZPRO ? pg[I] : decay_from_z(pg[I], eA, 16u * I + (l >> 2) < nrows ? g_min : 0.f);
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
        wave_lds_sync();
        if (vw) {
#pragma unroll
            for (int j = 0; j < VPW; ++j)
#pragma unroll
                for (int I = 0; I < 4; ++I)
                    vacc[j][I] = tr_read(&vst[(16 * I + 4 * lq + (l16 >> 2)) * LDVS + 16 * j + 4 * (l16 & 3)]);
        }
        if (kw) {
            float pcol[2][4];   // exp(G_ref(I)) of channel 32w + 16h + l16
            i16x4 qrec[4];      // the h = 0 half of each Q~ record block, stored with the h = 1 half
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                bf16x8 ga[2];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const bf16_t* b0 = &stA[(32 * s + 4 * lq + (l16 >> 2)) * LDG + 16 * h + 4 * (l16 & 3)];
                    ga[s] = cat(tr_read(b0), tr_read(b0 + 16 * LDG));
                }
                // D[r] = G for channel 32w + 16h + 4lq + r at token 16I + l16. The constant
                // operands are rebuilt here (a few VALU ops) rather than held across the chunk
                // loop: the empty asm hides that their inputs are loop-invariant.
                int lqv = lq, l16v = l16;
                asm volatile("" : "+v"(lqv), "+v"(l16v));
                const UFrags uf = ufrags(lqv, l16v);
                f32x4 G[4];
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    G[I] = mma32(ga[0], uf.get(I, 0), kZero4);
                    if (I >= 2) G[I] = mma32(ga[1], uf.get(I, 1), G[I]);
                }
                // Reference points: G_ref(I) = G at token 16I - 1 (0 for I = 0), broadcast from
                // lane 15 of the row that holds tile I - 1; gC = G at token 63. Every factor between
                // reference points is a product of the block decays D_J = e^{G_ref(J+1) - G_ref(J)}
                // and the tail E = e^{gC - G_ref(3)}, all <= 1: P_I = e^{G_ref(I)} (P_0 = 1),
                // Q_I = e^{gC - G_ref(I)}, f_IJ = e^{G_ref(I) - G_ref(J)}, gamma_C = Q_0.
                f32x4 Gref[4], P[4], Qt[4], D[3];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    Gref[0][r] = 0.f;
                    Gref[1][r] = row_bcast15(G[0][r]);
                    Gref[2][r] = row_bcast15(G[1][r]);
                    Gref[3][r] = row_bcast15(G[2][r]);
                    const float gC = row_bcast15(G[3][r]);
                    D[0][r] = __builtin_amdgcn_exp2f(Gref[1][r] * kLog2e);
                    D[1][r] = __builtin_amdgcn_exp2f((Gref[2][r] - Gref[1][r]) * kLog2e);
                    D[2][r] = __builtin_amdgcn_exp2f((Gref[3][r] - Gref[2][r]) * kLog2e);
                    Qt[3][r] = __builtin_amdgcn_exp2f((gC - Gref[3][r]) * kLog2e);
                    P[0][r] = 1.f;
                    P[1][r] = D[0][r];
                    P[2][r] = D[0][r] * D[1][r];
                    P[3][r] = P[2][r] * D[2][r];
                    Qt[2][r] = Qt[3][r] * D[2][r];
                    Qt[1][r] = Qt[2][r] * D[1][r];
                    Qt[0][r] = Qt[1][r] * D[0][r];
                }
                if (DEFER) gam[h] = Qt[0];
                else if (l16 == 15)
                    *reinterpret_cast<f32x4*>(rec + R::G * 1024 + (32 * w + 16 * h + 4 * lq) * 4) = Qt[0];
                if (l16 == 0) {   // f_IJ for the lane's four channels
                    const int cc = 32 * w + 16 * h + 4 * lq;
                    *reinterpret_cast<i16x4*>(&sm.fij[pair_index(1, 0)][cc]) = cvt4(D[0]);
                    *reinterpret_cast<i16x4*>(&sm.fij[pair_index(2, 1)][cc]) = cvt4(D[1]);
                    *reinterpret_cast<i16x4*>(&sm.fij[pair_index(3, 2)][cc]) = cvt4(D[2]);
                    *reinterpret_cast<i16x4*>(&sm.fij[pair_index(2, 0)][cc]) = cvt4(P[2]);
                    *reinterpret_cast<i16x4*>(&sm.fij[pair_index(3, 1)][cc]) = cvt4(D[1] * D[2]);
                    *reinterpret_cast<i16x4*>(&sm.fij[pair_index(3, 0)][cc]) = cvt4(P[3]);
                }
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    const f32x4 qf = unpack4f(__builtin_bit_cast(i16x4, qv[h][I]));
                    const f32x4 kf = unpack4f(__builtin_bit_cast(i16x4, kv[h][I]));
                    f32x4 oq, ok, oh, ob, orq;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        // within the 16-token block: e1 = exp(G - G_ref) <= 1, e2 = 1/e1 <= e^80
                        const float d2 = (G[I][r] - Gref[I][r]) * kLog2e;
                        const float e1 = __builtin_amdgcn_exp2f(d2);
                        const float e2 = __builtin_amdgcn_exp2f(-d2);
                        oq[r] = qf[r] * e1;
                        ok[r] = kf[r] * e1;
                        oh[r] = kf[r] * e2;
                        // record factors relative to the chunk start, each <= 1
                        orq[r] = oq[r] * P[I][r];
                        ob[r] = oh[r] * Qt[I][r];
                    }
                    // fragment blocks (I, ks = w): register elements e < 4 come from h = 0, e >= 4
                    // from h = 1, i.e. bytes 8h .. 8h + 7 of the lane's 16
                    *reinterpret_cast<i16x4*>(lblk(w, 0, I) + l * 16 + 8 * h) = cvt4(oq);
                    *reinterpret_cast<i16x4*>(lblk(w, 1, I) + l * 16 + 8 * h) = cvt4(ok);
                    *reinterpret_cast<i16x4*>(lblk(w, 2, I) + l * 16 + 8 * h) = cvt4(oh);
                    if (h == 0) qrec[I] = cvt4(orq);
                    else if (DEFER) qblk[I] = cat(qrec[I], cvt4(orq));
                    else *reinterpret_cast<bf16x8*>(blk(R::q(I, w))) = cat(qrec[I], cvt4(orq));
                    // K- token-major into the g stage columns 16h.. (already consumed above)
                    *reinterpret_cast<uint2*>(&stA[(16 * I + l16) * LDG + 16 * h + 4 * lq]) =
                        __builtin_bit_cast(uint2, cvt4(ob));
                }
                // P_I (I > 0) of local channel 16h + 4lq + r (every lane of row lq holds it), fp32,
                // into the g stage's padding columns, stage row (I - 1) 8 + 4h + lq: the solve's
                // accumulator layout wants it for channel 16h + l16, read back after the sync below
                // (a cross-row permute here would wait for this phase's LDS writes)
                if (l16 == 0) {
#pragma unroll
                    for (int I = 1; I < 4; ++I)
                        *reinterpret_cast<f32x4*>(reinterpret_cast<unsigned char*>(stA) +
                                                  ((I - 1) * 8 + 4 * h + lq) * (LDG * 2) + 64) = P[I];
                }
                // one 16-channel tile at a time: interleaving the two would double the live set
                __builtin_amdgcn_sched_barrier(0);
            }
            wave_lds_sync();
            if (!DEFER) store_kbar(rec);
            // P_I of the lane's column channel 32w + 16h + l16 (P_0 = 1), from the stage padding
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                pcol[h][0] = 1.f;
#pragma unroll
                for (int I = 1; I < 4; ++I)
                    pcol[h][I] = *reinterpret_cast<const float*>(reinterpret_cast<const unsigned char*>(stA) +
                                                                 ((I - 1) * 8 + 4 * h + (l16 >> 2)) * (LDG * 2) + 64 +
                                                                 (l16 & 3) * 4);
            }
            // K~ in accumulator layout from its own blocks: the 8-byte chunk addressed by lane
            // (lq, l16) is K~[16I + 4lq + l16/4][32w + 16h + 4(l16%4) ..], i.e. block lane
            // (l16 % 4, 4lq + l16/4), half h.
            // (block-relative there; times exp(G_ref(I)) of the column's channel: chunk-relative)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int I = 0; I < 4; ++I)
                    kacc[h][I] = cvt4(pcol[h][I] * unpack4f(tr_read(reinterpret_cast<const bf16_t*>(
                        lblk(w, 1, I) + ((l16 & 3) * 16 + 4 * lq + (l16 >> 2)) * 16 + 8 * h))));
        }
    }
    // K- record blocks (M = 2w + h, half) from the token-major stage: K-[32 half + k(e)][16M + l16]
    __device__ __forceinline__ void store_kbar(unsigned char* rec) {
        const bf16_t* stA = reinterpret_cast<const bf16_t*>(region());
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const bf16_t* b0 = &stA[(32 * half + 4 * lq + (l16 >> 2)) * LDG + 16 * h + 4 * (l16 & 3)];
                *reinterpret_cast<bf16x8*>(rec + R::k(2 * w + h, half) * 1024 + l * 16) = cat(tr_read(b0), tr_read(b0 + 16 * LDG));
            }
    }
    // DEFER: the record pieces decay() held back (Q~, gamma, K-). The K- stage stays intact until
    // the next chunk's decay().
    __device__ __forceinline__ void publish(unsigned char* rec) {
        if (!kw) return;
#pragma unroll
        for (int I = 0; I < 4; ++I) *reinterpret_cast<bf16x8*>(rec + R::q(I, w) * 1024 + l * 16) = qblk[I];
        if (l16 == 15) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
                *reinterpret_cast<f32x4*>(rec + R::G * 1024 + (32 * w + 16 * h + 4 * lq) * 4) = gam[h];
        }
        store_kbar(rec);
    }

    // Phase 2: Gram tiles from every wave's LDS blocks. Wave 0 forms the four diagonal blocks of
    // A_kk and inverts I + A_kk,II (lane: block lq, row l16); waves 1-3 take two off-diagonal pairs
    // each, then the diagonal A_qk blocks. SPLIT: no diagonal A_kk work; the six pairs and the four
    // diagonal A_qk blocks spread over the four waves.
    __device__ __forceinline__ void gram(unsigned char* rec) {
        if (SPLIT) {   // (each wave's own addresses, rebuilt per chunk)
            const int fl = fresh_lane();
            if (w == 0) { gram_pair(sm, rec, 1, 0, fl); gram_pair(sm, rec, 2, 0, fl); }
            if (w == 1) { gram_pair(sm, rec, 2, 1, fl); gram_pair(sm, rec, 3, 0, fl); }
            if (w == 2) { gram_pair(sm, rec, 3, 1, fl); diag_aqk_block(sm, rec, 0, fl); diag_aqk_block(sm, rec, 1, fl); }
            if (w == 3) { gram_pair(sm, rec, 3, 2, fl); diag_aqk_block(sm, rec, 2, fl); diag_aqk_block(sm, rec, 3, fl); }
            return;
        }
        if (w == 0) {
#pragma unroll
            for (int I = 0; I < 4; ++I) diag_akk_block(sm, I, l);
            wave_lds_sync();
            invert_row(sm, lq, l16, true);
        } else {
            const int I0 = w == 1 ? 1 : (w == 2 ? 2 : 3), J0 = w == 1 ? 0 : (w == 2 ? 1 : 1);
            const int I1 = w == 1 ? 2 : 3, J1 = w == 1 ? 0 : (w == 2 ? 0 : 2);
            gram_pair(sm, rec, I0, J0, l);
            gram_pair(sm, rec, I1, J1, l);
            // diagonal A_qk blocks: wave 1 takes I = 0, 1, wave 2 I = 2, wave 3 I = 3
            const int nd = w == 1 ? 2 : 1;
            for (int d = 0; d < nd; ++d) diag_aqk_block(sm, rec, w == 1 ? d : w, l);
        }
    }

    // Phase 3: (I + A_kk) [W | U] = Diag(beta) [K~ | V]; U and -W to the record.
    __device__ __forceinline__ void solve(unsigned char* rec) {
        auto blk = [&](int b) -> unsigned char* { return rec + b * 1024 + l * 16; };
        const SolveOps ops = solve_ops(sm, l);
        if (vw) {
#pragma unroll
            for (int j = 0; j < VPW; ++j) {
                f32x4 X[4];
                ut_solve(ops, unpack4f(vacc[j][0]), unpack4f(vacc[j][1]), unpack4f(vacc[j][2]), unpack4f(vacc[j][3]),
                         X[0], X[1], X[2], X[3]);
                const int n = vc0 / 16 + j;
                *reinterpret_cast<bf16x8*>(blk(R::u(n, 0))) = cat(cvt4(X[0]), cvt4(X[1]));
                *reinterpret_cast<bf16x8*>(blk(R::u(n, 1))) = cat(cvt4(X[2]), cvt4(X[3]));
            }
        }
        if (kw) {
            bf16_t* wt = reinterpret_cast<bf16_t*>(region());   // W^T [32 channels][64 tokens]
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f32x4 X[4];
                ut_solve(ops, unpack4f(kacc[h][0]), unpack4f(kacc[h][1]), unpack4f(kacc[h][2]), unpack4f(kacc[h][3]),
                         X[0], X[1], X[2], X[3]);
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
};

// The value side of one chunk for a wave that owns value tiles 2 vw, 2 vw + 1 (dv = 128) and key
// block I = vw of A_kk's diagonal, next to four ChunkWave<..., SPLIT> waves (the fused kernel's
// consumer): V rows loaded one chunk ahead, staged in LDS into accumulator layout; the diagonal
// block and its inverse (for every wave's solve); and U = (I + A_kk)^{-1} Diag(beta) V for its
// tiles, kept in registers as the bf16 values a record would hold.
template <int DK, int DV>
struct ValueWave {
    typedef IntraCfg<DK, DV> Cfg;
    static constexpr int LDVS = Cfg::LDVS;
    static_assert(DV == 128 && Cfg::VPW == 2, "two value tiles per wave");
    IntraSmem<DK, DV>& sm;
    bf16_t* vst;      // this wave's V stage: 64 rows of LDVS elements
    int vw;
    uint4 pv[4];      // V rows of the chunk being loaded
    i16x4 vacc[2][4]; // V rows 16I + 4lq + e, column 32 vw + 16j + l16
    // (each phase derives its lane offsets from fresh_lane(): the wave runs beside the state step,
    // whose registers leave none to hold them across the chunk loop)

    __device__ __forceinline__ ValueWave(IntraSmem<DK, DV>& s, bf16_t* stage, int wave) : sm(s), vst(stage), vw(wave) {}
    // rows row0 .. row0 + n - 1 of v (zeros from n on; n = 0 moves no data)
    __device__ __forceinline__ void load(const void* v, int64_t row0, uint32_t n) {
        const __amdgpu_buffer_rsrc_t rv = make_rsrc((const bf16_t*)v + row0 * DV, n * (DV * 2));
        const int l = fresh_lane();
        const uint32_t vo = (uint32_t)(((l / 4) * DV + 32 * vw + 8 * (l % 4)) * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[i] = buf_load16(rv, vo + i * 16 * DV * 2);
    }
    __device__ __forceinline__ void pin_inputs() {
#pragma unroll
        for (int i = 0; i < 4; ++i) pin(pv[i]);
    }
    // the loaded rows into accumulator layout through the stage
    __device__ __forceinline__ void stage() {
        const int l = fresh_lane(), l16 = l & 15, lq = l >> 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&vst[(i * 16 + l / 4) * LDVS + 8 * (l % 4)]) = pv[i];
        wave_lds_sync();
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int I = 0; I < 4; ++I)
                vacc[j][I] = tr_read(&vst[(16 * I + 4 * lq + (l16 >> 2)) * LDVS + 16 * j + 4 * (l16 & 3)]);
    }
    // diagonal block vw of A_kk and the inverse of I + A_kk,vw (the lanes of row group lq = 0 store it)
    __device__ __forceinline__ void diag_inverse() {
        const int l = fresh_lane(), l16 = l & 15, lq = l >> 4;
        diag_akk_block(sm, vw, l);
        wave_lds_sync();
        invert_row(sm, vw, l16, lq == 0);
    }
    // U of this wave's two tiles, in the record's rounding
    __device__ __forceinline__ void solve(i16x4 (&U)[2][4]) {
        const SolveOps ops = solve_ops(sm, fresh_lane());
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            f32x4 X[4];
            ut_solve(ops, unpack4f(vacc[j][0]), unpack4f(vacc[j][1]), unpack4f(vacc[j][2]), unpack4f(vacc[j][3]), X[0],
                     X[1], X[2], X[3]);
#pragma unroll
            for (int I = 0; I < 4; ++I) U[j][I] = cvt4(X[I]);
        }
    }
};

}  // namespace intra
}  // namespace kda

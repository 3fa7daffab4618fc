// KDA chunkwise prefill for gfx950, fp32 inputs (dk = 64): one fused chunk loop per (lane, block of
// value columns) on the fp32 MFMA, and the state copy used by T = 0 calls. bf16 inputs take the
// two-kernel path instead (intra-chunk records in kda_intra.hip, state pass in kda_inter.hip).
//
// Mathematics (Kimi K3 reading notes, liuzhao09.github.io/papers/kimi-k3.html, section 2.2,
// chunk equations; the pieces the page leaves unprinted are derived by unrolling the
// recurrence inside one chunk). For a chunk of C = 64 rows with entry state S, per key
// channel G_r = sum_{s<=r} log_alpha_s, Gamma_r = exp(G_r), gamma_C = Gamma_C:
//   Q~ = Q*Gamma, K~ = K*Gamma, K^ = K/Gamma, K-bar = K*gamma_C/Gamma
//   A_kk = Diag(beta) StrictTril(K~ K^T),   A_qk = Tril(Q~ K^T)   (incl. diagonal)
//   V~ = (I + A_kk)^{-1} Diag(beta) (V - K~ S)          (= U - W S of the UT transform)
//   O  = Q~ S + A_qk V~
//   S' = Diag(gamma_C) S + K-bar^T V~
// The fp32 path is planned without a sequence split: each workgroup walks all chunks of its lane.
//
// Work decomposition. Value columns are independent given the key-side quantities, so a
// workgroup owns a lane (b,h) and NW*16 state columns; each wave owns 16
// of those columns (its slice of S lives in MFMA accumulators, fp32) and a 1/NW share of the
// key channels for the per-chunk key-side preparation. Per chunk:
//   A  (wave-local) load rows of q,k,log_alpha,v (prefetched one chunk ahead), cumulative
//      log-decay across the 64 lanes (= rows), exponentials, operand tiles to LDS
//   B  per-wave K~ S and S^T Q~^T on MFMA; Gram tiles on MFMA spread over the waves; wave 0
//      inverts the four 16x16 diagonal blocks of (I + A_kk) in fp32
//   D  per-wave: R = beta (V - K~ S), blocked forward substitution with the inverted diagonal
//      blocks (V~), O^T += V~^T A_qk^T -> o, S <- gamma_C S + K-bar^T V~
// Three workgroup barriers per chunk.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int kC = 64;  // chunk length

template <class Op, int DK, int NW>
struct __align__(16) ChunkSmem {
    typedef typename Op::elem E;
    static constexpr int P = 16 / (int)sizeof(E);  // 16-byte row padding, in elements
    static constexpr int LDK = DK + P;             // stride of [*][DK] tiles
    static constexpr int LDC = kC + P;             // stride of [*][C] tiles
    static constexpr int LDT = 16 + P;             // stride of the inverted diagonal blocks
    static constexpr int LDB = 16 * 16 + 4;        // fp32 diagonal blocks (block stride, floats)
    E q[kC * LDK];          // Q~
    E k[kC * LDK];          // K~
    E kh[kC * LDK];         // K^
    E kbT[DK * LDC];        // K-bar^T
    E aqk[kC * LDC];        // A_qk (upper 16x16 blocks (0,1) and (2,3) kept at zero)
    E l[kC * LDC];          // A_kk, off-diagonal 16x16 blocks
    E td[4 * 16 * LDT];     // (I + L_II)^{-1}, I = 0..3
    float ld[4 * LDB];      // diagonal blocks of A_kk, fp32
    float gam[DK];          // gamma_C
    float beta[kC];
    E sT[NW][16 * LDK];     // per wave: S^T of its 16 columns (operand precision)
    E x[NW][16 * LDC];      // per wave: V^T, then X^T and V~^T
};

template <typename T> struct VecCount { static constexpr int value = 1; };

template <class Op, typename TIn, typename TOut, int DK, int NW>
__global__ __launch_bounds__(NW * 64) void chunk_kernel(ChunkLaunch p) {
    typedef ChunkSmem<Op, DK, NW> Sm;
    typedef typename Op::elem E;
    constexpr int LDK = Sm::LDK, LDC = Sm::LDC, LDT = Sm::LDT, LDB = Sm::LDB;
    constexpr int CPW = DK / NW;                       // key channels prepared per wave
    constexpr int EPV = 16 / (int)sizeof(TIn);         // input elements per 16-byte vector
    constexpr int NVK = CPW / EPV;                     // vectors per row per key-side tensor
    constexpr int NVV = 16 / EPV;                      // vectors per row of the wave's 16 v columns
    constexpr int NM = DK / 16;                        // 16-row tiles of the state
    static_assert(CPW % EPV == 0 && CPW % 4 == 0, "channel split");
    __shared__ Sm sm;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep it scalar
    const int l = tid & 63;
    const int l16 = l & 15;
    const int lq = l >> 4;
    const int W = NW * 16;
    const int64_t DV = p.dv;

    // ---- which lane and column block this workgroup owns ---------------------------------
    int64_t bid = blockIdx.x;
    const int64_t nblk = gridDim.x;
    if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);  // siblings share an XCD
    const int ncb = (int)(DV / W);
    const int cb = (int)(bid % ncb);
    const int64_t lane = bid / ncb;
    const int64_t T = p.T;
    const int64_t c_begin = 0;
    const int64_t c_end = (T + kC - 1) / kC;

    const int col0 = cb * W + 16 * w;                  // first column of this wave
    const int ch0 = w * CPW;                           // first key channel this wave prepares

    const TIn* qg = (const TIn*)p.q + lane * T * DK;
    const TIn* kg = (const TIn*)p.k + lane * T * DK;
    const TIn* gg = (const TIn*)p.la + lane * T * DK;
    const TIn* vg = (const TIn*)p.v + lane * T * DV;
    const TIn* bg = (const TIn*)p.beta + lane * T;

    // ---- entry state into accumulators and into the wave's S^T operand tile ---------------
    f32x4 Sacc[NM];
    {
        const float* entry = p.S0 ? p.S0 + lane * DK * DV : nullptr;
        if (entry) {
            // all loads issued together, one wait
            const float* e = entry + col0 + l16;
#pragma unroll
            for (int M = 0; M < NM; ++M)
#pragma unroll
                for (int r = 0; r < 4; ++r) Sacc[M][r] = e[(int64_t)(16 * M + 4 * lq + r) * DV];
        } else {
#pragma unroll
            for (int M = 0; M < NM; ++M) Sacc[M] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int M = 0; M < NM; ++M)
            store4(&sm.sT[w][l16 * LDK + 16 * M + 4 * lq], Sacc[M][0], Sacc[M][1], Sacc[M][2], Sacc[M][3]);
    }
    // A_qk blocks above the diagonal that the 32-wide K steps touch stay zero for the whole run.
    for (int i = tid; i < 2 * 256; i += NW * 64) {
        const int blk = i >> 8, e = i & 255;
        sm.aqk[(32 * blk + (e >> 4)) * LDC + 32 * blk + 16 + (e & 15)] = Op::cvt(0.f);
    }

    // ---- prefetch registers: this lane = row l of the chunk -------------------------------
    uint4 pq[NVK], pk[NVK], pg[NVK], pv[NVV];
    float pb = 0.f;
    auto load_chunk = [&](int64_t c) {
        const int64_t row = c * kC + l;
        const bool ok = row < T;
#pragma unroll
        for (int i = 0; i < NVK; ++i) {
            const int64_t off = row * DK + ch0 + i * EPV;
            pq[i] = ok ? *reinterpret_cast<const uint4*>(qg + off) : make_uint4(0, 0, 0, 0);
            pk[i] = ok ? *reinterpret_cast<const uint4*>(kg + off) : make_uint4(0, 0, 0, 0);
            pg[i] = ok ? *reinterpret_cast<const uint4*>(gg + off) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < NVV; ++i)
            pv[i] = ok ? *reinterpret_cast<const uint4*>(vg + row * DV + col0 + i * EPV)
                                  : make_uint4(0, 0, 0, 0);
        if (w == 0) pb = ok ? ld_f(bg + row) : 0.f;
    };
    if (c_begin < c_end) load_chunk(c_begin);

    for (int64_t c = c_begin; c < c_end; ++c) {
        // ================= phase A: key-side preparation (wave-local) =====================
        {
            // one 16-byte group of EPV key channels at a time keeps the live set small
            uint4 cq_[NVK], ck_[NVK], cg_[NVK], cv_[NVV];
#pragma unroll
            for (int i = 0; i < NVK; ++i) { cq_[i] = pq[i]; ck_[i] = pk[i]; cg_[i] = pg[i]; }
#pragma unroll
            for (int i = 0; i < NVV; ++i) cv_[i] = pv[i];
            const float bcur = pb;
            if (c + 1 < c_end) load_chunk(c + 1);
#pragma unroll
            for (int i = 0; i < NVK; ++i) {
                asm volatile("" ::: "memory");
                float qf[EPV], kf[EPV], G[EPV];
                unpack16(cq_[i], (const TIn*)nullptr, qf);
                unpack16(ck_[i], (const TIn*)nullptr, kf);
                unpack16(cg_[i], (const TIn*)nullptr, G);
                // cumulative log-decay over the 64 rows (= lanes), in log2 units
#pragma unroll
                for (int j = 0; j < EPV; ++j) G[j] = wave_prefix_sum(G[j] * kLog2e);
                float oq[EPV], ok_[EPV], okh[EPV];
                const int chg = ch0 + i * EPV;
#pragma unroll
                for (int j = 0; j < EPV; ++j) {
                    const float gC = __builtin_amdgcn_exp2f(lane_value(G[j], 63));  // gamma_C, wave-uniform
                    const float gam = __builtin_amdgcn_exp2f(G[j]);
                    const float kh = kf[j] * __builtin_amdgcn_exp2f(-G[j]);
                    oq[j] = qf[j] * gam;
                    ok_[j] = kf[j] * gam;
                    okh[j] = kh;
                    sm.kbT[(chg + j) * LDC + l] = Op::cvt(kh * gC);
                    if (l == j) sm.gam[chg + j] = gC;
                }
                if constexpr (EPV == 8) {
                    store8(&sm.q[l * LDK + chg], oq);
                    store8(&sm.k[l * LDK + chg], ok_);
                    store8(&sm.kh[l * LDK + chg], okh);
                } else {
                    store4(&sm.q[l * LDK + chg], oq[0], oq[1], oq[2], oq[3]);
                    store4(&sm.k[l * LDK + chg], ok_[0], ok_[1], ok_[2], ok_[3]);
                    store4(&sm.kh[l * LDK + chg], okh[0], okh[1], okh[2], okh[3]);
                }
            }
            if (w == 0) sm.beta[l] = bcur;
#pragma unroll
            for (int i = 0; i < NVV; ++i) {
                float vf[EPV];
                unpack16(cv_[i], (const TIn*)nullptr, vf);
#pragma unroll
                for (int n = 0; n < EPV; ++n) sm.x[w][(i * EPV + n) * LDC + l] = Op::cvt(vf[n]);
            }
        }
        __syncthreads();

        // ================= phase B: state products, Gram tiles, diagonal inverses ==========
        f32x4 Y[4], Ot[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) { Y[I] = f32x4{0.f, 0.f, 0.f, 0.f}; Ot[I] = Y[I]; }
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks) {
            asm volatile("" ::: "memory");  // bound how many fragments the scheduler hoists
            const auto sf = Op::load32(&sm.sT[w][l16 * LDK + 32 * ks + 8 * lq]);
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const auto a = Op::load32(&sm.k[(16 * I + l16) * LDK + 32 * ks + 8 * lq]);
                Y[I] = Op::mma32(a, sf, Y[I]);
                const auto b = Op::load32(&sm.q[(16 * I + l16) * LDK + 32 * ks + 8 * lq]);
                Ot[I] = Op::mma32(sf, b, Ot[I]);
            }
        }
        if (w == 0) {
            // diagonal blocks of A_kk (fp32, strictly lower, rows scaled by beta), then invert
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                asm volatile("" ::: "memory");
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < DK / 32; ++ks) {
                    const auto a = Op::load32(&sm.k[(16 * I + l16) * LDK + 32 * ks + 8 * lq]);
                    const auto b = Op::load32(&sm.kh[(16 * I + l16) * LDK + 32 * ks + 8 * lq]);
                    acc = Op::mma32(a, b, acc);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 4 * lq + r;
                    sm.ld[I * LDB + i * 16 + l16] = (l16 < i) ? sm.beta[16 * I + i] * acc[r] : 0.f;
                }
            }
            wave_lds_sync();
            // lane (I = l / 16, j = l % 16) solves column j of (I + L_II)^{-1} by forward substitution
            const float* Lb = &sm.ld[lq * LDB];
            float tc[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) tc[i] = 0.f;
            // row i+1 of L_II is loaded while row i is consumed; the compiler barrier keeps at
            // most two rows in registers
            float4 cur[4], nxt[4];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (i + 1 < 16) {
#pragma unroll
                    for (int mb = 0; mb < (i + 4) / 4; ++mb)
                        nxt[mb] = *reinterpret_cast<const float4*>(&Lb[(i + 1) * 16 + 4 * mb]);
                }
                asm volatile("" ::: "memory");
                float s = 0.f;
#pragma unroll
                for (int mb = 0; mb < (i + 3) / 4; ++mb)
                    s += cur[mb].x * tc[4 * mb] + cur[mb].y * tc[4 * mb + 1] + cur[mb].z * tc[4 * mb + 2] +
                         cur[mb].w * tc[4 * mb + 3];
                tc[i] = (i == l16) ? 1.f : ((i < l16) ? 0.f : -s);
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) cur[mb] = nxt[mb];
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sm.td[(lq * 16 + i) * LDT + l16] = Op::cvt(tc[i]);
        } else {
            // off-diagonal A_kk blocks (6), then A_qk blocks (10)
            const int ntiles = 16;
            for (int idx = w - 1; idx < ntiles; idx += NW - 1) {
                int I, J;
                const bool is_kk = idx < 6;
                if (is_kk) {
                    I = idx < 1 ? 1 : (idx < 3 ? 2 : 3);
                    J = idx - (I * (I - 1)) / 2;
                } else {
                    const int t = idx - 6;
                    I = t < 1 ? 0 : (t < 3 ? 1 : (t < 6 ? 2 : 3));
                    J = t - (I * (I + 1)) / 2;
                }
                const E* A = is_kk ? sm.k : sm.q;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < DK / 32; ++ks) {
                    const auto a = Op::load32(&A[(16 * I + l16) * LDK + 32 * ks + 8 * lq]);
                    const auto b = Op::load32(&sm.kh[(16 * J + l16) * LDK + 32 * ks + 8 * lq]);
                    acc = Op::mma32(a, b, acc);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * I + 4 * lq + r;
                    const int j = 16 * J + l16;
                    if (is_kk) sm.l[i * LDC + j] = Op::cvt(sm.beta[i] * acc[r]);
                    else sm.aqk[i * LDC + j] = Op::cvt(j <= i ? acc[r] : 0.f);
                }
            }
        }
        __syncthreads();

        // ================= phase D: per-wave solve, output, state update ====================
        E* xw = sm.x[w];
        {
            f32x4 R[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const int i0 = 16 * I + 4 * lq;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float vv = ld_f(&xw[l16 * LDC + i0 + r]);
                    R[I][r] = sm.beta[i0 + r] * (vv - Y[I][r]);
                }
            }
            // (I + A_kk) V~ = R, block rows I = 0..3
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                f32x4 X = R[I];
                if (I > 0) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    const int rowL = (16 * I + l16) * LDC;
                    if (I == 1) {
                        acc = Op::mma16(Op::load16(&sm.l[rowL + 4 * lq]), Op::load16(&xw[l16 * LDC + 4 * lq]), acc);
                    } else {
                        acc = Op::mma32(Op::load32(&sm.l[rowL + 8 * lq]), Op::load32(&xw[l16 * LDC + 8 * lq]), acc);
                        if (I == 3) {
                            // A fresh accumulator: one accumulation chain never mixes MFMA shapes
                            // (a 16x16x16 reading as SrcC the result of a 16x16x32 issued just
                            // before it was observed to see the stale value).
                            f32x4 acc16 = {0.f, 0.f, 0.f, 0.f};
                            acc16 = Op::mma16(Op::load16(&sm.l[rowL + 32 + 4 * lq]),
                                              Op::load16(&xw[l16 * LDC + 32 + 4 * lq]), acc16);
                            acc = acc + acc16;
                        }
                    }
                    X = X - acc;
                }
                E* xi = &xw[l16 * LDC + 16 * I + 4 * lq];
                store4(xi, X[0], X[1], X[2], X[3]);
                wave_lds_sync();
                f32x4 vt = {0.f, 0.f, 0.f, 0.f};
                vt = Op::mma16(Op::load16(&sm.td[(I * 16 + l16) * LDT + 4 * lq]), Op::load16(xi), vt);
                store4(xi, vt[0], vt[1], vt[2], vt[3]);
                wave_lds_sync();
            }
        }
        {
            TOut* og = (TOut*)p.o + lane * T * DV;
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                asm volatile("" ::: "memory");
#pragma unroll
                for (int ks = 0; ks < (I < 2 ? 1 : 2); ++ks) {
                    const auto a = Op::load32(&xw[l16 * LDC + 32 * ks + 8 * lq]);
                    const auto b = Op::load32(&sm.aqk[(16 * I + l16) * LDC + 32 * ks + 8 * lq]);
                    Ot[I] = Op::mma32(a, b, Ot[I]);
                }
                const int64_t row = c * kC + 16 * I + l16;
                if (row < T) store4(og + row * DV + col0 + 4 * lq, Ot[I][0], Ot[I][1], Ot[I][2], Ot[I][3]);
            }
        }
#pragma unroll
        for (int M = 0; M < NM; ++M) {
            asm volatile("" ::: "memory");
            const float4 g4 = *reinterpret_cast<const float4*>(&sm.gam[16 * M + 4 * lq]);
            f32x4 acc = Sacc[M];
            acc[0] *= g4.x; acc[1] *= g4.y; acc[2] *= g4.z; acc[3] *= g4.w;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const auto a = Op::load32(&sm.kbT[(16 * M + l16) * LDC + 32 * ks + 8 * lq]);
                const auto b = Op::load32(&xw[l16 * LDC + 32 * ks + 8 * lq]);
                acc = Op::mma32(a, b, acc);
            }
            Sacc[M] = acc;
            store4(&sm.sT[w][l16 * LDK + 16 * M + 4 * lq], acc[0], acc[1], acc[2], acc[3]);
        }
        __syncthreads();
    }

    // ---- exit state ------------------------------------------------------------------------
    if (p.S_T) {
        float* dst = p.S_T + lane * DK * DV;
#pragma unroll
        for (int M = 0; M < NM; ++M)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(int64_t)(16 * M + 4 * lq + r) * DV + col0 + l16] = Sacc[M][r];
    }
}

__global__ void copy_or_zero_kernel(float* dst, const float* src, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = src ? src[i] : 0.f;
}

template <class Op, typename TIn, typename TOut, int DK, int NW>
static hipError_t launch_t(const ChunkLaunch& a, hipStream_t st) {
    const int W = NW * 16;
    const int64_t blocks = a.lanes * (a.dv / W);
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL((chunk_kernel<Op, TIn, TOut, DK, NW>), dim3((unsigned)blocks), dim3(NW * 64), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_chunk(const ChunkLaunch& a, hipStream_t st) {
    // fp32 path (dk = 64): the generic kernel on fp32 MFMA
    return a.out_bf16 ? launch_t<OpF32, float, bf16_t, 64, 4>(a, st) : launch_t<OpF32, float, float, 64, 4>(a, st);
}

hipError_t launch_copy_or_zero(float* dst, const float* src, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(copy_or_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, dst, src, n);
    return hipGetLastError();
}

}  // namespace kda

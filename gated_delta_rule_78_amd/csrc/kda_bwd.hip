// KDA backward (training) of chunkwise prefill for gfx950, bf16 inputs, fp32 arithmetic.
//
// The pages print no backward (section 2.2 of the Kimi K3 reading notes,
// liuzhao09.github.io/papers/kimi-k3.html, says training uses chunkwise KDA); this is the chain
// rule through the chunk equations of that section. For one 64-token chunk with entry state S,
// G = cumsum(g) over the chunk's rows, E_ij = exp(G_i - G_j) per channel (i >= j, so <= 1 over
// the whole decay domain), gamma = exp(G_63):
//   A_kk[i][j] = beta_i sum_c K_ic K_jc E_ijc (i > j),   T = (I + A_kk)^{-1}
//   W = T Diag(beta) (K e^G),   U = T Diag(beta) V,   V~ = U - W S
//   A_qk[i][j] = sum_c Q_ic K_jc E_ijc (i >= j),   O = (Q e^G) S + A_qk V~
//   S' = Diag(gamma) S + K-^T V~,   K- = K e^{G_63 - G}
// Given dO and the exit-state gradient Gx = dL/dS':
//   dV~ = A_qk^T dO + K- Gx,   dS = (Q e^G)^T dO + Diag(gamma) Gx - W^T dV~       (to chunk c-1)
//   dA_qk = Tril(dO V~^T),  dQ~ = dO S^T,  dW = -dV~ S^T,  dK- = V~ Gx^T,  dgamma = rowsum(Gx*S)
//   [dX_K | dX_V] = T^T [dW | dV~],   dA_kk = -(dX_K W^T + dX_V U^T) below the diagonal
// and from there to dq, dk, dv, dbeta and dG elementwise (the pairwise sums carry E_ijc), then
// dg = reverse cumsum of dG over the chunk (dgamma lands on row 63).
//
// Three kernels after a forward recompute that stores every chunk's entry state:
//   bwd_prep_kernel    one workgroup per chunk: T, W, U, Q~, K-, A_qk, gamma (fp32 scratch)
//   bwd_state_kernel   one workgroup per (lane, 16 or 32 value columns), chunks in reverse: Gx of every
//                      chunk, dV~, and dS0
//   bwd_grad_kernel    one workgroup per chunk: dq, dk, dv, dlog_alpha, dbeta
// All arithmetic is fp32. The matrix products (the state pass, V~ and the value-column products,
// T^T [dW | dV~], dA_kk) run on the fp32 matrix cores (16x16x4 MFMA) from LDS operands laid out
// contiguous along the contraction index; the pairwise decay terms and the inverse run on the
// VALU. One workgroup per CU (each kernel's LDS arena takes most of it).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kC = 64;
constexpr int kT = 256;   // threads per workgroup (prep, state pass)
constexpr int kTG = 512;  // threads of the gradient kernel: two waves per SIMD on its LDS arena
constexpr int kTP = 512;  // threads of the prep kernel, likewise

// Per-chunk fp32 scratch written by the prep kernel (offsets in floats).
template <int DK, int DV>
struct BwdLayout {
    static constexpr int T = 0;                       // [64][64] T = (I + A_kk)^{-1}
    static constexpr int W = T + kC * kC;             // [64][DK]
    static constexpr int U = W + kC * DK;             // [64][DV]
    static constexpr int QT = U + kC * DV;            // [64][DK] Q e^G
    static constexpr int KB = QT + kC * DK;           // [64][DK] K e^{G_63 - G}
    static constexpr int AQK = KB + kC * DK;          // [64][64]
    static constexpr int GAM = AQK + kC * kC;         // [DK] gamma
    static constexpr int PREP = GAM + DK;
};

__device__ __forceinline__ float ldin(const bf16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
__device__ __forceinline__ float ldo(const bf16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
__device__ __forceinline__ float ldo(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ f32x4 kZero4f() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// The backward kernels never read back, inside a workgroup, what they write to global memory, so
// their barriers order LDS only (lds_barrier) and prefetches stay in flight across them.

template <int V>
struct IntC { static constexpr int value = V; };

// fp32 16x16x4 MFMA step: lane l = r + 16 g supplies A[r][g] and B[g][r]; the accumulator holds
// rows 4 g .. 4 g + 3 of column r
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Register tiles for cooperative global -> LDS copies by NT threads: every thread issues all of
// its loads before its first LDS write, so a block costs one memory round trip instead of one per
// element. Piece e of a block goes to thread e mod NT.
template <int ROWS, int COLS, int NT>
struct F32Tile {   // fp32 block, 16-byte pieces
    static constexpr int Q = COLS / 4, N = ROWS * Q, PER = (N + NT - 1) / NT;
    static_assert(COLS % 4 == 0, "fp32 tile columns");
    f32x4 r[PER];
    __device__ __forceinline__ void load(const float* src, int64_t ld) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = threadIdx.x + u * NT;
            if (N % NT == 0 || e < N) r[u] = *reinterpret_cast<const f32x4*>(src + (e / Q) * ld + (e % Q) * 4);
        }
    }
    // keep = false stores zeros (a missing operand read from a stand-in address)
    __device__ __forceinline__ void store(float* dst, int ld, bool keep = true) const {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = threadIdx.x + u * NT;
            if (N % NT == 0 || e < N) *reinterpret_cast<f32x4*>(dst + (e / Q) * ld + (e % Q) * 4) = keep ? r[u] : kZero4f();
        }
    }
};

// fp32 block stored transposed into LDS (dst[c][r] = src[r][c]). Each wave instruction covers 16
// rows x 16 columns: lane l takes row 16 rb + (l mod 16) and the four columns from
// 16 cb + 4 (l / 16), so with a destination row stride of 4 mod 32 floats the transposed stores of
// a half-wave fall in distinct banks.
template <int ROWS, int COLS, int NT>
struct F32TileT {
    static constexpr int RB = ROWS / 16, NBLK = RB * (COLS / 16), NW = NT / 64, PER = NBLK / NW;
    static_assert(ROWS % 16 == 0 && COLS % 16 == 0 && NBLK % NW == 0, "transposed tile");
    f32x4 r[PER];
    static __device__ __forceinline__ int row(int u) {
        return 16 * (((int)(threadIdx.x >> 6) + NW * u) % RB) + (threadIdx.x & 15);
    }
    static __device__ __forceinline__ int col(int u) {
        return 16 * (((int)(threadIdx.x >> 6) + NW * u) / RB) + 4 * ((threadIdx.x >> 4) & 3);
    }
    __device__ __forceinline__ void load(const float* src, int64_t ld) {
#pragma unroll
        for (int u = 0; u < PER; ++u) r[u] = *reinterpret_cast<const f32x4*>(src + row(u) * ld + col(u));
    }
    __device__ __forceinline__ void store_t(float* dst, int ld) const {
#pragma unroll
        for (int u = 0; u < PER; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[(col(u) + i) * ld + row(u)] = r[u][i];
    }
};

// Rows [0, nrows) of a bf16 or fp32 row-major block as fp32, in pieces of 8 elements (16 bytes of
// bf16, 32 of fp32). Rows past nrows read the last valid row (no branch, hence no wait at the
// load) and are stored as zeros; an optional per-row factor scales what is stored.
template <int ROWS, int COLS, int NT, typename TI>
struct InTile {
    static constexpr int Q = COLS / 8, N = ROWS * Q, PER = (N + NT - 1) / NT, W = sizeof(TI) / 2;
    static_assert(COLS % 8 == 0 && (sizeof(TI) == 2 || sizeof(TI) == 4), "input tile");
    uint4 r[PER * W];
    int nrows;
    __device__ __forceinline__ void load(const TI* src, int64_t ld, int nrows_) {
        nrows = nrows_;
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = threadIdx.x + u * NT, row = e / Q, rr = row < nrows_ ? row : nrows_ - 1;
            const uint4* p = reinterpret_cast<const uint4*>(src + rr * ld + (e % Q) * 8);
            if (N % NT == 0 || e < N)
#pragma unroll
                for (int w = 0; w < W; ++w) r[u * W + w] = p[w];
        }
    }
    __device__ __forceinline__ void store(float* dst, int ld, const float* rowscale = nullptr) const {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = threadIdx.x + u * NT, row = e / Q;
            if (!(N % NT == 0 || e < N)) continue;
            const float f = row < nrows ? (rowscale ? rowscale[row] : 1.f) : 0.f;
            float x[8];
            if (W == 1) {
                const uint4 v = r[u * W];
                const unsigned h[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[2 * i] = __uint_as_float(h[i] << 16);
                    x[2 * i + 1] = __uint_as_float(h[i] & 0xffff0000u);
                }
            } else {
#pragma unroll
                for (int w = 0; w < W; ++w) {
                    const uint4 v = r[u * W + w];
                    x[4 * w] = __uint_as_float(v.x); x[4 * w + 1] = __uint_as_float(v.y);
                    x[4 * w + 2] = __uint_as_float(v.z); x[4 * w + 3] = __uint_as_float(v.w);
                }
            }
            float* d = dst + row * ld + (e % Q) * 8;
            *reinterpret_cast<f32x4*>(d) = f32x4{f * x[0], f * x[1], f * x[2], f * x[3]};
            *reinterpret_cast<f32x4*>(d + 4) = f32x4{f * x[4], f * x[5], f * x[6], f * x[7]};
        }
    }
};

template <int DK, int DV>
struct __align__(16) PrepSmem {
    static constexpr int LP = DK + 4;   // padded rows: 16-byte reads of 8 rows fall in distinct banks
    float K[kC][LP], Q[kC][LP], G[kC][LP];
    float A[kC][kC + 1], T[kC][kC + 4];   // T rows 16-byte aligned for the MFMA operand reads
    float Y[3][16][17];                   // block products of the inverse's substitution levels
    float beta[kC];
    float Vx[DV > DK ? kC : 1][DV > DK ? DV : 4];   // beta V when it does not fit over Q
};

template <int DK, int DV>
__global__ __launch_bounds__(kTP) void bwd_prep_kernel(BwdArgs a) {
    typedef BwdLayout<DK, DV> L;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    PrepSmem<DK, DV>& sm = *reinterpret_cast<PrepSmem<DK, DV>*>(smem_raw);
    const int64_t lane = blockIdx.x / a.nchunks, c = blockIdx.x % a.nchunks;
    const int64_t row0 = lane * a.T + c * kC;
    const int nrows = (int)(a.T - c * kC < kC ? a.T - c * kC : kC);
    float* sc = a.prep + (int64_t)blockIdx.x * L::PREP;
    const int tid = threadIdx.x;
    // K, Q, log_alpha and V of the chunk in one round trip; V stays in registers until its LDS
    // place is free (a persistent grid that loads the next chunk's rows during the current one's
    // last phase was 3 % slower: its loop held 229 registers instead of 70)
    InTile<kC, DK, kTP, bf16_t> tk, tq, tg;
    InTile<kC, DV, kTP, bf16_t> tv;
    tk.load((const bf16_t*)a.k + row0 * DK, DK, nrows);
    tq.load((const bf16_t*)a.q + row0 * DK, DK, nrows);
    tg.load((const bf16_t*)a.la + row0 * DK, DK, nrows);
    tv.load((const bf16_t*)a.v + row0 * DV, DV, nrows);
    if (tid < kC) {
        const float b = ldin((const bf16_t*)a.beta, row0 + (tid < nrows ? tid : nrows - 1));
        sm.beta[tid] = tid < nrows ? b : 0.f;
    }
    tk.store(&sm.K[0][0], PrepSmem<DK, DV>::LP);
    tq.store(&sm.Q[0][0], PrepSmem<DK, DV>::LP);
    tg.store(&sm.G[0][0], PrepSmem<DK, DV>::LP);
    lds_barrier();
    for (int c = tid; c < DK; c += kTP) {   // G = inclusive cumulative sum of log_alpha down the rows
        float acc = 0.f;
        for (int t = 0; t < kC; ++t) { acc += sm.G[t][c]; sm.G[t][c] = acc; }
    }
    lds_barrier();

    // A_kk (i > j, beta-scaled) and A_qk (i >= j) by 16 x 16 blocks (I, J), I >= J, each on the fp32
    // MFMA with the factors exp(G_i - G_j) split at r = 16 I, the first row of block I, as
    // exp(G_i - G_r) exp(G_r - G_j) and folded into the operands. Off the diagonal both factors are
    // <= 1 (j < r <= i), so the whole decay domain stays in range; on a diagonal block the second
    // is at most e^{15 * 5} (the per-step bound of the decay), still inside the fp32 range.
    {   // A_qk above the diagonal blocks is zero: thread = (row i, every 8th column from the next block)
        const int i = tid >> 3;
        for (int j = (i & ~15) + 16 + (tid & 7); j < kC; j += 8) sc[L::AQK + i * kC + j] = 0.f;
    }
    const int wv = tid >> 6, lr = tid & 15, lg = (tid >> 4) & 3;
    // One 16 x 16 block (I, J), I >= J, of A_kk and A_qk on the fp32 MFMA (one wave). Inside a
    // diagonal block the second factor exp(G_r - G_j) is >= 1 but at most e^{15 * 5}, far inside
    // the fp32 range; the entries above the diagonal (whose product is not bounded) are masked out.
    auto gram_block = [&](int I, int J) {
        const int r = 16 * I, ia = r + lr, jb = 16 * J + lr;
        f32x4 ckk = kZero4f(), cqk = kZero4f();
        for (int kb = 0; kb < DK; kb += 16) {
            const int k0 = kb + 4 * lg;
            const f32x4 ka = *reinterpret_cast<const f32x4*>(&sm.K[ia][k0]);
            const f32x4 qa = *reinterpret_cast<const f32x4*>(&sm.Q[ia][k0]);
            const f32x4 ga = *reinterpret_cast<const f32x4*>(&sm.G[ia][k0]);
            const f32x4 gr = *reinterpret_cast<const f32x4*>(&sm.G[r][k0]);
            const f32x4 kbv = *reinterpret_cast<const f32x4*>(&sm.K[jb][k0]);
            const f32x4 gbv = *reinterpret_cast<const f32x4*>(&sm.G[jb][k0]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float fa = fexp(ga[q] - gr[q]), fb = kbv[q] * fexp(gr[q] - gbv[q]);
                ckk = mfma4(ka[q] * fa, fb, ckk);
                cqk = mfma4(qa[q] * fa, fb, cqk);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = r + 4 * lg + e, col = 16 * J + lr;
            sm.A[row][col] = col < row ? sm.beta[row] * ckk[e] : 0.f;   // always true off the diagonal
            sc[L::AQK + row * kC + col] = col <= row ? cqk[e] : 0.f;
        }
    };
    // One block per wave: the six off-diagonal blocks on waves 0 .. 5, diagonal blocks 0 and 1 on
    // waves 6 and 7. Diagonal blocks 2 and 3 go to waves 2 and 3 in the next phase, right before
    // they invert them (two blocks on one wave here made that wave the phase's critical path).
    if (wv < 6) {
        const int I = wv < 1 ? 1 : (wv < 3 ? 2 : 3);
        gram_block(I, wv - (I * (I - 1)) / 2);
    } else {
        gram_block(wv - 6, wv - 6);
    }
    lds_barrier();
    // T = (I + A_kk)^{-1} (unit lower triangular) by 16 x 16 blocks: waves 0-3 invert the diagonal
    // blocks (one column per lane in registers, rows in order) while waves 4-7 write Q~, K- and
    // gamma; then block forward substitution T_IJ = -T_II sum_{J <= K < I} A_IK T_KJ, one level
    // of I - J at a time, on the fp32 MFMA.
    if (wv < 4) {
        if (wv >= 2) {   // this wave's diagonal block of A_kk and A_qk first
            gram_block(wv, wv);
            wave_lds_sync();
        }
        const int o = 16 * wv, j = lr;
        float col[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float x = i == j ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) x -= sm.A[o + i][o + m] * col[m];
            col[i] = i >= j ? x : 0.f;
        }
        if ((tid & 63) < 16)
#pragma unroll
            for (int i = 0; i < 16; ++i) sm.T[o + i][o + j] = col[i];
        for (int e = tid & 63; e < 16 * (kC - o - 16); e += 64) sm.T[o + e / (kC - o - 16)][o + 16 + e % (kC - o - 16)] = 0.f;
    } else {
        // Q~ = Q e^G, K- = K e^{G_63 - G}, gamma: four channels per thread and step
        for (int e = tid - 256; e < kC * DK / 4; e += kTP - 256) {
            const int t = e / (DK / 4), ch = 4 * (e % (DK / 4));
            const f32x4 q4 = *reinterpret_cast<const f32x4*>(&sm.Q[t][ch]);
            const f32x4 k4 = *reinterpret_cast<const f32x4*>(&sm.K[t][ch]);
            const f32x4 g4 = *reinterpret_cast<const f32x4*>(&sm.G[t][ch]);
            const f32x4 gl = *reinterpret_cast<const f32x4*>(&sm.G[kC - 1][ch]);
            f32x4 qt, kb;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qt[i] = q4[i] * fexp(g4[i]);
                kb[i] = k4[i] * fexp(gl[i] - g4[i]);
            }
            *reinterpret_cast<f32x4*>(sc + L::QT + t * DK + ch) = qt;
            *reinterpret_cast<f32x4*>(sc + L::KB + t * DK + ch) = kb;
        }
        for (int ch = tid - 256; ch < DK; ch += kTP - 256) sc[L::GAM + ch] = fexp(sm.G[kC - 1][ch]);
    }
    lds_barrier();
#pragma unroll
    for (int d = 1; d <= 3; ++d) {
        const bool job = wv < 4 - d;
        const int J = wv, I = wv + d;
        if (job) {   // Y = sum_K A_IK T_KJ
            f32x4 y = kZero4f();
            for (int K = J; K < I; ++K)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    y = mfma4(sm.A[16 * I + lr][16 * K + 4 * lg + q], sm.T[16 * K + 4 * lg + q][16 * J + lr], y);
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.Y[wv][4 * lg + e][lr] = y[e];
        }
        lds_barrier();
        if (job) {   // T_IJ = -T_II Y
            f32x4 t4 = kZero4f();
            const f32x4 x = *reinterpret_cast<const f32x4*>(&sm.T[16 * I + lr][16 * I + 4 * lg]);
#pragma unroll
            for (int q = 0; q < 4; ++q) t4 = mfma4(x[q], sm.Y[wv][4 * lg + q][lr], t4);
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.T[16 * I + 4 * lg + e][16 * J + lr] = -t4[e];
        }
        lds_barrier();
    }
    lds_barrier();
    // right-hand sides in place: K <- Diag(beta) K e^G, and Diag(beta) V over Q (or its own
    // array when dv > dk), rows of DV floats
    float* Vs = DV <= DK ? &sm.Q[0][0] : &sm.Vx[0][0];
    for (int e = tid; e < kC * DK / 4; e += kTP) {
        const int t = e / (DK / 4), ch = 4 * (e % (DK / 4));
        f32x4& k4 = *reinterpret_cast<f32x4*>(&sm.K[t][ch]);
        const f32x4 g4 = *reinterpret_cast<const f32x4*>(&sm.G[t][ch]);
        const float b = sm.beta[t];
        f32x4 x = k4;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] *= b * fexp(g4[i]);
        k4 = x;
    }
    tv.store(Vs, DV, sm.beta);
    for (int e = tid; e < kC * kC / 4; e += kTP) {
        const int t = e / (kC / 4), m = 4 * (e % (kC / 4));
        *reinterpret_cast<f32x4*>(sc + L::T + t * kC + m) = *reinterpret_cast<const f32x4*>(&sm.T[t][m]);
    }
    lds_barrier();
    // W = T (beta K e^G), U = T (beta V) as 16x16x4 MFMA tiles. Row block b costs b + 1 steps
    // (T[t][m] = 0 past the diagonal block, so m stops there): wave w takes row blocks {0, 3}
    // (w even) or {1, 2} (w odd), five steps either way, and a quarter of the columns of W and U.
    {
        constexpr int NWT = DK / 64, NUT = DV / 64;
        const int cw = (DK / 4) * (wv >> 1), cu = (DV / 4) * (wv >> 1);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int rb = 16 * ((wv & 1) ? 1 + h : 3 * h);
            f32x4 aw[NWT], au[NUT];
#pragma unroll
            for (int ct = 0; ct < NWT; ++ct) aw[ct] = kZero4f();
#pragma unroll
            for (int ct = 0; ct < NUT; ++ct) au[ct] = kZero4f();
            for (int kb = 0; kb <= rb; kb += 16) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(&sm.T[rb + lr][kb + 4 * lg]);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int m = kb + 4 * lg + q;
#pragma unroll
                    for (int ct = 0; ct < NWT; ++ct) aw[ct] = mfma4(x[q], sm.K[m][cw + 16 * ct + lr], aw[ct]);
#pragma unroll
                    for (int ct = 0; ct < NUT; ++ct) au[ct] = mfma4(x[q], Vs[m * DV + cu + 16 * ct + lr], au[ct]);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = rb + 4 * lg + e;
#pragma unroll
                for (int ct = 0; ct < NWT; ++ct) sc[L::W + t * DK + cw + 16 * ct + lr] = aw[ct][e];
#pragma unroll
                for (int ct = 0; ct < NUT; ++ct) sc[L::U + t * DV + cu + 16 * ct + lr] = au[ct][e];
            }
        }
    }
}

// Reverse state pass for value columns [j0, j0 + NB) of one lane (NB = 16 or 32), on the fp32 matrix cores
// (16x16x4 MFMA). Per chunk, walking backwards:
//     dV~ = K- Gx + A_qk^T dO                     (64 x NB; wave w owns rows 16w .. 16w + 15)
//     Gx  <- Diag(gamma) Gx + Q~^T dO - W^T dV~   (DK x NB; wave w owns rows DK/4 w ..)
// Gx lives in the waves' accumulator registers for the whole pass. K-, dO and dV~ sit in LDS with
// the contraction index contiguous (dO and dV~ transposed while staged or stored), so a lane
// fetches its next four k values in one 16-byte read; Q~, -W and A_qk stay in their row-major
// layout, where the contraction index is the row, and a lane reads its four values one by one
// (consecutive lanes take consecutive columns). In a 16x16x4 step lane l = r + 16 g supplies row
// (or column) r at k = g; the k values a lane walks through are assigned as kb + 4 g + q for step
// q of a block of 16, the same on both sides.
// The chunk before the current one is loaded into registers while the current one computes; the
// barriers order LDS only, so that load stays in flight across them.
template <int DK, int NB>
struct __align__(16) StateSmem {
    static constexpr int LK = DK + 4, LS = kC + 4;
    float KB[kC][LK];     // K- [t][ch]
    float QT[kC][LK];     // Q~ [s][ch]
    float WN[kC][LK];     // -W [s][ch]
    float AQ[kC][LS];     // A_qk [s][t]
    float dOT[NB][LS];    // dO^T [j][s]
    float dVT[NB][LS];    // dV~^T [j][s]
    float GxT[NB][LK];    // Gx^T [j][ch]
    float gam[DK];
};

// one thread's share of a chunk's state-pass operands, held in registers between the global load
// and the LDS store. Each factor is read as one contiguous array: float4 number tid + 256 u, so a
// wave's load instruction covers 1 KiB of whole cache lines, and the LDS stores keep the layout
// (16-byte stores, no transposition). Reading the factors in 16 x 16 blocks instead (half cache
// lines per row, for transposed LDS stores) made the loads costlier to issue: 8K backward
// 2.272-2.278 ms against 2.224-2.231 ms.
template <int DK, typename TO, int NB>
struct StateFetch {
    static constexpr int NF = kC * DK / 4 / kT;   // float4s of one [64][DK] factor
    static constexpr int NA = kC * kC / 4 / kT;   // float4s of A_qk
    static constexpr int ND = kC * NB / kT;       // dO elements
    static_assert(kT == 256, "four waves");
    f32x4 kb[NF], qt[NF], w[NF], aqk[NA];
    f32x4 gam;
    TO dO[ND];     // raw, converted when stored to LDS
    int nrows;

    // The loads of one chunk as a flat list: [0, NF) K-, [NF, 2NF) Q~, [2NF, 3NF) W, then A_qk,
    // gamma and dO. load_part issues entries [LO, HI); a chunk's loads go out in three parts
    // between the state pass's products (issued in one piece they stalled the wave for about half
    // of each chunk's time).
    static constexpr int NLD = 3 * NF + NA + 1 + ND;
    template <typename L, int LO, int HI>
    __device__ __forceinline__ void load_part(const float* sc, const TO* dO_, int64_t orow, int nrows_, int j0, int dv) {
        if (LO == 0) nrows = nrows_;
#pragma unroll
        for (int i = LO; i < (HI < NLD ? HI : NLD); ++i) {
            if (i < 3 * NF) {
                const int u = i % NF, f = i / NF;
                const int off = 4 * ((int)threadIdx.x + kT * u);
                const f32x4 x = *reinterpret_cast<const f32x4*>(sc + (f == 0 ? L::KB : (f == 1 ? L::QT : L::W)) + off);
                if (f == 0) kb[u] = x; else if (f == 1) qt[u] = x; else w[u] = x;
            } else if (i < 3 * NF + NA) {
                const int u = i - 3 * NF;
                aqk[u] = *reinterpret_cast<const f32x4*>(sc + L::AQK + 4 * ((int)threadIdx.x + kT * u));
            } else if (i == 3 * NF + NA) {
                if ((int)threadIdx.x < DK / 4) gam = *reinterpret_cast<const f32x4*>(sc + L::GAM + threadIdx.x * 4);
            } else {
                // rows past the end read the last row (no branch, so no wait); they are zeroed when
                // the raw values go to LDS, so nothing here waits for the loads to land
                const int u = i - (3 * NF + NA + 1);
                const int e = threadIdx.x + u * kT, t = e / NB, j = e % NB, tr = t < nrows_ ? t : nrows_ - 1;
                dO[u] = dO_[(orow + tr) * dv + j0 + j];
            }
        }
    }
    template <typename L>
    __device__ __forceinline__ void load(const float* sc, const TO* dO_, int64_t orow, int nrows_, int j0, int dv) {
        load_part<L, 0, NLD>(sc, dO_, orow, nrows_, j0, dv);
    }

    template <typename SS>
    __device__ __forceinline__ void store(SS& sm) const {
#pragma unroll
        for (int u = 0; u < NF; ++u) {
            const int e = (int)threadIdx.x + kT * u, r = e / (DK / 4), c = 4 * (e % (DK / 4));
            *reinterpret_cast<f32x4*>(&sm.KB[r][c]) = kb[u];
            *reinterpret_cast<f32x4*>(&sm.QT[r][c]) = qt[u];
            *reinterpret_cast<f32x4*>(&sm.WN[r][c]) = -w[u];
        }
#pragma unroll
        for (int u = 0; u < NA; ++u) {
            const int e = (int)threadIdx.x + kT * u;
            *reinterpret_cast<f32x4*>(&sm.AQ[e / (kC / 4)][4 * (e % (kC / 4))]) = aqk[u];
        }
        if ((int)threadIdx.x < DK / 4) *reinterpret_cast<f32x4*>(&sm.gam[threadIdx.x * 4]) = gam;
#pragma unroll
        for (int u = 0; u < ND; ++u) {
            const int e = threadIdx.x + u * kT;
            sm.dOT[e % NB][e / NB] = e / NB < nrows ? ldo(&dO[u], 0) : 0.f;
        }
    }
};

template <int DK, int DV, typename TO, int NB>
__global__ __launch_bounds__(kT) void bwd_state_kernel(BwdArgs a) {
    typedef BwdLayout<DK, DV> L;
    typedef StateSmem<DK, NB> SS;
    typedef StateFetch<DK, TO, NB> F;
    constexpr int RT = DK / 64;   // 16-row tiles of Gx per wave
    constexpr int CT = NB / 16;   // 16-column tiles of the block
    static_assert(DV % NB == 0 && DK % 64 == 0 && (kC * DK / 4) % kT == 0 && (kC * kC / 4) % kT == 0, "state tiles");
    extern __shared__ __align__(16) unsigned char smem_raw[];
    SS& sm = *reinterpret_cast<SS*>(smem_raw);
    const int nblk = DV / NB;
    // the column blocks of a lane run on one XCD (block index = lane mod 8 there) when the lane
    // count allows, so they share the lane's factors in that XCD's L2
    int64_t lane, cb;
    if (a.lanes % 8 == 0) {
        const int64_t bid = blockIdx.x;
        cb = (bid >> 3) % nblk;
        lane = (bid / (8 * nblk)) * 8 + (bid & 7);
    } else {
        lane = blockIdx.x / nblk;
        cb = blockIdx.x % nblk;
    }
    const int j0 = (int)cb * NB;
    const TO* dO = (const TO*)a.dO;
    const int wv = threadIdx.x >> 6, lr = threadIdx.x & 15, lg = (threadIdx.x >> 4) & 3;
    // Gx accumulators: gx[rt][ct][i] = Gx[gr0 + 16 rt + 4 lg + i][16 ct + lr]
    const int gr0 = wv * (DK / 4);
    f32x4 gx[RT][CT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ch = gr0 + 16 * rt + 4 * lg + i, j = 16 * ct + lr;
                gx[rt][ct][i] = a.dST ? a.dST[(lane * DK + ch) * DV + j0 + j] : 0.f;
            }
    auto put_gxt = [&]() {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
                *reinterpret_cast<f32x4*>(&sm.GxT[16 * ct + lr][gr0 + 16 * rt + 4 * lg]) = gx[rt][ct];
    };
    put_gxt();
    auto chunk_rows = [&](int64_t c) { return (int)(a.T - c * kC < kC ? a.T - c * kC : kC); };
    F f;
    {
        const int64_t c = a.nchunks - 1;
        f.template load<L>(a.prep + (lane * a.nchunks + c) * L::PREP, dO, lane * a.T + c * kC, chunk_rows(c), j0, DV);
    }
    for (int64_t c = a.nchunks - 1; c >= 0; --c) {
        float* gst = a.gst + (lane * a.nchunks + c) * (int64_t)(DK * DV);
        float* dvt = a.dvt + (lane * a.nchunks + c) * (int64_t)(kC * DV);
        lds_barrier();   // the previous chunk is done with every staged array; its Gx^T is in place
        f.store(sm);
        // the state gradient entering this chunk (from its end), for the gradient kernel
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    gst[(gr0 + 16 * rt + 4 * lg + i) * DV + j0 + 16 * ct + lr] = gx[rt][ct][i];
        // the next chunk's operands travel while this one computes, in three parts: a quarter before
        // barrier B, a quarter after the dV~ products, half after the first of the four blocks of
        // the Gx products (8K backward: 2.134 ms; half after all of them 2.150, half before them
        // 2.170, a quarter before and a quarter after 2.159; thirds, an eighth / eighth / rest and
        // nothing / quarter / rest were slower still)
        constexpr int P1 = F::NLD / 4, P2 = F::NLD / 2;
        const float* nsc = a.prep + (lane * a.nchunks + c - 1) * L::PREP;
        const int64_t norow = lane * a.T + (c - 1) * kC;
        const int nrows_next = c > 0 ? chunk_rows(c - 1) : 1;
        if (c > 0) f.template load_part<L, 0, P1>(nsc, dO, norow, nrows_next, j0, DV);
        lds_barrier();
        // dV~ rows 16 wv .. 16 wv + 15 = K- Gx + A_qk^T dO (A_qk^T[t][s] = 0 for s < t)
        {
            f32x4 dv[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) dv[ct] = kZero4f();
            const int t0 = 16 * wv;
            for (int kb = 0; kb < DK; kb += 16) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(&sm.KB[t0 + lr][kb + 4 * lg]);
                f32x4 y[CT];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) y[ct] = *reinterpret_cast<const f32x4*>(&sm.GxT[16 * ct + lr][kb + 4 * lg]);
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) dv[ct] = mfma4(x[q], y[ct][q], dv[ct]);
            }
            for (int kb = t0; kb < kC; kb += 16) {
                f32x4 x;
#pragma unroll
                for (int q = 0; q < 4; ++q) x[q] = sm.AQ[kb + 4 * lg + q][t0 + lr];
                f32x4 y[CT];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) y[ct] = *reinterpret_cast<const f32x4*>(&sm.dOT[16 * ct + lr][kb + 4 * lg]);
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) dv[ct] = mfma4(x[q], y[ct][q], dv[ct]);
            }
            if (c > 0) f.template load_part<L, P1, P2>(nsc, dO, norow, nrows_next, j0, DV);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                *reinterpret_cast<f32x4*>(&sm.dVT[16 * ct + lr][t0 + 4 * lg]) = dv[ct];
#pragma unroll
                for (int i = 0; i < 4; ++i) dvt[(t0 + 4 * lg + i) * DV + j0 + 16 * ct + lr] = dv[ct][i];
            }
        }
        lds_barrier();
        // Gx <- Diag(gamma) Gx + Q~^T dO - W^T dV~
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const f32x4 g4 = *reinterpret_cast<const f32x4*>(&sm.gam[gr0 + 16 * rt + 4 * lg]);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) gx[rt][ct] *= g4;
        }
#pragma unroll
        for (int kb = 0; kb < kC; kb += 16) {
            f32x4 xq[RT], xw[RT];
            if (kb == 16 && c > 0) f.template load_part<L, P2, F::NLD>(nsc, dO, norow, nrows_next, j0, DV);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    xq[rt][q] = sm.QT[kb + 4 * lg + q][gr0 + 16 * rt + lr];
                    xw[rt][q] = sm.WN[kb + 4 * lg + q][gr0 + 16 * rt + lr];
                }
            }
            f32x4 o[CT], v[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                o[ct] = *reinterpret_cast<const f32x4*>(&sm.dOT[16 * ct + lr][kb + 4 * lg]);
                v[ct] = *reinterpret_cast<const f32x4*>(&sm.dVT[16 * ct + lr][kb + 4 * lg]);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) gx[rt][ct] = mfma4(xq[rt][q], o[ct][q], gx[rt][ct]);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) gx[rt][ct] = mfma4(xw[rt][q], v[ct][q], gx[rt][ct]);
                }
        }
        put_gxt();   // nothing reads Gx^T between the dV~ products above and the next chunk's
    }
    if (a.dS0)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    a.dS0[(lane * DK + gr0 + 16 * rt + 4 * lg + i) * DV + j0 + 16 * ct + lr] = gx[rt][ct][i];
}

// Gradient kernel LDS arena, reused by phase (offsets in floats; rows padded by 4 floats):
//   phase 1 (twice, one half of the value columns each): S_h, Gx_h [DK][NH+4], W [64][DK+4],
//           dO_h, dV~_h, V~_h [64][NH+4]
//   phase 2: dA_kk [64][68] at 0 (kept), then T^T [64][68], dW^T [DK][68], dV~^T [DV][68] for
//           dX = T^T [dW | dV~], then dX_K [64][DK+4], dX_V [64][DV+4], W, U for dA_kk
//   phase 3: dA_kk, dA_qk [64][68], K, Q, G [64][DK+4] for the pairwise terms; then dG over Q
template <int DK, int DV>
struct GradArena {
    static constexpr int NH = DV / 2, LH = NH + 4, LK = DK + 4, LV = DV + 4, LA = kC + 4;
    // phase 1
    static constexpr int P1_S = 0, P1_GX = P1_S + DK * LH, P1_W = P1_GX + DK * LH, P1_DO = P1_W + kC * LK,
                         P1_DVT = P1_DO + kC * LH, P1_VT = P1_DVT + kC * LH, P1_END = P1_VT + kC * LH;
    // phase 2 / 3
    static constexpr int AKK = 0, P2_T = AKK + kC * LA, P2_DW = P2_T + kC * LA, P2_DVT = P2_DW + DK * LA,
                         P2A_END = P2_DVT + DV * LA;
    static constexpr int P2_XK = AKK + kC * LA, P2_XV = P2_XK + kC * LK, P2_W = P2_XV + kC * LV,
                         P2_U = P2_W + kC * LK, P2B_END = P2_U + kC * LV;
    static constexpr int AQK = AKK + kC * LA, P3_K = AQK + kC * LA, P3_Q = P3_K + kC * LK, P3_G = P3_Q + kC * LK,
                         P3_END = P3_G + kC * LK;
    static constexpr int SMALL = (P1_END > P2B_END ? (P1_END > P3_END ? P1_END : P3_END)
                                                   : (P2B_END > P3_END ? P2B_END : P3_END));
    // BETA: beta per row; DLGAM: gamma dgamma per channel; DB: dX_V . V per row from each of the
    // two waves that share a row block (summed in that order); DLP: each wave's sum of dK- K- over
    // its 8 rows per channel (summed in wave order). Fixed-order sums: the gradients are the same
    // bit for bit from run to run.
    static constexpr int BETA = SMALL, DLGAM = BETA + kC, DB = DLGAM + DK, DLP = DB + 2 * kC,
                         TOTAL = DLP + (kTG / 64) * DK;
    static_assert(P2A_END <= TOTAL && TOTAL * 4 <= 160 * 1024, "arena fits the LDS of a CU");
};

template <int DK, int DV, typename TO>
__global__ __launch_bounds__(kTG) void bwd_grad_kernel(BwdArgs a) {
    typedef BwdLayout<DK, DV> L;
    typedef GradArena<DK, DV> A;
    constexpr int NH = A::NH, LH = A::LH, LK = A::LK, LV = A::LV, LA = A::LA;
    constexpr int NGR = kTG / kC;     // threads per row
    constexpr int CG = DK / NGR;      // channels per thread: thread = (row t, channel group)
    extern __shared__ __align__(16) unsigned char smem_raw[];
    float* ar = reinterpret_cast<float*>(smem_raw);
    float* beta = ar + A::BETA;
    float* dlgam = ar + A::DLGAM;     // gamma dgamma per channel (joins row 63 of dG)
    float* sdb = ar + A::DB;          // [2][kC] dX_V . V per row, by column half (joins dbeta)
    float* dlp = ar + A::DLP;         // [waves][DK] per-wave sums of dK- K- (join row 63 of dG)
    const int64_t lane = blockIdx.x / a.nchunks, c = blockIdx.x % a.nchunks;
    const int64_t row0 = lane * a.T + c * kC;
    const int nrows = (int)(a.T - c * kC < kC ? a.T - c * kC : kC);
    const float* sc = a.prep + (int64_t)blockIdx.x * L::PREP;
    const float* Gx = a.gst + (int64_t)blockIdx.x * (DK * DV);
    const float* dVt = a.dvt + (int64_t)blockIdx.x * (kC * DV);
    // entry state: S0 (or zero) for the first chunk, else the forward's state after chunk c - 1
    const float* S = c == 0 ? (a.S0 ? a.S0 + lane * (int64_t)(DK * DV) : nullptr)
                            : a.ckpt + (lane * a.ck_stride + c - 1) * (int64_t)(DK * DV);
    const TO* dO = (const TO*)a.dO;
    const int tid = threadIdx.x;
    const int t = tid / NGR;                 // row of this thread in the (row, group) tiles
    const int gi = tid % NGR;
    const int c0 = gi * CG;                  // its channels
    // beta of the chunk's rows, loaded ahead of the first tiles and written to LDS after them by
    // every thread (thread tid writes row tid mod 64; the eight writers of a row store the same
    // value). A store under a branch would take the load into the branch with it, where the load
    // is waited for at once, ahead of the tile loads.
    const int brow = tid & (kC - 1);
    const bf16_t beta_raw = ((const bf16_t*)a.beta)[row0 + (brow < nrows ? brow : nrows - 1)];

    // ---------------- phase 1: V~ = U - W S, and the products over the value columns ----------
    // fp32 16x16x4 MFMA tiles (lane l = lr + 16 lg supplies row / column lr at k = lg; the k
    // values of a block of 16 are kb + 4 lg + q at step q, on both operands). Wave w owns rows
    // t0 = 16 (w mod 4) of every product and a quarter of the columns given by w / 4:
    //   V~_h     cols vb + 16 ct (NVT tiles)    dQ~, dW, dK- cols cm + 16 ct (NCT tiles)
    //   dA_qk    cols sb + 16 ct (2 tiles)
    // An accumulator tile holds rows t0 + 4 lg + i, i = 0..3, of column lr.
    constexpr int NCT = DK / 32, NVT = NH / 32;
    const int wv = tid >> 6, lr = tid & 15, lg = (tid >> 4) & 3;
    const int t0 = 16 * (wv & 3), vb = (NH / 2) * (wv >> 2), cm = (DK / 2) * (wv >> 2), sb = 32 * (wv >> 2);
    f32x4 mq[NCT], mw[NCT], mk[NCT], mqk[2];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) { mq[ct] = kZero4f(); mw[ct] = kZero4f(); mk[ct] = kZero4f(); }
    mqk[0] = kZero4f();
    mqk[1] = kZero4f();
    float dgam = 0.f;
    float* sS = ar + A::P1_S;
    float* sGx = ar + A::P1_GX;
    float* sW = ar + A::P1_W;
    float* sdO = ar + A::P1_DO;
    float* sdVt = ar + A::P1_DVT;
    float* sVt = ar + A::P1_VT;
    // operands of each phase are loaded into registers during the phase before it
    F32Tile<kC, DK, kTG> tw;
    F32Tile<DK, NH, kTG> ts, tgx;
    F32Tile<kC, NH, kTG> tdv;
    InTile<kC, NH, kTG, TO> tdo;
    F32TileT<kC, kC, kTG> tT;
    F32TileT<kC, DV, kTG> tdv2;
    const float* Ssrc = S ? S : Gx;   // a stand-in of the same shape when there is no entry state
    // U_h in the V~_h tile layout (V~ = U - W S), loaded with the half's tiles
    f32x4 uin[NVT];
    auto load_uin = [&](int jh) {
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) uin[ct][i] = sc[L::U + (t0 + 4 * lg + i) * DV + jh + vb + 16 * ct + lr];
    };
    tw.load(sc + L::W, DK);
    ts.load(Ssrc, DV);
    tgx.load(Gx, DV);
    tdv.load(dVt, DV);
    tdo.load(dO + row0 * DV, DV, nrows);
    load_uin(0);
    tw.store(sW, LK);
    beta[brow] = brow < nrows ? bf16_bits_to_f32(beta_raw) : 0.f;
    // the two halves are written out (no loop) so that the registers a prefetch fills are the ones
    // the next half reads, with no copies that would wait for the loads
    auto half = [&](auto hc) {
        constexpr int h = decltype(hc)::value;
        ts.store(sS, LH, S != nullptr);
        tgx.store(sGx, LH);
        tdv.store(sdVt, LH);
        tdo.store(sdO, LH);
        f32x4 acc[NVT];
#pragma unroll
        for (int ct = 0; ct < NVT; ++ct) acc[ct] = kZero4f();
        const f32x4 u0 = uin[0], u1 = uin[NVT - 1];
        lds_barrier();
        if constexpr (h == 0) {
            ts.load(Ssrc + NH, DV);
            tgx.load(Gx + NH, DV);
            tdv.load(dVt + NH, DV);
            tdo.load(dO + row0 * DV + NH, DV, nrows);
            load_uin(NH);
        } else {
            tT.load(sc + L::T, kC);
            tdv2.load(dVt, DV);
        }
        {   // W S_h for rows t0 .., columns vb + 16 ct; S_h's column is strided in LDS (4 reads)
#pragma unroll 2
            for (int kb = 0; kb < DK; kb += 16) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(sW + (t0 + lr) * LK + kb + 4 * lg);
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int ct = 0; ct < NVT; ++ct)
                        acc[ct] = mfma4(x[q], sS[(kb + 4 * lg + q) * LH + vb + 16 * ct + lr], acc[ct]);
            }
#pragma unroll
            for (int ct = 0; ct < NVT; ++ct) {
                const f32x4 uu = ct == 0 ? u0 : u1;
#pragma unroll
                for (int i = 0; i < 4; ++i) sVt[(t0 + 4 * lg + i) * LH + vb + 16 * ct + lr] = uu[i] - acc[ct][i];
            }
        }
        if (tid < DK) {
            float sacc = 0.f;
#pragma unroll 4
            for (int j = 0; j < NH; ++j) sacc += sGx[tid * LH + j] * sS[tid * LH + j];
            dgam += sacc;
        }
        lds_barrier();
        // dQ~ += dO S^T, dW += dV~ S^T (negated when stored), dK- += V~ Gx^T, dA_qk += dO V~^T
#pragma unroll 1
        for (int kb = 0; kb < NH; kb += 16) {
            const f32x4 xo = *reinterpret_cast<const f32x4*>(sdO + (t0 + lr) * LH + kb + 4 * lg);
            const f32x4 xd = *reinterpret_cast<const f32x4*>(sdVt + (t0 + lr) * LH + kb + 4 * lg);
            const f32x4 xv = *reinterpret_cast<const f32x4*>(sVt + (t0 + lr) * LH + kb + 4 * lg);
            f32x4 ys[NCT], yg[NCT], yv[2];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                ys[ct] = *reinterpret_cast<const f32x4*>(sS + (cm + 16 * ct + lr) * LH + kb + 4 * lg);
                yg[ct] = *reinterpret_cast<const f32x4*>(sGx + (cm + 16 * ct + lr) * LH + kb + 4 * lg);
            }
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) yv[ct] = *reinterpret_cast<const f32x4*>(sVt + (sb + 16 * ct + lr) * LH + kb + 4 * lg);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    mq[ct] = mfma4(xo[q], ys[ct][q], mq[ct]);
                    mw[ct] = mfma4(xd[q], ys[ct][q], mw[ct]);
                    mk[ct] = mfma4(xv[q], yg[ct][q], mk[ct]);
                }
                mqk[0] = mfma4(xo[q], yv[0][q], mqk[0]);
                mqk[1] = mfma4(xo[q], yv[1][q], mqk[1]);
            }
        }
        lds_barrier();
    };
    half(IntC<0>{});
    half(IntC<1>{});
    if (tid < DK) dlgam[tid] = sc[L::GAM + tid] * dgam;
    // dQ~ and dK- go from the tile layout to the (row t, channels c0 ..) layout of phase 3
    // through the free phase-1 space
    float accQ[CG], accK[CG];
    {
        float* xq = ar;
        float* xk = ar + kC * LK;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                xq[(t0 + 4 * lg + i) * LK + cm + 16 * ct + lr] = mq[ct][i];
                xk[(t0 + 4 * lg + i) * LK + cm + 16 * ct + lr] = mk[ct][i];
            }
        lds_barrier();
#pragma unroll
        for (int u = 0; u < CG; u += 4) {
            const f32x4 q4 = *reinterpret_cast<const f32x4*>(xq + t * LK + c0 + u);
            const f32x4 k4 = *reinterpret_cast<const f32x4*>(xk + t * LK + c0 + u);
#pragma unroll
            for (int e = 0; e < 4; ++e) { accQ[u + e] = q4[e]; accK[u + e] = k4[e]; }
        }
        lds_barrier();
    }

    // ---------------- phase 2: [dX_K | dX_V] = T^T [dW | dV~], then dA_kk ---------------------
    // MFMA tiles as in phase 1, every operand k-contiguous in LDS: T^T [t][m], dW^T [ch][m] and
    // dV~^T [j][m] for dX; dX_K [i][ch], dX_V [i][jj], W [j][ch], U [j][jj] for dA_kk
    constexpr int NXV = DV / 32;   // dX_V column tiles per wave
    const int xb = (DV / 2) * (wv >> 2);
    float* sAkk = ar + A::AKK;
    float* sTT = ar + A::P2_T;
    float* sdWT = ar + A::P2_DW;
    float* sdVT = ar + A::P2_DVT;
    tT.store_t(sTT, LA);
    tdv2.store_t(sdVT, LA);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) *reinterpret_cast<f32x4*>(sdWT + (cm + 16 * ct + lr) * LA + t0 + 4 * lg) = -mw[ct];
    lds_barrier();
    F32Tile<kC, DK, kTG> tw2;
    F32Tile<kC, DV, kTG> tu;
    tw2.load(sc + L::W, DK);
    tu.load(sc + L::U, DV);
    f32x4 mxk[NCT], mxv[NXV];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) mxk[ct] = kZero4f();
#pragma unroll
    for (int ct = 0; ct < NXV; ++ct) mxv[ct] = kZero4f();
    // V of this wave's dX_V entries, for dbeta: loaded before the products (rows past the end read
    // the last row; no branch, so nothing waits for them until they are used)
    bf16_t vdb[NXV][4];
#pragma unroll
    for (int ct = 0; ct < NXV; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = t0 + 4 * lg + i, rr = r < nrows ? r : nrows - 1;
            vdb[ct][i] = ((const bf16_t*)a.v)[(row0 + rr) * DV + xb + 16 * ct + lr];
        }
    for (int kb = t0; kb < kC; kb += 16) {   // T^T[t][m] = 0 for m < t
        const f32x4 x = *reinterpret_cast<const f32x4*>(sTT + (t0 + lr) * LA + kb + 4 * lg);
        f32x4 yw[NCT], yv[NXV];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) yw[ct] = *reinterpret_cast<const f32x4*>(sdWT + (cm + 16 * ct + lr) * LA + kb + 4 * lg);
#pragma unroll
        for (int ct = 0; ct < NXV; ++ct) yv[ct] = *reinterpret_cast<const f32x4*>(sdVT + (xb + 16 * ct + lr) * LA + kb + 4 * lg);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) mxk[ct] = mfma4(x[q], yw[ct][q], mxk[ct]);
#pragma unroll
            for (int ct = 0; ct < NXV; ++ct) mxv[ct] = mfma4(x[q], yv[ct][q], mxv[ct]);
        }
    }
    {   // dv = beta dX_V; dbeta gets dX_V . V (row sums over the 16 lanes of a tile, then one LDS
        // slot per row and column half: waves w and w + 4 share rows t0 .. t0 + 15)
        float pb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ct = 0; ct < NXV; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = t0 + 4 * lg + i, j = xb + 16 * ct + lr;
                if (r < nrows) {
                    a.dv_[(row0 + r) * DV + j] = beta[r] * mxv[ct][i];
                    pb[i] += mxv[ct][i] * bf16_bits_to_f32(vdb[ct][i]);
                }
            }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int m = 1; m < 16; m <<= 1) pb[i] += __shfl_xor(pb[i], m);
            if (lr == 0) sdb[(wv >> 2) * kC + t0 + 4 * lg + i] = pb[i];
        }
    }
    lds_barrier();   // T^T, dW^T, dV~^T are done; the dA_kk operands take their place
    float* sXK = ar + A::P2_XK;
    float* sXV = ar + A::P2_XV;
    float* sW2 = ar + A::P2_W;
    float* sU = ar + A::P2_U;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) sXK[(t0 + 4 * lg + i) * LK + cm + 16 * ct + lr] = mxk[ct][i];
#pragma unroll
    for (int ct = 0; ct < NXV; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) sXV[(t0 + 4 * lg + i) * LV + xb + 16 * ct + lr] = mxv[ct][i];
    tw2.store(sW2, LK);
    tu.store(sU, LV);
    lds_barrier();
    InTile<kC, DK, kTG, bf16_t> tk, tq, tg;
    tk.load((const bf16_t*)a.k + row0 * DK, DK, nrows);
    tq.load((const bf16_t*)a.q + row0 * DK, DK, nrows);
    tg.load((const bf16_t*)a.la + row0 * DK, DK, nrows);
    float xk[CG];   // dX_K in the (row t, channels c0 ..) layout of phase 3
#pragma unroll
    for (int u = 0; u < CG; u += 4) {
        const f32x4 x4 = *reinterpret_cast<const f32x4*>(sXK + t * LK + c0 + u);
#pragma unroll
        for (int e = 0; e < 4; ++e) xk[u + e] = x4[e];
    }
    {   // dA_kk = -(dX_K W^T + dX_V U^T) below the diagonal: the ten 16 x 16 tiles (R, C), C <= R,
        // as tile codes 4 R + C, one per wave and a second on waves 0 and 1 (three tiles per SIMD
        // at most: waves w and w + 4 share one); waves 2-7 also zero one tile above the diagonal
        // each. The tiles of a wave run interleaved, each one accumulation chain in step order.
        const int codeA = (int)((0xEC84D950u >> (4 * wv)) & 15u), codeB = (int)((0xAFu >> (4 * wv)) & 15u);
        const bool two = wv < 2;
        const int rA = 16 * (codeA >> 2), cA = 16 * (codeA & 3), rB = 16 * (codeB >> 2), cB = 16 * (codeB & 3);
        f32x4 akA = kZero4f(), akB = kZero4f();
#pragma unroll 2
        for (int kb = 0; kb < DK; kb += 16) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(sXK + (rA + lr) * LK + kb + 4 * lg);
            const f32x4 y = *reinterpret_cast<const f32x4*>(sW2 + (cA + lr) * LK + kb + 4 * lg);
#pragma unroll
            for (int q = 0; q < 4; ++q) akA = mfma4(x[q], y[q], akA);
            if (two) {
                const f32x4 xb = *reinterpret_cast<const f32x4*>(sXK + (rB + lr) * LK + kb + 4 * lg);
                const f32x4 yb = *reinterpret_cast<const f32x4*>(sW2 + (cB + lr) * LK + kb + 4 * lg);
#pragma unroll
                for (int q = 0; q < 4; ++q) akB = mfma4(xb[q], yb[q], akB);
            }
        }
#pragma unroll 2
        for (int kb = 0; kb < DV; kb += 16) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(sXV + (rA + lr) * LV + kb + 4 * lg);
            const f32x4 y = *reinterpret_cast<const f32x4*>(sU + (cA + lr) * LV + kb + 4 * lg);
#pragma unroll
            for (int q = 0; q < 4; ++q) akA = mfma4(x[q], y[q], akA);
            if (two) {
                const f32x4 xb = *reinterpret_cast<const f32x4*>(sXV + (rB + lr) * LV + kb + 4 * lg);
                const f32x4 yb = *reinterpret_cast<const f32x4*>(sU + (cB + lr) * LV + kb + 4 * lg);
#pragma unroll
                for (int q = 0; q < 4; ++q) akB = mfma4(xb[q], yb[q], akB);
            }
        }
        lds_barrier();   // everyone has read dX / W / U before dA_qk and K, Q, G land on them
        const int codeZ = (int)((0xB7632100u >> (4 * wv)) & 15u), rZ = 16 * (codeZ >> 2), cZ = 16 * (codeZ & 3);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * lg + e, col = lr;
            sAkk[(rA + r) * LA + cA + col] = cA + col < rA + r ? -akA[e] : 0.f;
            if (two) sAkk[(rB + r) * LA + cB + col] = cB + col < rB + r ? -akB[e] : 0.f;
            else sAkk[(rZ + r) * LA + cZ + col] = 0.f;
        }
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = t0 + 4 * lg + e, col = sb + 16 * ct + lr;
                ar[A::AQK + r * LA + col] = col <= r ? mqk[ct][e] : 0.f;
            }
    }

    // ---------------- phase 3: decay factors, pairwise terms, reverse cumsum -----------------
    float* sK = ar + A::P3_K;
    float* sQ = ar + A::P3_Q;
    float* sG = ar + A::P3_G;
    const float* sAqk = ar + A::AQK;
    tk.store(sK, LK);
    tq.store(sQ, LK);
    tg.store(sG, LK);
    lds_barrier();
    for (int ch = tid; ch < DK; ch += kTG) {   // G = inclusive cumsum of log_alpha down the rows
        float acc = 0.f;
        for (int tt = 0; tt < kC; ++tt) { acc += sG[tt * LK + ch]; sG[tt * LK + ch] = acc; }
    }
    lds_barrier();
    float dq[CG], dk[CG], dG[CG];
    float dbeta = 0.f;
    const float bt = beta[t];
#pragma unroll
    for (int u = 0; u < CG; u += 4) {
        const f32x4 g4 = *reinterpret_cast<const f32x4*>(sG + t * LK + c0 + u);
        const f32x4 k4 = *reinterpret_cast<const f32x4*>(sK + t * LK + c0 + u);
        const f32x4 q4 = *reinterpret_cast<const f32x4*>(sQ + t * LK + c0 + u);
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(sG + (kC - 1) * LK + c0 + u);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float eg = fexp(g4[e]);
            const float kbf = fexp(l4[e] - g4[e]);   // K- = K kbf
            dq[u + e] = accQ[u + e] * eg;
            dk[u + e] = accK[u + e] * kbf + bt * xk[u + e] * eg;
            dG[u + e] = accQ[u + e] * q4[e] * eg - accK[u + e] * k4[e] * kbf + bt * xk[u + e] * k4[e] * eg;
            dbeta += xk[u + e] * k4[e] * eg;
            accK[u + e] *= k4[e] * kbf;   // accK is not needed past this point: it becomes dK- K-
        }
    }
    // sum of dK- K- down the rows: over the wave's 8 rows (lanes 8 apart) here, into the wave's
    // own LDS slot per channel; the eight wave sums are added in wave order where row 63 of dG
    // takes them
#pragma unroll
    for (int u = 0; u < CG; ++u) {
        float v = accK[u];
        v += __shfl_xor(v, 8);
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if ((tid & 63) < NGR) dlp[wv * DK + c0 + u] = v;
    }
    // pairwise terms, per channel c (E_ij = exp(G_i - G_j), i >= j):
    //   row sums     rq = sum_{j<=t} A_qk[t][j] K_j E_tj,   rk = sum_{j<t} A_kk[t][j] K_j E_tj
    //   column sums  cc = sum_{i>=t} (A_qk[i][t] Q_i + beta_i A_kk[i][t] K_i) E_it
    // then dq += rq, dk += beta_t rk + cc, dG += Q_t rq + beta_t K_t rk - K_t cc and
    // dbeta += K_t . rk, all by 16-row blocks on the fp32 MFMA below.
    {   // By 16-row blocks, with E split at a reference row r. Wave w takes channel tile ct (16
        // channels, column lr of its tiles); with DK = 128 every wave does both kinds of job, with
        // DK = 64 waves 0-3 the row blocks and 4-7 the column blocks.
        //   rows of block I = 0..3, r = 16 I:  [Rq | Rk] = exp(G_i - G_r) (A[I rows, j < r + 16] Khat_r),
        //                                      Khat_r[j] = K_j exp(G_r - G_j)
        //   rows of block J = 0..2, r = 16 (J + 1), the later blocks:
        //       Cc = exp(G_r - G_t) (A_qk[i >= r, t]^T Qchk_r + (beta A_kk)[i >= r, t]^T Kchk_r),
        //       Qchk_r[i] = Q_i exp(G_i - G_r), Kchk_r[i] = K_i exp(G_i - G_r)
        //   rows of block J = 0..3, r = 16 J, the block itself: the same with i in [r, r + 16).
        // Off the diagonal both factors are <= 1. Inside a diagonal block one of them is >= 1 but at
        // most e^{15 * 5}; the entries of A above the diagonal, whose products it does not bound,
        // are zero in LDS.
        constexpr int NCTc = DK / 16;
        const bool rows_job = NCTc == 8 || wv < 4, cols_job = NCTc == 8 || wv >= 4;
        const int ch = 16 * (wv % NCTc) + lr;
        f32x4 mrq[4], mrk[4], mcc[3], mcd[4];
#pragma unroll
        for (int I = 0; I <= 3; ++I) {
            mrq[I] = kZero4f();
            mrk[I] = kZero4f();
            if (!rows_job) continue;
            const int r = 16 * I;
            const float gr = sG[r * LK + ch];
#pragma unroll 1
            for (int kb = 0; kb <= r; kb += 16) {
                const f32x4 xq = *reinterpret_cast<const f32x4*>(sAqk + (r + lr) * LA + kb + 4 * lg);
                const f32x4 xk = *reinterpret_cast<const f32x4*>(sAkk + (r + lr) * LA + kb + 4 * lg);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int j = kb + 4 * lg + q;
                    const float bj = sK[j * LK + ch] * fexp(gr - sG[j * LK + ch]);
                    mrq[I] = mfma4(xq[q], bj, mrq[I]);
                    mrk[I] = mfma4(xk[q], bj, mrk[I]);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float f = fexp(sG[(r + 4 * lg + e) * LK + ch] - gr);
                mrq[I][e] *= f;
                mrk[I][e] *= f;
            }
        }
#pragma unroll
        for (int J = 0; J <= 2; ++J) {
            mcc[J] = kZero4f();
            if (!cols_job) continue;
            const int r = 16 * (J + 1), tc = 16 * J + lr;
            const float gr = sG[r * LK + ch];
#pragma unroll 1
            for (int kb = r; kb < kC; kb += 16) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int i = kb + 4 * lg + q;
                    const float f = fexp(sG[i * LK + ch] - gr);
                    mcc[J] = mfma4(sAqk[i * LA + tc], sQ[i * LK + ch] * f, mcc[J]);
                    mcc[J] = mfma4(beta[i] * sAkk[i * LA + tc], sK[i * LK + ch] * f, mcc[J]);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) mcc[J][e] *= fexp(gr - sG[(16 * J + 4 * lg + e) * LK + ch]);
        }
#pragma unroll
        for (int J = 0; J <= 3; ++J) {   // the diagonal blocks of the column sums
            mcd[J] = kZero4f();
            if (!cols_job) continue;
            const int r = 16 * J, tc = r + lr;
            const float gr = sG[r * LK + ch];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int i = r + 4 * lg + q;
                const float f = fexp(sG[i * LK + ch] - gr);
                mcd[J] = mfma4(sAqk[i * LA + tc], sQ[i * LK + ch] * f, mcd[J]);
                mcd[J] = mfma4(beta[i] * sAkk[i * LA + tc], sK[i * LK + ch] * f, mcd[J]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) mcd[J][e] *= fexp(gr - sG[(r + 4 * lg + e) * LK + ch]);
        }
        // this thread's K_t and Q_t again (not kept in registers across the jobs above)
        float kt2[CG], qt2[CG];
#pragma unroll
        for (int u = 0; u < CG; u += 4) {
            const f32x4 k4 = *reinterpret_cast<const f32x4*>(sK + t * LK + c0 + u);
            const f32x4 q4 = *reinterpret_cast<const f32x4*>(sQ + t * LK + c0 + u);
#pragma unroll
            for (int e = 0; e < 4; ++e) { kt2[u + e] = k4[e]; qt2[u + e] = q4[e]; }
        }
        lds_barrier();   // every read of K, Q, G is done: they take the block results
#pragma unroll
        for (int I = 0; I <= 3; ++I)
            if (rows_job)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sK[(16 * I + 4 * lg + e) * LK + ch] = mrq[I][e];
                    sG[(16 * I + 4 * lg + e) * LK + ch] = mrk[I][e];
                }
#pragma unroll
        for (int J = 0; J <= 3; ++J)
            if (cols_job)
#pragma unroll
                for (int e = 0; e < 4; ++e) sQ[(16 * J + 4 * lg + e) * LK + ch] = (J <= 2 ? mcc[J][e] : 0.f) + mcd[J][e];
        lds_barrier();
        // the block results of this thread's row: rq, rk and cc of its 16 channels
#pragma unroll
        for (int u = 0; u < CG; u += 4) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(sK + t * LK + c0 + u);
            const f32x4 y = *reinterpret_cast<const f32x4*>(sG + t * LK + c0 + u);
            const f32x4 z = *reinterpret_cast<const f32x4*>(sQ + t * LK + c0 + u);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dq[u + e] += x[e];
                dk[u + e] += bt * y[e] + z[e];
                dG[u + e] += qt2[u + e] * x[e] + kt2[u + e] * (bt * y[e] - z[e]);
                dbeta += kt2[u + e] * y[e];
            }
        }
    }
    lds_barrier();
    // dG into LDS over Q, dgamma's share on row 63, then the reverse cumsum per channel. dq and dk
    // go to LDS too (over K and G: this thread's own row and channels, which only it has read),
    // so that all three leave in whole rows below.
#pragma unroll
    for (int u = 0; u < CG; ++u) {
        float last = 0.f;   // row 63: gamma dgamma + sum_t dK-_t K-_t, in a fixed order
        if (t == kC - 1) {
            last = dlgam[c0 + u];
#pragma unroll
            for (int w = 0; w < kTG / 64; ++w) last += dlp[w * DK + c0 + u];
        }
        sQ[t * LK + c0 + u] = dG[u] + last;
        sK[t * LK + c0 + u] = dq[u];
        sG[t * LK + c0 + u] = dk[u];
    }
    lds_barrier();
    for (int ch = tid; ch < DK; ch += kTG) {
        float acc = 0.f;
        for (int tt = kC - 1; tt >= 0; --tt) { acc += sQ[tt * LK + ch]; sQ[tt * LK + ch] = acc; }
    }
    lds_barrier();
#pragma unroll
    for (int m = 1; m < NGR; m <<= 1) dbeta += __shfl_xor(dbeta, m);
    if (t < nrows && gi == 0) a.dbeta[row0 + t] = dbeta + (sdb[t] + sdb[kC + t]);
    // dq, dk, dlog_alpha row by row: consecutive lanes write consecutive channels, so every store
    // instruction covers whole rows (thread-per-(row, channel group) stores scattered 4-byte words
    // over 8 rows and took about a fifth of the kernel's time)
#pragma unroll
    for (int v = 0; v < kC * DK / kTG; ++v) {
        const int f = tid + kTG * v, r = f / DK, ch = f % DK;
        if (r < nrows) {
            const int64_t o = (row0 + r) * DK + ch;
            a.dq[o] = sK[r * LK + ch];
            a.dk_[o] = sG[r * LK + ch];
            a.dla[o] = sQ[r * LK + ch];
        }
    }
}

template <int DK, int DV, typename TO>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t st) {
    const int64_t chunks = a.lanes * a.nchunks;
    if (chunks <= 0) return hipSuccess;
    // state pass: blocks of 16 value columns when blocks of 32 would leave compute units idle
    const bool narrow = a.lanes * (DV / 32) < compute_units(stream_device(st));
    const size_t prep_smem = sizeof(PrepSmem<DK, DV>);
    const size_t state_smem = narrow ? sizeof(StateSmem<DK, 16>) : sizeof(StateSmem<DK, 32>);
    const void* state_fn = narrow ? (const void*)bwd_state_kernel<DK, DV, TO, 16> : (const void*)bwd_state_kernel<DK, DV, TO, 32>;
    const size_t grad_smem = GradArena<DK, DV>::TOTAL * sizeof(float);
    // each kernel takes more than the default dynamic LDS limit: raise it, and stop at the first
    // error (a later launch would otherwise hide it)
    hipError_t e = hipFuncSetAttribute((const void*)bwd_prep_kernel<DK, DV>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)prep_smem);
    if (e == hipSuccess)
        e = hipFuncSetAttribute(state_fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)state_smem);
    if (e == hipSuccess)
        e = hipFuncSetAttribute((const void*)bwd_grad_kernel<DK, DV, TO>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)grad_smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_prep_kernel<DK, DV>), dim3((unsigned)chunks), dim3(kTP), prep_smem, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (narrow)
        hipLaunchKernelGGL((bwd_state_kernel<DK, DV, TO, 16>), dim3((unsigned)(a.lanes * (DV / 16))), dim3(kT),
                           state_smem, st, a);
    else
        hipLaunchKernelGGL((bwd_state_kernel<DK, DV, TO, 32>), dim3((unsigned)(a.lanes * (DV / 32))), dim3(kT),
                           state_smem, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_grad_kernel<DK, DV, TO>), dim3((unsigned)chunks), dim3(kTG), grad_smem, st, a);
    return hipGetLastError();
}

template <typename TO>
hipError_t launch_bwd_o(const BwdArgs& a, hipStream_t st) {
    if (a.dk == 128) return a.dv == 128 ? launch_bwd_t<128, 128, TO>(a, st) : launch_bwd_t<128, 64, TO>(a, st);
    return a.dv == 128 ? launch_bwd_t<64, 128, TO>(a, st) : launch_bwd_t<64, 64, TO>(a, st);
}

}  // namespace

size_t bwd_prep_floats(int64_t dk, int64_t dv) {
    return dk == 128 ? (dv == 128 ? BwdLayout<128, 128>::PREP : BwdLayout<128, 64>::PREP)
                     : (dv == 128 ? BwdLayout<64, 128>::PREP : BwdLayout<64, 64>::PREP);
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t st) {
    return a.dO_bf16 ? launch_bwd_o<bf16_t>(a, st) : launch_bwd_o<float>(a, st);
}

}  // namespace kda

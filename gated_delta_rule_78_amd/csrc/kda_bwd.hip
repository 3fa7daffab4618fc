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
//   bwd_state_kernel   one workgroup per (lane, 32 value columns), chunks in reverse: Gx of every
//                      chunk, dV~, and dS0
//   bwd_grad_kernel    one workgroup per chunk: dq, dk, dv, dlog_alpha, dbeta
// Plain fp32 loops over LDS / L2-resident scratch: correctness first, one workgroup per CU.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kC = 64;
constexpr int kT = 256;   // threads per workgroup

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
    // gradient-kernel scratch
    static constexpr int VT = 0;                      // [64][DV] V~
    static constexpr int DW = VT + kC * DV;           // [64][DK]
    static constexpr int XK = DW + kC * DK;           // [64][DK] dX_K
    static constexpr int XV = XK + kC * DK;           // [64][DV] dX_V
    static constexpr int GRAD = XV + kC * DV;
};

__device__ __forceinline__ float ldin(const bf16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
__device__ __forceinline__ float ldo(const bf16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
__device__ __forceinline__ float ldo(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// Rows [0, nrows) of the chunk into LDS as fp32 (zeros past the end), and the cumulative decay.
template <int DK>
__device__ void load_chunk_kgq(const BwdArgs& a, int64_t row0, int nrows, float (*Ks)[DK], float (*Qs)[DK],
                               float (*Gs)[DK], float* bs) {
    const bf16_t* k = (const bf16_t*)a.k;
    const bf16_t* q = (const bf16_t*)a.q;
    const bf16_t* la = (const bf16_t*)a.la;
    for (int e = threadIdx.x; e < kC * DK; e += kT) {
        const int t = e / DK, c = e % DK;
        const bool ok = t < nrows;
        Ks[t][c] = ok ? ldin(k, (row0 + t) * DK + c) : 0.f;
        Qs[t][c] = ok ? ldin(q, (row0 + t) * DK + c) : 0.f;
        Gs[t][c] = ok ? ldin(la, (row0 + t) * DK + c) : 0.f;
    }
    if (threadIdx.x < kC) bs[threadIdx.x] = threadIdx.x < nrows ? ldin((const bf16_t*)a.beta, row0 + threadIdx.x) : 0.f;
    __syncthreads();
    for (int c = threadIdx.x; c < DK; c += kT) {   // inclusive cumulative sum down the rows
        float acc = 0.f;
        for (int t = 0; t < kC; ++t) { acc += Gs[t][c]; Gs[t][c] = acc; }
    }
    __syncthreads();
}

template <int DK, int DV>
struct __align__(16) PrepSmem {
    float K[kC][DK], Q[kC][DK], G[kC][DK];
    float A[kC][kC + 1], T[kC][kC + 1];
    float beta[kC];
};

template <int DK, int DV>
__global__ __launch_bounds__(kT) void bwd_prep_kernel(BwdArgs a) {
    typedef BwdLayout<DK, DV> L;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    PrepSmem<DK, DV>& sm = *reinterpret_cast<PrepSmem<DK, DV>*>(smem_raw);
    const int64_t lane = blockIdx.x / a.nchunks, c = blockIdx.x % a.nchunks;
    const int64_t row0 = lane * a.T + c * kC;
    const int nrows = (int)(a.T - c * kC < kC ? a.T - c * kC : kC);
    float* sc = a.prep + (int64_t)blockIdx.x * L::PREP;
    load_chunk_kgq<DK>(a, row0, nrows, sm.K, sm.Q, sm.G, sm.beta);

    // A_kk (i > j, beta-scaled) and A_qk (i >= j)
    for (int e = threadIdx.x; e < kC * kC; e += kT) {
        const int i = e / kC, j = e % kC;
        float akk = 0.f, aqk = 0.f;
        if (j <= i) {
            for (int ch = 0; ch < DK; ++ch) {
                const float f = sm.K[j][ch] * fexp(sm.G[i][ch] - sm.G[j][ch]);
                akk += sm.K[i][ch] * f;
                aqk += sm.Q[i][ch] * f;
            }
        }
        sm.A[i][j] = j < i ? sm.beta[i] * akk : 0.f;
        sc[L::AQK + e] = aqk;
    }
    __syncthreads();
    // T = (I + A)^{-1}, unit lower triangular: one column per thread, rows in order
    if (threadIdx.x < kC) {
        const int j = threadIdx.x;
        for (int i = 0; i < kC; ++i) {
            float v = i == j ? 1.f : 0.f;
            if (i > j)
                for (int m = j; m < i; ++m) v -= sm.A[i][m] * sm.T[m][j];
            sm.T[i][j] = i >= j ? v : 0.f;
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < kC * kC; e += kT) sc[L::T + e] = sm.T[e / kC][e % kC];
    // W = T Diag(beta) K e^G,  Q~ = Q e^G,  K- = K e^{G_63 - G}
    for (int e = threadIdx.x; e < kC * DK; e += kT) {
        const int t = e / DK, ch = e % DK;
        float w = 0.f;
        for (int m = 0; m <= t; ++m) w += sm.T[t][m] * sm.beta[m] * sm.K[m][ch] * fexp(sm.G[m][ch]);
        sc[L::W + e] = w;
        sc[L::QT + e] = sm.Q[t][ch] * fexp(sm.G[t][ch]);
        sc[L::KB + e] = sm.K[t][ch] * fexp(sm.G[kC - 1][ch] - sm.G[t][ch]);
    }
    // U = T Diag(beta) V
    const bf16_t* v = (const bf16_t*)a.v;
    for (int e = threadIdx.x; e < kC * DV; e += kT) {
        const int t = e / DV, j = e % DV;
        float u = 0.f;
        for (int m = 0; m <= t && m < nrows; ++m) u += sm.T[t][m] * sm.beta[m] * ldin(v, (lane * a.T + c * kC + m) * DV + j);
        sc[L::U + e] = u;
    }
    for (int ch = threadIdx.x; ch < DK; ch += kT) sc[L::GAM + ch] = fexp(sm.G[kC - 1][ch]);
}

// Reverse state pass for value columns [j0, j0 + 32) of one lane.
template <int DK, int DV, typename TO>
__global__ __launch_bounds__(kT) void bwd_state_kernel(BwdArgs a) {
    typedef BwdLayout<DK, DV> L;
    constexpr int NB = 32;
    __shared__ float Gx[DK][NB];
    __shared__ float X[kC][NB];
    const int nblk = DV / NB;
    const int64_t lane = blockIdx.x / nblk;
    const int j0 = (int)(blockIdx.x % nblk) * NB;
    const TO* dO = (const TO*)a.dO;
    for (int e = threadIdx.x; e < DK * NB; e += kT) {
        const int ch = e / NB, j = e % NB;
        Gx[ch][j] = a.dST ? a.dST[(lane * DK + ch) * DV + j0 + j] : 0.f;
    }
    __syncthreads();
    for (int64_t c = a.nchunks - 1; c >= 0; --c) {
        const float* sc = a.prep + (lane * a.nchunks + c) * L::PREP;
        float* gst = a.gst + (lane * a.nchunks + c) * (int64_t)(DK * DV);
        float* dvt = a.dvt + (lane * a.nchunks + c) * (int64_t)(kC * DV);
        const int nrows = (int)(a.T - c * kC < kC ? a.T - c * kC : kC);
        const int64_t orow = lane * a.T + c * kC;
        for (int e = threadIdx.x; e < DK * NB; e += kT) {
            const int ch = e / NB, j = e % NB;
            gst[ch * DV + j0 + j] = Gx[ch][j];
        }
        // dV~ = K- Gx + A_qk^T dO
        for (int e = threadIdx.x; e < kC * NB; e += kT) {
            const int t = e / NB, j = e % NB;
            float x = 0.f;
            for (int ch = 0; ch < DK; ++ch) x += sc[L::KB + t * DK + ch] * Gx[ch][j];
            for (int i = t; i < nrows; ++i) x += sc[L::AQK + i * kC + t] * ldo(dO, (orow + i) * DV + j0 + j);
            X[t][j] = x;
            dvt[t * DV + j0 + j] = x;
        }
        __syncthreads();
        // Gx <- Diag(gamma) Gx + Q~^T dO - W^T dV~
        float gn[DK * NB / kT];
#pragma unroll
        for (int r = 0; r < DK * NB / kT; ++r) {
            const int e = threadIdx.x + r * kT;
            const int ch = e / NB, j = e % NB;
            float g = sc[L::GAM + ch] * Gx[ch][j];
#pragma nounroll
            for (int t = 0; t < nrows; ++t) g += sc[L::QT + t * DK + ch] * ldo(dO, (orow + t) * DV + j0 + j);
#pragma nounroll
            for (int t = 0; t < kC; ++t) g -= sc[L::W + t * DK + ch] * X[t][j];
            gn[r] = g;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < DK * NB / kT; ++r) {
            const int e = threadIdx.x + r * kT;
            Gx[e / NB][e % NB] = gn[r];
        }
        __syncthreads();
    }
    if (a.dS0)
        for (int e = threadIdx.x; e < DK * NB; e += kT) {
            const int ch = e / NB, j = e % NB;
            a.dS0[(lane * DK + ch) * DV + j0 + j] = Gx[ch][j];
        }
}

template <int DK, int DV>
struct __align__(16) GradSmem {
    float K[kC][DK], Q[kC][DK], G[kC][DK];
    float dAqk[kC][kC + 1], dAkk[kC][kC + 1];   // dAkk first holds T
    float beta[kC];
    float dlgam[DK];                             // gamma dgamma + sum_t dK-_t K-_t, joins row 63
};

template <int DK, int DV, typename TO>
__global__ __launch_bounds__(kT) void bwd_grad_kernel(BwdArgs a) {
    typedef BwdLayout<DK, DV> L;
    constexpr int CG = DK / 4;        // channels per thread: thread = (row t, channel group of CG)
    constexpr int VG = DV / 4;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    GradSmem<DK, DV>& sm = *reinterpret_cast<GradSmem<DK, DV>*>(smem_raw);
    const int64_t lane = blockIdx.x / a.nchunks, c = blockIdx.x % a.nchunks;
    const int64_t row0 = lane * a.T + c * kC;
    const int nrows = (int)(a.T - c * kC < kC ? a.T - c * kC : kC);
    const float* sc = a.prep + (int64_t)blockIdx.x * L::PREP;
    float* gs = a.gscr + (int64_t)blockIdx.x * L::GRAD;
    const float* Gx = a.gst + (int64_t)blockIdx.x * (DK * DV);
    const float* dVt = a.dvt + (int64_t)blockIdx.x * (kC * DV);
    // entry state: S0 (or zero) for the first chunk, else the forward's state after chunk c - 1
    const float* S = c == 0 ? (a.S0 ? a.S0 + lane * (int64_t)(DK * DV) : nullptr)
                            : a.ckpt + (lane * a.ck_stride + c - 1) * (int64_t)(DK * DV);
    const TO* dO = (const TO*)a.dO;
    load_chunk_kgq<DK>(a, row0, nrows, sm.K, sm.Q, sm.G, sm.beta);

    const int t = threadIdx.x >> 2;          // row of this thread
    const int c0 = (threadIdx.x & 3) * CG;   // its channels c0 .. c0 + CG - 1
    const int j0 = (threadIdx.x & 3) * VG;   // its value columns
    auto dO_at = [&](int tt, int j) -> float { return tt < nrows ? ldo(dO, (row0 + tt) * DV + j) : 0.f; };
    auto S_at = [&](int ch, int j) -> float { return S ? S[ch * DV + j] : 0.f; };

    // V~ = U - W S
    for (int e = threadIdx.x; e < kC * DV; e += kT) {
        const int tt = e / DV, j = e % DV;
        float x = sc[L::U + e];
        for (int ch = 0; ch < DK; ++ch) x -= sc[L::W + tt * DK + ch] * S_at(ch, j);
        gs[L::VT + e] = x;
    }
    // T into the dAkk slot; dgamma-part of dlgam
    for (int e = threadIdx.x; e < kC * kC; e += kT) sm.dAkk[e / kC][e % kC] = sc[L::T + e];
    for (int ch = threadIdx.x; ch < DK; ch += kT) {
        float s = 0.f;
        for (int j = 0; j < DV; ++j) s += Gx[ch * DV + j] * S_at(ch, j);
        sm.dlgam[ch] = sc[L::GAM + ch] * s;
    }
    __syncthreads();
    // dA_qk = Tril(dO V~^T)
    for (int e = threadIdx.x; e < kC * kC; e += kT) {
        const int i = e / kC, j = e % kC;
        float x = 0.f;
        if (j <= i)
            for (int jj = 0; jj < DV; ++jj) x += dO_at(i, jj) * gs[L::VT + j * DV + jj];
        sm.dAqk[i][j] = x;
    }
    // per (t, channel group): dQ~ = dO S^T, dK- = V~ Gx^T, dW = -dV~ S^T
    float dq[CG], dk[CG], dG[CG];
    float dbeta = 0.f;
    for (int u = 0; u < CG; ++u) {
        const int ch = c0 + u;
        float xq = 0.f, xb = 0.f, xw = 0.f;
        for (int j = 0; j < DV; ++j) {
            const float s = S_at(ch, j);
            xq += dO_at(t, j) * s;
            xb += gs[L::VT + t * DV + j] * Gx[ch * DV + j];
            xw -= dVt[t * DV + j] * s;
        }
        const float eg = fexp(sm.G[t][ch]);
        const float kb = sc[L::KB + t * DK + ch];
        dq[u] = xq * eg;
        dk[u] = xb * fexp(sm.G[kC - 1][ch] - sm.G[t][ch]);
        dG[u] = xq * sm.Q[t][ch] * eg - xb * kb;
        gs[L::DW + t * DK + ch] = xw;
        atomicAdd(&sm.dlgam[ch], xb * kb);
    }
    __syncthreads();
    // [dX_K | dX_V] = T^T [dW | dV~]
    for (int u = 0; u < CG; ++u) {
        const int ch = c0 + u;
        float x = 0.f;
        for (int m = t; m < kC; ++m) x += sm.dAkk[m][t] * gs[L::DW + m * DK + ch];
        gs[L::XK + t * DK + ch] = x;
        const float kt = sm.K[t][ch] * fexp(sm.G[t][ch]);   // K~
        dk[u] += sm.beta[t] * x * fexp(sm.G[t][ch]);
        dG[u] += sm.beta[t] * x * kt;
        dbeta += x * kt;
    }
    float dv[VG];
    for (int u = 0; u < VG; ++u) {
        const int j = j0 + u;
        float x = 0.f;
        for (int m = t; m < kC; ++m) x += sm.dAkk[m][t] * dVt[m * DV + j];
        gs[L::XV + t * DV + j] = x;
        dv[u] = sm.beta[t] * x;
        if (t < nrows) dbeta += x * ldin((const bf16_t*)a.v, (row0 + t) * DV + j);
    }
    __syncthreads();
    // dA_kk = -(dX_K W^T + dX_V U^T), strictly below the diagonal (replaces T)
    for (int e = threadIdx.x; e < kC * kC; e += kT) {
        const int i = e / kC, j = e % kC;
        float x = 0.f;
        if (j < i) {
            for (int ch = 0; ch < DK; ++ch) x -= gs[L::XK + i * DK + ch] * sc[L::W + j * DK + ch];
            for (int jj = 0; jj < DV; ++jj) x -= gs[L::XV + i * DV + jj] * sc[L::U + j * DV + jj];
        }
        sm.dAkk[i][j] = x;
    }
    __syncthreads();
    // pairwise terms: row sums (this thread's row t against j <= t) and column sums (rows i >= t)
    for (int u = 0; u < CG; ++u) {
        const int ch = c0 + u;
        const float kt = sm.K[t][ch], qt = sm.Q[t][ch], gt = sm.G[t][ch], bt = sm.beta[t];
        float rq = 0.f, rk = 0.f, rg = 0.f, rb = 0.f, ck = 0.f, cg = 0.f;
        for (int j = 0; j <= t; ++j) {
            const float e = fexp(gt - sm.G[j][ch]);
            const float aq = sm.dAqk[t][j], ak = j < t ? sm.dAkk[t][j] : 0.f;
            const float kj = sm.K[j][ch] * e;
            rq += aq * kj;
            rk += bt * ak * kj;
            rg += (aq * qt + bt * ak * kt) * kj;
            rb += ak * kt * kj;
        }
        for (int i = t; i < kC; ++i) {
            const float e = fexp(sm.G[i][ch] - gt);
            const float aq = sm.dAqk[i][t], ak = i > t ? sm.dAkk[i][t] : 0.f;
            const float w = (aq * sm.Q[i][ch] + sm.beta[i] * ak * sm.K[i][ch]) * e;
            ck += w;
            cg += w * kt;
        }
        dq[u] += rq;
        dk[u] += rk + ck;
        dG[u] += rg - cg;
        dbeta += rb;
    }
    __syncthreads();
    // dG into LDS (reusing Q), dgamma's share on row 63, then reverse cumsum per channel
    for (int u = 0; u < CG; ++u) sm.Q[t][c0 + u] = dG[u] + (t == kC - 1 ? sm.dlgam[c0 + u] : 0.f);
    __syncthreads();
    for (int ch = threadIdx.x; ch < DK; ch += kT) {
        float acc = 0.f;
        for (int tt = kC - 1; tt >= 0; --tt) { acc += sm.Q[tt][ch]; sm.Q[tt][ch] = acc; }
    }
    __syncthreads();
    dbeta += __shfl_xor(dbeta, 1);
    dbeta += __shfl_xor(dbeta, 2);
    if (t < nrows) {
        const int64_t r = row0 + t;
        for (int u = 0; u < CG; ++u) {
            a.dq[r * DK + c0 + u] = dq[u];
            a.dk_[r * DK + c0 + u] = dk[u];
            a.dla[r * DK + c0 + u] = sm.Q[t][c0 + u];
        }
        for (int u = 0; u < VG; ++u) a.dv_[r * DV + j0 + u] = dv[u];
        if ((threadIdx.x & 3) == 0) a.dbeta[r] = dbeta;
    }
}

template <int DK, int DV, typename TO>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t st) {
    const int64_t chunks = a.lanes * a.nchunks;
    if (chunks <= 0) return hipSuccess;
    const size_t prep_smem = sizeof(PrepSmem<DK, DV>), grad_smem = sizeof(GradSmem<DK, DV>);
    hipFuncSetAttribute((const void*)bwd_prep_kernel<DK, DV>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)prep_smem);
    hipFuncSetAttribute((const void*)bwd_grad_kernel<DK, DV, TO>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)grad_smem);
    hipLaunchKernelGGL((bwd_prep_kernel<DK, DV>), dim3((unsigned)chunks), dim3(kT), prep_smem, st, a);
    hipLaunchKernelGGL((bwd_state_kernel<DK, DV, TO>), dim3((unsigned)(a.lanes * (DV / 32))), dim3(kT), 0, st, a);
    hipLaunchKernelGGL((bwd_grad_kernel<DK, DV, TO>), dim3((unsigned)chunks), dim3(kT), grad_smem, st, a);
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
size_t bwd_grad_floats(int64_t dk, int64_t dv) {
    return dk == 128 ? (dv == 128 ? BwdLayout<128, 128>::GRAD : BwdLayout<128, 64>::GRAD)
                     : (dv == 128 ? BwdLayout<64, 128>::GRAD : BwdLayout<64, 64>::GRAD);
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t st) {
    return a.dO_bf16 ? launch_bwd_o<bf16_t>(a, st) : launch_bwd_o<float>(a, st);
}

}  // namespace kda

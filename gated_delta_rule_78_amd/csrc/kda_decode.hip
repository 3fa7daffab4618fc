// KDA single-token decode step for gfx950.
//
// One token of the recurrence in section 2.2 of the Kimi K3 reading notes
// (liuzhao09.github.io/papers/kimi-k3.html):
//   S' = Diag(alpha) S                           (decay, alpha = exp(log_alpha) per key channel)
//   r  = S'^T k,   p = S'^T q                     (two reductions over the key dimension)
//   delta = beta (v - r)
//   S'' = S' + k delta^T                          (written back in place)
//   o  = S''^T q = p + (k^T q) delta              (read after the write)
// The fp32 state is ~99% of the bytes, so the kernel is HBM-bound: each state slab is read once
// and written once with 16-byte coalesced accesses and kept in registers in between.
//
// Work mapping: one workgroup of 256 threads per (sequence, head, block of NC value columns).
// Thread t owns column quad t % NQ (4 value columns, float4) of the block and rows rg, rg + NRG,
// ... with rg = t / NQ, so each wave's loads cover whole row segments.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// Fused prologue / epilogue (Gating): alpha = exp(g_min * sigmoid(exp(A_h) * z)) replaces
// exp(log_alpha); o is replaced by sigmoid(gate) * w * o / sqrt(mean(o^2) + eps).
__device__ __forceinline__ float sigmoidf_fast(float x) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * kLog2e));
}

template <int DK, int DV, int NC, typename TIn, typename TOut>
__global__ __launch_bounds__(256) void decode_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                     const TIn* __restrict__ v, const TIn* __restrict__ la,
                                                     const TIn* __restrict__ beta, float* __restrict__ S,
                                                     TOut* __restrict__ o, int64_t lanes, int64_t H, Gating gt) {
    constexpr int NQ = NC / 4;        // column quads of this workgroup's block
    constexpr int NRG = 256 / NQ;     // row groups
    constexpr int RPT = DK / NRG;     // rows per thread
    constexpr int NB = DV / NC;       // column blocks per (sequence, head)
    constexpr int RGW = 64 / NQ;      // row groups per wave
    static_assert(RPT * NRG == DK && NB * NC == DV && RGW >= 1, "shape");
    __shared__ float red[4][NQ][9];   // per-wave partial sums: r (4), p (4), k^T q

    const int t = threadIdx.x;
    const int cq = t % NQ;
    const int rg = t / NQ;

    for (int64_t item = blockIdx.x; item < lanes * NB; item += gridDim.x) {
        const int64_t lane = item / NB;
        const int col0 = (int)(item % NB) * NC + 4 * cq;   // this thread's first column
        float* Sl = S + lane * (int64_t)(DK * DV);
        const TIn* ql = q + lane * DK;
        const TIn* kl = k + lane * DK;
        const TIn* lal = (gt.z ? (const TIn*)gt.z : la) + lane * DK;
        const TIn* vl = v + lane * DV;
        const float eA = gt.z ? __builtin_amdgcn_exp2f(gt.A_log[lane % H] * kLog2e) : 0.f;

        // the state streams through once per step: non-temporal loads and stores
        float4 s[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sl + (int64_t)(rg + NRG * i) * DV + col0));
            s[i] = make_float4(x[0], x[1], x[2], x[3]);
        }

        float kr[RPT], qr[RPT];
        float rs[4] = {0.f, 0.f, 0.f, 0.f}, ps[4] = {0.f, 0.f, 0.f, 0.f};
        float kq = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int row = rg + NRG * i;
            kr[i] = ld_f(kl + row);
            qr[i] = ld_f(ql + row);
            const float x = ld_f(lal + row);
            const float a = __builtin_amdgcn_exp2f((gt.z ? gt.g_min * sigmoidf_fast(eA * x) : x) * kLog2e);
            s[i].x *= a; s[i].y *= a; s[i].z *= a; s[i].w *= a;
            rs[0] += kr[i] * s[i].x; rs[1] += kr[i] * s[i].y; rs[2] += kr[i] * s[i].z; rs[3] += kr[i] * s[i].w;
            ps[0] += qr[i] * s[i].x; ps[1] += qr[i] * s[i].y; ps[2] += qr[i] * s[i].z; ps[3] += qr[i] * s[i].w;
            kq += kr[i] * qr[i];
        }
        // sums over the rows: first across the row groups of a wave (lanes NQ apart), then
        // across the four waves through LDS
#pragma unroll
        for (int m = NQ; m < 64; m <<= 1) {
#pragma unroll
            for (int j = 0; j < 4; ++j) { rs[j] += __shfl_xor(rs[j], m); ps[j] += __shfl_xor(ps[j], m); }
            kq += __shfl_xor(kq, m);
        }
        const int wv = t >> 6;
        if ((t & 63) < NQ) {
#pragma unroll
            for (int j = 0; j < 4; ++j) { red[wv][cq][j] = rs[j]; red[wv][cq][4 + j] = ps[j]; }
            red[wv][cq][8] = kq;
        }
        __syncthreads();
        float r4[4] = {0.f, 0.f, 0.f, 0.f}, p4[4] = {0.f, 0.f, 0.f, 0.f};
        float kqt = 0.f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
#pragma unroll
            for (int j = 0; j < 4; ++j) { r4[j] += red[g][cq][j]; p4[j] += red[g][cq][4 + j]; }
            kqt += red[g][cq][8];
        }
        const float b = ld_f(beta + lane);
        float d4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) d4[j] = b * (ld_f(vl + col0 + j) - r4[j]);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            s[i].x += kr[i] * d4[0]; s[i].y += kr[i] * d4[1]; s[i].z += kr[i] * d4[2]; s[i].w += kr[i] * d4[3];
            __builtin_nontemporal_store(f32x4{s[i].x, s[i].y, s[i].z, s[i].w},
                                        reinterpret_cast<f32x4*>(Sl + (int64_t)(rg + NRG * i) * DV + col0));
        }
        if (rg == 0) {   // threads 0 .. NQ-1 of wave 0 hold the block's output columns
            TOut* ol = o + lane * DV + col0;
            float y[4] = {p4[0] + kqt * d4[0], p4[1] + kqt * d4[1], p4[2] + kqt * d4[2], p4[3] + kqt * d4[3]};
            if (NC == DV && gt.gate) {   // the epilogue needs the whole row: launched with NC = DV
                float ss = y[0] * y[0] + y[1] * y[1] + y[2] * y[2] + y[3] * y[3];
#pragma unroll
                for (int m = 1; m < NQ; m <<= 1) ss += __shfl_xor(ss, m);
                const float rstd = __builtin_amdgcn_rsqf(ss * (1.f / (float)DV) + gt.eps);
                const TIn* gl = (const TIn*)gt.gate + lane * DV + col0;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    y[j] *= rstd * (gt.norm_w ? gt.norm_w[col0 + j] : 1.f) * sigmoidf_fast(ld_f(gl + j));
            }
            store4(ol, y[0], y[1], y[2], y[3]);
        }
        __syncthreads();  // red[] is reused by the next item of a grid-stride loop
    }
}

// Columns per workgroup: a (sequence, head) state splits into independent column blocks (each
// column of S only meets its own column of v), which keeps fewer registers per thread and more
// workgroups in flight; the fused epilogue normalises a whole row, so it keeps NC = DV.
constexpr int kDecodeCols = 64;

template <int DK, int DV, int NC, typename TIn, typename TOut>
static hipError_t launch_decode_nc(const DecodeArgs& a, hipStream_t st) {
    const int64_t items = a.N * a.H * (DV / NC);
    const int64_t grid = items < (int64_t)1 << 30 ? items : (int64_t)1 << 30;
    hipLaunchKernelGGL((decode_kernel<DK, DV, NC, TIn, TOut>), dim3((unsigned)grid), dim3(256), 0, st,
                       (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v, (const TIn*)a.la, (const TIn*)a.beta,
                       a.S, (TOut*)a.o, a.N * a.H, a.H, a.gt);
    return hipGetLastError();
}

template <int DK, int DV, typename TIn, typename TOut>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
    constexpr int NC = kDecodeCols < DV ? kDecodeCols : DV;
    if (a.gt.gate || NC == DV) return launch_decode_nc<DK, DV, DV, TIn, TOut>(a, st);
    return launch_decode_nc<DK, DV, NC, TIn, TOut>(a, st);
}

template <int DK, int DV>
static hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t st) {
    if (a.in_bf16 && a.out_bf16) return launch_decode_t<DK, DV, bf16_t, bf16_t>(a, st);
    if (a.in_bf16) return launch_decode_t<DK, DV, bf16_t, float>(a, st);
    if (a.out_bf16) return launch_decode_t<DK, DV, float, bf16_t>(a, st);
    return launch_decode_t<DK, DV, float, float>(a, st);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
    if (a.dk == 128 && a.dv == 128) return launch_decode_d<128, 128>(a, st);
    if (a.dk == 128 && a.dv == 64) return launch_decode_d<128, 64>(a, st);
    if (a.dk == 64 && a.dv == 128) return launch_decode_d<64, 128>(a, st);
    return launch_decode_d<64, 64>(a, st);
}

}  // namespace kda

// KDA fused prefill for gfx950, bf16 inputs: the intra-chunk work and the state step of every
// chunk in one kernel, so that a chunk's record (kda_record.h) never leaves the compute unit
// (Kimi K3 reading notes, liuzhao09.github.io/papers/kimi-k3.html, section 2.2 chunk equations;
// section 2.5 for the sequence split that gives each workgroup its own segment).
//
// One 8-wave workgroup per (lane, segment). Waves 0-3 (producer) run the key side of the
// intra-chunk work with the intra-chunk kernel's per-wave code (intra::ChunkWave, SPLIT): decay
// factors, the off-diagonal Gram tiles and A_qk, the W half of the UT solve, into an LDS record
// buffer. Waves 4-7 (consumer) hold the fp32 state in MFMA accumulators, 32 columns each, and
// take the value side (intra::ValueWave): their V rows, A_kk's diagonal block and its inverse,
// the U half of the solve (U stays in their registers), then the state step. Chunk c's record is
// built while the consumer steps through chunk c - 1's:
//   epoch c:  producer: decay factors of chunk c        | consumer: state step of chunk c - 1
//             ---- barrier 1: the consumer is done with the record buffer ----
//             producer: record pieces held back, loads  | consumer: o rows of chunk c - 1, V of
//                       of chunk c + 1, Gram tiles      |   chunk c staged, loads of V of chunk
//                                                       |   c + 1, A_kk's diagonal blocks and
//                                                       |   their inverses
//             ---- barrier 2 ----
//             producer: W                               | consumer: U of chunk c
//             ---- barrier 3: chunk c's record is complete ----
// The two roles run separate loops with the same barriers (every barrier orders LDS only), so
// the registers of one role are free for the other. Per chunk the kernel reads q, k, v,
// log_alpha and beta and writes o: the two-kernel path also writes and reads the record
// (71 KiB per chunk at d = 128) through HBM. Every product is the two-kernel path's, in the same
// order, so the outputs are the same bit for bit.
//
// Entry states: S0 for segment 0, else the window's S~ (ChunkLaunch::ws_entry, from a kPassWindow
// launch); a lane with an inexact window (ws_flag) is left to the two-kernel fallback. Lanes of
// equal-length and packed batches (LaneSpan); state checkpoints, the fused decay prologue
// (producer) and the gated RMSNorm epilogue (consumer) as in the two-kernel path.
#include "kda_intra_chunk.h"
#include "kda_step.h"

namespace kda {
namespace {

using intra::ChunkWave;
using intra::IntraSmem;
using intra::ValueWave;
using intra::kC;

constexpr int kThreads = 512;

// The record buffer's U blocks are never written (U stays with the consumer): the consumer's V
// stages live there, the fourth one after the record.
template <int DK, int DV>
struct __align__(16) FusedSmem {
    typedef RecordLayout<DK, DV> R;
    static constexpr int VSTAGE = kC * intra::IntraCfg<DK, DV>::LDVS * 2;
    static_assert(3 * VSTAGE <= 2 * R::NV * 1024, "three V stages fit the U blocks");
    IntraSmem<DK, DV> ip;                              // the producer's stages
    unsigned char rec[R::BYTES];                       // the record of the chunk in flight
    unsigned char vst3[VSTAGE];                        // the fourth consumer wave's V stage
    float ssq[4][kC];                                  // gated epilogue: per-wave sums of o^2 per token
    float norm_w[DV];                                  // gated epilogue: the RMSNorm weight
    __device__ __forceinline__ bf16_t* vstage(int cw) {
        return reinterpret_cast<bf16_t*>(cw < 3 ? rec + R::U * 1024 + cw * VSTAGE : vst3);
    }
};

// Barrier over the whole workgroup that orders LDS accesses only (global loads stay in flight).
__device__ __forceinline__ void epoch_barrier() { lds_barrier(); }

// A consumer wave's columns col0 .. col0 + 16 NT - 1 of a dk x dv fp32 state at dst, through a
// buffer descriptor: the lane's offset in a register, each (nt, M, r) offset a scalar constant
// (64-bit addresses per element would hold dozens of registers in the chunk loop).
template <int DK, int DV, int NT>
__device__ __forceinline__ void store_state(float* dst, const f32x4 (&S)[NT][DK / 16], int col0, int lq, int l16) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(dst, (uint32_t)(DK * DV * 4));
    const int lane_off = (4 * lq * DV + col0 + l16) * 4;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int M = 0; M < DK / 16; ++M)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[nt][M][rr]), r, lane_off,
                                                      ((16 * M + rr) * DV + 16 * nt) * 4, 0);
}

template <int DK, int DV, bool ZPRO>
__device__ __forceinline__ void producer(const ChunkLaunch& p, FusedSmem<DK, DV>& sm, int64_t lane, const LaneSpan& span,
                                         int64_t cb, int64_t ce) {
    ChunkWave<DK, DV, ZPRO, true> cw(sm.ip);
    unsigned char* rec = sm.rec;
    const int64_t T = span.len;
    const int64_t row_base = span.row_base;
    auto rows_of = [&](int64_t c) -> uint32_t { return c < ce ? (uint32_t)(T - c * kC < kC ? T - c * kC : kC) : 0u; };
    auto load = [&](int64_t c) {
        cw.load(p.q, p.k, ZPRO ? p.gt.z : p.la, p.v, p.beta, row_base + (c < ce ? c : 0) * kC, rows_of(c));
    };
    // the fused decay prologue: exp(A_h) of the lane's head (lane = b * H + h, or s * H + h packed)
    const float eA = ZPRO ? __builtin_amdgcn_exp2f(p.gt.A_log[lane % p.map.H] * kLog2e) : 0.f;
    load(cb);
    cw.pin_inputs();
    for (int64_t c = cb; c < ce; ++c) {
        cw.template decay<true>(rec, eA, ZPRO ? p.gt.g_min : 0.f, rows_of(c));
        epoch_barrier();   // 1
        cw.publish(rec);
        load(c + 1);
        cw.gram(rec);
        epoch_barrier();   // 2
        cw.pin_inputs();
        cw.solve(rec);
        epoch_barrier();   // 3
    }
    // the consumer's last chunk
    epoch_barrier();
    epoch_barrier();
    epoch_barrier();
}

template <typename TOut, int DK, int DV, bool GATED, bool CKPT>
__device__ __forceinline__ void consumer(const ChunkLaunch& p, FusedSmem<DK, DV>& sm, int64_t lane, int seg,
                                         bool last, const LaneSpan& span, int64_t cb, int64_t ce) {
    constexpr int NT = DV / 64;
    constexpr int NM = DK / 16;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);
    const int l = tid & 63;
    const int l16 = l & 15;
    const int lq = l >> 4;
    const int64_t DVl = DV;
    const int64_t T = span.len;
    const int64_t row_base = span.row_base;
    const int col0 = w * 16 * NT;
    ValueWave<DK, DV> vw(sm.ip, sm.vstage(w), w);
    auto load = [&](int64_t c) {
        uint32_t n = 0;
        if (c < ce) n = (uint32_t)(T - c * kC < kC ? T - c * kC : kC);
        vw.load(p.v, row_base + (c < ce ? c : 0) * kC, n);
    };
    load(cb);
    // S[nt][M] holds rows 16M + 4lq + r, column col0 + 16nt + l16
    f32x4 S[NT][NM];
    const float* entry = seg > 0 ? p.ws_entry + ((lane * p.nseg + seg) * DK) * DVl : (p.S0 ? p.S0 + lane * DK * DVl : nullptr);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int M = 0; M < NM; ++M)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[nt][M][r] = entry ? entry[(16 * M + 4 * lq + r) * DVl + col0 + 16 * nt + l16] : 0.f;
    // wait for the entry state here: left to its first use, the wait would sit at the top of the
    // chunk loop and, run every chunk, also wait for the stores and loads in flight there
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int M = 0; M < NM; ++M)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float x = S[nt][M][r];
                asm volatile("" : "+v"(x));
                S[nt][M][r] = x;
            }
    const __amdgpu_buffer_rsrc_t ro = make_rsrc((const TOut*)p.o + row_base * DVl, (uint32_t)(T * DVl * sizeof(TOut)));
    constexpr bool PAIRED = sizeof(TOut) == 2 && NT % 2 == 0;
    constexpr int NP = NT / 2 > 0 ? NT / 2 : 1;

    // State checkpoints (ChunkLaunch::ckpt): the lane's j-th at ck_base + (j - 1) ck_stride.
    const int64_t ck_base = span.ck_base, ck_stride = span.ck_stride;
    // Gated epilogue: the gate rows of chunk c are loaded into registers after chunk c's U solve,
    // in the layout of chunk c's o stores, and wait there through the next state step (a whole
    // step to arrive) until those rows are stored; per-token sums of o^2 meet across the four
    // consumer waves in LDS. The loads are issued on every path, like the V loads (past the last
    // chunk the rows lie beyond the lane and read as zeros). The row goes in the range-checked
    // vector offset, rebuilt at each use from fresh_lane().
    const __amdgpu_buffer_rsrc_t rgt =
        make_rsrc(GATED ? (const bf16_t*)p.gt.gate + row_base * DVl : nullptr, GATED ? (uint32_t)(T * DVl * 2) : 0u);
    uint2 gpend[NT][4];   // fp32 output: gate values of columns col0 + 16nt + 4lq .. + 3, row 16I + l16
    uint4 gq[NP][4];      // bf16 output: columns col0 + 32np + pair_col(lq) .. + 7, row 16I + l16
    if (GATED) {   // the weights (ones when absent) in LDS: read at each use, held in no register
        for (int i = l; i < 16 * NT; i += 64) sm.norm_w[col0 + i] = p.gt.norm_w ? p.gt.norm_w[col0 + i] : 1.f;
        wave_lds_sync();
    }
    auto weights = [&](int c0) -> f32x4 { return *reinterpret_cast<const f32x4*>(&sm.norm_w[c0]); };
    auto load_gate = [&](int64_t c) {
        if (!GATED) return;
        const int fl = fresh_lane();
        const uint32_t vo =
            (uint32_t)(((uint32_t)(c * kC) + (uint32_t)(fl & 15)) * (uint32_t)DV + (uint32_t)col0 +
                       (PAIRED ? pair_col(fl >> 4) : 4u * (uint32_t)(fl >> 4))) * 2u;
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            if constexpr (PAIRED) {
#pragma unroll
                for (int np = 0; np < NP; ++np) gq[np][I] = buf_load16(rgt, vo + (uint32_t)(16 * I * DV + 32 * np) * 2u);
            } else {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) gpend[nt][I] = buf_load8(rgt, vo + (uint32_t)(16 * I * DV + 16 * nt) * 2u);
            }
        }
    };
    const float inv_dv = 1.f / (float)DV;

    f32x4 O[NT][4];
    i16x4 U[NT][4];   // U of the chunk the next state step takes
    for (int64_t c = cb; c <= ce; ++c) {
        const bool prev = c > cb;   // chunk c - 1's record is in the buffer
        const bool cur = c < ce;    // chunk c is being built
        if (prev) {
            chunk_step<TOut, DK, DV, NT, 0, NT, true>(sm.rec, S, col0, DV / 16 - col0 / 16, O, false, ro, nullptr, w, U);
            if (CKPT && c % p.ck_chunks == 0 && c * kC <= T) {   // S is the state after chunk c - 1
                const int64_t idx = ck_base + (c / p.ck_chunks - 1) * ck_stride;
                if (idx < p.ck_cap) store_state<DK, DV, NT>(p.ckpt + idx * DK * DVl, S, col0, lq, l16);
            }
            if (GATED) {   // this wave's part of each token's sum of o^2
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    float ss = 0.f;
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                        for (int r = 0; r < 4; ++r) ss += O[nt][I][r] * O[nt][I][r];
                    ss += __shfl_xor(ss, 16);
                    ss += __shfl_xor(ss, 32);
                    if (lq == 0) sm.ssq[w][16 * I + l16] = ss;
                }
            }
        }
        epoch_barrier();   // 1
        if (prev) {
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const uint32_t row = (uint32_t)((c - 1) * kC + 16 * I + l16);
                float rstd = 0.f;
                if (GATED)
                    rstd = __builtin_amdgcn_rsqf((sm.ssq[0][16 * I + l16] + sm.ssq[1][16 * I + l16] + sm.ssq[2][16 * I + l16] +
                                                  sm.ssq[3][16 * I + l16]) * inv_dv + p.gt.eps);
                if constexpr (PAIRED) {
#pragma unroll
                    for (int np = 0; np < NP; ++np) {
                        f32x4 a, b;
                        swap_pair(O[2 * np][I], O[2 * np + 1][I], a, b);
                        if (GATED) {
                            const int wc = col0 + 32 * np + (int)pair_col(lq);
                            a = gated_norm(a, make_uint2(gq[np][I].x, gq[np][I].y), weights(wc), rstd);
                            b = gated_norm(b, make_uint2(gq[np][I].z, gq[np][I].w), weights(wc + 4), rstd);
                        }
                        store_bf16x8(ro, row * (uint32_t)DV + (uint32_t)(col0 + 32 * np) + pair_col(lq), a, b);
                    }
                } else {
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        const f32x4 y = GATED ? gated_norm(O[nt][I], gpend[nt][I], weights(col0 + 16 * nt + 4 * lq), rstd)
                                              : O[nt][I];
                        store_out(ro, (row * (uint32_t)DV + col0 + 16 * nt + 4 * lq) * (uint32_t)sizeof(TOut), y,
                                  (TOut*)nullptr);
                    }
                }
            }
        }
        // V of chunk c into the stage (its wait also covers the o stores just issued: measured
        // faster than staging V before the stores), the next V rows, the diagonal inverse
        if (cur) {
            vw.pin_inputs();
            vw.stage();
            load(c + 1);
            vw.diag_inverse();
        }
        epoch_barrier();   // 2
        if (cur) vw.solve(U);
        load_gate(c);
        epoch_barrier();   // 3
    }
    if (last && p.S_T) store_state<DK, DV, NT>(p.S_T + lane * DK * DVl, S, col0, lq, l16);
}

template <typename TOut, int DK, int DV, bool ZPRO, bool GATED, bool CKPT>
__global__ __launch_bounds__(kThreads, 1) void fused_kernel(ChunkLaunch p) {
    __shared__ FusedSmem<DK, DV> sm;
    const int64_t lane = uniform64(blockIdx.x / p.nseg);
    const int seg = (int)uniform64(blockIdx.x % p.nseg);
    if (p.nseg > 1 && !window_split_exact(p.ws_flag + lane * p.nseg, p.nseg)) return;   // the fallback's lane
    const LaneSpan span = lane_span(p, lane);
    // the lane's last live segment runs to its last chunk and stores S_T; the ones past it (a
    // packed lane shorter than the plan's longest) do nothing
    const int64_t nch = (span.len + kC - 1) / kC;
    const int live = live_segments(p, nch);
    if (seg >= live) return;
    int64_t cb = (int64_t)seg * p.chunks_per_seg;
    int64_t ce = seg == live - 1 ? nch : cb + p.chunks_per_seg;
    if (ce > nch) ce = nch;
    if (cb > ce) cb = ce;
    cb = uniform64(cb);
    ce = uniform64(ce);
    // the role split is wave-uniform (a scalar branch), so each wave runs only its own loop
    if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) < 4)
        producer<DK, DV, ZPRO>(p, sm, lane, span, cb, ce);
    else
        consumer<TOut, DK, DV, GATED, CKPT>(p, sm, lane, seg, seg == live - 1, span, cb, ce);
}

// One workgroup: the lanes whose flags are not all 1, in increasing order (a block-wide prefix
// count per 1024 lanes).
__global__ __launch_bounds__(1024, 1) void fallback_lanes_kernel(const int32_t* flag, int64_t lanes, int nseg,
                                                                 int32_t* list, int32_t* count) {
    __shared__ int32_t pre[1024];
    int32_t base = 0;
    for (int64_t l0 = 0; l0 < lanes; l0 += 1024) {
        const int64_t lane = l0 + threadIdx.x;
        const int32_t need = lane < lanes && !window_split_exact(flag + lane * nseg, nseg) ? 1 : 0;
        pre[threadIdx.x] = need;
        __syncthreads();
        for (int d = 1; d < 1024; d <<= 1) {   // inclusive Hillis-Steele scan
            const int32_t x = threadIdx.x >= (unsigned)d ? pre[threadIdx.x - d] : 0;
            __syncthreads();
            pre[threadIdx.x] += x;
            __syncthreads();
        }
        if (need) list[base + pre[threadIdx.x] - 1] = (int32_t)lane;
        base += pre[1023];
        __syncthreads();
    }
    if (threadIdx.x == 0) *count = base;
}

}  // namespace

template <typename TOut, bool ZPRO, bool GATED>
void launch_g(const ChunkLaunch& a, int64_t blocks, hipStream_t st) {
    if (a.ckpt)
        hipLaunchKernelGGL((fused_kernel<TOut, 128, 128, ZPRO, GATED, true>), dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL((fused_kernel<TOut, 128, 128, ZPRO, GATED, false>), dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
}

template <typename TOut>
void launch_o(const ChunkLaunch& a, int64_t blocks, hipStream_t st) {
    if (a.gt.z) {
        if (a.gt.gate) launch_g<TOut, true, true>(a, blocks, st);
        else launch_g<TOut, true, false>(a, blocks, st);
    } else {
        if (a.gt.gate) launch_g<TOut, false, true>(a, blocks, st);
        else launch_g<TOut, false, false>(a, blocks, st);
    }
}

hipError_t launch_fused(const ChunkLaunch& a, hipStream_t st) {
    const int64_t blocks = a.lanes * (int64_t)a.nseg;
    if (blocks <= 0) return hipSuccess;
    if (a.out_bf16) launch_o<bf16_t>(a, blocks, st);
    else launch_o<float>(a, blocks, st);
    return hipGetLastError();
}

hipError_t launch_fallback_lanes(const int32_t* flag, int64_t lanes, int nseg, int32_t* list, int32_t* count,
                                 hipStream_t st) {
    hipLaunchKernelGGL(fallback_lanes_kernel, dim3(1), dim3(1024), 0, st, flag, lanes, nseg, list, count);
    return hipGetLastError();
}

}  // namespace kda

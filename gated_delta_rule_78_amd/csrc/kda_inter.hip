// KDA inter-chunk state pass for gfx950: the sequential part of chunkwise prefill (Kimi K3
// reading notes, liuzhao09.github.io/papers/kimi-k3.html, section 2.2 chunk equations; section
// 2.5 affine pair for the sequence split). For each chunk of a lane, with the chunk's record
// (kda_record.h) and entry state S:
//   V~ = U - W S,   O = Q~ S + A_qk V~,   S <- Diag(gamma_C) S + K-^T V~
// (the record holds -W, so V~ is one MFMA accumulation started from U).
//
// One workgroup (4 waves) per (lane, segment) walks the segment's chunks in order. The fp32 state
// stays in MFMA accumulators: wave w owns 16*NT state columns, rows = key channels. Records
// stream HBM -> LDS with direct-to-LDS buffer loads (each wave a quarter of the blocks), double
// buffered one chunk ahead; every operand read from LDS is one conflict-free 16-byte fragment
// read. The chunk loop is bound by that record stream; the stores of a chunk's output are issued
// one chunk late, so that the wait for the next record copies does not also wait for them.
//
// A lane is one (batch, head) pair of a fixed-length batch or one (sequence, head) pair of a packed
// batch of variable-length sequences (ChunkLaunch::map); a FINISH segment also stores the state
// at every checkpoint interval it closes.
//
// With a fused epilogue (ChunkLaunch::gt.gate), FINISH stores y = sigmoid(gate) * w * o * rstd(o)
// instead of o (the per-head RMSNorm and output gate that follow the core in section 2.2).
//
// Roles (one launch may mix them, see ChunkLaunch):
//   FINISH  columns [0, dv): exact entry state in, o written, exit state stored as asked.
//   SUMMARY columns [0, dv + dk) = [S~ | M] with entry [0 | I] and U = 0 on the M columns: the
//           affine pair S_out = S~ + M S_in of the segment, no o.
//   WINDOW  (the start of a FINISH segment s > 0 in the first launch of a split, SplitPass) the
//           SUMMARY products over the last few chunks before the segment, on this wave's FINISH
//           columns of S~ and its share of M's columns. A decay strong enough to drive M to exactly
//           zero in fp32 within the window makes S~ the exact entry state (everything earlier
//           reaches the boundary only through M), and the segment goes on from it at once;
//           otherwise the workgroup computes the segment's SUMMARY for the fallback instead.
#include "kda_internal.h"
#include "kda_mfma.h"
#include "kda_record.h"
#include "kda_step.h"

namespace kda {
namespace {

constexpr int kC = 64;
constexpr int kThreads = 256;

template <int DK, int DV>
struct __align__(16) InterSmem {
    unsigned char rec[2][RecordLayout<DK, DV>::BYTES];
    float ssq[2][4][64];    // fused epilogue: per-wave partial sums of o^2 per token, by chunk parity
    int nonzero[4];         // WINDOW: per wave, whether its share of M has a nonzero entry
};

// WINDOW ahead of FINISH segment seg > 0 of a lane: chunks [wb, we) with we = the segment's first
// chunk and wb = max(0, we - win_chunks), from S~ = 0 (S0 when wb = 0) on this wave's FINISH columns
// and M = I on its share of M's columns (16 MT consecutive ones). Stores the lane's flag for the
// boundary and returns whether the window is exact (M = 0 in fp32, or wb = 0); then S holds S~.
template <typename TOut, int DK, int DV, int NT>
__device__ __forceinline__ bool window_entry(const ChunkLaunch& p, InterSmem<DK, DV>& sm, int64_t lane, int seg,
                                             const unsigned char* rec0, int64_t we, int col0, f32x4 (&S)[NT][DK / 16]) {
    typedef RecordLayout<DK, DV> R;
    constexpr int NM = R::NM;
    constexpr int BYTES = R::BYTES;
    constexpr int MT = DK / 64;
    constexpr int NW = NT + MT;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int l16 = l & 15;
    const int lq = l >> 4;
    const int64_t DVl = DV;
    const int64_t wb = we > p.win_chunks ? we - p.win_chunks : 0;
    const float* s0 = wb == 0 && p.S0 ? p.S0 + lane * DK * DVl : nullptr;
    f32x4 X[NW][NM];
#pragma unroll
    for (int nt = 0; nt < NW; ++nt) {
        const int mc = 16 * MT * w + 16 * (nt - NT) + l16;   // M column of an M tile
#pragma unroll
        for (int M = 0; M < NM; ++M)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * M + 4 * lq + r;
                X[nt][M][r] = nt < NT ? (s0 ? s0[row * DVl + col0 + 16 * nt + l16] : 0.f) : (row == mc ? 1.f : 0.f);
            }
    }
    f32x4 unused[NW][4];   // (no output rows: written only by FINISH products)
    if (wb < we) copy_record<DK, DV, false>(make_rsrc(rec0 + wb * BYTES, BYTES), 0u, sm.rec[0], w, l);
    for (int64_t c = wb; c < we; ++c) {
        const int buf = (int)((c - wb) & 1);
        __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0): this wave's copies of chunk c landed
        __syncthreads();                        // ... and everyone's; buffer buf^1 is free again
        chunk_step<TOut, DK, DV, NW, 0, NW, false>(sm.rec[buf], X, col0, NT, unused, c + 1 < we,
                                                  make_rsrc(rec0 + (c + 1) * BYTES, BYTES), sm.rec[buf ^ 1], w);
    }
    int nz = 0;
#pragma unroll
    for (int j = 0; j < MT; ++j)
#pragma unroll
        for (int M = 0; M < NM; ++M)
#pragma unroll
            for (int r = 0; r < 4; ++r) nz |= X[NT + j][M][r] != 0.f;   // NaN counts as nonzero
    const bool wave_nz = __ballot(nz) != 0;
    if (l == 0) sm.nonzero[w] = wave_nz ? 1 : 0;
    __syncthreads();   // also: every wave is done with both record buffers
    const bool exact = wb == 0 || !(sm.nonzero[0] | sm.nonzero[1] | sm.nonzero[2] | sm.nonzero[3]);
    if (tid == 0) p.ws_flag[lane * p.nseg + seg - 1] = exact ? 1 : 0;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int M = 0; M < NM; ++M) S[nt][M] = X[nt][M];
    return exact;
}

// One segment of one lane in the given role. Returns false when a FINISH segment's window was not
// exact (nothing of the segment was written then).
template <typename TOut, int DK, int DV, int NT, bool FIN, bool GATED>
__device__ __forceinline__ bool run_segment(const ChunkLaunch& p, InterSmem<DK, DV>& sm, int64_t lane, int seg) {
    typedef RecordLayout<DK, DV> R;
    constexpr int NM = R::NM;
    constexpr int BYTES = R::BYTES;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int l16 = l & 15;
    const int lq = l >> 4;
    const int64_t DVl = DV;

    // ---- where the lane's rows, records and checkpoints are (see SeqMap) ---------------------
    const LaneSpan span = lane_span(p, lane);
    const int64_t row_base = span.row_base, len = span.len, slot0 = span.slot0;
    const int64_t ck_base = span.ck_base, ck_stride = span.ck_stride;
    const int64_t nchunks = (len + kC - 1) / kC;
    // the lane's last live segment runs to its last chunk; a segment past it does nothing, and
    // the window passes mark its boundary exact (no SUMMARY is needed for the last live one: the
    // scan stops before it)
    const int live = live_segments(p, nchunks);
    if (seg >= live || (!FIN && seg == live - 1)) {
        if (FIN && (p.split == kPassWindow || p.split == kPassWindowFinish) && tid == 0)
            p.ws_flag[lane * p.nseg + seg - 1] = 1;
        return true;
    }
    int64_t c_begin = (int64_t)seg * p.chunks_per_seg;
    int64_t c_end = seg == live - 1 ? nchunks : c_begin + p.chunks_per_seg;
    if (c_end > nchunks) c_end = nchunks;
    if (c_begin > c_end) c_begin = c_end;
    const int col0 = w * 16 * NT;   // FINISH: in [0, dv); SUMMARY: in [0, dv + dk)
    // one descriptor per chunk record: a lane's records may exceed 32-bit offsets
    const unsigned char* rec0 = p.rec + slot0 * (int64_t)BYTES;

    // ---- entry state: S[nt][M] holds rows 16M + 4lq + r, column col0 + 16nt + l16 ----------
    f32x4 S[NT][NM];
    if (FIN && p.split == kPassWindow) {
        // the window alone: its flag and S~ (the segment's entry state where the flag is 1)
        window_entry<TOut, DK, DV, NT>(p, sm, lane, seg, rec0, c_begin, col0, S);
        float* dst = p.ws_entry + ((lane * p.nseg + seg) * DK) * DVl;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int M = 0; M < NM; ++M)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[(int64_t)(16 * M + 4 * lq + r) * DVl + col0 + 16 * nt + l16] = S[nt][M][r];
        return true;
    }
    if (FIN && p.split == kPassWindowFinish && seg > 0) {
        // from the window before the segment; an inexact one leaves the segment to the fallback
        if (!window_entry<TOut, DK, DV, NT>(p, sm, lane, seg, rec0, c_begin, col0, S)) return false;
    } else {
        if (FIN) {
            const float* entry = nullptr;
            if (seg > 0) entry = p.ws_entry + ((lane * p.nseg + seg) * DK) * DVl;
            else if (p.S0) entry = p.S0 + lane * DK * DVl;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int M = 0; M < NM; ++M)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        S[nt][M][r] = entry ? entry[(16 * M + 4 * lq + r) * DVl + col0 + 16 * nt + l16] : 0.f;
        } else {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int diag = col0 + 16 * nt + l16 - DV;   // M column -> its unit row
#pragma unroll
                for (int M = 0; M < NM; ++M)
#pragma unroll
                    for (int r = 0; r < 4; ++r) S[nt][M][r] = (16 * M + 4 * lq + r == diag) ? 1.f : 0.f;
            }
        }
    }

    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc(FIN ? (const TOut*)p.o + row_base * DVl : nullptr, FIN ? (uint32_t)(len * DVl * sizeof(TOut)) : 0u);
    // State checkpoint after chunk cc when it closes a checkpoint interval inside the lane
    // (FINISH only: the state is exact there). Stored right after the wait at the top of the
    // next iteration, like the output, so that the wait does not cover these stores.
    // (a macro, not a lambda: a lambda capturing the state array would put it in scratch)
#define KDA_CKPT_STORE(cc)                                                                          \
    do {                                                                                            \
        const int64_t cc_ = (cc);                                                                   \
        if (FIN && p.ckpt && (cc_ + 1) % p.ck_chunks == 0 && (cc_ + 1) * kC <= len) {               \
            const int64_t idx_ = ck_base + ((cc_ + 1) / p.ck_chunks - 1) * ck_stride;               \
            if (idx_ < p.ck_cap) {                                                                  \
                float* dst_ = p.ckpt + idx_ * DK * DVl;                                             \
                _Pragma("unroll") for (int nt = 0; nt < NT; ++nt)                                   \
                _Pragma("unroll") for (int M = 0; M < NM; ++M)                                      \
                _Pragma("unroll") for (int r = 0; r < 4; ++r)                                       \
                    dst_[(int64_t)(16 * M + 4 * lq + r) * DVl + col0 + 16 * nt + l16] = S[nt][M][r]; \
            }                                                                                       \
        }                                                                                           \
    } while (0)

    // Output of the previous chunk, stored one iteration late: vmcnt counts loads and stores
    // alike, so stores issued right after the wait complete in the shadow of the next chunk
    // instead of being waited for with its copies.
    f32x4 Opend[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int I = 0; I < 4; ++I) Opend[nt][I] = kZero4;

    // Fused epilogue (FINISH with a gate): the gate rows of a chunk load one iteration ahead of
    // their use, like the records; per-token sums of o^2 meet in LDS across the four waves.
    constexpr bool gated = FIN && GATED;
    const __amdgpu_buffer_rsrc_t rgt =
        make_rsrc(gated ? (const bf16_t*)p.gt.gate + row_base * DVl : nullptr, gated ? (uint32_t)(len * DVl * 2) : 0u);
    // bf16 output with an even tile count leaves in 16-byte row pieces (the layout swap_pair leaves):
    // the gate rows are then loaded in the same pieces and the epilogue applied after the swap
    constexpr bool PAIRED = sizeof(TOut) == 2 && NT % 2 == 0;
    constexpr int NP = NT / 2 > 0 ? NT / 2 : 1;
    f32x4 nw[NT];
    uint2 gpend[NT][4];
    f32x4 nwp[NP][2];    // PAIRED: weights of the lane's 8 columns of each tile pair
    uint4 gq[NP][4];     // PAIRED: gate values of those columns, one 16-byte piece per token row
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        nw[nt] = f32x4{1.f, 1.f, 1.f, 1.f};
        if (gated && p.gt.norm_w) nw[nt] = *reinterpret_cast<const f32x4*>(p.gt.norm_w + col0 + 16 * nt + 4 * lq);
#pragma unroll
        for (int I = 0; I < 4; ++I) gpend[nt][I] = make_uint2(0u, 0u);
    }
#pragma unroll
    for (int np = 0; np < NP; ++np) {
        nwp[np][0] = nwp[np][1] = f32x4{1.f, 1.f, 1.f, 1.f};
        if (PAIRED && gated && p.gt.norm_w) {
            const float* wp = p.gt.norm_w + col0 + 32 * np + pair_col(lq);
            nwp[np][0] = *reinterpret_cast<const f32x4*>(wp);
            nwp[np][1] = *reinterpret_cast<const f32x4*>(wp + 4);
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) gq[np][I] = make_uint4(0u, 0u, 0u, 0u);
    }
    const float inv_dv = 1.f / (float)DV;
    // sum of o^2 over the lane's columns, then over the four 16-lane rows, into LDS
#define KDA_EPI_PARTIAL(cc)                                                                         \
    do {                                                                                            \
        _Pragma("unroll") for (int I = 0; I < 4; ++I) {                                             \
            float ss_ = 0.f;                                                                        \
            _Pragma("unroll") for (int nt = 0; nt < NT; ++nt)                                       \
                _Pragma("unroll") for (int r = 0; r < 4; ++r) ss_ += Opend[nt][I][r] * Opend[nt][I][r]; \
            ss_ += __shfl_xor(ss_, 16);                                                             \
            ss_ += __shfl_xor(ss_, 32);                                                             \
            if (lq == 0) sm.ssq[(cc) & 1][w][16 * I + l16] = ss_;                                   \
        }                                                                                           \
    } while (0)
    // store the output of chunk cc (after a barrier that made every wave's partial sums visible)
#define KDA_STORE_O(cc)                                                                             \
    do {                                                                                            \
        _Pragma("unroll") for (int I = 0; I < 4; ++I) {                                             \
            const uint32_t row = (uint32_t)((cc) * kC + 16 * I + l16);                              \
            float rstd_ = 0.f;                                                                      \
            if (gated) {                                                                            \
                const float* ps_ = &sm.ssq[(cc) & 1][0][16 * I + l16];                              \
                rstd_ = __builtin_amdgcn_rsqf((ps_[0] + ps_[64] + ps_[128] + ps_[192]) * inv_dv + p.gt.eps); \
            }                                                                                       \
            if constexpr (PAIRED) {                                                                 \
                _Pragma("unroll") for (int np = 0; np < NP; ++np) {                                 \
                    f32x4 a_, b_;                                                                   \
                    swap_pair(Opend[2 * np][I], Opend[2 * np + 1][I], a_, b_);                      \
                    if (gated) {                                                                    \
                        a_ = gated_norm(a_, make_uint2(gq[np][I].x, gq[np][I].y), nwp[np][0], rstd_); \
                        b_ = gated_norm(b_, make_uint2(gq[np][I].z, gq[np][I].w), nwp[np][1], rstd_); \
                    }                                                                               \
                    store_bf16x8(ro, row * (uint32_t)DV + (uint32_t)(col0 + 32 * np) + pair_col(lq), a_, b_); \
                }                                                                                   \
            } else {                                                                                \
                _Pragma("unroll") for (int nt = 0; nt < NT; ++nt) {                                 \
                    const f32x4 y_ = gated ? gated_norm(Opend[nt][I], gpend[nt][I], nw[nt], rstd_) : Opend[nt][I]; \
                    store_out(ro, (row * (uint32_t)DV + col0 + 16 * nt + 4 * lq) * (uint32_t)sizeof(TOut), y_, \
                              (TOut*)nullptr);                                                      \
                }                                                                                   \
            }                                                                                       \
        }                                                                                           \
    } while (0)
    // gate rows of chunk cc for the lane's output tiles
#define KDA_LOAD_GATE(cc)                                                                           \
    do {                                                                                            \
        if (gated && PAIRED) {                                                                      \
            _Pragma("unroll") for (int I = 0; I < 4; ++I)                                           \
                _Pragma("unroll") for (int np = 0; np < NP; ++np)                                   \
                    gq[np][I] = buf_load16(rgt, (((uint32_t)((cc) * kC) + 16 * I + l16) * (uint32_t)DV + col0 + 32 * np + pair_col(lq)) * 2u); \
        } else if (gated) {                                                                         \
            _Pragma("unroll") for (int I = 0; I < 4; ++I)                                           \
                _Pragma("unroll") for (int nt = 0; nt < NT; ++nt)                                   \
                    gpend[nt][I] = buf_load8(rgt, (((uint32_t)((cc) * kC) + 16 * I + l16) * (uint32_t)DV + col0 + 16 * nt + 4 * lq) * 2u); \
        }                                                                                           \
    } while (0)

    if (c_begin < c_end) copy_record<DK, DV, FIN>(make_rsrc(rec0 + c_begin * BYTES, BYTES), 0u, sm.rec[0], w, l);
    for (int64_t c = c_begin; c < c_end; ++c) {
        const int buf = (int)((c - c_begin) & 1);
        __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0): this wave's copies of chunk c landed
        __syncthreads();                        // ... and everyone's; buffer buf^1 is free again
        if (FIN && c > c_begin) {
            KDA_CKPT_STORE(c - 1);
            KDA_STORE_O(c - 1);
        }
        KDA_LOAD_GATE(c);
        chunk_step<TOut, DK, DV, NT, 0, NT, FIN>(sm.rec[buf], S, col0, (int)(DV / 16) - col0 / 16, Opend, c + 1 < c_end,
                                                 make_rsrc(rec0 + (c + 1) * BYTES, BYTES), sm.rec[buf ^ 1], w);
        if (gated) KDA_EPI_PARTIAL(c);
    }
    if (FIN && c_begin < c_end) {
        KDA_CKPT_STORE(c_end - 1);
        if (gated) {
            __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0): the last chunk's gate rows
            __syncthreads();                        // every wave's partial sums of the last chunk
        }
        KDA_STORE_O(c_end - 1);
    }
#undef KDA_EPI_PARTIAL
#undef KDA_STORE_O
#undef KDA_LOAD_GATE

#undef KDA_CKPT_STORE
    // ---- exit state --------------------------------------------------------------------------
    float* dst = nullptr;
    int64_t ld_dst = DVl;
    if (!FIN) {
        dst = p.ws_pair + (lane * p.nseg + seg) * DK * (DVl + DK);
        ld_dst = DVl + DK;
    } else if (seg == live - 1) {
        dst = p.S_T ? p.S_T + lane * DK * DVl : nullptr;
    } else if (seg == 0) {   // segment 1's entry state, for the fallback's scan
        dst = p.ws_entry + ((lane * p.nseg + 1) * DK) * DVl;
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
    return true;
}

template <typename TOut, int DK, int DV, bool GATED>
__global__ __launch_bounds__(kThreads, 1) void inter_kernel(ChunkLaunch p) {
    __shared__ InterSmem<DK, DV> sm;
    const int64_t bid = blockIdx.x;
    const int64_t n_fin = p.lanes * p.fin_nseg;
    if (bid < n_fin) {
        const int64_t lane = uniform64(bid / p.fin_nseg);
        const int seg = (int)uniform64(p.fin_seg_lo + bid % p.fin_nseg);
        if (p.skip_flag && window_split_exact(p.skip_flag + lane * p.nseg, p.nseg)) return;   // a fused lane
        // the fallback's pass 2 finishes only the segments whose window was not exact
        if (p.split == kPassFinish && p.ws_flag[lane * p.nseg + seg - 1] != 0) return;
        // A segment whose window was not exact computes its own affine pair instead (a middle
        // segment; the scan needs no pair for the last one), so that under slow decay the
        // summaries run beside segment 0 as in a plain two-pass split.
        if (!run_segment<TOut, DK, DV, DV / 64, true, GATED>(p, sm, lane, seg) && seg < p.nseg - 1)
            run_segment<TOut, DK, DV, (DV + DK) / 64, false, false>(p, sm, lane, seg);
    } else {
        const int64_t b2 = bid - n_fin;
        const int64_t lane = uniform64(b2 / p.sum_nseg);
        const int seg = (int)uniform64(p.sum_seg_lo + b2 % p.sum_nseg);
        if (p.skip_flag && window_split_exact(p.skip_flag + lane * p.nseg, p.nseg)) return;   // a fused lane
        // pass 1 of the fallback: the pairs the first launch did not compute (segments whose
        // window was exact, in lanes where another window was not)
        if (p.split == kPassCarry &&
            (window_split_exact(p.ws_flag + lane * p.nseg, p.nseg) || p.ws_flag[lane * p.nseg + seg - 1] == 0))
            return;
        run_segment<TOut, DK, DV, (DV + DK) / 64, false, false>(p, sm, lane, seg);
    }
}

template <typename TOut, int DK, int DV>
hipError_t launch_t(const ChunkLaunch& a, hipStream_t st) {
    const int64_t blocks = a.lanes * ((int64_t)a.fin_nseg + (int64_t)a.sum_nseg);
    if (blocks <= 0) return hipSuccess;
    if (a.gt.gate)
        hipLaunchKernelGGL((inter_kernel<TOut, DK, DV, true>), dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL((inter_kernel<TOut, DK, DV, false>), dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <typename TOut>
hipError_t launch_o(const ChunkLaunch& a, hipStream_t st) {
    if (a.dk == 128) return a.dv == 128 ? launch_t<TOut, 128, 128>(a, st) : launch_t<TOut, 128, 64>(a, st);
    return a.dv == 128 ? launch_t<TOut, 64, 128>(a, st) : launch_t<TOut, 64, 64>(a, st);
}

}  // namespace

hipError_t launch_inter(const ChunkLaunch& a, hipStream_t st) {
    return a.out_bf16 ? launch_o<bf16_t>(a, st) : launch_o<float>(a, st);
}

}  // namespace kda

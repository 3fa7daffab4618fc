// Segment scan of the sequence split (Kimi K3 reading notes, liuzhao09.github.io/papers/kimi-k3.html,
// section 2.5: a segment acts on the state as the affine map S_out = S~ + M S_in, and such maps
// compose associatively). Given entry_1 (the exit state of segment 0) and the pairs (S~_s, M_s)
// of the middle segments, it forms the exact entry states entry_{s+1} = S~_s + M_s entry_s for
// s = 1 .. live - 2, in fp32 (live: the lane's segments that hold chunks, nseg but for a packed
// lane shorter than the longest). Lanes whose window flags are all set (see SplitPass) are skipped.
//
// One workgroup per (lane, 16 state columns), one wave per 16-row output tile (8 waves at dk = 128,
// two per SIMD, so that one wave's operand-load issue overlaps the other's products). The current
// entry tile (dk x 16) lives in LDS, transposed; each step is a (dk x dk) x (dk x 16) product on
// the fp32 MFMA (16x16x4), its A operands (rows of M_s) streaming from the workspace two steps
// ahead. The k index of the e-th value of a lane's j-th 16-byte vector is 16 j + 4 lq + e,
// the same for A and B: each lane reads whole 16-byte vectors, and the four lane groups of a row
// read 64 contiguous bytes per instruction (a blocked k = (dk/4) lq + .. layout made every
// instruction touch four times as many cache lines).
#include "kda_internal.h"
#include "kda_mfma.h"
#include "kda_step.h"

namespace kda {
namespace {

template <int DK>
__global__ __launch_bounds__(DK == 128 ? 512 : 256) void segment_scan_kernel(ChunkLaunch p) {
    constexpr int NTH = DK == 128 ? 512 : 256;   // one 16-row output tile per wave
    constexpr int TPW = DK / (16 * (NTH / 64));   // 16-row output tiles per wave
    constexpr int KJ = DK / 4;     // k values per lane group
    constexpr int LDE = DK + 4;
    __shared__ __align__(16) float Et[16][LDE];   // Et[column][row] of the current entry tile

    const int64_t DV = p.dv;
    const int64_t LDP = DV + DK;
    const int ncb = (int)(DV / 16);
    // Workgroups are dealt to the 8 XCDs round-robin by block index. When the lane count allows,
    // the ncb workgroups of a lane get indices that are equal mod 8, so they share one XCD's L2
    // and each M_s is read from HBM once per lane.
    int64_t lane, cb;
    const int64_t bid = blockIdx.x;
    if ((p.lanes & 7) == 0) {
        cb = (bid >> 3) % ncb;
        lane = (bid / (8 * ncb)) * 8 + (bid & 7);
    } else {
        cb = bid % ncb;
        lane = bid / ncb;
    }
    lane = uniform64(lane);
    cb = uniform64(cb);
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int l16 = l & 15;
    const int lq = l >> 4;
    const int64_t col = 16 * cb + l16;
    const int nseg = p.nseg;
    // a lane that the fused kernel finished, or whose entry states all came from the window
    // launch, has nothing to scan
    if (p.skip_flag && window_split_exact(p.skip_flag + lane * nseg, nseg)) return;
    if (window_split_exact(p.ws_flag + lane * nseg, nseg)) return;
    const int64_t nch = (lane_span(p, lane).len + 63) / 64;   // the lane's chunks of 64 tokens
    const int ns = live_segments(p, nch);   // steps s = 1 .. ns - 2
    if (ns <= 2) return;

    // entry tile: every load issued before the first LDS store (one memory round trip)
    const float* e1 = p.ws_entry + (lane * nseg + 1) * DK * DV;
    constexpr int NE = DK * 16 / NTH;
    float ev[NE];
#pragma unroll
    for (int u = 0; u < NE; ++u) {
        const int i = tid + NTH * u;
        ev[u] = e1[(int64_t)(i >> 4) * DV + 16 * cb + (i & 15)];
    }
#pragma unroll
    for (int u = 0; u < NE; ++u) {
        const int i = tid + NTH * u;
        Et[i & 15][i >> 4] = ev[u];
    }

    // operands of step s: A = rows 16 (TPW w + t) + l16 of M_s, k = 16 j4 + 4 lq + e;
    // st = S~_s at the tile's accumulator positions
    f32x4 a[TPW][KJ / 4], st[TPW];
    auto load_step = [&](int s, f32x4 (*aa)[KJ / 4], f32x4* ss) {
        const float* P = p.ws_pair + (lane * nseg + s) * DK * LDP;
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int row0 = 16 * (TPW * w + t);
            const float* Arow = P + (int64_t)(row0 + l16) * LDP + DV + 4 * lq;
#pragma unroll
            for (int j4 = 0; j4 < KJ / 4; ++j4) aa[t][j4] = *reinterpret_cast<const f32x4*>(Arow + 16 * j4);
#pragma unroll
            for (int r = 0; r < 4; ++r) ss[t][r] = P[(int64_t)(row0 + 4 * lq + r) * LDP + col];
        }
    };
    // Operands two steps ahead in three buffers: at the top of step s, before its products, the
    // loads of step s + 2 go into the buffer step s - 1 has released, so they are issued while
    // this step's MFMA chain runs. The loop is unrolled by three so that no buffer is ever copied
    // (a register copy would wait for the loads filling its source).
    f32x4 a1[TPW][KJ / 4], st1[TPW], a2[TPW][KJ / 4], st2[TPW];
    load_step(1, a, st);
    if (ns > 3) load_step(2, a1, st1);
    // Barriers below order the LDS tile only: a full barrier would also wait for the operand
    // loads in flight for later steps. The entry states stored here are read by a later kernel.
    lds_barrier();
    // (a macro, not a lambda, so that the operand arrays stay in registers)
#define KDA_SCAN_STEP(S_, A_, ST_, NA_, NST_)                                                       \
    do {                                                                                            \
        const int s_ = (S_);                                                                        \
        if (s_ + 3 < ns) load_step(s_ + 2, NA_, NST_);                                              \
        f32x4 acc[TPW];                                                                             \
        _Pragma("unroll") for (int t = 0; t < TPW; ++t) acc[t] = ST_[t];                            \
        _Pragma("unroll") for (int j4 = 0; j4 < KJ / 4; ++j4) {                                     \
            const f32x4 b = *reinterpret_cast<const f32x4*>(&Et[l16][16 * j4 + 4 * lq]);           \
            _Pragma("unroll") for (int e = 0; e < 4; ++e)                                           \
            _Pragma("unroll") for (int t = 0; t < TPW; ++t)                                         \
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(A_[t][j4][e], b[e], acc[t], 0, 0, 0); \
        }                                                                                           \
        lds_barrier();   /* every wave has read the old entry tile */                               \
        float* dst = p.ws_entry + (lane * nseg + s_ + 1) * DK * DV;                                 \
        _Pragma("unroll") for (int t = 0; t < TPW; ++t) {                                           \
            const int row0 = 16 * (TPW * w + t);                                                    \
            *reinterpret_cast<f32x4*>(&Et[l16][row0 + 4 * lq]) = acc[t];                            \
            _Pragma("unroll") for (int r = 0; r < 4; ++r)                                           \
                dst[(int64_t)(row0 + 4 * lq + r) * DV + col] = acc[t][r];                           \
        }                                                                                           \
        lds_barrier();                                                                              \
    } while (0)
    for (int s = 1; s + 1 < ns; s += 3) {
        KDA_SCAN_STEP(s, a, st, a2, st2);
        if (s + 2 < ns) KDA_SCAN_STEP(s + 1, a1, st1, a, st);
        if (s + 3 < ns) KDA_SCAN_STEP(s + 2, a2, st2, a1, st1);
    }
#undef KDA_SCAN_STEP
}

}  // namespace

hipError_t launch_segment_scan(const ChunkLaunch& a, hipStream_t st) {
    if (a.nseg <= 2) return hipSuccess;
    const int64_t blocks = a.lanes * (a.dv / 16);
    if (a.dk == 128) hipLaunchKernelGGL(segment_scan_kernel<128>, dim3((unsigned)blocks), dim3(512), 0, st, a);
    else hipLaunchKernelGGL(segment_scan_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace kda

// KDA intra-chunk kernel for gfx950, bf16 inputs: everything of a 64-token chunk that does not
// depend on the recurrent state (Kimi K3 reading notes, liuzhao09.github.io/papers/kimi-k3.html,
// section 2.2: cumulative decay Gamma, the decay-weighted Gram tiles and the UT transform).
//
// Every chunk of every lane is independent. A persistent grid of two workgroups (4 waves each) per
// compute unit walks the record slots (the chunks of every lane; for a packed batch of
// variable-length sequences, the chunk slots of every head, which a small table maps to rows),
// loading the next chunk's raw rows into registers while it solves the current one (and while
// the other workgroup on the compute unit runs). A chunk still costs a workgroup about 8 us, most
// of it dependent-instruction and LDS latency, of which the two workgroups per compute unit (the
// LDS budget) hide part. Input loads are row-contiguous (64 bytes per row per wave). Output: the chunk's record
// (kda_record.h) in the workspace. Steps, with G = cumsum(log alpha) over the chunk's rows:
//   1. per wave, 32 key channels: G^T = g^T U (U[s][t] = (s <= t)) on the MFMA. Decay factors are
//      taken against reference points so that none exceeds e^80 over the whole domain
//      log alpha in [-5, 0] (decay lower-bound equation of section 2.2, with the 16-token
//      sub-tiles of Figure 3): for the Gram tiles, relative to the start of each 16-token block,
//      G_ref(I) = G at token 16I - 1, i.e. Q~_I = Q e^{G - G_ref(I)}, K~_I = K e^{G - G_ref(I)}
//      (<= 1) and K^_I = K e^{G_ref(I) - G} (<= e^{16*5}); for the record, relative to the chunk
//      start: Q~ = Q e^{G}, K~ = K e^{G} and K- = K e^{G_C - G} (all <= 1). Factors are fp32,
//      rounded once to bf16. Q~ and K- go to the record; the block-relative Q~, K~, K^ go to LDS
//      as fragment blocks.
//   2. Gram tiles from the LDS blocks. A diagonal 16x16 block uses one reference point; an
//      off-diagonal block (I > J) rescales K^_J channel-wise by f_IJ = e^{G_ref(I) - G_ref(J)}
//      (<= 1). The diagonal blocks of A_kk = Diag(beta) StrictTril(K~K^^T) are formed in fp32
//      (wave 0, which then inverts I + A_kk's four 16x16 diagonal blocks by substitution); waves
//      1-3 take two off-diagonal block pairs each, rescaling K^_J once for both the A_kk block (bf16,
//      to LDS) and the A_qk = Tril(Q~K^^T) block (to the record), then the diagonal A_qk blocks.
//   3. blocked forward substitution (I + A_kk) [W | U] = Diag(beta) [K~ | V] on the MFMA, 16
//      columns per tile, right-hand sides and results in registers; U goes to the record, -W is
//      transposed through LDS into fragment order.
#include "kda_intra_chunk.h"

namespace kda {
namespace {

using intra::ChunkWave;
using intra::IntraSmem;
using intra::kC;

template <int DK, int DV, bool PACKED, bool ZPRO>
__global__ __launch_bounds__(256, 2) void intra_kernel(IntraArgs p) {
    __shared__ IntraSmem<DK, DV> sm;
    ChunkWave<DK, DV, ZPRO> cw(sm);

    // work items: record slots, `slots` per head (packed batch) or per lane (fixed length),
    // fewer than 2^31 in all; `rows` rows of every row-major input per head / lane. A fixed-length
    // batch may walk a subset (IntraArgs): `nl` lanes of `per_lane` chunks each.
    const uint32_t slots = (uint32_t)(PACKED ? p.map.slots : p.nchunks);
    const int64_t rows = PACKED ? p.map.rows : p.T;
    const uint32_t nl = PACKED ? 1u : (p.lane_list ? (uint32_t)*p.lane_count : (uint32_t)p.lanes);
    // window chunks per boundary: the whole previous segment when a segment is shorter than the window
    const uint32_t wspan = !PACKED && p.win_chunks > 0 ? (uint32_t)(p.win_chunks < p.chunks_per_seg ? p.win_chunks : p.chunks_per_seg) : 0u;
    const uint32_t per_lane = wspan ? (uint32_t)(p.nseg - 1) * wspan : slots;
    if (p.run_if && *p.run_if == 0) return;
    const uint32_t total = PACKED ? (p.slot_list ? (uint32_t)*p.slot_count : (uint32_t)(p.map.H * (int64_t)slots))
                                  : nl * per_lane;
    const int64_t nheads = p.map.H > 0 ? p.map.H : 1;

    // First row and valid rows of item (h, j) in the row-major inputs; no rows (zeros, no
    // traffic) for !ok.
    auto chunk_rows = [&](bool ok, uint32_t h, uint32_t j, int64_t& row0, uint32_t& n) {
        row0 = 0;
        n = 0;
        if (!ok) return;
        if (PACKED) {
            const SlotEntry e = p.slot_tab[j];
            row0 = (int64_t)h * rows + e.row0;
            n = (uint32_t)e.nrows;
        } else {
            row0 = (int64_t)h * rows + (int64_t)j * kC;
            n = (uint32_t)(rows - (int64_t)j * kC < kC ? rows - (int64_t)j * kC : kC);
        }
    };

    // Persistent: workgroup b takes items b, b + gridDim.x, ..., so the loads of the next chunk
    // overlap the Gram tiles and solve of this one. Item u -> (head or lane h, slot j). Packed
    // batch: head-major, in slot order. Fixed length: chunk-major from the last chunk down, lanes
    // fastest: the records written last, the ones still in the last-level cache when the state
    // pass starts, are then the first chunks of every lane, which the state pass reads first (in
    // lane-major order only the last-written lanes found theirs there, and the first pass waited
    // for the others).
    // A window subset walks, per lane, window r / wspan's chunk r % wspan (the window before
    // boundary s = r / wspan + 1 ends at chunk s * chunks_per_seg).
    const uint32_t G = gridDim.x;
    auto item_of = [&](uint32_t u, uint32_t& h, uint32_t& j) {
        if (PACKED) {
            const uint32_t e = p.slot_list ? (uint32_t)p.slot_list[u] : u;
            h = e / slots;
            j = e % slots;
            return;
        }
        h = u % nl;
        const uint32_t r = u / nl;
        j = wspan ? (r / wspan + 1u) * (uint32_t)p.chunks_per_seg - wspan + r % wspan : slots - 1u - r;
        if (p.lane_list) h = (uint32_t)p.lane_list[h];
    };
    uint32_t t = blockIdx.x;
    uint32_t hn = 0, jn = 0;   // the item whose rows are (being) loaded
    if (t < total) item_of(t, hn, jn);
    {
        int64_t row0;
        uint32_t n;
        chunk_rows(t < total, hn, jn, row0, n);
        cw.load(p.q, p.k, ZPRO ? p.gt.z : p.la, p.v, p.beta, row0, n);
    }
    // taken here too, so that the loop head (which merges this path with the loop's back edge)
    // carries no wait for loads
    cw.pin_inputs();
    for (; t < total; t += G) {
        const uint32_t hc = hn, jc = jn;   // this item
        unsigned char* rec = p.rec + ((int64_t)hc * slots + jc) * RecordLayout<DK, DV>::BYTES;
        // exp(A_h) of this chunk's head for the fused decay prologue (head = lane % H for a fixed batch)
        const float eA = ZPRO ? __builtin_amdgcn_exp2f(p.gt.A_log[PACKED ? hc : hc % nheads] * kLog2e) : 0.f;
        // valid rows of this chunk: with the fused prologue, padded rows (zeros, so z = 0) must not
        // decay, g = 0 there rather than g_min / 2
        uint32_t nrows = kC;
        if (ZPRO) {
            if (PACKED) nrows = (uint32_t)p.slot_tab[jc].nrows;
            else nrows = (uint32_t)(rows - (int64_t)jc * kC < kC ? rows - (int64_t)jc * kC : kC);
        }
        if (t + G < total) item_of(t + G, hn, jn);   // the next item

        cw.template decay<false>(rec, eA, ZPRO ? p.gt.g_min : 0.f, nrows);
        // the next chunk's rows load during the Gram phase: issued here rather than right after this
        // chunk's staging, they no longer queue behind the previous chunk's record stores at the top
        // of the chunk, and their registers stay free through the decay phase; issued after the
        // barrier rather than before it, a wave stalled on issuing them no longer holds up the other
        // three
        __syncthreads();
        {
            int64_t row0;
            uint32_t n;
            chunk_rows(t + G < total, hn, jn, row0, n);
            cw.load(p.q, p.k, ZPRO ? p.gt.z : p.la, p.v, p.beta, row0, n);
        }
        cw.gram(rec);
        __syncthreads();
        // the next chunk's rows have had the Gram phase to arrive; take them now, before this
        // chunk's solve issues its record stores
        cw.pin_inputs();
        cw.solve(rec);
        __syncthreads();   // the next chunk rewrites the stages, beta and the A_kk blocks
    }
}

template <int DK, int DV>
hipError_t launch_dd(const IntraArgs& a, hipStream_t st) {
    int64_t blocks = a.slot_tab ? a.map.H * a.map.slots : a.lanes * a.nchunks;
    if (a.win_chunks > 0) {
        const int64_t span = a.win_chunks < a.chunks_per_seg ? a.win_chunks : a.chunks_per_seg;
        blocks = a.lanes * (a.nseg - 1) * span;
    }
    if (blocks <= 0) return hipSuccess;
    const int64_t resident = 2 * (int64_t)compute_units(stream_device(st));   // two per CU (the LDS budget)
    if (blocks > resident) blocks = resident;
    const dim3 grid((unsigned)blocks), block(256);
    if (a.slot_tab) {
        if (a.gt.z) hipLaunchKernelGGL((intra_kernel<DK, DV, true, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((intra_kernel<DK, DV, true, false>), grid, block, 0, st, a);
    } else {
        if (a.gt.z) hipLaunchKernelGGL((intra_kernel<DK, DV, false, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((intra_kernel<DK, DV, false, false>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_intra(const IntraArgs& a, hipStream_t st) {
    if (a.dk == 128) return a.dv == 128 ? launch_dd<128, 128>(a, st) : launch_dd<128, 64>(a, st);
    return a.dv == 128 ? launch_dd<64, 128>(a, st) : launch_dd<64, 64>(a, st);
}

}  // namespace kda

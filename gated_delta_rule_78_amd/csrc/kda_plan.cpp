// Launch plan and dispatch of a bf16 prefill call (see kda_plan.h).
#include "kda_plan.h"

#include <hip/hip_runtime.h>

#include <atomic>

#include "kda_record.h"

namespace kda {

int stream_device(hipStream_t st) {
    int dev = 0;
    if (hipStreamGetDevice(st, &dev) == hipSuccess) return dev;
    return hipGetDevice(&dev) == hipSuccess ? dev : 0;
}

// Cached per device; concurrent first calls from several host threads store the same value.
int compute_units(int dev) {
    static std::atomic<int> cached[64];
    if (dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Sequence split of the bf16 state pass. One state-pass workgroup occupies a compute unit; with
// n segments, pass 1 runs segment 0 plus n - 2 summaries per lane, pass 2 the n - 1 later
// segments, each pass taking chunks_per_seg steps per round of `cus` workgroups (one per compute
// unit). Pick the n with the fewest sequential chunk steps (the segment scan adds about two per
// segment).
static int64_t auto_segments(int64_t lanes, int64_t nchunks, int64_t cus) {
    int64_t best = 1;
    int64_t best_cost = nchunks * ceil_div(lanes, cus);
    const int64_t nmax = nchunks / 4 < 64 ? nchunks / 4 : 64;
    for (int64_t n = 3; n <= nmax; ++n) {
        const int64_t cps = ceil_div(nchunks, n);
        const int64_t nn = ceil_div(nchunks, cps);
        if (nn < 3) continue;
        const int64_t rounds = ceil_div(lanes * (nn - 1), cus);
        const int64_t cost = cps * 2 * rounds + 2 * (nn - 2);
        if (cost < best_cost) { best_cost = cost; best = nn; }
    }
    return best;
}

Plan make_plan(const Geometry& g) {
    Plan p{};
    const int64_t nchunks = g.max_chunks;
    p.nchunks = nchunks;
    int64_t nseg = 1;
    if (g.in_dtype == KDA_BF16 && nchunks > 0) nseg = g.segments > 0 ? g.segments : auto_segments(g.long_lanes, nchunks, g.cus > 0 ? g.cus : 256);
    if (nseg > nchunks) nseg = nchunks > 0 ? nchunks : 1;
    int64_t cps = nchunks > 0 ? ceil_div(nchunks, nseg) : 1;
    if (cps < 1) cps = 1;
    nseg = nchunks > 0 ? ceil_div(nchunks, cps) : 1;  // no segment past the longest lane
    p.nseg = (int)nseg;
    p.chunks_per_seg = cps;
    if (g.in_dtype == KDA_BF16 && nchunks > 0) {
        p.rec_bytes = (size_t)g.slots * (size_t)record_bytes(g.dk, g.dv);
        if (nseg > 1) {
            p.pair_bytes = (size_t)g.lanes * (size_t)nseg * (size_t)(g.dk * (g.dv + g.dk)) * sizeof(float);
            p.entry_bytes = (size_t)g.lanes * (size_t)nseg * (size_t)(g.dk * g.dv) * sizeof(float);
        }
        p.tab_bytes = (size_t)g.tab_slots * sizeof(SlotEntry);
    }
    p.ws_bytes = p.rec_bytes + p.pair_bytes + p.entry_bytes + p.tab_bytes;
    return p;
}

// bf16 prefill after validation: records of every chunk (state independent, fully parallel),
// then the sequential state pass, split in two passes around the segment scan when the plan
// has more than one segment per lane.
kda_status run_bf16(ChunkLaunch& a, const Plan& plan, unsigned char* ws, hipStream_t st) {
    IntraArgs ia{};
    ia.lanes = a.lanes; ia.T = a.T; ia.nchunks = a.nchunks; ia.dk = a.dk; ia.dv = a.dv;
    ia.q = a.q; ia.k = a.k; ia.v = a.v; ia.la = a.la; ia.beta = a.beta;
    ia.rec = ws;
    ia.map = a.map;
    ia.gt = a.gt;
    ia.slot_tab = a.map.cu ? reinterpret_cast<const SlotEntry*>(ws + plan.rec_bytes + plan.pair_bytes + plan.entry_bytes)
                           : nullptr;
    if (launch_intra(ia, st) != hipSuccess) return KDA_ERR_HIP;
    a.rec = ws;
    a.ws_pair = plan.pair_bytes ? reinterpret_cast<float*>(ws + plan.rec_bytes) : nullptr;
    a.ws_entry = plan.entry_bytes ? reinterpret_cast<float*>(ws + plan.rec_bytes + plan.pair_bytes) : nullptr;
    if (plan.nseg == 1) {
        a.fin_seg_lo = 0; a.fin_nseg = 1; a.sum_seg_lo = 0; a.sum_nseg = 0;
        return launch_inter(a, st) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    // pass 1: segment 0 from the known entry state; summaries of the middle segments
    a.fin_seg_lo = 0; a.fin_nseg = 1; a.sum_seg_lo = 1; a.sum_nseg = plan.nseg - 2;
    if (launch_inter(a, st) != hipSuccess) return KDA_ERR_HIP;
    // exact entry state of every later segment
    if (launch_segment_scan(a, st) != hipSuccess) return KDA_ERR_HIP;
    // pass 2: every later segment from its exact entry state
    a.fin_seg_lo = 1; a.fin_nseg = plan.nseg - 1; a.sum_seg_lo = 0; a.sum_nseg = 0;
    return launch_inter(a, st) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace kda

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

// Sequence split of the bf16 state pass, with n segments per lane (SplitPass): one FINISH launch
// over lanes * n workgroups in which segments 1 .. n - 1 first run a kWindowChunks-chunk window
// (and, where it is inexact under slow decay, compute their affine pair instead); then, only for
// lanes with an inexact window, the missing pairs, the segment scan and the inexact segments.
//
// Modelled time of one state-pass launch, in microseconds: `cps` chunk steps per round of `cus`
// workgroups. A step takes the longer of the chunk's dependent chain (about 3.5 us with FINISH
// workgroups in the round, 3.2 us with SUMMARY ones only) and the record bytes the round's
// workgroups move at about 5 TB/s: 87 KiB per FINISH step (record and output rows), 49 KiB per
// SUMMARY step (fitted to kernel traces of 8K, 64K and 1M calls; at 1M, 192 FINISH workgroups
// took 3.47 us per step and 256 took 4.45 us).
static double pass_us(int64_t cps, int64_t fin, int64_t sum, int64_t cus) {
    double t = 0.0;
    for (int64_t left = fin + sum; left > 0;) {
        const int64_t r = left < cus ? left : cus;
        const int64_t f = fin < r ? fin : r;
        const double bw = (87.0 * (double)f + 49.0 * (double)(r - f)) / 5000.0;
        const double chain = f > 0 ? 3.5 : 3.2;
        t += (double)cps * (bw > chain ? bw : chain);
        fin -= f;
        left -= r;
    }
    return t;
}

// Pick n: the most segments whose FINISH workgroups (lanes * n) still run in one round on the
// device's compute units, among the n whose fallback (a window that is not exact: slow decay)
// stays within 20 % of the best fallback plan, unless one unsplit pass is modelled faster. (The
// model's step times alone do not rank the splits: with fewer workgroups than compute units a
// step is shorter, but at 8K the sweep n = 6, 7, 8 measured 0.2228, 0.2187, 0.2117 ms, and at 1M
// n = 6 lost 1.3 % to n = 8.)
constexpr int64_t kMaxSeg = 256;

static int64_t auto_segments(int64_t lanes, int64_t nchunks, int64_t cus, double* us) {
    const int64_t nmax = nchunks < kMaxSeg ? nchunks : kMaxSeg;
    double fast[kMaxSeg + 1], fallback[kMaxSeg + 1];
    bool valid[kMaxSeg + 1] = {};
    double best_fallback = 0.0;
    for (int64_t n = 1; n <= nmax; ++n) {
        const int64_t cps = ceil_div(nchunks, n);
        if (ceil_div(nchunks, cps) != n) continue;   // the same split as a smaller n
        if (n == 1) {
            fast[n] = fallback[n] = pass_us(nchunks, lanes, 0, cus);
        } else {
            const int64_t w = kWindowChunks < nchunks ? kWindowChunks : nchunks;
            const double empty = 4.5;   // a launch whose workgroups all return at once
            const double scan = n > 2 ? 16.0 + 2.0 * (double)(n - 2) : 0.0;
            fast[n] = pass_us(cps + w, lanes * n, 0, cus) + (n > 2 ? 3.0 : 1.0) * empty;
            // (segments 1 .. n - 2 compute their pairs in the first launch, beside segment 0; with
            // n = 2 the last segment needs no pair and its workgroups stop after the window, so
            // the fallback is segment 0, then segment 1 from its exit state)
            if (n == 2)
                fallback[n] = pass_us(cps, lanes, lanes, cus) + empty + pass_us(cps, lanes, 0, cus);
            else
                fallback[n] = pass_us(cps + w, lanes, lanes * (n - 1), cus) + empty + scan + pass_us(cps, lanes * (n - 1), 0, cus);
        }
        valid[n] = true;
        if (n == 1 || fallback[n] < best_fallback) best_fallback = fallback[n];
    }
    int64_t best = 1;
    for (int64_t n = 2; n <= nmax; ++n)
        if (valid[n] && lanes * n <= cus && fallback[n] <= 1.2 * best_fallback) best = n;
    if (fast[best] >= fast[1]) best = 1;
    *us = fast[best];
    return best;
}

// Modelled time of the intra-chunk kernel over `slots` chunks: two workgroups per compute unit at
// about 14 us per chunk and workgroup (8K: 8 chunks per workgroup in 120 us; 1M: 1,024 chunks in
// 13.9 ms, where the record bytes at the device's copy rate bind as much).
static double intra_us(int64_t slots, int64_t cus) { return 14.0 * (double)ceil_div(slots, 2 * cus); }

// Modelled time of the two-kernel state pass with n segments (n = 0: the plan's choice).
static double two_kernel_state_us(int64_t lanes, int64_t nchunks, int64_t cus, int64_t n) {
    double us = 0.0;
    if (n <= 0) {
        auto_segments(lanes, nchunks, cus, &us);
        return us;
    }
    const int64_t cps = ceil_div(nchunks, n);
    n = ceil_div(nchunks, cps);
    if (n == 1) return pass_us(nchunks, lanes, 0, cus);
    const int64_t w = kWindowChunks < nchunks ? kWindowChunks : nchunks;
    return pass_us(cps + w, lanes * n, 0, cus) + (n > 2 ? 3.0 : 1.0) * 4.5;
}

// The fused plan: one 8-wave workgroup per (lane, segment) and compute unit; each chunk is a
// dependent step of about kFusedStepUs (kernel traces: 7.45 us at 64K, 6.9 us at 1M), plus one
// step to fill the pipeline and a few microseconds for the entry and exit states. n = the most
// segments whose workgroups run in one round (n = 1 when the lanes alone fill the device). With
// n > 1 the windows come first: the intra-chunk kernel over their (n - 1) * min(8, cps) chunks per
// lane and the window launch (about 6 us plus 2.4 us per window step), and after the fused kernel
// six launches that return at once (about 4.5 us each). At 8K (32 heads, 16 chunks per segment)
// this models 235 us against 232 us for the two-kernel path, measured 240 and 235.
constexpr double kFusedStepUs = 7.0;
static int64_t fused_segments(int64_t lanes, int64_t nchunks, int64_t cus, int64_t forced, double* us) {
    int64_t n = forced > 0 ? forced : (lanes < cus ? cus / lanes : 1);
    if (n > kMaxSeg) n = kMaxSeg;
    if (n > nchunks) n = nchunks;
    const int64_t cps = ceil_div(nchunks, n);
    n = ceil_div(nchunks, cps);
    double t = (double)ceil_div(lanes * n, cus) * ((double)(cps + 1) * kFusedStepUs + 8.0);
    if (n > 1) {
        const int64_t w = kWindowChunks < cps ? kWindowChunks : cps;
        t += intra_us(lanes * (n - 1) * w, cus) + 6.0 + 2.4 * (double)w + 6.0 * 4.5;
    }
    *us = t;
    return n;
}

Plan make_plan(const Geometry& g) {
    Plan p{};
    const int64_t nchunks = g.max_chunks;
    p.nchunks = nchunks;
    const int64_t cus = g.cus > 0 ? g.cus : 256;
    int64_t nseg = 1;
    if (g.in_dtype == KDA_BF16 && nchunks > 0) {
        double two_us = 0.0, fused_us = 0.0;
        if (g.segments > 0) nseg = g.segments;
        else nseg = auto_segments(g.long_lanes, nchunks, cus, &two_us);
        if (g.fused_ok && g.state_pass != 1) {
            const int64_t nf = fused_segments(g.lanes, nchunks, cus, g.segments, &fused_us);
            if (g.state_pass == 0) two_us = intra_us(g.slots, cus) + two_kernel_state_us(g.long_lanes, nchunks, cus, g.segments);
            if (g.state_pass == 2 || fused_us < two_us) {
                p.fused = true;
                nseg = nf;
            }
        }
    }
    if (nseg > nchunks) nseg = nchunks > 0 ? nchunks : 1;
    int64_t cps = nchunks > 0 ? ceil_div(nchunks, nseg) : 1;
    if (cps < 1) cps = 1;
    nseg = nchunks > 0 ? ceil_div(nchunks, cps) : 1;  // no segment past the longest lane
    p.nseg = (int)nseg;
    p.chunks_per_seg = cps;
    p.win_chunks = kWindowChunks;   // also past a shorter segment's start: a shorter window is never exact
    if (g.in_dtype == KDA_BF16 && nchunks > 0) {
        p.rec_bytes = (size_t)g.slots * (size_t)record_bytes(g.dk, g.dv);
        if (nseg > 1) {
            p.pair_bytes = (size_t)g.lanes * (size_t)nseg * (size_t)(g.dk * (g.dv + g.dk)) * sizeof(float);
            p.entry_bytes = (size_t)g.lanes * (size_t)nseg * (size_t)(g.dk * g.dv) * sizeof(float);
            p.flag_bytes = (size_t)g.lanes * (size_t)nseg * sizeof(int32_t);
            if (p.fused) {
                p.pre_bytes = p.flag_bytes;
                p.list_bytes = ((size_t)(g.lanes + 1) * sizeof(int32_t) + 15) & ~(size_t)15;
                if (g.tab_slots > 0)
                    p.wlist_bytes = ((size_t)(g.lanes * (nseg - 1) * kWindowChunks + 1) * sizeof(int32_t) + 15) & ~(size_t)15;
            }
        }
        p.tab_bytes = (size_t)g.tab_slots * sizeof(SlotEntry);
    }
    p.ws_bytes = p.rec_bytes + p.pair_bytes + p.entry_bytes + p.tab_bytes + p.flag_bytes + p.pre_bytes + p.list_bytes +
                 p.wlist_bytes;
    return p;
}

// The fused plan: the windows' records and the window launch (n > 1), the fused kernel for every
// lane whose windows are all exact, then the two-kernel window split below for the other lanes
// (their full records first: in a packed batch, every record when any lane falls back), each
// launch of which skips the fused lanes.
static kda_status run_fused(ChunkLaunch& a, const Plan& plan, const IntraArgs& ia, unsigned char* ws, hipStream_t st) {
    if (plan.nseg == 1) {
        a.split = kPassAll;
        return launch_fused(a, st) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    const size_t pre_off = plan.rec_bytes + plan.pair_bytes + plan.entry_bytes + plan.tab_bytes + plan.flag_bytes;
    int32_t* pre = reinterpret_cast<int32_t*>(ws + pre_off);
    int32_t* list = reinterpret_cast<int32_t*>(ws + pre_off + plan.pre_bytes);
    int32_t* count = list + a.lanes;
    IntraArgs iw = ia;   // the window chunks of every lane
    if (a.map.cu) {      // packed: their slots, listed on the device from cu_seqlens
        int32_t* wlist = reinterpret_cast<int32_t*>(ws + pre_off + plan.pre_bytes + plan.list_bytes);
        WindowSlots wsl{};
        wsl.cu = a.map.cu; wsl.N = a.lanes / a.map.H; wsl.H = a.map.H; wsl.rows = a.map.rows;
        wsl.max_len = a.map.max_len; wsl.slots = a.map.slots; wsl.nseg = plan.nseg;
        wsl.chunks_per_seg = plan.chunks_per_seg; wsl.win_chunks = plan.win_chunks;
        wsl.list = wlist; wsl.count = wlist + a.lanes * (plan.nseg - 1) * plan.win_chunks;
        if (launch_window_slots(wsl, st) != hipSuccess) return KDA_ERR_HIP;
        iw.slot_list = wsl.list; iw.slot_count = wsl.count;
    } else {
        iw.win_chunks = plan.win_chunks; iw.chunks_per_seg = plan.chunks_per_seg; iw.nseg = plan.nseg;
    }
    if (launch_intra(iw, st) != hipSuccess) return KDA_ERR_HIP;
    ChunkLaunch w = a;   // their flags and S~
    w.split = kPassWindow; w.ws_flag = pre;
    w.fin_seg_lo = 1; w.fin_nseg = plan.nseg - 1; w.sum_seg_lo = 0; w.sum_nseg = 0;
    if (launch_inter(w, st) != hipSuccess) return KDA_ERR_HIP;
    ChunkLaunch f = a;
    f.split = kPassAll; f.ws_flag = pre;
    if (launch_fused(f, st) != hipSuccess) return KDA_ERR_HIP;
    if (launch_fallback_lanes(pre, a.lanes, plan.nseg, list, count, st) != hipSuccess) return KDA_ERR_HIP;
    IntraArgs il = ia;   // the fallback lanes' records (packed: every record, when any lane falls back)
    if (a.map.cu) il.run_if = count;
    else { il.lane_list = list; il.lane_count = count; }
    if (launch_intra(il, st) != hipSuccess) return KDA_ERR_HIP;
    a.skip_flag = pre;
    return KDA_OK;
}

// bf16 prefill after validation: records of every chunk (state independent, fully parallel),
// then the sequential state pass, split as above when the plan has more than one segment.
kda_status run_bf16(ChunkLaunch& a, const Plan& plan, unsigned char* ws, hipStream_t st) {
    IntraArgs ia{};
    ia.lanes = a.lanes; ia.T = a.T; ia.nchunks = a.nchunks; ia.dk = a.dk; ia.dv = a.dv;
    ia.q = a.q; ia.k = a.k; ia.v = a.v; ia.la = a.la; ia.beta = a.beta;
    ia.rec = ws;
    ia.map = a.map;
    ia.gt = a.gt;
    const size_t tab_off = plan.rec_bytes + plan.pair_bytes + plan.entry_bytes;
    ia.slot_tab = a.map.cu ? reinterpret_cast<const SlotEntry*>(ws + tab_off) : nullptr;
    a.rec = ws;
    a.ws_pair = plan.pair_bytes ? reinterpret_cast<float*>(ws + plan.rec_bytes) : nullptr;
    a.ws_entry = plan.entry_bytes ? reinterpret_cast<float*>(ws + plan.rec_bytes + plan.pair_bytes) : nullptr;
    a.ws_flag = plan.flag_bytes ? reinterpret_cast<int32_t*>(ws + tab_off + plan.tab_bytes) : nullptr;
    a.win_chunks = plan.win_chunks;
    if (plan.fused) {
        const kda_status fs = run_fused(a, plan, ia, ws, st);
        if (fs != KDA_OK || plan.nseg == 1) return fs;
    } else if (launch_intra(ia, st) != hipSuccess) {
        return KDA_ERR_HIP;
    }
    if (plan.nseg == 1) {
        a.split = kPassAll;
        a.fin_seg_lo = 0; a.fin_nseg = 1; a.sum_seg_lo = 0; a.sum_nseg = 0;
        return launch_inter(a, st) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    // every segment, the later ones from the window before them where it is exact
    a.split = kPassWindowFinish;
    a.fin_seg_lo = 0; a.fin_nseg = plan.nseg; a.sum_seg_lo = 0; a.sum_nseg = 0;
    if (launch_inter(a, st) != hipSuccess) return KDA_ERR_HIP;
    // lanes with an inexact window: the pairs of middle segments whose window was exact, the
    // exact entry states from the segment scan, then the segments whose window was inexact
    a.split = kPassCarry;
    a.fin_seg_lo = 0; a.fin_nseg = 0; a.sum_seg_lo = 1; a.sum_nseg = plan.nseg - 2;
    if (launch_inter(a, st) != hipSuccess) return KDA_ERR_HIP;
    if (launch_segment_scan(a, st) != hipSuccess) return KDA_ERR_HIP;
    a.split = kPassFinish;
    a.fin_seg_lo = 1; a.fin_nseg = plan.nseg - 1; a.sum_seg_lo = 0; a.sum_nseg = 0;
    return launch_inter(a, st) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace kda

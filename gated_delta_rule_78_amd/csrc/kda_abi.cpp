// C ABI of the KDA library: argument validation, launch planning and dispatch.
// See include/kda.h for the contract of every entry point.
#include "kda.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "kda_internal.h"
#include "kda_record.h"

namespace {

constexpr int64_t kChunk = 64;
constexpr int64_t kTargetBlocks = 256;  // one workgroup per compute unit

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};
Range range_of(const void* p, int64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + (uintptr_t)bytes};
}
bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

bool valid_dtype(int32_t d) { return d == KDA_F32 || d == KDA_BF16; }
int64_t elem_bytes(int32_t d) { return d == KDA_BF16 ? 2 : 4; }

// Segments per lane, chunks per segment and workspace of a prefill call.
struct Plan {
    int nseg;
    int64_t nchunks, chunks_per_seg;
    size_t rec_bytes;    // intra-chunk records (bf16 path): [lanes][nchunks]
    size_t pair_bytes;   // affine pairs [lanes][nseg][dk][dv + dk] (nseg > 1)
    size_t entry_bytes;  // entry states [lanes][nseg][dk][dv] (nseg > 1)
    size_t ws_bytes;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Sequence split of the bf16 state pass. One state-pass workgroup occupies a compute unit; with
// n segments, pass 1 runs segment 0 plus n - 2 summaries per lane, pass 2 the n - 1 later
// segments, each pass taking chunks_per_seg steps per round of kTargetBlocks workgroups. Pick the
// n with the fewest sequential chunk steps (the segment scan adds about two per segment).
int64_t auto_segments(int64_t lanes, int64_t nchunks) {
    int64_t best = 1;
    int64_t best_cost = nchunks * ceil_div(lanes, kTargetBlocks);
    const int64_t nmax = nchunks / 4 < 64 ? nchunks / 4 : 64;
    for (int64_t n = 3; n <= nmax; ++n) {
        const int64_t cps = ceil_div(nchunks, n);
        const int64_t nn = ceil_div(nchunks, cps);
        if (nn < 3) continue;
        const int64_t rounds = ceil_div(lanes * (nn - 1), kTargetBlocks);
        const int64_t cost = cps * 2 * rounds + 2 * (nn - 2);
        if (cost < best_cost) { best_cost = cost; best = nn; }
    }
    return best;
}

Plan make_plan(const kda_chunk_desc* d) {
    Plan p{};
    const int64_t lanes = d->B * d->H;
    const int64_t nchunks = (d->T + kChunk - 1) / kChunk;
    p.nchunks = nchunks;
    int64_t nseg = 1;
    if (d->in_dtype == KDA_BF16 && nchunks > 0) nseg = d->segments > 0 ? d->segments : auto_segments(lanes, nchunks);
    if (nseg > nchunks) nseg = nchunks > 0 ? nchunks : 1;
    int64_t cps = nchunks > 0 ? ceil_div(nchunks, nseg) : 1;
    if (cps < 1) cps = 1;
    nseg = nchunks > 0 ? ceil_div(nchunks, cps) : 1;  // no empty segment
    p.nseg = (int)nseg;
    p.chunks_per_seg = cps;
    if (d->in_dtype == KDA_BF16 && nchunks > 0) {
        p.rec_bytes = (size_t)lanes * (size_t)nchunks * (size_t)kda::record_bytes(d->dk, d->dv);
        if (nseg > 1) {
            p.pair_bytes = (size_t)lanes * (size_t)nseg * (size_t)(d->dk * (d->dv + d->dk)) * sizeof(float);
            p.entry_bytes = (size_t)lanes * (size_t)nseg * (size_t)(d->dk * d->dv) * sizeof(float);
        }
    }
    p.ws_bytes = p.rec_bytes + p.pair_bytes + p.entry_bytes;
    return p;
}

kda_status check_chunk_desc(const kda_chunk_desc* d) {
    if (!d) return KDA_ERR_INVALID_ARG;
    if (d->B < 1 || d->H < 1 || d->T < 0 || d->dk < 1 || d->dv < 1 || d->segments < 0)
        return KDA_ERR_INVALID_ARG;
    if (!valid_dtype(d->in_dtype) || !valid_dtype(d->out_dtype)) return KDA_ERR_INVALID_ARG;
    if (d->chunk != kChunk) return KDA_ERR_UNSUPPORTED;
    if ((d->dk != 64 && d->dk != 128) || (d->dv != 64 && d->dv != 128)) return KDA_ERR_UNSUPPORTED;
    if (d->in_dtype == KDA_F32 && d->dk != 64) return KDA_ERR_UNSUPPORTED;
    // the bf16 kernel addresses one lane's rows with 32-bit buffer offsets
    if (d->in_dtype == KDA_BF16 && d->T * (d->dk > d->dv ? d->dk : d->dv) * 4 >= ((int64_t)1 << 31))
        return KDA_ERR_UNSUPPORTED;
    // element counts must fit comfortably in 64-bit byte offsets
    const double elems = (double)d->B * (double)d->H * (double)(d->T > 0 ? d->T : 1) * (double)(d->dk + d->dv);
    if (elems > 1e17) return KDA_ERR_INVALID_ARG;
    return KDA_OK;
}

}  // namespace

extern "C" {

const char* kda_status_string(int32_t status) {
    switch (status) {
        case KDA_OK: return "KDA_OK: success";
        case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG: null, negative, misaligned or overlapping argument";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: shape or type not implemented";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
        case KDA_ERR_HIP: return "KDA_ERR_HIP: the HIP runtime reported an error";
        default: return "unknown kda_status";
    }
}

const char* kda_version(void) { return "kda-gfx950 0.1.0"; }

size_t kda_chunk_fwd_workspace_bytes(const kda_chunk_desc* d) {
    if (check_chunk_desc(d) != KDA_OK) return 0;
    return make_plan(d).ws_bytes;
}

kda_status kda_chunk_fwd(const kda_chunk_desc* d, const void* q, const void* k, const void* v,
                         const void* log_alpha, const void* beta, const float* S0, void* o, float* S_T,
                         void* workspace, size_t workspace_bytes, void* stream) {
    const kda_status ds = check_chunk_desc(d);
    if (ds != KDA_OK) return ds;
    const int64_t lanes = d->B * d->H;
    const int64_t ein = elem_bytes(d->in_dtype), eout = elem_bytes(d->out_dtype);
    const int64_t state_bytes = lanes * d->dk * d->dv * (int64_t)sizeof(float);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);

    if (S0 && !aligned(S0, 16)) return KDA_ERR_INVALID_ARG;
    if (S_T && !aligned(S_T, 16)) return KDA_ERR_INVALID_ARG;
    if (S0 && S_T && S0 != S_T && overlaps(range_of(S0, state_bytes), range_of(S_T, state_bytes)))
        return KDA_ERR_INVALID_ARG;

    if (d->T == 0) {
        if (!S_T || S_T == S0) return KDA_OK;
        return kda::launch_copy_or_zero(S_T, S0, state_bytes / 4, st) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }

    if (!q || !k || !v || !log_alpha || !beta || !o) return KDA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(log_alpha, 16) || !aligned(o, 16) ||
        !aligned(beta, (uintptr_t)ein))
        return KDA_ERR_INVALID_ARG;
    const Range ro = range_of(o, lanes * d->T * d->dv * eout);
    const Range rin[] = {range_of(q, lanes * d->T * d->dk * ein), range_of(k, lanes * d->T * d->dk * ein),
                         range_of(v, lanes * d->T * d->dv * ein), range_of(log_alpha, lanes * d->T * d->dk * ein),
                         range_of(beta, lanes * d->T * ein)};
    for (const Range& r : rin)
        if (overlaps(ro, r)) return KDA_ERR_INVALID_ARG;
    if (S0 && overlaps(ro, range_of(S0, state_bytes))) return KDA_ERR_INVALID_ARG;
    if (S_T && overlaps(ro, range_of(S_T, state_bytes))) return KDA_ERR_INVALID_ARG;

    const Plan plan = make_plan(d);
    if (plan.ws_bytes > 0) {
        if (!workspace || workspace_bytes < plan.ws_bytes) return KDA_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return KDA_ERR_INVALID_ARG;
        const Range rw = range_of(workspace, (int64_t)plan.ws_bytes);
        if (overlaps(rw, ro)) return KDA_ERR_INVALID_ARG;
        for (const Range& r : rin)
            if (overlaps(rw, r)) return KDA_ERR_INVALID_ARG;
        if ((S0 && overlaps(rw, range_of(S0, state_bytes))) || (S_T && overlaps(rw, range_of(S_T, state_bytes))))
            return KDA_ERR_INVALID_ARG;
    }

    kda::ChunkLaunch a{};
    a.lanes = lanes; a.T = d->T; a.dk = d->dk; a.dv = d->dv;
    a.nchunks = plan.nchunks;
    a.in_bf16 = d->in_dtype == KDA_BF16; a.out_bf16 = d->out_dtype == KDA_BF16;
    a.nseg = plan.nseg; a.chunks_per_seg = plan.chunks_per_seg;
    a.q = q; a.k = k; a.v = v; a.la = log_alpha; a.beta = beta;
    a.S0 = S0; a.o = o; a.S_T = S_T;
    if (!a.in_bf16) {
        a.fin_seg_lo = 0; a.fin_nseg = 1; a.sum_seg_lo = 0; a.sum_nseg = 0;
        return kda::launch_chunk(a, st) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }

    // bf16: records of every chunk (state independent, fully parallel) ...
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    kda::IntraArgs ia{};
    ia.lanes = lanes; ia.T = d->T; ia.nchunks = plan.nchunks; ia.dk = d->dk; ia.dv = d->dv;
    ia.q = q; ia.k = k; ia.v = v; ia.la = log_alpha; ia.beta = beta;
    ia.rec = ws;
    if (kda::launch_intra(ia, st) != hipSuccess) return KDA_ERR_HIP;
    a.rec = ws;
    a.ws_pair = plan.pair_bytes ? reinterpret_cast<float*>(ws + plan.rec_bytes) : nullptr;
    a.ws_entry = plan.entry_bytes ? reinterpret_cast<float*>(ws + plan.rec_bytes + plan.pair_bytes) : nullptr;

    // ... then the sequential state pass
    if (plan.nseg == 1) {
        a.fin_seg_lo = 0; a.fin_nseg = 1; a.sum_seg_lo = 0; a.sum_nseg = 0;
        return kda::launch_inter(a, st) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    // pass 1: segment 0 from the known entry state; summaries of the middle segments
    a.fin_seg_lo = 0; a.fin_nseg = 1; a.sum_seg_lo = 1; a.sum_nseg = plan.nseg - 2;
    if (kda::launch_inter(a, st) != hipSuccess) return KDA_ERR_HIP;
    // exact entry state of every later segment
    if (kda::launch_segment_scan(a, st) != hipSuccess) return KDA_ERR_HIP;
    // pass 2: every later segment from its exact entry state
    a.fin_seg_lo = 1; a.fin_nseg = plan.nseg - 1; a.sum_seg_lo = 0; a.sum_nseg = 0;
    return kda::launch_inter(a, st) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_decode_step(const kda_decode_desc* d, const void* q, const void* k, const void* v,
                           const void* log_alpha, const void* beta, float* S, void* o, void* stream) {
    if (!d) return KDA_ERR_INVALID_ARG;
    if (d->N < 1 || d->H < 1 || d->dk < 1 || d->dv < 1) return KDA_ERR_INVALID_ARG;
    if (!valid_dtype(d->in_dtype) || !valid_dtype(d->out_dtype)) return KDA_ERR_INVALID_ARG;
    if ((d->dk != 64 && d->dk != 128) || (d->dv != 64 && d->dv != 128)) return KDA_ERR_UNSUPPORTED;
    if (!q || !k || !v || !log_alpha || !beta || !S || !o) return KDA_ERR_INVALID_ARG;
    const int64_t ein = elem_bytes(d->in_dtype), eout = elem_bytes(d->out_dtype);
    if (!aligned(S, 16) || !aligned(o, (uintptr_t)eout) || !aligned(q, (uintptr_t)ein) ||
        !aligned(k, (uintptr_t)ein) || !aligned(v, (uintptr_t)ein) || !aligned(log_alpha, (uintptr_t)ein) ||
        !aligned(beta, (uintptr_t)ein))
        return KDA_ERR_INVALID_ARG;
    // output rows are stored 4 columns at a time
    if (!aligned(o, (uintptr_t)(4 * eout))) return KDA_ERR_INVALID_ARG;
    const int64_t lanes = d->N * d->H;
    const Range ro = range_of(o, lanes * d->dv * eout);
    const Range others[] = {range_of(S, lanes * d->dk * d->dv * 4), range_of(q, lanes * d->dk * ein),
                            range_of(k, lanes * d->dk * ein), range_of(v, lanes * d->dv * ein),
                            range_of(log_alpha, lanes * d->dk * ein), range_of(beta, lanes * ein)};
    for (const Range& r : others)
        if (overlaps(ro, r)) return KDA_ERR_INVALID_ARG;
    for (int i = 1; i < 6; ++i)
        if (overlaps(others[0], others[i])) return KDA_ERR_INVALID_ARG;
    kda::DecodeArgs a{};
    a.N = d->N; a.H = d->H; a.dk = d->dk; a.dv = d->dv;
    a.in_bf16 = d->in_dtype == KDA_BF16; a.out_bf16 = d->out_dtype == KDA_BF16;
    a.q = q; a.k = k; a.v = v; a.la = log_alpha; a.beta = beta; a.S = S; a.o = o;
    return kda::launch_decode(a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"

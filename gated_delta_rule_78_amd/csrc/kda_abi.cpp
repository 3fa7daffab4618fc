// C ABI of the KDA library: argument validation, launch planning and dispatch.
// See include/kda.h for the contract of every entry point.
#include "kda.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "kda_internal.h"

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

// Segments per lane and chunks per segment for a prefill call.
struct Plan {
    int nseg;
    int64_t chunks_per_seg;
    int nw, nt;  // waves per workgroup, 16-column state tiles per wave
    size_t ws_bytes;
};

// Workgroup shape: 128 state columns per workgroup (4 waves x 2 tiles) wherever 128 divides
// both the value width and the augmented width, else 4 waves x 1 tile (64 columns).
void pick_shape(const kda_chunk_desc* d, int* nw, int* nt) {
    const bool w128 = (d->dv % 128 == 0) && ((d->dv + d->dk) % 128 == 0) && d->dk == 128;
    // dk = dv = 128: eight waves, one 16-column state tile each (measured faster than four
    // waves holding two tiles: more waves hide the LDS and exp latency of the chunk prologue).
    *nw = w128 ? 8 : 4;
    *nt = 1;
    // Launch-shape override for tuning sweeps: KDA_NW=8 (8 waves x 1 tile), 4 (4 x 1) or 4x2.
    if (const char* e = getenv("KDA_NW")) {
        if (!strcmp(e, "8") && w128) { *nw = 8; *nt = 1; }
        else if (!strcmp(e, "4")) { *nw = 4; *nt = 1; }
        else if (!strcmp(e, "4x2") && w128) { *nw = 4; *nt = 2; }
    }
}

Plan make_plan(const kda_chunk_desc* d) {
    Plan p{};
    const int64_t lanes = d->B * d->H;
    const int64_t nchunks = (d->T + kChunk - 1) / kChunk;
    int64_t nseg = 1;
    if (d->segments > 0) {
        nseg = d->segments;
    } else if (d->in_dtype == KDA_BF16 && lanes < kTargetBlocks && nchunks >= 16) {
        // Too few lanes to fill the chip: split each sequence into segments (at least 8 chunks
        // each) so that lanes x segments is about one workgroup per compute unit.
        nseg = kTargetBlocks / lanes;
        if (nseg > nchunks / 8) nseg = nchunks / 8;
        if (nseg < 1) nseg = 1;
    }
    if (nseg > nchunks) nseg = nchunks > 0 ? nchunks : 1;
    if (d->in_dtype == KDA_F32) nseg = 1;  // the fp32 path runs one pass
    int64_t cps = nchunks > 0 ? (nchunks + nseg - 1) / nseg : 1;
    if (cps < 1) cps = 1;
    nseg = nchunks > 0 ? (nchunks + cps - 1) / cps : 1;  // no empty segment
    p.nseg = (int)nseg;
    p.chunks_per_seg = cps;
    pick_shape(d, &p.nw, &p.nt);
    if (nseg == 1) {
        p.ws_bytes = 0;
    } else {
        p.ws_bytes = (size_t)lanes * (size_t)nseg * (size_t)d->dk * (size_t)(2 * d->dv + d->dk) * sizeof(float);
    }
    if (d->in_dtype == KDA_F32) { p.nw = 4; p.nt = 1; }
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
    a.in_bf16 = d->in_dtype == KDA_BF16; a.out_bf16 = d->out_dtype == KDA_BF16;
    a.nseg = plan.nseg; a.chunks_per_seg = plan.chunks_per_seg;
    a.q = q; a.k = k; a.v = v; a.la = log_alpha; a.beta = beta;
    a.S0 = S0; a.o = o; a.S_T = S_T;
    float* ws = static_cast<float*>(workspace);
    a.ws_pair = plan.ws_bytes ? ws : nullptr;
    a.ws_entry = plan.ws_bytes ? ws + (size_t)lanes * plan.nseg * d->dk * (d->dv + d->dk) : nullptr;

    a.nw = plan.nw;
    a.nt = plan.nt;
    if (plan.nseg == 1) {
        a.fin_seg_lo = 0; a.fin_nseg = 1; a.sum_seg_lo = 0; a.sum_nseg = 0;
        return kda::launch_chunk(a, st) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    // pass 1: segment 0 from the known entry state; summaries of the middle segments
    a.fin_seg_lo = 0; a.fin_nseg = 1; a.sum_seg_lo = 1; a.sum_nseg = plan.nseg - 2;
    if (kda::launch_chunk(a, st) != hipSuccess) return KDA_ERR_HIP;
    // exact entry state of every later segment
    if (kda::launch_segment_scan(a, st) != hipSuccess) return KDA_ERR_HIP;
    // pass 2: every later segment from its exact entry state
    a.fin_seg_lo = 1; a.fin_nseg = plan.nseg - 1; a.sum_seg_lo = 0; a.sum_nseg = 0;
    return kda::launch_chunk(a, st) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
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

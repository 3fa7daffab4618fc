// C ABI of the KDA library: argument validation, launch planning and dispatch.
// See include/kda.h for the contract of every entry point.
#include "kda.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "kda_internal.h"
#include "kda_plan.h"
#include "kda_record.h"

namespace {

using kda::kChunk;
using kda::Geometry;
using kda::Plan;
using kda::ceil_div;
using kda::make_plan;
using kda::run_bf16;

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

// The plan (and so the workspace) depends on the compute-unit count of the device: a call plans
// for its stream's device, a workspace query for the current device.
int64_t current_cus() {
    int dev = 0;
    return kda::compute_units(hipGetDevice(&dev) == hipSuccess ? dev : 0);
}

// `forward`: a kda_chunk_fwd call (the fused kernel may take it); else the backward's recompute.
Geometry fixed_geometry(const kda_chunk_desc* d, int64_t cus, bool forward = true) {
    const int64_t nchunks = ceil_div(d->T, kChunk);
    Geometry g{d->B * d->H, nchunks, d->B * d->H * nchunks, d->dk, d->dv, d->in_dtype, d->segments, 0,
               d->B * d->H, cus};
    g.state_pass = forward ? d->state_pass : 1;
    g.fused_ok = forward && d->in_dtype == KDA_BF16 && d->dk == 128 && d->dv == 128;
    return g;
}

kda_status check_chunk_desc(const kda_chunk_desc* d) {
    if (!d) return KDA_ERR_INVALID_ARG;
    if (d->B < 1 || d->H < 1 || d->T < 0 || d->dk < 1 || d->dv < 1 || d->segments < 0 || d->state_pass < 0 ||
        d->state_pass > 2)
        return KDA_ERR_INVALID_ARG;
    if (!valid_dtype(d->in_dtype) || !valid_dtype(d->out_dtype)) return KDA_ERR_INVALID_ARG;
    if (d->chunk != kChunk) return KDA_ERR_UNSUPPORTED;
    if ((d->dk != 64 && d->dk != 128) || (d->dv != 64 && d->dv != 128)) return KDA_ERR_UNSUPPORTED;
    if (d->in_dtype == KDA_F32 && d->dk != 64) return KDA_ERR_UNSUPPORTED;
    if (d->in_dtype == KDA_BF16 && d->state_pass == 2 && (d->dk != 128 || d->dv != 128)) return KDA_ERR_UNSUPPORTED;
    // the bf16 kernel addresses one lane's rows with 32-bit buffer offsets
    if (d->in_dtype == KDA_BF16 && d->T * (d->dk > d->dv ? d->dk : d->dv) * 4 >= ((int64_t)1 << 31))
        return KDA_ERR_UNSUPPORTED;
    // element counts must fit comfortably in 64-bit byte offsets
    const double elems = (double)d->B * (double)d->H * (double)(d->T > 0 ? d->T : 1) * (double)(d->dk + d->dv);
    if (elems > 1e17) return KDA_ERR_INVALID_ARG;
    // the intra-chunk kernel numbers its chunks with 32 bits
    if (d->in_dtype == KDA_BF16 && (double)d->B * (double)d->H * (double)ceil_div(d->T, kChunk) >= 2147483648.0)
        return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

// Checks the kda_gating fields that are set; the tensors' extents are checked by the caller.
kda_status check_gating(const kda_gating* g) {
    if (!g) return KDA_OK;
    if (g->z) {
        if (!g->A_log || !aligned(g->A_log, 4) || !aligned(g->z, 16)) return KDA_ERR_INVALID_ARG;
        if (!(g->g_min < 0.f) || g->g_min < -3.0e38f) return KDA_ERR_INVALID_ARG;   // NaN fails too
    }
    if (g->gate) {
        if (!(g->eps > 0.f) || g->eps > 3.0e38f || !aligned(g->gate, 16)) return KDA_ERR_INVALID_ARG;
        if (g->norm_weight && !aligned(g->norm_weight, 16)) return KDA_ERR_INVALID_ARG;
    }
    return KDA_OK;
}

kda::Gating to_gating(const kda_gating* g) {
    kda::Gating r{};
    if (g) {
        r.z = g->z; r.A_log = g->A_log; r.g_min = g->g_min;
        r.gate = g->gate; r.norm_w = g->norm_weight; r.eps = g->eps;
    }
    return r;
}

kda_status check_varlen_desc(const kda_varlen_desc* d) {
    if (!d) return KDA_ERR_INVALID_ARG;
    if (d->N < 1 || d->H < 1 || d->T < 0 || d->max_len < 0 || d->dk < 1 || d->dv < 1 || d->segments < 0 ||
        d->ckpt_every < 0 || (d->packed != 0 && d->packed != 1) || d->state_pass < 0 || d->state_pass > 2)
        return KDA_ERR_INVALID_ARG;
    if (d->ckpt_every % kChunk != 0) return KDA_ERR_INVALID_ARG;
    if (!valid_dtype(d->in_dtype) || !valid_dtype(d->out_dtype)) return KDA_ERR_INVALID_ARG;
    if (d->chunk != kChunk) return KDA_ERR_UNSUPPORTED;
    if ((d->dk != 64 && d->dk != 128) || (d->dv != 64 && d->dv != 128)) return KDA_ERR_UNSUPPORTED;
    if (d->in_dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (d->state_pass == 2 && (d->dk != 128 || d->dv != 128)) return KDA_ERR_UNSUPPORTED;
    // the state pass addresses one sequence's output rows with 32-bit offsets; slot rows are int32
    const int64_t dmax = d->dk > d->dv ? d->dk : d->dv;
    const int64_t longest = d->packed ? d->max_len : d->T;
    if (longest * dmax * 4 >= ((int64_t)1 << 31) || d->T >= ((int64_t)1 << 31) - 64) return KDA_ERR_UNSUPPORTED;
    const double elems = (double)d->N * (double)d->H * (double)(d->T > 0 ? d->T : 1) * (double)(d->dk + d->dv);
    if (elems > 1e17) return KDA_ERR_INVALID_ARG;
    // the intra-chunk kernel numbers its chunk slots with 32 bits
    const double items = d->packed ? (double)d->H * (double)(d->T / kChunk + d->N)
                                   : (double)d->N * (double)d->H * (double)ceil_div(d->T, kChunk);
    if (items >= 2147483648.0) return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

// Packed batch: T/64 + N record slots per head (the lengths are only known on the device).
// Equal lengths: the fixed-length geometry with B = N.
Geometry varlen_geometry(const kda_varlen_desc* d, int64_t cus) {
    if (!d->packed) {
        const int64_t nchunks = ceil_div(d->T, kChunk);
        Geometry g{d->N * d->H, nchunks, d->N * d->H * nchunks, d->dk, d->dv, d->in_dtype, d->segments, 0,
                   d->N * d->H, cus};
        g.state_pass = d->state_pass;
        g.fused_ok = d->dk == 128 && d->dv == 128;
        return g;
    }
    const int64_t max_len = d->max_len < d->T ? d->max_len : d->T;
    const int64_t max_chunks = ceil_div(max_len, kChunk);
    const int64_t slots = d->T / kChunk + d->N;
    // The split is planned for the lanes that can have max_chunks chunks: at most T / max_len
    // sequences reach max_len (a shorter lane has fewer live segments, and the launches' workgroups
    // of its dead ones return at once). Measured on 12 sequences x 32 heads, 8192 tokens, longest
    // 2500 (96 such lanes: 2 segments): 0.263 ms unsplit, 0.237 ms in 2 segments, 0.242 in 3.
    int64_t can_be_long = max_len > 0 ? d->T / max_len : d->N;
    if (can_be_long < 1) can_be_long = 1;
    if (can_be_long > d->N) can_be_long = d->N;
    Geometry g{d->N * d->H, max_chunks, d->H * slots, d->dk, d->dv, d->in_dtype, d->segments, slots, can_be_long * d->H,
               cus};
    g.state_pass = d->state_pass;
    g.fused_ok = d->dk == 128 && d->dv == 128;
    return g;
}

// Backward workspace, in order: the forward's own workspace (records, pairs, entries), every
// chunk's exit state, the forward's output (discarded), then the backward's per-chunk scratch.
struct BwdPlan {
    Plan fwd;
    int64_t ck_stride;
    size_t ckpt_off, o_off, prep_off, gst_off, dvt_off, ws_bytes;
};

BwdPlan make_bwd_plan(const kda_chunk_desc* d, int64_t cus) {
    BwdPlan b{};
    b.fwd = make_plan(fixed_geometry(d, cus, false));
    const int64_t lanes = d->B * d->H;
    const int64_t nchunks = ceil_div(d->T, kChunk);
    const size_t chunks = (size_t)(lanes * nchunks);
    b.ck_stride = d->T / kChunk;
    auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
    b.ckpt_off = align(b.fwd.ws_bytes);
    b.o_off = align(b.ckpt_off + (size_t)(lanes * b.ck_stride * d->dk * d->dv) * 4);
    b.prep_off = align(b.o_off + (size_t)(lanes * d->T * d->dv) * (size_t)elem_bytes(d->out_dtype));
    b.gst_off = align(b.prep_off + chunks * kda::bwd_prep_floats(d->dk, d->dv) * 4);
    b.dvt_off = align(b.gst_off + chunks * (size_t)(d->dk * d->dv) * 4);
    b.ws_bytes = b.dvt_off + chunks * (size_t)(kChunk * d->dv) * 4;
    return b;
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
        case KDA_ERR_SCRATCH:
            return "KDA_ERR_SCRATCH: the call needs more workspace than the library's fixed scratch "
                   "(KDA_NOALLOC_SCRATCH_BYTES); use kda_chunk_fwd with a workspace";
        default: return "unknown kda_status";
    }
}

const char* kda_version(void) { return "kda-gfx950 0.1.0"; }

size_t kda_chunk_fwd_workspace_bytes(const kda_chunk_desc* d) {
    if (check_chunk_desc(d) != KDA_OK) return 0;
    return make_plan(fixed_geometry(d, current_cus())).ws_bytes;
}

kda_status kda_chunk_fwd(const kda_chunk_desc* d, const void* q, const void* k, const void* v,
                         const void* log_alpha, const void* beta, const float* S0, void* o, float* S_T,
                         void* workspace, size_t workspace_bytes, void* stream) {
    return kda::chunk_fwd_impl(d, q, k, v, log_alpha, beta, S0, o, S_T, workspace, workspace_bytes, stream, nullptr);
}

}  // extern "C"

namespace kda {

// kda_chunk_fwd, or with `scratch_of` set kda_chunk_fwd_noalloc: the workspace is then the fixed
// scratch of the stream's device, looked up only once every argument has passed validation and
// the plan is known to fit it.
kda_status chunk_fwd_impl(const kda_chunk_desc* d, const void* q, const void* k, const void* v,
                          const void* log_alpha, const void* beta, const float* S0, void* o, float* S_T,
                          void* workspace, size_t workspace_bytes, void* stream, void* (*scratch_of)(int)) {
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
    const Range rst = range_of(S_T, S_T ? state_bytes : 0);
    for (const Range& r : rin)
        if (overlaps(ro, r) || overlaps(rst, r)) return KDA_ERR_INVALID_ARG;
    if (S0 && overlaps(ro, range_of(S0, state_bytes))) return KDA_ERR_INVALID_ARG;
    if (S_T && overlaps(ro, range_of(S_T, state_bytes))) return KDA_ERR_INVALID_ARG;

    const int dev = kda::stream_device(st);
    const Plan plan = make_plan(fixed_geometry(d, kda::compute_units(dev)));
    if (scratch_of && plan.ws_bytes > 0) {
        if (plan.ws_bytes > (size_t)KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_SCRATCH;
        workspace = scratch_of(dev);
        if (!workspace) return KDA_ERR_HIP;
        workspace_bytes = (size_t)KDA_NOALLOC_SCRATCH_BYTES;
    }
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
    a.map.H = d->H;
    if (!a.in_bf16) {
        a.fin_seg_lo = 0; a.fin_nseg = 1; a.sum_seg_lo = 0; a.sum_nseg = 0;
        return kda::launch_chunk(a, st) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    return run_bf16(a, plan, static_cast<unsigned char*>(workspace), st);
}

}  // namespace kda

extern "C" {

size_t kda_chunk_fwd_varlen_workspace_bytes(const kda_varlen_desc* d) {
    if (check_varlen_desc(d) != KDA_OK) return 0;
    return make_plan(varlen_geometry(d, current_cus())).ws_bytes;
}

kda_status kda_chunk_fwd_varlen(const kda_varlen_desc* d, const void* q, const void* k, const void* v,
                                const void* log_alpha, const void* beta, const int32_t* cu_seqlens,
                                const float* S0, void* o, float* S_T, float* S_ckpt, int32_t* ckpt_offsets,
                                const kda_gating* gating, void* workspace, size_t workspace_bytes, void* stream) {
    const kda_status ds = check_varlen_desc(d);
    if (ds != KDA_OK) return ds;
    const kda_status gs = check_gating(gating);
    if (gs != KDA_OK) return gs;
    const void* z = gating ? gating->z : nullptr;
    const void* gate = gating ? gating->gate : nullptr;
    const bool packed = d->packed != 0;
    if (packed != (cu_seqlens != nullptr)) return KDA_ERR_INVALID_ARG;
    const int64_t lanes = d->N * d->H;
    const int64_t row_lanes = packed ? d->H : lanes;   // row blocks of the row-major tensors
    const int64_t eout = elem_bytes(d->out_dtype);
    const int64_t state_bytes = lanes * d->dk * d->dv * (int64_t)sizeof(float);
    const int64_t ck_states = d->ckpt_every > 0 ? (packed ? d->T / d->ckpt_every : d->N * (d->T / d->ckpt_every)) * d->H : 0;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);

    if (S0 && !aligned(S0, 16)) return KDA_ERR_INVALID_ARG;
    if (S_T && !aligned(S_T, 16)) return KDA_ERR_INVALID_ARG;
    if (S0 && S_T && S0 != S_T && overlaps(range_of(S0, state_bytes), range_of(S_T, state_bytes)))
        return KDA_ERR_INVALID_ARG;
    if (d->ckpt_every > 0) {
        if (ck_states > 0 && (!S_ckpt || !aligned(S_ckpt, 16))) return KDA_ERR_INVALID_ARG;
        if (packed && !ckpt_offsets) return KDA_ERR_INVALID_ARG;
    }
    if (cu_seqlens && !aligned(cu_seqlens, 4)) return KDA_ERR_INVALID_ARG;
    if (ckpt_offsets && !aligned(ckpt_offsets, 4)) return KDA_ERR_INVALID_ARG;
    const Range rck = range_of(S_ckpt, ck_states * d->dk * d->dv * (int64_t)sizeof(float));
    const Range rcko = range_of(ckpt_offsets, d->ckpt_every > 0 && ckpt_offsets ? (d->N + 1) * 4 : 0);
    const Range rcu = range_of(cu_seqlens, packed ? (d->N + 1) * 4 : 0);
    const Range rs0 = range_of(S0, S0 ? state_bytes : 0), rst = range_of(S_T, S_T ? state_bytes : 0);
    const Range outs[] = {rck, rcko};
    for (const Range& r : outs)
        if (overlaps(r, rs0) || overlaps(r, rst) || overlaps(r, rcu)) return KDA_ERR_INVALID_ARG;
    if (overlaps(rck, rcko) || overlaps(rcu, rst)) return KDA_ERR_INVALID_ARG;

    const Geometry g = varlen_geometry(d, kda::compute_units(kda::stream_device(st)));
    const Plan plan = make_plan(g);
    kda::VarlenPrep vp{};
    vp.cu = cu_seqlens; vp.N = d->N; vp.rows = d->T; vp.max_len = packed ? d->max_len : d->T;
    vp.ck_off = d->ckpt_every > 0 ? ckpt_offsets : nullptr; vp.ck_every = d->ckpt_every;

    if (plan.nchunks == 0) {   // every sequence is empty
        if (vp.ck_off && kda::launch_varlen_prep(vp, st) != hipSuccess) return KDA_ERR_HIP;
        if (!S_T || S_T == S0) return KDA_OK;
        return kda::launch_copy_or_zero(S_T, S0, state_bytes / 4, st) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }

    if (!q || !k || !v || (!log_alpha && !z) || !beta || !o) return KDA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(log_alpha, 16) || !aligned(o, 16) ||
        !aligned(beta, 2))
        return KDA_ERR_INVALID_ARG;
    const int64_t nrow = row_lanes * d->T;
    const Range ro = range_of(o, nrow * d->dv * eout);
    const Range rin[] = {range_of(q, nrow * d->dk * 2), range_of(k, nrow * d->dk * 2), range_of(v, nrow * d->dv * 2),
                         range_of(z ? nullptr : log_alpha, z ? 0 : nrow * d->dk * 2), range_of(beta, nrow * 2), rcu,
                         range_of(z, z ? nrow * d->dk * 2 : 0), range_of(gate, gate ? nrow * d->dv * 2 : 0),
                         range_of(z ? gating->A_log : nullptr, z ? d->H * 4 : 0),
                         range_of(gate ? gating->norm_weight : nullptr, gate && gating->norm_weight ? d->dv * 4 : 0)};
    for (const Range& r : rin)
        if (overlaps(ro, r) || overlaps(rck, r) || overlaps(rcko, r) || overlaps(rst, r)) return KDA_ERR_INVALID_ARG;
    if (overlaps(ro, rs0) || overlaps(ro, rst) || overlaps(ro, rck) || overlaps(ro, rcko)) return KDA_ERR_INVALID_ARG;

    if (!workspace || workspace_bytes < plan.ws_bytes) return KDA_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return KDA_ERR_INVALID_ARG;
    const Range rw = range_of(workspace, (int64_t)plan.ws_bytes);
    if (overlaps(rw, ro) || overlaps(rw, rs0) || overlaps(rw, rst) || overlaps(rw, rck) || overlaps(rw, rcko))
        return KDA_ERR_INVALID_ARG;
    for (const Range& r : rin)
        if (overlaps(rw, r)) return KDA_ERR_INVALID_ARG;

    unsigned char* ws = static_cast<unsigned char*>(workspace);
    kda::ChunkLaunch a{};
    a.lanes = lanes; a.T = d->T; a.dk = d->dk; a.dv = d->dv;
    a.nchunks = plan.nchunks;
    a.in_bf16 = true; a.out_bf16 = d->out_dtype == KDA_BF16;
    a.nseg = plan.nseg; a.chunks_per_seg = plan.chunks_per_seg;
    a.q = q; a.k = k; a.v = v; a.la = log_alpha; a.beta = beta;
    a.S0 = S0; a.o = o; a.S_T = S_T;
    a.map.H = d->H;
    a.gt = to_gating(gating);
    if (packed) {
        a.map.cu = cu_seqlens; a.map.H = d->H; a.map.rows = d->T; a.map.max_len = d->max_len;
        a.map.slots = g.tab_slots;
        vp.slots = g.tab_slots;
        vp.slot_tab = reinterpret_cast<kda::SlotEntry*>(ws + plan.rec_bytes + plan.pair_bytes + plan.entry_bytes);
    }
    if (d->ckpt_every > 0 && ck_states > 0) {
        a.ckpt = S_ckpt; a.ck_chunks = d->ckpt_every / kChunk; a.ck_cap = ck_states;
        a.ck_per_lane = d->T / d->ckpt_every; a.ck_off = ckpt_offsets;
    }
    if ((packed || vp.ck_off) && kda::launch_varlen_prep(vp, st) != hipSuccess) return KDA_ERR_HIP;
    return run_bf16(a, plan, ws, st);
}

size_t kda_chunk_bwd_workspace_bytes(const kda_chunk_desc* d) {
    if (check_chunk_desc(d) != KDA_OK || d->in_dtype != KDA_BF16 || d->T == 0) return 0;
    return make_bwd_plan(d, current_cus()).ws_bytes;
}

kda_status kda_chunk_bwd(const kda_chunk_desc* d, const void* q, const void* k, const void* v,
                         const void* log_alpha, const void* beta, const float* S0, const void* dO,
                         const float* dS_T, float* dq, float* dk, float* dv, float* dlog_alpha, float* dbeta,
                         float* dS0, void* workspace, size_t workspace_bytes, void* stream) {
    const kda_status ds = check_chunk_desc(d);
    if (ds != KDA_OK) return ds;
    if (d->in_dtype != KDA_BF16 || d->state_pass == 2) return KDA_ERR_UNSUPPORTED;
    const int64_t lanes = d->B * d->H;
    const int64_t eout = elem_bytes(d->out_dtype);
    const int64_t state_bytes = lanes * d->dk * d->dv * 4;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if ((S0 && !aligned(S0, 16)) || (dS_T && !aligned(dS_T, 16)) || (dS0 && !aligned(dS0, 16)))
        return KDA_ERR_INVALID_ARG;
    const Range rs0 = range_of(S0, S0 ? state_bytes : 0), rdst = range_of(dS_T, dS_T ? state_bytes : 0);
    const Range rds0 = range_of(dS0, dS0 ? state_bytes : 0);
    if (overlaps(rds0, rs0) || overlaps(rds0, rdst)) return KDA_ERR_INVALID_ARG;
    if (d->T == 0) {   // no tokens: dS0 = dS_T
        if (!dS0) return KDA_OK;
        return kda::launch_copy_or_zero(dS0, dS_T, state_bytes / 4, st) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    if (!q || !k || !v || !log_alpha || !beta || !dO || !dq || !dk || !dv || !dlog_alpha || !dbeta)
        return KDA_ERR_INVALID_ARG;
    // the forward recompute reads q, k, v, log_alpha with the 16-byte loads kda_chunk_fwd needs
    const void* ins[] = {q, k, v, log_alpha, dO};
    for (const void* p : ins)
        if (!aligned(p, 16)) return KDA_ERR_INVALID_ARG;
    const void* outs[] = {dq, dk, dv, dlog_alpha, dbeta};
    for (const void* p : outs)
        if (!aligned(p, 4)) return KDA_ERR_INVALID_ARG;
    if (!aligned(beta, 2)) return KDA_ERR_INVALID_ARG;
    const int64_t nk = lanes * d->T * d->dk, nv = lanes * d->T * d->dv, nt = lanes * d->T;
    const Range rin[] = {range_of(q, nk * 2), range_of(k, nk * 2), range_of(v, nv * 2), range_of(log_alpha, nk * 2),
                         range_of(beta, nt * 2), range_of(dO, nv * eout), rs0, rdst};
    const Range rout[] = {range_of(dq, nk * 4), range_of(dk, nk * 4), range_of(dv, nv * 4),
                          range_of(dlog_alpha, nk * 4), range_of(dbeta, nt * 4), rds0};
    for (int i = 0; i < 6; ++i) {
        for (const Range& r : rin)
            if (overlaps(rout[i], r)) return KDA_ERR_INVALID_ARG;
        for (int j = i + 1; j < 6; ++j)
            if (overlaps(rout[i], rout[j])) return KDA_ERR_INVALID_ARG;
    }
    const BwdPlan bp = make_bwd_plan(d, kda::compute_units(kda::stream_device(st)));
    if (!workspace || workspace_bytes < bp.ws_bytes) return KDA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return KDA_ERR_INVALID_ARG;
    const Range rw = range_of(workspace, (int64_t)bp.ws_bytes);
    for (const Range& r : rin)
        if (overlaps(rw, r)) return KDA_ERR_INVALID_ARG;
    for (const Range& r : rout)
        if (overlaps(rw, r)) return KDA_ERR_INVALID_ARG;

    unsigned char* ws = static_cast<unsigned char*>(workspace);
    // forward recompute: every chunk's exit state into the workspace (lane-major checkpoints)
    kda::ChunkLaunch a{};
    a.lanes = lanes; a.T = d->T; a.dk = d->dk; a.dv = d->dv;
    a.nchunks = bp.fwd.nchunks;
    a.in_bf16 = true; a.out_bf16 = d->out_dtype == KDA_BF16;
    a.nseg = bp.fwd.nseg; a.chunks_per_seg = bp.fwd.chunks_per_seg;
    a.q = q; a.k = k; a.v = v; a.la = log_alpha; a.beta = beta;
    a.S0 = S0; a.o = ws + bp.o_off; a.S_T = nullptr;
    a.map.H = 1;   // checkpoint j of lane l at index l * ck_per_lane + j - 1
    if (bp.ck_stride > 0) {
        a.ckpt = reinterpret_cast<float*>(ws + bp.ckpt_off);
        a.ck_chunks = 1; a.ck_cap = lanes * bp.ck_stride; a.ck_per_lane = bp.ck_stride;
    }
    const kda_status fs = run_bf16(a, bp.fwd, ws, st);
    if (fs != KDA_OK) return fs;
    kda::BwdArgs b{};
    b.lanes = lanes; b.T = d->T; b.nchunks = bp.fwd.nchunks; b.dk = d->dk; b.dv = d->dv;
    b.q = q; b.k = k; b.v = v; b.la = log_alpha; b.beta = beta; b.S0 = S0;
    b.dO = dO; b.dO_bf16 = d->out_dtype == KDA_BF16; b.dST = dS_T;
    b.ckpt = reinterpret_cast<const float*>(ws + bp.ckpt_off); b.ck_stride = bp.ck_stride;
    b.prep = reinterpret_cast<float*>(ws + bp.prep_off);
    b.gst = reinterpret_cast<float*>(ws + bp.gst_off);
    b.dvt = reinterpret_cast<float*>(ws + bp.dvt_off);
    b.dq = dq; b.dk_ = dk; b.dv_ = dv; b.dla = dlog_alpha; b.dbeta = dbeta; b.dS0 = dS0;
    return kda::launch_bwd(b, st) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_decode_step_gated(const kda_decode_desc* d, const void* q, const void* k, const void* v,
                                 const void* log_alpha, const void* beta, const kda_gating* gating, float* S,
                                 void* o, void* stream) {
    if (!d) return KDA_ERR_INVALID_ARG;
    if (d->N < 1 || d->H < 1 || d->dk < 1 || d->dv < 1) return KDA_ERR_INVALID_ARG;
    if (!valid_dtype(d->in_dtype) || !valid_dtype(d->out_dtype)) return KDA_ERR_INVALID_ARG;
    if ((d->dk != 64 && d->dk != 128) || (d->dv != 64 && d->dv != 128)) return KDA_ERR_UNSUPPORTED;
    const kda_status gs = check_gating(gating);
    if (gs != KDA_OK) return gs;
    const void* z = gating ? gating->z : nullptr;
    const void* gate = gating ? gating->gate : nullptr;
    if (!q || !k || !v || (!log_alpha && !z) || !beta || !S || !o) return KDA_ERR_INVALID_ARG;
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
                            range_of(z ? nullptr : log_alpha, z ? 0 : lanes * d->dk * ein),
                            range_of(beta, lanes * ein),
                            range_of(z, z ? lanes * d->dk * ein : 0), range_of(gate, gate ? lanes * d->dv * ein : 0),
                            range_of(z ? gating->A_log : nullptr, z ? d->H * 4 : 0),
                            range_of(gate ? gating->norm_weight : nullptr, gate && gating->norm_weight ? d->dv * 4 : 0)};
    for (const Range& r : others)
        if (overlaps(ro, r)) return KDA_ERR_INVALID_ARG;
    for (int i = 1; i < (int)(sizeof(others) / sizeof(others[0])); ++i)
        if (overlaps(others[0], others[i])) return KDA_ERR_INVALID_ARG;
    kda::DecodeArgs a{};
    a.N = d->N; a.H = d->H; a.dk = d->dk; a.dv = d->dv;
    a.in_bf16 = d->in_dtype == KDA_BF16; a.out_bf16 = d->out_dtype == KDA_BF16;
    a.q = q; a.k = k; a.v = v; a.la = log_alpha; a.beta = beta; a.S = S; a.o = o;
    a.gt = to_gating(gating);
    return kda::launch_decode(a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_decode_step(const kda_decode_desc* d, const void* q, const void* k, const void* v,
                           const void* log_alpha, const void* beta, float* S, void* o, void* stream) {
    return kda_decode_step_gated(d, q, k, v, log_alpha, beta, nullptr, S, o, stream);
}

}  // extern "C"

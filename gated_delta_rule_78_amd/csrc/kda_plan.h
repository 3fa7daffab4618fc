// Launch plan and dispatch of a bf16 prefill call (fixed-length or packed): how many sequence
// segments each lane's state pass is split into, the workspace that plan needs, and the launch
// sequence intra-chunk kernel -> state pass (-> segment scan -> state pass). Internal to the
// library; the C ABI validates arguments before it plans.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "kda.h"
#include "kda_internal.h"

namespace kda {

constexpr int64_t kChunk = 64;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// What a bf16 prefill call covers, for planning: `lanes` (batch or sequence, head) pairs whose
// longest one has `max_chunks` chunks, and `slots` record slots in all.
struct Geometry {
    int64_t lanes, max_chunks, slots, dk, dv;
    int32_t in_dtype, segments;
    int64_t tab_slots;   // slot-table entries (packed batches), 0 otherwise
    int64_t long_lanes;  // lanes that can have max_chunks chunks (plans the sequence split)
    int64_t cus;         // compute units of the device the call runs on
    int32_t state_pass;  // kda_chunk_desc::state_pass (0 = choose, 1 = two kernels, 2 = fused)
    bool fused_ok;       // the call can take the fused kernel (see launch_fused)
};

// Chunks in the window that looks for an exact segment entry state (SplitPass): a decay of
// about e^-16 per chunk per key channel (log alpha averaging -0.25 per token) leaves nothing of
// the state 7 chunks back in fp32.
constexpr int64_t kWindowChunks = 8;

// Segments per lane, chunks per segment and workspace of a prefill call. The workspace holds,
// in this order: records, affine pairs, entry states, slot table, window flags and, for the
// fused plan, the window launch's flags, the list of lanes left to the two-kernel fallback and
// (packed batches) the list of the windows' record slots.
struct Plan {
    bool fused;          // the fused kernel (with the two-kernel path as the fallback of lanes
                         // with an inexact window)
    int nseg;
    int64_t nchunks, chunks_per_seg;
    int64_t win_chunks;  // chunks per window (nseg > 1), kWindowChunks
    size_t rec_bytes;    // intra-chunk records (bf16 path): one per slot
    size_t pair_bytes;   // affine pairs [lanes][nseg][dk][dv + dk] (nseg > 1)
    size_t entry_bytes;  // entry states [lanes][nseg][dk][dv] (nseg > 1)
    size_t tab_bytes;    // slot table (packed batches)
    size_t flag_bytes;   // window flags [lanes][nseg] int32 (nseg > 1)
    size_t pre_bytes;    // fused plan, nseg > 1: the window launch's flags [lanes][nseg] int32
    size_t list_bytes;   // fused plan, nseg > 1: fallback lanes [lanes] int32, then their count
    size_t wlist_bytes;  // fused plan of a packed batch, nseg > 1: the windows' slots, then their count
    size_t ws_bytes;
};

Plan make_plan(const Geometry& g);

// Launch a validated bf16 prefill on `st`: `a` carries the call's tensors and geometry, `ws` the
// workspace of `plan` (at least plan.ws_bytes). Every workspace byte a launch reads was written
// earlier in the same call. Returns KDA_ERR_HIP if a launch fails.
kda_status run_bf16(ChunkLaunch& a, const Plan& plan, unsigned char* ws, hipStream_t st);

// kda_chunk_fwd (scratch_of == NULL) or kda_chunk_fwd_noalloc (scratch_of returns the device address
// of a device's fixed scratch, KDA_NOALLOC_SCRATCH_BYTES long, or NULL on failure).
kda_status chunk_fwd_impl(const kda_chunk_desc* d, const void* q, const void* k, const void* v,
                          const void* log_alpha, const void* beta, const float* S0, void* o, float* S_T,
                          void* workspace, size_t workspace_bytes, void* stream, void* (*scratch_of)(int));

}  // namespace kda

// Internal launcher interfaces between the C ABI layer (kda_abi.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Fused prologue / epilogue (kda_gating), all NULL when not asked for: with z, the log decay is
// g_min * sigmoid(exp(A_log[h]) * z); with gate, o receives sigmoid(gate) * w * o * rstd(o).
struct Gating {
    const void* z;
    const float* A_log;
    float g_min, eps;
    const void* gate;
    const float* norm_w;
};

struct DecodeArgs {
    int64_t N, H, dk, dv;
    bool in_bf16, out_bf16;
    const void *q, *k, *v, *la, *beta;
    float* S;
    void* o;
    Gating gt;
};

// Where the rows of one lane live. Fixed-length batches: lane = b*H + h owns rows
// [lane*T, lane*T + T) of q, k, v, log_alpha, beta and o, and records [lane*nchunks, ...).
// Packed variable-length batches (cu != NULL): lane = s*H + h, sequence s is rows
// [cu[s], cu[s+1]) of head h's block of `rows` rows, and its chunk c has record slot
// h*slots + cu[s]/64 + s + c (a slot index that never collides, whatever the lengths).
struct SeqMap {
    const int32_t* cu;      // [N + 1] device cumulative lengths, or NULL for equal lengths T
    int64_t H;              // heads (lanes = N * H; set in both modes)
    int64_t rows;           // packed rows per head (cu != NULL) or T
    int64_t max_len;        // longest sequence processed (longer ones are cut to it)
    int64_t slots;          // record slots per head (cu != NULL) or per lane (= nchunks)
};

// Per-chunk slot table entry of a packed batch: first row of the chunk inside its head's block
// and the number of valid rows (0 for a slot no chunk owns).
struct SlotEntry {
    int32_t row0, nrows;
};

// Launches of a sequence split (ChunkLaunch::split; kda_plan.cpp runs them in this order):
//   kPassWindowFinish  FINISH of every segment of every lane. A segment s > 0 first runs the
//                SUMMARY products over the last win_chunks chunks of the lane before it (from the
//                lane's first chunk, with S0, if the window reaches it). When the window's
//                transition M is exactly zero in fp32 (or the window starts at chunk 0), its S~ is
//                the segment's exact entry state and the segment goes on from it; otherwise the
//                workgroup computes the segment's affine pair (s < nseg - 1). Flag [lane][s - 1]
//                says which (1: exact). Segment 0 also stores its exit state (segment 1's entry).
//   kPassCarry   SUMMARY of segments 1 .. nseg - 2 whose flag is 1, in lanes with a flag 0.
//   (segment scan, skipped by lanes whose flags are all 1)
//   kPassFinish  FINISH of segments 1 .. nseg - 1 whose flag is 0, from the scanned entry states.
// kPassAll is a single-segment call (and the fp32 path).
// The fused plan (launch_fused) runs the windows first, on their own: kPassWindow runs the window
// before each boundary s = 1 .. nseg - 1 (the FINISH blocks of segments 1 .. nseg - 1), stores its
// flag and S~ (the segment's entry state where the flag is 1) and nothing else. The fused kernel
// then finishes every lane whose flags are all 1, and the launches above run the other lanes
// (ChunkLaunch::skip_flag).
enum SplitPass { kPassAll = 0, kPassWindowFinish = 1, kPassCarry = 2, kPassFinish = 3, kPassWindow = 4 };

// One launch of the chunk kernels. Blocks [0, n_fin) run FINISH work (exact entry state, write
// o and, for the lane's last segment, S_T); the following n_sum blocks run SUMMARY work (affine
// pair of a segment, no o). Every segment covers `chunks_per_seg` chunks of 64 tokens; the last
// segment of a lane runs to the lane's last chunk. A packed lane shorter than the plan's longest
// has fewer segments (ceil(chunks / chunks_per_seg), at least 1): the later ones do nothing,
// and their window flags are set (exact).
struct ChunkLaunch {
    int64_t lanes, T, dk, dv;
    int64_t nchunks;
    bool in_bf16, out_bf16;
    int nseg;               // segments per lane
    int64_t chunks_per_seg;
    int fin_seg_lo, fin_nseg;   // FINISH segments [fin_seg_lo, fin_seg_lo + fin_nseg)
    int sum_seg_lo, sum_nseg;   // SUMMARY segments [sum_seg_lo, sum_seg_lo + sum_nseg)
    const void *q, *k, *v, *la, *beta;
    const float* S0;        // entry state of segment 0 (NULL = zero)
    void* o;
    float* S_T;             // exit state of the last segment (NULL = not stored)
    const unsigned char* rec;   // intra-chunk records (bf16 path), see SeqMap
    float* ws_pair;         // [lanes][nseg][dk][dv + dk]   affine pairs [S~ | M]
    float* ws_entry;        // [lanes][nseg][dk][dv]        exact entry state of each segment
    int32_t* ws_flag;       // [lanes][nseg]                window flags (see SplitPass)
    int split;              // SplitPass of this launch
    int64_t win_chunks;     // kPassWindowFinish, kPassWindow: chunks per window
    // [lanes][nseg] flags of a kPassWindow launch, or NULL: lanes whose flags there are all 1 were
    // finished by the fused kernel, and the launches of a two-kernel split skip them.
    const int32_t* skip_flag;
    SeqMap map;
    // State checkpoints (bf16 path): after every ck_chunks chunks of a lane (s, h), the state
    // goes to ckpt[(ck_off[s] + j - 1) * H + h] (packed) or ckpt[(s * ck_per_lane + j - 1) * H + h]
    // (equal lengths), dk x dv fp32 each, with H = map.H; indices at or beyond ck_cap states are
    // dropped.
    float* ckpt;            // NULL = no checkpoints
    int64_t ck_chunks, ck_cap, ck_per_lane;
    const int32_t* ck_off;  // [N + 1] (packed batches)
    Gating gt;              // the epilogue fields are read by the state pass
};

// The intra-chunk kernel over every record slot (bf16 inputs): slots = map.slots per head of
// map.H heads (packed) or per lane of `lanes` lanes (fixed).
struct IntraArgs {
    int64_t lanes, T, nchunks, dk, dv;
    const void *q, *k, *v, *la, *beta;
    unsigned char* rec;     // record_bytes(dk, dv) per slot
    const SlotEntry* slot_tab;  // [map.slots] for a packed batch, NULL for a fixed one
    SeqMap map;
    Gating gt;              // the prologue fields are read by the intra-chunk kernel
    // Subsets of a fixed-length batch's chunks (both off: every chunk). With win_chunks > 0, only
    // the chunks of the windows before segment boundaries 1 .. nseg - 1 (chunks_per_seg chunks per
    // segment; see SplitPass). With lane_list set, only the lanes lane_list[0 .. *lane_count)
    // (both device memory).
    int64_t win_chunks, chunks_per_seg;
    int nseg;
    const int32_t* lane_list;
    const int32_t* lane_count;
    // Packed batch: with slot_list set, only the record slots slot_list[0 .. *slot_count) (global
    // indices h * slots + j). With run_if set, the launch does nothing when *run_if is 0.
    const int32_t* slot_list;
    const int32_t* slot_count;
    const int32_t* run_if;
};

// The record slots of a packed batch that the windows before segment boundaries 1 .. nseg - 1
// read (kPassWindow; every window ends at its segment's first chunk, and a boundary at or past
// the sequence's last chunk has none), each once, in increasing (lane, boundary, chunk) order:
// list[0 .. *count).
struct WindowSlots {
    const int32_t* cu;
    int64_t N, H, rows, max_len, slots;
    int nseg;
    int64_t chunks_per_seg, win_chunks;
    int32_t* list;
    int32_t* count;
};
hipError_t launch_window_slots(const WindowSlots& a, hipStream_t st);

// Slot table and checkpoint offsets of a packed batch.
struct VarlenPrep {
    const int32_t* cu;
    int64_t N, rows, max_len, slots;
    SlotEntry* slot_tab;    // [slots]
    int32_t* ck_off;        // [N + 1] or NULL
    int64_t ck_every;       // tokens per checkpoint (> 0 when ck_off is set)
};

// Backward of chunkwise prefill (bf16 inputs, fp32 gradients), after a forward recompute that
// stored every chunk's exit state in ckpt ([lanes][ck_stride] states, dk x dv each).
struct BwdArgs {
    int64_t lanes, T, nchunks, dk, dv;
    const void *q, *k, *v, *la, *beta;   // bf16 [lanes][T][d]
    const float* S0;                      // [lanes][dk][dv] or NULL (zero)
    const void* dO;                       // [lanes][T][dv], bf16 or fp32
    bool dO_bf16;
    const float* dST;                     // [lanes][dk][dv] or NULL (zero)
    const float* ckpt;                    // forward exit state of chunk c at [lane * ck_stride + c]
    int64_t ck_stride;
    float* prep;                          // [lanes * nchunks][bwd_prep_floats]
    float* gst;                           // [lanes * nchunks][dk][dv]  exit-state gradient of each chunk
    float* dvt;                           // [lanes * nchunks][64][dv]  dV~ of each chunk
    float *dq, *dk_, *dv_, *dla, *dbeta, *dS0;   // outputs (dS0 may be NULL)
};
size_t bwd_prep_floats(int64_t dk, int64_t dv);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t st);

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);
// fp32-input prefill (one pass, generic chunk kernel).
hipError_t launch_chunk(const ChunkLaunch& a, hipStream_t st);
// bf16-input prefill: records of every chunk, then the inter-chunk state pass.
hipError_t launch_intra(const IntraArgs& a, hipStream_t st);
// The device a stream launches on (the current device for the null stream), and the number of
// compute units of a device (cached per device; 256 if the runtime cannot tell).
int stream_device(hipStream_t st);
int compute_units(int dev);
hipError_t launch_inter(const ChunkLaunch& a, hipStream_t st);
// The fused single-pass prefill (bf16, dk = dv = 128, lanes of equal length; checkpoints and the
// fused gating as ChunkLaunch says): one workgroup per (lane, segment) builds each chunk's record
// in LDS and runs the state step on it;
// segments s > 0 start from ws_entry (a kPassWindow launch), and lanes with an inexact window
// (ws_flag) are left alone.
hipError_t launch_fused(const ChunkLaunch& a, hipStream_t st);
// The lanes whose flags [lanes][nseg] are not all 1, in increasing order: list[0 .. *count).
hipError_t launch_fallback_lanes(const int32_t* flag, int64_t lanes, int nseg, int32_t* list, int32_t* count,
                                 hipStream_t st);
// entry_{s+1} = S~_s + M_s entry_s for s in [1, nseg-1), entry_1 already stored.
hipError_t launch_segment_scan(const ChunkLaunch& a, hipStream_t st);
hipError_t launch_varlen_prep(const VarlenPrep& a, hipStream_t st);
// dst[i] = src ? src[i] : 0 for n floats (graph-capture safe replacement for memcpy/memset).
hipError_t launch_copy_or_zero(float* dst, const float* src, int64_t n, hipStream_t st);

}  // namespace kda

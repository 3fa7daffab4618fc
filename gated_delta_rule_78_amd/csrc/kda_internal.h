// Internal launcher interfaces between the C ABI layer (kda_abi.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct DecodeArgs {
    int64_t N, H, dk, dv;
    bool in_bf16, out_bf16;
    const void *q, *k, *v, *la, *beta;
    float* S;
    void* o;
};

// One launch of the chunk kernels. Blocks [0, n_fin) run FINISH work (exact entry state, write
// o and, for the last segment, S_T); the following n_sum blocks run SUMMARY work (affine pair
// of a segment, no o). Every segment covers `chunks_per_seg` chunks of 64 tokens.
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
    const unsigned char* rec;   // [lanes][nchunks] intra-chunk records (bf16 path)
    float* ws_pair;         // [lanes][nseg][dk][dv + dk]   affine pairs [S~ | M]
    float* ws_entry;        // [lanes][nseg][dk][dv]        exact entry state of each segment
};

// The intra-chunk kernel over every chunk of every lane (bf16 inputs).
struct IntraArgs {
    int64_t lanes, T, nchunks, dk, dv;
    const void *q, *k, *v, *la, *beta;
    unsigned char* rec;     // [lanes][nchunks] records, record_bytes(dk, dv) each
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);
// fp32-input prefill (one pass, generic chunk kernel).
hipError_t launch_chunk(const ChunkLaunch& a, hipStream_t st);
// bf16-input prefill: records of every chunk, then the inter-chunk state pass.
hipError_t launch_intra(const IntraArgs& a, hipStream_t st);
hipError_t launch_inter(const ChunkLaunch& a, hipStream_t st);
// entry_{s+1} = S~_s + M_s entry_s for s in [1, nseg-1), entry_1 already stored.
hipError_t launch_segment_scan(const ChunkLaunch& a, hipStream_t st);
// dst[i] = src ? src[i] : 0 for n floats (graph-capture safe replacement for memcpy/memset).
hipError_t launch_copy_or_zero(float* dst, const float* src, int64_t n, hipStream_t st);

}  // namespace kda

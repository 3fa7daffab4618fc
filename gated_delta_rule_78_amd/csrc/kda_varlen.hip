// Set-up of a packed batch of variable-length sequences for the bf16 prefill: the record-slot
// table that the intra-chunk kernel walks, and the per-sequence checkpoint offsets (also for a
// batch of equal lengths, cu == NULL, where only the offsets are made).
//
// Sequence s is rows [cu[s], cu[s+1]) of every head's block of `rows` rows. Its chunk c (64
// rows, the last one ragged) gets record slot start(s) + c with start(s) = cu[s]/64 + s: the
// slots of consecutive sequences never overlap (a sequence of length L starting at row r spans
// at most ceil(L/64) <= (r+L)/64 - r/64 + 1 slots), and the highest slot is below
// rows/64 + N, so a head needs rows/64 + N slots whatever the lengths. A slot no chunk owns
// (at most one per sequence) gets nrows = 0, and the intra-chunk kernel writes a zero record
// there that no state pass reads.
//
// cu is clamped exactly as the state pass clamps it (rows into [0, rows], lengths to max_len),
// so malformed lengths give wrong numbers but never an access outside the tensors.
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void seq_rows(const VarlenPrep& p, int64_t s, int64_t& c0, int64_t& len) {
    if (!p.cu) {   // N sequences of `rows` tokens each (checkpoint offsets only)
        c0 = s * p.rows;
        len = p.rows;
        return;
    }
    int64_t a = p.cu[s], b = p.cu[s + 1];
    a = a < 0 ? 0 : (a > p.rows ? p.rows : a);
    b = b < a ? a : (b > p.rows ? p.rows : b);
    c0 = a;
    len = b - a < p.max_len ? b - a : p.max_len;
}

// Block 0: exclusive scan of floor(len_s / ck_every) into ck_off[0..N] (when asked for).
// Blocks 1..: one slot per thread; the owner is the last sequence whose first slot is <= j.
__global__ __launch_bounds__(kThreads) void varlen_prep_kernel(VarlenPrep p) {
    if (blockIdx.x == 0) {
        if (!p.ck_off) return;
        __shared__ int64_t part[kThreads];
        int64_t carry = 0;
        for (int64_t base = 0; base < p.N; base += kThreads) {
            const int64_t s = base + threadIdx.x;
            int64_t v = 0;
            if (s < p.N) {
                int64_t c0, len;
                seq_rows(p, s, c0, len);
                v = len / p.ck_every;
            }
            part[threadIdx.x] = v;
            __syncthreads();
            for (int d = 1; d < kThreads; d <<= 1) {   // inclusive Hillis-Steele scan
                const int64_t add = threadIdx.x >= (unsigned)d ? part[threadIdx.x - d] : 0;
                __syncthreads();
                part[threadIdx.x] += add;
                __syncthreads();
            }
            if (s < p.N) p.ck_off[s] = (int32_t)(carry + part[threadIdx.x] - v);
            carry += part[kThreads - 1];
            __syncthreads();
        }
        if (threadIdx.x == 0) p.ck_off[p.N] = (int32_t)carry;
        return;
    }
    const int64_t j = (int64_t)(blockIdx.x - 1) * kThreads + threadIdx.x;
    if (j >= p.slots) return;
    // largest s in [0, N) with start(s) <= j (start(0) = 0 <= j)
    int64_t lo = 0, hi = p.N - 1;
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        int64_t c0, len;
        seq_rows(p, mid, c0, len);
        if ((c0 >> 6) + mid <= j) lo = mid; else hi = mid - 1;
    }
    int64_t c0, len;
    seq_rows(p, lo, c0, len);
    const int64_t c = j - ((c0 >> 6) + lo);
    SlotEntry e{0, 0};
    if (c >= 0 && c * 64 < len) {
        e.row0 = (int32_t)(c0 + 64 * c);
        e.nrows = (int32_t)(len - 64 * c < 64 ? len - 64 * c : 64);
    }
    p.slot_tab[j] = e;
}

// One workgroup: the window slots of every lane (WindowSlots). Candidate u = ((lane * (nseg - 1)
// + b - 1) * win + r) is chunk b * cps - win + r of the lane's sequence; it is kept when boundary b
// lies inside the sequence's n_s chunks (b * cps < n_s: the boundaries past a shorter sequence's
// end have no window), when it is >= 0, and when it is not already in boundary b - 1's window
// (>= (b - 1) * cps).
__global__ __launch_bounds__(1024, 1) void window_slots_kernel(WindowSlots p) {
    __shared__ int32_t pre[1024];
    const int64_t lanes = p.N * p.H;
    const int64_t per_lane = (int64_t)(p.nseg - 1) * p.win_chunks;
    const int64_t total = lanes * per_lane;
    VarlenPrep vp{};
    vp.cu = p.cu; vp.rows = p.rows; vp.max_len = p.max_len;
    int32_t base = 0;
    for (int64_t u0 = 0; u0 < total; u0 += 1024) {
        const int64_t u = u0 + threadIdx.x;
        int32_t slot = -1;
        if (u < total) {
            const int64_t lane = u / per_lane, rest = u % per_lane;
            const int64_t b = 1 + rest / p.win_chunks, r = rest % p.win_chunks;
            const int64_t s = lane / p.H, h = lane % p.H;
            int64_t c0, len;
            seq_rows(vp, s, c0, len);
            const int64_t n = (len + 63) / 64;
            const int64_t cb = b * p.chunks_per_seg, cp = cb - p.chunks_per_seg;
            const int64_t c = cb - p.win_chunks + r;
            if (cb < n && c >= 0 && c >= cp) slot = (int32_t)(h * p.slots + (c0 >> 6) + s + c);
        }
        const int32_t need = slot >= 0 ? 1 : 0;
        pre[threadIdx.x] = need;
        __syncthreads();
        for (int d = 1; d < 1024; d <<= 1) {   // inclusive Hillis-Steele scan
            const int32_t x = threadIdx.x >= (unsigned)d ? pre[threadIdx.x - d] : 0;
            __syncthreads();
            pre[threadIdx.x] += x;
            __syncthreads();
        }
        if (need) p.list[base + pre[threadIdx.x] - 1] = slot;
        base += pre[1023];
        __syncthreads();
    }
    if (threadIdx.x == 0) *p.count = base;
}

}  // namespace

hipError_t launch_window_slots(const WindowSlots& a, hipStream_t st) {
    hipLaunchKernelGGL(window_slots_kernel, dim3(1), dim3(1024), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_varlen_prep(const VarlenPrep& a, hipStream_t st) {
    const int64_t blocks = 1 + (a.slots + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(varlen_prep_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace kda

/*
 * kda.h -- C ABI of the Kimi Delta Attention (KDA) hot path for AMD Instinct MI355X (gfx950).
 *
 * The operation (Kimi K3 reading notes, liuzhao09.github.io/papers/kimi-k3.html, section 2.2,
 * state recurrence equation): per (batch b, head h) lane a fixed-size state S in R^{dk x dv}
 * (rows are key channels) evolves token by token as
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T q_t,
 *
 * with per-channel retention alpha_t = exp(log_alpha_t) in (0,1]^{dk} and write strength beta_t.
 * Prefill evaluates it in the chunkwise form of the same section (cumulative decay
 * gamma^{i->j}, UT transform, causal matrix including the diagonal); decode applies one step.
 * The carried initial / final state is the KDA checkpoint restored at a prefix-cache hit
 * (section 2.5, Figure 12).
 *
 * Conventions shared by every entry point
 *  - All data pointers are DEVICE pointers, owned by the caller, who allocates and frees them.
 *    The library never allocates device memory, never synchronises and keeps no per-call state.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default stream). A returned
 *    KDA_OK means the work was enqueued; a kernel fault surfaces at the caller's next sync.
 *  - Arguments are validated before any device work. On any error nothing is enqueued and
 *    no output is touched. No entry point aborts or throws.
 *  - Element types: kda_dtype. Inputs q,k,v,log_alpha,beta share `in_dtype`; the output o
 *    uses `out_dtype`; states (S0, S_T, S) are always fp32.
 *  - q and k are used as given (the library does not L2-normalise them); no 1/sqrt(d) scale.
 *  - Every tensor is dense and row-major with the last dimension contiguous; tensor base
 *    pointers must be 16-byte aligned (beta: aligned to its element size).
 *  - Decay domain: log_alpha must lie in [-5, 0] (the lower bound g_min = -5 of the decay
 *    equation in section 2.2); bf16 prefill and decode accept the whole domain. The fp32
 *    prefill path (dk = 64) additionally requires every per-channel sum of log_alpha over one
 *    64-token chunk to be >= -80 (true whenever log_alpha >= -1.25). Outside these ranges
 *    results are undefined (no check is made: it would need a pass over the data).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = -1, /* null/negative/misaligned/overlapping argument            */
    KDA_ERR_UNSUPPORTED = -2, /* well-formed but not implemented (e.g. dk not in {64,128}) */
    KDA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than the query reports      */
    KDA_ERR_HIP = -4,         /* the HIP runtime reported an error while enqueuing        */
    KDA_ERR_SCRATCH = -5      /* kda_chunk_fwd_noalloc: the call needs more workspace than
                                 the library's fixed scratch (KDA_NOALLOC_SCRATCH_BYTES)  */
} kda_status;

typedef enum kda_dtype {
    KDA_F32 = 0,  /* IEEE fp32                                    */
    KDA_BF16 = 1  /* bfloat16 (round-to-nearest-even on output)   */
} kda_dtype;

/* Shape and types of one chunkwise prefill call. */
typedef struct kda_chunk_desc {
    int64_t B;          /* batch, >= 1                                                   */
    int64_t H;          /* heads, >= 1                                                   */
    int64_t T;          /* tokens per lane, >= 0; a ragged last chunk is fine; bf16 inputs
                           need T * max(dk,dv) * 4 < 2^31 (T < 4,194,304 at d = 128)     */
    int64_t dk;         /* key dimension: 64 or 128                                      */
    int64_t dv;         /* value dimension: 64 or 128                                    */
    int32_t chunk;      /* chunk length C: must be 64                                    */
    int32_t in_dtype;   /* kda_dtype of q,k,v,log_alpha,beta (KDA_F32 needs dk == 64)    */
    int32_t out_dtype;  /* kda_dtype of o                                                */
    int32_t segments;   /* sequence segments per lane: 0 = library's choice, n >= 1 = n  */
    int32_t state_pass; /* bf16 inputs: 0 = library's choice; 1 = two kernels (every chunk's
                           factors through the workspace); 2 = the fused kernel (dk = dv =
                           128 only, else KDA_ERR_UNSUPPORTED). kda_chunk_bwd uses 1 for its
                           forward and accepts 0 or 1. The fp32 path ignores it.         */
} kda_chunk_desc;

/* Shape and types of one decode step over N independent sequences. */
typedef struct kda_decode_desc {
    int64_t N;          /* sequences, >= 1                 */
    int64_t H;          /* heads, >= 1                     */
    int64_t dk;         /* key dimension: 64 or 128        */
    int64_t dv;         /* value dimension: 64 or 128      */
    int32_t in_dtype;   /* kda_dtype of q,k,v,log_alpha,beta */
    int32_t out_dtype;  /* kda_dtype of o                  */
} kda_decode_desc;

/*
 * Bytes of device workspace kda_chunk_fwd needs for `desc` (0 when the call needs none, and
 * 0 for an invalid desc). For bf16 inputs the workspace holds, in this order:
 *  - one record per 64-token chunk of every (b,h) lane: the chunk's state-independent factors
 *    W = (I+A_kk)^{-1} Diag(beta) K~, U = (I+A_kk)^{-1} Diag(beta) V, Q~, K- = K gamma_C / Gamma,
 *    A_qk and gamma_C (the UT transform and decay factors of section 2.2 of the Kimi K3 reading
 *    notes), (12 dk/32 + 7 + 2 dv/16) KiB per chunk, about 1.1x the bytes of q, k, v and
 *    log_alpha together;
 *  - with more than one sequence segment per lane, per-segment affine pairs (M, S~) with
 *    S_out = S~ + M S_in and the exact entry state of each segment (section 2.5: segment
 *    transforms compose associatively, and a prefix scan gives every segment its entry state),
 *    then one 4-byte flag per (lane, segment). The library first runs each segment boundary's
 *    last 8 chunks from a zero state; where the decay drives that window's M to exactly zero
 *    in fp32, the window's S~ is the boundary's exact state and the lane needs neither the
 *    full-length affine pairs nor the scan;
 *  - with the fused kernel (state_pass, or the library's choice for long lanes) and more than one
 *    segment, the window launch's own flags (4 bytes per lane and segment) and the list of lanes
 *    with an inexact window (4 bytes per lane, then the count; 16-byte multiple). The fused kernel
 *    keeps every chunk's factors in on-chip memory; the records are still reserved, for the lanes
 *    that fall back to the two-kernel path, and only the windows' chunks are written otherwise.
 * The fp32 path needs no workspace.
 */
size_t kda_chunk_fwd_workspace_bytes(const kda_chunk_desc* desc);

/*
 * Chunkwise KDA prefill: kda_chunk_fwd(q,k,v,log_alpha,beta,S0) -> (o, S_T).
 *   q, k, log_alpha : [B,H,T,dk] in_dtype      v : [B,H,T,dv] in_dtype
 *   beta            : [B,H,T]    in_dtype      o : [B,H,T,dv] out_dtype (written)
 *   S0              : [B,H,dk,dv] fp32 entry state, or NULL for the zero state
 *   S_T             : [B,H,dk,dv] fp32 state after token T-1 (written), or NULL to skip;
 *                     may be the same pointer as S0 (in-place update), must not partially
 *                     overlap it
 *   workspace       : at least kda_chunk_fwd_workspace_bytes(desc) bytes (may be NULL if 0)
 * Neither o nor S_T may overlap an input. T == 0 writes S_T = S0 (or zeros) and touches nothing else.
 * Source: section 2.2 (recurrence and chunk equations) and section 2.5 (affine pair,
 * in-device sequence split) of the Kimi K3 reading notes.
 */
kda_status kda_chunk_fwd(const kda_chunk_desc* desc,
                         const void* q, const void* k, const void* v,
                         const void* log_alpha, const void* beta,
                         const float* S0, void* o, float* S_T,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_fwd without a workspace argument, for callers that cannot allocate device memory
 * (code under stream capture, tight serving loops, harnesses that forbid allocation). Same
 * arguments, layouts, validation and results as kda_chunk_fwd (the same kernels and plan); the
 * workspace kda_chunk_fwd_workspace_bytes(desc) reports is taken from a scratch array of
 * KDA_NOALLOC_SCRATCH_BYTES that the library owns: one copy per device, allocated when the
 * library's code is loaded on that device and held until the process ends. The call allocates
 * nothing. A call that needs more returns KDA_ERR_SCRATCH (about 2,700 chunk records at
 * d = 128: e.g. 32 heads x 5,500 tokens, or 8 heads x 22,000 tokens, with the library's plan).
 * Every call on one device shares that device's scratch: calls that overlap in time on one
 * device (two streams, or two host threads) race and give undefined results; serialise them.
 * No part of the scratch needs clearing: each call writes every scratch byte it reads first.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (192u << 20)
kda_status kda_chunk_fwd_noalloc(const kda_chunk_desc* desc,
                                 const void* q, const void* k, const void* v,
                                 const void* log_alpha, const void* beta,
                                 const float* S0, void* o, float* S_T, void* stream);

/*
 * Optional fused prologue and epilogue around the KDA core (section 2.2 of the Kimi K3 reading
 * notes: the decay lower-bound equation, and the per-head RMSNorm with the full-rank sigmoid
 * output gate that follow the core). Only their elementwise parts: the projections that produce
 * z and the gate pre-activation, and W_o after the gate, are the caller's.
 *  Prologue (z != NULL): the per-channel log decay is computed from the decay pre-activation z
 *    (same shape and type as log_alpha, which is then ignored and may be NULL) as
 *        g = g_min * sigmoid(exp(A_log[h]) * z),   alpha = exp(g),
 *    in fp32; g_min < 0 (K3 uses -5; every g then lies in (g_min, 0), inside the decay domain when
 *    g_min >= -5). The bf16 prefill rounds g to bf16 before its cumulative sum, as a bf16
 *    log_alpha input would be; decode keeps it in fp32.
 *  Epilogue (gate != NULL): o receives, instead of the core output o_t,
 *        y_t = sigmoid(gate_t) * norm_weight * o_t / sqrt(mean(o_t^2) + eps)
 *    per (token, head), the mean over the dv columns of the head (gate: same shape and type as v;
 *    norm_weight: [dv] fp32 shared by the heads, NULL = ones; eps > 0), computed from the fp32
 *    core output before o is rounded.
 */
typedef struct kda_gating {
    const void* z;              /* decay pre-activation, or NULL = use log_alpha              */
    const float* A_log;         /* [H] fp32 head-wise log scale (required with z)            */
    float g_min;                /* decay lower bound, < 0 (required with z)                   */
    float eps;                  /* RMSNorm epsilon, > 0 (required with gate)                  */
    const void* gate;           /* gate pre-activation W_g x, or NULL = no epilogue           */
    const float* norm_weight;   /* [dv] fp32 RMSNorm weight, or NULL = ones                   */
} kda_gating;

/* Shape and types of one prefill call over a batch of sequences with checkpoints. */
typedef struct kda_varlen_desc {
    int64_t N;          /* sequences, >= 1                                                */
    int64_t H;          /* heads, >= 1                                                    */
    int64_t T;          /* packed: rows per head (= cu_seqlens[N]); else tokens per
                           sequence. >= 0                                                 */
    int64_t max_len;    /* packed: bound on every sequence length (plans the sequence
                           split); ignored otherwise. max_len * max(dk,dv) * 4 < 2^31     */
    int64_t dk;         /* key dimension: 64 or 128                                       */
    int64_t dv;         /* value dimension: 64 or 128                                     */
    int32_t chunk;      /* chunk length C: must be 64                                     */
    int32_t in_dtype;   /* must be KDA_BF16                                               */
    int32_t out_dtype;  /* kda_dtype of o                                                 */
    int32_t segments;   /* sequence segments per lane: 0 = library's choice, n >= 1 = n   */
    int32_t ckpt_every; /* 0 = no checkpoints, else a positive multiple of 64 (e.g. 512)  */
    int32_t packed;     /* 1: sequences packed along T, described by cu_seqlens;
                           0: N sequences of T tokens in kda_chunk_fwd's layout (B = N)   */
    int32_t state_pass; /* as kda_chunk_desc::state_pass; 2 (the fused kernel) needs
                           dk = dv = 128, else KDA_ERR_UNSUPPORTED                        */
} kda_varlen_desc;

/* Bytes of device workspace kda_chunk_fwd_varlen needs for `desc` (0 for an invalid desc).
 * The same records, affine pairs, entry states and flags as kda_chunk_fwd's workspace; a packed
 * batch lays out records in T/64 + N chunk slots per head (sequence s's chunk c in slot
 * cu_seqlens[s]/64 + s + c, which never collide whatever the lengths) and adds a table of
 * 8 bytes per slot (before the flags). A packed batch on the fused kernel with more than one
 * segment also lists the record slots of the windows (4 bytes per lane, boundary and window
 * chunk, then the count; at the end). The segments are planned for the longest sequence
 * (max_len); a shorter sequence ends in an earlier segment, which finishes it. */
size_t kda_chunk_fwd_varlen_workspace_bytes(const kda_varlen_desc* desc);

/*
 * Chunkwise KDA prefill over a batch of sequences, with state checkpoints:
 * kda_chunk_fwd_varlen(q,k,v,log_alpha,beta,cu_seqlens,S0) -> (o, S_T, S_ckpt, ckpt_offsets).
 * Each (sequence s, head h) pair is an independent lane computing exactly what
 * kda_chunk_fwd computes for one lane (its chunks start at the sequence's first token).
 *  packed = 1: q, k, log_alpha : [H,T,dk] bf16   v : [H,T,dv] bf16   beta : [H,T] bf16
 *              o : [H,T,dv] out_dtype. Sequence s is rows cu_seqlens[s] .. cu_seqlens[s+1]-1
 *              of every head (the [1,H,T,d] tensors of kda_chunk_fwd with the sequences
 *              back to back along T). cu_seqlens: DEVICE int32 [N+1], cu_seqlens[0] = 0,
 *              non-decreasing, cu_seqlens[N] = T, every length <= max_len. The library reads
 *              it on the device only. Lengths that break these rules give undefined numbers but
 *              no access outside the tensors (rows are clamped into [0, T], lengths cut to
 *              max_len; o rows past a cut length are left untouched).
 *  packed = 0: cu_seqlens must be NULL; tensors as kda_chunk_fwd with B = N.
 *  S0, S_T    : [N,H,dk,dv] fp32 as in kda_chunk_fwd (S0 NULL = zero state, S_T NULL = skip,
 *               S_T may be S0).
 *  Checkpoints (ckpt_every = E > 0): after every E tokens of a sequence (tokens counted from
 *  the sequence's first row, i.e. from the state S0 stands for), the state of every head is
 *  written: for sequence s and j = 1 .. floor(len_s / E), the state after its first j*E tokens
 *  goes to S_ckpt[(ckpt_offsets[s] + j - 1) * H + h] (dk x dv fp32 each): one checkpoint holds
 *  all heads of a sequence at one endpoint, the unit a prefix cache restores. ckpt_offsets
 *  (DEVICE int32 [N+1], written) receives the exclusive prefix sum of floor(len_s / E), its
 *  last entry the total. S_ckpt must hold floor(T/E) * H states (packed) or N * floor(T/E) * H
 *  (packed = 0); checkpoints beyond that capacity are dropped. With packed = 0, ckpt_offsets
 *  may be NULL (its values are s * floor(T/E)); with packed = 1 it is required.
 *  With E = 0, S_ckpt and ckpt_offsets are ignored.
 *  gating     : fused prologue / epilogue (see kda_gating), or NULL for none; the head of
 *               A_log[h] is the lane's head in both layouts.
 *  workspace  : at least kda_chunk_fwd_varlen_workspace_bytes(desc) bytes.
 * No output may overlap an input or another output (S_T = S0 aside). A call whose sequences
 * are all empty writes S_T = S0 (or zeros) and the offsets, nothing else.
 * Source: section 2.5 of the Kimi K3 reading notes and its Figure 12 (a prefix cache with
 * 6144-token physical blocks and 512-token hash blocks keeps KDA checkpoints only at the
 * hash-queryable endpoints; a hit at boundary B restores the checkpoint and continues prefill
 * from B); the per-lane arithmetic is section 2.2's, as in kda_chunk_fwd.
 */
kda_status kda_chunk_fwd_varlen(const kda_varlen_desc* desc,
                                const void* q, const void* k, const void* v,
                                const void* log_alpha, const void* beta,
                                const int32_t* cu_seqlens, const float* S0, void* o, float* S_T,
                                float* S_ckpt, int32_t* ckpt_offsets, const kda_gating* gating,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace kda_chunk_bwd needs for `desc` (0 for an invalid desc, fp32 inputs or
 * T = 0). It holds the forward's workspace, the state after every 64-token chunk (fp32), the
 * recomputed output, and per-chunk fp32 scratch (with the checkpoint about 0.32 MiB per chunk of
 * a lane at d = 128). */
size_t kda_chunk_bwd_workspace_bytes(const kda_chunk_desc* desc);

/*
 * Backward of chunkwise KDA prefill (training): for L with dL/do = dO and dL/dS_T = dS_T, writes
 * dL/dq, dL/dk, dL/dv, dL/dlog_alpha, dL/dbeta and dL/dS0.
 *   inputs as kda_chunk_fwd (in_dtype must be KDA_BF16; S0 NULL = zero state)
 *   dO              : [B,H,T,dv] out_dtype        dS_T : [B,H,dk,dv] fp32, or NULL (zero)
 *   dq, dk, dlog_alpha : [B,H,T,dk] fp32 (written)   dv : [B,H,T,dv] fp32   dbeta : [B,H,T] fp32
 *   dS0             : [B,H,dk,dv] fp32 (written), or NULL to skip
 *   workspace       : at least kda_chunk_bwd_workspace_bytes(desc) bytes, 256-byte aligned
 * The call recomputes the forward (with a state checkpoint after every chunk) and then runs the
 * reverse pass; gradient outputs must not overlap each other, the inputs or the workspace.
 * q, k, v, log_alpha and dO need 16-byte aligned bases (the forward's loads), beta its element
 * alignment, the fp32 outputs 4 bytes. Every reduction runs in a fixed order: the same inputs give
 * the same gradients bit for bit on every call.
 * Source: the pages print no backward; section 2.2 of the Kimi K3 reading notes gives the
 * recurrence and chunk equations this differentiates, and says training uses chunkwise KDA.
 */
kda_status kda_chunk_bwd(const kda_chunk_desc* desc,
                         const void* q, const void* k, const void* v,
                         const void* log_alpha, const void* beta, const float* S0,
                         const void* dO, const float* dS_T,
                         float* dq, float* dk, float* dv, float* dlog_alpha, float* dbeta, float* dS0,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * One KDA decode step: kda_decode_step(q,k,v,log_alpha,beta,S) -> (o, S').
 *   q, k, log_alpha : [N,H,dk] in_dtype        v : [N,H,dv] in_dtype
 *   beta            : [N,H]    in_dtype        o : [N,H,dv] out_dtype (written)
 *   S               : [N,H,dk,dv] fp32, read and overwritten in place with S'
 * o must not overlap S or any input. Source: the recurrence of section 2.2 (one token), and
 * section 2.5's decode regime (a fixed-size state, one launch per step, no KV growth).
 */
kda_status kda_decode_step(const kda_decode_desc* desc,
                           const void* q, const void* k, const void* v,
                           const void* log_alpha, const void* beta,
                           float* S, void* o, void* stream);

/*
 * kda_decode_step with the fused prologue / epilogue of kda_gating (z [N,H,dk] in_dtype replaces
 * log_alpha, which may then be NULL; gate [N,H,dv] in_dtype). gating == NULL is kda_decode_step.
 * Source: as kda_decode_step, plus the decay lower-bound and output-gate equations of section 2.2.
 */
kda_status kda_decode_step_gated(const kda_decode_desc* desc,
                                 const void* q, const void* k, const void* v,
                                 const void* log_alpha, const void* beta, const kda_gating* gating,
                                 float* S, void* o, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* kda_status_string(int32_t status);

/* Static version string of the library, e.g. "kda-gfx950 0.1.0". */
const char* kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */

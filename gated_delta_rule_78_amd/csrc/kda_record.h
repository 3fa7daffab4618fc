// Per-chunk record written by the intra-chunk kernel and streamed by the inter-chunk state pass.
//
// For one 64-token chunk of one (batch, head) lane (Kimi K3 reading notes, section 2.2 chunk
// equations; U and W are the outputs of the UT transform there):
//   W  = (I + A_kk)^{-1} Diag(beta) K~      [64 x dk], stored negated
//   U  = (I + A_kk)^{-1} Diag(beta) V       [64 x dv]
//   Q~ = Q * Gamma                          [64 x dk]
//   K- = K * gamma_C / Gamma                [64 x dk]
//   A_qk = Tril(Q~ K^^T)                    [64 x 64], diagonal included
//   gamma_C = Gamma of the chunk's last row [dk]
// so that, for the entry state S of the chunk,
//   V~ = U - W S,   O = Q~ S + A_qk V~,   S' = Diag(gamma_C) S + K-^T V~.
// W is stored as -W so that V~ is one MFMA accumulation started from U.
//
// Every matrix is stored as 1 KiB "fragment blocks": 64 lanes x 16 bytes, lane l holding the
// 8 bf16 values of its MFMA operand fragment (register order e = 0..7), so the state pass copies
// blocks into LDS unchanged and each lane reads its fragment with one conflict-free 16-byte
// read. With l16 = l % 16, lq = l / 16 and k(e) = 16*(e/4) + 4*lq + e%4:
//   W  block (I, ks), I < 4, ks < dk/32: -W [16I + l16][32ks + k(e)]         (A of -W S)
//   Q~ block (I, ks):                     Q~[16I + l16][32ks + k(e)]         (B of S^T Q~^T)
//   K- block (M, h), M < dk/16, h < 2:    K-[32h + k(e)][16M + l16]          (A of K-^T V~)
//   A  block (I, h), h < (I < 2 ? 1 : 2): A_qk[16I + l16][32h + k(e)]        (B of V~^T A_qk^T)
//   U  block (n, p), n < dv/16, p < 2:    e < 4: U[32p + 4lq + e][16n + l16]
//                                         e >= 4: U[32p + 16 + 4lq + e - 4][16n + l16]
//                                         (the accumulator layout of two 16-row tiles)
//   gamma: dk floats, then zero padding to a whole block.
#pragma once

#include <stdint.h>

namespace kda {

template <int DK, int DV>
struct RecordLayout {
    static constexpr int NKS = DK / 32;      // 32-wide channel windows
    static constexpr int NM = DK / 16;       // 16-channel tiles
    static constexpr int NV = DV / 16;       // 16-column value tiles
    static constexpr int W = 0;
    static constexpr int Q = W + 4 * NKS;
    static constexpr int K = Q + 4 * NKS;
    static constexpr int A = K + 2 * NM;
    static constexpr int U = A + 6;
    static constexpr int G = U + 2 * NV;
    static constexpr int BLOCKS = G + 1;
    static constexpr int BYTES = BLOCKS * 1024;
    __host__ __device__ static constexpr int w(int I, int ks) { return W + I * NKS + ks; }
    __host__ __device__ static constexpr int q(int I, int ks) { return Q + I * NKS + ks; }
    __host__ __device__ static constexpr int k(int M, int h) { return K + 2 * M + h; }
    __host__ __device__ static constexpr int a(int I, int h) { return A + (I < 2 ? I : 2 + 2 * (I - 2) + h); }
    __host__ __device__ static constexpr int u(int n, int p) { return U + 2 * n + p; }
    static_assert(DK * 4 <= 1024, "gamma fits one block");
};

// Record bytes for runtime dk, dv (both in {64, 128}).
inline int64_t record_bytes(int64_t dk, int64_t dv) {
    return (12 * (dk / 32) + 7 + 2 * (dv / 16)) * 1024;
}

}  // namespace kda

// Internal interface of the outer-orthogonalisation kernels (polar.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dlk {

// Output tiles (128 x 128) of an M x N product; a launch takes at most
// kGemmMaxTiles of them (one workgroup of 256 threads each, the grid padded
// to a multiple of 8).
constexpr int64_t kGemmMaxTiles = (int64_t(1) << 24) - 8;
inline int64_t gemm_tiles(int64_t M, int64_t N) { return ((M + 127) / 128) * ((N + 127) / 128); }

// Bytes of workspace polar_iterate needs for a batch of rows x cols matrices.
int64_t polar_workspace_bytes(int64_t rows, int64_t cols, int64_t batch);

// Newton-Schulz iteration towards the polar factor P of A (rows x cols,
// row-major fp32) for each matrix b of a batch, with A = src[b], or A =
// src[b] - sub[b] when sub is not null.  `quintic` + `cubic` >= 1 steps.
// The result goes to out[0] (batch 1 only), or, when theta is not null,
// theta[b] = theta[b] - scale * P (theta[b] may be src[b]).  The batch's
// products run as one launch each.  `ws` holds polar_workspace_bytes bytes,
// 256-byte aligned.
hipError_t polar_iterate(const float* const* src, const float* const* sub, float* const* out,
                         float* const* theta, float scale, int64_t batch, int64_t rows,
                         int64_t cols, int quintic, int cubic, void* ws, hipStream_t s);

// Workspace bytes for the stream-K split of a batch of M x N x K products
// (partial sums of the tiles cut between workgroups).
int64_t matmul_workspace_bytes(int64_t M, int64_t N, int64_t K, bool sym, int64_t batch);

// Whether the main block of such a batch runs on the large-tile kernel when
// its operands are 16-byte aligned and contiguous (leading dimension K) and
// the workspace holds ws_bytes.
bool matmul_large_tiles(int64_t M, int64_t N, int64_t K, bool sym, int64_t batch,
                        int64_t ws_bytes);

// A batch of fp32 MFMA products, matrix b: C_b = alpha * op(A_b, B_b) + beta
// * Y_b + diag * I with A_b = A + b*sa, B_b = B + b*sb, C_b = C + b*sc, Y_b =
// Y + b*sy (Y may be null or equal C):  tn: sum_k A[k*lda + i] * B[k*ldb + j];
// nt: sum_k A[i*lda + k] * B[j*ldb + k]; i < M, j < N.  With sym (M == N, a
// symmetric result and a symmetric or null Y) only the upper triangle is
// computed and mirrored.  With ws_bytes >= matmul_workspace_bytes the work
// is spread stream-K; otherwise (ws may be null) one workgroup per tile.
hipError_t matmul(bool tn, const float* A, int64_t lda, int64_t sa, const float* B, int64_t ldb,
                  int64_t sb, int64_t M, int64_t N, int64_t K, float* C, int64_t ldc, int64_t sc,
                  const float* Y, int64_t sy, float alpha, float beta, float diag, bool sym,
                  int64_t batch, void* ws, int64_t ws_bytes, hipStream_t s);

}  // namespace dlk

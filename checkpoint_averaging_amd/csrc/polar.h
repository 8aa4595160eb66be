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

// Bytes of workspace polar_iterate needs for a rows x cols matrix.
int64_t polar_workspace_bytes(int64_t rows, int64_t cols);

// Newton-Schulz iteration towards the polar factor of A (rows x cols,
// row-major fp32), with A = src, or A = src - sub when sub is not null.
// `quintic` + `cubic` >= 1 steps.  The result goes to `out` (if not null),
// or, when `theta` is not null, theta = theta - scale * P (theta may be src).
// `ws` holds polar_workspace_bytes(rows, cols) bytes, 256-byte aligned.
hipError_t polar_iterate(const float* src, const float* sub, float* out, float* theta, float scale,
                         int64_t rows, int64_t cols, int quintic, int cubic, void* ws,
                         hipStream_t s);

// Workspace bytes for the stream-K split of an M x N x K product (partial
// sums of the tiles cut between workgroups).
int64_t matmul_workspace_bytes(int64_t M, int64_t N, int64_t K, bool sym);

// One fp32 MFMA product C = alpha * op(A, B) + beta * Y + diag * I (Y may be
// null or equal C):  tn: sum_k A[k*lda + i] * B[k*ldb + j];
//                    nt: sum_k A[i*lda + k] * B[j*ldb + k]; i < M, j < N.
// With sym (M == N, a symmetric result and a symmetric or null Y) only the
// upper triangle is computed and mirrored.  With ws_bytes >=
// matmul_workspace_bytes the work is spread stream-K; otherwise (ws may be
// null) one workgroup per output tile.
hipError_t matmul(bool tn, const float* A, int64_t lda, const float* B, int64_t ldb, int64_t M,
                  int64_t N, int64_t K, float* C, int64_t ldc, const float* Y, float alpha,
                  float beta, float diag, bool sym, void* ws, int64_t ws_bytes, hipStream_t s);

}  // namespace dlk

// Outer orthogonalisation for CDNA4 (gfx950): the polar factor of an averaged
// update, computed with a Newton-Schulz iteration on fp32 MFMA.
//
// The DiffuRefill-1B technical report (section "What we measured",
// "Optimisers") tried replacing the averaged outer update by its polar
// factor: for a weight matrix whose averaged update is A = U S V^T (thin
// SVD), the update becomes U V^T.  Here U V^T is reached by iterating on
// X_0 = A / ||A||_F (all singular values in (0, 1]):
//   quintic steps  X <- X (a I + b G + c G^2),  G = X^T X,
//                  (a, b, c) = (3.4445, -4.7750, 2.0315): small singular
//                  values grow by 3.44x per step, large ones stay in
//                  [0.68, 1.2];
//   cubic steps    X <- X (1.5 I - 0.5 G): Newton-Schulz, quadratic
//                  convergence to 1 from that range.
// 12 + 6 steps bring every singular value with s / ||A||_F >= 1.4e-7 to 1
// within fp32 rounding.  For a wide matrix (rows < cols) the same runs on
// G = X X^T with X <- M X.
//
// Every product is a plain GEMM of fp32 on MFMA (v_mfma_f32_32x32x2f32):
// workgroups of 4 wave64 compute 128 x 128 output tiles, each wave a 64 x 64
// quarter as 2 x 2 MFMA blocks of 32 x 32, over K in steps of 16 staged
// through LDS (row stride 129 floats: no bank conflicts on the transposed
// writes or the operand reads).  The epilogue is fused: out = alpha*acc +
// beta*Y + (i == j ? d : 0), which forms a I + b G + c G^2 in the G^2 product,
// 1.5 I - 0.5 G in the Gram product, and theta - s*P in the last product.
// The Frobenius norm is a deterministic two-stage fp64 reduction (no
// atomics: the same input gives the same bits).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "polar.h"

namespace dlk {

namespace {

constexpr int kTileM = 128;
constexpr int kTileN = 128;
constexpr int kTileK = 32;
constexpr int kLdsRow = kTileK + 4;   // LDS row of one operand row's K-tile (floats)
constexpr int kGemmThreads = 256;
constexpr int kXcds = 8;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct Epilogue {
    float* c;
    int64_t ldc;
    const float* y;      // may be null; may equal c
    int64_t ldy;
    float alpha, beta, diag;
};

// One operand's K-tile: 128 operand rows (i for A, j for B) x 32 k, held as
// 4 float4 per thread and stored to LDS as [row][k] (16-byte rows, so the
// MFMA operand reads below are ds_read_b128).
//   k-major storage, element (row, k) at P[k*ld + row] (both operands of TN):
//     thread t owns row t%128 and k = 4*(t/128) + 8p + c, p, c = 0..3; each
//     of the 16 scalar loads is coalesced across the wave (consecutive rows);
//   row-major storage, element (row, k) at P[row*ld + k] (both of NT):
//     thread t owns rows t/8 + 32p and k = 4*(t%8) + c: one float4 load each
//     where `vec` says the row is 16-byte aligned and the 4 k are in range.
template <bool KMajor>
__device__ __forceinline__ void load_tile(const float* __restrict__ P, int64_t ld, int64_t r0,
                                          int64_t R, int64_t k0, int64_t K, bool vec, int tid,
                                          f32x4 (&v)[4]) {
    if constexpr (KMajor) {
        const int64_t row = r0 + (tid & 127);
        const int kg = 4 * (tid >> 7);
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int64_t k = k0 + kg + 8 * p + c;
                v[p][c] = (row < R && k < K) ? P[k * ld + row] : 0.0f;
            }
    } else {
        const int64_t k = k0 + 4 * (tid & 7);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int64_t row = r0 + (tid >> 3) + 32 * p;
            if (vec && row < R && k + 3 < K) {
                v[p] = *reinterpret_cast<const f32x4*>(P + row * ld + k);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    v[p][c] = (row < R && k + c < K) ? P[row * ld + k + c] : 0.0f;
            }
        }
    }
}

template <bool KMajor>
__device__ __forceinline__ void store_tile(float (*S)[kLdsRow], const f32x4 (&v)[4], int tid) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        float* dst = KMajor ? &S[tid & 127][4 * (tid >> 7) + 8 * p]
                            : &S[(tid >> 3) + 32 * p][4 * (tid & 7)];
        *reinterpret_cast<f32x4*>(dst) = v[p];
    }
}

// C[i][j] = epi( sum_k opA[i][k] * opB[k][j] ) for i < M, j < N, with
//   TN:  opA[i][k] = A[k*lda + i],  opB[k][j] = B[k*ldb + j]
//   NT:  opA[i][k] = A[i*lda + k],  opB[k][j] = B[j*ldb + k]
// A 128 x 128 output tile per workgroup; wave w computes the 64 x 64 quarter
// (w/2, w%2) as 2 x 2 blocks of v_mfma_f32_32x32x2f32.  The K loop is
// double-buffered: the next K-tile's global loads are in flight while the
// MFMAs consume the current one from LDS; one barrier per K-tile.  Within a
// K-tile, lane half h of MFMA step s carries k = 16h + s (the same k for the
// A and B operands), so each lane reads its 16 k of a row with 4 b128 reads.
template <bool TN>
__global__ __launch_bounds__(kGemmThreads) void k_gemm(const float* __restrict__ A, int64_t lda,
                                                       const float* __restrict__ B, int64_t ldb,
                                                       int64_t M, int64_t N, int64_t K,
                                                       uint32_t tiles_n, uint32_t tiles,
                                                       uint32_t per_xcd, bool vec_a, bool vec_b,
                                                       Epilogue e) {
    __shared__ __align__(16) float As[2][kTileM][kLdsRow];
    __shared__ __align__(16) float Bs[2][kTileN][kLdsRow];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;        // 2 x 2 waves of 64 x 64
    // Workgroups are dealt to the 8 XCDs round-robin; give each XCD a
    // contiguous run of tiles (row-major over the tile grid) so that the
    // tiles sharing an A row band meet in the same L2.
    // (tile counts stay below 2^24, so the index arithmetic is 32-bit)
    const uint32_t t = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (t >= tiles) return;   // padding workgroup: the whole group leaves before any barrier
    const int64_t i0 = static_cast<int64_t>(t / tiles_n) * kTileM;
    const int64_t j0 = static_cast<int64_t>(t % tiles_n) * kTileN;

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    const int64_t ktiles = (K + kTileK - 1) / kTileK;
    f32x4 ra[4], rb[4];
    if (ktiles > 0) {
        load_tile<TN>(A, lda, i0, M, 0, K, vec_a, tid, ra);
        load_tile<TN>(B, ldb, j0, N, 0, K, vec_b, tid, rb);
        store_tile<TN>(As[0], ra, tid);
        store_tile<TN>(Bs[0], rb, tid);
    }
    __syncthreads();
    const int h = lane >> 5, rl = lane & 31;
    for (int64_t kt = 0; kt < ktiles; ++kt) {
        const int cur = static_cast<int>(kt & 1);
        const bool more = kt + 1 < ktiles;
        if (more) {
            load_tile<TN>(A, lda, i0, M, (kt + 1) * kTileK, K, vec_a, tid, ra);
            load_tile<TN>(B, ldb, j0, N, (kt + 1) * kTileK, K, vec_b, tid, rb);
        }
        f32x4 a[2][4], b[2][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
                a[mb][q] = *reinterpret_cast<const f32x4*>(&As[cur][wr * 64 + mb * 32 + rl][16 * h + 4 * q]);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
                b[nb][q] = *reinterpret_cast<const f32x4*>(&Bs[cur][wc * 64 + nb * 32 + rl][16 * h + 4 * q]);
        }
#pragma unroll
        for (int st = 0; st < kTileK / 2; ++st) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                        a[mb][st >> 2][st & 3], b[nb][st >> 2][st & 3], acc[mb][nb], 0, 0, 0);
        }
        if (more) {
            store_tile<TN>(As[cur ^ 1], ra, tid);
            store_tile<TN>(Bs[cur ^ 1], rb, tid);
        }
        __syncthreads();
    }

    // ---- epilogue: accumulator r of lane l holds C[8(r/4) + 4(l/32) + r%4][l%32]
    //      of its 32 x 32 block --------------------------------------------------
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t i = i0 + wr * 64 + bi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int64_t j = j0 + wc * 64 + bj * 32 + (lane & 31);
                if (i < M && j < N) {
                    float v = e.alpha * acc[bi][bj][r];
                    if (e.y) v = v + e.beta * e.y[i * e.ldy + j];
                    if (i == j) v = v + e.diag;
                    e.c[i * e.ldc + j] = v;
                }
            }
}

// ---- Frobenius norm (two-stage fp64 reduction, fixed order) ---------------

constexpr int kRedBlocks = 1024;
constexpr int kRedThreads = 256;

// Stage 1: block b sums the squares of its grid-stride elements in fp64.
// With `y`, the element is x - y (rounded in fp32) and is also written to d.
__global__ __launch_bounds__(kRedThreads) void k_sumsq_partial(const float* __restrict__ x,
                                                               const float* __restrict__ y,
                                                               float* __restrict__ d, int64_t n,
                                                               double* __restrict__ partial) {
    __shared__ double red[kRedThreads];
    double s = 0.0;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * kRedThreads + threadIdx.x; e < n;
         e += static_cast<int64_t>(gridDim.x) * kRedThreads) {
        float v = x[e];
        if (y) {
            v = v - y[e];
            d[e] = v;
        }
        s += static_cast<double>(v) * static_cast<double>(v);
    }
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = kRedThreads / 2; w > 0; w >>= 1) {
        if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) partial[blockIdx.x] = red[0];
}

// Stage 2 (one block): inv = 1 / sqrt(sum of partials), or 0 for a zero matrix.
__global__ __launch_bounds__(kRedThreads) void k_sumsq_final(const double* __restrict__ partial,
                                                             int nparts, float* __restrict__ inv) {
    __shared__ double red[kRedThreads];
    double s = 0.0;
    for (int p = threadIdx.x; p < nparts; p += kRedThreads) s += partial[p];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = kRedThreads / 2; w > 0; w >>= 1) {
        if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) inv[0] = red[0] > 0.0 ? static_cast<float>(1.0 / sqrt(red[0])) : 0.0f;
}

// x[e] = src[e] * inv[0]
// (x may be src: each element is read and written by the same thread)
__global__ __launch_bounds__(256) void k_scale(float* x, const float* src,
                                               const float* __restrict__ inv, int64_t n) {
    const float s = inv[0];
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < n;
         e += static_cast<int64_t>(gridDim.x) * 256)
        x[e] = src[e] * s;
}

constexpr float kQa = 3.4445f, kQb = -4.7750f, kQc = 2.0315f;

int64_t align256(int64_t b) { return (b + 255) / 256 * 256; }

hipError_t gemm(bool tn, const float* A, int64_t lda, const float* B, int64_t ldb, int64_t M,
                int64_t N, int64_t K, const Epilogue& e, hipStream_t s) {
    const int64_t tiles_n = (N + kTileN - 1) / kTileN;
    const int64_t tiles = (M + kTileM - 1) / kTileM * tiles_n;
    const int64_t per_xcd = (tiles + kXcds - 1) / kXcds;
    const dim3 grid(static_cast<unsigned>(per_xcd * kXcds));
    const uint32_t tn32 = static_cast<uint32_t>(tiles_n), t32 = static_cast<uint32_t>(tiles),
                   px32 = static_cast<uint32_t>(per_xcd);
    // float4 loads of row-major operands need 16-byte aligned rows
    const bool vec_a = reinterpret_cast<uintptr_t>(A) % 16 == 0 && lda % 4 == 0;
    const bool vec_b = reinterpret_cast<uintptr_t>(B) % 16 == 0 && ldb % 4 == 0;
    if (tn)
        hipLaunchKernelGGL((k_gemm<true>), grid, dim3(kGemmThreads), 0, s, A, lda, B, ldb, M, N, K,
                           tn32, t32, px32, vec_a, vec_b, e);
    else
        hipLaunchKernelGGL((k_gemm<false>), grid, dim3(kGemmThreads), 0, s, A, lda, B, ldb, M, N, K,
                           tn32, t32, px32, vec_a, vec_b, e);
    return hipGetLastError();
}

}  // namespace

int64_t polar_workspace_bytes(int64_t rows, int64_t cols) {
    const int64_t r = rows < cols ? rows : cols;
    return align256(kRedBlocks * 8) + 256 + 2 * align256(rows * cols * 4) + 2 * align256(r * r * 4);
}

hipError_t polar_iterate(const float* src, const float* sub, float* out, float* theta, float scale,
                         int64_t rows, int64_t cols, int quintic, int cubic, void* ws,
                         hipStream_t s) {
    const int64_t n = rows * cols;
    const bool tall = rows >= cols;
    const int64_t r = tall ? cols : rows;
    char* p = static_cast<char*>(ws);
    double* partial = reinterpret_cast<double*>(p);
    p += align256(kRedBlocks * 8);
    float* inv = reinterpret_cast<float*>(p);
    p += 256;
    float* xa = reinterpret_cast<float*>(p);
    p += align256(n * 4);
    float* xb = reinterpret_cast<float*>(p);
    p += align256(n * 4);
    float* g = reinterpret_cast<float*>(p);
    p += align256(r * r * 4);
    float* m = reinterpret_cast<float*>(p);

    // X0 = A / ||A||_F, with A = src (or src - sub, formed in fp32 into xa)
    hipLaunchKernelGGL(k_sumsq_partial, dim3(kRedBlocks), dim3(kRedThreads), 0, s, src, sub,
                       sub ? xa : nullptr, n, partial);
    hipLaunchKernelGGL(k_sumsq_final, dim3(1), dim3(kRedThreads), 0, s, partial, kRedBlocks, inv);
    hipLaunchKernelGGL(k_scale, dim3(4096), dim3(256), 0, s, xa, sub ? xa : src, inv, n);
    if (hipError_t err = hipGetLastError()) return err;

    float* x = xa;
    float* xn = xb;
    const int steps = quintic + cubic;
    for (int st = 0; st < steps; ++st) {
        const bool quin = st < quintic;
        // Gram matrix (r x r) of the current iterate; for the cubic steps the
        // epilogue forms M = 1.5 I - 0.5 G directly.
        const Epilogue eg{quin ? g : m, r, nullptr, 0, quin ? 1.0f : -0.5f, 0.0f,
                          quin ? 0.0f : 1.5f};
        hipError_t err = tall ? gemm(true, x, cols, x, cols, r, r, rows, eg, s)      // X^T X
                              : gemm(false, x, cols, x, cols, r, r, cols, eg, s);   // X X^T
        if (err) return err;
        if (quin) {   // M = c G^2 + b G + a I  (G symmetric: G G = G^T G)
            const Epilogue em{m, r, g, r, kQc, kQb, kQa};
            if ((err = gemm(true, g, r, g, r, r, r, r, em, s))) return err;
        }
        // next iterate: X M (tall) or M X (wide); the last step writes the
        // result: the polar factor to out, or theta - scale * P onto theta
        const bool last = st == steps - 1;
        Epilogue ex{xn, cols, nullptr, 0, 1.0f, 0.0f, 0.0f};
        if (last && out) ex.c = out;
        if (last && theta) ex = Epilogue{theta, cols, theta, cols, -scale, 1.0f, 0.0f};
        err = tall ? gemm(false, x, cols, m, r, rows, cols, r, ex, s)    // C[i][j] = sum_k X[i][k] M[j][k]
                   : gemm(true, m, r, x, cols, rows, cols, r, ex, s);    // C[i][j] = sum_k M[k][i] X[k][j]
        if (err) return err;
        float* t = x;
        x = xn;
        xn = t;
    }
    return hipGetLastError();
}

hipError_t gemm_probe(bool tn, const float* A, int64_t lda, const float* B, int64_t ldb,
                      int64_t M, int64_t N, int64_t K, float* C, int64_t ldc, const float* Y,
                      float alpha, float beta, float diag, hipStream_t s) {
    const Epilogue e{C, ldc, Y, ldc, alpha, beta, diag};
    return gemm(tn, A, lda, B, ldb, M, N, K, e, s);
}

}  // namespace dlk

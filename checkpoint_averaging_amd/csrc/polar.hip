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

constexpr int kTileElems = kTileM * kTileN;

// How one product is cut into workgroups: output tiles (all of them, or only
// the upper triangle of a symmetric square result), times `splits` ranges of
// K of `kchunk` elements each.  With `partial`, each workgroup writes its raw
// 128 x 128 sums to its own slot of a partial buffer, and k_reduce_tiles adds
// the K ranges in a fixed order, applies the epilogue and writes C (and the
// mirror image for a symmetric result).
struct Tiling {
    uint32_t tiles_n;    // tiles along N (and along M when symmetric)
    uint32_t tiles;      // output tiles computed
    uint32_t splits;     // K ranges
    uint32_t per_xcd;    // workgroups per XCD; the grid is 8 * per_xcd
    int64_t kchunk;      // K elements per range, a multiple of the K-tile
    bool sym;
    bool partial;
};

// Output tile t -> (tile row, tile column): row-major over the tile grid, or
// over the upper triangle (ti <= tj), where row ti holds tiles_n - ti tiles.
__device__ __forceinline__ void tile_coords(uint32_t t, const Tiling& tl, uint32_t& ti,
                                            uint32_t& tj) {
    const uint32_t n = tl.tiles_n;
    if (!tl.sym) {
        ti = t / n;
        tj = t % n;
        return;
    }
    // first tile of row r: r*n - r*(r-1)/2, increasing in r; the row of t is
    // the last r with first(r) <= t (binary search, integer arithmetic)
    auto first = [n](uint32_t r) { return r * n - (r * (r - 1)) / 2; };
    uint32_t lo = 0, hi = n;      // first(lo) <= t < first(hi)
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) / 2;
        if (first(mid) <= t) lo = mid;
        else hi = mid;
    }
    ti = lo;
    tj = lo + (t - first(lo));
}

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
    // k0: first k of the tile; K: end of this workgroup's K range
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
                                                       Tiling tl, bool vec_a, bool vec_b,
                                                       Epilogue e, float* __restrict__ part) {
    __shared__ __align__(16) float As[2][kTileM][kLdsRow];
    __shared__ __align__(16) float Bs[2][kTileN][kLdsRow];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;        // 2 x 2 waves of 64 x 64
    // Workgroups are dealt to the 8 XCDs round-robin; give each XCD a
    // contiguous run of tiles (row-major over the tile grid) so that the
    // tiles sharing an A row band meet in the same L2.
    // Consecutive workgroups of one XCD share a K range and neighbouring
    // tiles.  (Workgroup counts stay below 2^24: 32-bit index arithmetic.)
    const uint32_t L = (blockIdx.x % kXcds) * tl.per_xcd + blockIdx.x / kXcds;
    if (L >= tl.tiles * tl.splits) return;   // padding: the whole group leaves before any barrier
    const uint32_t split = L / tl.tiles, t = L % tl.tiles;
    uint32_t ti, tj;
    tile_coords(t, tl, ti, tj);
    const int64_t i0 = static_cast<int64_t>(ti) * kTileM;
    const int64_t j0 = static_cast<int64_t>(tj) * kTileN;
    const int64_t kb = static_cast<int64_t>(split) * tl.kchunk;
    const int64_t ke = K < kb + tl.kchunk ? K : kb + tl.kchunk;

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    const int64_t ktiles = ke > kb ? (ke - kb + kTileK - 1) / kTileK : 0;
    f32x4 ra[4], rb[4];
    if (ktiles > 0) {
        load_tile<TN>(A, lda, i0, M, kb, ke, vec_a, tid, ra);
        load_tile<TN>(B, ldb, j0, N, kb, ke, vec_b, tid, rb);
        store_tile<TN>(As[0], ra, tid);
        store_tile<TN>(Bs[0], rb, tid);
    }
    __syncthreads();
    const int h = lane >> 5, rl = lane & 31;
    for (int64_t kt = 0; kt < ktiles; ++kt) {
        const int cur = static_cast<int>(kt & 1);
        const bool more = kt + 1 < ktiles;
        if (more) {
            load_tile<TN>(A, lda, i0, M, kb + (kt + 1) * kTileK, ke, vec_a, tid, ra);
            load_tile<TN>(B, ldb, j0, N, kb + (kt + 1) * kTileK, ke, vec_b, tid, rb);
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
    if (tl.partial) {
        float* pt = part + (static_cast<int64_t>(split) * tl.tiles + t) * kTileElems;
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int bj = 0; bj < 2; ++bj)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int li = wr * 64 + bi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    const int lj = wc * 64 + bj * 32 + (lane & 31);
                    pt[li * kTileN + lj] = acc[bi][bj][r];
                }
        return;
    }
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

// Sum of the K ranges' partial tiles (in range order), epilogue, and C.
// Workgroup b handles rows 32(b%4) .. +31 of output tile b/4; thread t owns
// columns 4(t%32) .. +3 of rows t/32 + 8p.  For a symmetric result the
// elements with i <= j are written in place and those with i < j also to
// C[j][i] through an LDS transpose (rows of 32 consecutive i per store).
__global__ __launch_bounds__(256) void k_reduce_tiles(const float* __restrict__ part, Tiling tl,
                                                      int64_t M, int64_t N, Epilogue e) {
    __shared__ float tr[32][kTileN + 1];
    const uint32_t t = blockIdx.x >> 2;
    const int q = static_cast<int>(blockIdx.x & 3);
    uint32_t ti, tj;
    tile_coords(t, tl, ti, tj);
    const int tid = threadIdx.x;
    const int lj = 4 * (tid & 31);
    const int64_t stride = static_cast<int64_t>(tl.tiles) * kTileElems;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int ll = (tid >> 5) + 8 * p;                    // row within the quarter
        const int li = 32 * q + ll;
        const float* src = part + static_cast<int64_t>(t) * kTileElems + li * kTileN + lj;
        f32x4 v = *reinterpret_cast<const f32x4*>(src);
        for (uint32_t sp = 1; sp < tl.splits; ++sp) {
            const f32x4 w = *reinterpret_cast<const f32x4*>(src + sp * stride);
#pragma unroll
            for (int c = 0; c < 4; ++c) v[c] = v[c] + w[c];
        }
        const int64_t i = static_cast<int64_t>(ti) * kTileM + li;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int64_t j = static_cast<int64_t>(tj) * kTileN + lj + c;
            float o = e.alpha * v[c];
            // a symmetric result reads Y and writes C only on and above the
            // diagonal (Y may be C: the mirror writes below never meet a read)
            if (i < M && j < N && (!tl.sym || i <= j)) {
                if (e.y) o = o + e.beta * e.y[i * e.ldy + j];
                if (i == j) o = o + e.diag;
                e.c[i * e.ldc + j] = o;
            }
            tr[ll][lj + c] = o;
        }
    }
    if (!tl.sym) return;      // uniform across the workgroup
    __syncthreads();
    const int ii = tid & 31;
    const int64_t i = static_cast<int64_t>(ti) * kTileM + 32 * q + ii;
#pragma unroll 4
    for (int p = 0; p < 16; ++p) {
        const int jj = (tid >> 5) + 8 * p;
        const int64_t j = static_cast<int64_t>(tj) * kTileN + jj;
        if (i < j && j < M) e.c[j * e.ldc + i] = tr[ii][jj];
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

constexpr int64_t kTargetGroups = 512;          // two resident workgroups on each of 256 CUs
constexpr int64_t kMinSplitK = 8 * kTileK;      // each K range spans at least 8 K-tiles
constexpr int64_t kMaxSplits = 16;

// The cut of an M x N x K product (see Tiling).  ws_bytes bounds the partial
// buffer; fewer K ranges are used if it is short.  Returns false if a
// symmetric product cannot get even one range's partial tiles.
bool plan_gemm(int64_t M, int64_t N, int64_t K, bool sym, int64_t ws_bytes, Tiling& tl,
               int64_t* need_bytes = nullptr) {
    const int64_t tn = (N + kTileN - 1) / kTileN, tm = (M + kTileM - 1) / kTileM;
    const int64_t tiles = sym ? tn * (tn + 1) / 2 : tm * tn;
    int64_t splits = 1;
    if (K > 0) {
        const int64_t want = (kTargetGroups + tiles - 1) / tiles;
        int64_t most = K / kMinSplitK;
        if (most > kMaxSplits) most = kMaxSplits;
        if (most < 1) most = 1;
        splits = want < most ? want : most;
    }
    const int64_t tile_bytes = static_cast<int64_t>(kTileElems) * 4;
    while (splits > 1 && splits * tiles * tile_bytes > ws_bytes) --splits;
    const bool partial = sym || splits > 1;
    if (partial && splits * tiles * tile_bytes > ws_bytes) return false;
    int64_t kchunk = 0;
    if (K > 0) {
        kchunk = ((K + splits - 1) / splits + kTileK - 1) / kTileK * kTileK;
        splits = (K + kchunk - 1) / kchunk;
    }
    tl.tiles_n = static_cast<uint32_t>(tn);
    tl.tiles = static_cast<uint32_t>(tiles);
    tl.splits = static_cast<uint32_t>(splits);
    tl.per_xcd = static_cast<uint32_t>((tiles * splits + kXcds - 1) / kXcds);
    tl.kchunk = kchunk;
    tl.sym = sym;
    tl.partial = partial;
    if (need_bytes) *need_bytes = partial ? splits * tiles * tile_bytes : 0;
    return true;
}

// Partial-buffer bytes the preferred cut of a product needs (0 if none).
int64_t gemm_partial_bytes(int64_t M, int64_t N, int64_t K, bool sym) {
    Tiling tl;
    int64_t need = 0;
    plan_gemm(M, N, K, sym, INT64_MAX, tl, &need);
    return need;
}

hipError_t gemm(bool tn, const float* A, int64_t lda, const float* B, int64_t ldb, int64_t M,
                int64_t N, int64_t K, const Epilogue& e, bool sym, float* part,
                int64_t part_bytes, hipStream_t s) {
    Tiling tl;
    if (!plan_gemm(M, N, K, sym, part ? part_bytes : 0, tl)) return hipErrorInvalidValue;
    const dim3 grid(tl.per_xcd * kXcds);
    // float4 loads of row-major operands need 16-byte aligned rows
    const bool vec_a = reinterpret_cast<uintptr_t>(A) % 16 == 0 && lda % 4 == 0;
    const bool vec_b = reinterpret_cast<uintptr_t>(B) % 16 == 0 && ldb % 4 == 0;
    if (tn)
        hipLaunchKernelGGL((k_gemm<true>), grid, dim3(kGemmThreads), 0, s, A, lda, B, ldb, M, N, K,
                           tl, vec_a, vec_b, e, part);
    else
        hipLaunchKernelGGL((k_gemm<false>), grid, dim3(kGemmThreads), 0, s, A, lda, B, ldb, M, N, K,
                           tl, vec_a, vec_b, e, part);
    if (tl.partial)
        hipLaunchKernelGGL(k_reduce_tiles, dim3(tl.tiles * 4), dim3(256), 0, s, part, tl, M, N, e);
    return hipGetLastError();
}

}  // namespace

namespace {

// Partial-buffer bytes of the iteration's three products on a rows x cols
// matrix: the symmetric Gram matrix, its symmetric square, the next iterate.
int64_t polar_partial_bytes(int64_t rows, int64_t cols) {
    const int64_t r = rows < cols ? rows : cols, L = rows < cols ? cols : rows;
    int64_t b = gemm_partial_bytes(r, r, L, true);
    const int64_t sq = gemm_partial_bytes(r, r, r, true);
    const int64_t nx = gemm_partial_bytes(rows, cols, r, false);
    if (sq > b) b = sq;
    if (nx > b) b = nx;
    return b;
}

}  // namespace

int64_t polar_workspace_bytes(int64_t rows, int64_t cols) {
    const int64_t r = rows < cols ? rows : cols;
    return align256(kRedBlocks * 8) + 256 + 2 * align256(rows * cols * 4) + 2 * align256(r * r * 4) +
           align256(polar_partial_bytes(rows, cols));
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
    p += align256(r * r * 4);
    float* part = reinterpret_cast<float*>(p);
    const int64_t part_bytes = align256(polar_partial_bytes(rows, cols));

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
        // Both r x r results are symmetric: only their upper triangles are
        // computed, and the lower ones are mirror images (exactly symmetric).
        hipError_t err =
            tall ? gemm(true, x, cols, x, cols, r, r, rows, eg, true, part, part_bytes, s)   // X^T X
                 : gemm(false, x, cols, x, cols, r, r, cols, eg, true, part, part_bytes, s); // X X^T
        if (err) return err;
        if (quin) {   // M = c G^2 + b G + a I  (G symmetric: G G = G^T G)
            const Epilogue em{m, r, g, r, kQc, kQb, kQa};
            if ((err = gemm(true, g, r, g, r, r, r, r, em, true, part, part_bytes, s))) return err;
        }
        // next iterate: X M (tall) or M X (wide); the last step writes the
        // result: the polar factor to out, or theta - scale * P onto theta
        const bool last = st == steps - 1;
        Epilogue ex{xn, cols, nullptr, 0, 1.0f, 0.0f, 0.0f};
        if (last && out) ex.c = out;
        if (last && theta) ex = Epilogue{theta, cols, theta, cols, -scale, 1.0f, 0.0f};
        err = tall ? gemm(false, x, cols, m, r, rows, cols, r, ex, false, part, part_bytes, s)
                   : gemm(true, m, r, x, cols, rows, cols, r, ex, false, part, part_bytes, s);
        // (tall: C[i][j] = sum_k X[i][k] M[j][k]; wide: C[i][j] = sum_k M[k][i] X[k][j])
        if (err) return err;
        float* t = x;
        x = xn;
        xn = t;
    }
    return hipGetLastError();
}

int64_t matmul_workspace_bytes(int64_t M, int64_t N, int64_t K, bool sym) {
    return gemm_partial_bytes(M, N, K, sym);
}

hipError_t matmul(bool tn, const float* A, int64_t lda, const float* B, int64_t ldb, int64_t M,
                  int64_t N, int64_t K, float* C, int64_t ldc, const float* Y, float alpha,
                  float beta, float diag, bool sym, void* ws, int64_t ws_bytes, hipStream_t s) {
    const Epilogue e{C, ldc, Y, ldc, alpha, beta, diag};
    return gemm(tn, A, lda, B, ldb, M, N, K, e, sym, static_cast<float*>(ws), ws ? ws_bytes : 0, s);
}

}  // namespace dlk

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
// Every product is a GEMM of fp32 on MFMA (v_mfma_f32_32x32x2f32), on one
// of two kernels.  Products large enough to fill the CUs with 256 x 256
// tiles run those on k_gemm_big: one workgroup per CU, one wave per SIMD,
// each wave a 128 x 128 quarter whose sums fill the accumulation registers,
// K-tiles of 16 double-buffered in LDS.  Everything else (and the ragged
// strips past the last whole 256 rows and columns) runs on k_gemm:
// workgroups of 4 wave64 compute 128 x 128 output tiles, each wave a 64 x 64
// quarter as 2 x 2 MFMA blocks of 32 x 32, over K in tiles of 32 staged
// through LDS with the next tile's loads in flight.  On k_gemm the work of a
// product (output tiles x K-tiles; for a batch of equally shaped matrices,
// all their tiles) goes to as many workgroups as the GPU holds at once:
// whole tiles in rounds, then the last round or two's worth split stream-K;
// tiles cut between workgroups are summed in K order by a second kernel, so
// results are deterministic.  A product with fewer tiles than workgroups
// over a long K is split along K instead, its (K range, tile) units dealt
// range by range so that the workgroups of an XCD read the same operand
// rows together, and each tile's pieces summed in K order; k_gemm_big cuts
// the last round's tiles along K the same way.  Edge tiles take the plain
// loads with clamped rows where the layout allows it.  The Gram matrix and its square are symmetric: only
// their upper tiles are computed and the lower ones are written as mirror
// images.  The epilogue is fused: out = alpha*acc + beta*Y + (i == j ? d :
// 0), which forms a I + b G + c G^2 in the G^2 product, 1.5 I - 0.5 G in the
// Gram product, and theta - s*P in the last product of a single matrix (a
// batch finishes with an elementwise pass of the same arithmetic).  The
// Frobenius norm is a deterministic two-stage fp64 reduction (no atomics:
// the same input gives the same bits).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

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
    int64_t sc = 0, sy = 0;   // element strides between the matrices of a batch
};

constexpr int kTileElems = kTileM * kTileN;

// How one product is spread over workgroups.  It has `tiles` output tiles
// of 128 x 128 (all of them, or the upper triangle of a symmetric result)
// and `kt` K-tiles of 32 per output tile.  With `groups` workgroups:
//   * first, dp_rounds rounds of whole tiles: in round r workgroup w takes
//     tile r * groups + w, so the workgroups running together work on
//     neighbouring tiles (and share operand rows in L2);
//   * then the remaining sk_tiles tiles, stream-K: their units = sk_tiles *
//     kt K-tiles, tile after tile, are dealt out as contiguous runs,
//     workgroup w taking [begin(w), begin(w + 1)), begin(w) = floor(units *
//     w / groups): whole tiles, with possibly a piece of a tile at either
//     end.  A piece stores its raw sums in partial slot 2w (the workgroup's
//     first stream-K piece) or 2w + 1 (its last one), and k_reduce_pieces
//     adds the pieces of each cut tile in K order.
// Without a workspace: groups = tiles, one round of whole tiles, no pieces.
// Split mode (ksplit > 1; few tiles over a long K): K is cut into ksplit
// ranges of kspan K-tiles, and the units (range r, tile t), numbered
// r * tiles + t, are dealt out in rounds (round n: workgroup w takes unit
// n * groups + w).  The workgroups running together then work on the same K
// range of neighbouring tiles, so an XCD's workgroups read the same operand
// rows at about the same time (one fetch into its L2 serves them all).
// Every unit is a piece, stored in partial slot = its number, and
// k_reduce_splits adds each tile's pieces in K order.
// A batch of equally shaped products is one product whose tiles are the
// batch's tiles, matrix after matrix.
struct Work {
    uint32_t tiles_n;    // tiles along N (and along M when symmetric)
    uint32_t tiles_per;  // output tiles computed per matrix of the batch
    uint32_t tiles;      // output tiles computed in all (tiles_per * batch)
    uint32_t kt;         // K-tiles per output tile (at least 1)
    uint32_t groups;     // workgroups with work
    uint32_t per_xcd;    // the grid is 8 * per_xcd workgroups
    uint32_t dp_rounds;  // rounds of whole tiles
    uint32_t units;      // stream-K units: (tiles - dp_rounds * groups) * kt, below 2^32
    uint32_t ksplit;     // split mode: K ranges (0 or 1: off)
    uint32_t kspan;      // split mode: K-tiles per range
    bool sym;
};

// floor(units * w / groups), in 32-bit arithmetic (stream-K splits have at
// most 512 workgroups, so r * w stays below 2^18)
__device__ __forceinline__ uint32_t unit_begin(const Work& wk, uint32_t w) {
    const uint32_t q = wk.units / wk.groups, r = wk.units % wk.groups;
    return q * w + r * w / wk.groups;
}

// Output tile t -> (tile row, tile column): row-major over the tile grid, or
// over the upper triangle (ti <= tj), where row ti holds tiles_n - ti tiles.
__device__ __forceinline__ void tile_coords(uint32_t t, const Work& wk, uint32_t& ti,
                                            uint32_t& tj) {
    const uint32_t n = wk.tiles_n;
    if (!wk.sym) {
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

// One operand's K-tile: 128 operand rows (i for A, j for B) x 32 k, loaded
// as 4 float4 per thread and stored to LDS as [row][k] (16-byte rows, so the
// MFMA operand reads below are ds_read_b128).
//   k-major storage, element (row, k) at P[k*ld + row] (both operands of TN):
//     thread t loads rows 4j .. 4j+3, j = (t/2)%32, of k = 4g .. 4g+3,
//     g = 2(t/64) + t%2: four float4 loads along the rows (each load of a
//     wave covers two runs of 512 contiguous bytes), transposed in registers
//     into four [row][k] float4 stores; pairing neighbouring lanes on two k
//     groups puts every 8 consecutive lanes' stores in distinct LDS banks;
//   row-major storage, element (row, k) at P[row*ld + k] (both of NT):
//     thread t loads rows t/8 + 32p, k = 4(t%8) .. +3: one float4 each.
// Guard = false (full K-tiles, 16-byte aligned rows): plain float4 loads,
// rows past the operand's last clamped to it (a k-major operand's rows come
// in groups of 4, so it needs R % 4 == 0: a group is then wholly in or out);
// the clamped rows only feed outputs past the last row, which are never
// stored.  Guard = true (a partial K-tile, or an edge that cannot be
// clamped): every element from a clamped, valid address, 0 outside the
// operand or the K range (no branches).  k0: first k of the tile; K: end of
// the K range; R: rows.
template <bool KMajor, bool Guard>
__device__ __forceinline__ void load_tile(const float* __restrict__ P, int64_t ld, int64_t r0,
                                          int64_t R, int64_t k0, int64_t K, int tid,
                                          f32x4 (&v)[4]) {
    if constexpr (KMajor) {
        const int64_t row = r0 + 4 * ((tid >> 1) & 31);
        const int64_t kq = k0 + 4 * (2 * (tid >> 6) + (tid & 1));
        if constexpr (!Guard) {
            const int64_t rc = row < R - 4 ? row : R - 4;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                v[kk] = *reinterpret_cast<const f32x4*>(P + (kq + kk) * ld + rc);
        } else {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int64_t k = kq + kk, rr = row + c;
                    const float x = P[(k < K ? k : K - 1) * ld + (rr < R ? rr : R - 1)];
                    v[kk][c] = (k < K && rr < R) ? x : 0.0f;
                }
        }
    } else {
        const int64_t k = k0 + 4 * (tid & 7);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int64_t row = r0 + (tid >> 3) + 32 * p;
            if constexpr (!Guard) {
                const int64_t rc = row < R - 1 ? row : R - 1;
                v[p] = *reinterpret_cast<const f32x4*>(P + rc * ld + k);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int64_t kc = k + c;
                    const float x = P[(row < R ? row : R - 1) * ld + (kc < K ? kc : K - 1)];
                    v[p][c] = (row < R && kc < K) ? x : 0.0f;
                }
            }
        }
    }
}

template <bool KMajor>
__device__ __forceinline__ void store_tile(float (*S)[kLdsRow], const f32x4 (&v)[4], int tid) {
    if constexpr (KMajor) {
        const int row = 4 * ((tid >> 1) & 31), k = 4 * (2 * (tid >> 6) + (tid & 1));
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const f32x4 w = {v[0][c], v[1][c], v[2][c], v[3][c]};
            *reinterpret_cast<f32x4*>(&S[row + c][k]) = w;
        }
    } else {
#pragma unroll
        for (int p = 0; p < 4; ++p)
            *reinterpret_cast<f32x4*>(&S[(tid >> 3) + 32 * p][4 * (tid & 7)]) = v[p];
    }
}

typedef float LdsRow[kLdsRow];
constexpr int kLdsFloats = 2 * (kTileM + kTileN) * kLdsRow;   // two buffers of A and B tiles
constexpr int kStage = kTileN + 1;                             // staged output tile row (floats)
static_assert(kTileM * kStage <= kLdsFloats, "the staged output tile reuses the operand buffers");

__device__ __forceinline__ LdsRow* lds_a(float* smem, int buf) {
    return reinterpret_cast<LdsRow*>(smem + buf * (kTileM + kTileN) * kLdsRow);
}
__device__ __forceinline__ LdsRow* lds_b(float* smem, int buf) {
    return reinterpret_cast<LdsRow*>(smem + (buf * (kTileM + kTileN) + kTileM) * kLdsRow);
}

// Loads of the next K-tile inside one step of the K loop.
enum class Next { None, Plain, Guarded };

struct TileCtx {
    const float* A;
    int64_t lda;
    const float* B;
    int64_t ldb;
    int64_t M, N, i0, j0, kb, ke;
    float* smem;
    bool clamp_rows;   // edge tiles may take the plain loads with clamped rows
};

// One K-tile: the next tile's loads (if any) in flight while the MFMAs
// consume the current one from LDS buffer kt % 2; then the next tile goes
// to the other buffer and one barrier closes the step.  Within a K-tile,
// lane half h of MFMA step s carries k = 16h + s (the same k for the A and
// B operands), so each lane reads its 16 k of a row with four b128 reads.
// In the plain steps, scheduling barriers spread the global loads and LDS
// stores among the MFMAs instead of leaving them bunched.
template <bool TN, Next L>
__device__ __forceinline__ void k_step_tile(const TileCtx& c, int64_t kt, f32x4 (&ra)[4],
                                            f32x4 (&rb)[4], f32x16 (&acc)[2][2]) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    const int cur = static_cast<int>(kt & 1);
    if constexpr (L != Next::None) {
        const int64_t k0 = c.kb + (kt + 1) * kTileK;
        load_tile<TN, L == Next::Guarded>(c.A, c.lda, c.i0, c.M, k0, c.ke, tid, ra);
        load_tile<TN, L == Next::Guarded>(c.B, c.ldb, c.j0, c.N, k0, c.ke, tid, rb);
    }
    LdsRow* as = lds_a(c.smem, cur);
    LdsRow* bs = lds_b(c.smem, cur);
    const int h = lane >> 5, rl = lane & 31;
    f32x4 a[2][4], b[2][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
            a[mb][q] = *reinterpret_cast<const f32x4*>(&as[wr * 64 + mb * 32 + rl][16 * h + 4 * q]);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
            b[nb][q] = *reinterpret_cast<const f32x4*>(&bs[wc * 64 + nb * 32 + rl][16 * h + 4 * q]);
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
    if constexpr (L != Next::None) {
        store_tile<TN>(lds_a(c.smem, cur ^ 1), ra, tid);
        store_tile<TN>(lds_b(c.smem, cur ^ 1), rb, tid);
    }
    if constexpr (L == Next::Plain && !TN) {
        // row-major operands: operand reads first, the next tile's global
        // loads one per 4 MFMAs over the first half, its LDS stores one per 4
        // MFMAs over the second half
        __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        }
    }
    if constexpr (L == Next::Plain && TN) {
        // k-major operands: loads first, then the operand reads, and the LDS
        // stores one per MFMA over the last eight
        __builtin_amdgcn_sched_group_barrier(0x020, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 56, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        }
    }

    __syncthreads();
}

// acc = opA[i0.., kb..ke) * opB[kb..ke), j0..] for one 128 x 128 tile.
// Tiles with 16-byte aligned rows run their full K-tiles through a
// branch-free loop of plain loads (edge tiles too, with clamped rows, when
// the rows allow it); a partial K-tile, and edge tiles that cannot be
// clamped, use guarded loads.  Ends with a barrier: LDS is free afterwards.
template <bool TN>
__device__ __forceinline__ void mma_tile(const TileCtx& c, bool vec_a, bool vec_b,
                                         f32x16 (&acc)[2][2]) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;
    const int tid = threadIdx.x;
    const int64_t span = c.ke > c.kb ? c.ke - c.kb : 0;
    const int64_t ktiles = (span + kTileK - 1) / kTileK, nfull = span / kTileK;
    const bool plain =
        vec_a && vec_b && (c.clamp_rows || (c.i0 + kTileM <= c.M && c.j0 + kTileN <= c.N));
    f32x4 ra[4], rb[4];
    if (ktiles > 0) {
        if (plain && nfull > 0) {
            load_tile<TN, false>(c.A, c.lda, c.i0, c.M, c.kb, c.ke, tid, ra);
            load_tile<TN, false>(c.B, c.ldb, c.j0, c.N, c.kb, c.ke, tid, rb);
        } else {
            load_tile<TN, true>(c.A, c.lda, c.i0, c.M, c.kb, c.ke, tid, ra);
            load_tile<TN, true>(c.B, c.ldb, c.j0, c.N, c.kb, c.ke, tid, rb);
        }
        store_tile<TN>(lds_a(c.smem, 0), ra, tid);
        store_tile<TN>(lds_b(c.smem, 0), rb, tid);
    }
    __syncthreads();
    int64_t kt = 0;
    if (plain)
        for (; kt + 1 < nfull; ++kt) k_step_tile<TN, Next::Plain>(c, kt, ra, rb, acc);
    for (; kt + 1 < ktiles; ++kt) k_step_tile<TN, Next::Guarded>(c, kt, ra, rb, acc);
    if (kt < ktiles) k_step_tile<TN, Next::None>(c, kt, ra, rb, acc);
}

// Position of accumulator r of the calling lane in its wave's 32 x 32 block
// (bi, bj): row 8(r/4) + 4(l/32) + r%4, column l%32, within the 128 x 128 tile.
__device__ __forceinline__ int acc_row(int bi, int r) {
    const int lane = threadIdx.x & 63, wr = (threadIdx.x >> 6) >> 1;
    return wr * 64 + bi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__device__ __forceinline__ int acc_col(int bj) {
    const int lane = threadIdx.x & 63, wc = (threadIdx.x >> 6) & 1;
    return wc * 64 + bj * 32 + (lane & 31);
}

// C[i][j] = epi( sum_k opA[i][k] * opB[k][j] ) for i < M, j < N, with
//   TN:  opA[i][k] = A[k*lda + i],  opB[k][j] = B[k*ldb + j]
//   NT:  opA[i][k] = A[i*lda + k],  opB[k][j] = B[j*ldb + k]
// over the stream-K split `wk` (see Work).  For a symmetric result, whole
// tiles write C[i][j] for i <= j in place and C[j][i] for i < j from the
// tile staged in LDS (rows of consecutive i per store).
template <bool TN>
__global__ __launch_bounds__(kGemmThreads) void k_gemm(const float* __restrict__ A, int64_t lda,
                                                       const float* __restrict__ B, int64_t ldb,
                                                       int64_t M, int64_t N, int64_t K,
                                                       int64_t sa, int64_t sb, Work wk,
                                                       bool vec_a, bool vec_b, Epilogue e,
                                                       float* __restrict__ part) {
    __shared__ __align__(16) float smem[kLdsFloats];
    // Workgroups are dealt to the 8 XCDs round-robin; give each XCD a
    // contiguous run of workgroup indices, hence of tiles, so that tiles
    // sharing operand rows meet in the same L2.  (Workgroup and tile counts
    // stay below 2^24: 32-bit index arithmetic.)
    const uint32_t w = (blockIdx.x % kXcds) * wk.per_xcd + blockIdx.x / kXcds;
    if (w >= wk.groups) return;   // padding: the whole group leaves before any barrier
    // whole tiles first, then this workgroup's stream-K run; everything here
    // is uniform across the workgroup
    const uint32_t dp_tiles = wk.dp_rounds * wk.groups;
    const uint32_t u_end = wk.units ? unit_begin(wk, w + 1) : 0;
    uint32_t u = wk.units ? unit_begin(wk, w) : 0;
    bool first_piece = true;
    const bool split = wk.ksplit > 1;
    const uint32_t split_units = split ? wk.tiles * wk.ksplit : 0;
    for (uint32_t seg = 0;
         split ? seg * wk.groups + w < split_units : (seg < wk.dp_rounds || u < u_end); ++seg) {
        uint32_t t, seg_end = 0, slot = 0;
        int64_t kb = 0, ke = K;
        bool whole = true;
        if (split) {
            slot = seg * wk.groups + w;
            const uint32_t r = slot / wk.tiles;
            t = slot - r * wk.tiles;
            kb = static_cast<int64_t>(r) * wk.kspan * kTileK;
            ke = kb + static_cast<int64_t>(wk.kspan) * kTileK;
            if (ke > K) ke = K;
            whole = false;
        } else if (seg < wk.dp_rounds) {
            t = seg * wk.groups + w;
        } else {
            const uint32_t ts = u / wk.kt;
            const uint32_t t_begin = ts * wk.kt, t_end = t_begin + wk.kt;
            seg_end = u_end < t_end ? u_end : t_end;
            kb = static_cast<int64_t>(u - t_begin) * kTileK;
            ke = static_cast<int64_t>(seg_end - t_begin) * kTileK;
            if (ke > K) ke = K;
            whole = u == t_begin && seg_end == t_end;
            t = dp_tiles + ts;
            slot = 2 * w + (first_piece ? 0 : 1);
        }
        // matrix mb of the batch, tile tm within it
        const uint32_t mb = t / wk.tiles_per, tm = t - mb * wk.tiles_per;
        uint32_t ti, tj;
        tile_coords(tm, wk, ti, tj);
        const int64_t i0 = static_cast<int64_t>(ti) * kTileM;
        const int64_t j0 = static_cast<int64_t>(tj) * kTileN;
        f32x16 acc[2][2];
        const TileCtx ctx{A + mb * sa, lda, B + mb * sb, ldb, M, N, i0, j0, kb, ke, smem,
                          TN ? ((M | N) & 3) == 0 : true};
        mma_tile<TN>(ctx, vec_a, vec_b, acc);
        float* const ec = e.c + mb * e.sc;
        const float* const ey = e.y ? e.y + mb * e.sy : nullptr;

        // Stage the tile's sums in LDS (free after mma_tile), then store
        // from there: rows of 128 consecutive columns per store, with
        // per-thread indices that are cheap to recompute.
#pragma unroll
        for (int bi = 0; bi < 2; ++bi)
#pragma unroll
            for (int bj = 0; bj < 2; ++bj)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    smem[acc_row(bi, r) * kStage + acc_col(bj)] = acc[bi][bj][r];
        __syncthreads();
        const int tid = threadIdx.x;
        const int col = tid & (kTileN - 1);
        if (!whole) {
            // a piece: raw sums to its slot (stream-K: the workgroup's first
            // or last; split mode: the unit's number)
            float* pt = part + static_cast<int64_t>(slot) * kTileElems;
#pragma unroll 4
            for (int p = 0; p < kTileElems / kGemmThreads; ++p) {
                const int row = 2 * p + (tid >> 7);
                pt[row * kTileN + col] = smem[row * kStage + col];
            }
        } else {
            // a whole tile: epilogue and C.  A symmetric result reads Y and
            // writes C in place only on and above the diagonal (Y may be C:
            // the mirror writes below never meet a read); its final values
            // go back to the staged tile for the mirror pass.
            const int64_t j = j0 + col;
#pragma unroll 2
            for (int p = 0; p < kTileElems / kGemmThreads; ++p) {
                const int row = 2 * p + (tid >> 7);
                const int64_t i = i0 + row;
                float v = e.alpha * smem[row * kStage + col];
                if (i < M && j < N && (!wk.sym || i <= j)) {
                    if (ey) v = v + e.beta * ey[i * e.ldy + j];
                    if (i == j) v = v + e.diag;
                    ec[i * e.ldc + j] = v;
                }
                if (wk.sym) smem[row * kStage + col] = v;
            }
            if (wk.sym) {   // uniform
                __syncthreads();
                // C[j][i] for i < j: rows jj of the mirror, consecutive i per store
                const int64_t i = i0 + col;
#pragma unroll 2
                for (int p = 0; p < kTileElems / kGemmThreads; ++p) {
                    const int jj = 2 * p + (tid >> 7);
                    const int64_t jm = j0 + jj;
                    if (i < jm && jm < M) ec[jm * e.ldc + i] = smem[col * kStage + jj];
                }
            }
        }
        if (!split && seg >= wk.dp_rounds) {
            first_piece = false;
            u = seg_end;
        }
        __syncthreads();   // LDS is reused by the next tile
    }
}

// ---- large-tile kernel ------------------------------------------------------
//
// C = alpha * sum + beta * Y (+ diag where i == j) over the main block of a
// product: M and N multiples of 256, K of 16.  Row-major operands (NT: A is
// M x K, B is N x K) or k-major ones (TN: A is K x M, B is K x N; each 4 x 4
// piece transposed in registers on its way to LDS), LDS holding [row][k]
// either way.  One workgroup per CU (4 waves, one per SIMD), each wave a 128
// x 128 quarter of a 256 x 256 tile as 4 x 4 MFMA blocks of 32 x 32 whose
// sums fill the 256 accumulation registers.  With one wave per SIMD the
// latency is hidden inside the wave: K-tiles of 16 in two LDS buffers; the
// operands of a K-tile come in two halves of 4 k-steps (k = 8h + 4c + e for
// lane half h, chunk c), the second half read while the first runs and the
// next K-tile's first half read while the second runs; the next K-tile's
// LDS stores, the loads of the one after and the operand reads are spread
// among the MFMAs, one per two, by scheduling barriers; one barrier per
// K-tile.  A symmetric result has only its upper tiles computed: an
// off-diagonal tile is written and mirrored, a diagonal one writes its
// elements with i <= j and mirrors those with i < j.
//
// Work items are dealt in rounds, the 32 workgroups of an XCD on
// consecutive items (sharing operand rows in L2): first the whole tiles 0 ..
// dp - 1, then the last `tail` tiles in `ksplit` pieces of K each, dealt
// piece by piece (the workgroups running together work on the same K range
// of neighbouring tiles).  A piece's raw sums go to the partial buffer, and
// k_reduce_big adds each tail tile's pieces in K order before the epilogue.
constexpr int kBigM = 256, kBigN = 256, kBigK = 16;
constexpr int kBigRow = kBigK + 4;                    // LDS row (floats): 16 k + 4 padding
constexpr int kBigTile = kBigM * kBigRow;             // one operand tile of one buffer
constexpr int kBigGroups = 256;                       // one workgroup per CU
constexpr int64_t kBigElems = kBigM * kBigN;          // one tile's sums (a piece)

struct BigWork {
    uint32_t tiles_n;    // tiles along N (and along M when symmetric)
    uint32_t tiles_per;  // tiles per matrix of the batch: the grid or its upper triangle
    uint32_t dp;         // tiles 0 .. dp - 1: whole
    uint32_t tail;       // tiles dp .. dp + tail - 1: in ksplit pieces each
    uint32_t ksplit;     // pieces per tail tile
    uint32_t kspan;      // K-tiles per piece (the last piece: the rest)
    uint32_t nk;         // K-tiles of a tile
    bool sym;
};

// tile t -> matrix mb of the batch, tile row ti, tile column tj (row-major
// over the grid, or over the upper triangle, whose row r starts at
// r n - r (r - 1) / 2)
__device__ __forceinline__ void big_coords(uint32_t t, const BigWork& wk, uint32_t& mb,
                                           uint32_t& ti, uint32_t& tj) {
    mb = t / wk.tiles_per;
    const uint32_t u = t - mb * wk.tiles_per, n = wk.tiles_n;
    if (!wk.sym) {
        ti = u / n;
        tj = u - ti * n;
        return;
    }
    uint32_t r = 0;
    while (r + 1 < n && (r + 1) * n - ((r + 1) * r) / 2 <= u) ++r;
    ti = r;
    tj = u - (r * n - (r * (r - 1)) / 2) + r;
}

// One K-tile of an operand, from P (row-major: the tile's first row at the
// K-tile's first k; k-major: the K-tile's first k at the tile's first
// column).  Row-major: thread t loads rows t/4 + 64p, k 4(t%4) .. +3;
// k-major: k 4(t%4) + p, columns 4(t/4) .. +3.  `off` is the lane's byte
// offset (below 2^32); P plus the p term is uniform, so each load takes a
// scalar base and the one 32-bit lane offset.
template <bool KM>
__device__ __forceinline__ uint32_t big_offset(int64_t ld, int tid) {
    return KM ? static_cast<uint32_t>((4 * (tid & 3) * ld + 4 * (tid >> 2)) * 4)
              : static_cast<uint32_t>(((tid >> 2) * ld + 4 * (tid & 3)) * 4);
}
template <bool KM>
__device__ __forceinline__ void big_load(const float* __restrict__ P, int64_t ld, uint32_t off,
                                         f32x4 (&g)[4]) {
#pragma unroll
    for (int p = 0; p < 4; ++p)
        g[p] = *reinterpret_cast<const f32x4*>(
            reinterpret_cast<const char*>(P + (KM ? p : 64 * p) * ld) + off);
}
// to LDS as [row][k]: row-major, row t/4 + 64p gets load p; k-major, row
// 4(t/4) + p gets element p of the four loads (k 4(t%4) .. +3)
template <bool KM>
__device__ __forceinline__ void big_store(float* S, int tid, const f32x4 (&g)[4]) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        if (KM) {
            const f32x4 v = {g[0][p], g[1][p], g[2][p], g[3][p]};
            *reinterpret_cast<f32x4*>(S + (4 * (tid >> 2) + p) * kBigRow + 4 * (tid & 3)) = v;
        } else {
            *reinterpret_cast<f32x4*>(S + ((tid >> 2) + 64 * p) * kBigRow + 4 * (tid & 3)) =
                g[p];
        }
    }
}
// chunk c of this lane's operand rows base + 32 i + l%32 (i < 4)
__device__ __forceinline__ void big_read(const float* S, int base, int lane, int c,
                                         f32x4 (&r)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r[i] = *reinterpret_cast<const f32x4*>(S + (base + 32 * i + (lane & 31)) * kBigRow +
                                               8 * (lane >> 5) + 4 * c);
}
__device__ __forceinline__ void big_mma(int e, const f32x4 (&a)[4], const f32x4 (&b)[4],
                                        f32x16 (&acc)[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][e], b[j][e], acc[i][j], 0, 0,
                                                             0);
}

// f(integral_constant<int, b>) for the 16 MFMA blocks b of a wave's quarter,
// so that every accumulator index is a constant
template <class F, int... Bs>
__device__ __forceinline__ void each_block_(F&& f, std::integer_sequence<int, Bs...>) {
    (f(std::integral_constant<int, Bs>{}), ...);
}
template <class F>
__device__ __forceinline__ void each_block(F&& f) {
    each_block_(f, std::make_integer_sequence<int, 16>{});
}

template <bool KM>
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_big(
    const float* __restrict__ A, int64_t lda, int64_t sa, const float* __restrict__ B,
    int64_t ldb, int64_t sb, BigWork wk, Epilogue e, float* __restrict__ part) {
    __shared__ __align__(16) float smem[4 * kBigTile];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    const uint32_t per_xcd = kBigGroups / kXcds;
    const uint32_t w = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    const uint32_t offa = big_offset<KM>(lda, tid), offb = big_offset<KM>(ldb, tid);
    const int64_t stepa = KM ? kBigK * lda : kBigK;   // one K-tile further
    const int64_t stepb = KM ? kBigK * ldb : kBigK;
    const uint32_t items = wk.dp + wk.tail * wk.ksplit;
    for (uint32_t it = w; it < items; it += kBigGroups) {
        uint32_t t = it, k0 = 0, nk = wk.nk;
        int64_t slot = -1;   // a piece's partial slot (uniform)
        if (it >= wk.dp) {
            const uint32_t v = it - wk.dp, seg = v / wk.tail;
            t = wk.dp + (v - seg * wk.tail);
            k0 = seg * wk.kspan;
            nk = wk.nk - k0 < wk.kspan ? wk.nk - k0 : wk.kspan;
            slot = v;
        }
        uint32_t mb, ti, tj;
        big_coords(t, wk, mb, ti, tj);
        const int64_t ri = static_cast<int64_t>(ti) * kBigM, rj = static_cast<int64_t>(tj) * kBigN;
        const float* Ab = A + mb * sa + k0 * stepa + (KM ? ri : ri * lda);
        const float* Bb = B + mb * sb + k0 * stepb + (KM ? rj : rj * ldb);
        f32x16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
        f32x4 ga[4], gb[4], a0[4], b0[4], a1[4], b1[4];
        big_load<KM>(Ab, lda, offa, ga);
        big_load<KM>(Bb, ldb, offb, gb);
        big_store<KM>(smem, tid, ga);
        big_store<KM>(smem + kBigTile, tid, gb);
        __syncthreads();
        big_read(smem, wr * 128, lane, 0, a0);
        big_read(smem + kBigTile, wc * 128, lane, 0, b0);
        if (nk > 1) {
            big_load<KM>(Ab + stepa, lda, offa, ga);
            big_load<KM>(Bb + stepb, ldb, offb, gb);
        }
        // K-tile kt (in buffer kt % 2, chunk 0 already in a0/b0): store
        // K-tile kt+1 (in ga/gb) to the other buffer, load K-tile kt+2, read
        // chunk 1 into a1/b1, barrier, read chunk 0 of K-tile kt+1.
        auto ktile = [&](int64_t kt, bool store_next, bool load_next2) {
            const int cur = static_cast<int>(kt & 1), nxt = cur ^ 1;
            const float* sa_ = smem + 2 * cur * kBigTile;
            const float* sb_ = sa_ + kBigTile;
            float* na = smem + 2 * nxt * kBigTile;
            float* nb = na + kBigTile;
            big_mma(0, a0, b0, acc);
            if (store_next) {
                big_store<KM>(na, tid, ga);
                big_store<KM>(nb, tid, gb);
            }
            big_mma(1, a0, b0, acc);
            if (load_next2) {
                big_load<KM>(Ab + (kt + 2) * stepa, lda, offa, ga);
                big_load<KM>(Bb + (kt + 2) * stepb, ldb, offb, gb);
            }
            big_mma(2, a0, b0, acc);
            big_read(sa_, wr * 128, lane, 1, a1);
            big_read(sb_, wc * 128, lane, 1, b1);
            big_mma(3, a0, b0, acc);
            if (store_next && load_next2) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // LDS store
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // global load
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            __syncthreads();
            big_mma(0, a1, b1, acc);
            if (store_next) {
                big_read(na, wr * 128, lane, 0, a0);
                big_read(nb, wc * 128, lane, 0, b0);
            }
            big_mma(1, a1, b1, acc);
            big_mma(2, a1, b1, acc);
            big_mma(3, a1, b1, acc);
            if (store_next && load_next2) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 48, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        int64_t kt = 0;
        for (; kt + 2 < nk; ++kt) ktile(kt, true, true);   // branch-free body
        if (kt + 1 < nk) {
            ktile(kt, true, false);
            ++kt;
        }
        if (kt < nk) ktile(kt, false, false);
        __syncthreads();   // LDS is free for the next item
        // accumulator r of block (i, j) is row 32i + 8(r/4) + r%4 + 4(l/32),
        // column 32j + l%32 of the wave's quarter: a per-lane base plus a
        // uniform offset.  Blocks leave the accumulation registers one at a
        // time (the empty asm pins the move there; moved all at once, they
        // would not fit beside the rest).
        const int hr = 4 * (lane >> 5), cc = lane & 31;
        if (slot >= 0) {   // a piece: raw sums, 256 x 256 row-major
            float* const pp = part + slot * kBigElems + (wr * 128 + hr) * kBigN + wc * 128 + cc;
            each_block([&](auto bk) {
                constexpr int b = decltype(bk)::value;
                f32x16 v = acc[b >> 2][b & 3];
                asm volatile("" : "+v"(v));
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    pp[(32 * (b >> 2) + 8 * (r >> 2) + (r & 3)) * kBigN + 32 * (b & 3)] = v[r];
            });
            continue;
        }
        const int64_t i0 = ri + wr * 128 + hr, j0 = rj + wc * 128 + cc;
        float* const ec = e.c + mb * e.sc + i0 * e.ldc + j0;
        float* const em = e.c + mb * e.sc + j0 * e.ldc + i0;   // mirror: C[j][i]
        const float* const ey = e.y ? e.y + mb * e.sy + i0 * e.ldy + j0 : nullptr;
        // block b of the quarter, at block row 4 wr + b/4 and column 4 wc +
        // b%4 of the tile: 0 nothing, 1 written, 2 written and mirrored,
        // 3 a diagonal block of a symmetric result (element-wise)
        auto mode = [&](int b) {
            const int bi = 4 * wr + (b >> 2), bj = 4 * wc + (b & 3);
            if (!wk.sym) return 1;
            if (ti != tj) return 2;
            return bi < bj ? 2 : (bi == bj ? 3 : 0);
        };
        auto on_diag = [&](int b) { return ti == tj && 4 * wr + (b >> 2) == 4 * wc + (b & 3); };
        // Y of block b + 1 is loaded before block b is stored (Y is C itself
        // or apart from it, so every element's Y is read before its C is
        // written), which keeps 16 loads in flight
        float yv[2][16];
        auto load_y = [&](int b, float (&y)[16]) {
            if (!ey || mode(b) == 0) return;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                y[r] = ey[(32 * (b >> 2) + 8 * (r >> 2) + (r & 3)) * e.ldy + 32 * (b & 3)];
        };
        load_y(0, yv[0]);
        each_block([&](auto bk) {
            constexpr int b = decltype(bk)::value;
            if (b + 1 < 16) load_y(b + 1, yv[(b + 1) & 1]);
            const int md = mode(b);
            if (md == 0) return;
            f32x16 v = acc[b >> 2][b & 3];
            asm volatile("" : "+v"(v));
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                x[r] = e.alpha * v[r];
                if (ey) x[r] = x[r] + e.beta * yv[b & 1][r];
            }
            const int64_t bo = 32 * (b >> 2), bc = 32 * (b & 3);   // block row, column
            if (on_diag(b)) {
                // element r sits on row hr + 8(r/4) + r%4 and column cc of
                // the block: i - j = that row - cc
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int d = hr + 8 * (r >> 2) + (r & 3) - cc;
                    if (d == 0) x[r] = x[r] + e.diag;
                    const int64_t o = (bo + 8 * (r >> 2) + (r & 3)) * e.ldc + bc;
                    if (md != 3 || d <= 0) ec[o] = x[r];
                    if (md == 3 && d < 0) em[bc * e.ldc + bo + 8 * (r >> 2) + (r & 3)] = x[r];
                }
                if (md == 3) return;
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    ec[(bo + 8 * (r >> 2) + (r & 3)) * e.ldc + bc] = x[r];
            }
            if (md == 2) {   // rows 8g .. 8g + 3 (plus the lane's 4) of column bc: one float4
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 m4 = {x[4 * g], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3]};
                    *reinterpret_cast<f32x4*>(em + bc * e.ldc + bo + 8 * g) = m4;
                }
            }
        });
    }
}

// One tile's pieces summed in K order (piece(0) + piece(1) + ... +
// piece(count - 1), each a 128 x 128 tile of raw sums), then the epilogue and
// C, for rows 32q .. 32q + 31 of the tile.  Thread t owns columns 4(t%32) ..
// +3 of rows t/32 + 8p.  For a symmetric result the elements with i <= j are
// written in place and those with i < j also to C[j][i] through an LDS
// transpose (rows of 32 consecutive i).
template <class Piece>
__device__ __forceinline__ void reduce_tile_rows(const Piece& piece, uint32_t count, uint32_t t,
                                                 int q, const Work& wk, int64_t M, int64_t N,
                                                 const Epilogue& e) {
    __shared__ float tr[32][kTileN + 1];
    const uint32_t mb = t / wk.tiles_per;
    uint32_t ti, tj;
    tile_coords(t - mb * wk.tiles_per, wk, ti, tj);
    float* const ec = e.c + mb * e.sc;
    const float* const ey = e.y ? e.y + mb * e.sy : nullptr;
    const int tid = threadIdx.x;
    const int lj = 4 * (tid & 31);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int ll = (tid >> 5) + 8 * p;                    // row within the quarter
        const int li = 32 * q + ll;
        f32x4 v = *reinterpret_cast<const f32x4*>(piece(0) + li * kTileN + lj);
        for (uint32_t n = 1; n < count; ++n) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(piece(n) + li * kTileN + lj);
#pragma unroll
            for (int c = 0; c < 4; ++c) v[c] = v[c] + x[c];
        }
        const int64_t i = static_cast<int64_t>(ti) * kTileM + li;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int64_t j = static_cast<int64_t>(tj) * kTileN + lj + c;
            float o = e.alpha * v[c];
            if (i < M && j < N && (!wk.sym || i <= j)) {
                if (ey) o = o + e.beta * ey[i * e.ldy + j];
                if (i == j) o = o + e.diag;
                ec[i * e.ldc + j] = o;
            }
            tr[ll][lj + c] = o;
        }
    }
    if (!wk.sym) return;      // uniform across the workgroup
    __syncthreads();
    const int ii = tid & 31;
    const int64_t i = static_cast<int64_t>(ti) * kTileM + 32 * q + ii;
#pragma unroll 4
    for (int p = 0; p < 16; ++p) {
        const int jj = (tid >> 5) + 8 * p;
        const int64_t j = static_cast<int64_t>(tj) * kTileN + jj;
        if (i < j && j < M) ec[j * e.ldc + i] = tr[ii][jj];
    }
}

// The tiles cut between workgroups (stream-K): workgroup 4b + q looks at the
// start of workgroup b (b >= 1); if that falls inside a tile and no earlier
// workgroup start does, it sums that tile's pieces (workgroup b - 1's piece,
// then the first pieces of b, b + 1, ... that start inside the tile) for
// rows 32q .. 32q + 31.
__global__ __launch_bounds__(256) void k_reduce_pieces(const float* __restrict__ part, Work wk,
                                                       int64_t M, int64_t N, Epilogue e) {
    const uint32_t b = blockIdx.x >> 2;
    const int q = static_cast<int>(blockIdx.x & 3);
    if (b == 0 || b >= wk.groups || wk.units == 0) return;
    const uint32_t ub = unit_begin(wk, b);
    const uint32_t ts = ub / wk.kt;                  // stream-K tile
    const uint32_t t_begin = ts * wk.kt, t_end = t_begin + wk.kt;
    if (ub == t_begin) return;                       // a start between whole tiles
    const uint32_t prev = unit_begin(wk, b - 1);
    if (prev > t_begin) return;                      // handled at an earlier start
    // workgroup b - 1 holds the tile's first piece: its first slot if it
    // starts at the tile, else its last slot
    const float* first = part + (2 * static_cast<int64_t>(b - 1) + (prev < t_begin ? 1 : 0)) *
                                    kTileElems;
    uint32_t last = b;                               // workgroups b .. last start inside the tile
    while (last + 1 < wk.groups && unit_begin(wk, last + 1) < t_end) ++last;
    auto piece = [&](uint32_t n) {
        return n == 0 ? first : part + 2 * static_cast<int64_t>(b + n - 1) * kTileElems;
    };
    reduce_tile_rows(piece, last - b + 2, wk.dp_rounds * wk.groups + ts, q, wk, M, N, e);
}

// Split mode: workgroup 4t + q sums the ksplit pieces of tile t (slots
// r * tiles + t, r = 0 .. ksplit - 1, in K order) for rows 32q .. 32q + 31.
__global__ __launch_bounds__(256) void k_reduce_splits(const float* __restrict__ part, Work wk,
                                                       int64_t M, int64_t N, Epilogue e) {
    const uint32_t t = blockIdx.x >> 2;
    const int q = static_cast<int>(blockIdx.x & 3);
    if (t >= wk.tiles) return;
    auto piece = [&](uint32_t r) {
        return part + (static_cast<int64_t>(r) * wk.tiles + t) * kTileElems;
    };
    reduce_tile_rows(piece, wk.ksplit, t, q, wk, M, N, e);
}

// The tail tiles of the large-tile kernel: tile dp + tt's ksplit pieces
// (slots s * tail + tt) summed in K order (piece 0 + piece 1 + ...), then
// the epilogue, for rows 32q .. 32q + 31 and columns 64h .. 64h + 63 of the
// tile (workgroup 32 tt + 4q + h: 32 per tile, so that a tail of a few
// tiles still spreads over the CUs).  Thread t owns columns 4(t%16) .. +3
// of that block's rows t/16 and t/16 + 16.  A symmetric result is mirrored
// as in the large-tile kernel, through LDS (rows of 32 consecutive i per
// store).
__global__ __launch_bounds__(256) void k_reduce_big(const float* __restrict__ part, BigWork wk,
                                                    Epilogue e) {
    __shared__ float tr[64][33];
    const uint32_t tt = blockIdx.x >> 5;
    const int q = static_cast<int>((blockIdx.x >> 2) & 7), h = static_cast<int>(blockIdx.x & 3);
    if (tt >= wk.tail) return;
    uint32_t mb, ti, tj;
    big_coords(wk.dp + tt, wk, mb, ti, tj);
    const int tid = threadIdx.x, cl = 4 * (tid & 15), lj = 64 * h + cl;
    const bool dtile = wk.sym && ti == tj;
    float* const c = e.c + mb * e.sc;
    const float* const y = e.y ? e.y + mb * e.sy : nullptr;
    const int64_t ri = static_cast<int64_t>(ti) * kBigM, rj = static_cast<int64_t>(tj) * kBigN;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int lr = (tid >> 4) + 16 * p;   // row within the block
        const int li = 32 * q + lr;           // row within the tile
        const int64_t off = static_cast<int64_t>(li) * kBigN + lj;
        f32x4 v = *reinterpret_cast<const f32x4*>(part + tt * kBigElems + off);
        for (uint32_t s = 1; s < wk.ksplit; ++s) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(
                part + (static_cast<int64_t>(s) * wk.tail + tt) * kBigElems + off);
            v = v + x;
        }
        const int64_t gi = ri + li;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int64_t gj = rj + lj + x;
            float o = e.alpha * v[x];
            if (y) o = o + e.beta * y[gi * e.ldy + gj];
            if (gi == gj) o = o + e.diag;
            if (!dtile || gi <= gj) c[gi * e.ldc + gj] = o;
            if (wk.sym) tr[cl + x][lr] = o;
        }
    }
    if (wk.sym) {   // uniform: C[j][i] for the block's (i, j), 32 consecutive i per row
        __syncthreads();
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int idx = p * 256 + tid;
            const int mr = idx >> 5, mc = idx & 31;   // block column, block row
            const int64_t gi = ri + 32 * q + mc, gj = rj + 64 * h + mr;
            if (!dtile || gi < gj) c[gj * e.ldc + gi] = tr[mr][mc];
        }
    }
}

// ---- Frobenius norm (two-stage fp64 reduction, fixed order) ---------------

constexpr int kRedBlocks = 1024;
constexpr int kRedThreads = 256;

// A batch's elementwise passes run as one launch each, matrix blockIdx.y of
// the batch per grid row; every matrix is split into blocks exactly as it
// would be alone, so a batch gives each matrix the same bits.
constexpr int kMaxBatch = 64;   // matrices per launch (the C ABI's limit)
struct MatPtrs {                // one pointer per matrix, passed by value
    const float* p[kMaxBatch];
};
struct MatPtrsW {
    float* p[kMaxBatch];
};

// Whether a matrix's elementwise pass can take 16-byte packs: n a multiple
// of 4 and every (non-null) pointer 16-byte aligned.
__device__ __forceinline__ bool vec4_ok(const void* a, const void* b, const void* c, int64_t n) {
    const uintptr_t u = reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) |
                        reinterpret_cast<uintptr_t>(c);
    return (n & 3) == 0 && (u & 15) == 0;
}

// Stage 1: block b of matrix m sums the squares of its grid-stride elements
// in fp64 into partial[m * gridDim.x + b].  With ys.p[m], the element is x -
// y (rounded in fp32) and is also written to d0 + m * sd.
__global__ __launch_bounds__(kRedThreads) void k_sumsq_partial(MatPtrs xs, MatPtrs ys,
                                                               float* __restrict__ d0, int64_t sd,
                                                               int64_t n,
                                                               double* __restrict__ partial) {
    __shared__ double red[kRedThreads];
    const int m = static_cast<int>(blockIdx.y);
    const float* __restrict__ x = xs.p[m];
    const float* __restrict__ y = ys.p[m];
    float* __restrict__ d = d0 + m * sd;
    double s = 0.0;
    const int64_t first = static_cast<int64_t>(blockIdx.x) * kRedThreads + threadIdx.x;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kRedThreads;
    if (vec4_ok(x, y, y ? d : nullptr, n)) {   // uniform: 16-byte packs, squares in pack order
        for (int64_t e = first; e < n / 4; e += stride) {
            f32x4 v = reinterpret_cast<const f32x4*>(x)[e];
            if (y) {
                v = v - reinterpret_cast<const f32x4*>(y)[e];
                reinterpret_cast<f32x4*>(d)[e] = v;
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) s += static_cast<double>(v[c]) * static_cast<double>(v[c]);
        }
    } else {
        for (int64_t e = first; e < n; e += stride) {
            float v = x[e];
            if (y) {
                v = v - y[e];
                d[e] = v;
            }
            s += static_cast<double>(v) * static_cast<double>(v);
        }
    }
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = kRedThreads / 2; w > 0; w >>= 1) {
        if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) partial[static_cast<int64_t>(m) * gridDim.x + blockIdx.x] = red[0];
}

// Stage 2 (block m for matrix m): inv[m] = 1 / sqrt(sum of its partials),
// or 0 for a zero matrix.
__global__ __launch_bounds__(kRedThreads) void k_sumsq_final(const double* __restrict__ partial,
                                                             int nparts, float* __restrict__ inv) {
    __shared__ double red[kRedThreads];
    const double* __restrict__ pm = partial + static_cast<int64_t>(blockIdx.x) * nparts;
    double s = 0.0;
    for (int p = threadIdx.x; p < nparts; p += kRedThreads) s += pm[p];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = kRedThreads / 2; w > 0; w >>= 1) {
        if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0)
        inv[blockIdx.x] = red[0] > 0.0 ? static_cast<float>(1.0 / sqrt(red[0])) : 0.0f;
}

// x_m[e] = src_m[e] * inv[m], x_m = x0 + m * sx, src_m = srcs.p[m] or (when
// null) x_m itself: each element is read and written by the same thread
__global__ __launch_bounds__(256) void k_scale(float* x0, int64_t sx, MatPtrs srcs,
                                               const float* __restrict__ inv, int64_t n) {
    const int m = static_cast<int>(blockIdx.y);
    float* x = x0 + m * sx;
    const float* src = srcs.p[m] ? srcs.p[m] : x;
    const float s = inv[m];
    const int64_t first = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    if (vec4_ok(x, src, nullptr, n)) {
        for (int64_t e = first; e < n / 4; e += stride)
            reinterpret_cast<f32x4*>(x)[e] = reinterpret_cast<const f32x4*>(src)[e] * s;
    } else {
        for (int64_t e = first; e < n; e += stride) x[e] = src[e] * s;
    }
}

constexpr float kQa = 3.4445f, kQb = -4.7750f, kQc = 2.0315f;

int64_t align256(int64_t b) { return (b + 255) / 256 * 256; }

constexpr int64_t kStreamGroups = 512;          // two resident workgroups on each of 256 CUs
constexpr int64_t kMinUnits = 8;                // K-tiles per workgroup at least
constexpr int64_t kSplitMinSpan = 64;           // split mode: K-tiles per range at least

// The split of a batch of M x N x K products (see Work).  With a workspace
// of at least 2 * groups tiles the units are spread over up to
// kStreamGroups workgroups; otherwise each workgroup takes one whole tile.
void plan_gemm(int64_t M, int64_t N, int64_t K, bool sym, int64_t batch, int64_t ws_bytes,
               Work& wk, int64_t* need_bytes = nullptr) {
    const int64_t tn = (N + kTileN - 1) / kTileN, tm = (M + kTileM - 1) / kTileM;
    const int64_t per = sym ? tn * (tn + 1) / 2 : tm * tn;
    const int64_t tiles = per * batch;
    const int64_t kt = K > 0 ? (K + kTileK - 1) / kTileK : 1;
    const int64_t units = tiles * kt;
    int64_t g = units / kMinUnits;
    if (g > kStreamGroups) g = kStreamGroups;
    if (g >= kXcds) g -= g % kXcds;
    if (g < 1) g = 1;
    const int64_t need = 2 * g * kTileElems * 4;
    // whole-tile rounds for all but the last one or two rounds' worth of
    // tiles, which are split stream-K
    const int64_t rounds = tiles >= 2 * g ? tiles / g - 1 : 0;
    const int64_t sk_units = (tiles - rounds * g) * kt;
    const bool stream = need <= ws_bytes && sk_units <= static_cast<int64_t>(UINT32_MAX) &&
                        g != tiles;
    const int64_t groups = stream ? g : tiles;
    wk.ksplit = 0;
    wk.kspan = 0;
    // Split mode, for fewer tiles than resident workgroups over a long K:
    // R rounds of units (range, tile) with S = R * 512 / tiles ranges (at
    // least kSplitMinSpan K-tiles each); taken when some R brings the
    // busiest workgroup's K-tiles within 3% of an even stream-K split.
    if (tiles < kStreamGroups && kt >= 2 * kSplitMinSpan) {
        int64_t best = INT64_MAX, best_s = 0, best_span = 0;
        for (int64_t R = 1; R <= 8; ++R) {
            int64_t S = R * kStreamGroups / tiles;
            if (S * kSplitMinSpan > kt) S = kt / kSplitMinSpan;
            if (S < 2) continue;
            const int64_t span = (kt + S - 1) / S;
            S = (kt + span - 1) / span;                // ranges actually needed
            const int64_t load = (tiles * S + kStreamGroups - 1) / kStreamGroups * span;
            if (load < best) {
                best = load;
                best_s = S;
                best_span = span;
            }
        }
        const int64_t even = (units + kStreamGroups - 1) / kStreamGroups;
        const int64_t split_need = tiles * best_s * kTileElems * 4;
        if (best_s > 1 && best * 100 <= even * 103 && split_need <= ws_bytes) {
            wk.tiles_n = static_cast<uint32_t>(tn);
            wk.tiles_per = static_cast<uint32_t>(per);
            wk.tiles = static_cast<uint32_t>(tiles);
            wk.kt = static_cast<uint32_t>(kt);
            const int64_t sg = tiles * best_s < kStreamGroups ? tiles * best_s : kStreamGroups;
            wk.groups = static_cast<uint32_t>(sg);
            wk.per_xcd = static_cast<uint32_t>((sg + kXcds - 1) / kXcds);
            wk.dp_rounds = 0;
            wk.units = 0;
            wk.ksplit = static_cast<uint32_t>(best_s);
            wk.kspan = static_cast<uint32_t>(best_span);
            wk.sym = sym;
            if (need_bytes) *need_bytes = split_need;
            return;
        }
    }
    wk.tiles_n = static_cast<uint32_t>(tn);
    wk.tiles_per = static_cast<uint32_t>(per);
    wk.tiles = static_cast<uint32_t>(tiles);
    wk.kt = static_cast<uint32_t>(kt);
    wk.groups = static_cast<uint32_t>(groups);
    wk.per_xcd = static_cast<uint32_t>((groups + kXcds - 1) / kXcds);
    wk.dp_rounds = stream ? static_cast<uint32_t>(rounds) : 1;
    wk.units = stream ? static_cast<uint32_t>(sk_units) : 0;
    wk.sym = sym;
    if (need_bytes) *need_bytes = need;
}


// A batch of `batch` products on k_gemm: operand b at A + b*sa and B + b*sb,
// result and Y at e.c + b*e.sc and e.y + b*e.sy.
hipError_t gemm_general(bool tn, const float* A, int64_t lda, int64_t sa, const float* B,
                        int64_t ldb, int64_t sb, int64_t M, int64_t N, int64_t K,
                        const Epilogue& e, bool sym, int64_t batch, float* part,
                        int64_t part_bytes, hipStream_t s) {
    Work wk;
    plan_gemm(M, N, K, sym, batch, part ? part_bytes : 0, wk);
    const dim3 grid(wk.per_xcd * kXcds);
    // float4 loads of row-major operands need 16-byte aligned rows (and
    // batch strides)
    const bool vec_a = reinterpret_cast<uintptr_t>(A) % 16 == 0 && lda % 4 == 0 && sa % 4 == 0;
    const bool vec_b = reinterpret_cast<uintptr_t>(B) % 16 == 0 && ldb % 4 == 0 && sb % 4 == 0;
    if (tn)
        hipLaunchKernelGGL((k_gemm<true>), grid, dim3(kGemmThreads), 0, s, A, lda, B, ldb, M, N, K,
                           sa, sb, wk, vec_a, vec_b, e, part);
    else
        hipLaunchKernelGGL((k_gemm<false>), grid, dim3(kGemmThreads), 0, s, A, lda, B, ldb, M, N, K,
                           sa, sb, wk, vec_a, vec_b, e, part);
    if (wk.ksplit > 1)                                         // every tile in pieces
        hipLaunchKernelGGL(k_reduce_splits, dim3(wk.tiles * 4), dim3(256), 0, s, part, wk, M, N, e);
    else if (wk.units != 0 && (wk.units / wk.kt) % wk.groups != 0)   // pieces of cut tiles to add
        hipLaunchKernelGGL(k_reduce_pieces, dim3(wk.groups * 4), dim3(256), 0, s, part, wk, M, N, e);
    return hipGetLastError();
}

// Whether a product's main block can run on k_gemm_big: K a multiple of 16,
// 16-byte aligned operand rows (and batch strides) with leading dimensions
// below 2^24 (32-bit lane offsets); a symmetric result square with M a
// multiple of 256 (no ragged strips) and 16-byte aligned rows (mirrored
// float4 stores).  A diagonal term needs the result's diagonal inside the
// main block: a non-symmetric product with one and ragged strips runs
// wholly on k_gemm (a strip's own diagonal is not the result's).
bool big_fits(bool sym, const Epilogue& e, const float* A, int64_t lda, int64_t sa,
              const float* B, int64_t ldb, int64_t sb, int64_t M, int64_t N, int64_t K) {
    if (K < kBigK || K % kBigK != 0 || M < kBigM || N < kBigN) return false;
    if (e.diag != 0.0f && (M % kBigM != 0 || N % kBigN != 0)) return false;
    if (reinterpret_cast<uintptr_t>(A) % 16 || reinterpret_cast<uintptr_t>(B) % 16 ||
        lda % 4 || ldb % 4 || sa % 4 || sb % 4)
        return false;
    if (lda >= (int64_t{1} << 24) || ldb >= (int64_t{1} << 24)) return false;
    if (sym && (M != N || M % kBigM != 0 || reinterpret_cast<uintptr_t>(e.c) % 16 ||
                e.ldc % 4 || e.sc % 4))
        return false;
    return true;
}

// Time model of the large-tile kernel: a tile of K takes 2 * 256^2 * K
// flops at a 256th of 145 TFLOP/s on its CU; each piece of a split tile adds
// its partial sums written and read back (512 KiB at 5 TB/s), and the split
// a reduction launch.
constexpr double kBigCuFlops = 145e12 / kBigGroups;
constexpr double kBigPieceSeconds = 2.0 * kBigElems * 4 / 5e12;
constexpr double kBigReduceSeconds = 10e-6;

// How k_gemm_big spreads a product (main block M/256 x N/256 tiles, or its
// upper triangle): whole tiles in rounds of 256, and possibly the last
// round's tiles in pieces along K (one round of pieces at most, each piece
// 256 KiB of part_bytes), whichever the time model finishes first.  Taken
// when that time is within 12% of the work spread evenly over all CUs;
// false otherwise.  need_bytes: the partial-buffer bytes of the choice.
bool plan_big(int64_t M, int64_t N, int64_t K, bool sym, int64_t batch, int64_t part_bytes,
              BigWork& wk, int64_t* need_bytes = nullptr) {
    const int64_t tn = N / kBigN, tm = M / kBigM;
    const int64_t per = sym ? tn * (tn + 1) / 2 : tm * tn;
    const int64_t tiles = per * batch, nk = K / kBigK;
    if (tiles < 1 || nk < 1 || tiles > (int64_t{1} << 30)) return false;
    const double tile_s = 2.0 * kBigElems * static_cast<double>(K) / kBigCuFlops;
    double best = static_cast<double>((tiles + kBigGroups - 1) / kBigGroups) * tile_s;
    int64_t best_s = 1, best_span = nk;
    const int64_t dp = tiles / kBigGroups * kBigGroups, R = tiles - dp;
    for (int64_t S = 2; R > 0 && S <= nk && R * S <= kBigGroups; ++S) {
        const int64_t span = (nk + S - 1) / S, se = (nk + span - 1) / span;
        const int64_t pieces = R * se;
        if (pieces * kBigElems * 4 > part_bytes) break;
        const double t = static_cast<double>(dp / kBigGroups) * tile_s +
                         tile_s * static_cast<double>(span) / static_cast<double>(nk) +
                         static_cast<double>(pieces) * kBigPieceSeconds + kBigReduceSeconds;
        if (t < best) {
            best = t;
            best_s = se;
            best_span = span;
        }
    }
    const double even = static_cast<double>(tiles) * tile_s / kBigGroups;
    if (best > even * 1.12) return false;
    wk.tiles_n = static_cast<uint32_t>(tn);
    wk.tiles_per = static_cast<uint32_t>(per);
    wk.nk = static_cast<uint32_t>(nk);
    wk.sym = sym;
    const bool split = best_s > 1;
    wk.dp = static_cast<uint32_t>(split ? dp : tiles);
    wk.tail = static_cast<uint32_t>(split ? R : 0);
    wk.ksplit = static_cast<uint32_t>(best_s);
    wk.kspan = static_cast<uint32_t>(best_span);
    if (need_bytes) *need_bytes = split ? R * best_s * kBigElems * 4 : 0;
    return true;
}

// Partial-buffer bytes of the preferred split of a batch of products (on
// k_gemm, or on k_gemm_big for aligned operands).
int64_t gemm_partial_bytes(int64_t M, int64_t N, int64_t K, bool sym, int64_t batch = 1) {
    Work wk;
    int64_t need = 0;
    plan_gemm(M, N, K, sym, batch, INT64_MAX, wk, &need);
    BigWork bw;
    int64_t big = 0;
    if (K % kBigK == 0 && M >= kBigM && N >= kBigN && (!sym || (M == N && M % kBigM == 0)) &&
        plan_big(M, N, K, sym, batch, INT64_MAX, bw, &big) && big > need)
        need = big;
    return need;
}

// A batch of `batch` products: operand b at A + b*sa and B + b*sb, result and
// Y at e.c + b*e.sc and e.y + b*e.sy.  The main block on k_gemm_big when it
// fits and pays, the strips past the last whole 256 rows and columns (not
// for a symmetric result, whose M is a multiple of 256 there) on k_gemm;
// otherwise everything on k_gemm.
hipError_t gemm(bool tn, const float* A, int64_t lda, int64_t sa, const float* B, int64_t ldb,
                int64_t sb, int64_t M, int64_t N, int64_t K, const Epilogue& e, bool sym,
                int64_t batch, float* part, int64_t part_bytes, hipStream_t s) {
    BigWork wk;
    if (!big_fits(sym, e, A, lda, sa, B, ldb, sb, M, N, K) ||
        !plan_big(M, N, K, sym, batch, part ? part_bytes : 0, wk))
        return gemm_general(tn, A, lda, sa, B, ldb, sb, M, N, K, e, sym, batch, part, part_bytes,
                            s);
    if (tn)
        hipLaunchKernelGGL(k_gemm_big<true>, dim3(kBigGroups), dim3(kGemmThreads), 0, s, A, lda,
                           sa, B, ldb, sb, wk, e, part);
    else
        hipLaunchKernelGGL(k_gemm_big<false>, dim3(kBigGroups), dim3(kGemmThreads), 0, s, A, lda,
                           sa, B, ldb, sb, wk, e, part);
    if (wk.tail != 0)
        hipLaunchKernelGGL(k_reduce_big, dim3(wk.tail * 32), dim3(256), 0, s, part, wk, e);
    if (hipError_t err = hipGetLastError()) return err;
    const int64_t mm = M / kBigM * kBigM, nm = N / kBigN * kBigN;
    if (mm < M) {   // rows mm .. M-1, every column
        Epilogue eb = e;
        eb.c = e.c + mm * e.ldc;
        eb.y = e.y ? e.y + mm * e.ldy : nullptr;
        if (hipError_t err = gemm_general(tn, tn ? A + mm : A + mm * lda, lda, sa, B, ldb, sb,
                                          M - mm, N, K, eb, false, batch, part, part_bytes, s))
            return err;
    }
    if (nm < N) {   // rows 0 .. mm-1, columns nm .. N-1
        Epilogue er = e;
        er.c = e.c + nm;
        er.y = e.y ? e.y + nm : nullptr;
        if (hipError_t err = gemm_general(tn, A, lda, sa, tn ? B + nm : B + nm * ldb, ldb, sb, mm,
                                          N - nm, K, er, false, batch, part, part_bytes, s))
            return err;
    }
    return hipSuccess;
}

}  // namespace

namespace {

// Partial-buffer bytes of the iteration's three products on a batch of
// rows x cols matrices: the symmetric Gram matrix, its symmetric square, the
// next iterate.
int64_t polar_partial_bytes(int64_t rows, int64_t cols, int64_t batch) {
    const int64_t r = rows < cols ? rows : cols, L = rows < cols ? cols : rows;
    int64_t b = gemm_partial_bytes(r, r, L, true, batch);
    const int64_t sq = gemm_partial_bytes(r, r, r, true, batch);
    const int64_t nx = gemm_partial_bytes(rows, cols, r, false, batch);
    if (sq > b) b = sq;
    if (nx > b) b = nx;
    return b;
}

// Workspace layout of a batch: per matrix the norm partials, then the
// inverse norms, then per matrix two iterates and the Gram and polynomial
// matrices (each region 256-byte aligned per matrix), then the partial tiles.
struct PolarSpace {
    double* partial;
    float* inv;
    float *xa, *xb, *g, *m, *part;
    int64_t sx, sg, part_bytes, total;
};

PolarSpace polar_space(void* ws, int64_t rows, int64_t cols, int64_t batch) {
    const int64_t n = rows * cols, r = rows < cols ? rows : cols;
    PolarSpace sp{};
    sp.sx = align256(n * 4) / 4;
    sp.sg = align256(r * r * 4) / 4;
    sp.part_bytes = align256(polar_partial_bytes(rows, cols, batch));
    char* p = static_cast<char*>(ws);
    const int64_t o_inv = align256(batch * kRedBlocks * 8);
    const int64_t o_xa = o_inv + align256(batch * 4);
    const int64_t o_xb = o_xa + batch * sp.sx * 4;
    const int64_t o_g = o_xb + batch * sp.sx * 4;
    const int64_t o_m = o_g + batch * sp.sg * 4;
    const int64_t o_part = o_m + batch * sp.sg * 4;
    sp.total = o_part + sp.part_bytes;
    if (p) {
        sp.partial = reinterpret_cast<double*>(p);
        sp.inv = reinterpret_cast<float*>(p + o_inv);
        sp.xa = reinterpret_cast<float*>(p + o_xa);
        sp.xb = reinterpret_cast<float*>(p + o_xb);
        sp.g = reinterpret_cast<float*>(p + o_g);
        sp.m = reinterpret_cast<float*>(p + o_m);
        sp.part = reinterpret_cast<float*>(p + o_part);
    }
    return sp;
}

// theta_m = theta_m - scale * P_m (matrix blockIdx.y, P_m = P0 + m * sp), the
// same two roundings as the fused epilogue: fl(fl(-scale * P) + theta).
__global__ __launch_bounds__(256) void k_step(MatPtrsW thetas, const float* __restrict__ P0,
                                              int64_t sp, float scale, int64_t n) {
    const int m = static_cast<int>(blockIdx.y);
    float* __restrict__ theta = thetas.p[m];
    const float* __restrict__ P = P0 + m * sp;
    const float ns = -scale;
    const int64_t first = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    if (vec4_ok(theta, P, nullptr, n)) {
        f32x4* t4 = reinterpret_cast<f32x4*>(theta);
        const f32x4* p4 = reinterpret_cast<const f32x4*>(P);
        for (int64_t e = first; e < n / 4; e += stride) t4[e] = ns * p4[e] + t4[e];
    } else {
        for (int64_t e = first; e < n; e += stride) theta[e] = ns * P[e] + theta[e];
    }
}

}  // namespace

int64_t polar_workspace_bytes(int64_t rows, int64_t cols, int64_t batch) {
    return polar_space(nullptr, rows, cols, batch).total;
}

hipError_t polar_iterate(const float* const* src, const float* const* sub, float* const* out,
                         float* const* theta, float scale, int64_t batch, int64_t rows,
                         int64_t cols, int quintic, int cubic, void* ws, hipStream_t s) {
    if (batch < 1 || batch > kMaxBatch || (batch > 1 && (out || !theta)))
        return hipErrorInvalidValue;
    const int64_t n = rows * cols;
    const bool tall = rows >= cols;
    const int64_t r = tall ? cols : rows;
    const PolarSpace sp = polar_space(ws, rows, cols, batch);

    // X0 = A / ||A||_F per matrix, with A = src (or src - sub, formed in fp32
    // into the first iterate); one launch per pass for the whole batch
    MatPtrs ps{}, pu{}, pscale{};
    for (int64_t b = 0; b < batch; ++b) {
        ps.p[b] = src[b];
        pu.p[b] = sub ? sub[b] : nullptr;
        pscale.p[b] = sub ? nullptr : src[b];   // scale the difference in place
    }
    const unsigned nb = static_cast<unsigned>(batch);
    hipLaunchKernelGGL(k_sumsq_partial, dim3(kRedBlocks, nb), dim3(kRedThreads), 0, s, ps, pu,
                       sp.xa, sp.sx, n, sp.partial);
    hipLaunchKernelGGL(k_sumsq_final, dim3(nb), dim3(kRedThreads), 0, s, sp.partial, kRedBlocks,
                       sp.inv);
    hipLaunchKernelGGL(k_scale, dim3(4096, nb), dim3(256), 0, s, sp.xa, sp.sx, pscale, sp.inv, n);
    if (hipError_t err = hipGetLastError()) return err;

    // A single matrix writes its result straight from the last product's
    // epilogue; a batch writes P to the workspace and finishes per matrix.
    const bool direct = batch == 1;
    float* x = sp.xa;
    float* xn = sp.xb;
    const int steps = quintic + cubic;
    for (int st = 0; st < steps; ++st) {
        const bool quin = st < quintic;
        // Gram matrix (r x r) of the current iterate; for the cubic steps the
        // epilogue forms M = 1.5 I - 0.5 G directly.
        Epilogue eg{quin ? sp.g : sp.m, r, nullptr, 0, quin ? 1.0f : -0.5f, 0.0f,
                    quin ? 0.0f : 1.5f};
        eg.sc = sp.sg;
        // Both r x r results are symmetric: only their upper triangles are
        // computed, and the lower ones are mirror images (exactly symmetric).
        hipError_t err =
            tall ? gemm(true, x, cols, sp.sx, x, cols, sp.sx, r, r, rows, eg, true, batch,
                        sp.part, sp.part_bytes, s)                                    // X^T X
                 : gemm(false, x, cols, sp.sx, x, cols, sp.sx, r, r, cols, eg, true, batch,
                        sp.part, sp.part_bytes, s);                                   // X X^T
        if (err) return err;
        if (quin) {   // M = c G^2 + b G + a I  (G exactly symmetric: G G = G G^T, so the
                      // row-major (NT) path, the faster one, applies)
            Epilogue em{sp.m, r, sp.g, r, kQc, kQb, kQa};
            em.sc = sp.sg;
            em.sy = sp.sg;
            if ((err = gemm(false, sp.g, r, sp.sg, sp.g, r, sp.sg, r, r, r, em, true, batch,
                            sp.part, sp.part_bytes, s)))
                return err;
        }
        // next iterate: X M (tall) or M X (wide); the last step of a single
        // matrix writes the result: the polar factor to out, or theta -
        // scale * P onto theta
        const bool last = st == steps - 1;
        Epilogue ex{xn, cols, nullptr, 0, 1.0f, 0.0f, 0.0f};
        ex.sc = sp.sx;
        if (last && direct && out) ex = Epilogue{out[0], cols, nullptr, 0, 1.0f, 0.0f, 0.0f};
        if (last && direct && theta)
            ex = Epilogue{theta[0], cols, theta[0], cols, -scale, 1.0f, 0.0f};
        err = tall ? gemm(false, x, cols, sp.sx, sp.m, r, sp.sg, rows, cols, r, ex, false, batch,
                          sp.part, sp.part_bytes, s)
                   : gemm(true, sp.m, r, sp.sg, x, cols, sp.sx, rows, cols, r, ex, false, batch,
                          sp.part, sp.part_bytes, s);
        // (tall: C[i][j] = sum_k X[i][k] M[j][k]; wide: C[i][j] = sum_k M[k][i] X[k][j])
        if (err) return err;
        float* t = x;
        x = xn;
        xn = t;
    }
    if (!direct) {   // x holds the batch's polar factors
        MatPtrsW pt{};
        for (int64_t b = 0; b < batch; ++b) pt.p[b] = theta[b];
        hipLaunchKernelGGL(k_step, dim3(4096, nb), dim3(256), 0, s, pt, x, sp.sx, scale, n);
    }
    return hipGetLastError();
}

int64_t matmul_workspace_bytes(int64_t M, int64_t N, int64_t K, bool sym, int64_t batch) {
    return gemm_partial_bytes(M, N, K, sym, batch);
}

bool matmul_large_tiles(int64_t M, int64_t N, int64_t K, bool sym, int64_t batch,
                        int64_t ws_bytes) {
    // contiguous operands: leading dimension K (row-major) or M and N (k-major)
    const int64_t kMaxLd = int64_t{1} << 24;
    if (K % kBigK != 0 || M < kBigM || N < kBigN || (sym && (M != N || M % kBigM != 0)) ||
        K >= kMaxLd || M >= kMaxLd || N >= kMaxLd)
        return false;
    BigWork wk;
    return plan_big(M, N, K, sym, batch, ws_bytes, wk);
}

hipError_t matmul(bool tn, const float* A, int64_t lda, int64_t sa, const float* B, int64_t ldb,
                  int64_t sb, int64_t M, int64_t N, int64_t K, float* C, int64_t ldc, int64_t sc,
                  const float* Y, int64_t sy, float alpha, float beta, float diag, bool sym,
                  int64_t batch, void* ws, int64_t ws_bytes, hipStream_t s) {
    Epilogue e{C, ldc, Y, ldc, alpha, beta, diag};
    e.sc = sc;
    e.sy = sy;
    return gemm(tn, A, lda, sa, B, ldb, sb, M, N, K, e, sym, batch, static_cast<float*>(ws),
                ws ? ws_bytes : 0, s);
}

}  // namespace dlk

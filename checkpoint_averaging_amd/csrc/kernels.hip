// Streaming kernels of the DiLoCo outer-step merge for CDNA4 (gfx950).
//
// Every kernel is elementwise over a flat fp32 parameter range: no element
// depends on another, so the work is pure HBM streaming with a few binary32
// operations per element and no use for MFMA or LDS.  Design points:
//
//  * 128-bit global accesses.  A lane moves one 4-element pack per stream
//    (16 B of fp32, 8 B of bf16); consecutive lanes take consecutive packs, so
//    each wavefront instruction reads or writes one dense 1 KiB span.
//  * Several packs per lane (UNROLL), all loads issued before any store, so a
//    lane keeps UNROLL x (streams) 16-byte loads in flight to cover HBM
//    latency.
//  * Non-temporal loads and stores for ranges too large to stay in the
//    Infinity Cache; ordinary (cached) accesses for small ranges, where a
//    fragment's accumulator can still be resident at the next fold.
//  * No workgroup reuses another's data, so the block -> XCD round-robin
//    placement needs no remapping; each block takes one contiguous tile.
//  * The element operation is written once, as a scalar function, and used by
//    the vector body, the scalar fallback and the ragged tail alike.
//  * Arithmetic is IEEE binary32 with one rounding per operation: the file is
//    built with -ffp-contract=off (plus the pragma below), no fast-math,
//    correctly rounded division and subnormals kept, so the result follows
//    the operation order the merge defines.
//
// The merge definitions come from the DiffuRefill-1B technical report
// (section "Training system", Table 2: rows "Outer step" and "Side
// averages"), the DiffuRefill-1B model card ("How it is trained": Merging and
// EMA bullets) and the GradientMail post "Pythia-14M on four rented GPUs and a
// bucket" (section "Getting updates through the bucket": token-weighted mean
// of deltas and outer Nesterov, learning rate 0.7, momentum 0.9).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

#pragma clang fp contract(off)

namespace dlk {

namespace {

constexpr int kBlock = 256;     // 4 wave64 per workgroup
constexpr int kUnroll = 4;      // packs per lane per tile
constexpr int kPack = 4;        // elements per pack

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <bool NT, typename T>
__device__ __forceinline__ T ld(const T* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <bool NT, typename T>
__device__ __forceinline__ void st(T* p, T v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// ---- checkpoint element types ---------------------------------------------

// bfloat16 is the high half of a binary32 word: widening is a 16-bit shift,
// exact for every bit pattern.
__device__ __forceinline__ float widen_bf16(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

template <typename CT> struct Ckpt;

template <> struct Ckpt<float> {
    using pack_t = f32x4;
    static __device__ __forceinline__ float one(const float* c, int64_t j) { return c[j]; }
    template <bool NT>
    static __device__ __forceinline__ f32x4 pack(const float* c, int64_t p) {
        return ld<NT>(reinterpret_cast<const f32x4*>(c) + p);
    }
};

template <> struct Ckpt<uint16_t> {
    using pack_t = u32x2;
    static __device__ __forceinline__ float one(const uint16_t* c, int64_t j) {
        return widen_bf16(c[j]);
    }
    // 4 bf16 = 8 bytes; element 2k sits in the low half of word k.
    template <bool NT>
    static __device__ __forceinline__ f32x4 pack(const uint16_t* c, int64_t p) {
        u32x2 w = ld<NT>(reinterpret_cast<const u32x2*>(c) + p);
        f32x4 v;
        v.x = __uint_as_float(w.x << 16);
        v.y = __uint_as_float(w.x & 0xFFFF0000u);
        v.z = __uint_as_float(w.y << 16);
        v.w = __uint_as_float(w.y & 0xFFFF0000u);
        return v;
    }
};

// ---- element operations (one binary32 rounding per operator) ---------------

struct FoldSumOp {          // running fp32 sum: S = c (first) or S + c
    __device__ __forceinline__ float operator()(float s, float c, bool first) const {
        return first ? c : s + c;
    }
};

struct FoldDeltaOp {        // weighted delta: A = w*(theta - c) (first) or A + w*(theta - c)
    float w;
    __device__ __forceinline__ float operator()(float a, float theta, float c, bool first) const {
        float d = theta - c;
        float p = w * d;
        return first ? p : a + p;
    }
};

struct EmaOp {              // e' = beta*e + (1 - beta)*x
    float beta, omega;
    __device__ __forceinline__ float operator()(float e, float x) const {
        float a = beta * e;
        float b = omega * x;
        return a + b;
    }
};

struct MeanOp {             // g = S / N
    float count;
    __device__ __forceinline__ float operator()(float s) const { return s / count; }
};

struct NesterovOp {         // dbar = A/W; m' = mu*m + dbar; u = dbar + mu*m'; theta' = theta - lr*u
    float total, lr, mu;
    __device__ __forceinline__ void operator()(float a, float& theta, float& m) const {
        float dbar = a / total;
        float mm = mu * m;
        float m_new = mm + dbar;
        float mu_m = mu * m_new;
        float u = dbar + mu_m;
        float step = lr * u;
        theta = theta - step;
        m = m_new;
    }
};

// ---- tiling helpers ---------------------------------------------------------

// Packs are assigned as: tile t = blockIdx.x covers packs
// [t*kBlock*kUnroll, (t+1)*kBlock*kUnroll); lane l of the block takes packs
// t*kBlock*kUnroll + k*kBlock + l for k < kUnroll.  VEC = 1 runs the same
// scheme with one-element "packs" (scalar fallback for unaligned pointers).
__device__ __forceinline__ int64_t tile_base() {
    return static_cast<int64_t>(blockIdx.x) * (kBlock * kUnroll) + threadIdx.x;
}

// Elements past the last whole pack (fewer than kPack) are handled by the
// first lanes of the last block.
__device__ __forceinline__ int64_t tail_index(int64_t npacks, int64_t n) {
    if (blockIdx.x != gridDim.x - 1) return -1;
    int64_t j = npacks * kPack + threadIdx.x;
    return j < n ? j : -1;
}

// ---- kernels ----------------------------------------------------------------

template <typename CT, bool FIRST, bool VEC4, bool NT>
__global__ __launch_bounds__(kBlock) void k_fold_sum(float* __restrict__ acc,
                                                     const CT* __restrict__ c, int64_t n) {
    const FoldSumOp op;
    if constexpr (VEC4) {
        const int64_t npacks = n / kPack;
        const int64_t p0 = tile_base();
        f32x4 cv[kUnroll], sv[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t p = p0 + k * kBlock;
            if (p < npacks) {
                cv[k] = Ckpt<CT>::template pack<NT>(c, p);
                if (!FIRST) sv[k] = ld<NT>(reinterpret_cast<const f32x4*>(acc) + p);
            }
        }
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t p = p0 + k * kBlock;
            if (p < npacks) {
                f32x4 r;
#pragma unroll
                for (int i = 0; i < kPack; ++i) r[i] = op(FIRST ? 0.0f : sv[k][i], cv[k][i], FIRST);
                st<NT>(reinterpret_cast<f32x4*>(acc) + p, r);
            }
        }
        const int64_t j = tail_index(npacks, n);
        if (j >= 0) acc[j] = op(FIRST ? 0.0f : acc[j], Ckpt<CT>::one(c, j), FIRST);
    } else {
        const int64_t j0 = tile_base();
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t j = j0 + k * kBlock;
            if (j < n) acc[j] = op(FIRST ? 0.0f : acc[j], Ckpt<CT>::one(c, j), FIRST);
        }
    }
}

template <typename CT, bool FIRST, bool VEC4, bool NT>
__global__ __launch_bounds__(kBlock) void k_fold_delta(float* __restrict__ acc,
                                                       const float* __restrict__ theta,
                                                       const CT* __restrict__ c, float w,
                                                       int64_t n) {
    const FoldDeltaOp op{w};
    if constexpr (VEC4) {
        const int64_t npacks = n / kPack;
        const int64_t p0 = tile_base();
        f32x4 cv[kUnroll], tv[kUnroll], av[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t p = p0 + k * kBlock;
            if (p < npacks) {
                tv[k] = ld<NT>(reinterpret_cast<const f32x4*>(theta) + p);
                cv[k] = Ckpt<CT>::template pack<NT>(c, p);
                if (!FIRST) av[k] = ld<NT>(reinterpret_cast<const f32x4*>(acc) + p);
            }
        }
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t p = p0 + k * kBlock;
            if (p < npacks) {
                f32x4 r;
#pragma unroll
                for (int i = 0; i < kPack; ++i)
                    r[i] = op(FIRST ? 0.0f : av[k][i], tv[k][i], cv[k][i], FIRST);
                st<NT>(reinterpret_cast<f32x4*>(acc) + p, r);
            }
        }
        const int64_t j = tail_index(npacks, n);
        if (j >= 0) acc[j] = op(FIRST ? 0.0f : acc[j], theta[j], Ckpt<CT>::one(c, j), FIRST);
    } else {
        const int64_t j0 = tile_base();
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t j = j0 + k * kBlock;
            if (j < n) acc[j] = op(FIRST ? 0.0f : acc[j], theta[j], Ckpt<CT>::one(c, j), FIRST);
        }
    }
}

// out may be the same array as sum (in place); each element is read and then
// written by the same lane, so the two pointers are not marked restrict.
template <bool EMA, bool VEC4, bool NT>
__global__ __launch_bounds__(kBlock) void k_finalize_mean(float* out, const float* sum,
                                                          float* __restrict__ ema, int64_t n,
                                                          MeanOp mean, EmaOp eop) {
    if constexpr (VEC4) {
        const int64_t npacks = n / kPack;
        const int64_t p0 = tile_base();
        f32x4 sv[kUnroll], ev[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t p = p0 + k * kBlock;
            if (p < npacks) {
                sv[k] = ld<NT>(reinterpret_cast<const f32x4*>(sum) + p);
                if (EMA) ev[k] = ld<NT>(reinterpret_cast<const f32x4*>(ema) + p);
            }
        }
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t p = p0 + k * kBlock;
            if (p < npacks) {
                f32x4 g, e;
#pragma unroll
                for (int i = 0; i < kPack; ++i) {
                    g[i] = mean(sv[k][i]);
                    if (EMA) e[i] = eop(ev[k][i], g[i]);
                }
                st<NT>(reinterpret_cast<f32x4*>(out) + p, g);
                if (EMA) st<NT>(reinterpret_cast<f32x4*>(ema) + p, e);
            }
        }
        const int64_t j = tail_index(npacks, n);
        if (j >= 0) {
            float g = mean(sum[j]);
            out[j] = g;
            if (EMA) ema[j] = eop(ema[j], g);
        }
    } else {
        const int64_t j0 = tile_base();
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t j = j0 + k * kBlock;
            if (j < n) {
                float g = mean(sum[j]);
                out[j] = g;
                if (EMA) ema[j] = eop(ema[j], g);
            }
        }
    }
}

template <bool EMA, bool VEC4, bool NT>
__global__ __launch_bounds__(kBlock) void k_nesterov(float* __restrict__ theta,
                                                     float* __restrict__ m,
                                                     const float* __restrict__ acc,
                                                     float* __restrict__ ema, int64_t n,
                                                     NesterovOp nop, EmaOp eop) {
    if constexpr (VEC4) {
        const int64_t npacks = n / kPack;
        const int64_t p0 = tile_base();
        f32x4 av[kUnroll], tv[kUnroll], mv[kUnroll], ev[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t p = p0 + k * kBlock;
            if (p < npacks) {
                av[k] = ld<NT>(reinterpret_cast<const f32x4*>(acc) + p);
                tv[k] = ld<NT>(reinterpret_cast<const f32x4*>(theta) + p);
                mv[k] = ld<NT>(reinterpret_cast<const f32x4*>(m) + p);
                if (EMA) ev[k] = ld<NT>(reinterpret_cast<const f32x4*>(ema) + p);
            }
        }
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t p = p0 + k * kBlock;
            if (p < npacks) {
                f32x4 t = tv[k], mm = mv[k], e;
#pragma unroll
                for (int i = 0; i < kPack; ++i) {
                    float ti = t[i], mi = mm[i];
                    nop(av[k][i], ti, mi);
                    t[i] = ti;
                    mm[i] = mi;
                    if (EMA) e[i] = eop(ev[k][i], ti);
                }
                st<NT>(reinterpret_cast<f32x4*>(theta) + p, t);
                st<NT>(reinterpret_cast<f32x4*>(m) + p, mm);
                if (EMA) st<NT>(reinterpret_cast<f32x4*>(ema) + p, e);
            }
        }
        const int64_t j = tail_index(npacks, n);
        if (j >= 0) {
            float t = theta[j], mj = m[j];
            nop(acc[j], t, mj);
            theta[j] = t;
            m[j] = mj;
            if (EMA) ema[j] = eop(ema[j], t);
        }
    } else {
        const int64_t j0 = tile_base();
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t j = j0 + k * kBlock;
            if (j < n) {
                float t = theta[j], mj = m[j];
                nop(acc[j], t, mj);
                theta[j] = t;
                m[j] = mj;
                if (EMA) ema[j] = eop(ema[j], t);
            }
        }
    }
}

template <bool VEC4, bool NT>
__global__ __launch_bounds__(kBlock) void k_ema(float* __restrict__ ema,
                                                const float* __restrict__ g, int64_t n,
                                                EmaOp eop) {
    if constexpr (VEC4) {
        const int64_t npacks = n / kPack;
        const int64_t p0 = tile_base();
        f32x4 ev[kUnroll], gv[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t p = p0 + k * kBlock;
            if (p < npacks) {
                ev[k] = ld<NT>(reinterpret_cast<const f32x4*>(ema) + p);
                gv[k] = ld<NT>(reinterpret_cast<const f32x4*>(g) + p);
            }
        }
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t p = p0 + k * kBlock;
            if (p < npacks) {
                f32x4 r;
#pragma unroll
                for (int i = 0; i < kPack; ++i) r[i] = eop(ev[k][i], gv[k][i]);
                st<NT>(reinterpret_cast<f32x4*>(ema) + p, r);
            }
        }
        const int64_t j = tail_index(npacks, n);
        if (j >= 0) ema[j] = eop(ema[j], g[j]);
    } else {
        const int64_t j0 = tile_base();
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t j = j0 + k * kBlock;
            if (j < n) ema[j] = eop(ema[j], g[j]);
        }
    }
}

// ---- launch helpers ---------------------------------------------------------

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

// Ranges of at least this many elements (64 MiB of fp32) stream with
// non-temporal accesses; smaller ones keep the default cache policy so that a
// fragment's accumulator can stay in the 256 MB Infinity Cache between folds.
constexpr int64_t kNontemporalMin = int64_t(1) << 24;

unsigned grid_for(int64_t n, bool vec4) {
    const int64_t units = vec4 ? n / kPack : n;
    int64_t blocks = (units + kBlock * kUnroll - 1) / (kBlock * kUnroll);
    if (blocks < 1) blocks = 1;       // the ragged tail still needs one block
    return static_cast<unsigned>(blocks);
}

// Dispatches a kernel template over the VEC4 x NT choices.
#define DLK_DISPATCH2(VEC4, NT, LAUNCH)                           \
    do {                                                          \
        if (VEC4) {                                               \
            if (NT) { LAUNCH(true, true); } else { LAUNCH(true, false); } \
        } else {                                                  \
            if (NT) { LAUNCH(false, true); } else { LAUNCH(false, false); } \
        }                                                         \
    } while (0)

}  // namespace

hipError_t launch_fold_sum(float* acc, const void* ckpt, bool bf16, int64_t n, bool first,
                           hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const bool vec4 = aligned16(acc) && (bf16 ? aligned8(ckpt) : aligned16(ckpt));
    const bool nt = n >= kNontemporalMin;
    const dim3 grid(grid_for(n, vec4)), block(kBlock);
#define L(V, N)                                                                              \
    if (bf16) {                                                                              \
        auto c = static_cast<const uint16_t*>(ckpt);                                         \
        if (first) hipLaunchKernelGGL((k_fold_sum<uint16_t, true, V, N>), grid, block, 0, s, acc, c, n); \
        else hipLaunchKernelGGL((k_fold_sum<uint16_t, false, V, N>), grid, block, 0, s, acc, c, n); \
    } else {                                                                                 \
        auto c = static_cast<const float*>(ckpt);                                            \
        if (first) hipLaunchKernelGGL((k_fold_sum<float, true, V, N>), grid, block, 0, s, acc, c, n); \
        else hipLaunchKernelGGL((k_fold_sum<float, false, V, N>), grid, block, 0, s, acc, c, n); \
    }
    DLK_DISPATCH2(vec4, nt, L);
#undef L
    return hipGetLastError();
}

hipError_t launch_fold_delta(float* acc, const float* theta, const void* ckpt, bool bf16,
                             float w, int64_t n, bool first, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const bool vec4 = aligned16(acc) && aligned16(theta) &&
                      (bf16 ? aligned8(ckpt) : aligned16(ckpt));
    const bool nt = n >= kNontemporalMin;
    const dim3 grid(grid_for(n, vec4)), block(kBlock);
#define L(V, N)                                                                              \
    if (bf16) {                                                                              \
        auto c = static_cast<const uint16_t*>(ckpt);                                         \
        if (first) hipLaunchKernelGGL((k_fold_delta<uint16_t, true, V, N>), grid, block, 0, s, acc, theta, c, w, n); \
        else hipLaunchKernelGGL((k_fold_delta<uint16_t, false, V, N>), grid, block, 0, s, acc, theta, c, w, n); \
    } else {                                                                                 \
        auto c = static_cast<const float*>(ckpt);                                            \
        if (first) hipLaunchKernelGGL((k_fold_delta<float, true, V, N>), grid, block, 0, s, acc, theta, c, w, n); \
        else hipLaunchKernelGGL((k_fold_delta<float, false, V, N>), grid, block, 0, s, acc, theta, c, w, n); \
    }
    DLK_DISPATCH2(vec4, nt, L);
#undef L
    return hipGetLastError();
}

hipError_t launch_finalize_mean(float* out, const float* sum, float count, float* ema,
                                float beta, float omega, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const bool vec4 = aligned16(out) && aligned16(sum) && (ema == nullptr || aligned16(ema));
    const bool nt = n >= kNontemporalMin;
    const dim3 grid(grid_for(n, vec4)), block(kBlock);
    const MeanOp mop{count};
    const EmaOp eop{beta, omega};
#define L(V, N)                                                                              \
    if (ema) hipLaunchKernelGGL((k_finalize_mean<true, V, N>), grid, block, 0, s, out, sum, ema, n, mop, eop); \
    else hipLaunchKernelGGL((k_finalize_mean<false, V, N>), grid, block, 0, s, out, sum, ema, n, mop, eop);
    DLK_DISPATCH2(vec4, nt, L);
#undef L
    return hipGetLastError();
}

hipError_t launch_nesterov(float* theta, float* m, const float* acc, float total, float lr,
                           float mu, float* ema, float beta, float omega, int64_t n,
                           hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const bool vec4 = aligned16(theta) && aligned16(m) && aligned16(acc) &&
                      (ema == nullptr || aligned16(ema));
    const bool nt = n >= kNontemporalMin;
    const dim3 grid(grid_for(n, vec4)), block(kBlock);
    const NesterovOp nop{total, lr, mu};
    const EmaOp eop{beta, omega};
#define L(V, N)                                                                              \
    if (ema) hipLaunchKernelGGL((k_nesterov<true, V, N>), grid, block, 0, s, theta, m, acc, ema, n, nop, eop); \
    else hipLaunchKernelGGL((k_nesterov<false, V, N>), grid, block, 0, s, theta, m, acc, ema, n, nop, eop);
    DLK_DISPATCH2(vec4, nt, L);
#undef L
    return hipGetLastError();
}

hipError_t launch_ema(float* ema, const float* g, float beta, float omega, int64_t n,
                      hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const bool vec4 = aligned16(ema) && aligned16(g);
    const bool nt = n >= kNontemporalMin;
    const dim3 grid(grid_for(n, vec4)), block(kBlock);
    const EmaOp eop{beta, omega};
#define L(V, N) hipLaunchKernelGGL((k_ema<V, N>), grid, block, 0, s, ema, g, n, eop);
    DLK_DISPATCH2(vec4, nt, L);
#undef L
    return hipGetLastError();
}

}  // namespace dlk

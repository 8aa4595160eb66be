// Streaming kernels of the DiLoCo outer-step merge for CDNA4 (gfx950).
//
// Every kernel is elementwise over a flat fp32 parameter range: no element
// depends on another, so the work is pure HBM streaming with a few binary32
// operations per element and no use for MFMA or LDS.  One engine runs every
// operation; an operation is a small functor that says which streams it
// loads and stores and what it computes per element.
//
//  * 128-bit global accesses.  A lane moves one 4-element pack per stream
//    (16 B of fp32, 8 B of bf16); consecutive lanes take consecutive packs, so
//    each wavefront instruction reads or writes one dense 1 KiB span.
//  * Every load of a tile is issued before its first store; HBM latency is
//    covered by many resident waves (one 1024-element tile per 256-lane
//    workgroup, about a million workgroups at 1.08B elements) rather than by
//    deep per-lane unrolling.
//  * Non-temporal loads and stores for ranges too large to stay in the
//    256 MB Infinity Cache; ordinary (cached) accesses for small ranges, where
//    a fragment's accumulator can still be resident at the next fold.  One
//    stream is always read through the cache: the global theta of the
//    fragment merge, which every pass over a fragment reads again (each fold
//    and the close).  Leaving the cache to it alone keeps part of theta there
//    from one pass to the next.  On MI355X the 1.08B fragment round took
//    1.7-3% less time that way (the library's builds alternating in one
//    process).  The close writes theta non-temporally: the next pass is
//    another fragment's, so a cached store would only leave dirty lines for
//    that pass to write back (same round time, measured).  Caching the
//    accumulator, momentum or EMA as well was slower, and so was caching the
//    running sum of the mean merge.
//  * Alternating direction: on non-temporal (large) ranges a pass may walk
//    its tiles from the last to the first, so that consecutive passes over
//    the same fragment meet where the previous one ended and find part of its
//    data still cached.  Elements are independent, so the direction never
//    changes a result.  Small, cache-resident ranges always walk forward.
//  * No workgroup reuses another's data, so the block -> XCD round-robin
//    placement needs no remapping; each block takes one contiguous tile.
//  * The element arithmetic is written once, as scalar functions, and used by
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
constexpr int kUnroll = 1;      // packs per lane per tile (1 measured fastest: many short
                                // workgroups keep more waves resident than deeper per-lane
                                // unrolling; 2, 4 and 8 were 2-6% slower on MI355X)
constexpr int kPack = 4;        // elements per pack
constexpr int64_t kTile = int64_t(kBlock) * kUnroll;   // packs (or scalars) per block

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

template <bool NT>
__device__ __forceinline__ f32x4 ld4(const float* base, int64_t p) {
    return ld<NT>(reinterpret_cast<const f32x4*>(base) + p);
}

template <bool NT>
__device__ __forceinline__ void st4(float* base, int64_t p, f32x4 v) {
    st<NT>(reinterpret_cast<f32x4*>(base) + p, v);
}

// ---- checkpoint element types ---------------------------------------------

// bfloat16 is the high half of a binary32 word: widening is a 16-bit shift,
// exact for every bit pattern.
__device__ __forceinline__ float widen_bf16(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

template <typename CT> struct Ckpt;

template <> struct Ckpt<float> {
    static __device__ __forceinline__ float one(const float* c, int64_t j) { return c[j]; }
    template <bool NT>
    static __device__ __forceinline__ f32x4 pack(const float* c, int64_t p) {
        return ld4<NT>(c, p);
    }
};

template <> struct Ckpt<uint16_t> {
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

// ---- element arithmetic (one binary32 rounding per operator) ---------------

// running fp32 sum: S = c for the first arrival, S + c after
__device__ __forceinline__ float fold_sum(float s, float c, bool first) {
    return first ? c : s + c;
}

// weighted delta: A = w*(theta - c) for the first arrival, A + w*(theta - c) after
__device__ __forceinline__ float fold_delta(float a, float theta, float c, float w, bool first) {
    const float d = theta - c;
    const float p = w * d;
    return first ? p : a + p;
}

// e' = beta*e + (1 - beta)*x
__device__ __forceinline__ float ema_step(float e, float x, float beta, float omega) {
    const float a = beta * e;
    const float b = omega * x;
    return a + b;
}

// dbar = A/W; m' = mu*m + dbar; u = dbar + mu*m'; theta' = theta - lr*u
__device__ __forceinline__ void nesterov_step(float a, float total, float lr, float mu,
                                              float& theta, float& m) {
    const float dbar = a / total;
    const float mm = mu * m;
    const float m_new = mm + dbar;
    const float mu_m = mu * m_new;
    const float u = dbar + mu_m;
    const float step = lr * u;
    theta = theta - step;
    m = m_new;
}

// ---- operations ---------------------------------------------------------------
//
// Each operation provides
//   struct Regs                       the loaded values of one pack
//   load<NT>(p, Regs&)                loads pack p of every input stream
//   store<NT>(p, const Regs&)         computes and stores pack p
//   scalar(j)                         the same for element j alone
// Pointers are already offset to the fragment.

template <typename CT, bool FIRST>
struct FoldSum {                // acc = c (first) or acc + c
    float* acc;
    const CT* c;
    struct Regs { f32x4 c, s; };
    template <bool NT> __device__ void load(int64_t p, Regs& r) const {
        r.c = Ckpt<CT>::template pack<NT>(c, p);
        if constexpr (!FIRST) r.s = ld4<NT>(acc, p);
    }
    template <bool NT> __device__ void store(int64_t p, const Regs& r) const {
        f32x4 o;
#pragma unroll
        for (int i = 0; i < kPack; ++i) o[i] = fold_sum(FIRST ? 0.0f : r.s[i], r.c[i], FIRST);
        st4<NT>(acc, p, o);
    }
    __device__ void scalar(int64_t j) const {
        acc[j] = fold_sum(FIRST ? 0.0f : acc[j], Ckpt<CT>::one(c, j), FIRST);
    }
};

template <typename CT, bool FIRST>
struct FoldDelta {              // acc = w*(theta - c) (first) or acc + w*(theta - c)
    float* acc;
    const float* theta;
    const CT* c;
    float w;
    struct Regs { f32x4 a, t, c; };
    template <bool NT> __device__ void load(int64_t p, Regs& r) const {
        r.t = ld4<false>(theta, p);             // cached: every pass reads theta again
        r.c = Ckpt<CT>::template pack<NT>(c, p);
        if constexpr (!FIRST) r.a = ld4<NT>(acc, p);
    }
    template <bool NT> __device__ void store(int64_t p, const Regs& r) const {
        f32x4 o;
#pragma unroll
        for (int i = 0; i < kPack; ++i)
            o[i] = fold_delta(FIRST ? 0.0f : r.a[i], r.t[i], r.c[i], w, FIRST);
        st4<NT>(acc, p, o);
    }
    __device__ void scalar(int64_t j) const {
        acc[j] = fold_delta(FIRST ? 0.0f : acc[j], theta[j], Ckpt<CT>::one(c, j), w, FIRST);
    }
};

template <bool EMA>
struct MeanClose {              // out = S / N; ema = beta*ema + omega*out.  out may be sum.
    float* out;
    const float* sum;
    float* ema;
    float count, beta, omega;
    struct Regs { f32x4 s, e; };
    template <bool NT> __device__ void load(int64_t p, Regs& r) const {
        r.s = ld4<NT>(sum, p);
        if constexpr (EMA) r.e = ld4<NT>(ema, p);
    }
    template <bool NT> __device__ void store(int64_t p, const Regs& r) const {
        f32x4 g, e;
#pragma unroll
        for (int i = 0; i < kPack; ++i) {
            g[i] = r.s[i] / count;
            if constexpr (EMA) e[i] = ema_step(r.e[i], g[i], beta, omega);
        }
        st4<NT>(out, p, g);
        if constexpr (EMA) st4<NT>(ema, p, e);
    }
    __device__ void scalar(int64_t j) const {
        const float g = sum[j] / count;
        out[j] = g;
        if constexpr (EMA) ema[j] = ema_step(ema[j], g, beta, omega);
    }
};

template <bool EMA>
struct NesterovClose {          // outer Nesterov from the accumulated weighted deltas (+ EMA)
    float* theta;
    float* m;
    const float* acc;
    float* ema;
    float total, lr, mu, beta, omega;
    struct Regs { f32x4 a, t, m, e; };
    template <bool NT> __device__ void load(int64_t p, Regs& r) const {
        r.a = ld4<NT>(acc, p);
        r.t = ld4<false>(theta, p);             // cached: every pass reads theta again
        r.m = ld4<NT>(m, p);
        if constexpr (EMA) r.e = ld4<NT>(ema, p);
    }
    template <bool NT> __device__ void store(int64_t p, const Regs& r) const {
        f32x4 t = r.t, mm = r.m, e;
#pragma unroll
        for (int i = 0; i < kPack; ++i) {
            float ti = t[i], mi = mm[i];
            nesterov_step(r.a[i], total, lr, mu, ti, mi);
            t[i] = ti;
            mm[i] = mi;
            if constexpr (EMA) e[i] = ema_step(r.e[i], ti, beta, omega);
        }
        st4<NT>(theta, p, t);
        st4<NT>(m, p, mm);
        if constexpr (EMA) st4<NT>(ema, p, e);
    }
    __device__ void scalar(int64_t j) const {
        float t = theta[j], mj = m[j];
        nesterov_step(acc[j], total, lr, mu, t, mj);
        theta[j] = t;
        m[j] = mj;
        if constexpr (EMA) ema[j] = ema_step(ema[j], t, beta, omega);
    }
};

// The round's last arrival folded and the fragment closed in one pass: the
// sum is completed in registers and never written back.  Same operations, in
// the same order, as FoldSum followed by MeanClose.  out may be sum.
template <typename CT, bool FIRST, bool EMA>
struct FoldMeanClose {
    float* out;
    const float* sum;
    const CT* c;
    float* ema;
    float count, beta, omega;
    struct Regs { f32x4 s, c, e; };
    template <bool NT> __device__ void load(int64_t p, Regs& r) const {
        r.c = Ckpt<CT>::template pack<NT>(c, p);
        if constexpr (!FIRST) r.s = ld4<NT>(sum, p);
        if constexpr (EMA) r.e = ld4<NT>(ema, p);
    }
    template <bool NT> __device__ void store(int64_t p, const Regs& r) const {
        f32x4 g, e;
#pragma unroll
        for (int i = 0; i < kPack; ++i) {
            const float s = fold_sum(FIRST ? 0.0f : r.s[i], r.c[i], FIRST);
            g[i] = s / count;
            if constexpr (EMA) e[i] = ema_step(r.e[i], g[i], beta, omega);
        }
        st4<NT>(out, p, g);
        if constexpr (EMA) st4<NT>(ema, p, e);
    }
    __device__ void scalar(int64_t j) const {
        const float s = fold_sum(FIRST ? 0.0f : sum[j], Ckpt<CT>::one(c, j), FIRST);
        const float g = s / count;
        out[j] = g;
        if constexpr (EMA) ema[j] = ema_step(ema[j], g, beta, omega);
    }
};

// The round's last arrival folded and the outer Nesterov step taken in one
// pass: theta is read once for both the delta and the update, and the
// accumulator is completed in registers and never written back.  Same
// operations, in the same order, as FoldDelta followed by NesterovClose.
template <typename CT, bool FIRST, bool EMA>
struct FoldNesterovClose {
    float* theta;
    float* m;
    const float* acc;
    const CT* c;
    float* ema;
    float w, total, lr, mu, beta, omega;
    struct Regs { f32x4 a, t, c, m, e; };
    template <bool NT> __device__ void load(int64_t p, Regs& r) const {
        r.t = ld4<false>(theta, p);             // cached: every pass reads theta again
        r.c = Ckpt<CT>::template pack<NT>(c, p);
        if constexpr (!FIRST) r.a = ld4<NT>(acc, p);
        r.m = ld4<NT>(m, p);
        if constexpr (EMA) r.e = ld4<NT>(ema, p);
    }
    template <bool NT> __device__ void store(int64_t p, const Regs& r) const {
        f32x4 t = r.t, mm = r.m, e;
#pragma unroll
        for (int i = 0; i < kPack; ++i) {
            const float a = fold_delta(FIRST ? 0.0f : r.a[i], r.t[i], r.c[i], w, FIRST);
            float ti = t[i], mi = mm[i];
            nesterov_step(a, total, lr, mu, ti, mi);
            t[i] = ti;
            mm[i] = mi;
            if constexpr (EMA) e[i] = ema_step(r.e[i], ti, beta, omega);
        }
        st4<NT>(theta, p, t);
        st4<NT>(m, p, mm);
        if constexpr (EMA) st4<NT>(ema, p, e);
    }
    __device__ void scalar(int64_t j) const {
        float t = theta[j], mj = m[j];
        const float a = fold_delta(FIRST ? 0.0f : acc[j], t, Ckpt<CT>::one(c, j), w, FIRST);
        nesterov_step(a, total, lr, mu, t, mj);
        theta[j] = t;
        m[j] = mj;
        if constexpr (EMA) ema[j] = ema_step(ema[j], t, beta, omega);
    }
};

// ---- several arrivals in one pass ----------------------------------------------
//
// A merger that already holds several arrivals of a fragment (they came in
// while it waited for its quorum, or a restarted merger finds them waiting)
// folds them in one pass.  Every arrival's pack is loaded, then the
// operations of the one-arrival passes run in registers, in arrival order, so
// the results are those passes' bit for bit; the accumulator (and, when the
// pass also closes, the global, momentum and EMA) is read and written once
// instead of once per arrival.  k is a kernel argument: the unrolled loops
// test it with a uniform branch, so a pass loads only its k checkpoints.
constexpr int kMaxArrivals = 8;

template <typename CT>
struct Arrivals {
    const CT* c[kMaxArrivals];   // fragment-length checkpoints, in arrival order
    float w[kMaxArrivals];       // token weights (delta folds only)
    int k;                       // 1 <= k <= kMaxArrivals

    template <bool NT> __device__ void load(int64_t p, f32x4 (&v)[kMaxArrivals]) const {
#pragma unroll
        for (int i = 0; i < kMaxArrivals; ++i)
            if (i < k) v[i] = Ckpt<CT>::template pack<NT>(c[i], p);
    }
    // S = c_0 (first) or S + c_0, then S + c_i for each later arrival
    __device__ f32x4 sum(f32x4 s, const f32x4 (&v)[kMaxArrivals], bool first) const {
#pragma unroll
        for (int e = 0; e < kPack; ++e) s[e] = fold_sum(s[e], v[0][e], first);
#pragma unroll
        for (int i = 1; i < kMaxArrivals; ++i)
            if (i < k) {
#pragma unroll
                for (int e = 0; e < kPack; ++e) s[e] = fold_sum(s[e], v[i][e], false);
            }
        return s;
    }
    // A = w_0*(theta - c_0) (first) or A + w_0*(theta - c_0), then A + w_i*(theta - c_i)
    __device__ f32x4 delta(f32x4 a, f32x4 t, const f32x4 (&v)[kMaxArrivals], bool first) const {
#pragma unroll
        for (int e = 0; e < kPack; ++e) a[e] = fold_delta(a[e], t[e], v[0][e], w[0], first);
#pragma unroll
        for (int i = 1; i < kMaxArrivals; ++i)
            if (i < k) {
#pragma unroll
                for (int e = 0; e < kPack; ++e) a[e] = fold_delta(a[e], t[e], v[i][e], w[i], false);
            }
        return a;
    }
    __device__ float sum_one(float s, int64_t j, bool first) const {
        s = fold_sum(s, Ckpt<CT>::one(c[0], j), first);
#pragma unroll
        for (int i = 1; i < kMaxArrivals; ++i)
            if (i < k) s = fold_sum(s, Ckpt<CT>::one(c[i], j), false);
        return s;
    }
    __device__ float delta_one(float a, float t, int64_t j, bool first) const {
        a = fold_delta(a, t, Ckpt<CT>::one(c[0], j), w[0], first);
#pragma unroll
        for (int i = 1; i < kMaxArrivals; ++i)
            if (i < k) a = fold_delta(a, t, Ckpt<CT>::one(c[i], j), w[i], false);
        return a;
    }
};

template <typename CT, bool FIRST>
struct FoldSumMany {            // FoldSum of each arrival in turn
    float* acc;
    Arrivals<CT> in;
    struct Regs { f32x4 s; f32x4 c[kMaxArrivals]; };
    template <bool NT> __device__ void load(int64_t p, Regs& r) const {
        in.template load<NT>(p, r.c);
        if constexpr (!FIRST) r.s = ld4<NT>(acc, p);
    }
    template <bool NT> __device__ void store(int64_t p, const Regs& r) const {
        st4<NT>(acc, p, in.sum(FIRST ? f32x4{} : r.s, r.c, FIRST));
    }
    __device__ void scalar(int64_t j) const {
        acc[j] = in.sum_one(FIRST ? 0.0f : acc[j], j, FIRST);
    }
};

template <typename CT, bool FIRST>
struct FoldDeltaMany {          // FoldDelta of each arrival in turn
    float* acc;
    const float* theta;
    Arrivals<CT> in;
    struct Regs { f32x4 a, t; f32x4 c[kMaxArrivals]; };
    template <bool NT> __device__ void load(int64_t p, Regs& r) const {
        r.t = ld4<false>(theta, p);             // cached: later passes read theta again
        in.template load<NT>(p, r.c);
        if constexpr (!FIRST) r.a = ld4<NT>(acc, p);
    }
    template <bool NT> __device__ void store(int64_t p, const Regs& r) const {
        st4<NT>(acc, p, in.delta(FIRST ? f32x4{} : r.a, r.t, r.c, FIRST));
    }
    __device__ void scalar(int64_t j) const {
        acc[j] = in.delta_one(FIRST ? 0.0f : acc[j], theta[j], j, FIRST);
    }
};

// The fragment's remaining arrivals folded and the fragment closed with the
// mean (+ EMA) in one pass: FoldSumMany followed by MeanClose.  out may be sum.
template <typename CT, bool FIRST, bool EMA>
struct FoldManyMeanClose {
    float* out;
    const float* sum;
    Arrivals<CT> in;
    float* ema;
    float count, beta, omega;
    struct Regs { f32x4 s, e; f32x4 c[kMaxArrivals]; };
    template <bool NT> __device__ void load(int64_t p, Regs& r) const {
        in.template load<NT>(p, r.c);
        if constexpr (!FIRST) r.s = ld4<NT>(sum, p);
        if constexpr (EMA) r.e = ld4<NT>(ema, p);
    }
    template <bool NT> __device__ void store(int64_t p, const Regs& r) const {
        const f32x4 s = in.sum(FIRST ? f32x4{} : r.s, r.c, FIRST);
        f32x4 g, e;
#pragma unroll
        for (int i = 0; i < kPack; ++i) {
            g[i] = s[i] / count;
            if constexpr (EMA) e[i] = ema_step(r.e[i], g[i], beta, omega);
        }
        st4<NT>(out, p, g);
        if constexpr (EMA) st4<NT>(ema, p, e);
    }
    __device__ void scalar(int64_t j) const {
        const float g = in.sum_one(FIRST ? 0.0f : sum[j], j, FIRST) / count;
        out[j] = g;
        if constexpr (EMA) ema[j] = ema_step(ema[j], g, beta, omega);
    }
};

// The fragment's remaining arrivals folded (token-weighted deltas) and the
// outer Nesterov step (+ EMA) taken in one pass: FoldDeltaMany followed by
// NesterovClose.  Theta is read once for every delta and the update.
template <typename CT, bool FIRST, bool EMA>
struct FoldManyNesterovClose {
    float* theta;
    float* m;
    const float* acc;
    Arrivals<CT> in;
    float* ema;
    float total, lr, mu, beta, omega;
    struct Regs { f32x4 a, t, m, e; f32x4 c[kMaxArrivals]; };
    template <bool NT> __device__ void load(int64_t p, Regs& r) const {
        r.t = ld4<false>(theta, p);             // cached, as in the one-arrival close
        in.template load<NT>(p, r.c);
        if constexpr (!FIRST) r.a = ld4<NT>(acc, p);
        r.m = ld4<NT>(m, p);
        if constexpr (EMA) r.e = ld4<NT>(ema, p);
    }
    template <bool NT> __device__ void store(int64_t p, const Regs& r) const {
        const f32x4 a = in.delta(FIRST ? f32x4{} : r.a, r.t, r.c, FIRST);
        f32x4 t = r.t, mm = r.m, e;
#pragma unroll
        for (int i = 0; i < kPack; ++i) {
            float ti = t[i], mi = mm[i];
            nesterov_step(a[i], total, lr, mu, ti, mi);
            t[i] = ti;
            mm[i] = mi;
            if constexpr (EMA) e[i] = ema_step(r.e[i], ti, beta, omega);
        }
        st4<NT>(theta, p, t);
        st4<NT>(m, p, mm);
        if constexpr (EMA) st4<NT>(ema, p, e);
    }
    __device__ void scalar(int64_t j) const {
        float t = theta[j], mj = m[j];
        const float a = in.delta_one(FIRST ? 0.0f : acc[j], t, j, FIRST);
        nesterov_step(a, total, lr, mu, t, mj);
        theta[j] = t;
        m[j] = mj;
        if constexpr (EMA) ema[j] = ema_step(ema[j], t, beta, omega);
    }
};

// Keep-local-drift adoption on a worker: theta = theta + (g - pushed), the
// difference rounded first.
template <typename CT>
struct AdoptKeepDrift {
    float* theta;
    const float* g;
    const CT* pushed;
    struct Regs { f32x4 t, g, p; };
    template <bool NT> __device__ void load(int64_t p, Regs& r) const {
        r.t = ld4<NT>(theta, p);
        r.g = ld4<NT>(g, p);
        r.p = Ckpt<CT>::template pack<NT>(pushed, p);
    }
    template <bool NT> __device__ void store(int64_t p, const Regs& r) const {
        f32x4 o;
#pragma unroll
        for (int i = 0; i < kPack; ++i) {
            const float shift = r.g[i] - r.p[i];
            o[i] = r.t[i] + shift;
        }
        st4<NT>(theta, p, o);
    }
    __device__ void scalar(int64_t j) const {
        const float shift = g[j] - Ckpt<CT>::one(pushed, j);
        theta[j] = theta[j] + shift;
    }
};

// Mean of K snapshots read in one pass: S = s_0; S = S + s_i for i = 1..K-1
// in the given order; out = S / K.  K is a template argument so each count
// holds only the registers it reads (higher occupancy for small K).
constexpr int kMaxSnapshots = 16;

template <int K>
struct SnapshotMean {
    float* out;
    const float* snap[K];
    float count;
    struct Regs { f32x4 s[K]; };
    template <bool NT> __device__ void load(int64_t p, Regs& r) const {
#pragma unroll
        for (int i = 0; i < K; ++i) r.s[i] = ld4<NT>(snap[i], p);
    }
    template <bool NT> __device__ void store(int64_t p, const Regs& r) const {
        f32x4 g;
#pragma unroll
        for (int e = 0; e < kPack; ++e) {
            float acc = r.s[0][e];
#pragma unroll
            for (int i = 1; i < K; ++i) acc = fold_sum(acc, r.s[i][e], false);
            g[e] = acc / count;
        }
        st4<NT>(out, p, g);
    }
    __device__ void scalar(int64_t j) const {
        float acc = snap[0][j];
#pragma unroll
        for (int i = 1; i < K; ++i) acc = fold_sum(acc, snap[i][j], false);
        out[j] = acc / count;
    }
};

struct Ema {                    // ema = beta*ema + omega*g
    float* ema;
    const float* g;
    float beta, omega;
    struct Regs { f32x4 e, g; };
    template <bool NT> __device__ void load(int64_t p, Regs& r) const {
        r.e = ld4<NT>(ema, p);
        r.g = ld4<NT>(g, p);
    }
    template <bool NT> __device__ void store(int64_t p, const Regs& r) const {
        f32x4 o;
#pragma unroll
        for (int i = 0; i < kPack; ++i) o[i] = ema_step(r.e[i], r.g[i], beta, omega);
        st4<NT>(ema, p, o);
    }
    __device__ void scalar(int64_t j) const { ema[j] = ema_step(ema[j], g[j], beta, omega); }
};

// ---- the engine -----------------------------------------------------------------

// 128-bit path.  Traversal position q (blocks take q = blockIdx.x,
// blockIdx.x + gridDim.x, ...) is tile q (forward) or tile ntiles-1-q
// (backward); lane l of a tile takes packs tile*kTile + k*kBlock + l,
// k < kUnroll.  The fewer than kPack elements past the last whole pack are
// done by the first lanes of the last block.  The grid is capped (a launch
// may hold at most 2^32 - 1 work-items), so very large ranges loop.
template <class Op, bool NT>
__global__ __launch_bounds__(kBlock) void k_stream(Op op, int64_t n, int backward) {
    const int64_t npacks = n / kPack;
    const int64_t ntiles = (npacks + kTile - 1) / kTile;
    for (int64_t q = blockIdx.x; q < ntiles; q += gridDim.x) {
        const int64_t tile = backward ? ntiles - 1 - q : q;
        const int64_t p0 = tile * kTile + threadIdx.x;
        typename Op::Regs r[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t p = p0 + k * kBlock;
            if (p < npacks) op.template load<NT>(p, r[k]);
        }
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t p = p0 + k * kBlock;
            if (p < npacks) op.template store<NT>(p, r[k]);
        }
    }
    if (blockIdx.x == gridDim.x - 1) {
        const int64_t j = npacks * kPack + threadIdx.x;
        if (j < n) op.scalar(j);
    }
}

// Scalar path (a pointer is not aligned for 128-bit access): one element per
// lane and unroll step, same tiling and grid cap.
template <class Op>
__global__ __launch_bounds__(kBlock) void k_stream_scalar(Op op, int64_t n) {
    const int64_t ntiles = (n + kTile - 1) / kTile;
    for (int64_t q = blockIdx.x; q < ntiles; q += gridDim.x) {
        const int64_t j0 = q * kTile + threadIdx.x;
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t j = j0 + k * kBlock;
            if (j < n) op.scalar(j);
        }
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }
bool ckpt_aligned(const void* c, bool bf16) { return bf16 ? aligned8(c) : aligned16(c); }

// Ranges of at least this many elements (64 MiB of fp32) stream with
// non-temporal accesses; smaller ones keep the default cache policy so that a
// fragment's accumulator can stay in the 256 MB Infinity Cache between folds.
constexpr int64_t kNontemporalMin = int64_t(1) << 24;

// At most this many workgroups per launch (4M x 256 lanes = 2^30 work-items,
// well inside the 2^32 - 1 a launch may hold); beyond 4M tiles blocks loop.
constexpr int64_t kMaxBlocks = int64_t(1) << 22;

int64_t grid_blocks(int64_t tiles) {
    if (tiles < 1) return 1;                     // the ragged tail still needs one block
    return tiles < kMaxBlocks ? tiles : kMaxBlocks;
}

// Launches op over n elements: 128-bit path when `vec4`, else scalar.
template <class Op>
hipError_t launch(const Op& op, int64_t n, bool vec4, bool backward, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const dim3 block(kBlock);
    if (vec4) {
        const dim3 grid(static_cast<unsigned>(grid_blocks((n / kPack + kTile - 1) / kTile)));
        if (n >= kNontemporalMin)
            hipLaunchKernelGGL((k_stream<Op, true>), grid, block, 0, s, op, n, backward ? 1 : 0);
        else
            hipLaunchKernelGGL((k_stream<Op, false>), grid, block, 0, s, op, n, 0);
    } else {
        const dim3 grid(static_cast<unsigned>(grid_blocks((n + kTile - 1) / kTile)));
        hipLaunchKernelGGL((k_stream_scalar<Op>), grid, block, 0, s, op, n);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fold_sum(float* acc, const void* ckpt, bool bf16, int64_t n, bool first,
                           bool backward, hipStream_t s) {
    const bool vec4 = aligned16(acc) && ckpt_aligned(ckpt, bf16);
    if (bf16) {
        auto c = static_cast<const uint16_t*>(ckpt);
        if (first) return launch(FoldSum<uint16_t, true>{acc, c}, n, vec4, backward, s);
        return launch(FoldSum<uint16_t, false>{acc, c}, n, vec4, backward, s);
    }
    auto c = static_cast<const float*>(ckpt);
    if (first) return launch(FoldSum<float, true>{acc, c}, n, vec4, backward, s);
    return launch(FoldSum<float, false>{acc, c}, n, vec4, backward, s);
}

hipError_t launch_fold_delta(float* acc, const float* theta, const void* ckpt, bool bf16,
                             float w, int64_t n, bool first, bool backward, hipStream_t s) {
    const bool vec4 = aligned16(acc) && aligned16(theta) && ckpt_aligned(ckpt, bf16);
    if (bf16) {
        auto c = static_cast<const uint16_t*>(ckpt);
        if (first) return launch(FoldDelta<uint16_t, true>{acc, theta, c, w}, n, vec4, backward, s);
        return launch(FoldDelta<uint16_t, false>{acc, theta, c, w}, n, vec4, backward, s);
    }
    auto c = static_cast<const float*>(ckpt);
    if (first) return launch(FoldDelta<float, true>{acc, theta, c, w}, n, vec4, backward, s);
    return launch(FoldDelta<float, false>{acc, theta, c, w}, n, vec4, backward, s);
}

hipError_t launch_finalize_mean(float* out, const float* sum, float count, float* ema,
                                float beta, float omega, int64_t n, bool backward,
                                hipStream_t s) {
    const bool vec4 = aligned16(out) && aligned16(sum) && (ema == nullptr || aligned16(ema));
    if (ema) return launch(MeanClose<true>{out, sum, ema, count, beta, omega}, n, vec4, backward, s);
    return launch(MeanClose<false>{out, sum, ema, count, beta, omega}, n, vec4, backward, s);
}

hipError_t launch_nesterov(float* theta, float* m, const float* acc, float total, float lr,
                           float mu, float* ema, float beta, float omega, int64_t n,
                           bool backward, hipStream_t s) {
    const bool vec4 = aligned16(theta) && aligned16(m) && aligned16(acc) &&
                      (ema == nullptr || aligned16(ema));
    if (ema)
        return launch(NesterovClose<true>{theta, m, acc, ema, total, lr, mu, beta, omega}, n,
                      vec4, backward, s);
    return launch(NesterovClose<false>{theta, m, acc, ema, total, lr, mu, beta, omega}, n, vec4,
                  backward, s);
}

hipError_t launch_fold_finalize_mean(float* out, const float* sum, const void* ckpt, bool bf16,
                                     bool first, float count, float* ema, float beta,
                                     float omega, int64_t n, bool backward, hipStream_t s) {
    const bool vec4 = aligned16(out) && aligned16(sum) && ckpt_aligned(ckpt, bf16) &&
                      (ema == nullptr || aligned16(ema));
#define DLK_FMC(CT, FIRST, EMA)                                                              \
    return launch(FoldMeanClose<CT, FIRST, EMA>{out, sum, static_cast<const CT*>(ckpt), ema,  \
                                                count, beta, omega},                         \
                  n, vec4, backward, s)
    if (bf16) {
        if (first) { if (ema) DLK_FMC(uint16_t, true, true); else DLK_FMC(uint16_t, true, false); }
        else { if (ema) DLK_FMC(uint16_t, false, true); else DLK_FMC(uint16_t, false, false); }
    }
    if (first) { if (ema) DLK_FMC(float, true, true); else DLK_FMC(float, true, false); }
    if (ema) DLK_FMC(float, false, true);
    DLK_FMC(float, false, false);
#undef DLK_FMC
}

hipError_t launch_fold_nesterov(float* theta, float* m, const float* acc, const void* ckpt,
                                bool bf16, bool first, float w, float total, float lr, float mu,
                                float* ema, float beta, float omega, int64_t n, bool backward,
                                hipStream_t s) {
    const bool vec4 = aligned16(theta) && aligned16(m) && aligned16(acc) &&
                      ckpt_aligned(ckpt, bf16) && (ema == nullptr || aligned16(ema));
#define DLK_FNC(CT, FIRST, EMA)                                                              \
    return launch(FoldNesterovClose<CT, FIRST, EMA>{theta, m, acc,                           \
                                                    static_cast<const CT*>(ckpt), ema, w,    \
                                                    total, lr, mu, beta, omega},             \
                  n, vec4, backward, s)
    if (bf16) {
        if (first) { if (ema) DLK_FNC(uint16_t, true, true); else DLK_FNC(uint16_t, true, false); }
        else { if (ema) DLK_FNC(uint16_t, false, true); else DLK_FNC(uint16_t, false, false); }
    }
    if (first) { if (ema) DLK_FNC(float, true, true); else DLK_FNC(float, true, false); }
    if (ema) DLK_FNC(float, false, true);
    DLK_FNC(float, false, false);
#undef DLK_FNC
}

namespace {

bool valid_arrivals(int k) { return k >= 1 && k <= kMaxArrivals; }

// The arrivals of one pass; *vec4 is cleared if a checkpoint is not aligned
// for the 128-bit path.  Slots past k stay null and are never read.
template <typename CT>
Arrivals<CT> arrivals(const void* const* ckpts, const float* w, int k, bool* vec4) {
    Arrivals<CT> in{};
    in.k = k;
    for (int i = 0; i < k; ++i) {
        in.c[i] = static_cast<const CT*>(ckpts[i]);
        in.w[i] = w != nullptr ? w[i] : 0.0f;
        *vec4 = *vec4 && ckpt_aligned(ckpts[i], sizeof(CT) == 2);
    }
    return in;
}

}  // namespace

int max_arrivals_per_pass() { return kMaxArrivals; }

hipError_t launch_fold_sum_many(float* acc, const void* const* ckpts, int k, bool bf16,
                                int64_t n, bool first, bool backward, hipStream_t s) {
    if (!valid_arrivals(k)) return hipErrorInvalidValue;
    bool vec4 = aligned16(acc);
#define DLK_FSM(CT)                                                                         \
    {                                                                                        \
        const Arrivals<CT> in = arrivals<CT>(ckpts, nullptr, k, &vec4);                      \
        if (first) return launch(FoldSumMany<CT, true>{acc, in}, n, vec4, backward, s);      \
        return launch(FoldSumMany<CT, false>{acc, in}, n, vec4, backward, s);                \
    }
    if (bf16) DLK_FSM(uint16_t);
    DLK_FSM(float);
#undef DLK_FSM
}

hipError_t launch_fold_delta_many(float* acc, const float* theta, const void* const* ckpts,
                                  const float* w, int k, bool bf16, int64_t n, bool first,
                                  bool backward, hipStream_t s) {
    if (!valid_arrivals(k)) return hipErrorInvalidValue;
    bool vec4 = aligned16(acc) && aligned16(theta);
#define DLK_FDM(CT)                                                                          \
    {                                                                                         \
        const Arrivals<CT> in = arrivals<CT>(ckpts, w, k, &vec4);                             \
        if (first) return launch(FoldDeltaMany<CT, true>{acc, theta, in}, n, vec4, backward, s); \
        return launch(FoldDeltaMany<CT, false>{acc, theta, in}, n, vec4, backward, s);        \
    }
    if (bf16) DLK_FDM(uint16_t);
    DLK_FDM(float);
#undef DLK_FDM
}

hipError_t launch_fold_many_finalize_mean(float* out, const float* sum, const void* const* ckpts,
                                          int k, bool bf16, bool first, float count, float* ema,
                                          float beta, float omega, int64_t n, bool backward,
                                          hipStream_t s) {
    if (!valid_arrivals(k)) return hipErrorInvalidValue;
    bool vec4 = aligned16(out) && aligned16(sum) && (ema == nullptr || aligned16(ema));
#define DLK_FMMC(CT, FIRST, EMA)                                                             \
    return launch(FoldManyMeanClose<CT, FIRST, EMA>{out, sum, in, ema, count, beta, omega}, n, \
                  vec4, backward, s)
#define DLK_FMMC_CT(CT)                                                                      \
    {                                                                                         \
        const Arrivals<CT> in = arrivals<CT>(ckpts, nullptr, k, &vec4);                       \
        if (first) { if (ema) DLK_FMMC(CT, true, true); else DLK_FMMC(CT, true, false); }     \
        if (ema) DLK_FMMC(CT, false, true);                                                   \
        DLK_FMMC(CT, false, false);                                                           \
    }
    if (bf16) DLK_FMMC_CT(uint16_t);
    DLK_FMMC_CT(float);
#undef DLK_FMMC_CT
#undef DLK_FMMC
}

hipError_t launch_fold_many_nesterov(float* theta, float* m, const float* acc,
                                     const void* const* ckpts, const float* w, int k, bool bf16,
                                     bool first, float total, float lr, float mu, float* ema,
                                     float beta, float omega, int64_t n, bool backward,
                                     hipStream_t s) {
    if (!valid_arrivals(k)) return hipErrorInvalidValue;
    bool vec4 = aligned16(theta) && aligned16(m) && aligned16(acc) &&
                (ema == nullptr || aligned16(ema));
#define DLK_FMNC(CT, FIRST, EMA)                                                             \
    return launch(FoldManyNesterovClose<CT, FIRST, EMA>{theta, m, acc, in, ema, total, lr, mu, \
                                                        beta, omega},                        \
                  n, vec4, backward, s)
#define DLK_FMNC_CT(CT)                                                                      \
    {                                                                                         \
        const Arrivals<CT> in = arrivals<CT>(ckpts, w, k, &vec4);                             \
        if (first) { if (ema) DLK_FMNC(CT, true, true); else DLK_FMNC(CT, true, false); }     \
        if (ema) DLK_FMNC(CT, false, true);                                                   \
        DLK_FMNC(CT, false, false);                                                           \
    }
    if (bf16) DLK_FMNC_CT(uint16_t);
    DLK_FMNC_CT(float);
#undef DLK_FMNC_CT
#undef DLK_FMNC
}

namespace {

template <int K>
hipError_t launch_snapshot_mean_k(float* out, const float* const* snaps, int64_t n,
                                  hipStream_t s) {
    SnapshotMean<K> op{};
    op.out = out;
    op.count = static_cast<float>(K);
    bool vec4 = aligned16(out);
    for (int i = 0; i < K; ++i) {
        op.snap[i] = snaps[i];
        vec4 = vec4 && aligned16(snaps[i]);
    }
    return launch(op, n, vec4, false, s);
}

template <int K>
hipError_t dispatch_snapshot_mean(int k, float* out, const float* const* snaps, int64_t n,
                                  hipStream_t s) {
    if (k == K) return launch_snapshot_mean_k<K>(out, snaps, n, s);
    if constexpr (K < kMaxSnapshots) return dispatch_snapshot_mean<K + 1>(k, out, snaps, n, s);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_snapshot_mean(float* out, const float* const* snaps, int k, int64_t n,
                               hipStream_t s) {
    if (k < 1 || k > kMaxSnapshots) return hipErrorInvalidValue;
    return dispatch_snapshot_mean<1>(k, out, snaps, n, s);
}

hipError_t launch_adopt_keep_drift(float* theta, const float* g, const void* pushed, bool bf16,
                                   int64_t n, hipStream_t s) {
    const bool vec4 = aligned16(theta) && aligned16(g) && ckpt_aligned(pushed, bf16);
    if (bf16)
        return launch(AdoptKeepDrift<uint16_t>{theta, g, static_cast<const uint16_t*>(pushed)}, n,
                      vec4, false, s);
    return launch(AdoptKeepDrift<float>{theta, g, static_cast<const float*>(pushed)}, n, vec4,
                  false, s);
}

hipError_t launch_ema(float* ema, const float* g, float beta, float omega, int64_t n,
                      hipStream_t s) {
    const bool vec4 = aligned16(ema) && aligned16(g);
    return launch(Ema{ema, g, beta, omega}, n, vec4, false, s);
}

}  // namespace dlk

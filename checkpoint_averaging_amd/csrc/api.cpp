// C ABI of the merge (declared in include/dlmerge.h): the round state machine
// and argument validation on the host, then one kernel launch per call.
//
// Round rules follow the pages: checkpoints must carry the current round's
// tag (DiffuRefill-1B technical report, "Training system", failure rule iii),
// a round closes once its quorum of checkpoints is in (Table 2, row "Merger";
// GradientMail post, "Getting updates through the bucket": quorum 3 per
// fragment, four fragments), quorum 1 drains the leftovers of dead workers
// (Table 2, row "Recovery"), arrivals are folded in the order they come (model
// card, "How it is trained", Merging bullet), and two rounds may be open at
// once (GradientMail post, same section).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <new>
#include <stdexcept>
#include <vector>

#include "dlmerge.h"
#include "kernels.h"
#include "noalloc.h"
#include "polar.h"

namespace {

constexpr int kMaxFrags = 4096;
constexpr int kMaxWorkers = 65536;

struct Fragment {
    bool closed = false;
    std::vector<int> arrivals;       // worker ids in arrival order
    int64_t tokens = 0;              // exact sum (DL_DELTA_NESTEROV)
    const float* global = nullptr;   // global the deltas were taken against
    int passes = 0;                  // kernel passes over this fragment so far
};

struct Span {
    uintptr_t lo, hi;                // [lo, hi)
    bool overlaps(const Span& o) const { return lo < o.hi && o.lo < hi; }
    bool same(const Span& o) const { return lo == o.lo && hi == o.hi; }
};

Span span_of(const void* p, int64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Span{a, a + static_cast<uintptr_t>(bytes)};
}

// A HIP error left pending on this thread by earlier work (a failed call, or
// an asynchronous fault the runtime has reported) is the caller's to see:
// the library neither launches over it nor clears it.  "Not ready" from an
// event or stream query is a status, not a failure: it is consumed so that
// the launch status read after this call's own launch is that launch's.
bool hip_error_pending() {
    const hipError_t e = hipPeekAtLastError();
    if (e == hipErrorNotReady) {
        (void)hipGetLastError();
        return false;
    }
    return e != hipSuccess;
}

// The span must lie inside one device allocation known to the HIP runtime.
// A host pointer or a span running past its allocation is rejected here
// instead of faulting the GPU.  Every call reaches this check before its
// launch, so a pending HIP error is reported here as DL_E_HIP, before the
// runtime is asked anything.
int check_device_span(const void* p, int64_t bytes) {
    if (p == nullptr) return DL_E_INVAL;
    if (hip_error_pending()) return DL_E_HIP;
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, const_cast<void*>(p)) != hipSuccess) {
        (void)hipGetLastError();     // do not leave the failure as a sticky error
        return DL_E_INVAL;
    }
    const uintptr_t b = reinterpret_cast<uintptr_t>(base);
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    if (a < b || bytes < 0 || static_cast<uint64_t>(bytes) > size - (a - b)) return DL_E_INVAL;
    return DL_OK;
}

bool aligned_to(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// 1 - beta, one binary32 subtraction (exact for beta in [0.5, 1]).
float one_minus(float beta) { return 1.0f - beta; }

}  // namespace

struct dl_round {
    uint64_t tag = 0;
    int mode = DL_MEAN;
    int64_t n_params = 0;
    std::vector<int64_t> offsets;
    int quorum = 1;
    int max_workers = 1;
    float* acc = nullptr;
    hipStream_t stream = nullptr;
    bool failed = false;
    std::vector<Fragment> frags;

    int64_t off(int f) const { return offsets[f]; }
    int64_t len(int f) const { return offsets[f + 1] - offsets[f]; }
    int n_frags() const { return static_cast<int>(frags.size()); }
};

namespace {

// Checks shared by every call that folds an arrival: state, indices, tag,
// duplicate, mode-specific arguments, alignment.  Sets *esize to the
// checkpoint element size.  A call folding several arrivals checks each one
// after those before it: `tokens_before` is their token sum and `seen` marks
// every worker already folded into the fragment or earlier in the call.
int check_arrival(const dl_round* r, int frag, int worker_id, uint64_t ckpt_round_tag,
                  const void* ckpt, int dtype, const float* global, int64_t tokens,
                  int64_t* esize, int64_t tokens_before = 0,
                  const std::vector<char>* seen = nullptr) {
    if (r->failed) return DL_E_STATE;
    if (frag < 0 || frag >= r->n_frags()) return DL_E_INVAL;
    const Fragment& F = r->frags[frag];
    if (F.closed) return DL_E_STATE;
    if (worker_id < 0 || worker_id >= r->max_workers) return DL_E_INVAL;
    if (dtype != DL_F32 && dtype != DL_BF16) return DL_E_INVAL;
    if (ckpt_round_tag != r->tag) return DL_E_STALE;
    if (seen != nullptr ? (*seen)[static_cast<size_t>(worker_id)] != 0
                        : std::find(F.arrivals.begin(), F.arrivals.end(), worker_id) !=
                              F.arrivals.end())
        return DL_E_DUP;
    if (r->mode == DL_MEAN) {
        if (global != nullptr) return DL_E_INVAL;
    } else {
        if (global == nullptr || tokens <= 0) return DL_E_INVAL;
        if (F.tokens + tokens_before > INT64_MAX - tokens) return DL_E_INVAL;
        if (F.global != nullptr && F.global != global) return DL_E_INVAL;
    }
    if (ckpt == nullptr) return DL_E_INVAL;
    *esize = dtype == DL_BF16 ? 2 : 4;
    if (!aligned_to(ckpt, static_cast<uintptr_t>(*esize))) return DL_E_ALIGN;
    if (global != nullptr && !aligned_to(global, alignof(float))) return DL_E_ALIGN;
    return DL_OK;
}

// Makes room for `count` more arrivals in the fragment's record before
// anything is launched, so that recording them after the launch cannot fail.
int reserve_arrival(Fragment& F, int count = 1) {
    try {
        F.arrivals.reserve(F.arrivals.size() + static_cast<size_t>(count));
    } catch (const std::bad_alloc&) {
        return DL_E_NOMEM;
    } catch (const std::length_error&) {
        return DL_E_NOMEM;
    }
    return DL_OK;
}

// Records a launch's outcome: a failed launch fails the round.
int after_launch(dl_round* r, hipError_t err) {
    if (err != hipSuccess) {
        r->failed = true;
        return DL_E_HIP;
    }
    return DL_OK;
}

// True if s overlaps any of the n spans at ck.
bool overlaps_any(const Span& s, const Span* ck, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (s.overlaps(ck[i])) return true;
    return false;
}

// Validates the buffers of a mean close over fragment frag.  `ck[0..nck)` are
// the spans of the arrivals folded in the same pass (none for a plain close).
int check_mean_close(dl_round* r, int frag, float* out_global, float* ema, const Span* ck,
                     size_t nck, float** out, float** e) {
    if (out_global == nullptr) return DL_E_INVAL;
    if (!aligned_to(out_global, alignof(float)) || (ema && !aligned_to(ema, alignof(float))))
        return DL_E_ALIGN;
    const int64_t off = r->off(frag), n = r->len(frag);
    float* acc = r->acc + off;
    *out = out_global + off;
    const Span acc_s = span_of(acc, n * 4), out_s = span_of(*out, n * 4);
    if (!out_s.same(acc_s) && out_s.overlaps(acc_s)) return DL_E_INVAL;
    if (overlaps_any(out_s, ck, nck)) return DL_E_INVAL;
    *e = nullptr;
    if (ema != nullptr) {
        *e = ema + off;
        const Span e_s = span_of(*e, n * 4);
        if (e_s.overlaps(acc_s) || e_s.overlaps(out_s) || overlaps_any(e_s, ck, nck))
            return DL_E_INVAL;
        if (int st = check_device_span(*e, n * 4)) return st;
    }
    if (int st = check_device_span(acc, n * 4)) return st;
    return check_device_span(*out, n * 4);
}

// Validates the buffers of a Nesterov close over fragment frag (arrival spans
// as in check_mean_close).
int check_nesterov_close(dl_round* r, int frag, float* global, float* momentum, float* ema,
                         const Span* ck, size_t nck, float** theta, float** m, float** e) {
    if (global == nullptr || momentum == nullptr) return DL_E_INVAL;
    if (!aligned_to(global, alignof(float)) || !aligned_to(momentum, alignof(float)) ||
        (ema && !aligned_to(ema, alignof(float))))
        return DL_E_ALIGN;
    const int64_t off = r->off(frag), n = r->len(frag);
    float* acc = r->acc + off;
    *theta = global + off;
    *m = momentum + off;
    const Span acc_s = span_of(acc, n * 4), th_s = span_of(*theta, n * 4),
               m_s = span_of(*m, n * 4);
    if (th_s.overlaps(acc_s) || m_s.overlaps(acc_s) || m_s.overlaps(th_s)) return DL_E_INVAL;
    if (overlaps_any(th_s, ck, nck) || overlaps_any(m_s, ck, nck)) return DL_E_INVAL;
    *e = nullptr;
    if (ema != nullptr) {
        *e = ema + off;
        const Span e_s = span_of(*e, n * 4);
        if (e_s.overlaps(acc_s) || e_s.overlaps(th_s) || e_s.overlaps(m_s) ||
            overlaps_any(e_s, ck, nck))
            return DL_E_INVAL;
        if (int st = check_device_span(*e, n * 4)) return st;
    }
    if (int st = check_device_span(acc, n * 4)) return st;
    if (int st = check_device_span(*theta, n * 4)) return st;
    return check_device_span(*m, n * 4);
}

// The arrivals of one call that folds several, validated.
struct Arrivals {
    int64_t esize = 0;
    int64_t tokens = 0;                  // exact sum of the call's token counts
    std::vector<float> w;                // each count rounded once (DL_DELTA_NESTEROV)
    std::vector<Span> spans;             // checkpoint spans
};

// Validates `count` arrivals for fragment frag as that many dl_fold_checkpoint
// calls in array order would (duplicates within the call included), without
// recording anything.  Host rules only; check_arrival_spans does the rest.
int check_arrivals(const dl_round* r, int frag, int count, const int* worker_ids,
                   const uint64_t* ckpt_round_tags, const void* const* ckpts, int dtype,
                   const float* global, const int64_t* tokens, Arrivals* a) {
    if (r->failed) return DL_E_STATE;
    if (frag < 0 || frag >= r->n_frags()) return DL_E_INVAL;
    const Fragment& F = r->frags[frag];
    if (F.closed) return DL_E_STATE;
    if (count < 1 || count > r->max_workers) return DL_E_INVAL;
    if (worker_ids == nullptr || ckpt_round_tags == nullptr || ckpts == nullptr)
        return DL_E_INVAL;
    if (r->mode == DL_DELTA_NESTEROV && tokens == nullptr) return DL_E_INVAL;
    std::vector<char> seen;
    try {
        seen.assign(static_cast<size_t>(r->max_workers), 0);
        a->w.reserve(static_cast<size_t>(count));
        a->spans.reserve(static_cast<size_t>(count));
    } catch (const std::bad_alloc&) {
        return DL_E_NOMEM;
    }
    for (int wk : F.arrivals) seen[static_cast<size_t>(wk)] = 1;
    const int64_t off = r->off(frag), n = r->len(frag);
    const Span acc_s = span_of(r->acc + off, n * 4);
    const Span th_s = global != nullptr ? span_of(global + off, n * 4) : Span{0, 0};
    for (int i = 0; i < count; ++i) {
        const int64_t t = r->mode == DL_DELTA_NESTEROV ? tokens[i] : 0;
        if (int st = check_arrival(r, frag, worker_ids[i], ckpt_round_tags[i], ckpts[i], dtype,
                                   global, t, &a->esize, a->tokens, &seen))
            return st;
        const Span ck_s = span_of(ckpts[i], n * a->esize);
        if (ck_s.overlaps(acc_s) || ck_s.overlaps(th_s)) return DL_E_INVAL;
        seen[static_cast<size_t>(worker_ids[i])] = 1;
        a->tokens += t;
        a->w.push_back(static_cast<float>(t));    // nearest-even
        a->spans.push_back(ck_s);
    }
    return DL_OK;
}

// The device-side checks of a validated call's buffers (after every host rule,
// as in the one-arrival calls).
int check_arrival_spans(const dl_round* r, int frag, const void* const* ckpts,
                        const float* global, const Arrivals& a) {
    const int64_t off = r->off(frag), n = r->len(frag);
    if (global != nullptr)
        if (int st = check_device_span(global + off, n * 4)) return st;
    if (int st = check_device_span(r->acc + off, n * 4)) return st;
    for (size_t i = 0; i < a.spans.size(); ++i)
        if (int st = check_device_span(ckpts[i], n * a.esize)) return st;
    return DL_OK;
}

// The buffers and parameters of a close taken in the same pass as the last
// arrivals (pointers already offset to the fragment).
struct CloseArgs {
    float* out = nullptr;                // mean: new global
    float* theta = nullptr;              // Nesterov: global, momentum
    float* m = nullptr;
    float* ema = nullptr;
    float lr = 0, mu = 0, beta = 0;
};

// Launches the folds of a validated call in passes of at most
// dlk::max_arrivals_per_pass() arrivals, in order; with `close` the last pass
// also closes the fragment.  Records the arrivals once every pass is launched.
int fold_passes(dl_round* r, int frag, int count, const int* worker_ids,
                const void* const* ckpts, int dtype, const float* global, const Arrivals& a,
                const CloseArgs* close) {
    Fragment& F = r->frags[frag];
    const int64_t off = r->off(frag), n = r->len(frag);
    float* acc = r->acc + off;
    const bool bf16 = dtype == DL_BF16;
    const int kmax = dlk::max_arrivals_per_pass();
    for (int i = 0; i < count; i += kmax) {
        const int k = std::min(kmax, count - i);
        const bool first = i == 0 && F.arrivals.empty();
        const bool backward = (F.passes & 1) != 0;
        const bool closing = close != nullptr && i + k == count;
        hipError_t err;
        if (r->mode == DL_MEAN) {
            if (closing) {
                const float cnt = static_cast<float>(F.arrivals.size() + count);
                err = dlk::launch_fold_many_finalize_mean(close->out, acc, ckpts + i, k, bf16,
                                                          first, cnt, close->ema, close->beta,
                                                          one_minus(close->beta), n, backward,
                                                          r->stream);
            } else {
                err = dlk::launch_fold_sum_many(acc, ckpts + i, k, bf16, n, first, backward,
                                                r->stream);
            }
        } else {
            const float* theta = global + off;
            if (closing) {
                const float total = static_cast<float>(F.tokens + a.tokens);   // exact sum, rounded once
                err = dlk::launch_fold_many_nesterov(close->theta, close->m, acc, ckpts + i,
                                                     a.w.data() + i, k, bf16, first, total,
                                                     close->lr, close->mu, close->ema,
                                                     close->beta, one_minus(close->beta), n,
                                                     backward, r->stream);
            } else {
                err = dlk::launch_fold_delta_many(acc, theta, ckpts + i, a.w.data() + i, k, bf16,
                                                  n, first, backward, r->stream);
            }
        }
        if (int st = after_launch(r, err)) return st;
        F.passes += 1;
    }
    F.arrivals.insert(F.arrivals.end(), worker_ids, worker_ids + count);   // reserved
    if (r->mode == DL_DELTA_NESTEROV) {
        F.tokens += a.tokens;
        F.global = global;
    }
    if (close != nullptr) F.closed = true;
    return DL_OK;
}

}  // namespace

extern "C" {

int dl_round_begin(dl_round** out, uint64_t round_tag, int mode, int64_t n_params, int n_frags,
                   const int64_t* frag_offsets, int quorum, int max_workers, float* acc,
                   void* stream) {
    if (out == nullptr) return DL_E_INVAL;
    *out = nullptr;
    if (mode != DL_MEAN && mode != DL_DELTA_NESTEROV) return DL_E_INVAL;
    if (n_params < 1 || n_frags < 1 || n_frags > kMaxFrags || frag_offsets == nullptr)
        return DL_E_INVAL;
    if (max_workers < 1 || max_workers > kMaxWorkers || quorum < 1 || quorum > max_workers)
        return DL_E_INVAL;
    if (acc == nullptr) return DL_E_INVAL;
    if (!aligned_to(acc, alignof(float))) return DL_E_ALIGN;
    if (frag_offsets[0] != 0 || frag_offsets[n_frags] != n_params) return DL_E_INVAL;
    for (int f = 0; f < n_frags; ++f)
        if (frag_offsets[f + 1] <= frag_offsets[f]) return DL_E_INVAL;
    if (n_params > INT64_MAX / static_cast<int64_t>(sizeof(float))) return DL_E_INVAL;

    dl_round* r = new (std::nothrow) dl_round;
    if (r == nullptr) return DL_E_NOMEM;
    try {
        r->offsets.assign(frag_offsets, frag_offsets + n_frags + 1);
        r->frags.resize(static_cast<size_t>(n_frags));
    } catch (const std::bad_alloc&) {
        delete r;
        return DL_E_NOMEM;
    }
    r->tag = round_tag;
    r->mode = mode;
    r->n_params = n_params;
    r->quorum = quorum;
    r->max_workers = max_workers;
    r->acc = acc;
    r->stream = static_cast<hipStream_t>(stream);
    *out = r;
    return DL_OK;
}

int dl_fold_checkpoint(dl_round* r, int frag, int worker_id, uint64_t ckpt_round_tag,
                       const void* ckpt, int dtype, const float* global, int64_t tokens) {
    if (r == nullptr) return DL_E_INVAL;
    int64_t esize = 0;
    if (int st = check_arrival(r, frag, worker_id, ckpt_round_tag, ckpt, dtype, global, tokens,
                               &esize))
        return st;
    Fragment& F = r->frags[frag];
    const int64_t off = r->off(frag), n = r->len(frag);
    float* acc = r->acc + off;
    const Span acc_s = span_of(acc, n * 4), ck_s = span_of(ckpt, n * esize);
    if (acc_s.overlaps(ck_s)) return DL_E_INVAL;
    const float* theta = nullptr;
    if (global != nullptr) {
        theta = global + off;
        const Span th_s = span_of(theta, n * 4);
        if (th_s.overlaps(acc_s) || th_s.overlaps(ck_s)) return DL_E_INVAL;
        if (int e = check_device_span(theta, n * 4)) return e;
    }
    if (int e = check_device_span(acc, n * 4)) return e;
    if (int e = check_device_span(ckpt, n * esize)) return e;

    if (int st = reserve_arrival(F)) return st;
    const bool first = F.arrivals.empty();
    const bool backward = (F.passes & 1) != 0;
    hipError_t err;
    if (r->mode == DL_MEAN) {
        err = dlk::launch_fold_sum(acc, ckpt, dtype == DL_BF16, n, first, backward, r->stream);
    } else {
        const float w = static_cast<float>(tokens);   // nearest-even
        err = dlk::launch_fold_delta(acc, theta, ckpt, dtype == DL_BF16, w, n, first, backward,
                                     r->stream);
    }
    if (int st = after_launch(r, err)) return st;
    F.arrivals.push_back(worker_id);
    F.passes += 1;
    if (r->mode == DL_DELTA_NESTEROV) {
        F.tokens += tokens;
        F.global = global;
    }
    return DL_OK;
}

int dl_finalize_mean(dl_round* r, int frag, float* out_global, float* ema, float beta) {
    if (r == nullptr) return DL_E_INVAL;
    if (r->failed || r->mode != DL_MEAN) return DL_E_STATE;
    if (frag < 0 || frag >= r->n_frags()) return DL_E_INVAL;
    Fragment& F = r->frags[frag];
    if (F.closed) return DL_E_STATE;
    if (static_cast<int>(F.arrivals.size()) < r->quorum) return DL_E_QUORUM;
    float *out = nullptr, *e = nullptr;
    if (int st = check_mean_close(r, frag, out_global, ema, nullptr, 0, &out, &e)) return st;

    const float count = static_cast<float>(F.arrivals.size());
    const hipError_t err =
        dlk::launch_finalize_mean(out, r->acc + r->off(frag), count, e, beta, one_minus(beta),
                                  r->len(frag), (F.passes & 1) != 0, r->stream);
    if (int st = after_launch(r, err)) return st;
    F.passes += 1;
    F.closed = true;
    return DL_OK;
}

int dl_outer_nesterov(dl_round* r, int frag, float* global, float* momentum, float lr, float mu,
                      float* ema, float beta) {
    if (r == nullptr) return DL_E_INVAL;
    if (r->failed || r->mode != DL_DELTA_NESTEROV) return DL_E_STATE;
    if (frag < 0 || frag >= r->n_frags()) return DL_E_INVAL;
    Fragment& F = r->frags[frag];
    if (F.closed) return DL_E_STATE;
    if (static_cast<int>(F.arrivals.size()) < r->quorum) return DL_E_QUORUM;
    if (global == nullptr || global != F.global) return DL_E_INVAL;
    float *theta = nullptr, *m = nullptr, *e = nullptr;
    if (int st = check_nesterov_close(r, frag, global, momentum, ema, nullptr, 0, &theta, &m, &e))
        return st;

    const float total = static_cast<float>(F.tokens);    // exact int64 sum, rounded once
    const hipError_t err = dlk::launch_nesterov(theta, m, r->acc + r->off(frag), total, lr, mu,
                                                e, beta, one_minus(beta), r->len(frag),
                                                (F.passes & 1) != 0, r->stream);
    if (int st = after_launch(r, err)) return st;
    F.passes += 1;
    F.closed = true;
    return DL_OK;
}

int dl_fold_and_finalize_mean(dl_round* r, int frag, int worker_id, uint64_t ckpt_round_tag,
                              const void* ckpt, int dtype, float* out_global, float* ema,
                              float beta) {
    if (r == nullptr) return DL_E_INVAL;
    if (r->mode != DL_MEAN) return DL_E_STATE;
    int64_t esize = 0;
    if (int st = check_arrival(r, frag, worker_id, ckpt_round_tag, ckpt, dtype, nullptr, 0,
                               &esize))
        return st;
    Fragment& F = r->frags[frag];
    if (static_cast<int>(F.arrivals.size()) + 1 < r->quorum) return DL_E_QUORUM;
    const int64_t off = r->off(frag), n = r->len(frag);
    const Span ck_s = span_of(ckpt, n * esize);
    if (span_of(r->acc + off, n * 4).overlaps(ck_s)) return DL_E_INVAL;
    float *out = nullptr, *e = nullptr;
    if (int st = check_mean_close(r, frag, out_global, ema, &ck_s, 1, &out, &e)) return st;
    if (int st = check_device_span(ckpt, n * esize)) return st;
    if (int st = reserve_arrival(F)) return st;

    const bool first = F.arrivals.empty();
    const float count = static_cast<float>(F.arrivals.size() + 1);
    const hipError_t err = dlk::launch_fold_finalize_mean(
        out, r->acc + off, ckpt, dtype == DL_BF16, first, count, e, beta, one_minus(beta), n,
        (F.passes & 1) != 0, r->stream);
    if (int st = after_launch(r, err)) return st;
    F.arrivals.push_back(worker_id);
    F.passes += 1;
    F.closed = true;
    return DL_OK;
}

int dl_fold_and_outer_nesterov(dl_round* r, int frag, int worker_id, uint64_t ckpt_round_tag,
                               const void* ckpt, int dtype, int64_t tokens, float* global,
                               float* momentum, float lr, float mu, float* ema, float beta) {
    if (r == nullptr) return DL_E_INVAL;
    if (r->mode != DL_DELTA_NESTEROV) return DL_E_STATE;
    int64_t esize = 0;
    if (int st = check_arrival(r, frag, worker_id, ckpt_round_tag, ckpt, dtype, global, tokens,
                               &esize))
        return st;
    Fragment& F = r->frags[frag];
    if (static_cast<int>(F.arrivals.size()) + 1 < r->quorum) return DL_E_QUORUM;
    const int64_t off = r->off(frag), n = r->len(frag);
    const Span ck_s = span_of(ckpt, n * esize);
    if (span_of(r->acc + off, n * 4).overlaps(ck_s)) return DL_E_INVAL;
    float *theta = nullptr, *m = nullptr, *e = nullptr;
    if (int st = check_nesterov_close(r, frag, global, momentum, ema, &ck_s, 1, &theta, &m, &e))
        return st;
    if (int st = check_device_span(ckpt, n * esize)) return st;
    if (int st = reserve_arrival(F)) return st;

    const bool first = F.arrivals.empty();
    const float w = static_cast<float>(tokens);               // nearest-even
    const float total = static_cast<float>(F.tokens + tokens);  // exact int64 sum, rounded once
    const hipError_t err = dlk::launch_fold_nesterov(
        theta, m, r->acc + off, ckpt, dtype == DL_BF16, first, w, total, lr, mu, e, beta,
        one_minus(beta), n, (F.passes & 1) != 0, r->stream);
    if (int st = after_launch(r, err)) return st;
    F.arrivals.push_back(worker_id);
    F.tokens += tokens;
    F.global = global;
    F.passes += 1;
    F.closed = true;
    return DL_OK;
}

int dl_fold_checkpoints(dl_round* r, int frag, int count, const int* worker_ids,
                        const uint64_t* ckpt_round_tags, const void* const* ckpts, int dtype,
                        const float* global, const int64_t* tokens) {
    if (r == nullptr) return DL_E_INVAL;
    Arrivals a;
    if (int st = check_arrivals(r, frag, count, worker_ids, ckpt_round_tags, ckpts, dtype, global,
                                tokens, &a))
        return st;
    if (int st = check_arrival_spans(r, frag, ckpts, global, a)) return st;
    if (int st = reserve_arrival(r->frags[frag], count)) return st;
    return fold_passes(r, frag, count, worker_ids, ckpts, dtype, global, a, nullptr);
}

int dl_fold_checkpoints_and_finalize_mean(dl_round* r, int frag, int count,
                                          const int* worker_ids, const uint64_t* ckpt_round_tags,
                                          const void* const* ckpts, int dtype, float* out_global,
                                          float* ema, float beta) {
    if (r == nullptr) return DL_E_INVAL;
    if (r->mode != DL_MEAN) return DL_E_STATE;
    Arrivals a;
    if (int st = check_arrivals(r, frag, count, worker_ids, ckpt_round_tags, ckpts, dtype,
                                nullptr, nullptr, &a))
        return st;
    Fragment& F = r->frags[frag];
    if (static_cast<int64_t>(F.arrivals.size()) + count < r->quorum) return DL_E_QUORUM;
    CloseArgs c;
    if (int st = check_mean_close(r, frag, out_global, ema, a.spans.data(), a.spans.size(),
                                  &c.out, &c.ema))
        return st;
    if (int st = check_arrival_spans(r, frag, ckpts, nullptr, a)) return st;
    if (int st = reserve_arrival(F, count)) return st;
    c.beta = beta;
    return fold_passes(r, frag, count, worker_ids, ckpts, dtype, nullptr, a, &c);
}

int dl_fold_checkpoints_and_outer_nesterov(dl_round* r, int frag, int count,
                                           const int* worker_ids,
                                           const uint64_t* ckpt_round_tags,
                                           const void* const* ckpts, int dtype,
                                           const int64_t* tokens, float* global, float* momentum,
                                           float lr, float mu, float* ema, float beta) {
    if (r == nullptr) return DL_E_INVAL;
    if (r->mode != DL_DELTA_NESTEROV) return DL_E_STATE;
    Arrivals a;
    if (int st = check_arrivals(r, frag, count, worker_ids, ckpt_round_tags, ckpts, dtype, global,
                                tokens, &a))
        return st;
    Fragment& F = r->frags[frag];
    if (static_cast<int64_t>(F.arrivals.size()) + count < r->quorum) return DL_E_QUORUM;
    CloseArgs c;
    if (int st = check_nesterov_close(r, frag, global, momentum, ema, a.spans.data(),
                                      a.spans.size(), &c.theta, &c.m, &c.ema))
        return st;
    if (int st = check_arrival_spans(r, frag, ckpts, global, a)) return st;
    if (int st = reserve_arrival(F, count)) return st;
    c.lr = lr;
    c.mu = mu;
    c.beta = beta;
    return fold_passes(r, frag, count, worker_ids, ckpts, dtype, global, a, &c);
}

int dl_ema_update(float* ema, const float* global, int64_t n, float beta, void* stream) {
    if (n < 0) return DL_E_INVAL;
    if (n == 0) return DL_OK;
    if (ema == nullptr || global == nullptr) return DL_E_INVAL;
    if (n > INT64_MAX / 4) return DL_E_INVAL;
    if (!aligned_to(ema, alignof(float)) || !aligned_to(global, alignof(float))) return DL_E_ALIGN;
    if (span_of(ema, n * 4).overlaps(span_of(global, n * 4))) return DL_E_INVAL;
    if (int st = check_device_span(ema, n * 4)) return st;
    if (int st = check_device_span(global, n * 4)) return st;
    const hipError_t err = dlk::launch_ema(ema, global, beta, one_minus(beta), n,
                                           static_cast<hipStream_t>(stream));
    return err == hipSuccess ? DL_OK : DL_E_HIP;
}

int dl_swa_fold(float* sum, const float* global, int64_t n, int64_t folded_before,
                void* stream) {
    if (n < 0 || folded_before < 0) return DL_E_INVAL;
    if (n == 0) return DL_OK;
    if (sum == nullptr || global == nullptr || n > INT64_MAX / 4) return DL_E_INVAL;
    if (!aligned_to(sum, alignof(float)) || !aligned_to(global, alignof(float))) return DL_E_ALIGN;
    if (span_of(sum, n * 4).overlaps(span_of(global, n * 4))) return DL_E_INVAL;
    if (int st = check_device_span(sum, n * 4)) return st;
    if (int st = check_device_span(global, n * 4)) return st;
    const hipError_t err = dlk::launch_fold_sum(sum, global, false, n, folded_before == 0, false,
                                                static_cast<hipStream_t>(stream));
    return err == hipSuccess ? DL_OK : DL_E_HIP;
}

int dl_swa_average(float* out, const float* sum, int64_t n, int64_t count, void* stream) {
    if (n < 0 || count < 1) return DL_E_INVAL;
    if (n == 0) return DL_OK;
    if (out == nullptr || sum == nullptr || n > INT64_MAX / 4) return DL_E_INVAL;
    if (!aligned_to(out, alignof(float)) || !aligned_to(sum, alignof(float))) return DL_E_ALIGN;
    const Span out_s = span_of(out, n * 4), sum_s = span_of(sum, n * 4);
    if (!out_s.same(sum_s) && out_s.overlaps(sum_s)) return DL_E_INVAL;
    if (int st = check_device_span(out, n * 4)) return st;
    if (int st = check_device_span(sum, n * 4)) return st;
    const hipError_t err = dlk::launch_finalize_mean(out, sum, static_cast<float>(count), nullptr,
                                                     0.0f, 0.0f, n, false,
                                                     static_cast<hipStream_t>(stream));
    return err == hipSuccess ? DL_OK : DL_E_HIP;
}

int dl_snapshot_average(float* out, const float* const* snapshots, int k, int64_t n,
                        void* stream) {
    if (n < 0 || k < 1 || k > DL_MAX_SNAPSHOTS || snapshots == nullptr) return DL_E_INVAL;
    if (n == 0) return DL_OK;
    if (out == nullptr || n > INT64_MAX / 4) return DL_E_INVAL;
    if (!aligned_to(out, alignof(float))) return DL_E_ALIGN;
    const Span out_s = span_of(out, n * 4);
    for (int i = 0; i < k; ++i) {
        if (snapshots[i] == nullptr) return DL_E_INVAL;
        if (!aligned_to(snapshots[i], alignof(float))) return DL_E_ALIGN;
        if (span_of(snapshots[i], n * 4).overlaps(out_s)) return DL_E_INVAL;
    }
    if (int st = check_device_span(out, n * 4)) return st;
    for (int i = 0; i < k; ++i)
        if (int st = check_device_span(snapshots[i], n * 4)) return st;
    const hipError_t err =
        dlk::launch_snapshot_mean(out, snapshots, k, n, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? DL_OK : DL_E_HIP;
}

int dl_adopt_keep_drift(float* theta, const float* global, const void* pushed, int pushed_dtype,
                        int64_t n, void* stream) {
    if (n < 0) return DL_E_INVAL;
    if (pushed_dtype != DL_F32 && pushed_dtype != DL_BF16) return DL_E_INVAL;
    if (n == 0) return DL_OK;
    if (theta == nullptr || global == nullptr || pushed == nullptr || n > INT64_MAX / 4)
        return DL_E_INVAL;
    const int64_t esize = pushed_dtype == DL_BF16 ? 2 : 4;
    if (!aligned_to(theta, alignof(float)) || !aligned_to(global, alignof(float)) ||
        !aligned_to(pushed, static_cast<uintptr_t>(esize)))
        return DL_E_ALIGN;
    const Span t_s = span_of(theta, n * 4), g_s = span_of(global, n * 4),
               p_s = span_of(pushed, n * esize);
    if (t_s.overlaps(g_s) || t_s.overlaps(p_s)) return DL_E_INVAL;
    if (int st = check_device_span(theta, n * 4)) return st;
    if (int st = check_device_span(global, n * 4)) return st;
    if (int st = check_device_span(pushed, n * esize)) return st;
    const hipError_t err = dlk::launch_adopt_keep_drift(theta, global, pushed,
                                                        pushed_dtype == DL_BF16, n,
                                                        static_cast<hipStream_t>(stream));
    return err == hipSuccess ? DL_OK : DL_E_HIP;
}

int dl_matmul_workspace_bytes_batch(int64_t m, int64_t n, int64_t k, int symmetric, int batch,
                                    int64_t* bytes) {
    if (bytes == nullptr || m < 0 || n < 0 || k < 0) return DL_E_INVAL;
    if (symmetric != 0 && symmetric != 1) return DL_E_INVAL;
    if (symmetric && m != n) return DL_E_INVAL;
    if (batch < 1 || batch > DL_MAX_BATCH) return DL_E_INVAL;
    if (m > (int64_t(1) << 31) || n > (int64_t(1) << 31) ||
        dlk::gemm_tiles(m, n) * batch > dlk::kGemmMaxTiles)
        return DL_E_INVAL;
    *bytes = (m == 0 || n == 0) ? 0
                                : dlk::matmul_workspace_bytes(m, n, k, symmetric != 0, batch);
    return DL_OK;
}

int dl_matmul_workspace_bytes(int64_t m, int64_t n, int64_t k, int symmetric, int64_t* bytes) {
    return dl_matmul_workspace_bytes_batch(m, n, k, symmetric, 1, bytes);
}

int dl_matmul_large_tiles(int64_t m, int64_t n, int64_t k, int symmetric, int batch,
                          int64_t workspace_bytes, int* large) {
    int64_t unused = 0;
    if (large == nullptr || workspace_bytes < 0) return DL_E_INVAL;
    if (const int rc = dl_matmul_workspace_bytes_batch(m, n, k, symmetric, batch, &unused))
        return rc;
    *large = (m > 0 && n > 0 &&
              dlk::matmul_large_tiles(m, n, k, symmetric != 0, batch, workspace_bytes))
                 ? 1
                 : 0;
    return DL_OK;
}

int dl_matmul_f32_batch(int form, const float* a, int64_t lda, int64_t stride_a, const float* b,
                        int64_t ldb, int64_t stride_b, int64_t m, int64_t n, int64_t k, float* c,
                        int64_t ldc, int64_t stride_c, const float* y, int64_t stride_y,
                        float alpha, float beta, float diag, int symmetric, int batch,
                        void* workspace, int64_t workspace_bytes, void* stream) {
    if (form != DL_TN && form != DL_NT) return DL_E_INVAL;
    if (m < 0 || n < 0 || k < 0 || workspace_bytes < 0) return DL_E_INVAL;
    if (symmetric != 0 && symmetric != 1) return DL_E_INVAL;
    if (symmetric && m != n) return DL_E_INVAL;
    if (batch < 1 || batch > DL_MAX_BATCH) return DL_E_INVAL;
    if (m == 0 || n == 0) return DL_OK;
    if (a == nullptr || b == nullptr || c == nullptr) return DL_E_INVAL;
    if (m > (int64_t(1) << 31) || n > (int64_t(1) << 31) ||
        dlk::gemm_tiles(m, n) * batch > dlk::kGemmMaxTiles)
        return DL_E_INVAL;
    const bool tn = form == DL_TN;
    // the operands' extents: TN reads A as k x lda (cols i < m), NT as m x lda (cols k)
    if (tn ? (lda < m || ldb < n) : (lda < k || ldb < k)) return DL_E_INVAL;
    if (ldc < n) return DL_E_INVAL;
    if (!aligned_to(a, alignof(float)) || !aligned_to(b, alignof(float)) ||
        !aligned_to(c, alignof(float)) || (y && !aligned_to(y, alignof(float))))
        return DL_E_ALIGN;
    if (workspace != nullptr && !aligned_to(workspace, 256)) return DL_E_ALIGN;
    const int64_t ws_bytes = workspace ? workspace_bytes : 0;
    const int64_t a_one = 4 * (tn ? (k > 0 ? (k - 1) * lda + m : 0) : (m - 1) * lda + k);
    const int64_t b_one = 4 * (tn ? (k > 0 ? (k - 1) * ldb + n : 0) : (n - 1) * ldb + k);
    const int64_t c_one = 4 * ((m - 1) * ldc + n);
    // results must not overlap each other: C strides at least one matrix
    if (batch > 1 && (stride_c < 0 || 4 * stride_c < c_one)) return DL_E_INVAL;
    if (stride_a < 0 || stride_b < 0 || stride_y < 0) return DL_E_INVAL;
    const int64_t bm = batch - 1;
    const int64_t a_bytes = a_one + 4 * bm * stride_a, b_bytes = b_one + 4 * bm * stride_b;
    const int64_t c_bytes = c_one + 4 * bm * stride_c, y_bytes = c_one + 4 * bm * stride_y;
    const Span c_s = span_of(c, c_bytes);
    if (k > 0 && (c_s.overlaps(span_of(a, a_bytes)) || c_s.overlaps(span_of(b, b_bytes))))
        return DL_E_INVAL;
    if (y != nullptr && !(y == c && stride_y == stride_c) && c_s.overlaps(span_of(y, y_bytes)))
        return DL_E_INVAL;
    if (ws_bytes > 0) {
        const Span w_s = span_of(workspace, ws_bytes);
        if (w_s.overlaps(c_s) || (y && w_s.overlaps(span_of(y, y_bytes))) ||
            (k > 0 && (w_s.overlaps(span_of(a, a_bytes)) || w_s.overlaps(span_of(b, b_bytes)))))
            return DL_E_INVAL;
    }
    if (k > 0) {
        if (int st = check_device_span(a, a_bytes)) return st;
        if (int st = check_device_span(b, b_bytes)) return st;
    }
    if (int st = check_device_span(c, c_bytes)) return st;
    if (y != nullptr)
        if (int st = check_device_span(y, y_bytes)) return st;
    if (ws_bytes > 0)
        if (int st = check_device_span(workspace, ws_bytes)) return st;
    const hipError_t err = dlk::matmul(tn, a, lda, stride_a, b, ldb, stride_b, m, n, k, c, ldc,
                                       stride_c, y, stride_y, alpha, beta, diag, symmetric != 0,
                                       batch, workspace, ws_bytes,
                                       static_cast<hipStream_t>(stream));
    return err == hipSuccess ? DL_OK : DL_E_HIP;
}

int dl_matmul_f32(int form, const float* a, int64_t lda, const float* b, int64_t ldb, int64_t m,
                  int64_t n, int64_t k, float* c, int64_t ldc, const float* y, float alpha,
                  float beta, float diag, int symmetric, void* workspace, int64_t workspace_bytes,
                  void* stream) {
    return dl_matmul_f32_batch(form, a, lda, 0, b, ldb, 0, m, n, k, c, ldc, 0, y, 0, alpha, beta,
                               diag, symmetric, 1, workspace, workspace_bytes, stream);
}

int dl_polar_workspace_bytes_batch(int64_t rows, int64_t cols, int batch, int64_t* bytes) {
    if (bytes == nullptr || rows < 1 || cols < 1 || batch < 1 || batch > DL_MAX_BATCH)
        return DL_E_INVAL;
    if (rows > (int64_t(1) << 31) || cols > (int64_t(1) << 31) ||
        dlk::gemm_tiles(rows, cols) * batch > dlk::kGemmMaxTiles)
        return DL_E_INVAL;
    *bytes = dlk::polar_workspace_bytes(rows, cols, batch);
    return DL_OK;
}

int dl_polar_workspace_bytes(int64_t rows, int64_t cols, int64_t* bytes) {
    return dl_polar_workspace_bytes_batch(rows, cols, 1, bytes);
}

namespace {

int check_polar_args(int64_t rows, int64_t cols, int batch, int quintic, int cubic, void* ws,
                     int64_t ws_bytes, int64_t* need) {
    if (int st = dl_polar_workspace_bytes_batch(rows, cols, batch, need)) return st;
    if (quintic < 0 || cubic < 0 || quintic + cubic < 1 || quintic > 64 || cubic > 64)
        return DL_E_INVAL;
    if (ws == nullptr || ws_bytes < *need) return DL_E_INVAL;
    if (!aligned_to(ws, 256)) return DL_E_ALIGN;
    return DL_OK;
}

}  // namespace

int dl_polar_factor(float* out, const float* update, int64_t rows, int64_t cols, int quintic_steps,
                    int cubic_steps, void* workspace, int64_t workspace_bytes, void* stream) {
    int64_t need = 0;
    if (int st = check_polar_args(rows, cols, 1, quintic_steps, cubic_steps, workspace,
                                  workspace_bytes, &need))
        return st;
    if (out == nullptr || update == nullptr) return DL_E_INVAL;
    if (!aligned_to(out, alignof(float)) || !aligned_to(update, alignof(float))) return DL_E_ALIGN;
    const int64_t bytes = rows * cols * 4;
    const Span o_s = span_of(out, bytes), u_s = span_of(update, bytes), w_s = span_of(workspace, need);
    if (o_s.overlaps(w_s) || u_s.overlaps(w_s)) return DL_E_INVAL;
    if (!o_s.same(u_s) && o_s.overlaps(u_s)) return DL_E_INVAL;
    if (int st = check_device_span(workspace, need)) return st;
    if (int st = check_device_span(out, bytes)) return st;
    if (int st = check_device_span(update, bytes)) return st;
    const hipError_t err = dlk::polar_iterate(&update, nullptr, &out, nullptr, 0.0f, 1, rows, cols,
                                              quintic_steps, cubic_steps, workspace,
                                              static_cast<hipStream_t>(stream));
    return err == hipSuccess ? DL_OK : DL_E_HIP;
}

int dl_outer_orthogonal_step_batch(float* const* theta, const float* const* averaged, int batch,
                                   int64_t rows, int64_t cols, float scale, int quintic_steps,
                                   int cubic_steps, void* workspace, int64_t workspace_bytes,
                                   void* stream) {
    int64_t need = 0;
    if (int st = check_polar_args(rows, cols, batch, quintic_steps, cubic_steps, workspace,
                                  workspace_bytes, &need))
        return st;
    if (theta == nullptr || averaged == nullptr) return DL_E_INVAL;
    const int64_t bytes = rows * cols * 4;
    const Span w_s = span_of(workspace, need);
    for (int b = 0; b < batch; ++b) {
        if (theta[b] == nullptr || averaged[b] == nullptr) return DL_E_INVAL;
        if (!aligned_to(theta[b], alignof(float)) || !aligned_to(averaged[b], alignof(float)))
            return DL_E_ALIGN;
        const Span t_s = span_of(theta[b], bytes), a_s = span_of(averaged[b], bytes);
        if (t_s.overlaps(a_s) || t_s.overlaps(w_s) || a_s.overlaps(w_s)) return DL_E_INVAL;
        // the matrices are written: no theta may meet another matrix's theta or averaged
        for (int c = 0; c < b; ++c)
            if (t_s.overlaps(span_of(theta[c], bytes)) || t_s.overlaps(span_of(averaged[c], bytes)) ||
                a_s.overlaps(span_of(theta[c], bytes)))
                return DL_E_INVAL;
    }
    if (int st = check_device_span(workspace, need)) return st;
    for (int b = 0; b < batch; ++b) {
        if (int st = check_device_span(theta[b], bytes)) return st;
        if (int st = check_device_span(averaged[b], bytes)) return st;
    }
    const hipError_t err = dlk::polar_iterate(theta, averaged, nullptr, theta, scale, batch, rows,
                                              cols, quintic_steps, cubic_steps, workspace,
                                              static_cast<hipStream_t>(stream));
    return err == hipSuccess ? DL_OK : DL_E_HIP;
}

int dl_outer_orthogonal_step(float* theta, const float* averaged, int64_t rows, int64_t cols,
                             float scale, int quintic_steps, int cubic_steps, void* workspace,
                             int64_t workspace_bytes, void* stream) {
    return dl_outer_orthogonal_step_batch(&theta, &averaged, 1, rows, cols, scale, quintic_steps,
                                          cubic_steps, workspace, workspace_bytes, stream);
}

int dl_outer_orthogonal_step_noalloc(float* theta, const float* averaged, int64_t rows,
                                     int64_t cols, float scale, int quintic_steps,
                                     int cubic_steps, void* stream) {
    int64_t need = 0;
    if (int st = dl_polar_workspace_bytes_batch(rows, cols, 1, &need)) return st;
    if (quintic_steps < 0 || cubic_steps < 0 || quintic_steps + cubic_steps < 1 ||
        quintic_steps > 64 || cubic_steps > 64)
        return DL_E_INVAL;
    if (need > dlk::kNoallocScratchBytes) return DL_E_TOO_LARGE;
    if (theta == nullptr || averaged == nullptr) return DL_E_INVAL;
    if (!aligned_to(theta, alignof(float)) || !aligned_to(averaged, alignof(float)))
        return DL_E_ALIGN;
    const int64_t bytes = rows * cols * 4;
    if (span_of(theta, bytes).overlaps(span_of(averaged, bytes))) return DL_E_INVAL;
    if (int st = check_device_span(theta, bytes)) return st;
    if (int st = check_device_span(averaged, bytes)) return st;
    // the scratch is looked up on the calling thread's current device, which
    // must be the stream's
    const hipStream_t s = static_cast<hipStream_t>(stream);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return DL_E_HIP;
    if (s != nullptr) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(s, &sdev) != hipSuccess) return DL_E_HIP;
        if (sdev != dev) return DL_E_INVAL;
    }
    void* ws = nullptr;
    if (dlk::noalloc_scratch(dev, &ws) != hipSuccess) return DL_E_HIP;
    const hipError_t err = dlk::polar_iterate(&theta, &averaged, nullptr, &theta, scale, 1, rows,
                                              cols, quintic_steps, cubic_steps, ws, s);
    return err == hipSuccess ? DL_OK : DL_E_HIP;
}

int dl_frag_range(const dl_round* r, int frag, int64_t* offset, int64_t* length) {
    if (r == nullptr || offset == nullptr || length == nullptr) return DL_E_INVAL;
    if (frag < 0 || frag >= r->n_frags()) return DL_E_INVAL;
    *offset = r->off(frag);
    *length = r->len(frag);
    return DL_OK;
}

int dl_round_participants(const dl_round* r, int frag, int* count, int* workers, int capacity) {
    if (r == nullptr || count == nullptr) return DL_E_INVAL;
    if (frag < 0 || frag >= r->n_frags()) return DL_E_INVAL;
    const std::vector<int>& a = r->frags[frag].arrivals;
    *count = static_cast<int>(a.size());
    if (workers == nullptr) return DL_OK;
    if (capacity < *count) return DL_E_CAPACITY;
    std::copy(a.begin(), a.end(), workers);
    return DL_OK;
}

int dl_round_tokens(const dl_round* r, int frag, int64_t* total_tokens) {
    if (r == nullptr || total_tokens == nullptr) return DL_E_INVAL;
    if (frag < 0 || frag >= r->n_frags()) return DL_E_INVAL;
    *total_tokens = r->frags[frag].tokens;
    return DL_OK;
}

int dl_round_end(dl_round* r) {
    delete r;
    return DL_OK;
}

const char* dl_strerror(int status) {
    switch (status) {
        case DL_OK: return "ok";
        case DL_E_INVAL: return "invalid argument";
        case DL_E_STALE: return "checkpoint carries another round's tag";
        case DL_E_DUP: return "worker already folded into this fragment";
        case DL_E_QUORUM: return "fewer arrivals than the quorum";
        case DL_E_STATE: return "call not allowed in this state";
        case DL_E_ALIGN: return "pointer not aligned to its element type";
        case DL_E_HIP: return "HIP error (pending before the call, or at launch)";
        case DL_E_CAPACITY: return "output array too small";
        case DL_E_NOMEM: return "host memory exhausted";
        case DL_E_TOO_LARGE:
            return "matrix needs more workspace than the allocation-free entry point's scratch";
        default: return "unknown status";
    }
}

}  // extern "C"

// Internal launch interface of the merge kernels (not part of the C ABI).
// Each function launches exactly one kernel on stream s over n elements and
// returns the launch status (hipGetLastError after the launch); n <= 0
// launches nothing.  Pointers are device pointers already offset to the
// fragment; the caller has validated them.  `backward` walks the tiles from
// last to first (no effect on results: elements are independent).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dlk {

// acc[j] = c[j] (first) or acc[j] + c[j]; c is fp32, or bf16 if bf16 is set.
hipError_t launch_fold_sum(float* acc, const void* ckpt, bool bf16, int64_t n, bool first,
                           bool backward, hipStream_t s);

// acc[j] = w*(theta[j] - c[j]) (first) or acc[j] + w*(theta[j] - c[j]).
hipError_t launch_fold_delta(float* acc, const float* theta, const void* ckpt, bool bf16,
                             float w, int64_t n, bool first, bool backward, hipStream_t s);

// out[j] = sum[j] / count; if ema: ema[j] = beta*ema[j] + omega*out[j].
// out may equal sum.
hipError_t launch_finalize_mean(float* out, const float* sum, float count, float* ema,
                                float beta, float omega, int64_t n, bool backward,
                                hipStream_t s);

// dbar = acc/total; m = mu*m + dbar; theta -= lr*(dbar + mu*m);
// if ema: ema = beta*ema + omega*theta.
hipError_t launch_nesterov(float* theta, float* m, const float* acc, float total, float lr,
                           float mu, float* ema, float beta, float omega, int64_t n,
                           bool backward, hipStream_t s);

// launch_fold_sum followed by launch_finalize_mean in one pass; the completed
// sum is not written back.  out may equal sum.  `first`: this is the only
// arrival (sum is not read).
hipError_t launch_fold_finalize_mean(float* out, const float* sum, const void* ckpt, bool bf16,
                                     bool first, float count, float* ema, float beta,
                                     float omega, int64_t n, bool backward, hipStream_t s);

// launch_fold_delta followed by launch_nesterov in one pass; the completed
// accumulator is not written back.
hipError_t launch_fold_nesterov(float* theta, float* m, const float* acc, const void* ckpt,
                                bool bf16, bool first, float w, float total, float lr, float mu,
                                float* ema, float beta, float omega, int64_t n, bool backward,
                                hipStream_t s);

// The passes above for k arrivals at once, 1 <= k <= max_arrivals_per_pass():
// ckpts[0..k) are the arrivals in arrival order (all fp32, or all bf16), w[i]
// the token weight of arrival i.  Each gives the bits of k one-arrival passes
// in that order (the closing ones: k - 1 folds, then the fold and close),
// with the accumulator read and written once.  `first`: acc holds no earlier
// arrival of the fragment (it is not read).  k out of range:
// hipErrorInvalidValue, nothing launched.
int max_arrivals_per_pass();
hipError_t launch_fold_sum_many(float* acc, const void* const* ckpts, int k, bool bf16,
                                int64_t n, bool first, bool backward, hipStream_t s);
hipError_t launch_fold_delta_many(float* acc, const float* theta, const void* const* ckpts,
                                  const float* w, int k, bool bf16, int64_t n, bool first,
                                  bool backward, hipStream_t s);
hipError_t launch_fold_many_finalize_mean(float* out, const float* sum, const void* const* ckpts,
                                          int k, bool bf16, bool first, float count, float* ema,
                                          float beta, float omega, int64_t n, bool backward,
                                          hipStream_t s);
hipError_t launch_fold_many_nesterov(float* theta, float* m, const float* acc,
                                     const void* const* ckpts, const float* w, int k, bool bf16,
                                     bool first, float total, float lr, float mu, float* ema,
                                     float beta, float omega, int64_t n, bool backward,
                                     hipStream_t s);

// out[j] = (((s_0[j] + s_1[j]) + ...) + s_{k-1}[j]) / k, 1 <= k <= 16, in one pass.
// out must not overlap any snapshot.
hipError_t launch_snapshot_mean(float* out, const float* const* snaps, int k, int64_t n,
                               hipStream_t s);

// theta[j] = theta[j] + (g[j] - pushed[j]); pushed is fp32, or bf16 if bf16 is set.
hipError_t launch_adopt_keep_drift(float* theta, const float* g, const void* pushed, bool bf16,
                                   int64_t n, hipStream_t s);

// ema[j] = beta*ema[j] + omega*g[j].
hipError_t launch_ema(float* ema, const float* g, float beta, float omega, int64_t n,
                      hipStream_t s);

}  // namespace dlk

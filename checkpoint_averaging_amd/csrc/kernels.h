// Internal launch interface of the merge kernels (not part of the C ABI).
// Each function launches exactly one kernel on stream s over n elements and
// returns the launch status (hipGetLastError after the launch); n <= 0
// launches nothing.  Pointers are device pointers already offset to the
// fragment; the caller has validated them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dlk {

// acc[j] = c[j] (first) or acc[j] + c[j]; c is fp32, or bf16 if bf16 is set.
hipError_t launch_fold_sum(float* acc, const void* ckpt, bool bf16, int64_t n, bool first,
                           hipStream_t s);

// acc[j] = w*(theta[j] - c[j]) (first) or acc[j] + w*(theta[j] - c[j]).
hipError_t launch_fold_delta(float* acc, const float* theta, const void* ckpt, bool bf16,
                             float w, int64_t n, bool first, hipStream_t s);

// out[j] = sum[j] / count; if ema: ema[j] = beta*ema[j] + omega*out[j].
// out may equal sum.
hipError_t launch_finalize_mean(float* out, const float* sum, float count, float* ema,
                                float beta, float omega, int64_t n, hipStream_t s);

// dbar = acc/total; m = mu*m + dbar; theta -= lr*(dbar + mu*m);
// if ema: ema = beta*ema + omega*theta.
hipError_t launch_nesterov(float* theta, float* m, const float* acc, float total, float lr,
                           float mu, float* ema, float beta, float omega, int64_t n,
                           hipStream_t s);

// ema[j] = beta*ema[j] + omega*g[j].
hipError_t launch_ema(float* ema, const float* g, float beta, float omega, int64_t n,
                      hipStream_t s);

}  // namespace dlk

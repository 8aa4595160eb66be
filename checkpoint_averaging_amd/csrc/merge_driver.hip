// dlmerge_driver: runs merge rounds through the C ABI (include/dlmerge.h) on
// buffers it allocates with hipMalloc, with no other GPU work besides a fill
// pass and an optional plain copy kernel of known size.  It is a minimal C
// consumer of the library and the program hardware counters are collected
// on (a copy of known size calibrates the byte counters).
//
//   dlmerge_driver --n N [--offsets 0,o1,...,N] [--mode mean|delta]
//                  [--workers W] [--dtype f32|bf16] [--ema 0|1]
//                  [--rounds R] [--warmup R0] [--copy-mib M] [--fused 0|1]
//                  [--streams S] [--side 1] [--inplace 0|1] [--host-timing 1]
//                  [--batched 0|1|2]
//
// Round structure matches the benchmark: for each fragment, every worker is
// folded (token-weighted delta in delta mode) and the fragment is closed
// (mean, or outer Nesterov lr 0.7 / momentum 0.9), with the EMA (beta 0.9)
// fused in when enabled.  With --fused 1 (default) the last worker is folded
// in the same pass as the close.  With --inplace 1 (default) a mean round
// writes the new global over the running sum and the two buffers swap roles
// for the next round, as the benchmark does; --inplace 0 writes it to a
// separate global buffer.  With --host-timing 1 the driver also reports the
// host time each C-ABI call takes to return (validation, the allocation-range
// checks and the launch; the kernels run asynchronously), averaged per call
// kind over the timed rounds, and the time of one allocation-range query on
// its own.  With --batched 1 each fragment's arrivals go to the library in
// one several-arrival call (with --fused 1 the call also closes: one pass
// per fragment); --batched 2 alternates the two schedules round by round
// (odd rounds batched), so one counter run covers both.  With --streams S > 1 every fragment's round
// is its own handle on one of S streams (rounds in flight together), the
// arrivals issued round-robin across fragments.  With --side 1 a round is
// instead the side averages and the worker adoption over the whole buffer:
// one fold of a global into the uniform-average sum, the average of 130
// globals, the means of the last 3 and last 5 snapshots (the checkpoints
// stand in for them; --workers >= 5), and the keep-local-drift adoption.
// Buffer contents are a deterministic pattern; the timing does not depend on
// them.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <chrono>
#include <map>
#include <utility>
#include <vector>

#include "dlmerge.h"

#define HIPCHECK(x)                                                                   \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_),  \
                         __LINE__);                                                   \
            std::exit(1);                                                             \
        }                                                                             \
    } while (0)

#define DLCHECK(x)                                                                    \
    do {                                                                              \
        int s_ = (x);                                                                 \
        if (s_ != DL_OK) {                                                            \
            std::fprintf(stderr, "dlmerge error %s at line %d\n", dl_strerror(s_),    \
                         __LINE__);                                                   \
            std::exit(1);                                                             \
        }                                                                             \
    } while (0)

namespace {

__device__ __forceinline__ uint32_t mix(uint64_t x) {
    x ^= x >> 33;
    x *= 0xff51afd7ed558ccdull;
    x ^= x >> 33;
    return static_cast<uint32_t>(x);
}

// value ~ 0.02 * uniform(-0.5, 0.5) + 1e-3 * stream offset pattern
__global__ void fill_f32(float* p, int64_t n, uint32_t stream) {
    for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x) {
        const float u = static_cast<float>(mix(uint64_t(i) * 0x9E3779B97F4A7C15ull + stream) >> 8) *
                        (1.0f / 16777216.0f);
        p[i] = 0.02f * (u - 0.5f) + 1e-3f * static_cast<float>(stream % 7);
    }
}

__global__ void fill_bf16(uint16_t* p, int64_t n, uint32_t stream) {
    for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x) {
        const float u = static_cast<float>(mix(uint64_t(i) * 0x9E3779B97F4A7C15ull + stream) >> 8) *
                        (1.0f / 16777216.0f);
        const float v = 0.02f * (u - 0.5f);
        p[i] = static_cast<uint16_t>(__float_as_uint(v) >> 16);
    }
}

// Plain copy of known size: reads npacks * 16 bytes, writes npacks * 16 bytes.
__global__ void plain_copy(const float4* __restrict__ src, float4* __restrict__ dst,
                           int64_t npacks) {
    for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < npacks;
         i += int64_t(gridDim.x) * blockDim.x)
        dst[i] = src[i];
}

struct Args {
    int64_t n = 0;
    std::vector<int64_t> offsets;
    bool delta = false;
    int workers = 5;
    bool bf16 = false;
    bool ema = true;
    int rounds = 1;
    int warmup = 1;
    int copy_mib = 0;
    bool fused = true;
    int streams = 1;
    bool side = false;
    bool inplace = true;
    bool host_timing = false;
    int batched = 0;
};

[[noreturn]] void usage() {
    std::fprintf(stderr,
                 "usage: dlmerge_driver --n N [--offsets 0,o1,...,N] [--mode mean|delta]\n"
                 "       [--workers W] [--dtype f32|bf16] [--ema 0|1] [--rounds R]\n"
                 "       [--warmup R0] [--copy-mib M] [--fused 0|1] [--streams S]\n"
                 "       [--side 0|1] [--inplace 0|1] [--host-timing 0|1] [--batched 0|1|2]\n");
    std::exit(2);
}

Args parse(int argc, char** argv) {
    Args a;
    for (int i = 1; i < argc; ++i) {
        std::string k = argv[i];
        if (i + 1 >= argc) usage();
        std::string v = argv[++i];
        if (k == "--n") a.n = std::atoll(v.c_str());
        else if (k == "--offsets") {
            size_t pos = 0;
            while (pos <= v.size()) {
                size_t c = v.find(',', pos);
                if (c == std::string::npos) c = v.size();
                a.offsets.push_back(std::atoll(v.substr(pos, c - pos).c_str()));
                pos = c + 1;
            }
        } else if (k == "--mode") a.delta = (v == "delta");
        else if (k == "--workers") a.workers = std::atoi(v.c_str());
        else if (k == "--dtype") a.bf16 = (v == "bf16");
        else if (k == "--ema") a.ema = std::atoi(v.c_str()) != 0;
        else if (k == "--rounds") a.rounds = std::atoi(v.c_str());
        else if (k == "--warmup") a.warmup = std::atoi(v.c_str());
        else if (k == "--copy-mib") a.copy_mib = std::atoi(v.c_str());
        else if (k == "--fused") a.fused = std::atoi(v.c_str()) != 0;
        else if (k == "--streams") a.streams = std::atoi(v.c_str());
        else if (k == "--side") a.side = std::atoi(v.c_str()) != 0;
        else if (k == "--inplace") a.inplace = std::atoi(v.c_str()) != 0;
        else if (k == "--host-timing") a.host_timing = std::atoi(v.c_str()) != 0;
        else if (k == "--batched") a.batched = std::atoi(v.c_str());
        else usage();
    }
    if (a.n <= 0 || a.workers < 1 || a.rounds < 0 || a.warmup < 0 || a.streams < 1 ||
        a.streams > 16 || (a.side && (a.workers < 5 || a.bf16 || !a.ema)) ||
        a.batched < 0 || a.batched > 2 || (a.batched && (a.streams > 1 || a.side)))
        usage();
    if (a.offsets.empty()) a.offsets = {0, a.n};
    return a;
}

}  // namespace

int main(int argc, char** argv) {
    const Args a = parse(argc, argv);
    const int n_frags = static_cast<int>(a.offsets.size()) - 1;
    const size_t fbytes = size_t(a.n) * sizeof(float);
    const size_t cbytes = size_t(a.n) * (a.bf16 ? 2 : 4);

    hipStream_t s;
    HIPCHECK(hipStreamCreate(&s));
    float *theta = nullptr, *m = nullptr, *e = nullptr, *acc = nullptr;
    HIPCHECK(hipMalloc(&theta, fbytes));
    HIPCHECK(hipMalloc(&acc, fbytes));
    if (a.delta) HIPCHECK(hipMalloc(&m, fbytes));
    if (a.ema) HIPCHECK(hipMalloc(&e, fbytes));
    std::vector<void*> ck(a.workers);
    for (auto& p : ck) HIPCHECK(hipMalloc(&p, cbytes));

    const dim3 fg(4096), fb(256);
    hipLaunchKernelGGL(fill_f32, fg, fb, 0, s, theta, a.n, 0u);
    if (m) HIPCHECK(hipMemsetAsync(m, 0, fbytes, s));
    if (e) hipLaunchKernelGGL(fill_f32, fg, fb, 0, s, e, a.n, 0u);
    for (int i = 0; i < a.workers; ++i) {
        if (a.bf16) hipLaunchKernelGGL(fill_bf16, fg, fb, 0, s, static_cast<uint16_t*>(ck[i]), a.n, uint32_t(i + 1));
        else hipLaunchKernelGGL(fill_f32, fg, fb, 0, s, static_cast<float*>(ck[i]), a.n, uint32_t(i + 1));
    }
    HIPCHECK(hipGetLastError());
    HIPCHECK(hipStreamSynchronize(s));

    if (a.copy_mib > 0) {
        const int64_t nb = int64_t(a.copy_mib) << 20;
        void *src = nullptr, *dst = nullptr;
        HIPCHECK(hipMalloc(&src, nb));
        HIPCHECK(hipMalloc(&dst, nb));
        HIPCHECK(hipMemsetAsync(src, 0, nb, s));
        hipLaunchKernelGGL(plain_copy, dim3(8192), dim3(256), 0, s, static_cast<const float4*>(src),
                           static_cast<float4*>(dst), nb / 16);
        HIPCHECK(hipGetLastError());
        HIPCHECK(hipStreamSynchronize(s));
        std::printf("copy calibration: plain_copy read %lld bytes, wrote %lld bytes\n",
                    (long long)nb, (long long)nb);
        HIPCHECK(hipFree(src));
        HIPCHECK(hipFree(dst));
    }

    hipEvent_t e0, e1;
    HIPCHECK(hipEventCreate(&e0));
    HIPCHECK(hipEventCreate(&e1));
    // extra streams for --streams: each waits for s at the start of a round,
    // and s waits for each at its end
    std::vector<hipStream_t> fs(a.streams, s);
    std::vector<hipEvent_t> joins(a.streams);
    for (int i = 1; i < a.streams; ++i) HIPCHECK(hipStreamCreate(&fs[i]));
    for (auto& ev : joins) HIPCHECK(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
    const int dt = a.bf16 ? DL_BF16 : DL_F32;
    const int64_t esz = a.bf16 ? 2 : 4;
    // host time per call kind over the timed rounds (--host-timing)
    std::map<std::string, std::pair<double, long>> host_us;
    auto timed = [&](const char* kind, bool on, auto&& call) {
        if (!a.host_timing || !on) return call();
        const auto t0 = std::chrono::steady_clock::now();
        const int st = call();
        const double us =
            std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count();
        auto& h = host_us[kind];
        h.first += us;
        h.second += 1;
        return st;
    };
    for (int r = 0; r < a.warmup + a.rounds; ++r) {
        const bool tr = r >= a.warmup;
        if (r == a.warmup) HIPCHECK(hipEventRecord(e0, s));
        if (a.side) {
            const float* snaps[5];
            for (int i = 0; i < 5; ++i) snaps[i] = static_cast<const float*>(ck[i]);
            DLCHECK(dl_swa_fold(acc, theta, a.n, r, s));
            DLCHECK(dl_swa_average(e, acc, a.n, 130, s));
            DLCHECK(dl_snapshot_average(e, snaps, 3, a.n, s));
            DLCHECK(dl_snapshot_average(e, snaps, 5, a.n, s));
            DLCHECK(dl_adopt_keep_drift(e, theta, ck[1], DL_F32, a.n, s));
            continue;
        }
        const uint64_t tag = uint64_t(r) + 1;
        const bool batched = a.batched == 1 || (a.batched == 2 && (r & 1));
        HIPCHECK(hipEventRecord(joins[0], s));
        for (int i = 1; i < a.streams; ++i) HIPCHECK(hipStreamWaitEvent(fs[i], joins[0], 0));
        std::vector<dl_round*> rd(a.streams > 1 ? n_frags : 1, nullptr);
        for (size_t h = 0; h < rd.size(); ++h)
            DLCHECK(timed("round_begin", tr, [&] {
                return dl_round_begin(&rd[h], tag, a.delta ? DL_DELTA_NESTEROV : DL_MEAN, a.n,
                                      n_frags, a.offsets.data(), 1, a.workers, acc,
                                      fs[h % a.streams]);
            }));
        // Batched: one several-arrival call per fragment (plus the close
        // when it is not fused).
        for (int f = 0; batched && f < n_frags; ++f) {
            dl_round* h = rd[0];
            std::vector<int> ids(a.workers);
            std::vector<uint64_t> tags(a.workers, tag);
            std::vector<int64_t> toks(a.workers);
            std::vector<const void*> bases(a.workers);
            for (int i = 0; i < a.workers; ++i) {
                ids[i] = i;
                toks[i] = 19660800 + 1000 * int64_t(i);
                bases[i] = static_cast<const char*>(ck[i]) + a.offsets[f] * esz;
            }
            float* out = a.inplace ? acc : theta;
            if (a.fused && a.delta)
                DLCHECK(timed("fold_checkpoints_and_outer_nesterov", tr, [&] {
                    return dl_fold_checkpoints_and_outer_nesterov(
                        h, f, a.workers, ids.data(), tags.data(), bases.data(), dt, toks.data(),
                        theta, m, 0.7f, 0.9f, e, 0.9f);
                }));
            else if (a.fused)
                DLCHECK(timed("fold_checkpoints_and_finalize_mean", tr, [&] {
                    return dl_fold_checkpoints_and_finalize_mean(h, f, a.workers, ids.data(),
                                                                 tags.data(), bases.data(), dt,
                                                                 out, e, 0.9f);
                }));
            else {
                DLCHECK(timed("fold_checkpoints", tr, [&] {
                    return dl_fold_checkpoints(h, f, a.workers, ids.data(), tags.data(),
                                               bases.data(), dt, a.delta ? theta : nullptr,
                                               toks.data());
                }));
                if (a.delta)
                    DLCHECK(timed("outer_nesterov", tr, [&] {
                        return dl_outer_nesterov(h, f, theta, m, 0.7f, 0.9f, e, 0.9f);
                    }));
                else
                    DLCHECK(timed("finalize_mean", tr, [&] {
                        return dl_finalize_mean(h, f, out, e, 0.9f);
                    }));
            }
        }
        // One stream: one handle, fragment after fragment (as the benchmark
        // issues a round).  Several streams: one handle per fragment, the
        // arrivals round-robin across fragments.
        for (int step = 0; !batched && step < a.workers * n_frags; ++step) {
            const int f = a.streams > 1 ? step % n_frags : step / a.workers;
            const int i = a.streams > 1 ? step / n_frags : step % a.workers;
            {
                dl_round* h = rd[a.streams > 1 ? f : 0];
                const char* base = static_cast<const char*>(ck[i]) + a.offsets[f] * esz;
                const int64_t tok = 19660800 + 1000 * int64_t(i);
                const bool last = i == a.workers - 1;
                float* out = a.inplace ? acc : theta;   // mean rounds: where the mean lands
                if (last && a.fused) {
                    if (a.delta)
                        DLCHECK(timed("fold_and_outer_nesterov", tr, [&] {
                            return dl_fold_and_outer_nesterov(h, f, i, tag, base, dt, tok, theta,
                                                              m, 0.7f, 0.9f, e, 0.9f);
                        }));
                    else
                        DLCHECK(timed("fold_and_finalize_mean", tr, [&] {
                            return dl_fold_and_finalize_mean(h, f, i, tag, base, dt, out, e, 0.9f);
                        }));
                    continue;
                }
                DLCHECK(timed("fold_checkpoint", tr, [&] {
                    return dl_fold_checkpoint(h, f, i, tag, base, dt, a.delta ? theta : nullptr,
                                              tok);
                }));
                if (last) {
                    if (a.delta)
                        DLCHECK(timed("outer_nesterov", tr, [&] {
                            return dl_outer_nesterov(h, f, theta, m, 0.7f, 0.9f, e, 0.9f);
                        }));
                    else
                        DLCHECK(timed("finalize_mean", tr, [&] {
                            return dl_finalize_mean(h, f, out, e, 0.9f);
                        }));
                }
            }
        }
        for (auto h : rd) DLCHECK(timed("round_end", tr, [&] { return dl_round_end(h); }));
        if (!a.delta && a.inplace) std::swap(theta, acc);   // the sum's buffer holds the new global
        for (int i = 1; i < a.streams; ++i) {
            HIPCHECK(hipEventRecord(joins[i], fs[i]));
            HIPCHECK(hipStreamWaitEvent(s, joins[i], 0));
        }
    }
    HIPCHECK(hipEventRecord(e1, s));
    HIPCHECK(hipEventSynchronize(e1));
    if (a.rounds > 0) {
        float ms = 0.f;
        HIPCHECK(hipEventElapsedTime(&ms, e0, e1));
        std::printf("%d rounds: %.4f ms per round\n", a.rounds, ms / a.rounds);
    }
    if (a.host_timing) {
        for (const auto& kv : host_us)
            std::printf("host time per call: %-26s %8.2f us (%ld calls)\n", kv.first.c_str(),
                        kv.second.first / kv.second.second, kv.second.second);
        // one allocation-range query alone, as the library makes per device span
        const int reps = 10000;
        const auto t0 = std::chrono::steady_clock::now();
        for (int k = 0; k < reps; ++k) {
            hipDeviceptr_t base = nullptr;
            size_t size = 0;
            HIPCHECK(hipMemGetAddressRange(&base, &size, acc + k));
        }
        const double us =
            std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count();
        std::printf("host time per call: %-26s %8.2f us (%d calls)\n", "hipMemGetAddressRange",
                    us / reps, reps);
    }

    for (int i = 1; i < a.streams; ++i) HIPCHECK(hipStreamDestroy(fs[i]));
    for (auto ev : joins) HIPCHECK(hipEventDestroy(ev));
    for (auto p : ck) HIPCHECK(hipFree(p));
    HIPCHECK(hipFree(theta));
    HIPCHECK(hipFree(acc));
    if (m) HIPCHECK(hipFree(m));
    if (e) HIPCHECK(hipFree(e));
    HIPCHECK(hipStreamDestroy(s));
    return 0;
}

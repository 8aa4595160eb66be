// dlpolar_driver: runs the orthogonalised outer step through the C ABI
// (include/dlmerge.h) on buffers it allocates with hipMalloc, with no other
// GPU work besides a fill pass and an optional plain copy kernel of known
// size.  It is the program hardware counters are collected on for the
// orthogonalisation kernels.
//
//   dlpolar_driver --shapes RxC:count[,RxC:count...] [--batch B] [--steps S]
//                  [--warmup W] [--quintic Q] [--cubic C] [--copy-mib M]
//                  (--batch 0: each shape's matrices split evenly into as few
//                  batches of at most DL_MAX_BATCH as hold them)
//   dlpolar_driver --gemm TN|NT:MxNxK[:sym][:nows] [--batch B] [--steps S]
//                  [--warmup W]
//
// The second form times one launch of dl_matmul_f32_batch over B products
// of that shape (S launches, each bracketed by events) with the workspace of
// dl_matmul_workspace_bytes_batch (none with :nows); `sym` declares the
// results symmetric (A = B, M = N).
//
// One step runs theta = theta - s * P(theta - averaged) once for every
// matrix of the list (count matrices of each shape, in list order), in
// batches of up to B equally shaped matrices (dl_outer_orthogonal_step_batch;
// B = 1: one by one), on one stream with one workspace sized for the
// largest batch.  The batches of a step share B theta / averaged pairs of
// the largest size (the kernels' work does not depend on where the buffers
// sit).  Prints the average time per
// step and per shape, and the algorithmic TFLOP/s (symmetric Gram products
// counted at their distinct outputs).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>
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

// p[i] = base[i] + scale * uniform(-0.5, 0.5)  (base may be null: 0)
__global__ void fill(float* p, const float* base, float scale, int64_t n, uint32_t stream) {
    for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x) {
        const float u = static_cast<float>(mix(uint64_t(i) * 0x9E3779B97F4A7C15ull + stream) >> 8) *
                        (1.0f / 16777216.0f);
        p[i] = (base ? base[i] : 0.0f) + scale * (u - 0.5f);
    }
}

// Plain copy of known size: reads npacks * 16 bytes, writes npacks * 16 bytes.
__global__ void plain_copy(const float4* __restrict__ src, float4* __restrict__ dst,
                           int64_t npacks) {
    for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < npacks;
         i += int64_t(gridDim.x) * blockDim.x)
        dst[i] = src[i];
}

struct Shape {
    int64_t rows, cols;
    int count;
};

struct Gemm {
    bool tn = true, sym = false, ws = true;
    int64_t m = 0, n = 0, k = 0;
};

struct Args {
    std::vector<Shape> shapes;
    Gemm gemm;
    bool has_gemm = false;
    int steps = 1;
    int warmup = 1;
    int quintic = 12;
    int cubic = 6;
    int copy_mib = 0;
    int batch = 1;
};

[[noreturn]] void usage() {
    std::fprintf(stderr,
                 "usage: dlpolar_driver --shapes RxC:count[,RxC:count...] [--batch B]\n"
                 "       [--steps S] [--warmup W] [--quintic Q] [--cubic C] [--copy-mib M]\n"
                 "       dlpolar_driver --gemm TN|NT:MxNxK[:sym][:nows] [--batch B] [--steps S]\n"
                 "       [--warmup W]\n");
    std::exit(2);
}

Args parse(int argc, char** argv) {
    Args a;
    for (int i = 1; i < argc; ++i) {
        std::string k = argv[i];
        if (i + 1 >= argc) usage();
        std::string v = argv[++i];
        if (k == "--shapes") {
            size_t pos = 0;
            while (pos < v.size()) {
                size_t c = v.find(',', pos);
                if (c == std::string::npos) c = v.size();
                const std::string item = v.substr(pos, c - pos);
                Shape s{0, 0, 1};
                if (std::sscanf(item.c_str(), "%ldx%ld:%d", &s.rows, &s.cols, &s.count) < 2)
                    usage();
                a.shapes.push_back(s);
                pos = c + 1;
            }
        } else if (k == "--gemm") {
            char form[3] = {0, 0, 0};
            if (std::sscanf(v.c_str(), "%2[TN]:%ldx%ldx%ld", form, &a.gemm.m, &a.gemm.n,
                            &a.gemm.k) != 4)
                usage();
            a.gemm.tn = std::string(form) == "TN";
            a.gemm.sym = v.find(":sym") != std::string::npos;
            a.gemm.ws = v.find(":nows") == std::string::npos;
            a.has_gemm = true;
        } else if (k == "--steps") a.steps = std::atoi(v.c_str());
        else if (k == "--warmup") a.warmup = std::atoi(v.c_str());
        else if (k == "--quintic") a.quintic = std::atoi(v.c_str());
        else if (k == "--cubic") a.cubic = std::atoi(v.c_str());
        else if (k == "--copy-mib") a.copy_mib = std::atoi(v.c_str());
        else if (k == "--batch") a.batch = std::atoi(v.c_str());
        else usage();
    }
    if ((a.shapes.empty() && !a.has_gemm) || a.steps < 1 || a.warmup < 0 || a.batch < 0 ||
        a.batch > DL_MAX_BATCH || (a.has_gemm && a.batch < 1))
        usage();
    if (a.has_gemm && (a.gemm.m < 1 || a.gemm.n < 1 || a.gemm.k < 1 ||
                       (a.gemm.sym && a.gemm.m != a.gemm.n)))
        usage();
    for (const Shape& s : a.shapes)
        if (s.rows < 1 || s.cols < 1 || s.count < 1) usage();
    return a;
}

// Algorithmic flops of the iteration on one matrix (see the orthogonalise
// module): symmetric Gram products at their distinct outputs.
double flops(const Shape& s, int quintic, int cubic) {
    const double r = s.rows < s.cols ? s.rows : s.cols, L = s.rows < s.cols ? s.cols : s.rows;
    const double sym = r * (r + 1) / 2;
    return (quintic + cubic) * (2 * sym * L + 2 * L * r * r) + quintic * 2 * sym * r;
}

// Sizes of the batches `count` matrices of one shape run in: chunks of
// `batch`, or (batch 0) an even split into ceil(count / DL_MAX_BATCH).
std::vector<int> batches(int count, int batch) {
    std::vector<int> out;
    if (batch > 0) {
        for (int c = 0; c < count; c += batch) out.push_back(count - c < batch ? count - c : batch);
        return out;
    }
    const int n = (count + DL_MAX_BATCH - 1) / DL_MAX_BATCH;
    for (int i = 0; i < n; ++i) out.push_back(count / n + (i < count % n ? 1 : 0));
    return out;
}

}  // namespace

// One batched product launch, timed launch by launch.  A and B are filled
// with a pattern; for a symmetric result B is A (A^T A as TN, A A^T as NT).
int run_gemm(const Args& a) {
    const Gemm& g = a.gemm;
    const int bt = a.batch;
    const int64_t na = g.tn ? g.k * g.m : g.m * g.k;
    const int64_t nb = g.tn ? g.k * g.n : g.n * g.k;
    float *A = nullptr, *B = nullptr, *C = nullptr;
    void* ws = nullptr;
    int64_t wsb = 0;
    DLCHECK(dl_matmul_workspace_bytes_batch(g.m, g.n, g.k, g.sym ? 1 : 0, bt, &wsb));
    HIPCHECK(hipMalloc(&A, bt * na * sizeof(float)));
    if (!g.sym) HIPCHECK(hipMalloc(&B, bt * nb * sizeof(float)));
    HIPCHECK(hipMalloc(&C, bt * g.m * g.n * sizeof(float)));
    if (g.ws && wsb > 0) HIPCHECK(hipMalloc(&ws, wsb));
    hipLaunchKernelGGL(fill, dim3(4096), dim3(256), 0, nullptr, A, nullptr, 0.04f, bt * na, 3u);
    if (!g.sym)
        hipLaunchKernelGGL(fill, dim3(4096), dim3(256), 0, nullptr, B, nullptr, 0.04f, bt * nb, 4u);
    HIPCHECK(hipGetLastError());
    HIPCHECK(hipDeviceSynchronize());
    const float* Bp = g.sym ? A : B;
    const int64_t lda = g.tn ? g.m : g.k, ldb = g.tn ? g.n : g.k;
    auto launch = [&]() {
        DLCHECK(dl_matmul_f32_batch(g.tn ? DL_TN : DL_NT, A, lda, na, Bp, ldb, g.sym ? na : nb,
                                    g.m, g.n, g.k, C, g.n, g.m * g.n, nullptr, 0, 1.0f, 0.0f,
                                    0.0f, g.sym ? 1 : 0, bt, ws, ws ? wsb : 0, nullptr));
    };
    for (int w = 0; w < a.warmup; ++w) launch();
    HIPCHECK(hipDeviceSynchronize());
    std::vector<hipEvent_t> ev(2 * a.steps);
    for (hipEvent_t& x : ev) HIPCHECK(hipEventCreate(&x));
    for (int st = 0; st < a.steps; ++st) {
        HIPCHECK(hipEventRecord(ev[2 * st], nullptr));
        launch();
        HIPCHECK(hipEventRecord(ev[2 * st + 1], nullptr));
    }
    HIPCHECK(hipDeviceSynchronize());
    double tot = 0.0, best = 1e30;
    for (int st = 0; st < a.steps; ++st) {
        float ms = 0.0f;
        HIPCHECK(hipEventElapsedTime(&ms, ev[2 * st], ev[2 * st + 1]));
        tot += ms;
        if (ms < best) best = ms;
    }
    const double outs = g.sym ? double(g.m) * (g.m + 1) / 2 : double(g.m) * g.n;
    const double fl = 2.0 * outs * g.k * bt, avg = tot / a.steps;
    std::printf("[driver] gemm %s %ldx%ldx%ld%s%s batch %d: avg %.4f ms (%.2f TFLOP/s), best "
                "%.4f ms (%.2f TFLOP/s), workspace %ld bytes\n",
                g.tn ? "TN" : "NT", g.m, g.n, g.k, g.sym ? " sym" : "", ws ? "" : " nows", bt, avg,
                fl / (avg / 1e3) / 1e12, best, fl / (best / 1e3) / 1e12, ws ? wsb : 0);
    HIPCHECK(hipFree(A));
    if (B) HIPCHECK(hipFree(B));
    HIPCHECK(hipFree(C));
    if (ws) HIPCHECK(hipFree(ws));
    return 0;
}

int main(int argc, char** argv) {
    const Args a = parse(argc, argv);
    if (a.has_gemm) return run_gemm(a);
    // slot b of the theta / averaged pairs holds the largest matrix that
    // runs in a batch of more than b
    int64_t ws_max = 0;
    int b_max = 0;
    std::vector<int64_t> slot;
    for (const Shape& s : a.shapes) {
        for (int b : batches(s.count, a.batch)) {
            int64_t ws = 0;
            DLCHECK(dl_polar_workspace_bytes_batch(s.rows, s.cols, b, &ws));
            if (ws > ws_max) ws_max = ws;
            if (b > b_max) b_max = b;
            if (static_cast<int>(slot.size()) < b) slot.resize(b, 0);
            for (int i = 0; i < b; ++i)
                if (s.rows * s.cols > slot[i]) slot[i] = s.rows * s.cols;
        }
    }
    const int64_t n_max = slot.empty() ? 0 : slot[0];
    std::vector<float*> theta(b_max, nullptr), avg(b_max, nullptr);
    void* ws = nullptr;
    for (int b = 0; b < b_max; ++b) {
        HIPCHECK(hipMalloc(&theta[b], slot[b] * sizeof(float)));
        HIPCHECK(hipMalloc(&avg[b], slot[b] * sizeof(float)));
        hipLaunchKernelGGL(fill, dim3(4096), dim3(256), 0, nullptr, theta[b], nullptr, 0.04f,
                           slot[b], 1u + 2u * b);
        hipLaunchKernelGGL(fill, dim3(4096), dim3(256), 0, nullptr, avg[b], theta[b], 2e-3f,
                           slot[b], 2u + 2u * b);
    }
    HIPCHECK(hipMalloc(&ws, ws_max));
    HIPCHECK(hipGetLastError());
    HIPCHECK(hipDeviceSynchronize());
    std::printf("[driver] %zu shape(s), batch %d, theta/averaged %ld floats each, workspace %ld "
                "bytes\n",
                a.shapes.size(), a.batch, n_max, ws_max);
    std::fflush(stdout);

    if (a.copy_mib > 0) {
        const int64_t nb = int64_t(a.copy_mib) << 20;
        float4 *src = nullptr, *dst = nullptr;
        HIPCHECK(hipMalloc(&src, nb));
        HIPCHECK(hipMalloc(&dst, nb));
        HIPCHECK(hipMemset(src, 0, nb));
        hipLaunchKernelGGL(plain_copy, dim3(4096), dim3(256), 0, nullptr, src, dst, nb / 16);
        HIPCHECK(hipGetLastError());
        HIPCHECK(hipDeviceSynchronize());
        HIPCHECK(hipFree(src));
        HIPCHECK(hipFree(dst));
        std::printf("[driver] plain copy: %ld bytes read, %ld bytes written\n", nb, nb);
    }

    const float scale = 1e-4f;
    auto step = [&](std::vector<double>* shape_ms, std::vector<hipEvent_t>& ev) {
        size_t e = 0;
        for (size_t i = 0; i < a.shapes.size(); ++i) {
            const Shape& s = a.shapes[i];
            if (shape_ms) HIPCHECK(hipEventRecord(ev[e], nullptr));
            for (int b : batches(s.count, a.batch)) {
                DLCHECK(dl_outer_orthogonal_step_batch(theta.data(), avg.data(), b, s.rows, s.cols,
                                                       scale, a.quintic, a.cubic, ws, ws_max,
                                                       nullptr));
            }
            if (shape_ms) HIPCHECK(hipEventRecord(ev[e + 1], nullptr));
            e += 2;
        }
    };
    std::vector<hipEvent_t> ev(2 * a.shapes.size());
    for (hipEvent_t& x : ev) HIPCHECK(hipEventCreate(&x));
    for (int w = 0; w < a.warmup; ++w) step(nullptr, ev);
    HIPCHECK(hipDeviceSynchronize());
    std::vector<double> shape_ms(a.shapes.size(), 0.0);
    hipEvent_t t0, t1;
    HIPCHECK(hipEventCreate(&t0));
    HIPCHECK(hipEventCreate(&t1));
    double total_ms = 0.0;
    for (int st = 0; st < a.steps; ++st) {
        HIPCHECK(hipEventRecord(t0, nullptr));
        step(&shape_ms, ev);
        HIPCHECK(hipEventRecord(t1, nullptr));
        HIPCHECK(hipEventSynchronize(t1));
        float ms = 0.0f;
        HIPCHECK(hipEventElapsedTime(&ms, t0, t1));
        total_ms += ms;
        for (size_t i = 0; i < a.shapes.size(); ++i) {
            float m = 0.0f;
            HIPCHECK(hipEventElapsedTime(&m, ev[2 * i], ev[2 * i + 1]));
            shape_ms[i] += m;
        }
        std::printf("[driver] step %d: %.2f ms\n", st, ms);
        std::fflush(stdout);
    }
    double fl_total = 0.0;
    for (size_t i = 0; i < a.shapes.size(); ++i) {
        const Shape& s = a.shapes[i];
        const double f = flops(s, a.quintic, a.cubic) * s.count;
        fl_total += f;
        const double ms = shape_ms[i] / a.steps;
        std::printf("[driver] %ldx%ld x%d: %.3f ms per matrix, %.2f TFLOP/s\n", s.rows, s.cols,
                    s.count, ms / s.count, f / (ms / 1e3) / 1e12);
    }
    const double ms = total_ms / a.steps;
    std::printf("[driver] step: %.2f ms, %.2f TFLOP/s (%.3e flops)\n", ms,
                fl_total / (ms / 1e3) / 1e12, fl_total);
    for (int b = 0; b < b_max; ++b) {
        HIPCHECK(hipFree(theta[b]));
        HIPCHECK(hipFree(avg[b]));
    }
    HIPCHECK(hipFree(ws));
    return 0;
}

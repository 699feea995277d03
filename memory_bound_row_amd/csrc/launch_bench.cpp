// launch_bench.cpp -- host-side cost of the decode-shaped LayerNorm forward:
// `rows` x `cols` rows of one storage type, mean/rstd not saved (inference
// keeps no intermediates), N back-to-back ln_fwd calls on one stream.
//
// Prints one JSON object with the microseconds per call of
//   cpp_loop_us  a plain C++ loop of N calls, timed with steady_clock from the
//                first call to the end of one stream synchronisation;
//   graph_us     the same N calls captured into one HIP graph and replayed.
// A benchmark tool next to the library it measures; it is not part of the
// library.  Usage: launch_bench [rows cols calls dtype(0 f32, 1 f16, 2 bf16)]
#include <hip/hip_runtime.h>

#include <chrono>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "mbrow_ln.h"

namespace {

bool ok(hipError_t e, const char* what) {
    if (e != hipSuccess) {
        std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
        return false;
    }
    return true;
}

bool ok(ln_status_t s, const char* what) {
    if (s != LN_OK) {
        std::fprintf(stderr, "%s: %s\n", what, ln_status_string(s));
        return false;
    }
    return true;
}

// Host bit patterns of 1.0 (x, gamma) and 0.5 (beta) in the storage type.
void fill(std::vector<uint8_t>& h, int64_t n, int dt, float v) {
    const size_t es = dt == 0 ? 4 : 2;
    h.resize((size_t)n * es);
    uint32_t bits32;
    std::memcpy(&bits32, &v, 4);
    const uint16_t bits16 = dt == 2 ? (uint16_t)(bits32 >> 16)   // exact for 1.0 and 0.5
                                    : (uint16_t)(v == 1.0f ? 0x3C00 : 0x3800);
    for (int64_t i = 0; i < n; ++i) {
        if (es == 4) std::memcpy(&h[(size_t)i * 4], &bits32, 4);
        else std::memcpy(&h[(size_t)i * 2], &bits16, 2);
    }
}

}  // namespace

int main(int argc, char** argv) {
    const int64_t rows = argc > 1 ? std::atoll(argv[1]) : 1;
    const int64_t cols = argc > 2 ? std::atoll(argv[2]) : 4096;
    const int calls = argc > 3 ? std::atoi(argv[3]) : 10000;
    const int dt = argc > 4 ? std::atoi(argv[4]) : 1;
    if (rows <= 0 || cols <= 0 || calls <= 0 || dt < 0 || dt > 2) {
        std::fprintf(stderr, "usage: launch_bench [rows cols calls dtype]\n");
        return 2;
    }
    std::vector<uint8_t> hx, hg, hb;
    fill(hx, rows * cols, dt, 1.0f);
    fill(hg, cols, dt, 1.0f);
    fill(hb, cols, dt, 0.5f);

    void *x = nullptr, *g = nullptr, *b = nullptr, *y = nullptr;
    hipStream_t s = nullptr;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    int rc = 1;
    const ln_dtype_t dtype = static_cast<ln_dtype_t>(dt);
    double loop_us = 0.0, graph_us = 0.0;
    auto enqueue = [&]() {
        return ln_fwd(x, g, b, y, nullptr, nullptr, rows, cols, 1e-5f, dtype, s);
    };
    do {
        if (!ok(hipMalloc(&x, hx.size()), "hipMalloc x") ||
            !ok(hipMalloc(&y, hx.size()), "hipMalloc y") ||
            !ok(hipMalloc(&g, hg.size()), "hipMalloc gamma") ||
            !ok(hipMalloc(&b, hb.size()), "hipMalloc beta") ||
            !ok(hipMemcpy(x, hx.data(), hx.size(), hipMemcpyHostToDevice), "copy x") ||
            !ok(hipMemcpy(g, hg.data(), hg.size(), hipMemcpyHostToDevice), "copy gamma") ||
            !ok(hipMemcpy(b, hb.data(), hb.size(), hipMemcpyHostToDevice), "copy beta") ||
            !ok(hipStreamCreate(&s), "hipStreamCreate"))
            break;
        bool good = true;
        for (int i = 0; i < 200 && good; ++i) good = ok(enqueue(), "ln_fwd");
        if (!good || !ok(hipStreamSynchronize(s), "sync")) break;

        const auto t0 = std::chrono::steady_clock::now();
        for (int i = 0; i < calls && good; ++i) good = ok(enqueue(), "ln_fwd");
        if (!good || !ok(hipStreamSynchronize(s), "sync")) break;
        const auto t1 = std::chrono::steady_clock::now();
        loop_us = std::chrono::duration<double, std::micro>(t1 - t0).count() / calls;

        if (!ok(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal), "begin capture"))
            break;
        for (int i = 0; i < calls && good; ++i) good = ok(enqueue(), "ln_fwd (capture)");
        if (!ok(hipStreamEndCapture(s, &graph), "end capture") || !good) break;
        if (!ok(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0), "instantiate") ||
            !ok(hipGraphLaunch(exec, s), "graph launch") ||
            !ok(hipStreamSynchronize(s), "sync"))
            break;
        const auto t2 = std::chrono::steady_clock::now();
        if (!ok(hipGraphLaunch(exec, s), "graph launch") || !ok(hipStreamSynchronize(s), "sync"))
            break;
        const auto t3 = std::chrono::steady_clock::now();
        graph_us = std::chrono::duration<double, std::micro>(t3 - t2).count() / calls;
        rc = 0;
    } while (false);

    if (exec) hipGraphExecDestroy(exec);
    if (graph) hipGraphDestroy(graph);
    if (s) hipStreamDestroy(s);
    hipFree(x);
    hipFree(y);
    hipFree(g);
    hipFree(b);
    if (rc == 0)
        std::printf("{\"rows\": %lld, \"cols\": %lld, \"dtype\": %d, \"calls\": %d, "
                    "\"cpp_loop_us\": %.3f, \"graph_us\": %.3f}\n",
                    (long long)rows, (long long)cols, dt, calls, loop_us, graph_us);
    return rc;
}

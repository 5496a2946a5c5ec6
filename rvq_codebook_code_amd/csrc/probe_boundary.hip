// Cost of a kernel boundary: the time per kernel of `launches` back-to-back
// launches of one trivial kernel, captured as one graph and replayed (the
// regime of the batched path's frames) or launched on a stream.  The kernel
// does nothing, writes `n` floats, or reads `n` floats, on `blocks`
// workgroups of 256 threads.  Built into libqp_probe.so; bench.py
// --boundary-probe prints a table.
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace {

// kind 0: no work; 1: writes p[0..n); 2: reads p[0..n) (one store per
// workgroup only if the sum were an impossible value, so the loads stay)
__global__ __launch_bounds__(256) void k_boundary(float* p, size_t n, int kind) {
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    const size_t i0 = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (kind == 1) {
        for (size_t i = i0; i < n; i += stride) p[i] = static_cast<float>(i);
    } else if (kind == 2) {
        float s = 0.f;
        for (size_t i = i0; i < n; i += stride) s += p[i];
        if (s == -1234.5f) p[blockIdx.x] = s;
    }
}

}  // namespace

extern "C" {

// Best-of-`reps` microseconds per kernel.  kind 0, 1 or 2; blocks in
// [1, 4096]; n <= 2^26 floats (256 MiB); launches in [1, 1000]; graph != 0
// captures the launches as one graph (replayed reps times), else launches
// them on a stream.  Returns 0, -1 for unsupported settings, else a HIP
// error code.
int qp_probe_boundary(int kind, int blocks, size_t n, int launches, int graph, int reps, float* us_per_kernel) {
    if (kind < 0 || kind > 2 || blocks < 1 || blocks > 4096 || n > (static_cast<size_t>(1) << 26) ||
        launches < 1 || launches > 1000 || reps < 1)
        return -1;
    if (kind != 0 && n < static_cast<size_t>(blocks)) return -1;
    float* buf = nullptr;
    hipStream_t st = nullptr;
    hipGraph_t g = nullptr;
    hipGraphExec_t ge = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    const size_t nbuf = n > 0 ? n : 1;
    hipError_t e = hipMalloc(&buf, nbuf * 4);
    if (e == hipSuccess) e = hipMemset(buf, 0, nbuf * 4);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    auto enqueue = [&]() {
        for (int i = 0; i < launches; ++i) hipLaunchKernelGGL(k_boundary, dim3(blocks), dim3(256), 0, st, buf, n, kind);
        return hipGetLastError();
    };
    if (e == hipSuccess && graph) {
        e = hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal);
        if (e == hipSuccess) {
            const hipError_t le = enqueue();
            e = hipStreamEndCapture(st, &g);
            if (e == hipSuccess) e = le;
        }
        if (e == hipSuccess) e = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
    }
    float best = 1e30f;
    for (int r = 0; r < reps + 1 && e == hipSuccess; ++r) {   // the first round warms up
        e = hipEventRecord(e0, st);
        if (e == hipSuccess) e = graph ? hipGraphLaunch(ge, st) : enqueue();
        if (e == hipSuccess) e = hipEventRecord(e1, st);
        if (e == hipSuccess) e = hipEventSynchronize(e1);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
        if (e == hipSuccess && r > 0 && ms < best) best = ms;
    }
    if (st) (void)hipStreamSynchronize(st);
    if (ge) (void)hipGraphExecDestroy(ge);
    if (g) (void)hipGraphDestroy(g);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (st) (void)hipStreamDestroy(st);
    (void)hipFree(buf);
    if (e != hipSuccess) return static_cast<int>(e);
    *us_per_kernel = best * 1e3f / launches;
    return 0;
}

}  // extern "C"

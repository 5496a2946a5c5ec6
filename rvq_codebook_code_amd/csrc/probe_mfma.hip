// Measured peak of the bf16 matrix-core instruction the batched products use
// (v_mfma_f32_16x16x32_bf16), for quoting matrix-core utilisation against a
// number taken on the same GPU beside the vendor's dense figure.  Built into
// its own library (libqp_probe.so); bench.py --mfma-peak calls it.
//
// Every wave runs `iters` rounds of 8 independent accumulation chains, so
// the matrix unit never waits on a result; wgs_per_cu workgroups of 4 waves
// per compute unit.  flops = waves * iters * 8 * (2 * 16 * 16 * 32).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_mfma_peak(float* out, int iters) {
    const int t = threadIdx.x;
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = static_cast<__bf16>(1.0f + 1e-3f * static_cast<float>((t + i) & 7));
        b[i] = static_cast<__bf16>(1.0f - 1e-3f * static_cast<float>((t * 3 + i) & 7));
    }
    f32x4_t c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
    out[blockIdx.x * blockDim.x + t] = s;
}

}  // namespace

extern "C" {

// Runs the probe on the current device: returns 0 on success, else the HIP
// error code.  ms_out: the best of `reps` timed launches; tflops_out: the
// dense bf16 rate of that launch in TFLOP/s.
int qp_probe_mfma_bf16(int wgs_per_cu, int iters, int reps, float* ms_out, double* tflops_out) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return static_cast<int>(e);
    const int wgs = cus * wgs_per_cu;
    float* out = nullptr;
    e = hipMalloc(&out, static_cast<size_t>(wgs) * 256 * sizeof(float));
    if (e != hipSuccess) return static_cast<int>(e);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    (void)hipEventCreate(&e0);
    (void)hipEventCreate(&e1);
    float best = 1e30f;
    for (int r = 0; r < reps + 1 && e == hipSuccess; ++r) {   // the first launch warms up
        hipEventRecord(e0, nullptr);
        hipLaunchKernelGGL(k_mfma_peak, dim3(wgs), dim3(256), 0, nullptr, out, iters);
        hipEventRecord(e1, nullptr);
        e = hipEventSynchronize(e1);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
        if (r > 0 && ms < best) best = ms;
    }
    if (e == hipSuccess) e = hipGetLastError();
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    (void)hipFree(out);
    if (e != hipSuccess) return static_cast<int>(e);
    const double flops = static_cast<double>(wgs) * 4.0 * iters * 8.0 * (2.0 * 16 * 16 * 32);
    *ms_out = best;
    *tflops_out = flops / (best * 1e-3) / 1e12;
    return 0;
}

}  // extern "C"

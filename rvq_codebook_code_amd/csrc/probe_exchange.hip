// Cost of one hand-off through tagged records, the exchange the dataflow
// kernels are built on.  One cooperative launch of 256 workgroups repeats
// `phases` times: every workgroup writes its share of a set of R 64-bit
// records (phase tag in the high word), then `consumers` workgroups wait
// until they have seen all R records carry the phase's tag, `waves` waves
// each pulling a slice with `loads` 16-byte device-coherent loads per lane
// in flight.  Every phase writes a fresh region, so nothing is overwritten
// while a slow consumer still reads it.  Built into libqp_probe.so; bench.py
// --exchange-probe prints the time per phase for a grid of settings.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kNwg = 256;
constexpr int kDevScope = 16;   // buffer cache policy: device-coherent

template <int NW, int NL>
__global__ __launch_bounds__(NW * 64) void k_exchange(uint64_t* buf, int R, int consumers, int phases,
                                                      uint32_t tag0, float* sink, unsigned* err) {
    const int wg = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float acc = 0.f;
    for (int ph = 0; ph < phases; ++ph) {
        uint64_t* b = buf + static_cast<size_t>(ph) * R;
        const uint32_t tag = tag0 + ph + 1;
        const int per = R / kNwg;
        for (int i = threadIdx.x; i < per; i += NW * 64) {
            const uint64_t u = (static_cast<uint64_t>(tag) << 32) | __float_as_uint(acc + i);
            __hip_atomic_store(b + static_cast<size_t>(wg) * per + i, u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (wg < consumers) {
            const int q = R / NW;                   // records of this wave's slice
            const auto r = __builtin_amdgcn_make_buffer_rsrc(b + static_cast<size_t>(wave) * q, static_cast<short>(0),
                                                             q * 8, 0x00020000);
            const int nj = q / 128;                 // 16-byte loads per lane (two records each)
            for (int j0 = 0; j0 < nj; j0 += NL) {
                const int n = nj - j0 < NL ? nj - j0 : NL;
                uint32_t pend = (1u << n) - 1u;
                unsigned spins = 0;
                while (true) {
                    decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0u, 0u, 0)) u[NL];
#pragma unroll
                    for (int j = 0; j < NL; ++j)
                        if ((pend >> j) & 1u)
                            u[j] = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16u, 1024u * (j0 + j), kDevScope);
#pragma unroll
                    for (int j = 0; j < NL; ++j)
                        if (((pend >> j) & 1u) && static_cast<uint32_t>(u[j][1]) == tag &&
                            static_cast<uint32_t>(u[j][3]) == tag) {
                            acc += __int_as_float(u[j][0]) + __int_as_float(u[j][2]);
                            pend &= ~(1u << j);
                        }
                    if (!__any(pend != 0u)) break;
                    __builtin_amdgcn_s_sleep(1);
                    if (++spins > (1u << 22)) {   // bounded: a lost record flags and ends the wait
                        atomicOr(err, 1u);
                        break;
                    }
                }
            }
        }
        __syncthreads();
    }
    if (acc == 1234.5f) sink[threadIdx.x] = acc;   // keeps the loads
}

}  // namespace

extern "C" {

// Best-of-`reps` microseconds per phase for R records (R a multiple of 256,
// R / waves a multiple of 128, R <= 49152), `consumers` in [1, 256], waves
// 4, 8 or 16 with 8 loads per lane in flight, or 4 with 16.  Returns 0, -1
// for unsupported settings, 1 if a wait timed out, else a HIP error code.
int qp_probe_exchange(int R, int consumers, int waves, int loads, int phases, int reps, float* us_per_phase) {
    if (R <= 0 || R % 256 || R > 49152 || consumers < 1 || consumers > kNwg || phases < 1 || phases > 400 ||
        (R / waves) % 128)
        return -1;
    const void* fn = nullptr;
    if (waves == 4 && loads == 8) fn = reinterpret_cast<const void*>(&k_exchange<4, 8>);
    else if (waves == 4 && loads == 16) fn = reinterpret_cast<const void*>(&k_exchange<4, 16>);
    else if (waves == 8 && loads == 8) fn = reinterpret_cast<const void*>(&k_exchange<8, 8>);
    else if (waves == 16 && loads == 8) fn = reinterpret_cast<const void*>(&k_exchange<16, 8>);
    else return -1;
    uint64_t* buf = nullptr;
    float* sink = nullptr;
    unsigned* err = nullptr;
    const size_t bytes = static_cast<size_t>(R) * phases * 8;
    hipError_t e = hipMalloc(&buf, bytes);
    if (e == hipSuccess) e = hipMalloc(&sink, 4096);
    if (e == hipSuccess) e = hipMalloc(&err, 4);
    if (e == hipSuccess) e = hipMemset(buf, 0, bytes);
    if (e == hipSuccess) e = hipMemset(err, 0, 4);
    float best = 1e30f;
    uint32_t tag = 0;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (e == hipSuccess) e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    for (int r = 0; r < reps + 1 && e == hipSuccess; ++r) {   // the first launch warms up
        int Rv = R, cv = consumers, pv = phases;
        uint32_t tv = tag;
        void* args[] = {&buf, &Rv, &cv, &pv, &tv, &sink, &err};
        hipEventRecord(e0, nullptr);
        e = hipLaunchCooperativeKernel(fn, dim3(kNwg), dim3(waves * 64), args, 0, nullptr);
        hipEventRecord(e1, nullptr);
        if (e == hipSuccess) e = hipEventSynchronize(e1);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
        if (r > 0 && ms < best) best = ms;
        tag += phases + 2;
    }
    unsigned flag = 0;
    if (e == hipSuccess) e = hipMemcpy(&flag, err, 4, hipMemcpyDeviceToHost);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    (void)hipFree(buf);
    (void)hipFree(sink);
    (void)hipFree(err);
    if (e != hipSuccess) return static_cast<int>(e);
    *us_per_phase = best * 1e3f / phases;
    return flag ? 1 : 0;
}

}  // extern "C"

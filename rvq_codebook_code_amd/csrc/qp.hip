// Host side of the code-predictor library: the C ABI declared in qp.h,
// create-time weight preparation, and the frame drivers: the dataflow kernel
// (small batches of the 1.7B geometry), the batched matrix-core path (one
// kernel per phase) and the generic path (one persistent cooperative kernel
// per frame, or one kernel per phase).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "qp.h"
#include "qp_common.h"
#include "qp_phases.h"
#include "qp_stream.h"
#include "qp_tiled.h"
#include "qp_flow.h"
#include "qp_sample.h"

using namespace qp;

// ---------------------------------------------------------------------------
// device kernels
// ---------------------------------------------------------------------------

namespace {

// Grid barrier.  Workgroups arrive on one of 8 group counters (contention is
// what makes a single counter slow), the last arriver of a group bumps the top
// counter and the last group publishes the barrier's generation; everybody
// polls the generation word.  All words are 64-bit and only grow, so no reset
// is needed between launches: the host passes how many barriers came before.
// Phase data moves with device-scope loads/stores (ld_act/st_act), so the
// barrier only has to make this workgroup's stores complete before arriving.
constexpr int kBarGroups = 8;
constexpr int kBarStride = 16;  // 128-byte spacing between barrier words

__device__ void grid_sync(unsigned long long* bar, unsigned long long idx, unsigned* err, int wg, int nwg) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's stores are complete
    __syncthreads();
    if (threadIdx.x == 0) {
        const int ngroups = nwg < kBarGroups ? nwg : kBarGroups;
        const int g = wg % ngroups;
        const unsigned long long gsize = static_cast<unsigned long long>((nwg - g + ngroups - 1) / ngroups);
        unsigned long long* top = bar + kBarGroups * kBarStride;
        unsigned long long* gen = top + kBarStride;
        const unsigned long long old =
            __hip_atomic_fetch_add(bar + g * kBarStride, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old == idx * gsize - 1) {
            const unsigned long long t =
                __hip_atomic_fetch_add(top, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (t == idx * static_cast<unsigned long long>(ngroups) - 1)
                __hip_atomic_store(gen, idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        unsigned spins = 0;
        while (__hip_atomic_load(gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < idx) {
            __builtin_amdgcn_s_sleep(1);
            ++spins;
            // bounded wait: a barrier that never completes flags the frame
            // and lets every workgroup run to its end
            if ((spins & 1023u) == 0u) {
                if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kErrBarrierTimeout)
                    break;
                if (spins > (1u << 24)) {
                    atomicOr(err, kErrBarrierTimeout);
                    break;
                }
            }
        }
    }
    __syncthreads();
}

template <int WT>
__global__ __launch_bounds__(kThreads) void k_persistent(Model m, RunArgs a) {
    __shared__ float lds[kLdsFloats];
    const int wg = blockIdx.x, nwg = gridDim.x;
    unsigned long long bi = a.bar_base;
    auto sync = [&]() { grid_sync(m.bar, ++bi, m.err, wg, nwg); };
    phase_init<WT>(m, a, lds, wg, nwg);
    for (int s = 1; s <= kSteps; ++s) {
        for (int l = 0; l < m.L; ++l) {
            sync();
            phase_qkv<WT>(m, a, s, l, lds, wg, nwg);
            sync();
            phase_attn(m, a, s, l, lds, wg, nwg);
            sync();
            phase_oproj<WT>(m, a, s, l, lds, wg, nwg);
            sync();
            phase_up<WT>(m, a, s, l, lds, wg, nwg);
            sync();
            phase_down<WT>(m, a, s, l, lds, wg, nwg);
        }
        sync();
        phase_lm<WT>(m, a, s, lds, wg, nwg);
        sync();
        phase_next(m, a, s, wg, nwg);
    }
}

template <int WT>
__global__ __launch_bounds__(kThreads) void k_phase(Model m, RunArgs a, int ph, int s, int l) {
    __shared__ float lds[kLdsFloats];
    run_phase<WT>(m, a, ph, s, l, lds, blockIdx.x, gridDim.x);
}

// 32-bit word copy (staging of a frame's inputs and outputs)
__global__ void k_copy32(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst, size_t n) {
    for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        dst[i] = src[i];
}

// Staging of a call's rows into a prepared graph's buffers: the first n
// words are copied, the rest up to n_total (the padding rows of the batch
// bucket) are zeroed, so padded rows compute on valid inputs (H = 0, token 0).
__global__ void k_stage32(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst, size_t n, size_t n_total) {
    for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n_total;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        dst[i] = i < n ? src[i] : 0u;
}

// 64-bit word fill (clearing the dataflow kernel's records)
__global__ void k_fill64(uint64_t* __restrict__ dst, size_t n) {
    for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        dst[i] = 0ull;
}

// --- create-time kernels ----------------------------------------------------

// EMA codebook: E[v][k] = S[v][k] / (u[v] + 1e-7), fp32 add then fp32 divide.
__global__ void k_ema(const float* S, const float* u, float* E, int V, int dT) {
    const size_t n = static_cast<size_t>(V) * dT;
    for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * blockDim.x) {
        const int v = static_cast<int>(i / dT);
        E[i] = S[i] / (u[v] + 1e-7f);
    }
}

__device__ float mat_elem(const Mat& W, int wt, int K, int n, int k) {
    const size_t off = static_cast<size_t>(n) * K + k;
    if (wt == WT_F32) return static_cast<const float*>(W.w)[off];
    if (wt == WT_BF16) return bf16_to_f32(static_cast<const uint16_t*>(W.w)[off]);
    return static_cast<float>(static_cast<const int8_t*>(W.w)[off]) *
           W.scale[static_cast<size_t>(n) * (K / 32) + (k >> 5)];
}

// Projected codebook tables: P[j][v][n] = sum_k W_p[n][k] * E_j[v][k] + b_p[n]
// for j = 0..14 (fp32, 64x64 output tiles, 32-wide k slices through LDS).
__global__ __launch_bounds__(256) void k_ptab(Model m, float* P) {
    __shared__ float As[32][65];  // [k][v]
    __shared__ float Bs[32][65];  // [k][n]
    const int j = blockIdx.z;
    const int v0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < m.dT; k0 += 32) {
        for (int idx = threadIdx.x; idx < 32 * 64; idx += 256) {
            const int kk = idx & 31, rr = idx >> 5;
            const int v = v0 + rr, n = n0 + rr, k = k0 + kk;
            As[kk][rr] = (v < m.V && k < m.dT) ? emb_elem(m, j, v, k) : 0.f;
            Bs[kk][rr] = (n < m.dP && k < m.dT) ? mat_elem(m.proj, m.wt, m.dT, n, k) : 0.f;
        }
        __syncthreads();
        for (int kk = 0; kk < 32; ++kk) {
            float av[4], bv[4];
            for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
            for (int i = 0; i < 4; ++i) bv[i] = Bs[kk][tx * 4 + i];
            for (int i = 0; i < 4; ++i)
                for (int q = 0; q < 4; ++q) acc[i][q] = fmaf(av[i], bv[q], acc[i][q]);
        }
        __syncthreads();
    }
    for (int i = 0; i < 4; ++i) {
        const int v = v0 + ty * 4 + i;
        if (v >= m.V) continue;
        for (int q = 0; q < 4; ++q) {
            const int n = n0 + tx * 4 + q;
            if (n < m.dP) P[(static_cast<size_t>(j) * m.V + v) * m.dP + n] = acc[i][q] + m.proj_b[n];
        }
    }
}

// Layer 0's q/k/v rows for every row of the projected tables P_1 .. P_14:
//   Q0[j-1][v][n] = rsqrt(mean_k P_j[v][k]^2 + eps) * sum_k W_qkv[n][k] g[k] P_j[v][k]
// with g = layer 0's attn_norm (the fused q/k/v projection of the RMSNorm of
// the row; fp32, 64x64 output tiles as in k_ptab).  From step 2 on a
// position's layer-0 input is such a row, chosen by the previous token.
__global__ __launch_bounds__(256) void k_qkv0(Model m, const float* g, float* Q0) {
    __shared__ float As[32][65];  // [k][v]
    __shared__ float Bs[32][65];  // [k][n]
    const int j = blockIdx.z + 1;
    const int v0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const Mat w = m.layers[0].qkv;
    const float* P = m.ptab + static_cast<size_t>(j) * m.V * m.dP;
    float acc[4][4] = {};
    float ss[4] = {};
    for (int k0 = 0; k0 < m.dP; k0 += 32) {
        for (int idx = threadIdx.x; idx < 32 * 64; idx += 256) {
            const int kk = idx & 31, rr = idx >> 5;
            const int v = v0 + rr, n = n0 + rr, k = k0 + kk;
            As[kk][rr] = (v < m.V && k < m.dP) ? P[static_cast<size_t>(v) * m.dP + k] : 0.f;
            Bs[kk][rr] = (n < m.nqkv && k < m.dP) ? mat_elem(w, m.wt, m.dP, n, k) * g[k] : 0.f;
        }
        __syncthreads();
        for (int kk = 0; kk < 32; ++kk) {
            float av[4], bv[4];
            for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
            for (int i = 0; i < 4; ++i) bv[i] = Bs[kk][tx * 4 + i];
            for (int i = 0; i < 4; ++i) {
                ss[i] = fmaf(av[i], av[i], ss[i]);
                for (int q = 0; q < 4; ++q) acc[i][q] = fmaf(av[i], bv[q], acc[i][q]);
            }
        }
        __syncthreads();
    }
    for (int i = 0; i < 4; ++i) {
        const int v = v0 + ty * 4 + i;
        if (v >= m.V) continue;
        const float rinv = 1.0f / sqrtf(ss[i] / static_cast<float>(m.dP) + m.eps);
        for (int q = 0; q < 4; ++q) {
            const int n = n0 + tx * 4 + q;
            if (n < m.nqkv) Q0[(static_cast<size_t>(j - 1) * m.V + v) * m.nqkv + n] = acc[i][q] * rinv;
        }
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// static scratch of qp_run_frames_noalloc
// ---------------------------------------------------------------------------

namespace noalloc {
namespace S = qp::stream;
constexpr int kMaxB = 2;                         // requests the scratch holds
// the dataflow kernel's records (two rows per request) ...
constexpr size_t kRecs = static_cast<size_t>(2 * kMaxB) * (S::DP + S::NQKV + S::QD + S::F) +
                         2ull * S::kNwg * kMaxB;
// ... and its KV cache, [kMaxL][kMaxB][16][NKV][HD] fp32 for keys, then values
constexpr size_t kKV = static_cast<size_t>(S::kMaxL) * kMaxB * kPositions * S::NKV * S::HD;
constexpr size_t kBytes = kRecs * 8 + 2 * kKV * 4;   // 1,646,592 B
static_assert(kRecs * 8 % 256 == 0 && kKV * 4 % 256 == 0, "256-byte aligned parts");
constexpr int kDevices = 64;
}  // namespace noalloc

// One copy per GPU, held until the process ends.  In host code this name is a
// stand-in, not a device address: host code uses the address that
// hipGetSymbolAddress returns for the current device (noalloc_dev below).
static __device__ __align__(256) unsigned char scratch[noalloc::kBytes];

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

struct qp_handle {
    int device = 0;
    int nwg = 0;
    Model m{};
    std::vector<void*> allocs;
    unsigned long long bar_base = 0;
    uint32_t last_flags = 0;
    // dataflow kernel for small batches of the 1.7B predictor geometry
    bool stream_ok = false;
    qp::stream::Recs recs{};
    size_t nrecs = 0;   // records in the allocation at recs.X
    uint32_t seq = 0;
    // dataflow kernel with matrix-core products for 3 <= B <= 16 (1.7B
    // geometry, bf16 weights)
    bool flow_ok = false;
    qp::flow::Recs frecs{};
    uint64_t* frec_base = nullptr;
    uint32_t fseq = 0;
    // batched matrix-core path
    bool tiled_ok = false;
    bool q4 = false;   // Q4_0 weights: 4-bit fragments on the batched path
    std::vector<LayerDev> layers_host;
    qp::tiled::FMat t_proj{};
    std::vector<qp::tiled::FMat> t_qkv, t_o, t_gate, t_up, t_down;
    qp::tiled::FMat t_lm[kSteps]{};
    unsigned long long* t_keys = nullptr;   // [max_batch][V/16] per-tile argmax keys
    float* t_part = nullptr;                // split-K partial tiles
    size_t t_part_floats = 0;
    unsigned* t_ctr = nullptr;              // split-K tile counters
    size_t t_nctr = 0;
    // one frame of the batched path captured as a graph per batch bucket
    // (greedy, and sampled where the handle can sample), all built by
    // qp_create and kept until qp_destroy; each reads and writes handle-owned
    // staging buffers, and a call with B rows replays the smallest bucket
    // that holds them, its extra rows zero-padded
    struct FrameGraph {
        int B = 0;
        bool sampled = false;
        hipGraph_t graph = nullptr;
        hipGraphExec_t exec = nullptr;
    };
    std::vector<FrameGraph> graphs;
    hipStream_t cap_stream = nullptr;
    float* st_H = nullptr;                  // [max_batch][dT]
    int* st_q0 = nullptr;                   // [max_batch]
    int* st_tok = nullptr;                  // [max_batch][15]
    float* st_emb = nullptr;                // [max_batch][dT]
    uint16_t* t_xg = nullptr;               // bf16(g_next * x), 2*max_batch rows (rounded up to 16) of width dP, fragment order
    float* t_ss = nullptr;                  // [2*max_batch][dP/16] 16-column sums of x^2
    // sampled frames (batched path, V <= 4096)
    bool sample_ok = false;
    float* t_logits = nullptr;              // [max_batch][V] one step's logits
    int* t_sampled = nullptr;               // [max_batch] one step's drawn tokens
    float* st_u = nullptr;                  // [max_batch][15] staged uniforms
    qp::sample::Params* st_samp = nullptr;  // the call's sampling parameters
};

namespace {

thread_local std::string g_last_error;

// QP_LOG set (to anything) in the environment: every failure is also
// written to stderr, one line each
bool log_failures() {
    static const bool on = std::getenv("QP_LOG") != nullptr;
    return on;
}

qp_status fail(qp_status st, const std::string& msg) {
    g_last_error = msg;
    if (log_failures()) std::fprintf(stderr, "qp: %s (%s)\n", msg.c_str(), qp_status_string(st));
    return st;
}

struct DeviceGuard {
    int prev = -1;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        (void)hipSetDevice(dev);
    }
    ~DeviceGuard() {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

float half_to_float(uint16_t h) {
    const uint32_t sign = (h & 0x8000u) << 16;
    const uint32_t exp = (h >> 10) & 0x1Fu;
    const uint32_t man = h & 0x3FFu;
    float f;
    if (exp == 0) {
        f = std::ldexp(static_cast<float>(man), -24);  // zero or subnormal
    } else if (exp == 31) {
        uint32_t bits = 0x7F800000u | (man << 13);
        std::memcpy(&f, &bits, 4);
    } else {
        uint32_t bits = ((exp + 112u) << 23) | (man << 13);
        std::memcpy(&f, &bits, 4);
    }
    uint32_t b;
    std::memcpy(&b, &f, 4);
    b |= sign;
    std::memcpy(&f, &b, 4);
    return f;
}

struct Uploader {
    std::vector<void*>* allocs;   // the owning handle's allocation list
    qp_status st = QP_OK;
    std::string msg;

    void* alloc(size_t bytes) {
        if (st != QP_OK) return nullptr;
        void* p = nullptr;
        if (bytes == 0) bytes = 4;
        if (hipMalloc(&p, bytes) != hipSuccess) {
            st = QP_ERR_OOM;
            msg = "hipMalloc of " + std::to_string(bytes) + " bytes failed";
            (void)hipGetLastError();
            return nullptr;
        }
        allocs->push_back(p);
        return p;
    }
    void* upload(const void* src, size_t bytes) {
        void* p = alloc(bytes);
        if (!p) return nullptr;
        if (hipMemcpy(p, src, bytes, hipMemcpyHostToDevice) != hipSuccess) {
            st = QP_ERR_HIP;
            msg = "hipMemcpy to device failed";
            return nullptr;
        }
        return p;
    }
    // A matrix on the host in row-major storage: f32 / bf16 elements, or the
    // Q8_0 rows split into int8 codes [N][K] and fp32 block scales [N][K/32].
    struct HostMat {
        std::vector<uint8_t> w;
        std::vector<float> scale;
        size_t N = 0;
        int K = 0, wt = 0;
    };
    // Vertically stack matrices [N_i][K] of one storage type.
    static HostMat build(const std::vector<const void*>& parts, const std::vector<int>& rows, int K, int wt) {
        HostMat hm;
        hm.K = K;
        hm.wt = wt;
        for (int r : rows) hm.N += static_cast<size_t>(r);
        if (wt == WT_F32 || wt == WT_BF16) {
            const size_t esz = wt == WT_F32 ? 4 : 2;
            hm.w.resize(hm.N * K * esz);
            size_t off = 0;
            for (size_t i = 0; i < parts.size(); ++i) {
                const size_t nb = static_cast<size_t>(rows[i]) * K * esz;
                std::memcpy(hm.w.data() + off, parts[i], nb);
                off += nb;
            }
            return hm;
        }
        // Q8_0 / Q4_0: int8 codes (Q4_0: code - 8) and fp32 block scales
        const int nb = K / 32;
        const size_t bbytes = wt == WT_Q4 ? 18 : 34;
        hm.w.resize(hm.N * K);
        hm.scale.resize(hm.N * nb);
        size_t row = 0;
        for (size_t i = 0; i < parts.size(); ++i) {
            const uint8_t* src = static_cast<const uint8_t*>(parts[i]);
            for (int r = 0; r < rows[i]; ++r, ++row) {
                const uint8_t* rp = src + static_cast<size_t>(r) * nb * bbytes;
                for (int bk = 0; bk < nb; ++bk) {
                    const uint8_t* blk = rp + static_cast<size_t>(bk) * bbytes;
                    hm.scale[row * nb + bk] = half_to_float(static_cast<uint16_t>(blk[0] | (blk[1] << 8)));
                    int8_t* dst = reinterpret_cast<int8_t*>(&hm.w[row * K + static_cast<size_t>(bk) * 32]);
                    if (wt == WT_Q4) {
                        for (int j = 0; j < 16; ++j) {
                            dst[j] = static_cast<int8_t>((blk[2 + j] & 15) - 8);
                            dst[j + 16] = static_cast<int8_t>((blk[2 + j] >> 4) - 8);
                        }
                    } else {
                        std::memcpy(dst, blk + 2, 32);
                    }
                }
            }
        }
        return hm;
    }
    // Row-major device copy (Q4_0 as int8 codes with block scales, i.e. the
    // Q8_0 layout)
    Mat rowmajor(const HostMat& hm) {
        Mat out{nullptr, nullptr};
        out.w = upload(hm.w.data(), hm.w.size());
        if (hm.wt == WT_Q8 || hm.wt == WT_Q4)
            out.scale = static_cast<const float*>(upload(hm.scale.data(), hm.scale.size() * 4));
        return out;
    }
    // MFMA fragment order: fragment (n/16, k/32) holds, for lane
    // l = (n % 16) + 16 * ((k % 32) / 8), the 8 elements k .. k+7 of row n
    // (bf16: 16 bytes; Q8_0: 8 int8 codes; Q4_0: 8 codes + 8 as nibbles of
    // one 32-bit word, element k + i in bits 4i .. 4i+3).
    qp::tiled::FMat fragments(const HostMat& hm) {
        qp::tiled::FMat out{nullptr, nullptr};
        const size_t N = hm.N, K = static_cast<size_t>(hm.K), KB = K / 32;
        const size_t esz = hm.wt == WT_BF16 ? 2 : 1;
        const size_t chunk = hm.wt == WT_BF16 ? 16 : (hm.wt == WT_Q8 ? 8 : 4);
        std::vector<uint8_t> f(N / 16 * KB * 64 * chunk);
        for (size_t nb = 0; nb < N / 16; ++nb)
            for (size_t kb = 0; kb < KB; ++kb)
                for (size_t lane = 0; lane < 64; ++lane) {
                    const size_t n = nb * 16 + (lane & 15), k = kb * 32 + (lane >> 4) * 8;
                    uint8_t* dst = &f[((nb * KB + kb) * 64 + lane) * chunk];
                    if (hm.wt == WT_Q4) {
                        uint32_t word = 0;
                        for (int i = 0; i < 8; ++i)
                            word |= static_cast<uint32_t>((static_cast<int8_t>(hm.w[n * K + k + i]) + 8) & 15) << (4 * i);
                        std::memcpy(dst, &word, 4);
                    } else {
                        std::memcpy(dst, &hm.w[(n * K + k) * esz], 8 * esz);
                    }
                }
        out.w = upload(f.data(), f.size());
        if (hm.wt == WT_Q8 || hm.wt == WT_Q4) {
            std::vector<float> sc(hm.scale.size());
            for (size_t nb = 0; nb < N / 16; ++nb)
                for (size_t kb = 0; kb < KB; ++kb)
                    for (size_t r = 0; r < 16; ++r) sc[(nb * KB + kb) * 16 + r] = hm.scale[(nb * 16 + r) * KB + kb];
            out.scale = static_cast<const float*>(upload(sc.data(), sc.size() * 4));
        }
        return out;
    }
    Mat stack(const std::vector<const void*>& parts, const std::vector<int>& rows, int K, int wt) {
        return rowmajor(build(parts, rows, K, wt));
    }
    Mat one(const void* p, int N, int K, int wt) { return stack({p}, {N}, K, wt); }
};

bool check_hip(hipError_t e, const char* what, qp_status* st) {
    if (e == hipSuccess) return true;
    *st = fail(QP_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
    return false;
}

qp_status validate_geometry(const qp_geometry* g) {
    if (g->n_codebooks != QP_N_CODEBOOKS)
        return fail(QP_ERR_GEOMETRY, "n_codebooks must be 16");
    if (g->d_talker <= 0 || g->d_model <= 0 || g->n_layers < 0 || g->n_q_heads <= 0 ||
        g->n_kv_heads <= 0 || g->head_dim <= 0 || g->d_ffn <= 0 || g->vocab <= 0)
        return fail(QP_ERR_GEOMETRY, "every dimension must be positive (n_layers >= 0)");
    if (g->n_layers > 256) return fail(QP_ERR_GEOMETRY, "n_layers above 256");
    if (g->n_q_heads % g->n_kv_heads != 0)
        return fail(QP_ERR_GEOMETRY, "n_q_heads must be a multiple of n_kv_heads");
    if (g->head_dim != 64 && g->head_dim != 128 && g->head_dim != 256)
        return fail(QP_ERR_GEOMETRY, "head_dim must be 64, 128 or 256");
    if (!(g->rms_eps > 0.f) || !(g->rope_base > 0.f) || !std::isfinite(g->rope_base))
        return fail(QP_ERR_GEOMETRY, "rms_eps and rope_base must be positive");
    if (g->max_batch < 1 || g->max_batch > 65536)
        return fail(QP_ERR_GEOMETRY, "max_batch must be in [1, 65536]");
    if (g->weight_dtype < QP_WEIGHT_F32 || g->weight_dtype > QP_WEIGHT_Q4_0)
        return fail(QP_ERR_DTYPE, "unknown weight_dtype");
    if (g->emb_format < QP_EMB_F32 || g->emb_format > QP_EMB_EMA)
        return fail(QP_ERR_DTYPE, "unknown emb_format");
    const int qd = g->n_q_heads * g->head_dim;
    const int ins[4] = {g->d_talker, g->d_model, qd, g->d_ffn};
    const int align = (g->weight_dtype == QP_WEIGHT_Q8_0 || g->weight_dtype == QP_WEIGHT_Q4_0) ? 32 : 8;
    for (int k : ins) {
        if (k % align != 0)
            return fail(QP_ERR_SHAPE, "every input width (dT, dP, nq*hd, F) must be a multiple of " +
                                          std::to_string(align) + " for this weight dtype");
        if (k > kLdsFloats) return fail(QP_ERR_SHAPE, "an input width exceeds 16384");
    }
    return QP_OK;
}

qp_status validate_weights(const qp_weights* w, const qp_geometry* g) {
    if (!w->proj_w || !w->proj_b || !w->out_norm) return fail(QP_ERR_INVALID_ARG, "NULL projection/out_norm");
    for (int j = 0; j < QP_N_CODEBOOKS; ++j) {
        if (g->emb_format == QP_EMB_EMA) {
            if (!w->ema_sum[j] || !w->ema_usage[j]) return fail(QP_ERR_INVALID_ARG, "NULL EMA table");
        } else if (!w->emb[j]) {
            return fail(QP_ERR_INVALID_ARG, "NULL codebook table");
        }
    }
    for (int k = 0; k < QP_N_STEPS; ++k)
        if (!w->lm_head[k]) return fail(QP_ERR_INVALID_ARG, "NULL lm_head");
    if (g->n_layers > 0 && !w->layers) return fail(QP_ERR_INVALID_ARG, "NULL layers");
    for (int l = 0; l < g->n_layers; ++l) {
        const qp_layer_weights& L = w->layers[l];
        if (!L.attn_norm || !L.wq || !L.wk || !L.wv || !L.wo || !L.q_norm || !L.k_norm || !L.ffn_norm ||
            !L.w_gate || !L.w_up || !L.w_down)
            return fail(QP_ERR_INVALID_ARG, "NULL tensor in layer " + std::to_string(l));
    }
    return QP_OK;
}

void free_all(qp_handle* h) {
    for (void* p : h->allocs) (void)hipFree(p);
    h->allocs.clear();
}

// Per-device state of the static scratch: its device address (from
// hipGetSymbolAddress with that device current), and the next record tag of
// the dataflow frames that run on it (shared by every call on the device, so
// no stale record can carry a current tag).
struct NoallocDev {
    uint64_t* base = nullptr;
    uint32_t seq = 0;
};
std::mutex g_noalloc_mu;
NoallocDev g_noalloc[noalloc::kDevices];

// Once per device, with the device current (qp_create): look up the scratch's
// address and clear its records (tag 0 is never current; the KV part needs no
// clearing, a frame writes every position before reading it).
qp_status noalloc_setup(int device) {
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    if (device < 0 || device >= noalloc::kDevices) return QP_OK;   // the entry point rejects such devices
    NoallocDev& d = g_noalloc[device];
    if (d.base) return QP_OK;
    void* ptr = nullptr;
    qp_status st = QP_OK;
    if (!check_hip(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress (static scratch)", &st))
        return st;
    hipLaunchKernelGGL(k_fill64, dim3(64), dim3(256), 0, 0, static_cast<uint64_t*>(ptr), noalloc::kRecs);
    if (!check_hip(hipGetLastError(), "static scratch clear", &st) ||
        !check_hip(hipDeviceSynchronize(), "static scratch clear", &st))
        return st;
    d.base = static_cast<uint64_t*>(ptr);
    d.seq = 0;
    return QP_OK;
}

// Wait for the device (no replay of the handle's graphs is in flight after
// that), free the graphs, the capture stream and every buffer, and the handle.
void destroy_handle(qp_handle* h) {
    {
        DeviceGuard guard(h->device);
        (void)hipDeviceSynchronize();
        for (auto& e : h->graphs) {
            if (e.exec) (void)hipGraphExecDestroy(e.exec);
            if (e.graph) (void)hipGraphDestroy(e.graph);
        }
        h->graphs.clear();
        if (h->cap_stream) (void)hipStreamDestroy(h->cap_stream);
        h->cap_stream = nullptr;
        free_all(h);
    }
    delete h;
}

}  // namespace

namespace {

// --- batched matrix-core path ---------------------------------------------

// Launch indices of a frame's kernels for the timeline build (QP_TSTAMP):
// launch_tiled numbers its launches from 0 in order and records each one's
// role; every other build numbers nothing.  Host-side state of that
// measurement build only, not safe for concurrent captures.
enum TlKind : int { TL_PROJ = 1, TL_QKV, TL_ATTN, TL_ATTN_TOK, TL_O, TL_SWIGLU, TL_DOWN, TL_LM, TL_START, TL_NEXT };
#ifdef QP_TIMELINE
int g_tl_next = 0;
int g_tl_kind[qp::kTiledLaunches];
void tl_reset() { g_tl_next = 0; }
int tl_index(int kind) {
    const int i = g_tl_next++;
    if (i < qp::kTiledLaunches) g_tl_kind[i] = kind;
    return i;
}
#else
void tl_reset() {}
int tl_index(int) { return -1; }
#endif

// Launches one product; returns the number of column tiles (gridDim.x).
// h: any handle with the split-K scratch (t_part, t_part_floats, t_ctr, t_nctr).
template <int WT, int SRC, int EPI, class Handle>
int tiled_gemm(const Handle* h, qp::tiled::GemmArgs g, hipStream_t stream) {
    namespace T = qp::tiled;
    // one 16-row tile per workgroup up to 32 rows (more workgroups per CU to
    // cover memory latency; the weights are re-read from L2 per row tile),
    // two above (measured: B = 64 Q8_0 +27 %, B = 128 bf16 +11 % over tiles
    // of up to 64 rows; B = 64 Q8_0 +1.5 % over one row tile up to 64 rows).
    // Residual products (N = dP) keep one row tile at any M: with two they
    // need the split-K fixup to fill the chip, and its extra round trips cost
    // more (B = 128 bf16: 4.15 against 4.29 ms per frame-batch; one row tile
    // for the other products was slower).  SwiGLU keeps one row tile up to
    // 64 rows (with fragment-ordered operands: B = 64 Q8_0 +3 %, no change
    // at 128 rows)
    const int RT = (g.M <= 32 || EPI == T::EPI_RESID || (EPI == T::EPI_SWIGLU && g.M <= 64)) ? 1 : 2;
    // one row tile: one 16-column fragment per workgroup (twice the
    // workgroups streaming weights); SwiGLU always pairs gate and up
    const int CT = (RT == 1 && EPI != T::EPI_SWIGLU) ? 1 : 2;
    const int gx = EPI == T::EPI_SWIGLU ? g.N / 16 : g.N / (16 * CT);
    const int gy = (g.M + 16 * RT - 1) / (16 * RT);
    // The projection of H (N = dP, few output tiles) with more than one row
    // tile also splits K over workgroups: the smallest split (into whole
    // pairs of 32-wide blocks per wave, at most 4) that fills 256 workgroups.
    // With a single row tile the ordered fixup costs more than it saves.
    const int tiles = gx * gy;
    int KS = 1;
    if (EPI == T::EPI_BIAS && RT > 1 && tiles < 256 && static_cast<size_t>(tiles) <= h->t_nctr) {
        for (int c = 2; c <= T::kMaxKS; ++c) {
            // whole pairs of 32-wide blocks for each of the 4 waves
            if ((g.K / 256) % c != 0) continue;
            if (static_cast<size_t>(c) * tiles * RT * CT * 256 > h->t_part_floats) break;
            KS = c;
            if (c * tiles >= 256) break;
        }
    }
    g.KS = KS;
    g.part = h->t_part;
    g.part_bytes = static_cast<uint32_t>(h->t_part_floats * 4);
    g.ctr = h->t_ctr;
    // Workgroups go to the 8 XCDs round-robin by linear id x + gx (y + gy z).
    // With gx a multiple of 8 (every product of the 1.7B predictor and the
    // Talker: gx = N/16 or N/32 with N a multiple of 256), every row tile and
    // K split of column tile x runs on XCD x mod 8, so each weight slice is
    // fetched into one XCD's L2 only; the activation rows, read by all, are
    // small.
    const dim3 grid(gx, gy, KS);
    if (RT == 1) {
        // up to 16 rows there is little work per output: 8 waves per
        // workgroup keep twice the weight bytes in flight where K splits into
        // 16 pairs of blocks (M = 1: 5 % faster per Talker step than 4 waves,
        // from the residual products).  Above 16 rows 4 waves are faster
        // (M = 64 Q8_0: 3.5 % per frame-batch), and so is SwiGLU, whose
        // workgroups read two fragments, at any M (B = 16: 0.5 %).
        const bool w8 = EPI != T::EPI_SWIGLU && g.M <= 16 && (g.K / 32) % 16 == 0;
        constexpr int C1 = EPI == T::EPI_SWIGLU ? 2 : 1;
        if (w8)
            hipLaunchKernelGGL((T::k_gemm<WT, 1, SRC, EPI, 8, C1>), grid, dim3(512), 0, stream, g);
        else
            hipLaunchKernelGGL((T::k_gemm<WT, 1, SRC, EPI, 4, C1>), grid, dim3(256), 0, stream, g);
    } else {
        hipLaunchKernelGGL((T::k_gemm<WT, 2, SRC, EPI, 4, 2>), grid, dim3(256), 0, stream, g);
    }
    return gx;
}

template <int WT>
qp_status launch_tiled(qp_handle* h, const RunArgs& a, hipStream_t stream) {
    namespace T = qp::tiled;
    qp_status st = QP_OK;
    const Model& m = h->m;
    const int B = a.B, qd = m.nq * m.hd, nss = m.dP / 16;
    const int nb = B < 1024 ? B : 1024;
    // the gain of the first reader of a position's input row
    const float* gain0 = m.L > 0 ? h->layers_host[0].attn_norm : m.out_norm;
    // the bf16 activations' layout for this batch (qp_tiled.h, act_index)
    const int frag = B >= T::kFragMinRows ? 1 : 0;
    T::TokArgs ta{};
    ta.B = B;
    ta.frag = frag;
    ta.dT = m.dT;
    ta.dP = m.dP;
    ta.V = m.V;
    ta.emb_bf16 = m.emb_bf16;
    ta.q0 = a.q0;
    ta.force = a.force;
    ta.tok_out = a.tok_out;
    ta.embsum = a.embsum;
    ta.keys = h->t_keys;
    ta.x = m.x;
    ta.xg = h->t_xg;
    ta.ss = h->t_ss;
    ta.gain0 = gain0;
    ta.err = m.err;
    ta.emb = m.emb[0];
    ta.ptab = m.ptab;
    ta.qkv = m.qkv;
    ta.nqkv = m.nqkv;
    tl_reset();
    ta.tl = tl_index(TL_START);
    hipLaunchKernelGGL(T::k_start, dim3(nb), dim3(T::kThreadsT), 0, stream, ta);
    ta.tl = -1;
    T::AttnArgs aa{};
    aa.B = B;
    aa.frag = frag;
    aa.nq = m.nq;
    aa.nkv = m.nkv;
    aa.nqkv = m.nqkv;
    aa.max_batch = m.max_batch;
    aa.eps = m.eps;
    aa.attn_scale = m.attn_scale;
    aa.qkv = m.qkv;
    aa.kc = m.kc;
    aa.vc = m.vc;
    aa.rope_cos = m.rope_cos;
    aa.rope_sin = m.rope_sin;
    T::GemmArgs g{};
    g.eps = m.eps;
    g.frag = frag;
    // x[position 0] = W_p . H + b_p
    g.a = a.H;
    g.lda = m.dT;
    g.M = B;
    g.N = m.dP;
    g.K = m.dT;
    g.w0 = h->t_proj;
    g.out = m.x;
    g.ldo = m.dP;
    g.bias = m.proj_b;
    g.xg = h->t_xg;
    g.g_next = gain0;
    g.ss_out = h->t_ss;
    g.tl = tl_index(TL_PROJ);
    tiled_gemm<WT, T::SRC_F32, T::EPI_BIAS>(h, g, stream);
    uint16_t* ao = reinterpret_cast<uint16_t*>(m.ao);
    uint16_t* hb = reinterpret_cast<uint16_t*>(m.hb);
    for (int s = 1; s <= kSteps; ++s) {
        const int M = s == 1 ? 2 * B : B;
        for (int l = 0; l < m.L; ++l) {
            const LayerDev& L = h->layers_host[l];
            const float* g_after = l + 1 < m.L ? h->layers_host[l + 1].attn_norm : m.out_norm;
            // q, k, v = W_qkv . RMSNorm(x); from step 2 on, with the layer-0
            // table, k_next has already copied layer 0's rows
            if (l > 0 || s == 1 || !m.qkv0) {
                g = T::GemmArgs{};
                g.eps = m.eps;
                g.frag = frag;
                g.M = M;
                g.a = h->t_xg;
                g.lda = m.dP;
                g.ss_in = h->t_ss;
                g.nss = nss;
                g.N = m.nqkv;
                g.K = m.dP;
                g.w0 = h->t_qkv[l];
                g.out = m.qkv;
                g.ldo = m.nqkv;
                g.tl = tl_index(TL_QKV);
                tiled_gemm<WT, T::SRC_BF16_NORM, T::EPI_SCALE>(h, g, stream);
            }
            // attention (layer 0 from step 2 on, with the table: also the
            // previous step's token decision, handed over below)
            aa.s = s;
            aa.l = l;
            aa.tok_on = (l == 0 && s > 1 && m.qkv0) ? 1 : 0;
            aa.tl = tl_index(aa.tok_on ? TL_ATTN_TOK : TL_ATTN);
            aa.k_norm = L.k_norm;
            aa.q_norm = L.q_norm;
            aa.ao = ao;
            const dim3 ag(B * m.nkv);
            if (aa.tok_on) {
                switch (m.hd) {
                    case 64: hipLaunchKernelGGL((T::k_attn<64, true>), ag, dim3(T::kThreadsT), 0, stream, aa); break;
                    case 128: hipLaunchKernelGGL((T::k_attn<128, true>), ag, dim3(T::kThreadsT), 0, stream, aa); break;
                    default: hipLaunchKernelGGL((T::k_attn<256, true>), ag, dim3(T::kThreadsT), 0, stream, aa); break;
                }
            } else {
                switch (m.hd) {
                    case 64: hipLaunchKernelGGL((T::k_attn<64, false>), ag, dim3(T::kThreadsT), 0, stream, aa); break;
                    case 128: hipLaunchKernelGGL((T::k_attn<128, false>), ag, dim3(T::kThreadsT), 0, stream, aa); break;
                    default: hipLaunchKernelGGL((T::k_attn<256, false>), ag, dim3(T::kThreadsT), 0, stream, aa); break;
                }
            }
            // x += W_o . attention; publishes bf16(ffn_norm * x)
            g = T::GemmArgs{};
            g.eps = m.eps;
            g.frag = frag;
            g.M = M;
            g.a = ao;
            g.lda = qd;
            g.N = m.dP;
            g.K = qd;
            g.w0 = h->t_o[l];
            g.out = m.x;
            g.ldo = m.dP;
            g.xg = h->t_xg;
            g.g_next = L.ffn_norm;
            g.ss_out = h->t_ss;
            g.tl = tl_index(TL_O);
            tiled_gemm<WT, T::SRC_BF16, T::EPI_RESID>(h, g, stream);
            // h = silu(W_g . RMSNorm(x)) * (W_u . RMSNorm(x)), bf16
            g = T::GemmArgs{};
            g.eps = m.eps;
            g.frag = frag;
            g.M = M;
            g.a = h->t_xg;
            g.lda = m.dP;
            g.ss_in = h->t_ss;
            g.nss = nss;
            g.N = m.F;
            g.K = m.dP;
            g.w0 = h->t_gate[l];
            g.w1 = h->t_up[l];
            g.outb = hb;
            g.tl = tl_index(TL_SWIGLU);
            tiled_gemm<WT, T::SRC_BF16_NORM, T::EPI_SWIGLU>(h, g, stream);
            // x += W_d . h (and the residual tap); publishes the next reader's operand
            g = T::GemmArgs{};
            g.eps = m.eps;
            g.frag = frag;
            g.M = M;
            g.a = hb;
            g.lda = m.F;
            g.N = m.dP;
            g.K = m.F;
            g.w0 = h->t_down[l];
            g.out = m.x;
            g.ldo = m.dP;
            g.xg = h->t_xg;
            g.g_next = g_after;
            g.ss_out = h->t_ss;
            g.taps = a.taps;
            g.tap_s = s;
            g.tap_l = l;
            g.tap_L = m.L;
            g.tap_B = B;
            g.tl = tl_index(TL_DOWN);
            tiled_gemm<WT, T::SRC_BF16, T::EPI_RESID>(h, g, stream);
        }
        // lm_head[s-1] . RMSNorm(x at position s) -> per-tile argmax keys
        const size_t row0 = s == 1 ? static_cast<size_t>(B) : 0;
        g = T::GemmArgs{};
        g.eps = m.eps;
        g.frag = frag;
        g.a = h->t_xg;
        g.a_row0 = static_cast<int>(row0);
        g.lda = m.dP;
        g.ss_in = h->t_ss + row0 * nss;
        g.nss = nss;
        g.M = B;
        g.N = m.V;
        g.K = m.dP;
        g.w0 = h->t_lm[s - 1];
        g.keys = h->t_keys;
        if (a.logits_out) {
            g.logits = a.logits_out + static_cast<size_t>(s - 1) * m.V;
            g.logit_ld = static_cast<size_t>(kSteps) * m.V;
        } else if (a.uniforms) {
            g.logits = h->t_logits;
            g.logit_ld = m.V;
        }
        g.tl = tl_index(TL_LM);
        ta.nkt = tiled_gemm<WT, T::SRC_BF16_NORM, T::EPI_ARGMAX>(h, g, stream);
        if (a.uniforms) {
            // the step's token drawn from its logits with the caller's uniform
            hipLaunchKernelGGL(qp::sample::sample_kernel(m.V), dim3(B), dim3(qp::sample::kThreadsSm), 0, stream, g.logits,
                               static_cast<long long>(g.logit_ld), m.V, qp::sample::Params{}, h->st_samp,
                               a.uniforms + (s - 1), kSteps, h->t_sampled);
            ta.sampled = h->t_sampled;
        }
        ta.s = s;
        ta.emb = m.emb[s];
        ta.ptab = s < kSteps ? m.ptab + static_cast<size_t>(s) * m.V * m.dP : nullptr;
        ta.qkv0 = s < kSteps && m.qkv0 ? m.qkv0 + static_cast<size_t>(s - 1) * m.V * m.nqkv : nullptr;
        if (ta.qkv0) {
            // the next step's layer-0 attention decides this step's token and
            // reads its q/k/v rows from the table: no k_next launch
            aa.tok = ta;
        } else {
            ta.tl = tl_index(TL_NEXT);
            hipLaunchKernelGGL(T::k_next, dim3(nb), dim3(T::kThreadsT), 0, stream, ta);
            ta.tl = -1;
        }
    }
    if (!check_hip(hipGetLastError(), "batched path kernel launch", &st)) return st;
    return QP_OK;
}

void copy32(const void* src, void* dst, size_t words, hipStream_t stream) {
    const int blocks = static_cast<int>(std::min<size_t>((words + 255) / 256, 1024));
    hipLaunchKernelGGL(k_copy32, dim3(blocks), dim3(256), 0, stream, static_cast<const uint32_t*>(src),
                       static_cast<uint32_t*>(dst), words);
}

// Row buckets of the prepared graphs: 1, 2, 4, 8, 16, 32, then 48, 64, 96,
// 128, 192, 256, ... (alternately x1.5 and x4/3, so every bucket above 16 is
// a whole number of 16-row tiles), those below max_batch, and max_batch.
std::vector<int> batch_buckets(int max_batch) {
    std::vector<int> b;
    for (int v = 1; v < max_batch;) {
        b.push_back(v);
        if (v < 32) v *= 2;
        else v = (v & (v - 1)) == 0 ? v + v / 2 : (v / 3) * 4;
    }
    b.push_back(max_batch);
    return b;
}

void stage32(const void* src, void* dst, size_t words, size_t total, hipStream_t stream) {
    const int blocks = static_cast<int>(std::min<size_t>((total + 255) / 256, 1024));
    hipLaunchKernelGGL(k_stage32, dim3(blocks), dim3(256), 0, stream, static_cast<const uint32_t*>(src),
                       static_cast<uint32_t*>(dst), words, total);
}

// Capture one frame of bucket Bk (greedy or sampled) on the handle's capture
// stream and instantiate it; the graph reads and writes the staging buffers.
// Nothing in it clears memory with a memset node: the split-K counters are
// left at zero by the kernels themselves.
template <int WT>
qp_status capture_tiled_graph(qp_handle* h, int Bk, bool sampled) {
    qp_status st = QP_OK;
    RunArgs sa{};
    sa.B = Bk;
    sa.H = h->st_H;
    sa.q0 = h->st_q0;
    sa.tok_out = h->st_tok;
    sa.embsum = h->st_emb;
    sa.uniforms = sampled ? h->st_u : nullptr;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    if (!check_hip(hipStreamBeginCapture(h->cap_stream, hipStreamCaptureModeThreadLocal), "hipStreamBeginCapture", &st))
        return st;
    const qp_status lst = launch_tiled<WT>(h, sa, h->cap_stream);
    const hipError_t ce = hipStreamEndCapture(h->cap_stream, &graph);
    if (lst != QP_OK) {
        if (graph) (void)hipGraphDestroy(graph);
        return lst;
    }
    if (!check_hip(ce, "hipStreamEndCapture", &st)) return st;
    if (!check_hip(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0), "hipGraphInstantiate", &st)) {
        (void)hipGraphDestroy(graph);
        return st;
    }
    qp_handle::FrameGraph fg;
    fg.B = Bk;
    fg.sampled = sampled;
    fg.graph = graph;
    fg.exec = exec;
    h->graphs.push_back(fg);
    return QP_OK;
}

// All graphs of a handle (qp_create, after the tables are built).
qp_status prepare_tiled_graphs(qp_handle* h) {
    qp_status st = QP_OK;
    if (!check_hip(hipStreamCreateWithFlags(&h->cap_stream, hipStreamNonBlocking), "hipStreamCreate", &st)) return st;
    for (int Bk : batch_buckets(h->m.max_batch)) {
        for (int sampled = 0; sampled < (h->sample_ok ? 2 : 1); ++sampled) {
            if (h->m.wt == WT_BF16) st = capture_tiled_graph<WT_BF16>(h, Bk, sampled != 0);
            else if (h->q4) st = capture_tiled_graph<WT_Q4>(h, Bk, sampled != 0);
            else st = capture_tiled_graph<WT_Q8>(h, Bk, sampled != 0);
            if (st != QP_OK) return st;
        }
    }
    return QP_OK;
}

// The batched path without test hooks: the call's inputs are staged into the
// handle's buffers (rows past B up to the bucket zeroed), the bucket's
// prepared graph replays the frame (about 400 kernels), and B rows of the
// outputs are copied back.  Nothing is captured, instantiated or freed here.
qp_status launch_tiled_graph(qp_handle* h, const RunArgs& a, hipStream_t stream) {
    qp_status st = QP_OK;
    const Model& m = h->m;
    const int B = a.B;
    const bool sampled = a.uniforms != nullptr;
    const qp_handle::FrameGraph* fg = nullptr;
    for (const auto& e : h->graphs)
        if (e.sampled == sampled && e.B >= B && (!fg || e.B < fg->B)) fg = &e;
    if (!fg) return fail(QP_ERR_HIP, "no prepared graph for B=" + std::to_string(B));
    const size_t Bk = static_cast<size_t>(fg->B);
    stage32(a.H, h->st_H, static_cast<size_t>(B) * m.dT, Bk * m.dT, stream);
    stage32(a.q0, h->st_q0, static_cast<size_t>(B), Bk, stream);
    if (sampled) stage32(a.uniforms, h->st_u, static_cast<size_t>(B) * kSteps, Bk * kSteps, stream);
    if (!check_hip(hipGraphLaunch(fg->exec, stream), "hipGraphLaunch", &st)) return st;
    copy32(h->st_tok, a.tok_out, static_cast<size_t>(B) * kSteps, stream);
    copy32(h->st_emb, a.embsum, static_cast<size_t>(B) * m.dT, stream);
    if (!check_hip(hipGetLastError(), "staging copy launch", &st)) return st;
    return QP_OK;
}

// The moderate-batch dataflow kernel: one cooperative launch per frame.
qp_status launch_flow(qp_handle* h, const RunArgs& a, hipStream_t stream) {
    namespace FL = qp::flow;
    qp_status st = QP_OK;
    const Model& m = h->m;
    const uint32_t ppf = static_cast<uint32_t>(FL::phases_per_frame(m.L));
    if (h->fseq > 0xFFFFFFFFu - 2u * ppf) {
        // the 32-bit phase tags would wrap: clear every record (tag 0 is never
        // current) so that no record left from long ago can match a new tag
        hipLaunchKernelGGL(k_fill64, dim3(64), dim3(256), 0, stream, h->frec_base, FL::kRecsTotal);
        if (!check_hip(hipGetLastError(), "record clear", &st)) return st;
        h->fseq = 0;
    }
    FL::FArgs fa{};
    for (int l = 0; l < m.L; ++l) {
        fa.lay[l].qkv = static_cast<const uint8_t*>(h->t_qkv[l].w);
        fa.lay[l].o = static_cast<const uint8_t*>(h->t_o[l].w);
        fa.lay[l].gate = static_cast<const uint8_t*>(h->t_gate[l].w);
        fa.lay[l].up = static_cast<const uint8_t*>(h->t_up[l].w);
        fa.lay[l].down = static_cast<const uint8_t*>(h->t_down[l].w);
    }
    fa.proj = static_cast<const uint8_t*>(h->t_proj.w);
    for (int k = 0; k < kSteps; ++k) fa.lm[k] = static_cast<const uint8_t*>(h->t_lm[k].w);
    RunArgs ra = a;
    ra.seq0 = h->fseq;
    Model mm = m;
    FL::Recs rc = h->frecs;
    void* args[] = {&mm, &ra, &rc, &fa};
    if (!check_hip(hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&FL::k_flow), dim3(FL::kNwg),
                                              dim3(FL::kThreadsF), args, 0, stream),
                   "cooperative launch (moderate-batch dataflow kernel)", &st))
        return st;
    h->fseq += ppf;
    return QP_OK;
}

template <int WT>
qp_status launch_frame(qp_handle* h, const RunArgs& a, hipStream_t stream, bool stepwise, bool generic, bool tiled,
                       bool flow = false) {
    qp_status st = QP_OK;
    const Model& m = h->m;
    if constexpr (WT == WT_BF16) {
        // 3 <= B <= 16 greedy frames (any B <= 16 under QP_FLAG_FLOW) of the
        // 1.7B geometry with bf16 weights: the moderate-batch dataflow kernel
        if (h->flow_ok && !a.uniforms && !stepwise && !generic && !tiled && a.B <= qp::flow::kMaxB &&
            (flow || a.B >= 3))
            return launch_flow(h, a, stream);
    }
    if constexpr (WT == WT_BF16 || WT == WT_Q8) {
        // the batched path for B > 2, and for any B that the dataflow kernel
        // cannot take (Q8_0 and Q4_0 weights, other geometries)
        if (tiled || (!stepwise && !generic && h->tiled_ok && (a.B > 2 || !h->stream_ok))) {
            const bool hooks = a.force || a.logits_out || a.taps;
            if (!hooks) return launch_tiled_graph(h, a, stream);
            if (WT == WT_Q8 && h->q4) return launch_tiled<WT_Q4>(h, a, stream);
            return launch_tiled<WT>(h, a, stream);
        }
    }
    if constexpr (WT == WT_BF16 || WT == WT_Q8) {
        if (!stepwise && !generic && h->stream_ok && a.B <= 2) {
            const uint32_t ppf = static_cast<uint32_t>(qp::stream::phases_per_frame(m.L));
            if (h->seq > 0xFFFFFFFFu - 2u * ppf) {
                // the 32-bit phase tags would wrap: clear every record (tag 0 is
                // never current) so no record left from long ago can match a new tag
                hipLaunchKernelGGL(k_fill64, dim3(64), dim3(256), 0, stream, h->recs.X, h->nrecs);
                if (!check_hip(hipGetLastError(), "record clear", &st)) return st;
                h->seq = 0;
            }
            RunArgs ra = a;
            ra.seq0 = h->seq;
            Model mm = m;
            qp::stream::Recs rc = h->recs;
            void* args[] = {&mm, &ra, &rc};
            const void* fn = a.B == 1 ? reinterpret_cast<const void*>(&qp::stream::k_stream<2, WT>)
                                      : reinterpret_cast<const void*>(&qp::stream::k_stream<4, WT>);
            if (!check_hip(hipLaunchCooperativeKernel(fn, dim3(qp::stream::kNwg), dim3(qp::stream::kThreadsS), args,
                                                      0, stream),
                           "cooperative launch (dataflow kernel)", &st))
                return st;
            h->seq += ppf;
            return QP_OK;
        }
    }
    if (stepwise) {
        auto go = [&](int ph, int s, int l) {
            hipLaunchKernelGGL(k_phase<WT>, dim3(h->nwg), dim3(kThreads), 0, stream, m, a, ph, s, l);
        };
        go(PH_INIT, 0, 0);
        for (int s = 1; s <= kSteps; ++s) {
            for (int l = 0; l < m.L; ++l) {
                go(PH_QKV, s, l);
                go(PH_ATTN, s, l);
                go(PH_OPROJ, s, l);
                go(PH_UP, s, l);
                go(PH_DOWN, s, l);
            }
            go(PH_LM, s, 0);
            go(PH_NEXT, s, 0);
        }
        if (!check_hip(hipGetLastError(), "phase kernel launch", &st)) return st;
        return QP_OK;
    }
    RunArgs ra = a;
    ra.bar_base = h->bar_base;
    Model mm = m;
    void* args[] = {&mm, &ra};
    if (!check_hip(hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&k_persistent<WT>), dim3(h->nwg),
                                              dim3(kThreads), args, 0, stream),
                   "cooperative launch", &st))
        return st;
    h->bar_base += static_cast<unsigned long long>(phases_per_frame(m.L) - 1);
    return QP_OK;
}

}  // namespace

extern "C" {

const char* qp_status_string(int32_t s) {
    switch (s) {
        case QP_OK: return "ok";
        case QP_ERR_INVALID_ARG: return "invalid argument";
        case QP_ERR_GEOMETRY: return "invalid geometry";
        case QP_ERR_SHAPE: return "shape not supported by the weight format";
        case QP_ERR_DTYPE: return "unknown dtype";
        case QP_ERR_OOM: return "device out of memory";
        case QP_ERR_HIP: return "HIP runtime error";
        case QP_ERR_BATCH: return "batch size out of range";
        case QP_ERR_DEVICE_FLAG: return "device flagged bad input or a barrier timeout";
        default: return "unknown status";
    }
}

const char* qp_last_error(void) { return g_last_error.c_str(); }

qp_status qp_create(const qp_weights* w, const qp_geometry* g, int32_t device, qp_handle** out) {
    if (!out) return fail(QP_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!w || !g) return fail(QP_ERR_INVALID_ARG, "weights or geometry is NULL");
    qp_status st = validate_geometry(g);
    if (st != QP_OK) return st;
    st = validate_weights(w, g);
    if (st != QP_OK) return st;

    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0) {
        (void)hipGetLastError();
        return fail(QP_ERR_HIP, "no HIP device");
    }
    if (device < 0 || device >= ndev) return fail(QP_ERR_INVALID_ARG, "device index out of range");
    DeviceGuard guard(device);

    qp_handle* h = new qp_handle();
    h->device = device;
    int cus = 0;
    if (!check_hip(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device),
                   "hipDeviceGetAttribute", &st)) {
        delete h;
        return st;
    }
    h->nwg = cus;

    Model& m = h->m;
    m.dT = g->d_talker;
    m.dP = g->d_model;
    m.L = g->n_layers;
    m.nq = g->n_q_heads;
    m.nkv = g->n_kv_heads;
    m.hd = g->head_dim;
    m.F = g->d_ffn;
    m.V = g->vocab;
    // Q4_0 weights run as int8 codes on every path but the batched one
    h->q4 = g->weight_dtype == QP_WEIGHT_Q4_0;
    m.wt = h->q4 ? WT_Q8 : g->weight_dtype;
    m.nqkv = (m.nq + 2 * m.nkv) * m.hd;
    m.max_batch = g->max_batch;
    m.eps = g->rms_eps;
    m.attn_scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(m.hd)));

    Uploader up{&h->allocs};
    const int wt = h->q4 ? WT_Q4 : m.wt;   // storage format of the host weights
    // batched matrix-core path: bf16, Q8_0 or Q4_0 weights whose widths tile into
    // 32 x 256 blocks (every K split four ways into whole 32-wide blocks,
    // two at a time; every N a whole number of 32-column tiles)
    h->tiled_ok = (wt == WT_BF16 || wt == WT_Q8 || wt == WT_Q4) && m.dT % 256 == 0 && m.dP % 256 == 0 && m.dP <= 4096 && m.dT <= 4096 &&
                  (m.nq * m.hd) % 256 == 0 && m.F % 256 == 0 && m.nqkv % 32 == 0 && m.V % 32 == 0;
    {
        const Uploader::HostMat hm = Uploader::build({w->proj_w}, {m.dP}, m.dT, wt);
        m.proj = up.rowmajor(hm);
        if (h->tiled_ok) h->t_proj = up.fragments(hm);
    }
    m.proj_b = static_cast<const float*>(up.upload(w->proj_b, sizeof(float) * m.dP));
    const size_t tab = static_cast<size_t>(m.V) * m.dT;
    if (g->emb_format == QP_EMB_EMA) {
        m.emb_bf16 = 0;
        float* S = static_cast<float*>(up.alloc(tab * 4));
        float* U = static_cast<float*>(up.alloc(static_cast<size_t>(m.V) * 4));
        for (int j = 0; j < kCodebooks && up.st == QP_OK; ++j) {
            float* E = static_cast<float*>(up.alloc(tab * 4));
            if (up.st != QP_OK) break;
            if (!check_hip(hipMemcpy(S, w->ema_sum[j], tab * 4, hipMemcpyHostToDevice), "hipMemcpy", &st) ||
                !check_hip(hipMemcpy(U, w->ema_usage[j], static_cast<size_t>(m.V) * 4, hipMemcpyHostToDevice),
                           "hipMemcpy", &st)) {
                up.st = st;
                break;
            }
            hipLaunchKernelGGL(k_ema, dim3(1024), dim3(256), 0, 0, S, U, E, m.V, m.dT);
            if (!check_hip(hipDeviceSynchronize(), "EMA kernel", &st)) {
                up.st = st;
                break;
            }
            m.emb[j] = E;
        }
    } else {
        m.emb_bf16 = g->emb_format == QP_EMB_BF16 ? 1 : 0;
        const size_t esz = m.emb_bf16 ? 2 : 4;
        for (int j = 0; j < kCodebooks; ++j) m.emb[j] = up.upload(w->emb[j], tab * esz);
    }
    std::vector<LayerDev> layers(static_cast<size_t>(m.L));
    const int kd = m.nkv * m.hd, qd = m.nq * m.hd;
    for (int l = 0; l < m.L && up.st == QP_OK; ++l) {
        const qp_layer_weights& lw = w->layers[l];
        LayerDev& d = layers[l];
        const Uploader::HostMat hq = Uploader::build({lw.wq, lw.wk, lw.wv}, {qd, kd, kd}, m.dP, wt);
        const Uploader::HostMat ho = Uploader::build({lw.wo}, {m.dP}, qd, wt);
        const Uploader::HostMat hg = Uploader::build({lw.w_gate}, {m.F}, m.dP, wt);
        const Uploader::HostMat hu = Uploader::build({lw.w_up}, {m.F}, m.dP, wt);
        const Uploader::HostMat hd = Uploader::build({lw.w_down}, {m.dP}, m.F, wt);
        d.qkv = up.rowmajor(hq);
        d.o = up.rowmajor(ho);
        d.gate = up.rowmajor(hg);
        d.up = up.rowmajor(hu);
        d.down = up.rowmajor(hd);
        if (h->tiled_ok) {
            h->t_qkv.push_back(up.fragments(hq));
            h->t_o.push_back(up.fragments(ho));
            h->t_gate.push_back(up.fragments(hg));
            h->t_up.push_back(up.fragments(hu));
            h->t_down.push_back(up.fragments(hd));
        }
        d.attn_norm = static_cast<const float*>(up.upload(lw.attn_norm, sizeof(float) * m.dP));
        d.q_norm = static_cast<const float*>(up.upload(lw.q_norm, sizeof(float) * m.hd));
        d.k_norm = static_cast<const float*>(up.upload(lw.k_norm, sizeof(float) * m.hd));
        d.ffn_norm = static_cast<const float*>(up.upload(lw.ffn_norm, sizeof(float) * m.dP));
    }
    h->layers_host = layers;
    // a geometry without layers still gets a (never read) one-entry table:
    // the copy source must be a real host array
    if (layers.empty()) layers.push_back(LayerDev{});
    m.layers = static_cast<const LayerDev*>(up.upload(layers.data(), sizeof(LayerDev) * layers.size()));
    m.out_norm = static_cast<const float*>(up.upload(w->out_norm, sizeof(float) * m.dP));
    for (int k = 0; k < kSteps && up.st == QP_OK; ++k) {
        const Uploader::HostMat hl = Uploader::build({w->lm_head[k]}, {m.V}, m.dP, wt);
        m.lm[k] = up.rowmajor(hl);
        if (h->tiled_ok) h->t_lm[k] = up.fragments(hl);
    }

    // RoPE table, fp64 then rounded: angle(p, i) = p * base^(-2i/hd)
    const int half = m.hd / 2;
    std::vector<float> rc(static_cast<size_t>(kPositions) * half), rs(rc.size());
    for (int p = 0; p < kPositions; ++p)
        for (int i = 0; i < half; ++i) {
            const double ang = p * std::pow(static_cast<double>(g->rope_base), -2.0 * i / m.hd);
            rc[static_cast<size_t>(p) * half + i] = static_cast<float>(std::cos(ang));
            rs[static_cast<size_t>(p) * half + i] = static_cast<float>(std::sin(ang));
        }
    m.rope_cos = static_cast<const float*>(up.upload(rc.data(), rc.size() * 4));
    m.rope_sin = static_cast<const float*>(up.upload(rs.data(), rs.size() * 4));

    // scratch for max_batch requests
    const size_t rows = 2 * static_cast<size_t>(m.max_batch);
    const size_t rows16 = (rows + 15) / 16 * 16;   // the batched path's bf16 operands, in whole row fragments
    m.x = static_cast<float*>(up.alloc(rows * m.dP * 4));
    m.qkv = static_cast<float*>(up.alloc(rows * m.nqkv * 4));
    m.ao = static_cast<float*>(up.alloc(std::max(rows * qd * 4, rows16 * qd * 2)));
    m.hb = static_cast<float*>(up.alloc(std::max(rows * m.F * 4, rows16 * m.F * 2)));
    const size_t kvn = static_cast<size_t>(m.L > 0 ? m.L : 1) * m.max_batch * kPositions * kd;
    m.kc = static_cast<float*>(up.alloc(kvn * 4));
    m.vc = static_cast<float*>(up.alloc(kvn * 4));
    m.amax = static_cast<unsigned long long*>(up.alloc(static_cast<size_t>(m.max_batch) * 8));
    m.err = static_cast<unsigned*>(up.alloc(256));
    m.bar = static_cast<unsigned long long*>(up.alloc(4096));
    float* ptab = static_cast<float*>(up.alloc(static_cast<size_t>(kSteps) * m.V * m.dP * 4));
    float* qkv0 = nullptr;
    m.ptab = ptab;
    if (h->tiled_ok) {
        // argmax keys of the lm_head tiles; split-K partial tiles and counters
        // for the products with N = dP (split K only when M <= 2 * max_batch
        // rows leave fewer than 256 tiles)
        h->t_keys = static_cast<unsigned long long*>(up.alloc(static_cast<size_t>(m.max_batch) * (m.V / 16) * 8));
        // K is split only while tiles * KS < 2 * 256, so 512 partial tiles
        // of up to 4 row fragments x 2 column fragments suffice
        h->t_part_floats = 512ull * 4 * 2 * 256;
        h->t_part = static_cast<float*>(up.alloc(h->t_part_floats * 4));
        h->t_nctr = 256;  // split K (the projection of H) only applies below 256 tiles
        h->t_ctr = static_cast<unsigned*>(up.alloc(h->t_nctr * 4));
        h->t_xg = static_cast<uint16_t*>(up.alloc(rows16 * m.dP * 2));
        h->st_H = static_cast<float*>(up.alloc(static_cast<size_t>(m.max_batch) * m.dT * 4));
        h->st_q0 = static_cast<int*>(up.alloc(static_cast<size_t>(m.max_batch) * 4));
        h->st_tok = static_cast<int*>(up.alloc(static_cast<size_t>(m.max_batch) * kSteps * 4));
        h->st_emb = static_cast<float*>(up.alloc(static_cast<size_t>(m.max_batch) * m.dT * 4));
        h->t_ss = static_cast<float*>(up.alloc(rows * (m.dP / 16) * 4));
        h->sample_ok = m.V <= qp::sample::kMaxV;
        if (h->sample_ok) {
            h->t_logits = static_cast<float*>(up.alloc(static_cast<size_t>(m.max_batch) * m.V * 4));
            h->t_sampled = static_cast<int*>(up.alloc(static_cast<size_t>(m.max_batch) * 4));
            h->st_u = static_cast<float*>(up.alloc(static_cast<size_t>(m.max_batch) * kSteps * 4));
            h->st_samp = static_cast<qp::sample::Params*>(up.alloc(256));
        }
    }

    // records of the dataflow kernel (1.7B geometry, bf16, Q8_0 or Q4_0 weights, B <= 2)
    {
        namespace S = qp::stream;
        h->stream_ok = m.dT == S::DT && m.dP == S::DP && m.nq == S::NQ && m.nkv == S::NKV && m.hd == S::HD &&
                       m.F == S::F && m.V == S::V && (wt == WT_BF16 || wt == WT_Q8 || wt == WT_Q4) && m.L >= 1 &&
                       m.L <= S::kMaxL;
        if (h->stream_ok) {
            constexpr int MR = 4;
            const size_t nrec = static_cast<size_t>(MR) * (S::DP + S::NQKV + S::QD + S::F) + 2ull * S::kNwg * 2;
            uint64_t* r = static_cast<uint64_t*>(up.alloc(nrec * 8));
            if (r) {
                h->nrecs = nrec;
                h->recs.X = r;
                h->recs.QKV = h->recs.X + MR * S::DP;
                h->recs.AO = h->recs.QKV + MR * S::NQKV;
                h->recs.H = h->recs.AO + MR * S::QD;
                h->recs.KEY = h->recs.H + MR * S::F;
                if (hipMemset(r, 0, nrec * 8) != hipSuccess) {
                    up.st = QP_ERR_HIP;
                    up.msg = "hipMemset of the record buffers failed";
                }
            }
            // layer 0's q/k/v rows of every table row (k_qkv0, after k_ptab);
            // the batched path's layer-0 attention then also moves each
            // request to its token, a slice of kTokPer elements per thread
            // and kv head
            static_assert(S::DT <= qp::tiled::kTokPer * qp::tiled::kThreadsT * S::NKV &&
                              S::DP <= qp::tiled::kTokPer * qp::tiled::kThreadsT * S::NKV,
                          "token move slices exceed the registers set aside for them");
            qkv0 = static_cast<float*>(up.alloc(static_cast<size_t>(kSteps - 1) * m.V * m.nqkv * 4));
            m.qkv0 = qkv0;
        }
    }
    // records of the moderate-batch dataflow kernel (same geometry, bf16
    // weights in fragment order)
    {
        namespace FL = qp::flow;
        h->flow_ok = h->stream_ok && h->tiled_ok && wt == WT_BF16;
        if (h->flow_ok) {
            uint64_t* r = static_cast<uint64_t*>(up.alloc(FL::kRecsTotal * 8));
            if (r) {
                h->frec_base = r;
                h->frecs.XG = r;
                h->frecs.SS = h->frecs.XG + static_cast<size_t>(FL::kMaxRows) * (FL::DP / 2);
                h->frecs.QKV = h->frecs.SS + static_cast<size_t>(FL::kNOwn) * FL::kMaxRows;
                h->frecs.AO = h->frecs.QKV + static_cast<size_t>(FL::kMaxRows) * FL::NQKV;
                h->frecs.HH = h->frecs.AO + static_cast<size_t>(FL::kMaxRows) * (FL::QD / 2);
                h->frecs.KEY = h->frecs.HH + static_cast<size_t>(FL::kMaxRows) * (FL::F / 2);
                if (hipMemset(r, 0, FL::kRecsTotal * 8) != hipSuccess) {
                    up.st = QP_ERR_HIP;
                    up.msg = "hipMemset of the record buffers failed";
                }
            }
        }
    }

    if (up.st != QP_OK) {
        st = fail(up.st, up.msg);
        free_all(h);
        delete h;
        return st;
    }
    if (!check_hip(hipMemset(m.amax, 0, static_cast<size_t>(m.max_batch) * 8), "hipMemset", &st) ||
        !check_hip(hipMemset(m.err, 0, 256), "hipMemset", &st) ||
        !check_hip(hipMemset(m.bar, 0, 4096), "hipMemset", &st) ||
        (h->tiled_ok && !check_hip(hipMemset(h->t_ctr, 0, h->t_nctr * 4), "hipMemset", &st))) {
        free_all(h);
        delete h;
        return st;
    }
    hipLaunchKernelGGL(k_ptab, dim3((m.dP + 63) / 64, (m.V + 63) / 64, kSteps), dim3(256), 0, 0, m, ptab);
    if (qkv0)
        hipLaunchKernelGGL(k_qkv0, dim3((m.nqkv + 63) / 64, (m.V + 63) / 64, kSteps - 1), dim3(256), 0, 0, m,
                           h->layers_host[0].attn_norm, qkv0);
    if (!check_hip(hipGetLastError(), "projected-table kernel launch", &st) ||
        !check_hip(hipDeviceSynchronize(), "projected-table kernel", &st)) {
        free_all(h);
        delete h;
        return st;
    }
    // the static scratch of qp_run_frames_noalloc on this device
    if (h->stream_ok) {
        st = noalloc_setup(device);
        if (st != QP_OK) {
            destroy_handle(h);
            return st;
        }
    }
    // every graph a later call can replay, built now so that no call
    // captures, instantiates or frees one
    if (h->tiled_ok) {
        st = prepare_tiled_graphs(h);
        if (st != QP_OK) {
            destroy_handle(h);
            return st;
        }
    }
    // testing only: the dataflow kernel's first record epoch, so that a test
    // reaches the tag-restart path without running 11 million frames first
    if (const char* e = std::getenv("QP_TEST_EPOCH0")) h->seq = h->fseq = static_cast<uint32_t>(std::strtoul(e, nullptr, 0));
    *out = h;
    return QP_OK;
}


qp_status qp_run_frames_ex(qp_handle* h, int32_t B, const float* H, const int32_t* q0, int32_t* tokens_out,
                           float* embsum_out, void* stream, const int32_t* force_tokens, float* logits_out,
                           float* taps_out, uint32_t flags) {
    if (!h) return fail(QP_ERR_INVALID_ARG, "handle is NULL");
    if (B < 0 || B > h->m.max_batch)
        return fail(QP_ERR_BATCH, "B=" + std::to_string(B) + " outside [0, " + std::to_string(h->m.max_batch) + "]");
    if (flags & ~(QP_FLAG_STEPWISE | QP_FLAG_GENERIC | QP_FLAG_TILED | QP_FLAG_FLOW))
        return fail(QP_ERR_INVALID_ARG, "unknown flag bits");
    const bool tiled = (flags & QP_FLAG_TILED) != 0;
    const bool flow = (flags & QP_FLAG_FLOW) != 0;
    if (tiled && (flags & (QP_FLAG_STEPWISE | QP_FLAG_GENERIC)))
        return fail(QP_ERR_INVALID_ARG, "QP_FLAG_TILED excludes the other driver flags");
    if (flow && (flags & (QP_FLAG_STEPWISE | QP_FLAG_GENERIC | QP_FLAG_TILED)))
        return fail(QP_ERR_INVALID_ARG, "QP_FLAG_FLOW excludes the other driver flags");
    if (tiled && !h->tiled_ok)
        return fail(QP_ERR_INVALID_ARG, "the batched matrix-core path does not support this geometry or weight dtype");
    if (flow && (!h->flow_ok || B > qp::flow::kMaxB))
        return fail(QP_ERR_INVALID_ARG,
                    "the moderate-batch dataflow kernel takes the 1.7B predictor geometry with bf16 weights and "
                    "B <= 16 only");
    if (B == 0) return QP_OK;
    if (!H || !q0 || !tokens_out || !embsum_out) return fail(QP_ERR_INVALID_ARG, "NULL input or output pointer");
    DeviceGuard guard(h->device);
    RunArgs a{};
    a.B = B;
    a.H = H;
    a.q0 = q0;
    a.tok_out = tokens_out;
    a.embsum = embsum_out;
    a.force = force_tokens;
    a.logits_out = logits_out;
    a.taps = taps_out;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const bool stepwise = (flags & QP_FLAG_STEPWISE) != 0;
    const bool generic = (flags & QP_FLAG_GENERIC) != 0;
    switch (h->m.wt) {
        case WT_F32: return launch_frame<WT_F32>(h, a, s, stepwise, generic, false);
        case WT_BF16: return launch_frame<WT_BF16>(h, a, s, stepwise, generic, tiled, flow);
        default: return launch_frame<WT_Q8>(h, a, s, stepwise, generic, tiled);
    }
}

qp_status qp_run_frames(qp_handle* h, int32_t B, const float* H, const int32_t* q0, int32_t* tokens_out,
                        float* embsum_out, void* stream) {
    return qp_run_frames_ex(h, B, H, q0, tokens_out, embsum_out, stream, nullptr, nullptr, nullptr, 0u);
}

qp_status qp_run_frames_noalloc(qp_handle* h, int32_t B, const float* H, const int32_t* q0, int32_t* tokens_out,
                                float* embsum_out, void* stream) {
    namespace S = qp::stream;
    if (!h) return fail(QP_ERR_INVALID_ARG, "handle is NULL");
    if (!h->stream_ok)
        return fail(QP_ERR_INVALID_ARG,
                    "the allocation-free entry point runs the small-batch dataflow kernel: the 1.7B predictor "
                    "geometry with bf16, Q8_0 or Q4_0 weights only");
    const int bmax = std::min(noalloc::kMaxB, h->m.max_batch);
    if (B < 0 || B > bmax)
        return fail(QP_ERR_BATCH, "B=" + std::to_string(B) + " outside [0, " + std::to_string(bmax) +
                                      "]: the static scratch holds " + std::to_string(noalloc::kMaxB) +
                                      " requests (and B may not exceed max_batch)");
    if (B == 0) return QP_OK;
    if (!H || !q0 || !tokens_out || !embsum_out) return fail(QP_ERR_INVALID_ARG, "NULL input or output pointer");
    if (h->device >= noalloc::kDevices) return fail(QP_ERR_INVALID_ARG, "device index beyond the static scratch table");
    DeviceGuard guard(h->device);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    qp_status st = QP_OK;
    const uint32_t ppf = static_cast<uint32_t>(S::phases_per_frame(h->m.L));
    uint64_t* base = nullptr;
    uint32_t seq0 = 0;
    {
        std::lock_guard<std::mutex> lock(g_noalloc_mu);
        NoallocDev& d = g_noalloc[h->device];
        if (!d.base) return fail(QP_ERR_HIP, "the static scratch of this device was not set up");
        if (d.seq > 0xFFFFFFFFu - 2u * ppf) {
            // the 32-bit tags would wrap: clear the records, restart the tags
            hipLaunchKernelGGL(k_fill64, dim3(64), dim3(256), 0, s, d.base, noalloc::kRecs);
            if (!check_hip(hipGetLastError(), "static scratch clear", &st)) return st;
            d.seq = 0;
        }
        base = d.base;
        seq0 = d.seq;
        d.seq += ppf;
    }
    // the kernel's records and KV cache in the static scratch (the records'
    // row stride is the kernel's 4 rows; the KV cache holds 2 requests)
    S::Recs rc{};
    rc.X = base;
    rc.QKV = rc.X + 4 * S::DP;
    rc.AO = rc.QKV + 4 * S::NQKV;
    rc.H = rc.AO + 4 * S::QD;
    rc.KEY = rc.H + 4 * S::F;
    Model mm = h->m;
    mm.kc = reinterpret_cast<float*>(base + noalloc::kRecs);
    mm.vc = mm.kc + noalloc::kKV;
    mm.max_batch = noalloc::kMaxB;
    RunArgs ra{};
    ra.B = B;
    ra.H = H;
    ra.q0 = q0;
    ra.tok_out = tokens_out;
    ra.embsum = embsum_out;
    ra.seq0 = seq0;
    void* args[] = {&mm, &ra, &rc};
    const void* fn;
    if (h->m.wt == WT_BF16)
        fn = B == 1 ? reinterpret_cast<const void*>(&S::k_stream<2, WT_BF16>)
                    : reinterpret_cast<const void*>(&S::k_stream<4, WT_BF16>);
    else
        fn = B == 1 ? reinterpret_cast<const void*>(&S::k_stream<2, WT_Q8>)
                    : reinterpret_cast<const void*>(&S::k_stream<4, WT_Q8>);
    if (!check_hip(hipLaunchCooperativeKernel(fn, dim3(S::kNwg), dim3(S::kThreadsS), args, 0, s),
                   "cooperative launch (dataflow kernel, static scratch)", &st))
        return st;
    return QP_OK;
}

namespace {
bool sampling_valid(const qp_sampling* sp, std::string* why) {
    if (!sp) {
        *why = "sampling parameters are NULL";
        return false;
    }
    if (!(sp->temperature > 0.0f) || !std::isfinite(sp->temperature)) {
        *why = "temperature must be finite and > 0";
        return false;
    }
    if (sp->top_k < 0) {
        *why = "top_k must be >= 0";
        return false;
    }
    if (!(sp->top_p > 0.0f && sp->top_p <= 1.0f)) {
        *why = "top_p must lie in (0, 1]";
        return false;
    }
    return true;
}
}  // namespace

qp_status qp_run_frames_sampled(qp_handle* h, int32_t B, const float* H, const int32_t* q0,
                                const qp_sampling* sampling, const float* uniforms, int32_t* tokens_out,
                                float* embsum_out, void* stream, const int32_t* force_tokens, float* logits_out) {
    if (!h) return fail(QP_ERR_INVALID_ARG, "handle is NULL");
    if (B < 0 || B > h->m.max_batch)
        return fail(QP_ERR_BATCH, "B=" + std::to_string(B) + " outside [0, " + std::to_string(h->m.max_batch) + "]");
    std::string why;
    if (!sampling_valid(sampling, &why)) return fail(QP_ERR_INVALID_ARG, why);
    if (!h->tiled_ok || !h->sample_ok)
        return fail(QP_ERR_INVALID_ARG,
                    "sampled frames run on the batched matrix-core path, which does not support this geometry, "
                    "weight dtype or vocabulary size");
    if (B == 0) return QP_OK;
    if (!H || !q0 || !uniforms || !tokens_out || !embsum_out)
        return fail(QP_ERR_INVALID_ARG, "NULL input or output pointer");
    DeviceGuard guard(h->device);
    RunArgs a{};
    a.B = B;
    a.H = H;
    a.q0 = q0;
    a.tok_out = tokens_out;
    a.embsum = embsum_out;
    a.force = force_tokens;
    a.logits_out = logits_out;
    a.uniforms = uniforms;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const qp::sample::Params p{sampling->temperature, sampling->top_k, sampling->top_p};
    hipLaunchKernelGGL(qp::sample::k_set_params, dim3(1), dim3(64), 0, s, p, h->st_samp);
    switch (h->m.wt) {
        case WT_BF16: return launch_frame<WT_BF16>(h, a, s, false, false, true);
        default: return launch_frame<WT_Q8>(h, a, s, false, false, true);
    }
}

qp_status qp_sample_logits(const float* logits, int32_t rows, int32_t V, int64_t row_stride,
                           const qp_sampling* sampling, const float* uniforms, int32_t uniform_stride,
                           int32_t* tokens_out, void* stream) {
    std::string why;
    if (!sampling_valid(sampling, &why)) return fail(QP_ERR_INVALID_ARG, why);
    if (rows < 0) return fail(QP_ERR_INVALID_ARG, "rows must be >= 0");
    if (V < 1 || V > qp::sample::kMaxV)
        return fail(QP_ERR_INVALID_ARG, "V must lie in [1, " + std::to_string(qp::sample::kMaxV) + "]");
    if (row_stride < V) return fail(QP_ERR_INVALID_ARG, "row_stride must be >= V");
    if (uniform_stride < 1) return fail(QP_ERR_INVALID_ARG, "uniform_stride must be >= 1");
    if (rows == 0) return QP_OK;
    if (!logits || !uniforms || !tokens_out) return fail(QP_ERR_INVALID_ARG, "NULL input or output pointer");
    const qp::sample::Params p{sampling->temperature, sampling->top_k, sampling->top_p};
    hipLaunchKernelGGL(qp::sample::sample_kernel(V), dim3(rows), dim3(qp::sample::kThreadsSm), 0,
                       static_cast<hipStream_t>(stream), logits, static_cast<long long>(row_stride), V, p,
                       static_cast<const qp::sample::Params*>(nullptr), uniforms, uniform_stride, tokens_out);
    qp_status st = QP_OK;
    if (!check_hip(hipGetLastError(), "sampling kernel launch", &st)) return st;
    return QP_OK;
}

qp_status qp_get_error(qp_handle* h) {
    if (!h) return fail(QP_ERR_INVALID_ARG, "handle is NULL");
    DeviceGuard guard(h->device);
    qp_status st = QP_OK;
    if (!check_hip(hipDeviceSynchronize(), "hipDeviceSynchronize", &st)) return st;
    unsigned flags = 0;
    if (!check_hip(hipMemcpy(&flags, h->m.err, 4, hipMemcpyDeviceToHost), "hipMemcpy", &st)) return st;
    h->last_flags = flags;
    if (flags == 0) return QP_OK;
    if (!check_hip(hipMemset(h->m.err, 0, 4), "hipMemset", &st)) return st;
    if (flags & kErrBarrierTimeout) {
        // the barrier count is unknown after a timeout: restart it
        if (!check_hip(hipMemset(h->m.bar, 0, 4096), "hipMemset", &st)) return st;
        h->bar_base = 0;
    }
    char hex[16];
    std::snprintf(hex, sizeof(hex), "0x%x", flags);
    return fail(QP_ERR_DEVICE_FLAG, std::string("device flags ") + hex);
}

uint32_t qp_last_device_flags(qp_handle* h) { return h ? h->last_flags : 0u; }

void qp_destroy(qp_handle* h) {
    if (!h) return;
    destroy_handle(h);
}

}  // extern "C"

// the Talker decode step (include/qp_talker.h)
#include "qp_talker_host.h"

#ifdef QP_TIMELINE
// Timeline build only (QP_TSTAMP): copies the batched path's kernel stamps,
// uint64 [kTiledLaunches][kTiledWgs][3] (at most `bytes` of them), and the
// role (TlKind) of each launch of the frame last captured or launched (at
// most `cap`); returns the number of launches in that frame, or -1 if the
// copy fails.
extern "C" int qp_timeline_tiled(void* stamps, size_t bytes, int* kinds, int cap) {
    const size_t n = std::min(bytes, sizeof(qp::g_tiled_stamps));
    if (hipDeviceSynchronize() != hipSuccess) return -1;
    if (hipMemcpyFromSymbol(stamps, HIP_SYMBOL(qp::g_tiled_stamps), n, 0, hipMemcpyDeviceToHost) != hipSuccess)
        return -1;
    for (int i = 0; i < cap && i < qp::kTiledLaunches; ++i) kinds[i] = g_tl_kind[i];
    return g_tl_next;
}
#endif

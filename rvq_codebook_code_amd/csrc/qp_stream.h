// Dataflow frame kernel for small batches (B <= 2) of the 1.7B-shaped
// predictor with bf16 weights.
//
// One persistent workgroup per CU (256), each with four compute waves and
// one poller wave, and no grid barrier at all:
//  * every value that crosses workgroups is published as a 64-bit record
//    (epoch << 32 | fp32 bits) with a device-scope store; the epoch is unique
//    per phase instance, so a consumer knows a value is current by its tag;
//  * the poller wave waits for exactly the records its workgroup needs next,
//    copies them into one of two LDS slots, computes the RMS statistics, and
//    releases the compute waves with one workgroup barrier per phase;
//  * the compute waves never wait on remote data, so each phase's weight
//    loads are issued one phase ahead into registers and land while the
//    workgroup waits for that phase's inputs (only the poller issues polling
//    loads, whose completion would otherwise be ordered behind them).
// Ownership (256 workgroups x 4 compute waves = 1024 waves):
//    q/k/v rows 16*wg + 4*w + {0..3}, O / down / projection row 4*wg + w,
//    gate/up rows 12*wg + 3*w + {0..2}, lm_head rows 8*wg + 2*w + {0,1},
//    attention unit (request b, kv head g) on workgroup b*8 + g,
//    embedding-sum elements 8*wg .. 8*wg+7.
#pragma once

#include "qp_common.h"
#include "qp_phases.h"

namespace qp {
namespace stream {

// the Qwen3-TTS 1.7B code-predictor geometry
constexpr int DT = 2048, DP = 1024, NQ = 16, NKV = 8, HD = 128, F = 3072, V = 2048;
constexpr int QD = NQ * HD, NQKV = (NQ + 2 * NKV) * HD;
constexpr int kCW = 4;                   // compute waves
constexpr int kThreadsS = (kCW + 1) * 64;
constexpr int kNwg = 256;
constexpr int kGW = kNwg * kCW;          // compute waves in the grid
static_assert(NQKV == 16 * kNwg && DP == 4 * kNwg && F == 12 * kNwg && V == 8 * kNwg && DT == 8 * kNwg,
              "row ownership assumes the 1.7B predictor geometry");

__host__ __device__ constexpr int phases_per_frame(int L) { return 1 + kSteps * (5 * L + 1) + 1; }
__host__ __device__ constexpr int slot_floats(int MR) { return MR * F; }

struct Recs {
    uint64_t* X;    // [MR][DP]
    uint64_t* QKV;  // [MR][NQKV]
    uint64_t* AO;   // [MR][QD]
    uint64_t* H;    // [MR][F]
    uint64_t* KEY;  // [Bmax][kGW][2]
};

__device__ __forceinline__ void st_rec(uint64_t* p, float v, uint32_t tag) {
    const uint64_t u = (static_cast<uint64_t>(tag) << 32) | __float_as_uint(v);
    __hip_atomic_store(p, u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_rec_u(uint64_t* p, uint32_t v, uint32_t tag) {
    const uint64_t u = (static_cast<uint64_t>(tag) << 32) | v;
    __hip_atomic_store(p, u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_rec(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// frame-relative phase indices
__device__ __forceinline__ int ph_layer(int L, int s, int l, int t) { return 1 + (s - 1) * (5 * L + 1) + 5 * l + t; }
__device__ __forceinline__ int ph_lm(int L, int s) { return 1 + (s - 1) * (5 * L + 1) + 5 * L; }
enum { T_QKV = 0, T_ATTN = 1, T_O = 2, T_UP = 3, T_DOWN = 4 };

__device__ __forceinline__ bool timed_out(const unsigned* err) {
    return __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kErrBarrierTimeout;
}

// ---------------------------------------------------------------------------
// poller side
// ---------------------------------------------------------------------------

__device__ __forceinline__ bool spin_wait(unsigned& spins, unsigned* err) {
    __builtin_amdgcn_s_sleep(1);
    if ((++spins & 255u) == 0u) {
        if (timed_out(err)) return false;
        if (spins > (1u << 22)) {
            atomicOr(err, kErrBarrierTimeout);
            return false;
        }
    }
    return true;
}

// Wait for the 64*N records src[0 .. 64N) carrying `tag` and copy their
// values to dst[0 .. 64N).  Every missing record is re-read each round; all of
// a round's loads are in flight together.
template <int N>
__device__ __forceinline__ void poll_vec(const uint64_t* src, uint32_t tag, float* dst, unsigned* err) {
    static_assert(N <= 64, "at most 64 records per lane");
    const int lane = threadIdx.x & 63;
    uint64_t pend = (N == 64) ? ~0ull : ((1ull << N) - 1ull);
    const uint64_t* p = src + lane;
    unsigned spins = 0;
    while (true) {
        uint64_t u[N];
#pragma unroll
        for (int i = 0; i < N; ++i)
            if ((pend >> i) & 1ull) u[i] = ld_rec(p + 64 * i);
#pragma unroll
        for (int i = 0; i < N; ++i) {
            if (((pend >> i) & 1ull) && static_cast<uint32_t>(u[i] >> 32) == tag) {
                dst[lane + 64 * i] = __uint_as_float(static_cast<uint32_t>(u[i]));
                pend &= ~(1ull << i);
            }
        }
        if (!__any(pend != 0ull)) break;
        if (!spin_wait(spins, err)) break;
    }
}

// The four head vectors one attention unit needs from a q/k/v row: q heads
// 2g and 2g+1, k head g, v head g (HD = 128 each) -> dst[0..512).
__device__ __forceinline__ void poll_heads(const uint64_t* row, int g, uint32_t tag, float* dst, unsigned* err) {
    const int lane = threadIdx.x & 63;
    const int col[4] = {(2 * g) * HD, (2 * g + 1) * HD, (NQ + g) * HD, (NQ + NKV + g) * HD};
    uint32_t pend = 0xFFu;
    unsigned spins = 0;
    while (true) {
        uint64_t u[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if ((pend >> j) & 1u) u[j] = ld_rec(row + col[j >> 1] + lane + 64 * (j & 1));
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (((pend >> j) & 1u) && static_cast<uint32_t>(u[j] >> 32) == tag) {
                dst[(j >> 1) * HD + lane + 64 * (j & 1)] = __uint_as_float(static_cast<uint32_t>(u[j]));
                pend &= ~(1u << j);
            }
        }
        if (!__any(pend != 0u)) break;
        if (!spin_wait(spins, err)) break;
    }
}

// 64 consecutive fp32 values (device-coherent) straight into LDS, one per
// lane, without passing through registers: src and dst are wave-uniform.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void gbl_void_t;
__device__ __forceinline__ void dma64(const float* src, float* dst) {
    const int lane = threadIdx.x & 63;
    __builtin_amdgcn_global_load_lds((gbl_void_t*)(src + lane), (lds_void_t*)(dst), 4, 0,
                                     16 /* device scope */);
}

// Sum of squares of n LDS values, fixed order, lane-uniform result.
__device__ __forceinline__ float lds_sumsq(const float* x, int n) {
    const int lane = threadIdx.x & 63;
    float t = 0.f;
    for (int k = lane; k < n; k += 64) t = fmaf(x[k], x[k], t);
    return wave_sum(t);
}

// Global argmax over the per-wave key records of every request: returns the
// token of request `b` in lane-uniform form.  Records: [b][gw][0] = ordered
// logit bits, [b][gw][1] = vocabulary index, both tagged.
__device__ int poll_argmax(const uint64_t* key, int b, uint32_t tag, unsigned* err) {
    const int lane = threadIdx.x & 63;
    uint64_t best = 0;
    // 2*kGW records per request; poll them 64*32 at a time
    const uint64_t* src = key + static_cast<size_t>(b) * kGW * 2;
    constexpr int PER = 32;
    for (int f0 = 0; f0 < 2 * kGW; f0 += 64 * PER) {
        uint32_t val[PER];
        uint32_t pending = 0xFFFFFFFFu;
        unsigned spins = 0;
        while (true) {
            uint64_t u[PER];
#pragma unroll
            for (int i = 0; i < PER; ++i)
                if (pending & (1u << i)) u[i] = ld_rec(src + f0 + 2 * lane + 128 * (i >> 1) + (i & 1));
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                if ((pending & (1u << i)) && static_cast<uint32_t>(u[i] >> 32) == tag) {
                    val[i] = static_cast<uint32_t>(u[i]);
                    pending &= ~(1u << i);
                }
            }
            if (!__any(pending != 0u)) break;
            if (!spin_wait(spins, err)) break;
        }
#pragma unroll
        for (int i = 0; i < PER; i += 2) {
            // larger logit first, lower index on ties
            const uint64_t k = (static_cast<uint64_t>(val[i]) << 32) | (0xFFFFFFFFu - val[i + 1]);
            best = k > best ? k : best;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint64_t o = (static_cast<uint64_t>(__shfl_xor(static_cast<unsigned>(best >> 32), off, 64)) << 32) |
                           __shfl_xor(static_cast<unsigned>(best & 0xFFFFFFFFu), off, 64);
        best = o > best ? o : best;
    }
    return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best & 0xFFFFFFFFu));
}

// ---------------------------------------------------------------------------
// compute side helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float dot8(const uint4 w, const float a[8], float acc) {
    acc = fmaf(__uint_as_float(w.x << 16), a[0], acc);
    acc = fmaf(__uint_as_float(w.x & 0xFFFF0000u), a[1], acc);
    acc = fmaf(__uint_as_float(w.y << 16), a[2], acc);
    acc = fmaf(__uint_as_float(w.y & 0xFFFF0000u), a[3], acc);
    acc = fmaf(__uint_as_float(w.z << 16), a[4], acc);
    acc = fmaf(__uint_as_float(w.z & 0xFFFF0000u), a[5], acc);
    acc = fmaf(__uint_as_float(w.w << 16), a[6], acc);
    acc = fmaf(__uint_as_float(w.w & 0xFFFF0000u), a[7], acc);
    return acc;
}

// Weights stream through buffer loads: the matrix base lives in a scalar
// resource (with the matrix size as its bound), the lane offset in one VGPR,
// the row offset in an SGPR, so no per-row 64-bit addresses are kept.
using rsrc_t = __amdgpu_buffer_rsrc_t;
__device__ __forceinline__ rsrc_t wrsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0), static_cast<int>(bytes),
                                             0x00020000);
}
// 8 bf16 weights of row `row` (K wide) at k = kc*512 + lane*8
__device__ __forceinline__ uint4 ldw(rsrc_t r, int row, int K, int kc, uint32_t lane16) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, lane16 + static_cast<uint32_t>(kc) * 1024u,
                                                         static_cast<uint32_t>(row) * static_cast<uint32_t>(K) * 2u, 0);
    return make_uint4(static_cast<uint32_t>(v[0]), static_cast<uint32_t>(v[1]), static_cast<uint32_t>(v[2]),
                      static_cast<uint32_t>(v[3]));
}

__device__ __forceinline__ void lds8(const float* p, float a[8]) {
    const float4 u = *reinterpret_cast<const float4*>(p);
    const float4 v = *reinterpret_cast<const float4*>(p + 4);
    a[0] = u.x; a[1] = u.y; a[2] = u.z; a[3] = u.w;
    a[4] = v.x; a[5] = v.y; a[6] = v.z; a[7] = v.w;
}

__device__ __forceinline__ void gain8(const float4 g0, const float4 g1, float a[8]) {
    a[0] *= g0.x; a[1] *= g0.y; a[2] *= g0.z; a[3] *= g0.w;
    a[4] *= g1.x; a[5] *= g1.y; a[6] *= g1.z; a[7] *= g1.w;
}

__device__ __forceinline__ uint32_t ordered_bits(float v) {
    uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ void ld_gain(const float* g, int lane, float4 out[4]) {
    // the 16 gains a lane needs for K = 1024: k = lane*8..+7 and 512 + lane*8..+7
    const float4* p = reinterpret_cast<const float4*>(g + lane * 8);
    const float4* q = reinterpret_cast<const float4*>(g + 512 + lane * 8);
    out[0] = p[0]; out[1] = p[1]; out[2] = q[0]; out[3] = q[1];
}

__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

constexpr int kMaxL = 5;  // layers whose norm gains fit the LDS table
// LDS gain table: attn_norm[l], ffn_norm[l] (DP each), out_norm (DP), then
// q_norm[l], k_norm[l] (HD each)
constexpr int kGainFloats = (2 * kMaxL + 1) * DP + 2 * kMaxL * HD;

template <int MR>
__global__ __launch_bounds__(kThreadsS) void k_stream(Model m, RunArgs a, Recs rc) {
    constexpr int SLOT = slot_floats(MR);
    __shared__ float slot[2][SLOT];
    __shared__ float ssq[2][MR];
    __shared__ float rope_s[2][kPositions * (HD / 2)];
    __shared__ float gains[kGainFloats];
    __shared__ LayerDev lay_s[kMaxL];
    const int wg = blockIdx.x;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int B = a.B;
    const int L = m.L;
    const uint32_t seq0 = a.seq0;
    auto tag_of = [&](int ph) { return seq0 + static_cast<uint32_t>(ph) + 1u; };
    const float eps = m.eps;
    // the layer table lives in device memory; read it once into LDS so that
    // no phase waits on a pointer load
    if (threadIdx.x < L) lay_s[threadIdx.x] = m.layers[threadIdx.x];
    __syncthreads();
    const LayerDev* LD = lay_s;
    auto g_attn = [&](int l) { return gains + (2 * l) * DP; };
    auto g_ffn = [&](int l) { return gains + (2 * l + 1) * DP; };
    const float* g_out = gains + 2 * kMaxL * DP;
    auto g_q = [&](int l) { return gains + (2 * kMaxL + 1) * DP + (2 * l) * HD; };
    auto g_k = [&](int l) { return gains + (2 * kMaxL + 1) * DP + (2 * l + 1) * HD; };

    if (wave == kCW) {
        // ======================= poller wave =======================
        int fed[2] = {0, 0};
        float es = 0.f;  // embedding-sum element: request lane/8, column 8*wg + lane%8
        const int eb = lane >> 3, ek = 8 * wg + (lane & 7);
        // INIT: H rows, q0
        for (int b = 0; b < B; ++b) {
            int q = a.q0[b];
            if (q < 0 || q >= V) {
                if (lane == 0 && wg == 0) atomicOr(m.err, kErrBadQ0);
                q = 0;
            }
            fed[b] = q;
            const float4* hr = reinterpret_cast<const float4*>(a.H + static_cast<size_t>(b) * DT);
            for (int k = lane; k < DT / 4; k += 64) reinterpret_cast<float4*>(slot[0] + b * DT)[k] = hr[k];
        }
        if (eb < B) es = emb_elem(m, 0, fed[eb], ek);
        __syncthreads();
        int ph = 1;
        auto decide = [&](int s_prev) {
            // tokens of step s_prev from the key records; returns via fed[]
            const uint32_t lt = tag_of(ph_lm(L, s_prev));
            for (int b = 0; b < B; ++b) {
                const int tok = poll_argmax(rc.KEY, b, lt, m.err);
                if (wg == 0 && lane == 0) a.tok_out[b * kSteps + (s_prev - 1)] = tok;
                int f = a.force ? a.force[b * kSteps + (s_prev - 1)] : tok;
                if (f < 0 || f >= V) {
                    if (wg == 0 && lane == 0) atomicOr(m.err, kErrBadForced);
                    f = 0;
                }
                fed[b] = f;
            }
        };
        for (int s = 1; s <= kSteps; ++s) {
            const int M = (s == 1) ? 2 * B : B;
            for (int l = 0; l < L; ++l) {
                // ---- QKV(l): x rows
                {
                    float* dst = slot[ph & 1];
                    if (l == 0) {
                        if (s == 1) {
                            for (int b = 0; b < B; ++b) poll_vec<DP / 64>(rc.X + b * DP, tag_of(0), dst + b * DP, m.err);
                        } else {
                            decide(s - 1);
                            if (eb < B) es += emb_elem(m, s - 1, fed[eb], ek);
                        }
                        const int r0 = (s == 1) ? B : 0;
                        for (int b = 0; b < B; ++b) {
                            const float4* prow =
                                reinterpret_cast<const float4*>(m.ptab + (static_cast<size_t>(s - 1) * V + fed[b]) * DP);
                            float4* d4 = reinterpret_cast<float4*>(dst + (r0 + b) * DP);
#pragma unroll
                            for (int i = 0; i < DP / 256; ++i) d4[lane + 64 * i] = prow[lane + 64 * i];
                        }
                    } else {
                        const uint32_t t = tag_of(ph_layer(L, s, l - 1, T_DOWN));
                        for (int r = 0; r < M; ++r) poll_vec<DP / 64>(rc.X + r * DP, t, dst + r * DP, m.err);
                    }
                    for (int r = 0; r < M; ++r) {
                        const float t = lds_sumsq(dst + r * DP, DP);
                        if (lane == 0) ssq[ph & 1][r] = t;
                    }
                    __syncthreads();
                    ++ph;
                }
                // ---- ATTN(l): q/k/v head vectors of the unit + cached keys/values
                {
                    float* dst = slot[ph & 1];
                    if (wg < B * NKV) {
                        const int b = wg / NKV, g = wg % NKV;
                        const int pf = (s == 1) ? 0 : s;
                        const size_t kvb = ((static_cast<size_t>(l) * m.max_batch + b) * kPositions) * NKV * HD;
                        // cached keys/values of earlier positions: LDS-direct loads,
                        // all in flight while the new head vectors are polled
                        for (int t = 0; t < pf; ++t) {
                            const size_t off = kvb + (static_cast<size_t>(t) * NKV + g) * HD;
                            dma64(m.kc + off, dst + t * HD);
                            dma64(m.kc + off + 64, dst + t * HD + 64);
                            dma64(m.vc + off, dst + 2048 + t * HD);
                            dma64(m.vc + off + 64, dst + 2048 + t * HD + 64);
                        }
                        const uint32_t qt = tag_of(ph_layer(L, s, l, T_QKV));
                        poll_heads(rc.QKV + static_cast<size_t>(b) * NQKV, g, qt, dst + 4096, m.err);
                        if (s == 1) poll_heads(rc.QKV + static_cast<size_t>(B + b) * NQKV, g, qt, dst + 4096 + 512, m.err);
                        __builtin_amdgcn_s_waitcnt(0);
                    }
                    __syncthreads();
                    ++ph;
                }
                // ---- O(l): attention output rows
                {
                    const uint32_t t = tag_of(ph_layer(L, s, l, T_ATTN));
                    for (int r = 0; r < M; ++r) poll_vec<QD / 64>(rc.AO + r * QD, t, slot[ph & 1] + r * QD, m.err);
                    __syncthreads();
                    ++ph;
                }
                // ---- UP(l): x rows after the attention residual
                {
                    const uint32_t t = tag_of(ph_layer(L, s, l, T_O));
                    float* dst = slot[ph & 1];
                    for (int r = 0; r < M; ++r) poll_vec<DP / 64>(rc.X + r * DP, t, dst + r * DP, m.err);
                    for (int r = 0; r < M; ++r) {
                        const float q = lds_sumsq(dst + r * DP, DP);
                        if (lane == 0) ssq[ph & 1][r] = q;
                    }
                    __syncthreads();
                    ++ph;
                }
                // ---- DOWN(l): SwiGLU rows
                {
                    const uint32_t t = tag_of(ph_layer(L, s, l, T_UP));
                    for (int r = 0; r < M; ++r) poll_vec<F / 64>(rc.H + r * F, t, slot[ph & 1] + r * F, m.err);
                    __syncthreads();
                    ++ph;
                }
            }
            // ---- LM(s): the rows at position s
            {
                const int r0 = (s == 1) ? B : 0;
                const uint32_t t = tag_of(ph_layer(L, s, L - 1, T_DOWN));
                float* dst = slot[ph & 1];
                for (int b = 0; b < B; ++b) poll_vec<DP / 64>(rc.X + (r0 + b) * DP, t, dst + b * DP, m.err);
                for (int b = 0; b < B; ++b) {
                    const float q = lds_sumsq(dst + b * DP, DP);
                    if (lane == 0) ssq[ph & 1][b] = q;
                }
                __syncthreads();
                ++ph;
            }
        }
        // ---- FINAL: last token, embedding sum out
        decide(kSteps);
        if (eb < B) {
            es += emb_elem(m, kSteps, fed[eb], ek);
            a.embsum[static_cast<size_t>(eb) * DT + ek] = es;
        }
        return;
    }

    // ======================= compute waves =======================
    const int gw = wg * kCW + wave;
    const int ctid = threadIdx.x;  // 0 .. 255 over the compute waves
    uint4 wP[4], wQ[8], wO[4], wU[12], wD[6], wL[4];
    float xr[MR];

    const uint32_t lane16 = static_cast<uint32_t>(lane) * 16u;
    auto load_wQ = [&](int l) {
        const rsrc_t W = wrsrc(LD[l].qkv.w, NQKV * DP * 2);
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int c = 0; c < 2; ++c) wQ[q * 2 + c] = ldw(W, 16 * wg + 4 * wave + q, DP, c, lane16);
    };
    auto load_wO = [&](int l) {
        const rsrc_t W = wrsrc(LD[l].o.w, DP * QD * 2);
#pragma unroll
        for (int c = 0; c < 4; ++c) wO[c] = ldw(W, 4 * wg + wave, QD, c, lane16);
    };
    auto load_wU = [&](int l) {
        const rsrc_t Wg = wrsrc(LD[l].gate.w, F * DP * 2);
        const rsrc_t Wu = wrsrc(LD[l].up.w, F * DP * 2);
#pragma unroll
        for (int q = 0; q < 3; ++q)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                wU[q * 2 + c] = ldw(Wg, 12 * wg + 3 * wave + q, DP, c, lane16);
                wU[6 + q * 2 + c] = ldw(Wu, 12 * wg + 3 * wave + q, DP, c, lane16);
            }
    };
    auto load_wD = [&](int l) {
        const rsrc_t W = wrsrc(LD[l].down.w, DP * F * 2);
#pragma unroll
        for (int c = 0; c < 6; ++c) wD[c] = ldw(W, 4 * wg + wave, F, c, lane16);
    };
    auto load_wL = [&](int s) {
        const rsrc_t W = wrsrc(m.lm[s - 1].w, V * DP * 2);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int c = 0; c < 2; ++c) wL[q * 2 + c] = ldw(W, 8 * wg + 2 * wave + q, DP, c, lane16);
    };
    // select vals[t] for a lane-dependent t (vals is a small register array)
    auto pick = [&](const float* vals, int count, int t) {
        float v = 0.f;
#pragma unroll
        for (int i = 0; i < 4 * MR; ++i)
            if (i < count && i == t) v = vals[i];
        return v;
    };
    // gain-weighted activations for k = c*512 + lane*8 .. +7
    auto act8 = [&](const float* xrow, const float* g, int c, float x8[8]) {
        float g8[8];
        lds8(xrow + c * 512 + lane * 8, x8);
        lds8(g + c * 512 + lane * 8, g8);
#pragma unroll
        for (int j = 0; j < 8; ++j) x8[j] *= g8[j];
    };

    // kernel start: weights of the first two phases in flight, then the RoPE
    // and norm-gain tables into LDS
    {
        const rsrc_t W = wrsrc(m.proj.w, DP * DT * 2);
#pragma unroll
        for (int c = 0; c < 4; ++c) wP[c] = ldw(W, 4 * wg + wave, DT, c, lane16);
    }
    load_wQ(0);
    sched_fence();
    for (int i = ctid; i < kPositions * (HD / 2); i += kCW * 64) {
        rope_s[0][i] = m.rope_cos[i];
        rope_s[1][i] = m.rope_sin[i];
    }
    for (int l = 0; l < L; ++l)
        for (int i = ctid; i < DP; i += kCW * 64) {
            gains[(2 * l) * DP + i] = LD[l].attn_norm[i];
            gains[(2 * l + 1) * DP + i] = LD[l].ffn_norm[i];
        }
    for (int i = ctid; i < DP; i += kCW * 64) gains[2 * kMaxL * DP + i] = m.out_norm[i];
    for (int l = 0; l < L; ++l)
        for (int i = ctid; i < HD; i += kCW * 64) {
            gains[(2 * kMaxL + 1) * DP + (2 * l) * HD + i] = LD[l].q_norm[i];
            gains[(2 * kMaxL + 1) * DP + (2 * l + 1) * HD + i] = LD[l].k_norm[i];
        }

    // ---- INIT: x rows at position 0 = W_p . H + b_p
    __syncthreads();
    int ph = 0;
    {
        const float* Hs = slot[0];
        float acc[MR / 2];
#pragma unroll
        for (int r = 0; r < MR / 2; ++r) acc[r] = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int r = 0; r < MR / 2; ++r) {
                if (r < B) {
                    float x8[8];
                    lds8(Hs + r * DT + c * 512 + lane * 8, x8);
                    acc[r] = dot8(wP[c], x8, acc[r]);
                }
            }
        const int n = 4 * wg + wave;
        const float bias = m.proj_b[n];
#pragma unroll
        for (int r = 0; r < MR / 2; ++r) {
            if (r < B) {
                const float v = wave_sum(acc[r]) + bias;
                if (lane == r) st_rec(rc.X + static_cast<size_t>(r) * DP + n, v, tag_of(0));
            }
        }
    }
    ph = 1;

    for (int s = 1; s <= kSteps; ++s) {
        const int M = (s == 1) ? 2 * B : B;
        for (int l = 0; l < L; ++l) {
            // ================= QKV(l) =================
            __syncthreads();
            {
                const float* xs = slot[ph & 1];
                const float* ss = ssq[ph & 1];
                if (l == 0) {
#pragma unroll
                    for (int r = 0; r < MR; ++r) xr[r] = (r < M) ? xs[r * DP + 4 * wg + wave] : 0.f;
                }
                float acc[4 * MR];
#pragma unroll
                for (int i = 0; i < 4 * MR; ++i) acc[i] = 0.f;
#pragma unroll
                for (int c = 0; c < 2; ++c) {
#pragma unroll
                    for (int r = 0; r < MR; ++r) {
                        if (r < M) {
                            float x8[8];
                            act8(xs + r * DP, g_attn(l), c, x8);
#pragma unroll
                            for (int q = 0; q < 4; ++q) acc[q * MR + r] = dot8(wQ[q * 2 + c], x8, acc[q * MR + r]);
                        }
                    }
                    sched_fence();
                }
                float res[4 * MR];
#pragma unroll
                for (int r = 0; r < MR; ++r) {
                    const float rinv = (r < M) ? 1.0f / sqrtf(ss[r] / static_cast<float>(DP) + eps) : 0.f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) res[q * MR + r] = (r < M) ? wave_sum(acc[q * MR + r]) * rinv : 0.f;
                }
                if (lane < 4 * M) {
                    const int q = lane / M, r = lane - q * M;
                    st_rec(rc.QKV + static_cast<size_t>(r) * NQKV + 16 * wg + 4 * wave + q,
                           pick(res, 4 * MR, q * MR + r), tag_of(ph));
                }
            }
            ++ph;
            // ================= ATTN(l) =================
            __syncthreads();
            load_wO(l);
            sched_fence();
            if (wg < B * NKV && wave < 2) {
                const float* sl = slot[ph & 1];
                const int b = wg / NKV, g = wg % NKV, h = 2 * g + wave;
                const int pf = (s == 1) ? 0 : s;
                const int npos = (s == 1) ? 2 : 1;
                const size_t kvb = ((static_cast<size_t>(l) * m.max_batch + b) * kPositions) * NKV * HD;
                const float* gq = g_q(l);
                const float* gk = g_k(l);
                float kn[2][2] = {{0.f, 0.f}, {0.f, 0.f}}, vn[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
#pragma unroll
                for (int pi = 0; pi < 2; ++pi) {
                    if (pi >= npos) break;
                    const int p = pf + pi;
                    const int r = (s == 1) ? pi * B + b : b;
                    const float* nd = sl + 4096 + pi * 512;
                    const float c0 = rope_s[0][p * (HD / 2) + lane], s0 = rope_s[1][p * (HD / 2) + lane];
                    {   // key: per-head RMSNorm, rotate-half RoPE (pair lane, lane+64)
                        const float k0 = nd[256 + lane], k1 = nd[256 + lane + 64];
                        const float rv = 1.0f / sqrtf(wave_sum(k0 * k0 + k1 * k1) / static_cast<float>(HD) + eps);
                        const float a0 = gk[lane] * (k0 * rv), a1 = gk[lane + 64] * (k1 * rv);
                        kn[pi][0] = a0 * c0 - a1 * s0;
                        kn[pi][1] = a1 * c0 + a0 * s0;
                        vn[pi][0] = nd[384 + lane];
                        vn[pi][1] = nd[384 + lane + 64];
                    }
                    if (wave == 0) {
                        const size_t off = kvb + (static_cast<size_t>(p) * NKV + g) * HD;
                        st_act(m.kc + off + lane, kn[pi][0]);
                        st_act(m.kc + off + lane + 64, kn[pi][1]);
                        st_act(m.vc + off + lane, vn[pi][0]);
                        st_act(m.vc + off + lane + 64, vn[pi][1]);
                    }
                    float q0v, q1v;
                    {
                        const float x0 = nd[wave * HD + lane], x1 = nd[wave * HD + lane + 64];
                        const float rv = 1.0f / sqrtf(wave_sum(x0 * x0 + x1 * x1) / static_cast<float>(HD) + eps);
                        const float a0 = gq[lane] * (x0 * rv), a1 = gq[lane + 64] * (x1 * rv);
                        q0v = a0 * c0 - a1 * s0;
                        q1v = a1 * c0 + a0 * s0;
                    }
                    float sc[kPositions];
                    float mx = -__builtin_huge_valf();
#pragma unroll
                    for (int t = 0; t < kPositions; ++t) {
                        if (t <= p) {
                            float d;
                            if (t < pf) {
                                d = q0v * sl[t * HD + lane] + q1v * sl[t * HD + lane + 64];
                            } else {
                                const bool j0 = (t == pf);
                                d = q0v * (j0 ? kn[0][0] : kn[1][0]) + q1v * (j0 ? kn[0][1] : kn[1][1]);
                            }
                            d = wave_sum(d) * m.attn_scale;
                            sc[t] = d;
                            mx = fmaxf(mx, d);
                        }
                    }
                    float den = 0.f;
#pragma unroll
                    for (int t = 0; t < kPositions; ++t)
                        if (t <= p) {
                            sc[t] = expf(sc[t] - mx);
                            den += sc[t];
                        }
                    float o0 = 0.f, o1 = 0.f;
#pragma unroll
                    for (int t = 0; t < kPositions; ++t) {
                        if (t <= p) {
                            const float pt = sc[t] / den;
                            float v0, v1;
                            if (t < pf) {
                                v0 = sl[2048 + t * HD + lane];
                                v1 = sl[2048 + t * HD + lane + 64];
                            } else {
                                const bool j0 = (t == pf);
                                v0 = j0 ? vn[0][0] : vn[1][0];
                                v1 = j0 ? vn[0][1] : vn[1][1];
                            }
                            o0 = fmaf(pt, v0, o0);
                            o1 = fmaf(pt, v1, o1);
                        }
                    }
                    uint64_t* orow = rc.AO + static_cast<size_t>(r) * QD + h * HD;
                    st_rec(orow + lane, o0, tag_of(ph));
                    st_rec(orow + lane + 64, o1, tag_of(ph));
                }
            }
            ++ph;
            // ================= O(l) =================
            __syncthreads();
            load_wU(l);
            sched_fence();
            {
                const float* as = slot[ph & 1];
                float acc[MR];
#pragma unroll
                for (int r = 0; r < MR; ++r) acc[r] = 0.f;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
#pragma unroll
                    for (int r = 0; r < MR; ++r)
                        if (r < M) {
                            float x8[8];
                            lds8(as + r * QD + c * 512 + lane * 8, x8);
                            acc[r] = dot8(wO[c], x8, acc[r]);
                        }
                    sched_fence();
                }
                const int n = 4 * wg + wave;
                float res[MR];
#pragma unroll
                for (int r = 0; r < MR; ++r) {
                    res[r] = 0.f;
                    if (r < M) {
                        xr[r] += wave_sum(acc[r]);
                        res[r] = xr[r];
                    }
                }
                if (lane < M) st_rec(rc.X + static_cast<size_t>(lane) * DP + n, pick(res, MR, lane), tag_of(ph));
            }
            ++ph;
            // ================= UP(l) =================
            __syncthreads();
            load_wD(l);
            sched_fence();
            {
                const float* xs = slot[ph & 1];
                const float* ss = ssq[ph & 1];
                float ag[3 * MR], au[3 * MR];
#pragma unroll
                for (int i = 0; i < 3 * MR; ++i) { ag[i] = 0.f; au[i] = 0.f; }
#pragma unroll
                for (int c = 0; c < 2; ++c) {
#pragma unroll
                    for (int r = 0; r < MR; ++r)
                        if (r < M) {
                            float x8[8];
                            act8(xs + r * DP, g_ffn(l), c, x8);
#pragma unroll
                            for (int q = 0; q < 3; ++q) {
                                ag[q * MR + r] = dot8(wU[q * 2 + c], x8, ag[q * MR + r]);
                                au[q * MR + r] = dot8(wU[6 + q * 2 + c], x8, au[q * MR + r]);
                            }
                        }
                    sched_fence();
                }
                float res[3 * MR];
#pragma unroll
                for (int r = 0; r < MR; ++r) {
                    const float rinv = (r < M) ? 1.0f / sqrtf(ss[r] / static_cast<float>(DP) + eps) : 0.f;
#pragma unroll
                    for (int q = 0; q < 3; ++q) {
                        res[q * MR + r] = 0.f;
                        if (r < M) {
                            const float gv = wave_sum(ag[q * MR + r]) * rinv;
                            const float uv = wave_sum(au[q * MR + r]) * rinv;
                            res[q * MR + r] = (gv / (1.0f + expf(-gv))) * uv;
                        }
                    }
                }
                if (lane < 3 * M) {
                    const int q = lane / M, r = lane - q * M;
                    st_rec(rc.H + static_cast<size_t>(r) * F + 12 * wg + 3 * wave + q, pick(res, 3 * MR, q * MR + r),
                           tag_of(ph));
                }
            }
            ++ph;
            // ================= DOWN(l) =================
            __syncthreads();
            if (l + 1 < L) load_wQ(l + 1); else load_wL(s);
            sched_fence();
            {
                const float* hs = slot[ph & 1];
                float acc[MR];
#pragma unroll
                for (int r = 0; r < MR; ++r) acc[r] = 0.f;
#pragma unroll
                for (int c = 0; c < 6; ++c) {
#pragma unroll
                    for (int r = 0; r < MR; ++r)
                        if (r < M) {
                            float x8[8];
                            lds8(hs + r * F + c * 512 + lane * 8, x8);
                            acc[r] = dot8(wD[c], x8, acc[r]);
                        }
                    sched_fence();
                }
                const int n = 4 * wg + wave;
                float res[MR];
#pragma unroll
                for (int r = 0; r < MR; ++r) {
                    res[r] = 0.f;
                    if (r < M) {
                        xr[r] += wave_sum(acc[r]);
                        res[r] = xr[r];
                    }
                }
                if (lane < M) {
                    const float v = pick(res, MR, lane);
                    st_rec(rc.X + static_cast<size_t>(lane) * DP + n, v, tag_of(ph));
                    if (a.taps) {
                        const int pos = (s == 1) ? (lane >= B ? 1 : 0) : s;
                        const int b = (s == 1 && lane >= B) ? lane - B : lane;
                        a.taps[((static_cast<size_t>(pos) * L + l) * B + b) * DP + n] = v;
                    }
                }
            }
            ++ph;
        }
        // ================= LM(s) =================
        __syncthreads();
        if (s < kSteps) load_wQ(0);
        sched_fence();
        {
            const float* xs = slot[ph & 1];
            const float* ss = ssq[ph & 1];
            constexpr int BM = MR / 2;
            float acc[2 * BM];
#pragma unroll
            for (int i = 0; i < 2 * BM; ++i) acc[i] = 0.f;
#pragma unroll
            for (int b = 0; b < BM; ++b)
                if (b < B) {
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        float x8[8];
                        act8(xs + b * DP, g_out, c, x8);
#pragma unroll
                        for (int q = 0; q < 2; ++q) acc[q * BM + b] = dot8(wL[q * 2 + c], x8, acc[q * BM + b]);
                    }
                }
            const int v0 = 8 * wg + 2 * wave;
#pragma unroll
            for (int b = 0; b < BM; ++b) {
                if (b < B) {
                    const float rinv = 1.0f / sqrtf(ss[b] / static_cast<float>(DP) + eps);
                    const float l0 = wave_sum(acc[b]) * rinv;
                    const float l1 = wave_sum(acc[BM + b]) * rinv;
                    if (a.logits_out && lane < 2)
                        a.logits_out[(static_cast<size_t>(b) * kSteps + (s - 1)) * V + v0 + lane] = lane ? l1 : l0;
                    const bool second = ordered_bits(l1) > ordered_bits(l0);
                    const uint32_t ob = ordered_bits(second ? l1 : l0);
                    const uint32_t idx = static_cast<uint32_t>(v0 + (second ? 1 : 0));
                    uint64_t* kr = rc.KEY + (static_cast<size_t>(b) * kGW + gw) * 2;
                    if (lane == 0) st_rec_u(kr, ob, tag_of(ph));
                    if (lane == 1) st_rec_u(kr + 1, idx, tag_of(ph));
                }
            }
        }
        ++ph;
    }
}

}  // namespace stream
}  // namespace qp

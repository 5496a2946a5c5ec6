// Dataflow frame kernel for small batches (B <= 2) of the 1.7B-shaped
// predictor with bf16 weights, or Q8_0 / Q4_0 weights held as int8 codes
// with fp32 block scales.
//
// One persistent workgroup of four waves per CU (256) and no grid barrier:
//  * every value that crosses workgroups is published as a 64-bit record
//    (epoch << 32 | fp32 bits) with a device-scope store; the epoch is unique
//    per phase instance, so a consumer knows a value is current by its tag;
//  * at the start of a phase the four waves each wait for a quarter of the
//    records the workgroup needs (16-byte device-scope loads, two records per
//    lane), stage them in one of two LDS slots and meet at one workgroup
//    barrier; a single wave cannot pull the inputs fast enough alone;
//  * the matrix-vector products round their activations to bf16 pairs and
//    use the pairwise bf16 dot instruction with fp32 accumulation (the same
//    operand rounding as the batched matrix-core path); norms, softmax,
//    SwiGLU and the residual stream stay fp32;
//  * each phase's weights are requested at the end of the previous phase,
//    right after that phase's records were stored (a CU's memory requests
//    drain roughly in order, so a store issued behind a weight burst would
//    leave only after the burst), and land while the inputs are awaited.
// Ownership (256 workgroups x 4 waves = 1024 waves):
//    q/k/v rows 16*wg + 4*w + {0..3}, O / down / projection row 4*wg + w,
//    gate/up rows 12*wg + 3*w + {0..2}, lm_head rows 8*wg + 2*w + {0,1},
//    attention unit (request b, kv head g) on workgroup b*8 + g,
//    embedding-sum elements 8*wg .. 8*wg+7 (wave 3).
#pragma once

#include "qp_common.h"
#include "qp_phases.h"

namespace qp {
namespace stream {

// the Qwen3-TTS 1.7B code-predictor geometry
constexpr int DT = 2048, DP = 1024, NQ = 16, NKV = 8, HD = 128, F = 3072, V = 2048;
constexpr int QD = NQ * HD, NQKV = (NQ + 2 * NKV) * HD;
constexpr int kW = 4;                    // waves per workgroup
constexpr int kThreadsS = kW * 64;
constexpr int kNwg = 256;
static_assert(NQKV == 16 * kNwg && DP == 4 * kNwg && F == 12 * kNwg && V == 8 * kNwg && DT == 8 * kNwg,
              "row ownership assumes the 1.7B predictor geometry");

// INIT, then per step 5 phases per layer and the lm_head, then FINAL
__host__ __device__ constexpr int phases_per_frame(int L) { return 1 + kSteps * (5 * L + 1) + 1; }
__host__ __device__ constexpr int slot_floats(int MR) { return MR * F; }

struct Recs {
    uint64_t* X;    // [MR][DP]
    uint64_t* QKV;  // [MR][NQKV]
    uint64_t* AO;   // [MR][QD]
    uint64_t* H;    // [MR][F]
    uint64_t* KEY;  // [Bmax][kNwg][2]: ordered logit bits, vocabulary index
};

__device__ __forceinline__ void st_rec(uint64_t* p, float v, uint32_t tag) {
    const uint64_t u = (static_cast<uint64_t>(tag) << 32) | __float_as_uint(v);
    __hip_atomic_store(p, u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_rec_u(uint64_t* p, uint32_t v, uint32_t tag) {
    const uint64_t u = (static_cast<uint64_t>(tag) << 32) | v;
    __hip_atomic_store(p, u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// frame-relative phase indices
__device__ __forceinline__ int ph_layer(int L, int s, int l, int t) { return 1 + (s - 1) * (5 * L + 1) + 5 * l + t; }
__device__ __forceinline__ int ph_lm(int L, int s) { return 1 + (s - 1) * (5 * L + 1) + 5 * L; }
enum { T_QKV = 0, T_ATTN = 1, T_O = 2, T_UP = 3, T_DOWN = 4 };

__device__ __forceinline__ bool timed_out(const unsigned* err) {
    return __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kErrBarrierTimeout;
}

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

// Weights stream through buffer loads: the matrix base lives in a scalar
// resource (with the matrix size as its bound), the lane offset in one VGPR,
// the row offset in an SGPR, so no per-row 64-bit addresses are kept.
using rsrc_t = __amdgpu_buffer_rsrc_t;
// A pointer read from LDS is, to the compiler, a per-lane value; every lane
// holds the same one, so move it to scalar registers.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
    return reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ const float* uniform_f(const float* p) {
    return static_cast<const float*>(uniform_ptr(p));
}
__device__ __forceinline__ rsrc_t wrsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0), static_cast<int>(bytes),
                                             0x00020000);
}
// A weight matrix as buffer resources: the values (bf16, or int8 codes) and,
// for the block formats, the fp32 scales [N][K/32].
struct WSrc {
    rsrc_t w, s;
};
template <int WT>
__device__ __forceinline__ WSrc wsrc(const void* w, const float* scale, int N, int K) {
    if constexpr (WT == WT_BF16) {
        const rsrc_t r = wrsrc(w, N * K * 2);
        return {r, r};
    } else {
        return {wrsrc(w, N * K), wrsrc(scale, N * (K / 32) * 4)};
    }
}
// The 8 weights of row `row` (K wide) at k = kc*512 + lane*8: bf16, or for
// the block formats 8 int8 codes (x, y) and their block's scale (z bits).
template <int WT>
__device__ __forceinline__ uint4 ldw(const WSrc& r, int row, int K, int kc, uint32_t lane16) {
    if constexpr (WT == WT_BF16) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r.w, lane16 + static_cast<uint32_t>(kc) * 1024u,
                                                             static_cast<uint32_t>(row) * static_cast<uint32_t>(K) * 2u, 0);
        return make_uint4(static_cast<uint32_t>(v[0]), static_cast<uint32_t>(v[1]), static_cast<uint32_t>(v[2]),
                          static_cast<uint32_t>(v[3]));
    } else {
        const uint32_t lane = lane16 >> 4;
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r.w, lane * 8u + static_cast<uint32_t>(kc) * 512u,
                                                            static_cast<uint32_t>(row) * static_cast<uint32_t>(K), 0);
        const uint32_t sc = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(
            r.s, ((lane >> 2) + static_cast<uint32_t>(kc) * 16u) * 4u,
            static_cast<uint32_t>(row) * static_cast<uint32_t>(K / 32) * 4u, 0));
        return make_uint4(static_cast<uint32_t>(v[0]), static_cast<uint32_t>(v[1]), sc, 0u);
    }
}

// ---------------------------------------------------------------------------
// waiting for records
// ---------------------------------------------------------------------------

constexpr int kDeviceScope = 16;  // buffer-load cache policy bit: device-coherent

// This wave's quarter of a row of K tagged records: records
// [w*K/4, (w+1)*K/4), two per lane per 16-byte load.  Values go to dst[k]
// (dst = the row's LDS base); returns this wave's part of the row's sum of
// squares (fixed order).
template <int K>
__device__ __forceinline__ float poll_share(const uint64_t* row, int wave, uint32_t tag, float* dst, unsigned* err) {
    constexpr int NJ = K / 512;  // 16-byte loads per lane
    static_assert(NJ >= 1 && NJ <= 16, "row width");
    const int lane = threadIdx.x & 63;
    const rsrc_t r = wrsrc(row + wave * (K / 4), (K / 4) * 8);
    float* d = dst + wave * (K / 4);
    uint32_t pend = (1u << NJ) - 1u;
    float v[2 * NJ];
    unsigned spins = 0;
    while (true) {
        decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0u, 0u, 0)) u[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            if ((pend >> j) & 1u) u[j] = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16u, 1024u * j, kDeviceScope);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if (((pend >> j) & 1u) && static_cast<uint32_t>(u[j][1]) == tag && static_cast<uint32_t>(u[j][3]) == tag) {
                v[2 * j] = __int_as_float(u[j][0]);
                v[2 * j + 1] = __int_as_float(u[j][2]);
                pend &= ~(1u << j);
            }
        }
        if (!__any(pend != 0u)) break;
        if (!spin_wait(spins, err)) break;
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        *reinterpret_cast<float2*>(d + 2 * (lane + 64 * j)) = make_float2(v[2 * j], v[2 * j + 1]);
        ss = fmaf(v[2 * j], v[2 * j], ss);
        ss = fmaf(v[2 * j + 1], v[2 * j + 1], ss);
    }
    return wave_sum(ss);
}

// Wave 0 alone waits until some record of the first NC KiB at rec carries
// tag (one 16-byte load per lane per attempt, its chunks in turn); then all
// waves meet at the barrier.
template <int NC>
__device__ __forceinline__ void gate_rec(const uint64_t* rec, uint32_t tag, unsigned* err) {
    if ((threadIdx.x >> 6) == 0) {
        const int lane = threadIdx.x & 63;
        const rsrc_t r = wrsrc(rec, NC * 1024);
        uint32_t probe = 0;
        unsigned spins = 0;
        while (true) {
            const auto u = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16u, 1024u * probe, kDeviceScope);
            if (__any(static_cast<uint32_t>(u[1]) == tag || static_cast<uint32_t>(u[3]) == tag)) break;
            probe = probe + 1 == NC ? 0 : probe + 1;
            if (!spin_wait(spins, err)) break;
        }
    }
    __syncthreads();
}

// One head vector (HD = 128 tagged records) -> dst[0..128).
__device__ __forceinline__ void poll_head(const uint64_t* src, uint32_t tag, float* dst, unsigned* err) {
    const int lane = threadIdx.x & 63;
    const rsrc_t r = wrsrc(src, HD * 8);
    unsigned spins = 0;
    while (true) {
        const auto u = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16u, 0u, kDeviceScope);
        const bool ok = static_cast<uint32_t>(u[1]) == tag && static_cast<uint32_t>(u[3]) == tag;
        if (__all(ok)) {
            *reinterpret_cast<float2*>(dst + 2 * lane) = make_float2(__int_as_float(u[0]), __int_as_float(u[2]));
            break;
        }
        if (!spin_wait(spins, err)) break;
    }
}

// Token of request b from the per-workgroup key records of one lm_head phase
// (largest logit, lowest index on ties); lane-uniform.
__device__ __forceinline__ int poll_argmax(const uint64_t* key, int b, uint32_t tag, unsigned* err) {
    const int lane = threadIdx.x & 63;
    constexpr int NJ = kNwg / 64;
    const rsrc_t r = wrsrc(key + static_cast<size_t>(b) * kNwg * 2, kNwg * 16);
    uint32_t ord[NJ], idx[NJ];
    uint32_t pend = (1u << NJ) - 1u;
    unsigned spins = 0;
    while (true) {
        decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0u, 0u, 0)) u[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            if ((pend >> j) & 1u) u[j] = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16u, 1024u * j, kDeviceScope);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if (((pend >> j) & 1u) && static_cast<uint32_t>(u[j][1]) == tag && static_cast<uint32_t>(u[j][3]) == tag) {
                ord[j] = static_cast<uint32_t>(u[j][0]);
                idx[j] = static_cast<uint32_t>(u[j][2]);
                pend &= ~(1u << j);
            }
        }
        if (!__any(pend != 0u)) break;
        if (!spin_wait(spins, err)) break;
    }
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const uint64_t k = (static_cast<uint64_t>(ord[j]) << 32) | (0xFFFFFFFFu - idx[j]);
        best = k > best ? k : best;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint64_t o = (static_cast<uint64_t>(__shfl_xor(static_cast<unsigned>(best >> 32), off, 64)) << 32) |
                           __shfl_xor(static_cast<unsigned>(best & 0xFFFFFFFFu), off, 64);
        best = o > best ? o : best;
    }
    return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best & 0xFFFFFFFFu));
}

// 64 consecutive fp32 values (device-coherent) straight into LDS, one per
// lane, without passing through registers: src and dst are wave-uniform.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void gbl_void_t;
__device__ __forceinline__ void dma64(const float* src, float* dst) {
    const int lane = threadIdx.x & 63;
    __builtin_amdgcn_global_load_lds((gbl_void_t*)(src + lane), (lds_void_t*)(dst), 4, 0, kDeviceScope);
}

// The cached keys and values of positions 0 .. pf-1 of one (request, kv head)
// (rows of HD floats, position stride NKV * HD in the cache) into LDS: keys
// at hist[t * HD], values at hist[2048 + t * HD].  16 bytes per lane, so one
// load moves two positions' rows (lanes 32..63 the second); the loads are
// dealt round-robin over the nw waves from wave w0.  With pf odd, the last
// load's upper half re-reads row pf - 1 into row pf, which the caller
// overwrites with the current position after its barrier.
__device__ __forceinline__ void hist_dma(const float* kc, const float* vc, size_t kvb, int g, int pf, float* hist,
                                         int wave, int w0, int nw) {
    const int lane = threadIdx.x & 63;
    const int np = (pf + 1) >> 1;             // loads per matrix
    for (int i = wave - w0; i < 2 * np; i += nw) {
        if (i < 0) continue;
        const int j = i < np ? i : i - np;     // position pair
        const int tt = min(2 * j + (lane >> 5), pf - 1);
        const float* src = (i < np ? kc : vc) + kvb + (static_cast<size_t>(tt) * NKV + g) * HD + (lane & 31) * 4;
        float* dst = hist + (i < np ? 0 : 2048) + 2 * j * HD;
        __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)dst, 16, 0, kDeviceScope);
    }
}

// ---------------------------------------------------------------------------
// compute side helpers
// ---------------------------------------------------------------------------

// activations packed to bf16 pairs (round to nearest even), element 2i in
// the low half: the operand order of the weights' bf16 pairs
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void pack8(const float a[8], bf16x2_t p[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_convertvector(f32x2_t{a[2 * i], a[2 * i + 1]}, bf16x2_t);
}
// acc + w . a over 8 bf16 products (pairwise dot instructions)
__device__ __forceinline__ float dot8p(const uint4 w, const bf16x2_t p[4], float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x), p[0], acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y), p[1], acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z), p[2], acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w), p[3], acc, false);
    return acc;
}

// acc + w . x over 8 weights: bf16 weights against the activations' bf16
// pairs (p), or int8 codes (exact in fp32) against the fp32 activations (x),
// the block's sum times its scale
template <int WT>
__device__ __forceinline__ float wdot8(const uint4 w, const float x[8], const bf16x2_t p[4], float acc) {
    if constexpr (WT == WT_BF16) {
        return dot8p(w, p, acc);
    } else {
        const uint32_t c[2] = {w.x, w.y};
        float blk = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            blk = fmaf(static_cast<float>(static_cast<int8_t>((c[i >> 2] >> (8 * (i & 3))) & 0xFFu)), x[i], blk);
        return fmaf(__uint_as_float(w.z), blk, acc);
    }
}
// the activations' bf16 pairs, needed by the bf16 products only
template <int WT>
__device__ __forceinline__ void pack8w(const float a[8], bf16x2_t p[4]) {
    if constexpr (WT == WT_BF16) pack8(a, p);
}

__device__ __forceinline__ void lds8(const float* p, float a[8]) {
    const float4 u = *reinterpret_cast<const float4*>(p);
    const float4 v = *reinterpret_cast<const float4*>(p + 4);
    a[0] = u.x; a[1] = u.y; a[2] = u.z; a[3] = u.w;
    a[4] = v.x; a[5] = v.y; a[6] = v.z; a[7] = v.w;
}

__device__ __forceinline__ uint32_t ordered_bits(float v) {
    uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

constexpr int kMaxL = 5;  // layers whose norm gains fit the LDS table
// LDS gain table: attn_norm[l], ffn_norm[l] (DP each), out_norm (DP), then
// q_norm[l], k_norm[l] (HD each)
constexpr int kGainFloats = (2 * kMaxL + 1) * DP + 2 * kMaxL * HD;

template <int MR, int WT>
__global__ __launch_bounds__(kThreadsS) void k_stream(Model m, RunArgs a, Recs rc) {
    constexpr int BM = MR / 2;  // requests
    constexpr int SLOT = slot_floats(MR);
    __shared__ float slot[2][SLOT];
    __shared__ float ssp[2][kW][MR];          // per-wave partial sums of squares
    __shared__ uint64_t lmk[kW][BM];          // per-wave lm_head keys
    __shared__ __align__(16) float rope_s[2][kPositions * (HD / 2)];
    __shared__ __align__(16) float gains[kGainFloats];
    __shared__ LayerDev lay_s[kMaxL];
    // the tokens fed at codebooks 0..15 (q0, then each step's), per request:
    // the embedding sum gathers its 16 rows once, at the end of the frame,
    // instead of one dependent load per step on the step's critical path
    __shared__ int tok_s[kSteps + 1][BM];

    const int wg = blockIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int lane = threadIdx.x & 63;
    const int B = a.B;
    const int L = m.L;
    const uint32_t seq0 = a.seq0;
    auto tag_of = [&](int ph) { return seq0 + static_cast<uint32_t>(ph) + 1u; };
    const float eps = m.eps;
    unsigned* err = m.err;
    // layer 0's q/k/v rows of every table row P_j[v] (j = 1..14), computed at
    // create time: from step 2 on, layer 0 takes its head vectors from here
    const float* t0 = m.qkv0;

    // ---- tables into LDS: layer pointers, norm gains, RoPE.  The tables go
    // straight into LDS, 16 bytes per lane, every request issued before any
    // is awaited; they are complete at the barrier that ends INIT's staging
    // (a wait for every load in flight precedes it).
    auto dma_tab = [&](const float* src, float* dst, int n) {   // n: a multiple of 4 floats
        for (int o = wave * 256; o < n; o += kW * 256)
            if (o + 4 * lane < n)
                __builtin_amdgcn_global_load_lds((gbl_void_t*)(src + o + 4 * lane), (lds_void_t*)(dst + o), 16, 0, 0);
    };
    dma_tab(m.rope_cos, rope_s[0], kPositions * (HD / 2));
    dma_tab(m.rope_sin, rope_s[1], kPositions * (HD / 2));
    dma_tab(m.out_norm, gains + 2 * kMaxL * DP, DP);
    if (threadIdx.x < L) lay_s[threadIdx.x] = m.layers[threadIdx.x];
    __syncthreads();
    const LayerDev* LD = lay_s;
    for (int l = 0; l < L; ++l) {
        dma_tab(LD[l].attn_norm, gains + (2 * l) * DP, DP);
        dma_tab(LD[l].ffn_norm, gains + (2 * l + 1) * DP, DP);
        dma_tab(LD[l].q_norm, gains + (2 * kMaxL + 1) * DP + (2 * l) * HD, HD);
        dma_tab(LD[l].k_norm, gains + (2 * kMaxL + 1) * DP + (2 * l + 1) * HD, HD);
    }
    auto g_attn = [&](int l) { return gains + (2 * l) * DP; };
    auto g_ffn = [&](int l) { return gains + (2 * l + 1) * DP; };
    const float* g_out = gains + 2 * kMaxL * DP;
    auto g_q = [&](int l) { return gains + (2 * kMaxL + 1) * DP + (2 * l) * HD; };
    auto g_k = [&](int l) { return gains + (2 * kMaxL + 1) * DP + (2 * l + 1) * HD; };

    // ---- weights in registers, one phase ahead
    const uint32_t lane16 = static_cast<uint32_t>(lane) * 16u;
    uint4 wP[4], wQ[8], wO[4], wU[12], wD[6], wL[4];
    auto load_wQ = [&](int l) {
        const WSrc W = wsrc<WT>(uniform_ptr(LD[l].qkv.w), uniform_f(LD[l].qkv.scale), NQKV, DP);
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int c = 0; c < 2; ++c) wQ[q * 2 + c] = ldw<WT>(W, 16 * wg + 4 * wave + q, DP, c, lane16);
    };
    auto load_wO = [&](int l) {
        const WSrc W = wsrc<WT>(uniform_ptr(LD[l].o.w), uniform_f(LD[l].o.scale), DP, QD);
#pragma unroll
        for (int c = 0; c < 4; ++c) wO[c] = ldw<WT>(W, 4 * wg + wave, QD, c, lane16);
    };
    auto load_wU = [&](int l) {
        const WSrc Wg = wsrc<WT>(uniform_ptr(LD[l].gate.w), uniform_f(LD[l].gate.scale), F, DP);
        const WSrc Wu = wsrc<WT>(uniform_ptr(LD[l].up.w), uniform_f(LD[l].up.scale), F, DP);
#pragma unroll
        for (int q = 0; q < 3; ++q)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                wU[q * 2 + c] = ldw<WT>(Wg, 12 * wg + 3 * wave + q, DP, c, lane16);
                wU[6 + q * 2 + c] = ldw<WT>(Wu, 12 * wg + 3 * wave + q, DP, c, lane16);
            }
    };
    auto load_wD = [&](int l) {
        const WSrc W = wsrc<WT>(uniform_ptr(LD[l].down.w), uniform_f(LD[l].down.scale), DP, F);
#pragma unroll
        for (int c = 0; c < 6; ++c) wD[c] = ldw<WT>(W, 4 * wg + wave, F, c, lane16);
    };
    auto load_wL = [&](int s) {
        const WSrc W = wsrc<WT>(m.lm[s - 1].w, m.lm[s - 1].scale, V, DP);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int c = 0; c < 2; ++c) wL[q * 2 + c] = ldw<WT>(W, 8 * wg + 2 * wave + q, DP, c, lane16);
    };
    {
        const WSrc W = wsrc<WT>(m.proj.w, m.proj.scale, DP, DT);
#pragma unroll
        for (int c = 0; c < 4; ++c) wP[c] = ldw<WT>(W, 4 * wg + wave, DT, c, lane16);
    }
    load_wQ(0);
    sched_fence();

    // gain-weighted activations for k = c*512 + lane*8 .. +7
    auto act8 = [&](const float* xrow, const float* g, int c, float x8[8]) {
        float g8[8];
        lds8(xrow + c * 512 + lane * 8, x8);
        lds8(g + c * 512 + lane * 8, g8);
#pragma unroll
        for (int j = 0; j < 8; ++j) x8[j] *= g8[j];
    };
    // sum of squares of LDS row r after the barrier: fixed order over waves
    auto row_ss = [&](int par, int r) { return ((ssp[par][0][r] + ssp[par][1][r]) + ssp[par][2][r]) + ssp[par][3][r]; };
    // x rows of the next phase: each wave waits for its quarter
    auto gather_x = [&](const uint64_t* base, int nrows, uint32_t tg, int par) {
        for (int r = 0; r < nrows; ++r) {
            const float q = poll_share<DP>(base + static_cast<size_t>(r) * DP, wave, tg, slot[par] + r * DP, err);
            if (lane == 0) ssp[par][wave][r] = q;
        }
    };

    // decide the tokens of step sp from the key records; all waves do it
    int fed[BM];
    auto decide = [&](int sp, int ph_lm_idx) {
        const uint32_t lt = tag_of(ph_lm_idx);
#pragma unroll
        for (int b = 0; b < BM; ++b) {
            if (b < B) {
                const int tok = poll_argmax(rc.KEY, b, lt, err);
                if (wg == 0 && wave == 0 && lane == 0) a.tok_out[b * kSteps + (sp - 1)] = tok;
                int f = a.force ? a.force[b * kSteps + (sp - 1)] : tok;
                if (f < 0 || f >= V) {
                    if (wg == 0 && wave == 0 && lane == 0) atomicOr(err, kErrBadForced);
                    f = 0;
                }
                fed[b] = f;
            }
        }
    };

    // ---- INIT: q0, H rows
    // wave 3 keeps the tokens fed at codebook j for the embedding sum
    // (element: request lane/8, column 8*wg + lane%8), written and read by
    // wave 3 alone
    const int eb = lane >> 3, ek = 8 * wg + (lane & 7);
    auto keep_tokens = [&](int j) {
        if (wave == 3 && lane < B) {
            int fb = fed[0];
#pragma unroll
            for (int b = 1; b < BM; ++b)
                if (b == lane) fb = fed[b];
            tok_s[j][lane] = fb;
        }
    };
#pragma unroll
    for (int b = 0; b < BM; ++b) {
        if (b < B) {
            int q = a.q0[b];
            if (q < 0 || q >= V) {
                if (wg == 0 && wave == 0 && lane == 0) atomicOr(err, kErrBadQ0);
                q = 0;
            }
            fed[b] = q;
            const float4* hr = reinterpret_cast<const float4*>(a.H + static_cast<size_t>(b) * DT) + wave * (DT / 16);
            float4* d4 = reinterpret_cast<float4*>(slot[0] + b * DT) + wave * (DT / 16);
#pragma unroll
            for (int i = 0; i < DT / 1024; ++i) d4[lane + 64 * i] = hr[lane + 64 * i];
        }
    }
    keep_tokens(0);
    __builtin_amdgcn_s_waitcnt(0);   // this wave's table requests too
    __syncthreads();
    {
        const float* Hs = slot[0];
        const int n = 4 * wg + wave;
        const float bias = m.proj_b[n];
#pragma unroll
        for (int r = 0; r < BM; ++r) {
            if (r < B) {
                float acc = 0.f;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    float x8[8];
                    lds8(Hs + r * DT + c * 512 + lane * 8, x8);
                    bf16x2_t p8[4];
                    pack8w<WT>(x8, p8);
                    acc = wdot8<WT>(wP[c], x8, p8, acc);
                }
                const float v = wave_sum(acc) + bias;
                if (lane == 0) st_rec(rc.X + static_cast<size_t>(r) * DP + n, v, tag_of(0));
            }
        }
    }

    float xr[MR];  // this wave's residual-stream element (column 4*wg + wave) per row
    int ph = 1;
    for (int s = 1; s <= kSteps; ++s) {
        const int M = (s == 1) ? 2 * B : B;
        for (int l = 0; l < L; ++l) {
            // ================= QKV(l) =================
            if (l == 0 && s > 1 && t0) {
                // the input row is P_{s-1}[fed], whose q/k/v rows are in the
                // table: decide the tokens and take this wave's residual
                // element.  The attention units first request their layer-0
                // history, which does not depend on the token (attention's
                // slot: its last reader, the lm_head phase, ended at a barrier).
                if (wg < B * NKV) {
                    const size_t kvb = (static_cast<size_t>(wg / NKV) * kPositions) * NKV * HD;
                    hist_dma(m.kc, m.vc, kvb, wg % NKV, s, slot[(ph + 1) & 1], wave, 0, kW);
                }
                decide(s - 1, ph_lm(L, s - 1));
                keep_tokens(s - 1);
#pragma unroll
                for (int r = 0; r < MR; ++r) xr[r] = 0.f;
#pragma unroll
                for (int b = 0; b < BM; ++b)
                    if (b < B) xr[b] = m.ptab[(static_cast<size_t>(s - 1) * V + fed[b]) * DP + 4 * wg + wave];
                ++ph;
            } else {
                const int par = ph & 1;
                float* xs = slot[par];
                QP_STAMP(a.taps, wg, ph, 0);
                if (l == 0) {
                    if (s == 1) {
                        gather_x(rc.X, B, tag_of(0), par);
                    } else {
                        decide(s - 1, ph_lm(L, s - 1));
                        keep_tokens(s - 1);
                    }
                    // rows fed by the codebook tables: P_{s-1}[fed], a quarter per wave
                    const int r0 = (s == 1) ? B : 0;
#pragma unroll
                    for (int b = 0; b < BM; ++b) {
                        if (b < B) {
                            const float4* prow = reinterpret_cast<const float4*>(
                                                     m.ptab + (static_cast<size_t>(s - 1) * V + fed[b]) * DP) +
                                                 wave * (DP / 16);
                            float4* d4 = reinterpret_cast<float4*>(xs + (r0 + b) * DP) + wave * (DP / 16);
                            const float4 t = prow[lane];
                            d4[lane] = t;
                            const float q = wave_sum(t.x * t.x + t.y * t.y + t.z * t.z + t.w * t.w);
                            if (lane == 0) ssp[par][wave][r0 + b] = q;
                        }
                    }
                } else {
                    gather_x(rc.X, M, tag_of(ph - 1), par);
                }
                __syncthreads();
                QP_STAMP(a.taps, wg, ph, 1);
                if (l == 0) {
#pragma unroll
                    for (int r = 0; r < MR; ++r) xr[r] = (r < M) ? xs[r * DP + 4 * wg + wave] : 0.f;
                }
                const float* ga = g_attn(l);
                for (int r = 0; r < M; ++r) {
                    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        float x8[8];
                        act8(xs + r * DP, ga, c, x8);
                        bf16x2_t p8[4];
                        pack8w<WT>(x8, p8);
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc[q] = wdot8<WT>(wQ[q * 2 + c], x8, p8, acc[q]);
                    }
                    const float rinv = __builtin_amdgcn_rsqf(row_ss(par, r) / static_cast<float>(DP) + eps);
                    wave_sums(acc);
                    float v = 0.f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) v = (lane == q) ? acc[q] * rinv : v;
                    if (lane < 4) st_rec(rc.QKV + static_cast<size_t>(r) * NQKV + 16 * wg + 4 * wave + lane, v, tag_of(ph));
                }
                QP_STAMP(a.taps, wg, ph, 2);
                if (wg < B * NKV && s > 1) {
                    // the attention unit's history, requested behind its
                    // q/k/v stores: it lands while the other producers'
                    // records are awaited.  The slot is attention's; its
                    // last reader (the previous phase) finished before this
                    // phase's staging barrier.
                    const size_t kvb = ((static_cast<size_t>(l) * m.max_batch + wg / NKV) * kPositions) * NKV * HD;
                    hist_dma(m.kc, m.vc, kvb, wg % NKV, s, slot[par ^ 1], wave, 0, kW);
                }
                ++ph;
            }
            // ================= ATTN(l) =================
            {
                const int par = ph & 1;
                if (wg < B * NKV) QP_STAMP(a.taps, wg, ph, 0);
                float* hist = slot[par];
                const bool unit = wg < B * NKV;
                const int b = wg / NKV, g = wg % NKV;
                const int pf = (s == 1) ? 0 : s;
                const int npos = (s == 1) ? 2 : 1;
                const size_t kvb = ((static_cast<size_t>(l) * m.max_batch + b) * kPositions) * NKV * HD;
                if (unit) {
                    // cached keys/values of earlier positions (LDS-direct
                    // loads) were requested by the unit already: at the end
                    // of its q/k/v phase, or (layer 0 from the table) ahead
                    // of the token decision
                    // new head vectors: wave w takes q 2g, q 2g+1, k g, v g
                    const int col = wave < 2 ? (2 * g + wave) * HD : (wave == 2 ? (NQ + g) * HD : (NQ + NKV + g) * HD);
                    if (l == 0 && s > 1 && t0) {
                        // from the table (one position): row P_{s-1}[fed[b]]
                        int fb = fed[0];
#pragma unroll
                        for (int bb = 1; bb < BM; ++bb)
                            if (bb == b) fb = fed[bb];
                        const float* trow = t0 + (static_cast<size_t>(s - 2) * V + fb) * NQKV + col;
                        *reinterpret_cast<float2*>(hist + 4096 + wave * HD + 2 * lane) =
                            *reinterpret_cast<const float2*>(trow + 2 * lane);
                    } else {
                        const uint32_t qt = tag_of(ph - 1);
                        for (int pi = 0; pi < npos; ++pi)
                            poll_head(rc.QKV + static_cast<size_t>(pi * B + b) * NQKV + col, qt,
                                      hist + 4096 + 512 * pi + wave * HD, err);
                    }
                    __builtin_amdgcn_s_waitcnt(0);
                }
                __syncthreads();
                if (unit) QP_STAMP(a.taps, wg, ph, 1);
                if (unit && wave < 2) {
                    // one wave per query head; all <= 16 scores at once: key t on
                    // lanes 4t..4t+3, each lane a 32-wide slice of the head
                    const int h = 2 * g + wave;
                    const float* gq = g_q(l);
                    const float* gk = g_k(l);
                    float* qb = hist + 5120 + 128 * wave;     // this wave's rotated query
                    float* eb = hist + 5376 + 16 * wave;      // its softmax weights
                    const int kt = lane >> 2, kq = (lane & 3) * 32;
                    for (int pi = 0; pi < npos; ++pi) {
                        const int p = pf + pi;
                        const int r = (s == 1) ? pi * B + b : b;
                        const float* nd = hist + 4096 + pi * 512;
                        // every LDS operand of this position first, then one wait
                        const float c0 = rope_s[0][p * (HD / 2) + lane], s0 = rope_s[1][p * (HD / 2) + lane];
                        const float k0 = nd[256 + lane], k1 = nd[256 + lane + 64];
                        const float x0 = nd[wave * HD + lane], x1 = nd[wave * HD + lane + 64];
                        const float vv0 = nd[384 + lane], vv1 = nd[384 + lane + 64];
                        const float gk0 = gk[lane], gk1 = gk[lane + 64], gq0 = gq[lane], gq1 = gq[lane + 64];
                        // key and this wave's query: per-head RMSNorm (both sums
                        // at once; hardware reciprocal square root), rotate-half
                        // RoPE (pair lane, lane + 64)
                        float sq[2] = {k0 * k0 + k1 * k1, x0 * x0 + x1 * x1};
                        wave_sums(sq);
                        const float rk = __builtin_amdgcn_rsqf(sq[0] / static_cast<float>(HD) + eps);
                        const float rq = __builtin_amdgcn_rsqf(sq[1] / static_cast<float>(HD) + eps);
                        float kv0, kv1;
                        {
                            const float a0 = gk0 * (k0 * rk), a1 = gk1 * (k1 * rk);
                            kv0 = a0 * c0 - a1 * s0;
                            kv1 = a1 * c0 + a0 * s0;
                        }
                        if (wave == 0) {
                            const size_t off = kvb + (static_cast<size_t>(p) * NKV + g) * HD;
                            st_act(m.kc + off + lane, kv0);
                            st_act(m.kc + off + lane + 64, kv1);
                            st_act(m.vc + off + lane, vv0);
                            st_act(m.vc + off + lane + 64, vv1);
                        }
                        // this position's key/value join the history (both waves
                        // write the same values, each before it reads them)
                        hist[p * HD + lane] = kv0;
                        hist[p * HD + lane + 64] = kv1;
                        hist[2048 + p * HD + lane] = vv0;
                        hist[2048 + p * HD + lane + 64] = vv1;
                        {
                            const float a0 = gq0 * (x0 * rq), a1 = gq1 * (x1 * rq);
                            qb[lane] = a0 * c0 - a1 * s0;
                            qb[lane + 64] = a1 * c0 + a0 * s0;
                        }
                        // scores
                        float sc = 0.f;
                        if (kt <= p) {
#pragma unroll
                            for (int i = 0; i < 32; i += 4) {
                                const float4 qv = *reinterpret_cast<const float4*>(qb + kq + i);
                                const float4 kv = *reinterpret_cast<const float4*>(hist + kt * HD + kq + i);
                                sc = fmaf(qv.x, kv.x, sc);
                                sc = fmaf(qv.y, kv.y, sc);
                                sc = fmaf(qv.z, kv.z, sc);
                                sc = fmaf(qv.w, kv.w, sc);
                            }
                        }
                        sc += dpp_or_zero<0xB1, 0xF>(sc);   // lanes of a quad: one key
                        sc += dpp_or_zero<0x4E, 0xF>(sc);
                        sc = (kt <= p) ? sc * m.attn_scale : -__builtin_huge_valf();
                        const float mx = wave_max(sc);
                        const float e = (kt <= p) ? __expf(sc - mx) : 0.f;
                        const float den = wave_sum((lane & 3) == 0 ? e : 0.f);
                        if ((lane & 3) == 0) eb[kt] = e;
                        // weighted values (weights are 0 beyond p; rows beyond p
                        // are read as row p, so no stale LDS enters the sum); all
                        // reads are issued before the first product
                        float va[kPositions], vb[kPositions], ew[kPositions];
#pragma unroll
                        for (int t = 0; t < kPositions; ++t) {
                            const int tt = t <= p ? t : p;
                            ew[t] = eb[t];
                            va[t] = hist[2048 + tt * HD + lane];
                            vb[t] = hist[2048 + tt * HD + lane + 64];
                        }
                        float o0 = 0.f, o1 = 0.f;
#pragma unroll
                        for (int t = 0; t < kPositions; ++t) {
                            o0 = fmaf(ew[t], va[t], o0);
                            o1 = fmaf(ew[t], vb[t], o1);
                        }
                        uint64_t* orow = rc.AO + static_cast<size_t>(r) * QD + h * HD;
                        const float rden = __builtin_amdgcn_rcpf(den);
                        st_rec(orow + lane, o0 * rden, tag_of(ph));
                        st_rec(orow + lane + 64, o1 * rden, tag_of(ph));
                    }
                }
                // next phase's weights, after this phase's stores have left
                sched_fence();
                load_wO(l);
                if (!unit) load_wU(l);
                sched_fence();
                if (unit) QP_STAMP(a.taps, wg, ph, 2);
                ++ph;
            }
            // ================= O(l) =================
            {
                const int par = ph & 1;
                float* as = slot[par];
                const uint32_t tg = tag_of(ph - 1);
                QP_STAMP(a.taps, wg, ph, 0);
                if (wg >= B * NKV) gate_rec<QD / 128>(rc.AO, tg, err);
                for (int r = 0; r < M; ++r) (void)poll_share<QD>(rc.AO + static_cast<size_t>(r) * QD, wave, tg, as + r * QD, err);
                __syncthreads();
                QP_STAMP(a.taps, wg, ph, 1);
                const int n = 4 * wg + wave;
                for (int r = 0; r < M; ++r) {
                    float acc = 0.f;
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        float x8[8];
                        lds8(as + r * QD + c * 512 + lane * 8, x8);
                        bf16x2_t p8[4];
                        pack8w<WT>(x8, p8);
                        acc = wdot8<WT>(wO[c], x8, p8, acc);
                    }
                    const float d = wave_sum(acc);
                    float nv = 0.f;
#pragma unroll
                    for (int i = 0; i < MR; ++i)
                        if (i == r) { xr[i] += d; nv = xr[i]; }
                    if (lane == 0) st_rec(rc.X + static_cast<size_t>(r) * DP + n, nv, tag_of(ph));
                }
                sched_fence();
                if (wg < B * NKV) load_wU(l);
                sched_fence();
                QP_STAMP(a.taps, wg, ph, 2);
                ++ph;
            }
            // ================= UP(l) =================
            {
                const int par = ph & 1;
                float* xs = slot[par];
                QP_STAMP(a.taps, wg, ph, 0);
                gather_x(rc.X, M, tag_of(ph - 1), par);
                __syncthreads();
                QP_STAMP(a.taps, wg, ph, 1);
                const float* gf = g_ffn(l);
                for (int r = 0; r < M; ++r) {
                    float ag[3] = {0.f, 0.f, 0.f}, au[3] = {0.f, 0.f, 0.f};
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        float x8[8];
                        act8(xs + r * DP, gf, c, x8);
                        bf16x2_t p8[4];
                        pack8w<WT>(x8, p8);
#pragma unroll
                        for (int q = 0; q < 3; ++q) {
                            ag[q] = wdot8<WT>(wU[q * 2 + c], x8, p8, ag[q]);
                            au[q] = wdot8<WT>(wU[6 + q * 2 + c], x8, p8, au[q]);
                        }
                    }
                    const float rinv = __builtin_amdgcn_rsqf(row_ss(par, r) / static_cast<float>(DP) + eps);
                    float gu[6] = {ag[0], ag[1], ag[2], au[0], au[1], au[2]};
                    wave_sums(gu);
                    float v = 0.f;
#pragma unroll
                    for (int q = 0; q < 3; ++q) {
                        const float gv = gu[q] * rinv;
                        const float uv = gu[3 + q] * rinv;
                        const float hv = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
                        v = (lane == q) ? hv : v;
                    }
                    if (lane < 3) st_rec(rc.H + static_cast<size_t>(r) * F + 12 * wg + 3 * wave + lane, v, tag_of(ph));
                }
                sched_fence();
                load_wD(l);
                sched_fence();
                QP_STAMP(a.taps, wg, ph, 2);
                ++ph;
            }
            // ================= DOWN(l) =================
            {
                const int par = ph & 1;
                float* hs = slot[par];
                const uint32_t tg = tag_of(ph - 1);
                QP_STAMP(a.taps, wg, ph, 0);
                for (int r = 0; r < M; ++r) (void)poll_share<F>(rc.H + static_cast<size_t>(r) * F, wave, tg, hs + r * F, err);
                __syncthreads();
                QP_STAMP(a.taps, wg, ph, 1);
                const int n = 4 * wg + wave;
                for (int r = 0; r < M; ++r) {
                    float acc = 0.f;
#pragma unroll
                    for (int c = 0; c < 6; ++c) {
                        float x8[8];
                        lds8(hs + r * F + c * 512 + lane * 8, x8);
                        bf16x2_t p8[4];
                        pack8w<WT>(x8, p8);
                        acc = wdot8<WT>(wD[c], x8, p8, acc);
                    }
                    const float d = wave_sum(acc);
                    float nv = 0.f;
#pragma unroll
                    for (int i = 0; i < MR; ++i)
                        if (i == r) { xr[i] += d; nv = xr[i]; }
                    if (lane == 0) {
                        st_rec(rc.X + static_cast<size_t>(r) * DP + n, nv, tag_of(ph));
                        if (kWriteTaps && a.taps) {
                            const int pos = (s == 1) ? (r >= B ? 1 : 0) : s;
                            const int bb = (s == 1 && r >= B) ? r - B : r;
                            a.taps[((static_cast<size_t>(pos) * L + l) * B + bb) * DP + n] = nv;
                        }
                    }
                }
                sched_fence();
                if (l + 1 < L) load_wQ(l + 1); else load_wL(s);
                sched_fence();
                QP_STAMP(a.taps, wg, ph, 2);
                ++ph;
            }
        }
        // ================= LM(s) =================
        {
            const int par = ph & 1;
            float* xs = slot[par];
            const int r0 = (s == 1) ? B : 0;
            QP_STAMP(a.taps, wg, ph, 0);
            gather_x(rc.X + static_cast<size_t>(r0) * DP, B, tag_of(ph - 1), par);
            __syncthreads();
            QP_STAMP(a.taps, wg, ph, 1);
            const int v0 = 8 * wg + 2 * wave;
#pragma unroll
            for (int b = 0; b < BM; ++b) {
                if (b < B) {
                    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        float x8[8];
                        act8(xs + b * DP, g_out, c, x8);
                        bf16x2_t p8[4];
                        pack8w<WT>(x8, p8);
                        acc0 = wdot8<WT>(wL[c], x8, p8, acc0);
                        acc1 = wdot8<WT>(wL[2 + c], x8, p8, acc1);
                    }
                    const float rinv = __builtin_amdgcn_rsqf(row_ss(par, b) / static_cast<float>(DP) + eps);
                    float lg[2] = {acc0, acc1};
                    wave_sums(lg);
                    const float l0 = lg[0] * rinv;
                    const float l1 = lg[1] * rinv;
                    if (a.logits_out && lane < 2)
                        a.logits_out[(static_cast<size_t>(b) * kSteps + (s - 1)) * V + v0 + lane] = lane ? l1 : l0;
                    const bool second = ordered_bits(l1) > ordered_bits(l0);
                    const uint64_t key = (static_cast<uint64_t>(ordered_bits(second ? l1 : l0)) << 32) |
                                         (0xFFFFFFFFu - static_cast<uint32_t>(v0 + (second ? 1 : 0)));
                    if (lane == 0) lmk[wave][b] = key;
                }
            }
            __syncthreads();
            if (wave == 0 && lane < B) {
                uint64_t best = 0;
#pragma unroll
                for (int w = 0; w < kW; ++w) {
                    uint64_t k = 0;
#pragma unroll
                    for (int b = 0; b < BM; ++b)
                        if (b == lane) k = lmk[w][b];
                    best = k > best ? k : best;
                }
                uint64_t* kr = rc.KEY + (static_cast<size_t>(lane) * kNwg + wg) * 2;
                st_rec_u(kr, static_cast<uint32_t>(best >> 32), tag_of(ph));
                st_rec_u(kr + 1, 0xFFFFFFFFu - static_cast<uint32_t>(best & 0xFFFFFFFFu), tag_of(ph));
            }
            sched_fence();
            if (s < kSteps && !t0) load_wQ(0);
            sched_fence();
            QP_STAMP(a.taps, wg, ph, 2);
            ++ph;
        }
    }
    // ================= FINAL: last token, embedding sum out =================
    decide(kSteps, ph_lm(L, kSteps));
    keep_tokens(kSteps);
    if (wave == 3 && eb < B) {
        // the 16 rows' elements requested together, summed in codebook order
        float ev[kSteps + 1];
#pragma unroll
        for (int j = 0; j <= kSteps; ++j) ev[j] = emb_elem(m, j, tok_s[j][eb], ek);
        float es = ev[0];
#pragma unroll
        for (int j = 1; j <= kSteps; ++j) es += ev[j];
        a.embsum[static_cast<size_t>(eb) * DT + ek] = es;
    }
}


}  // namespace stream
}  // namespace qp

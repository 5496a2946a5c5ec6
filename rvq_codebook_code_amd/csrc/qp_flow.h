// Dataflow frame kernel for moderate batches (3 <= B <= 16) of the 1.7B-shaped
// predictor with bf16 weights: the small-batch kernel's record exchange
// (qp_stream.h) with every product on the matrix cores.
//
// One cooperative launch of 256 workgroups of 16 waves (one per compute
// unit), no grid barrier.  Values cross workgroups as 64-bit records whose
// high word is the phase tag (unique per phase instance, as in qp_stream.h);
// activations travel as pairs of bf16 in the low word (half the bytes of an
// fp32 record per value), the q/k/v rows and the row sums of squares as
// fp32.  A consumer stages the rows it needs in LDS, one wave per row, all of
// a row's loads in flight at once (16 waves x up to 12 16-byte loads per
// lane: the per-unit pull of tagged records runs about three times faster
// than with 4 waves x 8 loads).
//
// Waiting: before a phase polls its rows, wave 0 alone waits for the first
// record of row 0 to carry the phase's tag (one 16-byte load per lane per
// attempt), the other waves at a barrier; then all sixteen poll their rows in
// full.  Most workgroups sit out several phases (the owners' O and down,
// the attention units), and sixteen waves polling whole rows through those
// waits took fabric bandwidth from the phases in flight (B = 16: 10,240 ->
// 11,360 frames/s with the gate).
//
// Products: [rows x K] . [K x 16] fragments on v_mfma_f32_16x16x32_bf16 over
// the batched path's fragment-ordered weights (qp_tiled.h), held in
// registers one active phase ahead; the 16 waves split K and their partial
// tiles are summed through LDS in wave order.  The RMSNorm fold is the
// batched path's: whoever owns residual-stream columns publishes
// bf16(g_next * x) and the columns' sums of x^2; the reader scales its
// output row by rsqrt(sum / dP + eps).
//
// Roles (workgroup w):
//   w >= 192: owner of residual columns 16 (w-192) .. +15 (the projection of
//             H, O and down products, x kept in registers across the frame),
//             of embedding-sum columns 32 (w-192) .. +31, and (w = 192) of
//             tokens_out;
//   every w:  q/k/v columns 16 w .. +15;
//   w < 192:  gate/up columns 16 w .. +15 (SwiGLU in the epilogue);
//   w < 128:  lm_head vocabulary columns 16 w .. +15 (per-row argmax keys);
//   w < 8 B:  attention unit (request w / 8, kv head w % 8).
// Layer 0's q/k/v rows of steps 2..15 come from the create-time table
// (Model::qkv0), as in qp_stream.h: the step starts with the token decision.
#pragma once

#include "qp_common.h"
#include "qp_phases.h"
#include "qp_stream.h"
#include "qp_tiled.h"

namespace qp {
namespace flow {

using stream::DP;
using stream::DT;
using stream::F;
using stream::HD;
using stream::NKV;
using stream::NQ;
using stream::NQKV;
using stream::QD;
using stream::V;
using stream::kMaxL;

constexpr int kW = 16;                  // waves per workgroup
constexpr int kThreadsF = kW * 64;
constexpr int kNwg = 256;
constexpr int kMaxB = 16;
constexpr int kMaxRows = 2 * kMaxB;     // step 1 holds positions 0 and 1
constexpr int kOwn0 = 192;              // first residual-column owner
constexpr int kNOwn = DP / 16;          // 64 owners
constexpr int kNUp = F / 16;            // 192 gate/up fragments
constexpr int kNLm = V / 16;            // 128 lm_head fragments
constexpr int kSRow = F + 8;            // LDS row stride of a staged operand (bf16), padded against bank conflicts
static_assert(NQKV / 16 == kNwg && kOwn0 + kNOwn == kNwg && kNUp == kOwn0 && kNLm <= kNUp && NKV * kMaxB <= kNLm,
              "role layout assumes the 1.7B predictor geometry");

__host__ __device__ constexpr int phases_per_frame(int L) { return 1 + kSteps * (5 * L + 1) + 1; }

// Record buffers (all zero-initialised; tag 0 is never current).
struct Recs {
    uint64_t* XG;    // [kMaxRows][DP / 2]   bf16 pairs of g_next * x
    uint64_t* SS;    // [kNOwn][kMaxRows]    sum of x^2 over each owner's 16 columns; owner-major,
                     // so that each owner writes its own block (rows of many
                     // writers sharing a segment made every reader wait longer)
    uint64_t* QKV;   // [kMaxRows][NQKV]     fp32
    uint64_t* AO;    // [kMaxRows][QD / 2]   bf16 pairs of the attention output
    uint64_t* HH;    // [kMaxRows][F / 2]    bf16 pairs of the SwiGLU output
    uint64_t* KEY;   // [kNLm][kMaxB][2]     ordered logit bits, vocabulary index; fragment-major,
                     // each lm_head workgroup writing its own block
};
constexpr size_t kRecsTotal = static_cast<size_t>(kMaxRows) * (DP / 2 + NQKV + QD / 2 + F / 2) +
                              static_cast<size_t>(kNOwn) * kMaxRows +
                              static_cast<size_t>(kMaxB) * kNLm * 2;

// Fragment-ordered bf16 weights ([N/16][K/32][64 lanes][8]) of one launch.
struct FLayer {
    const uint8_t* qkv;
    const uint8_t* o;
    const uint8_t* gate;
    const uint8_t* up;
    const uint8_t* down;
};
struct FArgs {
    FLayer lay[kMaxL];
    const uint8_t* proj;
    const uint8_t* lm[kSteps];
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
using stream::rsrc_t;
using stream::kDeviceScope;

__device__ __forceinline__ int ph_layer(int L, int s, int l, int t) { return 1 + (s - 1) * (5 * L + 1) + 5 * l + t; }
__device__ __forceinline__ int ph_lm(int L, int s) { return 1 + (s - 1) * (5 * L + 1) + 5 * L; }
enum { T_QKV = 0, T_ATTN = 1, T_O = 2, T_UP = 3, T_DOWN = 4 };

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
// One record, (tag << 32) | lo, at record index i of buffer r: a single
// 64-bit device-coherent store (the base lives in scalar registers, only the
// 32-bit offset in a vector register).
__device__ __forceinline__ void st_rec64(rsrc_t r, uint32_t i, uint32_t lo, uint32_t tag) {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{lo, tag}, r, i * 8u, 0u, kDeviceScope);
}
__device__ __forceinline__ rsrc_t rbuf(const void* p) { return stream::wrsrc(p, 0x7FFFFFF0u); }
// The lane index read afresh where it is used: the epilogues' record offsets
// derive from it, so the compiler cannot compute them once per frame and
// keep (or spill) them across the phase loop.
__device__ __forceinline__ int fresh_lane() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}
__device__ __forceinline__ float ldf(rsrc_t r, uint32_t i) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, i * 4u, 0u, 0));
}

__device__ __forceinline__ uint32_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }

// KBW consecutive 32-wide k-blocks of output fragment nb (K / 32 = KB blocks
// per fragment row), this wave's share, one 16-byte piece per lane each.
template <int KBW>
__device__ __forceinline__ void ld_frag(const uint8_t* W, int nb, int KB, int wave, int lane, uint4* out) {
    const rsrc_t r = rbuf(W);
    const uint32_t so = (static_cast<uint32_t>(nb) * KB + static_cast<uint32_t>(wave) * KBW) * 1024u;
#pragma unroll
    for (int k = 0; k < KBW; ++k) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<uint32_t>(lane) * 16u, so + k * 1024u, 0);
        out[k] = make_uint4(v[0], v[1], v[2], v[3]);
    }
}

// This wave's k-blocks of the staged rows (bf16 [16][kSRow] in LDS) against
// the fragment pieces in registers.
template <int KBW>
__device__ __forceinline__ f32x4_t mfma_slice(const uint16_t* stage, int wave, int lane, const uint4* w,
                                              f32x4_t acc) {
    const uint16_t* a = stage + (lane & 15) * kSRow + (lane >> 4) * 8 + wave * KBW * 32;
#pragma unroll
    for (int k = 0; k < KBW; ++k) {
        const uint4 av = *reinterpret_cast<const uint4*>(a + k * 32);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                      __builtin_bit_cast(bf16x8_t, w[k]), acc, 0, 0, 0);
    }
    return acc;
}

// Wait for one staged row: NJ 16-byte loads per lane of bf16-pair records
// (2 records = 4 values each) into dst (bf16, K = 256 NJ values).  With ss
// set, the wave also waits for its share of the fragment's sums of squares:
// owners 4 wave .. 4 wave + 3 (lane / 16), rows ss_row0 + lane % 16 below
// ss_row0 + ss_rows, into ss_dst[owner][lane % 16] (the row totals are taken
// after the workgroup barrier).  Bounded wait: a record that never arrives
// raises the timeout flag and the row keeps whatever arrived.
// Without a row of its own (have_row false: the fragment's rows end
// before this wave's) a wave still waits for its share of the sums and
// zeroes its staged row.
template <int NJ>
__device__ __forceinline__ void poll_row(const uint64_t* rec, uint32_t tag, uint16_t* dst, unsigned* err,
                                         const uint64_t* ss = nullptr, int ss_row0 = 0, int ss_rows = 0,
                                         float* ss_dst = nullptr, bool have_row = true) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const rsrc_t r = stream::wrsrc(rec, NJ * 1024);
    const rsrc_t rs = stream::wrsrc(ss ? ss : rec, 0x7FFFFFF0u);
    const int so = 4 * wave + (lane >> 4);                     // owner of this lane's sum
    const uint32_t soff = (static_cast<uint32_t>(so) * kMaxRows + ss_row0 + (lane & 15)) * 8u;
    uint32_t pend = have_row ? (1u << NJ) - 1u : 0u;
    bool spend = ss != nullptr && (lane & 15) < ss_rows;
    if (!have_row) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) *reinterpret_cast<uint2*>(dst + 4 * (j * 64 + lane)) = make_uint2(0u, 0u);
    }
    unsigned spins = 0;
    while (true) {
        decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0u, 0u, 0)) u[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            if ((pend >> j) & 1u) u[j] = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16u, 1024u * j, kDeviceScope);
        decltype(__builtin_amdgcn_raw_buffer_load_b64(rs, 0u, 0u, 0)) us{};
        if (spend) us = __builtin_amdgcn_raw_buffer_load_b64(rs, soff, 0u, kDeviceScope);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if (((pend >> j) & 1u) && static_cast<uint32_t>(u[j][1]) == tag && static_cast<uint32_t>(u[j][3]) == tag) {
                *reinterpret_cast<uint2*>(dst + 4 * (j * 64 + lane)) =
                    make_uint2(static_cast<uint32_t>(u[j][0]), static_cast<uint32_t>(u[j][2]));
                pend &= ~(1u << j);
            }
        }
        if (spend && static_cast<uint32_t>(us[1]) == tag) {
            ss_dst[so * 16 + (lane & 15)] = __uint_as_float(static_cast<uint32_t>(us[0]));
            spend = false;
        }
        if (!__any(pend != 0u || spend)) break;
        if (!stream::spin_wait(spins, err)) break;
    }
}

// Wave 0 alone waits until some record of row `rec` carries `tag` (one
// 16-byte load per lane per attempt, its chunks in turn); every wave then
// meets at the barrier and polls its own row in full.  A workgroup that
// waits long for a phase thus polls with one wave instead of sixteen, and
// the fabric is left to the phases in flight.
template <int NJ>
__device__ __forceinline__ void gate_row(const uint64_t* rec, uint32_t tag, unsigned* err) {
    if ((threadIdx.x >> 6) == 0) {
        const int lane = threadIdx.x & 63;
        const rsrc_t r = stream::wrsrc(rec, NJ * 1024);
        uint32_t probe = 0;
        unsigned spins = 0;
        while (true) {
            const auto u = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16u, 1024u * probe, kDeviceScope);
            if (__any(static_cast<uint32_t>(u[1]) == tag || static_cast<uint32_t>(u[3]) == tag)) break;
            probe = probe + 1 == NJ ? 0 : probe + 1;
            if (!stream::spin_wait(spins, err)) break;
        }
    }
    __syncthreads();
}

template <int NJ>
__device__ __forceinline__ void zero_row(uint16_t* dst) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < NJ; ++j) *reinterpret_cast<uint2*>(dst + 4 * (j * 64 + lane)) = make_uint2(0u, 0u);
}

// Token of request b from the lm_head fragments' key records (largest
// logit, lowest index on ties); lane-uniform.  One wave.
__device__ __forceinline__ int poll_token(const uint64_t* key, int b, uint32_t tag, unsigned* err) {
    const int lane = threadIdx.x & 63;
    constexpr int NJ = kNLm / 64;
    // fragment f = lane + 64 j: its record pair for request b
    const rsrc_t r = stream::wrsrc(key + static_cast<size_t>(b) * 2, kNLm * kMaxB * 16);
    uint32_t ord[NJ], idx[NJ];
    uint32_t pend = (1u << NJ) - 1u;
    unsigned spins = 0;
    while (true) {
        decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0u, 0u, 0)) u[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            if ((pend >> j) & 1u)
                u[j] = __builtin_amdgcn_raw_buffer_load_b128(r, lane * (kMaxB * 16u), j * 64u * kMaxB * 16u, kDeviceScope);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if (((pend >> j) & 1u) && static_cast<uint32_t>(u[j][1]) == tag && static_cast<uint32_t>(u[j][3]) == tag) {
                ord[j] = static_cast<uint32_t>(u[j][0]);
                idx[j] = static_cast<uint32_t>(u[j][2]);
                pend &= ~(1u << j);
            }
        }
        if (!__any(pend != 0u)) break;
        if (!stream::spin_wait(spins, err)) break;
    }
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const uint64_t k = (static_cast<uint64_t>(ord[j]) << 32) | (0xFFFFFFFFu - idx[j]);
        best = k > best ? k : best;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint64_t o = tiled::shfl_xor64(best, off);
        best = o > best ? o : best;
    }
    return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best & 0xFFFFFFFFu));
}

__global__ __launch_bounds__(kThreadsF) void k_flow(Model m, RunArgs a, Recs rc, FArgs fa) {
    __shared__ __attribute__((aligned(16))) uint16_t stage[16 * kSRow];   // staged operand rows (attention scratch too)
    __shared__ f32x4_t red[2][kW][64];                                   // partial tiles of the 16 waves
    __shared__ float rinv_s[16];
    __shared__ float ss_s[kNOwn * 16];                                   // [owner][fragment row] sums of x^2
    __shared__ float rope_s[2][kPositions * (HD / 2)];
    __shared__ float qk_s[kMaxL][2][HD];                                 // q_norm, k_norm gains
    __shared__ int fed_s[kMaxB];
    __shared__ LayerDev lay_s[kMaxL];
    // owners: the gains of their 16 columns (attn_norm[l], ffn_norm[l], then
    // out_norm), read by the epilogues without a memory round trip
    __shared__ float gain_s[2 * kMaxL + 1][16];

    const int wg = blockIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int B = a.B;
    const int L = m.L;
    const float eps = m.eps;
    unsigned* err = m.err;
    const uint32_t seq0 = a.seq0;
    auto tag_of = [&](int ph) { return seq0 + static_cast<uint32_t>(ph) + 1u; };

    const bool own = wg >= kOwn0;
    const int oc = wg - kOwn0;                 // owner column fragment
    const bool up_role = wg < kNUp;
    const bool lm_role = wg < kNLm;
    const bool unit = wg < B * NKV;
    const int ub = wg / NKV, ug = wg % NKV;    // attention unit: request, kv head

    // ---- tables into LDS
    if (threadIdx.x < L) lay_s[threadIdx.x] = m.layers[threadIdx.x];
    for (int i = threadIdx.x; i < kPositions * (HD / 2); i += kThreadsF) {
        rope_s[0][i] = m.rope_cos[i];
        rope_s[1][i] = m.rope_sin[i];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < L * HD; i += kThreadsF) {
        const int l = i / HD, d = i % HD;
        qk_s[l][0][d] = lay_s[l].q_norm[d];
        qk_s[l][1][d] = lay_s[l].k_norm[d];
    }
    if (own && threadIdx.x < (2 * kMaxL + 1) * 16) {
        const int j = threadIdx.x >> 4, c = 16 * (wg - kOwn0) + (threadIdx.x & 15);
        const float* g = j == 2 * kMaxL ? m.out_norm : (j < 2 * L ? ((j & 1) ? lay_s[j >> 1].ffn_norm : lay_s[j >> 1].attn_norm)
                                                                  : nullptr);
        gain_s[j][threadIdx.x & 15] = g ? g[c] : 0.f;
    }

    // ---- weights in registers, one active phase ahead
    // one buffer: a workgroup holds only the weights of its next active
    // phase (q/k/v 2, O 4, gate + up 2 + 2, down 6, lm_head 2, projection 4
    // pieces of 16 bytes per lane)
    uint4 wb[6];
    auto load_q = [&](int l) { ld_frag<2>(fa.lay[l].qkv, wg, DP / 32, wave, lane, wb); };
    auto load_o = [&](int l) { ld_frag<4>(fa.lay[l].o, oc, QD / 32, wave, lane, wb); };
    auto load_u = [&](int l) {
        ld_frag<2>(fa.lay[l].gate, wg, DP / 32, wave, lane, wb);
        ld_frag<2>(fa.lay[l].up, wg, DP / 32, wave, lane, wb + 2);
    };
    auto load_d = [&](int l) { ld_frag<6>(fa.lay[l].down, oc, F / 32, wave, lane, wb); };
    auto load_l = [&](int s) { ld_frag<2>(fa.lm[s - 1], wg, DP / 32, wave, lane, wb); };
    if (own) ld_frag<4>(fa.proj, oc, DT / 32, wave, lane, wb);
    else load_q(0);

    // ---- owner state (waves 0..3): x of row 16 rf + 4 (lane / 16) + wave,
    // column 16 oc + lane % 16; the epilogues split a tile's four row
    // components over waves 0..3 the same way
    float xr[2] = {0.f, 0.f};
    const int erw = 4 * (lane >> 4) + wave;      // this wave's row in a 16-row fragment (waves 0..3)
    const int ocol = 16 * oc + (lane & 15);
    // embedding sum: owner thread t < 32 B holds row t / 32, column 32 oc + t % 32
    float es = 0.f;
    const int erow = threadIdx.x >> 5, ecol = 32 * oc + (threadIdx.x & 31);
    const bool eown = own && erow < B;

    // component `wave` (< 4) of the 16 waves' partial tiles, summed in wave order
    auto reduce = [&](int which) {
        const float* r = reinterpret_cast<const float*>(&red[which][0][lane]) + wave;
        float t = r[0];
#pragma unroll
        for (int w = 1; w < kW; ++w) t += r[w * 64 * 4];
        return t;
    };
    // wave w: the RMSNorm scale of fragment row w from the owners' sums
    // (lane c holds owner c's; the fixed reduction tree), after the barrier
    // that follows the polls
    auto row_scale = [&]() {
        const float sq = wave_sum(ss_s[lane * 16 + wave]);
        if (lane == 0) rinv_s[wave] = __builtin_amdgcn_rsqf(sq / static_cast<float>(DP) + eps);
    };
    // owner epilogue (waves 0..3): publish bf16(gain * x) pairs and the
    // 16-column sum of x^2 of this wave's row of fragment rf, if below M
    auto publish_x = [&](int rf, int M, int gj, uint32_t tag) {
        const int ln = fresh_lane();
        const int row = 16 * rf + 4 * (ln >> 4) + wave;
        const float v = xr[rf];
        const uint32_t hb = bf16_bits(gain_s[gj][ln & 15] * v);
        const uint32_t nb = __shfl_xor(hb, 1, 64);
        const float sq = tiled::sum16(v * v);
        if (row < M) {
            const uint32_t col = 16 * oc + (ln & 15);
            if ((ln & 1) == 0) st_rec64(rbuf(rc.XG), static_cast<uint32_t>(row) * (DP / 2) + col / 2, hb | (nb << 16), tag);
            if ((ln & 15) == 0) st_rec64(rbuf(rc.SS), static_cast<uint32_t>(oc) * kMaxRows + row, __float_as_uint(sq), tag);
        }
    };
    // the tokens of step sp (owners: every request, one wave per request;
    // units: their request): forced or own, checked and clamped; the owner
    // of column fragment 0 writes tokens_out and raises the flags
    auto decide_rows = [&](int sp, uint32_t tag) {
        if (wave < B) {
            const int tok = poll_token(rc.KEY, wave, tag, err);
            int f = a.force ? a.force[wave * kSteps + (sp - 1)] : tok;
            const bool bad = f < 0 || f >= V;
            if (lane == 0) {
                if (oc == 0) {
                    a.tok_out[wave * kSteps + (sp - 1)] = tok;
                    if (bad) atomicOr(err, kErrBadForced);
                }
                fed_s[wave] = bad ? 0 : f;
            }
        }
        __syncthreads();
        if (eown) es += emb_elem(m, sp, fed_s[erow], ecol);
    };

    // ================= INIT: x = W_p . H + b_p (rows < B), P_0[q0] (rows B .. 2B-1)
    if (own) {
        // H rows as bf16 operand rows, one wave per row
        if (wave < B) {
            const float4* hr = reinterpret_cast<const float4*>(a.H + static_cast<size_t>(wave) * DT);
            uint16_t* dst = stage + wave * kSRow;
#pragma unroll
            for (int j = 0; j < DT / 256; ++j) {
                const float4 v = hr[j * 64 + lane];
                *reinterpret_cast<uint2*>(dst + 4 * (j * 64 + lane)) =
                    make_uint2(tiled::pack_bf16x2(v.x, v.y), tiled::pack_bf16x2(v.z, v.w));
            }
        } else {
            zero_row<DT / 256>(stage + wave * kSRow);
        }
        if (threadIdx.x < kMaxB) {
            int q = threadIdx.x < B ? a.q0[threadIdx.x] : 0;
            if (q < 0 || q >= V) {
                if (oc == 0) atomicOr(err, kErrBadQ0);
                q = 0;
            }
            fed_s[threadIdx.x] = q;
        }
        __syncthreads();
        if (eown) es = emb_elem(m, 0, fed_s[erow], ecol);
        red[0][wave][lane] = mfma_slice<4>(stage, wave, lane, wb, f32x4_t{0.f, 0.f, 0.f, 0.f});
        __syncthreads();
        if (wave < 4) {
            const float t = reduce(0);
            const float bias = m.proj_b[ocol];
#pragma unroll
            for (int rf = 0; rf < 2; ++rf) {
                const int row = 16 * rf + erw;
                if (rf == 0 && row < B) xr[rf] = t + bias;
                else if (row >= B && row < 2 * B) xr[rf] = ldf(rbuf(m.ptab), static_cast<uint32_t>(fed_s[row - B]) * DP + ocol);
            }
            publish_x(0, 2 * B, L > 0 ? 0 : 2 * kMaxL, tag_of(0));
            publish_x(1, 2 * B, L > 0 ? 0 : 2 * kMaxL, tag_of(0));
        }
        load_q(0);
    }

    const float* t0 = m.qkv0;
    for (int s = 1; s <= kSteps; ++s) {
        const int M = (s == 1) ? 2 * B : B;
        const int nrf = (M + 15) / 16;
        if (s > 1 && own) {
            // the previous step's tokens, and layer 0's residual rows P_{s-1}[t]
            decide_rows(s - 1, tag_of(ph_lm(L, s - 1)));
            if (wave < 4) {
                xr[0] = erw < B ? ldf(rbuf(m.ptab), (static_cast<uint32_t>(s - 1) * V + fed_s[erw]) * DP + ocol) : 0.f;
                xr[1] = 0.f;
            }
        }
        for (int l = 0; l < L; ++l) {
            // ================= QKV(l): all workgroups, columns 16 wg .. +15
            if (!(l == 0 && s > 1)) {
                const uint32_t tin = (l == 0) ? tag_of(0) : tag_of(ph_layer(L, s, l - 1, T_DOWN));
                const uint32_t tout = tag_of(ph_layer(L, s, l, T_QKV));
                QP_STAMP(a.taps, wg, ph_layer(L, s, l, T_QKV), 0);
                #pragma unroll
                for (int rf = 0; rf < 2; ++rf) {
                    if (rf >= nrf) break;
                    const int row = 16 * rf + wave;
                    if (rf == 0) gate_row<DP / 256>(rc.XG, tin, err);
                    poll_row<DP / 256>(rc.XG + static_cast<size_t>(row) * (DP / 2), tin, stage + wave * kSRow, err,
                                       rc.SS, 16 * rf, M - 16 * rf, ss_s, row < M);
                    __syncthreads();
                    if (rf == 0) QP_STAMP(a.taps, wg, ph_layer(L, s, l, T_QKV), 1);
                    if (row < M) row_scale();
                    red[0][wave][lane] = mfma_slice<2>(stage, wave, lane, wb, f32x4_t{0.f, 0.f, 0.f, 0.f});
                    __syncthreads();
                    if (wave < 4) {
                        const float t = reduce(0);
                        const int ln = fresh_lane();
                        const int er = 4 * (ln >> 4) + wave, r = 16 * rf + er;
                        if (r < M)
                            st_rec64(rbuf(rc.QKV), static_cast<uint32_t>(r) * NQKV + 16 * wg + (ln & 15),
                                     __float_as_uint(t * rinv_s[er]), tout);
                    }
                    __syncthreads();
                }
                QP_STAMP(a.taps, wg, ph_layer(L, s, l, T_QKV), 2);
                // the attention units fetch their gate/up weights after
                // attention: requested here, they would sit ahead of the
                // units' polls in the CU's in-order memory queue
                stream::sched_fence();
                if (own) load_o(l);
                else if (!unit) load_u(l);
                stream::sched_fence();
            }
            // ================= ATTN(l): units (request ub, kv head ug)
            if (unit) {
                QP_STAMP(a.taps, wg, ph_layer(L, s, l, T_ATTN), 0);
                float* sf = reinterpret_cast<float*>(stage);
                float* hist = sf;                  // K [16][HD], then V [16][HD] at 2048
                float* nd = sf + 4096;             // head vectors [2 positions][4][HD]
                float* qb = sf + 5120;             // rotated query [2 waves][HD]
                float* eb = sf + 5376;             // softmax weights [2 waves][16]
                const int pf = (s == 1) ? 0 : s;
                const int npos = (s == 1) ? 2 : 1;
                const size_t kvb = ((static_cast<size_t>(l) * m.max_batch + ub) * kPositions) * NKV * HD;
                int fed = 0;
                if (l == 0 && s > 1) {
                    // this request's token of the previous step; its q/k/v rows from the table
                    if (wave == 0) {
                        const int tok = poll_token(rc.KEY, ub, tag_of(ph_lm(L, s - 1)), err);
                        int f = a.force ? a.force[ub * kSteps + (s - 2)] : tok;
                        if (lane == 0) fed_s[0] = (f < 0 || f >= V) ? 0 : f;
                    }
                    __syncthreads();
                    fed = fed_s[0];
                }
                // history: keys and values of positions < pf, LDS-direct loads
                if (wave >= 8) stream::hist_dma(m.kc, m.vc, kvb, ug, pf, hist, wave, 8, kW - 8);
                // head vectors: wave 4 pi + v takes vector v (q 2g, q 2g+1, k g, v g) of position pi.
                // Polled (not from the table), the value vector is left to
                // the computing waves, which wait for it only after the
                // softmax: its columns come from the owners, which reach the
                // q/k/v phase last (they end the down phase)
                const bool tab = l == 0 && s > 1;
                if (wave < 4 * npos && (tab || (wave & 3) != 3)) {
                    const int pi = wave >> 2, v = wave & 3;
                    const int col = v < 2 ? (2 * ug + v) * HD : (v == 2 ? (NQ + ug) * HD : (NQ + NKV + ug) * HD);
                    float* dst = nd + (pi * 4 + v) * HD;
                    if (l == 0 && s > 1) {
                        const float* trow = t0 + (static_cast<size_t>(s - 2) * V + fed) * NQKV + col;
                        *reinterpret_cast<float2*>(dst + 2 * lane) = *reinterpret_cast<const float2*>(trow + 2 * lane);
                    } else {
                        const int row = (s == 1) ? pi * B + ub : ub;
                        stream::poll_head(rc.QKV + static_cast<size_t>(row) * NQKV + col,
                                          tag_of(ph_layer(L, s, l, T_QKV)), dst, err);
                    }
                }
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                QP_STAMP(a.taps, wg, ph_layer(L, s, l, T_ATTN), 1);
                if (wave < 2) {
                    const int h = 2 * ug + wave;
                    const float* gq = qk_s[l][0];
                    const float* gk = qk_s[l][1];
                    float* qw = qb + 128 * wave;
                    float* ew = eb + 16 * wave;
                    const int kt = lane >> 2, kq = (lane & 3) * 32;
                    for (int pi = 0; pi < npos; ++pi) {
                        const int p = pf + pi;
                        const int row = (s == 1) ? pi * B + ub : ub;
                        const float* hv = nd + pi * 4 * HD;
                        // norms and RoPE with lane holding elements lane and
                        // lane + 64 (the rotate-half pair of element lane)
                        const float k0 = hv[2 * HD + lane], k1 = hv[2 * HD + lane + 64];
                        const float x0 = hv[wave * HD + lane], x1 = hv[wave * HD + lane + 64];
                        const float ca = rope_s[0][p * (HD / 2) + lane], sa = rope_s[1][p * (HD / 2) + lane];
                        float sq2[2] = {k0 * k0 + k1 * k1, x0 * x0 + x1 * x1};
                        wave_sums(sq2);
                        const float rk = __builtin_amdgcn_rsqf(sq2[0] / static_cast<float>(HD) + eps);
                        const float rq = __builtin_amdgcn_rsqf(sq2[1] / static_cast<float>(HD) + eps);
                        const float a0 = gk[lane] * (k0 * rk), a1 = gk[lane + 64] * (k1 * rk);
                        const float kv0 = a0 * ca - a1 * sa, kv1 = a1 * ca + a0 * sa;
                        const size_t off = kvb + (static_cast<size_t>(p) * NKV + ug) * HD;
                        if (wave == 0) {
                            st_act(m.kc + off + lane, kv0);
                            st_act(m.kc + off + lane + 64, kv1);
                        }
                        // both waves write the same values before reading them
                        hist[p * HD + lane] = kv0;
                        hist[p * HD + lane + 64] = kv1;
                        {
                            const float b0 = gq[lane] * (x0 * rq), b1 = gq[lane + 64] * (x1 * rq);
                            qw[lane] = b0 * ca - b1 * sa;
                            qw[lane + 64] = b1 * ca + b0 * sa;
                        }
                        // scores: key t on lanes 4t .. 4t+3, a 32-wide slice each
                        float sc = 0.f;
                        if (kt <= p) {
#pragma unroll
                            for (int i = 0; i < 32; i += 4) {
                                const float4 qv = *reinterpret_cast<const float4*>(qw + kq + i);
                                const float4 kk = *reinterpret_cast<const float4*>(hist + kt * HD + kq + i);
                                sc = fmaf(qv.x, kk.x, sc);
                                sc = fmaf(qv.y, kk.y, sc);
                                sc = fmaf(qv.z, kk.z, sc);
                                sc = fmaf(qv.w, kk.w, sc);
                            }
                        }
                        sc += dpp_or_zero<0xB1, 0xF>(sc);
                        sc += dpp_or_zero<0x4E, 0xF>(sc);
                        sc = (kt <= p) ? sc * m.attn_scale : -__builtin_huge_valf();
                        const float mx = wave_max(sc);
                        const float e = (kt <= p) ? __expf(sc - mx) : 0.f;
                        const float den = wave_sum((lane & 3) == 0 ? e : 0.f);
                        if ((lane & 3) == 0) ew[kt] = e;
                        // this position's value vector joins the history (and
                        // the cache): from the table, or awaited only now
                        if (tab) {
                            const float vv0 = hv[3 * HD + lane], vv1 = hv[3 * HD + lane + 64];
                            if (wave == 0) {
                                st_act(m.vc + off + lane, vv0);
                                st_act(m.vc + off + lane + 64, vv1);
                            }
                            hist[2048 + p * HD + lane] = vv0;
                            hist[2048 + p * HD + lane + 64] = vv1;
                        } else {
                            float* vrow = hist + 2048 + p * HD;
                            stream::poll_head(rc.QKV + static_cast<size_t>(row) * NQKV + (NQ + NKV + ug) * HD,
                                              tag_of(ph_layer(L, s, l, T_QKV)), vrow, err);
                            if (wave == 0) {
                                // one 8-byte store per lane: the wave writes the row's 512 bytes contiguously
                                const uint64_t vv = *reinterpret_cast<const uint64_t*>(vrow + 2 * lane);
                                __hip_atomic_store(reinterpret_cast<uint64_t*>(m.vc + off + 2 * lane), vv, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
                            }
                        }
                        // weighted values, elements 2 lane and 2 lane + 1 (one
                        // record); each half's LDS reads issued before its products
                        float o0 = 0.f, o1 = 0.f;
#pragma unroll
                        for (int t0h = 0; t0h < kPositions; t0h += kPositions / 2) {
                            float w8[kPositions / 2];
                            float2 vr[kPositions / 2];
#pragma unroll
                            for (int t = 0; t < kPositions / 2; ++t) {
                                const int tt = t0h + t <= p ? t0h + t : p;     // weight 0 beyond p
                                w8[t] = ew[t0h + t];
                                vr[t] = *reinterpret_cast<const float2*>(hist + 2048 + tt * HD + 2 * lane);
                            }
#pragma unroll
                            for (int t = 0; t < kPositions / 2; ++t) {
                                o0 = fmaf(w8[t], vr[t].x, o0);
                                o1 = fmaf(w8[t], vr[t].y, o1);
                            }
                        }
                        const float rden = __builtin_amdgcn_rcpf(den);
                        st_rec64(rbuf(rc.AO), static_cast<uint32_t>(row) * (QD / 2) + h * (HD / 2) + fresh_lane(),
                                 bf16_bits(o0 * rden) | (bf16_bits(o1 * rden) << 16), tag_of(ph_layer(L, s, l, T_ATTN)));
                    }
                }
                __syncthreads();
                QP_STAMP(a.taps, wg, ph_layer(L, s, l, T_ATTN), 2);
                if (!(l == 0 && s > 1)) {   // layer 0 of later steps: fetched after the last lm_head
                    stream::sched_fence();
                    load_u(l);
                    stream::sched_fence();
                }
            }
            // ================= O(l): owners, x += W_o . attention
            if (own) {
                const uint32_t tin = tag_of(ph_layer(L, s, l, T_ATTN));
                QP_STAMP(a.taps, wg, ph_layer(L, s, l, T_O), 0);
                #pragma unroll
                for (int rf = 0; rf < 2; ++rf) {
                    if (rf >= nrf) break;
                    const int row = 16 * rf + wave;
                    if (rf == 0) gate_row<QD / 256>(rc.AO, tin, err);
                    if (row < M) poll_row<QD / 256>(rc.AO + static_cast<size_t>(row) * (QD / 2), tin, stage + wave * kSRow, err);
                    else zero_row<QD / 256>(stage + wave * kSRow);
                    __syncthreads();
                    if (rf == 0) QP_STAMP(a.taps, wg, ph_layer(L, s, l, T_O), 1);
                    red[0][wave][lane] = mfma_slice<4>(stage, wave, lane, wb, f32x4_t{0.f, 0.f, 0.f, 0.f});
                    __syncthreads();
                    if (wave < 4) {
                        xr[rf] += reduce(0);
                        publish_x(rf, M, 2 * l + 1, tag_of(ph_layer(L, s, l, T_O)));
                    }
                    __syncthreads();
                }
                QP_STAMP(a.taps, wg, ph_layer(L, s, l, T_O), 2);
                stream::sched_fence();
                load_d(l);
                stream::sched_fence();
            }
            // ================= UP(l): gate/up columns 16 wg .. +15, SwiGLU
            if (up_role) {
                const uint32_t tin = tag_of(ph_layer(L, s, l, T_O));
                const uint32_t tout = tag_of(ph_layer(L, s, l, T_UP));
                QP_STAMP(a.taps, wg, ph_layer(L, s, l, T_UP), 0);
                #pragma unroll
                for (int rf = 0; rf < 2; ++rf) {
                    if (rf >= nrf) break;
                    const int row = 16 * rf + wave;
                    if (rf == 0) gate_row<DP / 256>(rc.XG, tin, err);
                    poll_row<DP / 256>(rc.XG + static_cast<size_t>(row) * (DP / 2), tin, stage + wave * kSRow, err,
                                       rc.SS, 16 * rf, M - 16 * rf, ss_s, row < M);
                    __syncthreads();
                    if (rf == 0) QP_STAMP(a.taps, wg, ph_layer(L, s, l, T_UP), 1);
                    if (row < M) row_scale();
                    red[0][wave][lane] = mfma_slice<2>(stage, wave, lane, wb, f32x4_t{0.f, 0.f, 0.f, 0.f});
                    red[1][wave][lane] = mfma_slice<2>(stage, wave, lane, wb + 2, f32x4_t{0.f, 0.f, 0.f, 0.f});
                    __syncthreads();
                    if (wave < 4) {
                        const int ln = fresh_lane();
                        const int er = 4 * (ln >> 4) + wave, r = 16 * rf + er;
                        const float ri = rinv_s[er];
                        const float gv = reduce(0) * ri, uv = reduce(1) * ri;
                        const float hv = (gv / (1.0f + __expf(-gv))) * uv;
                        const uint32_t hb = bf16_bits(hv);
                        const uint32_t nb = __shfl_xor(hb, 1, 64);
                        if (r < M && (ln & 1) == 0)
                            st_rec64(rbuf(rc.HH), static_cast<uint32_t>(r) * (F / 2) + (16 * wg + (ln & 15)) / 2,
                                     hb | (nb << 16), tout);
                    }
                    __syncthreads();
                }
                QP_STAMP(a.taps, wg, ph_layer(L, s, l, T_UP), 2);
                stream::sched_fence();
                if (l + 1 < L) load_q(l + 1);
                else if (lm_role) load_l(s);
                else if (s < kSteps) load_u(0);
                stream::sched_fence();
            }
            // ================= DOWN(l): owners, x += W_d . h
            if (own) {
                const uint32_t tin = tag_of(ph_layer(L, s, l, T_UP));
                const uint32_t tout = tag_of(ph_layer(L, s, l, T_DOWN));
                const int gnext = (l + 1 < L) ? 2 * (l + 1) : 2 * kMaxL;   // gain row of the next reader
                QP_STAMP(a.taps, wg, ph_layer(L, s, l, T_DOWN), 0);
                #pragma unroll
                for (int rf = 0; rf < 2; ++rf) {
                    if (rf >= nrf) break;
                    const int row = 16 * rf + wave;
                    if (rf == 0) gate_row<F / 256>(rc.HH, tin, err);
                    if (row < M) poll_row<F / 256>(rc.HH + static_cast<size_t>(row) * (F / 2), tin, stage + wave * kSRow, err);
                    else zero_row<F / 256>(stage + wave * kSRow);
                    __syncthreads();
                    if (rf == 0) QP_STAMP(a.taps, wg, ph_layer(L, s, l, T_DOWN), 1);
                    red[0][wave][lane] = mfma_slice<6>(stage, wave, lane, wb, f32x4_t{0.f, 0.f, 0.f, 0.f});
                    __syncthreads();
                    if (wave < 4) {
                        xr[rf] += reduce(0);
                        publish_x(rf, M, gnext, tout);
                        const int r = 16 * rf + erw;
                        if (kWriteTaps && a.taps && r < M) {
                            const int pos = row_pos(s, B, r), bb = row_req(s, B, r);
                            a.taps[((static_cast<size_t>(pos) * L + l) * B + bb) * DP + ocol] = xr[rf];
                        }
                    }
                    __syncthreads();
                }
                QP_STAMP(a.taps, wg, ph_layer(L, s, l, T_DOWN), 2);
                stream::sched_fence();
                if (l + 1 < L) load_q(l + 1);
                else if (s < kSteps) load_o(0);
                stream::sched_fence();
            }
        }
        // ================= LM(s): vocabulary columns 16 wg .. +15, per-row argmax keys
        if (lm_role) {
            const uint32_t tin = tag_of(ph_layer(L, s, L - 1, T_DOWN));
            const uint32_t tout = tag_of(ph_lm(L, s));
            const int r0 = (s == 1) ? B : 0;
            QP_STAMP(a.taps, wg, ph_lm(L, s), 0);
            gate_row<DP / 256>(rc.XG + static_cast<size_t>(r0) * (DP / 2), tin, err);
            poll_row<DP / 256>(rc.XG + static_cast<size_t>(r0 + wave) * (DP / 2), tin, stage + wave * kSRow, err,
                               rc.SS, r0, B, ss_s, wave < B);
            __syncthreads();
            QP_STAMP(a.taps, wg, ph_lm(L, s), 1);
            if (wave < B) row_scale();
            red[0][wave][lane] = mfma_slice<2>(stage, wave, lane, wb, f32x4_t{0.f, 0.f, 0.f, 0.f});
            __syncthreads();
            if (wave < 4) {
                const int ln = fresh_lane();
                const int col = 16 * wg + (ln & 15);
                const int b = 4 * (ln >> 4) + wave;
                const float lg = reduce(0) * rinv_s[b];
                if (a.logits_out && b < B) a.logits_out[(static_cast<size_t>(b) * kSteps + (s - 1)) * V + col] = lg;
                uint64_t key = argmax_key(lg, col);
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) {
                    const uint64_t k2 = tiled::shfl_xor64(key, o);
                    key = k2 > key ? k2 : key;
                }
                if ((ln & 15) == 0 && b < B) {
                    const uint32_t kr = (static_cast<uint32_t>(wg) * kMaxB + b) * 2;
                    st_rec64(rbuf(rc.KEY), kr, static_cast<uint32_t>(key >> 32), tout);
                    st_rec64(rbuf(rc.KEY), kr + 1, static_cast<uint32_t>(argmax_index(key)), tout);
                }
            }
            __syncthreads();
            QP_STAMP(a.taps, wg, ph_lm(L, s), 2);
            stream::sched_fence();
            if (s < kSteps) load_u(0);
            stream::sched_fence();
        }
    }
    // ================= FINAL: the last tokens; the embedding sum out
    if (own) {
        decide_rows(kSteps, tag_of(ph_lm(L, kSteps)));
        if (eown) a.embsum[static_cast<size_t>(erow) * DT + ecol] = es;
    }
}

}  // namespace flow
}  // namespace qp

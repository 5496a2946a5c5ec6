// Talker decode step: one position per request through the long-context
// transformer that yields the frame hidden state H and the first codebook
// token q0 (mixtureofinsights OpenVINO port, section 1 diagram and sections
// 2.1-2.2; hackernews.jp translation of the Nari Labs post,
// "Qwen3-TTSの最適化方法").  Geometry, block tensors and the 3072-row codec
// table follow the rightkit-qts exporter README ("Loader contract" and
// "Expected verification shapes").
//
// The step is B rows wide, so its products are the batched matrix-core
// kernels (k_gemm: fragment-order weights on v_mfma_f32_16x16x32_bf16, the
// RMSNorm folded into the operand and the row scale).  What is new here:
//
//  * k_input: the caller's input rows enter the residual stream and publish
//    the first product's operand (bf16(attn_norm * x)) with 16-column sums
//    of x^2;
//  * k_attn: attention of one position over the request's whole history.
//    The history is a bf16 cache per request slot, laid out
//    [slot][layer][kv head][position][hd] so a head's keys stream
//    contiguously.  The context is split over workgroups (grid = splits x kv
//    heads x rows): each computes its query heads' norm and RoPE, scores
//    its chunk of positions (HD/8 lanes per position, one 16-byte load per
//    lane), the chunk's softmax statistics and weighted values, and
//    publishes (max, sum, values) with device-coherent stores; the last
//    split to arrive (one counter per request and kv head, left at zero)
//    combines them in split order.  The split holding the current position
//    also norms, rotates and rounds the new key and value, writes them to
//    the cache and uses them directly;
//  * k_final: H = output_norm * x / rms(x) and q0 from the codec head's
//    per-tile argmax keys.
//
// Positions: the multimodal RoPE's three position streams carry the same
// index for codec frames, so the rotation is rotate-half RoPE at the
// absolute position with one frequency ladder over the head.
#pragma once

#include "qp_common.h"
#include "qp_phases.h"
#include "qp_tiled.h"

namespace qp {
namespace talker {

constexpr int kThreadsK = 256;
constexpr int kMaxCh = 64;               // positions per attention split
constexpr unsigned kErrBadPos = 1u;      // a position outside [0, max_len)
constexpr unsigned kErrBadSlot = 2u;     // a slot outside [0, n_slots)

struct InArgs {
    int d;
    const float* x_in;     // [B][d] the caller's rows
    float* x;              // [B][d] residual stream
    uint16_t* xg;          // bf16(gain0 * x), width d (qp::tiled::act_index layout)
    float* ss;             // [B][d/16] 16-column sums of x^2
    const float* gain0;    // layer 0's attn_norm (output_norm without layers)
    int frag;              // activations in fragment order
};

__global__ __launch_bounds__(kThreadsK) void k_input(InArgs a) {
    const int b = blockIdx.x;
    const float* src = a.x_in + static_cast<size_t>(b) * a.d;
    float* dst = a.x + static_cast<size_t>(b) * a.d;
    for (int f = threadIdx.x; f < a.d / 16; f += kThreadsK) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 t = reinterpret_cast<const float4*>(src + 16 * f)[i];
            v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
            reinterpret_cast<float4*>(dst + 16 * f)[i] = t;
        }
        float s = 0.f;
        uint32_t pk[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            s = fmaf(v[2 * i], v[2 * i], s);
            s = fmaf(v[2 * i + 1], v[2 * i + 1], s);
            pk[i] = qp::tiled::pack_bf16x2(a.gain0[16 * f + 2 * i] * v[2 * i], a.gain0[16 * f + 2 * i + 1] * v[2 * i + 1]);
        }
        // eight consecutive columns from a multiple of 8 are contiguous in either layout
        *reinterpret_cast<uint4*>(a.xg + qp::tiled::act_index(b, 16 * f, a.d, a.frag)) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        *reinterpret_cast<uint4*>(a.xg + qp::tiled::act_index(b, 16 * f + 8, a.d, a.frag)) =
            make_uint4(pk[4], pk[5], pk[6], pk[7]);
        a.ss[static_cast<size_t>(b) * (a.d / 16) + f] = s;
    }
}

struct AttnArgs {
    int nkv, nqkv, qd, l, L, max_ctx, n_slots, ch, nsplit;
    float eps, scale;
    const float* qkv;                 // [B][nqkv]: q heads, k heads, v heads
    const float* q_norm;              // [hd]
    const float* k_norm;              // [hd]
    const float* rope_cos;            // [max_ctx][hd/2]
    const float* rope_sin;
    const int* slots;                 // [B]
    const int* pos;                   // [B] position of this step (= history length)
    uint16_t* kc;                     // [n_slots][L][nkv][max_ctx][hd] bf16
    uint16_t* vc;
    float* part;                      // [B][nq][nsplit][hd + 2]: max, sum, values
    unsigned* ctr;                    // [B][nkv] arrival counters, left at 0
    uint16_t* ao;                     // bf16 attention output, width qd (qp::tiled::act_index layout)
    int frag;                         // activations in fragment order
    unsigned* err;
    // prepared graphs (grid for max_ctx and a batch bucket): null, or the
    // call's limits written before the replay, {splits the call's max_len
    // covers, rows B}; rows at or past B are padding and exit at once
    const int* live;
};

__global__ void k_set_live(int* live, int nsplit, int B) {
    if (threadIdx.x == 0) {
        live[0] = nsplit;
        live[1] = B;
    }
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// R query heads share kv head g (R = nq / nkv, 1 or 2): waves 0..R-1 own the
// query heads, waves 2 and 3 the new key and value.
template <int HD, int R>
__global__ __launch_bounds__(kThreadsK) void k_attn(AttnArgs a) {
    static_assert(HD % 64 == 0 && HD <= 256 && (R == 1 || R == 2), "head layout");
    constexpr int J = HD / 64;          // elements per lane of a head vector
    constexpr int LP = HD / 8;          // lanes per position when scoring
    constexpr int PPW = 64 / LP;        // positions per wave per pass
    __shared__ float q_s[R][HD];
    __shared__ float kn_s[HD], vn_s[HD];
    __shared__ float w_s[R][kMaxCh];    // scores, then softmax weights
    __shared__ float red_s[4][R][HD];
    __shared__ float st_s[R][2];
    __shared__ int last_s;

    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int lim = a.nsplit;                  // splits the call's max_len covers
    if (a.live) {
        if (b >= a.live[1]) return;      // a padding row of the batch bucket
        lim = a.live[0];
    }
    int p = a.pos[b], slot = a.slots[b];
    // a row with a position or slot out of range raises the flag, is computed
    // at position 0 of slot 0 and writes nothing into the cache
    bool valid = true;
    if (p < 0 || p >= lim * a.ch || p >= a.max_ctx) {
        if (s == 0 && g == 0 && threadIdx.x == 0) atomicOr(a.err, kErrBadPos);
        p = 0;
        valid = false;
    }
    if (slot < 0 || slot >= a.n_slots) {
        if (s == 0 && g == 0 && threadIdx.x == 0) atomicOr(a.err, kErrBadSlot);
        slot = 0;
        valid = false;
    }
    const int n = p + 1;
    const int p0 = s * a.ch;
    if (p0 >= n) return;                 // past this request's history
    const int cnt = min(a.ch, n - p0);
    const int nsb = (n + a.ch - 1) / a.ch;
    const bool has_new = p < p0 + cnt;   // the split holding this step's position
    const size_t hbase = ((static_cast<size_t>(slot) * a.L + a.l) * a.nkv + g) * a.max_ctx;
    const uint16_t* kh = a.kc + hbase * HD;
    const uint16_t* vh = a.vc + hbase * HD;
    const float* row = a.qkv + static_cast<size_t>(b) * a.nqkv;

    // this wave's head vector of the step (query, or in the last split the
    // new key or value): requested first, since loads complete in order
    float hv[J];
    {
        int off = -1;
        if (wave < R) off = (g * R + wave) * HD;
        else if (has_new && wave == 2) off = a.qd + g * HD;
        else if (has_new && wave == 3) off = a.qd + (a.nkv + g) * HD;
#pragma unroll
        for (int j = 0; j < J; ++j) hv[j] = off >= 0 ? row[off + lane + 64 * j] : 0.f;
    }

    // the norm gains and the RoPE row of this wave's head, requested before
    // the history, so that the norm need not wait for it (the loads of a
    // wave complete in order)
    float hg[J];
    qp::tiled::RopeRow<HD> hr;
    qp::tiled::gain_fetch<HD>(wave < R ? a.q_norm : a.k_norm, hg);
    qp::tiled::rope_fetch<HD>(a.rope_cos, a.rope_sin, p, hr);

    // 0. the chunk's cached keys and values, requested before anything else
    //    (they do not depend on this step): LP lanes per position, 8
    //    elements (16 bytes) each, PPW positions per wave per pass, the same
    //    positions for keys and values
    constexpr int KP = kMaxCh / (4 * PPW);
    const int grp = lane / LP, sub = lane % LP;
    uint4 kraw[KP], vraw[KP];
#pragma unroll
    for (int i = 0; i < KP; ++i) {
        const int t = i * 4 * PPW + wave * PPW + grp;
        kraw[i] = make_uint4(0u, 0u, 0u, 0u);
        vraw[i] = make_uint4(0u, 0u, 0u, 0u);
        if (t < cnt && p0 + t != p) {
            kraw[i] = *reinterpret_cast<const uint4*>(kh + static_cast<size_t>(p0 + t) * HD + sub * 8);
            vraw[i] = *reinterpret_cast<const uint4*>(vh + static_cast<size_t>(p0 + t) * HD + sub * 8);
        }
    }

    // 1. queries (per-head norm, RoPE); in the last split also the new key
    //    and value, rounded to bf16 into the cache
    if (wave < R) {
        float o[J];
        qp::tiled::norm_rope_apply<HD>(hv, hg, hr, a.eps, o);
#pragma unroll
        for (int j = 0; j < J; ++j) q_s[wave][lane + 64 * j] = o[j];
    } else if (has_new && wave == 2) {
        float o[J];
        qp::tiled::norm_rope_apply<HD>(hv, hg, hr, a.eps, o);
        uint16_t* dst = a.kc + (hbase + p) * HD;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const uint16_t r16 = qp::tiled::to_bf16(o[j]);
            if (valid) dst[lane + 64 * j] = r16;
            kn_s[lane + 64 * j] = bf16_to_f32(r16);
        }
    } else if (has_new && wave == 3) {
        uint16_t* dst = a.vc + (hbase + p) * HD;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const uint16_t r16 = qp::tiled::to_bf16(hv[j]);
            if (valid) dst[lane + 64 * j] = r16;
            vn_s[lane + 64 * j] = bf16_to_f32(r16);
        }
    }
    __syncthreads();

    // 2. scores: LP lanes per position, 8 elements each
    float qr[R][8];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < 8; ++i) qr[r][i] = q_s[r][sub * 8 + i];
#pragma unroll
    for (int i = 0; i < KP; ++i) {
        const int t = i * 4 * PPW + wave * PPW + grp;
        float k8[8];
        if (p0 + t != p) {
            const uint32_t w4[4] = {kraw[i].x, kraw[i].y, kraw[i].z, kraw[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                k8[2 * e] = __uint_as_float(w4[e] << 16);
                k8[2 * e + 1] = __uint_as_float(w4[e] & 0xFFFF0000u);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) k8[e] = kn_s[sub * 8 + e];
        }
        float d[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            d[r] = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) d[r] = fmaf(qr[r][e], k8[e], d[r]);
#pragma unroll
            for (int o = 1; o < LP; o <<= 1) d[r] += __shfl_xor(d[r], o, 64);
        }
        if (t < cnt && sub == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) w_s[r][t] = d[r] * a.scale;
        }
    }
    __syncthreads();

    // 3. the chunk's softmax statistics (wave r: query head r)
    if (wave < R) {
        float mx = -__builtin_huge_valf();
        for (int t = lane; t < cnt; t += 64) mx = fmaxf(mx, w_s[wave][t]);
        mx = wave_max(mx);
        float sum = 0.f;
        for (int t = lane; t < cnt; t += 64) {
            const float e = __expf(w_s[wave][t] - mx);
            w_s[wave][t] = e;
            sum += e;
        }
        sum = wave_sum(sum);
        if (lane == 0) {
            st_s[wave][0] = mx;
            st_s[wave][1] = sum;
        }
    }
    __syncthreads();

    // 4. weighted values, over the positions of the scores: a lane sums
    //    elements sub*8 .. +7 over its positions, the PPW position groups of
    //    a wave are then added across lanes (the same result in every lane
    //    of a column), and the four waves through LDS in wave order
    float acc[R][8];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
#pragma unroll
    for (int i = 0; i < KP; ++i) {
        const int t = i * 4 * PPW + wave * PPW + grp;
        if (t < cnt) {
            float v8[8];
            if (p0 + t != p) {
                const uint32_t w4[4] = {vraw[i].x, vraw[i].y, vraw[i].z, vraw[i].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v8[2 * e] = __uint_as_float(w4[e] << 16);
                    v8[2 * e + 1] = __uint_as_float(w4[e] & 0xFFFF0000u);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v8[e] = vn_s[sub * 8 + e];
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float w = w_s[r][t];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(w, v8[e], acc[r][e]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
#pragma unroll
            for (int o = LP; o < 64; o <<= 1) acc[r][e] += __shfl_xor(acc[r][e], o, 64);
        }
    if (grp == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) red_s[wave][r][sub * 8 + e] = acc[r][e];
    }
    __syncthreads();
    float o[J];
    if (wave < R) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int e = lane * J + j;
            o[j] = ((red_s[0][wave][e] + red_s[1][wave][e]) + red_s[2][wave][e]) + red_s[3][wave][e];
        }
    }

    // 5. one split: the output directly; several: publish, the last combines
    const int nq = a.nkv * R;
    if (nsb == 1) {
        if (wave < R) {
            const float rl = 1.0f / st_s[wave][1];
#pragma unroll
            for (int j = 0; j < J; ++j)
                a.ao[qp::tiled::act_index(b, (g * R + wave) * HD + lane * J + j, a.qd, a.frag)] =
                    qp::tiled::to_bf16(o[j] * rl);
        }
        return;
    }
    if (wave < R) {
        float* ph = a.part + ((static_cast<size_t>(b) * nq + g * R + wave) * a.nsplit + s) * (HD + 2);
        const auto pw = __builtin_amdgcn_make_buffer_rsrc(ph, static_cast<short>(0), (HD + 2) * 4, 0x00020000);
#pragma unroll
        for (int j = 0; j < J; ++j)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, o[j]), pw,
                                                  static_cast<uint32_t>(2 + lane * J + j) * 4u, 0u, qp::tiled::kDevScope);
        if (lane == 0) {
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, st_s[wave][0]), pw, 0u, 0u, qp::tiled::kDevScope);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, st_s[wave][1]), pw, 4u, 0u, qp::tiled::kDevScope);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned* c = a.ctr + static_cast<size_t>(b) * a.nkv + g;
        const unsigned old = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = old == static_cast<unsigned>(nsb - 1);
        if (last) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_s = last;
    }
    __syncthreads();
    if (!last_s || wave >= R) return;
    // combine: lane z holds split z's (max, sum); the values are summed over
    // the splits in split order, lanes across the head's elements
    const float* ph0 = a.part + (static_cast<size_t>(b) * nq + g * R + wave) * a.nsplit * (HD + 2);
    const auto pr = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(ph0), static_cast<short>(0),
                                                      static_cast<int>(static_cast<size_t>(nsb) * (HD + 2) * 4), 0x00020000);
    float f = 0.f, Ls = 0.f;
    {
        float mz = -__builtin_huge_valf(), lz = 0.f;
        for (int z = lane; z < nsb; z += 64) {   // nsb <= 64 in practice; more splits wrap
            const float m1 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(pr, static_cast<uint32_t>(z) * (HD + 2) * 4u, 0u, qp::tiled::kDevScope));
            const float l1 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(pr, (static_cast<uint32_t>(z) * (HD + 2) + 1u) * 4u, 0u, qp::tiled::kDevScope));
            if (m1 > mz) {
                lz = lz * __expf(mz - m1) + l1;
                mz = m1;
            } else {
                lz += l1 * __expf(m1 - mz);
            }
        }
        // the maximum over the lanes, then every lane's sum rescaled to it
        const float M = wave_max(mz);
        Ls = wave_sum(lz * __expf(mz - M));
        f = M;                                   // the common maximum
    }
    const float M = f;
    float O[J];
#pragma unroll
    for (int j = 0; j < J; ++j) O[j] = 0.f;
    for (int z0 = 0; z0 < nsb; z0 += 8) {
        float mv[8], ov[8][J];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int z = z0 + u < nsb ? z0 + u : nsb - 1;
            mv[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(pr, static_cast<uint32_t>(z) * (HD + 2) * 4u, 0u, qp::tiled::kDevScope));
#pragma unroll
            for (int j = 0; j < J; ++j)
                ov[u][j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                    pr, (static_cast<uint32_t>(z) * (HD + 2) + 2u + static_cast<uint32_t>(lane * J + j)) * 4u, 0u,
                    qp::tiled::kDevScope));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (z0 + u < nsb) {
                const float w = __expf(mv[u] - M);
#pragma unroll
                for (int j = 0; j < J; ++j) O[j] = fmaf(ov[u][j], w, O[j]);
            }
        }
    }
    const float rl = 1.0f / Ls;
#pragma unroll
    for (int j = 0; j < J; ++j)
        a.ao[qp::tiled::act_index(b, (g * R + wave) * HD + lane * J + j, a.qd, a.frag)] = qp::tiled::to_bf16(O[j] * rl);
}

struct FinArgs {
    int d, nkt;
    float eps;
    const float* x;                   // [B][d] residual stream after the last layer
    const float* ss;                  // [B][d/16]
    const float* g_out;               // output_norm [d]
    const unsigned long long* keys;   // [B][nkt] codec head tile keys
    float* H_out;                     // [B][d]
    int* q0_out;                      // [B]
};

__global__ __launch_bounds__(kThreadsK) void k_final(FinArgs a) {
    __shared__ float red[kThreadsK / 64];
    __shared__ unsigned long long kred[kThreadsK / 64];
    const int b = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nf = a.d / 16;
    // the first 8 * kThreadsK elements of the row and the gains, requested
    // with the sums below (one round trip for the whole kernel at d <= 2048)
    constexpr int kU = 8;
    const float* xrow = a.x + static_cast<size_t>(b) * a.d;
    float xv[kU], gv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int c = min(u * kThreadsK + static_cast<int>(threadIdx.x), a.d - 1);
        xv[u] = xrow[c];
        gv[u] = a.g_out[c];
    }
    float t = 0.f;
    for (int f = threadIdx.x; f < nf; f += kThreadsK) t += a.ss[static_cast<size_t>(b) * nf + f];
    t = wave_sum(t);
    unsigned long long k = 0;
    for (int i = threadIdx.x; i < a.nkt; i += kThreadsK) k = qp::tiled::umax64(k, a.keys[static_cast<size_t>(b) * a.nkt + i]);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) k = qp::tiled::umax64(k, qp::tiled::shfl_xor64(k, off));
    if (lane == 0) {
        red[wave] = t;
        kred[wave] = k;
    }
    __syncthreads();
    const float tot = ((red[0] + red[1]) + red[2]) + red[3];
    const float rinv = 1.0f / sqrtf(tot / static_cast<float>(a.d) + a.eps);
    float* hrow = a.H_out + static_cast<size_t>(b) * a.d;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int c = u * kThreadsK + static_cast<int>(threadIdx.x);
        if (c < a.d) hrow[c] = gv[u] * (xv[u] * rinv);
    }
    for (int c0 = kU * kThreadsK; c0 < a.d; c0 += kU * kThreadsK) {   // d > 2048: the rest, 8 at a time
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int c = min(c0 + u * kThreadsK + static_cast<int>(threadIdx.x), a.d - 1);
            xv[u] = xrow[c];
            gv[u] = a.g_out[c];
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int c = c0 + u * kThreadsK + static_cast<int>(threadIdx.x);
            if (c < a.d) hrow[c] = gv[u] * (xv[u] * rinv);
        }
    }
    if (threadIdx.x == 0) {
        unsigned long long kk = kred[0];
        for (int w = 1; w < kThreadsK / 64; ++w) kk = qp::tiled::umax64(kk, kred[w]);
        a.q0_out[b] = argmax_index(kk);
    }
}

// a history of n positions for one slot: bf16 [L][n][nkv][hd] -> the cache
// layout [slot][L][nkv][max_ctx][hd]
__global__ void k_load_history(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, uint16_t* kc,
                               uint16_t* vc, int slot, int n, int L, int nkv, int hd, int max_ctx) {
    const size_t total = static_cast<size_t>(L) * n * nkv * hd;
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
         i += static_cast<size_t>(gridDim.x) * blockDim.x) {
        const int e = static_cast<int>(i % hd);
        size_t r = i / hd;
        const int g = static_cast<int>(r % nkv);
        r /= nkv;
        const int p = static_cast<int>(r % n);
        const int l = static_cast<int>(r / n);
        const size_t dst = ((((static_cast<size_t>(slot) * L + l) * nkv + g) * max_ctx) + p) * hd + e;
        kc[dst] = k[i];
        vc[dst] = v[i];
    }
}

}  // namespace talker
}  // namespace qp

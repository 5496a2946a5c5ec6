// Phases of one code-predictor frame, written as workgroup-strided device
// functions: each takes (wg, nwg) and does that workgroup's share, so the
// same code runs as one kernel per phase or inside one persistent kernel
// with grid barriers between phases.  Results never depend on nwg or on the
// batch composition: every output element is reduced in a fixed order that
// only depends on the geometry.
#pragma once

#include "qp_common.h"

namespace qp {

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or_zero(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

// Sum over the 64 lanes with DPP moves (pairs, quads, half rows, rows, then
// the two row broadcasts); the total lands in lane 63 and is broadcast.  The
// summation tree is fixed, so every call reduces in the same order.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_or_zero<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v += dpp_or_zero<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    v += dpp_or_zero<0x141, 0xF>(v);  // row_half_mirror
    v += dpp_or_zero<0x140, 0xF>(v);  // row_mirror
    v += dpp_or_zero<0x142, 0xA>(v);  // row_bcast15 into rows 1, 3
    v += dpp_or_zero<0x143, 0xC>(v);  // row_bcast31 into rows 2, 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// N independent wave sums, stage by stage, so that the DPP moves of one sum
// fill the wait states of the others; same tree (and result) as wave_sum.
template <int N>
__device__ __forceinline__ void wave_sums(float (&v)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp_or_zero<0xB1, 0xF>(v[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp_or_zero<0x4E, 0xF>(v[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp_or_zero<0x141, 0xF>(v[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp_or_zero<0x140, 0xF>(v[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp_or_zero<0x142, 0xA>(v[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp_or_zero<0x143, 0xC>(v[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[i]), 63));
}

// Maximum over the 64 lanes with DPP moves (lanes a move does not reach keep
// their own value); broadcast from lane 63.
template <unsigned CTRL, unsigned ROW_MASK>
__device__ __forceinline__ float dpp_or_self(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_or_self<0xB1, 0xF>(v));
    v = fmaxf(v, dpp_or_self<0x4E, 0xF>(v));
    v = fmaxf(v, dpp_or_self<0x141, 0xF>(v));
    v = fmaxf(v, dpp_or_self<0x140, 0xF>(v));
    v = fmaxf(v, dpp_or_self<0x142, 0xA>(v));
    v = fmaxf(v, dpp_or_self<0x143, 0xC>(v));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float block_sum(float v) {
    __shared__ float red[kWaves];
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) t += red[i];
    return t;
}

// Activations cross workgroups (and XCDs) between phases.  They move with
// device-scope loads and stores, which bypass the per-XCD L2 copies, so the
// grid barrier needs no cache writeback or invalidation.
__device__ __forceinline__ float ld_act(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_act(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ float emb_elem(const Model& m, int j, int row, int k) {
    const size_t off = static_cast<size_t>(row) * m.dT + k;
    return m.emb_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(m.emb[j])[off])
                      : static_cast<const float*>(m.emb[j])[off];
}

// Eight consecutive weights W[n][k0 .. k0+7] as fp32 (exact for every format).
template <int WT>
__device__ __forceinline__ void load_w8(const Mat& W, int K, int n, int k0, float w[8]) {
    const size_t off = static_cast<size_t>(n) * K + k0;
    if constexpr (WT == WT_F32) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(W.w) + off);
        const float4 a = p[0], b = p[1];
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else if constexpr (WT == WT_BF16) {
        const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W.w) + off);
        const uint32_t v[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[2 * i] = __uint_as_float(v[i] << 16);
            w[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
        }
    } else {
        const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const int8_t*>(W.w) + off);
        const float s = W.scale[static_cast<size_t>(n) * (K / 32) + (k0 >> 5)];
        const uint32_t v[2] = {u.x, u.y};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int8_t q = static_cast<int8_t>((v[i >> 2] >> (8 * (i & 3))) & 0xFF);
            w[i] = static_cast<float>(q) * s;
        }
    }
}

// Packed argmax key: larger logit wins, then lower index.  -0 is folded into
// +0 so that equal logits always tie.
__device__ __forceinline__ unsigned long long argmax_key(float v, int n) {
    uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (static_cast<unsigned long long>(u) << 32) |
           static_cast<unsigned long long>(0xFFFFFFFFu - static_cast<uint32_t>(n));
}

__device__ __forceinline__ int argmax_index(unsigned long long key) {
    return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key & 0xFFFFFFFFull));
}

// Block-cooperative RMSNorm of one row into LDS: dst = g * (x / rms(x)).
__device__ __forceinline__ void rms_row_to_lds(const float* x, const float* g, int K, float eps,
                                               float* dst) {
    float ss = 0.f;
    for (int k = threadIdx.x; k < K; k += kThreads) {
        const float v = ld_act(x + k);
        dst[k] = v;
        ss += v * v;
    }
    ss = block_sum(ss);
    const float rinv = 1.0f / sqrtf(ss / static_cast<float>(K) + eps);
    for (int k = threadIdx.x; k < K; k += kThreads) dst[k] = g[k] * (dst[k] * rinv);
}

__device__ __forceinline__ void copy_row_to_lds(const float* x, int K, float* dst) {
    for (int k = threadIdx.x; k < K; k += kThreads) dst[k] = ld_act(x + k);
}

// ---------------------------------------------------------------------------
// generic "rows x matrix" phase: out[r][n] = sum_k W[n][k] * in[r][k]
//   rows are staged in LDS (fp32) a few at a time by the prologue `pro`,
//   output columns are spread over every wave of the grid, each wave runs a
//   lane-strided dot product and a fixed butterfly reduction.
//   DUAL computes two matrices over the same input (gate and up).
// ---------------------------------------------------------------------------

template <int WT, bool DUAL, class Pro, class Epi>
__device__ void linear_phase(const Mat& W, const Mat& W2, int N, int K, int M, Pro pro, Epi epi,
                             float* lds, int wg, int nwg) {
    constexpr int RB = 4;   // output rows per wave pass
    constexpr int KC = 2;   // 512-wide k chunks whose loads are in flight together
    const int lane = threadIdx.x & 63;
    const int gw = wg * kWaves + (threadIdx.x >> 6);
    const int nw = nwg * kWaves;
    int R = kLdsFloats / K;
    if (R > kMaxRowsPerChunk) R = kMaxRowsPerChunk;
    for (int r0 = 0; r0 < M; r0 += R) {
        const int rc = (M - r0 < R) ? (M - r0) : R;
        __syncthreads();
        for (int i = 0; i < rc; ++i) pro(r0 + i, lds + i * K);
        __syncthreads();
        for (int nb = gw * RB; nb < N; nb += nw * RB) {
            float acc[kMaxRowsPerChunk][RB] = {};
            float acc2[kMaxRowsPerChunk][RB] = {};
            for (int kb = 0; kb < K; kb += 512 * KC) {
                float w[RB][KC][8], w2[RB][KC][8];
                // issue every load of this block before the arithmetic
#pragma unroll
                for (int q = 0; q < RB; ++q) {
#pragma unroll
                    for (int c = 0; c < KC; ++c) {
                        const int n = nb + q, k0 = kb + c * 512 + lane * 8;
                        if (n < N && k0 < K) {
                            load_w8<WT>(W, K, n, k0, w[q][c]);
                            if constexpr (DUAL) load_w8<WT>(W2, K, n, k0, w2[q][c]);
                        } else {
#pragma unroll
                            for (int j = 0; j < 8; ++j) { w[q][c][j] = 0.f; w2[q][c][j] = 0.f; }
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < kMaxRowsPerChunk; ++i) {
                    if (i < rc) {
#pragma unroll
                        for (int c = 0; c < KC; ++c) {
                            const int k0 = kb + c * 512 + lane * 8;
                            if (k0 < K) {
                                const float* a = lds + i * K + k0;
                                const float4 a0 = *reinterpret_cast<const float4*>(a);
                                const float4 a1 = *reinterpret_cast<const float4*>(a + 4);
                                const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
                                for (int q = 0; q < RB; ++q) {
                                    float s = acc[i][q], s2 = acc2[i][q];
#pragma unroll
                                    for (int j = 0; j < 8; ++j) {
                                        s = fmaf(w[q][c][j], av[j], s);
                                        if constexpr (DUAL) s2 = fmaf(w2[q][c][j], av[j], s2);
                                    }
                                    acc[i][q] = s;
                                    acc2[i][q] = s2;
                                }
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < kMaxRowsPerChunk; ++i) {
                if (i < rc) {
#pragma unroll
                    for (int q = 0; q < RB; ++q) {
                        acc[i][q] = wave_sum(acc[i][q]);
                        if constexpr (DUAL) acc2[i][q] = wave_sum(acc2[i][q]);
                    }
                }
            }
            if (lane == 0) {
                for (int i = 0; i < rc; ++i)
                    for (int q = 0; q < RB; ++q)
                        if (nb + q < N) epi(r0 + i, nb + q, acc[i][q], acc2[i][q]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// row bookkeeping: step s (1..15) runs M rows; step 1 is the two-position
// prefill (rows [0,B) = position 0, rows [B,2B) = position 1), later steps
// run one row per request at position s.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int step_rows(int s, int B) { return s == 1 ? 2 * B : B; }
__device__ __forceinline__ int row_pos(int s, int B, int r) { return s == 1 ? (r >= B ? 1 : 0) : s; }
__device__ __forceinline__ int row_req(int s, int B, int r) { return s == 1 ? (r >= B ? r - B : r) : r; }

// ---------------------------------------------------------------------------
// phases
// ---------------------------------------------------------------------------

// Frame start: x[pos 0] = W_p . H + b_p; x[pos 1] = P_0[q0]; embsum = E_0[q0].
template <int WT>
__device__ void phase_init(const Model& m, const RunArgs& a, float* lds, int wg, int nwg) {
    const int B = a.B;
    __shared__ int tok_s;
    for (int b = wg; b < B; b += nwg) {
        __syncthreads();
        if (threadIdx.x == 0) {
            int q = a.q0[b];
            if (q < 0 || q >= m.V) {
                atomicOr(m.err, kErrBadQ0);
                q = 0;
            }
            tok_s = q;
            __hip_atomic_store(m.amax + b, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        const int q = tok_s;
        const float* prow = m.ptab + static_cast<size_t>(q) * m.dP;
        float* xr = m.x + static_cast<size_t>(B + b) * m.dP;
        for (int k = threadIdx.x; k < m.dP; k += kThreads) st_act(xr + k, prow[k]);
        float* es = a.embsum + static_cast<size_t>(b) * m.dT;
        for (int k = threadIdx.x; k < m.dT; k += kThreads) es[k] = emb_elem(m, 0, q, k);
    }
    const Mat none{nullptr, nullptr};
    linear_phase<WT, false>(
        m.proj, none, m.dP, m.dT, B,
        [&](int r, float* dst) {
            const float* h = a.H + static_cast<size_t>(r) * m.dT;
            for (int k = threadIdx.x; k < m.dT; k += kThreads) dst[k] = h[k];
        },
        [&](int r, int n, float v, float) { st_act(m.x + static_cast<size_t>(r) * m.dP + n, v + m.proj_b[n]); },
        lds, wg, nwg);
}

// q/k/v projection of every row of the step, after the attention RMSNorm.
template <int WT>
__device__ void phase_qkv(const Model& m, const RunArgs& a, int s, int l, float* lds, int wg, int nwg) {
    const LayerDev& L = m.layers[l];
    const Mat none{nullptr, nullptr};
    linear_phase<WT, false>(
        L.qkv, none, m.nqkv, m.dP, step_rows(s, a.B),
        [&](int r, float* dst) {
            rms_row_to_lds(m.x + static_cast<size_t>(r) * m.dP, L.attn_norm, m.dP, m.eps, dst);
        },
        [&](int r, int n, float v, float) { st_act(m.qkv + static_cast<size_t>(r) * m.nqkv + n, v); },
        lds, wg, nwg);
}

// Per-head RMSNorm then rotate-half RoPE of one head vector, by one wave.
// Lane `lane` holds elements d = lane + 64*j, j < hd/64 (hd in {64,128,256}).
__device__ __forceinline__ void norm_rope_wave(const float* src, const float* gain, int hd, float eps,
                                               int pos, const float* rcos, const float* rsin,
                                               float out[4]) {
    const int lane = threadIdx.x & 63;
    const int J = hd >> 6;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    float ss = 0.f;
    for (int j = 0; j < J; ++j) {
        v[j] = ld_act(src + lane + 64 * j);
        ss += v[j] * v[j];
    }
    ss = wave_sum(ss);
    const float rinv = 1.0f / sqrtf(ss / static_cast<float>(hd) + eps);
    for (int j = 0; j < J; ++j) v[j] = gain[lane + 64 * j] * (v[j] * rinv);
    const int half = hd >> 1;
    const float* cp = rcos + static_cast<size_t>(pos) * half;
    const float* sp = rsin + static_cast<size_t>(pos) * half;
    if (hd == 64) {
        const float partner = __shfl_xor(v[0], 32, 64);
        const int i = lane & 31;
        const float c = cp[i], sn = sp[i];
        out[0] = (lane < 32) ? (v[0] * c - partner * sn) : (v[0] * c + partner * sn);
    } else {
        const int H2 = J >> 1;  // registers in each half
        for (int j = 0; j < H2; ++j) {
            const int i = lane + 64 * j;
            const float c = cp[i], sn = sp[i];
            const float x1 = v[j], x2 = v[j + H2];
            out[j] = x1 * c - x2 * sn;
            out[j + H2] = x2 * c + x1 * sn;
        }
    }
}

// Short-context GQA attention.  Work unit = (request, kv head); the unit
// handles every position of the step in order, so the prefill's position 1
// sees position 0's key and value.  The <= 16 cached keys/values of the
// unit's kv head are staged in LDS.
__device__ void phase_attn(const Model& m, const RunArgs& a, int s, int l, float* lds, int wg, int nwg) {
    const int B = a.B, hd = m.hd, nkv = m.nkv, grp = m.nq / m.nkv;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int J = hd >> 6;
    const LayerDev& L = m.layers[l];
    float* Ks = lds;                  // [16][hd]
    float* Vs = lds + kPositions * hd;
    const int npos = (s == 1) ? 2 : 1;
    const int p_first = (s == 1) ? 0 : s;
    for (int u = wg; u < B * nkv; u += nwg) {
        const int b = u / nkv, g = u % nkv;
        const size_t kvb = ((static_cast<size_t>(l) * m.max_batch + b) * kPositions) * nkv * hd;
        __syncthreads();
        for (int idx = threadIdx.x; idx < p_first * hd; idx += kThreads) {
            const int t = idx / hd, d = idx - t * hd;
            const size_t off = kvb + (static_cast<size_t>(t) * nkv + g) * hd + d;
            Ks[idx] = ld_act(m.kc + off);
            Vs[idx] = ld_act(m.vc + off);
        }
        for (int pi = 0; pi < npos; ++pi) {
            const int p = p_first + pi;
            const int r = (s == 1) ? pi * B + b : b;
            const float* row = m.qkv + static_cast<size_t>(r) * m.nqkv;
            __syncthreads();
            if (wave == 0) {
                float kr[4];
                norm_rope_wave(row + (m.nq + g) * hd, L.k_norm, hd, m.eps, p, m.rope_cos, m.rope_sin, kr);
                for (int j = 0; j < J; ++j) Ks[p * hd + lane + 64 * j] = kr[j];
            } else if (wave == 1) {
                const float* vr = row + (m.nq + nkv + g) * hd;
                for (int j = 0; j < J; ++j) Vs[p * hd + lane + 64 * j] = ld_act(vr + lane + 64 * j);
            }
            __syncthreads();
            for (int d = threadIdx.x; d < hd; d += kThreads) {
                const size_t off = kvb + (static_cast<size_t>(p) * nkv + g) * hd + d;
                st_act(m.kc + off, Ks[p * hd + d]);
                st_act(m.vc + off, Vs[p * hd + d]);
            }
            for (int i = wave; i < grp; i += kWaves) {
                const int h = g * grp + i;
                float q[4];
                norm_rope_wave(row + h * hd, L.q_norm, hd, m.eps, p, m.rope_cos, m.rope_sin, q);
                float sc[kPositions];
                float mx = -INFINITY;
#pragma unroll
                for (int t = 0; t < kPositions; ++t) {
                    if (t <= p) {
                        float d = 0.f;
                        for (int j = 0; j < J; ++j) d = fmaf(q[j], Ks[t * hd + lane + 64 * j], d);
                        d = wave_sum(d) * m.attn_scale;
                        sc[t] = d;
                        mx = fmaxf(mx, d);
                    }
                }
                float den = 0.f;
#pragma unroll
                for (int t = 0; t < kPositions; ++t) {
                    if (t <= p) {
                        sc[t] = expf(sc[t] - mx);
                        den += sc[t];
                    }
                }
                float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < kPositions; ++t) {
                    if (t <= p) {
                        const float pt = sc[t] / den;
                        for (int j = 0; j < J; ++j) o[j] = fmaf(pt, Vs[t * hd + lane + 64 * j], o[j]);
                    }
                }
                float* orow = m.ao + static_cast<size_t>(r) * (m.nq * hd) + h * hd;
                for (int j = 0; j < J; ++j) st_act(orow + lane + 64 * j, o[j]);
            }
        }
    }
}

// x += W_o . attention_output
template <int WT>
__device__ void phase_oproj(const Model& m, const RunArgs& a, int s, int l, float* lds, int wg, int nwg) {
    const LayerDev& L = m.layers[l];
    const Mat none{nullptr, nullptr};
    const int K = m.nq * m.hd;
    linear_phase<WT, false>(
        L.o, none, m.dP, K, step_rows(s, a.B),
        [&](int r, float* dst) { copy_row_to_lds(m.ao + static_cast<size_t>(r) * K, K, dst); },
        [&](int r, int n, float v, float) {
            float* xp = m.x + static_cast<size_t>(r) * m.dP + n;
            st_act(xp, ld_act(xp) + v);
        },
        lds, wg, nwg);
}

// h = silu(W_g . m) * (W_u . m), m = RMSNorm(x; ffn_norm)
template <int WT>
__device__ void phase_up(const Model& m, const RunArgs& a, int s, int l, float* lds, int wg, int nwg) {
    const LayerDev& L = m.layers[l];
    linear_phase<WT, true>(
        L.gate, L.up, m.F, m.dP, step_rows(s, a.B),
        [&](int r, float* dst) {
            rms_row_to_lds(m.x + static_cast<size_t>(r) * m.dP, L.ffn_norm, m.dP, m.eps, dst);
        },
        [&](int r, int n, float gv, float uv) {
            st_act(m.hb + static_cast<size_t>(r) * m.F + n, (gv / (1.0f + expf(-gv))) * uv);
        },
        lds, wg, nwg);
}

// x += W_d . h  (and the optional per-layer tap of the residual stream)
template <int WT>
__device__ void phase_down(const Model& m, const RunArgs& a, int s, int l, float* lds, int wg, int nwg) {
    const LayerDev& L = m.layers[l];
    const Mat none{nullptr, nullptr};
    const int B = a.B;
    linear_phase<WT, false>(
        L.down, none, m.dP, m.F, step_rows(s, B),
        [&](int r, float* dst) { copy_row_to_lds(m.hb + static_cast<size_t>(r) * m.F, m.F, dst); },
        [&](int r, int n, float v, float) {
            float* xp = m.x + static_cast<size_t>(r) * m.dP + n;
            const float nv = ld_act(xp) + v;
            st_act(xp, nv);
            if (a.taps) {
                const int pos = row_pos(s, B, r), b = row_req(s, B, r);
                a.taps[((static_cast<size_t>(pos) * m.L + l) * B + b) * m.dP + n] = nv;
            }
        },
        lds, wg, nwg);
}

// logits = lm_head[s-1] . RMSNorm(x; out_norm) for the rows at position s,
// folded into one packed argmax key per request.
template <int WT>
__device__ void phase_lm(const Model& m, const RunArgs& a, int s, float* lds, int wg, int nwg) {
    const int B = a.B;
    const int row0 = (s == 1) ? B : 0;
    const Mat none{nullptr, nullptr};
    linear_phase<WT, false>(
        m.lm[s - 1], none, m.V, m.dP, B,
        [&](int i, float* dst) {
            rms_row_to_lds(m.x + static_cast<size_t>(row0 + i) * m.dP, m.out_norm, m.dP, m.eps, dst);
        },
        [&](int b, int n, float v, float) {
            if (a.logits_out) a.logits_out[(static_cast<size_t>(b) * kSteps + (s - 1)) * m.V + n] = v;
            atomicMax(m.amax + b, argmax_key(v, n));
        },
        lds, wg, nwg);
}

// Decode step s's token; feed it (or the forced token) back: embsum += E_s[t]
// and, before the last step, the next position's input row P_s[t].
__device__ void phase_next(const Model& m, const RunArgs& a, int s, int wg, int nwg) {
    const int B = a.B;
    __shared__ int fed_s;
    for (int b = wg; b < B; b += nwg) {
        __syncthreads();
        if (threadIdx.x == 0) {
            const unsigned long long key =
                __hip_atomic_load(m.amax + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(m.amax + b, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int tok = argmax_index(key);
            a.tok_out[b * kSteps + (s - 1)] = tok;
            int fed = a.force ? a.force[b * kSteps + (s - 1)] : tok;
            if (fed < 0 || fed >= m.V) {
                atomicOr(m.err, a.force ? kErrBadForced : kErrBadQ0);
                fed = 0;
            }
            fed_s = fed;
        }
        __syncthreads();
        const int t = fed_s;
        float* es = a.embsum + static_cast<size_t>(b) * m.dT;
        for (int k = threadIdx.x; k < m.dT; k += kThreads) es[k] += emb_elem(m, s, t, k);
        if (s < kSteps) {
            const float* prow = m.ptab + (static_cast<size_t>(s) * m.V + t) * m.dP;
            float* xr = m.x + static_cast<size_t>(b) * m.dP;
            for (int k = threadIdx.x; k < m.dP; k += kThreads) st_act(xr + k, prow[k]);
        }
    }
}

enum PhaseId : int { PH_INIT = 0, PH_QKV, PH_ATTN, PH_OPROJ, PH_UP, PH_DOWN, PH_LM, PH_NEXT };

template <int WT>
__device__ __forceinline__ void run_phase(const Model& m, const RunArgs& a, int ph, int s, int l,
                                          float* lds, int wg, int nwg) {
    switch (ph) {
        case PH_INIT: phase_init<WT>(m, a, lds, wg, nwg); break;
        case PH_QKV: phase_qkv<WT>(m, a, s, l, lds, wg, nwg); break;
        case PH_ATTN: phase_attn(m, a, s, l, lds, wg, nwg); break;
        case PH_OPROJ: phase_oproj<WT>(m, a, s, l, lds, wg, nwg); break;
        case PH_UP: phase_up<WT>(m, a, s, l, lds, wg, nwg); break;
        case PH_DOWN: phase_down<WT>(m, a, s, l, lds, wg, nwg); break;
        case PH_LM: phase_lm<WT>(m, a, s, lds, wg, nwg); break;
        case PH_NEXT: phase_next(m, a, s, wg, nwg); break;
        default: break;
    }
}

// Phase order of one frame; the host walks the same list for the
// one-kernel-per-phase driver and the persistent kernel places a grid
// barrier between consecutive entries.
__host__ __device__ constexpr int phases_per_frame(int L) { return 1 + kSteps * (5 * L + 2); }

}  // namespace qp

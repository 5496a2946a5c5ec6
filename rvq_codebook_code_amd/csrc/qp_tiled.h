// Batched frame driver (any B; bf16 or Q8_0 weights): one kernel per phase,
// every projection on the matrix cores.
//
// The predictor step is the same as in the other drivers (Qwen3 decoder
// block: RMSNorm, fused q/k/v projection, per-head q/k RMSNorm, rotate-half
// RoPE, GQA attention over <= 16 cached positions, output projection,
// SwiGLU MLP, final RMSNorm, lm_head[k-1] argmax; Qwen3-TTS code predictor as
// described by the rightkit-qts exporter README, "Loader contract").  What
// changes with the batch is the shape of the work: every projection becomes
// a [rows x K] . [K x N] product, which runs here on
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
//
//  * Weights are repacked at create time into MFMA fragment order: for each
//    block of 16 output rows and 32 inputs, the 64 lanes' 8-element pieces
//    are stored contiguously in lane order (1 KiB per fragment for bf16,
//    512 B of int8 codes plus 16 fp32 block scales for Q8_0).  A wave's
//    weight load is one contiguous 1 KiB (or 512 B) read.
//  * Activations enter as bf16.  RMSNorm is applied as
//      W . (g * x / rms(x)) = (W . bf16(g * x)) / rms(x)
//    Whoever writes a residual-stream row also writes bf16(g * x) with the
//    gain of the row's next reader (ffn_norm after the output projection,
//    the next layer's attn_norm or out_norm after the MLP) and the row's sums
//    of x^2 over 32-column tiles; the reader's epilogue adds those sums up
//    (in tile order) for the row scale.  The operand is then a plain bf16
//    load, and the gain rides on it while the row scale rides on the output.
//  * Q8_0 codes are integers in [-128, 127], exact in bf16; one MFMA covers
//    exactly one 32-wide quantisation block, whose f16 scale (stored as fp32)
//    multiplies the block's partial sum before accumulation.  The weights
//    therefore enter the product exactly.
//  * A workgroup (4 waves) owns a tile of 16*RT rows x 32 output columns
//    (2 fragments wide; for SwiGLU the gate and up fragments of the same 16
//    columns).  The 4 waves split K and their partial tiles are summed through
//    LDS in wave order.  Small-N products also split K across KS workgroups:
//    every workgroup writes its partial tile, and the last to arrive (a
//    counter per tile) sums the KS partials in order and runs the epilogue,
//    so results do not depend on timing.
#pragma once

#include "qp_common.h"
#include "qp_phases.h"

#include <type_traits>

namespace qp {
namespace tiled {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreadsT = 256;
constexpr int kCT = 2;        // output fragments (16 columns each) per workgroup
constexpr int kMaxKS = 4;     // largest split of K across workgroups

// A weight matrix [N][K] in fragment order (see the file comment).
struct FMat {
    const void* w;        // bf16: uint16 [N/16][K/32][64][8]; Q8_0: int8 [N/16][K/32][64][8]
    const float* scale;   // Q8_0: [N/16][K/32][16]; bf16: null
};

enum Src : int { SRC_F32 = 0, SRC_BF16 = 1, SRC_BF16_NORM = 2 };
enum Epi : int { EPI_BIAS = 0, EPI_SCALE = 1, EPI_RESID = 2, EPI_SWIGLU = 3, EPI_ARGMAX = 4 };

struct GemmArgs {
    const void* a;          // A operand rows [M][lda]: fp32 (SRC_F32) or bf16
    int lda;
    int M, N, K, KS;        // N = output columns (for SwiGLU: F)
    FMat w0, w1;            // w1: the up matrix of SwiGLU
    // RMSNorm of the A rows (SRC_BF16_NORM): the rows are already g * x in
    // bf16; rms(x) comes from nss partial sums of squares per row
    const float* ss_in;     // [M][nss]
    int nss;
    float eps;
    // epilogue outputs
    float* out;             // fp32 rows [M][ldo] (BIAS, SCALE, RESID)
    int ldo;
    uint16_t* outb;         // bf16 rows [M][N] (SWIGLU)
    const float* bias;      // [N] (BIAS)
    // BIAS / RESID also publish the next consumer's operand and row sums:
    // xg = bf16(g_next * x) [M][ldo], ss_out[m][tile] = sum over the tile's 32 columns of x^2
    uint16_t* xg;
    const float* g_next;
    float* ss_out;
    unsigned long long* keys;  // [M][gridDim.x] per-tile argmax keys (ARGMAX)
    float* logits;          // row m's logits at logits + m * logit_ld (ARGMAX, optional)
    size_t logit_ld;
    float* taps;            // residual taps [16][L][B][dP] (RESID of the down projection, optional)
    int tap_s, tap_l, tap_L, tap_B;
    float* part;            // split-K partial tiles
    uint32_t part_bytes;
    unsigned* ctr;          // split-K arrival counters, one per tile, left at 0
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};  // round to nearest even
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// int8 code -> bf16 bits (exact: |q| <= 128 needs 8 significant bits)
__device__ __forceinline__ uint32_t q8pair(uint32_t w, int sh) {
    const float lo = static_cast<float>(static_cast<int>(w << (24 - sh)) >> 24);
    const float hi = static_cast<float>(static_cast<int>(w << (16 - sh)) >> 24);
    return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), m, 64);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), m, 64);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// sum over the 16 lanes of a row group (lanes with equal lane / 16), fixed order
__device__ __forceinline__ float sum16(float v) {
    v += __shfl_xor(v, 1, 64);
    v += __shfl_xor(v, 2, 64);
    v += __shfl_xor(v, 4, 64);
    v += __shfl_xor(v, 8, 64);
    return v;
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kDevScope = 16;   // buffer cache policy: device-coherent (sc1)

// ---------------------------------------------------------------------------
// [M x K] . [K x N] with a fused prologue (SRC) and epilogue (EPI).
// grid = (N / 32 (SwiGLU: N / 16), ceil(M / (16 RT)), KS), 256 threads.
// ---------------------------------------------------------------------------
template <int WT, int RT, int SRC, int EPI>
__global__ __launch_bounds__(kThreadsT) void k_gemm(GemmArgs g) {
    __shared__ f32x4_t red[4][RT][kCT][64];
    __shared__ int last_s;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int bx = blockIdx.x, by = blockIdx.y, kz = blockIdx.z;
    const int m0 = by * 16 * RT;
    const int KB = g.K >> 5;
    const int kbw = KB / (4 * g.KS);             // k-blocks per wave (even)
    const int kb0 = (kz * 4 + wave) * kbw;

    // output fragments of this workgroup
    int nb[kCT];
    const uint8_t* wp[kCT];
    const float* sp[kCT];
#pragma unroll
    for (int c = 0; c < kCT; ++c) {
        const FMat& W = (EPI == EPI_SWIGLU && c == 1) ? g.w1 : g.w0;
        nb[c] = (EPI == EPI_SWIGLU) ? bx : bx * kCT + c;
        const size_t frag0 = static_cast<size_t>(nb[c]) * KB;
        wp[c] = static_cast<const uint8_t*>(W.w) + frag0 * 64 * (WT == WT_Q8 ? 8 : 16);
        sp[c] = (WT == WT_Q8) ? W.scale + frag0 * 16 : nullptr;
    }

    // this lane's A row (per row tile) and k offset inside a block
    const int arow = lane & 15, akoff = (lane >> 4) * 8;
    bool rok[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) rok[rt] = m0 + 16 * rt + arow < g.M;

    // RMSNorm row scales of the row tiles this wave finishes, fetched before
    // the products: lane l sums a quarter of row (l % 16)'s tile sums, the
    // quarters are then combined across the lane groups (fixed order)
    float rss[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        rss[rt] = 0.f;
        if constexpr (SRC == SRC_BF16_NORM) {
            if ((rt & 3) == wave && rok[rt]) {
                const int q = g.nss >> 2;
                const float* sr = g.ss_in + static_cast<size_t>(m0 + 16 * rt + arow) * g.nss + (lane >> 4) * q;
                for (int t = 0; t < q; t += 2) {   // q = nss / 4 is even (dP % 256 == 0)
                    const float2 v = *reinterpret_cast<const float2*>(sr + t);
                    rss[rt] += v.x + v.y;
                }
            }
        }
    }

    f32x4_t acc[RT][kCT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int c = 0; c < kCT; ++c) acc[rt][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // one batch of UU k-blocks: every load first, then the products
    auto batch = [&](int kb, auto uu) {
        constexpr int UU = decltype(uu)::value;
        uint4 av[UU][RT];
        uint4 wv[UU][kCT];
        uint2 wq[UU][kCT];
        float ws[UU][kCT];
#pragma unroll
        for (int u = 0; u < UU; ++u) {
            const int k = (kb + u) * 32 + akoff;
#pragma unroll
            for (int c = 0; c < kCT; ++c) {
                if constexpr (WT == WT_Q8) {
                    wq[u][c] = *reinterpret_cast<const uint2*>(wp[c] + (static_cast<size_t>(kb + u) * 64 + lane) * 8);
                    ws[u][c] = sp[c][(kb + u) * 16 + (lane & 15)];
                } else {
                    wv[u][c] = *reinterpret_cast<const uint4*>(wp[c] + (static_cast<size_t>(kb + u) * 64 + lane) * 16);
                }
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const size_t row = static_cast<size_t>(m0 + 16 * rt + arow);
                if constexpr (SRC == SRC_F32) {
                    const float* src = static_cast<const float*>(g.a) + row * g.lda + k;
                    float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
                    if (rok[rt]) {
                        x0 = *reinterpret_cast<const float4*>(src);
                        x1 = *reinterpret_cast<const float4*>(src + 4);
                    }
                    av[u][rt] = make_uint4(pack_bf16x2(x0.x, x0.y), pack_bf16x2(x0.z, x0.w),
                                           pack_bf16x2(x1.x, x1.y), pack_bf16x2(x1.z, x1.w));
                } else {
                    const uint16_t* src = static_cast<const uint16_t*>(g.a) + row * g.lda + k;
                    av[u][rt] = rok[rt] ? *reinterpret_cast<const uint4*>(src) : make_uint4(0, 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < UU; ++u) {
#pragma unroll
            for (int c = 0; c < kCT; ++c) {
                uint4 w8;
                if constexpr (WT == WT_Q8) {
                    w8 = make_uint4(q8pair(wq[u][c].x, 0), q8pair(wq[u][c].x, 16), q8pair(wq[u][c].y, 0),
                                    q8pair(wq[u][c].y, 16));
                } else {
                    w8 = wv[u][c];
                }
                const bf16x8_t wb = __builtin_bit_cast(bf16x8_t, w8);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const bf16x8_t ab = __builtin_bit_cast(bf16x8_t, av[u][rt]);
                    if constexpr (WT == WT_Q8) {
                        const f32x4_t p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, wb, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                        const float sc = ws[u][c];
                        acc[rt][c] = f32x4_t{fmaf(sc, p[0], acc[rt][c][0]), fmaf(sc, p[1], acc[rt][c][1]),
                                             fmaf(sc, p[2], acc[rt][c][2]), fmaf(sc, p[3], acc[rt][c][3])};
                    } else {
                        acc[rt][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, wb, acc[rt][c], 0, 0, 0);
                    }
                }
            }
        }
    };
    int kb = kb0;
    const int kb1 = kb0 + kbw;
    if constexpr (RT == 1) {
        for (; kb + 8 <= kb1; kb += 8) batch(kb, std::integral_constant<int, 8>{});
    }
    for (; kb + 4 <= kb1; kb += 4) batch(kb, std::integral_constant<int, 4>{});
    for (; kb < kb1; kb += 2) batch(kb, std::integral_constant<int, 2>{});

    // ---- reduce the four waves' K ranges, in wave order ----
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int c = 0; c < kCT; ++c) red[wave][rt][c][lane] = acc[rt][c];
    __syncthreads();

    // wave w finishes row tiles w, w+4, ...
    f32x4_t tot[RT][kCT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        if ((rt & 3) != wave) continue;
#pragma unroll
        for (int c = 0; c < kCT; ++c) {
            f32x4_t t = red[0][rt][c][lane];
            t += red[1][rt][c][lane];
            t += red[2][rt][c][lane];
            t += red[3][rt][c][lane];
            tot[rt][c] = t;
        }
    }

    if (g.KS > 1) {
        // split K across workgroups: publish this partial tile with
        // device-coherent stores; the last arriver sums all of them in kz order
        const size_t tile = static_cast<size_t>(by) * gridDim.x + bx;
        const size_t tiles = static_cast<size_t>(gridDim.x) * gridDim.y;
        const auto pr = __builtin_amdgcn_make_buffer_rsrc(g.part, static_cast<short>(0), static_cast<int>(g.part_bytes),
                                                          0x00020000);
        auto poff = [&](int z, int rt, int c) {
            return static_cast<uint32_t>(((((static_cast<size_t>(z) * tiles + tile) * RT + rt) * kCT + c) * 64 + lane) * 16);
        };
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if ((rt & 3) != wave) continue;
#pragma unroll
            for (int c = 0; c < kCT; ++c)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, tot[rt][c]), pr, poff(kz, rt, c), 0u,
                                                       kDevScope);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0) {
            const unsigned old = __hip_atomic_fetch_add(g.ctr + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int last = old == static_cast<unsigned>(g.KS - 1);
            if (last) __hip_atomic_store(g.ctr + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last_s = last;
        }
        __syncthreads();
        if (!last_s) return;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if ((rt & 3) != wave) continue;
#pragma unroll
            for (int c = 0; c < kCT; ++c) {
                f32x4_t t = f32x4_t{0.f, 0.f, 0.f, 0.f};
                for (int z = 0; z < g.KS; ++z)
                    t += __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(pr, poff(z, rt, c), 0u, kDevScope));
                tot[rt][c] = t;
            }
        }
    }

    // ---- epilogue: lane holds rows 4*(lane/16)+i, column lane%16 of each fragment ----
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        if ((rt & 3) != wave) continue;
        float rinv[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (SRC == SRC_BF16_NORM) {
            float t = rss[rt];
            t += __shfl_xor(t, 16, 64);
            t += __shfl_xor(t, 32, 64);   // every lane: the sum for row lane % 16
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float sst = __shfl(t, 4 * (lane >> 4) + i, 64);
                rinv[i] = 1.0f / sqrtf(sst / static_cast<float>(g.K) + g.eps);
            }
        }
        if constexpr (EPI == EPI_ARGMAX) {
            uint64_t key[4] = {0, 0, 0, 0};
#pragma unroll
            for (int c = 0; c < kCT; ++c) {
                const int n = nb[c] * 16 + (lane & 15);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = m0 + 16 * rt + 4 * (lane >> 4) + i;
                    const float v = tot[rt][c][i] * rinv[i];
                    if (g.logits && m < g.M) g.logits[m * g.logit_ld + n] = v;
                    key[i] = umax64(key[i], argmax_key(v, n));
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) key[i] = umax64(key[i], shfl_xor64(key[i], o));
                const int m = m0 + 16 * rt + 4 * (lane >> 4) + i;
                if ((lane & 15) == 0 && m < g.M) g.keys[static_cast<size_t>(m) * gridDim.x + bx] = key[i];
            }
        } else if constexpr (EPI == EPI_SWIGLU) {
            const int n = nb[0] * 16 + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + 16 * rt + 4 * (lane >> 4) + i;
                if (m >= g.M) continue;
                const float gt = tot[rt][0][i] * rinv[i], ut = tot[rt][1][i] * rinv[i];
                g.outb[static_cast<size_t>(m) * g.N + n] = to_bf16((gt / (1.0f + expf(-gt))) * ut);
            }
        } else if constexpr (EPI == EPI_SCALE) {
#pragma unroll
            for (int c = 0; c < kCT; ++c) {
                const int n = nb[c] * 16 + (lane & 15);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = m0 + 16 * rt + 4 * (lane >> 4) + i;
                    if (m < g.M) g.out[static_cast<size_t>(m) * g.ldo + n] = tot[rt][c][i] * rinv[i];
                }
            }
        } else {
            // residual stream rows: x (fp32), xg = bf16(g_next * x), and the
            // sum of x^2 over this workgroup's 32 columns
            float sq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < kCT; ++c) {
                const int n = nb[c] * 16 + (lane & 15);
                const float gn = g.g_next[n];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = m0 + 16 * rt + 4 * (lane >> 4) + i;
                    if (m >= g.M) continue;
                    float* o = g.out + static_cast<size_t>(m) * g.ldo + n;
                    float nv;
                    if constexpr (EPI == EPI_BIAS) {
                        nv = tot[rt][c][i] + g.bias[n];
                    } else {
                        nv = *o + tot[rt][c][i];
                        if (g.taps) {
                            const int B = g.tap_B;
                            const int pos = row_pos(g.tap_s, B, m), b = row_req(g.tap_s, B, m);
                            g.taps[((static_cast<size_t>(pos) * g.tap_L + g.tap_l) * B + b) * g.ldo + n] = nv;
                        }
                    }
                    *o = nv;
                    g.xg[static_cast<size_t>(m) * g.ldo + n] = to_bf16(gn * nv);
                    sq[i] = fmaf(nv, nv, sq[i]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float t = sum16(sq[i]);
                const int m = m0 + 16 * rt + 4 * (lane >> 4) + i;
                if ((lane & 15) == 0 && m < g.M) g.ss_out[static_cast<size_t>(m) * (g.ldo / 32) + bx] = t;
            }
        }
    }
}

// One residual-stream row written whole (position inputs gathered from P_j):
// x, xg = bf16(g * x) and the per-32-column sums of x^2.  Thread j owns
// columns j, j + 256, ...; every load is issued before any arithmetic, and a
// tile's sum is reduced over the 32 threads that own it.
constexpr int kMaxRowPerThread = 16;   // dP <= 4096
__device__ __forceinline__ void put_row(const Model& m, const float* src, int row, const float* gain, uint16_t* xg,
                                        float* ss) {
    const int j = threadIdx.x;
    const int n_per = m.dP / kThreadsT;   // dP % 256 == 0
    float v[kMaxRowPerThread], gv[kMaxRowPerThread];
#pragma unroll
    for (int i = 0; i < kMaxRowPerThread; ++i) {
        if (i < n_per) {
            v[i] = src[j + kThreadsT * i];
            gv[i] = gain[j + kThreadsT * i];
        }
    }
    float* xr = m.x + static_cast<size_t>(row) * m.dP;
    uint16_t* gr = xg + static_cast<size_t>(row) * m.dP;
    float* sr = ss + static_cast<size_t>(row) * (m.dP / 32);
#pragma unroll
    for (int i = 0; i < kMaxRowPerThread; ++i) {
        if (i < n_per) {
            const int n = j + kThreadsT * i;
            xr[n] = v[i];
            gr[n] = to_bf16(gv[i] * v[i]);
            float q = v[i] * v[i];
            q += __shfl_xor(q, 1, 64);
            q += __shfl_xor(q, 2, 64);
            q += __shfl_xor(q, 4, 64);
            q += __shfl_xor(q, 8, 64);
            q += __shfl_xor(q, 16, 64);
            if ((j & 31) == 0) sr[n >> 5] = q;
        }
    }
}

// ---------------------------------------------------------------------------
// Attention of one step: one workgroup per (request, kv head).  Every
// position of the step is handled in order (the prefill's position 1 sees
// position 0).  Keys and values of earlier positions come from the fp32 KV
// cache; the new position's key gets its per-head RMSNorm and RoPE here and
// is appended to the cache.  Scores for all <= 16 keys are formed at once:
// key t on lanes 4t..4t+3, each lane a quarter of the head.
// Output: bf16 rows [M][nq*hd], the operand of the output projection.
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(kThreadsT) void k_attn(Model m, int B, int s, int l, uint16_t* ao) {
    constexpr int J = HD / 64;        // elements per lane in the lane + 64 j layout
    constexpr int SL = HD / 4;        // slice of the head per lane in the score
    __shared__ float Ks[kPositions][HD];
    __shared__ float Vs[kPositions][HD];
    __shared__ float qs[4][HD];
    __shared__ float es[4][kPositions];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nkv = m.nkv, grp = m.nq / m.nkv;
    const int b = blockIdx.x / nkv, g = blockIdx.x % nkv;
    const LayerDev& L = m.layers[l];
    const int npos = (s == 1) ? 2 : 1;
    const int pf = (s == 1) ? 0 : s;
    const size_t kvb = ((static_cast<size_t>(l) * m.max_batch + b) * kPositions) * nkv * HD;
    for (int idx = threadIdx.x; idx < pf * HD; idx += kThreadsT) {
        const int t = idx / HD, d = idx - t * HD;
        const size_t off = kvb + (static_cast<size_t>(t) * nkv + g) * HD + d;
        Ks[t][d] = m.kc[off];
        Vs[t][d] = m.vc[off];
    }
    for (int pi = 0; pi < npos; ++pi) {
        const int p = pf + pi;
        const int r = (s == 1) ? pi * B + b : b;
        const float* row = m.qkv + static_cast<size_t>(r) * m.nqkv;
        const size_t off = kvb + (static_cast<size_t>(p) * nkv + g) * HD;
        if (wave == 0) {
            float kr[4];
            norm_rope_wave(row + (m.nq + g) * HD, L.k_norm, HD, m.eps, p, m.rope_cos, m.rope_sin, kr);
#pragma unroll
            for (int j = 0; j < J; ++j) {
                Ks[p][lane + 64 * j] = kr[j];
                m.kc[off + lane + 64 * j] = kr[j];
            }
        } else if (wave == 1) {
            const float* vr = row + (m.nq + nkv + g) * HD;
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const float v = vr[lane + 64 * j];
                Vs[p][lane + 64 * j] = v;
                m.vc[off + lane + 64 * j] = v;
            }
        }
        __syncthreads();
        for (int i = wave; i < grp; i += 4) {
            const int h = g * grp + i;
            float q[4];
            norm_rope_wave(row + h * HD, L.q_norm, HD, m.eps, p, m.rope_cos, m.rope_sin, q);
#pragma unroll
            for (int j = 0; j < J; ++j) qs[wave][lane + 64 * j] = q[j];
            const int kt = lane >> 2, k0 = (lane & 3) * SL;
            float sc = 0.f;
            if (kt <= p) {
#pragma unroll
                for (int d = 0; d < SL; d += 4) {
                    const float4 qv = *reinterpret_cast<const float4*>(&qs[wave][k0 + d]);
                    const float4 kv = *reinterpret_cast<const float4*>(&Ks[kt][k0 + d]);
                    sc = fmaf(qv.x, kv.x, sc);
                    sc = fmaf(qv.y, kv.y, sc);
                    sc = fmaf(qv.z, kv.z, sc);
                    sc = fmaf(qv.w, kv.w, sc);
                }
            }
            sc += dpp_or_zero<0xB1, 0xF>(sc);
            sc += dpp_or_zero<0x4E, 0xF>(sc);
            sc = (kt <= p) ? sc * m.attn_scale : -__builtin_huge_valf();
            float mx = sc;
#pragma unroll
            for (int o = 32; o >= 4; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
            const float e = (kt <= p) ? expf(sc - mx) : 0.f;
            const float den = wave_sum((lane & 3) == 0 ? e : 0.f);
            if ((lane & 3) == 0) es[wave][kt] = e;
            float o[J];
#pragma unroll
            for (int j = 0; j < J; ++j) o[j] = 0.f;
#pragma unroll
            for (int t = 0; t < kPositions; ++t) {
                const int tt = t <= p ? t : p;     // weight 0 beyond p
                const float w = es[wave][t];
#pragma unroll
                for (int j = 0; j < J; ++j) o[j] = fmaf(w, Vs[tt][lane + 64 * j], o[j]);
            }
            uint16_t* orow = ao + static_cast<size_t>(r) * (m.nq * HD) + h * HD;
#pragma unroll
            for (int j = 0; j < J; ++j) orow[lane + 64 * j] = to_bf16(o[j] / den);
        }
        __syncthreads();
    }
}

// Frame start, per request: check q0, x[pos 1] = P_0[q0], embsum = E_0[q0].
// (x[pos 0] = W_p . H + b_p is a product of its own.)
__global__ __launch_bounds__(kThreadsT) void k_start(Model m, RunArgs a, const float* gain0, uint16_t* xg, float* ss) {
    __shared__ int tok_s;
    const int B = a.B;
    for (int b = blockIdx.x; b < B; b += gridDim.x) {
        __syncthreads();
        if (threadIdx.x == 0) {
            int q = a.q0[b];
            if (q < 0 || q >= m.V) {
                atomicOr(m.err, kErrBadQ0);
                q = 0;
            }
            tok_s = q;
        }
        __syncthreads();
        const int q = tok_s;
        put_row(m, m.ptab + static_cast<size_t>(q) * m.dP, B + b, gain0, xg, ss);
        float* es = a.embsum + static_cast<size_t>(b) * m.dT;
        for (int k = threadIdx.x; k < m.dT; k += kThreadsT) es[k] = emb_elem(m, 0, q, k);
    }
}

// Step s's token per request from the lm_head tiles' keys; the fed-back
// token (forced or own) adds E_s[t] to embsum and, before the last step,
// sets the next position's input row P_s[t].
__global__ __launch_bounds__(kThreadsT) void k_next(Model m, RunArgs a, int s, const unsigned long long* keys,
                                                    int nkt, const float* gain0, uint16_t* xg, float* ss) {
    __shared__ unsigned long long red[kThreadsT / 64];
    __shared__ int fed_s;
    const int B = a.B;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int b = blockIdx.x; b < B; b += gridDim.x) {
        uint64_t k = 0;
        for (int t = threadIdx.x; t < nkt; t += kThreadsT) k = umax64(k, keys[static_cast<size_t>(b) * nkt + t]);
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) k = umax64(k, shfl_xor64(k, o));
        __syncthreads();
        if (lane == 0) red[wave] = k;
        __syncthreads();
        if (threadIdx.x == 0) {
            uint64_t kk = red[0];
            for (int w = 1; w < kThreadsT / 64; ++w) kk = umax64(kk, red[w]);
            const int tok = argmax_index(kk);
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
        for (int k2 = threadIdx.x; k2 < m.dT; k2 += kThreadsT) es[k2] += emb_elem(m, s, t, k2);
        if (s < kSteps) put_row(m, m.ptab + (static_cast<size_t>(s) * m.V + t) * m.dP, b, gain0, xg, ss);
    }
}

}  // namespace tiled
}  // namespace qp

// Batched frame driver (any B; bf16, Q8_0 or Q4_0 weights): one kernel per phase,
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
//  * Activations enter as bf16.  From kFragMinRows rows per position on they
//    are held in the same fragment order as the weights: a matrix of width K
//    is [rows/16][K/32][64 lanes][8], lane l holding row l % 16, inputs
//    8 (l / 16) .. +7 of the 32-wide block (see frag_index).  Every writer of
//    a product's A operand (the residual and SwiGLU epilogues, attention, the
//    token steps) then stores in that order, and a wave's load of a 16 x 32
//    operand block touches 8 whole cache lines instead of 16 half-used ones
//    (the batched products are bound by each CU's vector-memory path).  With
//    fewer rows, row-major rows touch fewer lines (one per row), so they stay
//    row-major.  Buffers hold their rows rounded up to 16.
//  * RMSNorm is applied as
//      W . (g * x / rms(x)) = (W . bf16(g * x)) / rms(x)
//    Whoever writes a residual-stream row also writes bf16(g * x) with the
//    gain of the row's next reader (ffn_norm after the output projection,
//    the next layer's attn_norm or out_norm after the MLP) and the row's sums
//    of x^2 over 32-column tiles; the reader's epilogue adds those sums up
//    (in tile order) for the row scale.  The operand is then a plain bf16
//    load, and the gain rides on it while the row scale rides on the output.
//  * Q8_0 codes are integers in [-128, 127] and Q4_0 codes minus 8 are in
//    [-8, 7], both exact in bf16; one MFMA covers exactly one 32-wide
//    quantisation block, whose f16 scale (stored as fp32) multiplies the
//    block's partial sum before accumulation.  The weights therefore enter
//    the product exactly.  Q4_0 fragments hold a lane's 8 codes in one
//    32-bit word (256 B per fragment).
//  * A workgroup of NW waves owns a tile of 16*RT rows x 16*CT output
//    columns (for SwiGLU the gate and up fragments of the same 16 columns).
//    RT = 1 (up to 32 rows, and the residual products) takes CT = 1
//    (SwiGLU: its pair) and, except SwiGLU, NW = 8 up to 16 rows where K
//    holds 16 pairs of 32-wide blocks, else 4; RT = 2 takes CT = 2 and
//    NW = 4.  The NW waves split K and their partial tiles are summed through
//    LDS in wave order.  The sum and the epilogue are shared by four waves,
//    wave i taking component i of every lane's accumulator (one row of each
//    16-row fragment per lane), so they run four wide; the row scales reach
//    them through LDS from the wave that summed the row's squares.  The
//    projection of H (small N) with two row
//    fragments also splits K across KS workgroups:
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
constexpr int kMaxCT = 2;     // output fragments (16 columns each) per workgroup
constexpr int kMaxKS = 4;     // largest split of K across workgroups

// A weight matrix [N][K] in fragment order (see the file comment).
struct FMat {
    const void* w;        // bf16: uint16 [N/16][K/32][64][8]; Q8_0: int8 [N/16][K/32][64][8];
                          // Q4_0: uint32 [N/16][K/32][64], nibble i = code of element i
    const float* scale;   // Q8_0, Q4_0: [N/16][K/32][16]; bf16: null
};

enum Src : int { SRC_F32 = 0, SRC_BF16 = 1, SRC_BF16_NORM = 2 };
enum Epi : int { EPI_BIAS = 0, EPI_SCALE = 1, EPI_RESID = 2, EPI_SWIGLU = 3, EPI_ARGMAX = 4 };

struct GemmArgs {
    const void* a;          // A operand: fp32 rows [M][lda] (SRC_F32), or bf16 of width K (act_index),
                            // logical row m at physical row a_row0 + m
    int lda;
    int a_row0;
    int frag;               // the bf16 activations (A operand, xg, outb) are in fragment order
    int M, N, K, KS;        // N = output columns (for SwiGLU: F)
    FMat w0, w1;            // w1: the up matrix of SwiGLU
    // RMSNorm of the A rows (SRC_BF16_NORM): the rows are already g * x in
    // bf16; rms(x) comes from nss partial sums of squares per row
    const float* ss_in;     // [M][nss], nss = K / 16
    int nss;
    float eps;
    // epilogue outputs
    float* out;             // fp32 rows [M][ldo] (BIAS, SCALE, RESID)
    int ldo;
    uint16_t* outb;         // bf16, width N (act_index layout; SWIGLU)
    const float* bias;      // [N] (BIAS)
    // BIAS / RESID also publish the next consumer's operand and row sums:
    // xg = bf16(g_next * x) (width ldo, act_index layout), ss_out[m][f] = sum over the 16 columns
    // of fragment f of x^2
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
    int tl = -1;            // launch index in the frame (timeline build)
};

// Arguments of the token-step kernels, resolved on the host per launch and
// kept small: a kernel reads them in one batch at its start instead of a
// chain of dependent loads through a large structure.
struct TokArgs {
    int B, s, dT, dP, V, emb_bf16, nkt;
    const void* emb;                  // E_j of this launch's codebook (fp32 or bf16 [V][dT])
    const float* ptab;                // P_j [V][dP] of the next position's input; null at the last step
    const int* q0;                    // [B] (frame start)
    const int* force;                 // [B][15] or null
    int* tok_out;                     // [B][15]
    float* embsum;                    // [B][dT]
    const unsigned long long* keys;   // [B][nkt] lm_head tile keys
    const int* sampled;               // [B] drawn tokens of this step (sampled frames), or null
    float* x;                         // residual rows [2B][dP]
    uint16_t* xg;                     // bf16(gain0 * x), width dP (act_index layout)
    int frag;                         // activations in fragment order
    float* ss;                        // 16-column sums of x^2 [2B][dP/16]
    const float* gain0;               // attn_norm of layer 0 (out_norm without layers)
    unsigned* err;
    // layer 0's q/k/v rows of the next position's table rows [V][nqkv], or
    // null; when set, the fed token's row is copied to qkv [B][nqkv] and the
    // next step runs no layer-0 q/k/v product
    const float* qkv0;
    float* qkv;
    int nqkv;
    int tl = -1;                      // launch index in the frame (timeline build)
};

struct AttnArgs {
    int B, s, nq, nkv, nqkv, max_batch, l;
    float eps, attn_scale;
    const float* qkv;                 // [M][nqkv] step rows
    float* kc;                        // KV cache [L][max_batch][16][nkv][hd]
    float* vc;
    const float* k_norm;              // layer l's per-head gains [hd]
    const float* q_norm;
    const float* rope_cos;            // [16][hd/2]
    const float* rope_sin;
    uint16_t* ao;                     // bf16 output, width nq*hd (act_index layout)
    int frag;                         // activations in fragment order
    // layer 0 from step 2 on, with the layer-0 q/k/v table: the previous
    // step's token decision (tok.s = that step) happens here instead of in
    // k_next, and the head vectors come from tok.qkv0 [V][nqkv]
    int tok_on;
    TokArgs tok;
    int tl = -1;                      // launch index in the frame (timeline build)
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};  // round to nearest even
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// 8 Q4_0 codes (nibble i of w, value code - 8) -> 8 bf16 (exact)
__device__ __forceinline__ uint4 q4x8(uint32_t w) {
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = static_cast<float>(static_cast<int>((w >> (8 * i)) & 15u) - 8);
        const float hi = static_cast<float>(static_cast<int>((w >> (8 * i + 4)) & 15u) - 8);
        o[i] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
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

// Index of element (row p, column n) of a bf16 activation matrix of width K
// (a multiple of 32) in fragment order: the order in which a product's wave
// reads its A operand (lane l: row l % 16, columns 8 (l / 16) .. +7 of a
// 32-wide block), so that its load of one 16 x 32 block is 1 KiB of
// consecutive bytes.  Eight consecutive columns from a multiple of 8 are
// contiguous.
__device__ __forceinline__ size_t frag_index(int p, int n, int K) {
    return ((static_cast<size_t>(p >> 4) * (K >> 5) + (n >> 5)) * 64 + ((n & 31) >> 3) * 16 + (p & 15)) * 8 +
           (n & 7);
}

// The activation layout of a frame: fragment order from kFragMinRows rows
// per position, else row-major.  A 16 x 32 operand load touches 4 cache
// lines (up to 8 rows) or 8 in fragment order, and one line per row
// row-major.
constexpr int kFragMinRows = 5;
__device__ __forceinline__ size_t act_index(int p, int n, int K, int frag) {
    return frag ? frag_index(p, n, K) : static_cast<size_t>(p) * K + n;
}

// ---------------------------------------------------------------------------
// [M x K] . [K x N] with a fused prologue (SRC) and epilogue (EPI).
// grid = (N / (16 CT) (SwiGLU: N / 16), ceil(M / (16 RT)), KS), 64 * NW
// threads (NW waves split the workgroup's K range); CT output fragments of
// 16 columns per workgroup.
// ---------------------------------------------------------------------------
template <int WT, int RT, int SRC, int EPI, int NW, int CT>
__global__ __launch_bounds__(64 * NW) void k_gemm(GemmArgs g) {
    static_assert(EPI != EPI_SWIGLU || CT == 2, "SwiGLU pairs a gate and an up fragment");
    __shared__ f32x4_t red[NW][RT][CT][64];
    __shared__ float rinv_s[RT][16];   // RMSNorm row scales, for the component-split epilogue
    __shared__ int last_s;

    QP_TSTAMP(g.tl, 0);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int bx = blockIdx.x, by = blockIdx.y, kz = blockIdx.z;
    const int m0 = by * 16 * RT;
    const int KB = g.K >> 5;
    const int kbw = KB / (NW * g.KS);            // k-blocks per wave (even)
    const int kb0 = (kz * NW + wave) * kbw;

    // output fragments of this workgroup
    int nb[CT];
    const uint8_t* wp[CT];
    const float* sp[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) {
        const FMat& W = (EPI == EPI_SWIGLU && c == 1) ? g.w1 : g.w0;
        nb[c] = (EPI == EPI_SWIGLU) ? bx : bx * CT + c;
        const size_t frag0 = static_cast<size_t>(nb[c]) * KB;
        wp[c] = static_cast<const uint8_t*>(W.w) + frag0 * 64 * (WT == WT_Q8 ? 8 : (WT == WT_Q4 ? 4 : 16));
        sp[c] = (WT == WT_Q8 || WT == WT_Q4) ? W.scale + frag0 * 16 : nullptr;
    }

    // this lane's A row (per row tile) and k offset inside a block
    const int arow = lane & 15, akoff = (lane >> 4) * 8;
    bool rok[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) rok[rt] = m0 + 16 * rt + arow < g.M;
    // bf16 operands: this lane's 8 inputs of k-block 0 per row tile, and the
    // step from one k-block to the next (fragment order: one 512-element
    // block; row-major: 32 elements)
    const uint16_t* abase[RT];
    const int astep = g.frag ? 512 : 32;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int p = g.a_row0 + m0 + 16 * rt + arow;   // physical row
        abase[rt] = static_cast<const uint16_t*>(g.a) +
                    (g.frag ? (static_cast<size_t>(p >> 4) * KB * 64 + (lane >> 4) * 16 + (p & 15)) * 8
                            : static_cast<size_t>(p) * g.K + akoff);
    }

    // RMSNorm row scales of the row tiles this wave finishes: lane l sums a
    // quarter of row (l % 16)'s tile sums (q = nss / 4 of them, a multiple
    // of 4 since dP % 256 == 0), the quarters are then combined across the
    // lane groups (fixed order).  The first 32 are requested here, all at
    // once, and summed after the K loop, so that their round trip overlaps
    // the products instead of preceding them.
    // Every product but the projection of H (which may split K over
    // workgroups) finishes its tile with the four waves sharing the work:
    // wave i < 4 takes component i of every lane's accumulator (row
    // 4 (lane / 16) + i of each row fragment), so the reduction, the
    // epilogue arithmetic and the stores run four wide instead of on one
    // wave per row fragment.
    constexpr bool kSplitEpi = EPI != EPI_BIAS;
    static_assert(RT <= NW, "a wave finishes at most one row fragment's scales");
    constexpr int kRssHeld = 8;                  // float4 loads held across the K loop
    float rss[RT];
    float4 rsv[kRssHeld];
    const int rq = g.nss >> 2;
    const int rsv_n = rq >> 2 < kRssHeld ? rq >> 2 : kRssHeld;
    const bool rown = SRC == SRC_BF16_NORM && wave < RT && rok[wave < RT ? wave : 0];
    const float* rsrc = (SRC == SRC_BF16_NORM && wave < RT)
                            ? g.ss_in + static_cast<size_t>(m0 + 16 * wave + arow) * g.nss + (lane >> 4) * rq
                            : nullptr;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) rss[rt] = 0.f;
#pragma unroll
    for (int j = 0; j < kRssHeld; ++j) {
        rsv[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (rown && j < rsv_n) rsv[j] = *reinterpret_cast<const float4*>(rsrc + 4 * j);
    }

    // residual-stream epilogues: the old x tile, the next reader's gain and
    // the bias are fetched before the products
    float xo[RT][CT][4], gnx[CT], bia[CT];
    if constexpr (EPI == EPI_RESID || EPI == EPI_BIAS) {
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            const int n = nb[c] * 16 + (lane & 15);
            gnx[c] = g.g_next[n];
            bia[c] = (EPI == EPI_BIAS) ? g.bias[n] : 0.f;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = m0 + 16 * rt + 4 * (lane >> 4) + (kSplitEpi ? wave : i);
                    const bool mine = kSplitEpi ? (i == 0 && wave < 4) : rt % NW == wave;
                    xo[rt][c][i] = (EPI == EPI_RESID && mine && m < g.M)
                                       ? g.out[static_cast<size_t>(m) * g.ldo + n] : 0.f;
                }
            }
        }
    }

    f32x4_t acc[RT][CT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int c = 0; c < CT; ++c) acc[rt][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // one batch of UU k-blocks: every load first, then the products
    auto batch = [&](int kb, auto uu) {
        constexpr int UU = decltype(uu)::value;
        uint4 av[UU][RT];
        uint4 wv[UU][CT];
        uint2 wq[UU][CT];
        uint32_t w4[UU][CT];
        float ws[UU][CT];
#pragma unroll
        for (int u = 0; u < UU; ++u) {
            const int k = (kb + u) * 32 + akoff;
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                if constexpr (WT == WT_Q8) {
                    wq[u][c] = *reinterpret_cast<const uint2*>(wp[c] + (static_cast<size_t>(kb + u) * 64 + lane) * 8);
                    ws[u][c] = sp[c][(kb + u) * 16 + (lane & 15)];
                } else if constexpr (WT == WT_Q4) {
                    w4[u][c] = *reinterpret_cast<const uint32_t*>(wp[c] + (static_cast<size_t>(kb + u) * 64 + lane) * 4);
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
                    const uint16_t* src = abase[rt] + static_cast<size_t>(kb + u) * astep;
                    av[u][rt] = rok[rt] ? *reinterpret_cast<const uint4*>(src) : make_uint4(0, 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < UU; ++u) {
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                uint4 w8;
                if constexpr (WT == WT_Q8) {
                    w8 = make_uint4(q8pair(wq[u][c].x, 0), q8pair(wq[u][c].x, 16), q8pair(wq[u][c].y, 0),
                                    q8pair(wq[u][c].y, 16));
                } else if constexpr (WT == WT_Q4) {
                    w8 = q4x8(w4[u][c]);
                } else {
                    w8 = wv[u][c];
                }
                const bf16x8_t wb = __builtin_bit_cast(bf16x8_t, w8);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const bf16x8_t ab = __builtin_bit_cast(bf16x8_t, av[u][rt]);
                    if constexpr (WT == WT_Q8 || WT == WT_Q4) {
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

    QP_TSTAMP(g.tl, 1);
    if constexpr (SRC == SRC_BF16_NORM) {
        // the row-scale sums, in pairs in column order (rows past M add zeros)
        if (wave < RT) {
            float t = 0.f;
#pragma unroll
            for (int j = 0; j < kRssHeld; ++j) {
                if (j < rsv_n) {
                    t += rsv[j].x + rsv[j].y;
                    t += rsv[j].z + rsv[j].w;
                }
            }
            // d > 2048: the rest, 32 at a time, each group requested together
            for (int b = kRssHeld; rown && 4 * b < rq; b += kRssHeld) {
                float4 v[kRssHeld];
#pragma unroll
                for (int j = 0; j < kRssHeld; ++j)
                    if (4 * (b + j) < rq) v[j] = *reinterpret_cast<const float4*>(rsrc + 4 * (b + j));
#pragma unroll
                for (int j = 0; j < kRssHeld; ++j) {
                    if (4 * (b + j) < rq) {
                        t += v[j].x + v[j].y;
                        t += v[j].z + v[j].w;
                    }
                }
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                if (rt == wave) rss[rt] = t;
        }
    }
    // ---- reduce the four waves' K ranges, in wave order ----
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int c = 0; c < CT; ++c) red[wave][rt][c][lane] = acc[rt][c];
    if constexpr (kSplitEpi && SRC == SRC_BF16_NORM) {
        // the wave that summed row fragment rt's squares publishes its 16 row scales
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if (rt % NW != wave) continue;
            float t = rss[rt];
            t += __shfl_xor(t, 16, 64);
            t += __shfl_xor(t, 32, 64);   // every lane: the sum for row lane % 16
            if (lane < 16) rinv_s[rt][lane] = 1.0f / sqrtf(t / static_cast<float>(g.K) + g.eps);
        }
    }
    __syncthreads();

    if constexpr (kSplitEpi) {
        if (wave < 4) {
            const int i = wave;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int m = m0 + 16 * rt + 4 * (lane >> 4) + i;
                float rinv = 1.f;
                if constexpr (SRC == SRC_BF16_NORM) rinv = rinv_s[rt][4 * (lane >> 4) + i];
                // component i of the NW partial tiles, summed in wave order
                float v[CT];
#pragma unroll
                for (int c = 0; c < CT; ++c) {
                    const float* r = reinterpret_cast<const float*>(&red[0][rt][c][lane]) + i;
                    float t = r[0];
#pragma unroll
                    for (int w = 1; w < NW; ++w) t += r[w * RT * CT * 64 * 4];
                    v[c] = t;
                }
                if constexpr (EPI == EPI_ARGMAX) {
                    uint64_t key = 0;
#pragma unroll
                    for (int c = 0; c < CT; ++c) {
                        const int n = nb[c] * 16 + (lane & 15);
                        const float x = v[c] * rinv;
                        if (g.logits && m < g.M) g.logits[m * g.logit_ld + n] = x;
                        key = umax64(key, argmax_key(x, n));
                    }
#pragma unroll
                    for (int o = 1; o < 16; o <<= 1) key = umax64(key, shfl_xor64(key, o));
                    if ((lane & 15) == 0 && m < g.M) g.keys[static_cast<size_t>(m) * gridDim.x + bx] = key;
                } else if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
                    for (int pp = 0; pp < CT / 2; ++pp) {
                        const int n = nb[2 * pp] * 16 + (lane & 15);
                        if (m < g.M) {
                            const float gt = v[2 * pp] * rinv, ut = v[2 * pp + 1] * rinv;
                            g.outb[act_index(m, n, g.N, g.frag)] = to_bf16((gt / (1.0f + expf(-gt))) * ut);
                        }
                    }
                } else if constexpr (EPI == EPI_SCALE) {
#pragma unroll
                    for (int c = 0; c < CT; ++c) {
                        const int n = nb[c] * 16 + (lane & 15);
                        if (m < g.M) g.out[static_cast<size_t>(m) * g.ldo + n] = v[c] * rinv;
                    }
                } else {
                    // residual stream rows: x (fp32), xg = bf16(g_next * x), and
                    // the sum of x^2 over each 16-column fragment
#pragma unroll
                    for (int c = 0; c < CT; ++c) {
                        const int n = nb[c] * 16 + (lane & 15);
                        float sq = 0.f;
                        if (m < g.M) {
                            const float nv = xo[rt][c][0] + v[c];
                            if (g.taps) {
                                const int B = g.tap_B;
                                const int pos = row_pos(g.tap_s, B, m), b = row_req(g.tap_s, B, m);
                                g.taps[((static_cast<size_t>(pos) * g.tap_L + g.tap_l) * B + b) * g.ldo + n] = nv;
                            }
                            g.out[static_cast<size_t>(m) * g.ldo + n] = nv;
                            g.xg[act_index(m, n, g.ldo, g.frag)] = to_bf16(gnx[c] * nv);
                            sq = nv * nv;
                        }
                        const float t = sum16(sq);
                        if ((lane & 15) == 0 && m < g.M) g.ss_out[static_cast<size_t>(m) * (g.ldo / 16) + nb[c]] = t;
                    }
                }
            }
        }
        QP_TSTAMP(g.tl, 2);
        return;
    }

    // wave w finishes row tiles w, w + NW, ...
    f32x4_t tot[RT][CT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        if (rt % NW != wave) continue;
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            f32x4_t t = red[0][rt][c][lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) t += red[w][rt][c][lane];
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
            return static_cast<uint32_t>(((((static_cast<size_t>(z) * tiles + tile) * RT + rt) * CT + c) * 64 + lane) * 16);
        };
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if (rt % NW != wave) continue;
#pragma unroll
            for (int c = 0; c < CT; ++c)
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
        if (!last_s) {
            QP_TSTAMP(g.tl, 2);
            return;
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if (rt % NW != wave) continue;
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                // every partial requested first, then summed in kz order
                f32x4_t pz[kMaxKS];
#pragma unroll
                for (int z = 0; z < kMaxKS; ++z)
                    if (z < g.KS)
                        pz[z] = __builtin_bit_cast(f32x4_t,
                                                   __builtin_amdgcn_raw_buffer_load_b128(pr, poff(z, rt, c), 0u, kDevScope));
                f32x4_t t = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int z = 0; z < kMaxKS; ++z)
                    if (z < g.KS) t += pz[z];
                tot[rt][c] = t;
            }
        }
    }

    // ---- epilogue: lane holds rows 4*(lane/16)+i, column lane%16 of each fragment ----
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        if (rt % NW != wave) continue;
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
            for (int c = 0; c < CT; ++c) {
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
                g.outb[act_index(m, n, g.N, g.frag)] = to_bf16((gt / (1.0f + expf(-gt))) * ut);
            }
        } else if constexpr (EPI == EPI_SCALE) {
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                const int n = nb[c] * 16 + (lane & 15);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = m0 + 16 * rt + 4 * (lane >> 4) + i;
                    if (m < g.M) g.out[static_cast<size_t>(m) * g.ldo + n] = tot[rt][c][i] * rinv[i];
                }
            }
        } else {
            // residual stream rows: x (fp32), xg = bf16(g_next * x), and the
            // sum of x^2 over each 16-column fragment
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                float sq[4] = {0.f, 0.f, 0.f, 0.f};
                const int n = nb[c] * 16 + (lane & 15);
                const float gn = gnx[c];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = m0 + 16 * rt + 4 * (lane >> 4) + i;
                    if (m >= g.M) continue;
                    float* o = g.out + static_cast<size_t>(m) * g.ldo + n;
                    float nv;
                    if constexpr (EPI == EPI_BIAS) {
                        nv = tot[rt][c][i] + bia[c];
                    } else {
                        nv = xo[rt][c][i] + tot[rt][c][i];
                        if (g.taps) {
                            const int B = g.tap_B;
                            const int pos = row_pos(g.tap_s, B, m), b = row_req(g.tap_s, B, m);
                            g.taps[((static_cast<size_t>(pos) * g.tap_L + g.tap_l) * B + b) * g.ldo + n] = nv;
                        }
                    }
                    *o = nv;
                    g.xg[act_index(m, n, g.ldo, g.frag)] = to_bf16(gn * nv);
                    sq[i] = nv * nv;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float t = sum16(sq[i]);
                    const int m = m0 + 16 * rt + 4 * (lane >> 4) + i;
                    if ((lane & 15) == 0 && m < g.M) g.ss_out[static_cast<size_t>(m) * (g.ldo / 16) + nb[c]] = t;
                }
            }
        }
    }
    QP_TSTAMP(g.tl, 2);
}

// Row helpers of the token steps.  Thread j owns elements j, j + 256, ...
// (dT and dP are multiples of 256 and at most 4096); callers issue every
// load before any store so that one memory round trip covers a row.
constexpr int kMaxPer = 16;
// elements per thread of a workgroup's slice of the token move (k_attn with
// the token decision): the layer-0 table, and with it that variant, exists
// only for geometries whose slices fit (checked where the table is built)
constexpr int kTokPer = 1;

// x, xg = bf16(g * x) and the per-16-column sums of x^2 of residual-stream
// row `row` from values v (with gains gv) already in registers; a
// fragment's sum is reduced over the 16 threads that own it.
__device__ __forceinline__ void store_row(const TokArgs& ta, int row, const float (&v)[kMaxPer],
                                          const float (&gv)[kMaxPer]) {
    const int j = threadIdx.x, np = ta.dP / kThreadsT;
    float* xr = ta.x + static_cast<size_t>(row) * ta.dP;
    // element j + 256 i: 256 columns on is eight 32-wide blocks on in
    // fragment order, 256 elements on row-major
    uint16_t* gr = ta.xg + act_index(row, j, ta.dP, ta.frag);
    const int gstep = ta.frag ? 4096 : kThreadsT;
    float* sr = ta.ss + static_cast<size_t>(row) * (ta.dP / 16);
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
        if (i < np) {
            const int n = j + kThreadsT * i;
            xr[n] = v[i];
            gr[i * gstep] = to_bf16(gv[i] * v[i]);
            float q = v[i] * v[i];
            q += __shfl_xor(q, 1, 64);
            q += __shfl_xor(q, 2, 64);
            q += __shfl_xor(q, 4, 64);
            q += __shfl_xor(q, 8, 64);
            if ((j & 15) == 0) sr[n >> 4] = q;
        }
    }
}

__device__ __forceinline__ void load_vec(const float* src, int n_per, float (&v)[kMaxPer]) {
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i)
        if (i < n_per) v[i] = src[threadIdx.x + kThreadsT * i];
}

__device__ __forceinline__ void load_emb(const TokArgs& ta, int t, float (&e)[kMaxPer]) {
    const int ne = ta.dT / kThreadsT;
    const size_t row = static_cast<size_t>(t) * ta.dT;
    if (ta.emb_bf16) {
        const uint16_t* E = static_cast<const uint16_t*>(ta.emb) + row;
#pragma unroll
        for (int i = 0; i < kMaxPer; ++i)
            if (i < ne) e[i] = __uint_as_float(static_cast<uint32_t>(E[threadIdx.x + kThreadsT * i]) << 16);
    } else {
        const float* E = static_cast<const float*>(ta.emb) + row;
#pragma unroll
        for (int i = 0; i < kMaxPer; ++i)
            if (i < ne) e[i] = E[threadIdx.x + kThreadsT * i];
    }
}

// Per-head RMSNorm then rotate-half RoPE of a head vector held by one wave
// (element lane + 64 j in v[j]); the pair of element i is element i + hd/2.
// The gains and a position's rotation factors are fetched apart from the
// arithmetic, so that a caller can request them with its first reads (none
// depends on the data).
template <int HD>
struct RopeRow {
    static constexpr int H2 = HD / 128 > 0 ? HD / 128 : 1;
    float c[H2], s[H2];
};
template <int HD>
__device__ __forceinline__ void gain_fetch(const float* gain, float (&g)[HD / 64]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < HD / 64; ++j) g[j] = gain[lane + 64 * j];
}
template <int HD>
__device__ __forceinline__ void rope_fetch(const float* rcos, const float* rsin, int pos, RopeRow<HD>& r) {
    const int lane = threadIdx.x & 63;
    const float* cp = rcos + pos * (HD / 2);
    const float* sp = rsin + pos * (HD / 2);
    if constexpr (HD / 64 == 1) {
        r.c[0] = cp[lane & 31];
        r.s[0] = sp[lane & 31];
    } else {
#pragma unroll
        for (int j = 0; j < RopeRow<HD>::H2; ++j) {
            r.c[j] = cp[lane + 64 * j];
            r.s[j] = sp[lane + 64 * j];
        }
    }
}
template <int HD>
__device__ __forceinline__ void norm_rope_apply(const float (&v)[HD / 64], const float (&g)[HD / 64],
                                                const RopeRow<HD>& r, float eps, float (&out)[HD / 64]) {
    constexpr int J = HD / 64;
    const int lane = threadIdx.x & 63;
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) ss += v[j] * v[j];
    ss = wave_sum(ss);
    const float rinv = 1.0f / sqrtf(ss / static_cast<float>(HD) + eps);
    float w[J];
#pragma unroll
    for (int j = 0; j < J; ++j) w[j] = g[j] * (v[j] * rinv);
    if constexpr (J == 1) {
        const float partner = __shfl_xor(w[0], 32, 64);
        const float c = r.c[0], sn = r.s[0];
        out[0] = (lane < 32) ? (w[0] * c - partner * sn) : (w[0] * c + partner * sn);
    } else {
        constexpr int H2 = J / 2;
#pragma unroll
        for (int j = 0; j < H2; ++j) {
            const float c = r.c[j], sn = r.s[j];
            out[j] = w[j] * c - w[j + H2] * sn;
            out[j + H2] = w[j + H2] * c + w[j] * sn;
        }
    }
}

// ---------------------------------------------------------------------------
// Attention of one step: one workgroup per (request, kv head).  Every
// position of the step is handled in order (the prefill's position 1 sees
// position 0).  Keys and values of earlier positions come from the fp32 KV
// cache; the new position's key gets its per-head RMSNorm and RoPE here and
// is appended to the cache.  All global reads (history, the step's q/k/v
// rows) are issued before the first barrier.  Scores for all <= 16 keys are
// formed at once: key t on lanes 4t..4t+3, each lane a quarter of the head.
// Output: bf16 rows [M][nq*hd], the operand of the output projection.
// ---------------------------------------------------------------------------
// Step ta.s's token of request b from the lm_head tiles' keys (or the drawn
// token of a sampled frame), and the token fed back (forced or own), checked
// and clamped; block-wide, uniform result.  The writer also stores the token
// and raises the flags.  red: [kThreadsT / 64] LDS scratch, fed_s: one int.
__device__ __forceinline__ int decide_fed(const TokArgs& ta, int b, bool writer, uint64_t* red, int* fed_s) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nkt = ta.nkt;
    uint64_t k = 0;
    if (!ta.sampled)
        for (int t = threadIdx.x; t < nkt; t += kThreadsT) k = umax64(k, ta.keys[static_cast<size_t>(b) * nkt + t]);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) k = umax64(k, shfl_xor64(k, off));
    __syncthreads();
    if (lane == 0) red[wave] = k;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t kk = red[0];
        for (int w = 1; w < kThreadsT / 64; ++w) kk = umax64(kk, red[w]);
        const int tok = ta.sampled ? ta.sampled[b] : argmax_index(kk);
        int fed = ta.force ? ta.force[b * kSteps + (ta.s - 1)] : tok;
        const bool bad = fed < 0 || fed >= ta.V;
        if (writer) {
            ta.tok_out[b * kSteps + (ta.s - 1)] = tok;
            if (bad) atomicOr(ta.err, ta.force ? kErrBadForced : kErrBadQ0);
        }
        *fed_s = bad ? 0 : fed;
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(*fed_s);
}

template <int HD, bool TOK>
__global__ __launch_bounds__(kThreadsT, HD <= 128 ? 4 : 3) void k_attn(AttnArgs m) {
    constexpr int J = HD / 64;        // elements per lane in the lane + 64 j layout
    constexpr int SL = HD / 4;        // slice of the head per lane in the score
    constexpr int HPT = kPositions * HD / kThreadsT;   // history elements per thread (max)
    __shared__ float Ks[kPositions][HD];
    __shared__ float Vs[kPositions][HD];
    __shared__ float qs[4][HD];
    __shared__ float es[4][kPositions];
    __shared__ uint64_t red_s[kThreadsT / 64];
    __shared__ int fed_s;
    QP_TSTAMP(m.tl, 0);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int B = m.B, s = m.s, l = m.l;
    const int nkv = m.nkv, grp = m.nq / m.nkv;
    const int b = blockIdx.x / nkv, g = blockIdx.x % nkv;
    const int npos = (s == 1) ? 2 : 1;
    const int pf = (s == 1) ? 0 : s;
    const size_t kvb = ((static_cast<size_t>(l) * m.max_batch + b) * kPositions) * nkv * HD;

    // ---- every global read first ----
    float hk[HPT], hv[HPT];
#pragma unroll
    for (int i = 0; i < HPT; ++i) {
        const int idx = threadIdx.x + kThreadsT * i;
        hk[i] = hv[i] = 0.f;
        if (idx < pf * HD) {
            const int t = idx / HD, d = idx - t * HD;
            const size_t off = kvb + (static_cast<size_t>(t) * nkv + g) * HD + d;
            hk[i] = m.kc[off];
            hv[i] = m.vc[off];
        }
    }
    // the history into LDS
    auto stash_history = [&]() {
#pragma unroll
        for (int i = 0; i < HPT; ++i) {
            const int idx = threadIdx.x + kThreadsT * i;
            if (idx < pf * HD) {
                const int t = idx / HD, d = idx - t * HD;
                Ks[t][d] = hk[i];
                Vs[t][d] = hv[i];
            }
        }
    };
    // layer 0 with the table: the previous step's token first (the history
    // loads above are in flight meanwhile).  The request's move to the token
    // (embsum += E[t], residual row = P[t]) is shared by its nkv workgroups,
    // each taking a contiguous slice of both rows: a single workgroup doing
    // all of it ended about 6 us after the others at B = 128.
    const TokArgs& ta = m.tok;
    int fed = -1;
    float o_es[TOK ? kTokPer : 1], o_v[TOK ? kTokPer : 1];
    uint32_t o_e[TOK ? kTokPer : 1];    // E[t] elements as loaded: bf16 or fp32 bits
    const int eT = (ta.dT + nkv - 1) / nkv, eP = (ta.dP + nkv - 1) / nkv;   // slice lengths
    const int cT = g * eT, cP = g * eP;                                     // slice starts
    // this thread's element i of a slice [c0, c0 + len) of a row of n, or -1
    auto slot = [&](int i, int len, int c0, int n) {
        const int e = threadIdx.x + kThreadsT * i;
        return (e < len && c0 + e < n) ? c0 + e : -1;
    };
    float* const es_row = ta.embsum + static_cast<size_t>(b) * ta.dT;
    // Every load below is issued unconditionally from an in-range address (a
    // missing element reads element 0 and is not stored) and converted only
    // where it is used: with a branch or a conversion beside each load the
    // compiler waited for every load before issuing the next.
    if constexpr (TOK) {
#pragma unroll
        for (int i = 0; i < kTokPer; ++i) o_es[i] = es_row[max(slot(i, eT, cT, ta.dT), 0)];
        fed = decide_fed(ta, b, g == 0, red_s, &fed_s);
        // the history arrived before the keys (a wave's loads return in
        // order): into LDS now, freeing its registers for the loads below
        stash_history();
        const size_t erow = static_cast<size_t>(fed) * ta.dT;
        if (ta.emb_bf16) {
            const uint16_t* E = static_cast<const uint16_t*>(ta.emb) + erow;
#pragma unroll
            for (int i = 0; i < kTokPer; ++i) o_e[i] = E[max(slot(i, eT, cT, ta.dT), 0)];
        } else {
            const uint32_t* E = static_cast<const uint32_t*>(ta.emb) + erow;
#pragma unroll
            for (int i = 0; i < kTokPer; ++i) o_e[i] = E[max(slot(i, eT, cT, ta.dT), 0)];
        }
        const float* prow = ta.ptab + static_cast<size_t>(fed) * ta.dP;
#pragma unroll
        for (int i = 0; i < kTokPer; ++i) o_v[i] = prow[max(slot(i, eP, cP, ta.dP), 0)];
    }
    // the step's q/k/v row of position pi: from the table when fed >= 0
    auto qkv_row = [&](int pi) {
        const int r = (s == 1) ? pi * B + b : b;
        return fed >= 0 ? ta.qkv0 + static_cast<size_t>(fed) * m.nqkv : m.qkv + static_cast<size_t>(r) * m.nqkv;
    };
    // the per-head norm gains and the RoPE rows of the step's positions,
    // requested ahead of the head vectors (with them, they were requested
    // only after the history had been awaited: one more round trip for the
    // key, another after the barrier for the queries)
    float gk[J], gq[J];
    RopeRow<HD> rp[2];
    gain_fetch<HD>(m.k_norm, gk);
    gain_fetch<HD>(m.q_norm, gq);
#pragma unroll
    for (int pi = 0; pi < 2; ++pi) rope_fetch<HD>(m.rope_cos, m.rope_sin, pf + (pi < npos ? pi : 0), rp[pi]);
    auto rope_of = [&](int pi) {
        RopeRow<HD> r;
#pragma unroll
        for (int h = 0; h < RopeRow<HD>::H2; ++h) {
            r.c[h] = pi ? rp[1].c[h] : rp[0].c[h];
            r.s[h] = pi ? rp[1].s[h] : rp[0].s[h];
        }
        return r;
    };
    // wave 0: the step's key rows, wave 1: value rows, wave w: query head
    // g * grp + w (later heads of a large group are read when used)
    float pin[2][J];
#pragma unroll
    for (int pi = 0; pi < 2; ++pi) {
        const float* row = qkv_row(pi);
        const int col = wave == 0 ? (m.nq + g) * HD : (wave == 1 ? (m.nq + nkv + g) * HD : 0);
#pragma unroll
        for (int j = 0; j < J; ++j) pin[pi][j] = 0.f;
        if (pi < npos && wave < 2) {
#pragma unroll
            for (int j = 0; j < J; ++j) pin[pi][j] = row[col + lane + 64 * j];
        }
    }
    float qin[2][J];
#pragma unroll
    for (int pi = 0; pi < 2; ++pi) {
        const float* row = qkv_row(pi);
#pragma unroll
        for (int j = 0; j < J; ++j) qin[pi][j] = 0.f;
        if (pi < npos && wave < grp) {
#pragma unroll
            for (int j = 0; j < J; ++j) qin[pi][j] = row[(g * grp + wave) * HD + lane + 64 * j];
        }
    }
    // this workgroup's share of the request's move to the token (its loads
    // were issued before the head vectors', so this waits for nothing the
    // attention does not need); the residual row's next reader is layer 0's
    // residual add (its q/k/v come from the table), so x alone
    if constexpr (TOK) {
        float* x_row = ta.x + static_cast<size_t>(b) * ta.dP;
#pragma unroll
        for (int i = 0; i < kTokPer; ++i) {
            const int jt = slot(i, eT, cT, ta.dT), jp = slot(i, eP, cP, ta.dP);
            const float e = __uint_as_float(ta.emb_bf16 ? o_e[i] << 16 : o_e[i]);
            if (jt >= 0) es_row[jt] = o_es[i] + e;
            if (jp >= 0) x_row[jp] = o_v[i];
        }
    }
    if constexpr (!TOK) stash_history();

    for (int pi = 0; pi < npos; ++pi) {
        const int p = pf + pi;
        const int r = (s == 1) ? pi * B + b : b;
        float kr[J];
        if (wave == 0) {
            norm_rope_apply<HD>(pin[pi], gk, rope_of(pi), m.eps, kr);
#pragma unroll
            for (int j = 0; j < J; ++j) Ks[p][lane + 64 * j] = kr[j];
        } else if (wave == 1) {
#pragma unroll
            for (int j = 0; j < J; ++j) Vs[p][lane + 64 * j] = pin[pi][j];
        }
        __syncthreads();
        if (pi == 0) QP_TSTAMP(m.tl, 1);
        for (int i = wave; i < grp; i += 4) {
            const int h = g * grp + i;
            float qv[J], q[J];
            if (i == wave) {
#pragma unroll
                for (int j = 0; j < J; ++j) qv[j] = qin[pi][j];
            } else {
                const float* row = qkv_row(pi) + h * HD;
#pragma unroll
                for (int j = 0; j < J; ++j) qv[j] = row[lane + 64 * j];
            }
            norm_rope_apply<HD>(qv, gq, rope_of(pi), m.eps, q);
#pragma unroll
            for (int j = 0; j < J; ++j) qs[wave][lane + 64 * j] = q[j];
            const int kt = lane >> 2, k0 = (lane & 3) * SL;
            float sc = 0.f;
            if (kt <= p) {
#pragma unroll
                for (int d = 0; d < SL; d += 4) {
                    const float4 qq = *reinterpret_cast<const float4*>(&qs[wave][k0 + d]);
                    const float4 kk = *reinterpret_cast<const float4*>(&Ks[kt][k0 + d]);
                    sc = fmaf(qq.x, kk.x, sc);
                    sc = fmaf(qq.y, kk.y, sc);
                    sc = fmaf(qq.z, kk.z, sc);
                    sc = fmaf(qq.w, kk.w, sc);
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
            // columns lane + 64 j: 64 columns on is two 32-wide blocks on
            // in fragment order, 64 elements on row-major
            uint16_t* op = m.ao + act_index(r, h * HD + lane, m.nq * HD, m.frag);
            const int ostep = m.frag ? 1024 : 64;
#pragma unroll
            for (int j = 0; j < J; ++j) op[j * ostep] = to_bf16(o[j] / den);
        }
        // this position's key and value into the cache, after the position's
        // reads: a wave's loads and stores complete in one order, so a store
        // ahead of them made their waits wait for it too
        const size_t off = kvb + (static_cast<size_t>(p) * nkv + g) * HD;
        if (wave == 0) {
#pragma unroll
            for (int j = 0; j < J; ++j) m.kc[off + lane + 64 * j] = kr[j];
        } else if (wave == 1) {
#pragma unroll
            for (int j = 0; j < J; ++j) m.vc[off + lane + 64 * j] = pin[pi][j];
        }
        __syncthreads();
    }
    QP_TSTAMP(m.tl, 2);
}

// Frame start, per request: check q0, x[pos 1] = P_0[q0], embsum = E_0[q0].
// (x[pos 0] = W_p . H + b_p is a product of its own.)
__global__ __launch_bounds__(kThreadsT) void k_start(TokArgs ta) {
    __shared__ int tok_s;
    QP_TSTAMP(ta.tl, 0);
    const int B = ta.B, ne = ta.dT / kThreadsT, np = ta.dP / kThreadsT;
    float gv[kMaxPer], v[kMaxPer], e[kMaxPer];
    load_vec(ta.gain0, np, gv);
    for (int b = blockIdx.x; b < B; b += gridDim.x) {
        __syncthreads();
        if (threadIdx.x == 0) {
            int q = ta.q0[b];
            if (q < 0 || q >= ta.V) {
                atomicOr(ta.err, kErrBadQ0);
                q = 0;
            }
            tok_s = q;
        }
        __syncthreads();
        const int q = __builtin_amdgcn_readfirstlane(tok_s);
        load_vec(ta.ptab + static_cast<size_t>(q) * ta.dP, np, v);
        load_emb(ta, q, e);
        store_row(ta, B + b, v, gv);
        float* es = ta.embsum + static_cast<size_t>(b) * ta.dT;
#pragma unroll
        for (int i = 0; i < kMaxPer; ++i)
            if (i < ne) es[threadIdx.x + kThreadsT * i] = e[i];
    }
    QP_TSTAMP(ta.tl, 2);
}

// Step s's token per request from the lm_head tiles' keys; the fed-back
// token (forced or own) adds E_s[t] to embsum and, before the last step,
// sets the next position's input row P_s[t] (and, with the table, that row's
// layer-0 q/k/v rows).
__global__ __launch_bounds__(kThreadsT) void k_next(TokArgs ta) {
    __shared__ uint64_t red[kThreadsT / 64];
    __shared__ int fed_s;
    QP_TSTAMP(ta.tl, 0);
    const int B = ta.B;
    const int ne = ta.dT / kThreadsT, np = ta.dP / kThreadsT;
    float gv[kMaxPer], o[kMaxPer], v[kMaxPer], e[kMaxPer];
    if (ta.ptab) load_vec(ta.gain0, np, gv);
    for (int b = blockIdx.x; b < B; b += gridDim.x) {
        float* es = ta.embsum + static_cast<size_t>(b) * ta.dT;
        load_vec(es, ne, o);
        const int t = decide_fed(ta, b, true, red, &fed_s);
        load_emb(ta, t, e);
        if (ta.ptab) load_vec(ta.ptab + static_cast<size_t>(t) * ta.dP, np, v);
        if (ta.qkv0) {
            const float4* src = reinterpret_cast<const float4*>(ta.qkv0 + static_cast<size_t>(t) * ta.nqkv);
            float4* dst = reinterpret_cast<float4*>(ta.qkv + static_cast<size_t>(b) * ta.nqkv);
            for (int i = threadIdx.x; i < ta.nqkv / 4; i += kThreadsT) dst[i] = src[i];
        }
#pragma unroll
        for (int i = 0; i < kMaxPer; ++i)
            if (i < ne) es[threadIdx.x + kThreadsT * i] = o[i] + e[i];
        if (ta.ptab) store_row(ta, b, v, gv);
    }
    QP_TSTAMP(ta.tl, 2);
}

}  // namespace tiled
}  // namespace qp

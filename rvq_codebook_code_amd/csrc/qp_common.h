// Shared device-side definitions of the code-predictor library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qp {

constexpr int kThreads = 256;            // 4 wave64 per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kCodebooks = 16;
constexpr int kSteps = kCodebooks - 1;
constexpr int kPositions = kCodebooks;   // positions 0..15 per frame
constexpr int kLdsFloats = 16384;        // 64 KiB workgroup scratch
constexpr int kMaxHeadDim = 256;
constexpr int kMaxRowsPerChunk = 4;

// WT_Q4 only names the 4-bit fragment layout of the batched path; elsewhere
// Q4_0 weights are held as int8 codes (code - 8) with WT_Q8's block scales.
enum WeightType : int { WT_F32 = 0, WT_BF16 = 1, WT_Q8 = 2, WT_Q4 = 3 };

// Device error flag bits (also documented in qp.h).
// Phase timeline of the dataflow kernels, in a separate build of the same
// sources (libqp_timeline.so, compiled with QP_TIMELINE): thread 0 of
// workgroup wg writes the GPU's 100 MHz real-time counter at three points of
// phase ph (k = 0: the phase starts, 1: its inputs are staged, 2: its
// stores are issued) into the caller's taps buffer, read as uint64
// [256][kTimelinePhases][3].  That build writes no residual taps.  The
// product build compiles none of it.
constexpr int kTimelinePhases = 400;
#ifdef QP_TIMELINE
constexpr bool kWriteTaps = false;
#define QP_STAMP(taps, wg, ph, k)                                                                         \
    do {                                                                                                  \
        if ((taps) && threadIdx.x == 0 && (ph) < ::qp::kTimelinePhases)                                   \
            reinterpret_cast<unsigned long long*>(taps)[(static_cast<size_t>(wg) * ::qp::kTimelinePhases + \
                                                         (ph)) * 3 + (k)] = __builtin_amdgcn_s_memrealtime(); \
    } while (0)
#else
constexpr bool kWriteTaps = true;
#define QP_STAMP(taps, wg, ph, k) ((void)0)
#endif

// Kernel timeline of the batched path, in the same timeline build: every
// kernel launch of a frame carries its index (tl, -1 elsewhere), and thread
// 0 of each workgroup (linear id below kTiledWgs) writes the real-time
// counter at its start (k = 0), at the end of a product's K loop or once an
// attention's inputs are in LDS (k = 1) and at its end (k = 2) into a device
// array of [kTiledLaunches][kTiledWgs][3], read back with qp_timeline_tiled.
// The graph replays of a frame overwrite it; the product build compiles none
// of it.
constexpr int kTiledLaunches = 448, kTiledWgs = 1024;
#ifdef QP_TIMELINE
__device__ unsigned long long g_tiled_stamps[kTiledLaunches * kTiledWgs * 3];
#define QP_TSTAMP(tl, k)                                                                                     \
    do {                                                                                                     \
        if (threadIdx.x == 0 && (tl) >= 0 && (tl) < ::qp::kTiledLaunches) {                                  \
            const int lin_ = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);                 \
            if (lin_ < ::qp::kTiledWgs)                                                                      \
                ::qp::g_tiled_stamps[(static_cast<size_t>(tl) * ::qp::kTiledWgs + lin_) * 3 + (k)] =         \
                    __builtin_amdgcn_s_memrealtime();                                                        \
        }                                                                                                    \
    } while (0)
#else
#define QP_TSTAMP(tl, k) ((void)0)
#endif

constexpr unsigned kErrBadQ0 = 1u;
constexpr unsigned kErrBadForced = 2u;
constexpr unsigned kErrBarrierTimeout = 4u;

// A linear layer's weights on the device, row-major [N][K]:
//   WT_F32: float, WT_BF16: uint16 bf16, WT_Q8: int8 codes with one fp32
//   scale per 32-wide block along K in `scale` [N][K/32].
struct Mat {
    const void* w;
    const float* scale;
};

struct LayerDev {
    Mat qkv;          // [(nq+2nkv)*hd][dP]: q rows, then k rows, then v rows
    Mat o;            // [dP][nq*hd]
    Mat gate, up;     // [F][dP]
    Mat down;         // [dP][F]
    const float* attn_norm;
    const float* q_norm;
    const float* k_norm;
    const float* ffn_norm;
};

// Everything a launch needs that does not change between calls.
struct Model {
    int dT, dP, L, nq, nkv, hd, F, V, wt, emb_bf16, nqkv, max_batch;
    float eps, attn_scale;
    Mat proj;
    const float* proj_b;
    const void* emb[kCodebooks];   // [V][dT] fp32 or bf16
    const float* ptab;             // [15][V][dP]: W_p . E_j + b_p, j = 0..14
    const float* qkv0;             // [14][V][nqkv]: layer 0's q/k/v rows of P_j[v], j = 1..14
                                   // (dataflow kernel only; null elsewhere)
    const LayerDev* layers;        // device array [L]
    const float* out_norm;
    Mat lm[kSteps];
    const float* rope_cos;         // [16][hd/2]
    const float* rope_sin;
    // scratch (sized for max_batch)
    float* x;                      // [2*maxB][dP]   residual stream rows
    float* qkv;                    // [2*maxB][nqkv]
    float* ao;                     // [2*maxB][nq*hd] attention output (the batched path: bf16 in fragment order)
    float* hb;                     // [2*maxB][F]     SwiGLU activations (the batched path: bf16 in fragment order)
    float* kc;                     // [L][maxB][16][nkv][hd]
    float* vc;
    unsigned long long* amax;      // [maxB] packed (logit, index) argmax keys
    unsigned* err;                 // sticky flag word
    unsigned long long* bar;       // grid barrier counter
};

// Per-call arguments.
struct RunArgs {
    int B;
    const float* H;        // [B][dT]
    const int* q0;         // [B]
    int* tok_out;          // [B][15]
    float* embsum;         // [B][dT]
    const int* force;      // [B][15] or null
    float* logits_out;     // [B][15][V] or null
    float* taps;           // [16][L][B][dP] or null
    const float* uniforms; // [B][15] caller's draws for sampled frames, or null (greedy)
    unsigned long long bar_base;  // grid barriers completed by earlier launches
    uint32_t seq0;                // record epochs used by earlier launches
};

}  // namespace qp

// Caller-controlled sampling of one token per row from fp32 logits, in place
// of the argmax.  The pages leave sampling to the caller (rightkit-qts
// exporter README, "Qwen3-TTS 1.7B -> QTS GGUF", section "Usage") and describe
// the exported predictor as greedy; the controls taken here are the usual
// temperature, top-k and top-p, with one caller-supplied uniform per row:
//
//   rank order   descending logit, lower vocabulary index first on ties;
//   weights      w_r = exp((z_r - z_0) / T) for rank r (z_0 the largest);
//   top-k        ranks r < K (K = 0: all);
//   top-p        the shortest rank-order prefix of those whose weight
//                reaches P times their total (at least one);
//   draw         the first kept rank whose inclusive cumulative weight
//                exceeds u times the kept total (u clamped to [0, 1], NaN
//                as 0), else the last kept rank.
//
// One workgroup per row.  The row's keys (ordered fp32 bits of the logit,
// then the complement of the index) are sorted by a bitonic network with each
// thread holding a contiguous run of positions in registers: pairs inside a
// thread are exchanged in registers, pairs inside a wave by lane shuffles and
// only pairs across waves through LDS.  Each thread then owns a contiguous
// run of ranks, sums its weights in order and takes its offset from a
// block-wide scan; the top-p cut and the draw are block-wide minima over
// "first rank that passes".  The cumulative weights are fp32 sums in this
// order (at most 16 terms per thread, a 6-step wave scan, 3 cross-wave
// additions): only draws whose threshold lies within about 2e-6 of the total
// from a boundary can differ from an exact evaluation.
#pragma once

#include "qp_common.h"

namespace qp {
namespace sample {

constexpr int kThreadsSm = 256;
constexpr int kMaxV = 4096;  // LDS: 32 KiB of keys

struct Params {
    float temperature;  // > 0
    int top_k;          // 0 = every token
    float top_p;        // (0, 1]
};

// fp32 -> uint32 whose unsigned order is the float order (-0 as +0)
__device__ __forceinline__ uint32_t order_bits(float v) {
    const uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_order_bits(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// exclusive prefix of v over the block's threads (in thread order); *total
// receives the block sum.  red: 4 floats of LDS.
__device__ __forceinline__ float block_exclusive(float v, float* red, float* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) red[wave] = x;
    __syncthreads();
    float pre = 0.f;
    for (int w = 0; w < wave; ++w) pre += red[w];
    *total = ((red[0] + red[1]) + red[2]) + red[3];
    __syncthreads();
    return pre + (x - v);
}

__device__ __forceinline__ int block_min(int v, int* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const int y = __shfl_xor(v, o, 64);
        v = y < v ? y : v;
    }
    if (lane == 0) red[wave] = v;
    __syncthreads();
    int m = red[0];
    for (int w = 1; w < kThreadsSm / 64; ++w) m = red[w] < m ? red[w] : m;
    __syncthreads();
    return m;
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), m, 64);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), m, 64);
    return (static_cast<unsigned long long>(hi) << 32) | lo;
}

// One bitonic compare-exchange step for element e holding a, partner value b:
// within blocks of size k the order is descending where (e & k) == 0 and
// ascending elsewhere; the lower position of the pair takes the element that
// comes first in that order.
__device__ __forceinline__ unsigned long long bitonic_keep(unsigned long long a, unsigned long long b, int e, int j, int k) {
    const bool want_larger = ((e & k) == 0) == ((e & j) == 0);
    return ((a > b) == want_larger) ? a : b;
}

// rows x V logits (row stride ld floats); uniforms u[row * u_stride];
// parameters from *pd when pd is non-null, else p; token of row r -> out[r].
// KPT keys per thread: V <= 256 * KPT.
template <int KPT>
__global__ __launch_bounds__(kThreadsSm) void k_sample(const float* __restrict__ logits, long long ld, int V,
                                                       Params p, const Params* pd, const float* __restrict__ u,
                                                       int u_stride, int* __restrict__ out) {
    constexpr int Vp = kThreadsSm * KPT;
    __shared__ unsigned long long key_s[Vp];
    __shared__ float redf[kThreadsSm / 64];
    __shared__ int redi[kThreadsSm / 64];
    __shared__ float s2_s;
    const int row = blockIdx.x, tid = threadIdx.x;
    const Params q = pd ? *pd : p;
    const float* z = logits + static_cast<long long>(row) * ld;
    // thread tid holds positions e = tid * KPT + r, r < KPT
    unsigned long long key[KPT];
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
        const int i = tid * KPT + r;
        key[r] = i < V ? (static_cast<unsigned long long>(order_bits(z[i])) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(i))
                       : 0ull;
    }
    // bitonic sort, descending: partners within a thread in registers,
    // within a wave by lane shuffles, across waves through LDS
#pragma unroll
    for (int k = 2; k <= Vp; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            if (j < KPT) {
#pragma unroll
                for (int r = 0; r < KPT; ++r) {
                    const int r2 = r ^ j;
                    if (r2 > r) {
                        const int e = tid * KPT + r;
                        const unsigned long long a = key[r], b = key[r2];
                        key[r] = bitonic_keep(a, b, e, j, k);
                        key[r2] = bitonic_keep(b, a, e + j, j, k);
                    }
                }
            } else if (j / KPT < 64) {
                const int m = j / KPT;
#pragma unroll
                for (int r = 0; r < KPT; ++r) {
                    const unsigned long long b = shfl_xor_u64(key[r], m);
                    key[r] = bitonic_keep(key[r], b, tid * KPT + r, j, k);
                }
            } else {
                __syncthreads();
#pragma unroll
                for (int r = 0; r < KPT; ++r) key_s[tid * KPT + r] = key[r];
                __syncthreads();
                const int t2 = tid ^ (j / KPT);
#pragma unroll
                for (int r = 0; r < KPT; ++r) key[r] = bitonic_keep(key[r], key_s[t2 * KPT + r], tid * KPT + r, j, k);
            }
        }
    }
    // rank tid * KPT + r is key[r]; the largest logit is rank 0's
    __syncthreads();
    if (tid == 0) key_s[0] = key[0];
    __syncthreads();
    const float z0 = from_order_bits(static_cast<uint32_t>(key_s[0] >> 32));
    const int r0 = tid * KPT;
    const int n1 = (q.top_k <= 0 || q.top_k >= V) ? V : q.top_k;
    float c[KPT];
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        float w = 0.f;
        if (r0 + i < n1) w = __expf((from_order_bits(static_cast<uint32_t>(key[i] >> 32)) - z0) / q.temperature);
        acc += w;
        c[i] = acc;
    }
    float s1;
    const float off = block_exclusive(acc, redf, &s1);
#pragma unroll
    for (int i = 0; i < KPT; ++i) c[i] += off;
    // top-p cut: n2 = 1 + first rank whose cumulative weight reaches P * s1
    int n2 = n1;
    if (q.top_p < 1.0f) {
        const float thr = q.top_p * s1;
        int first = 0x7FFFFFFF;
#pragma unroll
        for (int i = KPT - 1; i >= 0; --i)
            if (r0 + i < n1 && c[i] >= thr) first = r0 + i;
        first = block_min(first, redi);
        if (first != 0x7FFFFFFF) n2 = first + 1;
    }
    // kept total: the cumulative weight at rank n2 - 1
#pragma unroll
    for (int i = 0; i < KPT; ++i)
        if (r0 + i == n2 - 1) s2_s = c[i];
    __syncthreads();
    const float s2 = s2_s;
    float uu = u[static_cast<long long>(row) * u_stride];
    uu = uu != uu ? 0.f : fminf(fmaxf(uu, 0.f), 1.f);
    const float thr = uu * s2;
    int first = 0x7FFFFFFF;
#pragma unroll
    for (int i = KPT - 1; i >= 0; --i)
        if (r0 + i < n2 && c[i] > thr) first = r0 + i;
    first = block_min(first, redi);
    const int rank = first != 0x7FFFFFFF ? first : n2 - 1;
#pragma unroll
    for (int i = 0; i < KPT; ++i)
        if (r0 + i == rank) out[row] = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key[i] & 0xFFFFFFFFu));
}

// the instantiation for a vocabulary of V (V <= kMaxV)
using SampleFn = void (*)(const float*, long long, int, Params, const Params*, const float*, int, int*);
inline SampleFn sample_kernel(int V) {
    if (V <= 256) return k_sample<1>;
    if (V <= 512) return k_sample<2>;
    if (V <= 1024) return k_sample<4>;
    if (V <= 2048) return k_sample<8>;
    return k_sample<16>;
}

__global__ void k_set_params(Params p, Params* dst) {
    if (threadIdx.x == 0) *dst = p;
}

}  // namespace sample
}  // namespace qp

// top2.hip -- top-2 logit margin monitor.
//
// The precision study on the page arxiv-daily-jp 2609.26621 finds that output
// flips concentrate where the two best candidates are close, and that
// recomputing the head only for such steps is what helped.  Per row: the
// argmax (ties to the lowest index) and margin = top1 - top2, top2 being the
// largest logit at any other index (a tie gives 0), one fp32 subtraction;
// V == 1 gives +inf; a NaN gives id -1 and margin NaN.
//
// One row per 1024-thread workgroup (each thread with kUnroll independent
// loads in flight: a decoding step has few rows, so a row's scan is
// latency-bound).  A thread keeps (top1 value, its index,
// top2 value); two such triples merge as: top1 = the better of the two top1s
// (larger value, equal values keep the lower index), top2 = the largest of the
// other top1 and both top2s.  Every piece is a maximum or a total-order choice,
// so the merge order does not change the result.
#include "bi_common.hpp"

namespace {

constexpr int kThreads = 1024;
constexpr int kUnroll = 8;

struct Top2 {
    float v1;
    int i1;
    float v2;
};

__device__ __forceinline__ Top2 merge(Top2 a, Top2 b)
{
    if (b.i1 < 0) return a;
    if (a.i1 < 0) return b;
    const bool b_wins = b.v1 > a.v1 || (b.v1 == a.v1 && b.i1 < a.i1);
    Top2 r;
    r.v1 = b_wins ? b.v1 : a.v1;
    r.i1 = b_wins ? b.i1 : a.i1;
    r.v2 = fmaxf(fmaxf(a.v2, b.v2), b_wins ? a.v1 : b.v1);
    return r;
}

__global__ __launch_bounds__(kThreads) void top2_kernel(const float* __restrict__ x, int64_t ld, int V,
                                                        int32_t* __restrict__ ids, float* __restrict__ margin)
{
    __shared__ float s_v1[kThreads / 64], s_v2[kThreads / 64];
    __shared__ int s_i1[kThreads / 64], s_nan[kThreads / 64];
    const int t = threadIdx.x;
    const float* row = x + (int64_t)blockIdx.x * ld;
    Top2 a{-INFINITY, -1, -INFINITY};
    int nan = 0;
    for (int64_t i0 = t; i0 < V; i0 += (int64_t)kThreads * kUnroll) {
        float v[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t i = i0 + (int64_t)k * kThreads;
            v[k] = i < V ? row[i] : 0.0f;
        }
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t i = i0 + (int64_t)k * kThreads;
            if (i < V) {
                if (v[k] != v[k]) nan = 1;
                else a = merge(a, Top2{v[k], (int)i, -INFINITY});
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        Top2 b;
        b.v1 = __shfl_xor(a.v1, off, 64);
        b.i1 = __shfl_xor(a.i1, off, 64);
        b.v2 = __shfl_xor(a.v2, off, 64);
        nan |= __shfl_xor(nan, off, 64);
        a = merge(a, b);
    }
    const int w = t >> 6;
    if ((t & 63) == 0) {
        s_v1[w] = a.v1;
        s_i1[w] = a.i1;
        s_v2[w] = a.v2;
        s_nan[w] = nan;
    }
    __syncthreads();
    if (t == 0) {
        a = Top2{s_v1[0], s_i1[0], s_v2[0]};
        nan = s_nan[0];
        for (int k = 1; k < kThreads / 64; ++k) {
            a = merge(a, Top2{s_v1[k], s_i1[k], s_v2[k]});
            nan |= s_nan[k];
        }
        ids[blockIdx.x] = nan ? -1 : a.i1;
        margin[blockIdx.x] = nan ? __builtin_nanf("") : (V == 1 ? INFINITY : a.v1 - a.v2);
    }
}

}  // namespace

extern "C" int bi_top2(const float* logits, int64_t ld, int64_t rows, int64_t V, int32_t* ids, float* margin,
                       void* stream)
{
    BI_TRY_BEGIN
    if (rows < 0 || V <= 0 || ld < V) return BI_ERR_INVALID_ARGUMENT;
    if (rows > 0 && (!logits || !ids || !margin || !bi_aligned(logits, 4) || !bi_aligned(ids, 4) ||
                     !bi_aligned(margin, 4)))
        return BI_ERR_INVALID_ARGUMENT;
    if (rows > 0x7fffffffLL || V > 0x7fffffffLL - kThreads) return BI_ERR_UNSUPPORTED;
    if (rows == 0) return BI_OK;
    hipLaunchKernelGGL(top2_kernel, dim3((unsigned)rows), dim3(kThreads), 0, (hipStream_t)stream, logits, ld,
                       (int)V, ids, margin);
    return bi_launch_status();
    BI_TRY_END
}

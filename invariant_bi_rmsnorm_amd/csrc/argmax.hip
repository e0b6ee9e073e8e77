// argmax.hip -- greedy token choice.
//
// Temperature 0 means taking the argmax at every step (page "la température
// zéro n'est pas déterministe", section "Le mensonge de la température zéro").
// One workgroup per row.  (value, index) pairs combine by "larger value wins,
// equal values keep the lower index", an associative and commutative rule, so
// the chosen index never depends on the reduction order; a NaN anywhere gives -1.
// 1024 threads per row, each with kUnroll independent loads in flight (a
// decoding step has few rows, so each row's scan is latency-bound).
#include "bi_common.hpp"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 8;

__device__ __forceinline__ void better(float& v, int& i, float v2, int i2)
{
    if (i2 >= 0 && (i < 0 || v2 > v || (v2 == v && i2 < i))) { v = v2; i = i2; }
}

__global__ __launch_bounds__(kThreads) void argmax_kernel(const float* __restrict__ x, int64_t ld,
                                                          int64_t V, int32_t* __restrict__ ids)
{
    __shared__ float s_v[kWaves];
    __shared__ int s_i[kWaves];
    __shared__ int s_nan[kWaves];
    const int64_t r = blockIdx.x;
    const float* row = x + r * ld;
    float bv = 0.0f;
    int bi = -1;
    int nan = 0;
    // this thread's entries in increasing index order (a strict > keeps the
    // lowest index among its equal values)
    for (int64_t j0 = threadIdx.x; j0 < V; j0 += (int64_t)kThreads * kUnroll) {
        float v[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t j = j0 + (int64_t)k * kThreads;
            v[k] = j < V ? row[j] : 0.0f;
        }
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int64_t j = j0 + (int64_t)k * kThreads;
            if (j < V) {
                if (v[k] != v[k]) nan = 1;
                else if (bi < 0 || v[k] > bv) { bv = v[k]; bi = (int)j; }
            }
        }
    }
    for (int off = 32; off >= 1; off >>= 1) {
        const float v2 = __shfl_xor(bv, off, 64);
        const int i2 = __shfl_xor(bi, off, 64);
        nan |= __shfl_xor(nan, off, 64);
        better(bv, bi, v2, i2);
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { s_v[w] = bv; s_i[w] = bi; s_nan[w] = nan; }
    __syncthreads();
    if (threadIdx.x == 0) {
        float v = s_v[0];
        int i = s_i[0];
        int n = s_nan[0];
        for (int k = 1; k < kWaves; ++k) { better(v, i, s_v[k], s_i[k]); n |= s_nan[k]; }
        ids[r] = n ? -1 : i;
    }
}

}  // namespace

extern "C" int bi_argmax(const float* logits, int64_t ld, int64_t rows, int64_t V, int32_t* ids,
                         void* stream)
{
    BI_TRY_BEGIN
    if (rows < 0 || V <= 0 || ld < V) return BI_ERR_INVALID_ARGUMENT;
    if (rows > 0 && (!logits || !ids)) return BI_ERR_INVALID_ARGUMENT;
    if (rows > 0 && (!bi_aligned(logits, 4) || !bi_aligned(ids, 4))) return BI_ERR_INVALID_ARGUMENT;
    if (V > 0x7fffffffLL || rows > 0x7fffffffLL) return BI_ERR_UNSUPPORTED;
    if (rows == 0) return BI_OK;
    hipLaunchKernelGGL(argmax_kernel, dim3((unsigned)rows), dim3(kThreads), 0, (hipStream_t)stream,
                       logits, ld, V, ids);
    return bi_launch_status();
    BI_TRY_END
}

// log_softmax.hip -- batch-invariant log_softmax over the last dimension.
//
// The post "論文／ブログ「Defeating Nondeterminism in LLM Inference」の技術的な
// ポイント" (mobiles-han.blogspot.com), section 他の演算子（RMSNorm, MatMul,
// mean/reduction etc.）, names log_softmax among the reductions the invariant
// library replaces, and asks that such reductions keep one order whatever the
// batch.  y_i = x_i - m - log(sum_j exp(x_j - m)), m = max_j x_j, fp32 in and
// out.
//
// One row per 512-thread workgroup, the same design as the RMSNorm kernel.
// The row maximum is exact (any order gives the same value).  The sum has one
// order that depends only on V: thread t adds exp(x_i - m) for i = t, t + 512,
// t + 1024, ... ascending; a xor butterfly 32, 16, ..., 1 inside each
// wavefront; the 8 wavefront sums as ((w0+w1)+(w2+w3))+((w4+w5)+(w6+w7)).
// exp and log are the hardware v_exp_f32 / v_log_f32 on base-2 arguments.
// Rows of up to 32768 entries are held in registers between the passes;
// longer rows are read again, visiting the entries in the same order, so the
// two paths give the same bits.  NaN anywhere in a row gives a NaN row; a row
// whose maximum is -inf or +inf gives NaN where the formula does.
#include "bi_common.hpp"

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kReg = 64;                               // cached entries per thread
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }

template <bool kCached>
__global__ __launch_bounds__(kThreads) void log_softmax_kernel(const float* x, int64_t ldx, float* y,
                                                               int64_t ldy, int V)
{
    __shared__ float s_max[kWaves];
    __shared__ float s_sum[kWaves];
    __shared__ int s_nan[kWaves];
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const float* xr = x + (int64_t)blockIdx.x * ldx;
    float* yr = y + (int64_t)blockIdx.x * ldy;

    float v[kCached ? kReg : 1];
    float m = -INFINITY;
    int nan = 0;
    if constexpr (kCached) {
#pragma unroll
        for (int k = 0; k < kReg; ++k) {
            const int i = t + k * kThreads;
            v[k] = i < V ? xr[i] : -INFINITY;
        }
#pragma unroll
        for (int k = 0; k < kReg; ++k) {
            m = fmaxf(m, v[k]);
            nan |= v[k] != v[k];
        }
    } else {
        for (int i = t; i < V; i += kThreads) {
            const float a = xr[i];
            m = fmaxf(m, a);
            nan |= a != a;
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        m = fmaxf(m, __shfl_xor(m, off, 64));
        nan |= __shfl_xor(nan, off, 64);
    }
    if (lane == 0) {
        s_max[wave] = m;
        s_nan[wave] = nan;
    }
    __syncthreads();
    m = s_max[0];
    nan = s_nan[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
        m = fmaxf(m, s_max[w]);
        nan |= s_nan[w];
    }

    float s = 0.0f;
    if constexpr (kCached) {
        // entries past V hold -inf: they add exp2(-inf) = +0, which leaves s unchanged
#pragma unroll
        for (int k = 0; k < kReg; ++k) s = s + hw_exp2((v[k] - m) * kLog2e);
    } else {
        for (int i = t; i < V; i += kThreads) s = s + hw_exp2((xr[i] - m) * kLog2e);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s = s + __shfl_xor(s, off, 64);
    if (lane == 0) s_sum[wave] = s;
    __syncthreads();
    const float total = ((s_sum[0] + s_sum[1]) + (s_sum[2] + s_sum[3])) +
                        ((s_sum[4] + s_sum[5]) + (s_sum[6] + s_sum[7]));
    const float lse = nan ? __builtin_nanf("") : m + hw_log2(total) * kLn2;

    if constexpr (kCached) {
#pragma unroll
        for (int k = 0; k < kReg; ++k) {
            const int i = t + k * kThreads;
            if (i < V) yr[i] = v[k] - lse;
        }
    } else {
        for (int i = t; i < V; i += kThreads) yr[i] = xr[i] - lse;
    }
}

}  // namespace

extern "C" int bi_log_softmax(const float* x, int64_t ldx, float* y, int64_t ldy, int64_t rows, int64_t V,
                              void* stream)
{
    BI_TRY_BEGIN
    if (rows < 0 || V <= 0 || ldx < V || ldy < V) return BI_ERR_INVALID_ARGUMENT;
    if (rows > 0 && (!x || !y || !bi_aligned(x, 4) || !bi_aligned(y, 4))) return BI_ERR_INVALID_ARGUMENT;
    if (x == y && ldx != ldy) return BI_ERR_INVALID_ARGUMENT;
    if (rows > 0x7fffffffLL || V > 0x7fffffffLL - kThreads) return BI_ERR_UNSUPPORTED;
    if (rows == 0) return BI_OK;
    if (V <= (int64_t)kThreads * kReg)
        hipLaunchKernelGGL(log_softmax_kernel<true>, dim3((unsigned)rows), dim3(kThreads), 0,
                           (hipStream_t)stream, x, ldx, y, ldy, (int)V);
    else
        hipLaunchKernelGGL(log_softmax_kernel<false>, dim3((unsigned)rows), dim3(kThreads), 0,
                           (hipStream_t)stream, x, ldx, y, ldy, (int)V);
    return bi_launch_status();
    BI_TRY_END
}

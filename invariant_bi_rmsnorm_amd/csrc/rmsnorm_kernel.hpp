// rmsnorm_kernel.hpp -- the RMSNorm kernel (see rmsnorm.hip for the design and
// the invariance argument).  kOrder 0 is the library's fixed reduction order,
// the only one bi_rmsnorm in libbi.so uses; kOrder 1 (chunks reversed, waves
// combined as (w0+w3)+(w1+w2)) exists only for the non-invariant baseline.
#pragma once
#include "bi_common.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxChunks = 8;                 // per thread: H <= 256 * 8 * 8 = 16384

template <int kOrder>
__global__ __launch_bounds__(kThreads) void rmsnorm_kernel(
    const uint16_t* x, int64_t ldx, const uint16_t* __restrict__ w,
    uint16_t* y, int64_t ldy, float* __restrict__ rstd, int H, float eps)
{
    __shared__ float wave_sum[4];
    const int64_t m = blockIdx.x;
    const int tid = threadIdx.x;
    const int nch = H >> 3;
    const uint16_t* xr = x + m * ldx;

    u32x4 xv[kMaxChunks];
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
        const int ch = tid + c * kThreads;
        xv[c] = zero_u32x4();
        if (ch < nch) xv[c] = ld16(xr + (int64_t)ch * 8);
    }
#pragma unroll
    for (int cc = 0; cc < kMaxChunks; ++cc) {
        const int c = kOrder == 1 ? kMaxChunks - 1 - cc : cc;     // order 1: chunks reversed
        const int ch = tid + c * kThreads;
        if (ch < nch) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float lo = bf16_to_f32(xv[c][e] & 0xffffu);
                const float hi = bf16_to_f32(xv[c][e] >> 16);
                acc = __fmaf_rn(lo, lo, acc);
                acc = __fmaf_rn(hi, hi, acc);
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc = acc + __shfl_xor(acc, off, 64);
    if ((tid & 63) == 0) wave_sum[tid >> 6] = acc;
    __syncthreads();
    const float total = kOrder == 1 ? (wave_sum[0] + wave_sum[3]) + (wave_sum[1] + wave_sum[2])
                                    : (wave_sum[0] + wave_sum[1]) + (wave_sum[2] + wave_sum[3]);
    const float ms = total / (float)H;
    const float r = 1.0f / sqrtf(ms + eps);
    if (tid == 0 && rstd) rstd[m] = r;

    uint16_t* yr = y + m * ldy;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
        const int ch = tid + c * kThreads;
        if (ch < nch) {
            const u32x4 wv = ld16(w + (int64_t)ch * 8);
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x0 = bf16_to_f32(xv[c][e] & 0xffffu);
                const float x1 = bf16_to_f32(xv[c][e] >> 16);
                const float w0 = bf16_to_f32(wv[e] & 0xffffu);
                const float w1 = bf16_to_f32(wv[e] >> 16);
                o[e] = pack_bf16x2((x0 * r) * w0, (x1 * r) * w1);
            }
            st16(yr + (int64_t)ch * 8, o);
        }
    }
}

static inline int rmsnorm_validate(const void* x, int64_t ldx, const void* w, const void* y, int64_t ldy,
                                   const float* rstd, int64_t M, int64_t H, float eps)
{
    if (M < 0 || H <= 0) return BI_ERR_INVALID_ARGUMENT;
    if (M > 0 && (!x || !w || !y)) return BI_ERR_INVALID_ARGUMENT;
    if (ldx < H || ldy < H) return BI_ERR_INVALID_ARGUMENT;
    if (!(eps >= 0.0f) || eps != eps) return BI_ERR_INVALID_ARGUMENT;
    if (M > 0 && (!bi_aligned(x, 16) || !bi_aligned(w, 16) || !bi_aligned(y, 16) ||
                  (rstd && !bi_aligned(rstd, 4))))
        return BI_ERR_INVALID_ARGUMENT;
    if ((ldx % 8) || (ldy % 8)) return BI_ERR_INVALID_ARGUMENT;
    if ((H % 8) || H > (int64_t)kThreads * kMaxChunks * 8) return BI_ERR_UNSUPPORTED;
    if (x == y && ldx != ldy) return BI_ERR_INVALID_ARGUMENT;
    if (M > 0x7fffffffLL) return BI_ERR_UNSUPPORTED;
    if (M == 0) return -1;
    return BI_OK;
}

template <int kOrder>
static inline int rmsnorm_launch(const void* x, int64_t ldx, const void* w, void* y, int64_t ldy,
                                 float* rstd, int64_t M, int64_t H, float eps, void* stream)
{
    hipLaunchKernelGGL(rmsnorm_kernel<kOrder>, dim3((unsigned)M), dim3(kThreads), 0, (hipStream_t)stream,
                       (const uint16_t*)x, ldx, (const uint16_t*)w, (uint16_t*)y, ldy, rstd,
                       (int)H, eps);
    return bi_launch_status();
}

}  // namespace

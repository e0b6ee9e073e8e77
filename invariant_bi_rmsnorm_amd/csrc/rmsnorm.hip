// rmsnorm.hip -- batch-invariant RMSNorm: one row per workgroup.
//
// Table row "RMSNorm" of the post "論文／ブログ「Defeating Nondeterminism in LLM
// Inference」の技術的なポイント" (mobiles-han.blogspot.com), section
// 対応策：バッチ不変なカーネル設計: standard kernels split a row's reduction over
// several cores when the batch is small, which changes the order; the fix is a
// data-parallel strategy whose per-row order never depends on the batch.
//
// Here: grid = M workgroups of 256 threads (4 wavefronts of 64), one row each.
// The reduction order of row m depends only on H:
//   1. thread t owns 8-element chunks t, t+256, t+512, ... (ascending) and
//      accumulates x*x for the 8 elements of each chunk in order with fmaf;
//   2. xor butterfly across the 64 lanes of a wave, offsets 32,16,8,4,2,1
//      (both partners compute a+b, which is commutative, so every lane ends
//      with the same bits);
//   3. the four wave sums are combined as (w0 + w1) + (w2 + w3).
// Nothing depends on M or on blockIdx; no atomics.  The row is read once into
// registers and reused for the output (4 B of HBM traffic per element).
#include "bi_common.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxChunks = 8;                 // per thread: H <= 256 * 8 * 8 = 16384

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
    for (int c = 0; c < kMaxChunks; ++c) {
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
    const float total = (wave_sum[0] + wave_sum[1]) + (wave_sum[2] + wave_sum[3]);
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

}  // namespace

extern "C" int bi_rmsnorm(const void* x, int64_t ldx, const void* w, void* y, int64_t ldy,
                          float* rstd, int64_t M, int64_t H, float eps, void* stream)
{
    BI_TRY_BEGIN
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
    if (M == 0) return BI_OK;
    hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)M), dim3(kThreads), 0, (hipStream_t)stream,
                       (const uint16_t*)x, ldx, (const uint16_t*)w, (uint16_t*)y, ldy, rstd,
                       (int)H, eps);
    return bi_launch_status();
    BI_TRY_END
}

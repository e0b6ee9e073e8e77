// rmsnorm_kernel.hpp -- the RMSNorm kernel (see rmsnorm.hip for the design and
// the invariance argument).  kOrder 0 is the library's fixed reduction order,
// the only one bi_rmsnorm in libbi.so uses; kOrder 1 (chunks reversed, waves
// combined as (w0+w3)+(w1+w2)) exists only for the non-invariant baseline.
#pragma once
#include "bi_common.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxChunks = 8;                 // per thread: H <= 256 * 8 * 8 = 16384

// kChunks: 16-byte chunks per thread the launch provides registers for
// (H <= 2048 kChunks); the chunks past H are skipped, so every kChunks gives
// the same bits for a given H.  kAdd: the row normalised is bf16(x + r), each
// element rounded as bi_add rounds it, and that sum is also stored to hsum
// (which may be x itself: each thread rewrites only the chunks it read).
template <int kOrder, int kChunks, bool kAdd = false>
__global__ __launch_bounds__(kThreads) void rmsnorm_kernel(
    const uint16_t* x, int64_t ldx, const uint16_t* __restrict__ w,
    uint16_t* y, int64_t ldy, float* __restrict__ rstd, int H, float eps,
    const uint16_t* r_add, int64_t ldr, uint16_t* hsum, int64_t ldh)
{
    __shared__ float wave_sum[4];
    const int64_t m = blockIdx.x;
    const int tid = threadIdx.x;
    const int nch = H >> 3;
    const uint16_t* xr = x + m * ldx;

    // the row and the weights are loaded together, so the weights need no
    // second memory round trip after the reduction
    u32x4 xv[kChunks], wv[kChunks];
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        const int ch = tid + c * kThreads;
        xv[c] = zero_u32x4();
        wv[c] = zero_u32x4();
        if (ch < nch) {
            xv[c] = ld16(xr + (int64_t)ch * 8);
            wv[c] = ld16(w + (int64_t)ch * 8);
        }
    }
    if constexpr (kAdd) {
        u32x4 rv[kChunks];
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            const int ch = tid + c * kThreads;
            rv[c] = ch < nch ? ld16(r_add + m * ldr + (int64_t)ch * 8) : zero_u32x4();
        }
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            const int ch = tid + c * kThreads;
            if (ch < nch) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    xv[c][e] = pack_bf16x2(bf16_to_f32(xv[c][e] & 0xffffu) + bf16_to_f32(rv[c][e] & 0xffffu),
                                           bf16_to_f32(xv[c][e] >> 16) + bf16_to_f32(rv[c][e] >> 16));
                st16(hsum + m * ldh + (int64_t)ch * 8, xv[c]);
            }
        }
    }
#pragma unroll
    for (int cc = 0; cc < kChunks; ++cc) {
        const int c = kOrder == 1 ? kChunks - 1 - cc : cc;        // order 1: chunks reversed
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
    for (int c = 0; c < kChunks; ++c) {
        const int ch = tid + c * kThreads;
        if (ch < nch) {
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x0 = bf16_to_f32(xv[c][e] & 0xffffu);
                const float x1 = bf16_to_f32(xv[c][e] >> 16);
                const float w0 = bf16_to_f32(wv[c][e] & 0xffffu);
                const float w1 = bf16_to_f32(wv[c][e] >> 16);
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

// kAdd launches normalise bf16(x + r) and store that sum to h (see the kernel)
template <int kOrder, bool kAdd = false>
static inline int rmsnorm_launch(const void* x, int64_t ldx, const void* w, void* y, int64_t ldy,
                                 float* rstd, int64_t M, int64_t H, float eps, void* stream,
                                 const void* r = nullptr, int64_t ldr = 0, void* h = nullptr, int64_t ldh = 0)
{
    const dim3 grid((unsigned)M), block(kThreads);
    const hipStream_t st = (hipStream_t)stream;
    if (H <= 2 * kThreads * 8)
        hipLaunchKernelGGL((rmsnorm_kernel<kOrder, 2, kAdd>), grid, block, 0, st, (const uint16_t*)x, ldx,
                           (const uint16_t*)w, (uint16_t*)y, ldy, rstd, (int)H, eps, (const uint16_t*)r, ldr,
                           (uint16_t*)h, ldh);
    else if (H <= 4 * kThreads * 8)
        hipLaunchKernelGGL((rmsnorm_kernel<kOrder, 4, kAdd>), grid, block, 0, st, (const uint16_t*)x, ldx,
                           (const uint16_t*)w, (uint16_t*)y, ldy, rstd, (int)H, eps, (const uint16_t*)r, ldr,
                           (uint16_t*)h, ldh);
    else
        hipLaunchKernelGGL((rmsnorm_kernel<kOrder, kMaxChunks, kAdd>), grid, block, 0, st, (const uint16_t*)x, ldx,
                           (const uint16_t*)w, (uint16_t*)y, ldy, rstd, (int)H, eps, (const uint16_t*)r, ldr,
                           (uint16_t*)h, ldh);
    return bi_launch_status();
}

// bi_add_rmsnorm's checks beyond bi_rmsnorm's: r like x, and y distinct from h
// (the sum is the residual the caller keeps)
static inline int add_rmsnorm_validate(const void* h, int64_t ldh, const void* r, int64_t ldr, const void* w,
                                       const void* y, int64_t ldy, const float* rstd, int64_t M, int64_t H,
                                       float eps)
{
    const int v = rmsnorm_validate(h, ldh, w, y, ldy, rstd, M, H, eps);
    if (v != BI_OK && v != -1) return v;
    if (ldr < H || (ldr % 8)) return BI_ERR_INVALID_ARGUMENT;
    if (M > 0 && (!r || !bi_aligned(r, 16) || y == h)) return BI_ERR_INVALID_ARGUMENT;
    return v;
}

}  // namespace

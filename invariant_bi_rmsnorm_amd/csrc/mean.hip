// mean.hip -- batch-invariant mean over the last dimension.
//
// The post "論文／ブログ「Defeating Nondeterminism in LLM Inference」の技術的な
// ポイント" (mobiles-han.blogspot.com), section 他の演算子（RMSNorm, MatMul,
// mean/reduction etc.）, names torch.mean among the reductions whose order
// must not follow the batch.  out[r] = (1/H) sum_j x[r][j], bf16 in, fp32 out.
//
// The RMSNorm kernel's design with the squares left out: one row per
// 256-thread workgroup; thread t adds the 8 values of each of its 16-byte
// chunks t, t + 256, ... in order; a xor butterfly 32, 16, ..., 1 inside the
// wavefront; the four wavefront sums as (w0 + w1) + (w2 + w3); one division
// by H.  The order depends only on H.
#include "bi_common.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxChunks = 8;                 // H <= 256 * 8 * 8 = 16384

__global__ __launch_bounds__(kThreads) void mean_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                        float* __restrict__ out, int H)
{
    __shared__ float wave_sum[4];
    const int tid = threadIdx.x;
    const int nch = H >> 3;
    const uint16_t* xr = x + (int64_t)blockIdx.x * ldx;
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
        const int ch = tid + c * kThreads;
        if (ch < nch) {
            const u32x4 v = ld16(xr + (int64_t)ch * 8);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc = acc + bf16_to_f32(v[e] & 0xffffu);
                acc = acc + bf16_to_f32(v[e] >> 16);
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc = acc + __shfl_xor(acc, off, 64);
    if ((tid & 63) == 0) wave_sum[tid >> 6] = acc;
    __syncthreads();
    if (tid == 0) out[blockIdx.x] = ((wave_sum[0] + wave_sum[1]) + (wave_sum[2] + wave_sum[3])) / (float)H;
}

}  // namespace

extern "C" int bi_mean(const void* x, int64_t ldx, float* out, int64_t rows, int64_t H, void* stream)
{
    BI_TRY_BEGIN
    if (rows < 0 || H <= 0 || ldx < H) return BI_ERR_INVALID_ARGUMENT;
    if (rows > 0 && (!x || !out || !bi_aligned(x, 16) || !bi_aligned(out, 4))) return BI_ERR_INVALID_ARGUMENT;
    if (ldx % 8) return BI_ERR_INVALID_ARGUMENT;
    if ((H % 8) || H > (int64_t)kThreads * kMaxChunks * 8 || rows > 0x7fffffffLL) return BI_ERR_UNSUPPORTED;
    if (rows == 0) return BI_OK;
    hipLaunchKernelGGL(mean_kernel, dim3((unsigned)rows), dim3(kThreads), 0, (hipStream_t)stream,
                       (const uint16_t*)x, ldx, out, (int)H);
    return bi_launch_status();
    BI_TRY_END
}

// lm_head_f32.hip -- the output head in fp32, for the rows whose top-2 margin
// is small.
//
// Page arxiv-daily-jp.pages.dev/paper/2609.26621 (abstract): greedy outputs
// flip between numeric paths where the top-2 logit margin at the LM head is
// small against the perturbation between the two candidates, and recomputing
// the head in FP32 only for those steps was the best low-cost intervention.
// The bf16 path here rounds the normalised hidden state to bf16 before the LM
// head GEMM (bi_rmsnorm, then bi_matmul with fp32 output).  This kernel
// computes the head from the unrounded state:
//     rstd      = the rstd bi_rmsnorm computes for the row (same order, same bits)
//     y_j       = (h_j * rstd) * w_j   in fp32, not rounded
//     out[r][v] = sum_j y_j * W[v][j]
// The sum has one order, whatever R, V or the row's place: lane l of a
// wavefront takes j = 512 c + 8 l + e for c = 0, 1, ... and e = 0..7 in that
// order, accumulating with fmaf from 0, and the 64 lane sums are combined by
// the xor butterfly 32, 16, ..., 1 (a + b and b + a round alike, so every lane
// ends with the same value).  A workgroup is 4 wavefronts over 64 vocabulary
// rows of one hidden row; y stays in registers, W is streamed once per row.
#include "bi_common.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kVPerWG = 64;                   // vocabulary rows per workgroup, 16 per wavefront
constexpr int kMaxH = 4096;                   // y in registers: H / 512 chunks of 8 per lane
constexpr int kRmsChunks = 8;                 // the RMSNorm kernel's per-thread chunk bound

template <int NC>
__global__ __launch_bounds__(kThreads) void lm_head_f32_kernel(
    const uint16_t* __restrict__ h, int64_t ldh, const uint16_t* __restrict__ w, float eps,
    const uint16_t* __restrict__ wt, int64_t ldw, float* __restrict__ out, int64_t ldo, int V,
    const float* __restrict__ margin, float threshold)
{
    constexpr int H = NC * 512;
    __shared__ float wave_sum[4];
    const int r = blockIdx.y;
    if (margin && margin[r] >= threshold) return;              // uniform: a NaN margin is recomputed
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const uint16_t* hr = h + (int64_t)r * ldh;

    // ---- rstd, exactly as the RMSNorm kernel forms it
    constexpr int nch = H >> 3;
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < kRmsChunks; ++c) {
        const int ch = tid + c * kThreads;
        if (ch < nch) {
            const u32x4 xv = ld16(hr + (int64_t)ch * 8);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float lo = bf16_to_f32(xv[e] & 0xffffu);
                const float hi = bf16_to_f32(xv[e] >> 16);
                acc = __fmaf_rn(lo, lo, acc);
                acc = __fmaf_rn(hi, hi, acc);
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc = acc + __shfl_xor(acc, off, 64);
    if (lane == 0) wave_sum[wave] = acc;
    __syncthreads();
    const float total = (wave_sum[0] + wave_sum[1]) + (wave_sum[2] + wave_sum[3]);
    const float ms = total / (float)H;
    const float rs = 1.0f / sqrtf(ms + eps);

    // ---- this lane's y_j, j = 512 c + 8 lane + e
    float y[NC][8];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const u32x4 xv = ld16(hr + 512 * c + 8 * lane);
        const u32x4 wv = ld16(w + 512 * c + 8 * lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            y[c][2 * e] = (bf16_to_f32(xv[e] & 0xffffu) * rs) * bf16_to_f32(wv[e] & 0xffffu);
            y[c][2 * e + 1] = (bf16_to_f32(xv[e] >> 16) * rs) * bf16_to_f32(wv[e] >> 16);
        }
    }

    // ---- 16 vocabulary rows per wavefront, 4 in flight
    const int v0 = blockIdx.x * kVPerWG + wave * (kVPerWG / 4);
    float* orow = out + (int64_t)r * ldo;
#pragma unroll 1
    for (int i0 = 0; i0 < kVPerWG / 4; i0 += 4) {
        u32x4 wv[4][NC];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int v = v0 + i0 + k;
#pragma unroll
            for (int c = 0; c < NC; ++c)
                wv[k][c] = v < V ? ld16(wt + (int64_t)v * ldw + 512 * c + 8 * lane) : zero_u32x4();
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float s = 0.0f;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    s = __fmaf_rn(y[c][2 * e], bf16_to_f32(wv[k][c][e] & 0xffffu), s);
                    s = __fmaf_rn(y[c][2 * e + 1], bf16_to_f32(wv[k][c][e] >> 16), s);
                }
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) s = s + __shfl_xor(s, off, 64);
            const int v = v0 + i0 + k;
            if (lane == 0 && v < V) orow[v] = s;
        }
    }
}

template <int NC>
void launch(const void* h, int64_t ldh, const void* w, float eps, const void* wt, int64_t ldw, float* out,
            int64_t ldo, int64_t R, int64_t V, const float* margin, float threshold, hipStream_t st)
{
    const dim3 grid((unsigned)((V + kVPerWG - 1) / kVPerWG), (unsigned)R);
    hipLaunchKernelGGL(lm_head_f32_kernel<NC>, grid, dim3(kThreads), 0, st, (const uint16_t*)h, ldh,
                       (const uint16_t*)w, eps, (const uint16_t*)wt, ldw, out, ldo, (int)V, margin, threshold);
}

}  // namespace

extern "C" int bi_lm_head_f32(const void* h, int64_t ldh, const void* norm_w, float eps, const void* lm_head,
                              int64_t ldw, float* out, int64_t ldo, int64_t R, int64_t V, int64_t H,
                              const float* margin, float threshold, void* stream)
{
    BI_TRY_BEGIN
    if (R < 0 || V <= 0 || H <= 0) return BI_ERR_INVALID_ARGUMENT;
    if (ldh < H || ldw < H || ldo < V || (ldh % 8) || (ldw % 8)) return BI_ERR_INVALID_ARGUMENT;
    if (!(eps >= 0.0f) || eps > 3.0e38f || threshold != threshold) return BI_ERR_INVALID_ARGUMENT;
    if (R > 0 && (!h || !norm_w || !lm_head || !out || !bi_aligned(h, 16) || !bi_aligned(norm_w, 16) ||
                  !bi_aligned(lm_head, 16) || !bi_aligned(out, 4) || (margin && !bi_aligned(margin, 4))))
        return BI_ERR_INVALID_ARGUMENT;
    if ((H % 512) || H > kMaxH || R > 65535 || V > 0x7fffffffLL - kVPerWG) return BI_ERR_UNSUPPORTED;
    if (R == 0) return BI_OK;
    const hipStream_t st = (hipStream_t)stream;
    switch (H / 512) {
        case 1: launch<1>(h, ldh, norm_w, eps, lm_head, ldw, out, ldo, R, V, margin, threshold, st); break;
        case 2: launch<2>(h, ldh, norm_w, eps, lm_head, ldw, out, ldo, R, V, margin, threshold, st); break;
        case 3: launch<3>(h, ldh, norm_w, eps, lm_head, ldw, out, ldo, R, V, margin, threshold, st); break;
        case 4: launch<4>(h, ldh, norm_w, eps, lm_head, ldw, out, ldo, R, V, margin, threshold, st); break;
        case 5: launch<5>(h, ldh, norm_w, eps, lm_head, ldw, out, ldo, R, V, margin, threshold, st); break;
        case 6: launch<6>(h, ldh, norm_w, eps, lm_head, ldw, out, ldo, R, V, margin, threshold, st); break;
        case 7: launch<7>(h, ldh, norm_w, eps, lm_head, ldw, out, ldo, R, V, margin, threshold, st); break;
        default: launch<8>(h, ldh, norm_w, eps, lm_head, ldw, out, ldo, R, V, margin, threshold, st); break;
    }
    return bi_launch_status();
    BI_TRY_END
}

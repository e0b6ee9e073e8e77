// misc.hip -- version, status strings and the MFMA layout probe.
#include "bi_common.hpp"

namespace {

// One wavefront: load a (16x32, row-major) and b (32x16, row-major) into the
// operand layout every kernel of the library assumes, run one MFMA, write c.
__global__ __launch_bounds__(64) void probe_kernel(const uint16_t* __restrict__ a,
                                                   const uint16_t* __restrict__ b,
                                                   float* __restrict__ c)
{
    const int l = threadIdx.x;
    const int col = l & 15;
    const int grp = l >> 4;
    const u32x4 av = ld16(a + col * 32 + 8 * grp);
    u32x4 bv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t lo = b[(8 * grp + 2 * e) * 16 + col];
        const uint32_t hi = b[(8 * grp + 2 * e + 1) * 16 + col];
        bv[e] = lo | (hi << 16);
    }
    const f32x4 acc = mfma16(as_bf16x8(av), as_bf16x8(bv), f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int r = 0; r < 4; ++r) c[(4 * grp + r) * 16 + col] = acc[r];
}

// Plain streaming copy, 16 bytes per lane per access, grid-stride: the
// reference for achievable HBM bandwidth and for scaling memory counters.
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        dst[i] = a;
        dst[i + stride] = b;
        dst[i + 2 * stride] = c;
        dst[i + 3 * stride] = d;
    }
    for (; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" int bi_abi_version(void) { return BI_ABI_VERSION; }

extern "C" const char* bi_status_string(int status)
{
    switch (status) {
        case BI_OK: return "ok";
        case BI_ERR_INVALID_ARGUMENT: return "invalid argument";
        case BI_ERR_UNSUPPORTED: return "unsupported shape or configuration";
        case BI_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case BI_ERR_NO_DEVICE: return "no device";
        case BI_ERR_LAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

extern "C" int bi_probe_mfma_bf16(const void* a, const void* b, float* c, void* stream)
{
    BI_TRY_BEGIN
    if (!a || !b || !c) return BI_ERR_INVALID_ARGUMENT;
    if (!bi_aligned(a, 16) || !bi_aligned(b, 2) || !bi_aligned(c, 4)) return BI_ERR_INVALID_ARGUMENT;
    hipLaunchKernelGGL(probe_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, (const uint16_t*)a,
                       (const uint16_t*)b, c);
    return bi_launch_status();
    BI_TRY_END
}

extern "C" int bi_probe_copy(const void* src, void* dst, int64_t bytes, void* stream)
{
    BI_TRY_BEGIN
    if (bytes < 0 || (bytes % 16)) return BI_ERR_INVALID_ARGUMENT;
    if (bytes > 0 && (!src || !dst || !bi_aligned(src, 16) || !bi_aligned(dst, 16)))
        return BI_ERR_INVALID_ARGUMENT;
    if (bytes == 0) return BI_OK;
    const int64_t n16 = bytes / 16;
    const int64_t want = (n16 + 255) / 256;
    const unsigned grid = (unsigned)(want < 256 * 16 ? want : 256 * 16);
    hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src,
                       (u32x4*)dst, n16);
    return bi_launch_status();
    BI_TRY_END
}

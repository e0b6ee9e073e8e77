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

// Plain streaming read: wavefront w of the grid reads the 8 KB blocks w,
// w + W, w + 2W, ... (W wavefronts in all), eight 16-byte loads per lane in
// flight, each covering 1 KB of the block: the achievable HBM read bandwidth.
// Each wavefront writes the xor of every 32-bit word it read to sink[w], so
// no load is dead and the sink words xor to the xor of the whole buffer.
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                   uint32_t* __restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    const int64_t W = (int64_t)gridDim.x * 4;
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    uint32_t acc = 0;
    for (int64_t b = w; b * 512 < n16; b += W) {          // 512 16-byte units per block
        u32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t i = b * 512 + 64 * j + lane;
            v[j] = i < n16 ? src[i] : zero_u32x4();
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
    }
    for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
    if (lane == 0) sink[w] = acc;
}

// Global -> LDS fill rate: each of the 8 wavefronts of a workgroup streams
// iters x 8 KB from src (1 KB global_load_lds_dwordx4 loads, the GEMM and
// attention kernels' staging instruction; 8 to 16 in flight per wavefront)
// into its own 8 KB of LDS, wrapping inside the first span_chunks KB of src.
// The span decides where the data comes from: a few MB stay in each XCD's L2,
// tens of MB in the last-level cache, a GB in HBM.
constexpr int kFillWaves = 8;
__global__ __launch_bounds__(64 * kFillWaves) void lds_fill_kernel(const uint16_t* __restrict__ src,
                                                                   int64_t span_chunks, int iters,
                                                                   uint32_t* __restrict__ sink)
{
    __shared__ __attribute__((aligned(1024))) uint16_t lds[kFillWaves * 8 * 512];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int64_t chunk = ((int64_t)blockIdx.x * kFillWaves + wave) * 8;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t c = (chunk + j) % span_chunks;
            __builtin_amdgcn_global_load_lds(src + c * 512 + lane * 8, lds + (wave * 8 + j) * 512, 16, 0, 0);
        }
        // at most the 8 loads just issued stay in flight (vmcnt 8; lgkmcnt, expcnt unconstrained)
        __builtin_amdgcn_s_waitcnt((8 & 0xF) | (0x7 << 4) | (0xF << 8));
        chunk += (int64_t)gridDim.x * kFillWaves * 8;
    }
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));   // vmcnt 0: every load has landed
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = lds[lane];
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

extern "C" int bi_probe_read(const void* src, int64_t bytes, uint32_t* sink, void* stream)
{
    BI_TRY_BEGIN
    if (bytes < 0 || (bytes % 16)) return BI_ERR_INVALID_ARGUMENT;
    if (bytes > 0 && (!src || !sink || !bi_aligned(src, 16) || !bi_aligned(sink, 4)))
        return BI_ERR_INVALID_ARGUMENT;
    if (bytes == 0) return BI_OK;
    const int64_t n16 = bytes / 16;
    const int64_t blocks = (n16 + 511) / 512;                  // 8 KB blocks, 4 wavefronts per workgroup
    const int64_t want = (blocks + 3) / 4;
    const unsigned grid = (unsigned)(want < 1024 ? want : 1024);   // 16 wavefronts per CU at most
    hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src, n16,
                       sink);
    return bi_launch_status();
    BI_TRY_END
}

extern "C" int bi_probe_lds_fill(const void* src, int64_t span_bytes, int32_t workgroups, int32_t iters,
                                 uint32_t* sink, void* stream)
{
    BI_TRY_BEGIN
    if (!src || !sink || !bi_aligned(src, 16) || !bi_aligned(sink, 4)) return BI_ERR_INVALID_ARGUMENT;
    if (span_bytes < 1024 || (span_bytes % 1024) || workgroups <= 0 || workgroups > BI_PROBE_SINK_WORDS ||
        iters <= 0)
        return BI_ERR_INVALID_ARGUMENT;
    hipLaunchKernelGGL(lds_fill_kernel, dim3(workgroups), dim3(64 * kFillWaves), 0, (hipStream_t)stream,
                       (const uint16_t*)src, span_bytes / 1024, iters, sink);
    return bi_launch_status();
    BI_TRY_END
}

// sample.hip -- seeded, batch-invariant sampling at temperature T > 0.
//
// Extends the greedy experiment of the page "la température zéro n'est pas
// déterministe" (section "Le mensonge de la température zéro": temperature 0
// is the argmax) to sampled decoding.  Gumbel-max rule:
//     id = argmax_i ( x_i / T + g_i ),   g_i = -log(-log(u_i)),
// which draws i with probability softmax(x / T)_i.  The uniforms come from the
// counter-based generator Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
// random numbers: as easy as 1, 2, 3", SC 2011), written here from that
// definition: key = the row's 64-bit seed, counter = (i, offset low, offset
// high, 0), u_i = ((first output word >> 8) + 0.5) * 2^-24.  Everything after
// the 32-bit word is double precision.
//
// A row's draw depends only on its logits, seed, offset and T: one row per
// workgroup, each thread scores its entries i = t, t + 512, ..., and the
// (score, index) pairs are combined by "larger score wins, equal scores keep
// the lower index", a total order, so the combining order does not matter.
// A NaN logit gives -1.
#include "bi_common.hpp"

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1)
{
    constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;   // round multipliers
    constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;   // key increments
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t hi0 = __umulhi(kM0, c0), lo0 = kM0 * c0;
        const uint32_t hi1 = __umulhi(kM1, c2), lo1 = kM1 * c2;
        const uint32_t n0 = hi1 ^ c1 ^ k0;
        const uint32_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
        k0 += kW0;
        k1 += kW1;
    }
    return c0;
}

__device__ __forceinline__ bool better(double s, int i, double bs, int bi)
{
    return s > bs || (s == bs && i < bi);
}

__global__ __launch_bounds__(kThreads) void sample_kernel(const float* __restrict__ x, int64_t ld, int V,
                                                          double temp, const uint64_t* __restrict__ seeds,
                                                          const uint64_t* __restrict__ offsets,
                                                          int32_t* __restrict__ ids)
{
    __shared__ double s_score[kWaves];
    __shared__ int s_idx[kWaves];
    __shared__ int s_nan[kWaves];
    const int r = blockIdx.x;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const float* xr = x + (int64_t)r * ld;
    const uint64_t seed = seeds[r], off = offsets[r];
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    const uint32_t c1 = (uint32_t)off, c2 = (uint32_t)(off >> 32);

    double bs = -INFINITY;
    int bi = 0x7fffffff;
    int nan = 0;
    for (int i = t; i < V; i += kThreads) {
        const float xi = xr[i];
        nan |= xi != xi;
        const uint32_t w = philox_word0((uint32_t)i, c1, c2, 0u, k0, k1);
        const double u = ((double)(w >> 8) + 0.5) * 0x1p-24;
        const double s = (double)xi / temp - log(-log(u));
        if (better(s, i, bs, bi)) {
            bs = s;
            bi = i;
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const double os = __shfl_xor(bs, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (better(os, oi, bs, bi)) {
            bs = os;
            bi = oi;
        }
        nan |= __shfl_xor(nan, o, 64);
    }
    if (lane == 0) {
        s_score[wave] = bs;
        s_idx[wave] = bi;
        s_nan[wave] = nan;
    }
    __syncthreads();
    if (t == 0) {
        for (int w = 1; w < kWaves; ++w) {
            if (better(s_score[w], s_idx[w], bs, bi)) {
                bs = s_score[w];
                bi = s_idx[w];
            }
            nan |= s_nan[w];
        }
        ids[r] = nan ? -1 : bi;
    }
}

}  // namespace

extern "C" int bi_sample(const float* logits, int64_t ld, int64_t rows, int64_t V, float temperature,
                         const uint64_t* seeds, const uint64_t* offsets, int32_t* ids, void* stream)
{
    BI_TRY_BEGIN
    if (rows < 0 || V <= 0 || ld < V) return BI_ERR_INVALID_ARGUMENT;
    if (!(temperature > 0.0f) || temperature > 3.0e38f) return BI_ERR_INVALID_ARGUMENT;
    if (rows > 0 && (!logits || !seeds || !offsets || !ids || !bi_aligned(logits, 4) ||
                     !bi_aligned(seeds, 8) || !bi_aligned(offsets, 8) || !bi_aligned(ids, 4)))
        return BI_ERR_INVALID_ARGUMENT;
    if (rows > 0x7fffffffLL || V > 0x7fffffffLL - kThreads) return BI_ERR_UNSUPPORTED;
    if (rows == 0) return BI_OK;
    hipLaunchKernelGGL(sample_kernel, dim3((unsigned)rows), dim3(kThreads), 0, (hipStream_t)stream, logits, ld,
                       (int)V, (double)temperature, seeds, offsets, ids);
    return bi_launch_status();
    BI_TRY_END
}

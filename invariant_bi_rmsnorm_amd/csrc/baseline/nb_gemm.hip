// nb_gemm.hip -- NON-invariant, shape-tuned baseline of bi_matmul and bi_addmm,
// built only into libbi_nb.so (measurement, and a check that the invariance
// tests can see a batch-dependent strategy).
//
// It does what the pages say ordinary libraries do (post 論文／ブログ「Defeating
// Nondeterminism in LLM Inference」の技術的なポイント, section 対応策：バッチ不変な
// カーネル設計, table row 行列乗算（MatMul）: the strategy follows the shape, with
// split-K for small batches), on the library's own tiles:
//   * M <= 64 where the 64 x 32 x 128 tiles number at most half the CUs
//     (N <= 4096 on MI355X): split-K.  That tile computes z = 0..Z-1 partial
//     products over k slices of K / Z into fp32 scratch, Z the largest of 2
//     and 4 that keeps the workgroups within the CU count (the fastest split
//     measured at N = 4096); a second kernel adds the partials in z order and
//     rounds.  Each output's sum is split into Z pieces -- and the rows of a
//     batch of 64 are summed differently from the same rows in a batch of 65.
//   * everything else: the library's tiles and rule (gemm_tiles.hpp), tagged
//     as this library's kernels.
// Every result is a correct fp32-accumulated product and run-to-run
// deterministic; only the order, hence the bits, depends on the batch.
#include "../gemm_tiles.hpp"

namespace {

using NbSmallTile = GemmTiles<1>::S;

constexpr size_t kNbScratchFloats = (size_t)16 << 20;     // 64 MiB of fp32 partials
static __device__ __align__(256) float nb_scratch[kNbScratchFloats];

static float* nb_scratch_ptr()
{
    static std::mutex mu;
    static void* addr[64] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev] && hipGetSymbolAddress(&addr[dev], HIP_SYMBOL(nb_scratch)) != hipSuccess) addr[dev] = nullptr;
    return (float*)addr[dev];
}

// c[m][n..n+3] = sum over z of the partials, z ascending, (+ bias), rounded
__global__ __launch_bounds__(256) void nb_splitk_reduce(const float* __restrict__ part, int splits,
                                                        int64_t split_stride, const uint16_t* __restrict__ bias,
                                                        void* __restrict__ c, int64_t ldc, int c_f32, int M, int N)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int nq = N / 4;
    if (q >= (int64_t)M * nq) return;
    const int m = (int)(q / nq);
    const int n = (int)(q % nq) * 4;
    const float* p = part + (int64_t)m * N + n;
    f32x4 v = *reinterpret_cast<const f32x4*>(p);
    for (int z = 1; z < splits; ++z) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(p + z * split_stride);
        v[0] = v[0] + w[0];
        v[1] = v[1] + w[1];
        v[2] = v[2] + w[2];
        v[3] = v[3] + w[3];
    }
    if (bias) {
        const u32x2 bb = *reinterpret_cast<const u32x2*>(bias + n);
        v[0] = v[0] + bf16_to_f32(bb[0] & 0xffffu);
        v[1] = v[1] + bf16_to_f32(bb[0] >> 16);
        v[2] = v[2] + bf16_to_f32(bb[1] & 0xffffu);
        v[3] = v[3] + bf16_to_f32(bb[1] >> 16);
    }
    if (c_f32) {
        *reinterpret_cast<f32x4*>((float*)c + (int64_t)m * ldc + n) = v;
    } else {
        u32x2 o;
        o[0] = pack_bf16x2(v[0], v[1]);
        o[1] = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<u32x2*>((uint16_t*)c + (int64_t)m * ldc + n) = o;
    }
}

static int nb_gemm(const void* a, int64_t lda, const void* wt, int64_t ldw, const void* bias, void* c,
                   int64_t ldc, int c_dtype, int64_t M, int64_t N, int64_t K, void* stream)
{
    if (M <= 64) {
        const int64_t tiles = (N + NbSmallTile::kBN - 1) / NbSmallTile::kBN;
        const int64_t cus = device_cus();
        int splits = 1;
        while (splits < 4 && tiles * splits * 2 <= cus && K % (2 * splits * NbSmallTile::kBK) == 0) splits *= 2;
        float* part = splits > 1 && (size_t)splits * M * N <= kNbScratchFloats ? nb_scratch_ptr() : nullptr;
        if (part) {
            int rc = gemm_launch<NbSmallTile, true>(a, lda, wt, ldw, nullptr, part, N, BI_F32, M, N, K / splits,
                                                    stream, splits, M * N);
            if (rc != BI_OK) return rc;
            const int64_t quads = M * N / 4;
            hipLaunchKernelGGL(nb_splitk_reduce, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0,
                               (hipStream_t)stream, (const float*)part, splits, (int64_t)(M * N),
                               (const uint16_t*)bias, c, ldc, c_dtype == BI_F32 ? 1 : 0, (int)M, (int)N);
            return bi_launch_status();
        }
    }
    return gemm_dispatch<1>(a, lda, wt, ldw, bias, c, ldc, c_dtype, M, N, K, stream);
}

}  // namespace

extern "C" int bi_matmul(const void* a, int64_t lda, const void* wt, int64_t ldw, void* c,
                         int64_t ldc, int c_dtype, int64_t M, int64_t N, int64_t K, void* stream)
{
    BI_TRY_BEGIN
    const int v = gemm_validate(a, lda, wt, ldw, c, ldc, c_dtype, M, N, K);
    if (v != BI_OK) return v < 0 ? BI_OK : v;
    return nb_gemm(a, lda, wt, ldw, nullptr, c, ldc, c_dtype, M, N, K, stream);
    BI_TRY_END
}

extern "C" int bi_addmm(const void* a, int64_t lda, const void* wt, int64_t ldw, const void* bias, void* c,
                        int64_t ldc, int c_dtype, int64_t M, int64_t N, int64_t K, void* stream)
{
    BI_TRY_BEGIN
    const int v = gemm_validate(a, lda, wt, ldw, c, ldc, c_dtype, M, N, K);
    if (v != BI_OK) return v < 0 ? BI_OK : v;
    if (!bias || !bi_aligned(bias, 8)) return BI_ERR_INVALID_ARGUMENT;
    return nb_gemm(a, lda, wt, ldw, bias, c, ldc, c_dtype, M, N, K, stream);
    BI_TRY_END
}

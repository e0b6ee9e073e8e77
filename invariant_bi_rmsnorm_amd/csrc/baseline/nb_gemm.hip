// nb_gemm.hip -- NON-invariant baseline of bi_matmul and bi_addmm, built only into
// libbi_nb.so for measurement and for checking that the invariance tests can
// see a batch-dependent strategy.
//
// It reproduces the failure the pages describe (post 論文／ブログ「Defeating
// Nondeterminism in LLM Inference」の技術的なポイント, section 対応策：バッチ不変な
// カーネル設計, table row 行列乗算（MatMul）: libraries change the reduction
// strategy with the batch size, e.g. split-K for small matrices): for
// M <= 128 the k chunks are accumulated in two interleaved chains (even / odd)
// added at the end, as a split-K would; above, the plain ascending chain.
// Every result is still a correct, run-to-run deterministic fp32-accumulated
// product; only the order, hence the bits, depend on M.
#include "../gemm_kernel.hpp"

extern "C" int bi_matmul(const void* a, int64_t lda, const void* wt, int64_t ldw, void* c,
                         int64_t ldc, int c_dtype, int64_t M, int64_t N, int64_t K, void* stream)
{
    BI_TRY_BEGIN
    const int v = gemm_validate(a, lda, wt, ldw, c, ldc, c_dtype, M, N, K);
    if (v != BI_OK) return v < 0 ? BI_OK : v;
    if (M <= 128) return gemm_launch<1>(a, lda, wt, ldw, nullptr, c, ldc, c_dtype, M, N, K, stream);
    return gemm_launch<0>(a, lda, wt, ldw, nullptr, c, ldc, c_dtype, M, N, K, stream);
    BI_TRY_END
}

extern "C" int bi_addmm(const void* a, int64_t lda, const void* wt, int64_t ldw, const void* bias, void* c,
                        int64_t ldc, int c_dtype, int64_t M, int64_t N, int64_t K, void* stream)
{
    BI_TRY_BEGIN
    const int v = gemm_validate(a, lda, wt, ldw, c, ldc, c_dtype, M, N, K);
    if (v != BI_OK) return v < 0 ? BI_OK : v;
    if (!bias || !bi_aligned(bias, 8)) return BI_ERR_INVALID_ARGUMENT;
    if (M <= 128) return gemm_launch<1>(a, lda, wt, ldw, bias, c, ldc, c_dtype, M, N, K, stream);
    return gemm_launch<0>(a, lda, wt, ldw, bias, c, ldc, c_dtype, M, N, K, stream);
    BI_TRY_END
}

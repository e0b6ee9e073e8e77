// nb_rmsnorm.hip -- NON-invariant baseline of bi_rmsnorm (libbi_nb.so only).
//
// Post 論文／ブログ「Defeating Nondeterminism in LLM Inference」の技術的なポイント,
// section 対応策：バッチ不変なカーネル設計, table row RMSNorm: at small batch
// sizes libraries switch to a split-reduction strategy, which reorders the
// row's sum.  Here a batch below 32 rows uses a different (still fixed,
// deterministic) per-row order than larger batches.
#include "../rmsnorm_kernel.hpp"

extern "C" int bi_rmsnorm(const void* x, int64_t ldx, const void* w, void* y, int64_t ldy,
                          float* rstd, int64_t M, int64_t H, float eps, void* stream)
{
    BI_TRY_BEGIN
    const int v = rmsnorm_validate(x, ldx, w, y, ldy, rstd, M, H, eps);
    if (v != BI_OK) return v < 0 ? BI_OK : v;
    if (M < 32) return rmsnorm_launch<1>(x, ldx, w, y, ldy, rstd, M, H, eps, stream);
    return rmsnorm_launch<0>(x, ldx, w, y, ldy, rstd, M, H, eps, stream);
    BI_TRY_END
}

// The residual add and the RMSNorm that follows it, in one launch: h = bf16(h + r)
// element by element (as bi_add), then y = the RMSNorm of the new h (as
// bi_rmsnorm above), so the bits equal those of the two calls in turn.
extern "C" int bi_add_rmsnorm(void* h, int64_t ldh, const void* r, int64_t ldr, const void* w, void* y,
                              int64_t ldy, float* rstd, int64_t M, int64_t H, float eps, void* stream)
{
    BI_TRY_BEGIN
    const int v = add_rmsnorm_validate(h, ldh, r, ldr, w, y, ldy, rstd, M, H, eps);
    if (v != BI_OK) return v < 0 ? BI_OK : v;
    if (M < 32) return rmsnorm_launch<1, true>(h, ldh, w, y, ldy, rstd, M, H, eps, stream, r, ldr, h, ldh);
    return rmsnorm_launch<0, true>(h, ldh, w, y, ldy, rstd, M, H, eps, stream, r, ldr, h, ldh);
    BI_TRY_END
}

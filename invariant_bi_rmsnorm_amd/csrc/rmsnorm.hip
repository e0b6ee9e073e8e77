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
#include "rmsnorm_kernel.hpp"

extern "C" int bi_rmsnorm(const void* x, int64_t ldx, const void* w, void* y, int64_t ldy,
                          float* rstd, int64_t M, int64_t H, float eps, void* stream)
{
    BI_TRY_BEGIN
    const int v = rmsnorm_validate(x, ldx, w, y, ldy, rstd, M, H, eps);
    if (v != BI_OK) return v < 0 ? BI_OK : v;
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
    return rmsnorm_launch<0, true>(h, ldh, w, y, ldy, rstd, M, H, eps, stream, r, ldr, h, ldh);
    BI_TRY_END
}

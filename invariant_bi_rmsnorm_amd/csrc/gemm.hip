// gemm.hip -- batch-invariant dense matmul: ONE MFMA tile configuration for
// every shape.
//
// Table row 行列乗算（MatMul） of the post "論文／ブログ「Defeating Nondeterminism
// in LLM Inference」の技術的なポイント" (mobiles-han.blogspot.com), section
// 対応策：バッチ不変なカーネル設計, and the same row in the post
// "元OpenAIの研究者ら、AIの応答が毎回違う理由をついに解明", section
// 解決へのアプローチ: libraries pick split-K or drop the matrix units for some
// sizes, which changes each output's reduction order with the batch; the fix
// is one kernel configuration, decided in advance, for all shapes.
//
// Reduction order of an output c[m][n] (the only thing batch invariance needs
// fixed): an fp32 accumulator starts at 0; one v_mfma_f32_16x16x32_bf16 per
// 32-wide k chunk, chunks in ascending k; inside a chunk, lane group g always
// supplies k = 8g..8g+7.  An MFMA result element depends only on its own row
// and column operands, so nothing in the chain depends on M, N, the tile's
// place in the grid or the row's place in the tile.  No split-K, no stream-K,
// no shape-dependent dispatch.
//
// The one configuration (chosen by measuring the whole M = 1..2048 sweep of
// Llama-8B projections on MI355X; small M is weight-streaming, large M is
// MFMA/L2 bound, and one tile has to serve both):
//   * workgroup tile 64 (m) x 32 (n) x 128 (k), 512 threads = 8 wavefronts in
//     a 4 (m) x 2 (n) arrangement, each wavefront one 16x16 MFMA tile; small
//     N-tiles give the weight-streaming small-M shapes more workgroups (a
//     CU streams from HBM at a bounded rate, so the number of CUs at work is
//     what sets their speed: N = 4096 gives 128 workgroups);
//   * operands go global -> LDS with global_load_lds_dwordx4 (no register
//     staging), three 24 KB stages (two in flight while one is consumed),
//     72 KB in all, so two workgroups share a CU at large M; a row's 128-wide
//     k slice is 256 contiguous bytes in HBM;
//   * LDS rows are 256 B with the 16-byte chunks XOR-swizzled by (row & 15):
//     the 16 rows of an MFMA operand read then hit distinct 16-byte slots and
//     the read has no bank conflicts on gfx950 (a (row & 7) swizzle costs 4
//     conflict cycles per read there);
//   * tiles are dealt to the 8 XCDs in contiguous ranges of a grouped order
//     (bands of 4 m-tiles, n-major inside a band), so the wavefronts running
//     together on one XCD share A and W slices in that XCD's L2;
//   * MFMAs of 16-row groups that lie entirely at m >= M are skipped (those
//     rows are never stored; every stored row runs the full chain).
// M and N tails: out-of-range rows are not loaded and not stored.
#include "gemm_kernel.hpp"

extern "C" int bi_matmul(const void* a, int64_t lda, const void* wt, int64_t ldw, void* c,
                         int64_t ldc, int c_dtype, int64_t M, int64_t N, int64_t K, void* stream)
{
    BI_TRY_BEGIN
    const int v = gemm_validate(a, lda, wt, ldw, c, ldc, c_dtype, M, N, K);
    if (v != BI_OK) return v < 0 ? BI_OK : v;
    return gemm_launch<0>(a, lda, wt, ldw, nullptr, c, ldc, c_dtype, M, N, K, stream);
    BI_TRY_END
}

// addmm: the same kernel and K chain, the bias row added to the fp32 result
// once, before the output rounding.
extern "C" int bi_addmm(const void* a, int64_t lda, const void* wt, int64_t ldw, const void* bias, void* c,
                        int64_t ldc, int c_dtype, int64_t M, int64_t N, int64_t K, void* stream)
{
    BI_TRY_BEGIN
    const int v = gemm_validate(a, lda, wt, ldw, c, ldc, c_dtype, M, N, K);
    if (v != BI_OK) return v < 0 ? BI_OK : v;
    if (!bias || !bi_aligned(bias, 8)) return BI_ERR_INVALID_ARGUMENT;
    return gemm_launch<0>(a, lda, wt, ldw, bias, c, ldc, c_dtype, M, N, K, stream);
    BI_TRY_END
}

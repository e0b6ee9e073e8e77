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
// The one configuration (BiTile in gemm_kernel.hpp), chosen by timing the
// whole M = 1..2048 sweep of Llama-8B projections (N = 4096 and 14336,
// K = 4096) on MI355X against a dozen tiles with the same chain:
//   * workgroup tile 128 (m) x 64 (n) x 128 (k), 512 threads = 8 wavefronts
//     in a 4 (m) x 2 (n) arrangement, each wavefront a 32 x 32 tile of four
//     16 x 16 MFMA tiles that share their operand reads (one 16-byte LDS read
//     per MFMA).  Large M is bound by what the L2 delivers into the CUs'
//     LDS, so the tile's flops per byte loaded (2 BM BN / (2 (BM + BN)) =
//     43 flop/B) set its speed; small M streams W, and 64-wide n tiles still
//     give N = 4096 sixty-four workgroups to stream it with;
//   * operands go global -> LDS with global_load_lds_dwordx4, three 48 KB
//     stages (144 KB, one workgroup per CU);
//   * the operands of k tile kt+1 are read from LDS while the MFMAs of k tile
//     kt run (two register sets), so the LDS latency is off the critical path;
//   * a tile wholly inside M, N and a whole number of k tiles runs a loop with
//     no guards and fixed wait counts; edge tiles run the same chain with
//     wave-uniform guards (rows out of range are neither loaded nor stored,
//     and MFMAs of 16-row groups entirely past M are skipped);
//   * LDS rows are 256 B with the 16-byte chunks XOR-swizzled by (row & 15):
//     the 16 rows of an MFMA operand read hit distinct 16-byte slots, no bank
//     conflicts on gfx950;
//   * tiles are dealt to the 8 XCDs in contiguous ranges of a grouped order
//     (bands of 4 m tiles, n-major inside a band).
// No split-K, no stream-K, no shape-dependent choice of tile, MFMA or k order.
#include "gemm_kernel.hpp"

extern "C" int bi_matmul(const void* a, int64_t lda, const void* wt, int64_t ldw, void* c,
                         int64_t ldc, int c_dtype, int64_t M, int64_t N, int64_t K, void* stream)
{
    BI_TRY_BEGIN
    const int v = gemm_validate(a, lda, wt, ldw, c, ldc, c_dtype, M, N, K);
    if (v != BI_OK) return v < 0 ? BI_OK : v;
    return gemm_launch<BiTile>(a, lda, wt, ldw, nullptr, c, ldc, c_dtype, M, N, K, stream);
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
    return gemm_launch<BiTile>(a, lda, wt, ldw, bias, c, ldc, c_dtype, M, N, K, stream);
    BI_TRY_END
}

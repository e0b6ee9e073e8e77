// gemm.hip -- batch-invariant dense matmul: ONE reduction chain per output
// element for every shape.
//
// Table row 行列乗算（MatMul） of the post "論文／ブログ「Defeating Nondeterminism
// in LLM Inference」の技術的なポイント" (mobiles-han.blogspot.com), section
// 対応策：バッチ不変なカーネル設計, and the same row in the post
// "元OpenAIの研究者ら、AIの応答が毎回違う理由をついに解明", section
// 解決へのアプローチ: libraries pick split-K or drop the matrix units for some
// sizes, which changes each output's reduction order with the batch; the fix
// is a kernel whose reduction order is decided in advance for all shapes.
//
// Reduction order of an output c[m][n] (the only thing batch invariance needs
// fixed): an fp32 accumulator starts at 0; one v_mfma_f32_16x16x32_bf16 per
// 32-wide k chunk, chunks in ascending k; inside a chunk, lane group g always
// supplies k = 8g..8g+7; the bias (addmm) is added once to the fp32 sum, then
// the result is rounded.  An MFMA result element depends only on its own row
// and column operands, so nothing in the chain depends on M, N, the tile's
// size, its place in the grid or the row's place in the tile.  No split-K, no
// stream-K, no other instruction or k order for any shape.
//
// What the shape does choose is how the outputs are dealt to workgroups: nine
// tiles of the one kernel template (gemm_kernel.hpp), all with that chain.
// Their results are identical bit for bit (checked for every M of the
// Llama-8B sweep against rows computed inside a 2048-row batch, and at edge
// shapes, by the GPU tests), so the choice changes speed only.  Rule, from
// timing the tiles at every M of the sweep (N = 4096 and 14336, K = 4096) on
// MI355X:
//   * M <= 64 is bound by streaming the weights, each read once per call:
//     weight loads are non-temporal.  When 64-wide n tiles still give three
//     quarters of the CU count in workgroups, 64 x 64 x 128; otherwise narrow
//     n tiles with deep k tiles, so that many weight bytes are in flight per
//     CU: 16 x 16 x 256 (M <= 16), 16 x 32 x 256 (M <= 32), 32 x 32 x 128
//     with six stages (M <= 64).  (Cold weights, N = 4096, M <= 16: 8.5-8.9 us
//     against 15.1-15.3 for the 64 x 32 x 128 tile; N = 14336: 22-26 us.)
//   * M > 64: the largest of 64 x 32 x 128, 64 x 64 x 128, 128 x 64 x 128,
//     128 x 128 x 64 and 256 x 128 x 64 (m x n x k; the last with 64 x 64
//     wavefront tiles, half the LDS reads per MFMA) no taller than M rounded
//     up to 64 that still gives three quarters of the CU count in workgroups
//     (512 x 14336: 66 us against 87 for 128 x 128 x 64).
// A tile that sticks out past M runs the unguarded loop with its extra rows
// reading row M-1; their results are never stored.  Common to all tiles:
//   * wavefront tiles of 16 x 16 MFMA tiles that share their operand reads;
//   * operands go global -> LDS with global_load_lds_dwordx4 through three
//     to six stages;
//   * the operands of k tile kt+1 are read from LDS while the MFMAs of k tile
//     kt run (two register sets), so the LDS latency is off the critical path;
//   * a tile inside N and a whole number of k tiles runs a loop with no
//     guards and fixed wait counts; edge tiles (columns past N, a k tail) run
//     the same chain with wave-uniform guards (rows out of range are neither
//     loaded nor stored, and MFMAs of 16-row groups entirely past M are
//     skipped);
//   * 16-byte LDS chunks XOR-swizzled by row: the 16 rows of an MFMA operand
//     read hit distinct 16-byte slots, no bank conflicts on gfx950;
//   * tiles are dealt to the 8 XCDs in contiguous ranges of a grouped order
//     (bands of 4 m tiles, n-major inside a band).
#include "gemm_tiles.hpp"

extern "C" int bi_matmul(const void* a, int64_t lda, const void* wt, int64_t ldw, void* c,
                         int64_t ldc, int c_dtype, int64_t M, int64_t N, int64_t K, void* stream)
{
    BI_TRY_BEGIN
    const int v = gemm_validate(a, lda, wt, ldw, c, ldc, c_dtype, M, N, K);
    if (v != BI_OK) return v < 0 ? BI_OK : v;
    return gemm_dispatch<0>(a, lda, wt, ldw, nullptr, c, ldc, c_dtype, M, N, K, stream);
    BI_TRY_END
}

// addmm: the same kernels and K chain, the bias row added to the fp32 result
// once, before the output rounding.
extern "C" int bi_addmm(const void* a, int64_t lda, const void* wt, int64_t ldw, const void* bias, void* c,
                        int64_t ldc, int c_dtype, int64_t M, int64_t N, int64_t K, void* stream)
{
    BI_TRY_BEGIN
    const int v = gemm_validate(a, lda, wt, ldw, c, ldc, c_dtype, M, N, K);
    if (v != BI_OK) return v < 0 ? BI_OK : v;
    if (!bias || !bi_aligned(bias, 8)) return BI_ERR_INVALID_ARGUMENT;
    return gemm_dispatch<0>(a, lda, wt, ldw, bias, c, ldc, c_dtype, M, N, K, stream);
    BI_TRY_END
}

// attn_prefill.hip -- causal (chunked) prefill attention over the paged cache.
//
// Table row アテンション (Attention) of the post "論文／ブログ「Defeating
// Nondeterminism in LLM Inference」の技術的なポイント" (mobiles-han.blogspot.com),
// section 対応策：バッチ不変なカーネル設計 (chunked prefill and prefix caching must
// not change the reduction path; cache and fresh tokens share one layout;
// fixed-size splits), and the FixedAttention sketch of the post
// 「非決定モード → 決定モード」に切り替える例, section 注意点・補足実装 (fixed chunk
// size whatever the cache state).
//
// Grid: (query tiles, KV heads, sequences).  A workgroup of 8 wavefronts takes
// 128/G query tokens x the G query heads of one KV head (G = Hq/Hkv); each
// wavefront owns 16 of those (token, head) rows as the 16 MFMA columns.  The
// workgroup reads its sequence's block ids into LDS once, then walks the
// ABSOLUTE 256-token splits 0, 1, ..., up to the split holding its last row.
// K and V^T of a split are staged in LDS with direct global-to-LDS loads,
// double-buffered against the math: V of split i streams in while the scores
// of split i are formed, K of split i+1 while its values are accumulated.
// Every split is evaluated through attn_core.hpp exactly as the decode kernel
// does, folding in registers.  Because splits are aligned to absolute position
// 0 and the arithmetic per split does not depend on which or how many other
// rows share the call, a row's output is the same whether its prompt arrived
// in one piece or in chunks, and equals decode at the same length.
#include "attn_prefill_kernel.hpp"

extern "C" int bi_attention_prefill(const void* q, int64_t ldq, const int32_t* q_start,
                                    const int32_t* kv_lens, const void* k_cache,
                                    const void* v_cache, int64_t num_blocks,
                                    const int32_t* block_table, int32_t max_blocks, void* out,
                                    int64_t ldo, int32_t S, int64_t T, int32_t Hq, int32_t Hkv,
                                    int32_t D, int32_t max_q_len, float scale, void* stream)
{
    return prefill_entry<false>(q, ldq, q_start, kv_lens, k_cache, v_cache, num_blocks, block_table,
                                max_blocks, out, ldo, S, T, Hq, Hkv, D, max_q_len, scale, stream);
}

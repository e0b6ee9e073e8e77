// nb_attn_prefill.hip -- NON-invariant baseline of bi_attention_prefill
// (libbi_nb.so only).
//
// Post 論文／ブログ「Defeating Nondeterminism in LLM Inference」の技術的なポイント,
// section 対応策：バッチ不変なカーネル設計, table row アテンション (Attention): when a
// prompt arrives in chunks, or part of it is already cached, an attention
// kernel that tiles the keys from where the current chunk starts reduces each
// row in an order that depends on how the prompt was cut.  Here the 256-token
// splits start at the chunk's first position, rounded down to its cache block
// (16 tokens), instead of at position 0; the first split starts below 0 and
// its negative positions are masked.  Same kernel and arithmetic per split;
// a prompt whose chunks all start at multiples of 256 (or a single-shot
// prompt) gives the library's bits, other chunkings do not.
#include "../attn_prefill_kernel.hpp"

extern "C" int bi_attention_prefill(const void* q, int64_t ldq, const int32_t* q_start,
                                    const int32_t* kv_lens, const void* k_cache,
                                    const void* v_cache, int64_t num_blocks,
                                    const int32_t* block_table, int32_t max_blocks, void* out,
                                    int64_t ldo, int32_t S, int64_t T, int32_t Hq, int32_t Hkv,
                                    int32_t D, int32_t max_q_len, float scale, void* stream)
{
    return prefill_entry<true>(q, ldq, q_start, kv_lens, k_cache, v_cache, num_blocks, block_table,
                               max_blocks, out, ldo, S, T, Hq, Hkv, D, max_q_len, scale, stream);
}

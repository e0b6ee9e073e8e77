// attn_decode.hip -- paged decode attention with fixed-SIZE KV splits.
//
// Table row アテンション (Attention) of the post "論文／ブログ「Defeating
// Nondeterminism in LLM Inference」の技術的なポイント" (mobiles-han.blogspot.com),
// section 対応策：バッチ不変なカーネル設計: Split-KV / FlashDecode must use a fixed
// split SIZE, so the split boundaries of a sequence never move with the batch,
// the length mix or the number of sequences.
//
// Two kernels:
//  1. decode_split_kernel: persistent workgroups over the work list of
//     (sequence, split) pairs, one KV head per grid row.  Each workgroup first
//     builds the prefix of split counts ceil(kv_len/256) of all sequences in
//     LDS (integer, exact), then takes items blockIdx.x, blockIdx.x + gridDim.x,
//     ...  Which workgroup computes an item has no influence on its arithmetic.
//     Per item: 4 wavefronts each score 64 of the split's 256 tokens for the
//     (up to 16) query heads of the KV group, the split max is taken across
//     the waves, the bf16 weights go to LDS as P^T, and each wave then runs
//     the values chain of the whole split for 32 of the 128 head dims.  The
//     split's (m, l, o[128]) is written, fp32, to the workspace.
//  2. decode_combine_kernel: per (sequence, query head), fold the splits in
//     ascending order and divide.
// All arithmetic goes through attn_core.hpp, shared with the prefill kernel,
// which is why decode at length L equals prefill row L-1 bit for bit.
#include "attn_decode_kernel.hpp"

extern "C" size_t bi_attention_workspace_bytes(int32_t S, int32_t Hq, int32_t D, int32_t max_kv_len)
{
    return decode_ws_bytes(S, Hq, D, max_kv_len, kSplit);
}

extern "C" int bi_attention_decode(const void* q, int64_t ldq, const void* k_cache,
                                   const void* v_cache, int64_t num_blocks,
                                   const int32_t* block_table, int32_t max_blocks,
                                   const int32_t* kv_lens, void* out, int64_t ldo, int32_t S,
                                   int32_t Hq, int32_t Hkv, int32_t D, int32_t max_kv_len,
                                   float scale, void* ws, size_t ws_bytes, void* stream)
{
    BI_TRY_BEGIN
    const int v = decode_validate(q, ldq, k_cache, v_cache, num_blocks, block_table, max_blocks, kv_lens,
                                  out, ldo, S, Hq, Hkv, D, max_kv_len, scale, ws);
    if (v != BI_OK) return v < 0 ? BI_OK : v;
    if (ws_bytes < decode_ws_bytes(S, Hq, D, max_kv_len, kSplit)) return BI_ERR_WORKSPACE_TOO_SMALL;
    return decode_launch(q, ldq, k_cache, v_cache, num_blocks, block_table, max_blocks, kv_lens, out, ldo,
                         S, Hq, Hkv, max_kv_len, scale, ws, kSplit, stream);
    BI_TRY_END
}

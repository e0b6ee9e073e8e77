// nb_attn_decode.hip -- NON-invariant baseline of bi_attention_decode
// (libbi_nb.so only).
//
// Post 論文／ブログ「Defeating Nondeterminism in LLM Inference」の技術的なポイント,
// section 対応策：バッチ不変なカーネル設計, table row アテンション (Attention), and
// post 「非決定モード → 決定モード」に切り替える例, section 注意点・補足実装: decode
// kernels usually pick the KV split from the batch (a split COUNT chosen to
// fill the GPU), so a sequence's split boundaries move with the load.  Here the
// split length is derived from the batch: about 1024 workgroups are wanted,
// i.e. 1024/(S*Hkv) splits per sequence, length = ceil(max_kv_len / that)
// rounded up to 32 and clamped to [32, 256].  Same kernels, same arithmetic per
// split; only the boundaries (hence the fold) depend on S and max_kv_len.
#include "../attn_decode_kernel.hpp"

static int nb_split_len(int32_t S, int32_t Hkv, int32_t max_kv_len)
{
    const int64_t per_seq = std::max<int64_t>(1, 1024 / ((int64_t)S * Hkv));
    int64_t len = ceil_div64(ceil_div64(max_kv_len, per_seq), 32) * 32;
    return (int)std::min<int64_t>(256, std::max<int64_t>(32, len));
}

extern "C" size_t bi_attention_workspace_bytes(int32_t S, int32_t Hq, int32_t D, int32_t max_kv_len)
{
    return decode_ws_bytes(S, Hq, D, max_kv_len, 32);        // room for the shortest split
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
    const int split_len = nb_split_len(S, Hkv, max_kv_len);
    if (ws_bytes < decode_ws_bytes(S, Hq, D, max_kv_len, split_len)) return BI_ERR_WORKSPACE_TOO_SMALL;
    return decode_launch(q, ldq, k_cache, v_cache, num_blocks, block_table, max_blocks, kv_lens, out, ldo,
                         S, Hq, Hkv, max_kv_len, scale, ws, split_len, stream);
    BI_TRY_END
}

// toy_driver.hip -- the greedy-decode step of a small Llama-style decoder,
// built only from the library's batch-invariant entry points.
//
// The experiment it serves: the same prompt decoded greedily 1000 times under
// varying server load gives many distinct completions with ordinary kernels
// and one with batch-invariant kernels (page "la température zéro n'est pas
// déterministe", introduction; post 論文／ブログ「Defeating Nondeterminism in LLM
// Inference」の技術的なポイント, section 実装上の工夫：ツールとライブラリ).
//
// One call = one engine step over a mixed batch: some sequences decode one
// token, others push a chunk of their prompt.  The caller owns every buffer
// (weights, per-layer paged KV caches, the step description, the workspace);
// the driver keeps no state between calls and allocates nothing.
//
// Per layer: RMSNorm -> QKV matmul -> RoPE on q,k and KV append (one launch) -> attention
// (decode kernel for the single-token sequences, prefill kernel for the
// chunks; both give the same bits for the same row) -> O matmul -> residual ->
// RMSNorm -> gate|up matmul -> SiLU*mul -> down matmul -> residual.  Each
// residual add that an RMSNorm follows runs in the same launch as that
// RMSNorm (bi_add_rmsnorm: the same bits as the two calls).
// Then the last row of each sequence (and any further rows the step asks for):
// RMSNorm -> LM head (fp32 logits) -> [rows with a small top-2 margin: the head
// again in fp32 from the unrounded norm, when asked] -> argmax.
#include "../../include/bi.h"
#include "../../include/bi_toy.h"
#include "bi_common.hpp"

namespace {

constexpr size_t kAlign = 256;

size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Layout {
    size_t h, xn, qkv, attn, tmp, gu, act, hl, xl, logits, marg, tids, dws, total;
};

Layout layout(const bi_toy_config* c, int64_t T, int64_t S, int32_t max_kv_len)
{
    const size_t H = c->hidden, D = c->head_dim, Hq = c->heads, Hkv = c->kv_heads, F = c->mlp;
    const size_t QKV = (Hq + 2 * Hkv) * D;
    Layout L{};
    size_t o = 0;
    L.h = o;      o += up((size_t)T * H * 2);   // first: the residual stream, left in place on return
    L.xn = o;     o += up((size_t)T * H * 2);
    L.qkv = o;    o += up((size_t)T * QKV * 2);
    L.attn = o;   o += up((size_t)T * Hq * D * 2);
    L.tmp = o;    o += up((size_t)T * H * 2);
    L.gu = o;     o += up((size_t)T * 2 * F * 2);
    L.act = o;    o += up((size_t)T * F * 2);
    L.hl = o;     o += up((size_t)S * H * 2);
    L.xl = o;     o += up((size_t)S * H * 2);
    L.logits = o; o += up((size_t)S * c->vocab * 4);
    L.marg = o;   o += up((size_t)S * 4);
    L.tids = o;   o += up((size_t)S * 4);
    L.dws = o;    o += up(bi_attention_workspace_bytes((int32_t)S, (int32_t)Hq, (int32_t)D, max_kv_len));
    L.total = o;
    return L;
}

bool cfg_ok(const bi_toy_config* c)
{
    return c && c->layers > 0 && c->hidden > 0 && c->heads > 0 && c->kv_heads > 0 &&
           c->heads % c->kv_heads == 0 && c->head_dim == BI_HEAD_DIM && c->mlp > 0 && c->vocab > 0 &&
           c->max_pos > 0 && c->hidden % 64 == 0 && c->mlp % 64 == 0;
}

#define CHECK(call)                   \
    do {                              \
        const int rc_ = (call);       \
        if (rc_ != BI_OK) return rc_; \
    } while (0)

}  // namespace

extern "C" size_t bi_toy_workspace_bytes(const bi_toy_config* cfg, int32_t max_tokens, int32_t max_seqs,
                                         int32_t max_kv_len)
{
    if (!cfg_ok(cfg) || max_tokens <= 0 || max_seqs <= 0 || max_kv_len <= 0) return 0;
    return layout(cfg, max_tokens, max_seqs, max_kv_len).total;
}

extern "C" int bi_toy_step(const bi_toy_config* c, const bi_toy_weights* w, const bi_toy_step_desc* st,
                           void* ws, size_t ws_bytes, int32_t* next_ids, float* logits_out, void* stream)
{
    BI_TRY_BEGIN
    if (!cfg_ok(c) || !w || !st || !ws || !next_ids) return BI_ERR_INVALID_ARGUMENT;
    if (!w->embed || !w->final_norm || !w->lm_head || !w->layer || !w->k_cache || !w->v_cache ||
        !w->rope_table || w->num_blocks <= 0)
        return BI_ERR_INVALID_ARGUMENT;
    if (st->T <= 0 || st->S <= 0 || st->n_decode < 0 || st->n_decode > st->S || st->S > st->T ||
        st->max_q_len <= 0 || st->max_kv_len <= 0 || st->max_blocks <= 0)
        return BI_ERR_INVALID_ARGUMENT;
    if (!st->ids || !st->pos || !st->slots || !st->q_start || !st->kv_lens || !st->block_table ||
        !st->logit_rows)
        return BI_ERR_INVALID_ARGUMENT;
    if (st->n_logit_rows < 0 || (st->n_logit_rows > 0 && (st->n_logit_rows < st->S || st->n_logit_rows > st->T)))
        return BI_ERR_INVALID_ARGUMENT;
    if (!(st->fp32_head_margin >= 0.0f)) return BI_ERR_INVALID_ARGUMENT;      // negative or NaN
    const int64_t R = st->n_logit_rows > 0 ? st->n_logit_rows : st->S;
    const Layout L = layout(c, st->T, R, st->max_kv_len);
    if (ws_bytes < L.total) return BI_ERR_WORKSPACE_TOO_SMALL;

    const int64_t T = st->T, H = c->hidden, D = c->head_dim;
    const int32_t Hq = c->heads, Hkv = c->kv_heads;
    const int64_t F = c->mlp, V = c->vocab, QKV = (int64_t)(Hq + 2 * Hkv) * D;
    const float scale = 1.0f / sqrtf((float)D);
    char* base = (char*)ws;
    void* h = base + L.h;
    void* xn = base + L.xn;
    uint16_t* qkv = (uint16_t*)(base + L.qkv);
    void* attn = base + L.attn;
    void* tmp = base + L.tmp;
    void* gu = base + L.gu;
    void* act = base + L.act;
    void* hl = base + L.hl;
    void* xl = base + L.xl;
    float* logits = logits_out ? logits_out : (float*)(base + L.logits);
    void* dws = base + L.dws;
    const size_t dws_bytes = L.total - L.dws;
    const int32_t nd = st->n_decode;
    const int32_t np = st->S - nd;

    CHECK(bi_embed(w->embed, V, H, st->ids, T, h, H, stream));
    for (int l = 0; l < c->layers; ++l) {
        const void* const* lw = w->layer + 6 * l;
        // (from the second layer on, with the previous layer's MLP residual add)
        if (l == 0)
            CHECK(bi_rmsnorm(h, H, lw[0], xn, H, nullptr, T, H, c->eps, stream));
        else
            CHECK(bi_add_rmsnorm(h, H, tmp, H, lw[0], xn, H, nullptr, T, H, c->eps, stream));
        CHECK(bi_matmul(xn, H, lw[1], H, qkv, QKV, BI_BF16, T, QKV, H, stream));
        CHECK(bi_rope_kv_append(qkv, QKV, Hq, Hkv, (int32_t)D, st->pos, st->slots, T, w->rope_table, c->max_pos,
                                w->k_cache[l], w->v_cache[l], w->num_blocks, stream));
        if (nd > 0)
            CHECK(bi_attention_decode(qkv, QKV, w->k_cache[l], w->v_cache[l], w->num_blocks,
                                      st->block_table, st->max_blocks, st->kv_lens, attn, (int64_t)Hq * D,
                                      nd, Hq, Hkv, (int32_t)D, st->max_kv_len, scale, dws, dws_bytes,
                                      stream));
        if (np > 0)
            CHECK(bi_attention_prefill(qkv, QKV, st->q_start + nd, st->kv_lens + nd, w->k_cache[l],
                                       w->v_cache[l], w->num_blocks,
                                       st->block_table + (int64_t)nd * st->max_blocks, st->max_blocks,
                                       attn, (int64_t)Hq * D, np, T, Hq, Hkv, (int32_t)D, st->max_q_len,
                                       scale, stream));
        CHECK(bi_matmul(attn, (int64_t)Hq * D, lw[2], (int64_t)Hq * D, tmp, H, BI_BF16, T, H,
                        (int64_t)Hq * D, stream));
        CHECK(bi_add_rmsnorm(h, H, tmp, H, lw[3], xn, H, nullptr, T, H, c->eps, stream));
        CHECK(bi_matmul(xn, H, lw[4], H, gu, 2 * F, BI_BF16, T, 2 * F, H, stream));
        CHECK(bi_silu_mul(gu, 2 * F, F, act, F, T, stream));
        CHECK(bi_matmul(act, F, lw[5], F, tmp, H, BI_BF16, T, H, F, stream));
    }
    CHECK(bi_add(h, tmp, h, T * H, stream));          // the last layer's MLP residual
    CHECK(bi_gather_rows(h, H, T, st->logit_rows, R, H, hl, H, stream));
    CHECK(bi_rmsnorm(hl, H, w->final_norm, xl, H, nullptr, R, H, c->eps, stream));
    CHECK(bi_matmul(xl, H, w->lm_head, H, logits, V, BI_F32, R, V, H, stream));
    if (st->fp32_head_margin > 0.0f) {
        // rows with a small top-2 margin: the head again, from the unrounded norm
        float* marg = (float*)(base + L.marg);
        CHECK(bi_top2(logits, V, R, V, (int32_t*)(base + L.tids), marg, stream));
        CHECK(bi_lm_head_f32(hl, H, w->final_norm, c->eps, w->lm_head, H, logits, V, R, V, H, marg,
                             st->fp32_head_margin, stream));
    }
    CHECK(bi_argmax(logits, V, R, V, next_ids, stream));
    return BI_OK;
    BI_TRY_END
}

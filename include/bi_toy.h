/*
 * bi_toy.h -- C ABI of the toy greedy-decode driver in libbi.so and of the
 * element-wise ops it needs besides bi.h.
 *
 * The experiment this serves is on the page "la température zéro n'est pas
 * déterministe" (introduction and section "Le prix d'une sortie bit à bit
 * identique"): one prompt decoded greedily (argmax at temperature 0) 1000
 * times by a served model under varying load; with batch-invariant kernels
 * every run gives the same completion.  The post 論文／ブログ「Defeating
 * Nondeterminism in LLM Inference」の技術的なポイント (mobiles-han.blogspot.com),
 * section 実装上の工夫：ツールとライブラリ, reports the same 1000-run result.
 * The pages name only a "Transformer"; the model here is a Llama-style
 * pre-norm decoder (RMSNorm, rotary embedding with rotate-half pairing,
 * grouped-query attention, SiLU-gated MLP, untied LM head, no biases).
 *
 * Conventions are those of bi.h: device pointers owned by the caller, void*
 * streams, bi_status return codes, full host validation before any launch,
 * nothing allocated by the library.
 */
#ifndef BI_TOY_H
#define BI_TOY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ element-wise ops */

/* out[t][0:H] = table[ids[t]][0:H] (bf16 copy; an id outside [0, V) gives zeros).
 * table [V][H]; out [T][ldo].  Requires H % 8 == 0, ldo % 8 == 0, 16-byte alignment. */
int bi_embed(const void* table, int64_t V, int64_t H, const int32_t* ids, int64_t T,
             void* out, int64_t ldo, void* stream);

/* Build the rotary table on the device: table[p][i] = (cos a, sin a),
 * a = p * theta^(-2i/D), i < D/2, p < max_pos, evaluated in double and stored
 * as fp32.  table: device float[max_pos * D]. */
int bi_rope_table(float* table, int32_t max_pos, int32_t D, double theta, void* stream);

/* Rotary embedding in place on heads 0..H-1 of each row of x [T][ldx] (bf16):
 * for pair (i, i + D/2) with (c, s) = table[pos[t]][i]:
 *   x[i] <- bf16(x[i] c - x[i+D/2] s),  x[i+D/2] <- bf16(x[i+D/2] c + x[i] s)
 * (fp32 arithmetic).  A position outside [0, max_pos) uses position 0. */
int bi_rope(void* x, int64_t ldx, int32_t H, int32_t D, const int32_t* pos, int64_t T,
            const float* table, int32_t max_pos, void* stream);

/* bi_rope on the q and k heads of a fused projection and bi_kv_append of its
 * k and v heads, in one launch, with the same bits as the two calls in turn:
 * row t of qkv [T][ld] holds Hq q heads, Hkv k heads and Hkv v heads of D;
 * the q and k heads are rotated in place (position pos[t], table as in
 * bi_rope), then k and v are written to k_cache [num_blocks][Hkv][16][D] and
 * v_cache [num_blocks][Hkv][D][16] at slot slots[t] (the cache layout of
 * include/bi.h, one layout for cached and fresh tokens; a slot outside the
 * pool writes no cache entry).  Requires D == 128, ld >= (Hq + 2 Hkv) D,
 * ld % 8 == 0, 16-byte aligned qkv and caches.  Device pointers. */
int bi_rope_kv_append(void* qkv, int64_t ld, int32_t Hq, int32_t Hkv, int32_t D, const int32_t* pos,
                      const int32_t* slots, int64_t T, const float* table, int32_t max_pos, void* k_cache,
                      void* v_cache, int64_t num_blocks, void* stream);

/* out = bf16(a + b), n bf16 elements (n % 8 == 0); out may alias a or b. */
int bi_add(const void* a, const void* b, void* out, int64_t n, void* stream);

/* A pre-norm decoder's residual add and the RMSNorm after it, in one launch:
 * for each of the M rows, h[m] <- bf16(h[m] + r[m]) element by element, then
 * y[m] = bi_rmsnorm of the new h[m] (rstd[m] as there, when rstd is not NULL).
 * The bits equal those of bi_add followed by bi_rmsnorm (the RMSNorm of
 * include/bi.h, table row RMSNorm of the post 論文／ブログ「Defeating
 * Nondeterminism in LLM Inference」の技術的なポイント); the same requirements
 * as bi_rmsnorm apply to h (as x), w, y and H, and r [M][ldr] is laid out like
 * h; y must not be h (BI_ERR_INVALID_ARGUMENT).  Device pointers. */
int bi_add_rmsnorm(void* h, int64_t ldh, const void* r, int64_t ldr, const void* w, void* y, int64_t ldy,
                   float* rstd, int64_t M, int64_t H, float eps, void* stream);

/* out[t][j] = bf16( silu(gu[t][j]) * gu[t][F + j] ), silu(g) = g / (1 + exp(-g)),
 * fp32 arithmetic; gu [T][ldgu] holds gate | up.  Requires F % 8 == 0. */
int bi_silu_mul(const void* gu, int64_t ldgu, int64_t F, void* out, int64_t ldo, int64_t T,
                void* stream);

/* dst[r][0:W] = src[rows[r]][0:W] (bf16); a row index outside [0, nsrc) gives zeros. */
int bi_gather_rows(const void* src, int64_t lds, int64_t nsrc, const int32_t* rows, int64_t R,
                   int64_t W, void* dst, int64_t ldd, void* stream);

/* ------------------------------------------------------------ the step driver */

typedef struct {
    int32_t layers, hidden, heads, kv_heads, head_dim, mlp, vocab;
    int32_t max_pos;      /* rows of the rotary table */
    float eps;            /* RMSNorm epsilon */
    float rope_theta;
} bi_toy_config;

typedef struct {
    const void* embed;              /* [vocab][hidden] bf16 */
    const void* final_norm;         /* [hidden] */
    const void* lm_head;            /* [vocab][hidden] (logits = h . lm_head^T) */
    const void* const* layer;       /* HOST array of 6*layers device pointers, per layer:
                                       attn_norm [hidden], wqkv [(heads+2 kv_heads) D][hidden],
                                       wo [hidden][heads D], mlp_norm [hidden],
                                       wgu [2 mlp][hidden] (gate rows then up rows),
                                       wd [hidden][mlp]                                      */
    void* const* k_cache;           /* HOST array of `layers` device pointers, [num_blocks][kv_heads][16][D] */
    void* const* v_cache;           /* HOST array of `layers` device pointers, [num_blocks][kv_heads][D][16] */
    int64_t num_blocks;
    const float* rope_table;        /* device, from bi_rope_table(max_pos, D, rope_theta) */
} bi_toy_weights;

typedef struct {
    int32_t T;                  /* tokens in this step                                          */
    int32_t S;                  /* sequences in this step                                       */
    int32_t n_decode;           /* sequences 0..n_decode-1 contribute exactly one token each     */
    int32_t max_q_len;          /* >= tokens of any one sequence in this step                    */
    int32_t max_kv_len;         /* >= every kv_lens[s]                                          */
    int32_t max_blocks;         /* columns of block_table                                       */
    const int32_t* ids;         /* device [T] token ids, grouped by sequence as q_start says     */
    const int32_t* pos;         /* device [T] absolute positions                                 */
    const int32_t* slots;       /* device [T] cache slots (block*16 + offset) of those positions */
    const int32_t* q_start;     /* device [S+1]                                                 */
    const int32_t* kv_lens;     /* device [S] cache length after this step's tokens             */
    const int32_t* block_table; /* device [S][max_blocks]                                       */
    const int32_t* logit_rows;  /* device [R] rows (in 0..T-1) whose logits are taken; row r < S
                                   is the one that picks sequence r's next token                */
    int32_t n_logit_rows;       /* R: 0 means S; S <= R <= T.  Rows past S give the logits (and
                                   argmax) after further tokens of a chunk, e.g. every token of a
                                   chunk that re-checks tokens proposed by another path          */
    float fp32_head_margin;     /* > 0: rows whose top-2 margin (bi_top2) is below this get their
                                   logits recomputed by bi_lm_head_f32 before the argmax; 0: off;
                                   +inf: every row                                               */
} bi_toy_step_desc;

/* Workspace bytes for steps of up to max_tokens tokens, max_seqs sequences (and
 * logit rows) and KV lengths up to max_kv_len; 0 if the configuration is
 * unsupported. */
size_t bi_toy_workspace_bytes(const bi_toy_config* cfg, int32_t max_tokens, int32_t max_seqs,
                              int32_t max_kv_len);

/* One greedy step: writes next_ids[r] (device int32 [R]) = argmax of the fp32
 * logits of row logit_rows[r]; logits_out (device float [R][vocab]) receives
 * those logits when non-NULL.  BI_ERR_INVALID_ARGUMENT when n_logit_rows is
 * negative, below S or above T, or fp32_head_margin is negative or NaN;
 * BI_ERR_WORKSPACE_TOO_SMALL when R rows do not fit the workspace.  Each row goes through the batch-invariant
 * kernels only, so next_ids[s] does not depend on which other sequences share
 * the step or on their order.  Requires head_dim == 128, hidden % 64 == 0,
 * mlp % 64 == 0 and the constraints of the bi.h entry points it calls.
 * On return the workspace begins with the residual stream after the last
 * layer: bf16 [T][hidden], row t for token t of the step (before the final
 * RMSNorm), for callers that inspect or check intermediate states. */
int bi_toy_step(const bi_toy_config* cfg, const bi_toy_weights* w, const bi_toy_step_desc* step,
                void* ws, size_t ws_bytes, int32_t* next_ids, float* logits_out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* BI_TOY_H */

/*
 * bi.h -- C ABI of libbi.so: batch-invariant transformer forward kernels for
 * AMD Instinct MI355X (gfx950, CDNA4).
 *
 * Batch invariance: for any one row (a token's activations, a query row of
 * attention), the bits of the result do not depend on the batch size, on the
 * row's position in the batch, on what else is in the batch, nor on the
 * KV-cache state (cache hit or fresh, chunked or single-shot prefill, decode).
 * The property and the three ops that need care are laid out in the post
 * "論文／ブログ「Defeating Nondeterminism in LLM Inference」の技術的なポイント"
 * (mobiles-han.blogspot.com, 2025-09-14 archive), sections
 * "バッチ不変性 (Batch Invariance) の意味" (definition) and
 * "対応策：バッチ不変なカーネル設計" (table: RMSNorm, MatMul, Attention).
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - bf16 tensors are passed as void* to 16-bit storage (IEEE binary32 top
 *    half); fp32 as float*; indices as int32_t*.  All tensor pointers are
 *    DEVICE pointers unless stated otherwise, allocated and owned by the
 *    caller.  The library never allocates or frees device memory and holds no
 *    mutable global state, except the scratch array that
 *    bi_attention_decode_noalloc uses instead of a caller workspace; every other
 *    entry point is safe to call from several threads.
 *  - Leading dimensions (ld*) are in elements.  Row-major everywhere.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Every call is asynchronous on that stream.
 *  - Return value: a bi_status.  Arguments are validated on the host, in full,
 *    before anything is launched; on error nothing is launched and nothing is
 *    written.  Device contents (lengths, block tables, slots) cannot be checked
 *    on the host; the kernels bounds-check every index they read and never
 *    access memory outside the buffers described by the size arguments
 *    (an out-of-range index produces unspecified output values, not a fault).
 *    Faults of an asynchronous launch surface at the caller's next
 *    synchronisation.  No C++ exception crosses this ABI.
 *  - Unsupported-but-valid shapes return BI_ERR_UNSUPPORTED; they are never
 *    routed to a different kernel, because a shape-dependent kernel switch is
 *    exactly what breaks batch invariance.
 *  - M == 0 / T == 0 / S == 0 is a valid no-op.
 */
#ifndef BI_H
#define BI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BI_ABI_VERSION 1

typedef enum {
    BI_OK = 0,
    BI_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative size, ld too small, misaligned  */
    BI_ERR_UNSUPPORTED = 2,        /* valid but outside what the kernels support              */
    BI_ERR_WORKSPACE_TOO_SMALL = 3,
    BI_ERR_NO_DEVICE = 4,
    BI_ERR_LAUNCH = 5              /* hipGetLastError() reported a launch failure             */
} bi_status;

typedef enum { BI_BF16 = 0, BI_F32 = 1 } bi_dtype;

/* Fixed strategy constants (compile-time properties of the kernels). */
#define BI_KV_BLOCK 16      /* tokens per KV-cache block                                 */
#define BI_KV_SPLIT 256     /* tokens per attention split, aligned to absolute position 0 */
#define BI_HEAD_DIM 128     /* the only supported head dimension                          */

int         bi_abi_version(void);
const char* bi_status_string(int status);

/*
 * RMSNorm, one row per workgroup with a fixed reduction order
 * (table row "RMSNorm" of the section 対応策：バッチ不変なカーネル設計: keep a
 * data-parallel strategy whatever the batch size so each row's reduction order
 * never changes).
 *
 *   rstd[m] = 1 / sqrt( (1/H) * sum_j x[m][j]^2 + eps )     (fp32 accumulation)
 *   y[m][j] = bf16( (x[m][j] * rstd[m]) * w[j] )             (fp32, one rounding to bf16)
 *
 * x   [M][ldx] bf16, w [H] bf16, y [M][ldy] bf16, rstd [M] fp32 or NULL.
 * Requires H % 8 == 0, 8 <= H <= 16384, ldx % 8 == 0, ldy % 8 == 0, x/w/y 16-byte
 * aligned.  y may alias x only if ldy == ldx (in-place).
 */
int bi_rmsnorm(const void* x, int64_t ldx, const void* w, void* y, int64_t ldy,
               float* rstd, int64_t M, int64_t H, float eps, void* stream);

/*
 * Dense matmul with ONE reduction chain per output element for every shape
 * (table row 行列乗算（MatMul） of the same section: a reduction order fixed in
 * advance for all shapes, no split-K, no switch of compute unit by size).  Each
 * c[m][n] is an fp32 sum from 0, one bf16 MFMA per 32-wide k chunk in ascending
 * k, rounded once; the shape only chooses how outputs are dealt to workgroups
 * (tiles), which changes no bit of any output.
 *
 *   c[m][n] = sum_{k=0..K-1} a[m][k] * wt[n][k]     (fp32 accumulation, ascending k)
 *
 * a  [M][lda] bf16; wt [N][ldw] bf16 = the logical weight W[K][N] stored
 * transposed (the K-contiguous layout of a linear layer); c [M][ldc], bf16
 * (round to nearest even) or fp32 per c_dtype.
 * Requires K % 32 == 0, N % 4 == 0, lda/ldw % 8 == 0, lda/ldw < 2^24, ldc % 4 == 0,
 * a/wt 16-byte aligned, c 8-byte (bf16) / 16-byte (fp32) aligned; M, N, K below
 * 2^31 - 256 and ceil(M/16) * ceil(N/16) below 2^31 - 8 (else BI_ERR_UNSUPPORTED).
 * M == 0 returns BI_OK without a launch.
 */
int bi_matmul(const void* a, int64_t lda, const void* wt, int64_t ldw,
              void* c, int64_t ldc, int c_dtype, int64_t M, int64_t N, int64_t K,
              void* stream);

/*
 * addmm (torch.addmm with alpha = beta = 1, one of the ops the post
 * "論文／ブログ「Defeating Nondeterminism in LLM Inference」の技術的なポイント",
 * section 他の演算子（RMSNorm, MatMul, mean/reduction etc.）, lists as replaced
 * by invariant kernels): c[m][n] = bias[n] + sum_k a[m][k] * wt[n][k].  The
 * same kernel and K chain as bi_matmul; the bf16 bias is added to the fp32
 * chain result once, then the output is rounded.  bias [N] bf16, device,
 * 8-byte aligned; every other argument as bi_matmul.
 */
int bi_addmm(const void* a, int64_t lda, const void* wt, int64_t ldw, const void* bias, void* c,
             int64_t ldc, int c_dtype, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * Append fresh keys/values to the paged cache, so that attention reads cached
 * and fresh tokens through one layout (table row アテンション (Attention) of the
 * same section: merge cache and current data into one consistent layout before
 * attending; the FixedAttention sketch of the post
 * 「非決定モード → 決定モード」に切り替える例, section 注意点・補足実装).
 *
 * k_new, v_new: token t, head h, dim d at [t*ld_new + h*D + d] (bf16).
 * slots [T]: slot = block*16 + offset of token t (int32); a slot outside
 *   [0, num_blocks*16) is skipped.
 * k_cache [num_blocks][Hkv][16][D] bf16 (token-major inside a block);
 * v_cache [num_blocks][Hkv][D][16] bf16 (dim-major inside a block).
 * Requires D == 128, ld_new >= Hkv*D, ld_new % 8 == 0, 16-byte aligned pointers.
 * A bitwise copy; no arithmetic.
 */
int bi_kv_append(const void* k_new, const void* v_new, int64_t ld_new, const int32_t* slots,
                 int64_t T, void* k_cache, void* v_cache, int64_t num_blocks,
                 int32_t Hkv, int32_t D, void* stream);

/*
 * Workspace for bi_attention_decode, laid out from its first 256-byte
 * boundary: 256 bytes for the work counter of the split kernel (zeroed by the
 * call itself, with a kernel, on its stream), then per split and query head a
 * row of D fp32 partial values, then 128 bytes per split and KV head for the
 * partial (max, sum) pairs (sized for Hkv == Hq, which needs the most).  Every
 * partial line is written whole by one wavefront.  Size: 255 + 256 +
 * S * Hq * ceil(max_kv_len/256) * (D + 32) * 4 bytes.
 */
size_t bi_attention_workspace_bytes(int32_t S, int32_t Hq, int32_t D, int32_t max_kv_len);

/*
 * Paged decode attention with FIXED-SIZE KV splits (same table row: use a fixed
 * split size for Split-KV / FlashDecode, never a split count derived from the
 * batch or the length).  One query token per sequence; the token's own K/V
 * must already be in the cache (bi_kv_append), and kv_lens counts it.
 *
 * Split i of sequence s covers absolute tokens [256 i, 256 i + 256).  Per split
 * and query head: split-local max, exp2 weights, their sum and the weighted
 * values (fp32, into the workspace); then a left fold over splits 0,1,2,...
 * For the same query row and the same cached K/V the result is bitwise equal
 * to row (kv_len - 1) of bi_attention_prefill.
 *
 * q [S rows][ldq] bf16, row s holds Hq heads of D; out likewise with ldo.
 * block_table [S][max_blocks] int32 physical block ids; kv_lens [S] int32 in
 * [1, max_kv_len] and <= max_blocks*16.  scale multiplies q.k (1/sqrt(D) usually).
 * kv_lens live on the device and are not checked on the host: a length of 0
 * or less gives that sequence an all-zero output row, and a length past the
 * limits is cut to min(max_blocks*16, max_kv_len rounded up to 256).
 * A block id outside [0, num_blocks) names no block: its 16 tokens take no part
 * in the attention (score -inf, value 0), here and in bi_attention_prefill
 * alike, so such a row still does not depend on the rest of the batch (a row
 * with no token left gets 0/0 = NaN).
 * ws: device workspace of at least bi_attention_workspace_bytes(S, Hq, D, max_kv_len);
 * its contents need no initialisation, and calls that share one ws must not
 * overlap in time.  Which workgroup computes which split is decided at run
 * time (a work counter), and has no influence on any result.
 * Requires D == 128, Hq % Hkv == 0, Hq/Hkv <= 16, Hkv <= 256,
 * 1 <= max_kv_len <= 1<<20, S <= 2048, S * ceil(max_kv_len/256) * Hkv <= 2^30
 * (else BI_ERR_UNSUPPORTED), 16-byte aligned q/out/caches, ldq/ldo % 8 == 0.
 */
int bi_attention_decode(const void* q, int64_t ldq, const void* k_cache, const void* v_cache,
                        int64_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                        const int32_t* kv_lens, void* out, int64_t ldo,
                        int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_kv_len,
                        float scale, void* ws, size_t ws_bytes, void* stream);

/*
 * Allocation-free bi_attention_decode, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, kernels and bits as bi_attention_decode,
 * without ws/ws_bytes: the split partials go to a scratch array that the
 * library holds in device memory, one per GPU, until the process ends.  The
 * call never allocates or frees memory (neither does the rest of the library).
 * Limit: bi_attention_workspace_bytes(S, Hq, D, max_kv_len) must not exceed
 * BI_ATTENTION_DECODE_NOALLOC_SCRATCH_BYTES (64 MiB; e.g. S * Hq *
 * ceil(max_kv_len/256) <= 104856 for D = 128), else BI_ERR_WORKSPACE_TOO_SMALL
 * is returned before any device work.  Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (other streams, other host
 * threads) race and must be serialised by the caller.  Nothing needs clearing
 * between calls (each call zeroes the array's work counter itself, with a
 * kernel on its stream).
 */
#define BI_ATTENTION_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int bi_attention_decode_noalloc(const void* q, int64_t ldq, const void* k_cache, const void* v_cache,
                                int64_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                                const int32_t* kv_lens, void* out, int64_t ldo,
                                int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_kv_len,
                                float scale, void* stream);

/*
 * Causal (chunked) prefill attention over the paged cache (same table row:
 * chunked prefill must not change the reduction path).  Sequence s contributes
 * T_s = q_start[s+1] - q_start[s] query tokens, which sit at absolute positions
 * [kv_lens[s] - T_s, kv_lens[s]) and whose K/V are already in the cache.  A query
 * at position p sees keys 0..p.  Splits are the same absolute 256-token splits
 * as decode, so the output of a row does not depend on how the prompt was
 * chunked, on what else is in the call, nor on whether the row is computed
 * here or by bi_attention_decode.
 *
 * q [T][ldq] bf16 (rows ordered by q_start), out [T][ldo] bf16;
 * q_start [S+1] int32 ascending with q_start[0] == 0 and q_start[S] == T;
 * kv_lens [S] int32; max_q_len >= every T_s (host-side bound for the grid).
 * Requires D == 128, Hq % Hkv == 0, Hq/Hkv in {1,2,4,8,16}, max_blocks <= 4096
 * (sequences up to 65536 positions), S <= 65535, Hkv <= 65535.
 */
int bi_attention_prefill(const void* q, int64_t ldq, const int32_t* q_start,
                         const int32_t* kv_lens, const void* k_cache, const void* v_cache,
                         int64_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                         void* out, int64_t ldo, int32_t S, int64_t T, int32_t Hq,
                         int32_t Hkv, int32_t D, int32_t max_q_len, float scale,
                         void* stream);

/*
 * Mean over the last dimension, batch-invariant (post "論文／ブログ「Defeating
 * Nondeterminism in LLM Inference」の技術的なポイント", section 他の演算子
 * （RMSNorm, MatMul, mean/reduction etc.）: torch.mean is one of the reductions
 * whose order must not follow the batch).  out[r] = (1/H) sum_j x[r][j] with
 * the RMSNorm kernel's reduction order (fixed by H alone).
 *
 * x [rows][ldx] bf16 (16-byte aligned, ldx % 8 == 0), out [rows] fp32, device
 * pointers.  H % 8 == 0 and H <= 16384, else BI_ERR_UNSUPPORTED.
 */
int bi_mean(const void* x, int64_t ldx, float* out, int64_t rows, int64_t H, void* stream);

/*
 * log_softmax over the last dimension, batch-invariant (post "論文／ブログ
 * 「Defeating Nondeterminism in LLM Inference」の技術的なポイント", section
 * 他の演算子（RMSNorm, MatMul, mean/reduction etc.）: log_softmax is one of the
 * reductions the invariant library replaces).  For every row r:
 *     y[r][i] = x[r][i] - m - log(sum_j exp(x[r][j] - m)),  m = max_j x[r][j]
 * with one reduction order that depends only on V (one row per workgroup;
 * see csrc/log_softmax.hip), so a row's bits do not depend on rows, on the
 * row's position or on the other rows.
 *
 * x [rows][ldx] fp32, y [rows][ldy] fp32, device pointers, 4-byte aligned;
 * ldx, ldy >= V; in place (x == y) only with ldx == ldy.  A row holding a NaN
 * becomes all NaN; a row whose maximum is -inf (all -inf) or +inf becomes NaN
 * where the formula gives NaN; -inf entries of other rows give -inf.
 * rows == 0 is a no-op; rows and V up to 2^31 - 513.
 */
int bi_log_softmax(const float* x, int64_t ldx, float* y, int64_t ldy, int64_t rows, int64_t V,
                   void* stream);

/*
 * Seeded sampling at temperature T > 0, batch-invariant: extends the greedy
 * choice below (page "la température zéro n'est pas déterministe", section
 * "Le mensonge de la température zéro") to sampled decoding.  Gumbel-max:
 *     ids[r] = argmax_i ( x[r][i] / T + g_i ),  g_i = -log(-log(u_i)),
 *     u_i = ((w_i >> 8) + 0.5) * 2^-24,
 * w_i = first output word of Philox4x32-10 (Salmon et al., SC 2011) with key
 * = seeds[r] (low word first) and counter = (i, offsets[r] low, offsets[r]
 * high, 0); the division, logs and sum in double precision; ties to the lower
 * index; -1 if the row holds a NaN.  This draws i with probability
 * softmax(x[r] / T)_i, and a row's draw depends only on its logits, seed,
 * offset and T.  Use a fresh offset (e.g. the token's position) per draw.
 *
 * logits [rows][ld] fp32; seeds, offsets [rows] uint64; ids [rows] int32;
 * device pointers.  T must be finite and > 0 (T = 0 is bi_argmax).
 */
int bi_sample(const float* logits, int64_t ld, int64_t rows, int64_t V, float temperature,
              const uint64_t* seeds, const uint64_t* offsets, int32_t* ids, void* stream);

/*
 * Top-2 logit margin monitor (page arxiv-daily-jp 2609.26621: output flips
 * concentrate where the two best candidates are close, and recomputing the
 * head only for such steps is what helped).  ids[r] = argmax of row r (ties
 * to the lowest index, as bi_argmax); margin[r] = top1 - top2 in fp32, top2
 * the largest logit at any other index (a tie gives 0); V == 1 gives +inf; a
 * NaN gives -1 and NaN.  Both are order-free (maxima and a total order).
 * logits [rows][ld] fp32, ids [rows] int32, margin [rows] fp32, device.
 */
int bi_top2(const float* logits, int64_t ld, int64_t rows, int64_t V, int32_t* ids, float* margin,
            void* stream);

/*
 * Output head in fp32 for the rows whose top-2 margin is small (page
 * arxiv-daily-jp.pages.dev/paper/2609.26621, abstract: recomputing the LM head
 * in FP32 only where the margin falls below a threshold).  For each row r of
 * h (bf16 [R][ldh], the hidden state before the final norm) whose margin is
 * not >= threshold (every row when margin is NULL; a NaN margin counts as
 * small):
 *   rstd      = the rstd bi_rmsnorm gives for the row (same order, same bits),
 *   y_j       = (h_j * rstd) * norm_w_j in fp32, not rounded to bf16,
 *   out[r][v] = sum_j y_j * lm_head[v][j], fp32, one fixed order: per lane
 *               j = 512 c + 8 lane + e ascending with fmaf, lanes combined by a
 *               fixed xor butterfly (batch-invariant per row).
 * Rows not selected are left untouched.  lm_head [V][ldw] bf16; out [R][ldo]
 * fp32; margin [R] fp32 or NULL; all device pointers, h / norm_w / lm_head
 * 16-byte aligned.  BI_ERR_UNSUPPORTED unless H % 512 == 0 and H <= 4096, or
 * when R > 65535.  threshold must not be NaN; eps finite and >= 0.
 */
int bi_lm_head_f32(const void* h, int64_t ldh, const void* norm_w, float eps, const void* lm_head,
                   int64_t ldw, float* out, int64_t ldo, int64_t R, int64_t V, int64_t H,
                   const float* margin, float threshold, void* stream);

/*
 * Greedy token choice (temperature 0 = argmax at every step; page
 * "la température zéro n'est pas déterministe", section "Le mensonge de la
 * température zéro").  ids[r] = index of the largest logit of row r, ties to
 * the lowest index, -1 if the row holds a NaN.  logits [rows][ld] fp32.
 */
int bi_argmax(const float* logits, int64_t ld, int64_t rows, int64_t V, int32_t* ids,
              void* stream);

/*
 * Diagnostic: one v_mfma_f32_16x16x32_bf16 on a [16][32] bf16 (row-major) and
 * b [32][16] bf16 (row-major) into c [16][16] fp32 (row-major), with the
 * operand/result lane layout the kernels assume.  The batch-invariance
 * argument of bi_matmul and of attention rests on the fact that an MFMA
 * result element depends only on its own row of a and column of b; tests use
 * this entry point to check that and the layout.  Device pointers.
 */
int bi_probe_mfma_bf16(const void* a, const void* b, float* c, void* stream);

/*
 * Diagnostic: dst[0:bytes] = src[0:bytes] with a plain streaming copy kernel
 * (16-byte accesses, grid-stride).  It measures the achievable HBM bandwidth
 * that the kernels' rooflines are compared with, and is the known-size
 * reference for scaling the memory-traffic counters.  bytes % 16 == 0,
 * 16-byte aligned device pointers, no overlap.
 */
int bi_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);

/* Words of the sink array the two probes below write (device uint32). */
#define BI_PROBE_SINK_WORDS 8192

/*
 * Diagnostic: reads src[0:bytes] once with a plain streaming kernel (each
 * wavefront reads whole 8 KB blocks, eight 16-byte loads per lane in flight,
 * up to 16 wavefronts per CU): the achievable HBM read
 * bandwidth, the ceiling of the weight-streaming GEMMs and of decode, which
 * read far more than they write.  Each wavefront writes the xor of the 32-bit
 * words it read to one word of sink (device uint32 [BI_PROBE_SINK_WORDS]), so
 * the xor of all sink words equals the xor of all words of src (words the
 * call does not use keep their contents).  bytes % 16 == 0, 16-byte aligned
 * src.
 */
int bi_probe_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

/*
 * Diagnostic: the global -> LDS fill rate of global_load_lds_dwordx4, the
 * instruction the GEMM and attention kernels stage their operands with.
 * `workgroups` workgroups of 8 wavefronts each move iters x 8 KB per
 * wavefront from src into LDS (1 KB per load, 8 to 16 loads in flight per
 * wavefront), reading the first span_bytes of src over and over: a span of a
 * few MB is served by each XCD's L2, tens of MB by the last-level cache, a GB
 * by HBM.  Total bytes moved: workgroups * 8 * iters * 8192.  sink (device
 * uint32 [BI_PROBE_SINK_WORDS]) receives one word per workgroup.
 * span_bytes % 1024 == 0 and >= 1024, 1 <= workgroups <= BI_PROBE_SINK_WORDS,
 * iters >= 1, 16-byte aligned src of at least span_bytes.
 */
int bi_probe_lds_fill(const void* src, int64_t span_bytes, int32_t workgroups, int32_t iters, uint32_t* sink,
                      void* stream);

#ifdef __cplusplus
}
#endif
#endif /* BI_H */

/*
 * oracle.c -- plain, slow, obviously-correct CPU reference for the
 * batch-invariant forward path (RMSNorm, dense matmul, causal attention,
 * greedy argmax and the toy decoder forward built from them).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant with
 * the HIP library; the only thing both sides see is the seeded input bits.
 *
 * What it computes.  The method on the pages (the post "Defeating
 * Nondeterminism in LLM Inference の技術的なポイント", mobiles-han.blogspot.com,
 * section 対応策：バッチ不変なカーネル設計, and the matching table in the post
 * "元OpenAIの研究者ら、AIの応答が毎回違う理由をついに解明", section
 * 解決へのアプローチ) changes only *which* fixed rounding order each row gets;
 * every op still computes an exact mathematical result up to rounding.  So the
 * oracle is that exact definition: products of bf16 values are exact in
 * double, every sum is a plain left-to-right double sum, and a single
 * round-to-nearest-even to bf16 happens at the very end.  No tiling, no
 * splitting, no fused reordering.
 *
 * Rows are independent; OpenMP parallelises over rows only and each row is a
 * sequential loop, so the result does not depend on the thread count.
 *
 * Every function that returns rounded data also has a double-precision twin
 * (suffix _f64) so a test can measure the error of a GPU result against the
 * unrounded value.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if defined(_OPENMP)
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* bf16 <-> double.  bf16 is the top half of an IEEE binary32.               */
/* ------------------------------------------------------------------------ */

static double bf16_bits_to_double(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f; /* exact */
}

static uint16_t float_bits_top(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/*
 * Round a double straight to bf16 (8 significant bits, binary32 exponent
 * range), ties to even.  Done on the value, not the bits: scale so that the
 * 8 kept bits sit left of the binary point, round with nearbyint() (default
 * mode = ties-to-even), scale back.  Below 2^-126 the spacing is the fixed
 * subnormal quantum 2^-133.  NaN stays NaN (quiet), overflow goes to inf.
 */
static uint16_t double_to_bf16(double x)
{
    if (isnan(x)) return (uint16_t)(signbit(x) ? 0xFFC0u : 0x7FC0u);
    if (isinf(x) || x == 0.0) return float_bits_top((float)x); /* exact */
    int e;
    (void)frexp(x, &e);            /* |x| = f * 2^e, 0.5 <= f < 1           */
    int q = e - 8;                 /* quantum exponent for 8 significant bits */
    if (q < -133) q = -133;        /* bf16/binary32 subnormal quantum         */
    double r = ldexp(nearbyint(ldexp(x, -q)), q);
    if (fabs(r) >= 0x1p128) return (uint16_t)(signbit(x) ? 0xFF80u : 0x7F80u);
    return float_bits_top((float)r); /* r is exact in binary32 and in bf16  */
}

void or_round_bf16(const double* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = double_to_bf16(in[i]);
}

void or_bf16_to_f64(const uint16_t* in, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_bits_to_double(in[i]);
}

/* ------------------------------------------------------------------------ */
/* RMSNorm.  The pages name the op (table row "RMSNorm" in the sections      */
/* cited above) but never write its formula; the oracle takes the usual      */
/* Llama form: mean of squares over the row (divide by H), eps inside the    */
/* square root, elementwise weight w multiplies:                             */
/*     rstd = 1 / sqrt( (1/H) * sum_j x_j^2 + eps )                          */
/*     y_j  = x_j * rstd * w_j                                               */
/* ------------------------------------------------------------------------ */

void or_rmsnorm_f64(const uint16_t* x, int64_t ldx, const uint16_t* w,
                    double* y, int64_t ldy, double* rstd,
                    int64_t M, int64_t H, double eps)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* xr = x + m * ldx;
        double ss = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            double v = bf16_bits_to_double(xr[j]);
            ss += v * v;
        }
        double r = 1.0 / sqrt(ss / (double)H + eps);
        if (rstd) rstd[m] = r;
        if (y) {
            for (int64_t j = 0; j < H; ++j)
                y[m * ldy + j] = bf16_bits_to_double(xr[j]) * r * bf16_bits_to_double(w[j]);
        }
    }
}

void or_rmsnorm(const uint16_t* x, int64_t ldx, const uint16_t* w,
                uint16_t* y, int64_t ldy, float* rstd,
                int64_t M, int64_t H, double eps)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* xr = x + m * ldx;
        double ss = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            double v = bf16_bits_to_double(xr[j]);
            ss += v * v;
        }
        double r = 1.0 / sqrt(ss / (double)H + eps);
        if (rstd) rstd[m] = (float)r;
        for (int64_t j = 0; j < H; ++j)
            y[m * ldy + j] = double_to_bf16(bf16_bits_to_double(xr[j]) * r *
                                            bf16_bits_to_double(w[j]));
    }
}

/* ------------------------------------------------------------------------ */
/* Dense matmul (table row 行列乗算（MatMul） in the sections cited above):  */
/*     C[m][n] = sum_k A[m][k] * W[k][n]                                     */
/* The logical weight is W[K][N]; it is stored transposed, Wt[n][k], the     */
/* K-contiguous layout of a linear layer.  Products of two bf16 values are   */
/* exact in double; the sum over k runs k = 0, 1, ..., K-1.                  */
/* ------------------------------------------------------------------------ */

void or_matmul_f64(const uint16_t* a, int64_t lda, const uint16_t* wt, int64_t ldw,
                   double* c, int64_t ldc, int64_t M, int64_t N, int64_t K)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* ar = a + m * lda;
        for (int64_t n = 0; n < N; ++n) {
            const uint16_t* wr = wt + n * ldw;
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k)
                s += bf16_bits_to_double(ar[k]) * bf16_bits_to_double(wr[k]);
            c[m * ldc + n] = s;
        }
    }
}

/* Matmul plus a bias row (torch.addmm with alpha = beta = 1, which the post */
/* "論文／ブログ「Defeating Nondeterminism in LLM Inference」の技術的なポイント",   */
/* section 他の演算子（RMSNorm, MatMul, mean/reduction etc.）, lists among the  */
/* ops replaced by invariant kernels): c[m][n] = bias[n] + sum_k a[m][k] w[n][k], */
/* exact in double (the bf16 products and the bias are exact there).          */
void or_addmm_f64(const uint16_t* a, int64_t lda, const uint16_t* wt, int64_t ldw,
                  const uint16_t* bias, double* c, int64_t ldc, int64_t M, int64_t N, int64_t K)
{
    or_matmul_f64(a, lda, wt, ldw, c, ldc, M, N, K);
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) c[m * ldc + n] += bf16_bits_to_double(bias[n]);
}

/* c_f32 != 0: C is float (one rounding double -> binary32);
 * c_f32 == 0: C is bf16 (one rounding double -> bf16). */
void or_matmul(const uint16_t* a, int64_t lda, const uint16_t* wt, int64_t ldw,
               void* c, int64_t ldc, int c_f32, int64_t M, int64_t N, int64_t K)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* ar = a + m * lda;
        for (int64_t n = 0; n < N; ++n) {
            const uint16_t* wr = wt + n * ldw;
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k)
                s += bf16_bits_to_double(ar[k]) * bf16_bits_to_double(wr[k]);
            if (c_f32) ((float*)c)[m * ldc + n] = (float)s;
            else       ((uint16_t*)c)[m * ldc + n] = double_to_bf16(s);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Causal attention over one sequence (table row アテンション (Attention) in  */
/* the sections cited above; the cache and the fresh tokens form one         */
/* sequence of keys, as the FixedAttention sketch in the post                */
/* 「非決定モード → 決定モード」に切り替える例 merges them before attending).   */
/*                                                                           */
/*   q   [T][Hq][D]   bf16, query rows; q_pos[t] = absolute position of row t */
/*   k,v [L][Hkv][D]  bf16, keys/values in logical order 0..L-1              */
/*   out [T][Hq][D]                                                          */
/* Query head h reads KV head h / (Hq/Hkv).  Row t sees keys j = 0..q_pos[t]. */
/*   s_j = scale * sum_d q[d] k_j[d]                                         */
/*   out = sum_j exp(s_j - max s) v_j / sum_j exp(s_j - max s)               */
/* The max shift changes nothing mathematically; it only keeps exp finite.   */
/* Decode is the special case T = 1, q_pos = L - 1.                          */
/* ------------------------------------------------------------------------ */

static void attention_row(const uint16_t* qr, const uint16_t* k, const uint16_t* v,
                          int64_t nvis, int32_t Hkv, int32_t D, int32_t g,
                          double scale, double* s, double* o)
{
    double mx = -INFINITY;
    for (int64_t j = 0; j < nvis; ++j) {
        const uint16_t* kr = k + (j * Hkv + g) * (int64_t)D;
        double dot = 0.0;
        for (int32_t d = 0; d < D; ++d)
            dot += bf16_bits_to_double(qr[d]) * bf16_bits_to_double(kr[d]);
        s[j] = scale * dot;
        if (s[j] > mx) mx = s[j];
    }
    double z = 0.0;
    for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
    for (int64_t j = 0; j < nvis; ++j) {
        double e = exp(s[j] - mx);
        z += e;
        const uint16_t* vr = v + (j * Hkv + g) * (int64_t)D;
        for (int32_t d = 0; d < D; ++d) o[d] += e * bf16_bits_to_double(vr[d]);
    }
    for (int32_t d = 0; d < D; ++d) o[d] /= z;
}

/* scratch_scores: caller provides T*Hq*L doubles (one L-slice per row), so
 * the oracle itself never allocates.  D <= 1024.  out_f64 and out_bf16 may
 * each be NULL. */
void or_attention(const uint16_t* q, int64_t T, const int32_t* q_pos,
                  const uint16_t* k, const uint16_t* v, int64_t L,
                  int32_t Hq, int32_t Hkv, int32_t D, double scale,
                  double* scratch_scores, double* out_f64, uint16_t* out_bf16)
{
    int32_t group = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t h = 0; h < Hq; ++h) {
            int64_t nvis = (int64_t)q_pos[t] + 1;
            if (nvis > L) nvis = L;
            double* s = scratch_scores + (t * Hq + h) * L;
            double o[1024];
            attention_row(q + (t * Hq + h) * (int64_t)D, k, v, nvis, Hkv, D,
                          h / group, scale, s, o);
            for (int32_t d = 0; d < D; ++d) {
                int64_t idx = (t * Hq + h) * (int64_t)D + d;
                if (out_f64) out_f64[idx] = o[d];
                if (out_bf16) out_bf16[idx] = double_to_bf16(o[d]);
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Greedy choice (temperature 0 means taking the argmax at every step, page  */
/* "la température zéro n'est pas déterministe", section "Le mensonge de la  */
/* température zéro").  Ties go to the lowest index.  A NaN anywhere in the  */
/* row gives -1.                                                             */
/* ------------------------------------------------------------------------ */

void or_argmax(const float* logits, int64_t ld, int64_t rows, int64_t V, int32_t* ids)
{
    for (int64_t r = 0; r < rows; ++r) {
        const float* x = logits + r * ld;
        int32_t best = -1;
        float bv = 0.0f;
        for (int64_t i = 0; i < V; ++i) {
            if (isnan(x[i])) { best = -1; break; }
            if (best < 0 || x[i] > bv) { best = (int32_t)i; bv = x[i]; }
        }
        ids[r] = best;
    }
}

/* ------------------------------------------------------------------------ */
/* Mean over the last dimension (post "論文／ブログ「Defeating Nondeterminism   */
/* in LLM Inference」の技術的なポイント", section 他の演算子（RMSNorm, MatMul,    */
/* mean/reduction etc.）: torch.mean is one of the reductions whose order the */
/* invariant library fixes).  out_r = (1/H) * sum_j x_rj, bf16 in, double.   */
/* ------------------------------------------------------------------------ */

void or_mean(const uint16_t* x, int64_t ldx, double* out, int64_t rows, int64_t H)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double s = 0.0;
        for (int64_t j = 0; j < H; ++j) s += bf16_bits_to_double(x[r * ldx + j]);
        out[r] = s / (double)H;
    }
}

/* ------------------------------------------------------------------------ */
/* log_softmax over the last dimension.  The page post "論文／ブログ          */
/* 「Defeating Nondeterminism in LLM Inference」の技術的なポイント", section     */
/* 他の演算子（RMSNorm, MatMul, mean/reduction etc.）, lists log_softmax among */
/* the reductions the invariant library replaces; the op itself is the usual */
/* one, written out:                                                         */
/*     y_i = x_i - m - log( sum_j exp(x_j - m) ),  m = max_j x_j             */
/* in double precision.  A row whose maximum is -inf (every entry -inf) or   */
/* +inf, or that holds a NaN, gives NaN where the formula does.              */
/* ------------------------------------------------------------------------ */

void or_log_softmax(const float* x, int64_t ldx, double* y, int64_t ldy, int64_t rows, int64_t V)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * ldx;
        double m = -INFINITY;
        int has_nan = 0;
        for (int64_t i = 0; i < V; ++i) {
            if (isnan(xr[i])) has_nan = 1;
            else if ((double)xr[i] > m) m = (double)xr[i];
        }
        double s = 0.0;
        for (int64_t i = 0; i < V; ++i) s += exp((double)xr[i] - m);
        const double lse = m + log(s);
        for (int64_t i = 0; i < V; ++i)
            y[r * ldy + i] = has_nan ? NAN : (double)xr[i] - lse;
    }
}

/* ------------------------------------------------------------------------ */
/* Seeded sampling at temperature T > 0 (extends the greedy experiment of    */
/* the page "la température zéro n'est pas déterministe" to sampled          */
/* decoding): the Gumbel-max rule                                            */
/*     id = argmax_i ( x_i / T + g_i ),   g_i = -log(-log(u_i))               */
/* picks i with probability softmax(x / T)_i.  The uniforms come from the    */
/* counter-based generator Philox4x32-10 (Salmon, Moraes, Dror, Shaw,        */
/* "Parallel random numbers: as easy as 1, 2, 3", SC 2011): key = the row's */
/* 64-bit seed, counter = (i, offset low, offset high, 0), first output word */
/*     u_i = ((word >> 8) + 0.5) * 2^-24   in (0, 1).                        */
/* Everything after the 32-bit word is double precision.  Ties go to the     */
/* lowest index; a NaN logit gives -1.                                       */
/* ------------------------------------------------------------------------ */

static void philox4x32_10(uint32_t ctr[4], uint32_t k0, uint32_t k1)
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;   /* round multipliers   */
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;   /* key schedule (Weyl) */
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)M0 * ctr[0];
        const uint64_t p1 = (uint64_t)M1 * ctr[2];
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        const uint32_t n0 = hi1 ^ ctr[1] ^ k0;
        const uint32_t n2 = hi0 ^ ctr[3] ^ k1;
        ctr[0] = n0;
        ctr[1] = lo1;
        ctr[2] = n2;
        ctr[3] = lo0;
        k0 += W0;
        k1 += W1;
    }
}

void or_philox4x32_10(const uint32_t* ctr_in, const uint32_t* key, uint32_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        uint32_t c[4] = {ctr_in[4 * i], ctr_in[4 * i + 1], ctr_in[4 * i + 2], ctr_in[4 * i + 3]};
        philox4x32_10(c, key[2 * i], key[2 * i + 1]);
        for (int j = 0; j < 4; ++j) out[4 * i + j] = c[j];
    }
}

static double gumbel_of(uint64_t seed, uint64_t offset, uint32_t i)
{
    uint32_t c[4] = {i, (uint32_t)offset, (uint32_t)(offset >> 32), 0u};
    philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
    const double u = ((double)(c[0] >> 8) + 0.5) * 0x1p-24;
    return -log(-log(u));
}

void or_sample(const float* logits, int64_t ld, int64_t rows, int64_t V, float temperature,
               const uint64_t* seeds, const uint64_t* offsets, int32_t* ids, double* scores)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float* x = logits + r * ld;
        int32_t best = -1;
        double bv = 0.0;
        for (int64_t i = 0; i < V; ++i) {
            if (isnan(x[i])) { best = -1; break; }
            const double sc = (double)x[i] / (double)temperature + gumbel_of(seeds[r], offsets[r], (uint32_t)i);
            if (scores) scores[r * V + i] = sc;
            if (best < 0 || sc > bv) { best = (int32_t)i; bv = sc; }
        }
        ids[r] = best;
    }
}

/* ------------------------------------------------------------------------ */
/* Top-2 logit margin (page arxiv-daily-jp 2609.26621, the precision study:  */
/* output flips concentrate where the two best candidates are close, and    */
/* recomputing the head only for such steps was what helped).  Per row: the */
/* argmax (ties to the lowest index) and margin = top1 - top2, where top2   */
/* is the largest logit at any other index (so a tie gives 0), computed as  */
/* one float subtraction; V == 1 gives +inf; a NaN gives id -1, margin NaN. */
/* ------------------------------------------------------------------------ */

void or_top2(const float* logits, int64_t ld, int64_t rows, int64_t V, int32_t* ids, float* margin)
{
    for (int64_t r = 0; r < rows; ++r) {
        const float* x = logits + r * ld;
        int32_t best = -1;
        int has_nan = 0;
        for (int64_t i = 0; i < V; ++i) {
            if (isnan(x[i])) { has_nan = 1; break; }
            if (best < 0 || x[i] > x[best]) best = (int32_t)i;
        }
        if (has_nan) { ids[r] = -1; margin[r] = NAN; continue; }
        float second = -INFINITY;
        int have_second = 0;
        for (int64_t i = 0; i < V; ++i)
            if (i != best && (!have_second || x[i] > second)) { second = x[i]; have_second = 1; }
        ids[r] = best;
        volatile float top1 = x[best];
        margin[r] = have_second ? top1 - second : INFINITY;
    }
}

/* ------------------------------------------------------------------------ */
/* Output head without the bf16 rounding of the normalized hidden state     */
/* (page arxiv-daily-jp.pages.dev/paper/2609.26621, abstract: output flips   */
/* follow from the top-2 logit margin at the LM head, and recomputing that  */
/* head in FP32 only where the margin is small was the best low-cost fix).  */
/* For each row r of h:  y = the unrounded RMSNorm of h_r (or_rmsnorm_f64),   */
/*     out[r][v] = sum_j y_j * W[v][j],   j = 0 .. H-1, in double.           */
/* ------------------------------------------------------------------------ */

void or_lm_head_f64(const uint16_t* h, int64_t ldh, const uint16_t* w, double eps,
                    const uint16_t* wt, int64_t ldw, double* out, int64_t ldo,
                    int64_t R, int64_t V, int64_t H)
{
    double* y = (double*)malloc((size_t)H * sizeof(double));
    if (!y) return;
    for (int64_t r = 0; r < R; ++r) {
        or_rmsnorm_f64(h + r * ldh, ldh, w, y, H, NULL, 1, H, eps);
#pragma omp parallel for schedule(static)
        for (int64_t v = 0; v < V; ++v) {
            const uint16_t* wr = wt + v * ldw;
            double s = 0.0;
            for (int64_t j = 0; j < H; ++j) s += y[j] * bf16_bits_to_double(wr[j]);
            out[r * ldo + v] = s;
        }
    }
    free(y);
}

/* thread count of the row-parallel loops (results do not depend on it) */
void or_set_num_threads(int n)
{
#if defined(_OPENMP)
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int or_num_threads(void)
{
#if defined(_OPENMP)
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ======================================================================== */
/* Toy decoder (greedy decoding of one prompt, the experiment of the page    */
/* "la température zéro n'est pas déterministe", introduction, and of the    */
/* post 論文／ブログ「Defeating Nondeterminism in LLM Inference」の技術的なポイント, */
/* section 実装上の工夫：ツールとライブラリ).  The pages name only a            */
/* "Transformer"; the layer is read as the usual Llama-style block:          */
/*   h += Wo . attn(rope(Wq xn), rope(Wk xn), Wv xn),  xn = rmsnorm(h)       */
/*   h += Wd . (silu(Wg xn) * (Wu xn)),                xn = rmsnorm(h)       */
/*   logits = Wlm . rmsnorm(h)                                               */
/* Every op is evaluated in double and rounded to bf16 where the model       */
/* stores a tensor (its storage format is part of its definition); logits    */
/* stay in double.                                                           */
/* ======================================================================== */

/* Rotary embedding, rotate-half pairing: pair (x[i], x[i + D/2]) turns by    */
/* angle pos * theta^(-2i/D).  In/out bf16 [T][H][D].                        */
void or_rope(const uint16_t* x, uint16_t* y, const int32_t* pos, int64_t T, int32_t H,
             int32_t D, double theta)
{
    int32_t half = D / 2;
    for (int64_t t = 0; t < T; ++t)
        for (int32_t h = 0; h < H; ++h) {
            const uint16_t* xr = x + (t * H + h) * (int64_t)D;
            uint16_t* yr = y + (t * H + h) * (int64_t)D;
            for (int32_t i = 0; i < half; ++i) {
                double ang = (double)pos[t] * pow(theta, -2.0 * (double)i / (double)D);
                double c = cos(ang), s = sin(ang);
                double a = bf16_bits_to_double(xr[i]);
                double b = bf16_bits_to_double(xr[i + half]);
                yr[i] = double_to_bf16(a * c - b * s);
                yr[i + half] = double_to_bf16(b * c + a * s);
            }
        }
}

/* act = silu(g) * u = g / (1 + exp(-g)) * u, bf16 in/out, n elements. */
void or_silu_mul(const uint16_t* g, const uint16_t* u, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        double gv = bf16_bits_to_double(g[i]);
        out[i] = double_to_bf16(gv / (1.0 + exp(-gv)) * bf16_bits_to_double(u[i]));
    }
}

/* out = a + b (bf16), n elements. */
void or_add(const uint16_t* a, const uint16_t* b, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = double_to_bf16(bf16_bits_to_double(a[i]) + bf16_bits_to_double(b[i]));
}

typedef struct {
    int32_t layers, hidden, heads, kv_heads, head_dim, mlp, vocab;
    double eps, rope_theta;
} or_toy_cfg;

/* layer_w: 6 pointers per layer in the order attn_norm [H], wqkv [(Hq+2Hkv)D][H],
 * wo [H][Hq D], mlp_norm [H], wgu [2F][H], wd [H][F].  Processes the T prompt
 * tokens of one sequence at positions 0..T-1 and writes the logits of the last
 * one.  scratch: caller-provided bytes, at least or_toy_scratch_bytes(cfg, T). */
int64_t or_toy_scratch_bytes(const or_toy_cfg* c, int64_t T)
{
    int64_t H = c->hidden, D = c->head_dim;
    int64_t qkv = (int64_t)(c->heads + 2 * c->kv_heads) * D;
    int64_t u16 = T * (H * 4 + qkv * 2 + (int64_t)c->heads * D * 2 + 2 * (int64_t)c->mlp * 2
                      + (int64_t)c->kv_heads * D * 4);
    int64_t f64 = T * (qkv > 2 * (int64_t)c->mlp ? qkv : 2 * (int64_t)c->mlp) + T * (int64_t)c->heads * T;
    return u16 * 2 + f64 * 8 + 4096;
}

void or_toy_forward(const or_toy_cfg* c, const uint16_t* embed, const uint16_t* const* layer_w,
                    const uint16_t* final_norm, const uint16_t* lm_head, const int32_t* ids,
                    int64_t T, void* scratch, double* logits)
{
    const int64_t H = c->hidden, D = c->head_dim, Hq = c->heads, Hkv = c->kv_heads, F = c->mlp;
    const int64_t QKV = (Hq + 2 * Hkv) * D;
    char* p = (char*)scratch;
    uint16_t* h = (uint16_t*)p;    p += T * H * 2;
    uint16_t* xn = (uint16_t*)p;   p += T * H * 2;
    uint16_t* tmp = (uint16_t*)p;  p += T * H * 2;
    uint16_t* attn = (uint16_t*)p; p += T * Hq * D * 2;
    uint16_t* qkv = (uint16_t*)p;  p += T * QKV * 2;
    uint16_t* qr = (uint16_t*)p;   p += T * Hq * D * 2;
    uint16_t* kk = (uint16_t*)p;   p += T * Hkv * D * 2;
    uint16_t* kr = (uint16_t*)p;   p += T * Hkv * D * 2;
    uint16_t* vv = (uint16_t*)p;   p += T * Hkv * D * 2;
    uint16_t* gu = (uint16_t*)p;   p += T * 2 * F * 2;
    uint16_t* act = (uint16_t*)p;  p += T * F * 2;
    uint16_t* gg = (uint16_t*)p;   p += T * F * 2;
    uint16_t* uu = (uint16_t*)p;   p += T * F * 2;
    p = (char*)(((uintptr_t)p + 15) & ~(uintptr_t)15);
    double* sc = (double*)p;       /* attention score scratch: T*Hq*T doubles */
    int32_t* pos = (int32_t*)malloc(sizeof(int32_t) * (size_t)T);
    for (int64_t t = 0; t < T; ++t) pos[t] = (int32_t)t;

    for (int64_t t = 0; t < T; ++t)
        memcpy(h + t * H, embed + (int64_t)ids[t] * H, (size_t)H * 2);

    for (int32_t l = 0; l < c->layers; ++l) {
        const uint16_t* const* w = layer_w + 6 * l;
        or_rmsnorm(h, H, w[0], xn, H, NULL, T, H, c->eps);
        or_matmul(xn, H, w[1], H, qkv, QKV, 0, T, QKV, H);
        for (int64_t t = 0; t < T; ++t) {
            memcpy(attn + t * Hq * D, qkv + t * QKV, (size_t)(Hq * D) * 2);         /* q */
            memcpy(kk + t * Hkv * D, qkv + t * QKV + Hq * D, (size_t)(Hkv * D) * 2);
            memcpy(vv + t * Hkv * D, qkv + t * QKV + (Hq + Hkv) * D, (size_t)(Hkv * D) * 2);
        }
        or_rope(attn, qr, pos, T, (int32_t)Hq, (int32_t)D, c->rope_theta);
        or_rope(kk, kr, pos, T, (int32_t)Hkv, (int32_t)D, c->rope_theta);
        or_attention(qr, T, pos, kr, vv, T, (int32_t)Hq, (int32_t)Hkv, (int32_t)D,
                     1.0 / sqrt((double)D), sc, NULL, attn);
        or_matmul(attn, Hq * D, w[2], Hq * D, tmp, H, 0, T, H, Hq * D);
        or_add(h, tmp, h, T * H);
        or_rmsnorm(h, H, w[3], xn, H, NULL, T, H, c->eps);
        or_matmul(xn, H, w[4], H, gu, 2 * F, 0, T, 2 * F, H);
        for (int64_t t = 0; t < T; ++t) {
            memcpy(gg + t * F, gu + t * 2 * F, (size_t)F * 2);
            memcpy(uu + t * F, gu + t * 2 * F + F, (size_t)F * 2);
        }
        or_silu_mul(gg, uu, act, T * F);
        or_matmul(act, F, w[5], F, tmp, H, 0, T, H, F);
        or_add(h, tmp, h, T * H);
    }
    or_rmsnorm(h + (T - 1) * H, H, final_norm, xn, H, NULL, 1, H, c->eps);
    or_matmul_f64(xn, H, lm_head, H, logits, c->vocab, 1, c->vocab, H);
    free(pos);
}

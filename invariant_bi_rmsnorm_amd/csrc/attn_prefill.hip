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
// Grid: (query tiles, KV heads, sequences).  A workgroup of 4 wavefronts takes
// 64/G query tokens x the G query heads of one KV head (G = Hq/Hkv); each
// wavefront owns 16 of those (token, head) rows as the 16 MFMA columns.  It
// walks the ABSOLUTE 256-token splits 0, 1, ..., up to the split holding its
// last row, staging K then V^T of each half split (128 tokens) in LDS, and
// evaluates every split through attn_core.hpp exactly as the decode kernel does,
// folding in registers.  Because splits are aligned to absolute position 0 and
// the arithmetic per split does not depend on which or how many other rows
// share the call, a row's output is the same whether its prompt arrived in one
// piece or in chunks, and equals decode at the same length.
#include "attn_core.hpp"

using namespace bi_attn;

namespace {

constexpr int kThreads = 256;
constexpr int kHalf = kSplit / 2;        // tokens staged at once
constexpr int kStride = kD + 8;          // bf16 per LDS row (both K and V^T stages)

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

__device__ __forceinline__ u32x4 keep_first(u32x4 v, int nvalid)
{
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int j = 2 * e;
        uint32_t w = v[e];
        if (j >= nvalid) w &= 0xffff0000u;
        if (j + 1 >= nvalid) w &= 0x0000ffffu;
        v[e] = w;
    }
    return v;
}

__global__ __launch_bounds__(kThreads) void prefill_kernel(
    const uint16_t* __restrict__ q, int64_t ldq, const int32_t* __restrict__ q_start,
    const int32_t* __restrict__ kv_lens, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, int64_t num_blocks, const int32_t* __restrict__ bt,
    int max_blocks, uint16_t* __restrict__ out, int64_t ldo, int64_t T, int Hq, int Hkv,
    float scale_log2)
{
    __shared__ __attribute__((aligned(16))) uint16_t s_buf[kHalf * kStride];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int s = blockIdx.z;
    const int g = blockIdx.y;
    const int G = Hq / Hkv;
    const int tpw = 16 / G;                 // tokens per wavefront
    const int QT = 4 * tpw;                 // tokens per workgroup
    const int qt = gridDim.x - 1 - blockIdx.x;   // longest rows first

    const int qs = q_start[s];
    const int Ts = q_start[s + 1] - qs;
    const int L = clamp_len(kv_lens[s], max_blocks * kBlock);
    const int p0 = L - Ts;                  // absolute position of the chunk's first token
    if (Ts <= 0 || p0 < 0 || qt * QT >= Ts) return;   // uniform over the workgroup
    if (qs < 0 || (int64_t)qs + Ts > T) return;        // inconsistent q_start: touch nothing
    const int32_t* btr = bt + (int64_t)s * max_blocks;

    const int tq = qt * QT + wave * tpw + col / G;    // token index inside this call's chunk
    const int h = g * G + col % G;
    const bool cvalid = tq < Ts;
    const int pos = cvalid ? p0 + tq : -1;
    const int last = min(Ts - 1, qt * QT + QT - 1);
    const int nsplit = (p0 + last) / kSplit + 1;

    bf16x8 qf[4];
    const uint16_t* qrow = q + (int64_t)(qs + tq) * ldq + (int64_t)h * kD + 8 * grp;
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) qf[dc] = as_bf16x8(cvalid ? ld16(qrow + 32 * dc) : zero_u32x4());

    float M = -INFINITY, Lam = 0.0f;
    f32x4 O[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int i = 0; i < nsplit; ++i) {
        const int t0 = i * kSplit;
        float sv[kChunks][8];
        // ---------------- scores
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
            __syncthreads();
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const int idx = tid + kThreads * it;
                const int tl = idx >> 4;
                const int ch = idx & 15;
                const int tok = t0 + kHalf * hs + tl;
                u32x4 v = zero_u32x4();
                if (tok < L) {
                    const int blk = btr[tok >> 4];
                    if (blk >= 0 && blk < num_blocks)
                        v = ld16(kc + (((int64_t)blk * Hkv + g) * kBlock + (tok & 15)) * kD + ch * 8);
                }
                st16(&s_buf[tl * kStride + ch * 8], v);
            }
            __syncthreads();
#pragma unroll
            for (int cl = 0; cl < 4; ++cl) {
                const int c = 4 * hs + cl;
#pragma unroll
                for (int th = 0; th < 2; ++th) {
                    const int tl = 32 * cl + score_row_token(col, th);
                    bf16x8 kf[4];
#pragma unroll
                    for (int dc = 0; dc < 4; ++dc)
                        kf[dc] = as_bf16x8(ld16(&s_buf[tl * kStride + 32 * dc + 8 * grp]));
                    const f32x4 acc = score_tile(kf, qf);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = 4 * th + r;
                        const bool valid = (t0 + 32 * c + 8 * grp + j) <= pos;
                        sv[c][j] = valid ? scaled_score(acc[r], scale_log2) : -INFINITY;
                    }
                }
            }
        }
        // ---------------- max, weights, sum
        float mx = -INFINITY;
#pragma unroll
        for (int c = 0; c < kChunks; ++c)
#pragma unroll
            for (int j = 0; j < 8; ++j) mx = fmaxf(mx, sv[c][j]);
        mx = colmax_finish(mx);
        bf16x8 pf[kChunks];
        float ls = 0.0f;
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            uint32_t wv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) wv[j] = weight_bf16(sv[c][j], mx, (t0 + 32 * c + 8 * grp + j) <= pos);
            pf[c] = pack_weights(wv);
            ls = lsum_add(ls, pf[c]);
        }
        ls = lsum_finish(ls);
        // ---------------- values
        f32x4 o[8];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
            __syncthreads();
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const int idx = tid + kThreads * it;
                const int b = idx >> 8;             // block within the half split
                const int rem = idx & 255;
                const int d = rem >> 1;
                const int half = rem & 1;
                const int tok = t0 + kHalf * hs + 16 * b + 8 * half;
                u32x4 v = zero_u32x4();
                if (tok < L) {
                    const int blk = btr[tok >> 4];
                    if (blk >= 0 && blk < num_blocks) {
                        v = ld16(vc + (((int64_t)blk * Hkv + g) * kD + d) * kBlock + 8 * half);
                        if (tok + 8 > L) v = keep_first(v, L - tok);
                    }
                }
                st16(&s_buf[d * kStride + 16 * b + 8 * half], v);
            }
            __syncthreads();
#pragma unroll
            for (int cl = 0; cl < 4; ++cl) {
                const int c = 4 * hs + cl;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) {
                    const bf16x8 vf = as_bf16x8(ld16(&s_buf[(16 * dt + col) * kStride + 32 * cl + 8 * grp]));
                    o[dt] = pv_step(vf, pf[c], o[dt]);
                }
            }
        }
        // ---------------- fold
        if (i == 0) {
            M = mx;
            Lam = ls;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) O[dt] = o[dt];
        } else if (pos >= t0) {
            float a, b;
            fold_scalars(M, Lam, mx, ls, a, b);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
#pragma unroll
                for (int r = 0; r < 4; ++r) O[dt][r] = fold_value(O[dt][r], o[dt][r], a, b);
        }
    }

    if (cvalid) {
        uint16_t* orow = out + (int64_t)(qs + tq) * ldo + (int64_t)h * kD + 4 * grp;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            u32x2 p;
            p[0] = pack_bf16x2(finish_value(O[dt][0], Lam), finish_value(O[dt][1], Lam));
            p[1] = pack_bf16x2(finish_value(O[dt][2], Lam), finish_value(O[dt][3], Lam));
            *reinterpret_cast<u32x2*>(orow + 16 * dt) = p;
        }
    }
}

}  // namespace

extern "C" int bi_attention_prefill(const void* q, int64_t ldq, const int32_t* q_start,
                                    const int32_t* kv_lens, const void* k_cache,
                                    const void* v_cache, int64_t num_blocks,
                                    const int32_t* block_table, int32_t max_blocks, void* out,
                                    int64_t ldo, int32_t S, int64_t T, int32_t Hq, int32_t Hkv,
                                    int32_t D, int32_t max_q_len, float scale, void* stream)
{
    BI_TRY_BEGIN
    if (S < 0 || T < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || max_blocks <= 0 || num_blocks <= 0 ||
        max_q_len < 0)
        return BI_ERR_INVALID_ARGUMENT;
    if (Hq % Hkv) return BI_ERR_INVALID_ARGUMENT;
    if (!(scale == scale)) return BI_ERR_INVALID_ARGUMENT;
    if (S > 0 && T > 0 && (!q || !q_start || !kv_lens || !k_cache || !v_cache || !block_table || !out))
        return BI_ERR_INVALID_ARGUMENT;
    if (ldq < (int64_t)Hq * D || ldo < (int64_t)Hq * D || (ldq % 8) || (ldo % 4))
        return BI_ERR_INVALID_ARGUMENT;
    if (S > 0 && T > 0 &&
        (!bi_aligned(q, 16) || !bi_aligned(k_cache, 16) || !bi_aligned(v_cache, 16) ||
         !bi_aligned(out, 8) || !bi_aligned(block_table, 4) || !bi_aligned(kv_lens, 4) ||
         !bi_aligned(q_start, 4)))
        return BI_ERR_INVALID_ARGUMENT;
    const int G = Hq / Hkv;
    if (D != kD || !(G == 1 || G == 2 || G == 4 || G == 8 || G == 16) || S > 65535 || Hkv > 65535 ||
        (int64_t)max_blocks * kBlock > (1 << 30))
        return BI_ERR_UNSUPPORTED;
    if (S == 0 || T == 0 || max_q_len == 0) return BI_OK;
    const int QT = 64 / G;
    const int ntiles = (max_q_len + QT - 1) / QT;
    hipLaunchKernelGGL(prefill_kernel, dim3(ntiles, Hkv, S), dim3(kThreads), 0, (hipStream_t)stream,
                       (const uint16_t*)q, ldq, q_start, kv_lens, (const uint16_t*)k_cache,
                       (const uint16_t*)v_cache, num_blocks, block_table, max_blocks,
                       (uint16_t*)out, ldo, T, Hq, Hkv, scale_log2_of(scale));
    return bi_launch_status();
    BI_TRY_END
}

// attn_core.hpp -- the ONE definition of a 256-token attention split, used by
// both bi_attention_decode and bi_attention_prefill.
//
// Table row アテンション (Attention) of the post "論文／ブログ「Defeating
// Nondeterminism in LLM Inference」の技術的なポイント" (mobiles-han.blogspot.com),
// section 対応策：バッチ不変なカーネル設計: split-KV / chunking strategies that vary
// with batch, length or cache state change the reduction path; the fix is
// fixed-SIZE splits over one KV layout.  The post 「非決定モード → 決定モード」に
// 切り替える例, section テスト・検証 (item 3), asks that prefill, decode and
// cache-hit paths agree; here they agree bit for bit because every path
// evaluates each split through the functions below, in the same order.
//
// Canonical arithmetic of split i (absolute tokens [256 i, 256 i + 256)) for one
// query row q (a column of the MFMA tiles; up to 16 rows share one K/V head):
//
//  scores  The split is 8 chunks of 32 tokens; each chunk is two MFMA tiles
//          S^T = K Q^T with 16 token-rows each.  Tile h of chunk c places token
//          32c + 8(i>>2) + 4h + (i&3) in MFMA row i, so that afterwards lane
//          (col = q, grp) holds tokens 32c + 8 grp + j, j = 0..7, in registers
//          (tile 0 rows -> j = 0..3, tile 1 rows -> j = 4..7).  Each tile is an
//          MFMA chain over the 4 head-dim chunks of 32 in ascending order from 0:
//          the raw score a (fp32).  Masked tokens get a = -inf.  With
//          c = |scale| * log2 e (fp32; for a negative scale the query is
//          negated, which negates every product and sum exactly):
//  max     m = fl(max over the split's valid tokens of a  *  c) (the max is
//          exact and order-free; -inf when no token is valid).
//  weights p = exp2(fma(a, c, -m)) (one rounding, v_exp_f32), rounded to bf16;
//          masked -> 0.
//  sum     l = the MFMA chain ones^T P^T over chunks c = 0..7 in ascending
//          order from 0 (the values' chain shape with an all-ones A operand),
//          so the weights are summed exactly as the values weight them.
//  values  O^T = V^T P^T, 8 head-dim tiles of 16; each an MFMA chain over the
//          chunks c = 0..7 in ascending order from 0, the B operand being the
//          lane's 8 bf16 weights (k-slot j <-> token 32c + 8 grp + j).
//  fold    state starts as split 0's (m, l, o); each later split folds in with
//          fold_scalars/fold_value below, splits in ascending order.  A split
//          with no visible token for this row is skipped.
//  out     bf16(o / l).
#pragma once

#include <algorithm>

#include "bi_common.hpp"

namespace bi_attn {

constexpr int kD = 128;           // head dim
constexpr int kBlock = 16;        // tokens per cache block
constexpr int kSplit = 256;       // tokens per split
constexpr int kChunks = kSplit / 32;

// MFMA row `row` of tile h (0/1) of a 32-token chunk holds this chunk-local token.
__device__ __forceinline__ int score_row_token(int row, int h)
{
    return 8 * (row >> 2) + 4 * h + (row & 3);
}

// Score tile: chain over the 4 head-dim chunks, ascending, from zero.
__device__ __forceinline__ f32x4 score_tile(const bf16x8 kf[4], const bf16x8 qf[4])
{
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) acc = mfma16(kf[dc], qf[dc], acc);
    return acc;
}

// The split's max m from the max of its raw scores (c = |scale| log2 e > 0,
// or 0 for a zero scale: a row with no valid token keeps m = -inf).
__device__ __forceinline__ float split_max(float raw_max, float c)
{
    return raw_max == -INFINITY ? -INFINITY : raw_max * c;
}

// Weight of one token before rounding: exp2(fma(a, c, -m)).  In a split with
// masked tokens (a = -inf) the masked form returns 0 for them.
__device__ __forceinline__ float weight_of(float a, float c, float m)
{
    return hw_exp2(__builtin_fmaf(a, c, -m));
}
__device__ __forceinline__ float weight_of_masked(float a, float c, float m)
{
    return a == -INFINITY ? 0.0f : weight_of(a, c, m);
}

// Queries enter with their sign flipped when the scale is negative, and the
// kernels use c = |scale log2 e|.
__device__ __forceinline__ u32x4 q_for_scale(u32x4 q, float scale_log2)
{
    return scale_log2 < 0.0f ? (q ^ u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u}) : q;
}
__device__ __forceinline__ float c_of_scale(float scale_log2) { return scale_log2 < 0.0f ? -scale_log2 : scale_log2; }

// Round 8 weights (j = 0..7) to bf16 and pack them into one MFMA operand.
__device__ __forceinline__ bf16x8 pack_weights(const float p[8])
{
    u32x4 v;
    v[0] = pack_bf16x2(p[0], p[1]);
    v[1] = pack_bf16x2(p[2], p[3]);
    v[2] = pack_bf16x2(p[4], p[5]);
    v[3] = pack_bf16x2(p[6], p[7]);
    return as_bf16x8(v);
}

// One step of the weight-sum chain: l tile += ones^T(chunk) * P^T(chunk).
// Every entry of the lane's accumulator ends up holding l of its column.
__device__ __forceinline__ bf16x8 ones_bf16x8()
{
    return as_bf16x8(u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
}
__device__ __forceinline__ f32x4 lsum_step(bf16x8 pf, f32x4 acc) { return mfma16(ones_bf16x8(), pf, acc); }

// Max across the four lane groups of one column (exact).
__device__ __forceinline__ float colmax_finish(float v)
{
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    v = fmaxf(v, __shfl_xor(v, 32, 64));
    return v;
}

// One step of the values chain: O^T tile += V^T(chunk) * P^T(chunk).
__device__ __forceinline__ f32x4 pv_step(bf16x8 vf, bf16x8 pf, f32x4 acc) { return mfma16(vf, pf, acc); }

// Fold split (mi, li, oi) into the running state (M, Lam, O) of one row.
__device__ __forceinline__ void fold_scalars(float& M, float& Lam, float mi, float li,
                                             float& a, float& b)
{
    const float Mn = fmaxf(M, mi);
    a = hw_exp2(M - Mn);
    b = hw_exp2(mi - Mn);
    Lam = Lam * a + li * b;
    M = Mn;
}

__device__ __forceinline__ float fold_value(float O, float oi, float a, float b) { return O * a + oi * b; }

__device__ __forceinline__ float finish_value(float O, float Lam) { return O / Lam; }

// Host: the score multiplier scale * log2(e) as one fp32 value, computed the
// same way for every entry point so all kernels see identical bits.
static inline float scale_log2_of(float scale)
{
    return (float)((double)scale * 1.4426950408889634074);
}

}  // namespace bi_attn

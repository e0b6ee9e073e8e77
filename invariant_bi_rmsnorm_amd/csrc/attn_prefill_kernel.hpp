// attn_prefill_kernel.hpp -- the causal (chunked) prefill kernel and its
// checked launch, shared by the library (splits aligned to position 0) and the
// non-invariant baseline (splits aligned to each chunk's start).
#pragma once
#include <type_traits>

#include "attn_core.hpp"

using namespace bi_attn;

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 16 * kWaves;          // (token, head) rows per workgroup
constexpr int kMaxBlocks = 4096;            // block-table width supported (65536 positions)

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

// LDS layouts of one split.  K: [256 token rows][128 dims], 16-byte chunk ch of
// row r at slot ch ^ kswz(r).  V^T: as in the cache, [16 blocks][128 dims][16
// tokens], unswizzled.  Both operand reads are free of bank conflicts on gfx950
// (SQ_LDS_BANK_CONFLICT for the whole kernel is under 1 cycle per 100 LDS
// instructions, so it cannot come from them); swapping the two 16-byte halves
// of every other group of 8 V^T dim rows, as a 32-bank layout would want,
// costs 4 conflict cycles per read here.
// Baseline alignment: split boundaries at the chunk's first position rounded
// down to a cache block (p0 & ~15), modulo the split length; split 0 starts
// at or below position 0 and its positions below 0 are masked.
__device__ __forceinline__ int chunk_split_base(int p0)
{
    const int o = (p0 & ~(kBlock - 1)) & (kSplit - 1);
    return o ? o - kSplit : 0;
}

__device__ __forceinline__ int kswz(int row) { return (row & 3) | (((row >> 3) & 3) << 2); }

template <bool kChunkAligned>
__global__ __launch_bounds__(kThreads) void prefill_kernel(
    const uint16_t* __restrict__ q, int64_t ldq, const int32_t* __restrict__ q_start,
    const int32_t* __restrict__ kv_lens, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, int64_t num_blocks, const int32_t* __restrict__ bt,
    int max_blocks, uint16_t* __restrict__ out, int64_t ldo, int64_t T, int Hq, int Hkv,
    float scale_log2)
{
    __shared__ __attribute__((aligned(1024))) uint16_t s_k[kSplit * kD];     // 64 KB
    __shared__ __attribute__((aligned(1024))) uint16_t s_v[kSplit * kD];     // 64 KB
    __shared__ int s_bt[kMaxBlocks];         // physical block of every cache block the workgroup reads
    __shared__ int s_bad[kMaxBlocks / (kSplit / kBlock) + 1];   // split reads a block id outside the pool

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int s = blockIdx.z;
    const int g = blockIdx.y;
    const int G = Hq / Hkv;
    const int tpw = 16 / G;                 // tokens per wavefront
    const int QT = kWaves * tpw;            // tokens per workgroup
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
    // rows of this wavefront: tokens tq0 .. tq0 + tpw - 1 of the chunk
    const int tq0 = qt * QT + wave * tpw;
    const bool wave_full = tq0 + tpw - 1 < Ts;       // every column is a real row
    const int wave_pos0 = p0 + tq0;                  // the smallest position among them
    // first position of split 0: 0, or (baseline only) at or before 0 so that
    // the boundaries fall on the chunk's first cache block
    const int base = kChunkAligned ? chunk_split_base(p0) : 0;
    const int nsplit = (p0 + last - base) / kSplit + 1;

    const float c_scale = c_of_scale(scale_log2);
    bf16x8 qf[4];
    const uint16_t* qrow = q + (int64_t)(qs + tq) * ldq + (int64_t)h * kD + 8 * grp;
#pragma unroll
    for (int dc = 0; dc < 4; ++dc)
        qf[dc] = as_bf16x8(q_for_scale(cvalid ? ld16(qrow + 32 * dc) : zero_u32x4(), scale_log2));

    // block ids of every cache block this workgroup reads, once (-1: none / invalid)
    const int nblk_used = min((L + kBlock - 1) / kBlock, (base + nsplit * kSplit) / kBlock);
    for (int b = tid; b < nblk_used; b += kThreads) {
        const int blk = btr[b];
        s_bt[b] = (blk >= 0 && blk < num_blocks) ? blk : -1;
    }
    auto issue_k = [&](int i) {                       // K rows of split i -> s_k
#pragma unroll
        for (int it = 0; it < kSplit / 4 / kWaves; ++it) {
            const int inst = wave + kWaves * it;
            const int row = 4 * inst + (lane >> 4);
            const int tok = base + i * kSplit + row;
            // the 4 rows of one load lie in one cache block: its id is wave-uniform
            const int tb = (base + i * kSplit + 4 * inst) >> 4;
            const int blk = __builtin_amdgcn_readfirstlane((!kChunkAligned || tb >= 0) && tb * kBlock < L ? s_bt[tb] : -1);
            if (blk >= 0 && tok < L) {
                const int gch = (lane & 15) ^ kswz(row);
                __builtin_amdgcn_global_load_lds(
                    kc + (((int64_t)blk * Hkv + g) * kBlock + (tok & 15)) * kD + gch * 8,
                    s_k + inst * 512, 16, 0, 0);
            }
        }
    };
    auto issue_v = [&](int i) {                       // V^T blocks of split i -> s_v
#pragma unroll
        for (int it = 0; it < kSplit / 4 / kWaves; ++it) {
            const int inst = wave + kWaves * it;      // block inst/4, dims 32*(inst%4) ...
            const int b = inst >> 2;
            const int d = 32 * (inst & 3) + (lane >> 1);
            const int tb = (base >> 4) + i * (kSplit / kBlock) + b;
            const int blk = __builtin_amdgcn_readfirstlane((!kChunkAligned || tb >= 0) && tb * kBlock < L ? s_bt[tb] : -1);
            if (blk >= 0)
                __builtin_amdgcn_global_load_lds(
                    vc + (((int64_t)blk * Hkv + g) * kD + d) * kBlock + (lane & 1) * 8,
                    s_v + inst * 512, 16, 0, 0);
        }
    };

    float M = -INFINITY, Lam = 0.0f;
    f32x4 O[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    __syncthreads();
    // tokens of a block whose id is outside the pool do not exist for the
    // arithmetic (score -inf, weight 0, value 0), exactly as in decode
    for (int sp = tid; sp < nsplit; sp += kThreads) {
        int bad = 0;
        const int b0 = (base >> 4) + sp * (kSplit / kBlock);
        for (int b = b0; b < min(nblk_used, b0 + kSplit / kBlock); ++b)
            bad |= (kChunkAligned && b < 0) || s_bt[b] < 0;   // positions below 0 do not exist
        s_bad[sp] = bad;
    }
    issue_k(0);

    for (int i = 0; i < nsplit; ++i) {
        const int t0 = base + i * kSplit;
        __syncthreads();                 // K of split i landed; every wave is done with s_v
        issue_v(i);
        const bool bad = s_bad[i] != 0;
        // ---------------- scores, max, weights, sum.  When every row of the
        // wavefront sees the whole split (all but the diagonal splits) the
        // causal mask is dropped: same values, fewer instructions.
        bf16x8 pf[kChunks];
        float mx = -INFINITY;
        f32x4 lacc = {0.f, 0.f, 0.f, 0.f};
        auto softmax_part = [&](auto masked) {
            constexpr bool kMasked = decltype(masked)::value;
            float sv[kChunks][8];
            // [step mod 3][dc]: the K operands of the next two tiles load while
            // this one multiplies
            bf16x8 kf[3][4];
            auto load_k = [&](int st, bf16x8 (&dst)[4]) __attribute__((always_inline)) {
                const int row = 32 * (st >> 1) + score_row_token(col, st & 1);
#pragma unroll
                for (int dc = 0; dc < 4; ++dc)
                    dst[dc] = *reinterpret_cast<const bf16x8*>(s_k + row * kD + (((4 * dc + grp) ^ kswz(row)) * 8));
            };
            load_k(0, kf[0]);
            load_k(1, kf[1]);
            float raw_max = -INFINITY;
#pragma unroll
            for (int c = 0; c < kChunks; ++c) {
#pragma unroll
                for (int th = 0; th < 2; ++th) {
                    const int st = 2 * c + th;
                    if (st + 2 < 2 * kChunks) load_k(st + 2, kf[(st + 2) % 3]);
                    // only VALU / SALU work may be scheduled across: the loads stay ahead
                    __builtin_amdgcn_sched_barrier(0x6);
                    const f32x4 acc = score_tile(kf[st % 3], qf);
                    bool blk_ok = true;
                    if constexpr (kMasked) {
                        const int tb = (t0 >> 4) + 2 * c + (grp >> 1);
                        blk_ok = !bad || ((!kChunkAligned || tb >= 0) && s_bt[tb] >= 0);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = 4 * th + r;
                        float a = acc[r];
                        if constexpr (kMasked) a = blk_ok && (t0 + 32 * c + 8 * grp + j) <= pos ? a : -INFINITY;
                        sv[c][j] = a;
                        raw_max = fmaxf(raw_max, a);
                    }
                }
            }
            mx = split_max(colmax_finish(raw_max), c_scale);
#pragma unroll
            for (int c = 0; c < kChunks; ++c) {
                float wv[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    wv[j] = kMasked ? weight_of_masked(sv[c][j], c_scale, mx) : weight_of(sv[c][j], c_scale, mx);
                pf[c] = pack_weights(wv);
                lacc = lsum_step(pf[c], lacc);
            }
        };
        if (wave_full && t0 + kSplit - 1 <= wave_pos0 && !bad)
            softmax_part(std::false_type{});
        else
            softmax_part(std::true_type{});
        __syncthreads();                 // V of split i landed; every wave is done with s_k
        if (i + 1 < nsplit) issue_k(i + 1);
        // ---------------- values.  In the split that holds the sequence end, the
        // value slots past it are stale LDS (possibly NaN) and are zeroed, as
        // are those of blocks with an id outside the pool (never loaded); every
        // other split is whole.
        f32x4 o[8];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto values_part = [&](auto tail) {
            constexpr bool kTail = decltype(tail)::value;
            u32x4 vf[3][4];              // [step mod 3][dt % 4]: the V operands of the next two half chunks load while this one multiplies
            auto load_v = [&](int st, u32x4 (&dst)[4]) __attribute__((always_inline)) {
                const int b = 2 * (st >> 1) + (grp >> 1);
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    dst[k] = ld16(s_v + b * (kD * kBlock) + (16 * (4 * (st & 1) + k) + col) * kBlock + (grp & 1) * 8);
            };
            load_v(0, vf[0]);
            load_v(1, vf[1]);
#pragma unroll
            for (int c = 0; c < kChunks; ++c) {
                const int tok = t0 + 32 * c + 8 * grp;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) {
                    const int st = 2 * c + (dt >> 2);
                    if ((dt & 3) == 0) {
                        if (st + 2 < 2 * kChunks) load_v(st + 2, vf[(st + 2) % 3]);
                        __builtin_amdgcn_sched_barrier(0x6);
                    }
                    u32x4 v = vf[st % 3][dt & 3];
                    if constexpr (kTail) {
                        if (tok + 8 > L) v = tok >= L ? zero_u32x4() : keep_first(v, L - tok);
                        if (bad && tok < L && ((kChunkAligned && tok < 0) || s_bt[tok >> 4] < 0)) v = zero_u32x4();
                    }
                    o[dt] = pv_step(as_bf16x8(v), pf[c], o[dt]);
                }
            }
        };
        if (t0 + kSplit <= L && !bad)
            values_part(std::false_type{});
        else
            values_part(std::true_type{});
        // ---------------- fold
        const float ls = lacc[0];
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

template <bool kChunkAligned>
int prefill_entry(const void* q, int64_t ldq, const int32_t* q_start,
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
        max_blocks > kMaxBlocks)
        return BI_ERR_UNSUPPORTED;
    if (S == 0 || T == 0 || max_q_len == 0) return BI_OK;
    const int QT = kRows / G;
    const int ntiles = (max_q_len + QT - 1) / QT;
    hipLaunchKernelGGL(prefill_kernel<kChunkAligned>, dim3(ntiles, Hkv, S), dim3(kThreads), 0, (hipStream_t)stream,
                       (const uint16_t*)q, ldq, q_start, kv_lens, (const uint16_t*)k_cache,
                       (const uint16_t*)v_cache, num_blocks, block_table, max_blocks,
                       (uint16_t*)out, ldo, T, Hq, Hkv, scale_log2_of(scale));
    return bi_launch_status();
    BI_TRY_END
}

}  // namespace

// attn_decode_kernel.hpp -- the paged decode kernels (see attn_decode.hip for
// the design).  Splits are `split_len` tokens; the library's bi_attention_decode
// always uses 256 (fixed-size splits), the non-invariant baseline derives the
// length from the batch.
#pragma once
#include "attn_core.hpp"

using namespace bi_attn;

namespace {

constexpr int kThreads = 256;
constexpr int kMaxSeqs = 2048;
// bf16 per row of the P^T buffer: a 32-byte pad makes the 16-byte operand
// reads and writes of one wavefront free of LDS bank conflicts on gfx950
// (a 16-byte pad costs 4 conflict cycles per access there)
constexpr int kPtStride = kSplit + 16;
static_assert(16 * kPtStride <= kSplit * kD, "P^T fits in the K buffer it aliases");

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

// zero elements j >= nvalid of an 8 x bf16 vector (nvalid in 0..8)
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

// workgroup barrier for LDS hand-offs: this wave's LDS accesses done, then
// s_barrier, without the memory fence of __syncthreads (which would also wait
// for the value loads still in flight)
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
}

// loads issued per lane per item for the values operands (all unconditional,
// so the count is fixed: the wait for K below leaves exactly these in flight)
constexpr int kVLoads = 2 * kChunks;

// K rows of a split are staged in LDS (256 B per token row); 16-byte chunk ch
// of row r sits at slot ch ^ kswz(r), so the 16 rows one MFMA operand read
// touches fall in distinct banks.
__device__ __forceinline__ int kswz(int row) { return (row & 3) | (((row >> 3) & 3) << 2); }

__global__ __launch_bounds__(kThreads) void decode_split_kernel(
    const uint16_t* __restrict__ q, int64_t ldq, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, int64_t num_blocks, const int32_t* __restrict__ bt,
    int max_blocks, const int32_t* __restrict__ kv_lens, int S, int Hq, int Hkv,
    int max_splits, int split_len, float scale_log2, float* __restrict__ ws, uint16_t* __restrict__ out,
    int64_t ldo)
{
    __shared__ int s_off[kMaxSeqs + 1];
    __shared__ int s_part[kThreads];
    __shared__ float s_max[4][16];
    __shared__ int s_blk[kSplit / kBlock];
    // K of the split [256][128] bf16; after the scores it holds P^T [16][kPtStride]
    __shared__ __attribute__((aligned(1024))) uint16_t s_k[kSplit * kD];
    uint16_t* const s_pt = s_k;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int g = blockIdx.y;
    const int G = Hq / Hkv;
    const int cap = min(max_blocks * kBlock, max_splits * split_len);

    // ---- exclusive prefix of split counts (integers: any order gives the same)
    const int per = (S + kThreads - 1) / kThreads;
    const int b0 = tid * per;
    int local = 0;
    for (int j = 0; j < per; ++j) {
        const int s = b0 + j;
        if (s < S) local += (clamp_len(kv_lens[s], cap) + split_len - 1) / split_len;
    }
    s_part[tid] = local;
    __syncthreads();
    for (int o = 1; o < kThreads; o <<= 1) {
        const int v = (tid >= o) ? s_part[tid - o] : 0;
        __syncthreads();
        s_part[tid] += v;
        __syncthreads();
    }
    int run = s_part[tid] - local;
    for (int j = 0; j < per; ++j) {
        const int s = b0 + j;
        if (s < S) {
            s_off[s] = run;
            run += (clamp_len(kv_lens[s], cap) + split_len - 1) / split_len;
        }
    }
    if (tid == kThreads - 1) s_off[S] = s_part[kThreads - 1];
    __syncthreads();
    const int total = s_off[S];

    for (int w = blockIdx.x; w < total; w += gridDim.x) {
        // sequence of item w: the largest s with s_off[s] <= w
        int lo = 0, hi = S - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_off[mid] <= w) lo = mid; else hi = mid - 1;
        }
        const int s = lo;
        const int i = w - s_off[s];
        const int Lseq = clamp_len(kv_lens[s], cap);
        const int t0 = i * split_len;
        // tokens of this split: [t0, L); with split_len == 256 (the library's
        // only value) L is the sequence length
        const int L = min(Lseq, t0 + split_len);
        const int32_t* btr = bt + (int64_t)s * max_blocks;

        // physical blocks of the split's 16 cache blocks (-1: none / invalid)
        if (tid < kSplit / kBlock) {
            const int tok = t0 + kBlock * tid;
            int blk = -1;
            if (tok < L) blk = btr[tok >> 4];
            s_blk[tid] = (blk >= 0 && blk < num_blocks) ? blk : -1;
        }
        lds_barrier();

        // tokens of a block whose id is outside the pool do not exist for the
        // arithmetic: score -inf, weight 0, value 0 (their K rows are never
        // loaded, so nothing stale from an earlier item can reach the result)
        int blk16[kSplit / kBlock];                  // the 16 ids in registers (broadcast reads, once)
#pragma unroll
        for (int b = 0; b < kSplit / kBlock; ++b) blk16[b] = s_blk[b];
        // block of this lane's tokens 32 c + 8 grp .. + 7 (blk16[2c] or blk16[2c+1]),
        // chosen with bit operations so the array is never indexed per lane
        const int hi_mask = -(grp >> 1);
        auto lane_blk = [&](int c) __attribute__((always_inline)) {
            return blk16[2 * c] ^ ((blk16[2 * c] ^ blk16[2 * c + 1]) & hi_mask);
        };
        bool bad = false;
#pragma unroll
        for (int b = 0; b < kSplit / kBlock; ++b) bad |= (t0 + kBlock * b < L) && blk16[b] < 0;
        // a split that ends before the sequence does and reads only valid
        // blocks needs no masking (the masked code gives the same values
        // there, with more instructions)
        const bool whole = t0 + kSplit <= L && !bad;

        // query operands: column col is query head g*G + col (columns past the
        // group read head g*G's row and are zeroed)
        const bool qok = col < G;
        const uint16_t* qrow = q + (int64_t)s * ldq + (int64_t)(g * G + (qok ? col : 0)) * kD + 8 * grp;
        u32x4 qraw[4];
#pragma unroll
        for (int dc = 0; dc < 4; ++dc) qraw[dc] = ld16(qrow + 32 * dc);

        // K of the split -> LDS, one 1 KB wave load = 4 token rows of 256 B
        // (rows past the sequence are not loaded; their scores are masked)
#pragma unroll
        for (int it = 0; it < kSplit / 4 / 4; ++it) {
            const int inst = wave + 4 * it;
            const int row = 4 * inst + (lane >> 4);          // row >> 4 == it: the 4 rows lie in block it
            const int tok = t0 + row;
            const int blk = tok < L ? blk16[it] : -1;
            if (blk >= 0) {
                const int gch = (lane & 15) ^ kswz(row);         // chunk landing at slot lane&15
                __builtin_amdgcn_global_load_lds(
                    kc + (((int64_t)blk * Hkv + g) * kBlock + (tok & 15)) * kD + gch * 8,
                    s_k + inst * 512, 16, 0, 0);
            }
        }

        // values operands of this wave's two head-dim tiles, all 8 chunks,
        // issued last so that they land while the scores are formed; every
        // lane loads (tokens without a block read block 0 and are zeroed at use)
        u32x4 vv[kChunks][2];
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            const int tok = t0 + 32 * c + 8 * grp;
            const int blk = tok < L ? lane_blk(c) : -1;
            const int b = blk >= 0 ? blk : 0;
#pragma unroll
            for (int dd = 0; dd < 2; ++dd) {
                const int d = 16 * (2 * wave + dd) + col;
                vv[c][dd] = ld16(vc + (((int64_t)b * Hkv + g) * kD + d) * kBlock + (tok & 15));
            }
        }
        // this wave's q and K loads have landed (only the kVLoads value loads,
        // issued after them, may still fly); then every wave's K has
        __builtin_amdgcn_s_waitcnt((kVLoads & 0xF) | ((kVLoads >> 4) << 14) | (0x7 << 4));
        asm volatile("s_barrier" ::: "memory");
        bf16x8 qf[4];
#pragma unroll
        for (int dc = 0; dc < 4; ++dc) qf[dc] = as_bf16x8(qok ? qraw[dc] : zero_u32x4());

        // scores of chunks 2*wave, 2*wave+1
        float sv[2][8];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            const int c = 2 * wave + cc;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int row = 32 * c + score_row_token(col, h);
                bf16x8 kf[4];
#pragma unroll
                for (int dc = 0; dc < 4; ++dc)
                    kf[dc] = *reinterpret_cast<const bf16x8*>(s_k + row * kD + (((4 * dc + grp) ^ kswz(row)) * 8));
                const f32x4 acc = score_tile(kf, qf);
                const bool blk_ok = whole || s_blk[2 * c + (grp >> 1)] >= 0;   // block of tokens 8 grp .. 8 grp + 7
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 4 * h + r;
                    const bool valid = whole || (blk_ok && (t0 + 32 * c + 8 * grp + j) < L);
                    sv[cc][j] = valid ? scaled_score(acc[r], scale_log2) : -INFINITY;
                }
            }
        }

        // split max across the four waves
        float mx = -INFINITY;
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int j = 0; j < 8; ++j) mx = fmaxf(mx, sv[cc][j]);
        mx = colmax_finish(mx);
        if (grp == 0) s_max[wave][col] = mx;
        lds_barrier();
        const float m = fmaxf(fmaxf(s_max[0][col], s_max[1][col]), fmaxf(s_max[2][col], s_max[3][col]));

        // bf16 weights -> LDS as P^T[q][token]
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            const int c = 2 * wave + cc;
            const bool blk_ok = whole || s_blk[2 * c + (grp >> 1)] >= 0;
            float wv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                wv[j] = weight_f32(sv[cc][j], m, whole || (blk_ok && (t0 + 32 * c + 8 * grp + j) < L));
            st16(&s_pt[col * kPtStride + 32 * c + 8 * grp], as_u32x4(pack_weights(wv)));
        }
        lds_barrier();

        // the value operands have landed; zero the slots of tokens past the
        // sequence or in a block outside the pool
        __builtin_amdgcn_s_waitcnt(0x0070);                      // vmcnt(0)
        if (!whole) {
#pragma unroll
            for (int c = 0; c < kChunks; ++c) {
                const int tok = t0 + 32 * c + 8 * grp;
                const bool ok = tok < L && lane_blk(c) >= 0;
#pragma unroll
                for (int dd = 0; dd < 2; ++dd) {
                    if (!ok) vv[c][dd] = zero_u32x4();
                    else if (tok + 8 > L) vv[c][dd] = keep_first(vv[c][dd], L - tok);
                }
            }
        }

        // values chain over the whole split for head-dim tiles 2*wave, 2*wave+1
        f32x4 o[2];
        o[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        o[1] = f32x4{0.f, 0.f, 0.f, 0.f};
        float ls = 0.0f;
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            const bf16x8 pf = as_bf16x8(ld16(&s_pt[col * kPtStride + 32 * c + 8 * grp]));
            ls = lsum_add(ls, pf);
#pragma unroll
            for (int dd = 0; dd < 2; ++dd) o[dd] = pv_step(as_bf16x8(vv[c][dd]), pf, o[dd]);
        }
        ls = lsum_finish(ls);

        if (col < G) {
            const int h = g * G + col;
            if (t0 == 0 && Lseq <= split_len) {
                // the sequence's only split: its fold is the split itself, so
                // the output is o / l, rounded, exactly what the combine would write
                uint16_t* orow = out + (int64_t)s * ldo + (int64_t)h * kD;
#pragma unroll
                for (int dd = 0; dd < 2; ++dd)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        orow[16 * (2 * wave + dd) + 4 * grp + r] =
                            (uint16_t)f32_to_bf16_rne(finish_value(o[dd][r], ls));
            } else {
                float* base = ws + (((int64_t)s * Hq + h) * max_splits + i) * (kD + 2);
#pragma unroll
                for (int dd = 0; dd < 2; ++dd)
#pragma unroll
                    for (int r = 0; r < 4; ++r) base[2 + 16 * (2 * wave + dd) + 4 * grp + r] = o[dd][r];
                if (wave == 0 && grp == 0) {
                    base[0] = m;
                    base[1] = ls;
                }
            }
        }
        lds_barrier();     // s_max / s_pt / s_blk are reused by the next item
    }
}

// Fold of the split partials of one (sequence, query head), 128 threads (one
// per head dim), splits taken 128 at a time (thread t owns split c0 + t of the
// chunk for the scalar part).  The left fold over splits i = 0, 1, ... is
//   M_i = max(M_{i-1}, m_i),  a_i = exp2(M_{i-1} - M_i),  b_i = exp2(m_i - M_i),
//   L_i = L_{i-1} a_i + l_i b_i,  O_i = O_{i-1} a_i + o_i b_i,
// starting from split 0's own (m, l, o).  The running maxima M_i are a prefix
// maximum, which is exact whatever the grouping, so they are formed with a
// wavefront scan; each thread then computes its split's (a_i, b_i) with exactly
// the operations of fold_scalars, and every thread runs the two rounding
// chains (L and its dim of O) in split order.  The bits equal those of the
// sequential fold_scalars / fold_value recurrence the prefill kernel runs in
// registers.  Partial values are loaded kPre splits at a time.
constexpr int kFoldChunk = kD;
constexpr int kPre = 32;

__global__ __launch_bounds__(kD) void decode_combine_kernel(
    const float* __restrict__ ws, const int32_t* __restrict__ kv_lens, int cap, int Hq,
    int max_splits, int split_len, uint16_t* __restrict__ out, int64_t ldo)
{
    __shared__ float s_a[kFoldChunk], s_b[kFoldChunk], s_l[kFoldChunk];
    __shared__ float s_wmax[2];
    const int s = blockIdx.y;
    const int h = blockIdx.x;
    const int d = threadIdx.x;
    const int lane = d & 63;
    const int L = clamp_len(kv_lens[s], cap);
    const int n = (L + split_len - 1) / split_len;
    uint16_t* o = out + (int64_t)s * ldo + (int64_t)h * kD + d;
    if (n == 0) {
        *o = 0;
        return;
    }
    if (n == 1) return;            // written by the split kernel
    const float* base = ws + ((int64_t)s * Hq + h) * max_splits * (kD + 2);
    float Mprev = -INFINITY, Lam = 0.f, O = 0.f;
    for (int c0 = 0; c0 < n; c0 += kFoldChunk) {
        const int cn = min(kFoldChunk, n - c0);
        const float* cb = base + (int64_t)c0 * (kD + 2);
        // ---- scalar part: thread d owns split c0 + d
        const bool own = d < cn;
        const float mi = own ? cb[(int64_t)d * (kD + 2)] : -INFINITY;
        const float li = own ? cb[(int64_t)d * (kD + 2) + 1] : 0.f;
        float v[kPre];
#pragma unroll
        for (int j = 0; j < kPre; ++j) v[j] = j < cn ? cb[(int64_t)j * (kD + 2) + 2 + d] : 0.f;
        float run = mi;                                   // inclusive prefix max inside the wave
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float t = __shfl_up(run, off, 64);
            if (lane >= off) run = fmaxf(run, t);
        }
        if (lane == 63) s_wmax[d >> 6] = run;
        __syncthreads();
        if (d >= 64) run = fmaxf(s_wmax[0], run);
        const float Mi = fmaxf(Mprev, run);               // M_{c0 + d}
        float Mim1 = __shfl_up(Mi, 1, 64);                // M_{c0 + d - 1}
        if (lane == 0) Mim1 = d == 0 ? Mprev : fmaxf(Mprev, s_wmax[0]);
        if (own) {
            s_a[d] = hw_exp2(Mim1 - Mi);
            s_b[d] = hw_exp2(mi - Mi);
            s_l[d] = li;
        }
        // carry: M after the chunk's last split
        const float chunk_max = cn > 64 ? fmaxf(s_wmax[0], s_wmax[1]) : s_wmax[0];
        __syncthreads();
        // ---- the two chains, in split order
        for (int i0 = 0; i0 < cn; i0 += kPre) {
            if (i0 > 0) {
#pragma unroll
                for (int j = 0; j < kPre; ++j)
                    v[j] = i0 + j < cn ? cb[(int64_t)(i0 + j) * (kD + 2) + 2 + d] : 0.f;
            }
#pragma unroll
            for (int j = 0; j < kPre; ++j) {
                const int i = i0 + j;
                if (i < cn) {
                    if (c0 == 0 && i == 0) {
                        Lam = s_l[0];
                        O = v[j];
                    } else {
                        Lam = Lam * s_a[i] + s_l[i] * s_b[i];
                        O = fold_value(O, v[j], s_a[i], s_b[i]);
                    }
                }
            }
        }
        Mprev = fmaxf(Mprev, chunk_max);
        __syncthreads();          // the chunk's LDS is reused by the next chunk
    }
    *o = (uint16_t)f32_to_bf16_rne(finish_value(O, Lam));
}

static inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Workspace of split partials when splits are `split_len` tokens long.
static inline size_t decode_ws_bytes(int32_t S, int32_t Hq, int32_t D, int32_t max_kv_len, int split_len)
{
    if (S <= 0 || Hq <= 0 || D <= 0 || max_kv_len <= 0) return 0;
    return (size_t)S * (size_t)Hq * (size_t)ceil_div64(max_kv_len, split_len) * (size_t)(D + 2) *
           sizeof(float);
}

// Host validation shared by every bi_attention_decode build: BI_OK to go on,
// -1 for the S == 0 no-op, else the status to return.
static inline int decode_validate(const void* q, int64_t ldq, const void* k_cache, const void* v_cache,
                                  int64_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                                  const int32_t* kv_lens, const void* out, int64_t ldo, int32_t S,
                                  int32_t Hq, int32_t Hkv, int32_t D, int32_t max_kv_len, float scale,
                                  const void* ws, bool caller_ws = true)
{
    if (S < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || max_blocks <= 0 || num_blocks <= 0)
        return BI_ERR_INVALID_ARGUMENT;
    if (max_kv_len <= 0 || (int64_t)max_kv_len > (int64_t)max_blocks * kBlock)
        return BI_ERR_INVALID_ARGUMENT;
    if (Hq % Hkv) return BI_ERR_INVALID_ARGUMENT;
    if (!(scale == scale)) return BI_ERR_INVALID_ARGUMENT;
    if (S > 0 && (!q || !k_cache || !v_cache || !block_table || !kv_lens || !out || (caller_ws && !ws)))
        return BI_ERR_INVALID_ARGUMENT;
    if (ldq < (int64_t)Hq * D || ldo < (int64_t)Hq * D || (ldq % 8) || (ldo % 8))
        return BI_ERR_INVALID_ARGUMENT;
    if (S > 0 && (!bi_aligned(q, 16) || !bi_aligned(k_cache, 16) || !bi_aligned(v_cache, 16) ||
                  !bi_aligned(out, 2) || (caller_ws && !bi_aligned(ws, 16)) || !bi_aligned(block_table, 4) ||
                  !bi_aligned(kv_lens, 4)))
        return BI_ERR_INVALID_ARGUMENT;
    if (D != kD || Hq / Hkv > 16 || S > kMaxSeqs || max_kv_len > (1 << 20) || Hkv > 65535)
        return BI_ERR_UNSUPPORTED;
    if (S == 0) return -1;
    return BI_OK;
}

// Launch split + combine with splits of split_len tokens (a multiple of 32,
// at most 256).  The invariant library always passes 256.
static inline int decode_launch(const void* q, int64_t ldq, const void* k_cache, const void* v_cache,
                                int64_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                                const int32_t* kv_lens, void* out, int64_t ldo, int32_t S, int32_t Hq,
                                int32_t Hkv, int32_t max_kv_len, float scale, void* ws, int split_len,
                                void* stream)
{
    const int max_splits = (int)ceil_div64(max_kv_len, split_len);
    const int64_t items_bound = (int64_t)S * max_splits;
    // persistent grid: as many workgroups as can be resident at once (a
    // second, partial round of workgroups would run at low occupancy)
    static const int resident = [] {
        int dev = 0, cus = 0, per_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_split_kernel, kThreads, 0) !=
                hipSuccess ||
            cus <= 0 || per_cu <= 0)
            return 1024;
        return cus * per_cu;
    }();
    const int64_t per_head = std::max<int64_t>(1, resident / Hkv);
    const int P = (int)std::min<int64_t>(items_bound, per_head);
    const float scale_log2 = scale_log2_of(scale);
    hipStream_t st = (hipStream_t)stream;
    hipLaunchKernelGGL(decode_split_kernel, dim3(P, Hkv), dim3(kThreads), 0, st,
                       (const uint16_t*)q, ldq, (const uint16_t*)k_cache, (const uint16_t*)v_cache,
                       num_blocks, block_table, max_blocks, kv_lens, S, Hq, Hkv, max_splits, split_len,
                       scale_log2, (float*)ws, (uint16_t*)out, ldo);
    int rc = bi_launch_status();
    if (rc != BI_OK) return rc;
    hipLaunchKernelGGL(decode_combine_kernel, dim3(Hq, S), dim3(kD), 0, st, (const float*)ws,
                       kv_lens, std::min(max_blocks * kBlock, max_splits * split_len), Hq, max_splits,
                       split_len, (uint16_t*)out, ldo);
    return bi_launch_status();
}

}  // namespace

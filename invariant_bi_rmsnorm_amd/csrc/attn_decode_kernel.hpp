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
// P^T buffer: the 16-byte unit of query column col, token group grp, chunk c
// (8 weights) sits at unit (4 c + grp) * 16 + col, so the 16 lanes of one
// group touch 256 contiguous bytes; measured on gfx950 this halves the
// split kernel's LDS bank-conflict cycles against rows padded to 544 bytes
// (528-byte rows are worse), for the same time: the kernel waits on HBM
__device__ __forceinline__ int pt_index(int c, int grp, int col) { return ((4 * c + grp) * 16 + col) * 8; }
// floats per item in the (m, l) region: one 128-byte line, the pairs of up to
// 16 query columns
constexpr int kMlFloats = 32;
static_assert(kSplit * 16 <= kSplit * kD, "P^T fits in the K buffer it aliases");

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

// The KV cache is read once per call, so its loads are marked non-temporal
// (cache policy NT; for the LDS-DMA builtin the policy argument): streamed
// through, they do not push the split partials out of L2 and the MALL, which
// measured 6 % faster at 256 sequences of up to 32K tokens.
constexpr int kStreamPolicy = 2;

// loads issued per lane per item for the values operands (all unconditional,
// so the count is fixed: the wait for K below leaves exactly these in flight)
constexpr int kVLoads = 2 * kChunks;

// K rows of a split are staged in LDS (256 B per token row); 16-byte chunk ch
// of row r sits at slot ch ^ kswz(r), so the 16 rows one MFMA operand read
// touches fall in distinct banks.
__device__ __forceinline__ int kswz(int row) { return (row & 3) | (((row >> 3) & 3) << 2); }

__global__ __launch_bounds__(kThreads, 2) void decode_split_kernel(
    const uint16_t* __restrict__ q, int64_t ldq, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, int64_t num_blocks, const int32_t* __restrict__ bt,
    int max_blocks, const int32_t* __restrict__ kv_lens, int S, int Hq, int Hkv,
    int max_splits, int split_len, float scale_log2, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    uint16_t* __restrict__ out, int64_t ldo, unsigned* __restrict__ tickets)
{
    __shared__ int s_off[kMaxSeqs + 1];
    __shared__ int s_part[kThreads];
    __shared__ float s_max[4][16];
    __shared__ int s_ticket;
    // K of the split [256][128] bf16; after the scores it holds P^T (pt_index)
    __shared__ __attribute__((aligned(1024))) uint16_t s_k[kSplit * kD];
    uint16_t* const s_pt = s_k;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 15;
    const int grp = lane >> 4;
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
    // work items are (split, KV head) pairs, ticket t = item * Hkv + head:
    // a workgroup takes tickets blockIdx.x and blockIdx.x + gridDim.x, then
    // draws 2 gridDim.x + (a counter the host zeroes before the launch), so
    // the workgroups that run faster take more items and all finish together
    const int n_tickets = total * Hkv;
    const int P = (int)gridDim.x;
    if ((int)blockIdx.x >= n_tickets) return;      // uniform over the workgroup

    // sequence and split index of item w: the largest s with s_off[s] <= w
    auto locate = [&](int w, int& s_, int& i_) __attribute__((always_inline)) {
        int lo = 0, hi = S - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_off[mid] <= w) lo = mid; else hi = mid - 1;
        }
        s_ = lo;
        i_ = w - s_off[lo];
    };
    // every lane loads the sequence length and the table entry of block
    // (lane & 15) of an item (16 blocks of 16 tokens cover a split); entries
    // past the sequence are read from inside the table row and masked later
    auto raw_len = [&](int s_) __attribute__((always_inline)) { return kv_lens[s_]; };
    auto raw_blk = [&](int s_, int i_) __attribute__((always_inline)) {
        const int b = min(((i_ * split_len) >> 4) + (tid & 15), max_blocks - 1);
        return bt[(int64_t)s_ * max_blocks + b];
    };

    // physical block of this lane's block (lane & 15) of the split starting at
    // token t0_: -1 where the block holds no token of the split or its id is
    // outside the pool.  Tokens of such a block do not exist for the
    // arithmetic (score -inf, weight 0, value 0; their K rows are never
    // loaded, so nothing stale from an earlier item can reach the result).
    auto lane_block = [&](int t0_, int Lseq_, int blk_raw) __attribute__((always_inline)) {
        const int L_ = min(Lseq_, t0_ + split_len);
        return (t0_ + kBlock * (tid & 15) < L_ && blk_raw >= 0 && blk_raw < num_blocks) ? blk_raw : -1;
    };

    // an item's length and block ids are loaded one item ahead (and taken
    // from registers after the wait for the previous item's values), and its
    // sequence is located two items ahead, so no item starts with a wait on
    // global memory
    // Results leave in as few store instructions as possible: each store
    // instruction holds up the CU's memory pipeline far longer than its bytes
    // take, so a wave gathers its values with cross-lane reads into one
    // full-width store (two or three for more than 7 query heads per KV head).
    // Lane (col, grp) holds dims 16 (2 wave + dd) + 4 grp + r of query column
    // col.  Every partial line is written whole by one wavefront (lines
    // written in part at different times cost HBM more).  The first store's
    // data and addresses are returned (it is issued later, with every lane
    // on: lanes without a value of their own repeat another lane's value and
    // address, so no branch makes the number of store instructions vary); any
    // other store is issued here.
    auto store_prepare = [&](const f32x4 (&o_)[2], float ls_, float m_, int s_, int i_, int g_, bool single,
                             u32x4& st_v, uint32_t*& st_p) __attribute__((always_inline)) {
        if (single) {
            // the sequence's only split: its fold is the split itself, so the
            // output is o / l, rounded, exactly what the combine would write.
            // Store lane t = 4 hh + j (hh < G): dims 32 wave + 8 j .. + 7 of
            // head g G + hh, from lanes (hh, 2 (j & 1)) and (hh, 2 (j & 1) + 1),
            // values dd = j >> 1.  (A shuffle reads the source lane's value:
            // both candidates are read and the destination lane picks.)
            u32x4 pk;                                   // this lane's 8 values, rounded
            pk[0] = pack_bf16x2(finish_value(o_[0][0], ls_), finish_value(o_[0][1], ls_));
            pk[1] = pack_bf16x2(finish_value(o_[0][2], ls_), finish_value(o_[0][3], ls_));
            pk[2] = pack_bf16x2(finish_value(o_[1][0], ls_), finish_value(o_[1][1], ls_));
            pk[3] = pack_bf16x2(finish_value(o_[1][2], ls_), finish_value(o_[1][3], ls_));
            const int t = lane % (4 * G);                // 4 G <= 64 lanes carry values
            const int hh = t >> 2;
            const int j = t & 3;
            const int srcA = hh + 16 * (2 * (j & 1));
            const int srcB = srcA + 16;
            const bool hi = (j >> 1) != 0;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const uint32_t a0 = (uint32_t)__shfl((int)pk[e], srcA, 64);
                const uint32_t a1 = (uint32_t)__shfl((int)pk[2 + e], srcA, 64);
                const uint32_t b0 = (uint32_t)__shfl((int)pk[e], srcB, 64);
                const uint32_t b1 = (uint32_t)__shfl((int)pk[2 + e], srcB, 64);
                st_v[e] = hi ? a1 : a0;
                st_v[2 + e] = hi ? b1 : b0;
            }
            st_p = (uint32_t*)(out + (int64_t)s_ * ldo + (int64_t)(g_ * G + hh) * kD + 32 * wave + 8 * j);
            return;
        }
        // o rows: store lane t = 8 hh + j (hh < G) writes dims 32 wave + 4 j
        // .. + 3 of head g G + hh, from lane (hh, j & 3), values dd = j >> 2;
        // on wave 0 the 8 lanes after them (when G <= 7) write the item's
        // (m, l) line: lane 8 G + k holds the pairs of columns 2k, 2k + 1
        const int n_o = 8 * G;
        const bool ml_inline = n_o + 8 <= 64;
        float* const mrow = ws_ml + (((int64_t)s_ * Hkv + g_) * max_splits + i_) * kMlFloats;
        // lanes of the first store without a value: lane l repeats lane
        // l mod n_store (n_store = the lanes with values)
        const int n_store = min(64, ml_inline && wave == 0 ? n_o + 8 : n_o);
        for (int base = 0; base < n_o; base += 64) {          // one pass while G <= 8
            const int t = base == 0 ? lane % n_store : base + lane;
            const int hh = (t >> 3) & 15;
            const int j = t & 7;
            const int src = hh + 16 * (j & 3);
            const bool hi = (j >> 2) != 0;
            f32x4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float v0 = __shfl(o_[0][r], src, 64);
                const float v1 = __shfl(o_[1][r], src, 64);
                v[r] = hi ? v1 : v0;
            }
            float* dst = ws_o + (((int64_t)s_ * Hq + g_ * G + hh) * max_splits + i_) * kD + 32 * wave + 4 * j;
            const bool on = t < n_o;
            if (base == 0 && ml_inline && wave == 0) {
                const int k = (t - n_o) & 7;
                f32x4 ml;
                ml[0] = __shfl(m_, 2 * k, 64);
                ml[1] = __shfl(ls_, 2 * k, 64);
                ml[2] = __shfl(m_, 2 * k + 1, 64);
                ml[3] = __shfl(ls_, 2 * k + 1, 64);
                if (!on) {
                    v = ml;
                    dst = mrow + 4 * k;
                }
            }
            if (base == 0) {
                st_v = __builtin_bit_cast(u32x4, v);
                st_p = (uint32_t*)dst;
            } else if (on) {
                *reinterpret_cast<f32x4*>(dst) = v;
            }
        }
        if (!ml_inline && wave == 0 && grp == 0) {
            f32x2_t ml;
            ml[0] = m_;
            ml[1] = ls_;
            *reinterpret_cast<f32x2_t*>(mrow + 2 * col) = ml;
        }
    };

    // An item's first store is issued after the next item's value loads, so
    // no counted wait of the wave waits for a fresh store (a store counts in
    // vmcnt like a load, and under load its completion comes back late): the
    // K wait allows the value loads and that one store to be in flight, the
    // value wait the store.  Every iteration issues exactly that one store
    // instruction; before the first item it writes zeros into the spare
    // second half of the ticket line.
    u32x4 st_v = {0u, 0u, 0u, 0u};
    uint32_t* st_p = (uint32_t*)((char*)tickets + 128 + 16 * (lane & 7));

    // sequence, split and KV head of ticket t (tickets past the last read the
    // last item's entries: their loads stay in bounds and are never used)
    auto ticket_item = [&](int t, int& s_, int& i_, int& g_) __attribute__((always_inline)) {
        const int tc = min(t, n_tickets - 1);
        const int item = tc / Hkv;
        g_ = tc - item * Hkv;
        locate(item, s_, i_);
    };
    int t_cur = blockIdx.x, t_next = blockIdx.x + P;
    int cs, ci, cg, ns, ni, ng;
    ticket_item(t_cur, cs, ci, cg);
    int c_Lseq = clamp_len(raw_len(cs), cap);
    int c_blk = lane_block(ci * split_len, c_Lseq, raw_blk(cs, ci));
    ticket_item(t_next, ns, ni, ng);

    while (t_cur < n_tickets) {
        // loads of the next item, and the ticket of the one after, issued
        // ahead of this item's operand loads
        const int n_len = raw_len(ns);
        const int n_blk = raw_blk(ns, ni);
        // (an increment-with-wrap at 2^32 - 1 is a plain increment; unlike an
        // add it is issued as one atomic whose result is waited for only where
        // it is used)
        unsigned drawn = 0;
        if (tid == 0) drawn = __builtin_amdgcn_atomic_inc32(tickets, 0xffffffffu, __ATOMIC_RELAXED, "agent");
        asm volatile("" ::: "memory");

        const int s = cs;
        const int i = ci;
        const int g = cg;
        const int Lseq = c_Lseq;
        const int t0 = i * split_len;
        // tokens of this split: [t0, L); with split_len == 256 (the library's
        // only value) L is the sequence length
        const int L = min(Lseq, t0 + split_len);
        const int my_blk = c_blk;
        int blk16[kSplit / kBlock];                  // the 16 ids, wave-uniform
#pragma unroll
        for (int b = 0; b < kSplit / kBlock; ++b) blk16[b] = __builtin_amdgcn_readlane(my_blk, b);
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
                    s_k + inst * 512, 16, 0, kStreamPolicy);
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
                vv[c][dd] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4*>(vc + (((int64_t)b * Hkv + g) * kD + d) * kBlock + (tok & 15)));
            }
        }
        __builtin_nontemporal_store(st_v, reinterpret_cast<u32x4*>(st_p));

        // this wave's q and K loads have landed (only the kVLoads value loads
        // and the store issued after them may still fly); then every wave's K has
        constexpr int kW1 = kVLoads + 1;
        __builtin_amdgcn_s_waitcnt((kW1 & 0xF) | ((kW1 >> 4) << 14) | (0x7 << 4));
        asm volatile("s_barrier" ::: "memory");
        // (the ticket drawn above has landed with the q and K loads; the other
        // waves read it after the next barrier)
        if (tid == 0) s_ticket = 2 * P + (int)drawn;
        bf16x8 qf[4];
#pragma unroll
        for (int dc = 0; dc < 4; ++dc) qf[dc] = as_bf16x8(q_for_scale(qok ? qraw[dc] : zero_u32x4(), scale_log2));

        // block of tokens 32 c + 8 grp .. + 7 for the two chunks c = 2 wave + cc
        // this wave scores (a lane read across the wave, no LDS round trip)
        bool blk_ok[2];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
            blk_ok[cc] = whole || __shfl(my_blk, 2 * (2 * wave + cc) + (grp >> 1), 64) >= 0;

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
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 4 * h + r;
                    const bool valid = whole || (blk_ok[cc] && (t0 + 32 * c + 8 * grp + j) < L);
                    sv[cc][j] = valid ? acc[r] : -INFINITY;
                }
            }
        }

        // split max across the four waves (of the raw scores; scaled once)
        float mx = -INFINITY;
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int j = 0; j < 8; ++j) mx = fmaxf(mx, sv[cc][j]);
        mx = colmax_finish(mx);
        if (grp == 0) s_max[wave][col] = mx;
        lds_barrier();
        const float c_scale = c_of_scale(scale_log2);
        const float m = split_max(fmaxf(fmaxf(s_max[0][col], s_max[1][col]), fmaxf(s_max[2][col], s_max[3][col])),
                                  c_scale);
        const int t_after = s_ticket;
        int s2, i2, g2;
        ticket_item(t_after, s2, i2, g2);

        // bf16 weights -> LDS as P^T[q][token]
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            const int c = 2 * wave + cc;
            float wv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                wv[j] = whole ? weight_of(sv[cc][j], c_scale, m) : weight_of_masked(sv[cc][j], c_scale, m);
            st16(&s_pt[pt_index(c, grp, col)], as_u32x4(pack_weights(wv)));
        }
        lds_barrier();

        // the value operands have landed; zero the slots of tokens past the
        // sequence or in a block outside the pool
        __builtin_amdgcn_s_waitcnt(0x0071);                      // vmcnt(1): the store may fly
        // (the next item's loads, issued before this item's, have landed too)
        const int n_Lseq = clamp_len(n_len, cap);
        const int n_myblk = lane_block(ni * split_len, n_Lseq, n_blk);
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
        f32x4 lacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            const bf16x8 pf = as_bf16x8(ld16(&s_pt[pt_index(c, grp, col)]));
            lacc = lsum_step(pf, lacc);
#pragma unroll
            for (int dd = 0; dd < 2; ++dd) o[dd] = pv_step(as_bf16x8(vv[c][dd]), pf, o[dd]);
        }
        const float ls = lacc[0];

        store_prepare(o, ls, m, s, i, g, t0 == 0 && Lseq <= split_len, st_v, st_p);
        lds_barrier();     // s_max / s_pt are reused by the next item
        c_Lseq = n_Lseq;
        c_blk = n_myblk;
        t_cur = t_next;
        t_next = t_after;
        cs = ns;
        ci = ni;
        cg = ng;
        ns = s2;
        ni = i2;
        ng = g2;
    }
    *reinterpret_cast<u32x4*>(st_p) = st_v;
}

// Runs before the split kernel: zeroes its ticket counter (a kernel rather
// than a memset, so the launch sequence can be captured in a HIP graph and
// replayed), and writes the zero output of every sequence with no token
// (kv_len <= 0), which no split covers.  Wavefront w of the grid takes
// sequence w; 256 threads per workgroup.
constexpr size_t kTicketBytes = 256;
__global__ __launch_bounds__(256) void decode_ticket_reset(unsigned* __restrict__ tickets,
                                                           const int32_t* __restrict__ kv_lens, int cap, int S,
                                                           int Hq, uint16_t* __restrict__ out, int64_t ldo)
{
    if (blockIdx.x == 0 && threadIdx.x == 0) *tickets = 0u;
    const int s = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (s >= S || clamp_len(kv_lens[s], cap) != 0) return;      // wave-uniform
    const int lane = threadIdx.x & 63;
    uint16_t* row = out + (int64_t)s * ldo;              // out is only 2-byte aligned
    for (int e = lane; e < Hq * kD; e += 64) row[e] = 0;
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
// registers.  Partial values are loaded kPre splits at a time, the next
// batch issued before the current one folds.
constexpr int kFoldChunk = kD;
constexpr int kPre = 32;

__global__ __launch_bounds__(kD) void decode_combine_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_ml, const int32_t* __restrict__ kv_lens,
    int cap, int Hq, int Hkv, int max_splits, int split_len, uint16_t* __restrict__ out, int64_t ldo)
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
    if (n <= 1) return;            // written by the split kernel (n = 1) or decode_ticket_reset (n = 0)
    const int G = Hq / Hkv;
    const int g = h / G;
    const float* base = ws_o + ((int64_t)s * Hq + h) * max_splits * kD;
    const float* mlb = ws_ml + ((int64_t)s * Hkv + g) * max_splits * kMlFloats + 2 * (h - g * G);
    float Mprev = -INFINITY, Lam = 0.f, O = 0.f;
    for (int c0 = 0; c0 < n; c0 += kFoldChunk) {
        const int cn = min(kFoldChunk, n - c0);
        const float* cb = base + (int64_t)c0 * kD;
        // ---- scalar part: thread d owns split c0 + d
        const bool own = d < cn;
        const float* ml = mlb + (int64_t)(c0 + d) * kMlFloats;
        const float mi = own ? ml[0] : -INFINITY;
        const float li = own ? ml[1] : 0.f;
        float v[kPre];
#pragma unroll
        for (int j = 0; j < kPre; ++j) v[j] = j < cn ? cb[(int64_t)j * kD + d] : 0.f;
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
        // ---- the two chains, in split order; the next kPre partials load
        // while this batch folds
        for (int i0 = 0; i0 < cn; i0 += kPre) {
            float vn[kPre];
            if (i0 + kPre < cn) {
#pragma unroll
                for (int j = 0; j < kPre; ++j)
                    vn[j] = i0 + kPre + j < cn ? cb[(int64_t)(i0 + kPre + j) * kD + d] : 0.f;
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
            if (i0 + kPre < cn) {
#pragma unroll
                for (int j = 0; j < kPre; ++j) v[j] = vn[j];
            }
        }
        Mprev = fmaxf(Mprev, chunk_max);
        __syncthreads();          // the chunk's LDS is reused by the next chunk
    }
    *o = (uint16_t)f32_to_bf16_rne(finish_value(O, Lam));
}

static inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Workspace when splits are `split_len` tokens long, from the first 256-byte
// boundary in it: the ticket counter of the split kernel (kTicketBytes), the o
// rows [S][Hq][splits][D] fp32, then one (m, l) line of kMlFloats per
// (sequence, KV head, split) item.  The host sizes the (m, l) region for
// Hkv == Hq (the size query takes no Hkv); Hkv < Hq uses less of it.
static inline size_t decode_ws_bytes(int32_t S, int32_t Hq, int32_t D, int32_t max_kv_len, int split_len)
{
    if (S <= 0 || Hq <= 0 || D <= 0 || max_kv_len <= 0) return 0;
    const size_t rows = (size_t)S * (size_t)Hq * (size_t)ceil_div64(max_kv_len, split_len);
    return 255 + kTicketBytes + rows * ((size_t)D + kMlFloats) * sizeof(float);
}

struct DecodeWs {
    unsigned* tickets;
    float* o;
    float* ml;
};

static inline DecodeWs decode_ws_layout(void* ws, int32_t S, int32_t Hq, int max_splits)
{
    char* a = (char*)(((uintptr_t)ws + 255) & ~(uintptr_t)255);
    DecodeWs w;
    w.tickets = (unsigned*)a;
    w.o = (float*)(a + kTicketBytes);
    w.ml = w.o + (size_t)S * Hq * max_splits * kD;
    return w;
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
    if (D != kD || Hq / Hkv > 16 || S > kMaxSeqs || max_kv_len > (1 << 20) || Hkv > 256)
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
    // tickets (and the counter's draws past them) stay far inside int range;
    // checked before any device call
    if (items_bound * Hkv > ((int64_t)1 << 30)) return BI_ERR_UNSUPPORTED;
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
    const int P = (int)std::min<int64_t>(items_bound * Hkv, resident);
    const float scale_log2 = scale_log2_of(scale);
    hipStream_t st = (hipStream_t)stream;
    const DecodeWs w = decode_ws_layout(ws, S, Hq, max_splits);
    const int cap = std::min(max_blocks * kBlock, max_splits * split_len);
    hipLaunchKernelGGL(decode_ticket_reset, dim3((S + 3) / 4), dim3(256), 0, st, w.tickets, kv_lens, cap, S, Hq,
                       (uint16_t*)out, ldo);
    int rc = bi_launch_status();
    if (rc != BI_OK) return rc;
    hipLaunchKernelGGL(decode_split_kernel, dim3(P), dim3(kThreads), 0, st,
                       (const uint16_t*)q, ldq, (const uint16_t*)k_cache, (const uint16_t*)v_cache,
                       num_blocks, block_table, max_blocks, kv_lens, S, Hq, Hkv, max_splits, split_len,
                       scale_log2, w.o, w.ml, (uint16_t*)out, ldo, w.tickets);
    rc = bi_launch_status();
    if (rc != BI_OK) return rc;
    // every sequence fits one split: the split kernel has written all outputs
    if (max_splits == 1) return BI_OK;
    hipLaunchKernelGGL(decode_combine_kernel, dim3(Hq, S), dim3(kD), 0, st, (const float*)w.o,
                       (const float*)w.ml, kv_lens, cap, Hq, Hkv, max_splits, split_len, (uint16_t*)out, ldo);
    return bi_launch_status();
}

}  // namespace

// gemm_kernel.hpp -- the GEMM kernel template.  libbi.so instantiates the
// tiles of gemm_tiles.hpp and picks one per call from the shape (gemm.hip
// states the rule and the invariance argument).  The non-invariant baseline
// library reuses the template with the same tiles and a split-K mode; nothing
// in libbi.so splits k.
//
// Per-element reduction order, identical for every tile of the template:
// an fp32 accumulator starts at 0; one v_mfma_f32_16x16x32_bf16 per 32-wide k
// chunk, chunks in ascending k; inside a chunk lane group g supplies
// k = 8g..8g+7; W is the MFMA's A operand (rows = n), A its B operand
// (columns = m).  An MFMA result element depends only on its own row and
// column operands, so the bits of c[m][n] do not depend on the tile, on where
// the tile sits in the grid or on where the row sits in the tile.
#pragma once
#include <type_traits>

#include "bi_common.hpp"

namespace {

// s_waitcnt vmcnt(<= N) lgkmcnt(0), expcnt unconstrained
template <int N>
__device__ __forceinline__ void gemm_wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    constexpr int imm = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4);
    __builtin_amdgcn_s_waitcnt(imm);
}

// the same with a run-time (wave-uniform) count, 0..63 (larger counts wait for 63)
__device__ __forceinline__ void gemm_wait_vm_upto(int n)
{
    switch (n) {
#define GEMM_WAIT_CASE(i) case i: gemm_wait_vm<i>(); break;
#define GEMM_WAIT_CASE8(i) GEMM_WAIT_CASE(i) GEMM_WAIT_CASE(i + 1) GEMM_WAIT_CASE(i + 2) GEMM_WAIT_CASE(i + 3) \
    GEMM_WAIT_CASE(i + 4) GEMM_WAIT_CASE(i + 5) GEMM_WAIT_CASE(i + 6) GEMM_WAIT_CASE(i + 7)
        GEMM_WAIT_CASE8(0) GEMM_WAIT_CASE8(8) GEMM_WAIT_CASE8(16) GEMM_WAIT_CASE8(24)
        GEMM_WAIT_CASE8(32) GEMM_WAIT_CASE8(40) GEMM_WAIT_CASE8(48)
        GEMM_WAIT_CASE(56) GEMM_WAIT_CASE(57) GEMM_WAIT_CASE(58) GEMM_WAIT_CASE(59) GEMM_WAIT_CASE(60)
        GEMM_WAIT_CASE(61) GEMM_WAIT_CASE(62)
#undef GEMM_WAIT_CASE8
#undef GEMM_WAIT_CASE
        default: gemm_wait_vm<63>(); break;
    }
}

// s_waitcnt lgkmcnt(0) only: this wave's LDS reads have returned
__device__ __forceinline__ void gemm_wait_lds() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// workgroup barrier without a memory fence (a fence would also wait for the
// loads still in flight for later stages)
__device__ __forceinline__ void gemm_barrier() { asm volatile("s_barrier" ::: "memory"); }

// one wavefront-wide 1 KB load: 16 bytes per lane, global -> LDS (the LDS
// destination is the wave's base address; lane l lands at byte 16 l); kPol is
// the cache policy (0 default, 2 non-temporal)
template <int kPol = 0>
__device__ __forceinline__ void gemm_load_lds16(const uint16_t* g, uint16_t* l)
{
    __builtin_amdgcn_global_load_lds(g, l, 16, 0, kPol);
}

// kLib tags which library instantiates the tile (0: libbi.so, 1: the baseline),
// so profiles tell their kernels apart; it has no other effect.  kWPol is the
// cache policy of the weight loads.
template <int BM, int BN, int BK, int WM, int WN, int STAGES, int kLib = 0, int WPOL = 0>
struct GemmTile {
    static constexpr int kBM = BM, kBN = BN, kBK = BK, kWM = WM, kWN = WN, kStages = STAGES;
    static constexpr int kWPol = WPOL;
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kChunks = BK / 8;              // 16-byte chunks per row of a k tile
    static constexpr int kRowsPerLoad = 64 / kChunks;   // rows one 1 KB wave load covers
    static constexpr int kALoads = BM / kRowsPerLoad;   // wave loads per stage, A and W
    static constexpr int kWLoads = BN / kRowsPerLoad;
    static constexpr int kAPer = kALoads / kWaves;      // ... per wavefront
    static constexpr int kWPer = kWLoads / kWaves;
    static constexpr int kPer = kAPer + kWPer;
    static constexpr int kStageA = BM * BK;             // bf16 elements per stage
    static constexpr int kStageW = BN * BK;
    static constexpr int kStage = kStageA + kStageW;
    static constexpr int kWRows = BM / WM;              // rows (m) of a wavefront's tile
    static constexpr int kWCols = BN / WN;              // columns (n) of a wavefront's tile
    static constexpr int kTM = kWRows / 16;             // 16 x 16 MFMA tiles per wavefront
    static constexpr int kTN = kWCols / 16;
    static constexpr int kKS = BK / 32;                 // 32-wide k chunks per k tile
    static constexpr int kLdsElems = STAGES * kStage;
    static_assert(kChunks == 8 || kChunks == 16 || kChunks == 32, "k tile of 64, 128 or 256");
    static_assert(kALoads % kWaves == 0 && kWLoads % kWaves == 0, "every wavefront issues the same loads");
    static_assert(kTM >= 1 && kTN >= 1 && kWRows % 16 == 0 && kWCols % 16 == 0, "wavefront tile");
    static_assert(STAGES >= 3, "one stage being read, at least one in flight, one being refilled");
    static_assert((STAGES - 1) * kPer <= 63, "loads in flight per wavefront fit the vmcnt counter");
    static_assert(kLdsElems * 2 <= 160 * 1024, "LDS of one CU");
    // LDS slot of 16-byte chunk c of row r (an involution).  The 16 rows one
    // MFMA operand read touches land in 16 distinct 16-byte slots of a 256-byte
    // bank row, so the reads are free of bank conflicts on gfx950.
    __device__ static __forceinline__ int slot(int row, int c)
    {
        return kChunks >= 16 ? (c ^ (row & 15)) : (c ^ ((row >> 1) & 7));
    }
};

// The 128 x 64 x 128 tile, one of the tiles the library deals outputs with
// (gemm_tiles.hpp); every tile computes each output with the same chain.
using BiTile = GemmTile<128, 64, 128, 4, 2, 3>;
constexpr int kGemmGroup = 4;          // m tiles per band of the tile order

// kSplitK (baseline library only): blockIdx.y = z computes the partial product
// over k in [z K, z K + K) of operands whose rows are longer than K, into the
// fp32 array c + z * c_split_stride.
template <class T, bool kSplitK>
__global__ __launch_bounds__(T::kThreads) void gemm_kernel(
    const uint16_t* __restrict__ a, int64_t lda, const uint16_t* __restrict__ wt, int64_t ldw,
    const uint16_t* __restrict__ bias, void* __restrict__ c, int64_t ldc, int c_f32, int M, int N, int K,
    int64_t c_split_stride)
{
    __shared__ __attribute__((aligned(1024))) uint16_t smem[T::kLdsElems];
    constexpr int BM = T::kBM, BN = T::kBN, BK = T::kBK, S = T::kStages, KS = T::kKS;
    constexpr int TM = T::kTM, TN = T::kTN;

    if (kSplitK) {
        a += (int64_t)blockIdx.y * K;
        wt += (int64_t)blockIdx.y * K;
        c = (float*)c + (int64_t)blockIdx.y * c_split_stride;
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % T::kWM;
    const int wn = wave / T::kWM;
    const int col = lane & 15;
    const int grp = lane >> 4;

    // ---- this workgroup's tile: the tiles in bands of kGemmGroup m tiles,
    // n-major inside a band; the XCDs take contiguous ranges of that order
    // (blocks are dealt to the 8 XCDs round-robin), so the workgroups running
    // together on one XCD share A rows and W rows in that XCD's L2
    const int mt = (M + BM - 1) / BM;
    const int ntl = (N + BN - 1) / BN;
    const int total = mt * ntl;
    const int per_xcd = (total + 7) / 8;
    const int t = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if (t >= total) return;
    const int band = t / (kGemmGroup * ntl);
    const int gm = min(kGemmGroup, mt - band * kGemmGroup);
    const int idx = t - band * kGemmGroup * ntl;
    const int m0 = (band * kGemmGroup + idx % gm) * BM;
    const int n0 = (idx / gm) * BN;

    const int lrow = lane / T::kChunks;      // row within a wave load
    const int lch = lane % T::kChunks;       // LDS slot this lane fills
    const int KT = (K + BK - 1) / BK;
    const int wrow0 = m0 + wm * T::kWRows;
    // 16-row groups of this wavefront holding at least one row < M
    const int tmv = max(0, min(TM, (M - wrow0 + 15) / 16));

    f32x4 acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // LDS offsets (elements, from a stage's base) of this lane's operand reads
    int offw[KS][TN], offa[KS][TM];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int i = 0; i < TN; ++i) {
            const int row = wn * T::kWCols + 16 * i + col;
            offw[ks][i] = T::kStageA + row * BK + T::slot(row, 4 * ks + grp) * 8;
        }
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const int row = wm * T::kWRows + 16 * j + col;
            offa[ks][j] = row * BK + T::slot(row, 4 * ks + grp) * 8;
        }
    }
    // operands of one k tile, all 32-wide chunks, from LDS slot s
    typedef bf16x8 OpW[KS][TN];
    typedef bf16x8 OpA[KS][TM];
    // (kGuard: skip k chunks past K and 16-row groups entirely past M)
    auto read_ops = [&](auto guard, int s, int nks, OpW& fw, OpA& fa) __attribute__((always_inline)) {
        constexpr bool kGuard = decltype(guard)::value;
        const uint16_t* st = smem + s * T::kStage;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (!kGuard || ks < nks) {
#pragma unroll
                for (int i = 0; i < TN; ++i) fw[ks][i] = *reinterpret_cast<const bf16x8*>(st + offw[ks][i]);
#pragma unroll
                for (int j = 0; j < TM; ++j)
                    if (!kGuard || j < tmv) fa[ks][j] = *reinterpret_cast<const bf16x8*>(st + offa[ks][j]);
            }
        }
    };
    // the chain steps of one k tile: chunks ascending
    auto mma = [&](auto guard, int nks, const OpW& fw, const OpA& fa) __attribute__((always_inline)) {
        constexpr bool kGuard = decltype(guard)::value;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            if (!kGuard || ks < nks)
#pragma unroll
                for (int j = 0; j < TM; ++j)
                    if (!kGuard || j < tmv)
#pragma unroll
                        for (int i = 0; i < TN; ++i) acc[i][j] = mfma16(fw[ks][i], fa[ks][j], acc[i][j]);
    };
    constexpr std::false_type kFull{};
    constexpr std::true_type kEdge{};

    // Pipeline (both paths): S LDS stages.  At step kt the MFMAs of k tile kt
    // run on operands read from LDS during step kt-1 while the operands of
    // k tile kt+1 are read, and stage kt+S is loaded into the slot stage kt
    // left once every wavefront has read it (its LDS reads done + barrier).
    OpW fw0, fw1;
    OpA fa0, fa1;
    if (n0 + BN <= N && K % BK == 0) {
        // ---- tile inside N and a whole number of k tiles: no guards.  Rows of
        // the tile past M load row M-1 instead (in bounds; their results are
        // computed and never stored, and no other output reads them)
        // per-lane element offsets from the tile's first row (fixed for the
        // whole k loop; k moves the wave-uniform base)
        uint32_t ga[T::kAPer], gw[T::kWPer];
#pragma unroll
        for (int i = 0; i < T::kAPer; ++i) {
            const int row = (wave + T::kWaves * i) * T::kRowsPerLoad + lrow;
            ga[i] = (uint32_t)(min(row, M - 1 - m0) * lda + T::slot(row, lch) * 8);
        }
#pragma unroll
        for (int i = 0; i < T::kWPer; ++i) {
            const int row = (wave + T::kWaves * i) * T::kRowsPerLoad + lrow;
            gw[i] = (uint32_t)(row * ldw + T::slot(row, lch) * 8);
        }
        const uint16_t* a_tile = a + (int64_t)m0 * lda;
        const uint16_t* w_tile = wt + (int64_t)n0 * ldw;
        auto issue = [&](int kt, int s) __attribute__((always_inline)) {
            uint16_t* sa = smem + s * T::kStage;
            uint16_t* sw = sa + T::kStageA;
            const uint16_t* ak = a_tile + kt * BK;
            const uint16_t* wk = w_tile + kt * BK;
#pragma unroll
            for (int i = 0; i < T::kAPer; ++i)
                gemm_load_lds16(ak + ga[i], sa + (wave + T::kWaves * i) * 512);
#pragma unroll
            for (int i = 0; i < T::kWPer; ++i)
                gemm_load_lds16<T::kWPol>(wk + gw[i], sw + (wave + T::kWaves * i) * 512);
        };
        // Every step issues one stage: past the last k tile it loads the last k
        // tile again into the slot just freed (never read again), so every
        // wait below counts the same loads and one loop covers all k tiles.
#pragma unroll
        for (int s = 0; s < S; ++s) issue(min(s, KT - 1), s);
        gemm_wait_vm<(S - 1) * T::kPer>();           // stage 0 landed (own loads)
        gemm_barrier();
        read_ops(kFull, 0, KS, fw0, fa0);
        auto step = [&](int kt, const OpW& fwc, const OpA& fac, OpW& fwn, OpA& fan) __attribute__((always_inline)) {
            gemm_wait_vm<(S - 2) * T::kPer>();       // stage kt+1 landed (own loads), own reads of kt done
            gemm_barrier();                          // ... for every wavefront
            issue(min(kt + S, KT - 1), kt % S);
            if (kt + 1 < KT) read_ops(kFull, (kt + 1) % S, KS, fwn, fan);
            mma(kFull, KS, fwc, fac);
        };
        int kt = 0;
        for (; kt + 1 < KT; kt += 2) {
            step(kt, fw0, fa0, fw1, fa1);
            step(kt + 1, fw1, fa1, fw0, fa0);
        }
        if (kt < KT) step(kt, fw0, fa0, fw1, fa1);
        gemm_wait_vm<0>();                           // no load may still write this LDS at exit
    } else {
        // ---- edge tile (columns past N, a K tail): rows out of
        // range are neither loaded nor stored; the load count per stage then
        // depends on how many rows are in range (wave-uniform)
        auto issue = [&](int kt, int s) __attribute__((always_inline)) {
            uint16_t* sa = smem + s * T::kStage;
            uint16_t* sw = sa + T::kStageA;
            const int kbase = kt * BK;
#pragma unroll
            for (int i = 0; i < T::kAPer; ++i) {
                const int inst = wave + T::kWaves * i;
                if (m0 + inst * T::kRowsPerLoad < M) {             // wave-uniform
                    const int row = inst * T::kRowsPerLoad + lrow;
                    const int gch = T::slot(row, lch);              // chunk landing at slot lch
                    if (m0 + row < M && kbase + gch * 8 < K)
                        gemm_load_lds16(a + (int64_t)(m0 + row) * lda + kbase + gch * 8, sa + inst * 512);
                }
            }
#pragma unroll
            for (int i = 0; i < T::kWPer; ++i) {
                const int inst = wave + T::kWaves * i;
                if (n0 + inst * T::kRowsPerLoad < N) {
                    const int row = inst * T::kRowsPerLoad + lrow;
                    const int gch = T::slot(row, lch);
                    if (n0 + row < N && kbase + gch * 8 < K)
                        gemm_load_lds16<T::kWPol>(wt + (int64_t)(n0 + row) * ldw + kbase + gch * 8, sw + inst * 512);
                }
            }
        };
        // loads this wavefront issues per stage (wave-uniform, the same for every stage;
        // a load whose first row is in range has at least one active lane)
        int per_stage = 0;
#pragma unroll
        for (int i = 0; i < T::kAPer; ++i) per_stage += (m0 + (wave + T::kWaves * i) * T::kRowsPerLoad < M);
#pragma unroll
        for (int i = 0; i < T::kWPer; ++i) per_stage += (n0 + (wave + T::kWaves * i) * T::kRowsPerLoad < N);
        auto nks_of = [&](int kt) { return min(BK, K - kt * BK) / 32; };
#pragma unroll
        for (int s = 0; s < S; ++s)
            if (s < KT) issue(s, s);
        gemm_wait_vm_upto(min(KT - 1, S - 1) * per_stage);
        gemm_barrier();
        if (tmv > 0) read_ops(kEdge, 0, nks_of(0), fw0, fa0);
        auto step = [&](int kt, const OpW& fwc, const OpA& fac, OpW& fwn, OpA& fan) __attribute__((always_inline)) {
            gemm_wait_lds();                                                    // own reads of stage kt done
            gemm_wait_vm_upto(max(0, min(KT - 2 - kt, S - 2)) * per_stage);     // stage kt+1 landed
            gemm_barrier();
            if (kt + S < KT) issue(kt + S, kt % S);
            if (tmv > 0) {
                if (kt + 1 < KT) read_ops(kEdge, (kt + 1) % S, nks_of(kt + 1), fwn, fan);
                mma(kEdge, nks_of(kt), fwc, fac);
            }
        };
        int kt = 0;
        for (; kt + 1 < KT; kt += 2) {
            step(kt, fw0, fa0, fw1, fa1);
            step(kt + 1, fw1, fa1, fw0, fa0);
        }
        if (kt < KT) step(kt, fw0, fa0, fw1, fa1);
    }

    // ---- epilogue: lane holds c[m = wrow0 + 16 j + col][n = .. + 4 grp + r], r = 0..3
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const int m = wrow0 + 16 * j + col;
            const int n = n0 + wn * T::kWCols + 16 * i + 4 * grp;
            if (m < M && n < N) {
                f32x4 v = acc[i][j];
                if (bias) {                               // addmm: the bias row, after the whole chain
                    const u32x2 bb = *reinterpret_cast<const u32x2*>(bias + n);
                    v[0] = v[0] + bf16_to_f32(bb[0] & 0xffffu);
                    v[1] = v[1] + bf16_to_f32(bb[0] >> 16);
                    v[2] = v[2] + bf16_to_f32(bb[1] & 0xffffu);
                    v[3] = v[3] + bf16_to_f32(bb[1] >> 16);
                }
                if (c_f32) {
                    *reinterpret_cast<f32x4*>((float*)c + (int64_t)m * ldc + n) = v;
                } else {
                    u32x2 p;
                    p[0] = pack_bf16x2(v[0], v[1]);
                    p[1] = pack_bf16x2(v[2], v[3]);
                    *reinterpret_cast<u32x2*>((uint16_t*)c + (int64_t)m * ldc + n) = p;
                }
            }
        }
    }
}

// Host-side validation shared by every bi_matmul build; returns BI_OK to go on,
// or the status to return (M == 0 returns the no-op marker -1).
static inline int gemm_validate(const void* a, int64_t lda, const void* wt, int64_t ldw, const void* c,
                                int64_t ldc, int c_dtype, int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N <= 0 || K <= 0) return BI_ERR_INVALID_ARGUMENT;
    if (c_dtype != BI_BF16 && c_dtype != BI_F32) return BI_ERR_INVALID_ARGUMENT;
    if (lda < K || ldw < K || ldc < N) return BI_ERR_INVALID_ARGUMENT;
    if (M > 0 && (!a || !wt || !c)) return BI_ERR_INVALID_ARGUMENT;
    if ((lda % 8) || (ldw % 8) || (ldc % 4)) return BI_ERR_INVALID_ARGUMENT;
    if (M > 0 && (!bi_aligned(a, 16) || !bi_aligned(wt, 16) ||
                  !bi_aligned(c, c_dtype == BI_F32 ? 16 : 8)))
        return BI_ERR_INVALID_ARGUMENT;
    if ((K % 32) || (N % 4)) return BI_ERR_UNSUPPORTED;
    // per-lane load offsets inside a tile are 32-bit: rows of up to 2^24 elements
    if (lda >= (1LL << 24) || ldw >= (1LL << 24)) return BI_ERR_UNSUPPORTED;
    // no tile dimension exceeds 256; no tile is smaller than 16 x 16
    if (M > 0x7fffffffLL - 256 || N > 0x7fffffffLL - 256 || K > 0x7fffffffLL - 256)
        return BI_ERR_UNSUPPORTED;
    const int64_t tiles = ((M + 15) / 16) * ((N + 15) / 16);
    if (tiles > 0x7fffffffLL - 8) return BI_ERR_UNSUPPORTED;
    if (M == 0) return -1;
    return BI_OK;
}

template <class T, bool kSplitK = false>
static inline int gemm_launch(const void* a, int64_t lda, const void* wt, int64_t ldw, const void* bias,
                              void* c, int64_t ldc, int c_dtype, int64_t M, int64_t N, int64_t K,
                              void* stream, int splits = 1, int64_t c_split_stride = 0)
{
    const int64_t tiles = ((M + T::kBM - 1) / T::kBM) * ((N + T::kBN - 1) / T::kBN);
    const unsigned grid = (unsigned)(((tiles + 7) / 8) * 8);
    hipLaunchKernelGGL((gemm_kernel<T, kSplitK>), dim3(grid, splits), dim3(T::kThreads), 0, (hipStream_t)stream,
                       (const uint16_t*)a, lda, (const uint16_t*)wt, ldw, (const uint16_t*)bias, c, ldc,
                       c_dtype == BI_F32 ? 1 : 0, (int)M, (int)N, (int)K, c_split_stride);
    return bi_launch_status();
}

}  // namespace

// gemm_kernel.hpp -- the one GEMM kernel of the library (see gemm.hip for the
// configuration and the invariance argument).  Template parameter kOrder
// selects the per-element reduction order: 0 is the library's fixed chain
// (the only order bi_matmul in libbi.so ever uses); 1 splits the chain into
// even and odd k chunks summed at the end, an order used only by the
// non-invariant baseline library to reproduce a batch-size-dependent switch.
#pragma once
#include "bi_common.hpp"

namespace {

constexpr int kBM = 64;
constexpr int kBN = 32;
constexpr int kBK = 128;
constexpr int kWM = 4;
constexpr int kWN = 2;
constexpr int kStages = 3;
constexpr int kGroup = 4;                         // m-tiles per band of the tile order
constexpr int kWaves = kWM * kWN;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunks = kBK / 8;                  // 16-byte chunks per row per k-tile
constexpr int kRowsPerInst = 64 / kChunks;        // rows covered by one 1 KB wave load
constexpr int kAPer = kBM / kRowsPerInst / kWaves;
constexpr int kWPer = kBN / kRowsPerInst / kWaves;
constexpr int kStageA = kBM * kBK;                // bf16 elements
constexpr int kStageW = kBN * kBK;
constexpr int kTM = kBM / kWM / 16;
constexpr int kTN = kBN / kWN / 16;
static_assert(kAPer * kRowsPerInst * kWaves == kBM && kWPer * kRowsPerInst * kWaves == kBN, "load split");

// vmcnt <= N and lgkmcnt == 0 (expcnt unconstrained)
template <int N>
__device__ __forceinline__ void wait_vm()
{
    constexpr int imm = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4);
    __builtin_amdgcn_s_waitcnt(imm);
}

__device__ __forceinline__ void wait_vm_upto(int n)
{
    static_assert(kAPer + kWPer <= 16, "wait table");
    switch (n) {
        case 0: wait_vm<0>(); break;
        case 1: wait_vm<1>(); break;
        case 2: wait_vm<2>(); break;
        case 3: wait_vm<3>(); break;
        case 4: wait_vm<4>(); break;
        case 5: wait_vm<5>(); break;
        case 6: wait_vm<6>(); break;
        case 7: wait_vm<7>(); break;
        case 8: wait_vm<8>(); break;
        case 9: wait_vm<9>(); break;
        case 10: wait_vm<10>(); break;
        case 11: wait_vm<11>(); break;
        case 12: wait_vm<12>(); break;
        case 13: wait_vm<13>(); break;
        case 14: wait_vm<14>(); break;
        case 15: wait_vm<15>(); break;
        default: wait_vm<16>(); break;
    }
}

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & (kChunks - 1)); }

template <int kOrder>
__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const uint16_t* __restrict__ a, int64_t lda, const uint16_t* __restrict__ wt, int64_t ldw,
    const uint16_t* __restrict__ bias, void* __restrict__ c, int64_t ldc, int c_f32, int M, int N, int K)
{
    __shared__ __attribute__((aligned(1024))) uint16_t smem[kStages * (kStageA + kStageW)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % kWM;
    const int wn = wave / kWM;
    const int col = lane & 15;
    const int grp = lane >> 4;

    // ---- tile of this workgroup: XCD-contiguous ranges of a grouped order
    const int mt = (M + kBM - 1) / kBM;
    const int ntl = (N + kBN - 1) / kBN;
    const int total = mt * ntl;
    const int per_xcd = (total + 7) / 8;
    const int t = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if (t >= total) return;
    const int band = t / (kGroup * ntl);
    const int gm = min(kGroup, mt - band * kGroup);
    const int idx = t - band * kGroup * ntl;
    const int m0 = (band * kGroup + idx % gm) * kBM;
    const int n0 = (idx / gm) * kBN;

    const int lrow = lane / kChunks;
    const int lch = lane % kChunks;
    const int KT = (K + kBK - 1) / kBK;

    auto issue = [&](int kt, int slot) {
        uint16_t* sa = smem + slot * (kStageA + kStageW);
        uint16_t* sw = sa + kStageA;
        const int kbase = kt * kBK;
#pragma unroll
        for (int i = 0; i < kAPer; ++i) {
            const int inst = wave + kWaves * i;
            if (m0 + inst * kRowsPerInst < M) {                 // wave-uniform
                const int row = inst * kRowsPerInst + lrow;
                const int gch = swz(row, lch);                  // chunk stored at LDS slot lch
                if (m0 + row < M && kbase + gch * 8 < K)
                    __builtin_amdgcn_global_load_lds(a + (int64_t)(m0 + row) * lda + kbase + gch * 8,
                                                     sa + inst * 512, 16, 0, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < kWPer; ++i) {
            const int inst = wave + kWaves * i;
            if (n0 + inst * kRowsPerInst < N) {
                const int row = inst * kRowsPerInst + lrow;
                const int gch = swz(row, lch);
                if (n0 + row < N && kbase + gch * 8 < K)
                    __builtin_amdgcn_global_load_lds(wt + (int64_t)(n0 + row) * ldw + kbase + gch * 8,
                                                     sw + inst * 512, 16, 0, 0);
            }
        }
    };

    // loads this wave issues per stage (wave-uniform, the same for every stage)
    int per_stage = 0;
#pragma unroll
    for (int i = 0; i < kAPer; ++i) per_stage += (m0 + (wave + kWaves * i) * kRowsPerInst < M);
#pragma unroll
    for (int i = 0; i < kWPer; ++i) per_stage += (n0 + (wave + kWaves * i) * kRowsPerInst < N);

    // 16-row groups of this wave that hold at least one row < M
    const int wrow0 = m0 + wm * (kBM / kWM);
    const int tmv = max(0, min(kTM, (M - wrow0 + 15) / 16));

    f32x4 acc[kTN][kTM];
    f32x4 acc2[kTN][kTM];          // second chain, used only by kOrder == 1
#pragma unroll
    for (int i = 0; i < kTN; ++i)
#pragma unroll
        for (int j = 0; j < kTM; ++j) {
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            acc2[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
        if (s < KT) issue(s, s);

    for (int kt = 0; kt < KT; ++kt) {
        // this wave's loads of stage kt have landed (later stages may still fly);
        // then every wave's have, after the barrier
        const int ahead = min(KT - 1 - kt, kStages - 2);
        wait_vm_upto(ahead * per_stage);
        asm volatile("s_barrier" ::: "memory");
        if (kt + kStages - 1 < KT) issue(kt + kStages - 1, (kt + kStages - 1) % kStages);

        const uint16_t* sa = smem + (kt % kStages) * (kStageA + kStageW);
        const uint16_t* sw = sa + kStageA;
        const int nks = min(kBK, K - kt * kBK) / 32;       // 32-wide k chunks in this tile
        // operands of one 32-wide k chunk, read from LDS
        auto read_ops = [&](int ks, bf16x8 (&fw)[kTN], bf16x8 (&fa)[kTM]) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < kTN; ++i) {
                const int row = wn * (kBN / kWN) + 16 * i + col;
                fw[i] = *reinterpret_cast<const bf16x8*>(sw + row * kBK + swz(row, 4 * ks + grp) * 8);
            }
#pragma unroll
            for (int j = 0; j < kTM; ++j) {
                const int row = wm * (kBM / kWM) + 16 * j + col;
                fa[j] = *reinterpret_cast<const bf16x8*>(sa + row * kBK + swz(row, 4 * ks + grp) * 8);
            }
        };
        // the chain step of one k chunk (ascending ks within the tile)
        auto chain = [&](int ks, const bf16x8 (&fw)[kTN], const bf16x8 (&fa)[kTM]) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < kTM; ++j) {
                if (j < tmv) {
#pragma unroll
                    for (int i = 0; i < kTN; ++i) {
                        if (kOrder == 1 && (ks & 1))
                            acc2[i][j] = mfma16(fw[i], fa[j], acc2[i][j]);
                        else
                            acc[i][j] = mfma16(fw[i], fa[j], acc[i][j]);
                    }
                }
            }
        };
        if (tmv > 0) {                                     // wave-uniform: rows < M in this wave's tile
            if (nks == kBK / 32) {
                // whole tile: every operand read is issued before the first MFMA,
                // so the LDS latency is paid once per tile, not once per k chunk
                bf16x8 fw[kBK / 32][kTN], fa[kBK / 32][kTM];
#pragma unroll
                for (int ks = 0; ks < kBK / 32; ++ks) read_ops(ks, fw[ks], fa[ks]);
                __builtin_amdgcn_sched_barrier(0);                 // keep the reads ahead
#pragma unroll
                for (int ks = 0; ks < kBK / 32; ++ks) chain(ks, fw[ks], fa[ks]);
            } else {
                for (int ks = 0; ks < nks; ++ks) {               // K tail
                    bf16x8 fw[kTN], fa[kTM];
                    read_ops(ks, fw, fa);
                    chain(ks, fw, fa);
                }
            }
        }
        // the next iteration's barrier orders these LDS reads before any wave
        // overwrites this slot
    }

    // lane holds c[m = .. + col][n = .. + 4 grp + r], r = 0..3
#pragma unroll
    for (int i = 0; i < kTN; ++i) {
#pragma unroll
        for (int j = 0; j < kTM; ++j) {
            const int m = wrow0 + 16 * j + col;
            const int n = n0 + wn * (kBN / kWN) + 16 * i + 4 * grp;
            if (m < M && n < N) {
                f32x4 v = acc[i][j];
                if (kOrder == 1) v = v + acc2[i][j];
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
    if (M > 0x7fffffffLL - kBM || N > 0x7fffffffLL - kBN || K > 0x7fffffffLL - kBK)
        return BI_ERR_UNSUPPORTED;
    const int64_t tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
    if (tiles > 0x7fffffffLL - 8) return BI_ERR_UNSUPPORTED;
    if (M == 0) return -1;
    return BI_OK;
}

template <int kOrder>
static inline int gemm_launch(const void* a, int64_t lda, const void* wt, int64_t ldw, const void* bias,
                              void* c, int64_t ldc, int c_dtype, int64_t M, int64_t N, int64_t K,
                              void* stream)
{
    const int64_t tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
    const unsigned grid = (unsigned)(((tiles + 7) / 8) * 8);
    hipLaunchKernelGGL(gemm_kernel<kOrder>, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                       (const uint16_t*)a, lda, (const uint16_t*)wt, ldw, (const uint16_t*)bias, c, ldc,
                       c_dtype == BI_F32 ? 1 : 0, (int)M, (int)N, (int)K);
    return bi_launch_status();
}

}  // namespace

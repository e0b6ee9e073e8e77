// gemm.hip -- batch-invariant dense matmul: ONE MFMA tile configuration for
// every shape.
//
// Table row 行列乗算（MatMul） of the post "論文／ブログ「Defeating Nondeterminism
// in LLM Inference」の技術的なポイント" (mobiles-han.blogspot.com), section
// 対応策：バッチ不変なカーネル設計, and the same row in the post
// "元OpenAIの研究者ら、AIの応答が毎回違う理由をついに解明", section
// 解決へのアプローチ: libraries pick split-K or drop the matrix units for some
// sizes, which changes each output's reduction order with the batch; the fix
// is one kernel configuration, decided in advance, for all shapes.
//
// The configuration: workgroup tile 128 (m) x 128 (n) x 64 (k), 256 threads
// = 4 wavefronts in a 2x2 arrangement, each wavefront 64x64 outputs as 4x4
// v_mfma_f32_16x16x32_bf16 tiles.  For an output element c[m][n] the
// accumulation is: fp32 accumulator starts at 0, then one MFMA per 32-wide k
// chunk, chunks in ascending k, always the same instruction with the same
// k-slot assignment.  Nothing in that chain depends on M, N, the tile's
// position in the grid or the row's position in the tile (an MFMA result
// element depends only on its own row and column operands).  No split-K, no
// stream-K, no shape-dependent dispatch.  M and N tails are zero-filled.
#include "bi_common.hpp"

namespace {

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBK = 64;
constexpr int kLds = kBK + 8;          // bf16 per LDS row: 64 + 16 B of padding
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(
    const uint16_t* __restrict__ a, int64_t lda, const uint16_t* __restrict__ wt, int64_t ldw,
    void* __restrict__ c, int64_t ldc, int c_f32, int M, int N, int K)
{
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][kBM * kLds];
    __shared__ __attribute__((aligned(16))) uint16_t sW[2][kBN * kLds];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1;
    const int wn = wave >> 1;
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int n0 = blockIdx.x * kBN;
    const int m0 = blockIdx.y * kBM;

    u32x4 ra[4], rw[4];
    auto gload = [&](int kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int v = tid + kThreads * i;
            const int row = v >> 3;
            const int ch = v & 7;
            const int m = m0 + row;
            const int n = n0 + row;
            ra[i] = zero_u32x4();
            rw[i] = zero_u32x4();
            if (m < M) ra[i] = ld16(a + (int64_t)m * lda + (int64_t)kt * kBK + ch * 8);
            if (n < N) rw[i] = ld16(wt + (int64_t)n * ldw + (int64_t)kt * kBK + ch * 8);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int v = tid + kThreads * i;
            const int row = v >> 3;
            const int ch = v & 7;
            st16(&sA[buf][row * kLds + ch * 8], ra[i]);
            st16(&sW[buf][row * kLds + ch * 8], rw[i]);
        }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int KT = K / kBK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 fw[4], fa[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                fw[i] = as_bf16x8(ld16(&sW[buf][(64 * wn + 16 * i + col) * kLds + 32 * ks + 8 * grp]));
                fa[i] = as_bf16x8(ld16(&sA[buf][(64 * wm + 16 * i + col) * kLds + 32 * ks + 8 * grp]));
            }
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) acc[ni][mi] = mfma16(fw[ni], fa[mi], acc[ni][mi]);
        }
        if (kt + 1 < KT) sstore(buf ^ 1);
        __syncthreads();
    }

    // lane holds c[m = .. + col][n = .. + 4 grp + r], r = 0..3
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int m = m0 + 64 * wm + 16 * mi + col;
            const int n = n0 + 64 * wn + 16 * ni + 4 * grp;
            if (m < M && n < N) {
                const f32x4 v = acc[ni][mi];
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

}  // namespace

extern "C" int bi_matmul(const void* a, int64_t lda, const void* wt, int64_t ldw, void* c,
                         int64_t ldc, int c_dtype, int64_t M, int64_t N, int64_t K, void* stream)
{
    BI_TRY_BEGIN
    if (M < 0 || N <= 0 || K <= 0) return BI_ERR_INVALID_ARGUMENT;
    if (c_dtype != BI_BF16 && c_dtype != BI_F32) return BI_ERR_INVALID_ARGUMENT;
    if (lda < K || ldw < K || ldc < N) return BI_ERR_INVALID_ARGUMENT;
    if (M > 0 && (!a || !wt || !c)) return BI_ERR_INVALID_ARGUMENT;
    if ((lda % 8) || (ldw % 8) || (ldc % 4)) return BI_ERR_INVALID_ARGUMENT;
    if (M > 0 && (!bi_aligned(a, 16) || !bi_aligned(wt, 16) ||
                  !bi_aligned(c, c_dtype == BI_F32 ? 16 : 8)))
        return BI_ERR_INVALID_ARGUMENT;
    if ((K % kBK) || (N % 4)) return BI_ERR_UNSUPPORTED;
    if (M > (int64_t)kBM * 65535 || N > 0x7fffffffLL - kBN || K > 0x7fffffffLL)
        return BI_ERR_UNSUPPORTED;
    if (M == 0) return BI_OK;
    dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM));
    hipLaunchKernelGGL(gemm_kernel, grid, dim3(kThreads), 0, (hipStream_t)stream,
                       (const uint16_t*)a, lda, (const uint16_t*)wt, ldw, c, ldc,
                       c_dtype == BI_F32 ? 1 : 0, (int)M, (int)N, (int)K);
    return bi_launch_status();
    BI_TRY_END
}

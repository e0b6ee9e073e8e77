// gemm_tiles.hpp -- the tiles bi_matmul deals outputs with and the rule that
// picks one from the shape (gemm.hip states why: every tile computes each
// output with the same chain, so the pick changes speed only).  kLib tags the
// instantiating library (0: libbi.so, 1: the non-invariant baseline, which
// uses the same rule where it does not split k) so that profiles tell their
// kernels apart.
#pragma once
#include <mutex>

#include "gemm_kernel.hpp"

namespace {

template <int kLib>
struct GemmTiles {
    using S = GemmTile<64, 32, 128, 4, 2, 3, kLib>;
    using Q = GemmTile<64, 64, 128, 2, 2, 3, kLib>;
    using M = GemmTile<128, 64, 128, 4, 2, 3, kLib>;
    using L = GemmTile<128, 128, 64, 2, 4, 3, kLib>;
    using G = GemmTile<256, 128, 64, 4, 2, 3, kLib>;      // 8 wavefronts of 64 x 64
    // M <= 64: weights read non-temporally (each is read once per call);
    // UpTo16/32/64 serve the M ranges where 64-wide tiles do not fill the CUs
    using Qn = GemmTile<64, 64, 128, 2, 2, 3, kLib, 2>;
    using UpTo16 = GemmTile<16, 16, 256, 1, 1, 4, kLib, 2>;
    using UpTo32 = GemmTile<16, 32, 256, 1, 2, 4, kLib, 2>;
    using UpTo64 = GemmTile<32, 32, 128, 2, 2, 6, kLib, 2>;
};
static_assert(std::is_same<GemmTiles<0>::M, BiTile>::value, "BiTile is the library's 128 x 64 x 128 tile");

inline int device_cus()
{
    static std::mutex mu;
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (cus[dev] <= 0) {
        int n = 0;
        cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
    }
    return cus[dev];
}

template <int kLib>
int gemm_dispatch(const void* a, int64_t lda, const void* wt, int64_t ldw, const void* bias, void* c,
                  int64_t ldc, int c_dtype, int64_t M, int64_t N, int64_t K, void* stream)
{
    using T = GemmTiles<kLib>;
    const int64_t need = (int64_t)device_cus() * 3 / 4;
    int pick = 0;                                    // 0 S, 1 Q, 2 M, 3 L, 4 Qn, 5-7 UpTo16/32/64, 8 G
    if (M <= 64) {
        pick = (N + 63) / 64 >= need ? 4 : M <= 16 ? 5 : M <= 32 ? 6 : 7;
    } else {
        const int64_t cap = (M + 63) / 64 * 64;      // no tile taller than M rounded up to 64
        const int64_t bm[5] = {64, 64, 128, 128, 256}, bn[5] = {32, 64, 64, 128, 128};
        const int code[5] = {0, 1, 2, 3, 8};
        for (int t = 0; t < 5; ++t)
            if (bm[t] <= cap && ((M + bm[t] - 1) / bm[t]) * ((N + bn[t] - 1) / bn[t]) >= need) pick = code[t];
    }
    switch (pick) {
    case 1: return gemm_launch<typename T::Q>(a, lda, wt, ldw, bias, c, ldc, c_dtype, M, N, K, stream);
    case 2: return gemm_launch<typename T::M>(a, lda, wt, ldw, bias, c, ldc, c_dtype, M, N, K, stream);
    case 3: return gemm_launch<typename T::L>(a, lda, wt, ldw, bias, c, ldc, c_dtype, M, N, K, stream);
    case 4: return gemm_launch<typename T::Qn>(a, lda, wt, ldw, bias, c, ldc, c_dtype, M, N, K, stream);
    case 5: return gemm_launch<typename T::UpTo16>(a, lda, wt, ldw, bias, c, ldc, c_dtype, M, N, K, stream);
    case 6: return gemm_launch<typename T::UpTo32>(a, lda, wt, ldw, bias, c, ldc, c_dtype, M, N, K, stream);
    case 7: return gemm_launch<typename T::UpTo64>(a, lda, wt, ldw, bias, c, ldc, c_dtype, M, N, K, stream);
    case 8: return gemm_launch<typename T::G>(a, lda, wt, ldw, bias, c, ldc, c_dtype, M, N, K, stream);
    default: return gemm_launch<typename T::S>(a, lda, wt, ldw, bias, c, ldc, c_dtype, M, N, K, stream);
    }
}

}  // namespace

// kv_append.hip -- write fresh K/V into the paged cache so that attention
// reads cached and fresh tokens through one layout.
//
// Table row アテンション (Attention) of the post "論文／ブログ「Defeating
// Nondeterminism in LLM Inference」の技術的なポイント" (mobiles-han.blogspot.com),
// section 対応策：バッチ不変なカーネル設計: merge cache and current data into one
// consistent layout before attending (the FixedAttention sketch of the post
// 「非決定モード → 決定モード」に切り替える例, section 注意点・補足実装, does it
// with a concatenation).  Attention never reads K/V from the projection output.
//
// Layout (one consistent layout for every token):
//   k_cache [num_blocks][Hkv][16][D]   token-major inside a block
//   v_cache [num_blocks][Hkv][D][16]   dim-major inside a block, so the values
//                                      operand of the MFMA (8 consecutive tokens
//                                      of one dim) is one 16-byte load
// A bitwise copy: no arithmetic.
#include "bi_common.hpp"

namespace {

constexpr int kD = 128;
constexpr int kThreads = 256;          // 32 lanes of 4 dims per head, 8 heads at a time

// one workgroup per token: lane group tid/32 takes heads tid/32, tid/32 + 8, ...;
// each lane moves 4 dims (8 bytes) of K and of V
__global__ __launch_bounds__(kThreads) void kv_append_kernel(
    const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn, int64_t ld,
    const int32_t* __restrict__ slots, uint16_t* __restrict__ kc, uint16_t* __restrict__ vc,
    int64_t num_blocks, int Hkv)
{
    const int64_t t = blockIdx.x;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_blocks * 16) return;
    const int64_t blk = slot >> 4;
    const int off = (int)(slot & 15);
    const int d4 = (threadIdx.x & 31) * 4;
    for (int h = threadIdx.x >> 5; h < Hkv; h += kThreads / 32) {
        const int64_t src = t * ld + (int64_t)h * kD + d4;
        const u32x2 kv = *reinterpret_cast<const u32x2*>(kn + src);
        const u32x2 vv = *reinterpret_cast<const u32x2*>(vn + src);
        *reinterpret_cast<u32x2*>(kc + ((blk * Hkv + h) * 16 + off) * kD + d4) = kv;
        uint16_t* vd = vc + ((blk * Hkv + h) * kD + d4) * 16 + off;
        vd[0] = (uint16_t)(vv[0] & 0xffffu);
        vd[16] = (uint16_t)(vv[0] >> 16);
        vd[32] = (uint16_t)(vv[1] & 0xffffu);
        vd[48] = (uint16_t)(vv[1] >> 16);
    }
}

}  // namespace

extern "C" int bi_kv_append(const void* k_new, const void* v_new, int64_t ld_new,
                            const int32_t* slots, int64_t T, void* k_cache, void* v_cache,
                            int64_t num_blocks, int32_t Hkv, int32_t D, void* stream)
{
    BI_TRY_BEGIN
    if (T < 0 || Hkv <= 0 || D <= 0 || num_blocks <= 0) return BI_ERR_INVALID_ARGUMENT;
    if (ld_new < (int64_t)Hkv * D || (ld_new % 8)) return BI_ERR_INVALID_ARGUMENT;
    if (T > 0 && (!k_new || !v_new || !slots || !k_cache || !v_cache)) return BI_ERR_INVALID_ARGUMENT;
    if (T > 0 && (!bi_aligned(k_new, 16) || !bi_aligned(v_new, 16) || !bi_aligned(k_cache, 16) ||
                  !bi_aligned(v_cache, 16) || !bi_aligned(slots, 4)))
        return BI_ERR_INVALID_ARGUMENT;
    if (D != kD || Hkv > 65535 || T > 0x7fffffffLL) return BI_ERR_UNSUPPORTED;
    if (T == 0) return BI_OK;
    hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)T), dim3(kThreads), 0, (hipStream_t)stream,
                       (const uint16_t*)k_new, (const uint16_t*)v_new, ld_new, slots,
                       (uint16_t*)k_cache, (uint16_t*)v_cache, num_blocks, Hkv);
    return bi_launch_status();
    BI_TRY_END
}

// attn_decode.hip -- paged decode attention with fixed-SIZE KV splits.
//
// Table row アテンション (Attention) of the post "論文／ブログ「Defeating
// Nondeterminism in LLM Inference」の技術的なポイント" (mobiles-han.blogspot.com),
// section 対応策：バッチ不変なカーネル設計: Split-KV / FlashDecode must use a fixed
// split SIZE, so the split boundaries of a sequence never move with the batch,
// the length mix or the number of sequences.
//
// Three kernels:
//  0. decode_ticket_reset zeroes the work counter at the head of the workspace
//     and writes the zero output of sequences with no token.
//  1. decode_split_kernel: persistent workgroups (as many as fit on the GPU at
//     once) over the work list of (sequence, split, KV head) items.  Each
//     workgroup first builds the prefix of split counts ceil(kv_len/256) of
//     all sequences in LDS (integer, exact), then takes two items by its index
//     and the rest from the counter, so faster workgroups take more items and
//     the grid drains together.  Which workgroup computes an item has no
//     influence on its arithmetic.  The next item's length and block ids are
//     loaded while the current one is computed; an item's results leave in
//     one store instruction per wavefront (gathered across lanes), issued
//     after the next item's value loads so that no wait covers it; the KV
//     cache is read with non-temporal loads.
//     Per item: 4 wavefronts each score 64 of the split's 256 tokens for the
//     (up to 16) query heads of the KV group, the split max is taken across
//     the waves, the bf16 weights go to LDS as P^T, and each wave then runs
//     the values chain of the whole split for 32 of the 128 head dims.  The
//     split's (m, l, o[128]) is written, fp32, to the workspace.
//  2. decode_combine_kernel: per (sequence, query head), fold the splits in
//     ascending order and divide; not launched when max_kv_len <= 256 (every
//     sequence is one split, finished by the split kernel).
// All arithmetic goes through attn_core.hpp, shared with the prefill kernel,
// which is why decode at length L equals prefill row L-1 bit for bit.
#include <mutex>

#include "attn_decode_kernel.hpp"

extern "C" size_t bi_attention_workspace_bytes(int32_t S, int32_t Hq, int32_t D, int32_t max_kv_len)
{
    return decode_ws_bytes(S, Hq, D, max_kv_len, kSplit);
}

extern "C" int bi_attention_decode(const void* q, int64_t ldq, const void* k_cache,
                                   const void* v_cache, int64_t num_blocks,
                                   const int32_t* block_table, int32_t max_blocks,
                                   const int32_t* kv_lens, void* out, int64_t ldo, int32_t S,
                                   int32_t Hq, int32_t Hkv, int32_t D, int32_t max_kv_len,
                                   float scale, void* ws, size_t ws_bytes, void* stream)
{
    BI_TRY_BEGIN
    const int v = decode_validate(q, ldq, k_cache, v_cache, num_blocks, block_table, max_blocks, kv_lens,
                                  out, ldo, S, Hq, Hkv, D, max_kv_len, scale, ws);
    if (v != BI_OK) return v < 0 ? BI_OK : v;
    if (ws_bytes < decode_ws_bytes(S, Hq, D, max_kv_len, kSplit)) return BI_ERR_WORKSPACE_TOO_SMALL;
    return decode_launch(q, ldq, k_cache, v_cache, num_blocks, block_table, max_blocks, kv_lens, out, ldo,
                         S, Hq, Hkv, max_kv_len, scale, ws, kSplit, stream);
    BI_TRY_END
}

// ---------------------------------------------------------------------------
// Allocation-free variant, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  The split partials go to `scratch`, an array of this library in
// device memory: each GPU the library runs on holds its own copy, at its own
// address, until the process ends.  The array's name is a host-side stand-in:
// host code only ever passes the address hipGetSymbolAddress returns for the
// current device.  The partials of a call are all written by its split kernel
// before its combine kernel reads them, and the work counter at the array's
// head is zeroed by the call's first kernel, so nothing has to be cleared
// between calls; calls that overlap on one GPU share the array and race.
constexpr size_t kNoAllocScratchBytes = BI_ATTENTION_DECODE_NOALLOC_SCRATCH_BYTES;
constexpr int kNoAllocMaxDevices = 64;
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

// Address of this device's copy of `scratch` (looked up once per device, with
// that device current), or nullptr with *status set.
static void* noalloc_scratch(int* status)
{
    static std::mutex mu;
    static void* addr[kNoAllocMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoAllocMaxDevices) {
        *status = BI_ERR_NO_DEVICE;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            *status = BI_ERR_NO_DEVICE;
            return nullptr;
        }
        addr[dev] = p;
    }
    return addr[dev];
}

extern "C" int bi_attention_decode_noalloc(const void* q, int64_t ldq, const void* k_cache,
                                           const void* v_cache, int64_t num_blocks,
                                           const int32_t* block_table, int32_t max_blocks,
                                           const int32_t* kv_lens, void* out, int64_t ldo, int32_t S,
                                           int32_t Hq, int32_t Hkv, int32_t D, int32_t max_kv_len,
                                           float scale, void* stream)
{
    BI_TRY_BEGIN
    const int v = decode_validate(q, ldq, k_cache, v_cache, num_blocks, block_table, max_blocks, kv_lens,
                                  out, ldo, S, Hq, Hkv, D, max_kv_len, scale, nullptr, false);
    if (v != BI_OK) return v < 0 ? BI_OK : v;
    // the size bound is checked on the host, before any device call
    if (decode_ws_bytes(S, Hq, D, max_kv_len, kSplit) > kNoAllocScratchBytes) return BI_ERR_WORKSPACE_TOO_SMALL;
    int status = BI_OK;
    void* ws = noalloc_scratch(&status);
    if (!ws) return status;
    return decode_launch(q, ldq, k_cache, v_cache, num_blocks, block_table, max_blocks, kv_lens, out, ldo,
                         S, Hq, Hkv, max_kv_len, scale, ws, kSplit, stream);
    BI_TRY_END
}

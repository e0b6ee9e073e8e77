// toy_ops.hip -- element-wise ops of the toy greedy-decode step: embedding
// gather, rotary embedding, residual add, SiLU * mul, row gather.
//
// The pages' experiment (page "la température zéro n'est pas déterministe",
// introduction; post 論文／ブログ「Defeating Nondeterminism in LLM Inference」の
// 技術的なポイント, section 実装上の工夫：ツールとライブラリ) decodes one prompt
// greedily 1000 times through a served transformer.  These ops are the parts of
// that transformer that do not reduce: each output element depends on a fixed
// set of input elements through a fixed expression, so they are batch
// invariant by construction (one thread per element or pair, no reduction).
#include <math.h>

#include "bi_common.hpp"

namespace {

__global__ void embed_kernel(const uint16_t* __restrict__ table, int64_t V, int64_t H,
                             const int32_t* __restrict__ ids, uint16_t* __restrict__ out, int64_t ldo)
{
    const int64_t t = blockIdx.x;
    const int64_t id = ids[t];
    const bool ok = id >= 0 && id < V;
    for (int64_t j = threadIdx.x * 8; j < H; j += blockDim.x * 8) {
        u32x4 v = zero_u32x4();
        if (ok) v = ld16(table + id * H + j);
        st16(out + t * ldo + j, v);
    }
}

// table[p][i] = (cos, sin) of p * theta^(-2i/D), evaluated in double, stored fp32
__global__ void rope_table_kernel(float* __restrict__ table, int max_pos, int half, int D, double theta)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= (int64_t)max_pos * half) return;
    const int p = (int)(k / half);
    const int i = (int)(k % half);
    const double ang = (double)p * pow(theta, -2.0 * (double)i / (double)D);
    table[2 * k] = (float)cos(ang);
    table[2 * k + 1] = (float)sin(ang);
}

// in place on [T][ldx] rows; heads [0, H) of each row; pair (i, i + D/2)
__global__ void rope_kernel(uint16_t* __restrict__ x, int64_t ldx, int D, const int32_t* __restrict__ pos,
                            const float* __restrict__ table, int max_pos)
{
    const int64_t t = blockIdx.x;
    const int h = blockIdx.y;
    const int half = D >> 1;
    int p = pos[t];
    if (p < 0 || p >= max_pos) p = 0;
    uint16_t* r = x + t * ldx + (int64_t)h * D;
    for (int i = threadIdx.x; i < half; i += blockDim.x) {
        const float c = table[2 * ((int64_t)p * half + i)];
        const float s = table[2 * ((int64_t)p * half + i) + 1];
        const float a = bf16_to_f32(r[i]);
        const float b = bf16_to_f32(r[i + half]);
        r[i] = (uint16_t)f32_to_bf16_rne(a * c - b * s);
        r[i + half] = (uint16_t)f32_to_bf16_rne(b * c + a * s);
    }
}

// Rotary embedding of q and k and the paged-cache append of k and v for one
// token per workgroup: the q heads are rotated in place; each k pair is
// rotated in registers, written back and written to the K cache; v is copied
// to the dim-major V cache.  The rotation is rope_kernel's arithmetic, the
// cache layout bi_kv_append's (k_cache [blocks][Hkv][16][D], v_cache
// [blocks][Hkv][D][16]); a slot outside the pool writes no cache entry.
constexpr int kRopeAppendThreads = 256;
__global__ __launch_bounds__(kRopeAppendThreads) void rope_kv_append_kernel(
    uint16_t* __restrict__ qkv, int64_t ld, int Hq, int Hkv, int D, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ slots, const float* __restrict__ table, int max_pos,
    uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, int64_t num_blocks)
{
    const int64_t t = blockIdx.x;
    const int half = D >> 1;
    int p = pos[t];
    if (p < 0 || p >= max_pos) p = 0;
    const int64_t slot = slots[t];
    const bool cached = slot >= 0 && slot < num_blocks * 16;
    const int64_t blk = slot >> 4;
    const int off = (int)(slot & 15);
    uint16_t* row = qkv + t * ld;
    const float* tab = table + 2 * (int64_t)p * half;
    // q heads 0..Hq-1 and k heads Hq..Hq+Hkv-1: pair i of head h
    for (int e = threadIdx.x; e < (Hq + Hkv) * half; e += kRopeAppendThreads) {
        const int h = e / half;
        const int i = e - h * half;
        const float c = tab[2 * i];
        const float sn = tab[2 * i + 1];
        uint16_t* r = row + (int64_t)h * D;
        const float a = bf16_to_f32(r[i]);
        const float b = bf16_to_f32(r[i + half]);
        const uint16_t ra = (uint16_t)f32_to_bf16_rne(a * c - b * sn);
        const uint16_t rb = (uint16_t)f32_to_bf16_rne(b * c + a * sn);
        r[i] = ra;
        r[i + half] = rb;
        if (h >= Hq && cached) {
            uint16_t* kd = kc + ((blk * Hkv + (h - Hq)) * 16 + off) * D;
            kd[i] = ra;
            kd[i + half] = rb;
        }
    }
    if (!cached) return;
    const uint16_t* v = row + (int64_t)(Hq + Hkv) * D;
    for (int e = threadIdx.x; e < Hkv * D; e += kRopeAppendThreads) {
        const int h = e / D;
        const int d = e - h * D;
        vc[((blk * Hkv + h) * D + d) * 16 + off] = v[e];
    }
}

__global__ void add_kernel(const uint16_t* __restrict__ a, const uint16_t* __restrict__ b,
                           uint16_t* __restrict__ out, int64_t n8)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n8) return;
    const u32x4 va = ld16(a + i * 8);
    const u32x4 vb = ld16(b + i * 8);
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        o[e] = pack_bf16x2(bf16_to_f32(va[e] & 0xffffu) + bf16_to_f32(vb[e] & 0xffffu),
                           bf16_to_f32(va[e] >> 16) + bf16_to_f32(vb[e] >> 16));
    st16(out + i * 8, o);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// out[t][j] = silu(gu[t][j]) * gu[t][F + j]
__global__ void silu_mul_kernel(const uint16_t* __restrict__ gu, int64_t ldgu, int64_t F,
                                uint16_t* __restrict__ out, int64_t ldo)
{
    const int64_t t = blockIdx.y;
    const int64_t j = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (j >= F) return;
    const u32x4 vg = ld16(gu + t * ldgu + j);
    const u32x4 vu = ld16(gu + t * ldgu + F + j);
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        o[e] = pack_bf16x2(silu(bf16_to_f32(vg[e] & 0xffffu)) * bf16_to_f32(vu[e] & 0xffffu),
                           silu(bf16_to_f32(vg[e] >> 16)) * bf16_to_f32(vu[e] >> 16));
    st16(out + t * ldo + j, o);
}

__global__ void gather_rows_kernel(const uint16_t* __restrict__ src, int64_t lds, const int32_t* __restrict__ rows,
                                   int64_t nsrc, int64_t W, uint16_t* __restrict__ dst, int64_t ldd)
{
    const int64_t r = blockIdx.x;
    const int64_t s = rows[r];
    const bool ok = s >= 0 && s < nsrc;
    for (int64_t j = threadIdx.x * 8; j < W; j += blockDim.x * 8) {
        u32x4 v = zero_u32x4();
        if (ok) v = ld16(src + s * lds + j);
        st16(dst + r * ldd + j, v);
    }
}

}  // namespace

extern "C" int bi_embed(const void* table, int64_t V, int64_t H, const int32_t* ids, int64_t T,
                        void* out, int64_t ldo, void* stream)
{
    BI_TRY_BEGIN
    if (T < 0 || V <= 0 || H <= 0 || ldo < H) return BI_ERR_INVALID_ARGUMENT;
    if (T > 0 && (!table || !ids || !out)) return BI_ERR_INVALID_ARGUMENT;
    if ((H % 8) || (ldo % 8)) return BI_ERR_UNSUPPORTED;
    if (T > 0 && (!bi_aligned(table, 16) || !bi_aligned(out, 16) || !bi_aligned(ids, 4)))
        return BI_ERR_INVALID_ARGUMENT;
    if (T == 0) return BI_OK;
    hipLaunchKernelGGL(embed_kernel, dim3((unsigned)T), dim3(256), 0, (hipStream_t)stream,
                       (const uint16_t*)table, V, H, ids, (uint16_t*)out, ldo);
    return bi_launch_status();
    BI_TRY_END
}

extern "C" int bi_rope_table(float* table, int32_t max_pos, int32_t D, double theta, void* stream)
{
    BI_TRY_BEGIN
    if (!table || max_pos <= 0 || D <= 0 || (D % 2) || !(theta > 0.0)) return BI_ERR_INVALID_ARGUMENT;
    const int64_t n = (int64_t)max_pos * (D / 2);
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, table, max_pos, D / 2, D, theta);
    return bi_launch_status();
    BI_TRY_END
}

extern "C" int bi_rope_kv_append(void* qkv, int64_t ld, int32_t Hq, int32_t Hkv, int32_t D, const int32_t* pos,
                                 const int32_t* slots, int64_t T, const float* table, int32_t max_pos,
                                 void* k_cache, void* v_cache, int64_t num_blocks, void* stream)
{
    BI_TRY_BEGIN
    if (T < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || max_pos <= 0 || num_blocks <= 0 ||
        ld < (int64_t)(Hq + 2 * Hkv) * D || (ld % 8))
        return BI_ERR_INVALID_ARGUMENT;
    if (T > 0 && (!qkv || !pos || !slots || !table || !k_cache || !v_cache)) return BI_ERR_INVALID_ARGUMENT;
    if (T > 0 && (!bi_aligned(qkv, 16) || !bi_aligned(k_cache, 16) || !bi_aligned(v_cache, 16) ||
                  !bi_aligned(pos, 4) || !bi_aligned(slots, 4) || !bi_aligned(table, 4)))
        return BI_ERR_INVALID_ARGUMENT;
    if (D != BI_HEAD_DIM || Hq + Hkv > 65535 || T > 0x7fffffffLL) return BI_ERR_UNSUPPORTED;
    if (T == 0) return BI_OK;
    hipLaunchKernelGGL(rope_kv_append_kernel, dim3((unsigned)T), dim3(kRopeAppendThreads), 0, (hipStream_t)stream,
                       (uint16_t*)qkv, ld, Hq, Hkv, D, pos, slots, table, max_pos, (uint16_t*)k_cache,
                       (uint16_t*)v_cache, num_blocks);
    return bi_launch_status();
    BI_TRY_END
}

extern "C" int bi_rope(void* x, int64_t ldx, int32_t H, int32_t D, const int32_t* pos, int64_t T,
                       const float* table, int32_t max_pos, void* stream)
{
    BI_TRY_BEGIN
    if (T < 0 || H <= 0 || D <= 0 || (D % 2) || max_pos <= 0 || ldx < (int64_t)H * D)
        return BI_ERR_INVALID_ARGUMENT;
    if (T > 0 && (!x || !pos || !table)) return BI_ERR_INVALID_ARGUMENT;
    if (H > 65535) return BI_ERR_UNSUPPORTED;
    if (T == 0) return BI_OK;
    hipLaunchKernelGGL(rope_kernel, dim3((unsigned)T, H), dim3(64), 0, (hipStream_t)stream,
                       (uint16_t*)x, ldx, D, pos, table, max_pos);
    return bi_launch_status();
    BI_TRY_END
}

extern "C" int bi_add(const void* a, const void* b, void* out, int64_t n, void* stream)
{
    BI_TRY_BEGIN
    if (n < 0) return BI_ERR_INVALID_ARGUMENT;
    if (n > 0 && (!a || !b || !out)) return BI_ERR_INVALID_ARGUMENT;
    if (n % 8) return BI_ERR_UNSUPPORTED;
    if (n > 0 && (!bi_aligned(a, 16) || !bi_aligned(b, 16) || !bi_aligned(out, 16)))
        return BI_ERR_INVALID_ARGUMENT;
    if (n == 0) return BI_OK;
    const int64_t n8 = n / 8;
    hipLaunchKernelGGL(add_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, (const uint16_t*)a, (const uint16_t*)b, (uint16_t*)out, n8);
    return bi_launch_status();
    BI_TRY_END
}

extern "C" int bi_silu_mul(const void* gu, int64_t ldgu, int64_t F, void* out, int64_t ldo, int64_t T,
                           void* stream)
{
    BI_TRY_BEGIN
    if (T < 0 || F <= 0 || ldgu < 2 * F || ldo < F) return BI_ERR_INVALID_ARGUMENT;
    if (T > 0 && (!gu || !out)) return BI_ERR_INVALID_ARGUMENT;
    if ((F % 8) || (ldgu % 8) || (ldo % 8) || T > 65535) return BI_ERR_UNSUPPORTED;
    if (T > 0 && (!bi_aligned(gu, 16) || !bi_aligned(out, 16))) return BI_ERR_INVALID_ARGUMENT;
    if (T == 0) return BI_OK;
    const int64_t n8 = F / 8;
    hipLaunchKernelGGL(silu_mul_kernel, dim3((unsigned)((n8 + 255) / 256), (unsigned)T), dim3(256), 0,
                       (hipStream_t)stream, (const uint16_t*)gu, ldgu, F, (uint16_t*)out, ldo);
    return bi_launch_status();
    BI_TRY_END
}

extern "C" int bi_gather_rows(const void* src, int64_t lds, int64_t nsrc, const int32_t* rows, int64_t R,
                              int64_t W, void* dst, int64_t ldd, void* stream)
{
    BI_TRY_BEGIN
    if (R < 0 || W <= 0 || nsrc < 0 || lds < W || ldd < W) return BI_ERR_INVALID_ARGUMENT;
    if (R > 0 && (!src || !rows || !dst)) return BI_ERR_INVALID_ARGUMENT;
    if ((W % 8) || (lds % 8) || (ldd % 8)) return BI_ERR_UNSUPPORTED;
    if (R > 0 && (!bi_aligned(src, 16) || !bi_aligned(dst, 16) || !bi_aligned(rows, 4)))
        return BI_ERR_INVALID_ARGUMENT;
    if (R == 0) return BI_OK;
    hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)R), dim3(256), 0, (hipStream_t)stream,
                       (const uint16_t*)src, lds, rows, nsrc, W, (uint16_t*)dst, ldd);
    return bi_launch_status();
    BI_TRY_END
}

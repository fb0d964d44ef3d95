// mla_cache.hip -- pkv_mla_cache_assemble: the MLA cache rows of a batch of
// tokens (page 1, kv_cache.rs, mla_cache_assemble: [kv_latent | k_rope]
// becomes the K row and [kv_latent | zeros] the V row of the single-head MLA
// cache, in one kernel).  The page's launcher handles one token; here the
// rows go to their slots through a slot mapping, like the other writes.
//
// A thread owns one 16-byte column of the cache row (cache_dim * elem bytes)
// and walks kMRun tokens: the latent column is loaded once and stored to
// both rows; K's rope columns come from k_rope; every column past the copied
// parts is zero.  Loads and stores are non-temporal.
#include "pkv_internal.h"

namespace pkv {

constexpr int kMThreads = 256;
constexpr int kMRun = 4;  // tokens per thread

__global__ __launch_bounds__(kMThreads) void mla_cache_assemble_kernel(
    const u32x4* __restrict__ latent, uint64_t latent_stride16, const u32x4* __restrict__ rope,
    uint64_t rope_stride16, const int64_t* __restrict__ slots, uint32_t num_tokens,
    uint32_t lora_cols, uint32_t rope_cols, uint32_t cols, uint32_t tpb, uint64_t num_slots,
    u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache)
{
    const uint32_t lane_tok = threadIdx.x / cols;
    const uint32_t col0 = threadIdx.x % cols;
    if (lane_tok >= tpb)
        return;
    const uint32_t col_step = cols < kMThreads ? cols : kMThreads;
    const uint64_t base = (uint64_t)blockIdx.x * tpb * kMRun;
    int64_t slot[kMRun];
    uint64_t tok[kMRun];
#pragma unroll
    for (int r = 0; r < kMRun; ++r) {
        tok[r] = base + (uint64_t)r * tpb + lane_tok;
        const int64_t s = tok[r] < num_tokens ? slots[tok[r]] : -1;
        slot[r] = (s >= 0 && (uint64_t)s < num_slots) ? s : -1;
    }
    const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
    for (uint32_t c = col0; c < cols; c += col_step) {
        u32x4 kv[kMRun], vv[kMRun];
#pragma unroll
        for (int r = 0; r < kMRun; ++r) {
            kv[r] = zero;
            vv[r] = zero;
            if (slot[r] < 0)
                continue;
            if (c < lora_cols) {
                kv[r] = load_nt(latent + tok[r] * latent_stride16 + c);
                vv[r] = kv[r];
            } else if (c < lora_cols + rope_cols) {
                kv[r] = load_nt(rope + tok[r] * rope_stride16 + (c - lora_cols));
            }
        }
#pragma unroll
        for (int r = 0; r < kMRun; ++r) {
            if (slot[r] < 0)
                continue;
            store_nt(k_cache + (uint64_t)slot[r] * cols + c, kv[r]);
            store_nt(v_cache + (uint64_t)slot[r] * cols + c, vv[r]);
        }
    }
}

}  // namespace pkv

extern "C" int pkv_mla_cache_assemble(const void* kv_latent, const void* k_rope, pkv_dtype dtype,
                                      uint64_t latent_stride, uint64_t rope_stride,
                                      const int64_t* slot_mapping, uint32_t num_tokens,
                                      uint32_t kv_lora, uint32_t rope, uint32_t cache_dim,
                                      uint32_t block_size, uint32_t num_blocks, void* k_cache,
                                      void* v_cache, void* stream)
{
    using namespace pkv;
    clear_error();
    if (num_tokens == 0)
        return PKV_OK;
    if (!kv_latent || !slot_mapping || !k_cache || !v_cache || (rope && !k_rope))
        return fail(PKV_ERR_INVALID,
                    "mla_cache_assemble: kv_latent, k_rope (rope > 0), slot_mapping and caches must be non-NULL");
    if (!valid_dtype(dtype))
        return fail(PKV_ERR_INVALID, "mla_cache_assemble: bad dtype %d", (int)dtype);
    if (dtype != PKV_BF16 && dtype != PKV_FP32)
        return fail(PKV_ERR_UNSUPPORTED, "mla_cache_assemble: dtype must be BF16 or FP32");
    if (cache_dim == 0 || block_size == 0 || num_blocks == 0 || kv_lora == 0)
        return fail(PKV_ERR_INVALID, "mla_cache_assemble: zero dimension");
    if ((uint64_t)kv_lora + rope > cache_dim)
        return fail(PKV_ERR_INVALID, "mla_cache_assemble: kv_lora + rope > cache_dim");
    if (latent_stride < kv_lora || (rope && rope_stride < rope))
        return fail(PKV_ERR_INVALID, "mla_cache_assemble: token stride smaller than a row");
    const uint64_t es = dtype_size(dtype);
    if ((kv_lora * es) % 16 || (rope * es) % 16 || (cache_dim * es) % 16 ||
        (latent_stride * es) % 16 || (rope && (rope_stride * es) % 16) || !aligned16(kv_latent) ||
        (rope && !aligned16(k_rope)) || !aligned16(k_cache) || !aligned16(v_cache))
        return fail(PKV_ERR_UNSUPPORTED,
                    "mla_cache_assemble: row parts, strides and pointers must be 16-byte aligned");
    const uint32_t cols = (uint32_t)(cache_dim * es / 16);
    const uint32_t tpb = cols <= (uint32_t)kMThreads ? (uint32_t)kMThreads / cols : 1u;
    const uint64_t per_block = (uint64_t)tpb * kMRun;
    const uint64_t blocks = (num_tokens + per_block - 1) / per_block;
    hipLaunchKernelGGL(mla_cache_assemble_kernel, dim3((uint32_t)blocks), dim3(kMThreads), 0,
                       (hipStream_t)stream, (const u32x4*)kv_latent, latent_stride * es / 16,
                       (const u32x4*)k_rope, rope ? rope_stride * es / 16 : 0, slot_mapping,
                       num_tokens, (uint32_t)(kv_lora * es / 16), (uint32_t)(rope * es / 16),
                       cols, tpb, (uint64_t)num_blocks * block_size, (u32x4*)k_cache,
                       (u32x4*)v_cache);
    return check_launch("mla_cache_assemble");
}

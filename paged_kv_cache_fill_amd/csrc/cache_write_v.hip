// cache_write_v.hip -- pkv_cache_write_v: the V reshape-and-cache copy
// (page 1, kv_cache.rs, reshape_and_cache_flash_v_only: V rows copied into
// the paged V pool at slot_mapping, leaving the K side to the fused K write),
// and its E4M3 form (page 1, reshape_and_cache_fp8: V stored as FP8 with a
// per-tensor v_scale), and the TurboQuant-style V forms (page 1,
// reshape_and_cache_bf16k_turbo{2,3,4}v; the format is stated with pkv_dtype).
//
// A token's V row (num_kv_heads * head_dim_v elements) is contiguous in the
// input and, under the [num_blocks, block_size, Hkv, Dv] layout, contiguous
// at its slot in the pool.  So the copy is a row gather/scatter in 16-byte
// pieces: each thread owns one 16-byte column of the row and walks a run of
// tokens, issuing all of a run's loads before its stores so that several
// kilobytes per wave are in flight.  Both sides are touched once: loads and
// stores are non-temporal.
#include "pkv_internal.h"

namespace pkv {

constexpr int kVThreads = 256;
// E4M3 store: tokens per thread per pass.  With the row loads independent of
// the slot loads, one token per thread measured fastest (64-sequence
// population write, 1.58 M tokens: 0.905 / 0.910 / 0.927 / 0.951 ms with
// 1 / 2 / 4 / 8 tokens per thread).
constexpr int kVRun = 1;
// The plain copy: one token per thread, so the most threads, each with one
// load in flight (population write of 1.09 M BF16 rows: 0.80 ms against
// 0.86 ms with four tokens per thread and 0.85 ms with two).
constexpr int kVRunCopy = 1;

// cols = row bytes / 16; tpb = tokens handled side by side by one block
// (kVThreads / cols when a row fits in a block, else 1 with a column loop).
__global__ __launch_bounds__(kVThreads) void cache_write_v_kernel(
    const u32x4* __restrict__ v, uint64_t in_stride16, const int64_t* __restrict__ slots,
    uint32_t num_tokens, uint32_t cols, uint32_t tpb, uint64_t num_slots,
    u32x4* __restrict__ cache)
{
    const uint32_t lane_tok = threadIdx.x / cols;       // which token of the block's group
    const uint32_t col0 = threadIdx.x % cols;
    if (lane_tok >= tpb)
        return;
    const uint32_t col_step = cols < kVThreads ? cols : kVThreads;  // columns per pass
    // Token runs: block b handles tokens [b * tpb * kVRunCopy, (b+1) * tpb * kVRunCopy),
    // token = base + r * tpb + lane_tok.
    const uint64_t base = (uint64_t)blockIdx.x * tpb * kVRunCopy;
    int64_t slot[kVRunCopy];
    uint64_t tok[kVRunCopy];
#pragma unroll
    for (int r = 0; r < kVRunCopy; ++r) {
        tok[r] = base + (uint64_t)r * tpb + lane_tok;
        int64_t s = tok[r] < num_tokens ? slots[tok[r]] : -1;
        slot[r] = (s >= 0 && (uint64_t)s < num_slots) ? s : -1;
    }
    // the row loads depend only on the token existing, not on its slot, so
    // they are in flight together with the slot loads
    for (uint32_t c = col0; c < cols; c += col_step) {
        u32x4 buf[kVRunCopy];
#pragma unroll
        for (int r = 0; r < kVRunCopy; ++r)
            if (tok[r] < num_tokens)
                buf[r] = load_nt(v + tok[r] * in_stride16 + c);
#pragma unroll
        for (int r = 0; r < kVRunCopy; ++r)
            if (slot[r] >= 0)
                store_nt(cache + (uint64_t)slot[r] * cols + c, buf[r]);
    }
}

// v / d for 2^-64 <= d <= 2^64 from the correctly rounded reciprocal
// r = RN(1/d): q0 = RN(x r), then one residual correction
// RN(q0 + (x - q0 d) r), the residual exact by FMA while it does not
// underflow (Markstein's division step).  For such d its E4M3 code (after
// the +-448 clamp) equals that of the correctly rounded quotient for every
// FP32 x: checked exhaustively over all 2^32 x for divisors across and at
// the ends of that range, an all-ones significand among them (near FLT_MIN
// the residual of tiny x underflows and some codes differ, hence the
// range); quotients of |q0| >= 1e30 saturate either way and are not
// corrected; the sign of q0 is kept so that -0 stays -0.
__device__ __forceinline__ float div_by_scale(float x, float d, float r)
{
    const float q0 = x * r;
    const float e = __builtin_fmaf(-q0, d, x);
    const float q1 = __builtin_fmaf(e, r, q0);
    return __builtin_copysignf(__builtin_fabsf(q0) < 1e30f ? q1 : q0, q0);
}

// E4M3 store: each thread owns 16 elements of the row, taken so that every
// load and store instruction of a wave covers consecutive bytes: with cols
// the row's 16-byte output columns, thread column c converts input chunks
// c + j * cols (j < 2 for BF16, 8 elements each; j < 4 for FP32, 4 each)
// and stores their codes as the 8- or 4-byte pieces c + j * cols of the
// output row.  (Two 16-byte loads per thread from one 32-byte span would
// make each load instruction touch every line of the row at half use.)
// Each thread walks kVRun tokens the same way.  The stored code is the E4M3
// rounding of fl32(v / v_scale): with FAST (2^-64 <= v_scale <= 2^64), by
// div_by_scale from the host's correctly rounded reciprocal; otherwise by
// the correctly rounded FP32 division.
template <int IN, bool FAST>   // IN: 0 = BF16 input, 2 = FP32 input
__global__ __launch_bounds__(kVThreads) void cache_write_v_e4m3_kernel(
    const u32x4* __restrict__ v, uint64_t in_stride16, const int64_t* __restrict__ slots,
    uint32_t num_tokens, uint32_t cols, uint32_t tpb, uint64_t num_slots, float v_scale,
    float v_rcp, uint8_t* __restrict__ cache)
{
    constexpr int NLD = IN == 0 ? 2 : 4;                // input chunks per thread and column
    constexpr int EPC = 16 / NLD;                       // elements (output bytes) per chunk
    const uint32_t lane_tok = threadIdx.x / cols;
    const uint32_t col0 = threadIdx.x % cols;
    if (lane_tok >= tpb)
        return;
    const uint32_t col_step = cols < kVThreads ? cols : kVThreads;
    const uint64_t base = (uint64_t)blockIdx.x * tpb * kVRun;
    int64_t slot[kVRun];
    uint64_t tok[kVRun];
#pragma unroll
    for (int r = 0; r < kVRun; ++r) {
        tok[r] = base + (uint64_t)r * tpb + lane_tok;
        int64_t s = tok[r] < num_tokens ? slots[tok[r]] : -1;
        slot[r] = (s >= 0 && (uint64_t)s < num_slots) ? s : -1;
    }
    const uint64_t row_bytes = (uint64_t)cols * 16;
    for (uint32_t c = col0; c < cols; c += col_step) {
        u32x4 buf[kVRun][NLD];
#pragma unroll
        for (int r = 0; r < kVRun; ++r)
            if (tok[r] < num_tokens)                    // independent of the slot loads
#pragma unroll
                for (int j = 0; j < NLD; ++j)
                    buf[r][j] = load_nt(v + tok[r] * in_stride16 + c + (uint64_t)j * cols);
#pragma unroll
        for (int r = 0; r < kVRun; ++r) {
            if (slot[r] < 0)
                continue;
            uint8_t* dst = cache + (uint64_t)slot[r] * row_bytes;
#pragma unroll
            for (int j = 0; j < NLD; ++j) {
                float x[EPC];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (IN == 0) {
                        x[2 * e] = bf16_lo(buf[r][j][e]);
                        x[2 * e + 1] = bf16_hi(buf[r][j][e]);
                    } else {
                        x[e] = __uint_as_float(buf[r][j][e]);
                    }
                }
                float y[EPC];
#pragma unroll
                for (int e = 0; e < EPC; ++e)
                    y[e] = FAST ? div_by_scale(x[e], v_scale, v_rcp) : x[e] / v_scale;
                const uint64_t off = ((uint64_t)c + (uint64_t)j * cols) * EPC;
                if constexpr (IN == 0)
                    __builtin_nontemporal_store(u32x2{e4m3_sat_x4(y[0], y[1], y[2], y[3]),
                                                      e4m3_sat_x4(y[4], y[5], y[6], y[7])},
                                                (u32x2*)(dst + off));
                else
                    __builtin_nontemporal_store(e4m3_sat_x4(y[0], y[1], y[2], y[3]),
                                                (uint32_t*)(dst + off));
            }
        }
    }
}

// TurboQuant-style V: one thread per (token, kv head, 16-element group).
// The grid is (token blocks, kv heads); a work-group's threads are (token,
// group) with the group index in the low `gshift` bits, so a wavefront covers
// consecutive tokens of one head, whose code rows and scale bytes are
// neighbours in the head's region of a cache block.  Codebook constants come
// from the host (tq.cpp): the encoder's thresholds (midpoints of adjacent
// magnitudes, +inf past the last), the magnitudes' E4M3 codes as an 8-byte
// lookup table, and their squares.
struct TqArgs {
    float thr[7];
    float sq[8];
    uint32_t mag_lo, mag_hi;
};

template <int IN, int BITS>   // IN: 0 = BF16 input, 2 = FP32 input
__global__ __launch_bounds__(256) void cache_write_v_tq_kernel(
    const uint8_t* __restrict__ v, uint64_t in_stride_bytes, const int64_t* __restrict__ slots,
    uint32_t num_tokens, uint32_t groups, uint32_t gshift, uint32_t D, uint32_t B,
    uint64_t num_slots, uint64_t blk_bytes, uint64_t region_bytes, TqArgs cb,
    uint8_t* __restrict__ cache)
{
    constexpr int M = 1 << (BITS - 1);                  // magnitudes
    const uint32_t q = threadIdx.x & ((1u << gshift) - 1);
    const uint32_t tok = (blockIdx.x << (8 - gshift)) + (threadIdx.x >> gshift);
    const uint32_t h = blockIdx.y;
    if (q >= groups || tok >= num_tokens)
        return;
    // slot and row loads in flight together (the row does not depend on it)
    const int64_t slot = slots[tok];

    float x[16];
    const uint8_t* src = v + (uint64_t)tok * in_stride_bytes + ((uint64_t)h * D + 16u * q) * (IN == 0 ? 2 : 4);
    if constexpr (IN == 0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const u32x4 w = load_nt((const u32x4*)src + j);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[8 * j + 2 * e] = bf16_lo(w[e]);
                x[8 * j + 2 * e + 1] = bf16_hi(w[e]);
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4 w = load_nt((const u32x4*)src + j);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                x[4 * j + e] = __uint_as_float(w[e]);
        }
    }
    if (slot < 0 || (uint64_t)slot >= num_slots)
        return;
    // The decisions below are taken in FP32 (in-order fused sum of squares,
    // the hardware reciprocal square root of the mean square, one product
    // per element, the scale from the hardware reciprocal and square root):
    // about a dozen roundings of at most an ulp or two each, so they equal
    // the exact definition's except within ~2^-20 (relative) of a decision
    // boundary.
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        ss = fmaf(x[i], x[i], ss);

    uint32_t w[2] = {0u, 0u};                           // codes of elements 0-7, 8-15
    uint32_t scale = 0;
    if (ss > 0.f) {
        // +inf for a mean square below the normal range (those groups' scale
        // rounds to zero), 0 for ss = +inf (codes 0, scale saturated)
        const float inv_r = __builtin_amdgcn_rsqf(ss * 0.0625f);
        [[maybe_unused]] float cn4 = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float u = x[i] * inv_r;
            const float au = fabsf(u);
            // magnitude index: the number of midpoints below |u| (ties stay
            // on the smaller magnitude), by binary search over the midpoints
            uint32_t m = 0;
#pragma unroll
            for (int step = M / 2; step >= 1; step /= 2) {
                float t = cb.thr[step - 1];
#pragma unroll
                for (int base = 2 * step; base + step - 1 < M - 1; base += 2 * step)
                    t = m == (uint32_t)base ? cb.thr[base + step - 1] : t;
                m += au > t ? (uint32_t)step : 0u;
            }
            if constexpr (BITS == 4) {
                const float mag = unpack_e4m3x2(__builtin_amdgcn_perm(cb.mag_hi, cb.mag_lo, m), false).x;
                cn4 = fmaf(mag, mag, cn4);
            }
            const uint32_t code = (u < 0.f ? (1u << (BITS - 1)) : 0u) | m;
            w[i / 8] |= code << (BITS * (i % 8));
        }
        // sum of the chosen magnitudes' squares: for 2- and 3-bit codes from
        // the counts of each magnitude index in the packed codes (exact: a
        // count times a square, summed, has few significant bits)
        float cn;
        if constexpr (BITS == 2) {
            const uint32_t n1 = __builtin_popcount((w[0] | (w[1] << 16)) & 0x55555555u);
            cn = fmaf((float)n1, cb.sq[1], (float)(16u - n1) * cb.sq[0]);
        } else if constexpr (BITS == 3) {
            uint32_t n1 = 0, n2 = 0, n3 = 0;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const uint32_t p0 = w[k] & 0x249249u, p1 = (w[k] >> 1) & 0x249249u;
                const uint32_t both = __builtin_popcount(p0 & p1);
                n3 += both;
                n1 += __builtin_popcount(p0) - both;
                n2 += __builtin_popcount(p1) - both;
            }
            cn = (float)(16u - n1 - n2 - n3) * cb.sq[0];
            cn = fmaf((float)n1, cb.sq[1], cn);
            cn = fmaf((float)n2, cb.sq[2], cn);
            cn = fmaf((float)n3, cb.sq[3], cn);
        } else {
            cn = cn4;
        }
        // the norm correction: scale so that |scale x levels| = |x|
        const float ratio = __builtin_amdgcn_sqrtf(ss * __builtin_amdgcn_rcpf(cn));
        scale = e4m3_sat_x4(ratio, 0.f, 0.f, 0.f) & 0xFFu;
    }
    // head h's region of the block: B code rows of D * BITS / 8 bytes, then
    // D / 16 scale rows (one per group) of B bytes
    const uint32_t blk = (uint32_t)slot / B;            // slots < 2^32 (checked by the host)
    const uint32_t t = (uint32_t)slot - blk * B;
    uint8_t* base = cache + (uint64_t)blk * blk_bytes + h * region_bytes;
    uint8_t* dst = base + (uint64_t)t * D * BITS / 8 + (uint64_t)q * 2 * BITS;
    if constexpr (BITS == 2) {
        *(uint32_t*)dst = w[0] | (w[1] << 16);
    } else if constexpr (BITS == 3) {
        uint16_t* d16 = (uint16_t*)dst;                 // 6 bytes, 2-byte aligned
        d16[0] = (uint16_t)w[0];
        d16[1] = (uint16_t)((w[0] >> 16) | (w[1] << 8));
        d16[2] = (uint16_t)(w[1] >> 8);
    } else {
        *(u32x2*)dst = u32x2{w[0], w[1]};
    }
    base[(uint64_t)B * D * BITS / 8 + (uint64_t)q * B + t] = (uint8_t)scale;
}

}  // namespace pkv

extern "C" int pkv_cache_write_v(const void* v, pkv_dtype in_dtype, uint64_t in_token_stride,
                                 const int64_t* slot_mapping, uint32_t num_tokens,
                                 uint32_t num_kv_heads, uint32_t head_dim_v, uint32_t block_size,
                                 uint32_t num_blocks, void* v_cache, pkv_dtype cache_dtype,
                                 float v_scale, void* stream)
{
    using namespace pkv;
    clear_error();
    if (num_tokens == 0)
        return PKV_OK;
    if (!v || !slot_mapping || !v_cache)
        return fail(PKV_ERR_INVALID, "cache_write_v: v, slot_mapping and v_cache must be non-NULL");
    if (!valid_dtype(in_dtype) || !(valid_dtype(cache_dtype) || is_tq(cache_dtype)))
        return fail(PKV_ERR_INVALID, "cache_write_v: bad dtype (%d, %d)", (int)in_dtype,
                    (int)cache_dtype);
    if (in_dtype != PKV_BF16 && in_dtype != PKV_FP32)
        return fail(PKV_ERR_UNSUPPORTED, "cache_write_v: input dtype must be BF16 or FP32");
    if (is_tq(cache_dtype)) {
        if (num_kv_heads == 0 || head_dim_v == 0 || block_size == 0 || num_blocks == 0)
            return fail(PKV_ERR_INVALID, "cache_write_v: zero dimension");
        if (head_dim_v % 16)
            return fail(PKV_ERR_UNSUPPORTED, "cache_write_v: TQ needs head_dim_v %% 16 == 0");
        // keeps every head region, and so every group's code store, naturally aligned
        if (((uint64_t)block_size * (head_dim_v / 16)) % 8)
            return fail(PKV_ERR_UNSUPPORTED,
                        "cache_write_v: TQ needs block_size * head_dim_v / 16 %% 8 == 0");
        const uint64_t es = dtype_size(in_dtype);
        if (in_token_stride < (uint64_t)num_kv_heads * head_dim_v)
            return fail(PKV_ERR_INVALID, "cache_write_v: in_token_stride smaller than a row");
        if ((in_token_stride * es) % 16 || !aligned16(v) || !aligned16(v_cache))
            return fail(PKV_ERR_UNSUPPORTED,
                        "cache_write_v: strides and pointers must be 16-byte aligned");
        const int bits = tq_bits(cache_dtype);
        const TqCodebook& book = tq_codebook(bits);
        TqArgs cb{};
        for (int j = 0; j < 7; ++j)
            cb.thr[j] = book.thr[j];
        for (int j = 0; j < 8; ++j)
            cb.sq[j] = book.mags[j] * book.mags[j];   // exact: E4M3 values
        for (int j = 0; j < 4; ++j) {
            cb.mag_lo |= (uint32_t)book.codes[j] << (8 * j);
            cb.mag_hi |= (uint32_t)book.codes[4 + j] << (8 * j);
        }
        const uint32_t groups = head_dim_v / 16;
        uint32_t gshift = 0;
        while ((1u << gshift) < groups)
            ++gshift;
        if (gshift > 8 || num_kv_heads > 65535 || (uint64_t)num_blocks * block_size >= (1ull << 32))
            return fail(PKV_ERR_UNSUPPORTED, "cache_write_v: TQ shape too large");
        const uint32_t tok_per_wg = 256u >> gshift;
        const uint64_t nblk = ((uint64_t)num_tokens + tok_per_wg - 1) / tok_per_wg;
        const uint64_t blk_bytes = tq_block_bytes(bits, block_size, num_kv_heads, head_dim_v);
        const uint64_t region_bytes = blk_bytes / num_kv_heads;
        hipStream_t st = (hipStream_t)stream;
#define PKV_TQW(IN, BITS)                                                                      \
    hipLaunchKernelGGL((cache_write_v_tq_kernel<IN, BITS>), dim3((uint32_t)nblk, num_kv_heads),     \
                       dim3(256), 0, st, (const uint8_t*)v, in_token_stride * es, slot_mapping, \
                       num_tokens, groups, gshift, head_dim_v, block_size,                      \
                       (uint64_t)num_blocks * block_size, blk_bytes, region_bytes, cb,          \
                       (uint8_t*)v_cache)
        if (in_dtype == PKV_BF16) {
            if (bits == 2) PKV_TQW(0, 2); else if (bits == 3) PKV_TQW(0, 3); else PKV_TQW(0, 4);
        } else {
            if (bits == 2) PKV_TQW(2, 2); else if (bits == 3) PKV_TQW(2, 3); else PKV_TQW(2, 4);
        }
#undef PKV_TQW
        return check_launch("cache_write_v");
    }
    if (cache_dtype != in_dtype && cache_dtype != PKV_FP8_E4M3)
        return fail(PKV_ERR_UNSUPPORTED, "cache_write_v: cache dtype must be the input's or E4M3");
    const bool e4m3 = cache_dtype == PKV_FP8_E4M3;
    if (e4m3 && !(v_scale > 0.0f && v_scale < INFINITY))
        return fail(PKV_ERR_INVALID, "cache_write_v: v_scale must be finite and > 0");
    if (num_kv_heads == 0 || head_dim_v == 0 || block_size == 0 || num_blocks == 0)
        return fail(PKV_ERR_INVALID, "cache_write_v: zero dimension");
    const uint64_t row_elems = (uint64_t)num_kv_heads * head_dim_v;
    const uint64_t row_bytes = row_elems * dtype_size(in_dtype);
    const uint64_t cache_row_bytes = row_elems * dtype_size(cache_dtype);
    if (in_token_stride < row_elems)
        return fail(PKV_ERR_INVALID, "cache_write_v: in_token_stride %llu < row of %llu elements",
                    (unsigned long long)in_token_stride, (unsigned long long)row_elems);
    const uint64_t stride_bytes = in_token_stride * dtype_size(in_dtype);
    if (row_bytes % 16 || cache_row_bytes % 16 || stride_bytes % 16 || !aligned16(v) ||
        !aligned16(v_cache))
        return fail(PKV_ERR_UNSUPPORTED,
                    "cache_write_v: rows, strides and pointers must be 16-byte aligned");
    const uint64_t cols64 = cache_row_bytes / 16;   // 16-byte columns of the cache row
    if (cols64 > (1u << 24))
        return fail(PKV_ERR_UNSUPPORTED, "cache_write_v: row too long");
    const uint32_t cols = (uint32_t)cols64;
    const uint32_t tpb = cols <= (uint32_t)kVThreads ? (uint32_t)kVThreads / cols : 1u;
    const uint64_t per_block = (uint64_t)tpb * (e4m3 ? kVRun : kVRunCopy);
    const uint64_t blocks = (num_tokens + per_block - 1) / per_block;
    if (blocks > 0x7FFFFFFFull)
        return fail(PKV_ERR_UNSUPPORTED, "cache_write_v: too many tokens for one call");
    const uint64_t num_slots = (uint64_t)num_blocks * block_size;
    hipStream_t st = (hipStream_t)stream;
    if (!e4m3)
        hipLaunchKernelGGL(cache_write_v_kernel, dim3((uint32_t)blocks), dim3(kVThreads), 0, st,
                           (const u32x4*)v, stride_bytes / 16, slot_mapping, num_tokens, cols,
                           tpb, num_slots, (u32x4*)v_cache);
    else {
        // the correctly rounded reciprocal: the double quotient is within
        // 2^-53 of 1/v_scale, which is never that close to a float midpoint
        // without being one, so rounding it to float rounds 1/v_scale once
        const float v_rcp = (float)(1.0 / (double)v_scale);
        const bool fast = v_scale >= 0x1p-64f && v_scale <= 0x1p64f;
#define PKV_E4V(IN, FAST)                                                                       \
    hipLaunchKernelGGL((cache_write_v_e4m3_kernel<IN, FAST>), dim3((uint32_t)blocks),          \
                       dim3(kVThreads), 0, st, (const u32x4*)v, stride_bytes / 16, slot_mapping, \
                       num_tokens, cols, tpb, num_slots, v_scale, v_rcp, (uint8_t*)v_cache)
        if (in_dtype == PKV_BF16) {
            if (fast) PKV_E4V(0, true); else PKV_E4V(0, false);
        } else {
            if (fast) PKV_E4V(2, true); else PKV_E4V(2, false);
        }
#undef PKV_E4V
    }
    return check_launch("cache_write_v");
}

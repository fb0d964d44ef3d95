// cache_write_k.hip -- pkv_cache_write_k_fused: RMSNorm -> RoPE -> one
// rounding, written into the paged K pool (page 1, kv_cache.rs,
// fused_k_norm_rope_cache_write_{bf16, bf16_mrope, fp8}: K kept in FP32
// between the three steps and rounded once at the cache write; page 2,
// kv_cache_fp8k.rs, module invariants: the FP8 store is k / k_scale as E4M3;
// page 3, mla_cuda.rs: NoPE skips the rotation).
//
// Lane layout.  A (token, kv head) row of D elements is split into 16-byte
// chunks of VEC elements (8 BF16 or 4 FP32).  A row is owned by L lanes;
// lane j of the row holds chunks j, j + L, j + 2L, ... (NC chunks).  L is
// chosen (host side) so that it divides the distance, in chunks, between
// the two halves of every rotation pair, so both members of every RoPE pair
// sit in the same lane and the rotation needs no cross-lane exchange.  Each
// load instruction of a row is L consecutive 16-byte chunks (coalesced).
// RMSNorm's sum of squares is reduced over the L lanes with xor shuffles.
//
// cos/sin of a (token, pair) angle are computed once per wave-unit by one
// lane and shared through LDS with all rows (kv heads) of the unit, so the
// transcendental work is per token, not per (token, head).
#include <cfloat>

#include "pkv_internal.h"

namespace pkv {

enum { IN_BF16 = 0, IN_F32 = 2 };
enum { OUT_BF16 = 0, OUT_FP8 = 1, OUT_F32 = 2 };

constexpr int kKThreads = 256;
constexpr int kKWaves = kKThreads / 64;
constexpr int kMaxHalf = 128;  // rotation pairs per row (rotary_dim <= 256)

struct KWriteArgs {
    const void* k_in;
    const void* norm_w;     // NULL: no RMSNorm
    const int32_t* pos_t;
    const int32_t* pos_h;   // MRoPE when pos_h and pos_w are both set
    const int32_t* pos_w;
    const int64_t* slots;
    void* k_cache;
    uint64_t in_stride;     // elements between tokens
    uint64_t num_slots;
    uint64_t num_units;     // tokens * units_per_token
    float eps;
    float theta;
    float k_scale;
    float inv_k_scale;      // 1 / k_scale for the E4M3 store, else 1
    float inv_d;            // 1 / head_dim
    uint32_t D;
    uint32_t Hkv;
    uint32_t rope_first;    // first rotated chunk (rope_offset / VEC)
    uint32_t rope_chunks;   // chunks in the first half of the rotation (R/2/VEC)
    uint32_t half;          // R/2 (0: no rotation)
    uint32_t rot_dim;       // R
    uint32_t L;             // lanes per row (power of two)
    uint32_t rows_per_wave; // 64 / L
    uint32_t units_per_token;
    uint32_t units_per_wave;
    // inverse frequencies fl32(theta^(-2i/R)), i < R/2: the FP64 power is
    // taken once per call on the host instead of twice per lane per wave
    float invf[kMaxHalf];
};

template <int IN>
struct InVec;
template <>
struct InVec<IN_BF16> {
    static constexpr int VEC = 8;
    __device__ static u32x4 raw(const void* base, uint64_t elem)
    {
        return load_nt((const u32x4*)((const uint16_t*)base + elem));
    }
    __device__ static void cvt(const u32x4& w, float* x)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_lo(w[i]);
            x[2 * i + 1] = bf16_hi(w[i]);
        }
    }
    __device__ static u32x4 raw_cached(const void* base, uint64_t elem)
    {
        return *(const u32x4*)((const uint16_t*)base + elem);
    }
};
template <>
struct InVec<IN_F32> {
    static constexpr int VEC = 4;
    __device__ static u32x4 raw(const void* base, uint64_t elem)
    {
        return load_nt((const u32x4*)((const float*)base + elem));
    }
    __device__ static void cvt(const u32x4& w, float* x)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            x[i] = __uint_as_float(w[i]);
    }
    __device__ static u32x4 raw_cached(const void* base, uint64_t elem)
    {
        return *(const u32x4*)((const float*)base + elem);
    }
};

// Store VEC FP32 values at element offset `elem` of the cache.
template <int OUT, int VEC>
__device__ __forceinline__ void store_chunk(void* cache, uint64_t elem, const float* y)
{
    if constexpr (OUT == OUT_BF16) {
        uint32_t w[VEC / 2];
#pragma unroll
        for (int i = 0; i < VEC / 2; ++i)
            w[i] = pack_bf16(y[2 * i], y[2 * i + 1]);
        uint16_t* p = (uint16_t*)cache + elem;
        if constexpr (VEC == 8) {
            store_nt((u32x4*)p, u32x4{w[0], w[1], w[2], w[3]});
        } else {
            __builtin_nontemporal_store(u32x2{w[0], w[1]}, (u32x2*)p);
        }
    } else if constexpr (OUT == OUT_FP8) {
        // y already carries the 1/k_scale factor (folded into the row scale)
        uint32_t w[VEC / 4];
#pragma unroll
        for (int j = 0; j < VEC / 4; ++j)
            w[j] = e4m3_sat_x4(y[4 * j], y[4 * j + 1], y[4 * j + 2], y[4 * j + 3]);
        uint8_t* p = (uint8_t*)cache + elem;
        if constexpr (VEC == 8) {
            __builtin_nontemporal_store(u32x2{w[0], w[1]}, (u32x2*)p);
        } else {
            __builtin_nontemporal_store(w[0], (uint32_t*)p);
        }
    } else {
        float* p = (float*)cache + elem;
#pragma unroll
        for (int i = 0; i < VEC; i += 4)
            store_nt((u32x4*)(p + i), u32x4{__float_as_uint(y[i]), __float_as_uint(y[i + 1]),
                                            __float_as_uint(y[i + 2]),
                                            __float_as_uint(y[i + 3])});
    }
}

// Per-token arrays are separate restrict parameters: the compiler may then
// read them with scalar loads (they cannot alias the cache being written).
template <int IN, int OUT, int NC>
__global__ __launch_bounds__(kKThreads) void cache_write_k_kernel(
    KWriteArgs a, const int64_t* __restrict__ slots, const int32_t* __restrict__ pos_t,
    const int32_t* __restrict__ pos_h, const int32_t* __restrict__ pos_w)
{
    constexpr int VEC = InVec<IN>::VEC;
    __shared__ float s_cos[kKWaves][kMaxHalf];
    __shared__ float s_sin[kKWaves][kMaxHalf];

    // wave index made explicitly uniform: the token cursors derived from it
    // then live in scalar registers and per-token loads are scalar loads
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const uint32_t lane = threadIdx.x % 64;
    const uint32_t rr = lane / a.L;         // row within the wave
    const uint32_t lir = lane % a.L;        // lane within the row

    // per-lane constants: norm weight of the lane's chunks (one 16-byte load
    // per chunk; converted once the first unit's loads are in flight too),
    // inverse frequencies
    u32x4 wr[NC];
    if (a.norm_w) {
#pragma unroll
        for (int k = 0; k < NC; ++k)
            wr[k] = InVec<IN>::raw_cached(a.norm_w, (uint64_t)(lir + a.L * k) * VEC);
    }
    float w[NC][VEC];
    auto convert_weights = [&]() {
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            if (a.norm_w) {
                InVec<IN>::cvt(wr[k], w[k]);
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    w[k][e] = 1.0f;
            }
        }
    };
    // invf_i = fl32(theta^(-2i/R)) (host table); lane takes pairs lane and lane + 64
    const float invf0 = a.invf[lane];
    const float invf1 = a.invf[lane + 64];
    const bool mrope = a.pos_h != nullptr && a.pos_w != nullptr;
    const uint32_t kp = a.half ? a.rope_chunks / a.L : 0;  // chunk-slot distance of a pair

    const uint64_t gwave = (uint64_t)blockIdx.x * kKWaves + wave;
    const uint64_t u0 = gwave * a.units_per_wave;
    const uint64_t u1 = u0 + a.units_per_wave < a.num_units ? u0 + a.units_per_wave : a.num_units;

    // Software pipeline over the wave's units: the rows, slots and positions
    // of the next two units are loaded while the current one is computed and
    // stored.  Loads are unconditional (rows past Hkv re-read the last head's
    // row), so the compiler's wait before each unit covers only that unit's
    // loads.
    struct Raw {
        u32x4 w[NC];
        int64_t slot;
        int32_t pt, ph, pw;
    };
    auto load_unit = [&](uint32_t t, uint32_t grp, Raw& r) {
        uint32_t h = grp * a.rows_per_wave + rr;
        h = h < a.Hkv ? h : a.Hkv - 1;
        const uint64_t src = (uint64_t)t * a.in_stride + (uint64_t)h * a.D;
#pragma unroll
        for (int k = 0; k < NC; ++k)
            r.w[k] = InVec<IN>::raw(a.k_in, src + (uint64_t)(lir + a.L * k) * VEC);
        r.slot = slots[t];
        if (a.half > 0) {
            r.pt = pos_t[t];
            r.ph = mrope ? pos_h[t] : r.pt;
            r.pw = mrope ? pos_w[t] : r.pt;
        }
    };

    auto process = [&](uint32_t t, uint32_t grp, const Raw& raw) {
        const int64_t slot = raw.slot;
        if (slot < 0 || (uint64_t)slot >= a.num_slots)
            return;                                     // padding slot: no write
        const uint32_t h = grp * a.rows_per_wave + rr;
        const bool row_ok = h < a.Hkv;

        float y[NC][VEC];
#pragma unroll
        for (int k = 0; k < NC; ++k)
            InVec<IN>::cvt(raw.w[k], y[k]);
        // angles of this token, one (token, pair) per lane, shared via LDS
        if (a.half > 0) {
            // positions are per token (wave-uniform), loaded with the row
            const int32_t pt = raw.pt, ph = raw.ph, pw = raw.pw;
#pragma unroll
            for (int rep = 0; rep < 2; ++rep) {
                const uint32_t i = lane + 64u * rep;
                if (i < a.half) {
                    const uint32_t ax = i % 3u;
                    const int32_t p = ax == 0 ? pt : ax == 1 ? ph : pw;
                    const float ang = (float)p * (rep ? invf1 : invf0);
                    // reduce the FP32 angle to [-1/2, 1/2] revolution in double
                    // (exact enough for any int32 position), then the hardware
                    // sin/cos, which take revolutions
                    const double rev = (double)ang * 0.15915494309189535;
                    const float f = (float)(rev - __builtin_rint(rev));
                    const float sn = __builtin_amdgcn_sinf(f);
                    const float cs = __builtin_amdgcn_cosf(f);
                    s_cos[wave][i] = cs;
                    s_sin[wave][i] = sn;
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

        // row factor: 1/rms (RMSNorm) times 1/k_scale (E4M3 store; 1 otherwise).
        // Rotation is linear, so scaling before it equals dividing the rotated
        // row by k_scale up to FP32 rounding.
        if (a.norm_w) {
            float ss = 0.f;
#pragma unroll
            for (int k = 0; k < NC; ++k)
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    ss = __builtin_fmaf(y[k][e], y[k][e], ss);
            // sum over the row's L lanes (L <= 16, aligned): DPP adds
            ss = group_sum(ss, a.L);
            const float r = rsqrtf(__builtin_fmaf(ss, a.inv_d, a.eps)) * a.inv_k_scale;
#pragma unroll
            for (int k = 0; k < NC; ++k)
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    y[k][e] = y[k][e] * r * w[k][e];
        } else if (OUT == OUT_FP8) {
#pragma unroll
            for (int k = 0; k < NC; ++k)
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    y[k][e] = y[k][e] * a.inv_k_scale;
        }

        if (a.half > 0) {
#pragma unroll
            for (int k = 0; k < NC; ++k) {
                const uint32_t ci = lir + a.L * k;
                if (ci >= a.rope_first && ci < a.rope_first + a.rope_chunks) {
                    const uint32_t i0 = (ci - a.rope_first) * VEC;
                    // partner chunk slot k + kp (kp >= 1 by construction)
#pragma unroll
                    for (int k2 = k + 1; k2 < NC; ++k2) {
                        if ((uint32_t)(k2 - k) == kp) {
#pragma unroll
                            for (int e = 0; e < VEC; ++e) {
                                const float cs = s_cos[wave][i0 + e];
                                const float sn = s_sin[wave][i0 + e];
                                const float x0 = y[k][e], x1 = y[k2][e];
                                y[k][e] = x0 * cs - x1 * sn;
                                y[k2][e] = x1 * cs + x0 * sn;
                            }
                        }
                    }
                }
            }
        }
        __builtin_amdgcn_wave_barrier();

        const uint64_t dst = ((uint64_t)slot * a.Hkv + h) * a.D;
        if constexpr (OUT == OUT_FP8 && IN == IN_BF16 && NC % 2 == 0) {
            // An E4M3 chunk is 8 bytes, so storing chunks in place would write
            // each row in half-line pieces.  Instead the row's lanes exchange
            // codes so that lane j stores 16-byte pieces P = j + L p (chunks
            // 2P and 2P + 1) and one store instruction covers whole rows.
            // Chunk c sits in lane c mod L, slot c / L; for L >= 2 both
            // chunks of piece P come from lanes 2j mod L and 2j mod L + 1,
            // slot 2p + (2j >= L).  Every lane takes part in the exchange.
            u32x2 c[NC];
#pragma unroll
            for (int k = 0; k < NC; ++k)
                c[k] = u32x2{e4m3_sat_x4(y[k][0], y[k][1], y[k][2], y[k][3]),
                             e4m3_sat_x4(y[k][4], y[k][5], y[k][6], y[k][7])};
            const int src0 = (int)(lane - lir + ((2 * lir) & (a.L - 1)));
            const int src1 = a.L > 1 ? src0 + 1 : src0;
            const bool upper = 2 * lir >= a.L;
            uint8_t* base = (uint8_t*)a.k_cache + dst;
#pragma unroll
            for (int p = 0; p < NC / 2; ++p) {
                u32x4 v;
                if (a.L == 1) {
                    v = u32x4{c[2 * p][0], c[2 * p][1], c[2 * p + 1][0], c[2 * p + 1][1]};
                } else {
                    const uint32_t a0 = __shfl(c[2 * p][0], src0, 64);
                    const uint32_t a1 = __shfl(c[2 * p][1], src0, 64);
                    const uint32_t a2 = __shfl(c[2 * p][0], src1, 64);
                    const uint32_t a3 = __shfl(c[2 * p][1], src1, 64);
                    const uint32_t b0 = __shfl(c[2 * p + 1][0], src0, 64);
                    const uint32_t b1 = __shfl(c[2 * p + 1][1], src0, 64);
                    const uint32_t b2 = __shfl(c[2 * p + 1][0], src1, 64);
                    const uint32_t b3 = __shfl(c[2 * p + 1][1], src1, 64);
                    v = upper ? u32x4{b0, b1, b2, b3} : u32x4{a0, a1, a2, a3};
                }
                if (row_ok)
                    store_nt((u32x4*)(base + (uint64_t)(lir + a.L * p) * 16), v);
            }
        } else if (row_ok) {
#pragma unroll
            for (int k = 0; k < NC; ++k)
                store_chunk<OUT, VEC>(a.k_cache, dst + (uint64_t)(lir + a.L * k) * VEC, y[k]);
        }
    };

    if (u0 < u1) {
        // (token, group) cursors instead of dividing the unit index each time
        const uint32_t U = a.units_per_token;
        // token indices fit 32 bits (num_tokens is a uint32); readfirstlane
        // keeps the cursors in scalar registers
        uint32_t lt = __builtin_amdgcn_readfirstlane((uint32_t)(u0 / U)), pt = lt;
        uint32_t lg = __builtin_amdgcn_readfirstlane((uint32_t)(u0 % U)), pg = lg;
        auto next = [&](uint32_t& t, uint32_t& g) {
            if (++g == U) {
                g = 0;
                ++t;
            }
        };
        const uint32_t n = (uint32_t)(u1 - u0);
        // loads run two units ahead of processing (a ring of three rows)
        Raw ra, rb, rc;
        load_unit(lt, lg, ra);
        next(lt, lg);
        if (n > 1) {
            load_unit(lt, lg, rb);
            next(lt, lg);
        }
        convert_weights();
        for (uint32_t i = 0;;) {
            if (i + 2 < n) {
                load_unit(lt, lg, rc);
                next(lt, lg);
            }
            process(pt, pg, ra);
            next(pt, pg);
            if (++i == n)
                break;
            if (i + 2 < n) {
                load_unit(lt, lg, ra);
                next(lt, lg);
            }
            process(pt, pg, rb);
            next(pt, pg);
            if (++i == n)
                break;
            if (i + 2 < n) {
                load_unit(lt, lg, rb);
                next(lt, lg);
            }
            process(pt, pg, rc);
            next(pt, pg);
            if (++i == n)
                break;
        }
    }
}

// ------------------------------------------------------------------ host

template <int IN, int OUT>
static bool launch_nc(int nc, dim3 grid, hipStream_t st, const KWriteArgs& a)
{
    switch (nc) {
    case 1: hipLaunchKernelGGL((cache_write_k_kernel<IN, OUT, 1>), grid, dim3(kKThreads), 0, st, a, a.slots, a.pos_t, a.pos_h, a.pos_w); return true;
    case 2: hipLaunchKernelGGL((cache_write_k_kernel<IN, OUT, 2>), grid, dim3(kKThreads), 0, st, a, a.slots, a.pos_t, a.pos_h, a.pos_w); return true;
    case 3: hipLaunchKernelGGL((cache_write_k_kernel<IN, OUT, 3>), grid, dim3(kKThreads), 0, st, a, a.slots, a.pos_t, a.pos_h, a.pos_w); return true;
    case 4: hipLaunchKernelGGL((cache_write_k_kernel<IN, OUT, 4>), grid, dim3(kKThreads), 0, st, a, a.slots, a.pos_t, a.pos_h, a.pos_w); return true;
    case 6: hipLaunchKernelGGL((cache_write_k_kernel<IN, OUT, 6>), grid, dim3(kKThreads), 0, st, a, a.slots, a.pos_t, a.pos_h, a.pos_w); return true;
    case 8: hipLaunchKernelGGL((cache_write_k_kernel<IN, OUT, 8>), grid, dim3(kKThreads), 0, st, a, a.slots, a.pos_t, a.pos_h, a.pos_w); return true;
    default: return false;
    }
}

template <int IN>
static bool launch_out(pkv_dtype out, int nc, dim3 grid, hipStream_t st, const KWriteArgs& a)
{
    switch (out) {
    case PKV_BF16: return launch_nc<IN, OUT_BF16>(nc, grid, st, a);
    case PKV_FP8_E4M3: return launch_nc<IN, OUT_FP8>(nc, grid, st, a);
    default: return launch_nc<IN, OUT_F32>(nc, grid, st, a);
    }
}

}  // namespace pkv

extern "C" int pkv_cache_write_k_fused(const void* k_in, pkv_dtype in_dtype,
                                       uint64_t in_token_stride, const void* norm_weight,
                                       float rms_eps, const int32_t* pos_t, const int32_t* pos_h,
                                       const int32_t* pos_w, float theta, uint32_t rope_offset,
                                       uint32_t rotary_dim, int nope,
                                       const int64_t* slot_mapping, uint32_t num_tokens,
                                       uint32_t num_kv_heads, uint32_t head_dim,
                                       uint32_t block_size, uint32_t num_blocks, void* k_cache,
                                       pkv_dtype cache_dtype, float k_scale, void* stream)
{
    using namespace pkv;
    clear_error();
    if (num_tokens == 0)
        return PKV_OK;
    if (!k_in || !slot_mapping || !k_cache)
        return fail(PKV_ERR_INVALID, "cache_write_k_fused: k_in, slot_mapping and k_cache must be non-NULL");
    if (!valid_dtype(in_dtype) || !valid_dtype(cache_dtype))
        return fail(PKV_ERR_INVALID, "cache_write_k_fused: bad dtype");
    if (in_dtype != PKV_BF16 && in_dtype != PKV_FP32)
        return fail(PKV_ERR_UNSUPPORTED, "cache_write_k_fused: in_dtype must be BF16 or FP32");
    if (num_kv_heads == 0 || head_dim == 0 || block_size == 0 || num_blocks == 0)
        return fail(PKV_ERR_INVALID, "cache_write_k_fused: zero dimension");
    if (head_dim != 64 && head_dim != 128 && head_dim != 192 && head_dim != 256)
        return fail(PKV_ERR_UNSUPPORTED, "cache_write_k_fused: head_dim %u not in {64,128,192,256}", head_dim);
    const uint64_t row = (uint64_t)num_kv_heads * head_dim;
    if (in_token_stride < row)
        return fail(PKV_ERR_INVALID, "cache_write_k_fused: in_token_stride smaller than a token row");
    const uint32_t es = (uint32_t)dtype_size(in_dtype);
    const uint32_t VEC = 16 / es;
    if ((in_token_stride * es) % 16 || !aligned16(k_in) || !aligned16(k_cache) ||
        (norm_weight && !aligned16(norm_weight)))
        return fail(PKV_ERR_UNSUPPORTED, "cache_write_k_fused: k_in/k_cache/norm_weight and the token stride must be 16-byte aligned");
    // 1/k_scale is folded into the row factor: a subnormal k_scale would make
    // it infinite (and 0 * inf a NaN code), so the scale must be a normal number
    if (cache_dtype == PKV_FP8_E4M3 && !(k_scale >= FLT_MIN && k_scale < INFINITY))
        return fail(PKV_ERR_INVALID, "cache_write_k_fused: k_scale must be finite and >= FLT_MIN (2^-126)");
    const bool rope = !nope && rotary_dim > 0;
    if (rope) {
        if (!pos_t)
            return fail(PKV_ERR_INVALID, "cache_write_k_fused: pos_t must be non-NULL when rotating");
        if ((pos_h == nullptr) != (pos_w == nullptr))
            return fail(PKV_ERR_INVALID, "cache_write_k_fused: pos_h and pos_w must be both set or both NULL");
        if (rotary_dim % 2 || (uint64_t)rope_offset + rotary_dim > head_dim)
            return fail(PKV_ERR_INVALID, "cache_write_k_fused: rotary_dim must be even and rope_offset + rotary_dim <= head_dim");
        if (rotary_dim / 2 > (uint32_t)kMaxHalf)
            return fail(PKV_ERR_UNSUPPORTED, "cache_write_k_fused: rotary_dim above 256");
        if (rope_offset % VEC || (rotary_dim / 2) % VEC)
            return fail(PKV_ERR_UNSUPPORTED, "cache_write_k_fused: rope_offset and rotary_dim/2 must be multiples of %u", VEC);
    }
    // lanes per row: the largest power of two <= 16 that divides the row's
    // chunk count and (when rotating) the pair distance in chunks, leaving a
    // supported number of chunks per lane
    const uint32_t chunks = head_dim / VEC;
    const uint32_t pair = rope ? (rotary_dim / 2) / VEC : 0;
    uint32_t L = 0, NC = 0;
    for (uint32_t l = 16; l >= 1; l >>= 1) {
        if (chunks % l || (rope && pair % l))
            continue;
        uint32_t nc = chunks / l;
        if (nc == 1 || nc == 2 || nc == 3 || nc == 4 || nc == 6 || nc == 8) {
            if (rope && nc < 2)
                continue;
            L = l;
            NC = nc;
            break;
        }
    }
    if (L == 0)
        return fail(PKV_ERR_UNSUPPORTED, "cache_write_k_fused: no lane layout for head_dim %u rotary_dim %u", head_dim, rotary_dim);

    KWriteArgs a{};
    a.k_in = k_in;
    a.norm_w = norm_weight;
    a.pos_t = pos_t;
    a.pos_h = pos_h;
    a.pos_w = pos_w;
    a.slots = slot_mapping;
    a.k_cache = k_cache;
    a.in_stride = in_token_stride;
    a.num_slots = (uint64_t)num_blocks * block_size;
    a.eps = rms_eps;
    a.theta = theta;
    a.k_scale = k_scale;
    a.inv_k_scale = cache_dtype == PKV_FP8_E4M3 ? 1.0f / k_scale : 1.0f;
    a.inv_d = 1.0f / (float)head_dim;
    a.D = head_dim;
    a.Hkv = num_kv_heads;
    a.rope_first = rope ? rope_offset / VEC : 0;
    a.rope_chunks = pair;
    a.half = rope ? rotary_dim / 2 : 0;
    a.rot_dim = rope ? rotary_dim : 1;
    for (uint32_t i = 0; i < (uint32_t)kMaxHalf; ++i)
        a.invf[i] = i < a.half ? (float)std::pow((double)theta, -(2.0 * (double)i) / (double)rotary_dim)
                               : 0.f;
    a.L = L;
    a.rows_per_wave = 64 / L;
    a.units_per_token = ceil_div(num_kv_heads, a.rows_per_wave);
    a.num_units = (uint64_t)num_tokens * a.units_per_token;
    // units per wave: one for BF16 and FP32 stores (the most waves in
    // flight), up to sixteen for E4M3 stores, whose lane exchange does more
    // per unit.  Population writes of 1.09 M (BF16) / 1.58 M (E4M3) tokens:
    // 0.812 / 0.852 / 0.866 / 0.871 ms (BF16) with at most 1 / 8 / 4 / 16
    // units, 1.036 / 0.913 / 0.918 / 0.946 ms (E4M3) with at most 1 / 2 /
    // 4 / 16 (one run each, rows loaded one unit ahead); with the slot and
    // positions loaded with the row and rows two units ahead, 0.920 / 0.919 /
    // 0.909 / 0.895 ms (E4M3) with at most 2 / 4 / 8 / 16 (means of two runs)
    // and 0.814 / 0.845 / 0.870 ms (BF16) with at most 1 / 2 / 4.
    const uint64_t target_waves = 256ull * 32;
    const uint64_t max_upw = cache_dtype == PKV_FP8_E4M3 ? 16 : 1;
    uint64_t upw = a.num_units / target_waves;
    upw = upw < 1 ? 1 : upw > max_upw ? max_upw : upw;
    a.units_per_wave = (uint32_t)upw;
    const uint64_t waves = (a.num_units + upw - 1) / upw;
    const uint64_t blocks = (waves + kKWaves - 1) / kKWaves;
    const dim3 grid((uint32_t)blocks);
    hipStream_t st = (hipStream_t)stream;
    bool ok = in_dtype == PKV_BF16 ? launch_out<IN_BF16>(cache_dtype, (int)NC, grid, st, a)
                                   : launch_out<IN_F32>(cache_dtype, (int)NC, grid, st, a);
    if (!ok)
        return fail(PKV_ERR_UNSUPPORTED, "cache_write_k_fused: chunk count %u per lane", NC);
    return check_launch("cache_write_k_fused");
}

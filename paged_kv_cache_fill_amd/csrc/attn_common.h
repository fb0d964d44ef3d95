// attn_common.h -- device pieces shared by the paged attention kernels of
// libpkv (decode and prefill, gfx950): cache block size, buffer-load flags,
// the K operand layout of the QK^T MFMA (coalesced row loads turned into
// MFMA operands through a swizzled LDS tile), lane reductions, BF16 pair
// packing, and the normalisation of a finished softmax row with an optional
// sink.  Not part of the public ABI.
#pragma once

#include "pkv_internal.h"

namespace pkv {

constexpr int kBS = 16;                 // tokens per cache block
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBufferFlags = 0x00020000; // buffer resource word 3: raw 32-bit dwords
constexpr int kNT = 2;                   // cache policy of streaming loads: non-temporal

__device__ __forceinline__ float wave_max_xor16_32(float v)
{
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    v = fmaxf(v, __shfl_xor(v, 32, 64));
    return v;
}

__device__ __forceinline__ float wave_sum_xor16_32(float v)
{
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

// The same reductions with gfx950's row swaps: v_permlane16_swap (v, v)
// returns v's xor-16 partners across the two results, v_permlane32_swap the
// xor-32 ones, so the max of the pair is the exchange-and-reduce step -- no
// lane-address arithmetic and no LDS round trip.
__device__ __forceinline__ float row_max_xor16_32(float v)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float row_sum_xor16_32(float v)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// bytes 2,3 of lo and 2,3 of hi -> one word (two BF16 from two FP32)
__device__ __forceinline__ uint32_t hi16_pair(uint32_t lo, uint32_t hi)
{
    return __builtin_amdgcn_perm(hi, lo, 0x07060302u);
}
// low halves of lo and hi -> one word
__device__ __forceinline__ uint32_t lo16_pair(uint32_t lo, uint32_t hi)
{
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Normalisation factor of a finished row: out = o * norm_factor(...).  With
// a sink (log2 units sk2) the denominator l 2^m gains 2^sk2; a row with no
// attended token (l = 0) stays zero.
__device__ __forceinline__ float norm_factor(float m, float l, const float* sinks, uint32_t h,
                                             float out_scale)
{
    if (!(l > 0.f))
        return 0.f;
    if (sinks) {
        const float sk2 = sinks[h] * kLog2e;
        const float mm = fmaxf(m, sk2);
        const float f = __builtin_amdgcn_exp2f(m - mm);
        return f * out_scale / (l * f + __builtin_amdgcn_exp2f(sk2 - mm));
    }
    return out_scale / l;
}

// KT: 0 = BF16 K, 1 = E4M3 K.  D: head dim of q and K (64 or 128).
//
// K reaches the MFMA in two steps.  (1) Coalesced loads: a K row of one head
// is CPR 16-byte chunks; load j of a lane covers row j * (64 / CPR) + lane /
// CPR, chunk lane % CPR, so each load instruction reads whole rows.  (2) A
// wave-private LDS tile [16 rows][CPR chunks] turns that into the MFMA
// operand layout (lane = token row ln, chunk group kg).  Chunk c of row r is
// stored at position c ^ swz(r), which makes both the row-wise writes and the
// column-wise operand reads free of bank conflicts.
template <int KT, int D>
struct KFrag {
    static constexpr int KES = KT == 0 ? 2 : 1;      // K element bytes
    static constexpr int CPR = D * KES / 16;         // 16-byte chunks per row
    static constexpr int RPL = 64 / CPR;             // rows per load instruction
    static constexpr int NL = 16 / RPL;              // loads (and LDS chunks) per lane
    static constexpr int NI = D / 32;                // MFMAs over the head dim (16x16x32)
    static constexpr int RP = 16 / CPR;              // rows per 256-byte LDS line
    __device__ static uint32_t swz(uint32_t row) { return (row / RP) & (CPR - 1); }
    // LDS byte offset of chunk c of row r
    __device__ static uint32_t lds_off(uint32_t r, uint32_t c) { return (r * CPR + (c ^ swz(r))) * 16; }
    // physical element of logical k = 8*kg + r of MFMA i (same permutation on q)
    __device__ static uint32_t phys(int i, int kg)
    {
        return KT == 0 ? 32u * i + 8u * kg : 64u * (i / 2) + 16u * kg + 8u * (i % 2);
    }
    // chunk holding the operand of MFMA i (BF16) or MFMAs 2i, 2i+1 (E4M3) for group kg
    __device__ static uint32_t op_chunk(int j, int kg) { return 4u * j + kg; }
    // MFMA operand i (8 BF16) from the operand chunks w[]
    __device__ static bf16x8 operand(const u32x4 (&w)[NL], int i)
    {
        if constexpr (KT == 0) {
            return __builtin_bit_cast(bf16x8, w[i]);
        } else {
            const u32x4 src = w[i / 2];
            const int base = (i % 2) * 2;     // words base, base+1 hold 8 codes
            u32x4 r;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                // E4M3 values are exact in BF16: widen each pair of codes in
                // one step (v_cvt_scalef32_pk_bf16_fp8, scale 1)
                const uint32_t word = src[base + q];
                r[2 * q] = __builtin_bit_cast(
                    uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, false));
                r[2 * q + 1] = __builtin_bit_cast(
                    uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, true));
            }
            return __builtin_bit_cast(bf16x8, r);
        }
    }
};

}  // namespace pkv

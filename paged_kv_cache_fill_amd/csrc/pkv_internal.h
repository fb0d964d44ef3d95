// pkv_internal.h -- shared device helpers and host-side status plumbing of
// libpkv (gfx950).  Not part of the public ABI (that is include/pkv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "pkv.h"

namespace pkv {

// ---------------------------------------------------------------- host side

// Records a message for pkv_last_error() and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the message (start of every entry point).
void clear_error();
// Checks the launch that just happened on the calling thread.
int check_launch(const char* what);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t dtype_size(pkv_dtype t)
{
    return t == PKV_BF16 ? 2 : t == PKV_FP32 ? 4 : 1;
}

inline bool valid_dtype(int t) { return t == PKV_BF16 || t == PKV_FP8_E4M3 || t == PKV_FP32; }

// TurboQuant-style V formats (V caches only)
inline bool is_tq(int t) { return t == PKV_TQ2 || t == PKV_TQ3 || t == PKV_TQ4; }
inline int tq_bits(int t) { return t - PKV_TQ2 + 2; }

// A TQ codebook: E4M3 codes and values of the 2^(b-1) positive magnitudes
// (ascending), the encoder's magnitude thresholds (midpoints; +inf past the
// last), and the decoder's 8-entry FP16 level table as byte-lookup words:
// f16_lut[0], [1] hold the low bytes of entries 0-3 and 4-7, f16_lut[2], [3]
// the high bytes.  Entry e is the level of code e (sign << (b-1) | index)
// for b = 2, 3 and the magnitude of index e for b = 4.
struct TqCodebook {
    int bits, mags_count;
    uint8_t codes[8];
    float mags[8];
    float thr[7];
    uint32_t f16_lut[4];
};
const TqCodebook& tq_codebook(int bits);
uint64_t tq_block_bytes(int bits, uint32_t B, uint32_t H, uint32_t D);

inline uint32_t ceil_div(uint64_t a, uint64_t b) { return (uint32_t)((a + b - 1) / b); }

// ---------------------------------------------------------------- device side

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Two BF16 halves of a 32-bit word -> FP32 (exact: BF16 is the top half of
// a binary32 pattern).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two FP32 -> packed BF16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b)
{
    bf16x2 v;
    v.x = (__bf16)a;
    v.y = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}

// Bitfield insert: bits of a where m is set, bits of b elsewhere (v_bfi_b32).
__device__ __forceinline__ uint32_t bit_insert(uint32_t m, uint32_t a, uint32_t b)
{
    return (a & m) | (b & ~m);
}

// Two FP32 -> packed FP16, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16(float a, float b)
{
    f16x2 v;
    v.x = (_Float16)a;
    v.y = (_Float16)b;
    return __builtin_bit_cast(uint32_t, v);
}

// Four FP32 -> four E4M3FN bytes in a word (v_cvt_pk_fp8_f32, round to
// nearest even).  Callers clamp finite magnitudes to 448 first.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Four FP32 -> four saturating E4M3FN codes: magnitudes above 448, infinite
// ones included, become +-448 (v_med3 clamp, then round to nearest even);
// NaN becomes the NaN code S.1111.111 with its sign.
__device__ __forceinline__ uint32_t e4m3_sat_x4(float a, float b, float c, float d)
{
    uint32_t w = pack_e4m3x4(__builtin_amdgcn_fmed3f(a, -448.0f, 448.0f),
                             __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f),
                             __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f),
                             __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f));
    if ((a != a) | (b != b) | (c != c) | (d != d)) {
        const float y[4] = {a, b, c, d};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (y[i] != y[i]) {
                const uint32_t code = 0x7Fu | ((__float_as_uint(y[i]) >> 24) & 0x80u);
                w = (w & ~(0xFFu << (8 * i))) | (code << (8 * i));
            }
        }
    }
    return w;
}

// Two E4M3FN bytes (selected by `hi`) -> two FP32, exact.
__device__ __forceinline__ f32x2 unpack_e4m3x2(uint32_t w, bool hi)
{
    return hi ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true)
              : __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
}

// DPP row operations (gfx9 encodings): lane i of each 16-lane row takes the
// value of lane i ^ 1, i ^ 2 (quad permutes), 7 - i within its half-row, or
// 15 - i within its row.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Sum over aligned groups of L = 2, 4, 8 or 16 consecutive lanes, left in
// every lane of the group (pairs, quads, mirrored half-rows, mirrored rows:
// one DPP add each, no LDS); L is wave-uniform.
__device__ __forceinline__ float group_sum(float v, uint32_t L)
{
    if (L >= 2)
        v += dpp_f32<kDppXor1>(v);
    if (L >= 4)
        v += dpp_f32<kDppXor2>(v);
    if (L >= 8)
        v += dpp_f32<kDppHalfMirror>(v);
    if (L >= 16)
        v += dpp_f32<kDppMirror>(v);
    return v;
}
__device__ __forceinline__ float row16_sum(float v) { return group_sum(v, 16); }

// Streaming (read-once / write-once) 16-byte accesses.
__device__ __forceinline__ u32x4 load_nt(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_nt(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

}  // namespace pkv

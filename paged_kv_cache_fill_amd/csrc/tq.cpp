// tq.cpp -- host side of the TurboQuant-style V formats (PKV_TQ2/3/4; page 1,
// kv_cache.rs, reshape_and_cache_bf16k_turbo{2,3,4}v: b-bit Lloyd-Max codes
// plus an FP8 per-group scale; page 2: one FP8 scale per 16 elements): the
// codebook with the decoder's FP16 level table, and the block-size query.
//
// Codebook: the positive levels of the 2^b-level Lloyd-Max quantiser of the
// standard normal distribution (the classical optimum tabulated by J. Max,
// "Quantizing for minimum distortion", IRE Trans. Inform. Theory, 1960:
// b = 2: 0.4528, 1.510; b = 3: 0.2451, 0.7560, 1.344, 2.152; b = 4: 0.1284,
// 0.3881, 0.6568, 0.9424, 1.256, 1.618, 2.069, 2.733), each rounded to the
// nearest E4M3 value (the closest to a rounding midpoint, 0.45278 against
// 0.453125, is 3e-4 clear of it), stored as E4M3 codes.  A decoded value, level x E4M3 scale, is then a
// product of two E4M3 numbers.
#include <cmath>
#include <cstring>
#include <mutex>

#include "pkv_internal.h"

namespace pkv {

static double e4m3_value(uint8_t c)
{
    const int field = (c >> 3) & 15, man = c & 7;
    const double v = field ? std::ldexp(1.0 + man / 8.0, field - 7) : std::ldexp(man / 8.0, -6);
    return (c & 0x80) ? -v : v;
}

// IEEE binary16 bits of a value that binary16 holds exactly (a normal number
// with at most 11 significant bits, as every E4M3 magnitude of the codebook).
static uint16_t f16_bits(double v)
{
    if (v == 0.0)
        return 0;
    const uint16_t sign = v < 0 ? 0x8000 : 0;
    int e2;
    const double f = std::frexp(std::fabs(v), &e2);   // |v| = f * 2^e2, f in [0.5, 1)
    const int field = e2 - 1 + 15;
    const int man = (int)std::ldexp(2.0 * f - 1.0, 10);
    return (uint16_t)(sign | field << 10 | man);
}

// E4M3 codes of the positive magnitudes, ascending (b = 2, 3, 4):
// 0x2E 0.4375, 0x3C 1.5; 0x28 0.25, 0x34 0.75, 0x3B 1.375, 0x41 2.25;
// 0x20 0.125, 0x2C 0.375, 0x33 0.6875, 0x37 0.9375, 0x3A 1.25, 0x3D 1.625,
// 0x40 2, 0x43 2.75.
static const uint8_t kMagCodes2[2] = {0x2E, 0x3C};
static const uint8_t kMagCodes3[4] = {0x28, 0x34, 0x3B, 0x41};
static const uint8_t kMagCodes4[8] = {0x20, 0x2C, 0x33, 0x37, 0x3A, 0x3D, 0x40, 0x43};

const TqCodebook& tq_codebook(int bits)
{
    static TqCodebook books[3];
    static std::once_flag once[3];
    const int i = bits - 2;
    std::call_once(once[i], [&] {
        TqCodebook& b = books[i];
        std::memset(&b, 0, sizeof b);
        b.bits = bits;
        b.mags_count = 1 << (bits - 1);
        const uint8_t* codes = bits == 2 ? kMagCodes2 : bits == 3 ? kMagCodes3 : kMagCodes4;
        for (int j = 0; j < b.mags_count; ++j) {
            b.codes[j] = codes[j];
            b.mags[j] = (float)e4m3_value(b.codes[j]);
        }
        for (int j = 0; j + 1 < b.mags_count; ++j)
            b.thr[j] = 0.5f * (b.mags[j] + b.mags[j + 1]);   // exact: E4M3 sums
        for (int j = b.mags_count - 1; j < 7; ++j)
            b.thr[j] = INFINITY;
        for (int e = 0; e < 8; ++e) {
            double v = 0.0;
            if (bits == 4)
                v = b.mags[e];
            else if (e < 2 * b.mags_count)
                v = e < b.mags_count ? b.mags[e] : -b.mags[e - b.mags_count];
            const uint16_t h = f16_bits(v);
            b.f16_lut[e / 4] |= (uint32_t)(h & 0xFF) << (8 * (e % 4));
            b.f16_lut[2 + e / 4] |= (uint32_t)(h >> 8) << (8 * (e % 4));
        }
    });
    return books[i];
}

uint64_t tq_block_bytes(int bits, uint32_t B, uint32_t H, uint32_t D)
{
    return (uint64_t)B * H * D * bits / 8 + (uint64_t)B * H * D / 16;
}

}  // namespace pkv

extern "C" size_t pkv_v_block_bytes(pkv_dtype v_dtype, uint32_t block_size, uint32_t num_kv_heads,
                                    uint32_t head_dim_v)
{
    using namespace pkv;
    if (is_tq(v_dtype))
        return head_dim_v % 16 ? 0
                               : (size_t)tq_block_bytes(tq_bits(v_dtype), block_size, num_kv_heads,
                                                        head_dim_v);
    if (!valid_dtype(v_dtype))
        return 0;
    return (size_t)block_size * num_kv_heads * head_dim_v * dtype_size(v_dtype);
}

extern "C" int pkv_tq_codebook(pkv_dtype v_dtype, uint8_t* mag_codes)
{
    using namespace pkv;
    clear_error();
    if (!is_tq(v_dtype) || !mag_codes)
        return fail(PKV_ERR_INVALID, "tq_codebook: a TQ dtype and a non-NULL output are needed");
    const TqCodebook& b = tq_codebook(tq_bits(v_dtype));
    std::memcpy(mag_codes, b.codes, (size_t)b.mags_count);
    return PKV_OK;
}

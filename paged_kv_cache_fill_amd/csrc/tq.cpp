// tq.cpp -- host side of the TurboQuant-style V formats (PKV_TQ2/3/4; page 1,
// kv_cache.rs, reshape_and_cache_bf16k_turbo{2,3,4}v: b-bit Lloyd-Max codes
// plus an FP8 per-group scale; page 2: one FP8 scale per 16 elements): the
// codebook, computed once per bit width (with the decoder's FP16 level
// table), and the block-size query.
//
// Codebook: Lloyd's iteration on the standard normal density -- cells at
// the midpoints between levels, each level moved to its cell's conditional
// mean (phi(a) - phi(b)) / (Phi(b) - Phi(a)) -- to a fixed point; the
// positive levels are then rounded to E4M3 (round to nearest even).
#include <cmath>
#include <cstring>
#include <mutex>

#include "pkv_internal.h"

namespace pkv {

// E4M3FN code of a finite x >= 0, round to nearest even, saturating at 448.
static uint8_t e4m3_code(double x)
{
    if (!(x > 0.0))
        return 0;
    if (x >= 448.0)
        return 0x7E;
    int e2;
    std::frexp(x, &e2);                  // x = f * 2^e2, f in [0.5, 1)
    int E = e2 - 1;                      // x in [2^E, 2^(E+1))
    if (E < -6)
        E = -6;                          // subnormal range: quantum 2^-9
    const double quantum = std::ldexp(1.0, E - 3);
    double m = std::nearbyint(x / quantum);   // default mode: ties to even
    if (m >= 16.0) {                     // rounded up into the next binade
        m = 8.0;
        ++E;
    }
    if (m < 8.0)                         // subnormal (E == -6)
        return (uint8_t)m;
    const int field = E + 7;
    if (field > 15 || (field == 15 && m > 14.0))
        return 0x7E;
    return (uint8_t)((field << 3) | ((int)m - 8));
}

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

static void lloyd_max(int bits, double* lv)
{
    const int L = 1 << bits;
    for (int k = 0; k < L; ++k)
        lv[k] = -3.0 + 6.0 * (k + 0.5) / L;
    const double inv_sqrt2pi = 0.3989422804014326779;
    auto pdf = [&](double x) { return std::isinf(x) ? 0.0 : inv_sqrt2pi * std::exp(-0.5 * x * x); };
    auto cdf = [](double x) { return 0.5 * std::erfc(-x * 0.70710678118654752440); };
    for (int it = 0; it < 100000; ++it) {
        double next[16], worst = 0.0, lo = -INFINITY;
        for (int k = 0; k < L; ++k) {
            const double hi = k + 1 < L ? 0.5 * (lv[k] + lv[k + 1]) : INFINITY;
            next[k] = (pdf(lo) - pdf(hi)) / (cdf(hi) - cdf(lo));
            lo = hi;
        }
        for (int k = 0; k < L; ++k) {
            worst = std::fmax(worst, std::fabs(next[k] - lv[k]));
            lv[k] = next[k];
        }
        if (worst < 1e-15)
            break;
    }
}

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
        double lv[16];
        lloyd_max(bits, lv);
        for (int j = 0; j < b.mags_count; ++j) {
            b.codes[j] = e4m3_code(lv[b.mags_count + j]);
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

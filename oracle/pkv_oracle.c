/*
 * pkv_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU definition of the paged KV-cache path:
 * slot mapping, the fused K cache write (RMSNorm -> RoPE -> one rounding),
 * the V reshape-and-cache copy and paged decode attention.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  The product (the HIP library) never links, loads or
 * calls it, and the two share no source, header, table or helper.
 *
 * Arithmetic is FP64 except where the pages fix the precision:
 *   - the K path is held in FP32 at the store (page 1, kv_cache.rs, doc of
 *     fused_k_norm_rope_cache_write_bf16: K is kept in FP32 through the
 *     three operations and rounded once, at the cache write), so the
 *     quantisation decision is taken on fl32 of the FP64 result;
 *   - the RoPE angle is an FP32 product of the FP32 position and an FP32
 *     inverse frequency (the FP32 regime of the same doc; our reading).
 *
 * Sources cited below are the three pages:
 *   p1 = docs.atlasinference.io .../spark_model/layers/ops/kv_cache.rs
 *   p2 = docs.metrale.ai .../metrale_model_layers/layers/ops/kv_cache_fp8k.rs
 *   p3 = docs.atlascybernetics.ai .../spark_model/kimi_k3/mla_cuda.rs
 * Where the pages leave a step open, the plainest reading is taken and
 * stated beside the code that makes it.
 *
 * Pins (tests/test_oracle_*.py) tie every function here to closed forms,
 * library routines, format specifications and invariants.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Element types.  Numbered like the product's enum only by convention; the
 * values are restated here, not included. */
enum { O_BF16 = 0, O_E4M3 = 1, O_F32 = 2, O_TQ2 = 3, O_TQ3 = 4, O_TQ4 = 5 };

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

/* bfloat16 -> binary32: bf16 is the upper half of a binary32 pattern. */
float pkvo_f32_from_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* binary32 -> bfloat16, IEEE round-to-nearest-even, written from the
 * definition: take the two bf16 neighbours of x (truncation toward zero and
 * the next value away from zero) and keep the nearer one, the one with an
 * even last bit on a tie.  A value past the largest finite bf16 rounds to
 * infinity exactly when IEEE says so (the "next" neighbour is then inf and
 * the tie/nearness test is done in double).  NaN returns a quiet NaN of the
 * same sign. */
uint16_t pkvo_bf16_from_f32(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if (isnan(x))
        return (uint16_t)((u >> 16) | 0x0040u);
    uint16_t lo = (uint16_t)(u >> 16);           /* |lo| <= |x|, same sign */
    if ((u & 0xFFFFu) == 0)
        return lo;                               /* exactly representable */
    uint16_t hi = (uint16_t)(lo + 1);            /* next bf16 away from zero */
    double dx = fabs((double)x);
    double dlo = fabs((double)pkvo_f32_from_bf16(lo));
    double dhi;
    if ((hi & 0x7FFFu) == 0x7F80u) {
        /* The neighbour past the largest finite value is infinity; IEEE
         * rounds to it when x is at or beyond the midpoint between the
         * largest finite value and 2^128 (the value the next step would
         * have had with an unbounded exponent). */
        dhi = ldexp(1.0, 128);
    } else {
        dhi = fabs((double)pkvo_f32_from_bf16(hi));
    }
    double elo = dx - dlo, ehi = dhi - dx;
    if (elo < ehi) return lo;
    if (ehi < elo) return hi;
    return (lo & 1u) ? hi : lo;                  /* tie: even last bit */
}

/* OCP 8-bit floating point, E4M3FN: 1 sign bit, 4 exponent bits (bias 7),
 * 3 mantissa bits, no infinities, NaN = S.1111.111, largest finite 448.
 * Value of a non-negative code c (c < 0x7F):
 *   exponent field e = c >> 3, mantissa m = c & 7
 *   e == 0 : m * 2^-9                  (subnormal)
 *   e >= 1 : (8 + m) * 2^(e - 10)      (normal)                        */
double pkvo_f64_from_e4m3(uint8_t c)
{
    int neg = (c & 0x80) != 0;
    int mag = c & 0x7F;
    if (mag == 0x7F)
        return neg ? -NAN : NAN;
    int e = mag >> 3, m = mag & 7;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return neg ? -v : v;
}

/* x -> E4M3FN by round-to-nearest-even over the 127 non-negative finite
 * codes, saturating: a magnitude above 448 (infinity included) becomes 448
 * (p1 kv_cache.rs, doc of fused_k_norm_rope_cache_write_fp8: the cast to
 * FP8 saturates).  NaN becomes the NaN code of the same
 * sign.  Zero keeps its sign.  Written as a nearest-value search over the
 * code table, so it follows the format definition directly. */
uint8_t pkvo_e4m3_from_f64(double x)
{
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    if (isnan(x))
        return (uint8_t)(sign | 0x7F);
    double a = fabs(x);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7E);
    int best = 0;
    double best_err = a;                         /* distance to code 0 */
    for (int c = 1; c <= 0x7E; ++c) {
        double err = fabs(a - pkvo_f64_from_e4m3((uint8_t)c));
        if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_err = err;
        }
    }
    return (uint8_t)(sign | best);
}

/* ------------------------------------------------------------------ */
/* Threading helper: split [0, n) over nthreads workers.               */
/* ------------------------------------------------------------------ */

typedef void (*range_fn)(void* ctx, uint64_t begin, uint64_t end);

typedef struct {
    range_fn fn;
    void* ctx;
    uint64_t begin, end;
} range_job;

static void* range_trampoline(void* p)
{
    range_job* j = (range_job*)p;
    j->fn(j->ctx, j->begin, j->end);
    return NULL;
}

static void parallel_for(uint64_t n, int nthreads, range_fn fn, void* ctx)
{
    if (nthreads < 1) nthreads = 1;
    if ((uint64_t)nthreads > n) nthreads = (int)(n ? n : 1);
    if (nthreads == 1) {
        fn(ctx, 0, n);
        return;
    }
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    range_job* jobs = (range_job*)malloc(sizeof(range_job) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) {
        jobs[i].fn = fn;
        jobs[i].ctx = ctx;
        jobs[i].begin = n * (uint64_t)i / (uint64_t)nthreads;
        jobs[i].end = n * (uint64_t)(i + 1) / (uint64_t)nthreads;
        pthread_create(&th[i], NULL, range_trampoline, &jobs[i]);
    }
    for (int i = 0; i < nthreads; ++i)
        pthread_join(th[i], NULL);
    free(th);
    free(jobs);
}

/* ------------------------------------------------------------------ */
/* (1) Slot mapping                                                    */
/* ------------------------------------------------------------------ */

/* For sequence s and its i-th token (p = start_pos[s] + i, i < count_s):
 *   slot = block_table[s][p / B] * B + p % B
 * (p1 kv_cache.rs, doc of fill_slots_from_block_table: slots are filled on
 * the device from a persistent block table, positions start_pos onward, with
 * block_size; slot_mapping is i64 per the doc of reshape_and_cache; a slot is
 * the flat row index of the [num_blocks, block_size] pool).  Batched: token range of sequence s
 * is [cu_counts[s], cu_counts[s+1]).  A position whose block index falls
 * outside the table, or a negative position, gives slot -1 (padding). */
void pkvo_fill_slots(int64_t* slots, const int32_t* block_tables, uint32_t max_blocks_per_seq,
                     const int32_t* start_pos, const int32_t* cu_counts, uint32_t num_seqs,
                     uint32_t total_tokens, uint32_t block_size)
{
    for (uint32_t i = 0; i < total_tokens; ++i)
        slots[i] = -1;
    for (uint32_t s = 0; s < num_seqs; ++s) {
        for (int64_t i = cu_counts[s]; i < cu_counts[s + 1]; ++i) {
            if (i < 0 || i >= (int64_t)total_tokens)
                continue;
            int64_t p = (int64_t)start_pos[s] + (i - cu_counts[s]);
            if (p < 0)
                continue;
            int64_t b = p / (int64_t)block_size;
            if (b >= (int64_t)max_blocks_per_seq)
                continue;
            int64_t blk = block_tables[(uint64_t)s * max_blocks_per_seq + (uint64_t)b];
            slots[i] = blk * (int64_t)block_size + p % (int64_t)block_size;
        }
    }
}

/* ------------------------------------------------------------------ */
/* (2) RoPE frequency                                                  */
/* ------------------------------------------------------------------ */

/* Inverse frequency of rotation pair i over rotary_dim R:
 *   theta^(-2i/R), rounded once to FP32.                              */
float pkvo_rope_inv_freq(float theta, uint32_t i, uint32_t rotary_dim)
{
    return (float)pow((double)theta, -(2.0 * (double)i) / (double)rotary_dim);
}

/* Angle of pair i at integer position pos: one FP32 product. */
float pkvo_rope_angle(int32_t pos, float inv_freq)
{
    volatile float p = (float)pos;               /* keep it a single fp32 multiply */
    volatile float a = p * inv_freq;
    return a;
}

/* Rotate y[offset .. offset+R) in place: NeoX rotate-half pairs (i, i+R/2).
 * For pair i:  a' = a cos(t) - b sin(t),   b' = b cos(t) + a sin(t),
 * t the FP32 angle of pair i, cos/sin evaluated in double. */
static void rope_rotate(double* y, uint32_t offset, uint32_t R, float theta,
                        const int32_t* pos3 /* pos for i%3 = 0,1,2 */)
{
    uint32_t half = R / 2;
    for (uint32_t i = 0; i < half; ++i) {
        float invf = pkvo_rope_inv_freq(theta, i, R);
        float ang = pkvo_rope_angle(pos3[i % 3], invf);
        double c = cos((double)ang), s = sin((double)ang);
        double a = y[offset + i], b = y[offset + i + half];
        y[offset + i] = a * c - b * s;
        y[offset + i + half] = b * c + a * s;
    }
}

static double load_elem(const void* base, int dtype, uint64_t idx)
{
    switch (dtype) {
    case O_BF16: return (double)pkvo_f32_from_bf16(((const uint16_t*)base)[idx]);
    case O_F32: return (double)((const float*)base)[idx];
    default: return pkvo_f64_from_e4m3(((const uint8_t*)base)[idx]);
    }
}

static size_t elem_size(int dtype)
{
    return dtype == O_BF16 ? 2 : dtype == O_F32 ? 4 : 1;
}

/* ------------------------------------------------------------------ */
/* (3) Fused K cache write                                             */
/* ------------------------------------------------------------------ */

typedef struct {
    const void* k_in; int in_dtype; uint64_t in_token_stride;
    const void* norm_weight; float eps;
    const int32_t *pos_t, *pos_h, *pos_w;
    float theta; uint32_t rope_offset, rotary_dim; int nope;
    const int64_t* slots; uint32_t num_kv_heads, head_dim;
    uint64_t num_slots; void* k_cache; int cache_dtype; float k_scale;
} kwrite_ctx;

static void kwrite_range(void* p, uint64_t t0, uint64_t t1)
{
    const kwrite_ctx* c = (const kwrite_ctx*)p;
    const uint32_t D = c->head_dim, H = c->num_kv_heads;
    double* y = (double*)malloc(sizeof(double) * D);
    for (uint64_t t = t0; t < t1; ++t) {
        int64_t slot = c->slots[t];
        if (slot < 0 || (uint64_t)slot >= c->num_slots)
            continue;                            /* padding slot: no write */
        for (uint32_t h = 0; h < H; ++h) {
            uint64_t src = t * c->in_token_stride + (uint64_t)h * D;
            for (uint32_t j = 0; j < D; ++j)
                y[j] = load_elem(c->k_in, c->in_dtype, src + j);
            /* RMSNorm over the whole head: y = x / sqrt(mean(x^2) + eps) * w
             * (p1 fused_k_norm_rope_cache_write_bf16: rms_norm with
             * k_norm_weight and rms_eps, first of the three fused steps) */
            if (c->norm_weight) {
                double ss = 0.0;
                for (uint32_t j = 0; j < D; ++j)
                    ss += y[j] * y[j];
                double r = 1.0 / sqrt(ss / (double)D + (double)c->eps);
                for (uint32_t j = 0; j < D; ++j)
                    y[j] = y[j] * r * load_elem(c->norm_weight, c->in_dtype, j);
            }
            /* RoPE at the token's position; the MRoPE variant picks the
             * position axis by pair index mod 3 (p1 doc of
             * fused_k_norm_rope_cache_write_bf16_mrope); NoPE skips it
             * (p3 module doc: NoPE skips rotate). */
            if (!c->nope && c->rotary_dim > 0) {
                int32_t pos3[3];
                pos3[0] = c->pos_t[t];
                pos3[1] = (c->pos_h && c->pos_w) ? c->pos_h[t] : pos3[0];
                pos3[2] = (c->pos_h && c->pos_w) ? c->pos_w[t] : pos3[0];
                rope_rotate(y, c->rope_offset, c->rotary_dim, c->theta, pos3);
            }
            /* One rounding at the store: the FP32 value of K, then BF16
             * round-to-nearest-even, or the saturating E4M3 cast of
             * k / k_scale (p2 module invariants: the write stores k/k_scale
             * as E4M3), or FP32 unchanged. */
            uint64_t dst = ((uint64_t)slot * H + h) * D;
            for (uint32_t j = 0; j < D; ++j) {
                float k32 = (float)y[j];
                switch (c->cache_dtype) {
                case O_BF16:
                    ((uint16_t*)c->k_cache)[dst + j] = pkvo_bf16_from_f32(k32);
                    break;
                case O_F32:
                    ((float*)c->k_cache)[dst + j] = k32;
                    break;
                default: {
                    float z = (float)((double)k32 / (double)c->k_scale); /* fl32(k/k_scale) */
                    ((uint8_t*)c->k_cache)[dst + j] = pkvo_e4m3_from_f64((double)z);
                }
                }
            }
        }
    }
    free(y);
}

void pkvo_cache_write_k(const void* k_in, int in_dtype, uint64_t in_token_stride,
                        const void* norm_weight, float eps,
                        const int32_t* pos_t, const int32_t* pos_h, const int32_t* pos_w,
                        float theta, uint32_t rope_offset, uint32_t rotary_dim, int nope,
                        const int64_t* slots, uint32_t num_tokens, uint32_t num_kv_heads,
                        uint32_t head_dim, uint32_t block_size, uint32_t num_blocks,
                        void* k_cache, int cache_dtype, float k_scale, int nthreads)
{
    kwrite_ctx c = {k_in, in_dtype, in_token_stride, norm_weight, eps, pos_t, pos_h, pos_w,
                    theta, rope_offset, rotary_dim, nope, slots, num_kv_heads, head_dim,
                    (uint64_t)num_blocks * block_size, k_cache, cache_dtype, k_scale};
    parallel_for(num_tokens, nthreads, kwrite_range, &c);
}

/* ------------------------------------------------------------------ */
/* TurboQuant-style V (p1 and p2: V as b-bit Lloyd-Max codes plus one  */
/* FP8 scale per group of 16 elements, with a norm correction)         */
/* ------------------------------------------------------------------ */

/* The pages name the ingredients (p1 reshape_and_cache_bf16k_turbo{2,3,4}v:
 * b-bit Lloyd-Max codes, an FP8 per-group scale, a matched-norm
 * correction; p2: one FP8 scale per 16 elements) and not their details.
 * Readings taken here:
 *  - codebook: the 2^b-level Lloyd-Max quantizer of the standard normal
 *    distribution, its levels rounded to E4M3 (so that a decoded value,
 *    scale x level, is a product of two E4M3 numbers); symmetric, code =
 *    sign << (b-1) | magnitude index, magnitudes ascending;
 *  - a group of 16 consecutive elements of a (token, kv head) row is coded
 *    as the nearest level of x / rms(x) (ties to the smaller magnitude, -0
 *    positive), and its scale is E4M3 of |x| / |levels of the codes| (the
 *    norm correction: the decoded group has the input's L2 norm up to the
 *    scale's rounding); an all-zero group stores scale 0 and code 0;
 *  - layout of a cache block of B tokens: one region per kv head h, at
 *    h * B * (D * b / 8 + D / 16); in it the code rows of tokens 0..B-1
 *    (token t at t * D * b / 8, group q at 2 b bytes each, element i at bits
 *    [b i, b i + b) of the group's little-endian bytes), then one scale row
 *    per group (scale of (t, q) at B * D * b / 8 + q * B + t).  A head's
 *    codes and scales of one block are thus contiguous (the pages fix no
 *    layout);
 *  - the encoder's decisions follow this definition in FP64 arithmetic:
 *    the rms, each x / rms, the nearest-level choice and the ratio of norms
 *    are exact up to FP64 rounding, and the ratio is rounded once, to E4M3;
 *  - no rotation; the decode is exact, and its sparse-V variant is
 *    pkvo_paged_decode_sparse_v. */

static double std_normal_pdf(double x) { return exp(-0.5 * x * x) / sqrt(2.0 * 3.14159265358979323846); }
static double std_normal_cdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

/* Lloyd's algorithm on N(0,1): alternate the nearest-neighbour cells
 * (midpoints) and the centroid condition (conditional means), to a fixed
 * point.  levels[2^bits], ascending. */
void pkvo_tq_lloyd_max(int bits, double* levels)
{
    int L = 1 << bits;
    for (int k = 0; k < L; ++k)
        levels[k] = -3.0 + 6.0 * (k + 0.5) / L;
    for (int it = 0; it < 100000; ++it) {
        double change = 0.0;
        double prev_t = -INFINITY;
        double nl[16];
        for (int k = 0; k < L; ++k) {
            double t = k + 1 < L ? 0.5 * (levels[k] + levels[k + 1]) : INFINITY;
            double pa = isinf(prev_t) ? 0.0 : std_normal_pdf(prev_t);
            double pb = isinf(t) ? 0.0 : std_normal_pdf(t);
            double mass = std_normal_cdf(t) - std_normal_cdf(prev_t);
            nl[k] = (pa - pb) / mass;
            prev_t = t;
        }
        for (int k = 0; k < L; ++k) {
            double d = fabs(nl[k] - levels[k]);
            if (d > change) change = d;
            levels[k] = nl[k];
        }
        if (change < 1e-15)
            break;
    }
}

/* E4M3 codes of the 2^(bits-1) positive magnitudes, ascending. */
void pkvo_tq_codebook(int bits, uint8_t* mag_codes)
{
    double lv[16];
    pkvo_tq_lloyd_max(bits, lv);
    int L = 1 << bits, M = L / 2;
    for (int j = 0; j < M; ++j)
        mag_codes[j] = pkvo_e4m3_from_f64(lv[M + j]);
}

static int tq_bits(int dtype) { return dtype - O_TQ2 + 2; }
static int is_tq(int dtype) { return dtype >= O_TQ2 && dtype <= O_TQ4; }

/* bytes of one cache block of B tokens x H heads x D elements: one region
 * per head, B code rows of D * bits / 8 bytes followed by D / 16 scale rows
 * (one per group) of B bytes */
static uint64_t tq_region_bytes(int bits, uint32_t B, uint32_t D)
{
    return (uint64_t)B * D * bits / 8 + (uint64_t)B * D / 16;
}

uint64_t pkvo_tq_block_bytes(int bits, uint32_t B, uint32_t H, uint32_t D)
{
    return H * tq_region_bytes(bits, B, D);
}

/* Decoded element (blk, t, h, d) of a TQ cache. */
static double tq_elem(const void* cache, int bits, uint32_t B, uint32_t H, uint32_t D,
                      const double* mags, uint64_t blk, uint32_t t, uint32_t h, uint32_t d)
{
    const uint8_t* base = (const uint8_t*)cache + blk * pkvo_tq_block_bytes(bits, B, H, D) +
                          h * tq_region_bytes(bits, B, D);
    const uint8_t* row = base + (uint64_t)t * D * bits / 8;
    uint32_t q = d / 16, i = d % 16;
    const uint8_t* grp = row + (uint64_t)q * 2 * bits;
    uint32_t bit = (uint32_t)bits * i, code = 0;
    for (int k = 0; k < bits; ++k, ++bit)
        code |= (uint32_t)((grp[bit / 8] >> (bit % 8)) & 1u) << k;
    uint8_t sc = base[(uint64_t)B * D * bits / 8 + (uint64_t)q * B + t];
    double mag = mags[code & ((1u << (bits - 1)) - 1)];
    double v = (code >> (bits - 1)) ? -mag : mag;
    return pkvo_f64_from_e4m3(sc) * v;
}

/* The E4M3 magnitudes of a TQ format and the midpoints between neighbours
 * (exact in FP64: sums of two E4M3 values). */
static int tq_levels(int bits, double* mags, double* thr)
{
    const int M = 1 << (bits - 1);
    uint8_t mc[8];
    pkvo_tq_codebook(bits, mc);
    for (int j = 0; j < M; ++j)
        mags[j] = pkvo_f64_from_e4m3(mc[j]);
    for (int j = 0; j + 1 < M; ++j)
        thr[j] = 0.5 * (mags[j] + mags[j + 1]);
    return M;
}

/* One group of 16 elements, by the definition, in FP64:
 *   rms   = sqrt(sum x_i^2 / 16);
 *   u_i   = x_i / rms;  code_i = sign(u_i) << (b-1) | the index of the
 *           nearest magnitude of |u_i| (on an exact midpoint the smaller
 *           one: the count of midpoints that |u_i| strictly exceeds; -0 and
 *           +0 are positive);
 *   ratio = |x| / |chosen levels| (the norm correction), scale = E4M3 of it
 *           (one rounding, nearest even, saturating at 448).
 * An all-zero group has codes 0 and scale 0.  u, the sum of squares and
 * the ratio are returned for callers that need to know how close a
 * decision was. */
static void tq_encode_group(const double* x, int bits, const double* mags, const double* thr,
                            uint32_t* codes, uint8_t* scale, double* u_out, double* ss_out,
                            double* ratio_out)
{
    const int M = 1 << (bits - 1);
    double ss = 0.0;
    for (int i = 0; i < 16; ++i)
        ss += x[i] * x[i];
    *ss_out = ss;
    *ratio_out = 0.0;
    *scale = 0;
    if (!(ss > 0.0)) {
        for (int i = 0; i < 16; ++i) {
            codes[i] = 0;
            u_out[i] = 0.0;
        }
        return;
    }
    const double rms = sqrt(ss / 16.0);
    double cn = 0.0;          /* exact: at most 16 squares of E4M3 values */
    for (int i = 0; i < 16; ++i) {
        const double u = x[i] / rms;
        const double au = fabs(u);
        uint32_t m = 0;
        while ((int)m + 1 < M && au > thr[m])
            ++m;
        codes[i] = (u < 0.0 ? 1u : 0u) << (bits - 1) | m;
        cn += mags[m] * mags[m];
        u_out[i] = u;
    }
    *ratio_out = sqrt(ss) / sqrt(cn);
    *scale = pkvo_e4m3_from_f64(*ratio_out);
}

/* Writes V rows of the tokens with valid slots into a TQ cache (each group
 * coded by tq_encode_group). */
void pkvo_cache_write_v_tq(const void* v, int in_dtype, uint64_t in_token_stride,
                           const int64_t* slots, uint32_t num_tokens, uint32_t num_kv_heads,
                           uint32_t head_dim_v, uint32_t block_size, uint32_t num_blocks,
                           void* v_cache, int bits)
{
    const uint32_t H = num_kv_heads, D = head_dim_v, B = block_size;
    double mags[8], thr[8];
    tq_levels(bits, mags, thr);
    uint64_t blk_bytes = pkvo_tq_block_bytes(bits, B, H, D);
    uint64_t num_slots = (uint64_t)num_blocks * B;
    for (uint64_t tok = 0; tok < num_tokens; ++tok) {
        int64_t slot = slots[tok];
        if (slot < 0 || (uint64_t)slot >= num_slots)
            continue;
        uint64_t blk = (uint64_t)slot / B;
        uint32_t t = (uint32_t)((uint64_t)slot % B);
        for (uint32_t h = 0; h < H; ++h) {
            uint8_t* base = (uint8_t*)v_cache + blk * blk_bytes + h * tq_region_bytes(bits, B, D);
            uint8_t* row = base + (uint64_t)t * D * bits / 8;
            for (uint32_t q = 0; q < D / 16; ++q) {
                double x[16], u[16], ss, ratio;
                for (int i = 0; i < 16; ++i)
                    x[i] = load_elem(v, in_dtype, tok * in_token_stride + (uint64_t)h * D + q * 16 + i);
                uint32_t codes[16];
                uint8_t scale;
                tq_encode_group(x, bits, mags, thr, codes, &scale, u, &ss, &ratio);
                uint8_t* grp = row + (uint64_t)q * 2 * bits;
                memset(grp, 0, 2 * (size_t)bits);
                for (int i = 0; i < 16; ++i)
                    for (int k = 0; k < bits; ++k) {
                        uint32_t bit = (uint32_t)bits * i + k;
                        grp[bit / 8] |= (uint8_t)(((codes[i] >> k) & 1u) << (bit % 8));
                    }
                base[(uint64_t)B * D * bits / 8 + (uint64_t)q * B + t] = scale;
            }
        }
    }
}

/* The encoder's inputs to its decisions for rows v [T, H, D] (token stride
 * in_token_stride): u [T, H, D] = x / rms of each element's group, and per
 * group [T, H, D/16] the sum of squares and the ratio of norms, all FP64 as
 * tq_encode_group takes them, plus the codes [T, H, D] and scale bytes it
 * chooses.  For tests that must tell a decision taken close to a rounding
 * boundary from a wrong one. */
void pkvo_tq_encode_diag(const void* v, int in_dtype, uint64_t in_token_stride,
                         uint32_t num_tokens, uint32_t num_kv_heads, uint32_t head_dim_v,
                         int bits, double* u_out, double* ss_out, double* ratio_out,
                         uint8_t* codes_out, uint8_t* scales_out)
{
    const uint32_t H = num_kv_heads, D = head_dim_v, NG = D / 16;
    double mags[8], thr[8];
    tq_levels(bits, mags, thr);
    for (uint64_t tok = 0; tok < num_tokens; ++tok)
        for (uint32_t h = 0; h < H; ++h)
            for (uint32_t q = 0; q < NG; ++q) {
                double x[16];
                for (int i = 0; i < 16; ++i)
                    x[i] = load_elem(v, in_dtype, tok * in_token_stride + (uint64_t)h * D + q * 16 + i);
                const uint64_t g = (tok * H + h) * NG + q;
                uint32_t codes[16];
                tq_encode_group(x, bits, mags, thr, codes, &scales_out[g], &u_out[g * 16],
                                &ss_out[g], &ratio_out[g]);
                for (int i = 0; i < 16; ++i)
                    codes_out[g * 16 + i] = (uint8_t)codes[i];
            }
}

/* ------------------------------------------------------------------ */
/* (4) V reshape-and-cache                                             */
/* ------------------------------------------------------------------ */

/* Same dtype in and out: v_cache[slot, h, :] = v[t, h, :] byte for byte
 * (p1 reshape_and_cache_flash_v_only: the V-only write that leaves the K side
 * of the cache to the fused K kernel).  E4M3 cache: each element is stored as
 * the saturating E4M3 cast of fl32(v / v_scale), the same store as an FP8 K
 * cache (p1 reshape_and_cache_fp8 writes K and V to FP8 with k_scale and
 * v_scale; p2 module invariants fix the store as value / scale).  Padding
 * slots (negative or past the pool) are skipped. */
void pkvo_cache_write_v(const void* v, int in_dtype, uint64_t in_token_stride,
                        const int64_t* slots, uint32_t num_tokens, uint32_t num_kv_heads,
                        uint32_t head_dim_v, uint32_t block_size, uint32_t num_blocks,
                        void* v_cache, int cache_dtype, float v_scale)
{
    if (is_tq(cache_dtype)) {
        pkvo_cache_write_v_tq(v, in_dtype, in_token_stride, slots, num_tokens, num_kv_heads,
                              head_dim_v, block_size, num_blocks, v_cache, tq_bits(cache_dtype));
        return;
    }
    size_t es = elem_size(in_dtype);
    uint64_t row_elems = (uint64_t)num_kv_heads * head_dim_v;
    uint64_t num_slots = (uint64_t)num_blocks * block_size;
    for (uint64_t t = 0; t < num_tokens; ++t) {
        int64_t slot = slots[t];
        if (slot < 0 || (uint64_t)slot >= num_slots)
            continue;
        if (cache_dtype == in_dtype) {
            memcpy((char*)v_cache + (uint64_t)slot * row_elems * es,
                   (const char*)v + t * in_token_stride * es, row_elems * es);
            continue;
        }
        for (uint64_t e = 0; e < row_elems; ++e) {
            double x = load_elem(v, in_dtype, t * in_token_stride + e);
            float z = (float)(x / (double)v_scale);               /* fl32(v/v_scale) */
            ((uint8_t*)v_cache)[(uint64_t)slot * row_elems + e] = pkvo_e4m3_from_f64((double)z);
        }
    }
}

/* ------------------------------------------------------------------ */
/* (5) Paged decode attention                                          */
/* ------------------------------------------------------------------ */

typedef struct {
    const void* q; int q_dtype; uint64_t q_seq_stride;
    const void* k_cache; int k_dtype; float k_scale;
    const void* v_cache; int v_dtype; float v_scale;
    const int32_t* block_tables; uint32_t max_blocks_per_seq;
    const int32_t* seq_lens; uint32_t num_blocks;
    uint32_t Hq, Hkv, Dqk, Dv, B; float scale;
    uint32_t window; const float* sinks;
    int q_rope; float q_rope_theta; uint32_t q_rope_offset, q_rope_dim;
    const float* gate; float* out;
    double tq_mags[8];          /* decoded codebook magnitudes of a TQ V cache */
    double spv_tau;             /* sparse-V threshold (with spv_bound) */
    float* spv_bound;           /* NULL: exact decode; else the sparse-V bound rows */
} decode_ctx;

/* Dequantised cache element: BF16 and FP32 exactly, E4M3 exactly times its
 * per-tensor scale (p2 module invariants: the decode multiplies by k_scale). */
static double cache_elem(const void* base, int dtype, float scl, uint64_t idx)
{
    double x = load_elem(base, dtype, idx);
    return dtype == O_E4M3 ? x * (double)scl : x;
}

static void tq_fill_mags(decode_ctx* c)
{
    if (!is_tq(c->v_dtype))
        return;
    int bits = tq_bits(c->v_dtype);
    uint8_t mc[8];
    pkvo_tq_codebook(bits, mc);
    for (int j = 0; j < (1 << (bits - 1)); ++j)
        c->tq_mags[j] = pkvo_f64_from_e4m3(mc[j]);
}

/* Scores of one query vector q (kv head g) of sequence s over the positions
 * [lo, end): sc[t] = scale * <q, k_t> for the attended t (ok[t] = 1);
 * tokens outside the window, of an unmapped block or past the table are
 * excluded (ok[t] = 0).  Returns the largest score (-inf if none). */
static double score_pass(const decode_ctx* c, uint32_t s, uint32_t g, int32_t end, int32_t lo,
                         const double* q, double* sc, unsigned char* ok)
{
    double m = -INFINITY;
    for (int32_t t = 0; t < end; ++t) {
        uint32_t b = (uint32_t)t / c->B;
        ok[t] = 0;
        if (t < lo)
            continue;                        /* outside the window */
        if (b >= c->max_blocks_per_seq)
            continue;
        int32_t blk = c->block_tables[(uint64_t)s * c->max_blocks_per_seq + b];
        if (blk < 0 || (uint32_t)blk >= c->num_blocks)
            continue;                        /* unmapped block: token excluded */
        uint64_t row = (uint64_t)blk * c->B + (uint32_t)t % c->B;
        uint64_t koff = (row * c->Hkv + g) * c->Dqk;
        double dot = 0.0;
        for (uint32_t j = 0; j < c->Dqk; ++j)
            dot += q[j] * cache_elem(c->k_cache, c->k_dtype, c->k_scale, koff + j);
        sc[t] = (double)c->scale * dot;
        ok[t] = 1;
        if (sc[t] > m) m = sc[t];
    }
    return m;
}

/* Element d of the V row of position t (kv head g) of sequence s, whose
 * block is mapped. */
static double v_value(const decode_ctx* c, uint32_t s, int32_t t, uint32_t g, uint32_t d)
{
    uint32_t b = (uint32_t)t / c->B;
    int32_t blk = c->block_tables[(uint64_t)s * c->max_blocks_per_seq + b];
    if (is_tq(c->v_dtype))
        return tq_elem(c->v_cache, tq_bits(c->v_dtype), c->B, c->Hkv, c->Dv, c->tq_mags,
                       (uint64_t)blk, (uint32_t)t % c->B, g, d);
    uint64_t row = (uint64_t)blk * c->B + (uint32_t)t % c->B;
    return cache_elem(c->v_cache, c->v_dtype, c->v_scale, (row * c->Hkv + g) * c->Dv + d);
}

/* Attention of one query vector q (kv head g, query head h) of sequence s
 * over the positions [lo, end) of its cache, written to dst[Dv]:
 *   softmax over s_t = scale * <q, k_t> (t attended), times v_t, summed.
 * Tokens of an unmapped block or past the table are excluded; with no
 * attended token the row is zero. */
static void attend(const decode_ctx* c, uint32_t s, uint32_t g, uint32_t h, int32_t end,
                   int32_t lo, const double* q, double* o, const float* gate_row, float* dst)
{
    for (uint32_t d = 0; d < c->Dv; ++d)
        o[d] = 0.0;
    if (end <= 0) {
        for (uint32_t d = 0; d < c->Dv; ++d)
            dst[d] = 0.0f;
        return;
    }
    /* pass 1: scores and their maximum */
    double* sc = (double*)malloc(sizeof(double) * (size_t)end);
    unsigned char* ok = (unsigned char*)malloc((size_t)end);
    const double m = score_pass(c, s, g, end, lo, q, sc, ok);
    /* pass 2: softmax weights and the weighted sum of V rows */
    double l = 0.0;
    for (int32_t t = 0; t < end; ++t) {
        if (!ok[t]) continue;
        double pt = exp(sc[t] - m);
        l += pt;
        for (uint32_t d = 0; d < c->Dv; ++d)
            o[d] += pt * v_value(c, s, t, g, d);
    }
    /* Attention sink (p1 mla_paged_decode_fp8 takes a `sinks` pointer,
     * semantics unstated; our reading): one logit per query head, in the
     * units of the scaled scores, that joins the softmax normalisation
     * and carries no value, i.e. the denominator gains exp(sink - m).
     * With no attended token the output stays zero. */
    if (c->sinks && l > 0.0) {
        double sk = (double)c->sinks[h];
        double mm = sk > m ? sk : m;
        double f = exp(m - mm);
        l = l * f + exp(sk - mm);
        for (uint32_t d = 0; d < c->Dv; ++d)
            o[d] *= f;
    }
    for (uint32_t d = 0; d < c->Dv; ++d) {
        double val = l > 0.0 ? o[d] / l : 0.0;
        /* optional elementwise output gate (p3 module doc: SDPA + gate) */
        if (gate_row)
            val *= (double)gate_row[d];
        dst[d] = (float)val;
    }
    free(sc);
    free(ok);
}

/* Sparse-V skip (p1 Turbo-V decode docs: the V loads and dequantisation are
 * sparse on both the batched and the remainder paths; p2
 * paged_decode_attn_fp8k_turbo3v: a position's V load and dequantisation
 * are skipped when its attention weight is at most
 * TQ_PLUS_SPARSE_V_THRESHOLD, a value the pages do not give).  Reading taken: the attention weight of position t is its softmax
 * weight w_t = exp(s_t) / Z with Z the exact decode's denominator (sinks
 * included); a skipped position leaves the sum over V and stays in Z (its
 * score is computed either way).  With threshold tau, for query head h:
 *   dst[d]  = sum over attended t with w_t >  tau of w_t v_t[d]   (x gate[d])
 *   bdst[d] = sum over attended t with w_t <= tau of w_t |v_t[d]| (x |gate[d]|)
 * so that the exact output differs from dst by at most bdst, and so does
 * the result of leaving out any subset of the positions with w_t <= tau.
 * tau = 0 gives the exact decode (every weight is positive). */
static void attend_sparse_v(const decode_ctx* c, double tau, uint32_t s, uint32_t g, uint32_t h,
                            int32_t end, int32_t lo, const double* q, double* o, double* bnd,
                            const float* gate_row, float* dst, float* bdst)
{
    for (uint32_t d = 0; d < c->Dv; ++d)
        o[d] = bnd[d] = 0.0;
    if (end > 0) {
        double* sc = (double*)malloc(sizeof(double) * (size_t)end);
        unsigned char* ok = (unsigned char*)malloc((size_t)end);
        const double m = score_pass(c, s, g, end, lo, q, sc, ok);
        int any = 0;
        for (int32_t t = 0; t < end; ++t)
            any |= ok[t];
        if (any) {
            /* Z relative to the larger of the top score and the sink */
            double mm = m;
            if (c->sinks && (double)c->sinks[h] > mm)
                mm = (double)c->sinks[h];
            double z = c->sinks ? exp((double)c->sinks[h] - mm) : 0.0;
            for (int32_t t = 0; t < end; ++t)
                if (ok[t])
                    z += exp(sc[t] - mm);
            for (int32_t t = 0; t < end; ++t) {
                if (!ok[t]) continue;
                const double w = exp(sc[t] - mm) / z;
                for (uint32_t d = 0; d < c->Dv; ++d) {
                    const double v = v_value(c, s, t, g, d);
                    if (w > tau)
                        o[d] += w * v;
                    else
                        bnd[d] += w * fabs(v);
                }
            }
        }
        free(sc);
        free(ok);
    }
    for (uint32_t d = 0; d < c->Dv; ++d) {
        const double gd = gate_row ? (double)gate_row[d] : 1.0;
        dst[d] = (float)(o[d] * gd);
        bdst[d] = (float)(bnd[d] * fabs(gd));
    }
}

/* Sliding window of W tokens (p1/p3 decode launchers take a sliding_window
 * argument, semantics unstated; our reading): a query at position p sees the
 * W most recent positions, [p + 1 - W, p + 1); W = 0 means no window. */
static int32_t window_start(uint32_t window, int32_t end)
{
    return (window > 0 && (int64_t)end > (int64_t)window) ? end - (int32_t)window : 0;
}

static void decode_range(void* p, uint64_t u0, uint64_t u1)
{
    const decode_ctx* c = (const decode_ctx*)p;
    const uint32_t G = c->Hq / c->Hkv;
    double* q = (double*)malloc(sizeof(double) * c->Dqk);
    double* o = (double*)malloc(sizeof(double) * c->Dv);
    double* bnd = (double*)malloc(sizeof(double) * c->Dv);
    for (uint64_t u = u0; u < u1; ++u) {
        uint32_t s = (uint32_t)(u / c->Hq), h = (uint32_t)(u % c->Hq);
        uint32_t g = h / G;                      /* GQA: contiguous groups */
        uint64_t orow = ((uint64_t)s * c->Hq + h) * c->Dv;
        int32_t n = c->seq_lens[s];              /* the query is the token at n - 1 */
        uint64_t qoff = (uint64_t)s * c->q_seq_stride + (uint64_t)h * c->Dqk;
        for (uint32_t j = 0; j < c->Dqk; ++j)
            q[j] = n > 0 ? load_elem(c->q, c->q_dtype, qoff + j) : 0.0;
        if (n > 0 && c->q_rope && c->q_rope_dim > 0) {
            int32_t pos3[3] = {n - 1, n - 1, n - 1};
            rope_rotate(q, c->q_rope_offset, c->q_rope_dim, c->q_rope_theta, pos3);
        }
        if (c->spv_bound)
            attend_sparse_v(c, c->spv_tau, s, g, h, n, window_start(c->window, n), q, o, bnd,
                            c->gate ? c->gate + orow : NULL, c->out + orow, c->spv_bound + orow);
        else
            attend(c, s, g, h, n, window_start(c->window, n), q, o,
                   c->gate ? c->gate + orow : NULL, c->out + orow);
    }
    free(q);
    free(o);
    free(bnd);
}

void pkvo_paged_decode(const void* q, int q_dtype, uint64_t q_seq_stride,
                       const void* k_cache, int k_dtype, float k_scale,
                       const void* v_cache, int v_dtype, float v_scale,
                       const int32_t* block_tables, uint32_t max_blocks_per_seq,
                       const int32_t* seq_lens, uint32_t num_seqs, uint32_t num_blocks,
                       uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim_qk,
                       uint32_t head_dim_v, uint32_t block_size, float scale,
                       uint32_t sliding_window, const float* sinks,
                       int q_rope, float q_rope_theta, uint32_t q_rope_offset,
                       uint32_t q_rope_dim, const float* gate, float* out, int nthreads)
{
    decode_ctx c = {q, q_dtype, q_seq_stride, k_cache, k_dtype, k_scale, v_cache, v_dtype,
                    v_scale, block_tables, max_blocks_per_seq, seq_lens, num_blocks,
                    num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, block_size, scale,
                    sliding_window, sinks, q_rope, q_rope_theta, q_rope_offset, q_rope_dim, gate, out,
                    {0}, 0.0, NULL};
    tq_fill_mags(&c);
    parallel_for((uint64_t)num_seqs * num_q_heads, nthreads, decode_range, &c);
}

/* The decode with the sparse-V skip at threshold tau >= 0 (attend_sparse_v):
 * out as for pkvo_paged_decode but summing only the positions whose weight
 * exceeds tau, bound[S, Hq, Dv] the weighted |V| of the others. */
void pkvo_paged_decode_sparse_v(const void* q, int q_dtype, uint64_t q_seq_stride,
                                const void* k_cache, int k_dtype, float k_scale,
                                const void* v_cache, int v_dtype, float v_scale,
                                const int32_t* block_tables, uint32_t max_blocks_per_seq,
                                const int32_t* seq_lens, uint32_t num_seqs, uint32_t num_blocks,
                                uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim_qk,
                                uint32_t head_dim_v, uint32_t block_size, float scale,
                                uint32_t sliding_window, const float* sinks, const float* gate,
                                double tau, float* out, float* bound, int nthreads)
{
    decode_ctx c = {q, q_dtype, q_seq_stride, k_cache, k_dtype, k_scale, v_cache, v_dtype,
                    v_scale, block_tables, max_blocks_per_seq, seq_lens, num_blocks,
                    num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, block_size, scale,
                    sliding_window, sinks, 0, 0.0f, 0, 0, gate, out, {0}, tau, bound};
    tq_fill_mags(&c);
    parallel_for((uint64_t)num_seqs * num_q_heads, nthreads, decode_range, &c);
}

/* ------------------------------------------------------------------ */
/* (6) Paged prefill attention (N new tokens per sequence)             */
/* ------------------------------------------------------------------ */

typedef struct {
    decode_ctx d;                 /* cache, tables, heads, scale, window, sinks */
    uint64_t q_token_stride;
    const int32_t* cu_q;          /* [S + 1] */
    uint32_t num_seqs;
} prefill_ctx;

/* Page 1 names batched prefill variants (N tokens) of the paged kernels and
 * gives no more; the reading taken is causal attention over the same cache:
 * the q_len = cu_q[s+1] - cu_q[s] queries of sequence s are its last q_len
 * tokens (their K/V rows already written), query i at position
 * p = seq_len - q_len + i, and it attends to positions [lo, p] (lo from the
 * sliding window, as for decode).  A query with p < 0 gives a zero row. */
static void prefill_range(void* pp, uint64_t u0, uint64_t u1)
{
    const prefill_ctx* c = (const prefill_ctx*)pp;
    const decode_ctx* d = &c->d;
    const uint32_t G = d->Hq / d->Hkv;
    double* q = (double*)malloc(sizeof(double) * d->Dqk);
    double* o = (double*)malloc(sizeof(double) * d->Dv);
    for (uint64_t u = u0; u < u1; ++u) {
        uint64_t t = u / d->Hq;
        uint32_t h = (uint32_t)(u % d->Hq);
        uint32_t s = 0;                          /* sequence holding query token t */
        while (s + 1 < c->num_seqs && (uint64_t)c->cu_q[s + 1] <= t)
            ++s;
        int32_t qlen = c->cu_q[s + 1] - c->cu_q[s];
        int32_t i = (int32_t)(t - (uint64_t)c->cu_q[s]);
        int32_t end = d->seq_lens[s] - qlen + i + 1;   /* attends to [lo, end) */
        uint64_t qoff = t * c->q_token_stride + (uint64_t)h * d->Dqk;
        for (uint32_t j = 0; j < d->Dqk; ++j)
            q[j] = load_elem(d->q, d->q_dtype, qoff + j);
        attend(d, s, h / G, h, end, window_start(d->window, end), q, o, NULL,
               d->out + (t * d->Hq + h) * d->Dv);
    }
    free(q);
    free(o);
}

void pkvo_paged_prefill(const void* q, int q_dtype, uint64_t q_token_stride, const int32_t* cu_q,
                        const void* k_cache, int k_dtype, float k_scale,
                        const void* v_cache, int v_dtype, float v_scale,
                        const int32_t* block_tables, uint32_t max_blocks_per_seq,
                        const int32_t* seq_lens, uint32_t num_seqs, uint32_t num_blocks,
                        uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim_qk,
                        uint32_t head_dim_v, uint32_t block_size, float scale,
                        uint32_t sliding_window, const float* sinks, float* out, int nthreads)
{
    prefill_ctx c;
    memset(&c, 0, sizeof c);
    decode_ctx d = {q, q_dtype, 0, k_cache, k_dtype, k_scale, v_cache, v_dtype, v_scale,
                    block_tables, max_blocks_per_seq, seq_lens, num_blocks, num_q_heads,
                    num_kv_heads, head_dim_qk, head_dim_v, block_size, scale, sliding_window,
                    sinks, 0, 0.0f, 0, 0, NULL, out, {0}, 0.0, NULL};
    tq_fill_mags(&d);
    c.d = d;
    c.q_token_stride = q_token_stride;
    c.cu_q = cu_q;
    c.num_seqs = num_seqs;
    uint64_t total = num_seqs ? (uint64_t)cu_q[num_seqs] : 0;
    parallel_for(total * num_q_heads, nthreads, prefill_range, &c);
}

/* ------------------------------------------------------------------ */
/* (7) MLA cache assembly                                              */
/* ------------------------------------------------------------------ */

/* Page 1, mla_cache_assemble: [kv_latent | k_rope] becomes the K row and
 * [kv_latent | zeros] the V row of the single-head MLA cache.  Batched here
 * over tokens through a slot mapping (padding slots skipped); a cache row
 * longer than kv_lora + rope is zero past the copied parts.  Byte copies in
 * the input dtype. */
void pkvo_mla_cache_assemble(const void* kv_latent, const void* k_rope, int dtype,
                             uint64_t latent_stride, uint64_t rope_stride,
                             const int64_t* slots, uint32_t num_tokens, uint32_t kv_lora,
                             uint32_t rope, uint32_t cache_dim, uint32_t block_size,
                             uint32_t num_blocks, void* k_cache, void* v_cache)
{
    size_t es = elem_size(dtype);
    uint64_t num_slots = (uint64_t)num_blocks * block_size;
    for (uint64_t t = 0; t < num_tokens; ++t) {
        int64_t slot = slots[t];
        if (slot < 0 || (uint64_t)slot >= num_slots)
            continue;
        char* krow = (char*)k_cache + (uint64_t)slot * cache_dim * es;
        char* vrow = (char*)v_cache + (uint64_t)slot * cache_dim * es;
        memset(krow, 0, cache_dim * es);
        memset(vrow, 0, cache_dim * es);
        memcpy(krow, (const char*)kv_latent + t * latent_stride * es, (size_t)kv_lora * es);
        memcpy(krow + (size_t)kv_lora * es, (const char*)k_rope + t * rope_stride * es,
               (size_t)rope * es);
        memcpy(vrow, (const char*)kv_latent + t * latent_stride * es, (size_t)kv_lora * es);
    }
}

/* ------------------------------------------------------------------ */
/* Array forms of the converters (for the pin tests).                  */
/* ------------------------------------------------------------------ */

void pkvo_bf16_from_f32_array(const float* x, uint16_t* out, uint64_t n)
{
    for (uint64_t i = 0; i < n; ++i)
        out[i] = pkvo_bf16_from_f32(x[i]);
}

void pkvo_e4m3_from_f32_array(const float* x, uint8_t* out, uint64_t n)
{
    for (uint64_t i = 0; i < n; ++i)
        out[i] = pkvo_e4m3_from_f64((double)x[i]);
}

void pkvo_f64_from_e4m3_array(const uint8_t* c, double* out, uint64_t n)
{
    for (uint64_t i = 0; i < n; ++i)
        out[i] = pkvo_f64_from_e4m3(c[i]);
}

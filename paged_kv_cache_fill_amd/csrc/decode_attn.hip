// decode_attn.hip -- pkv_paged_decode_attn: one-query-token paged decode
// attention with GQA, split-K over the token range and a log-sum-exp merge
// (page 1, kv_cache.rs, paged_decode_attn_fp8 and its BF16 sibling: Q, K/V
// pools, block_tables i32, seq_lens i32, num_q_heads / num_kv_heads,
// inv_sqrt_d, k_scale, v_scale; the sliding_window of its decode launchers
// and the sinks of mla_paged_decode_fp8; page 3, mla_cuda.rs: RoPE on q
// then SDPA + gate).  The attended range of a sequence of n tokens is
// [n - W, n) for a window of W tokens (W = 0: all of it); a sink adds
// exp(sink) to the softmax denominator of its query head.
//
// Work decomposition.  A work-group handles a piece of work for a group of
// kv heads, one wavefront per kv head: either one (sequence, split) pair, a
// split being `chunk_blocks` consecutive cache blocks of the sequence, or
// (balanced plan) an equal range of the batch's attended blocks taken in
// sequence order, which may hold pieces of several sequences.  The work-group's waves read
// neighbouring rows of the same pool blocks, so together they stream whole
// blocks ([block_size, Hkv, D] is contiguous).  Every query head of a kv
// head's GQA group is served by the same wave from the same K/V registers:
// K and V are read from HBM exactly once.
//
// BF16 / FP8-K caches (MFMA path).  Per 16-token cache block a wave computes
//   S^T[t, g] = K[t, :] . q[g, :]    v_mfma_f32_16x16x32_bf16  (M=t, N=g)
//   O[g, d]  += P[g, t] V[t, d]      v_mfma_f32_16x16x16_bf16  (M=g, N=d)
// The S^T accumulator layout (lane = t-group x g) is exactly the A-operand
// layout of the PV product, so softmax weights never leave their lanes.  The
// head dimension is permuted consistently on q and K so that every lane
// loads 16 contiguous bytes; V's columns are permuted so that a lane's 16-byte
// load feeds all eight N-tiles.  P is split into hi + lo BF16 parts (two PV
// MFMAs), which keeps the weights to ~16 bits; BF16 q x BF16 (or E4M3) K
// products are exact in FP32.  E4M3 V codes are widened exactly to BF16 for
// the PV product and v_scale is applied with the final normalisation.
// Online softmax runs in the log2 domain.
//
// TQ V caches may skip V per block (page 2, paged_decode_attn_fp8k_turbo3v:
// the sparse-V skip at a caller's threshold): separate instantiations score
// a block first and load, decode and multiply its V only when some weight
// exceeds the threshold.
//
// FP32 caches (VALU path).  Four tokens per wave step (16 lanes per token
// row, 16-byte loads), one online-softmax stream per row, merged at the end.
#include <mutex>
#include <type_traits>

#include "attn_common.h"

namespace pkv {


// Launch shape of the MFMA path.
constexpr uint32_t kKvPerGroup = 2;     // kv heads (waves) per work-group, at most
constexpr int kPrefetch = 1;            // cache blocks loaded ahead of the one in use
// Sparse-V loop: K blocks loaded ahead.  On the 256-sequence 3-bit TQ V
// workload with one heavy key every 64 positions, 1, 2 and 3 blocks gave the
// same call time (0.386-0.403 ms, batch-averaged).
constexpr int kPrefetchSpv = 1;
constexpr bool kKDirect = false;        // K loaded straight into the operand layout
constexpr uint64_t kTargetGroups = 768; // (sequence, split, kv group) work-groups wanted
// FP32 path: (sequence, kv head, split) waves wanted -- about one per CU.
// Long splits stream faster here than many short ones: on the 64-head,
// 4096-token MLA-style workload the call took 58.9 / 60.0 / 61.4 / 63.8 us
// with 1024- / 512- / 256- / 96-token splits (256 to 2752 waves).
constexpr uint64_t kTargetWavesF32 = 256;
constexpr uint32_t kMinChunk = 4;       // blocks per split, automatic choice: at least
constexpr int kBtRegs = 2;              // table entries held per lane (split mode)
constexpr uint32_t kMaxChunk = 64 * kBtRegs;  // ... so at most this many blocks per split
constexpr int kBtRegsBal = 8;           // table entries held per lane (balanced mode)
constexpr uint32_t kMaxRange = 64 * kBtRegsBal;  // ... so at most this many blocks per range

struct DecodeArgs {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* bt;
    const int32_t* seq_lens;
    const float* gate;
    const float* sinks;     // [Hq] logits, or NULL
    float* out;
    float* part_o;          // [rows][Hq][Dv]; rows = S * max_splits, or ranges + S
    float* part_ml;         // [rows][Hq][2]  (max in log2 units, sum)
    uint64_t q_stride;      // elements between sequences
    uint32_t M;             // max_blocks_per_seq
    uint32_t num_blocks;
    uint32_t Hq, Hkv, G;
    uint32_t chunk_blocks;
    uint32_t max_splits;
    uint32_t S;             // sequences
    uint32_t ranges;        // balanced mode: block ranges per kv group (0 = split mode)
    uint32_t* cu;           // balanced mode, ranges > 1: [S + 1] attended blocks before s
    float qk_scale;         // scale * log2(e) (* k_scale for E4M3 K)
    float out_scale;        // output factor: v_scale (E4M3 V), 2^-15 for FP16 weights
    uint32_t window;        // sliding window in tokens, 0 = none
    // TurboQuant-style V: the FP16 level table as byte-lookup words (low
    // bytes of entries 0-3, 4-7, high bytes of 0-3, 4-7), and block bytes
    uint32_t tq_f16[4];
    uint32_t v_blk_bytes;
    // query rotation (FP32 path); inverse frequencies fl32(theta^(-2i/dim))
    // from the host, as for the K write
    uint32_t q_rope;
    float q_rope_theta;
    uint32_t q_rope_offset;
    uint32_t q_rope_dim;
    float q_invf[128];
    float spv_thr;          // sparse-V skip (TQ V): threshold x 2^15, the units of the FP16 weights
};

// ------------------------------------------------------------------ helpers

// Cache blocks of a sequence of n tokens that the table can address; tokens
// whose block index is past the table are excluded.
__device__ __forceinline__ uint32_t seq_blocks(int32_t n, uint32_t M)
{
    const uint32_t nb = n > 0 ? ((uint32_t)n + kBS - 1) / kBS : 0;
    return nb < M ? nb : M;
}

// Attended tokens [lo, n) of a sequence and the cache blocks [blo, nblk)
// that hold them; split i covers blocks blo + i * chunk_blocks onwards.
struct SeqRange {
    int32_t n, lo;
    uint32_t blo, nblk, nsplit;
};
__device__ __forceinline__ SeqRange seq_range(const DecodeArgs& a, uint32_t s)
{
    SeqRange r;
    r.n = a.seq_lens[s];
    r.nblk = seq_blocks(r.n, a.M);
    r.lo = (a.window > 0 && r.n > (int32_t)a.window) ? r.n - (int32_t)a.window : 0;
    r.blo = (uint32_t)r.lo / kBS;
    r.nsplit = r.nblk > r.blo ? (r.nblk - r.blo + a.chunk_blocks - 1) / a.chunk_blocks : 0;
    return r;
}

// Attended blocks of sequence s.
__device__ __forceinline__ uint32_t att_blocks(const DecodeArgs& a, uint32_t s)
{
    const SeqRange r = seq_range(a, s);
    return r.nblk > r.blo ? r.nblk - r.blo : 0u;
}

// Sum over the wave (DPP within rows, then the gfx950 row swaps).
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v)
{
    v += dpp_u32<kDppXor1>(v);
    v += dpp_u32<kDppXor2>(v);
    v += dpp_u32<kDppHalfMirror>(v);
    v += dpp_u32<kDppMirror>(v);
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = a[0] + a[1];
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return b[0] + b[1];
}

// Balanced mode.  The attended blocks of all sequences, in sequence order,
// form one list of T blocks; range w of every kv group is the list's blocks
// [w C, (w + 1) C), C = ceil(T / ranges) <= kMaxRange (the host sizes `ranges` from
// an upper bound of T).  A sequence whose blocks lie in one range is finished
// by that range's work-group; otherwise each range writes a partial row for
// it at slot w + s (unique: every slot step is a range or a sequence start),
// and the merge combines slots first + s .. last + s.  Every wave recomputes
// T from seq_lens (at most 1024 sequences); work-group 0 also writes the
// prefix sums to the workspace for the merge.
__device__ __forceinline__ uint32_t range_blocks(uint32_t T, uint32_t ranges)
{
    const uint32_t c = T == 0 ? 1u : (T + ranges - 1) / ranges;
    return c < kMaxRange ? c : kMaxRange;
}

// Total attended blocks T of the batch (all lanes).
__device__ __forceinline__ uint32_t total_blocks(const DecodeArgs& a, int lane)
{
    uint32_t T = 0;
    for (uint32_t c = 0; c < a.S; c += 64) {
        const uint32_t s = c + (uint32_t)lane;
        T += wave_sum_u32(s < a.S ? att_blocks(a, s) : 0u);
    }
    return T;
}

// Writes the finished or partial result of one wave.
// o[nt][r]: row g = 4*(lane/16) + r of the GQA group, column d = DPL*(lane%16) + nt.
template <int DV>
__device__ __forceinline__ void emit_mfma(const DecodeArgs& a, uint32_t s, uint32_t kvh,
                                          bool direct, uint64_t prow_base, int lane,
                                          const f32x4 (&o)[DV / 16], float m, float l)
{
    constexpr int NT = DV / 16, DPL = DV / 16;
    const int kg = lane >> 4, n = lane & 15;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t g = 4 * kg + r;
        const float lg = __shfl(l, (int)g, 64);
        const float mg = __shfl(m, (int)g, 64);
        if (g >= a.G)
            continue;
        const uint32_t h = kvh * a.G + g;
        float vals[NT];
        if (direct) {
            const float inv = norm_factor(mg, lg, a.sinks, h, a.out_scale);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                vals[nt] = o[nt][r] * inv;
            const uint64_t base = ((uint64_t)s * a.Hq + h) * DV + (uint64_t)DPL * n;
            if (a.gate) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    vals[nt] *= a.gate[base + nt];
            }
#pragma unroll
            for (int nt = 0; nt < NT; nt += 4)
                *(f32x4*)(a.out + base + nt) = f32x4{vals[nt], vals[nt + 1], vals[nt + 2], vals[nt + 3]};
        } else {
            const uint64_t prow = prow_base + h;
            const uint64_t base = prow * DV + (uint64_t)DPL * n;
#pragma unroll
            for (int nt = 0; nt < NT; nt += 4)
                *(f32x4*)(a.part_o + base + nt) = f32x4{o[nt][r], o[nt + 1][r], o[nt + 2][r], o[nt + 3][r]};
            if (n == 0)
                *(f32x2*)(a.part_ml + prow * 2) = f32x2{mg, lg};
        }
    }
}

// ------------------------------------------------------------------ FP16 PV

// FP16 A operands of the PV product from the weights p[0..3] of the lane's
// tokens (scaled by 2^15 by the caller): a hi part, and the rounding error
// of it as a lo part, so that hi + lo keeps the weights to ~22 bits.
struct F16Weights {
    f16x4 hi, lo;
};
__device__ __forceinline__ F16Weights f16_weights(const float (&p)[4])
{
    F16Weights w;
    const uint32_t h01 = pack_f16(p[0], p[1]), h23 = pack_f16(p[2], p[3]);
    const f16x2 a = __builtin_bit_cast(f16x2, h01), b = __builtin_bit_cast(f16x2, h23);
    const f16x2 c = __builtin_bit_cast(f16x2, pack_f16(p[0] - (float)a[0], p[1] - (float)a[1]));
    const f16x2 d = __builtin_bit_cast(f16x2, pack_f16(p[2] - (float)b[0], p[3] - (float)b[1]));
    w.hi = f16x4{a[0], a[1], b[0], b[1]};
    w.lo = f16x4{c[0], c[1], d[0], d[1]};
    return w;
}

// ------------------------------------------------------------------ TQ V

// The PV product of one 16-token block over a TurboQuant-style V cache (head
// dim 128).  Lane (ln, kg) holds the weights p[r] of tokens t = 4kg + r (A
// operand, row g = ln) and the raw V words of those tokens for its columns
// 8 ln .. 8 ln + 7 (one half of a 16-element group): the codes, and a word
// of the group's scale row whose byte `ssel` selects belongs to the token.
//
// Decoding works on two tokens at a time, so that every lookup already
// yields the (t, t + 1) pairs that the FP16 B operand packs per column:
//  - the two tokens' codes of four columns are placed one per nibble,
//    [t: c0 c1 | t: c2 c3 | t+1: c0 c1 | t+1: c2 c3] (3-bit codes are spread
//    from their packed form by two shift-and-insert steps; 2- and 4-bit codes
//    need only byte moves);
//  - even and odd nibbles become byte selectors into the 8-entry FP16 level
//    table (low and high bytes looked up separately with v_perm; a 4-bit
//    code's sign bit goes straight to the FP16 sign);
//  - a v_perm pairs the low and high bytes into the two tokens' FP16 values
//    of one column, and one packed FP16 multiply applies the two tokens'
//    scales.  level x scale has at most 8 significant bits and lies in
//    [2^-12, 1232], so the FP16 product is exact.
// The weights are FP16 (scaled by 2^15 by the caller); the products
// accumulate in FP32.
template <int VT, int VW>
__device__ __forceinline__ void tq_pv(const DecodeArgs& a, const float (&p)[4],
                                      const uint32_t (&v)[4][VW], uint32_t shift, uint32_t ssel,
                                      f32x4 (&o)[8])
{
    constexpr uint32_t MSK = VT == 2 ? 0x03030303u : 0x07070707u;
    const F16Weights ap = f16_weights(p);
    uint32_t vb[2][8];                         // [token pair][column]: FP16 (t, t + 1)
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
        const int r0 = 2 * pr, r1 = 2 * pr + 1;
        const f32x2 sc = unpack_e4m3x2(__builtin_amdgcn_perm(v[r1][VW - 1], v[r0][VW - 1], ssel), false);
        const f16x2 scale = __builtin_bit_cast(f16x2, pack_f16(sc.x, sc.y));
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {       // columns 4 hh .. 4 hh + 3
            uint32_t nw;
            if constexpr (VT == 4) {
                nw = __builtin_amdgcn_perm(v[r1][0], v[r0][0], hh ? 0x07060302u : 0x05040100u);
            } else if constexpr (VT == 2) {
                const uint32_t x = __builtin_amdgcn_perm(v[r1][0], v[r0][0],
                                                         hh ? 0x0C050C01u : 0x0C040C00u);
                const uint32_t y = bit_insert(0xFF00FF00u, x << 4, x);
                nw = bit_insert(0xF0F0F0F0u, y << 2, y);
            } else {
                // the lane's 24 code bits start `shift` (0, 8, 16 or 24) bits
                // into the 8-byte window
                const uint32_t c0 = __builtin_amdgcn_alignbit(v[r0][1], v[r0][0], shift);
                const uint32_t c1 = __builtin_amdgcn_alignbit(v[r1][1], v[r1][0], shift);
                const uint32_t x = __builtin_amdgcn_perm(hh ? c1 >> 12 : c1, hh ? c0 >> 12 : c0,
                                                         0x05040100u);
                const uint32_t y = bit_insert(0xFF00FF00u, x << 2, x);
                nw = bit_insert(0xF0F0F0F0u, y << 1, y);
            }
#pragma unroll
            for (int odd = 0; odd < 2; ++odd) {
                const uint32_t sel = (odd ? nw >> 4 : nw) & MSK;
                const uint32_t lo = __builtin_amdgcn_perm(a.tq_f16[1], a.tq_f16[0], sel);
                uint32_t hi = __builtin_amdgcn_perm(a.tq_f16[3], a.tq_f16[2], sel);
                if constexpr (VT == 4)
                    hi |= (odd ? nw : nw << 4) & 0x80808080u;
                // selector bytes: [t: c_a, t: c_b, t+1: c_a, t+1: c_b]
                const int ca = 4 * hh + odd, cb = 4 * hh + 2 + odd;
                vb[pr][ca] = __builtin_bit_cast(
                    uint32_t, __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(hi, lo, 0x06020400u)) * scale);
                vb[pr][cb] = __builtin_bit_cast(
                    uint32_t, __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(hi, lo, 0x07030501u)) * scale);
            }
        }
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
        const f16x4 bv = __builtin_bit_cast(f16x4, u32x2{vb[0][nt], vb[1][nt]});
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x16f16(ap.hi, bv, o[nt], 0, 0, 0);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x16f16(ap.lo, bv, o[nt], 0, 0, 0);
    }
}

// The PV product of one 16-token block over an E4M3 V cache, in FP16: for
// each pair of tokens a v_perm puts their codes of two columns side by side
// and v_cvt_scalef32_pk_f16_fp8 (scale 1) widens each pair of codes to the
// FP16 pair (t, t + 1) of one column -- exact, every E4M3 value is an FP16
// number.  Weights as for TQ V (FP16, scaled by 2^15 by the caller).
template <int NT, int VW>
__device__ __forceinline__ void e4m3_pv(const float (&p)[4], const uint32_t (&v)[4][VW],
                                        f32x4 (&o)[NT])
{
    const F16Weights ap = f16_weights(p);
    uint32_t vb[2][NT];                        // [token pair][column]: FP16 (t, t + 1)
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
#pragma unroll
        for (int w = 0; w < VW; ++w) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {   // columns 4w + 2hh, 4w + 2hh + 1
                const uint32_t x = __builtin_amdgcn_perm(v[2 * pr + 1][w], v[2 * pr][w],
                                                         hh ? 0x07030602u : 0x05010400u);
                vb[pr][4 * w + 2 * hh] = __builtin_bit_cast(
                    uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false));
                vb[pr][4 * w + 2 * hh + 1] = __builtin_bit_cast(
                    uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true));
            }
        }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const f16x4 bv = __builtin_bit_cast(f16x4, u32x2{vb[0][nt], vb[1][nt]});
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x16f16(ap.hi, bv, o[nt], 0, 0, 0);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x16f16(ap.lo, bv, o[nt], 0, 0, 0);
    }
}

// ------------------------------------------------------------------ MFMA path

// KT: 0 = BF16, 1 = E4M3 K cache.  VT: 0 = BF16, 1 = E4M3, 2/3/4 = the
// TurboQuant-style V with that many bits per code (D = 128).  D: head dim
// of q, K and V (64 or 128).  The K operand layout is KFrag (attn_common.h).
// SPV (TQ V only): the sparse-V skip at threshold a.spv_thr.
//
template <int KT, int VT, int D, int PF, bool BAL, bool SPV>
__global__ __launch_bounds__(512) void decode_mfma_kernel(DecodeArgs a, uint32_t kv_groups)
{
    using KF = KFrag<KT, D>;
    constexpr int NI = KF::NI, NL = KF::NL;
    __shared__ u32x4 s_k[kKvPerGroup][16 * KF::CPR]; // one K tile per wave
    constexpr int NT = D / 16;                 // PV N-tiles
    constexpr int DPL = D / 16;                // V dims per lane
    constexpr bool TQ = VT >= 2;               // TurboQuant-style V, VT bits per code
    static_assert(!TQ || D == 128, "TQ V decode is for head dim 128");
    static_assert(TQ || !SPV, "the sparse-V skip is for TQ V");
    constexpr uint32_t VES = VT == 0 ? 2 : 1;  // V element bytes (BF16 / E4M3)
    // V words per lane per token: 4, 2 or 1; TQ: the codes (an 8-byte window
    // for 3-bit codes, else one word) + the scale byte
    constexpr int VW = TQ ? (VT == 3 ? 3 : 2) : DPL * VES / 4;
    constexpr uint32_t KES = KT == 0 ? 2 : 1;  // K element bytes

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int kg = lane >> 4;                  // 0..3
    const int ln = lane & 15;
    // Token of MFMA row m (K operand row, k index of the PV product): m for
    // BF16 / E4M3 V; for TQ V the 4 x 4 transpose, so that lane group kg,
    // register r holds token 4 r + kg and one V load instruction (fixed r)
    // reads four consecutive token rows of the head's contiguous region.
    auto row_token = [](int m) { return TQ ? 4 * (m & 3) + (m >> 2) : m; };
    // Dispatch order is split-major: x = sequence * kv_groups + kv group,
    // y = split.  Work-groups are dealt to the XCDs round-robin by linear id,
    // so each split "layer" spreads the sequences that reach it evenly over
    // the XCDs (a sequence-major order would pile the always-present early
    // splits onto the same XCDs).  The kv groups of one (sequence, split) are
    // neighbours, so they stream the same cache blocks at about the same time.
    const uint32_t kvh = (blockIdx.x % kv_groups) * (blockDim.x >> 6) + wave;
    if (kvh >= a.Hkv)
        return;

    // One piece of work: cache blocks [b0, b1) of sequence s (at most
    // kMaxRange of them), finished (direct) or written as partial rows
    // prow_base + query head.
    auto run = [&](uint32_t s, const SeqRange& R, uint32_t b0, uint32_t b1, bool direct,
                   uint64_t prow_base) {
    const int32_t n = R.n;

    // q fragments: B operand of S^T = K q^T; lane (g = ln, kg)
    bf16x8 qf[NI];
    {
        const uint32_t g = ln;
        const uint16_t* qrow = (const uint16_t*)a.q + (uint64_t)s * a.q_stride +
                               (uint64_t)(kvh * a.G + g) * D;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            u32x4 w = u32x4{0u, 0u, 0u, 0u};
            if (g < a.G)
                w = *(const u32x4*)(qrow + KF::phys(i, kg));
            qf[i] = __builtin_bit_cast(bf16x8, w);
        }
    }

    // block-table entries of this split, kBtRegs per lane (chunk_blocks <=
    // 64 kBtRegs): entry i is lane i % 64 of bt_lane[i / 64]; lanes past the
    // split re-read its last entry, so the loads are unconditional
    constexpr int NBT = BAL ? kBtRegsBal : kBtRegs;
    int32_t bt_lane[NBT];
#pragma unroll
    for (int h = 0; h < NBT; ++h) {
        const uint32_t idx = b0 + 64 * h + lane;
        bt_lane[h] = a.bt[(uint64_t)s * a.M + (idx < b1 ? idx : b1 - 1)];
    }
    auto table_entry = [&](uint32_t i) -> int32_t {
        int32_t r = bt_lane[0];
#pragma unroll
        for (int h = 1; h < NBT; ++h)
            r = i >= 64u * h ? bt_lane[h] : r;          // wave-uniform choice
        return __builtin_amdgcn_readlane(r, (int)(i & 63));
    };

    const uint8_t* kbase = (const uint8_t*)a.k_cache;
    const uint8_t* vbase = (const uint8_t*)a.v_cache;
    const uint64_t krow_stride = (uint64_t)a.Hkv * D * KES;   // bytes per cache row
    const uint64_t vrow_stride = (uint64_t)a.Hkv * D;         // elements per cache row

    f32x4 o[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
        o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;

    struct Stage {
        u32x4 k[NL];
        uint32_t v[4][VW];
    };

    // Addresses: the block id is wave-uniform, so each block gets a buffer
    // resource built in scalar registers (its record count bounds every access
    // to that block); each lane's byte offsets inside a block are
    // loop-invariant 32-bit values.
    const uint32_t kblk_bytes = (uint32_t)(kBS * krow_stride);
    const uint32_t vblk_bytes = TQ ? a.v_blk_bytes : (uint32_t)(kBS * vrow_stride * VES);
    const uint32_t koff = kKDirect
        ? (uint32_t)(ln * krow_stride + (uint64_t)kvh * D * KES + 16 * kg)
        : (uint32_t)((lane / KF::CPR) * krow_stride + (uint64_t)kvh * D * KES + 16 * (lane % KF::CPR));
    // next load: RPL rows down (row-wise loads) or 4 chunks right (operand loads)
    const uint32_t kstep = kKDirect ? 64u : (uint32_t)(KF::RPL * krow_stride);
    // LDS positions: written chunk of load j, operand chunk of MFMA group j
    uint32_t lds_w[NL], lds_r[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        lds_w[j] = KF::lds_off(j * KF::RPL + lane / KF::CPR, lane % KF::CPR);
        lds_r[j] = KF::lds_off(row_token(ln), KF::op_chunk(j, kg));
    }
    uint8_t* ktile = (uint8_t*)&s_k[wave][0];
    const uint32_t voff = (uint32_t)((4 * kg) * vrow_stride * VES + ((uint64_t)kvh * D + DPL * ln) * VES);
    const uint32_t vrow_bytes = (uint32_t)(vrow_stride * VES);
    // TQ: a block holds one contiguous region per kv head: 16 code rows of
    // 16 VT bytes, then 8 scale rows (one per 16-column group) of 16 bytes,
    // one per token.  Codes of columns 8 ln .. 8 ln + 7 are VT bytes at VT * ln
    // in the token's code row (a 16-bit or 32-bit load for 2- and 4-bit codes,
    // an 8-byte window from the dword at or below for 3-bit codes); the scales
    // of their group are row ln / 2, one 16-byte load, of which dword r, byte
    // kg belongs to token 4 r + kg = register r of lane group kg.
    constexpr uint32_t kTqRegion = kBS * (16u * VT + 8u);
    [[maybe_unused]] const uint32_t tq_coff =
        kvh * kTqRegion + kg * 16u * VT + (VT == 3 ? ((3u * ln) & ~3u) : VT * ln);
    [[maybe_unused]] const uint32_t tq_crow = 4u * 16u * VT;           // r -> r + 1: 4 rows
    [[maybe_unused]] const uint32_t tq_soff = kvh * kTqRegion + kBS * 16u * VT + (ln / 2) * 16u;
    [[maybe_unused]] const uint32_t tq_shift = 8u * ((3u * ln) & 3u);
    // v_perm selector taking byte kg of two scale dwords (tokens 4 r + kg of
    // a register pair) into bytes 0 and 1
    [[maybe_unused]] const uint32_t tq_ssel = (uint32_t)kg | (4u + kg) << 8 | 0x0C0C0000u;

    // An unmapped block is read from block 0 instead (always inside the pool):
    // compute_block masks all of its tokens, so what it holds never counts.
    // do_k / do_v (std::true_type or std::false_type) select the K and V
    // loads; vrec is the record count of the block's V resource (0: the V
    // loads return zeros and move no data).
    auto load_parts = [&](uint32_t bi, Stage& st, auto do_k, auto do_v, uint32_t vrec) {
        int32_t pb = table_entry(bi - b0);
        pb = (pb >= 0 && (uint32_t)pb < a.num_blocks) ? pb : 0;
        const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(kbase + (uint64_t)pb * kblk_bytes), 0, (int)kblk_bytes, kBufferFlags);
        const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(vbase + (uint64_t)pb * vblk_bytes), 0, (int)vrec, kBufferFlags);
        if constexpr (decltype(do_k)::value) {
#pragma unroll
            for (int j = 0; j < NL; ++j) {                                // K: token t = ln
                const u32x4 w = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, koff, j * kstep, kNT));
                st.k[j] = w;
            }
        }
        if constexpr (!decltype(do_v)::value)
            return;
        if constexpr (TQ) {                                               // scales of 16 tokens
            const u32x4 s4 = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(vr, tq_soff, 0, kNT));
#pragma unroll
            for (int r = 0; r < 4; ++r)
                st.v[r][VW - 1] = s4[r];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {                                     // V: t = 4kg + r
            if constexpr (TQ) {
                if constexpr (VT == 3) {
                    const u32x2 c2 = __builtin_bit_cast(
                        u32x2, __builtin_amdgcn_raw_buffer_load_b64(vr, tq_coff, r * tq_crow, kNT));
                    st.v[r][0] = c2[0];
                    st.v[r][1] = c2[1];
                } else if constexpr (VT == 4) {
                    st.v[r][0] = __builtin_amdgcn_raw_buffer_load_b32(vr, tq_coff, r * tq_crow, kNT);
                } else {
                    st.v[r][0] = __builtin_amdgcn_raw_buffer_load_b16(vr, tq_coff, r * tq_crow, kNT);
                }
            } else if constexpr (VW == 4) {
                const u32x4 t4 = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(vr, voff, r * vrow_bytes, kNT));
                st.v[r][0] = t4[0]; st.v[r][1] = t4[1]; st.v[r][2] = t4[2]; st.v[r][3] = t4[3];
            } else if constexpr (VW == 2) {
                const u32x2 t2 = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_raw_buffer_load_b64(vr, voff, r * vrow_bytes, kNT));
                st.v[r][0] = t2[0]; st.v[r][1] = t2[1];
            } else {
                st.v[r][0] = __builtin_amdgcn_raw_buffer_load_b32(vr, voff, r * vrow_bytes, kNT);
            }
        }
    };
    auto load_block = [&](uint32_t bi, Stage& st) {
        load_parts(bi, st, std::true_type{}, std::true_type{}, vblk_bytes);
    };

    // Scores of block bi from its K rows in st: the softmax weights p of the
    // lane's tokens relative to the new running maximum (FP16 PV paths: times
    // 2^15; tokens that do not count: 0) and the factor alpha that takes
    // values relative to the old maximum to the new one; m and l are
    // updated.  [tlo, ntok) are the block's tokens that count.
    auto score_block = [&](uint32_t bi, Stage& st, float (&p)[4], float& alpha, int& ntok_out,
                           int& tlo_out) {
        const int32_t pb = table_entry(bi - b0);
        const bool blk_ok = pb >= 0 && (uint32_t)pb < a.num_blocks;
        const int32_t rem = n - (int32_t)(bi * kBS);
        const int ntok = blk_ok ? (rem < kBS ? rem : kBS) : 0;
        const int tlo = R.lo - (int32_t)(bi * kBS);   // tokens below it are outside the window

        // K rows -> MFMA operand layout through the wave's LDS tile (lanes
        // exchange data: order the writes after the previous block's reads
        // and before this block's reads, at wavefront scope)
        u32x4 kop[NL];
        if constexpr (kKDirect) {
#pragma unroll
            for (int j = 0; j < NL; ++j)
                kop[j] = st.k[j];
        } else {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int j = 0; j < NL; ++j)
                *(u32x4*)(ktile + lds_w[j]) = st.k[j];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int j = 0; j < NL; ++j)
                kop[j] = *(const u32x4*)(ktile + lds_r[j]);
        }

        // S^T = K q^T : lane holds S[t = 4kg + r][g = ln]
        f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NI; ++i)
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(KF::operand(kop, i), qf[i], sacc, 0, 0, 0);

        // scaled scores, masked ones -inf (a block wholly inside the range
        // needs no mask)
        float sv[4];
        if (ntok == kBS && tlo <= 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sv[r] = sacc[r] * a.qk_scale;
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = row_token(4 * kg + r);
                sv[r] = (t < ntok && t >= tlo) ? sacc[r] * a.qk_scale : -INFINITY;
            }
        }
        float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        mx = row_max_xor16_32(mx);
        const float m_new = fmaxf(m, mx);
        // while no token has counted yet (m_new = -inf) use 0 as the reference:
        // masked scores give p = 0, and alpha = 0 leaves the zero state zero
        const float m_ref = m_new == -INFINITY ? 0.f : m_new;
        alpha = __builtin_amdgcn_exp2f(m - m_ref);
        // TQ and E4M3 V: the weights go to the PV product as FP16 scaled by
        // 2^15 (kept clear of FP16 subnormals; p <= 1); the normalisation
        // divides it out
        constexpr bool F16PV = TQ || VT == 1;
        constexpr float kPOff = F16PV ? 15.f : 0.f;
        // the exponent is the difference of the rounded scaled score and the
        // reference, never an FMA of the raw score: with kPOff = 0 the row's
        // largest score gives exactly 1 (one attended token returns its V row)
        {
#pragma clang fp contract(off)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                p[r] = __builtin_amdgcn_exp2f(sv[r] - (m_ref - kPOff));
        }
        const float psum = (p[0] + p[1]) + (p[2] + p[3]);
        l = F16PV ? __builtin_fmaf(psum, 1.f / 32768.f, l * alpha) : l * alpha + psum;
        m = m_new;
        ntok_out = ntok;
        tlo_out = tlo;
    };
    // O rows are g = 4kg + r; their factor lives in lane g
    auto rescale_o = [&](float alpha) {
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
            // O rows are g = 4kg + r; their factor lives in lane g
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ar = __shfl(alpha, 4 * kg + r, 64);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    o[nt][r] *= ar;
            }
        }
    };
    // masked tokens must not bring NaN/Inf into 0 * V
    auto mask_v = [&](Stage& st, int ntok, int tlo) {
        if (ntok < kBS || tlo > 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (row_token(4 * kg + r) >= ntok || row_token(4 * kg + r) < tlo)
#pragma unroll
                    for (int w = 0; w < VW; ++w)
                        st.v[r][w] = 0u;
        }
    };

    auto compute_block = [&](uint32_t bi, Stage& st) {
        float p[4], alpha;
        int ntok, tlo;
        score_block(bi, st, p, alpha, ntok, tlo);
        rescale_o(alpha);
        mask_v(st, ntok, tlo);
        if constexpr (TQ) {
            tq_pv<VT>(a, p, st.v, tq_shift, tq_ssel, o);
            return;
        } else if constexpr (VT == 1) {
            e4m3_pv<NT>(p, st.v, o);
            return;
        }

        // P as hi + lo BF16 (A operand: lane holds P[g = ln][t = 4kg + r])
        uint32_t ph[2], pl[2];
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
            const uint32_t hw = pack_bf16(p[2 * r2], p[2 * r2 + 1]);
            ph[r2] = hw;
            pl[r2] = pack_bf16(p[2 * r2] - bf16_lo(hw), p[2 * r2 + 1] - bf16_hi(hw));
        }
        const i16x4 a_hi = __builtin_bit_cast(i16x4, u32x2{ph[0], ph[1]});
        const i16x4 a_lo = __builtin_bit_cast(i16x4, u32x2{pl[0], pl[1]});

        // B operand of N-tile nt: element nt of the lane's DPL columns, rows
        // t = 4kg + 0..3
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            uint32_t b01, b23;
            const int w = nt >> 1;
            if (nt & 1) {
                b01 = hi16_pair(st.v[0][w], st.v[1][w]);
                b23 = hi16_pair(st.v[2][w], st.v[3][w]);
            } else {
                b01 = lo16_pair(st.v[0][w], st.v[1][w]);
                b23 = lo16_pair(st.v[2][w], st.v[3][w]);
            }
            const i16x4 bv = __builtin_bit_cast(i16x4, u32x2{b01, b23});
            o[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_hi, bv, o[nt], 0, 0, 0);
            o[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_lo, bv, o[nt], 0, 0, 0);
        }
    };

    if constexpr (SPV) {
        // Sparse-V skip (page 2, paged_decode_attn_fp8k_turbo3v: the V load
        // and dequantisation of a position are skipped when its attention
        // weight is at most the threshold).  The weight at hand when block b
        // is scored is p / 2^15 = exp(s - running max), at least the final
        // softmax weight, so every position left out has a weight at most the
        // threshold; its weight stays in l, and rows past the GQA group never
        // count.  V of block b is loaded only when some position is kept,
        // right after the block's scores; its PV product waits two blocks, so
        // that the load has a block of work to arrive under, and its weights
        // are rescaled to the running maximum meanwhile.  K is loaded
        // kPrefetchSpv blocks ahead.  Block b's K lives in kst[(b - b0) % KS],
        // its V in vst[(b - b0) % 2] and its pending weights in
        // pw[(b - b0) % 2].
        constexpr int KPF = kPrefetchSpv;          // K blocks loaded ahead
        constexpr int KS = KPF + 1;                 // K stages
        constexpr int P = KS % 2 ? 2 * KS : KS;     // unroll period: K stages and V parity
        static_assert(P == 2, "the two steps run ahead of the loop keep (b - b0) % P == u "
                              "at the loop's entry only for a period of two");
        Stage kst[KS], vst[2];                      // K in kst[].k, V in vst[].v
        float pw[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        bool keep[2] = {false, false};             // wave-uniform
        int pn[2] = {0, 0}, pt[2] = {0, 0};        // [tlo, ntok) of the pending blocks
        auto pv_pending = [&](int v) {
            if (keep[v]) {
                mask_v(vst[v], pn[v], pt[v]);
                tq_pv<VT>(a, pw[v], vst[v].v, tq_shift, tq_ssel, o);
            }
        };
        // block b = b0 + (multiple of P) + u
        auto step = [&](uint32_t b, int u, bool prefetch) {
            if (prefetch)
                load_parts(b + KPF, kst[(u + KPF) % KS], std::true_type{}, std::false_type{}, 0u);
            float p[4], alpha;
            int ntok, tlo;
            score_block(b, kst[u % KS], p, alpha, ntok, tlo);
            const int v = u % 2;
            pv_pending(v);                          // block b - 2, at the old maximum
            rescale_o(alpha);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                pw[v ^ 1][r] *= alpha;              // block b - 1 to the new maximum
            bool kept = false;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool k = p[r] > a.spv_thr;
                pw[v][r] = k ? p[r] : 0.f;
                kept |= k && (uint32_t)ln < a.G;
            }
            keep[v] = __builtin_amdgcn_ballot_w64(kept) != 0;
            pn[v] = ntok;
            pt[v] = tlo;
            // issued whether or not the block is kept (a skipped block's
            // resource holds no records, so its loads move no data): the
            // count of loads in flight stays fixed, which keeps the
            // compiler's waits to the loads each use needs
            load_parts(b, vst[v], std::false_type{}, std::true_type{}, keep[v] ? vblk_bytes : 0u);
        };
        // The first two steps run ahead of the loop, so that the loop is
        // entered with the loads in flight in the order of its back edge
        // (K of the next block behind V of the last one): the compiler's
        // waits, which must hold on both paths, then wait only for the loads
        // each use needs.
#pragma unroll
        for (int f = 0; f < KPF; ++f)
            load_parts(b0 + f < b1 ? b0 + f : b1 - 1, kst[f], std::true_type{}, std::false_type{}, 0u);
        step(b0, 0, b0 + KPF < b1);
        if (b0 + 1 < b1) {
            step(b0 + 1, 1, b0 + 1 + KPF < b1);
            uint32_t bi = b0 + 2;
            for (; bi + P + KPF - 1 < b1; bi += P) {
#pragma unroll
                for (int u = 0; u < P; ++u)
                    step(bi + u, u, true);
            }
#pragma unroll
            for (int u = 0; u < P + KPF - 1; ++u) {
                if (bi + u >= b1)
                    break;
                step(bi + u, u, bi + u + KPF < b1);
            }
        }
        pv_pending(0);
        pv_pending(1);
    } else {
    // Ring of PF + 1 register stages; block b lives in stage (b - b0) % NS.
    // The main loop prefetches unconditionally (every block it handles has a
    // block PF ahead), so the compiler's wait before each compute covers only
    // the stage in use; the tail handles the last blocks with conditional
    // prefetch.  The prologue clamps to the last block instead of branching.
    constexpr int NS = PF + 1;
    Stage st[NS];
#pragma unroll
    for (int f = 0; f < PF; ++f)
        load_block(b0 + f < b1 ? b0 + f : b1 - 1, st[f]);
    uint32_t bi = b0;
    for (; bi + NS + PF - 1 < b1; bi += NS) {
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            load_block(bi + u + PF, st[(u + PF) % NS]);
            compute_block(bi + u, st[u]);
        }
    }
#pragma unroll
    for (int u = 0; u < NS + PF - 1; ++u) {
        const uint32_t b = bi + u;
        if (b >= b1)
            break;
        if (b + PF < b1)
            load_block(b + PF, st[(u + PF) % NS]);
        compute_block(b, st[u % NS]);
    }
    }

    l = row_sum_xor16_32(l);
    emit_mfma<D>(a, s, kvh, direct, prow_base, lane, o, m, l);
    };

    // The work-group's pieces: one (sequence, split) in split mode; in
    // balanced mode the pieces of range w of the flattened block list (see
    // range_blocks), sequence by sequence.  One call site of run.
    constexpr bool balanced = BAL;
    const uint32_t w = blockIdx.x / kv_groups;
    uint32_t s = w, cu = 0, r0 = 0, r1 = 0, C = 1;
    if constexpr (balanced) {
        const uint32_t T = total_blocks(a, lane);
        if (a.cu && blockIdx.x == 0 && wave == 0) {
            // the prefix sums, for the merge (which runs after this kernel)
            uint32_t base = 0;
            for (uint32_t c = 0; c < a.S; c += 64) {
                const uint32_t si = c + (uint32_t)lane;
                const uint32_t nb = si < a.S ? att_blocks(a, si) : 0u;
                uint32_t incl = nb;
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) {
                    const uint32_t t = __shfl_up(incl, d, 64);
                    if (lane >= d)
                        incl += t;
                }
                if (si < a.S)
                    a.cu[si] = base + incl - nb;
                base += __builtin_amdgcn_readlane(incl, 63);
            }
            if (lane == 0)
                a.cu[a.S] = T;
        }
        C = range_blocks(T, a.ranges);
        r0 = w * C;
        if (r0 >= T)
            return;
        r1 = r0 + C < T ? r0 + C : T;
        // first sequence whose blocks reach past r0, and where its blocks start
        s = 0;
        uint32_t base = 0;
        for (uint32_t c = 0; c < a.S; c += 64) {
            const uint32_t si = c + (uint32_t)lane;
            const uint32_t nb = si < a.S ? att_blocks(a, si) : 0u;
            uint32_t incl = nb;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const uint32_t t = __shfl_up(incl, d, 64);
                if (lane >= d)
                    incl += t;
            }
            incl += base;
            const uint64_t hit = __builtin_amdgcn_ballot_w64(si < a.S && incl > r0);
            if (hit) {
                const int l0 = __builtin_ctzll(hit);
                s = c + (uint32_t)l0;
                cu = __builtin_amdgcn_readlane(incl - nb, l0);
                break;
            }
            base = __builtin_amdgcn_readlane(incl, 63);
        }
    }
    const uint32_t split = blockIdx.y;
    for (;;) {
        if (balanced && (s >= a.S || cu >= r1))
            break;
        const SeqRange R = seq_range(a, s);
        uint32_t b0, b1, nb = 0;
        bool direct;
        uint64_t prow_base;
        if constexpr (balanced) {
            nb = R.nblk > R.blo ? R.nblk - R.blo : 0u;
            const uint32_t lo = r0 > cu ? r0 : cu;
            const uint32_t hi = cu + nb < r1 ? cu + nb : r1;
            if (hi <= lo) {
                cu += nb;
                ++s;
                continue;
            }
            b0 = R.blo + (lo - cu);
            b1 = R.blo + (hi - cu);
            direct = cu / C == (cu + nb - 1) / C;
            prow_base = (uint64_t)(w + s) * a.Hq;
        } else {
            // split y of sequence s covers chunk_blocks blocks from R.blo
            if (split >= R.nsplit) {
                if (R.nsplit == 0 && split == 0) {
                    // nothing attended: zero output rows of this kv head's group
                    for (uint32_t idx = lane; idx < a.G * D; idx += 64)
                        a.out[((uint64_t)s * a.Hq + kvh * a.G) * D + idx] = 0.f;
                }
                return;
            }
            b0 = R.blo + split * a.chunk_blocks;
            b1 = min(b0 + a.chunk_blocks, R.nblk);
            direct = R.nsplit == 1;
            prow_base = ((uint64_t)s * a.max_splits + split) * a.Hq;
        }
        run(s, R, b0, b1, direct, prow_base);
        if (!balanced)
            break;
        cu += nb;
        ++s;
    }
}

// ------------------------------------------------------------------ FP32 path

// Maximum and sum over the 16 lanes of each row (DPP), then over the four
// rows (gfx950 row swaps): the result is in every lane of the wave.
__device__ __forceinline__ float row16_max(float v)
{
    v = fmaxf(v, dpp_f32<kDppXor1>(v));
    v = fmaxf(v, dpp_f32<kDppXor2>(v));
    v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f32<kDppMirror>(v));
    return v;
}
__device__ __forceinline__ float wave_max64(float v) { return row_max_xor16_32(row16_max(v)); }
__device__ __forceinline__ float wave_sum64(float v) { return row_sum_xor16_32(row16_sum(v)); }

// One wavefront per (sequence, kv head, split).  Lane row r = lane / 16
// holds tokens 4 i + r (i = 0..3) of each 16-token cache block, 16 lanes per
// row: lane c of the row reads 16 bytes at 16 c + 256 j of the head's K and V
// slices (JK and JV loads per token).  A block's whole load set is issued one
// block ahead (two register stages); each block gets buffer resources built
// in scalar registers from its table entry, the split's entries having been
// read once into lanes; an unmapped or past-the-split block gets a record
// count of 0, so its loads return zeros and move no data.  Per row, a block's
// four scores come from a DPP row reduction, and the row's softmax stream is
// rescaled once per block; the four row streams merge at the end.
template <int DQK, int DV, int G>
__global__ __launch_bounds__(64) void decode_f32_kernel(DecodeArgs a)
{
    constexpr int JK = DQK / 64;               // 16-byte loads of a K slice per lane
    constexpr int JV = DV / 64;                // 16-byte loads of a V slice per lane
    constexpr bool QREG = G * JK <= 12;        // q in registers, else read from LDS
    __shared__ float s_q[G][DQK];

    const int lane = threadIdx.x;
    const int row = lane >> 4;                 // token row 0..3
    const int c = lane & 15;
    // split-major dispatch order (see decode_mfma_kernel)
    const uint32_t kvh = blockIdx.x;
    const uint32_t s = blockIdx.y;
    const uint32_t split = blockIdx.z;

    const SeqRange R = seq_range(a, s);
    const int32_t n = R.n;
    const uint32_t nsplit = R.nsplit;
    const uint32_t b0 = R.blo + split * a.chunk_blocks;
    if (split >= nsplit) {
        if (nsplit == 0 && split == 0)
            for (uint32_t idx = lane; idx < (uint32_t)G * DV; idx += 64)
                a.out[((uint64_t)s * a.Hq + kvh * G) * DV + idx] = 0.f;
        return;
    }
    const uint32_t b1 = min(b0 + a.chunk_blocks, R.nblk);

    // block-table entries of the split, kBtRegs per lane (entry i at lane
    // i % 64 of bt_lane[i / 64]; lanes past the split re-read its last one)
    int32_t bt_lane[kBtRegs];
#pragma unroll
    for (int h = 0; h < kBtRegs; ++h) {
        const uint32_t idx = b0 + 64 * h + lane;
        bt_lane[h] = a.bt[(uint64_t)s * a.M + (idx < b1 ? idx : b1 - 1)];
    }

    // q rows of the group into LDS, rotated at position n - 1 if asked
    const float* qsrc = (const float*)a.q + (uint64_t)s * a.q_stride + (uint64_t)kvh * G * DQK;
    for (int idx = lane; idx < G * DQK; idx += 64)
        s_q[idx / DQK][idx % DQK] = qsrc[idx];
    __syncthreads();
    if (a.q_rope && a.q_rope_dim > 0) {
        const uint32_t half = a.q_rope_dim / 2;
        for (uint32_t idx = lane; idx < (uint32_t)G * half; idx += 64) {
            const uint32_t g = idx / half, i = idx % half;
            const float ang = (float)(n - 1) * a.q_invf[i];
            float sn, cs;
            sincosf(ang, &sn, &cs);
            const float x0 = s_q[g][a.q_rope_offset + i];
            const float x1 = s_q[g][a.q_rope_offset + i + half];
            s_q[g][a.q_rope_offset + i] = x0 * cs - x1 * sn;
            s_q[g][a.q_rope_offset + i + half] = x1 * cs + x0 * sn;
        }
        __syncthreads();
    }
    f32x4 qv[QREG ? G : 1][QREG ? JK : 1];
    if constexpr (QREG) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int j = 0; j < JK; ++j)
                qv[g][j] = *(const f32x4*)&s_q[g][64 * j + 4 * c];
    }
    auto q_chunk = [&](int g, int j) -> f32x4 {
        if constexpr (QREG)
            return qv[g][j];
        else
            return *(const f32x4*)&s_q[g][64 * j + 4 * c];
    };

    float m[G], l[G];
    f32x4 o[G][JV];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int j = 0; j < JV; ++j)
            o[g][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const uint8_t* kbase = (const uint8_t*)a.k_cache;
    const uint8_t* vbase = (const uint8_t*)a.v_cache;
    const uint32_t krow = a.Hkv * DQK * 4u, vrow = a.Hkv * DV * 4u;     // bytes per cache row
    const uint32_t kblk = kBS * krow, vblk = kBS * vrow;
    const uint32_t koff = row * krow + kvh * DQK * 4u + 16u * c;
    const uint32_t voff = row * vrow + kvh * DV * 4u + 16u * c;

    struct Stage {
        f32x4 k[4][JK];
        f32x4 v[4][JV];
    };
    auto block_ok = [&](uint32_t bi) -> int32_t {
        int32_t r = bt_lane[0];
#pragma unroll
        for (int h = 1; h < kBtRegs; ++h)
            r = bi - b0 >= 64u * h ? bt_lane[h] : r;        // wave-uniform choice
        const int32_t pb = __builtin_amdgcn_readlane(r, (int)((bi - b0) & 63));
        return (bi < b1 && pb >= 0 && (uint32_t)pb < a.num_blocks) ? pb : -1;
    };
    auto load_block = [&](uint32_t bi, Stage& st) {
        const int32_t pb = block_ok(bi);
        const uint64_t p = pb >= 0 ? (uint64_t)pb : 0;
        const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(kbase + p * kblk), 0, pb >= 0 ? (int)kblk : 0, kBufferFlags);
        const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(vbase + p * vblk), 0, pb >= 0 ? (int)vblk : 0, kBufferFlags);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int j = 0; j < JK; ++j)
                st.k[i][j] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, koff + 256u * j, 4u * i * krow, kNT));
#pragma unroll
            for (int j = 0; j < JV; ++j)
                st.v[i][j] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(vr, voff + 256u * j, 4u * i * vrow, kNT));
        }
    };
    auto compute_block = [&](uint32_t bi, Stage& st) {
        // tokens 4 i + row of the block; an unmapped block loaded zeros
        const int32_t t0 = (int32_t)(bi * kBS) + row;
        const bool full = block_ok(bi) >= 0 && (int32_t)(bi * kBS) >= R.lo &&
                          (int32_t)(bi * kBS) + kBS <= n;
        bool ok[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int32_t t = t0 + 4 * i;
            ok[i] = full || (block_ok(bi) >= 0 && t < n && t >= R.lo);
            if (!full && !ok[i]) {
#pragma unroll
                for (int j = 0; j < JV; ++j)
                    st.v[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};   // rows past n may hold anything
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float sc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float d = 0.f;
#pragma unroll
                for (int j = 0; j < JK; ++j) {
                    const f32x4 qq = q_chunk(g, j);
                    d += qq.x * st.k[i][j].x + qq.y * st.k[i][j].y + qq.z * st.k[i][j].z +
                         qq.w * st.k[i][j].w;
                }
                d = row16_sum(d);
                sc[i] = ok[i] ? d * a.qk_scale : -INFINITY;
            }
            const float mb = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
            const float m_new = fmaxf(m[g], mb);
            if (m_new != -INFINITY) {
                const float alpha = __builtin_amdgcn_exp2f(m[g] - m_new);
                float p[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    p[i] = __builtin_amdgcn_exp2f(sc[i] - m_new);
                l[g] = l[g] * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
                for (int j = 0; j < JV; ++j) {
                    f32x4 acc = o[g][j] * alpha;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc = acc + st.v[i][j] * p[i];
                    o[g][j] = acc;
                }
                m[g] = m_new;
            }
        }
    };

    // two register stages, one block ahead: the main loop's loads are
    // unconditional (so the wait before each block covers only that block's
    // loads), and a tail takes the last one or two blocks; every load issued
    // is consumed
    Stage sa, sb;
    load_block(b0, sa);
    uint32_t bi = b0;
    for (; bi + 2 < b1; bi += 2) {
        load_block(bi + 1, sb);
        compute_block(bi, sa);
        load_block(bi + 2, sa);
        compute_block(bi + 1, sb);
    }
    if (bi + 1 < b1) {
        load_block(bi + 1, sb);
        compute_block(bi, sa);
        compute_block(bi + 1, sb);
    } else {
        compute_block(bi, sa);
    }

    // merge the four row streams
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float mt = row_max_xor16_32(m[g]);
        const float f = mt == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[g] - mt);
        float lt = row_sum_xor16_32(l[g] * f);
#pragma unroll
        for (int j = 0; j < JV; ++j) {
            f32x4 v = o[g][j] * f;
            v.x = row_sum_xor16_32(v.x);
            v.y = row_sum_xor16_32(v.y);
            v.z = row_sum_xor16_32(v.z);
            v.w = row_sum_xor16_32(v.w);
            o[g][j] = v;
        }
        if (row != 0)
            continue;
        const uint32_t h = kvh * G + g;
        if (nsplit == 1) {
            const float inv = norm_factor(mt, lt, a.sinks, h, a.out_scale);
            const uint64_t base = ((uint64_t)s * a.Hq + h) * DV;
#pragma unroll
            for (int j = 0; j < JV; ++j) {
                f32x4 v = o[g][j] * inv;
                if (a.gate)
                    v = v * *(const f32x4*)(a.gate + base + 64 * j + 4 * c);
                *(f32x4*)(a.out + base + 64 * j + 4 * c) = v;
            }
        } else {
            const uint64_t prow = ((uint64_t)s * a.max_splits + split) * a.Hq + h;
#pragma unroll
            for (int j = 0; j < JV; ++j)
                *(f32x4*)(a.part_o + prow * DV + 64 * j + 4 * c) = o[g][j];
            if (c == 0)
                *(f32x2*)(a.part_ml + prow * 2) = f32x2{mt, lt};
        }
    }
}

// ------------------------------------------------------------------ merge

// One wavefront per (sequence, query head) with more than one split, four
// query heads per work-group:
//   M = max_i m_i, w_i = 2^(m_i - M), out = sum_i w_i o_i / sum_i w_i l_i.
// Lane i holds split i's (m, l) (64 splits per pass); each lane accumulates
// its DPL = Dv / 64 output columns over the splits in order.  An empty split
// (m = -inf, o = 0) gets weight 0; with every split empty the reference is 0
// instead of M, so no weight is NaN and the row stays zero.
constexpr uint32_t kMergeHeads = 4;
// Partial rows loaded together: 1 / 4 / 8 gave 5.6 / 5.8 / 6.9 us on the
// BF16 workload (a sequence has 1-3 pieces under the balanced plan) and
// 5.8 / 5.4 / 5.5 us on the E4M3-K one (4-8 pieces).
constexpr int kMergeRows = 4;
template <int DPL>
__global__ __launch_bounds__(64 * kMergeHeads) void decode_merge_kernel(DecodeArgs a)
{
    constexpr uint32_t DV = 64 * DPL;
    const uint32_t s = blockIdx.x;
    const uint32_t h = blockIdx.y * kMergeHeads + (threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63;
    if (h >= a.Hq)
        return;
    uint32_t nsplit;
    uint64_t prow0;
    const uint64_t oi = ((uint64_t)s * a.Hq + h) * DV + lane * DPL;
    if (a.ranges) {
        // balanced mode: the pieces of s are ranges first .. last, at slots
        // w + s; with one range every sequence was finished in place
        const uint32_t T = a.cu ? a.cu[a.S] : 0u;
        const uint32_t cu = a.cu ? a.cu[s] : 0u;
        const uint32_t nb = a.cu ? a.cu[s + 1] - cu : att_blocks(a, s);
        if (nb == 0) {
            // nothing attended: a zero row (no range wrote it)
#pragma unroll
            for (int k = 0; k < DPL; ++k)
                a.out[oi + k] = 0.f;
            return;
        }
        if (!a.cu)
            return;
        const uint32_t C = range_blocks(T, a.ranges);
        const uint32_t first = cu / C;
        uint32_t last = (cu + nb - 1) / C;
        last = last < a.ranges ? last : a.ranges - 1;   // always true for a consistent plan
        nsplit = first <= last ? last - first + 1 : 0u;
        prow0 = (uint64_t)(first + s) * a.Hq + h;
    } else {
        nsplit = seq_range(a, s).nsplit;
        prow0 = (uint64_t)s * a.max_splits * a.Hq + h;
    }
    if (nsplit <= 1)
        return;
    auto ml_of = [&](uint32_t i) {
        return *(const f32x2*)(a.part_ml + (prow0 + (uint64_t)i * a.Hq) * 2);
    };
    float g[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k)
        g[k] = a.gate ? a.gate[oi + k] : 1.f;

    const f32x2 ml0 = lane < nsplit ? ml_of(lane) : f32x2{-INFINITY, 0.f};
    float M = ml0[0];
    for (uint32_t i = lane + 64; i < nsplit; i += 64)
        M = fmaxf(M, ml_of(i)[0]);
    M = wave_max64(M);
    const float Mref = M == -INFINITY ? 0.f : M;

    float L = 0.f;
    float acc[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k)
        acc[k] = 0.f;
    for (uint32_t i0 = 0; i0 < nsplit; i0 += 64) {
        const f32x2 ml = i0 == 0 ? ml0
                                 : (i0 + lane < nsplit ? ml_of(i0 + lane) : f32x2{-INFINITY, 0.f});
        const float w = __builtin_amdgcn_exp2f(ml[0] - Mref);
        L = __builtin_fmaf(w, ml[1], L);
        const uint32_t n = nsplit - i0 < 64u ? nsplit - i0 : 64u;
        // kMergeRows partial rows in flight at a time (rows past n re-read
        // row n - 1, which exists, and are not accumulated)
        for (uint32_t j0 = 0; j0 < n; j0 += kMergeRows) {
            float o[kMergeRows][DPL];
#pragma unroll
            for (int u = 0; u < kMergeRows; ++u) {
                const uint32_t j = j0 + u < n ? j0 + u : n - 1;
                const float* orow = a.part_o + (prow0 + (uint64_t)(i0 + j) * a.Hq) * DV + lane * DPL;
                if constexpr (DPL == 2) {
                    const f32x2 t = *(const f32x2*)orow;
                    o[u][0] = t[0];
                    o[u][1] = t[1];
                } else {
                    o[u][0] = orow[0];
                }
            }
#pragma unroll
            for (int u = 0; u < kMergeRows; ++u) {
                if (j0 + u < n) {
                    const float wj = __int_as_float(
                        __builtin_amdgcn_readlane(__float_as_int(w), (int)(j0 + u)));
#pragma unroll
                    for (int k = 0; k < DPL; ++k)
                        acc[k] = __builtin_fmaf(wj, o[u][k], acc[k]);
                }
            }
        }
    }
    L = wave_sum64(L);
    const float inv = norm_factor(M, L, a.sinks, h, a.out_scale);
    if constexpr (DPL == 2) {
        *(f32x2*)(a.out + oi) = f32x2{acc[0] * inv * g[0], acc[1] * inv * g[1]};
    } else {
        a.out[oi] = acc[0] * inv * g[0];
    }
}

// ------------------------------------------------------------------ host

struct Plan {
    uint32_t chunk_blocks;
    uint32_t max_splits;
    uint32_t ranges;        // balanced mode: block ranges per kv group (0 = split mode)
    size_t workspace;
};

// Balanced mode (MFMA path, automatic split size, no sliding window): up to
// this many sequences per call (every wave scans seq_lens) and this many
// ranges.  A windowed decode attends a few hundred blocks per sequence, whose
// equal splits already balance, and measured slower in balanced mode.
constexpr uint32_t kBalancedMaxSeqs = 1024;
constexpr uint64_t kBalancedMaxRanges = 1u << 16;

// Split plan: enough (sequence, split) work-groups to cover the chip several
// times over, each split a whole number of blocks, at most 128 blocks (so a
// split's block-table entries fit two per lane).  A window of W tokens
// touches at most floor((W + 2B - 2) / B) blocks of size B, which bounds the
// attended blocks of every sequence.
static Plan make_plan(uint32_t num_seqs, uint32_t num_q_heads, uint32_t num_kv_heads,
                      uint32_t head_dim_v, uint32_t max_blocks_per_seq, uint32_t block_size,
                      uint32_t sliding_window, uint32_t split_tokens, bool mfma)
{
    Plan p{};
    if (sliding_window > 0) {
        const uint64_t wb = ((uint64_t)sliding_window + 2ull * block_size - 2) / block_size;
        if (wb < max_blocks_per_seq)
            max_blocks_per_seq = (uint32_t)wb;
    }
    uint32_t cb;
    if (split_tokens) {
        cb = ceil_div(split_tokens, block_size);
    } else {
        // MFMA path: (sequence, kv group) work-groups of two waves, about
        // kTargetGroups of them; FP32 path: one wave per (sequence, kv head,
        // split), about kTargetWavesF32 of them
        const uint32_t kv_groups = mfma ? ceil_div(num_kv_heads, kKvPerGroup) : num_kv_heads;
        const uint64_t target = mfma ? kTargetGroups : kTargetWavesF32;
        const uint64_t units = (uint64_t)num_seqs * kv_groups;
        const uint64_t want = units >= target ? 1 : (target + units - 1) / units;
        cb = ceil_div(max_blocks_per_seq, want);
        cb = cb < kMinChunk ? kMinChunk : cb;
        // equal splits: as few as the chunk cap allows, then evenly sized
        if (cb > kMaxChunk)
            cb = ceil_div(max_blocks_per_seq, ceil_div(max_blocks_per_seq, kMaxChunk));
    }
    cb = cb < 1 ? 1 : cb > kMaxChunk ? kMaxChunk : cb;
    p.chunk_blocks = cb;
    p.max_splits = ceil_div(max_blocks_per_seq, cb);
    if (p.max_splits > 1)
        p.workspace = (size_t)num_seqs * p.max_splits * num_q_heads * (head_dim_v + 2) * sizeof(float);
    if (mfma && !split_tokens && !sliding_window && num_seqs <= kBalancedMaxSeqs) {
        // enough ranges that ceil(T / ranges) <= kMaxRange for any T up to
        // num_seqs * max_blocks_per_seq (the attended-block bound), and the
        // work-group target, but no more than one range per kMinChunk blocks
        // of that bound; a single range finishes every sequence itself and
        // needs no workspace
        const uint32_t kv_groups = ceil_div(num_kv_heads, kKvPerGroup);
        const uint64_t bound = (uint64_t)num_seqs * max_blocks_per_seq;
        const uint64_t need = (bound + kMaxRange - 1) / kMaxRange;
        uint64_t spread = (kTargetGroups + kv_groups - 1) / kv_groups;
        const uint64_t small = (bound + kMinChunk - 1) / kMinChunk;
        spread = spread < small ? spread : small;
        uint64_t ranges = need > spread ? need : spread;
        ranges = ranges < 1 ? 1 : ranges;
        if (ranges <= kBalancedMaxRanges) {
            p.ranges = (uint32_t)ranges;
            p.workspace = ranges > 1
                ? (size_t)(ranges + num_seqs) * num_q_heads * (head_dim_v + 2) * sizeof(float) +
                      ((size_t)num_seqs + 1) * sizeof(uint32_t)
                : 0;
        }
    }
    return p;
}

// Device scratch of pkv_paged_decode_attn_noalloc: the split partials live
// here instead of in a caller workspace.  Each GPU the library runs on holds
// its own copy for the life of the process.  Host code never passes the
// array's name to a kernel (on the host it is a stand-in, not a device
// address): the address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[PKV_DECODE_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch (looked up on the first
// call on that device, with the device current).  `stream`, when not NULL,
// must belong to the current device.
static int scratch_address(hipStream_t stream, void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(PKV_ERR_HIP, "paged_decode_attn_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(PKV_ERR_UNSUPPORTED, "paged_decode_attn_noalloc: device %d beyond %d", dev, kMaxDevices);
    if (stream) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess)
            return fail(PKV_ERR_HIP, "paged_decode_attn_noalloc: hipStreamGetDevice: %s", hipGetErrorString(e));
        if (sdev != dev)
            return fail(PKV_ERR_INVALID, "paged_decode_attn_noalloc: the stream belongs to device %d, the current device is %d",
                        (int)sdev, dev);
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(PKV_ERR_HIP, "paged_decode_attn_noalloc: hipGetSymbolAddress(scratch): %s",
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return PKV_OK;
}

}  // namespace pkv

extern "C" size_t pkv_decode_workspace_bytes(uint32_t num_seqs, uint32_t num_q_heads,
                                             uint32_t num_kv_heads, uint32_t head_dim_v,
                                             uint32_t max_blocks_per_seq, uint32_t block_size,
                                             uint32_t sliding_window, uint32_t split_tokens)
{
    if (!num_seqs || !num_q_heads || !num_kv_heads || !head_dim_v || !max_blocks_per_seq ||
        !block_size)
        return 0;
    // the larger of the two modes' needs (the dtypes, which choose the mode,
    // are not arguments here)
    const size_t a = pkv::make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim_v,
                                    max_blocks_per_seq, block_size, sliding_window, split_tokens,
                                    false).workspace;
    const size_t b = pkv::make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim_v,
                                    max_blocks_per_seq, block_size, sliding_window, split_tokens,
                                    true).workspace;
    return a > b ? a : b;
}

namespace pkv {

// The decode call; with `static_scratch` the split partials go to the
// library's device scratch instead of `workspace` (which is then ignored).
static int paged_decode(const void* q, pkv_dtype q_dtype, uint64_t q_seq_stride,
                        const void* k_cache, pkv_dtype k_dtype, float k_scale,
                        const void* v_cache, pkv_dtype v_dtype, float v_scale,
                        float sparse_v_threshold, const int32_t* block_tables,
                        uint32_t max_blocks_per_seq, const int32_t* seq_lens, uint32_t num_seqs, uint32_t num_blocks,
                        uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim_qk,
                        uint32_t head_dim_v, uint32_t block_size, float scale,
                        uint32_t sliding_window, const float* sinks, int q_rope,
                        float q_rope_theta, uint32_t q_rope_offset, uint32_t q_rope_dim,
                        const float* gate, float* out, uint32_t split_tokens, void* workspace,
                        size_t workspace_bytes, bool static_scratch, void* stream)
{
    clear_error();
    if (num_seqs == 0)
        return PKV_OK;
    if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !out)
        return fail(PKV_ERR_INVALID, "paged_decode_attn: q, caches, block_tables, seq_lens and out must be non-NULL");
    if (!valid_dtype(q_dtype) || !valid_dtype(k_dtype) || !(valid_dtype(v_dtype) || is_tq(v_dtype)))
        return fail(PKV_ERR_INVALID, "paged_decode_attn: bad dtype");
    if (!num_q_heads || !num_kv_heads || !head_dim_qk || !head_dim_v || !max_blocks_per_seq ||
        !num_blocks || !block_size)
        return fail(PKV_ERR_INVALID, "paged_decode_attn: zero dimension");
    if (num_q_heads % num_kv_heads)
        return fail(PKV_ERR_INVALID, "paged_decode_attn: num_q_heads %% num_kv_heads != 0");
    if (block_size != (uint32_t)kBS)
        return fail(PKV_ERR_UNSUPPORTED, "paged_decode_attn: block_size must be 16");
    if (q_seq_stride < (uint64_t)num_q_heads * head_dim_qk)
        return fail(PKV_ERR_INVALID, "paged_decode_attn: q_seq_stride smaller than a query row");
    const uint32_t G = num_q_heads / num_kv_heads;
    const bool mfma_path = q_dtype == PKV_BF16 &&
                           (k_dtype == PKV_BF16 || k_dtype == PKV_FP8_E4M3) &&
                           (v_dtype == PKV_BF16 || v_dtype == PKV_FP8_E4M3 || is_tq(v_dtype));
    if (is_tq(v_dtype) && (head_dim_qk != 128 || head_dim_v != 128))
        return fail(PKV_ERR_UNSUPPORTED, "paged_decode_attn: TQ V needs head_dim 128");
    const bool f32_path = q_dtype == PKV_FP32 && k_dtype == PKV_FP32 && v_dtype == PKV_FP32;
    if (!mfma_path && !f32_path)
        return fail(PKV_ERR_UNSUPPORTED, "paged_decode_attn: dtypes (q,K,V) must be (BF16, BF16|E4M3, BF16|E4M3) or (FP32,FP32,FP32)");
    if ((q_seq_stride * dtype_size(q_dtype)) % 16 || !aligned16(q) || !aligned16(k_cache) ||
        !aligned16(v_cache) || !aligned16(out) || (gate && !aligned16(gate)))
        return fail(PKV_ERR_UNSUPPORTED, "paged_decode_attn: pointers and q stride must be 16-byte aligned");
    if (!(scale > 0.0f && scale < INFINITY))
        return fail(PKV_ERR_INVALID, "paged_decode_attn: scale must be finite and > 0");
    if (k_dtype == PKV_FP8_E4M3 && !(k_scale > 0.0f && k_scale < INFINITY))
        return fail(PKV_ERR_INVALID, "paged_decode_attn: k_scale must be finite and > 0");
    if (v_dtype == PKV_FP8_E4M3 && !(v_scale > 0.0f && v_scale < INFINITY))
        return fail(PKV_ERR_INVALID, "paged_decode_attn: v_scale must be finite and > 0");
    if (!(sparse_v_threshold >= 0.0f && sparse_v_threshold < 1.0f))
        return fail(PKV_ERR_INVALID, "paged_decode_attn: sparse_v_threshold must be in [0, 1)");
    if (sparse_v_threshold > 0.0f && !is_tq(v_dtype))
        return fail(PKV_ERR_UNSUPPORTED, "paged_decode_attn: the sparse-V skip is for TQ V caches");
    if (q_rope && q_rope_dim > 0) {
        if (!f32_path)
            return fail(PKV_ERR_UNSUPPORTED, "paged_decode_attn: query rotation is supported for FP32 q/K/V");
        if (q_rope_dim % 2 || (uint64_t)q_rope_offset + q_rope_dim > head_dim_qk)
            return fail(PKV_ERR_INVALID, "paged_decode_attn: q_rope_dim must be even and fit the head");
    }
    if (mfma_path) {
        if (head_dim_qk != head_dim_v || (head_dim_qk != 64 && head_dim_qk != 128))
            return fail(PKV_ERR_UNSUPPORTED, "paged_decode_attn: BF16/E4M3 caches need head_dim_qk == head_dim_v in {64,128}");
        if (G > 16)
            return fail(PKV_ERR_UNSUPPORTED, "paged_decode_attn: GQA group above 16");
    } else {
        if ((head_dim_qk != 64 && head_dim_qk != 128 && head_dim_qk != 192 && head_dim_qk != 256) ||
            (head_dim_v != 64 && head_dim_v != 128))
            return fail(PKV_ERR_UNSUPPORTED, "paged_decode_attn: FP32 path needs head_dim_qk in {64,128,192,256}, head_dim_v in {64,128}");
        if (G != 1 && G != 2 && G != 4 && G != 8)
            return fail(PKV_ERR_UNSUPPORTED, "paged_decode_attn: FP32 path needs a GQA group of 1, 2, 4 or 8");
    }
    const Plan plan = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim_v,
                                max_blocks_per_seq, block_size, sliding_window, split_tokens,
                                mfma_path);
    if (static_scratch) {
        workspace = nullptr;
        workspace_bytes = 0;
        if (plan.workspace > PKV_DECODE_SCRATCH_BYTES)
            return fail(PKV_ERR_WORKSPACE, "paged_decode_attn_noalloc: the split partials need %zu bytes, the "
                        "library's scratch holds %zu; call pkv_paged_decode_attn with a workspace",
                        plan.workspace, (size_t)PKV_DECODE_SCRATCH_BYTES);
    }
    // the remaining checks need no device; the scratch address is looked up
    // only once they have passed
    if (!static_scratch && plan.workspace > 0 && (workspace_bytes < plan.workspace || !workspace))
        return fail(PKV_ERR_WORKSPACE, "paged_decode_attn: workspace of %zu bytes needed, %zu given",
                    plan.workspace, workspace_bytes);
    if (plan.workspace > 0 && !aligned16(workspace))
        return fail(PKV_ERR_UNSUPPORTED, "paged_decode_attn: workspace must be 16-byte aligned");
    // the split index is a grid dimension (y, or z on the FP32 path, which
    // also puts the sequence in y): both are limited to 65535
    if (!plan.ranges && plan.max_splits > 65535u)
        return fail(PKV_ERR_UNSUPPORTED, "paged_decode_attn: %u splits per sequence (limit 65535); use a larger split_tokens",
                    plan.max_splits);
    if (!mfma_path && num_seqs > 65535u)
        return fail(PKV_ERR_UNSUPPORTED, "paged_decode_attn: FP32 caches support at most 65535 sequences per call");
    if (mfma_path && ((uint64_t)num_seqs * num_kv_heads > 0x7FFFFFFFull ||
                      (uint64_t)plan.ranges * num_kv_heads > 0x7FFFFFFFull))
        return fail(PKV_ERR_UNSUPPORTED, "paged_decode_attn: too many sequences for one call");
    if (static_scratch && plan.workspace > 0) {
        const int rc = scratch_address((hipStream_t)stream, &workspace);
        if (rc)
            return rc;
        workspace_bytes = PKV_DECODE_SCRATCH_BYTES;
    }

    DecodeArgs a{};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.bt = block_tables;
    a.seq_lens = seq_lens;
    a.gate = gate;
    a.sinks = sinks;
    a.out = out;
    a.part_o = (float*)workspace;
    const size_t part_rows = plan.ranges ? (size_t)plan.ranges + num_seqs
                                         : (size_t)num_seqs * plan.max_splits;
    a.part_ml = plan.workspace ? (float*)workspace + part_rows * num_q_heads * head_dim_v : nullptr;
    a.S = num_seqs;
    a.ranges = plan.ranges;
    a.cu = plan.ranges > 1 ? (uint32_t*)(a.part_ml + part_rows * num_q_heads * 2) : nullptr;
    a.q_stride = q_seq_stride;
    a.M = max_blocks_per_seq;
    a.num_blocks = num_blocks;
    a.Hq = num_q_heads;
    a.Hkv = num_kv_heads;
    a.G = G;
    a.chunk_blocks = plan.chunk_blocks;
    a.max_splits = plan.max_splits;
    a.qk_scale = scale * kLog2e * (k_dtype == PKV_FP8_E4M3 ? k_scale : 1.0f);
    // E4M3 and TQ V: the FP16 weights carry 2^15 (divided out here)
    a.out_scale = v_dtype == PKV_FP8_E4M3 ? v_scale / 32768.f : 1.0f;
    a.window = sliding_window;
    if (is_tq(v_dtype)) {
        const TqCodebook& book = tq_codebook(tq_bits(v_dtype));
        for (int i = 0; i < 4; ++i)
            a.tq_f16[i] = book.f16_lut[i];
        a.out_scale = 1.f / 32768.f;          // the 2^15 on the FP16 weights
        a.spv_thr = sparse_v_threshold * 32768.f;   // exact: a power-of-two factor
        a.v_blk_bytes = (uint32_t)tq_block_bytes(book.bits, kBS, num_kv_heads, head_dim_v);
    }
    a.q_rope = (q_rope && q_rope_dim > 0) ? 1u : 0u;
    a.q_rope_theta = q_rope_theta;
    a.q_rope_offset = q_rope_offset;
    a.q_rope_dim = q_rope_dim;
    for (uint32_t i = 0; i < 128; ++i)
        a.q_invf[i] = a.q_rope && i < q_rope_dim / 2
                          ? (float)std::pow((double)q_rope_theta, -(2.0 * (double)i) / (double)q_rope_dim)
                          : 0.f;
    hipStream_t st = (hipStream_t)stream;

    if (mfma_path) {
        uint32_t kvpb = kKvPerGroup;
        while (num_kv_heads % kvpb)
            kvpb >>= 1;
        const uint32_t kvg = num_kv_heads / kvpb;
        // balanced mode: range-major, the kv groups of a range side by side
        const dim3 grid = plan.ranges ? dim3(plan.ranges * kvg, 1) : dim3(num_seqs * kvg, plan.max_splits);
        const dim3 block(64 * kvpb);
        const int kt = k_dtype == PKV_FP8_E4M3;
        const int vt = is_tq(v_dtype) ? tq_bits(v_dtype) : v_dtype == PKV_FP8_E4M3;
#define PKV_MFMA_B(KT, VT, D, BAL, SPV)                                                         \
    if (kt == KT && vt == VT && head_dim_qk == D && bal == BAL && spv == SPV)                  \
        hipLaunchKernelGGL((decode_mfma_kernel<KT, VT, D, kPrefetch, BAL, SPV>), grid, block, 0, st, a, kvg);
#define PKV_MFMA(KT, VT, D) PKV_MFMA_B(KT, VT, D, false, false) PKV_MFMA_B(KT, VT, D, true, false)
#define PKV_MFMA_TQ(KT, VT)                                                                     \
    PKV_MFMA(KT, VT, 128) PKV_MFMA_B(KT, VT, 128, false, true) PKV_MFMA_B(KT, VT, 128, true, true)
        const bool bal = plan.ranges != 0;
        const bool spv = sparse_v_threshold > 0.0f;
        PKV_MFMA(0, 0, 128) PKV_MFMA(0, 0, 64) PKV_MFMA(1, 0, 128) PKV_MFMA(1, 0, 64)
        PKV_MFMA(0, 1, 128) PKV_MFMA(0, 1, 64) PKV_MFMA(1, 1, 128) PKV_MFMA(1, 1, 64)
        PKV_MFMA_TQ(0, 2) PKV_MFMA_TQ(0, 3) PKV_MFMA_TQ(0, 4)
        PKV_MFMA_TQ(1, 2) PKV_MFMA_TQ(1, 3) PKV_MFMA_TQ(1, 4)
#undef PKV_MFMA_TQ
#undef PKV_MFMA
#undef PKV_MFMA_B
    } else {
        const dim3 grid(num_kv_heads, num_seqs, plan.max_splits);
#define PKV_F32(DQK, DV, GG)                                                              \
    if (head_dim_qk == DQK && head_dim_v == DV && G == GG)                                \
        hipLaunchKernelGGL((decode_f32_kernel<DQK, DV, GG>), grid, dim3(64), 0, st, a);
#define PKV_F32_G(DQK, DV) PKV_F32(DQK, DV, 1) PKV_F32(DQK, DV, 2) PKV_F32(DQK, DV, 4) PKV_F32(DQK, DV, 8)
        PKV_F32_G(64, 64) PKV_F32_G(128, 64) PKV_F32_G(192, 64) PKV_F32_G(256, 64)
        PKV_F32_G(64, 128) PKV_F32_G(128, 128) PKV_F32_G(192, 128) PKV_F32_G(256, 128)
#undef PKV_F32_G
#undef PKV_F32
    }
    int rc = check_launch("paged_decode_attn");
    if (rc)
        return rc;
    if (plan.ranges || plan.max_splits > 1) {
        const dim3 mgrid(num_seqs, ceil_div(num_q_heads, kMergeHeads));
        if (head_dim_v == 128)
            hipLaunchKernelGGL(decode_merge_kernel<2>, mgrid, dim3(64 * kMergeHeads), 0, st, a);
        else
            hipLaunchKernelGGL(decode_merge_kernel<1>, mgrid, dim3(64 * kMergeHeads), 0, st, a);
        rc = check_launch("paged_decode_attn merge");
    }
    return rc;
}

}  // namespace pkv

extern "C" int pkv_paged_decode_attn(const void* q, pkv_dtype q_dtype, uint64_t q_seq_stride,
                                     const void* k_cache, pkv_dtype k_dtype, float k_scale,
                                     const void* v_cache, pkv_dtype v_dtype, float v_scale,
                                     float sparse_v_threshold,
                                     const int32_t* block_tables, uint32_t max_blocks_per_seq,
                                     const int32_t* seq_lens, uint32_t num_seqs,
                                     uint32_t num_blocks, uint32_t num_q_heads,
                                     uint32_t num_kv_heads, uint32_t head_dim_qk,
                                     uint32_t head_dim_v, uint32_t block_size, float scale,
                                     uint32_t sliding_window, const float* sinks,
                                     int q_rope, float q_rope_theta, uint32_t q_rope_offset,
                                     uint32_t q_rope_dim, const float* gate, float* out,
                                     uint32_t split_tokens, void* workspace,
                                     size_t workspace_bytes, void* stream)
{
    return pkv::paged_decode(q, q_dtype, q_seq_stride, k_cache, k_dtype, k_scale, v_cache,
                             v_dtype, v_scale, sparse_v_threshold, block_tables,
                             max_blocks_per_seq, seq_lens,
                             num_seqs, num_blocks, num_q_heads, num_kv_heads, head_dim_qk,
                             head_dim_v, block_size, scale, sliding_window, sinks, q_rope,
                             q_rope_theta, q_rope_offset, q_rope_dim, gate, out, split_tokens,
                             workspace, workspace_bytes, false, stream);
}

extern "C" int pkv_paged_decode_attn_noalloc(
    const void* q, pkv_dtype q_dtype, uint64_t q_seq_stride, const void* k_cache,
    pkv_dtype k_dtype, float k_scale, const void* v_cache, pkv_dtype v_dtype, float v_scale,
    float sparse_v_threshold, const int32_t* block_tables, uint32_t max_blocks_per_seq,
    const int32_t* seq_lens,
    uint32_t num_seqs, uint32_t num_blocks, uint32_t num_q_heads, uint32_t num_kv_heads,
    uint32_t head_dim_qk, uint32_t head_dim_v, uint32_t block_size, float scale,
    uint32_t sliding_window, const float* sinks, int q_rope, float q_rope_theta,
    uint32_t q_rope_offset, uint32_t q_rope_dim, const float* gate, float* out,
    uint32_t split_tokens, void* stream)
{
    return pkv::paged_decode(q, q_dtype, q_seq_stride, k_cache, k_dtype, k_scale, v_cache,
                             v_dtype, v_scale, sparse_v_threshold, block_tables,
                             max_blocks_per_seq, seq_lens,
                             num_seqs, num_blocks, num_q_heads, num_kv_heads, head_dim_qk,
                             head_dim_v, block_size, scale, sliding_window, sinks, q_rope,
                             q_rope_theta, q_rope_offset, q_rope_dim, gate, out, split_tokens,
                             nullptr, 0, true, stream);
}

// prefill_attn.hip -- pkv_paged_prefill_attn: causal attention of the N new
// tokens of every sequence over its paged KV cache (page 1, kv_cache.rs,
// the section on batched prefill variants of the paged kernels over N
// tokens; the reading:
// the q_len queries of a sequence are its last q_len tokens, already written
// to the cache, and query i at position p = seq_len - q_len + i attends to
// [lo, p], lo from the sliding window as in decode; sinks as in decode).
//
// Work decomposition.  Rows of the score matrix are (query token, query
// head) pairs of one kv head's GQA group, token-major (row = i * G + g).  A
// work-group takes 128 consecutive rows of one (sequence, kv head), four
// wavefronts of two 16-row tiles each, and walks the keys [lo_min, end_max)
// of its rows in steps of four cache blocks (two pairs).  Each step's K and V blocks are
// loaded once per work-group (one 16-byte chunk of each per thread and
// block), written to LDS -- K in the swizzled MFMA operand layout of KFrag, V
// row-major with a 16-byte pad per row -- and read by all four waves; the
// next step's loads are in flight while the current one is computed (two LDS
// buffers, one barrier per step).  Per wave, step and row tile:
//   S^T[t, row] = K[t, :] . q[row, :]   v_mfma_f32_16x16x32_bf16 (M=t, N=row),
//                                       per block
//   O[row, d]  += P[row, t] V[t, d]     v_mfma_f32_16x16x32_bf16 whose k spans
//                                       the two blocks' keys, once with the hi
//                                       and once with the lo BF16 halves of P
// with the causal / window mask per row and online softmax in the log2
// domain, as in decode.  All query tiles of one (sequence, kv head) are
// dealt to the same XCD (work-group id % 8), so their repeated K/V reads
// are served by that XCD's L2.
#include "attn_common.h"

namespace pkv {

constexpr int kPWaves = 4;                   // waves per work-group
// cache blocks per step (pairs of blocks, each pair one PV k span): four
// halve the barriers of two (612 against 592 TFLOP/s on the chunk-256
// workload); eight need 256 VGPRs, one wave per SIMD (397)
constexpr int kPStep = 4;
constexpr int kPPre = 1;                     // steps whose loads are in flight
constexpr int kPTiles = 2;                   // 16-row tiles per wave
constexpr int kXcds = 8;                     // XCDs work-groups are dealt to
// A row's exponent reference moves only when its running max passes it by
// more than this (log2 units): weights stay below 2^8, exact in the BF16
// hi + lo split and in FP32, and the O rescale becomes rare.
constexpr float kLazyRescale = 8.0f;

struct PrefillArgs {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* cu_q;
    const int32_t* bt;
    const int32_t* seq_lens;
    const float* sinks;
    float* out;
    uint64_t q_stride;      // elements between query tokens
    uint32_t total_q;       // rows of q and out
    uint32_t M;             // max_blocks_per_seq
    uint32_t num_blocks;
    uint32_t Hq, Hkv, G;
    uint32_t tiles;         // query tiles per (sequence, kv head) in the grid
    uint32_t units;         // num_seqs * Hkv
    float qk_scale;         // scale * log2(e) (* k_scale for E4M3 K)
    float out_scale;        // v_scale for E4M3 V, else 1
    uint32_t window;
};

__device__ __forceinline__ int32_t window_lo(uint32_t window, int32_t end)
{
    return (window > 0 && end > (int32_t)window) ? end - (int32_t)window : 0;
}

// NW waves of RT x 16 query rows, STEP cache blocks per step, PF steps of
// loads in flight (a ring of register stages; loads are unconditional --
// steps past the range re-read block 0 -- so the compiler's wait before a
// stage's LDS write covers that stage only).  A wave's RT row tiles share
// every K operand read from LDS and every V operand built from it.
// The block table is a restrict parameter of its own: its wave-uniform
// entries are then read through the scalar cache, and waiting for them does
// not drain the vector loads in flight.
template <int KT, int VT, int D, int NW, int STEP, int PF, int RT>
__global__ __launch_bounds__(64 * NW) void prefill_mfma_kernel(PrefillArgs a,
                                                               const int32_t* __restrict__ bt)
{
    using KF = KFrag<KT, D>;
    constexpr int kWRows = 16 * RT;                    // query rows per wave
    constexpr int kPRows = kWRows * NW;                // ... per work-group
    constexpr int kPThreads = 64 * NW;
    constexpr int kPStep = STEP;
    constexpr int NI = KF::NI, NL = KF::NL;
    constexpr int CPR = KF::CPR;                       // K chunks per row
    constexpr uint32_t KES = KT == 0 ? 2 : 1;
    constexpr uint32_t VES = VT == 0 ? 2 : 1;
    constexpr int NT = D / 16;                         // PV N-tiles
    constexpr int DPL = D / 16;                        // V columns per lane
    constexpr int VW = DPL * VES / 4;                  // V words per lane per row
    constexpr int VCPR = D * VES / 16;                 // V chunks per row
    constexpr int KTILE = 16 * CPR * 16;               // bytes of a K tile
    constexpr int VROW = D * VES + 16;                 // padded V row in LDS
    constexpr int VTILE = 16 * VROW;
    constexpr int BLK = KTILE + VTILE;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][kPStep][BLK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform (scalar) so that every wave-level bound and block test
    // below is a scalar value and its branches are uniform
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = lane >> 4;
    const int ln = lane & 15;

    // work-group -> (unit, tile): the tiles of a unit share id % 8 (one XCD)
    const uint32_t xcd = blockIdx.x % kXcds, k = blockIdx.x / kXcds;
    const uint32_t unit = xcd + kXcds * (k / a.tiles);
    const uint32_t tile = k % a.tiles;
    if (unit >= a.units)
        return;
    const uint32_t s = unit / a.Hkv, kvh = unit % a.Hkv;
    const int32_t q0 = a.cu_q[s];
    const int32_t qlen = a.cu_q[s + 1] - q0;
    const uint32_t G = a.G;
    const uint32_t row0 = tile * kPRows;
    if (qlen <= 0 || (uint64_t)row0 >= (uint64_t)qlen * G)
        return;
    const int32_t n = a.seq_lens[s];
    const int32_t first_pos = n - qlen;                // position of query 0

    // this lane's rows (S^T columns), one per row tile: query token, head
    const uint32_t wrow0 = row0 + kWRows * wave;
    int32_t end_r[RT], lo_r[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const uint32_t row = wrow0 + 16 * t + ln;
        const int32_t qi = (int32_t)(row / G);
        const bool ok = qi < qlen && (uint32_t)(q0 + qi) < a.total_q;
        end_r[t] = ok ? first_pos + qi + 1 : 0;      // keys [lo_r, end_r)
        lo_r[t] = window_lo(a.window, end_r[t]);
    }

    // key range of the work-group and of this wave (rows are token-major)
    const int32_t i_lo = (int32_t)(row0 / G);
    const int32_t i_hi = min(qlen, (int32_t)((row0 + kPRows + G - 1) / G)) - 1;
    const int32_t end_max = first_pos + i_hi + 1;
    const int32_t lo_min = window_lo(a.window, first_pos + i_lo + 1);
    const int32_t wi_lo = (int32_t)(wrow0 / G);
    const int32_t wi_hi = min(qlen, (int32_t)((wrow0 + kWRows + G - 1) / G)) - 1;
    const bool wave_live = wi_lo <= wi_hi;
    const int32_t w_end = first_pos + wi_hi + 1;
    const int32_t w_lo = window_lo(a.window, first_pos + wi_lo + 1);
    // keys every row of the wave attends to: [in_lo, in_end)
    const int32_t in_end = first_pos + wi_lo + 1;
    const int32_t in_lo = window_lo(a.window, w_end);

    uint32_t nblk = 0, blo = 0;
    if (end_max > 0) {
        nblk = min(((uint32_t)end_max + kBS - 1) / kBS, a.M);
        blo = (uint32_t)max(lo_min, 0) / kBS;
    }

    // q fragments (B operand of S^T = K q^T): lane (row ln, kg), per row tile
    bf16x8 qf[RT][NI];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const uint32_t row = wrow0 + 16 * t + ln;
        const int32_t qi = (int32_t)(row / G);
        const uint16_t* qrow = (const uint16_t*)a.q + (uint64_t)(q0 + qi) * a.q_stride +
                               (uint64_t)(kvh * G + row % G) * D;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            u32x4 w = u32x4{0u, 0u, 0u, 0u};
            if (qi < qlen && (uint32_t)(q0 + qi) < a.total_q)
                w = *(const u32x4*)(qrow + KF::phys(i, kg));
            qf[t][i] = __builtin_bit_cast(bf16x8, w);
        }
    }

    f32x4 o[RT][NT];
    float m[RT], l[RT], neg_m[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            o[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[t] = -INFINITY;
        neg_m[t] = 0.f;                                // -m, 0 while m is -inf
        l[t] = 0.f;
    }

    // cooperative loads: thread tid owns K chunk tid and V chunk tid of each
    // block of a step (16 rows x CPR / VCPR chunks)
    const uint8_t* kbase = (const uint8_t*)a.k_cache;
    const uint8_t* vbase = (const uint8_t*)a.v_cache;
    const uint64_t krow_bytes = (uint64_t)a.Hkv * D * KES;
    const uint64_t vrow_bytes = (uint64_t)a.Hkv * D * VES;
    // K chunks on threads [0, 16 CPR), V chunks on the next 16 VCPR threads
    // when the work-group has that many, else on threads [0, 16 VCPR) too
    // (every thread loads -- threads past the chunk count re-load a chunk and
    // do not store it -- so the loads are not behind an exec-mask branch)
    constexpr int V_FIRST = 16 * CPR + 16 * VCPR <= kPThreads ? 16 * CPR : 0;
    const int vtid = tid - V_FIRST;
    const bool k_loader = tid < 16 * CPR, v_loader = vtid >= 0 && vtid < 16 * VCPR;
    const uint32_t kt_ = (uint32_t)tid % (16 * CPR);
    const uint32_t vt_ = (uint32_t)(vtid + kPThreads) % (16 * VCPR);
    const uint32_t k_r = kt_ / CPR, k_c = kt_ % CPR;
    const uint32_t v_r = vt_ / VCPR, v_c = vt_ % VCPR;
    const uint64_t k_off = k_r * krow_bytes + (uint64_t)kvh * D * KES + 16u * k_c;
    const uint64_t v_off = v_r * vrow_bytes + (uint64_t)kvh * D * VES + 16u * v_c;
    const uint32_t k_lds = KF::lds_off(k_r, k_c);
    const uint32_t v_lds = KTILE + v_r * VROW + 16u * v_c;

    struct Stage {
        u32x4 k[kPStep], v[kPStep];
    };
    auto block_id = [&](uint32_t b) -> int32_t {
        const int32_t pb = b < nblk ? bt[(uint64_t)s * a.M + b] : -1;
        return pb;
    };
    // an unmapped block (or one past the range) is read from block 0 and masked
    auto load_step = [&](uint32_t b0, Stage& st) {
#pragma unroll
        for (int j = 0; j < kPStep; ++j) {
            int32_t pb = block_id(b0 + j);
            pb = (pb >= 0 && (uint32_t)pb < a.num_blocks) ? pb : 0;
            const uint64_t blk = (uint64_t)pb * kBS;
            // ordinary (cached) loads: the other query tiles of this (sequence,
            // kv head), on the same XCD, read the same blocks from its L2
            st.k[j] = *(const u32x4*)(kbase + blk * krow_bytes + k_off);
            st.v[j] = *(const u32x4*)(vbase + blk * vrow_bytes + v_off);
        }
    };
    auto store_step = [&](int buf, const Stage& st) {
#pragma unroll
        for (int j = 0; j < kPStep; ++j) {
            if (k_loader)
                *(u32x4*)&lds[buf][j][k_lds] = st.k[j];
            if (v_loader)
                *(u32x4*)&lds[buf][j][v_lds] = st.v[j];
        }
    };

    // LDS read positions: K operand chunk of MFMA group jj; V rows 4kg + r
    uint32_t lds_r[NL];
#pragma unroll
    for (int jj = 0; jj < NL; ++jj)
        lds_r[jj] = KF::lds_off(ln, KF::op_chunk(jj, kg));
    const uint32_t v_rd = KTILE + (4 * kg) * VROW + DPL * ln * VES;

    static_assert(kPStep % 2 == 0, "a step is whole pairs of blocks along the PV k");
    // one pair of blocks (j0, j0 + 1 of the step's LDS buffer)
    auto compute_pair = [&](int buf, int j0, uint32_t b0) {
        if (!wave_live)
            return;
        bool blk_ok[2], inner[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t b = b0 + j;
            const int32_t t0 = (int32_t)(b * kBS);
            const int32_t pb = block_id(b);
            blk_ok[j] = b < nblk && pb >= 0 && (uint32_t)pb < a.num_blocks && t0 < w_end &&
                        t0 + kBS > w_lo;
            // a block wholly inside every row's [lo, end) needs no mask
            inner[j] = blk_ok[j] && t0 >= in_lo && t0 + kBS <= in_end;
        }
        // a step with no attended key leaves m, l and o as they are
        if (!(blk_ok[0] | blk_ok[1]))
            return;

        // S^T = K q^T for both blocks and row tiles.  Both blocks are in LDS
        // (an unmapped one was read from block 0), so the MFMAs run
        // unconditionally; masking below drops the scores not attended.
        f32x4 sacc[RT][2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int t = 0; t < RT; ++t)
                sacc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            const uint8_t* kt = &lds[buf][j0 + j][0];
            u32x4 kop[NL];
#pragma unroll
            for (int jj = 0; jj < NL; ++jj)
                kop[jj] = *(const u32x4*)(kt + lds_r[jj]);
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const bf16x8 kf = KF::operand(kop, i);
#pragma unroll
                for (int t = 0; t < RT; ++t)
                    sacc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[t][i], sacc[t][j],
                                                                         0, 0, 0);
            }
        }

        // online softmax, part 1, per row tile: masks, row max, rescale.  The
        // lane holds row ln of tile t and keys (b0 + j) * 16 + 4kg + r; raw
        // scores, masked ones -inf (the scale is applied inside the exponent's
        // FMA and to the row max: scale > 0 keeps the order)
        float sr[RT][2][4];
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if (inner[j]) {                          // wave-uniform
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sr[t][j][r] = sacc[t][j][r];
                } else {
                    const int32_t tk = (int32_t)((b0 + j) * kBS) + 4 * kg;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        // bitwise &: no short-circuit control flow per element
                        const bool ok = blk_ok[j] & (tk + r >= lo_r[t]) & (tk + r < end_r[t]);
                        sr[t][j][r] = ok ? sacc[t][j][r] : -INFINITY;
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    mx = fmaxf(mx, sr[t][j][r]);
            }
            // m is the row's exponent reference (-inf until a key counts).  A
            // row's max passes m + kLazyRescale iff one of its 4 lanes' maxima
            // does, so the cross-lane reduction runs only then
            if (__builtin_amdgcn_ballot_w64(mx * a.qk_scale > m[t] + kLazyRescale)) {
                mx = row_max_xor16_32(mx) * a.qk_scale;
                // rows whose reference stays keep alpha = 1 (also when it is
                // -inf: -inf - -inf would be NaN); a first reference gives 0
                const bool move = mx > m[t] + kLazyRescale;
                const float m_new = move ? mx : m[t];
                const float alpha = move ? __builtin_amdgcn_exp2f(m[t] - m_new) : 1.f;
                l[t] *= alpha;
                m[t] = m_new;
                neg_m[t] = m_new == -INFINITY ? 0.f : -m_new;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float ar = __shfl(alpha, 4 * kg + r, 64);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        o[t][nt][r] *= ar;
                }
            }
        }

        // V rows 4kg + r of both blocks.  In a block that is not interior,
        // keys outside [w_lo, w_end) (past the sequence end, or in an unmapped
        // block read from block 0) read as zero
        uint32_t vr[2][4][VW];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint8_t* vt = &lds[buf][j0 + h][0] + v_rd;
            if (inner[h]) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if constexpr (VW == 4) {
                        const u32x4 x = *(const u32x4*)(vt + r * VROW);
#pragma unroll
                        for (int w = 0; w < 4; ++w) vr[h][r][w] = x[w];
                    } else if constexpr (VW == 2) {
                        const u32x2 x = *(const u32x2*)(vt + r * VROW);
#pragma unroll
                        for (int w = 0; w < 2; ++w) vr[h][r][w] = x[w];
                    } else {
                        vr[h][r][0] = *(const uint32_t*)(vt + r * VROW);
                    }
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int32_t tk = (int32_t)((b0 + h) * kBS) + 4 * kg + r;
                    const bool keep = blk_ok[h] & (tk >= w_lo) & (tk < w_end);
                    if constexpr (VW == 4) {
                        const u32x4 x = *(const u32x4*)(vt + r * VROW);
#pragma unroll
                        for (int w = 0; w < 4; ++w) vr[h][r][w] = keep ? x[w] : 0u;
                    } else if constexpr (VW == 2) {
                        const u32x2 x = *(const u32x2*)(vt + r * VROW);
#pragma unroll
                        for (int w = 0; w < 2; ++w) vr[h][r][w] = keep ? x[w] : 0u;
                    } else {
                        const uint32_t x = *(const uint32_t*)(vt + r * VROW);
                        vr[h][r][0] = keep ? x : 0u;
                    }
                }
            }
        }

        // B operand of column tile nt: k = 8kg + 0..3 -> keys 4kg + 0..3 of
        // block 0, k = 8kg + 4..7 -> the same keys of block 1
        auto v_operand = [&](int nt) -> bf16x8 {
            uint32_t bw[4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if constexpr (VT == 1) {
                    // the two rows' codes of column nt side by side, then
                    // widened exactly to a BF16 pair (v_cvt_scalef32_pk_bf16_fp8,
                    // scale 1)
                    const int w = nt / 4, e = nt % 4;
                    const uint32_t sel = e < 2 ? 0x05010400u : 0x07030602u;
                    const uint32_t x01 = __builtin_amdgcn_perm(vr[h][1][w], vr[h][0][w], sel);
                    const uint32_t x23 = __builtin_amdgcn_perm(vr[h][3][w], vr[h][2][w], sel);
                    const bf16x2 p01 = (e & 1) ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x01, 1.0f, true)
                                               : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x01, 1.0f, false);
                    const bf16x2 p23 = (e & 1) ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x23, 1.0f, true)
                                               : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x23, 1.0f, false);
                    bw[2 * h] = __builtin_bit_cast(uint32_t, p01);
                    bw[2 * h + 1] = __builtin_bit_cast(uint32_t, p23);
                } else {
                    const int w = nt >> 1;
                    if (nt & 1) {
                        bw[2 * h] = hi16_pair(vr[h][0][w], vr[h][1][w]);
                        bw[2 * h + 1] = hi16_pair(vr[h][2][w], vr[h][3][w]);
                    } else {
                        bw[2 * h] = lo16_pair(vr[h][0][w], vr[h][1][w]);
                        bw[2 * h + 1] = lo16_pair(vr[h][2][w], vr[h][3][w]);
                    }
                }
            }
            return __builtin_bit_cast(bf16x8, u32x4{bw[0], bw[1], bw[2], bw[3]});
        };
        // P of tile t: weights 2^(s * scale - m), their sum, and the A operands
        // (k as for V) of their hi and lo BF16 halves
        auto p_operands = [&](int t, bf16x8& a_hi, bf16x8& a_lo) {
            uint32_t ph[2][2], pl[2][2];
            float psum;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                float p[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    p[r] = __builtin_amdgcn_exp2f(fmaf(sr[t][j][r], a.qk_scale, neg_m[t]));
                const float bsum = (p[0] + p[1]) + (p[2] + p[3]);
                psum = j == 0 ? bsum : psum + bsum;
#pragma unroll
                for (int r2 = 0; r2 < 2; ++r2) {
                    uint32_t hw = pack_bf16(p[2 * r2], p[2 * r2 + 1]);
                    // an empty asm hides hw's origin, so the low half below is
                    // hw << 16 rather than a second conversion of p[2 * r2]
                    asm("" : "+v"(hw));
                    ph[j][r2] = hw;
                    pl[j][r2] = pack_bf16(p[2 * r2] - bf16_lo(hw), p[2 * r2 + 1] - bf16_hi(hw));
                }
            }
            l[t] += psum;
            a_hi = __builtin_bit_cast(bf16x8, u32x4{ph[0][0], ph[0][1], ph[1][0], ph[1][1]});
            a_lo = __builtin_bit_cast(bf16x8, u32x4{pl[0][0], pl[0][1], pl[1][0], pl[1][1]});
        };
        bf16x8 bv[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            bv[nt] = v_operand(nt);
        bf16x8 a_hi[RT], a_lo[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t)
            p_operands(t, a_hi[t], a_lo[t]);
#pragma unroll
        for (int t = 0; t < RT; ++t) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                o[t][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_hi[t], bv[nt], o[t][nt], 0, 0, 0);
                o[t][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_lo[t], bv[nt], o[t][nt], 0, 0, 0);
            }
        }
    };

    auto compute_step = [&](int buf, uint32_t b0) {
#pragma unroll
        for (int j0 = 0; j0 < kPStep; j0 += 2)
            compute_pair(buf, j0, b0 + j0);
    };

    if (nblk > blo) {
        const uint32_t nsteps = (nblk - blo + kPStep - 1) / kPStep;
        // step j lives in register stage j % PF until it is written to LDS
        // buffer j % 2 at the end of step j - 1
        Stage st[PF];
#pragma unroll
        for (int u = 0; u < PF; ++u)
            load_step(blo + u * kPStep, st[u]);
        store_step(0, st[0]);
        __syncthreads();
        for (uint32_t j0 = 0; j0 < nsteps; j0 += PF) {
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                const uint32_t j = j0 + u;
                if (j >= nsteps)
                    break;
                load_step(blo + (j + PF) * kPStep, st[u]);
                compute_step(j & 1, blo + j * kPStep);
                store_step((j + 1) & 1, st[(u + 1) % PF]);
                __syncthreads();
            }
        }
    }

    // finished rows: o[t][nt][r] is row 4kg + r of tile t, column DPL * ln + nt
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const float lt = row_sum_xor16_32(l[t]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t wr = 4 * kg + r;              // row within the tile
            const float lr = __shfl(lt, (int)wr, 64);
            const float mr = __shfl(m[t], (int)wr, 64);
            const uint32_t orow = wrow0 + 16 * t + wr;
            const int32_t oi = (int32_t)(orow / G);
            if (oi >= qlen || (uint32_t)(q0 + oi) >= a.total_q)
                continue;
            const uint32_t h = kvh * G + orow % G;
            const float inv = norm_factor(mr, lr, a.sinks, h, a.out_scale);
            float* dst = a.out + ((uint64_t)(q0 + oi) * a.Hq + h) * D + (uint64_t)DPL * ln;
#pragma unroll
            for (int nt = 0; nt < NT; nt += 4)
                *(f32x4*)(dst + nt) = f32x4{o[t][nt][r] * inv, o[t][nt + 1][r] * inv,
                                            o[t][nt + 2][r] * inv, o[t][nt + 3][r] * inv};
        }
    }
}

}  // namespace pkv

extern "C" int pkv_paged_prefill_attn(const void* q, pkv_dtype q_dtype, uint64_t q_token_stride,
                                      const int32_t* cu_q, uint32_t max_q_len, uint32_t total_q,
                                      const void* k_cache, pkv_dtype k_dtype, float k_scale,
                                      const void* v_cache, pkv_dtype v_dtype, float v_scale,
                                      const int32_t* block_tables, uint32_t max_blocks_per_seq,
                                      const int32_t* seq_lens, uint32_t num_seqs,
                                      uint32_t num_blocks, uint32_t num_q_heads,
                                      uint32_t num_kv_heads, uint32_t head_dim_qk,
                                      uint32_t head_dim_v, uint32_t block_size, float scale,
                                      uint32_t sliding_window, const float* sinks, float* out,
                                      void* stream)
{
    using namespace pkv;
    clear_error();
    if (num_seqs == 0 || max_q_len == 0 || total_q == 0)
        return PKV_OK;
    if (!q || !cu_q || !k_cache || !v_cache || !block_tables || !seq_lens || !out)
        return fail(PKV_ERR_INVALID, "paged_prefill_attn: q, cu_q, caches, block_tables, seq_lens and out must be non-NULL");
    if (!valid_dtype(q_dtype) || !valid_dtype(k_dtype) || !valid_dtype(v_dtype))
        return fail(PKV_ERR_INVALID, "paged_prefill_attn: bad dtype");
    if (!num_q_heads || !num_kv_heads || !head_dim_qk || !head_dim_v || !max_blocks_per_seq ||
        !num_blocks || !block_size)
        return fail(PKV_ERR_INVALID, "paged_prefill_attn: zero dimension");
    if (num_q_heads % num_kv_heads)
        return fail(PKV_ERR_INVALID, "paged_prefill_attn: num_q_heads %% num_kv_heads != 0");
    if (block_size != (uint32_t)kBS)
        return fail(PKV_ERR_UNSUPPORTED, "paged_prefill_attn: block_size must be 16");
    if (q_token_stride < (uint64_t)num_q_heads * head_dim_qk)
        return fail(PKV_ERR_INVALID, "paged_prefill_attn: q_token_stride smaller than a query row");
    const uint32_t G = num_q_heads / num_kv_heads;
    if (q_dtype != PKV_BF16 || (k_dtype != PKV_BF16 && k_dtype != PKV_FP8_E4M3) ||
        (v_dtype != PKV_BF16 && v_dtype != PKV_FP8_E4M3))
        return fail(PKV_ERR_UNSUPPORTED, "paged_prefill_attn: dtypes (q,K,V) must be (BF16, BF16|E4M3, BF16|E4M3)");
    if (head_dim_qk != head_dim_v || (head_dim_qk != 64 && head_dim_qk != 128))
        return fail(PKV_ERR_UNSUPPORTED, "paged_prefill_attn: head_dim_qk == head_dim_v in {64,128}");
    if (16 % G)
        return fail(PKV_ERR_UNSUPPORTED, "paged_prefill_attn: GQA group must be 1, 2, 4, 8 or 16");
    if ((q_token_stride * 2) % 16 || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
        !aligned16(out))
        return fail(PKV_ERR_UNSUPPORTED, "paged_prefill_attn: pointers and q stride must be 16-byte aligned");
    if (!(scale > 0.0f && scale < INFINITY))
        return fail(PKV_ERR_INVALID, "paged_prefill_attn: scale must be finite and > 0");
    if (k_dtype == PKV_FP8_E4M3 && !(k_scale > 0.0f && k_scale < INFINITY))
        return fail(PKV_ERR_INVALID, "paged_prefill_attn: k_scale must be finite and > 0");
    if (v_dtype == PKV_FP8_E4M3 && !(v_scale > 0.0f && v_scale < INFINITY))
        return fail(PKV_ERR_INVALID, "paged_prefill_attn: v_scale must be finite and > 0");
    constexpr int kPRows = 16 * kPWaves * kPTiles;
    const uint64_t tiles = ((uint64_t)max_q_len * G + kPRows - 1) / kPRows;
    const uint64_t units = (uint64_t)num_seqs * num_kv_heads;
    const uint64_t groups = (units + kXcds - 1) / kXcds * kXcds * tiles;
    if (groups >= (1ull << 31))
        return fail(PKV_ERR_UNSUPPORTED, "paged_prefill_attn: grid too large");

    PrefillArgs a{};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.cu_q = cu_q;
    a.bt = block_tables;
    a.seq_lens = seq_lens;
    a.sinks = sinks;
    a.out = out;
    a.q_stride = q_token_stride;
    a.total_q = total_q;
    a.M = max_blocks_per_seq;
    a.num_blocks = num_blocks;
    a.Hq = num_q_heads;
    a.Hkv = num_kv_heads;
    a.G = G;
    a.tiles = (uint32_t)tiles;
    a.units = (uint32_t)units;
    a.qk_scale = scale * kLog2e * (k_dtype == PKV_FP8_E4M3 ? k_scale : 1.0f);
    a.out_scale = v_dtype == PKV_FP8_E4M3 ? v_scale : 1.0f;
    a.window = sliding_window;
    hipStream_t st = (hipStream_t)stream;
    const int kt = k_dtype == PKV_FP8_E4M3, vt = v_dtype == PKV_FP8_E4M3;
    const dim3 grid((uint32_t)groups), block(64 * kPWaves);
#define PKV_PREFILL(KT, VT, D)                                                                  \
    if (kt == KT && vt == VT && head_dim_qk == D)                                              \
        hipLaunchKernelGGL((prefill_mfma_kernel<KT, VT, D, kPWaves, kPStep, kPPre, kPTiles>),  \
                           grid, block, 0, st, a, block_tables);
    PKV_PREFILL(0, 0, 128) PKV_PREFILL(0, 0, 64) PKV_PREFILL(1, 0, 128) PKV_PREFILL(1, 0, 64)
    PKV_PREFILL(0, 1, 128) PKV_PREFILL(0, 1, 64) PKV_PREFILL(1, 1, 128) PKV_PREFILL(1, 1, 64)
#undef PKV_PREFILL
    return check_launch("paged_prefill_attn");
}

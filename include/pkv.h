/*
 * pkv.h -- C ABI of libpkv: paged KV-cache write and paged decode attention
 * for AMD Instinct MI355X (gfx950).
 *
 * Six operations, each an asynchronous launch on a caller-given HIP stream:
 *
 *   pkv_fill_slots          slot mapping from per-sequence block tables
 *   pkv_cache_write_k_fused RMSNorm -> RoPE -> one rounding, into the K pool
 *   pkv_cache_write_v       V reshape-and-cache copy (or E4M3 / TurboQuant-style
 *                           b-bit store) into the V pool
 *   pkv_paged_decode_attn   one-query-token GQA attention through the tables
 *   pkv_paged_decode_attn_noalloc  the same, its split partials in a device
 *                           scratch of the library (for callers that cannot
 *                           allocate)
 *   pkv_paged_prefill_attn  causal attention of N new tokens per sequence
 *   pkv_mla_cache_assemble  MLA cache rows [latent | k_rope] -> K, [latent | 0] -> V
 *
 * and host-side queries: pkv_decode_workspace_bytes, pkv_v_block_bytes,
 * pkv_tq_codebook, pkv_last_error, pkv_version.
 *
 * Sources (the pages this library implements):
 *   [p1] docs.atlasinference.io, spark_model/layers/ops/kv_cache.rs
 *   [p2] docs.metrale.ai, metrale_model_layers/layers/ops/kv_cache_fp8k.rs
 *   [p3] docs.atlascybernetics.ai, spark_model/kimi_k3/mla_cuda.rs
 *
 * Conventions shared by every call
 * --------------------------------
 * Pointers.  Every array argument is DEVICE memory owned by the caller (for
 *   example a torch tensor's data pointer).  The library never allocates,
 *   frees, copies between host and device, synchronises, or keeps state
 *   between calls (pkv_paged_decode_attn_noalloc excepted: it keeps one
 *   device scratch array per GPU, allocated with the code object).  `stream` is a hipStream_t (NULL = the null stream).
 * Pool layout ("NHD"), [p1] doc of reshape_and_cache_fp8 and [p2] module
 *   invariants: a pool is [num_blocks, block_size, num_kv_heads, head_dim],
 *   row-major, addressed from its base.  A slot is a flat row index
 *   slot = block * block_size + offset; element (slot, h, d) sits at
 *   (slot * num_kv_heads + h) * head_dim + d.
 * Status.  0 on success.  A negative code is returned, before anything is
 *   launched, for arguments the host can check; pkv_last_error() then gives
 *   a message (thread-local, valid until the next call on that thread):
 *     PKV_ERR_INVALID     (-1) NULL pointer, zero dimension, bad dtype enum,
 *                              inconsistent sizes
 *     PKV_ERR_UNSUPPORTED (-2) a shape/dtype/alignment outside the supported
 *                              set listed at each call
 *     PKV_ERR_WORKSPACE   (-3) workspace smaller than required
 *     PKV_ERR_HIP         (-4) the launch itself failed (HIP error text)
 *   A call with no work (zero tokens or sequences) returns 0 and launches
 *   nothing ([p1] fill_slots_from_block_table returns early on count 0).
 * Device-side conditions are defined behaviour, not errors: a negative slot
 *   or one past the pool is skipped by the writes; a block-table entry
 *   outside [0, num_blocks) excludes its tokens from attention; seq_len <= 0
 *   gives an all-zero output row; table entries past ceil(seq_len /
 *   block_size), and those wholly before a sliding window, are never read.
 * Alignment.  Cache rows and input rows are read and written in 16-byte
 *   pieces: every data pointer and every row stride (in bytes) must be a
 *   multiple of 16, else PKV_ERR_UNSUPPORTED.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  PKV_FP8_E4M3 is OCP FP8 E4M3FN (bias 7, no infinities,
 * largest finite 448), the "FP8 E4M3" of [p1] and [p2].
 * PKV_TQ2 / TQ3 / TQ4 are V cache formats only: the TurboQuant-style V of
 * [p1] reshape_and_cache_bf16k_turbo{2,3,4}v and [p2] (b-bit Lloyd-Max codes
 * plus one FP8 scale per 16 elements, with a norm correction).  The pages
 * give no more; the format taken here:
 *   - codebook: the 2^b Lloyd-Max levels of the standard normal
 *     distribution, rounded to E4M3; code = sign << (b-1) | magnitude index
 *     (pkv_tq_codebook returns the magnitudes);
 *   - each group of 16 consecutive elements of a (token, kv head) V row is
 *     coded as the nearest level of x / rms(group) (ties to the smaller
 *     magnitude); its scale is the saturating E4M3 of |x| / |levels|, so the
 *     decoded group (scale x level) keeps the input's L2 norm up to the
 *     scale's rounding; an all-zero group has scale 0.  These decisions are
 *     taken in FP32 in this order: ss = fused multiply-add sum of x_i^2,
 *     i = 0..15; u_i = x_i * rsq(ss * 1/16); magnitude index = the number
 *     of midpoints between adjacent magnitudes that |u_i| exceeds; sign =
 *     u_i < 0; scale = E4M3(sqrt(ss * rcp(sum of chosen m^2))), with rsq,
 *     rcp and sqrt the hardware's approximations (about an ulp each), so a
 *     decision can differ from the exact one only within ~2^-20 (relative)
 *     of its boundary;
 *   - a cache block of B tokens holds one region of B * (D * b / 8 + D / 16)
 *     bytes per kv head h, in head order: the code rows of tokens 0..B-1
 *     (token t at t * D * b / 8, group q at 2 b bytes each, element i at
 *     bits [b i, b i + b) of the group's little-endian bytes), then one
 *     scale row of B bytes per group (scale of (t, q) at B * D * b / 8 +
 *     q * B + t), so a head's codes and scales of one block are contiguous
 *     (pkv_v_block_bytes gives the block size). */
typedef enum pkv_dtype {
    PKV_BF16 = 0,
    PKV_FP8_E4M3 = 1,
    PKV_FP32 = 2,
    PKV_TQ2 = 3,
    PKV_TQ3 = 4,
    PKV_TQ4 = 5
} pkv_dtype;

enum {
    PKV_OK = 0,
    PKV_ERR_INVALID = -1,
    PKV_ERR_UNSUPPORTED = -2,
    PKV_ERR_WORKSPACE = -3,
    PKV_ERR_HIP = -4
};

/* Message for the last non-zero status on this thread ("" if none). */
const char* pkv_last_error(void);

/* Library version as "major.minor.patch". */
const char* pkv_version(void);

/* Bytes of one V cache block of block_size tokens x num_kv_heads x
 * head_dim_v elements in v_dtype (the pool is num_blocks such blocks); 0 for
 * an unknown dtype or a TQ layout whose head_dim_v is not a multiple of 16. */
size_t pkv_v_block_bytes(pkv_dtype v_dtype, uint32_t block_size, uint32_t num_kv_heads,
                         uint32_t head_dim_v);

/* The E4M3 codes of a TQ format's 2^(b-1) positive codebook magnitudes,
 * ascending, into host memory mag_codes.  0, or PKV_ERR_INVALID for a
 * non-TQ dtype or NULL. */
int pkv_tq_codebook(pkv_dtype v_dtype, uint8_t* mag_codes);

/*
 * pkv_fill_slots -- [p1] fill_slots_from_block_table: fill paged-KV slot
 * mappings on the device from a persistent block table.
 *
 * For sequence s (s < num_seqs) and its i-th token, i in
 * [cu_counts[s], cu_counts[s+1]), position p = start_pos[s] + (i - cu_counts[s]):
 *     slots[i] = block_tables[s * max_blocks_per_seq + p / block_size]
 *                * block_size + p % block_size
 * Batched form of the page's one-sequence call (num_seqs = 1, cu_counts =
 * {0, count} is that call).  A token whose block index p / block_size is not
 * below max_blocks_per_seq, or whose p is negative, or that no sequence
 * covers (i >= cu_counts[num_seqs]), gets slot -1.  A negative table entry
 * gives a negative slot (skipped by the writes).
 *
 *   slots          out  int64 [total_tokens]
 *   block_tables   in   int32 [num_seqs, max_blocks_per_seq]
 *   start_pos      in   int32 [num_seqs]
 *   cu_counts      in   int32 [num_seqs + 1], non-decreasing, cu_counts[0] = 0
 *   total_tokens        length of `slots` (usually cu_counts[num_seqs])
 * Supported: block_size in 1..65536.
 */
int pkv_fill_slots(int64_t* slots, const int32_t* block_tables, uint32_t max_blocks_per_seq,
                   const int32_t* start_pos, const int32_t* cu_counts, uint32_t num_seqs,
                   uint32_t total_tokens, uint32_t block_size, void* stream);

/*
 * pkv_cache_write_k_fused -- [p1] fused_k_norm_rope_cache_write_{bf16,
 * bf16_mrope, fp8}: RMSNorm, then RoPE, then ONE rounding at the store, all
 * in FP32 in between ([p1] doc: K stays FP32 between the three operations;
 * [p2] module invariants: FP8 stores k / k_scale as E4M3).
 *
 * For each token t with 0 <= slot_mapping[t] < num_blocks * block_size and
 * each kv head h, with x = k_in[t, h, :] (FP32 of the input):
 *   RMSNorm (norm_weight != NULL):  y = x / sqrt(mean_j x_j^2 + rms_eps) * w
 *   RoPE (nope == 0, rotary_dim > 0), NeoX rotate-half pairs over dims
 *     [rope_offset, rope_offset + rotary_dim): for pair i < rotary_dim / 2,
 *     a = y[o + i], b = y[o + i + rotary_dim/2], angle = fl32(pos * invf_i),
 *     invf_i = fl32(theta^(-2i / rotary_dim)):
 *       a' = a cos(angle) - b sin(angle),  b' = b cos(angle) + a sin(angle)
 *     pos = pos_t[t]; when pos_h and pos_w are both non-NULL (MRoPE,
 *     [p1] ..._bf16_mrope), pair i uses {pos_t, pos_h, pos_w}[i % 3][t];
 *     with pos_t == pos_h == pos_w the result is bit-identical to the
 *     scalar form.
 *   Store into k_cache[slot, h, :]:
 *     PKV_BF16      round-to-nearest-even of the FP32 value
 *     PKV_FP8_E4M3  saturating E4M3 of fl32(value / k_scale): magnitudes
 *                   above 448 become +-448, NaN stays NaN
 *     PKV_FP32      the FP32 value
 *
 *   k_in          in  [num_tokens, num_kv_heads, head_dim] of in_dtype; token
 *                     t starts at element t * in_token_stride; heads packed
 *   norm_weight   in  [head_dim] of in_dtype, shared by all heads; NULL = no norm
 *   pos_t         in  int32 [num_tokens] (ignored when nope != 0 or rotary_dim == 0)
 *   pos_h, pos_w  in  int32 [num_tokens] or both NULL
 *   slot_mapping  in  int64 [num_tokens]
 *   k_cache       out [num_blocks, block_size, num_kv_heads, head_dim] of cache_dtype
 *   k_scale           FP8 only: per-tensor scale, finite and at least
 *                     FLT_MIN = 2^-126 (a normal number), else PKV_ERR_INVALID
 * Supported: in_dtype BF16 or FP32; cache_dtype BF16, FP8_E4M3 or FP32;
 *   head_dim in {64, 128, 192, 256}; rotary_dim even, rope_offset +
 *   rotary_dim <= head_dim, rope_offset and rotary_dim / 2 multiples of
 *   the 16-byte input vector (8 BF16 or 4 FP32 elements).
 */
int pkv_cache_write_k_fused(const void* k_in, pkv_dtype in_dtype, uint64_t in_token_stride,
                            const void* norm_weight, float rms_eps,
                            const int32_t* pos_t, const int32_t* pos_h, const int32_t* pos_w,
                            float theta, uint32_t rope_offset, uint32_t rotary_dim, int nope,
                            const int64_t* slot_mapping, uint32_t num_tokens,
                            uint32_t num_kv_heads, uint32_t head_dim, uint32_t block_size,
                            uint32_t num_blocks, void* k_cache, pkv_dtype cache_dtype,
                            float k_scale, void* stream);

/*
 * pkv_cache_write_v -- [p1] reshape_and_cache_flash_v_only: the V-only paged
 * cache write, companion of the fused K write so that the K side of the
 * cache is written by the fused kernel alone; with an E4M3 cache, the V half
 * of [p1] reshape_and_cache_fp8 (K and V to FP8 with k_scale and v_scale).
 *
 * For each token t with 0 <= slot_mapping[t] < num_blocks * block_size and
 * every kv head h:
 *   cache_dtype == in_dtype:  v_cache[slot, h, :] = v[t, h, :], byte for byte
 *   cache_dtype == TQ2/3/4:   the row's 16-element groups coded as stated
 *                             with pkv_dtype (finite inputs; v_scale unused)
 *   cache_dtype == FP8_E4M3:  v_cache[slot, h, d] = saturating E4M3 of
 *                             fl32(v[t, h, d] / v_scale) (correctly rounded
 *                             FP32 division, then round-to-nearest-even;
 *                             magnitudes above 448 become +-448, NaN stays NaN)
 *
 *   v             in  [num_tokens, num_kv_heads, head_dim_v] of in_dtype, token
 *                     stride in_token_stride elements
 *   slot_mapping  in  int64 [num_tokens]
 *   v_cache       out [num_blocks, block_size, num_kv_heads, head_dim_v] of cache_dtype
 *   v_scale           E4M3 cache only: per-tensor scale, finite and > 0
 * Supported: (in_dtype, cache_dtype) (BF16, BF16), (FP32, FP32),
 *   (BF16, FP8_E4M3), (FP32, FP8_E4M3), (BF16 or FP32, TQ2/3/4); the cache
 *   row num_kv_heads * head_dim_v elements a multiple of 16 bytes in both
 *   dtypes; for TQ, head_dim_v a multiple of 16 and block_size *
 *   head_dim_v / 16 a multiple of 8 (v_cache: num_blocks *
 *   pkv_v_block_bytes bytes, 16-byte aligned).
 */
int pkv_cache_write_v(const void* v, pkv_dtype in_dtype, uint64_t in_token_stride,
                      const int64_t* slot_mapping, uint32_t num_tokens, uint32_t num_kv_heads,
                      uint32_t head_dim_v, uint32_t block_size, uint32_t num_blocks,
                      void* v_cache, pkv_dtype cache_dtype, float v_scale, void* stream);

/*
 * pkv_decode_workspace_bytes -- bytes of device workspace that
 * pkv_paged_decode_attn needs for these sizes (split-K partial results:
 * (head_dim_v + 2) FP32 per sequence, query head and split).  0 means none is
 * needed.  Depends only on the arguments given; sliding_window and
 * split_tokens as for pkv_paged_decode_attn.
 */
size_t pkv_decode_workspace_bytes(uint32_t num_seqs, uint32_t num_q_heads,
                                  uint32_t num_kv_heads, uint32_t head_dim_v,
                                  uint32_t max_blocks_per_seq, uint32_t block_size,
                                  uint32_t sliding_window, uint32_t split_tokens);

/*
 * pkv_paged_decode_attn -- [p1] paged_decode_attn_fp8 and its BF16 sibling
 * (one query token per sequence, reading K/V through block_tables i32
 * [num_seqs * max_blocks_per_seq] and seq_lens i32 [num_seqs], GQA through
 * num_q_heads / num_kv_heads, scaled scores, FP8 K and V multiplied back by
 * k_scale and v_scale), with the sliding window of the [p1] decode launchers
 * and the attention sinks of [p1] mla_paged_decode_fp8, the optional
 * elementwise output gate of [p3] (SDPA + gate) and the optional query
 * rotation of [p3] (maybe_rope before SDPA).
 *
 * For sequence s, query head h, kv head g = h / (num_q_heads / num_kv_heads),
 * n = seq_lens[s], attended tokens t in [lo, n) with lo = n - sliding_window
 * when 0 < sliding_window < n, else 0, each at row P * block_size +
 * t % block_size with P = block_tables[s][t / block_size]:
 *   q' = q[s, h, :], rotated at position n - 1 when q_rope != 0 (same RoPE
 *        as the K write over [q_rope_offset, q_rope_offset + q_rope_dim),
 *        theta q_rope_theta)
 *   s_t = scale * <q', k_t>, k_t = k_cache row (E4M3 codes times k_scale)
 *   Z   = sum_t exp(s_t) (+ exp(sinks[h]) when sinks is given)
 *   out[s, h, :] = sum_t exp(s_t) / Z * v_t   (v_t: E4M3 codes times
 *                  v_scale), times gate[s, h, :] if given
 * The window and sink semantics are not stated by the pages; this is the
 * reading taken: the window holds the sliding_window most recent tokens
 * (0 = no window), and a sink is a per-query-head logit, in the units of
 * s_t, that joins the normalisation and carries no value.  A sequence with
 * no attended token gives an all-zero row.  Table entries of blocks wholly
 * before the window are never read.  Computed in FP32 with split-K over the
 * attended range and a log-sum-exp merge; out is FP32.
 *
 *   q             in  [num_seqs, num_q_heads, head_dim_qk] of q_dtype; sequence
 *                     s starts at element s * q_seq_stride
 *   k_cache       in  [num_blocks, block_size, num_kv_heads, head_dim_qk] of k_dtype
 *   v_cache       in  [num_blocks, block_size, num_kv_heads, head_dim_v] of v_dtype;
 *                     TQ: num_blocks blocks of pkv_v_block_bytes bytes, laid out
 *                     as stated with pkv_dtype
 *   k_scale, v_scale  E4M3 caches only: per-tensor scales, finite and > 0
 *   sparse_v_threshold  the sparse-V skip of TQ V caches ([p2]
 *                     paged_decode_attn_fp8k_turbo3v: a position's V is not
 *                     loaded or dequantised when its attention weight is at
 *                     most a threshold whose value the pages do not give;
 *                     [p1] describes its Turbo-V decodes as sparse in V).
 *                     0 = exact decode.  In (0, 1): a position whose weight
 *                     relative to the largest score seen so far in its
 *                     split-K piece, exp(s_t - running max), is at most the
 *                     threshold leaves the sum over V (it stays in Z).  That
 *                     weight is never below the softmax weight exp(s_t) / Z,
 *                     so the positions left out are a subset of those whose
 *                     weight is at most the threshold; which ones depends on
 *                     the order and the split-K pieces in which positions
 *                     are visited.  A 16-token block none of whose positions
 *                     is kept for any query head of the GQA group reads no V
 *                     bytes and skips the V decode and the PV product.
 *                     Outside [0, 1) (or NaN): PKV_ERR_INVALID; > 0 with a
 *                     non-TQ V cache: PKV_ERR_UNSUPPORTED
 *   scale             softmax scale of the scores, finite and > 0 (else
 *                     PKV_ERR_INVALID)
 *   block_tables  in  int32 [num_seqs, max_blocks_per_seq]
 *   seq_lens      in  int32 [num_seqs]; tokens past max_blocks_per_seq *
 *                     block_size are excluded
 *   sliding_window    tokens in the window, 0 = attend to all
 *   sinks         in  FP32 [num_q_heads] or NULL
 *   gate          in  FP32 [num_seqs, num_q_heads, head_dim_v] or NULL
 *   out           out FP32 [num_seqs, num_q_heads, head_dim_v]
 *   split_tokens  tokens per split-K piece, rounded up to whole blocks and
 *                 capped at 128 blocks; 0 = the library's choice: without a
 *                 sliding window and with at most 1024 sequences, equal ranges
 *                 (at most 512 blocks) of the batch's attended blocks taken in
 *                 sequence order, so that short sequences share a work-group
 *                 and long ones span several; otherwise enough pieces per
 *                 sequence to cover the GPU several times over.  The result
 *                 does not depend on it beyond FP32 rounding.
 *   workspace     device scratch of at least
 *                 pkv_decode_workspace_bytes(...) bytes (may be NULL if that is 0);
 *                 caller-owned, needs no initialisation, holds the split
 *                 partials between the call's kernels: calls that may run at
 *                 the same time (other streams) need workspaces of their own
 * Supported: (q, K, V) dtypes (BF16, BF16 or FP8_E4M3, BF16 or FP8_E4M3 or
 *   TQ2/3/4), (FP32, FP32, FP32); TQ V with head_dim 128; the decode of TQ V
 *   is exact unless sparse_v_threshold > 0; num_q_heads % num_kv_heads == 0;
 *   block_size 16;
 *   head_dim_qk in {64, 128, 192, 256}, head_dim_v in {64, 128} (BF16/E4M3
 *   caches: head_dim_qk == head_dim_v in {64, 128}, GQA group <= 16; FP32:
 *   group 1, 2, 4 or 8); q_rope (FP32 only) with q_rope_dim even and
 *   q_rope_offset + q_rope_dim <= head_dim_qk.  At most 65535 split-K pieces
 *   per sequence (a larger split_tokens lowers the count), at most 65535
 *   sequences per call with FP32 caches, and num_seqs * num_kv_heads below
 *   2^31 otherwise; beyond these PKV_ERR_UNSUPPORTED.
 */
int pkv_paged_decode_attn(const void* q, pkv_dtype q_dtype, uint64_t q_seq_stride,
                          const void* k_cache, pkv_dtype k_dtype, float k_scale,
                          const void* v_cache, pkv_dtype v_dtype, float v_scale,
                          float sparse_v_threshold, const int32_t* block_tables,
                          uint32_t max_blocks_per_seq, const int32_t* seq_lens,
                          uint32_t num_seqs, uint32_t num_blocks,
                          uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim_qk,
                          uint32_t head_dim_v, uint32_t block_size, float scale,
                          uint32_t sliding_window, const float* sinks,
                          int q_rope, float q_rope_theta, uint32_t q_rope_offset,
                          uint32_t q_rope_dim, const float* gate, float* out,
                          uint32_t split_tokens, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * pkv_paged_decode_attn_noalloc -- pkv_paged_decode_attn without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, computation, supported set and status codes as
 * pkv_paged_decode_attn (same kernels and split plan, so the output is
 * bit-identical to it), except that the split-K partials live in a device
 * scratch array of PKV_DECODE_SCRATCH_BYTES held by the library (one per GPU,
 * kept until the process ends; its address is looked up on the first call
 * on a device, with that device current).  The call allocates nothing and
 * calls no allocating routine.
 *   Limit: when pkv_decode_workspace_bytes(...) for these sizes exceeds
 *   PKV_DECODE_SCRATCH_BYTES (32 MiB: e.g. 256 sequences x 32 query heads
 *   need ~8.5 MiB, 64 x 64 ~10.6 MiB), PKV_ERR_WORKSPACE before any launch.
 *   The scratch needs no initialisation and keeps the last call's contents.
 *   Calls on one GPU that may overlap in time (other streams, other host
 *   threads with other streams) share it and RACE: serialise them on one
 *   stream, or use pkv_paged_decode_attn with workspaces of their own.
 *   `stream`, when not NULL, must belong to the current device, else
 *   PKV_ERR_INVALID.
 */
#define PKV_DECODE_SCRATCH_BYTES (32u << 20)

int pkv_paged_decode_attn_noalloc(const void* q, pkv_dtype q_dtype, uint64_t q_seq_stride,
                                  const void* k_cache, pkv_dtype k_dtype, float k_scale,
                                  const void* v_cache, pkv_dtype v_dtype, float v_scale,
                                  float sparse_v_threshold, const int32_t* block_tables,
                                  uint32_t max_blocks_per_seq,
                                  const int32_t* seq_lens, uint32_t num_seqs,
                                  uint32_t num_blocks, uint32_t num_q_heads,
                                  uint32_t num_kv_heads, uint32_t head_dim_qk,
                                  uint32_t head_dim_v, uint32_t block_size, float scale,
                                  uint32_t sliding_window, const float* sinks,
                                  int q_rope, float q_rope_theta, uint32_t q_rope_offset,
                                  uint32_t q_rope_dim, const float* gate, float* out,
                                  uint32_t split_tokens, void* stream);

/*
 * pkv_paged_prefill_attn -- [p1] the batched prefill variants of the paged
 * kernels over N tokens (the page names them and gives no more): causal
 * attention of the new tokens of every sequence over the same paged cache,
 * after their K/V rows have been written (pkv_cache_write_k_fused /
 * pkv_cache_write_v).  Reading taken: the q_len = cu_q[s+1] - cu_q[s]
 * queries of sequence s are its last q_len tokens; query i sits at position
 * p = seq_lens[s] - q_len + i and attends to positions [lo, p], lo = p + 1 -
 * sliding_window when 0 < sliding_window < p + 1, else 0; scores, E4M3
 * scales, the sink rule and the exclusion of unmapped blocks are those of
 * pkv_paged_decode_attn.  q_len = 1 is the decode call.
 *
 *   q             in  [total_q, num_q_heads, head_dim_qk] BF16, token t at
 *                     element t * q_token_stride (heads packed)
 *   cu_q          in  int32 [num_seqs + 1], non-decreasing, cu_q[0] = 0,
 *                     cu_q[num_seqs] <= total_q
 *   max_q_len         an upper bound of every q_len (host value: sizes the
 *                     grid); rows of a sequence past max_q_len are undefined
 *   total_q           rows of q and out; rows >= total_q are never touched
 *   seq_lens      in  int32 [num_seqs], including the new tokens; a query
 *                     with p < 0 gets an all-zero row
 *   sinks         in  FP32 [num_q_heads] or NULL
 *   out           out FP32 [total_q, num_q_heads, head_dim_v]; rows of the
 *                     queries only
 *   (other arguments as for pkv_paged_decode_attn)
 * Supported: q BF16; K and V BF16 or FP8_E4M3; head_dim_qk == head_dim_v in
 *   {64, 128}; GQA group 1, 2, 4, 8 or 16; block_size 16.  No workspace.
 */
int pkv_paged_prefill_attn(const void* q, pkv_dtype q_dtype, uint64_t q_token_stride,
                           const int32_t* cu_q, uint32_t max_q_len, uint32_t total_q,
                           const void* k_cache, pkv_dtype k_dtype, float k_scale,
                           const void* v_cache, pkv_dtype v_dtype, float v_scale,
                           const int32_t* block_tables, uint32_t max_blocks_per_seq,
                           const int32_t* seq_lens, uint32_t num_seqs, uint32_t num_blocks,
                           uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim_qk,
                           uint32_t head_dim_v, uint32_t block_size, float scale,
                           uint32_t sliding_window, const float* sinks, float* out,
                           void* stream);

/*
 * pkv_mla_cache_assemble -- [p1] mla_cache_assemble: the single-head MLA
 * cache rows of a token, K = [kv_latent | k_rope] and V = [kv_latent |
 * zeros], in one kernel.  Batched here over tokens through a slot mapping:
 * for each token t with 0 <= slot_mapping[t] < num_blocks * block_size,
 *   k_cache[slot, 0, :] = [kv_latent[t, :kv_lora], k_rope[t, :rope], 0 ...]
 *   v_cache[slot, 0, :] = [kv_latent[t, :kv_lora], 0 ...]
 * byte for byte in dtype; cache_dim >= kv_lora + rope (the rest is zero).
 *
 *   kv_latent     in  [num_tokens, >= kv_lora] of dtype, token stride latent_stride
 *   k_rope        in  [num_tokens, >= rope] of dtype, token stride rope_stride
 *                     (may be NULL when rope == 0)
 *   slot_mapping  in  int64 [num_tokens]
 *   k_cache, v_cache  out [num_blocks, block_size, 1, cache_dim] of dtype
 * Supported: dtype BF16 or FP32; kv_lora, rope, cache_dim and both strides
 *   multiples of 16 bytes.
 */
int pkv_mla_cache_assemble(const void* kv_latent, const void* k_rope, pkv_dtype dtype,
                           uint64_t latent_stride, uint64_t rope_stride,
                           const int64_t* slot_mapping, uint32_t num_tokens, uint32_t kv_lora,
                           uint32_t rope, uint32_t cache_dim, uint32_t block_size,
                           uint32_t num_blocks, void* k_cache, void* v_cache, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */

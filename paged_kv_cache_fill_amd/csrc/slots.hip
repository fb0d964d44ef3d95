// slots.hip -- pkv_fill_slots: slot mapping from per-sequence block tables
// (page 1, kv_cache.rs, fill_slots_from_block_table: slots filled on the
// device from a persistent block table; slot_mapping is i64).
//
// One thread per output token.  The owning sequence is found by binary
// search over cu_counts (num_seqs + 1 entries, read through L2; every probe
// stays inside the array whatever its contents), so a whole batch of
// sequences -- a decode step of hundreds of sequences or a prefill of
// thousands of tokens -- is one launch.
#include "pkv_internal.h"

namespace pkv {

__global__ __launch_bounds__(256) void fill_slots_kernel(
    int64_t* __restrict__ slots, const int32_t* __restrict__ block_tables,
    uint32_t max_blocks_per_seq, const int32_t* __restrict__ start_pos,
    const int32_t* __restrict__ cu_counts, uint32_t num_seqs, uint32_t total_tokens,
    uint32_t block_size)
{
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i >= total_tokens)
        return;
    // smallest j in [1, num_seqs] with cu_counts[j] > i  (j = num_seqs + 1: none)
    uint32_t lo = 1, hi = num_seqs + 1;
    while (lo < hi) {
        uint32_t mid = (lo + hi) >> 1;
        if ((int64_t)cu_counts[mid] > (int64_t)i)
            hi = mid;
        else
            lo = mid + 1;
    }
    int64_t slot = -1;
    if (lo <= num_seqs) {
        const uint32_t s = lo - 1;
        const int64_t first = cu_counts[s];
        if (first <= (int64_t)i) {
            const int64_t p = (int64_t)start_pos[s] + ((int64_t)i - first);
            if (p >= 0) {
                const uint64_t b = (uint64_t)p / block_size;
                if (b < max_blocks_per_seq) {
                    const int64_t blk = block_tables[(uint64_t)s * max_blocks_per_seq + b];
                    slot = blk * (int64_t)block_size + (int64_t)((uint64_t)p % block_size);
                }
            }
        }
    }
    slots[i] = slot;
}

}  // namespace pkv

extern "C" int pkv_fill_slots(int64_t* slots, const int32_t* block_tables,
                              uint32_t max_blocks_per_seq, const int32_t* start_pos,
                              const int32_t* cu_counts, uint32_t num_seqs,
                              uint32_t total_tokens, uint32_t block_size, void* stream)
{
    using namespace pkv;
    clear_error();
    if (total_tokens == 0)
        return PKV_OK;
    if (!slots || !cu_counts)
        return fail(PKV_ERR_INVALID, "fill_slots: slots and cu_counts must be non-NULL");
    if (num_seqs > 0 && (!block_tables || !start_pos))
        return fail(PKV_ERR_INVALID, "fill_slots: block_tables and start_pos must be non-NULL");
    if (num_seqs > 0 && max_blocks_per_seq == 0)
        return fail(PKV_ERR_INVALID, "fill_slots: max_blocks_per_seq must be > 0");
    if (block_size == 0 || block_size > 65536)
        return fail(PKV_ERR_UNSUPPORTED, "fill_slots: block_size %u outside 1..65536", block_size);
    hipLaunchKernelGGL(fill_slots_kernel, dim3(ceil_div(total_tokens, 256)), dim3(256), 0,
                       (hipStream_t)stream, slots, block_tables, max_blocks_per_seq, start_pos,
                       cu_counts, num_seqs, total_tokens, block_size);
    return check_launch("fill_slots");
}

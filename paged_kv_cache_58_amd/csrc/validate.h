// Contract checks of the index arrays the decode and append trust: the slot
// mapping, the block tables and the context lengths.  Release builds never
// look at them on the host or the device (reading device arrays on the host
// would synchronise); a PA_DEBUG build runs these checks on the device before
// every call and refuses the call on a violation.  The functions are plain
// C++ usable from host code too, so the rules are tested on the CPU with
// out-of-range ids that are never handed to a GPU kernel.
//
// The rules restate the contract of the calls: a slot is -1 (skip) or a row
// of the pool, row = physical block * block_size + offset ("Écriture dans le
// cache" of the nano-vLLM article writes row `slot` and skips -1); a
// sequence's attended tokens sit in the blocks its table lists, each a block
// of the pool (the page table of "PagedAttention KV cache comme mémoire
// virtuelle" in "Cache KV, attention et optimisation de l'inference").
#pragma once

#include <cstdint>

#if defined(__HIPCC__)
#define PA_HOST_DEVICE __host__ __device__
#else
#define PA_HOST_DEVICE
#endif

namespace pa {

// What a violation record's code says (the record is one 64-bit word: code
// in the top 8 bits, the offending element's index below; 0 = no violation).
enum IndexViolation : int32_t {
    kIndexOk = 0,
    kSlotRange = 1,        // slot_mapping[i] is neither -1 nor a slot of the pool
    kSlotDuplicate = 2,    // slot_mapping[i] repeats an earlier non-negative slot
    kContextNegative = 3,  // context_lens[b] < 0
    kContextRange = 4,     // context_lens[b] exceeds what the table (or max_context) holds
    kBlockRange = 5,       // a block id the call reads is outside [0, num_blocks)
    kCopyRange = 6,        // a copy pair names a negative block, or a block that is also a source
};

// Tokens per record index field (the code sits above it).
constexpr int kRecordIndexBits = 56;

PA_HOST_DEVICE inline uint64_t make_record(int32_t code, int64_t index) {
    return (static_cast<uint64_t>(code) << kRecordIndexBits) |
           (static_cast<uint64_t>(index) & ((uint64_t(1) << kRecordIndexBits) - 1));
}
PA_HOST_DEVICE inline int32_t record_code(uint64_t r) {
    return static_cast<int32_t>(r >> kRecordIndexBits);
}
PA_HOST_DEVICE inline int64_t record_index(uint64_t r) {
    return static_cast<int64_t>(r & ((uint64_t(1) << kRecordIndexBits) - 1));
}

// Slot i of an append's slot mapping (n tokens, a pool of num_slots rows).
// Duplicates are looked for only among the first kDupScan tokens (quadratic).
constexpr int32_t kDupScan = 4096;
PA_HOST_DEVICE inline int32_t check_slot(const int32_t *slots, int32_t n, int32_t i,
                                         int64_t num_slots) {
    const int32_t s = slots[i];
    if (s == -1) return kIndexOk;
    if (s < 0 || s >= num_slots) return kSlotRange;
    if (n <= kDupScan)
        for (int32_t j = 0; j < i; ++j)
            if (slots[j] == s) return kSlotDuplicate;
    return kIndexOk;
}

// First token a query of a sequence of length ctx reads: the start of its
// sliding window (window > 0), else 0.
PA_HOST_DEVICE inline int32_t first_token_read(int32_t ctx, int32_t window) {
    return (window > 0 && ctx > window) ? ctx - window : 0;
}

// Context length of one sequence: within [0, cap], cap = the table's
// capacity (max_blocks * block_size) or a tighter bound the call states.
PA_HOST_DEVICE inline int32_t check_context(int32_t ctx, int64_t cap) {
    if (ctx < 0) return kContextNegative;
    return static_cast<int64_t>(ctx) <= cap ? kIndexOk : kContextRange;
}

// Entry j of sequence b's block table (max_blocks entries per row): only the
// entries of blocks holding a token the call reads are checked (the rest,
// padding included, are never read).  Call after check_context passed.
PA_HOST_DEVICE inline int32_t check_table_entry(const int32_t *block_tables, int32_t max_blocks,
                                                int32_t b, int32_t j, int32_t ctx,
                                                int32_t block_size, int32_t window,
                                                int32_t num_blocks) {
    const int32_t first = first_token_read(ctx, window) / block_size;
    const int32_t last = (ctx + block_size - 1) / block_size;  // one past
    if (j < first || j >= last) return kIndexOk;
    const int32_t id = block_tables[static_cast<int64_t>(b) * max_blocks + j];
    return (id >= 0 && id < num_blocks) ? kIndexOk : kBlockRange;
}

// Copy pair i of a block copy: both ids non-negative, no destination that is
// also a source (among the first kDupScan pairs).  The pool's block count is
// not part of that call, so the upper bound is the caller's.
PA_HOST_DEVICE inline int32_t check_copy_pair(const int32_t *src, const int32_t *dst, int32_t n,
                                              int32_t i) {
    if (src[i] < 0 || dst[i] < 0) return kCopyRange;
    if (n <= kDupScan)
        for (int32_t j = 0; j < n; ++j)
            if (src[j] == dst[i]) return kCopyRange;
    return kIndexOk;
}

}  // namespace pa

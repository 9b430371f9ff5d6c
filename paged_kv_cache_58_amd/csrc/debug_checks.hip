// The device pass of a PA_DEBUG build (linked into libpa_debug.so only):
// before a call's own kernels, one kernel applies the contract checks of
// validate.h to every slot, context length or block-table entry the call will
// use, and a thread that finds a violation stores a record of it (one plain
// 64-bit store; when several threads find one, any of their records may
// remain).  The host then waits for the stream, reads the record and, on a
// violation, returns PA_ERR_INDEX without launching anything that would have
// read or written out of bounds.  Release builds contain none of this.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <string>

#include "hip_util.h"
#include "launch.h"
#include "validate.h"

namespace pa {
namespace {

constexpr int kCheckThreads = 256;
constexpr int kMaxDebugDevices = 64;

// The violation record of each GPU (one copy per device).  Host code uses
// only the address hipGetSymbolAddress returns for the current device.
__device__ __align__(8) uint64_t g_violation_record;

__global__ __launch_bounds__(kCheckThreads) void check_slots_kernel(uint64_t *record,
                                                                    const int32_t *slots,
                                                                    int32_t n, int64_t num_slots) {
    const int32_t i = static_cast<int32_t>(blockIdx.x) * kCheckThreads + static_cast<int32_t>(threadIdx.x);
    if (i >= n) return;
    const int32_t c = check_slot(slots, n, i, num_slots);
    if (c != kIndexOk) *record = make_record(c, i);
}

// One work-group per sequence.
__global__ __launch_bounds__(kCheckThreads) void check_tables_kernel(
    uint64_t *record, const int32_t *block_tables, const int32_t *context_lens,
    int32_t max_blocks, int32_t block_size, int32_t window, int32_t num_blocks, int64_t cap) {
    const int32_t b = static_cast<int32_t>(blockIdx.x);
    const int32_t ctx = context_lens[b];
    const int32_t cc = check_context(ctx, cap);
    if (cc != kIndexOk) {
        if (threadIdx.x == 0) *record = make_record(cc, b);
        return;
    }
    for (int32_t j = static_cast<int32_t>(threadIdx.x); j < max_blocks; j += kCheckThreads) {
        const int32_t c = check_table_entry(block_tables, max_blocks, b, j, ctx, block_size, window,
                                            num_blocks);
        if (c != kIndexOk) *record = make_record(c, static_cast<int64_t>(b) * max_blocks + j);
    }
}

__global__ __launch_bounds__(kCheckThreads) void check_copies_kernel(uint64_t *record,
                                                                     const int32_t *src,
                                                                     const int32_t *dst,
                                                                     int32_t n) {
    const int32_t i = static_cast<int32_t>(blockIdx.x) * kCheckThreads + static_cast<int32_t>(threadIdx.x);
    if (i >= n) return;
    const int32_t c = check_copy_pair(src, dst, n, i);
    if (c != kIndexOk) *record = make_record(c, i);
}

// Address of the current device's record, looked up once per device.
pa_status record_address(uint64_t **out, std::string *why) {
    static std::atomic<uint64_t *> cache[kMaxDebugDevices];
    int dev = 0;
    pa_status st = hip_status(hipGetDevice(&dev), why, "debug: hipGetDevice");
    if (st != PA_OK) return st;
    if (dev < 0 || dev >= kMaxDebugDevices) {
        if (why) *why = "debug: device index out of range";
        return PA_ERR_UNSUPPORTED;
    }
    uint64_t *p = cache[dev].load(std::memory_order_acquire);
    if (!p) {
        void *addr = nullptr;
        st = hip_status(hipGetSymbolAddress(&addr, HIP_SYMBOL(g_violation_record)), why,
                        "debug: hipGetSymbolAddress");
        if (st != PA_OK) return st;
        p = static_cast<uint64_t *>(addr);
        cache[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return PA_OK;
}

const char *violation_text(int32_t code) {
    switch (code) {
        case kSlotRange: return "slot_mapping entry is neither -1 nor a slot of the pool";
        case kSlotDuplicate: return "slot_mapping entry repeats an earlier slot";
        case kContextNegative: return "context length is negative";
        case kContextRange: return "context length exceeds what the block table holds";
        case kBlockRange: return "block id is outside [0, num_blocks)";
        case kCopyRange: return "copy pair names a negative block or a destination that is a source";
    }
    return "unknown violation";
}

// Clears the record, enqueues `check`, waits for the stream and reads the
// record back.
template <typename F>
pa_status run_check(void *stream_arg, const char *what, std::string *why, F &&check) {
    const hipStream_t stream = static_cast<hipStream_t>(stream_arg);
    uint64_t *record = nullptr;
    pa_status st = record_address(&record, why);
    if (st != PA_OK) return st;
    st = hip_status(hipMemsetAsync(record, 0, sizeof(uint64_t), stream), why, "debug: clear");
    if (st != PA_OK) return st;
    check(record, stream);
    st = hip_status(hipGetLastError(), why, "debug: check launch");
    if (st != PA_OK) return st;
    st = hip_status(hipStreamSynchronize(stream), why, "debug: synchronize");
    if (st != PA_OK) return st;
    uint64_t r = 0;
    st = hip_status(hipMemcpy(&r, record, sizeof(r), hipMemcpyDeviceToHost), why, "debug: read");
    if (st != PA_OK) return st;
    if (r == 0) return PA_OK;
    if (why)
        *why = std::string(what) + ": " + violation_text(record_code(r)) + " (element " +
               std::to_string(record_index(r)) + ")";
    return PA_ERR_INDEX;
}

}  // namespace

pa_status debug_check_slots(const int32_t *slots, int32_t n, int64_t num_slots, void *stream,
                            std::string *why) {
    if (n <= 0) return PA_OK;
    return run_check(stream, "append (debug check)", why, [&](uint64_t *rec, hipStream_t s) {
        hipLaunchKernelGGL(check_slots_kernel, dim3((n + kCheckThreads - 1) / kCheckThreads),
                           dim3(kCheckThreads), 0, s, rec, slots, n, num_slots);
    });
}

pa_status debug_check_tables(const int32_t *block_tables, const int32_t *context_lens,
                             int32_t num_seqs, int32_t max_blocks, int32_t block_size,
                             int32_t window, int32_t num_blocks, int64_t cap, void *stream,
                             std::string *why) {
    if (num_seqs <= 0) return PA_OK;
    return run_check(stream, "decode (debug check)", why, [&](uint64_t *rec, hipStream_t s) {
        hipLaunchKernelGGL(check_tables_kernel, dim3(num_seqs), dim3(kCheckThreads), 0, s, rec,
                           block_tables, context_lens, max_blocks, block_size, window, num_blocks,
                           cap);
    });
}

pa_status debug_check_copies(const int32_t *src, const int32_t *dst, int32_t n, void *stream,
                             std::string *why) {
    if (n <= 0) return PA_OK;
    return run_check(stream, "copy_blocks (debug check)", why, [&](uint64_t *rec, hipStream_t s) {
        hipLaunchKernelGGL(check_copies_kernel, dim3((n + kCheckThreads - 1) / kCheckThreads),
                           dim3(kCheckThreads), 0, s, rec, src, dst, n);
    });
}

}  // namespace pa

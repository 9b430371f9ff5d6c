// Whole-block copies inside one cache pool (gfx950): the copy half of
// copy-on-write, when a sequence appends into a partly filled block that
// another sequence still shares (PagedAttention's copy-on-write in the CS336
// lecture 10 notes, "核心概念与定义").  The block manager queues (source,
// destination) pairs; one launch per pool array (K, V, and the scales of an
// MXFP8 cache) copies them, 16 bytes per lane.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "hip_util.h"
#include "launch.h"

namespace pa {
namespace {

__global__ __launch_bounds__(256) void copy_blocks_kernel(char *__restrict__ pool,
                                                          int64_t block_bytes,
                                                          const int32_t *__restrict__ src,
                                                          const int32_t *__restrict__ dst) {
    const int i = blockIdx.y;
    const uint4 *from = reinterpret_cast<const uint4 *>(pool + static_cast<int64_t>(src[i]) * block_bytes);
    uint4 *to = reinterpret_cast<uint4 *>(pool + static_cast<int64_t>(dst[i]) * block_bytes);
    const int64_t n = block_bytes / 16;
    for (int64_t k = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; k < n;
         k += static_cast<int64_t>(gridDim.x) * blockDim.x)
        to[k] = from[k];
}

}  // namespace

pa_status launch_copy_blocks(void *pool, int64_t block_bytes, const int32_t *src,
                             const int32_t *dst, int32_t num_pairs, void *stream_arg,
                             std::string *why) {
    const hipStream_t stream = static_cast<hipStream_t>(stream_arg);
    if (num_pairs == 0) return PA_OK;
    const int64_t vecs = block_bytes / 16;
    const int64_t per = (vecs + 255) / 256;
    const dim3 grid(static_cast<unsigned>(per < 64 ? per : 64), static_cast<unsigned>(num_pairs));
    hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(256), 0, stream, static_cast<char *>(pool),
                       block_bytes, src, dst);
    return hip_status(hipGetLastError(), why, "block copy launch");
}

}  // namespace pa

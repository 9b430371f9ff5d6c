// Slot-mapped KV append: token i's K (and V) row goes to row slot_mapping[i]
// of the cache viewed as [num_blocks * block_size, row]; -1 skips the token.
// (Cache-write kernel of "Écriture dans le cache", nano-vLLM article: one
// program per token, a row of kv_heads * head_dim elements, slot -1 = return.)
//
// One work-group per token.  The row is moved as whole vectors of the widest
// size (16 bytes on every shape this library runs) that divides the row
// lengths, the token strides and the base addresses, so the copy is bitwise.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "hip_util.h"
#include "launch.h"

namespace pa {
namespace {

constexpr int kAppendThreads = 256;

template <int VEC> struct VecType;
template <> struct VecType<16> { using type = uint4; };
template <> struct VecType<8> { using type = uint2; };
template <> struct VecType<4> { using type = uint32_t; };
template <> struct VecType<2> { using type = uint16_t; };

template <int VEC>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(
    char *__restrict__ k_cache, char *__restrict__ v_cache, const char *__restrict__ k,
    int64_t k_token_bytes, const char *__restrict__ v, int64_t v_token_bytes,
    const int32_t *__restrict__ slot_mapping, int64_t k_row_bytes, int64_t v_row_bytes) {
    using V = typename VecType<VEC>::type;
    const int64_t i = blockIdx.x;
    const int nk = static_cast<int>(k_row_bytes / VEC);
    const int nv = static_cast<int>(v_row_bytes / VEC);
    const V *src_k = reinterpret_cast<const V *>(k + i * k_token_bytes);
    const V *src_v = reinterpret_cast<const V *>(v + i * v_token_bytes);
    // the token's first chunk of K and V is read before the slot is known
    // (the source rows exist whatever the slot), so that both loads and the
    // slot's share one memory round trip
    const int e0 = threadIdx.x;
    V k0{}, v0{};
    if (e0 < nk) k0 = src_k[e0];
    if (e0 < nv) v0 = src_v[e0];
    const int32_t slot = slot_mapping[i];
    if (slot < 0) return;  // -1: padding token, nothing to write
    V *dst_k = reinterpret_cast<V *>(k_cache + static_cast<int64_t>(slot) * k_row_bytes);
    if (e0 < nk) dst_k[e0] = k0;
    for (int e = e0 + kAppendThreads; e < nk; e += kAppendThreads) dst_k[e] = src_k[e];
    if (nv > 0) {
        V *dst_v = reinterpret_cast<V *>(v_cache + static_cast<int64_t>(slot) * v_row_bytes);
        if (e0 < nv) dst_v[e0] = v0;
        for (int e = e0 + kAppendThreads; e < nv; e += kAppendThreads) dst_v[e] = src_v[e];
    }
}

template <int VEC>
void enqueue(const AppendArgs &a, const AppendPlan &p, hipStream_t stream) {
    const int eb = a.dtype == PA_F32 ? 4 : 2;
    hipLaunchKernelGGL(append_kernel<VEC>, dim3(a.num_tokens), dim3(kAppendThreads), 0, stream,
                       static_cast<char *>(a.k_cache), static_cast<char *>(a.v_cache),
                       static_cast<const char *>(a.k), a.k_token_stride * eb,
                       static_cast<const char *>(a.v), a.v_token_stride * eb, a.slot_mapping,
                       p.k_row_bytes, p.v_row_bytes);
}

}  // namespace

pa_status launch_append(const AppendArgs &a, const AppendPlan &plan, void *stream_arg,
                        std::string *why) {
    const hipStream_t stream = static_cast<hipStream_t>(stream_arg);
    if (a.num_tokens == 0) return PA_OK;
    switch (plan.vec_bytes) {
        case 16: enqueue<16>(a, plan, stream); break;
        case 8: enqueue<8>(a, plan, stream); break;
        case 4: enqueue<4>(a, plan, stream); break;
        default: enqueue<2>(a, plan, stream); break;
    }
    return hip_status(hipGetLastError(), why, "append launch");
}

}  // namespace pa

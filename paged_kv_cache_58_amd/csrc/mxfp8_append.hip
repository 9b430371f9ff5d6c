// Quantizing KV append into MXFP8 caches for gfx950.
//
// Each new token's K and V rows go through the slot mapping into the paged
// caches as in the plain append (the cache-write kernel of "Écriture dans le
// cache", nano-vLLM article: one program per token, -1 = skip), but stored in
// MXFP8, the blockwise-scaled fp8 the CS336 lecture 10 notes point to
// ("常见陷阱": per-tensor scales lose outlier channels; MXFP8 named as the
// blockwise remedy).  OCP MX conversion of each block of 32 values:
//   X = floor(log2(max |v|)) - 8, clamped to [-127, 127] (-127 for an all-zero
//   block), stored as the E8M0 byte X + 127;
//   each v * 2^-X rounded to the nearest E4M3 value, ties to even, saturating
//   at +-448.
// Layouts: K codes [num_blocks, Hkv, bs, 128] (token rows); V codes
// [num_blocks, Hkv, 128, bs] (each (block, head) tile transposed, which is
// the operand order of the decode's value product); scales [num_blocks, Hkv,
// bs, 4].
//
// One wave per (token, KV head): lane l holds values 2l and 2l + 1 of the
// row, so the 16 lanes of a row of the wave hold one 32-value block and find
// its max with four lane exchanges.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "hip_util.h"
#include "launch.h"

namespace pa {
namespace {

// Nearest E4M3 byte of a finite float, ties to even, saturating at +-448.
// Below 2^-6 the spacing is the subnormal quantum 2^-9 (rint of a * 512, where
// 8 lands on 0x08, the smallest normal); above, the 23-bit mantissa is
// rounded to 3 bits by integer addition, a carry moving into the exponent.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float y) {
    const uint32_t sign = (as_u(y) >> 24) & 0x80u;
    const float a = fabsf(y);
    uint32_t code;
    if (a >= 448.f) {
        code = 0x7Eu;
    } else if (a < 0.015625f) {
        code = static_cast<uint32_t>(rintf(a * 512.f));
    } else {
        uint32_t u = as_u(a);
        u += 0x7FFFFu + ((u >> 20) & 1u);
        code = (((u >> 23) - 120u) << 3) | ((u >> 20) & 7u);
    }
    return code | sign;
}

// Scale exponent of a block whose largest magnitude is amax (a float's biased
// exponent field is floor(log2) + 127 for normal values; zero and subnormals
// land below -127 and clamp there).
__device__ __forceinline__ int mx_scale_exp(float amax) {
    const int x = static_cast<int>((as_u(amax) >> 23) & 0xFFu) - 127 - 8;
    return min(max(x, -127), 127);
}

// Largest |v| over the 16 lanes of a row (one 32-value block).
__device__ __forceinline__ float max_over_16(float x) {
    x = fmaxf(x, __shfl_xor(x, 1));
    x = fmaxf(x, __shfl_xor(x, 2));
    x = fmaxf(x, __shfl_xor(x, 4));
    x = fmaxf(x, __shfl_xor(x, 8));
    return x;
}

template <typename T>
__device__ __forceinline__ float load_f32(const T *p) {
    if constexpr (sizeof(T) == 4) {
        return *reinterpret_cast<const float *>(p);
    } else {
        return as_f(static_cast<uint32_t>(*reinterpret_cast<const uint16_t *>(p)) << 16);
    }
}

// Quantizes a row's two values of this lane; returns the two codes as the
// low 16 bits (value 2l first) and leaves the scale byte in *scale.
template <typename T>
__device__ __forceinline__ uint32_t quantize_pair(const T *row, int lane, uint32_t *scale) {
    const float x0 = load_f32(row + 2 * lane);
    const float x1 = load_f32(row + 2 * lane + 1);
    const int X = mx_scale_exp(max_over_16(fmaxf(fabsf(x0), fabsf(x1))));
    *scale = static_cast<uint32_t>(X + 127);
    return e4m3_rne_sat(ldexpf(x0, -X)) | (e4m3_rne_sat(ldexpf(x1, -X)) << 8);
}

template <typename T>
__global__ __launch_bounds__(kWave) void mx_append_kernel(
    uint8_t *__restrict__ k8, uint8_t *__restrict__ v8, uint8_t *__restrict__ ks,
    uint8_t *__restrict__ vs, const T *__restrict__ k, int64_t k_stride, const T *__restrict__ v,
    int64_t v_stride, const int32_t *__restrict__ slot_mapping, int block_size,
    int num_kv_heads) {
    const int i = blockIdx.x;
    const int h = blockIdx.y;
    const int lane = threadIdx.x;
    const int s = slot_mapping[i];
    if (s < 0) return;  // -1: the token is skipped
    const int p = s / block_size;
    const int r = s - p * block_size;
    const int64_t tile = static_cast<int64_t>(p) * num_kv_heads + h;
    constexpr int D = kMxHeadDim;
    constexpr int NS = D / kMxBlock;

    uint32_t sc;
    const uint32_t kc = quantize_pair(k + static_cast<int64_t>(i) * k_stride + h * D, lane, &sc);
    *reinterpret_cast<uint16_t *>(k8 + (tile * block_size + r) * D + 2 * lane) =
        static_cast<uint16_t>(kc);
    if ((lane & 15) == 0) ks[(tile * block_size + r) * NS + (lane >> 4)] = static_cast<uint8_t>(sc);

    const uint32_t vc = quantize_pair(v + static_cast<int64_t>(i) * v_stride + h * D, lane, &sc);
    uint8_t *vt = v8 + (tile * D + 2 * lane) * block_size + r;  // column r of the V tile
    vt[0] = static_cast<uint8_t>(vc);
    vt[block_size] = static_cast<uint8_t>(vc >> 8);
    if ((lane & 15) == 0) vs[(tile * block_size + r) * NS + (lane >> 4)] = static_cast<uint8_t>(sc);
}

}  // namespace

pa_status launch_append_mxfp8(const MxAppendArgs &a, void *stream_arg, std::string *why) {
    const hipStream_t stream = static_cast<hipStream_t>(stream_arg);
    if (a.num_tokens == 0) return PA_OK;
    const dim3 grid(a.num_tokens, a.num_kv_heads);
    uint8_t *k8 = static_cast<uint8_t *>(a.k_cache);
    uint8_t *v8 = static_cast<uint8_t *>(a.v_cache);
    uint8_t *ks = static_cast<uint8_t *>(a.k_scale);
    uint8_t *vs = static_cast<uint8_t *>(a.v_scale);
    if (a.dtype == PA_BF16)
        hipLaunchKernelGGL(mx_append_kernel<uint16_t>, grid, dim3(kWave), 0, stream, k8, v8, ks,
                           vs, static_cast<const uint16_t *>(a.k), a.k_token_stride,
                           static_cast<const uint16_t *>(a.v), a.v_token_stride, a.slot_mapping,
                           a.block_size, a.num_kv_heads);
    else
        hipLaunchKernelGGL(mx_append_kernel<float>, grid, dim3(kWave), 0, stream, k8, v8, ks, vs,
                           static_cast<const float *>(a.k), a.k_token_stride,
                           static_cast<const float *>(a.v), a.v_token_stride, a.slot_mapping,
                           a.block_size, a.num_kv_heads);
    return hip_status(hipGetLastError(), why, "mxfp8 append launch");
}

}  // namespace pa

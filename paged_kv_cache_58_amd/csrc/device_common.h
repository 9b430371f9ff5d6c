// Device helpers shared by the decode kernels of libpa (gfx950), and the
// stream-K log-sum-exp reduce both decode paths end with.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdlib>

#include "plan.h"

namespace pa {
namespace {

constexpr int kWave = 64;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kMaxDevices = 64;



typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float as_f(uint32_t x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ uint32_t as_u(float x) { return __builtin_bit_cast(uint32_t, x); }

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                          __builtin_bit_cast(bf16x2_t, b), c, false);
}

// The first dot product of a chain, accumulating onto the constant 0 (the
// VOP3 form; the compiler would otherwise zero a register for v_dot2c).
__device__ __forceinline__ float dot2_bf16_0(uint32_t a, uint32_t b) {
    float r;
    asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    bf16x2_t v;
    v[0] = static_cast<__bf16>(lo);  // round to nearest even
    v[1] = static_cast<__bf16>(hi);
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return as_f(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return as_f(x & 0xffff0000u); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return as_f(static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(as_u(x)), CTRL, 0xF, 0xF, true)));
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// x[l] and x[l ^ 16] (r16) or x[l] and x[l ^ 32] (r32) in every lane l, by
// gfx950's row swaps (a swap of a register with itself hands each lane its
// partner's value) rather than __shfl_xor, which goes through the LDS
// crossbar and waits for it.  max and + are symmetric, so both lanes of a
// pair get the same bits.
__device__ __forceinline__ float max_r16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(as_u(x), as_u(x), false, false);
    return fmaxf(as_f(r[0]), as_f(r[1]));
}
__device__ __forceinline__ float max_r32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(as_u(x), as_u(x), false, false);
    return fmaxf(as_f(r[0]), as_f(r[1]));
}
__device__ __forceinline__ float sum_r16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(as_u(x), as_u(x), false, false);
    return as_f(r[0]) + as_f(r[1]);
}
__device__ __forceinline__ float sum_r32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(as_u(x), as_u(x), false, false);
    return as_f(r[0]) + as_f(r[1]);
}

// LDS address of a __shared__ object (what M0 takes for an LDS-DMA load).
__device__ __forceinline__ uint32_t lds_offset(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (const __attribute__((address_space(3))) char *)(p)));
}

// One global_load_lds_dwordx4: every lane reads 16 bytes at sbase + voff and
// the wave's 64 x 16 bytes land in LDS at m0 + 16 * lane, without passing
// through VGPRs.  The nt bit marks the stream as read-once.  Issued from asm
// so that the compiler does not serialise the ring with vmcnt(0) before every
// LDS read; the kernel places the exact vmcnt waits itself (wait_vmem).
__device__ __forceinline__ void dma16(const void *sbase, uint32_t voff, uint32_t lds) {
    asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "{m0}"(lds)
                 : "memory");
}

// Five wait states after `base` is formed and before the first dma16 that
// reads it: a vector memory instruction may read an SGPR only 5 wait states
// after a VALU instruction wrote it, and a base built from a block id goes
// v_readfirstlane -> a few SALU instructions -> the load (the compiler does
// not look inside the asm for the hazard).  Taking `base` as an operand
// keeps the nop after the instructions that form it.
__device__ __forceinline__ void sgpr_settle(const void *base) {
    asm volatile("s_nop 4" ::"s"(base) : "memory");
}

// Wait until at most N vector-memory operations of this wave are in flight
// (they retire in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}


__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// One global_load_lds_dword: lane l's 4 bytes at sbase + voff land in LDS at
// m0 + 4 * l (used for the block ids of a segment).  The compiler does not
// look inside inline assembly for hazards, and a vector memory instruction
// may read an SGPR only 5 wait states after a VALU instruction wrote it (as
// v_readlane does when a spilled base pointer is reloaded right before):
// hence the s_nop 4.  This load runs once per 64 blocks; the hot-loop loads
// (dma16) take sgpr_settle once per block where their base comes from a
// block id, and a static test checks the compiled kernels for the pattern.
__device__ __forceinline__ void dma4(const void *sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds)
                 : "memory");
}

// s_waitcnt the compiler itself understands (it then knows its own loads,
// issued before, are complete): vmcnt(0), no wait on the other counters.
__device__ __forceinline__ void drain_vmem() {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    asm volatile("" ::: "memory");  // and no LDS read may be hoisted above it
}

// Marks a value loaded from global memory as settled: the compiler waits for
// its load here (it sees the asm read it), and every later use reads the
// asm's output, not a pending load.  Loads issued before the LDS-DMA ring
// starts go through this, or the compiler's own vmcnt waits in the loop (it
// cannot count the ring's asm loads) would drain the ring at every step.
template <typename V>
__device__ __forceinline__ void settle(V &v) {
    asm volatile("" : "+v"(v));
}
__device__ __forceinline__ void settle(uint4 &v) {
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    u4 x = __builtin_bit_cast(u4, v);
    asm volatile("" : "+v"(x));
    v = __builtin_bit_cast(uint4, x);
}

// Inclusive prefix sum across the wave.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int t = __shfl_up(v, d);
        if (lane >= d) v += t;
    }
    return v;
}

// Blocks each stream share takes: an equal part of all (sequence, segment,
// block) work, and at least kMinShare so that tiny batches do not split into
// fragments that cost more to merge than to run.
constexpr int kMinShare = 16;
__host__ __device__ __forceinline__ int stream_share(int total, int waves) {
    const int r = (total + waves - 1) / waves;
    return r > kMinShare ? r : kMinShare;
}

// Waves per team of the grouped partition kernels: a team shares one stream
// share, each of its waves streaming one KV head of the same blocks, so that
// at any time neighbouring head slices of a block's token rows are read
// together (longer runs of consecutive bytes per row than one wave's 256).
// The largest power of two that divides both the KV head count and the waves
// of a work-group (a team never spans two work-groups), for grouped heads
// (group > 1); with one query head per KV head (MHA) shares of about a
// segment's length already put neighbouring heads of a sequence on
// neighbouring waves, and teams measured slower there, so each wave streams
// its own share (1).  PA_TEAM_HEADS caps it.
inline int team_heads(int num_kv_heads, int waves_per_group, int group) {
    int cap = group > 1 ? waves_per_group : 1;
    if (const char *env = std::getenv("PA_TEAM_HEADS")) {
        const int v = std::atoi(env);
        if (v >= 1 && v < cap) cap = v;
    }
    int t = 1;
    while (2 * t <= cap && waves_per_group % (2 * t) == 0 && num_kv_heads % (2 * t) == 0) t *= 2;
    return t;
}

// Sliding window (per-layer local attention): with window w > 0 the query of
// a sequence of length L attends to tokens [max(0, L - w), L).  The first of
// them lies in block window_first_block(); the blocks a sequence contributes
// to the work are those from there to its last block.
__host__ __device__ __forceinline__ int window_start(int L, int window) {
    return (window > 0 && L > window) ? L - window : 0;
}
__host__ __device__ __forceinline__ int window_first_block(int L, int window, int bs) {
    return window_start(L, window) / bs;
}
__host__ __device__ __forceinline__ int window_blocks(int L, int window, int bs) {
    return (L + bs - 1) / bs - window_first_block(L, window, bs);
}

// Where stream share `sid` of `nshares` lies in the global (sequence,
// segment, block) order of a batch of bs-token blocks (the blocks of each
// sequence's window), each sequence holding `segs` segments: blocks [x0, x1),
// the first of them block `blk` of the window of segment (b, g), sequence b
// having nbb such blocks.  A segment is one KV head, or one chunk of KV heads
// that a team of waves streams together (one head per wave).  Share 0 also
// stores the per-sequence block prefix sums (num_seqs + 1 entries) that the
// reduce reads, if `writer`.  Uniform over the wave; returns false for a
// share past the end of the work.
struct ShareSpan {
    int x0, x1, b, nbb, g, blk;
};
__device__ __forceinline__ bool find_share(int sid, int nshares, int num_seqs, int segs, int bs,
                                           const int32_t *__restrict__ context_lens,
                                           int32_t *__restrict__ ws_prefix, int lane,
                                           ShareSpan &sp, int window = 0, bool writer = true) {
    // The block counts of the first kCached * 64 sequences are loaded once,
    // every load before any is used (clamped in bounds, num_seqs >= 1), and
    // serve both passes below: one memory round trip instead of one per
    // chunk and pass.
    constexpr int kCached = 4;
    int nb_c[kCached];
    {
        int len_c[kCached];
#pragma unroll
        for (int r = 0; r < kCached; ++r) len_c[r] = context_lens[min(r * kWave + lane, num_seqs - 1)];
#pragma unroll
        for (int r = 0; r < kCached; ++r)
            nb_c[r] = r * kWave + lane < num_seqs ? window_blocks(len_c[r], window, bs) : 0;
    }
    auto chunk_blocks = [&](int base) {  // this lane's block count in the chunk at base
        const int bb = base + lane;
        if (base < kCached * kWave) {
            int v = nb_c[0];
#pragma unroll
            for (int r = 1; r < kCached; ++r)
                if (base == r * kWave) v = nb_c[r];
            return v;
        }
        return bb < num_seqs ? window_blocks(context_lens[bb], window, bs) : 0;
    };
    int seq_blocks_total = 0;
    for (int base = 0; base < num_seqs; base += kWave) {
        const int bb = base + lane;
        const int nb = chunk_blocks(base);
        const int incl = wave_incl_scan(nb, lane);
        if (sid == 0 && writer && bb < num_seqs) ws_prefix[bb] = seq_blocks_total + incl - nb;
        seq_blocks_total += __builtin_amdgcn_readlane(incl, kWave - 1);
    }
    if (sid == 0 && writer && lane == 0) ws_prefix[num_seqs] = seq_blocks_total;
    const int total = segs * seq_blocks_total;
    const int share = stream_share(total, nshares);
    const int64_t x0l = static_cast<int64_t>(sid) * share;
    if (x0l >= total) return false;
    sp.x0 = static_cast<int>(x0l);
    sp.x1 = min(sp.x0 + share, total);

    // The sequence holding global block x0: first b whose blocks end past it.
    sp.b = 0;
    sp.nbb = 0;
    int cb = 0;
    for (int base = 0, carry = 0;; base += kWave) {
        const int bb = base + lane;
        const int nb = chunk_blocks(base);
        const int incl = wave_incl_scan(nb, lane);
        const bool past = bb < num_seqs &&
                          static_cast<int64_t>(segs) * (carry + incl) > sp.x0;
        const uint64_t hit = __builtin_amdgcn_ballot_w64(past);
        if (hit != 0) {
            const int f = __builtin_ctzll(hit);
            sp.b = base + f;
            sp.nbb = __builtin_amdgcn_readlane(nb, f);
            cb = carry + __builtin_amdgcn_readlane(incl, f) - sp.nbb;
            break;
        }
        carry += __builtin_amdgcn_readlane(incl, kWave - 1);
    }
    sp.g = (sp.x0 - segs * cb) / sp.nbb;
    sp.blk = (sp.x0 - segs * cb) - sp.g * sp.nbb;
    return true;
}

// ---------------------------------------------------------------------------
// Reduce over the stream-K partial slots of each (sequence, query, query
// head).  KV head g of sequence b has C = group * q_len columns, column
// i * group + h % group for query i and head h.  The partition kernels'
// stream shares run over (sequence, head chunk, block) with NC = Hkv /
// team_heads chunks of team_heads heads per sequence (team_heads = 1: one
// head per segment); share s leaves the partial of head g = ch * team_heads
// + hw in slot s + b * NC + ch, row ((slot * team_heads + hw) * C + column):
// O = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s, M = max_s m_s
// (O = 0 when no slot saw a token: an empty context).  One work-group of W
// waves per (query, query head, sequence), blockIdx.x = i * Hq + h; wave w
// takes slots w, w + W, ... of the segment.  out is [B, q_len, Hq, D].
// ---------------------------------------------------------------------------
template <typename T, int D, int W>
__global__ __launch_bounds__(kWave *W) void stream_reduce_kernel(
    T *__restrict__ out, const float *__restrict__ ws_acc, const float2 *__restrict__ ws_ml,
    const int32_t *__restrict__ ws_prefix, const int32_t *__restrict__ context_lens,
    int num_seqs, int num_kv_heads, int group, int block_size, int nshares, int team_heads,
    int q_len, int window, float *__restrict__ lse) {
    constexpr int DPL = D / kWave;
    const int num_q_heads = num_kv_heads * group;
    const int qi = blockIdx.x / num_q_heads;
    const int h = blockIdx.x - qi * num_q_heads;
    const int b = blockIdx.y;
    const int g = h / group;
    const int hh = qi * group + (h - g * group);  // column within the segment
    const int ncols = group * q_len;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    // the length and the prefix sums are read in one round trip (the prefix is
    // in bounds, and written by the partition whenever a context is non-empty)
    const int ctx = context_lens[b];
    const int pre_all = ws_prefix[num_seqs], pre_b = ws_prefix[b];
    asm volatile("" ::"s"(ctx), "s"(pre_all), "s"(pre_b));
    const int nb = window_blocks(ctx, window, block_size);
    T *o = out + ((static_cast<int64_t>(b) * q_len + qi) * num_q_heads + h) * D + lane * DPL;
    float *lse_row = lse ? lse + (static_cast<int64_t>(b) * q_len + qi) * num_q_heads + h : nullptr;

    __shared__ float s_max[W];
    __shared__ float s_num[W][D];
    __shared__ float s_den[W];

    if (nb <= 0) {  // empty context: O = 0, log-sum-exp -inf
        if (wave == 0)
#pragma unroll
            for (int d = 0; d < DPL; ++d) o[d] = static_cast<T>(0.f);
        if (lse_row && tid == 0) *lse_row = kNegInf;
        return;
    }
    const int nchunks = num_kv_heads / team_heads;
    const int ch = g / team_heads;
    const int hw = g - ch * team_heads;
    const int total = nchunks * pre_all;
    const int share = stream_share(total, nshares);
    const int seg_lo = nchunks * pre_b + ch * nb;
    const int w0 = seg_lo / share;
    const int n = (seg_lo + nb - 1) / share - w0 + 1;  // partial slots of this segment
    // row of slot w0 + b * NC + ch; consecutive slots are team_heads * C rows apart
    const int64_t first =
        ((static_cast<int64_t>(w0) + b * nchunks + ch) * team_heads + hw) * ncols + hh;
    const int64_t stride = static_cast<int64_t>(team_heads) * ncols;

    // This wave merges slots p = wave + W j, j < nw, kBatch at a time; the
    // first batch's loads (which need no weight) go out with the max pass, so
    // a short segment costs one round trip after the prefix.
    constexpr int kBatch = 8;
    const int nw = n > wave ? (n - wave + W - 1) / W : 0;
    float2 bml[kBatch];
    float bacc[kBatch][DPL];
    auto load_batch = [&](int j0) {
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int64_t r = first + static_cast<int64_t>(wave + W * min(j0 + j, nw - 1)) * stride;
            bml[j] = ws_ml[r];
            const float *a = ws_acc + r * D + lane * DPL;
            if constexpr (DPL % 2 == 0) {
#pragma unroll
                for (int d = 0; d < DPL; d += 2) {
                    const float2 v = *reinterpret_cast<const float2 *>(a + d);
                    bacc[j][d] = v.x;
                    bacc[j][d + 1] = v.y;
                }
            } else {
                bacc[j][0] = a[0];
            }
        }
    };
    if (nw > 0) load_batch(0);

    float M = kNegInf;
    for (int p = tid; p < n; p += kWave * W) M = fmaxf(M, ws_ml[first + p * stride].x);
    for (int sh = 32; sh >= 1; sh >>= 1) M = fmaxf(M, __shfl_xor(M, sh));
    if constexpr (W > 1) {
        if (lane == 0) s_max[wave] = M;
        __syncthreads();
        M = s_max[0];
#pragma unroll
        for (int w = 1; w < W; ++w) M = fmaxf(M, s_max[w]);
    }

    float num[DPL];
#pragma unroll
    for (int d = 0; d < DPL; ++d) num[d] = 0.f;
    float den = 0.f;
    if (M == kNegInf) {  // no slot saw a token (a query that sees nothing): O = 0
        if (wave == 0)
#pragma unroll
            for (int d = 0; d < DPL; ++d) o[d] = static_cast<T>(0.f);
        if (lse_row && tid == 0) *lse_row = kNegInf;
        return;
    }
    for (int j0 = 0; j0 < nw; j0 += kBatch) {
        if (j0 > 0) load_batch(j0);
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (j0 + j < nw) {  // (past nw the batch re-read this wave's last slot)
                const float wgt = exp2_fast(bml[j].x - M);
                den = fmaf(wgt, bml[j].y, den);
#pragma unroll
                for (int d = 0; d < DPL; ++d) num[d] = fmaf(wgt, bacc[j][d], num[d]);
            }
        }
    }
    if constexpr (W > 1) {
#pragma unroll
        for (int d = 0; d < DPL; ++d) s_num[wave][lane * DPL + d] = num[d];
        if (lane == 0) s_den[wave] = den;
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int w = 1; w < W; ++w) {
            den += s_den[w];
#pragma unroll
            for (int d = 0; d < DPL; ++d) num[d] += s_num[w][lane * DPL + d];
        }
    }
    // log-sum-exp of the scores in natural units: M and den are in log2 units
    if (lse_row && lane == 0) *lse_row = (M + log2f(den)) * 0.69314718055994531f;
    if constexpr (sizeof(T) == 2) {
        if constexpr (DPL % 2 == 0) {
#pragma unroll
            for (int d = 0; d < DPL; d += 2)
                *reinterpret_cast<uint32_t *>(o + d) = pack_bf16(num[d] / den, num[d + 1] / den);
        } else {
            const __bf16 r = static_cast<__bf16>(num[0] / den);
            o[0] = __builtin_bit_cast(T, r);
        }
    } else {
#pragma unroll
        for (int d = 0; d < DPL; ++d) o[d] = num[d] / den;
    }
}

// Enqueues the reduce: four waves per (sequence, query head) when there are
// few of them (long contexts with many partial slots each), else one, so that
// every row's short chain of dependent loads runs in a single pass of the grid.
template <typename T, int D>
hipError_t enqueue_stream_reduce(T *out, const float *ws_acc, const float2 *ws_ml,
                                 const int32_t *ws_prefix, const int32_t *context_lens,
                                 int num_seqs, int num_q_heads, int num_kv_heads, int group,
                                 int block_size, int nshares, int team_heads, hipStream_t stream,
                                 int q_len = 1, int window = 0, float *lse = nullptr) {
    const dim3 grid(num_q_heads * q_len, num_seqs);
    if (static_cast<int64_t>(num_seqs) * num_q_heads * q_len < 2048)
        hipLaunchKernelGGL((stream_reduce_kernel<T, D, 4>), grid, dim3(kWave * 4), 0, stream, out,
                           ws_acc, ws_ml, ws_prefix, context_lens, num_seqs, num_kv_heads, group,
                           block_size, nshares, team_heads, q_len, window, lse);
    else
        hipLaunchKernelGGL((stream_reduce_kernel<T, D, 1>), grid, dim3(kWave), 0, stream, out,
                           ws_acc, ws_ml, ws_prefix, context_lens, num_seqs, num_kv_heads, group,
                           block_size, nshares, team_heads, q_len, window, lse);
    return hipGetLastError();
}

// Stream shares of a partition kernel: one per wave slot it keeps resident
// on the current device, so that every share streams from start to end.
// Work-groups per CU = the smaller of the register limit (occupancy query)
// and the LDS limit (CU LDS / the kernel's static LDS), rounded down to a
// multiple of per_cu_multiple and at most max_per_cu (0: no limit);
// shares = work-groups x waves_per_group (each wave of a work-group streams
// its own share), capped by the workspace's slot count.  The value is cached
// per device and kernel: the kernel is a template argument, since the
// instantiations of one kernel template share a function type (a cache keyed
// by the type would hand one instantiation's count to another).
// PA_STREAM_WAVES overrides it (tuning and tests).  Launch
// ceil(shares / waves_per_group) work-groups.
template <auto kernel>
int stream_waves(int threads, int per_cu_multiple, int cap, int waves_per_group = 1,
                 int max_per_cu = 0) {
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
    int w = cache[dev].load(std::memory_order_relaxed);
    if (w == 0) {
        int cus = 0, per_cu = 0, lds_cu = 0;
        hipFuncAttributes attr{};
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess)
            per_cu = 0;
        if (hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                                  dev) == hipSuccess &&
            hipFuncGetAttributes(&attr, reinterpret_cast<const void *>(kernel)) == hipSuccess &&
            attr.sharedSizeBytes > 0) {
            const int by_lds = lds_cu / static_cast<int>(attr.sharedSizeBytes);
            if (by_lds < per_cu) per_cu = by_lds;
        }
        if (max_per_cu > 0 && per_cu > max_per_cu) per_cu = max_per_cu;
        if (per_cu >= per_cu_multiple) per_cu -= per_cu % per_cu_multiple;
        w = cus * per_cu * waves_per_group;
        if (w <= 0) w = 256;
        if (w > cap) w = cap;
        cache[dev].store(w, std::memory_order_relaxed);
    }
    if (const char *env = std::getenv("PA_STREAM_WAVES")) {  // tuning / tests
        const int v = std::atoi(env);
        if (v >= 1 && v <= cap) w = v;
    }
    return w;
}

}  // namespace
}  // namespace pa

// moe_microbench.hip -- measurement kernels declared in include/moe_microbench.h.
//
// None of these is part of the layer.  They measure, inside the library the
// layer runs in, what its design rests on: the streaming read rate of HBM, the
// cost of a dependent kernel boundary, and the cost of the grid-wide
// exchanges a persistent kernel would need instead of kernel boundaries.
// Every wait is bounded and reports a give-up through a counter, so a grid
// whose blocks are not all resident still ends.
#include <string.h>

#include "../../include/moe.h"
#include "../../include/moe_microbench.h"
#include "moe_internal.h"

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMbThreads = 256;
constexpr int kMaxExchangeBlocks = 2048;
constexpr uint32_t kSpinLimit = 1u << 18;
constexpr uint32_t kSinkMagic = 0x9E3779B9u;

// ---------------------------------------------------------------------------
// streaming read: block b reads the b-th of `gridDim.x` contiguous ranges,
// N 16-byte nontemporal loads per lane in flight before the first use
// ---------------------------------------------------------------------------
// DEP: the layer kernels' dependency first.  Every lane loads 16 bytes of the
// 2 KiB vector `dep` (written by the previous kernel, as the logits or the
// selection are), and its loads of the range start `off` 16-byte units in,
// off = (XOR of those words) & (kMbDepSlack - 1): no load of the range can
// issue before `dep` has arrived.  OUT: at the end block b < 512 writes word b
// of `out` (0 unless its data XOR to the magic constant).
constexpr uint64_t kMbDepSlack = 4096;  // 16-byte units past `bytes` that src must hold
template <int N, bool DEP, bool OUT>
__global__ __launch_bounds__(kMbThreads) void k_mb_read(const u32x4_t *__restrict__ p, uint64_t n16,
                                                        uint32_t *sink, const u32x4_t *__restrict__ dep,
                                                        uint32_t *out) {
    const uint64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    uint64_t begin = (uint64_t)blockIdx.x * per;
    uint64_t end = begin + per < n16 ? begin + per : n16;
    if constexpr (DEP) {
        const u32x4_t d = dep[threadIdx.x & 127];
        const uint64_t off = (uint64_t)((d.x ^ d.y ^ d.z ^ d.w) & (uint32_t)(kMbDepSlack - 1));
        begin += off;
        end += off;
    }
    uint32_t acc = 0;
    for (uint64_t i = begin + threadIdx.x; i < end; i += (uint64_t)kMbThreads * N) {
        u32x4_t v[N];
#pragma unroll
        for (int u = 0; u < N; ++u) {
            const uint64_t j = i + (uint64_t)u * kMbThreads;
            v[u] = __builtin_nontemporal_load(p + (j < end ? j : begin));  // past the range: re-read a valid word
        }
#pragma unroll
        for (int u = 0; u < N; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == kSinkMagic) sink[threadIdx.x & 3] = acc;
    if constexpr (OUT) {
        if (threadIdx.x == 0 && blockIdx.x < 512) out[blockIdx.x] = acc == kSinkMagic ? 1u : 0u;
    }
}

__global__ __launch_bounds__(kMbThreads) void k_mb_empty(uint32_t *p) {
    if (p && threadIdx.x == 0 && blockIdx.x == 0x7FFFFFFFu) p[0] = 0;
}

// ---------------------------------------------------------------------------
// exchanges.  Layout of the buffer in 32-bit words (one 256-byte line per
// counter): [0] give-ups, [64] generation, then `groups` arrival counters, a
// top counter, `groups` replicas of the generation, `groups` exit counters,
// an exit top counter, and one 64-bit slot per block.
// ---------------------------------------------------------------------------
struct XLayout {
    int groups;
    __host__ __device__ int gen() const { return 64; }
    __host__ __device__ int ctr(int g) const { return 128 + 64 * g; }
    __host__ __device__ int top() const { return 128 + 64 * groups; }
    __host__ __device__ int rep(int g) const { return 128 + 64 * (groups + 1) + 64 * g; }
    __host__ __device__ int exitc(int g) const { return 128 + 64 * (2 * groups + 1) + 64 * g; }
    __host__ __device__ int exit_top() const { return 128 + 64 * (3 * groups + 1); }
    __host__ __device__ int slots() const { return 128 + 64 * (3 * groups + 2); }
    __host__ __device__ size_t words(int blocks) const { return (size_t)slots() + 2 * (size_t)blocks; }
};

// polls are relaxed agent-scope loads (they bypass the caches that are not
// coherent across XCDs); a wait that succeeds is followed by one acquire
// fence (an acquire load in the loop would invalidate the L2 on every poll)
__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_release(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_acq_rel(uint32_t *p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void acquire_fence() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

// two-level arrival: returns true in the block that arrives last of all
// (both levels' counters are reset by their last arrivals)
__device__ __forceinline__ bool arrive_last(uint32_t *w, int c_first, int c_top, int g, int members, int groups) {
    const uint32_t old = add_acq_rel(w + c_first + 64 * g, 1u);
    if (old + 1 != (uint32_t)members) return false;
    st_release(w + c_first + 64 * g, 0u);
    const uint32_t old2 = add_acq_rel(w + c_top, 1u);
    if (old2 + 1 != (uint32_t)groups) return false;
    st_release(w + c_top, 0u);
    return true;
}

// the generation advances once every block has left (two-level exit
// counters).  Relaxed: these words guard no other data (the exchanged words
// carry their own tags), so no cache write-back or invalidation is needed
__device__ __forceinline__ uint32_t add_relaxed(uint32_t *p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void leave(uint32_t *w, const XLayout &L, int g, int members, int groups, uint32_t next) {
    if (add_relaxed(w + L.exitc(g), 1u) + 1 != (uint32_t)members) return;
    st_relaxed(w + L.exitc(g), 0u);
    if (add_relaxed(w + L.exit_top(), 1u) + 1 != (uint32_t)groups) return;
    st_relaxed(w + L.exit_top(), 0u);
    st_relaxed(w + L.gen(), next);
}

__global__ __launch_bounds__(kMbThreads) void k_mb_exchange(int kind, int groups, uint32_t *w) {
    const XLayout L{groups};
    const int b = blockIdx.x, g = b % groups, members = gridDim.x / groups;
    const int lane = threadIdx.x;
    if (kind == 0) {
        if (lane == 0) __hip_atomic_fetch_add(w + L.ctr(g), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    if (threadIdx.x >= 64) {  // only wave 0 takes part; the other waves wait at the block's end
        __syncthreads();
        return;
    }
    const uint32_t gen0 = ld_relaxed(w + L.gen());
    uint64_t *slot = (uint64_t *)(w + L.slots());
    if (kind == 1 || kind == 2) {
        if (lane == 0) {
            if (arrive_last(w, L.ctr(0), L.top(), g, members, groups)) {
                if (kind == 2)
                    for (int r = 0; r < groups; ++r) st_release(w + L.rep(r), gen0 + 1);
                st_release(w + L.gen(), gen0 + 1);
            }
            const uint32_t *poll = (kind == 2) ? w + L.rep(g) : w + L.gen();
            uint32_t spins = 0;
            while (ld_relaxed(poll) == gen0) {
                if (++spins > kSpinLimit) {
                    add_acq_rel(w, 1u);
                    break;
                }
            }
            acquire_fence();
        }
    } else if (kind == 3) {
        const uint32_t tag = gen0 + 1;
        if (lane == 0)
            __hip_atomic_store(slot + b, ((uint64_t)tag << 32) | (uint32_t)b, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        uint32_t spins = 0;
        while (true) {
            bool ok = true;
            for (int i = lane; i < (int)gridDim.x; i += 64) {
                const uint64_t v = __hip_atomic_load(slot + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ok = ok && (uint32_t)(v >> 32) == tag;
            }
            if (__all(ok)) break;
            if (++spins > kSpinLimit) {
                if (lane == 0) add_acq_rel(w, 1u);
                break;
            }
        }
        if (lane == 0) leave(w, L, g, members, groups, tag);
    } else {  // kind 4: the first half of the blocks produce, the second half consume
        const int P = gridDim.x / 2;
        const uint32_t tag = gen0 + 1;
        if (b < P) {
            if (lane == 0) {
                __hip_atomic_store(slot + b, ((uint64_t)tag << 32) | (uint32_t)b, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                add_relaxed(w + L.ctr(b % groups), 1u);  // the slot carries its own tag
            }
        } else {
            // lanes g < groups poll counter g until the producers have all arrived
            uint32_t spins = 0;
            while (true) {
                const uint32_t c = lane < groups ? ld_relaxed(w + L.ctr(lane)) : 0u;
                uint32_t tot = c;
                for (int d = 1; d < 64; d <<= 1) tot += __shfl_xor(tot, d);
                if (tot >= (uint32_t)P * tag) break;
                if (++spins > kSpinLimit) {
                    if (lane == 0) add_acq_rel(w, 1u);
                    break;
                }
            }
            // then every producer's word, which must carry this call's tag (a
            // word seen before its store landed is counted as a give-up)
            bool ok = true;
            for (int i = lane; i < P; i += 64) {
                const uint64_t v = __hip_atomic_load(slot + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ok = ok && (uint32_t)(v >> 32) == tag;
            }
            if (!__all(ok) && lane == 0) add_acq_rel(w, 1u);
        }
        if (lane == 0) leave(w, L, g, members, groups, tag);
    }
    __syncthreads();
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int hip_rc(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

bool exchange_args_ok(int32_t blocks, int32_t groups) {
    return blocks >= 1 && blocks <= kMaxExchangeBlocks && groups >= 1 && groups <= blocks && blocks % groups == 0;
}

}  // namespace

extern "C" {

int moe_mb_stream_read(const void *src, size_t bytes, int32_t blocks, int32_t in_flight, void *sink, void *stream) {
    if (!src || !sink || bytes < 16 || bytes % 16 != 0) return MOE_ERR_INVALID_ARG;
    if (blocks < 1 || blocks > 65536) return MOE_ERR_INVALID_ARG;
    if (!aligned(src, 16) || !aligned(sink, 16)) return MOE_ERR_ALIGNMENT;
    const hipStream_t st = (hipStream_t)stream;
    const u32x4_t *p = (const u32x4_t *)src;
    const uint64_t n16 = bytes / 16;
    (void)hipGetLastError();
    uint32_t *sk = (uint32_t *)sink;
    switch (in_flight) {
        case 1: hipLaunchKernelGGL((k_mb_read<1, false, false>), dim3(blocks), dim3(kMbThreads), 0, st, p, n16, sk, nullptr, nullptr); break;
        case 2: hipLaunchKernelGGL((k_mb_read<2, false, false>), dim3(blocks), dim3(kMbThreads), 0, st, p, n16, sk, nullptr, nullptr); break;
        case 4: hipLaunchKernelGGL((k_mb_read<4, false, false>), dim3(blocks), dim3(kMbThreads), 0, st, p, n16, sk, nullptr, nullptr); break;
        case 8: hipLaunchKernelGGL((k_mb_read<8, false, false>), dim3(blocks), dim3(kMbThreads), 0, st, p, n16, sk, nullptr, nullptr); break;
        default: return MOE_ERR_INVALID_ARG;
    }
    return hip_rc(hipGetLastError());
}

int moe_mb_dependent_read(const void *src, size_t bytes, int32_t blocks, int32_t in_flight, const void *dep,
                          void *out, void *sink, void *stream) {
    if (!src || !out || !sink || bytes < 16 || bytes % 16 != 0) return MOE_ERR_INVALID_ARG;
    if (blocks < 1 || blocks > 65536) return MOE_ERR_INVALID_ARG;
    if (!aligned(src, 16) || !aligned(dep, 16) || !aligned(out, 16) || !aligned(sink, 16)) return MOE_ERR_ALIGNMENT;
    const hipStream_t st = (hipStream_t)stream;
    const u32x4_t *p = (const u32x4_t *)src, *d = (const u32x4_t *)dep;
    uint32_t *sk = (uint32_t *)sink, *o = (uint32_t *)out;
    const uint64_t n16 = bytes / 16;
    (void)hipGetLastError();
#define MB_DEP(N)                                                                                         \
    if (d) hipLaunchKernelGGL((k_mb_read<N, true, true>), dim3(blocks), dim3(kMbThreads), 0, st, p, n16, sk, d, o); \
    else hipLaunchKernelGGL((k_mb_read<N, false, true>), dim3(blocks), dim3(kMbThreads), 0, st, p, n16, sk, d, o)
    switch (in_flight) {
        case 1: MB_DEP(1); break;
        case 2: MB_DEP(2); break;
        case 4: MB_DEP(4); break;
        case 8: MB_DEP(8); break;
        default: return MOE_ERR_INVALID_ARG;
    }
#undef MB_DEP
    return hip_rc(hipGetLastError());
}

int moe_mb_empty(int32_t blocks, void *stream) {
    if (blocks < 1 || blocks > 65536) return MOE_ERR_INVALID_ARG;
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_mb_empty, dim3(blocks), dim3(kMbThreads), 0, (hipStream_t)stream, nullptr);
    return hip_rc(hipGetLastError());
}

size_t moe_mb_exchange_bytes(int32_t blocks, int32_t groups) {
    if (!exchange_args_ok(blocks, groups)) return 0;
    return XLayout{groups}.words(blocks) * 4;
}

int moe_mb_exchange(int32_t kind, int32_t blocks, int32_t groups, void *buf, size_t buf_bytes, void *stream) {
    if (kind < 0 || kind > 4 || !exchange_args_ok(blocks, groups) || !buf) return MOE_ERR_INVALID_ARG;
    if (kind == 4 && (blocks < 2 || blocks % 2 != 0 || groups > 64)) return MOE_ERR_INVALID_ARG;
    if (!aligned(buf, 256)) return MOE_ERR_ALIGNMENT;
    if (buf_bytes < moe_mb_exchange_bytes(blocks, groups)) return MOE_ERR_WORKSPACE;
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_mb_exchange, dim3(blocks), dim3(kMbThreads), 0, (hipStream_t)stream, (int)kind,
                       (int)groups, (uint32_t *)buf);
    return hip_rc(hipGetLastError());
}

int moe_mb_exchange_failures(const void *buf, uint32_t *failures) {
    if (!buf || !failures) return MOE_ERR_INVALID_ARG;
    return hip_rc(hipMemcpy(failures, buf, 4, hipMemcpyDeviceToHost));
}

}  // extern "C"

// moe_gdn.hip -- the GatedDeltaNet recurrent-state update (include/moe_gdn.h).
//
// Per head the state S is 128 x 128 fp32 (64 KiB); row i of S sees only
// v_i and its own entries:
//     s = alpha S_i;  u_i = s . k;  S_i <- s + beta (v_i - u_i) k;  o_i = S_i . q
// so rows are independent and the update streams the state once: each row is
// read into registers, carried through the call's tokens, and written back.
// A wave holds two rows per row-step (32 lanes x 4 floats each), RW row-steps
// of one head; the two dot products per row and token reduce over 32 lanes
// on the VALU (DPP and v_permlane16_swap).  The state is 64 x 64 KiB = 4 MiB
// per layer at the pages' 64 heads: one token reads and writes it once, HBM
// bound (about 8.4 MB per token with q, k and v).  Sources: the linear-
// attention paragraph of "48GB内存运行397B模型：Flash-Moe的极端量化与SSD流式加载
// 实践", section "Metal GPU管线：手写Kernel与FMA优化" (the scale, matrix-vector
// and rank-one-update routines, 64 heads x 128 x 128).
#include "../../include/moe.h"
#include "../../include/moe_gdn.h"
#include "moe_device.h"

namespace {

using namespace moe;

constexpr int kGdnD = 128;   // d_k = d_v
constexpr int kGdnRw = 2;    // row-steps (two rows each) per wave
constexpr int kGdnStepsPerHead = kGdnD / 2;

__device__ __forceinline__ float dot4(const float4 a, const float4 b) {
    return fmaf(a.w, b.w, fmaf(a.z, b.z, fmaf(a.y, b.y, a.x * b.x)));
}

// The first 14 dwords of arguments (the sizes and every input's pointer) are
// preloaded into SGPRs (the library is built with kernel-argument preloading),
// so no load waits for a read of the argument segment; the output pointer,
// needed only at the stores, is read from it.
template <int RW>
__global__ __launch_bounds__(256) void k_gdn(int n_heads, int T, float *__restrict__ state,
                                             const float *__restrict__ qp, const float *__restrict__ kp,
                                             const float *__restrict__ vp, const float *__restrict__ alphap,
                                             const float *__restrict__ betap, float *__restrict__ outp) {
    static_assert(kGdnStepsPerHead % RW == 0, "a wave's row-steps belong to one head");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 31, half = lane >> 5;
    const int rs0 = (blockIdx.x * 4 + wave) * RW;  // the wave's first row-step
    if (rs0 >= n_heads * kGdnStepsPerHead) return;  // no barrier in this kernel
    const int h = rs0 / kGdnStepsPerHead;
    int row[RW];
    float4 S[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        row[r] = 2 * (rs0 + r - h * kGdnStepsPerHead) + half;  // row of the head's state
        // the state streams through once per call: nontemporal loads (3.76 -> 3.22 us
        // per update at 64 heads) and stores
        const float *src = state + ((size_t)h * kGdnD + row[r]) * kGdnD + 4 * lr;
        S[r] = make_float4(__builtin_nontemporal_load(src), __builtin_nontemporal_load(src + 1),
                           __builtin_nontemporal_load(src + 2), __builtin_nontemporal_load(src + 3));
    }
    for (int t = 0; t < T; ++t) {
        const size_t th = (size_t)t * n_heads + h;
        const float4 kv = *(const float4 *)(kp + th * kGdnD + 4 * lr);
        const float4 qv = *(const float4 *)(qp + th * kGdnD + 4 * lr);
        const float alpha = alphap[th], beta = betap[th];
        float vv[RW];
#pragma unroll
        for (int r = 0; r < RW; ++r) vv[r] = vp[th * kGdnD + row[r]];
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            // scale: the decayed state
            float4 s = make_float4(alpha * S[r].x, alpha * S[r].y, alpha * S[r].z, alpha * S[r].w);
            // matrix-vector product: the value the decayed state holds at k
            const float u = lane_sum<32>(dot4(s, kv));
            // rank-one update with the delta-rule correction beta (v - u)
            const float w = beta * (vv[r] - u);
            s.x = fmaf(w, kv.x, s.x);
            s.y = fmaf(w, kv.y, s.y);
            s.z = fmaf(w, kv.z, s.z);
            s.w = fmaf(w, kv.w, s.w);
            S[r] = s;
            // matrix-vector product: the head's output
            const float o = lane_sum<32>(dot4(s, qv));
            // (the empty asm keeps the output pointer's read out of the loop
            // head, so that the first token's loads do not wait for it)
            float *op = outp;
            asm volatile("" : "+s"(op));
            if (lr == 0) op[th * kGdnD + row[r]] = o;
        }
    }
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        float *dst = state + ((size_t)h * kGdnD + row[r]) * kGdnD + 4 * lr;
        __builtin_nontemporal_store(S[r].x, dst);
        __builtin_nontemporal_store(S[r].y, dst + 1);
        __builtin_nontemporal_store(S[r].z, dst + 2);
        __builtin_nontemporal_store(S[r].w, dst + 3);
    }
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

extern "C" int moe_gdn_update(int32_t n_heads, int32_t d_k, int32_t d_v, int32_t n_tokens, float *state,
                              const float *q, const float *k, const float *v, const float *alpha,
                              const float *beta, float *out, void *stream) {
    if (n_heads < 1 || n_heads > 4096 || d_k < 1 || d_v < 1 || n_tokens < 1 || n_tokens > 65535)
        return MOE_ERR_INVALID_ARG;
    if (d_k != kGdnD || d_v != kGdnD) return MOE_ERR_UNSUPPORTED;
    if (!state || !q || !k || !v || !alpha || !beta || !out) return MOE_ERR_INVALID_ARG;
    if (!aligned(state, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 4) || !aligned(alpha, 4) ||
        !aligned(beta, 4) || !aligned(out, 4))
        return MOE_ERR_ALIGNMENT;
    const int waves = n_heads * kGdnStepsPerHead / kGdnRw;
    const int blocks = (waves + 3) / 4;
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_gdn<kGdnRw>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (int)n_heads, (int)n_tokens,
                       state, q, k, v, alpha, beta, out);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

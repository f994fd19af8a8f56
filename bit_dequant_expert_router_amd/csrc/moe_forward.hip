// moe_forward.hip -- the expert layer as three stream-ordered kernels.
//
//   k_router : two-pass RMSNorm + router GEMV (E rows) + shared-gate logit
//   k_gateup : per block, softmax/top-K/renormalise from the logits, then the
//              fused gate+up dequant GEMV of one selected (or the shared)
//              expert with SwiGLU in registers
//   k_down   : down-projection dequant GEMV of all K+1 experts for a set of
//              output rows, weighted combine, sigmoid-gated shared expert and
//              residual, written once per row (no atomics, deterministic)
//
// Sources of each step: RMSNorm in two passes, the FMA form of the 4-bit
// dequant mat-vec, fused SwiGLU, fused combine + residual + sigmoid gate:
// "48GB内存运行397B模型：Flash-Moe的极端量化与SSD流式加载实践", section
// "Metal GPU管线：手写Kernel与FMA优化"; routing GEMV then softmax + top-K:
// flash-moe README translation, "Pipeline mỗi lớp".
//
// Quantised GEMV: a lane owns a contiguous slice of the reduction axis (its
// slice of the activation vector stays in registers) and walks rows.  Each
// 64-entry group is folded:  sum_i (q_i s + b) h_i = s * sum_i q_i h_i + b * X,
// X = sum_i h_i over the group (computed once per token) -- one FMA per weight,
// the kernel-level form of the pages' fma(nibble, scale*x, bias*x) rewrite.
#include "moe_internal.h"

namespace moe {

namespace {

__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_val(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// Sum over aligned groups of `width` lanes (a power of two <= 64); every lane
// of a group receives the group's sum.
__device__ __forceinline__ float lane_group_sum(float v, int width) {
    for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float sigmoidf_(float t) { return 1.0f / (1.0f + expf(-t)); }

// Order-preserving key: larger logit first, then smaller expert index.
__device__ __forceinline__ uint64_t route_key(float z, int e) {
    uint32_t u = (z == 0.0f) ? 0u : __float_as_uint(z);  // -0 and +0 are one key
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)(~(uint32_t)e);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
    return ((uint64_t)hi << 32) | lo;
}

// Softmax -> top-K -> renormalise for one token, by the 64 lanes of one wave.
// Results land in sel[K] / w[K] (LDS), written by lane 0.
__device__ void route_wave(const float *z, int E, int K, int *sel, float *w) {
    const int lane = threadIdx.x & 63;
    constexpr int kPer = kMaxExperts / 64;
    uint64_t key[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = lane + 64 * i;
        key[i] = (e < E) ? route_key(z[e], e) : 0ull;
    }
    float zsel[kMaxTopK];
    int isel[kMaxTopK];
    for (int k = 0; k < K; ++k) {
        uint64_t best = 0ull;
#pragma unroll
        for (int i = 0; i < kPer; ++i) best = key[i] > best ? key[i] : best;
        for (int o = 32; o > 0; o >>= 1) {
            const uint64_t other = shfl_xor_u64(best, o);
            best = other > best ? other : best;
        }
        const int e = (int)(~(uint32_t)best);
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            if (key[i] == best) key[i] = 0ull;
        isel[k] = e;
        zsel[k] = z[e];
    }
    // softmax restricted to the selection == renormalised full softmax
    float denom = 0.0f;
    for (int k = 0; k < K; ++k) denom += expf(zsel[k] - zsel[0]);
    if (lane == 0) {
        for (int k = 0; k < K; ++k) {
            sel[k] = isel[k];
            w[k] = expf(zsel[k] - zsel[0]) / denom;
        }
    }
}

// ---------------------------------------------------------------------------
// quantised dot product of one row slice with the lane's activation slice
// ---------------------------------------------------------------------------
template <int BITS, int CPL>
struct QSlice {
    static constexpr int C = 128 / BITS;          // codes per 16-byte chunk
    static constexpr int D = 32 / BITS;           // codes per dword
    static constexpr int NV = CPL * C;            // codes per lane per row
    static constexpr int GL = NV < 64 ? NV : 64;  // codes of one group inside the slice
    static constexpr int NGL = NV / GL;           // groups touched by the slice
    static constexpr uint32_t kByteMask = BITS == 4 ? 0x0F0F0F0Fu : 0x03030303u;
};

template <int BITS, int CPL>
__device__ __forceinline__ float qdot(const uint8_t *__restrict__ codes_row,
                                      const uint32_t *__restrict__ sb_row, int lr, int lpr,
                                      const float (&hv)[QSlice<BITS, CPL>::NV],
                                      const float (&X)[QSlice<BITS, CPL>::NGL], int g0) {
    using Q = QSlice<BITS, CPL>;
    float accg[Q::NGL];
#pragma unroll
    for (int g = 0; g < Q::NGL; ++g) accg[g] = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const uint4 v = *(const uint4 *)(codes_row + 16 * (lr + lpr * j));
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
#pragma unroll
            for (int n = 0; n < 8 / BITS; ++n) {
                const uint32_t m = (d[w4] >> (BITS * n)) & Q::kByteMask;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int i = j * Q::C + w4 * Q::D + 4 * n + b;
                    accg[i / Q::GL] = fmaf((float)((m >> (8 * b)) & 0xFFu), hv[i], accg[i / Q::GL]);
                }
            }
        }
    }
    float total = 0.0f;
#pragma unroll
    for (int g = 0; g < Q::NGL; ++g) {
        const uint32_t sb = sb_row[g0 + g];
        total = fmaf(bf16_lo(sb), accg[g], total);
        total = fmaf(bf16_hi(sb), X[g], total);
    }
    return total;
}

// ---------------------------------------------------------------------------
// k_router
// ---------------------------------------------------------------------------
template <int CPLR>
__global__ __launch_bounds__(256) void k_router(FwdArgs a) {
    const int t = blockIdx.y;
    const int H = a.s.H, E = a.s.E;
    const float *x = a.x + (size_t)t * H;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __shared__ float red[4];

    // pass 1: sum of squares
    float ss = 0.0f;
    for (int i = threadIdx.x; i < H; i += 256) ss = fmaf(x[i], x[i], ss);
    ss = lane_group_sum(ss, 64);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    const float total = (red[0] + red[1]) + (red[2] + red[3]);
    const float inv = 1.0f / sqrtf(total / (float)H + a.s.eps);

    // pass 2: scale (block 0 stores h for the expert kernels)
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i < H; i += 256) a.ws.h[(size_t)t * H + i] = x[i] * inv * bf16_val(a.gamma[i]);

    const int nch = H / 8;  // 16-byte chunks of 8 bf16 per router row
    const int lpr = nch < 64 ? nch : 64;
    const int rpi = 64 / lpr;
    const int lr = lane % lpr, rsub = lane / lpr;
    float hv[CPLR * 8];
#pragma unroll
    for (int j = 0; j < CPLR; ++j) {
        const int k0 = 8 * (lr + lpr * j);
#pragma unroll
        for (int m = 0; m < 8; ++m) hv[8 * j + m] = x[k0 + m] * inv * bf16_val(a.gamma[k0 + m]);
    }
    const int nrg = (E + 1 + rpi - 1) / rpi;
    for (int rg = blockIdx.x * 4 + wave; rg < nrg; rg += gridDim.x * 4) {
        const int r = rg * rpi + rsub;
        float acc = 0.0f;
        if (r <= E) {
            const uint16_t *row = (r < E) ? a.router + (size_t)r * H : a.sgate;
#pragma unroll
            for (int j = 0; j < CPLR; ++j) {
                const uint4 v = *(const uint4 *)(row + 8 * (lr + lpr * j));
                const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc = fmaf(bf16_lo(d[q]), hv[8 * j + 2 * q], acc);
                    acc = fmaf(bf16_hi(d[q]), hv[8 * j + 2 * q + 1], acc);
                }
            }
        }
        acc = lane_group_sum(acc, lpr);
        if (r <= E && lr == 0) {
            if (r < E)
                a.ws.z[(size_t)t * E + r] = acc;
            else
                a.ws.gs[t] = acc;
        }
    }
}

// ---------------------------------------------------------------------------
// k_gateup
// ---------------------------------------------------------------------------
template <int BITS, int CPL>
__global__ __launch_bounds__(256) void k_gateup(FwdArgs a) {
    using Q = QSlice<BITS, CPL>;
    const int t = blockIdx.z, slot = blockIdx.y;
    const int H = a.s.H, F = a.s.F, E = a.s.E, K = a.s.K;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __shared__ int s_sel[kMaxTopK];
    __shared__ float s_w[kMaxTopK];
    if (wave == 0) route_wave(a.ws.z + (size_t)t * E, E, K, s_sel, s_w);
    __syncthreads();
    if (blockIdx.x == 0 && slot == 0) {
        if (threadIdx.x < K) {
            const int k = threadIdx.x;
            a.ws.sel[t * K + k] = s_sel[k];
            a.ws.coef[t * (K + 1) + k] = s_w[k];
            if (a.route_idx) a.route_idx[t * K + k] = s_sel[k];
            if (a.route_w) a.route_w[t * K + k] = s_w[k];
        } else if (threadIdx.x == K) {
            a.ws.coef[t * (K + 1) + K] = sigmoidf_(a.ws.gs[t]);
        }
    }
    const uint8_t *ex = (slot < K) ? a.experts + (size_t)s_sel[slot] * a.L.bytes : a.shared;
    const QMat &G = a.L.m[0];
    const QMat &U = a.L.m[1];
    const int lpr = G.lpr, rpi = 64 / lpr;
    const int lr = lane % lpr, rsub = lane / lpr;
    const int k0 = lr * Q::NV;
    const float *h = a.ws.h + (size_t)t * H;
    float hv[Q::NV];
#pragma unroll
    for (int i = 0; i < Q::NV; ++i) hv[i] = h[k0 + i];
    float X[Q::NGL];
#pragma unroll
    for (int g = 0; g < Q::NGL; ++g) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < Q::GL; ++i) s += hv[g * Q::GL + i];
        X[g] = s;
    }
    const int g0 = k0 / kGroup;
    const int nrg = F / rpi;
    float *act = a.ws.act + ((size_t)t * (K + 1) + slot) * F;
    for (int rg = blockIdx.x * 4 + wave; rg < nrg; rg += gridDim.x * 4) {
        const int r = rg * rpi + rsub;
        float g = qdot<BITS, CPL>(ex + G.codes_off + (size_t)r * G.row_bytes,
                                  (const uint32_t *)(ex + G.sb_off) + (size_t)r * G.ngroups, lr, lpr, hv, X, g0);
        float u = qdot<BITS, CPL>(ex + U.codes_off + (size_t)r * U.row_bytes,
                                  (const uint32_t *)(ex + U.sb_off) + (size_t)r * U.ngroups, lr, lpr, hv, X, g0);
        g = lane_group_sum(g, lpr);
        u = lane_group_sum(u, lpr);
        if (lr == 0) act[r] = g * sigmoidf_(g) * u;
    }
}

// ---------------------------------------------------------------------------
// k_down
// ---------------------------------------------------------------------------
template <int BITS, int CPL, int RPW>
__global__ __launch_bounds__(256) void k_down(FwdArgs a) {
    using Q = QSlice<BITS, CPL>;
    const int t = blockIdx.y;
    const int H = a.s.H, F = a.s.F, E = a.s.E, K = a.s.K;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __shared__ int s_e[kMaxTopK + 1];
    __shared__ float s_c[kMaxTopK + 1];
    if (threadIdx.x <= K) {
        s_e[threadIdx.x] = threadIdx.x < K ? a.ws.sel[t * K + threadIdx.x] : E;
        s_c[threadIdx.x] = a.ws.coef[t * (K + 1) + threadIdx.x];
    }
    __syncthreads();
    const QMat &Dm = a.L.m[2];
    const int lpr = Dm.lpr, rpi = 64 / lpr;
    const int lr = lane % lpr, rsub = lane / lpr;
    const int k0 = lr * Q::NV;
    const int g0 = k0 / kGroup;
    const int nrg = H / rpi;
    const int rg0 = (blockIdx.x * 4 + wave) * RPW;
    float acc[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) acc[i] = 0.0f;
    for (int s = 0; s <= K; ++s) {
        const uint8_t *ex = (s < K) ? a.experts + (size_t)s_e[s] * a.L.bytes : a.shared;
        const float c = s_c[s];
        const float *av = a.ws.act + ((size_t)t * (K + 1) + s) * F + k0;
        float hv[Q::NV];
#pragma unroll
        for (int i = 0; i < Q::NV; ++i) hv[i] = av[i];
        float X[Q::NGL];
#pragma unroll
        for (int g = 0; g < Q::NGL; ++g) {
            float sum = 0.0f;
#pragma unroll
            for (int i = 0; i < Q::GL; ++i) sum += hv[g * Q::GL + i];
            X[g] = sum;
        }
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int rg = rg0 + i;
            if (rg < nrg) {
                const int r = rg * rpi + rsub;
                const float p = qdot<BITS, CPL>(ex + Dm.codes_off + (size_t)r * Dm.row_bytes,
                                                (const uint32_t *)(ex + Dm.sb_off) + (size_t)r * Dm.ngroups, lr,
                                                lpr, hv, X, g0);
                acc[i] = fmaf(c, p, acc[i]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int rg = rg0 + i;
        const float v = lane_group_sum(acc[i], lpr);
        if (rg < nrg && lr == 0) {
            const int r = rg * rpi + rsub;
            const size_t o = (size_t)t * H + r;
            a.y[o] = a.x[o] + v;
        }
    }
}

template <int BITS>
hipError_t launch_bits(const FwdArgs &a, hipStream_t st) {
    const int H = a.s.H, F = a.s.F, E = a.s.E, K = a.s.K, T = a.T;
    // router
    {
        const int nch = H / 8, lpr = nch < 64 ? nch : 64, cplr = nch / lpr, rpi = 64 / lpr;
        const int nrg = (E + 1 + rpi - 1) / rpi;
        const int blocks = (nrg + 3) / 4;
        dim3 grid(blocks, T);
        switch (cplr) {
            case 1: hipLaunchKernelGGL(k_router<1>, grid, dim3(256), 0, st, a); break;
            case 2: hipLaunchKernelGGL(k_router<2>, grid, dim3(256), 0, st, a); break;
            case 4: hipLaunchKernelGGL(k_router<4>, grid, dim3(256), 0, st, a); break;
            case 8: hipLaunchKernelGGL(k_router<8>, grid, dim3(256), 0, st, a); break;
            default: return hipErrorInvalidValue;
        }
    }
    // gate/up
    {
        const QMat &G = a.L.m[0];
        const int rpi = 64 / G.lpr;
        const int nrg = F / rpi;
        int blocks = (nrg + 7) / 8;  // ~2 row groups per wave
        if (blocks < 1) blocks = 1;
        dim3 grid(blocks, K + 1, T);
        switch (G.cpl) {
            case 1: hipLaunchKernelGGL((k_gateup<BITS, 1>), grid, dim3(256), 0, st, a); break;
            case 2: hipLaunchKernelGGL((k_gateup<BITS, 2>), grid, dim3(256), 0, st, a); break;
            default: return hipErrorInvalidValue;
        }
    }
    // down + combine
    {
        const QMat &Dm = a.L.m[2];
        const int rpi = 64 / Dm.lpr;
        const int nrg = H / rpi;
        constexpr int RPW = 2;
        const int blocks = (nrg + 4 * RPW - 1) / (4 * RPW);
        dim3 grid(blocks, T);
        switch (Dm.cpl) {
            case 1: hipLaunchKernelGGL((k_down<BITS, 1, RPW>), grid, dim3(256), 0, st, a); break;
            case 2: hipLaunchKernelGGL((k_down<BITS, 2, RPW>), grid, dim3(256), 0, st, a); break;
            default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_forward(const FwdArgs &a, hipStream_t stream) {
    (void)hipGetLastError();  // report only this call's launches
    if (a.s.bits == 4) return launch_bits<4>(a, stream);
    if (a.s.bits == 2) return launch_bits<2>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace moe

// moe_forward.hip -- the expert layer as three stream-ordered kernels.
//
//   k_router : two-pass RMSNorm + router GEMV (E rows) + shared-gate logit;
//              a few blocks also store h in the fixed-point limb form below
//   k_gateup : per wave, softmax/top-K/renormalise from the logits, then the
//              fused gate+up dequant GEMV of the selected experts and the
//              shared expert with SwiGLU in registers
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
// Dequantised dot products.  A lane owns a contiguous slice of the reduction
// axis and walks rows; a 64-entry group with scale s and bias b contributes
//     sum_i (q_i s + b) v_i = s * sum_i q_i v_i + b * sum_i v_i,
// the group-level form of the pages' fma(nibble, scale*x, bias*x) rewrite.
// The code products sum_i q_i v_i are taken exactly in integers: each group of
// the activation vector v is written as V_i * S with S a power of two
// (max|v| < 2^22 S) and V_i an integer split into three signed 8-bit limbs,
// V = L2*65536 + L1*256 + L0; v_dot4 instructions accumulate q * L per limb
// (4 codes per instruction, exact int32), and one fp32 combination per group
// restores s*S*(D2*65536 + D1*256 + D0).  The only roundings are the 22-bit
// fixed point of v (relative 2^-23 of the group maximum) and fp32 sums,
// comparable to an fp32 dot product; VALU work drops to ~1.2 instructions per
// weight from ~2.3 for convert-and-FMA.
#include "moe_internal.h"

namespace moe {

namespace {

__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

// Sum over aligned groups of `width` lanes (a power of two <= 64); every lane
// of a group receives the group's sum.
__device__ __forceinline__ float lane_group_sum(float v, int width) {
    for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

template <int W>
__device__ __forceinline__ float lane_sum(float v) {
#pragma unroll
    for (int o = W >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

template <int W>
__device__ __forceinline__ float lane_max(float v) {
#pragma unroll
    for (int o = W >> 1; o > 0; o >>= 1) {
        const float u = __shfl_xor(v, o, 64);
        v = (v != v || u != u) ? (v + u) : fmaxf(v, u);
    }
    return v;
}

__device__ __forceinline__ float sigmoidf_(float t) { return 1.0f / (1.0f + expf(-t)); }

// max that keeps a NaN (fmaxf would drop it)
__device__ __forceinline__ float nan_max(float a, float b) { return (a != a || b != b) ? (a + b) : fmaxf(a, b); }

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// streaming 16-byte load of weights that are read once per call
__device__ __forceinline__ uint4 ld_stream16(const void *p) {
    const u32x4_t v = __builtin_nontemporal_load((const u32x4_t *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld_stream4(const uint32_t *p) { return __builtin_nontemporal_load(p); }

// ---------------------------------------------------------------------------
// fixed-point limbs
// ---------------------------------------------------------------------------
// Exponent e with max|v| < 2^e, clamped so that 2^(e-22) and 2^(22-e) are
// normal floats.  NaN / inf maxima give e = 255 (flagged by limb_scale).
__device__ __forceinline__ int limb_exponent(float m) {
    const uint32_t E = (__float_as_uint(m) >> 23) & 0xFFu;
    int e = (E == 0 ? 1 : (int)E) - 126;  // m < 2^e
    return e < -100 ? -100 : e;
}
__device__ __forceinline__ float pow2f(int p) { return __uint_as_float((uint32_t)(p + 127) << 23); }
// scale S of a group: 2^(e-22), or NaN when the group holds a NaN or an inf
__device__ __forceinline__ float limb_scale(float m) {
    return (m <= 3.4028234663852886e38f) ? pow2f(limb_exponent(m) - 22) : __uint_as_float(0x7FC00000u);
}
// integer V = rint(v / S) for finite groups (|V| <= 2^22), 0 otherwise
__device__ __forceinline__ int limb_value(float v, float m) {
    if (!(m <= 3.4028234663852886e38f)) return 0;
    return (int)rintf(v * pow2f(22 - limb_exponent(m)));
}
__device__ __forceinline__ void limb_split(int V, int &l0, int &l1, int &l2) {
    l0 = ((V + 128) & 255) - 128;
    const int v1 = (V - l0) >> 8;
    l1 = ((v1 + 128) & 255) - 128;
    l2 = (v1 - l1) >> 8;
}

// ---------------------------------------------------------------------------
// routing: softmax -> top-K -> renormalise, by one wave.  Lane k < K ends up
// holding the k-th selected expert and its renormalised weight.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t route_key(float z, int e) {
    uint32_t u = (z == 0.0f) ? 0u : __float_as_uint(z);  // -0 and +0 are one key
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)(~(uint32_t)e);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)v, o, 64);
        const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
        const uint64_t other = ((uint64_t)hi << 32) | lo;
        v = other > v ? other : v;
    }
    return v;
}

__device__ __forceinline__ float route_key_value(uint64_t key) {
    const uint32_t u = (uint32_t)(key >> 32);
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

__device__ __forceinline__ void route_wave(const float *__restrict__ z, int E, int K, int &my_sel, float &my_w) {
    const int lane = threadIdx.x & 63;
    constexpr int kPer = kMaxExperts / 64;
    float zv[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {  // unconditional (clamped) loads: all in flight at once
        const int e = lane + 64 * i;
        zv[i] = z[e < E ? e : E - 1];
    }
    uint64_t key[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = lane + 64 * i;
        key[i] = (e < E) ? route_key(zv[i], e) : 0ull;
    }
    my_sel = 0;
    float my_z = 0.0f;
    for (int k = 0; k < K; ++k) {
        uint64_t best = 0ull;
#pragma unroll
        for (int i = 0; i < kPer; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_u64(best);
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            if (key[i] == best) key[i] = 0ull;
        if (lane == k) {
            my_sel = (int)(~(uint32_t)best);
            my_z = route_key_value(best);
        }
    }
    // softmax restricted to the selection == renormalised full softmax
    const float z0 = __shfl(my_z, 0, 64);
    const float p = (lane < K) ? expf(my_z - z0) : 0.0f;
    const float denom = lane_sum<64>(p);
    my_w = p / denom;
}

// ---------------------------------------------------------------------------
// dequantised dot product of one row slice with a lane's limb slice
// ---------------------------------------------------------------------------
template <int BITS, int CPL>
struct QSlice {
    static constexpr int C = 128 / BITS;          // codes per 16-byte chunk
    static constexpr int D = 32 / BITS;           // codes per dword
    static constexpr int NV = CPL * C;            // codes per lane per row
    static constexpr int NL = NV / 4;             // limb dwords per limb
    static constexpr int GL = NV < 64 ? NV : 64;  // codes of one group inside the slice
    static constexpr int NGL = NV / GL;           // groups touched by the slice
    static constexpr uint32_t kByteMask = BITS == 4 ? 0x0F0F0F0Fu : 0x03030303u;
};

template <int BITS, int CPL>
struct LimbSlice {
    using Q = QSlice<BITS, CPL>;
    int L[3][Q::NL];
    float S[Q::NGL];  // group scale (power of two)
    float X[Q::NGL];  // sum of the activations of the slice within the group
};

template <int BITS, int CPL>
__device__ __forceinline__ float qdot(const uint4 (&c)[CPL], const uint32_t (&sb)[QSlice<BITS, CPL>::NGL],
                                      const LimbSlice<BITS, CPL> &v) {
    using Q = QSlice<BITS, CPL>;
    int acc[Q::NGL][3];
#pragma unroll
    for (int g = 0; g < Q::NGL; ++g) acc[g][0] = acc[g][1] = acc[g][2] = 0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const uint32_t d[4] = {c[j].x, c[j].y, c[j].z, c[j].w};
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
#pragma unroll
            for (int n = 0; n < 8 / BITS; ++n) {
                const int m = (int)((d[w4] >> (BITS * n)) & Q::kByteMask);
                const int li = (j * Q::C + w4 * Q::D) / 4 + n;  // limb dword of these 4 codes
                const int g = (4 * li) / Q::GL;
#pragma unroll
                for (int x = 0; x < 3; ++x) acc[g][x] = __builtin_amdgcn_sdot4(m, v.L[x][li], acc[g][x], false);
            }
        }
    }
    float total = 0.0f;
#pragma unroll
    for (int g = 0; g < Q::NGL; ++g) {
        const float f = fmaf((float)acc[g][2], 65536.0f, fmaf((float)acc[g][1], 256.0f, (float)acc[g][0]));
        total = fmaf(bf16_lo(sb[g]) * v.S[g], f, total);
        total = fmaf(bf16_hi(sb[g]), v.X[g], total);
    }
    return total;
}

template <int BITS, int CPL>
__device__ __forceinline__ void load_row(const uint8_t *__restrict__ ex, const QMat &q, int r, int lr,
                                         uint4 (&c)[CPL], uint32_t (&sb)[QSlice<BITS, CPL>::NGL]) {
    using Q = QSlice<BITS, CPL>;
    const uint8_t *row = ex + q.codes_off + (size_t)r * q.row_bytes;
#pragma unroll
    for (int j = 0; j < CPL; ++j) c[j] = ld_stream16(row + 16 * (lr + q.lpr * j));
    const uint32_t *sbr = (const uint32_t *)(ex + q.sb_off) + (size_t)r * q.ngroups + (lr * Q::NV) / kGroup;
#pragma unroll
    for (int g = 0; g < Q::NGL; ++g) sb[g] = ld_stream4(sbr + g);
}

// ---------------------------------------------------------------------------
// k_router: one router row-step per wave; the first ceil(H/256) blocks also
// write the limb form of h for k_gateup.
// ---------------------------------------------------------------------------
template <int CPLR>
__global__ __launch_bounds__(256) void k_router(FwdArgs a) {
    const int t = blockIdx.y;
    const int H = a.s.H, E = a.s.E;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float *x = a.x + (size_t)t * H;
    const int nch = H / 8;  // 16-byte chunks of 8 bf16 per router row
    const int lpr = nch < 64 ? nch : 64;
    const int rpi = 64 / lpr;
    const int lr = lane % lpr, rsub = lane / lpr;
    const int nrs = (E + 1 + rpi - 1) / rpi;
    const int rs = blockIdx.x * 4 + wave;
    const int r = rs * rpi + rsub;
    const bool has_row = rs < nrs && r <= E;

    // issue the router row loads first
    uint4 wv[CPLR];
    if (has_row) {
        const uint16_t *row = (r < E) ? a.router + (size_t)r * H : a.sgate;
#pragma unroll
        for (int j = 0; j < CPLR; ++j) wv[j] = ld_stream16(row + 8 * (lr + lpr * j));
    }
    // the lane's slice of x and gamma
    float xv[CPLR * 8];
    uint4 gv[CPLR];
#pragma unroll
    for (int j = 0; j < CPLR; ++j) {
        const int k0 = 8 * (lr + lpr * j);
        const float4 x0 = *(const float4 *)(x + k0);
        const float4 x1 = *(const float4 *)(x + k0 + 4);
        xv[8 * j + 0] = x0.x; xv[8 * j + 1] = x0.y; xv[8 * j + 2] = x0.z; xv[8 * j + 3] = x0.w;
        xv[8 * j + 4] = x1.x; xv[8 * j + 5] = x1.y; xv[8 * j + 6] = x1.z; xv[8 * j + 7] = x1.w;
        gv[j] = *(const uint4 *)(a.gamma + k0);
    }
    // pass 1: sum of squares over the whole token (each lane group holds all of x)
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < CPLR * 8; ++i) ss = fmaf(xv[i], xv[i], ss);
    ss = lane_group_sum(ss, lpr);
    const float inv = 1.0f / sqrtf(ss / (float)H + a.s.eps);

    // pass 2 + router dot product
    if (has_row) {
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < CPLR; ++j) {
            const uint32_t w[4] = {wv[j].x, wv[j].y, wv[j].z, wv[j].w};
            const uint32_t g[4] = {gv[j].x, gv[j].y, gv[j].z, gv[j].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc = fmaf(bf16_lo(w[q]), xv[8 * j + 2 * q] * inv * bf16_lo(g[q]), acc);
                acc = fmaf(bf16_hi(w[q]), xv[8 * j + 2 * q + 1] * inv * bf16_hi(g[q]), acc);
            }
        }
        acc = lane_group_sum(acc, lpr);
        if (lr == 0) {
            if (r < E)
                a.ws.z[(size_t)t * E + r] = acc;
            else
                a.ws.gs[t] = acc;
        }
    } else {
        (void)lane_group_sum(0.0f, lpr);
    }

    // limb form of h[256 b .. 256 b + 255]: one wave = one group of 64
    const int k = blockIdx.x * 256 + threadIdx.x;
    if (blockIdx.x * 256 < H) {
        const float h = (k < H) ? x[k] * inv * __uint_as_float((uint32_t)a.gamma[k] << 16) : 0.0f;
        const float m = lane_max<64>(fabsf(h));
        const int V = limb_value(h, m);
        int l0, l1, l2;
        limb_split(V, l0, l1, l2);
        const float half = lane_sum<32>(h);
        if (k < H) {
            int8_t *hl = a.ws.hl + (size_t)t * 3 * H;
            hl[k] = (int8_t)l0;
            hl[H + k] = (int8_t)l1;
            hl[2 * H + k] = (int8_t)l2;
            if (lane == 0) a.ws.hs[(size_t)t * (H / 64) + k / 64] = limb_scale(m);
            if ((lane & 31) == 0) a.ws.hx[(size_t)t * (H / 32) + k / 32] = half;
        }
    }
}

// ---------------------------------------------------------------------------
// k_gateup: RPW row-steps per wave over the (K+1) x F gate/up row pairs
// ---------------------------------------------------------------------------
template <int BITS, int CPL, int RPW>
__global__ __launch_bounds__(256) void k_gateup(FwdArgs a) {
    using Q = QSlice<BITS, CPL>;
    const int t = blockIdx.y;
    const int H = a.s.H, F = a.s.F, E = a.s.E, K = a.s.K;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const QMat &G = a.L.m[0];
    const QMat &U = a.L.m[1];
    const int lpr = G.lpr, rpi = 64 / lpr;
    const int lr = lane % lpr, rsub = lane / lpr;
    const int nrs = (K + 1) * F / rpi;
    const int rs0 = (blockIdx.x * 4 + wave) * RPW;
    if (rs0 >= nrs) return;

    // the lane's limb slice of h
    const int k0 = lr * Q::NV;
    LimbSlice<BITS, CPL> hv;
    {
        const int8_t *hl = a.ws.hl + (size_t)t * 3 * H + k0;
#pragma unroll
        for (int x = 0; x < 3; ++x)
#pragma unroll
            for (int i = 0; i < Q::NL / 4; ++i) {
                const int4 v = *(const int4 *)(hl + (size_t)x * H + 16 * i);
                hv.L[x][4 * i + 0] = v.x; hv.L[x][4 * i + 1] = v.y;
                hv.L[x][4 * i + 2] = v.z; hv.L[x][4 * i + 3] = v.w;
            }
        if constexpr (Q::NL % 4 != 0) {
#pragma unroll
            for (int x = 0; x < 3; ++x)
#pragma unroll
                for (int i = (Q::NL / 4) * 4; i < Q::NL; ++i)
                    hv.L[x][i] = *(const int *)(hl + (size_t)x * H + 4 * i);
        }
#pragma unroll
        for (int g = 0; g < Q::NGL; ++g) {
            hv.S[g] = a.ws.hs[(size_t)t * (H / 64) + k0 / 64 + g];
            float xs = 0.0f;
#pragma unroll
            for (int hh = 0; hh < Q::GL / 32; ++hh) xs += a.ws.hx[(size_t)t * (H / 32) + (k0 + g * 64) / 32 + hh];
            hv.X[g] = xs;
        }
    }

    // routing (every wave that touches a routed expert computes it)
    int my_sel = 0;
    float my_w = 0.0f;
    if ((rs0 * rpi) / F < K) route_wave(a.ws.z + (size_t)t * E, E, K, my_sel, my_w);
    if (blockIdx.x == 0 && wave == 0) {
        if (lane < K) {
            a.ws.sel[t * K + lane] = my_sel;
            a.ws.coef[t * (K + 1) + lane] = my_w;
            if (a.route_idx) a.route_idx[t * K + lane] = my_sel;
            if (a.route_w) a.route_w[t * K + lane] = my_w;
        } else if (lane == K) {
            a.ws.coef[t * (K + 1) + K] = sigmoidf_(a.ws.gs[t]);
        }
    }

    // all weight loads of this wave
    uint4 gc[RPW][CPL], uc[RPW][CPL];
    uint32_t gsb[RPW][Q::NGL], usb[RPW][Q::NGL];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int rs = rs0 + i;
        if (rs < nrs) {
            const int p = rs * rpi + rsub;
            const int s = p / F, j = p % F;
            const int e = __shfl(my_sel, s < K ? s : 0, 64);
            const uint8_t *ex = (s < K) ? a.experts + (size_t)e * a.L.bytes : a.shared;
            load_row<BITS, CPL>(ex, G, j, lr, gc[i], gsb[i]);
            load_row<BITS, CPL>(ex, U, j, lr, uc[i], usb[i]);
        }
    }
    float *act = a.ws.act + (size_t)t * (K + 1) * F;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int rs = rs0 + i;
        if (rs < nrs) {
            float g = qdot<BITS, CPL>(gc[i], gsb[i], hv);
            float u = qdot<BITS, CPL>(uc[i], usb[i], hv);
            g = lane_group_sum(g, lpr);
            u = lane_group_sum(u, lpr);
            if (lr == 0) act[rs * rpi + rsub] = g * sigmoidf_(g) * u;
        }
    }
}

// ---------------------------------------------------------------------------
// k_down: RPW row-steps of the H output rows per wave, all K+1 experts, in
// batches of SB experts whose activations are turned into limbs in LDS.
// ---------------------------------------------------------------------------
template <int BITS, int CPL, int RPW, int SB>
__global__ __launch_bounds__(256) void k_down(FwdArgs a) {
    using Q = QSlice<BITS, CPL>;
    const int t = blockIdx.y;
    const int H = a.s.H, F = a.s.F, E = a.s.E, K = a.s.K;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const QMat &Dm = a.L.m[2];
    const int lpr = Dm.lpr, rpi = 64 / lpr;
    const int lr = lane % lpr, rsub = lane / lpr;
    const int nrs = H / rpi;
    const int rs0 = (blockIdx.x * 4 + wave) * RPW;
    const int k0 = lr * Q::NV;

    extern __shared__ __align__(16) unsigned char smem[];
    int8_t *sl = (int8_t *)smem;                          // [SB][3][F]
    float *ss = (float *)(smem + (size_t)SB * 3 * F);     // [SB][F/64]
    float *sx = ss + SB * (F / 64);                       // [SB][F/32]

    // lane s (s <= K) holds slot s: expert index and combine coefficient
    const int my_e = (lane < K) ? a.ws.sel[t * K + lane] : E;
    const float my_c = (lane <= K) ? a.ws.coef[t * (K + 1) + lane] : 0.0f;

    float acc[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) acc[i] = 0.0f;

    for (int s0 = 0; s0 <= K; s0 += SB) {
        const int nb = (K + 1 - s0) < SB ? (K + 1 - s0) : SB;
        // weight loads of this batch
        uint4 wc[SB][RPW][CPL];
        uint32_t wsb[SB][RPW][Q::NGL];
#pragma unroll
        for (int si = 0; si < SB; ++si) {
            if (si < nb) {
                const int e = __shfl(my_e, s0 + si, 64);
                const uint8_t *ex = (e < E) ? a.experts + (size_t)e * a.L.bytes : a.shared;
#pragma unroll
                for (int i = 0; i < RPW; ++i) {
                    const int rs = rs0 + i;
                    if (rs < nrs) load_row<BITS, CPL>(ex, Dm, rs * rpi + rsub, lr, wc[si][i], wsb[si][i]);
                }
            }
        }
        // limbs of this batch's activations, in LDS
        __syncthreads();
        const float *act = a.ws.act + ((size_t)t * (K + 1) + s0) * F;
        for (int v0 = threadIdx.x * 4; v0 < SB * F; v0 += 1024) {
            const bool live = v0 < nb * F;
            const float4 v = live ? *(const float4 *)(act + v0) : make_float4(0.f, 0.f, 0.f, 0.f);
            float m = nan_max(nan_max(fabsf(v.x), fabsf(v.y)), nan_max(fabsf(v.z), fabsf(v.w)));
            m = lane_max<16>(m);  // 16 lanes x 4 values = one group of 64
            int l[4][3];
            const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) limb_split(limb_value(vv[q], m), l[q][0], l[q][1], l[q][2]);
            const float half = lane_sum<8>(v.x + v.y + v.z + v.w);
            if (live) {
                const int sidx = v0 / F, j = v0 % F;
#pragma unroll
                for (int x = 0; x < 3; ++x) {
                    const uint32_t packed = (uint32_t)(l[0][x] & 255) | ((uint32_t)(l[1][x] & 255) << 8) |
                                            ((uint32_t)(l[2][x] & 255) << 16) | ((uint32_t)(l[3][x] & 255) << 24);
                    *(uint32_t *)(sl + ((size_t)sidx * 3 + x) * F + j) = packed;
                }
                if ((threadIdx.x & 15) == 0) ss[sidx * (F / 64) + j / 64] = limb_scale(m);
                if ((threadIdx.x & 7) == 0) sx[sidx * (F / 32) + j / 32] = half;
            }
        }
        __syncthreads();
        // products of this batch
#pragma unroll
        for (int si = 0; si < SB; ++si) {
            if (si < nb) {
                const float c = __shfl(my_c, s0 + si, 64);
                LimbSlice<BITS, CPL> av;
#pragma unroll
                for (int x = 0; x < 3; ++x)
#pragma unroll
                    for (int i = 0; i < Q::NL; ++i) av.L[x][i] = *(const int *)(sl + ((size_t)si * 3 + x) * F + k0 + 4 * i);
#pragma unroll
                for (int g = 0; g < Q::NGL; ++g) {
                    av.S[g] = ss[si * (F / 64) + k0 / 64 + g];
                    float xs = 0.0f;
#pragma unroll
                    for (int hh = 0; hh < Q::GL / 32; ++hh) xs += sx[si * (F / 32) + (k0 + g * 64) / 32 + hh];
                    av.X[g] = xs;
                }
#pragma unroll
                for (int i = 0; i < RPW; ++i)
                    if (rs0 + i < nrs) acc[i] = fmaf(c, qdot<BITS, CPL>(wc[si][i], wsb[si][i], av), acc[i]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int rs = rs0 + i;
        const float v = lane_group_sum(acc[i], lpr);
        if (rs < nrs && lr == 0) {
            const size_t o = (size_t)t * H + rs * rpi + rsub;
            a.y[o] = a.x[o] + v;
        }
    }
}

constexpr int kRpwGateUp = 5;
constexpr int kRpwDown = 2;
constexpr int kSlotBatch = 5;

template <int BITS>
hipError_t launch_stage(const FwdArgs &a, int stage, hipStream_t st) {
    const int H = a.s.H, F = a.s.F, E = a.s.E, K = a.s.K, T = a.T;
    if (stage == 0) {  // RMSNorm + router + limbs of h
        const int nch = H / 8, lpr = nch < 64 ? nch : 64, cplr = nch / lpr, rpi = 64 / lpr;
        const int nrs = (E + 1 + rpi - 1) / rpi;
        int blocks = (nrs + 3) / 4;
        const int enc_blocks = (H + 255) / 256;
        if (blocks < enc_blocks) blocks = enc_blocks;
        dim3 grid(blocks, T);
        switch (cplr) {
            case 1: hipLaunchKernelGGL(k_router<1>, grid, dim3(256), 0, st, a); break;
            case 2: hipLaunchKernelGGL(k_router<2>, grid, dim3(256), 0, st, a); break;
            case 4: hipLaunchKernelGGL(k_router<4>, grid, dim3(256), 0, st, a); break;
            case 8: hipLaunchKernelGGL(k_router<8>, grid, dim3(256), 0, st, a); break;
            default: return hipErrorInvalidValue;
        }
    } else if (stage == 1) {  // routing + gate/up + SwiGLU
        const QMat &G = a.L.m[0];
        const int rpi = 64 / G.lpr;
        const int nrs = (K + 1) * F / rpi;
        const int blocks = (nrs + 4 * kRpwGateUp - 1) / (4 * kRpwGateUp);
        dim3 grid(blocks, T);
        switch (G.cpl) {
            case 1: hipLaunchKernelGGL((k_gateup<BITS, 1, kRpwGateUp>), grid, dim3(256), 0, st, a); break;
            case 2: hipLaunchKernelGGL((k_gateup<BITS, 2, kRpwGateUp>), grid, dim3(256), 0, st, a); break;
            default: return hipErrorInvalidValue;
        }
    } else if (stage == 2) {  // down + combine + residual
        const QMat &Dm = a.L.m[2];
        const int rpi = 64 / Dm.lpr;
        const int nrs = H / rpi;
        const int blocks = (nrs + 4 * kRpwDown - 1) / (4 * kRpwDown);
        const size_t lds = (size_t)kSlotBatch * 3 * F + (size_t)kSlotBatch * (F / 64) * 4 + (size_t)kSlotBatch * (F / 32) * 4;
        dim3 grid(blocks, T);
        switch (Dm.cpl) {
            case 1: hipLaunchKernelGGL((k_down<BITS, 1, kRpwDown, kSlotBatch>), grid, dim3(256), lds, st, a); break;
            case 2: hipLaunchKernelGGL((k_down<BITS, 2, kRpwDown, kSlotBatch>), grid, dim3(256), lds, st, a); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_stage(const FwdArgs &a, int stage, hipStream_t stream) {
    (void)hipGetLastError();  // report only this call's launches
    if (a.s.bits == 4) return launch_stage<4>(a, stage, stream);
    if (a.s.bits == 2) return launch_stage<2>(a, stage, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_forward(const FwdArgs &a, hipStream_t stream) {
    for (int stage = 0; stage < kForwardStages; ++stage) {
        const hipError_t e = launch_forward_stage(a, stage, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace moe

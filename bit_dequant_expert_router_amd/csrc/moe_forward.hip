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
//
// Gate/up (activation h, the normalised token): the code products sum_i q_i h_i
// are taken exactly in integers.  Each group of h is written as V_i * S with S a
// power of two (max|h| < 2^26 S) and V_i an integer split into seven signed
// base-16 digits (limbs) V = sum_x L_x 16^x, L_x in [-8, 7].  Eight limbs of
// consecutive entries are packed per dword, the operand form of v_dot8_i32_i4;
// the codes q, made signed as q - 8 by one XOR per 8 codes (4-bit), are the other
// operand, so one instruction accumulates 8 exact code x limb products.  Per group
// and limb the sums stay below 2^12; one fp32 combination restores
// s*S*sum_x D_x 16^x, and the -8 folds into the bias term, (b + 8 s) * sum h.
// Values within a factor 4 of their group's maximum are represented exactly
// (a float has 24 significant bits), smaller ones with an absolute error below
// 2^-27 of it, so the result matches an fp32 dot product; the VALU does 1.0
// instruction per weight against ~2.3 for convert-and-FMA.
//
// Down (activation a = SwiGLU output, widely spread magnitudes): fp32, codes
// converted with v_cvt_f32_ubyte (byte code order) and folded per group.
#include "moe_internal.h"

namespace moe {

namespace {

__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// cross-lane reductions on the VALU: DPP quad permutations and row mirrors
// inside 16-lane rows, then v_permlane16_swap / v_permlane32_swap across rows.
// Each step is one VALU instruction (no LDS round trip).  Callers keep every
// lane of a reduced group active.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i inside each half row
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i inside each row

struct SumOp {
    __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};
struct MaxOp {  // keeps a NaN (fmaxf would drop it)
    __device__ __forceinline__ float operator()(float a, float b) const {
        return (a != a || b != b) ? (a + b) : fmaxf(a, b);
    }
};

// reduce over aligned groups of W lanes (W a power of two <= 64); every lane
// of a group receives the result
template <int W, typename Op>
__device__ __forceinline__ float lane_reduce(float v, Op op) {
    if constexpr (W >= 2) v = op(v, __uint_as_float(dpp_u<kDppXor1>(__float_as_uint(v))));
    if constexpr (W >= 4) v = op(v, __uint_as_float(dpp_u<kDppXor2>(__float_as_uint(v))));
    if constexpr (W >= 8) v = op(v, __uint_as_float(dpp_u<kDppHalfMirror>(__float_as_uint(v))));
    if constexpr (W >= 16) v = op(v, __uint_as_float(dpp_u<kDppMirror>(__float_as_uint(v))));
    if constexpr (W >= 32) {
        const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = op(__uint_as_float(p[0]), __uint_as_float(p[1]));
    }
    if constexpr (W >= 64) {
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = op(__uint_as_float(p[0]), __uint_as_float(p[1]));
    }
    return v;
}

template <int W>
__device__ __forceinline__ float lane_sum(float v) { return lane_reduce<W>(v, SumOp()); }
template <int W>
__device__ __forceinline__ float lane_max(float v) { return lane_reduce<W>(v, MaxOp()); }

// sum over aligned groups of a runtime width (uniform across the wave)
__device__ __forceinline__ float lane_group_sum(float v, int width) {
    switch (width) {
        case 1: return v;
        case 2: return lane_sum<2>(v);
        case 4: return lane_sum<4>(v);
        case 8: return lane_sum<8>(v);
        case 16: return lane_sum<16>(v);
        case 32: return lane_sum<32>(v);
        default: return lane_sum<64>(v);
    }
}

// value of a wave-uniform lane index
__device__ __forceinline__ int lane_bcast(int v, int src) { return __builtin_amdgcn_readlane(v, src); }
__device__ __forceinline__ float lane_bcast(float v, int src) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

__device__ __forceinline__ float sigmoidf_(float t) { return 1.0f / (1.0f + expf(-t)); }

__device__ __forceinline__ float nan_max(float a, float b) { return MaxOp()(a, b); }

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
constexpr int kLimbs = 7;                  // signed base-16 digits
constexpr int kFixBits = 4 * kLimbs - 2;   // |V| <= 2^26

// Exponent e with max|v| < 2^e, clamped so that 2^(e-26) and 2^(26-e) are
// normal floats.  NaN / inf maxima are flagged by limb_scale.
__device__ __forceinline__ int limb_exponent(float m) {
    const uint32_t E = (__float_as_uint(m) >> 23) & 0xFFu;
    int e = (E == 0 ? 1 : (int)E) - 126;  // m < 2^e
    return e < -90 ? -90 : e;
}
__device__ __forceinline__ float pow2f(int p) { return __uint_as_float((uint32_t)(p + 127) << 23); }
// scale S of a group: 2^(e-26), or NaN when the group holds a NaN or an inf
__device__ __forceinline__ float limb_scale(float m) {
    return (m <= 3.4028234663852886e38f) ? pow2f(limb_exponent(m) - kFixBits) : __uint_as_float(0x7FC00000u);
}
// integer V = rint(v / S) for finite groups (|V| <= 2^26), 0 otherwise
__device__ __forceinline__ int limb_value(float v, float m) {
    if (!(m <= 3.4028234663852886e38f)) return 0;
    return (int)rintf(v * pow2f(kFixBits - limb_exponent(m)));
}
// balanced base-16 digits: V = sum_x l[x] 16^x, l[0..5] in [-8, 7], l[6] in [-4, 4]
__device__ __forceinline__ void limb_split(int V, int (&l)[kLimbs]) {
#pragma unroll
    for (int x = 0; x < kLimbs - 1; ++x) {
        l[x] = ((V + 8) & 15) - 8;
        V = (V - l[x]) >> 4;
    }
    l[kLimbs - 1] = V;
}

// OR over aligned groups of 8 lanes (every lane receives the result)
__device__ __forceinline__ uint32_t lane_or8(uint32_t v) {
    v |= dpp_u<kDppXor1>(v);
    v |= dpp_u<kDppXor2>(v);
    v |= dpp_u<kDppHalfMirror>(v);
    return v;
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

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint32_t blo, uint32_t bhi) {
    const uint64_t b = ((uint64_t)bhi << 32) | blo;
    return b > a ? b : a;
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t v) {
    return max_u64(v, dpp_u<CTRL>((uint32_t)v), dpp_u<CTRL>((uint32_t)(v >> 32)));
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = dpp_max_u64<kDppXor1>(v);
    v = dpp_max_u64<kDppXor2>(v);
    v = dpp_max_u64<kDppHalfMirror>(v);
    v = dpp_max_u64<kDppMirror>(v);
    {
        const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
        v = max_u64(((uint64_t)hi[0] << 32) | lo[0], lo[1], hi[1]);
    }
    {
        const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
        v = max_u64(((uint64_t)hi[0] << 32) | lo[0], lo[1], hi[1]);
    }
    return v;
}

__device__ __forceinline__ float route_key_value(uint64_t key) {
    const uint32_t u = (uint32_t)(key >> 32);
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// the router logits of one token, EPL per lane (clamped index: all loads in flight at once)
template <int EPL>
__device__ __forceinline__ void load_logits(const float *__restrict__ z, int E, float (&zv)[EPL]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        zv[i] = z[e < E ? e : E - 1];
    }
}

// bitonic sort of n = EPL keys, descending
template <int EPL>
__device__ __forceinline__ void sort_desc(uint64_t (&key)[EPL]) {
#pragma unroll
    for (int k = 2; k <= EPL; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const int l = i ^ j;
                if (l > i) {
                    const bool desc = (i & k) == 0;
                    const uint64_t a = key[i], b = key[l];
                    const bool swap = desc ? (a < b) : (a > b);
                    key[i] = swap ? b : a;
                    key[l] = swap ? a : b;
                }
            }
}

// Softmax -> top-K -> renormalise by one wave.  Each lane sorts its EPL keys;
// every round takes the wave maximum of the list heads and the winning lane
// pops its head.  Lane k < K ends with the k-th selected expert and weight.
template <int EPL>
__device__ __forceinline__ void route_wave(const float (&zv)[EPL], int E, int K, int &my_sel, float &my_w) {
    const int lane = threadIdx.x & 63;
    uint64_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        key[i] = (e < E) ? route_key(zv[i], e) : 0ull;
    }
    sort_desc<EPL>(key);
    my_sel = 0;
    float my_z = 0.0f;
    for (int k = 0; k < K; ++k) {
        const uint64_t best = wave_max_u64(key[0]);
        const bool win = key[0] == best;  // keys are unique: the index is part of the key
#pragma unroll
        for (int i = 0; i < EPL - 1; ++i) key[i] = win ? key[i + 1] : key[i];
        key[EPL - 1] = win ? 0ull : key[EPL - 1];
        if (lane == k) {
            my_sel = (int)(~(uint32_t)best);
            my_z = route_key_value(best);
        }
    }
    // softmax restricted to the selection == renormalised full softmax
    const float z0 = lane_bcast(my_z, 0);
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
    static constexpr int NL = NV / 8;             // limb dwords per limb (8 nibbles each)
    static constexpr int GL = NV < 64 ? NV : 64;  // codes of one group inside the slice
    static constexpr int NGL = NV / GL;           // groups touched by the slice
    static constexpr uint32_t kByteMask = BITS == 4 ? 0x0F0F0F0Fu : 0x03030303u;
    static constexpr float kCodeOffset = BITS == 4 ? 8.0f : 0.0f;  // signed code = q - offset
};

template <int BITS, int CPL>
struct LimbSlice {
    using Q = QSlice<BITS, CPL>;
    int L[kLimbs][Q::NL];
    float S[Q::NGL];  // group scale (power of two)
    float X[Q::NGL];  // sum of the activations of the slice within the group
};

// nibble-order codes (gate, up) against the lane's limb slice
template <int BITS, int CPL>
__device__ __forceinline__ float qdot(const uint4 (&c)[CPL], const uint32_t (&sb)[QSlice<BITS, CPL>::NGL],
                                      const LimbSlice<BITS, CPL> &v) {
    using Q = QSlice<BITS, CPL>;
    int acc[Q::NGL][kLimbs];
#pragma unroll
    for (int g = 0; g < Q::NGL; ++g)
#pragma unroll
        for (int x = 0; x < kLimbs; ++x) acc[g][x] = 0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const uint32_t d[4] = {c[j].x, c[j].y, c[j].z, c[j].w};
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
            if constexpr (BITS == 4) {
                const int q = (int)(d[w4] ^ 0x88888888u);  // eight signed codes q - 8
                const int li = j * 4 + w4;
                const int g = (8 * li) / Q::GL;
#pragma unroll
                for (int x = 0; x < kLimbs; ++x) acc[g][x] = __builtin_amdgcn_sdot8(q, v.L[x][li], acc[g][x], false);
            } else {
                const int qa = (int)(d[w4] & 0x33333333u);         // codes 0..7 of the dword
                const int qb = (int)((d[w4] >> 2) & 0x33333333u);  // codes 8..15
                const int li = j * 8 + 2 * w4;
                const int g = (8 * li) / Q::GL;
#pragma unroll
                for (int x = 0; x < kLimbs; ++x) {
                    acc[g][x] = __builtin_amdgcn_sdot8(qa, v.L[x][li], acc[g][x], false);
                    acc[g][x] = __builtin_amdgcn_sdot8(qb, v.L[x][li + 1], acc[g][x], false);
                }
            }
        }
    }
    float total = 0.0f;
#pragma unroll
    for (int g = 0; g < Q::NGL; ++g) {
        float f = (float)acc[g][kLimbs - 1];
#pragma unroll
        for (int x = kLimbs - 2; x >= 0; --x) f = fmaf(f, 16.0f, (float)acc[g][x]);
        const float s = bf16_lo(sb[g]);
        total = fmaf(s * v.S[g], f, total);
        total = fmaf(fmaf(Q::kCodeOffset, s, bf16_hi(sb[g])), v.X[g], total);
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
constexpr int kRouterWaves = 2;

template <int CPLR>
__global__ __launch_bounds__(64 * kRouterWaves) void k_router(FwdArgs a) {
    const int t = blockIdx.y;
    const int H = a.s.H, E = a.s.E;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float *x = a.x + (size_t)t * H;
    const int nch = H / 8;  // 16-byte chunks of 8 bf16 per router row
    const int lpr = nch < 64 ? nch : 64;
    const int rpi = 64 / lpr;
    const int lr = lane % lpr, rsub = lane / lpr;
    const int nrs = (E + 1 + rpi - 1) / rpi;
    const int rs = blockIdx.x * kRouterWaves + wave;
    const int r = rs * rpi + rsub;
    const bool has_row = rs < nrs && r <= E;

    // issue the router row loads first
    uint4 wv[CPLR];
#pragma unroll
    for (int j = 0; j < CPLR; ++j) wv[j] = make_uint4(0u, 0u, 0u, 0u);
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

    // pass 2 + router dot product (lanes without a row add zeros)
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
    if (has_row && lr == 0) {
        if (r < E)
            a.ws.z[(size_t)t * E + r] = acc;
        else
            a.ws.gs[t] = acc;
    }

    // limb form of h[64 kRouterWaves b ..]: one wave = one group of 64
    const int k = blockIdx.x * 64 * kRouterWaves + threadIdx.x;
    if (blockIdx.x * 64 * kRouterWaves < H) {
        const float h = (k < H) ? x[k] * inv * __uint_as_float((uint32_t)a.gamma[k] << 16) : 0.0f;
        const float m = lane_max<64>(fabsf(h));
        int l[kLimbs];
        limb_split(limb_value(h, m), l);
        const float half = lane_sum<32>(h);
        uint32_t packed[kLimbs];
#pragma unroll
        for (int xl = 0; xl < kLimbs; ++xl) packed[xl] = lane_or8((uint32_t)(l[xl] & 15) << (4 * (lane & 7)));
        if (k < H) {
            uint32_t *hl = (uint32_t *)a.ws.hl + (size_t)t * kLimbs * (H / 8);
            if ((lane & 7) == 0) {
#pragma unroll
                for (int xl = 0; xl < kLimbs; ++xl) hl[(size_t)xl * (H / 8) + k / 8] = packed[xl];
            }
            if (lane == 0) a.ws.hs[(size_t)t * (H / 64) + k / 64] = limb_scale(m);
            if ((lane & 31) == 0) a.ws.hx[(size_t)t * (H / 32) + k / 32] = half;
        }
    }
}

// ---------------------------------------------------------------------------
// k_gateup: RPW row-steps per wave over the (K+1) x F gate/up row pairs
// ---------------------------------------------------------------------------
template <int BITS, int CPL, int RPW, int EPL>
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
    const bool active = rs0 < nrs;
    // row-steps are slot-major: the block needs the routing iff its first row is routed
    const bool block_routed = (blockIdx.x * 4 * RPW * rpi) / F < K;
    const bool wave_shared_only = (rs0 * rpi) / F >= K;

    __shared__ int s_sel[kMaxTopK];
    __shared__ float s_w[kMaxTopK];
    __shared__ __align__(16) uint32_t s_hl[kLimbs * kMaxDim / 8];  // limbs of h, [kLimbs][H/8]
    __shared__ float s_hs[kMaxDim / 64];
    __shared__ float s_hx[kMaxDim / 32];

    // wave 0 routes for the whole block: its logit loads go first (loads complete in order)
    float zv[EPL];
    if (block_routed && wave == 0) load_logits<EPL>(a.ws.z + (size_t)t * E, E, zv);

    // stage the limb form of h in LDS, once per block
    {
        const int4 *src = (const int4 *)((const uint32_t *)a.ws.hl + (size_t)t * kLimbs * (H / 8));
        const int n16 = kLimbs * H / 32;
        constexpr int kStage = (kLimbs * kMaxDim / 32 + 255) / 256;
        int4 st0, st1, st2, st3;  // kStage == 4 staged 16-byte pieces per thread
        static_assert(kStage == 4, "staging assumes 4 pieces per thread");
        {
            const int i0 = threadIdx.x, i1 = threadIdx.x + 256, i2 = threadIdx.x + 512, i3 = threadIdx.x + 768;
            st0 = src[i0 < n16 ? i0 : 0];
            st1 = src[i1 < n16 ? i1 : 0];
            st2 = src[i2 < n16 ? i2 : 0];
            st3 = src[i3 < n16 ? i3 : 0];
        }
        float hs = 0.0f, hx = 0.0f;
        if (threadIdx.x < H / 64) hs = a.ws.hs[(size_t)t * (H / 64) + threadIdx.x];
        if (threadIdx.x < H / 32) hx = a.ws.hx[(size_t)t * (H / 32) + threadIdx.x];
        if (block_routed && wave == 0) {
            int my_sel;
            float my_w;
            route_wave<EPL>(zv, E, K, my_sel, my_w);
            if (lane < K) {
                s_sel[lane] = my_sel;
                s_w[lane] = my_w;
            }
            if (blockIdx.x == 0) {
                if (lane < K) {
                    a.ws.sel[t * K + lane] = my_sel;
                    a.ws.coef[t * (K + 1) + lane] = my_w;
                    if (a.route_idx) a.route_idx[t * K + lane] = my_sel;
                    if (a.route_w) a.route_w[t * K + lane] = my_w;
                } else if (lane == K) {
                    a.ws.coef[t * (K + 1) + K] = sigmoidf_(a.ws.gs[t]);
                }
            }
        }
        {
            int4 *dst = (int4 *)s_hl;
            const int i0 = threadIdx.x, i1 = threadIdx.x + 256, i2 = threadIdx.x + 512, i3 = threadIdx.x + 768;
            if (i0 < n16) dst[i0] = st0;
            if (i1 < n16) dst[i1] = st1;
            if (i2 < n16) dst[i2] = st2;
            if (i3 < n16) dst[i3] = st3;
        }
        if (threadIdx.x < H / 64) s_hs[threadIdx.x] = hs;
        if (threadIdx.x < H / 32) s_hx[threadIdx.x] = hx;
    }

    // weight loads: shared-only waves issue theirs before the routing is known
    uint4 gc[RPW][CPL], uc[RPW][CPL];
    uint32_t gsb[RPW][Q::NGL], usb[RPW][Q::NGL];
    auto issue_loads = [&]() {
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int rs = rs0 + i;
            if (rs < nrs) {
                const int p = rs * rpi + rsub;
                const int s = p / F, j = p % F;
                const uint8_t *ex = (s < K) ? a.experts + (size_t)s_sel[s] * a.L.bytes : a.shared;
                load_row<BITS, CPL>(ex, G, j, lr, gc[i], gsb[i]);
                load_row<BITS, CPL>(ex, U, j, lr, uc[i], usb[i]);
            }
        }
    };
    if (active && wave_shared_only) issue_loads();
    __syncthreads();
    if (!active) return;
    if (!wave_shared_only) issue_loads();

    // the lane's limb slice of h, from LDS
    const int k0 = lr * Q::NV;
    LimbSlice<BITS, CPL> hv;
#pragma unroll
    for (int x = 0; x < kLimbs; ++x)
#pragma unroll
        for (int i = 0; i < Q::NL / 4; ++i) {
            const int4 v = *(const int4 *)(s_hl + x * (H / 8) + k0 / 8 + 4 * i);
            hv.L[x][4 * i + 0] = v.x; hv.L[x][4 * i + 1] = v.y;
            hv.L[x][4 * i + 2] = v.z; hv.L[x][4 * i + 3] = v.w;
        }
#pragma unroll
    for (int g = 0; g < Q::NGL; ++g) {
        hv.S[g] = s_hs[k0 / 64 + g];
        float xs = 0.0f;
#pragma unroll
        for (int hh = 0; hh < Q::GL / 32; ++hh) xs += s_hx[(k0 + g * 64) / 32 + hh];
        hv.X[g] = xs;
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
// k_down: RPW row-steps of the H output rows per wave, all K+1 experts in
// batches of SB slots whose loads are all in flight together.  The SwiGLU
// activations vary widely in magnitude, so this product stays in fp32:
// codes are converted with v_cvt_f32_ubyte and folded per group as
// s * sum(q a) + b * sum(a).
// ---------------------------------------------------------------------------
template <int BITS, int CPL>
__device__ __forceinline__ float qdot_f32(const uint4 (&c)[CPL], const uint32_t (&sb)[QSlice<BITS, CPL>::NGL],
                                          const float (&av)[QSlice<BITS, CPL>::NV],
                                          const float (&X)[QSlice<BITS, CPL>::NGL]) {
    using Q = QSlice<BITS, CPL>;
    constexpr int NS = 8 / BITS;  // code slots per byte
    // one accumulator per slot: slot n holds q << (BITS n) once masked in place,
    // and the power of two is removed once per group
    float acc[Q::NGL][NS];
#pragma unroll
    for (int g = 0; g < Q::NGL; ++g)
#pragma unroll
        for (int n = 0; n < NS; ++n) acc[g][n] = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const uint32_t d[4] = {c[j].x, c[j].y, c[j].z, c[j].w};
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
#pragma unroll
            for (int n = 0; n < NS; ++n) {
                const uint32_t m = d[w4] & (Q::kByteMask << (BITS * n));
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int i = j * Q::C + w4 * Q::D + 4 * n + b;
                    acc[i / Q::GL][n] = fmaf((float)((m >> (8 * b)) & 0xFFu), av[i], acc[i / Q::GL][n]);
                }
            }
        }
    }
    float total = 0.0f;
#pragma unroll
    for (int g = 0; g < Q::NGL; ++g) {
        float qa = acc[g][NS - 1];
#pragma unroll
        for (int n = NS - 2; n >= 0; --n) qa = fmaf(qa, 1.0f / (float)(1 << BITS), acc[g][n]);
        total = fmaf(bf16_lo(sb[g]), qa, total);
        total = fmaf(bf16_hi(sb[g]), X[g], total);
    }
    return total;
}

// k_down processes the K+1 slots in batches of at most kDownBatch; a batch's
// activations and their half-group sums are staged in LDS once per block.
constexpr int kDownBatch = 5;
constexpr int kDownStageValues = 5120;  // activations staged per batch (batch * F <= this)

template <int BITS, int CPL, int RPW>
__global__ __launch_bounds__(256) void k_down(FwdArgs a, int batch) {
    using Q = QSlice<BITS, CPL>;
    const int t = blockIdx.y;
    const int H = a.s.H, F = a.s.F, E = a.s.E, K = a.s.K;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const QMat &Dm = a.L.m[2];
    const int lpr = Dm.lpr, rpi = 64 / lpr;
    const int lr = lane % lpr, rsub = lane / lpr;
    const int nrs = H / rpi;
    const int rs0 = (blockIdx.x * 4 + wave) * RPW;
    const bool active = rs0 < nrs;
    const int k0 = lr * Q::NV;

    extern __shared__ __align__(16) unsigned char smem[];
    float *s_act = (float *)smem;              // [batch][F]
    float *s_half = s_act + (size_t)batch * F;  // [batch][F/32]

    // lane s (s <= K) holds slot s: expert index and combine coefficient
    const int my_e = (lane < K) ? a.ws.sel[t * K + lane] : E;
    const float my_c = (lane <= K) ? a.ws.coef[t * (K + 1) + lane] : 0.0f;

    float acc[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) acc[i] = 0.0f;

    // slot positions run shared, 0, 1, ..., K-1: the shared expert's loads need no routing
    constexpr int kStageMax = kDownStageValues / 1024;  // float4 pieces per thread and batch
    for (int b0 = 0; b0 <= K; b0 += batch) {
        const int nb = (K + 1 - b0) < batch ? (K + 1 - b0) : batch;
        // this batch's activations first: the staging then waits on them only
        // (loads complete in order), while the weight loads stay in flight
        float4 stv[kStageMax];
#pragma unroll
        for (int r = 0; r < kStageMax; ++r) {
            const int v0 = threadIdx.x * 4 + 1024 * r;
            stv[r] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (v0 < nb * F) {
                const int si = v0 / F, j = v0 % F;
                const int s = (b0 + si == 0) ? K : b0 + si - 1;
                stv[r] = *(const float4 *)(a.ws.act + ((size_t)t * (K + 1) + s) * F + j);
            }
        }
        // weights of up to kDownBatch slots of this batch, all in flight together
        uint4 wc[kDownBatch][RPW][CPL];
        uint32_t wsb[kDownBatch][RPW][Q::NGL];
#pragma unroll
        for (int si = 0; si < kDownBatch; ++si) {
            if (si < nb && active) {
                const int s = (b0 + si == 0) ? K : b0 + si - 1;
                const int e = (s == K) ? E : lane_bcast(my_e, s);
                const uint8_t *ex = (e < E) ? a.experts + (size_t)e * a.L.bytes : a.shared;
#pragma unroll
                for (int i = 0; i < RPW; ++i) {
                    const int rs = rs0 + i;
                    if (rs < nrs) load_row<BITS, CPL>(ex, Dm, rs * rpi + rsub, lr, wc[si][i], wsb[si][i]);
                }
            }
        }
        // stage this batch's activations and half-group sums
        if (b0 > 0) __syncthreads();  // the previous batch is done with the LDS
#pragma unroll
        for (int r = 0; r < kStageMax; ++r) {
            const int v0 = threadIdx.x * 4 + 1024 * r;
            if (1024 * r < batch * F) {  // uniform: whole 8-thread groups are live or not
                const bool live = v0 < nb * F;
                if (live) *(float4 *)(s_act + v0) = stv[r];
                const float4 v = stv[r];
                const float half = lane_sum<8>((v.x + v.y) + (v.z + v.w));  // 8 threads = 32 values
                if (live && (threadIdx.x & 7) == 0) s_half[v0 / 32] = half;
            }
        }
        __syncthreads();
        if (active) {
#pragma unroll
            for (int si = 0; si < kDownBatch; ++si) {
                if (si < nb) {
                    const int s = (b0 + si == 0) ? K : b0 + si - 1;
                    const float c = lane_bcast(my_c, s);
                    float av[Q::NV];
#pragma unroll
                    for (int i = 0; i < Q::NV / 4; ++i) {
                        const float4 v = *(const float4 *)(s_act + (size_t)si * F + k0 + 4 * i);
                        av[4 * i] = v.x; av[4 * i + 1] = v.y; av[4 * i + 2] = v.z; av[4 * i + 3] = v.w;
                    }
                    float X[Q::NGL];
#pragma unroll
                    for (int g = 0; g < Q::NGL; ++g) {
                        float x = 0.0f;
#pragma unroll
                        for (int hh = 0; hh < Q::GL / 32; ++hh) x += s_half[si * (F / 32) + (k0 + g * 64) / 32 + hh];
                        X[g] = x;
                    }
#pragma unroll
                    for (int i = 0; i < RPW; ++i)
                        if (rs0 + i < nrs) acc[i] = fmaf(c, qdot_f32<BITS, CPL>(wc[si][i], wsb[si][i], av, X), acc[i]);
                }
            }
        }
    }
    if (!active) return;
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

constexpr int kRpwGateUp = 3;
constexpr int kRpwDown = 2;

template <int BITS>
hipError_t launch_stage(const FwdArgs &a, int stage, hipStream_t st) {
    const int H = a.s.H, F = a.s.F, E = a.s.E, K = a.s.K, T = a.T;
    if (stage == 0) {  // RMSNorm + router + limbs of h
        const int nch = H / 8, lpr = nch < 64 ? nch : 64, cplr = nch / lpr, rpi = 64 / lpr;
        const int nrs = (E + 1 + rpi - 1) / rpi;
        int blocks = (nrs + kRouterWaves - 1) / kRouterWaves;
        const int enc_blocks = (H + 64 * kRouterWaves - 1) / (64 * kRouterWaves);
        if (blocks < enc_blocks) blocks = enc_blocks;
        dim3 grid(blocks, T);
        const dim3 blk(64 * kRouterWaves);
        switch (cplr) {
            case 1: hipLaunchKernelGGL(k_router<1>, grid, blk, 0, st, a); break;
            case 2: hipLaunchKernelGGL(k_router<2>, grid, blk, 0, st, a); break;
            case 4: hipLaunchKernelGGL(k_router<4>, grid, blk, 0, st, a); break;
            case 8: hipLaunchKernelGGL(k_router<8>, grid, blk, 0, st, a); break;
            default: return hipErrorInvalidValue;
        }
    } else if (stage == 1) {  // routing + gate/up + SwiGLU
        const QMat &G = a.L.m[0];
        const int rpi = 64 / G.lpr;
        const int nrs = (K + 1) * F / rpi;
        const int blocks = (nrs + 4 * kRpwGateUp - 1) / (4 * kRpwGateUp);
        dim3 grid(blocks, T);
        const bool wide = E > 512;
        switch (G.cpl * 2 + (wide ? 1 : 0)) {
            case 2: hipLaunchKernelGGL((k_gateup<BITS, 1, kRpwGateUp, 8>), grid, dim3(256), 0, st, a); break;
            case 3: hipLaunchKernelGGL((k_gateup<BITS, 1, kRpwGateUp, 16>), grid, dim3(256), 0, st, a); break;
            case 4: hipLaunchKernelGGL((k_gateup<BITS, 2, kRpwGateUp, 8>), grid, dim3(256), 0, st, a); break;
            case 5: hipLaunchKernelGGL((k_gateup<BITS, 2, kRpwGateUp, 16>), grid, dim3(256), 0, st, a); break;
            default: return hipErrorInvalidValue;
        }
    } else if (stage == 2) {  // down + combine + residual
        const QMat &Dm = a.L.m[2];
        const int rpi = 64 / Dm.lpr;
        const int nrs = H / rpi;
        const int blocks = (nrs + 4 * kRpwDown - 1) / (4 * kRpwDown);
        dim3 grid(blocks, T);
        const size_t per_slot = (size_t)F * 4 + (size_t)(F / 32) * 4;
        int batch = kDownStageValues / F;
        if (batch > kDownBatch) batch = kDownBatch;
        if (batch > K + 1) batch = K + 1;
        if (batch < 1) batch = 1;
        const size_t lds = per_slot * batch;
        switch (Dm.cpl) {
            case 1: hipLaunchKernelGGL((k_down<BITS, 1, kRpwDown>), grid, dim3(256), lds, st, a, batch); break;
            case 2: hipLaunchKernelGGL((k_down<BITS, 2, kRpwDown>), grid, dim3(256), lds, st, a, batch); break;
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

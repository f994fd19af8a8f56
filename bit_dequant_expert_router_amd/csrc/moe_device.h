// moe_device.h -- device helpers shared by the layer kernels (library-internal).
//
// Dequantised dot products.  A lane owns a contiguous slice of the reduction
// axis and walks rows; a 64-entry group with scale s and bias b contributes
//     sum_i (q_i s + b) v_i = s * sum_i q_i v_i + b * sum_i v_i,
// the group-level form of the pages' fma(nibble, scale*x, bias*x) rewrite.
//
// Gate/up (activation h, the normalised token): the code products sum_i q_i h_i
// are taken exactly in integers.  Each group of h is written as V_i * S with S a
// power of two (max|h| < 2^22 S) and V_i an integer split into six signed
// base-16 digits (limbs) V = sum_x L_x 16^x, L_x in [-8, 7].  Eight limbs of
// consecutive entries are packed per dword, the operand form of v_dot8_i32_i4;
// the codes q, made signed as q - 8 by one XOR per 8 codes (4-bit), are the other
// operand, so one instruction accumulates 8 exact code x limb products.  Per group
// and limb the sums stay below 2^12; one fp32 combination restores
// s*S*sum_x D_x 16^x, and the -8 folds into the bias term, (b + 8 s) * sum h.
// Every entry is rounded to a multiple of S, an error of at most 2^-23 of the
// group's power-of-two bound (fp32 rounds an entry at 2^-24 of itself); the
// products and their sums are exact.  The VALU does about one instruction
// per weight against ~2.3 for convert-and-FMA.
//
// Down (activation a = SwiGLU output, widely spread magnitudes): fixed point
// per lane slice, not per group.  The single-token kernel (qdot_limbs) writes
// the NV activations of a lane slice as V = rint(a 2^(22-e)) with one exponent
// e for the slice, in three byte limbs; four codes masked into the bytes of a
// word (byte code order) meet four values' limbs in one v_dot4 per limb.  The
// grouped kernels take the activations in the six-limb form above (one
// exponent per group, from k_encode_act), in the nibble order of the byte-order
// codes, with v_dot8.
#pragma once
#include "moe_internal.h"

namespace moe {

namespace {

__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

// bf16 bits of f rounded to nearest even (NaN stays a quiet NaN)
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Entries 16u .. 16u+15 of vector t (length n) as three bf16 parts (hi, then
// the bf16 of what hi leaves, then of what both leave: 24 significant bits),
// stored in the operand order of v_mfma_f32_32x32x16_bf16 over 32 vectors:
// fragment (t / 32, u, part) holds lane t % 32 (entries 0..7) and lane
// t % 32 + 32 (entries 8..15), 8 bf16 per lane.
__device__ __forceinline__ void store_split_fragments(uint16_t *base, int n, int t, int u, const float (&v)[16]) {
    uint16_t *f = base + ((size_t)(t >> 5) * (n / 16) + u) * 3 * 512 + (t & 31) * 8;
    float r[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = v[i];
#pragma unroll
    for (int p = 0; p < 3; ++p) {
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t lo = bf16_rne_bits(r[2 * i]), hi = bf16_rne_bits(r[2 * i + 1]);
            w[i] = lo | (hi << 16);
            r[2 * i] -= __uint_as_float(lo << 16);
            r[2 * i + 1] -= __uint_as_float(hi << 16);
        }
        *(uint4 *)(f + p * 512) = make_uint4(w[0], w[1], w[2], w[3]);
        *(uint4 *)(f + p * 512 + 32 * 8) = make_uint4(w[4], w[5], w[6], w[7]);
    }
}

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
constexpr int kLimbs = 6;                  // signed base-16 digits
constexpr int kFixBits = 4 * kLimbs - 2;   // |V| <= 2^22

// Exponent e with max|v| < 2^e, clamped so that 2^(e-22) and 2^(22-e) are
// normal floats.  NaN / inf maxima are flagged by limb_scale.
__device__ __forceinline__ int limb_exponent(float m) {
    const uint32_t E = (__float_as_uint(m) >> 23) & 0xFFu;
    int e = (E == 0 ? 1 : (int)E) - 126;  // m < 2^e
    return e < -90 ? -90 : e;
}
__device__ __forceinline__ float pow2f(int p) { return __uint_as_float((uint32_t)(p + 127) << 23); }
// scale S of a group: 2^(e-22), or NaN when the group holds a NaN or an inf
__device__ __forceinline__ float limb_scale(float m) {
    return (m <= 3.4028234663852886e38f) ? pow2f(limb_exponent(m) - kFixBits) : __uint_as_float(0x7FC00000u);
}
// integer V = rint(v / S) for finite groups (|V| <= 2^22), 0 otherwise
__device__ __forceinline__ int limb_value(float v, float m) {
    if (!(m <= 3.4028234663852886e38f)) return 0;
    return (int)rintf(v * pow2f(kFixBits - limb_exponent(m)));
}
// balanced base-16 digits: V = sum_x l[x] 16^x, l[0..4] in [-8, 7], l[5] in [-4, 4]
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

__device__ __forceinline__ float route_key_value(uint64_t key) {
    const uint32_t u = (uint32_t)(key >> 32);
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
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

// 32-bit maximum over the wave (DPP row steps, then the row and half swaps)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
    v = mx(v, dpp_u<kDppXor1>(v));
    v = mx(v, dpp_u<kDppXor2>(v));
    v = mx(v, dpp_u<kDppHalfMirror>(v));
    v = mx(v, dpp_u<kDppMirror>(v));
    {
        const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        v = mx(p[0], p[1]);
    }
    {
        const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        v = mx(p[0], p[1]);
    }
    return v;
}

// The K largest of the wave's keys (logit order in the high word, the
// complemented index in the low word; N per lane, 0 = no key).  Each lane
// sorts its keys; every round takes the wave maximum of the heads' high
// words, and the lane holding it (one ballot bit, or after an exact tie the
// largest low word, i.e. the lowest index) pops its head.  Lane k < K ends
// with the k-th (0 when the wave holds fewer).
template <int N>
__device__ __forceinline__ uint64_t wave_top_keys(uint64_t (&key)[N], int K) {
    const int lane = threadIdx.x & 63;
    sort_desc<N>(key);
    uint64_t mine = 0;
    for (int k = 0; k < K; ++k) {
        const uint32_t hi = (uint32_t)(key[0] >> 32), lo = (uint32_t)key[0];
        const uint32_t m = wave_max_u32(hi);
        uint64_t cand = __ballot(hi == m);
        if (__popcll(cand) > 1) {  // exact tie of the high words: the largest low word (lowest index)
            const uint32_t m2 = wave_max_u32(hi == m ? lo : 0u);
            cand = __ballot(hi == m && lo == m2);
        }
        const int w = __ffsll((unsigned long long)cand) - 1;
        const uint32_t lo_w = __builtin_amdgcn_readlane(lo, w);
        const bool win = lane == w;
#pragma unroll
        for (int i = 0; i < N - 1; ++i) key[i] = win ? key[i + 1] : key[i];
        key[N - 1] = win ? 0ull : key[N - 1];
        if (lane == k) mine = ((uint64_t)m << 32) | lo_w;
    }
    return mine;
}

// Softmax -> top-K -> renormalise by the 4 waves of a block, in two steps
// around a block barrier that the caller places.
//
// route_candidates: each wave selects the K largest keys of its quarter of
// the logits (z[q] of lane l in wave w is expert e = 256 q + 64 w + l) and
// stores them at s_cand[w K + k] (s_cand: 4 * kMaxTopK keys of LDS, 16-byte
// aligned).
template <int EPW>
__device__ __forceinline__ void route_candidates(const float (&zq)[EPW], int E, int K, uint64_t *s_cand) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t key[EPW];
#pragma unroll
    for (int q = 0; q < EPW; ++q) {
        const int e = 256 * q + 64 * wave + lane;
        key[q] = (e < E) ? route_key(zq[q], e) : 0ull;
    }
    const uint64_t best = wave_top_keys<EPW>(key, K);
    if (lane < K) s_cand[wave * K + lane] = best;
}

// route_select, after the barrier, in any wave: lane i < 4K takes candidate i
// and counts the candidates above it.  The keys of experts are distinct and
// nonzero (absent ones are 0), so the candidates of rank k < K are the K
// largest logits in selection order, without further rounds.  The weights
// are the softmax restricted to the selection, which equals the full softmax
// renormalised over it.  rank == K marks a lane outside the selection.
struct RouteSel {
    int rank;
    int sel;
    float w;
};

__device__ __forceinline__ RouteSel route_select(int K, const uint64_t *s_cand) {
    const int lane = threadIdx.x & 63, n = 4 * K;
    const uint64_t mine = s_cand[lane < n ? lane : 0];
    int above = 0;
    // 8 keys per step, read together (s_cand holds 64; n is a multiple of 4,
    // so only the upper half of a step can lie past n: read and ignored)
    for (int j0 = 0; j0 < n; j0 += 8) {
        uint64_t c[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) c[u] = s_cand[j0 + u];
        int lo = 0, hi = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            lo += c[u] > mine ? 1 : 0;
            hi += c[u + 4] > mine ? 1 : 0;
        }
        above += lo + (j0 + 4 < n ? hi : 0);
    }
    const bool in = lane < n && above < K;
    const float z = in ? route_key_value(mine) : 0.0f;
    // the candidate of rank 0 holds the largest logit
    const uint64_t top = __ballot(in && above == 0);
    const float zmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), __ffsll((unsigned long long)top) - 1));
    const float p = in ? expf(z - zmax) : 0.0f;
    RouteSel r;
    r.rank = in ? above : K;
    r.sel = (int)(~(uint32_t)mine);
    r.w = p / lane_sum<64>(p);
    return r;
}

// ---------------------------------------------------------------------------
// routing by one wave over all E logits of a token (E <= 64 EPL), without LDS
// or barriers.  Lane l holds the keys of experts EPL l .. EPL l + EPL - 1 (the
// high word of route_key; 0 = absent or already taken).  A round takes the wave
// maximum of the lanes' best keys.  Among equal keys the lowest lane holds the
// lowest expert, and inside a lane the lowest position does (the first maximum
// is kept), so the key order (logit descending, index ascending) needs no
// second comparison.  The winner's key is cleared.  The expert of slot s is the
// winner of round s: a wave that serves slot s stops after s + 1 rounds.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t logit_key(float z) { return (uint32_t)(route_key(z, 0) >> 32); }
__device__ __forceinline__ float logit_of_key(uint32_t m) { return route_key_value((uint64_t)m << 32); }

// the lane's EPL logits of one token, from a row of ZS floats (a multiple of
// 16, 32-byte aligned) with 16-byte loads; a lane whose experts all lie past
// the row reads its last EPL entries instead (read, never used as logits)
template <int EPL>
__device__ __forceinline__ void load_logits_lane(const float *__restrict__ z, int ZS, float (&v)[EPL]) {
    const int lane = threadIdx.x & 63;
    const int base = EPL * lane < ZS - EPL ? EPL * lane : ZS - EPL;
#pragma unroll
    for (int i = 0; i < EPL / 4; ++i) {
        const float4 f = *(const float4 *)(z + base + 4 * i);
        v[4 * i] = f.x;
        v[4 * i + 1] = f.y;
        v[4 * i + 2] = f.z;
        v[4 * i + 3] = f.w;
    }
}

template <int EPL>
__device__ __forceinline__ void logit_keys(const float (&v)[EPL], int E, uint32_t (&key)[EPL]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < EPL; ++q) key[q] = (EPL * lane + q < E) ? logit_key(v[q]) : 0u;
}

// one round: the expert holding the wave's largest remaining key (wave-uniform,
// clamped below E), whose key is then cleared; m receives that key.  The
// dependent chain is kept short: the lane's best key by a tree of 3-input
// maxima, its first position (a bit mask of the equal keys, lowest bit) formed
// while the DPP wave maximum runs, and only the winning entry rewritten.
template <int EPL>
__device__ __forceinline__ uint32_t lane_best_key(const uint32_t (&key)[EPL]) {
    // groups of three (v_max3_u32), then the group maxima the same way
    uint32_t t[(EPL + 2) / 3];
#pragma unroll
    for (int i = 0; i < (EPL + 2) / 3; ++i) {
        uint32_t v = key[3 * i];
        if (3 * i + 1 < EPL) v = max(v, key[3 * i + 1]);
        if (3 * i + 2 < EPL) v = max(v, key[3 * i + 2]);
        t[i] = v;
    }
    uint32_t b = t[0];
#pragma unroll
    for (int i = 1; i < (EPL + 2) / 3; ++i) b = max(b, t[i]);
    return b;
}

template <int EPL>
__device__ __forceinline__ int route_round(uint32_t (&key)[EPL], int E, uint32_t &m) {
    const int lane = threadIdx.x & 63;
    const uint32_t best = lane_best_key<EPL>(key);
    uint32_t pm = 0;
#pragma unroll
    for (int q = 0; q < EPL; ++q) pm |= (key[q] == best) ? (1u << q) : 0u;
    const int bq = __builtin_ctz(pm);  // best is one of the keys: pm != 0
    m = wave_max_u32(best);
    const int w = __ffsll((unsigned long long)__ballot(best == m)) - 1;
    const int qw = __builtin_amdgcn_readlane(bq, w);
#pragma unroll
    for (int q = 0; q < EPL; ++q) key[q] = (q == qw && lane == w) ? 0u : key[q];
    const int e = w * EPL + qw;
    return e < E ? e : E - 1;
}

// the expert of slot s (s + 1 rounds; the keys are consumed)
template <int EPL>
__device__ __forceinline__ int route_slot(uint32_t (&key)[EPL], int E, int s) {
    int e = 0;
    uint32_t m;
    for (int r = 0; r <= s; ++r) e = route_round<EPL>(key, E, m);
    return e;
}

// softmax -> top-K -> renormalise: lane k < K ends with the k-th selected
// expert (key order) and its weight, the softmax restricted to the selection
// (which equals the full softmax renormalised over it); other lanes hold w = 0
struct RouteK {
    int sel;
    float w;
};

template <int EPL>
__device__ __forceinline__ RouteK route_all(uint32_t (&key)[EPL], int E, int K) {
    const int lane = threadIdx.x & 63;
    uint32_t my_m = 0;
    int my_e = 0;
    for (int r = 0; r < K; ++r) {
        uint32_t m;
        const int e = route_round<EPL>(key, E, m);
        my_m = (lane == r) ? m : my_m;
        my_e = (lane == r) ? e : my_e;
    }
    const bool in = lane < K;
    const float z = in ? logit_of_key(my_m) : 0.0f;
    const float zmax = lane_bcast(z, 0);  // round 0 took the largest logit
    const float p = in ? expf(z - zmax) : 0.0f;
    RouteK r;
    r.sel = my_e;
    r.w = p / lane_sum<64>(p);
    return r;
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

// NR rows of codes as stored (4-bit nibbles hold q XOR 8, the signed q - 8 that
// v_dot8_i32_i4 reads; 2-bit codes are masked per dot) against one vector's
// lane slice held in LDS.
// The limb words are read one limb at a time, limb-major, so that only 8 of
// them are live; each row keeps two integer Horner accumulators (limbs 5-4 and
// 3-0, each below 2^25), combined in fp32 as hi * 2^16 + lo.  s: the rows'
// group scales; o: b + 8 s (4-bit) or b (2-bit), unpacked by the caller once
// per row.  limbs: [kLimbs][n/8] words; S: [n/64] group scales; Xh: [n/32]
// half-group sums.
template <int BITS, int CPL, int NR>
__device__ __forceinline__ void rows_dot_lds(const uint4 (&c)[NR][CPL], const float (&s)[NR][QSlice<BITS, CPL>::NGL],
                                             const float (&o)[NR][QSlice<BITS, CPL>::NGL], const uint32_t *limbs,
                                             const float *S_all, const float *Xh_all, int n, int k0, float (&out)[NR]) {
    using Q = QSlice<BITS, CPL>;
    constexpr int ND = BITS == 4 ? CPL * 4 : CPL * 8;  // limb words per limb in the slice
    constexpr int DPG = ND / Q::NGL;                    // ... per group
    const uint32_t *lw = limbs + k0 / 8;
    const float *S = S_all + k0 / 64;
    const float *Xh = Xh_all + k0 / 32;
#pragma unroll
    for (int r = 0; r < NR; ++r) out[r] = 0.0f;
#pragma unroll
    for (int g = 0; g < Q::NGL; ++g) {
        int hi[NR], lo[NR];
        auto limb = [&](int x, int (&acc)[NR], bool first) {
            int L[DPG];
#pragma unroll
            for (int i = 0; i < DPG / 4; ++i) {
                const int4 v = *(const int4 *)(lw + x * (n / 8) + g * DPG + 4 * i);
                L[4 * i] = v.x; L[4 * i + 1] = v.y; L[4 * i + 2] = v.z; L[4 * i + 3] = v.w;
            }
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                int a = first ? 0 : (acc[r] << 4);
#pragma unroll
                for (int i = 0; i < DPG; ++i) {
                    const int di = g * DPG + i;  // limb word of the slice
                    int op;
                    if constexpr (BITS == 4) {
                        const uint4 cj = c[r][di / 4];
                        const uint32_t w[4] = {cj.x, cj.y, cj.z, cj.w};
                        op = (int)w[di % 4];
                    } else {
                        const uint4 cj = c[r][di / 8];
                        const uint32_t w[4] = {cj.x, cj.y, cj.z, cj.w};
                        const uint32_t d = w[(di % 8) / 2];
                        op = (int)((di & 1) ? ((d >> 2) & 0x33333333u) : (d & 0x33333333u));
                    }
                    a = __builtin_amdgcn_sdot8(op, L[i], a, false);
                }
                acc[r] = a;
            }
        };
        // limbs one at a time (the loops are kept rolled so that the limb
        // words of only one limb are live)
        limb(kLimbs - 1, hi, true);
#pragma unroll 1
        for (int x = kLimbs - 2; x >= 4; --x) limb(x, hi, false);
        limb(3, lo, true);
#pragma unroll 1
        for (int x = 2; x >= 0; --x) limb(x, lo, false);
        float xs = 0.0f;
#pragma unroll
        for (int hh = 0; hh < Q::GL / 32; ++hh) xs += Xh[g * 2 + hh];
        const float Sg = S[g];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const float f = fmaf((float)hi[r], 65536.0f, (float)lo[r]);
            out[r] = fmaf(s[r][g] * Sg, f, out[r]);
            out[r] = fmaf(o[r][g], xs, out[r]);
        }
    }
}

// ---------------------------------------------------------------------------
// several partial sums reduced at once over aligned groups of W lanes
// (N <= W, both powers of two).  The first log2(N) exchange steps halve the
// list (a lane keeps the half its lane bit selects and adds its partner's copy
// of that half), the remaining steps are plain sums.  Lane l ends with list
// entry j = sum over the halving steps s of bit b_s(l) * N / 2^(s+1), where
// b_s = log2(W) - 1 - s; every lane of the sub-group W / N shares it.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ float xchg(float v) {  // partner's copy of v across lane bit log2(D)
    if constexpr (D == 32) {
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        return __uint_as_float((threadIdx.x & 32) ? p[0] : p[1]);
    } else if constexpr (D == 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        return __uint_as_float((threadIdx.x & 16) ? p[0] : p[1]);
    } else {
        constexpr int C = D == 8 ? kDppMirror : D == 4 ? kDppHalfMirror : D == 2 ? kDppXor2 : kDppXor1;
        return __uint_as_float(dpp_u<C>(__float_as_uint(v)));
    }
}

template <int D>
__device__ __forceinline__ float halve(float a, float b) {  // keep a (lane bit clear) or b (set), plus partner's
    if constexpr (D == 32) {
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        return __uint_as_float(p[0]) + __uint_as_float(p[1]);
    } else if constexpr (D == 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        return __uint_as_float(p[0]) + __uint_as_float(p[1]);
    } else {
        const bool hi = (threadIdx.x & D) != 0;
        return (hi ? b : a) + xchg<D>(hi ? a : b);
    }
}

template <int D>
__device__ __forceinline__ float plain_reduce(float x) {
    if constexpr (D >= 1) return plain_reduce<D / 2>(x + xchg<D>(x));
    else return x;
}

template <int N, int W, int D = W / 2>
__device__ __forceinline__ float multi_reduce(float (&v)[N]) {
    static_assert(N <= W, "one list entry per lane at least");
    if constexpr (N == 1) {
        return plain_reduce<D>(v[0]);
    } else {
        float h[N / 2];
#pragma unroll
        for (int i = 0; i < N / 2; ++i) h[i] = halve<D>(v[i], v[i + N / 2]);
        return multi_reduce<N / 2, W, D / 2>(h);
    }
}

// list index held by the lane after multi_reduce<N, W>
template <int N, int W>
__device__ __forceinline__ int multi_index(int lane) {
    if constexpr (N == 1) return 0;
    else return ((lane & (W / 2)) ? N / 2 : 0) + multi_index<N / 2, W / 2>(lane);
}

template <int BITS, int CPL>
__device__ __forceinline__ void load_row(const uint8_t *__restrict__ ex, const QMat &q, int r, int lr,
                                         uint4 (&c)[CPL], uint32_t (&sb)[QSlice<BITS, CPL>::NGL]) {
    using Q = QSlice<BITS, CPL>;
    // 32-bit offsets from the expert's base (an expert is far below 4 GiB): with
    // a wave-uniform base the loads take the scalar-base form, one 32-bit
    // offset per lane instead of a 64-bit address
    const uint32_t row = (uint32_t)q.codes_off + (uint32_t)r * (uint32_t)q.row_bytes;
#pragma unroll
    for (int j = 0; j < CPL; ++j) c[j] = ld_stream16(ex + (row + 16u * (uint32_t)(lr + q.lpr * j)));
    const uint32_t sbr =
        (uint32_t)q.sb_off + 4u * ((uint32_t)r * (uint32_t)q.ngroups + (uint32_t)((lr * Q::NV) / kGroup));
#pragma unroll
    for (int g = 0; g < Q::NGL; ++g) sb[g] = ld_stream4((const uint32_t *)(ex + (sbr + 4u * g)));
}

// ---------------------------------------------------------------------------
// down projection: codes against byte limbs of the activations
// ---------------------------------------------------------------------------
// Byte limbs of a fixed-point value |V| <= 2^22: V = L2 2^16 + L1 2^8 + L0,
// L0 and L1 unsigned, L2 signed (in [-64, 64]).  Four values give one word per
// limb, value b in byte b.
__device__ __forceinline__ void byte_limbs(int v0, int v1, int v2, int v3, uint32_t &l0, uint32_t &l1,
                                           uint32_t &l2) {
    // v_perm_b32: byte k of the result is byte sel_k of {hi : lo} (lo = bytes 0-3)
    const uint32_t t01 = __builtin_amdgcn_perm((uint32_t)v1, (uint32_t)v0, 0x05010400u);  // v0.0 v1.0 v0.1 v1.1
    const uint32_t t23 = __builtin_amdgcn_perm((uint32_t)v3, (uint32_t)v2, 0x05010400u);
    const uint32_t u01 = __builtin_amdgcn_perm((uint32_t)v1, (uint32_t)v0, 0x07030602u);  // v0.2 v1.2 v0.3 v1.3
    const uint32_t u23 = __builtin_amdgcn_perm((uint32_t)v3, (uint32_t)v2, 0x07030602u);
    l0 = __builtin_amdgcn_perm(t23, t01, 0x05040100u);
    l1 = __builtin_amdgcn_perm(t23, t01, 0x07060302u);
    l2 = __builtin_amdgcn_perm(u23, u01, 0x05040100u);
}

// 32-bit maximum over aligned groups of W lanes
template <int W>
__device__ __forceinline__ uint32_t lane_max_u32(uint32_t v) {
    auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
    if constexpr (W >= 2) v = mx(v, dpp_u<kDppXor1>(v));
    if constexpr (W >= 4) v = mx(v, dpp_u<kDppXor2>(v));
    if constexpr (W >= 8) v = mx(v, dpp_u<kDppHalfMirror>(v));
    if constexpr (W >= 16) v = mx(v, dpp_u<kDppMirror>(v));
    if constexpr (W >= 32) {
        const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        v = mx(p[0], p[1]);
    }
    if constexpr (W >= 64) {
        const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        v = mx(p[0], p[1]);
    }
    return v;
}

// One row's dequantised dot product over the lane's slice of NV codes.  The
// four codes 4n..4n+3 of a dword, masked into the bytes of a word, meet the
// byte limbs of the same four activations in one v_dot4 per limb (u8 x u8 for
// L0 and L1, i8 x i8 for L2; codes are below 16).  Per group of 64 codes the
// integer sums give sum(q V) = 2^16 S2 + 2^8 S1 + S0 (S1 2^8 + S0 < 2^32),
// sum(q a) = sum(q V) * lsc (the slice's 2^(e-22)), and the group folds as
// s * sum(q a) + b * sum(a).
template <int BITS, int CPL>
__device__ __forceinline__ float qdot_limbs(const uint4 (&c)[CPL], const uint32_t (&sb)[QSlice<BITS, CPL>::NGL],
                                            const uint32_t (&L)[3][QSlice<BITS, CPL>::NV / 4], float lsc,
                                            const float (&X)[QSlice<BITS, CPL>::NGL]) {
    using Q = QSlice<BITS, CPL>;
    constexpr int NS = 8 / BITS;   // four-code groups per dword
    constexpr int PG = Q::GL / 4;  // four-code groups per quantisation group
    uint32_t s0[Q::NGL], s1[Q::NGL];
    int s2[Q::NGL];
#pragma unroll
    for (int g = 0; g < Q::NGL; ++g) s0[g] = s1[g] = 0u, s2[g] = 0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const uint32_t d[4] = {c[j].x, c[j].y, c[j].z, c[j].w};
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
#pragma unroll
            for (int n = 0; n < NS; ++n) {
                const uint32_t q = (d[w4] >> (BITS * n)) & Q::kByteMask;
                const int pc = (j * 4 + w4) * NS + n, g = pc / PG;
                s0[g] = __builtin_amdgcn_udot4(q, L[0][pc], s0[g], false);
                s1[g] = __builtin_amdgcn_udot4(q, L[1][pc], s1[g], false);
                s2[g] = __builtin_amdgcn_sdot4((int)q, (int)L[2][pc], s2[g], false);
            }
        }
    }
    float total = 0.0f;
#pragma unroll
    for (int g = 0; g < Q::NGL; ++g) {
        const float lo = (float)((s1[g] << 8) + s0[g]);
        const float qa = fmaf((float)s2[g], 65536.0f, lo) * lsc;
        total = fmaf(bf16_lo(sb[g]), qa, total);
        total = fmaf(bf16_hi(sb[g]), X[g], total);
    }
    return total;
}

}  // namespace

}  // namespace moe

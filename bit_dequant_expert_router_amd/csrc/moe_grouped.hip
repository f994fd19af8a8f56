// moe_grouped.hip -- the expert layer for a batch of tokens, grouped by expert.
//
// A batch of T decode tokens routes T*K (token, slot) assignments over the
// experts; with T = 32 and K = 10 (the model's native routing, juejin post on
// Flash-MoE, "为什么 397B 的模型能塞进 48GB") about 240 of 512 experts are
// touched, most by one or two tokens.  Reading each touched expert once and
// applying it to all of its tokens is what saves HBM bytes; the per-expert
// token counts are far too small for a dense tile, so the routed experts stay
// on the dequant-GEMV kernels with a loop over each expert's tokens.
//
//   k_norm_batch, k_router_mfma (moe_batch_router.hip) RMSNorm, limb and bf16
//                   forms of h, router logits on the matrix cores
//   k_route_tokens  one block per token: softmax/top-K/renormalise
//   k_group         one block: histogram of assignments per expert, exclusive
//                   scan, stable scatter (token order kept inside each expert)
//                   and the compact list of touched experts
//   k_grouped_gateup  one block per (touched expert, row chunk): gate+up rows read
//                   once, applied to every token of the expert, SwiGLU; the shared
//                   expert gets its own blocks over all tokens
//   k_grouped_down  same for the down projection, writing one output vector per
//                   (token, slot)
//   k_combine       out = x + sum_k w_k y_k + sigmoid(g_s) y_shared, in slot order
#include <mutex>

#include "moe_device.h"

namespace moe {

namespace {

struct GroupView {
    int G;  // bound on touched experts
    const int32_t *n_touched;
    const int32_t *expert;
    const int32_t *first;
    const int32_t *count;
    const int32_t *perm;
};

__device__ __forceinline__ GroupView group_view(const FwdArgs &a) {
    GroupView g;
    g.G = (a.T * a.s.K < a.s.E) ? a.T * a.s.K : a.s.E;
    g.n_touched = a.ws.grp;
    g.expert = a.ws.grp + 4;
    g.first = g.expert + (g.G + 1);
    g.count = g.first + (g.G + 1);
    g.perm = g.count + (g.G + 1);
    return g;
}

// exclusive prefix sums of NV values per thread over a block of NT threads
// (thread order); tot receives the block totals.  s_tmp: NT / 64 * NV ints.
template <int NV, int NT>
__device__ __forceinline__ void block_excl_scan(int (&v)[NV], int (&tot)[NV], int *s_tmp) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) incl[j] = v[j];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int u = __shfl_up(incl[j], o, 64);
            if (lane >= o) incl[j] += u;
        }
    }
    if (lane == 63) {
#pragma unroll
        for (int j = 0; j < NV; ++j) s_tmp[wave * NV + j] = incl[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        int pre = 0, t = 0;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) {
            const int x = s_tmp[w * NV + j];
            pre += w < wave ? x : 0;
            t += x;
        }
        v[j] = pre + incl[j] - v[j];
        tot[j] = t;
    }
}

// ---------------------------------------------------------------------------
// routing of every token and grouping of assignments by expert
// ---------------------------------------------------------------------------
// logits of token t that a wave of its block routes (experts 256 i + 64 w +
// lane, route_candidates' layout) and the shared-gate logit: the KS partial sums of
// the router GEMM, every load issued at once, added in a fixed order
template <int EPL>
__device__ __forceinline__ void token_logits(const FwdArgs &a, int t, float (&zv)[EPL], float &gs) {
    const int E = a.s.E, T = a.T, ksn = router_ksplit(a.s.H);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float *zt = a.ws.zp + (size_t)t * (E + 1);
    const size_t kstride = (size_t)T * (E + 1);
    float z[kMaxKsplit][EPL], g[kMaxKsplit];
#pragma unroll
    for (int ks = 0; ks < kMaxKsplit; ++ks) {
        const float *zk = zt + (size_t)(ks < ksn ? ks : 0) * kstride;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = 256 * i + 64 * wave + lane;
            z[ks][i] = zk[e < E ? e : E - 1];
        }
        g[ks] = zk[E];
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) zv[i] = z[0][i];
    gs = g[0];
#pragma unroll
    for (int ks = 1; ks < kMaxKsplit; ++ks) {
        if (ks < ksn) {
#pragma unroll
            for (int i = 0; i < EPL; ++i) zv[i] += z[ks][i];
            gs += g[ks];
        }
    }
}

// ---------------------------------------------------------------------------
// pass records of the two streaming launches (0: gate/up, 1: down), written by
// the grouping block: the shared expert over token chunks of tp first (the
// heaviest passes start first; none when the launch runs the shared expert on
// the matrix cores), then every touched expert over chunks of tp of its
// assignments (token order), in expert order.  s_pv holds the assignments
// sorted by (expert, token) as output indices t * (K+1) + slot.
// ---------------------------------------------------------------------------
constexpr int kGroupThreads = 1024;

// ceil(c / tp) for 0 <= c <= 2^20 without an integer division: a float
// quotient, then exact integer corrections
__device__ __forceinline__ int passes_of(int c, int tp, float inv_tp) {
    int q = (int)((float)c * inv_tp);
    if (q * tp > c) --q;
    if ((q + 1) * tp <= c) ++q;  // q = floor(c / tp)
    return q + (q * tp < c ? 1 : 0);
}

// s_pp[launch][e]: first pass of expert e (the scan in group_assignments)
__device__ void build_passes(const FwdArgs &a, const StreamPlan &P0, const StreamPlan &P1, const int *s_cnt,
                             const int *s_off, const int *s_pv, const int (*s_pp)[kMaxExperts]) {
    constexpr int NT = kGroupThreads;
    const int T = a.T, E = a.s.E, K = a.s.K;
    // records: thread x takes (launch, shared pass or expert) items
    for (int launch = 0; launch < 2; ++launch) {
        const StreamPlan &P = launch == 0 ? P0 : P1;
        const int tp = P.tp;
        int32_t *rec = a.ws.sched + (size_t)launch * sched_launch_ints(T, K) + 4;
        const int n_shared = P.n_mfma > 0 ? 0 : (T + tp - 1) / tp;
        for (int x = threadIdx.x; x < n_shared + E; x += NT) {
            if (x < n_shared) {
                int32_t *r = rec + (size_t)x * kPassRecord;
                const int nv = min(tp, T - x * tp);
                r[0] = E;
                r[1] = nv;
                for (int v = 0; v < nv; ++v) r[2 + v] = (x * tp + v) * (K + 1) + K;
            } else {
                const int e = x - n_shared;
                const int cnt = s_cnt[e];
                const int first = s_off[e] - cnt;
                int32_t *r = rec + (size_t)s_pp[launch][e] * kPassRecord;
                for (int q0 = 0; q0 < cnt; q0 += tp, r += kPassRecord) {
                    const int nv = min(tp, cnt - q0);
                    r[0] = e;
                    r[1] = nv;
                    for (int v = 0; v < nv; ++v) r[2 + v] = s_pv[first + q0 + v];
                }
            }
        }
    }
}

// grouping of all T*K assignments by expert, by one block of 1024 threads:
// histogram, exclusive scans, the compact list of touched experts, and a
// stable scatter (token order kept inside each expert); then the pass
// records of the two streaming launches

__device__ void group_assignments(const FwdArgs &a, const StreamPlan &p0, const StreamPlan &p1) {
    constexpr int NT = kGroupThreads;
    const int T = a.T, E = a.s.E, K = a.s.K;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int TK = T * K;
    GroupView gv = group_view(a);
    int32_t *expert = (int32_t *)gv.expert;
    int32_t *first = (int32_t *)gv.first;
    int32_t *count = (int32_t *)gv.count;
    int32_t *perm = (int32_t *)gv.perm;

    __shared__ int s_sel[kGroupMaxAssign];
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int s_off[kMaxExperts];
    __shared__ int s_tch[kMaxExperts];
    __shared__ uint32_t s_mask[kMaxExperts];
    __shared__ int s_pv[kGroupMaxAssign];
    __shared__ int s_pp[2][kMaxExperts];  // first pass of each expert, per streaming launch
    __shared__ int s_scan[NT / 64 * 4];

    for (int i = threadIdx.x; i < E; i += NT) s_cnt[i] = 0;
    for (int i = threadIdx.x; i < TK; i += NT) s_sel[i] = a.ws.sel[i];
    __syncthreads();
    for (int i = threadIdx.x; i < TK; i += NT) atomicAdd(&s_cnt[s_sel[i]], 1);
    __syncthreads();
    // one block-wide exclusive scan over the experts (thread e holds expert e,
    // E <= 1024): assignment counts, touched flags and the passes of the two
    // streaming launches
    {
        static_assert(kMaxExperts <= NT, "one expert per thread");
        const int n_sh0 = p0.n_mfma > 0 ? 0 : (T + p0.tp - 1) / p0.tp;
        const int n_sh1 = p1.n_mfma > 0 ? 0 : (T + p1.tp - 1) / p1.tp;
        const int e = threadIdx.x;
        const int c = e < E ? s_cnt[e] : 0;
        int v[4] = {c, c > 0 ? 1 : 0, passes_of(c, p0.tp, 1.0f / (float)p0.tp), passes_of(c, p1.tp, 1.0f / (float)p1.tp)};
        int tot[4];
        block_excl_scan<4, NT>(v, tot, s_scan);
        if (e < E) {
            s_off[e] = v[0];
            s_tch[e] = v[1];
            s_pp[0][e] = n_sh0 + v[2];
            s_pp[1][e] = n_sh1 + v[3];
        }
        if (threadIdx.x == 0) {
            a.ws.grp[0] = tot[1];  // number of touched experts
            int32_t *h0 = a.ws.sched, *h1 = a.ws.sched + sched_launch_ints(T, K);
            h0[0] = n_sh0 + tot[2];
            h0[1] = p0.n_mfma + (n_sh0 + tot[2]) * p0.rpp;
            h1[0] = n_sh1 + tot[3];
            h1[1] = p1.n_mfma + (n_sh1 + tot[3]) * p1.rpp;
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += NT) {
        if (s_cnt[e] > 0) {
            const int u = s_tch[e];
            expert[u] = e;
            first[u] = s_off[e];
            count[u] = s_cnt[e];
        }
    }
    // stable scatter, 32 tokens at a time: bit t - c0 of s_mask[e] marks token t
    // as a user of expert e (the K experts of a token are distinct), so the rank
    // of (t, e) among e's assignments is the users before c0 (s_off advanced
    // chunk by chunk) plus the bits below t - c0
    for (int c0 = 0; c0 < T; c0 += 32) {
        for (int e = threadIdx.x; e < E; e += NT) s_mask[e] = 0u;
        __syncthreads();
        const int i0 = c0 * K, i1 = min(T, c0 + 32) * K;
        for (int i = i0 + threadIdx.x; i < i1; i += NT) atomicOr(&s_mask[s_sel[i]], 1u << (i / K - c0));
        __syncthreads();
        for (int i = i0 + threadIdx.x; i < i1; i += NT) {
            const int e = s_sel[i];
            const uint32_t below = s_mask[e] & ((1u << (i / K - c0)) - 1u);
            perm[s_off[e] + __popc(below)] = i;
            s_pv[s_off[e] + __popc(below)] = i + i / K;  // t * (K+1) + slot
        }
        __syncthreads();
        for (int e = threadIdx.x; e < E; e += NT) s_off[e] += __popc(s_mask[e]);
        __syncthreads();
    }
    // s_off[e] now ends expert e's assignments: its first is s_off[e] - s_cnt[e]
    build_passes(a, p0, p1, s_cnt, s_off, s_pv, s_pp);
}

// ---------------------------------------------------------------------------
// k_route_tokens: one block of four waves per token sums the partial logits of
// the router GEMM (a quarter of the experts per wave) and routes (softmax ->
// top-K -> renormalise, route_candidates and route_select).  k_group then groups the assignments of
// the whole batch in one block.  (A last-block-done counter inside one kernel
// would need an L2 write-back per block and same-address atomics across the
// XCDs, both slower here than the kernel boundary.)
// ---------------------------------------------------------------------------
template <int EPW>
__global__ __launch_bounds__(256) void k_route_tokens(FwdArgs a) {
    const int t = blockIdx.x, K = a.s.K, E = a.s.E;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __shared__ __align__(16) uint64_t s_cand[4 * kMaxTopK];
    float zq[EPW], gs;
    token_logits<EPW>(a, t, zq, gs);
    route_candidates<EPW>(zq, E, K, s_cand);
    __syncthreads();
    if (wave == 0) {
        const RouteSel rt = route_select(K, s_cand);
        if (rt.rank < K) {
            a.ws.sel[t * K + rt.rank] = rt.sel;
            a.ws.coef[t * (K + 1) + rt.rank] = rt.w;
            if (a.route_idx) a.route_idx[t * K + rt.rank] = rt.sel;
            if (a.route_w) a.route_w[t * K + rt.rank] = rt.w;
        }
        if (lane == 0) a.ws.coef[t * (K + 1) + K] = sigmoidf_(gs);
    }
}

__global__ __launch_bounds__(kGroupThreads) void k_group(FwdArgs a, StreamPlan p0, StreamPlan p1) {
    group_assignments(a, p0, p1);
}

// the pass records of a streaming launch, read through the constant address
// space: scalar loads, which the weight loads' wait counter does not include
typedef const int32_t __attribute__((address_space(4))) const_i32;

struct SchedView {
    const const_i32 *head;  // [0] passes, [1] runs
    const const_i32 *rec;   // kPassRecord ints per pass
};

__device__ __forceinline__ SchedView sched_view(const FwdArgs &a, int launch) {
    SchedView v;
    v.head = (const const_i32 *)(a.ws.sched + (size_t)launch * sched_launch_ints(a.T, a.s.K));
    v.rec = v.head + 4;
    return v;
}

// ---------------------------------------------------------------------------
// k_encode_act: limb form of every (token, slot) activation vector, in the
// order of the down projection's byte-order codes.  A thread takes 16
// consecutive activations, four threads one group of 64.
//   4-bit: the code dword covering k = 8w .. 8w+7 holds k = 8w + m in nibble
//          2 (m % 4) + m / 4, so the limb dword w puts k = 8w + (n >> 1) + 4 (n & 1)
//          in nibble n.
//   2-bit: the code dword covering k = 16w .. 16w+15 holds k = 16w + m in byte
//          m % 4 at bit 2 (m / 4); its two masked halves (bits 0-1, bits 2-3 of
//          each nibble) are dotted with limb dwords 2w and 2w+1, which put
//          k = 16w + (n >> 1) + 4 p + 8 (n & 1) in nibble n (p = 0, 1).
// ---------------------------------------------------------------------------
// sks > 0: the shared expert's gate and up sums arrive as sks partial sums
// of matrix-core units over reduction chunks, and its down product runs on
// the matrix cores too: blocks past pair_blocks add the partials in chunk
// order, apply SwiGLU and write that slot's bf16 fragments and half-group
// sums (a thread per 4 values, every partial's load issued at once); the
// pair blocks skip the slot.
__device__ __forceinline__ void shared_act(const FwdArgs &a, int sks, int b) {
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    const int F = a.s.F, K = a.s.K, T = a.T;
    const int gt = b * 256 + threadIdx.x;
    const int t = gt / (F / 4), k0 = (gt % (F / 4)) * 4;
    if (t >= T) return;  // whole groups of 8 lanes (F / 4 is a multiple of 8)
    f32x4v q[kMaxMfmaKsplit][2];
#pragma unroll
    for (int kc = 0; kc < kMaxMfmaKsplit; ++kc)
#pragma unroll
        for (int m = 0; m < 2; ++m)
            q[kc][m] = *(const f32x4v *)(a.ws.sp + ((size_t)((kc < sks ? kc : 0) * 2 + m) * T + t) * F + k0);
    f32x4v g = q[0][0], u = q[0][1];
#pragma unroll
    for (int kc = 1; kc < kMaxMfmaKsplit; ++kc) {
        g = kc < sks ? g + q[kc][0] : g;
        u = kc < sks ? u + q[kc][1] : u;
    }
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = g[i] * u[i] * __builtin_amdgcn_rcpf(1.0f + __expf(-g[i]));
    // fragments: values k0 .. k0+3 of token t, three bf16 parts
    uint16_t *f = a.ws.ab + ((size_t)(t >> 5) * (F / 16) + k0 / 16) * 3 * 512 + ((t & 31) + 32 * ((k0 % 16) / 8)) * 8 +
                  (k0 % 8);
    float r[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
    for (int p = 0; p < 3; ++p) {
        uint32_t w[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t lo = bf16_rne_bits(r[2 * i]), hi = bf16_rne_bits(r[2 * i + 1]);
            w[i] = lo | (hi << 16);
            r[2 * i] -= __uint_as_float(lo << 16);
            r[2 * i + 1] -= __uint_as_float(hi << 16);
        }
        *(uint2 *)(f + p * 512) = make_uint2(w[0], w[1]);
    }
    // half-group sums: 8 threads of 4 values
    float sum = (v[0] + v[1]) + (v[2] + v[3]);
    sum += __shfl_xor(sum, 1, 64);
    sum += __shfl_xor(sum, 2, 64);
    sum += __shfl_xor(sum, 4, 64);
    if ((k0 & 31) == 0) a.ws.ax[((size_t)t * (K + 1) + K) * (F / 32) + k0 / 32] = sum;
}

template <int BITS>
__global__ __launch_bounds__(256) void k_encode_act(FwdArgs a, int n_pairs, int sks, int pair_blocks) {
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    if (BITS == 4 && (int)blockIdx.x >= pair_blocks) {
        shared_act(a, sks, blockIdx.x - pair_blocks);
        return;
    }
    const int F = a.s.F, K = a.s.K;
    const int tpp = F / 16;  // threads per pair (a multiple of 8)
    const int p = blockIdx.x * (256 / tpp) + threadIdx.x / tpp;
    const int u = threadIdx.x % tpp;
    const bool live = p < n_pairs && !(sks > 0 && p % (K + 1) == K);
    float v[16];
    {
        const f32x4v *src = (const f32x4v *)(a.ws.act + (size_t)(p < n_pairs ? p : 0) * F + 16 * u);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4v q = src[i];
            v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
        }
    }
    float m = 0.0f, sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        m = nan_max(m, fabsf(v[i]));
        sum += v[i];
    }
    sum += __shfl_xor(sum, 1, 64);  // half group (32 values)
    m = nan_max(m, __shfl_xor(m, 1, 64));
    m = nan_max(m, __shfl_xor(m, 2, 64));  // group of 64
    uint32_t pk[kLimbs][2];
#pragma unroll
    for (int x = 0; x < kLimbs; ++x) pk[x][0] = pk[x][1] = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        int l[kLimbs];
        limb_split(limb_value(v[i], m), l);
        int dw, nib;
        if constexpr (BITS == 4) {
            const int mm = i % 8;
            dw = i / 8;
            nib = 2 * (mm % 4) + mm / 4;
        } else {
            dw = (i / 4) % 2;
            nib = 2 * (i % 4) + i / 8;
        }
#pragma unroll
        for (int x = 0; x < kLimbs; ++x) pk[x][dw] |= (uint32_t)(l[x] & 15) << (4 * nib);
    }
    if (live) {
        uint32_t *al = (uint32_t *)a.ws.al + (size_t)p * kLimbs * (F / 8) + 2 * u;
#pragma unroll
        for (int x = 0; x < kLimbs; ++x) *(uint2 *)(al + (size_t)x * (F / 8)) = make_uint2(pk[x][0], pk[x][1]);
        if ((u & 1) == 0) a.ws.ax[(size_t)p * (F / 32) + u / 2] = sum;
        if ((u & 3) == 0) a.ws.as[(size_t)p * (F / 64) + u / 4] = limb_scale(m);
        // the shared slot also as bf16 fragments, the operand of its matrix-core down product
        if (BITS == 4 && p % (K + 1) == K) store_split_fragments(a.ws.ab, F, p / (K + 1), u, v);  // sks == 0
    }
}

// ---------------------------------------------------------------------------
// k_grouped_stream: the dequant GEMV of the expert matrix pair (gate + up, with
// SwiGLU) or of the down matrix, for every pass of a launch.
//
// A pass applies one expert's rows to up to tp of its vectors (tokens h for
// gate/up, (token, slot) activations for down); the shared expert's passes
// take chunks of tp tokens.  Passes are cut into runs of block-steps, and the
// grid is persistent: block b takes run b, then claims further runs from the
// counter of its group, one run ahead, so that the grid drains evenly however
// fast each block streams (fixed per-block work leaves a tail as long as one
// block at partial occupancy).  For each run a block stages the pass's
// vectors in LDS; every wave streams its row slots: the weights of the next
// block-step (across run boundaries too) are loaded into one register set
// while the current one is computed from the other, so HBM requests stay in
// flight through the compute, and each step's rows are applied to every
// staged vector.  No block waits on another: the claims are the only shared
// state, and the last block to leave resets the counters.
// ---------------------------------------------------------------------------
// words of one staged vector of length n: limbs [kLimbs][n/8], scales [n/64], half
// sums [n/32], rounded up to 16 bytes
MOE_HD int stage_words(int n) { return (kLimbs * (n / 8) + n / 64 + n / 32 + 3) & ~3; }

template <int BITS, int CPL, int NM, int RPW>
struct StepWeights {
    using Q = QSlice<BITS, CPL>;
    uint4 c[NM][RPW][CPL];
    uint32_t sb[NM][RPW][Q::NGL];
};

// block barrier for LDS only: no wait for global loads or stores in flight
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// a run: its expert matrices, pass and row-step range
struct StreamRun {
    const uint8_t *ex;
    int pass, rs_lo, rs_hi, nsteps;
};

// ---------------------------------------------------------------------------
// The shared expert on the matrix cores (4-bit codes).  Every token of the
// batch uses it, so it is a dense product [rows x n] x [n x T].  A unit is 128
// rows (32 per wave) by one tile of 32 tokens over the whole reduction, on
// v_mfma_f32_32x32x16_bf16: the codes enter as 16 + q, exact in bf16; the
// activations as their three bf16 parts (hi, mid, lo; written in fragment
// order by k_norm_batch and k_encode_act); the fp32 product C of each group
// of 64 is folded as s * C + (b - 16 s) * sum(v).  The block stages every
// group's fragments, per-row scale s and offset b - 16 s, and per-token sums
// in a ring of three LDS buffers, two groups ahead.
// Lane layouts of the 32x32x16 product: A lane l holds row l % 32 and the
// step's reduction entries 8 (l / 32) .. +7; B lane l holds those entries of
// token l % 32; result v of lane l is row 8 (v / 4) + 4 (l / 32) + v % 4,
// token l % 32.  A lane loads the 16-byte chunk (32 codes) of its row that
// covers half l / 32 of the group; one v_permlane32_swap per two dwords gives
// each lane the 8-code dword of every step.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

constexpr int kMfmaFrag = 12 * 64;     // 16-byte fragments of a group: 4 steps x 3 parts x 64 lanes
constexpr int kMfmaMinTokens = 32;     // smaller batches keep the shared expert in passes (a half-empty tile measured slower)
MOE_HD int mfma_buf_words(bool down) { return kMfmaFrag * 4 + (down ? 1 : 2) * 256 + 32; }
MOE_HD int mfma_lds_bytes(bool down) { return 3 * mfma_buf_words(down) * 4; }

// the 8 codes of a dword as bf16 values 16 + q in reduction order (4 dwords,
// value 2j in the low half of dword j): one byte-select and one shift-or per
// two codes.  Nibble order: code j in nibble j, stored as q XOR 8; byte order:
// code j in byte j % 4 at bit 4 (j / 4).
template <bool BYTE_CODES>
__device__ __forceinline__ u32x4v codes_bf16(uint32_t d) {
    if constexpr (!BYTE_CODES) d ^= 0x88888888u;
    const uint32_t lo = d & 0x0F0F0F0Fu, hi = (d >> 4) & 0x0F0F0F0Fu;
    u32x4v r;
    if constexpr (BYTE_CODES) {
        r.x = __builtin_amdgcn_perm(hi, lo, 0x0C010C00u);
        r.y = __builtin_amdgcn_perm(hi, lo, 0x0C030C02u);
        r.z = __builtin_amdgcn_perm(hi, lo, 0x0C050C04u);
        r.w = __builtin_amdgcn_perm(hi, lo, 0x0C070C06u);
    } else {
        r.x = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u);
        r.y = __builtin_amdgcn_perm(hi, lo, 0x0C050C01u);
        r.z = __builtin_amdgcn_perm(hi, lo, 0x0C060C02u);
        r.w = __builtin_amdgcn_perm(hi, lo, 0x0C070C03u);
    }
    return (r << 3u) | 0x41804180u;  // bf16(16 + q) = 0x4180 | q << 3
}

// unit = (token tile, row block, reduction chunk), the chunk fastest; with
// ks > 1 chunks the unit writes fp32 partial sums (gate/up only), which
// k_encode_act adds in chunk order
template <bool DOWN>
__device__ void shared_mfma_unit(const FwdArgs &a, int unit, int ks, uint32_t *lds) {
    constexpr int NM = DOWN ? 1 : 2;
    constexpr int NSB = NM * 128;  // scale/bias words of a group: NM matrices x 128 rows
    const int H = a.s.H, F = a.s.F, K = a.s.K, T = a.T;
    const int n = DOWN ? F : H, rows = DOWN ? H : F;
    const int nrb = rows / 128, gpu = (n / 64) / ks;  // groups per unit (>= 2)
    const int kc = unit % ks, rt = unit / ks;
    const int tt = rt / nrb, rb = rt - tt * nrb;
    const int g0 = kc * gpu, ng = g0 + gpu;  // the unit's groups: g0 .. ng-1
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5;
    const int row = rb * 128 + wave * 32 + (lane & 31);
    const QMat &M0 = a.L.m[DOWN ? 2 : 0];
    const QMat &M1 = a.L.m[1];
    const u32x4v *frag = (const u32x4v *)(DOWN ? a.ws.ab : a.ws.hb) + (size_t)tt * (n / 16) * 3 * 64;
    const int bw = mfma_buf_words(DOWN);
    // staging of group g, loads: fragments i, i+256, i+512 of thread i; the
    // scale/bias word of row i % NSB (a thread past NSB re-reads row i % NSB);
    // the group sum of token i % 32 (clamped to the batch)
    auto stage_load = [&](int g, u32x4v (&fp)[3], uint32_t &sbw, float &xs) {
        const u32x4v *src = frag + (size_t)g * kMfmaFrag;
#pragma unroll
        for (int j = 0; j < 3; ++j) fp[j] = src[threadIdx.x + 256 * j];
        const int i = threadIdx.x & (NSB - 1);
        const QMat &M = (i >> 7) ? M1 : M0;
        sbw = ld_stream4((const uint32_t *)(a.shared + M.sb_off) + (size_t)(rb * 128 + (i & 127)) * M.ngroups + g);
        const int tok = tt * 32 + (threadIdx.x & 31);
        const int tc = tok < T ? tok : T - 1;
        const float *hx = DOWN ? a.ws.ax + (size_t)(tc * (K + 1) + K) * (F / 32) : a.ws.hx + (size_t)tc * (H / 32);
        xs = hx[2 * g] + hx[2 * g + 1];
    };
    // stores (every index in range: duplicate writers store equal values)
    auto stage_store = [&](int g, const u32x4v (&fp)[3], uint32_t sbw, float xs) {
        uint32_t *buf = lds + (g % 3) * bw;
#pragma unroll
        for (int j = 0; j < 3; ++j) ((u32x4v *)buf)[threadIdx.x + 256 * j] = fp[j];
        const float sc = bf16_lo(sbw);
        float *so = (float *)(buf + kMfmaFrag * 4) + 2 * (threadIdx.x & (NSB - 1));
        so[0] = sc;
        so[1] = fmaf(-16.0f, sc, bf16_hi(sbw));
        ((float *)buf)[kMfmaFrag * 4 + 2 * NSB + (threadIdx.x & 31)] = xs;
    };
    // the lane's code chunk of group g: logical chunk 2 g + half of its row
    auto load_codes = [&](int g, uint4 (&ac)[NM]) {
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const QMat &M = m ? M1 : M0;
            const int L = 2 * g + half;
            ac[m] = ld_stream16(a.shared + M.codes_off + (size_t)row * M.row_bytes + 16 * (L / M.cpl + M.lpr * (L % M.cpl)));
        }
    };

    f32x16_t acc[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[m] = f32x16_t{};
    {
        u32x4v fp[3];
        uint32_t sbw;
        float xs;
        stage_load(g0, fp, sbw, xs);
        stage_store(g0, fp, sbw, xs);
        stage_load(g0 + 1, fp, sbw, xs);  // at least two groups per unit
        stage_store(g0 + 1, fp, sbw, xs);
    }
    uint4 ac[NM];
    load_codes(g0, ac);
    for (int g = g0; g < ng; ++g) {
        lds_barrier();  // group g's buffer is complete; group g - 1's is free
        // group g + 2 into the freed buffer (past the end: the last group again,
        // into a buffer no later group reads), the next group's codes
        const int g2 = g + 2 < ng ? g + 2 : ng - 1;
        u32x4v fp[3];
        uint32_t sbw;
        float xs;
        stage_load(g2, fp, sbw, xs);
        uint4 an[NM];
        load_codes(g + 1 < ng ? g + 1 : g, an);
        const uint32_t *buf = lds + (g % 3) * bw;
        const u32x4v *bf = (const u32x4v *)buf;
        const float X = ((const float *)buf)[kMfmaFrag * 4 + 2 * NSB + (lane & 31)];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const auto p01 = __builtin_amdgcn_permlane32_swap(ac[m].x, ac[m].y, false, false);
            const auto p23 = __builtin_amdgcn_permlane32_swap(ac[m].z, ac[m].w, false, false);
            const uint32_t dw[4] = {p01[0], p23[0], p01[1], p23[1]};  // the dword of steps 0 .. 3
            f32x16_t c = f32x16_t{};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const bf16x8_t av = __builtin_bit_cast(bf16x8_t, codes_bf16<DOWN>(dw[st]));
#pragma unroll
                for (int p = 2; p >= 0; --p)
                    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8_t, bf[(st * 3 + p) * 64 + lane]),
                                                                c, 0, 0, 0);
            }
            // fold: rows 8 j + 4 half + i of the wave's 32, (s, b - 16 s) pairs
            const float *so = (const float *)(buf + kMfmaFrag * 4) + 2 * (m * 128 + wave * 32 + 4 * half);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x4v q0 = *(const u32x4v *)(so + 16 * j);
                const u32x4v q1 = *(const u32x4v *)(so + 16 * j + 4);
                const float sv[4] = {__uint_as_float(q0.x), __uint_as_float(q0.z), __uint_as_float(q1.x),
                                     __uint_as_float(q1.z)};
                const float ov[4] = {__uint_as_float(q0.y), __uint_as_float(q0.w), __uint_as_float(q1.y),
                                     __uint_as_float(q1.w)};
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[m][4 * j + i] = fmaf(sv[i], c[4 * j + i], fmaf(ov[i], X, acc[m][4 * j + i]));
            }
        }
        stage_store(g2, fp, sbw, xs);
#pragma unroll
        for (int m = 0; m < NM; ++m) ac[m] = an[m];
    }
    const int tok = tt * 32 + (lane & 31);
    if (tok < T) {
        const size_t pv = (size_t)tok * (K + 1) + K;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = rb * 128 + wave * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
            if constexpr (DOWN) {
                a.ws.ys[pv * H + r] = acc[0][v];
            } else if (ks > 1) {
                a.ws.sp[((size_t)(kc * 2 + 0) * T + tok) * F + r] = acc[0][v];
                a.ws.sp[((size_t)(kc * 2 + 1) * T + tok) * F + r] = acc[1][v];
            } else {
                const float g = acc[0][v];
                a.ws.act[pv * F + r] = g * acc[1][v] * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
            }
        }
    }
}

// LPR: lanes per row when the partial sums of a step are reduced together
// (16, 32 or 64); 0: any other width, one reduction per row
template <int BITS, int CPL, int RPW, bool DOWN, int LPR>
__global__ __launch_bounds__(256) void k_grouped_stream(FwdArgs a, StreamPlan plan) {
    using Q = QSlice<BITS, CPL>;
    using W = StepWeights<BITS, CPL, DOWN ? 1 : 2, RPW>;
    constexpr int NM = DOWN ? 1 : 2;
    constexpr int NV = NM * RPW;  // partial sums per lane per step and vector
    constexpr int launch = DOWN ? 1 : 0;
    extern __shared__ uint4 s_dyn[];
    uint32_t *s_vec = (uint32_t *)s_dyn;
    __shared__ int s_out[kMaxPassVectors];  // output vector index (t * (K+1) + slot) per staged vector
    __shared__ int s_next;                    // the run claimed for after the next one
    __shared__ int s_first;                   // after a matrix-core unit: the first streaming run
    const int H = a.s.H, F = a.s.F, K = a.s.K, E = a.s.E;
    const int n = DOWN ? F : H;  // reduction length
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const GroupView gv = group_view(a);
    const SchedView sv = sched_view(a, launch);
    const int grp = blockIdx.x % kClaimGroups;
    uint32_t *run_ctr = a.ws.ctrl + ctrl_run_counter(launch, grp);
    uint32_t *exit_ctr = a.ws.ctrl + ctrl_exit_counter(launch, grp);
    const QMat &M0 = a.L.m[DOWN ? 2 : 0];
    const QMat &M1 = a.L.m[1];
    const int lpr = LPR ? LPR : M0.lpr, rpi = 64 / lpr;
    const int lr = lane % lpr, rsub = lane / lpr;
    const int nrs = M0.rows / rpi;
    const int words = stage_words(n);
    const int k0 = lr * Q::NV;
    const int out_len = DOWN ? H : F;
    float *out_base = DOWN ? a.ws.ys : a.ws.act;
    const int nb = (int)gridDim.x;
    const int n_runs = sv.head[1];

    // runs 0 .. n_mfma-1 are matrix-core units of the shared expert; run r
    // after them is run r - n_mfma of the passes
    auto run_of = [&](int r) {
        StreamRun R;
        r -= plan.n_mfma;
        R.pass = r / plan.rpp;
        const int b0 = (r - R.pass * plan.rpp) * plan.run_items;
        const int b1 = min(plan.nbs, b0 + plan.run_items);
        const int expert = sv.rec[(size_t)R.pass * kPassRecord];
        R.ex = expert == E ? a.shared : a.experts + (size_t)expert * a.L.bytes;
        R.rs_lo = b0 * 4 * RPW;
        R.rs_hi = min(nrs, b1 * 4 * RPW);
        R.nsteps = b1 - b0;
        return R;
    };
    // unconditional loads (rows past the run re-read its last row, unused)
    // so that no wait separates them
    auto load_step = [&](const uint8_t *ex, int rs_lo, int rs_hi, int s, W &w) {
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int r0 = rs_lo + (s * 4 + wave) * RPW + i;
            const int rs = r0 < rs_hi ? r0 : rs_hi - 1;
            load_row<BITS, CPL>(ex, M0, rs * rpi + rsub, lr, w.c[0][i], w.sb[0][i]);
            if constexpr (NM == 2) load_row<BITS, CPL>(ex, M1, rs * rpi + rsub, lr, w.c[1][i], w.sb[1][i]);
        }
    };
    auto compute_step = [&](const StreamRun &R, int s, int np, W &w) {
        const int rs0 = R.rs_lo + (s * 4 + wave) * RPW;
        float sc[NV][Q::NGL], of[NV][Q::NGL];
#pragma unroll
        for (int i = 0; i < RPW; ++i)
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                // the down matrix's 4-bit codes (byte order) made signed, q XOR 8, as
                // the gate and up codes are stored
                if constexpr (DOWN && BITS == 4) {
#pragma unroll
                    for (int j = 0; j < CPL; ++j) {
                        uint4 &c = w.c[m][i][j];
                        c = make_uint4(c.x ^ 0x88888888u, c.y ^ 0x88888888u, c.z ^ 0x88888888u, c.w ^ 0x88888888u);
                    }
                }
#pragma unroll
                for (int g = 0; g < Q::NGL; ++g) {
                    sc[NM * i + m][g] = bf16_lo(w.sb[m][i][g]);
                    of[NM * i + m][g] = fmaf(Q::kCodeOffset, sc[NM * i + m][g], bf16_hi(w.sb[m][i][g]));
                }
            }
        // row-major list of the step's rows: entry NM * i + m
        uint4 cl[NV][CPL];
#pragma unroll
        for (int i = 0; i < RPW; ++i)
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int j = 0; j < CPL; ++j) cl[NM * i + m][j] = w.c[m][i][j];
        for (int v = 0; v < np; ++v) {
            const uint32_t *vec = s_vec + (size_t)v * words;
            float *out = out_base + (size_t)s_out[v] * out_len;
            float part[NV];
            rows_dot_lds<BITS, CPL, NV>(cl, sc, of, vec, (const float *)(vec + kLimbs * (n / 8)),
                                        (const float *)(vec + kLimbs * (n / 8) + n / 64), n, k0, part);
            if constexpr (LPR != 0) {
                // every row of the step at once; rows past the run are computed
                // on stale registers and not written
                const float r = multi_reduce<NV, LPR>(part);
                constexpr int DL = LPR / NV;  // lanes sharing one reduced entry
                const int j = multi_index<NV, LPR>(lane);
                const int rs = rs0 + j / NM;
                if constexpr (DOWN) {
                    if ((lane & (DL - 1)) == 0 && rs < R.rs_hi) out[rs * rpi + rsub] = r;
                } else {
                    const float up = xchg<DL>(r);  // the up sum sits across the last halving bit
                    const float act = r * up * __builtin_amdgcn_rcpf(1.0f + __expf(-r));
                    if ((lane & (2 * DL - 1)) == 0 && rs < R.rs_hi) out[rs * rpi + rsub] = act;
                }
            } else {
#pragma unroll
                for (int i = 0; i < RPW; ++i) {
                    const int rs = rs0 + i;
                    if (rs < R.rs_hi) {
                        if constexpr (DOWN) {
                            const float y = lane_group_sum(part[i], lpr);
                            if (lr == 0) out[rs * rpi + rsub] = y;
                        } else {
                            const float g = lane_group_sum(part[2 * i], lpr);
                            const float up = lane_group_sum(part[2 * i + 1], lpr);
                            if (lr == 0) out[rs * rpi + rsub] = g * up * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
                        }
                    }
                }
            }
        }
    };
    // stage a run's vectors: limbs as 16-byte pieces, then scales and half
    // sums, every load of a vector issued before its single wait (indices
    // clamped, stores guarded); returns the vector count
    auto stage = [&](const StreamRun &R) {
        constexpr int kPieces = (kLimbs * kMaxDim / 32 + 255) / 256;
        const const_i32 *rec = sv.rec + (size_t)R.pass * kPassRecord;
        const int np = rec[1];
        const int nl = kLimbs * n / 32, ng = n / 64, nh = n / 32;
        for (int v = 0; v < np; ++v) {
            const int pv = rec[2 + v];
            const int t = pv / (K + 1);
            if (threadIdx.x == 0) s_out[v] = pv;
            const uint4 *hl = DOWN ? (const uint4 *)((const uint32_t *)a.ws.al + (size_t)pv * kLimbs * (F / 8))
                                   : (const uint4 *)((const uint32_t *)a.ws.hl + (size_t)t * kLimbs * (H / 8));
            const float *hs = DOWN ? a.ws.as + (size_t)pv * (F / 64) : a.ws.hs + (size_t)t * (H / 64);
            const float *hx = DOWN ? a.ws.ax + (size_t)pv * (F / 32) : a.ws.hx + (size_t)t * (H / 32);
            // every index wraps (i mod count): past the end a lane rewrites
            // an entry that another lane writes too, with the same value, at
            // its own address (a guarded store would let the compiler sink its
            // load into the guard, one wait per load; a clamped one would put
            // every such lane on one LDS word)
            // (a native vector type: an array of uint4 here keeps dead copies in
            // scratch memory, each store waiting for its load)
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            int li[kPieces];
            u32x4 lp[kPieces];
#pragma unroll
            for (int j = 0; j < kPieces; ++j) {
                li[j] = (int)((threadIdx.x + 256u * j) % (unsigned)nl);
                lp[j] = ((const u32x4 *)hl)[li[j]];
            }
            const int gi = threadIdx.x & (ng - 1), xi = threadIdx.x & (nh - 1);  // ng, nh: powers of two
            const float gs = hs[gi];
            const float xs = hx[xi];
            uint32_t *dst = s_vec + (size_t)v * words;
#pragma unroll
            for (int j = 0; j < kPieces; ++j) ((u32x4 *)dst)[li[j]] = lp[j];
            dst[kLimbs * (n / 8) + gi] = __float_as_uint(gs);
            dst[kLimbs * (n / 8) + ng + xi] = __float_as_uint(xs);
        }
        return np;
    };

    uint32_t claim = 0;  // thread 0: the counter value of the last claim
    // thread 0, once the claim made earlier has returned: publish its run (or
    // -1 past the last) and claim the run after it
    auto take_claim = [&]() {
        const int r = nb + kClaimGroups * (int)claim + grp;
        s_next = r < n_runs ? r : -1;
        if (r < n_runs) claim = atomicAdd(run_ctr, 1u);
    };
    int cur_r = blockIdx.x;
    if constexpr (BITS == 4) {
        // matrix-core units first: a block's claims come in increasing order,
        // so every unit precedes every streaming run
        while (cur_r >= 0 && cur_r < plan.n_mfma) {
            shared_mfma_unit<DOWN>(a, cur_r, plan.mfma_ks, s_vec);
            if (threadIdx.x == 0) {
                claim = atomicAdd(run_ctr, 1u);
                const int r = nb + kClaimGroups * (int)claim + grp;
                s_first = r < n_runs ? r : -1;
            }
            lds_barrier();  // the unit is done with LDS; s_first visible
            cur_r = s_first;
        }
    }
    if (cur_r >= 0 && cur_r < n_runs) {
        if (threadIdx.x == 0) claim = atomicAdd(run_ctr, 1u);
        StreamRun cur = run_of(cur_r);
        W w0, w1;
        load_step(cur.ex, cur.rs_lo, cur.rs_hi, 0, w0);  // in flight while the vectors are staged
        int np = stage(cur);
        if (threadIdx.x == 0) take_claim();  // after the staging loads' wait
        lds_barrier();
        int nxt_r = s_next;
        StreamRun nxt = run_of(nxt_r >= 0 ? nxt_r : cur_r);
        int s = 0;  // step of `cur` computed next
        // one block-step: load the one after it (the next step, else the next
        // run's first, else this one again, unused: the loads are
        // unconditional, since a load issued on one path only would make the
        // waits after the join count for the path without it), compute this
        // one, and cross into the next run at the end of this one.  At the
        // crossing the claim made one run earlier is read (its wait also
        // covers the next step's weights, which the staging waits for anyway)
        // and the next claim goes out just before the staging loads.
        auto advance = [&](W &wc, W &wl) {
            const bool in_cur = s + 1 < cur.nsteps;
            const bool to_nxt = !in_cur && nxt_r >= 0;
            const uint8_t *lex = to_nxt ? nxt.ex : cur.ex;
            const int llo = to_nxt ? nxt.rs_lo : cur.rs_lo, lhi = to_nxt ? nxt.rs_hi : cur.rs_hi;
            const int ls = in_cur ? s + 1 : (to_nxt ? 0 : s);
            load_step(lex, llo, lhi, ls, wl);
            compute_step(cur, s, np, wc);
            if (in_cur) {
                ++s;
                return true;
            }
            if (nxt_r < 0) return false;
            lds_barrier();  // the run is done with LDS
            cur_r = nxt_r;
            cur = nxt;
            if (threadIdx.x == 0) take_claim();  // the new claim returns with the staging loads
            np = stage(cur);
            lds_barrier();  // staged vectors and s_next visible
            nxt_r = s_next;
            nxt = run_of(nxt_r >= 0 ? nxt_r : cur_r);
            s = 0;
            return true;
        };
        while (advance(w0, w1) && advance(w1, w0)) {
        }
    }
    // the last block of the group to leave resets the group's counters for
    // the next launch (its own last claim has returned: the exit count
    // depends on it)
    if (threadIdx.x == 0) {
        const uint32_t prior = atomicAdd(exit_ctr, claim != 0xffffffffu ? 1u : 2u);
        if (prior == (uint32_t)(nb / kClaimGroups) - 1u) {
            atomicExch(run_ctr, 0u);
            atomicExch(exit_ctr, 0u);
        }
    }
}

// ---------------------------------------------------------------------------
// k_combine: out = x + sum_k w_k y_k + sigmoid(g_s) y_shared, in slot order
// (k = 0 .. K, the shared slot last).  A thread takes four outputs; the loads
// of every slot are issued at once (slot index clamped, the extra terms
// dropped by a select, not a branch: a load used only under a branch would
// be sunk into it and wait there, one slot at a time).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_combine(FwdArgs a) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const int H = a.s.H, K = a.s.K;
    const int t = blockIdx.y;
    const int o = (blockIdx.x * 64 + threadIdx.x) * 4;
    if (o >= H) return;
    const float *c = a.ws.coef + (size_t)t * (K + 1);
    const float *ys = a.ws.ys + (size_t)t * (K + 1) * H + o;
    f32x4 acc = *(const f32x4 *)(a.x + (size_t)t * H + o);
    f32x4 v[kMaxTopK + 1];
    float w[kMaxTopK + 1];
#pragma unroll
    for (int k = 0; k <= kMaxTopK; ++k) {
        const int kk = k <= K ? k : K;
        v[k] = *(const f32x4 *)(ys + (size_t)kk * H);
        w[k] = c[kk];
    }
#pragma unroll
    for (int k = 0; k <= kMaxTopK; ++k) {
        f32x4 r;
        r.x = fmaf(w[k], v[k].x, acc.x);
        r.y = fmaf(w[k], v[k].y, acc.y);
        r.z = fmaf(w[k], v[k].z, acc.z);
        r.w = fmaf(w[k], v[k].w, acc.w);
        acc = k <= K ? r : acc;
    }
    *(f32x4 *)(a.y + (size_t)t * H + o) = acc;
}

// row-slots per wave and step of k_grouped_stream: two register sets of
// weights stay within ~80 VGPRs
constexpr int stream_rpw(int cpl) { return cpl == 1 ? 4 : 2; }
// block-steps per run (8 rows per gate/up step, 32 per down step): short runs
// keep the end of the grid tight, since a block holds its current run and the
// one it has claimed ahead (runs of 8 and 4 steps left the last blocks ~40 us
// behind the median in a 200 us gate/up launch; 4 and 2 halve that)
constexpr int kGateUpRunItems = 4;
constexpr int kDownRunItems = 2;

// vectors staged per pass: as many as fit the block's LDS budget (48 KiB for
// gate/up, 40 KiB for down), at most 16.  The grid is as many blocks as the
// occupancy query allows at that LDS size: registers make it two per CU for
// gate/up (three, with the registers capped to fit, measured no faster) and
// four for down.
inline int stream_vectors(int n, bool down) {
    const int budget = (down ? 40 : 48) * 1024;
    const int v = budget / (stage_words(n) * 4);
    return v < kMaxPassVectors ? v : kMaxPassVectors;
}

// block slots of the GPU for a kernel (cached per kernel, LDS size and device)
hipError_t stream_block_slots(const void *fn, size_t lds, int &slots) {
    struct Entry {
        const void *fn;
        size_t lds;
        int dev, slots;
    };
    static std::mutex mu;
    static Entry cache[64];
    static int n_cache = 0;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < n_cache; ++i)
        if (cache[i].fn == fn && cache[i].lds == lds && cache[i].dev == dev) {
            slots = cache[i].slots;
            return hipSuccess;
        }
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, lds);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (per_cu < 1 || cus < 1) return hipErrorInvalidConfiguration;
    slots = per_cu * cus;
    if (n_cache < 64) cache[n_cache++] = Entry{fn, lds, dev, slots};
    return hipSuccess;
}

// the plan of one streaming launch (and, with launch set, the launch itself)
struct StreamOp {
    const FwdArgs *a;
    hipStream_t st;
    bool launch;
    StreamPlan plan;
    template <int BITS, int CPL, bool DOWN, int LPR>
    hipError_t run() {
        constexpr int rpw = stream_rpw(CPL);
        auto fn = k_grouped_stream<BITS, CPL, rpw, DOWN, LPR>;
        const QMat &M = a->L.m[DOWN ? 2 : 0];
        const int rpi = 64 / M.lpr;
        const int nrs = M.rows / rpi;
        const int n = DOWN ? a->s.F : a->s.H;
        StreamPlan p;
        p.tp = stream_vectors(n, DOWN);
        p.nbs = (nrs + 4 * rpw - 1) / (4 * rpw);
        p.run_items = DOWN ? kDownRunItems : kGateUpRunItems;
        p.rpp = (p.nbs + p.run_items - 1) / p.run_items;
        size_t lds = (size_t)p.tp * stage_words(n) * 4;
        p.n_mfma = 0;
        p.mfma_ks = 1;
        if (BITS == 4 && a->T >= kMfmaMinTokens) {
            // the shared expert on the matrix cores: one unit per 128 rows and
            // 32-token tile, each a block's first run
            const size_t lds_m = lds > (size_t)mfma_lds_bytes(DOWN) ? lds : (size_t)mfma_lds_bytes(DOWN);
            // gate/up: chunks of 8 groups (a unit's groups run one after the
            // other, each waiting on HBM: 64 in a row made the units the
            // critical path); down: the whole reduction (16 groups at F = 1024).
            // The split depends on the shape only, so that a token's result
            // does not depend on its batch.
            const int ng = n / 64;
            const int ks = DOWN ? 1 : (ng > 8 ? ng / 8 : 1);
            if (ks <= kMaxMfmaKsplit) {
                p.n_mfma = token_tiles(a->T) * (M.rows / 128) * ks;
                p.mfma_ks = ks;
                lds = lds_m;
            }
        }
        const hipError_t e = stream_block_slots((const void *)fn, lds, p.nb);
        if (e != hipSuccess) return e;
        p.nb = (p.nb + kClaimGroups - 1) / kClaimGroups * kClaimGroups;
        plan = p;
        if (launch) hipLaunchKernelGGL(fn, dim3((unsigned)p.nb), dim3(256), lds, st, *a, p);
        return hipSuccess;
    }
};

// the butterfly reduction needs lanes per row >= partial sums per lane
template <int BITS, int CPL, bool DOWN>
hipError_t dispatch_lpr(StreamOp &op) {
    constexpr int nv = (DOWN ? 1 : 2) * stream_rpw(CPL);
    switch (op.a->L.m[DOWN ? 2 : 0].lpr) {
        case 64: return op.template run<BITS, CPL, DOWN, 64>();
        case 32: return op.template run<BITS, CPL, DOWN, (nv <= 32 ? 32 : 0)>();
        case 16: return op.template run<BITS, CPL, DOWN, (nv <= 16 ? 16 : 0)>();
        default: return op.template run<BITS, CPL, DOWN, 0>();
    }
}

template <int BITS, bool DOWN>
hipError_t dispatch_stream(StreamOp &op) {
    const int cpl = op.a->L.m[DOWN ? 2 : 0].cpl;
    if (cpl == 1) return dispatch_lpr<BITS, 1, DOWN>(op);
    if constexpr (BITS == 4) {
        if (cpl == 2) return dispatch_lpr<4, 2, DOWN>(op);  // 2-bit rows of 4096 or fewer codes take one chunk per lane
    }
    return hipErrorInvalidValue;
}

template <int BITS>
hipError_t stream_op(const FwdArgs &a, bool down, bool launch, hipStream_t st, StreamPlan &plan) {
    StreamOp op{&a, st, launch, StreamPlan{}};
    const hipError_t e = down ? dispatch_stream<BITS, true>(op) : dispatch_stream<BITS, false>(op);
    plan = op.plan;
    return e;
}

template <int BITS>
hipError_t launch_grouped_bits(const FwdArgs &a, int stage, hipStream_t st) {
    const int H = a.s.H, F = a.s.F, E = a.s.E, K = a.s.K, T = a.T;
    switch (stage) {
        case 2: {
            StreamPlan p0, p1;
            hipError_t e = stream_op<BITS>(a, false, false, st, p0);
            if (e == hipSuccess) e = stream_op<BITS>(a, true, false, st, p1);
            if (e != hipSuccess) return e;
            if (E > 512)
                hipLaunchKernelGGL(k_route_tokens<4>, dim3((unsigned)T), dim3(256), 0, st, a);
            else
                hipLaunchKernelGGL(k_route_tokens<2>, dim3((unsigned)T), dim3(256), 0, st, a);
            hipLaunchKernelGGL(k_group, dim3(1), dim3(kGroupThreads), 0, st, a, p0, p1);
            break;
        }
        case 3:
        case 5: {
            StreamPlan p;
            const hipError_t e = stream_op<BITS>(a, stage == 5, true, st, p);
            if (e != hipSuccess) return e;
            break;
        }
        case 4: {
            StreamPlan p0;
            const hipError_t e = stream_op<BITS>(a, false, false, st, p0);
            if (e != hipSuccess) return e;
            const int sks = (p0.n_mfma > 0 && p0.mfma_ks > 1) ? p0.mfma_ks : 0;
            const int n_pairs = T * (K + 1);
            const int ppb = 256 / (F / 16);
            const int pair_blocks = (n_pairs + ppb - 1) / ppb;
            const int shared_blocks = sks > 0 ? (T * (F / 4) + 255) / 256 : 0;
            hipLaunchKernelGGL(k_encode_act<BITS>, dim3((unsigned)(pair_blocks + shared_blocks)), dim3(256), 0, st, a,
                               n_pairs, sks, pair_blocks);
            break;
        }
        case 6:
            hipLaunchKernelGGL(k_combine, dim3((unsigned)((H / 4 + 63) / 64), (unsigned)T), dim3(64), 0, st, a);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

// stages 0 and 1: batched RMSNorm and router GEMM
hipError_t launch_grouped_stage(const FwdArgs &a, int stage, hipStream_t stream) {
    (void)hipGetLastError();
    if (stage < 2) return launch_batch_router(a, stage, stream);
    if (a.s.bits == 4) return launch_grouped_bits<4>(a, stage, stream);
    if (a.s.bits == 2) return launch_grouped_bits<2>(a, stage, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_grouped(const FwdArgs &a, hipStream_t stream) {
    for (int stage = 0; stage < kGroupedStages; ++stage) {
        const hipError_t e = launch_grouped_stage(a, stage, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace moe

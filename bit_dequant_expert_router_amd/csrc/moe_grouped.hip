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
//   k_route_tokens  one wave per token: softmax/top-K/renormalise
//   k_group         one block: histogram of assignments per expert, exclusive
//                   scan, stable scatter (token order kept inside each expert)
//                   and the compact list of touched experts
//   k_grouped_gateup  one block per (touched expert, row chunk): gate+up rows read
//                   once, applied to every token of the expert, SwiGLU; the shared
//                   expert gets its own blocks over all tokens
//   k_grouped_down  same for the down projection, writing one output vector per
//                   (token, slot)
//   k_combine       out = x + sum_k w_k y_k + sigmoid(g_s) y_shared, in slot order
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

// exclusive prefix sum over the 64 lanes of a wave (small, one-time use)
__device__ __forceinline__ int wave_excl_scan(int v) {
    const int lane = threadIdx.x & 63;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
    }
    return incl - v;
}

// ---------------------------------------------------------------------------
// routing of every token and grouping of assignments by expert
// ---------------------------------------------------------------------------
// logits of token t: the KS partial sums of the router GEMM, every load issued
// at once, added in a fixed order
template <int EPL>
__device__ __forceinline__ void token_logits(const FwdArgs &a, int t, float (&zv)[EPL], float &gs) {
    const int E = a.s.E, T = a.T, ksn = router_ksplit(a.s.H);
    const int lane = threadIdx.x & 63;
    const float *zt = a.ws.zp + (size_t)t * (E + 1);
    const size_t kstride = (size_t)T * (E + 1);
    float z[kMaxKsplit][EPL], g[kMaxKsplit];
#pragma unroll
    for (int ks = 0; ks < kMaxKsplit; ++ks) {
        const float *zk = zt + (size_t)(ks < ksn ? ks : 0) * kstride;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
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

// grouping of all T*K assignments by expert, by one block of 256 threads:
// histogram, exclusive scans, the compact list of touched experts, and a
// stable scatter (token order kept inside each expert)
constexpr int kGroupThreads = 1024;

__device__ void group_assignments(const FwdArgs &a) {
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

    for (int i = threadIdx.x; i < E; i += NT) s_cnt[i] = 0;
    for (int i = threadIdx.x; i < TK; i += NT) s_sel[i] = a.ws.sel[i];
    __syncthreads();
    for (int i = threadIdx.x; i < TK; i += NT) atomicAdd(&s_cnt[s_sel[i]], 1);
    __syncthreads();
    // exclusive scans of the counts and of the touched flags (E <= 1024: 16 per lane)
    if (wave == 0) {
        constexpr int kPer = kMaxExperts / 64;
        int c[kPer];
        int sc = 0, sf = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = lane * kPer + i;
            c[i] = (e < E) ? s_cnt[e] : 0;
            sc += c[i];
            sf += c[i] > 0 ? 1 : 0;
        }
        int pc = wave_excl_scan(sc), pf = wave_excl_scan(sf);
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = lane * kPer + i;
            if (e < E) {
                s_off[e] = pc;
                s_tch[e] = pf;
            }
            pc += c[i];
            pf += c[i] > 0 ? 1 : 0;
        }
        if (lane == 63) a.ws.grp[0] = pf;  // number of touched experts
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
        }
        __syncthreads();
        for (int e = threadIdx.x; e < E; e += NT) s_off[e] += __popc(s_mask[e]);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// k_route_tokens: one wave per token sums the partial logits and routes
// (softmax -> top-K -> renormalise).  k_group then groups the assignments of
// the whole batch in one block.  (A last-block-done counter inside one kernel
// would need an L2 write-back per block and same-address atomics across the
// XCDs, both slower here than the kernel boundary.)
// ---------------------------------------------------------------------------
template <int EPL>
__global__ __launch_bounds__(64) void k_route_tokens(FwdArgs a) {
    const int t = blockIdx.x, K = a.s.K, E = a.s.E;
    const int lane = threadIdx.x & 63;
    float zv[EPL], gs;
    token_logits<EPL>(a, t, zv, gs);
    int my_sel;
    float my_w;
    route_wave<EPL>(zv, E, K, my_sel, my_w);
    if (lane < K) {
        a.ws.sel[t * K + lane] = my_sel;
        a.ws.coef[t * (K + 1) + lane] = my_w;
        if (a.route_idx) a.route_idx[t * K + lane] = my_sel;
        if (a.route_w) a.route_w[t * K + lane] = my_w;
    } else if (lane == K) {
        a.ws.coef[t * (K + 1) + K] = sigmoidf_(gs);
    }
}

__global__ __launch_bounds__(kGroupThreads) void k_group(FwdArgs a) { group_assignments(a); }

// unit of work of the grouped kernels: a touched expert (or the shared expert
// and a chunk of the batch's tokens) and a chunk of rows
struct Unit {
    bool live;
    bool shared;
    int expert;
    int first;   // first assignment in perm (routed) or first token (shared)
    int count;   // assignments (routed) or tokens (shared)
};

// units 0 .. n_shared-1: the shared expert over token chunks (the heaviest units
// are dispatched first); then one unit per touched routed expert
__device__ __forceinline__ Unit decode_unit(const FwdArgs &a, const GroupView &gv, int ui, int shared_tok_chunk) {
    Unit u;
    u.live = false;
    u.shared = false;
    const int n_shared = (a.T + shared_tok_chunk - 1) / shared_tok_chunk;
    if (ui < n_shared) {
        u.shared = true;
        u.expert = a.s.E;
        u.first = ui * shared_tok_chunk;
        u.count = (a.T - u.first) < shared_tok_chunk ? (a.T - u.first) : shared_tok_chunk;
        u.live = u.count > 0;
    } else {
        // r < G always: the four loads go out together
        const int r = ui - n_shared;
        const int nt = *gv.n_touched;
        u.expert = gv.expert[r];
        u.first = gv.first[r];
        u.count = gv.count[r];
        u.live = r < nt;
    }
    return u;
}

// (token, slot) of the i-th assignment of a unit
__device__ __forceinline__ void unit_item(const FwdArgs &a, const GroupView &gv, const Unit &u, int i, int &t,
                                          int &slot) {
    const int K = a.s.K;
    if (u.shared) {
        t = u.first + i;
        slot = K;
    } else {
        const int asg = gv.perm[u.first + i];
        t = asg / K;
        slot = asg % K;
    }
}

// lane slice [k0, k0 + NV) of one vector in limb form: limbs [7][n/8] dwords,
// group scales [n/64], half-group sums [n/32]
template <int BITS, int CPL>
__device__ __forceinline__ void load_limb_slice(const uint32_t *hl, const float *hs, const float *hx, int n, int k0,
                                                LimbSlice<BITS, CPL> &hv) {
    using Q = QSlice<BITS, CPL>;
    hl += k0 / 8;
#pragma unroll
    for (int x = 0; x < kLimbs; ++x)
#pragma unroll
        for (int i = 0; i < Q::NL / 4; ++i) {
            const int4 v = *(const int4 *)(hl + (size_t)x * (n / 8) + 4 * i);
            hv.L[x][4 * i + 0] = v.x; hv.L[x][4 * i + 1] = v.y;
            hv.L[x][4 * i + 2] = v.z; hv.L[x][4 * i + 3] = v.w;
        }
#pragma unroll
    for (int g = 0; g < Q::NGL; ++g) {
        hv.S[g] = hs[k0 / 64 + g];
        float xs = 0.0f;
#pragma unroll
        for (int hh = 0; hh < Q::GL / 32; ++hh) xs += hx[(k0 + g * 64) / 32 + hh];
        hv.X[g] = xs;
    }
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
template <int BITS>
__global__ __launch_bounds__(256) void k_encode_act(FwdArgs a, int n_pairs) {
    const int F = a.s.F;
    const int tpp = F / 16;  // threads per pair (a multiple of 8)
    const int p = blockIdx.x * (256 / tpp) + threadIdx.x / tpp;
    const int u = threadIdx.x % tpp;
    const bool live = p < n_pairs;
    float v[16];
    const float *src = a.ws.act + (size_t)(live ? p : 0) * F + 16 * u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 q = *(const float4 *)(src + 4 * i);
        v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
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
    }
}

// ---------------------------------------------------------------------------
// k_grouped_stream: the dequant GEMV of one expert matrix pair (gate + up, with
// SwiGLU) or of the down matrix, for the tokens of one unit and a range of rows.
//
// A block takes one unit (a touched expert, or the shared expert and a chunk of
// tokens) and a range of row-steps.  It stages the limb form of up to TP
// vectors of the unit (tokens h for gate/up, (token, slot) activations for
// down) in LDS once, then every wave streams its row-steps: the weights of
// step s+1 are loaded into one register set while step s is computed from the
// other, so HBM requests stay in flight through the compute.  Each step's
// rows are applied to every staged vector (weights read from HBM once per
// pass; a unit with more than TP vectors takes several passes).
// ---------------------------------------------------------------------------
// words of one staged vector of length n: limbs [7][n/8], scales [n/64], half
// sums [n/32], rounded up to 16 bytes
MOE_HD int stage_words(int n) { return (kLimbs * (n / 8) + n / 64 + n / 32 + 3) & ~3; }

template <int BITS, int CPL, int NM, int RPW>
struct StepWeights {
    using Q = QSlice<BITS, CPL>;
    uint4 c[NM][RPW][CPL];
    uint32_t sb[NM][RPW][Q::NGL];
};

// LPR: lanes per row when the partial sums of a step are reduced together
// (16, 32 or 64); 0: any other width, one reduction per row
template <int BITS, int CPL, int RPW, bool DOWN, int LPR>
__global__ __launch_bounds__(256) void k_grouped_stream(FwdArgs a, int chunks, int shared_tok_chunk, int tp) {
    using Q = QSlice<BITS, CPL>;
    constexpr int NM = DOWN ? 1 : 2;
    constexpr int NV = NM * RPW;  // partial sums per lane per step and vector
    extern __shared__ uint4 s_dyn[];
    uint32_t *s_vec = (uint32_t *)s_dyn;
    __shared__ int s_out[16];  // output vector index (t * (K+1) + slot) per staged vector
    const int H = a.s.H, F = a.s.F, K = a.s.K;
    const int n = DOWN ? F : H;  // reduction length
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const GroupView gv = group_view(a);
    const Unit u = decode_unit(a, gv, blockIdx.x / chunks, shared_tok_chunk);
    if (!u.live) return;
    const QMat &M0 = a.L.m[DOWN ? 2 : 0];
    const QMat &M1 = a.L.m[1];
    const int lpr = LPR ? LPR : M0.lpr, rpi = 64 / lpr;
    const int lr = lane % lpr, rsub = lane / lpr;
    const int nrs = M0.rows / rpi;
    const int per_block = (nrs + chunks - 1) / chunks;
    const int rs_lo = (blockIdx.x % chunks) * per_block;
    const int rs_hi = min(nrs, rs_lo + per_block);
    const int nsteps = (rs_hi - rs_lo + 4 * RPW - 1) / (4 * RPW);
    const uint8_t *ex = u.shared ? a.shared : a.experts + (size_t)u.expert * a.L.bytes;
    const int words = stage_words(n);
    const int k0 = lr * Q::NV;
    const int out_len = DOWN ? H : F;
    float *out_base = DOWN ? a.ws.ys : a.ws.act;

    // unconditional loads (rows past the range re-read its last row, unused)
    // so that no wait separates them
    auto load_step = [&](int s, StepWeights<BITS, CPL, NM, RPW> &w) {
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int r0 = rs_lo + (s * 4 + wave) * RPW + i;
            const int rs = r0 < rs_hi ? r0 : rs_hi - 1;
            load_row<BITS, CPL>(ex, M0, rs * rpi + rsub, lr, w.c[0][i], w.sb[0][i]);
            if constexpr (NM == 2) load_row<BITS, CPL>(ex, M1, rs * rpi + rsub, lr, w.c[1][i], w.sb[1][i]);
        }
    };
    auto compute_step = [&](int s, StepWeights<BITS, CPL, NM, RPW> &w, int np) {
        const int rs0 = rs_lo + (s * 4 + wave) * RPW;
        // row-major list of the step's rows: entry NM * i + m
        uint4 (&c)[NV][CPL] = *reinterpret_cast<uint4 (*)[NV][CPL]>(&w.c[0][0][0]);
        float sc[NV][Q::NGL], of[NV][Q::NGL];
#pragma unroll
        for (int i = 0; i < RPW; ++i)
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                prep_codes<BITS, CPL>(w.c[m][i]);
#pragma unroll
                for (int g = 0; g < Q::NGL; ++g) {
                    sc[NM * i + m][g] = bf16_lo(w.sb[m][i][g]);
                    of[NM * i + m][g] = fmaf(Q::kCodeOffset, sc[NM * i + m][g], bf16_hi(w.sb[m][i][g]));
                }
            }
        uint4 cl[NV][CPL];
#pragma unroll
        for (int i = 0; i < RPW; ++i)
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int j = 0; j < CPL; ++j) cl[NM * i + m][j] = w.c[m][i][j];
        (void)c;
        for (int v = 0; v < np; ++v) {
            const uint32_t *vec = s_vec + (size_t)v * words;
            float *out = out_base + (size_t)s_out[v] * out_len;
            float part[NV];
            rows_dot_lds<BITS, CPL, NV>(cl, sc, of, vec, (const float *)(vec + kLimbs * (n / 8)),
                                        (const float *)(vec + kLimbs * (n / 8) + n / 64), n, k0, part);
            if constexpr (LPR != 0) {
                // every row of the step at once; rows past the block's range
                // are computed on stale registers and not written
                const float r = multi_reduce<NV, LPR>(part);
                constexpr int DL = LPR / NV;  // lanes sharing one reduced entry
                const int j = multi_index<NV, LPR>(lane);
                const int rs = rs0 + j / NM;
                if constexpr (DOWN) {
                    if ((lane & (DL - 1)) == 0 && rs < rs_hi) out[rs * rpi + rsub] = r;
                } else {
                    const float up = xchg<DL>(r);  // the up sum sits across the last halving bit
                    const float act = r * up * __builtin_amdgcn_rcpf(1.0f + __expf(-r));
                    if ((lane & (2 * DL - 1)) == 0 && rs < rs_hi) out[rs * rpi + rsub] = act;
                }
            } else {
#pragma unroll
                for (int i = 0; i < RPW; ++i) {
                    const int rs = rs0 + i;
                    if (rs < rs_hi) {
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

    for (int p0 = 0; p0 < u.count; p0 += tp) {
        const int np = min(tp, u.count - p0);
        StepWeights<BITS, CPL, NM, RPW> wa, wb;
        load_step(0, wa);  // in flight while the vectors are staged
        if (p0 > 0) __syncthreads();  // the previous pass is done with LDS
        // stage the np vectors: limbs as 16-byte pieces, then scales and half sums
        for (int v = 0; v < np; ++v) {
            int t, slot;
            unit_item(a, gv, u, p0 + v, t, slot);
            const int pv = t * (K + 1) + slot;
            if (threadIdx.x == 0) s_out[v] = pv;
            const uint32_t *hl = DOWN ? (const uint32_t *)a.ws.al + (size_t)pv * kLimbs * (F / 8)
                                      : (const uint32_t *)a.ws.hl + (size_t)t * kLimbs * (H / 8);
            const float *hs = DOWN ? a.ws.as + (size_t)pv * (F / 64) : a.ws.hs + (size_t)t * (H / 64);
            const float *hx = DOWN ? a.ws.ax + (size_t)pv * (F / 32) : a.ws.hx + (size_t)t * (H / 32);
            uint32_t *dst = s_vec + (size_t)v * words;
            for (int i = threadIdx.x; i < kLimbs * n / 32; i += 256) ((uint4 *)dst)[i] = ((const uint4 *)hl)[i];
            for (int i = threadIdx.x; i < n / 64; i += 256) dst[kLimbs * (n / 8) + i] = __float_as_uint(hs[i]);
            for (int i = threadIdx.x; i < n / 32; i += 256) dst[kLimbs * (n / 8) + n / 64 + i] = __float_as_uint(hx[i]);
        }
        __syncthreads();
        // the prefetches are unconditional (past the last step they re-read
        // it, from cache): a load issued on one path only would make the
        // waits after the join count for the path without it, i.e. wait for
        // the prefetch itself
        for (int s = 0; s < nsteps; s += 2) {
            load_step(s + 1 < nsteps ? s + 1 : nsteps - 1, wb);
            compute_step(s, wa, np);
            load_step(s + 2 < nsteps ? s + 2 : nsteps - 1, wa);
            if (s + 1 < nsteps) compute_step(s + 1, wb, np);
        }
    }
}

// ---------------------------------------------------------------------------
// k_combine: out = x + sum_k w_k y_k + sigmoid(g_s) y_shared (slot order)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_combine(FwdArgs a) {
    const int H = a.s.H, K = a.s.K;
    const int t = blockIdx.y;
    const int o = blockIdx.x * 256 + threadIdx.x;
    if (o >= H) return;
    const float *c = a.ws.coef + (size_t)t * (K + 1);
    const float *ys = a.ws.ys + (size_t)t * (K + 1) * H + o;
    float acc = a.x[(size_t)t * H + o];
    for (int k = 0; k <= K; ++k) acc = fmaf(c[k], ys[(size_t)k * H], acc);
    a.y[(size_t)t * H + o] = acc;
}

// row-slots per wave and step of k_grouped_stream: two register sets of
// weights stay within ~80 VGPRs
constexpr int stream_rpw(int cpl) { return cpl == 1 ? 4 : 2; }
constexpr int kStreamStepsPerWave = 8;  // row-steps a wave streams per block
constexpr int kStreamMaxVectors = 16;

// vectors staged per pass: as many as fit the block's LDS budget (48 KiB for
// gate/up: three blocks per CU; 40 KiB for down, whose registers allow four),
// at most 16
inline int stream_vectors(int n, bool down) {
    const int budget = (down ? 40 : 48) * 1024;
    const int v = budget / (stage_words(n) * 4);
    return v < kStreamMaxVectors ? v : kStreamMaxVectors;
}

template <int BITS, int CPL, bool DOWN, int LPR>
void launch_stream(const FwdArgs &a, hipStream_t st) {
    const QMat &M = a.L.m[DOWN ? 2 : 0];
    const int rpi = 64 / M.lpr;
    const int nrs = M.rows / rpi;
    constexpr int rpw = stream_rpw(CPL);
    const int chunks = (nrs + 4 * rpw * kStreamStepsPerWave - 1) / (4 * rpw * kStreamStepsPerWave);
    const int n = DOWN ? a.s.F : a.s.H;
    const int tp = stream_vectors(n, DOWN);
    // shared-expert units of tp tokens: one pass each
    const int units = touched_bound(a.s, a.T) + (a.T + tp - 1) / tp;
    const size_t lds = (size_t)tp * stage_words(n) * 4;
    hipLaunchKernelGGL((k_grouped_stream<BITS, CPL, rpw, DOWN, LPR>), dim3((unsigned)(units * chunks)), dim3(256), lds, st,
                       a, chunks, tp, tp);
}

// the butterfly reduction needs lanes per row >= partial sums per lane
template <int BITS, int CPL, bool DOWN>
void launch_grouped_mats(const FwdArgs &a, hipStream_t st) {
    constexpr int nv = (DOWN ? 1 : 2) * stream_rpw(CPL);
    switch (a.L.m[DOWN ? 2 : 0].lpr) {
        case 64: launch_stream<BITS, CPL, DOWN, 64>(a, st); break;
        case 32: launch_stream<BITS, CPL, DOWN, (nv <= 32 ? 32 : 0)>(a, st); break;
        case 16: launch_stream<BITS, CPL, DOWN, (nv <= 16 ? 16 : 0)>(a, st); break;
        default: launch_stream<BITS, CPL, DOWN, 0>(a, st); break;
    }
}

template <int BITS>
hipError_t launch_grouped_bits(const FwdArgs &a, int stage, hipStream_t st) {
    const int H = a.s.H, F = a.s.F, E = a.s.E, K = a.s.K, T = a.T;
    switch (stage) {
        case 2:
            if (E > 512)
                hipLaunchKernelGGL(k_route_tokens<16>, dim3((unsigned)T), dim3(64), 0, st, a);
            else
                hipLaunchKernelGGL(k_route_tokens<8>, dim3((unsigned)T), dim3(64), 0, st, a);
            hipLaunchKernelGGL(k_group, dim3(1), dim3(kGroupThreads), 0, st, a);
            break;
        case 3:
        case 5: {
            const bool down = stage == 5;
            const int cpl = a.L.m[down ? 2 : 0].cpl;
            if (cpl == 1) {
                if (down) launch_grouped_mats<BITS, 1, true>(a, st);
                else launch_grouped_mats<BITS, 1, false>(a, st);
            } else if (BITS == 4 && cpl == 2) {  // 2-bit rows of 4096 or fewer codes take one chunk per lane
                if (down) launch_grouped_mats<4, 2, true>(a, st);
                else launch_grouped_mats<4, 2, false>(a, st);
            } else {
                return hipErrorInvalidValue;
            }
            break;
        }
        case 4: {
            const int n_pairs = T * (K + 1);
            const int ppb = 256 / (F / 16);
            hipLaunchKernelGGL(k_encode_act<BITS>, dim3((unsigned)((n_pairs + ppb - 1) / ppb)), dim3(256), 0, st, a,
                               n_pairs);
            break;
        }
        case 6:
            hipLaunchKernelGGL(k_combine, dim3((unsigned)((H + 255) / 256), (unsigned)T), dim3(256), 0, st, a);
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

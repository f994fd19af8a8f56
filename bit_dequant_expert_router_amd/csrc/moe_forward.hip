// moe_forward.hip -- the expert layer as three stream-ordered kernels.
//
//   k_router : two-pass RMSNorm + router GEMV (E rows) + shared-gate logit;
//              a few blocks also store h in the fixed-point limb form below
//              (k_router_split for H = 2048 / 4096, one token per block;
//              k_router_tokens from 4 tokens, four per block; k_router else)
//   k_gateup : per wave, the routing rounds its slot needs (block 0 also
//              the whole softmax/top-K/renormalise), then the fused gate+up
//              dequant GEMV of its rows of the selected or the shared expert
//              with SwiGLU in registers
//   k_down   : down-projection dequant GEMV of all K+1 experts for a set of
//              output rows, weighted combine, sigmoid-gated shared expert and
//              residual, written once per row (no atomics, deterministic)
//
// A batch runs one row of blocks per token (grid.y); batches from 100
// assignments (tokens x top-K) take the grouped kernels instead.
//
// Tiered residency (experts read from cache slots) runs k_router, then
// k_route (the routing alone, its selection also written to host memory),
// then, once the host has chosen the slots, k_fetch (the missing experts
// from host memory into their slots) and the TIER variants of k_gateup (no
// routing) and k_down, which address the selected experts by slot.
//
// Sources of each step: RMSNorm in two passes, the FMA form of the 4-bit
// dequant mat-vec, fused SwiGLU, fused combine + residual + sigmoid gate:
// "48GB内存运行397B模型：Flash-Moe的极端量化与SSD流式加载实践", section
// "Metal GPU管线：手写Kernel与FMA优化"; routing GEMV then softmax + top-K:
// flash-moe README translation, "Pipeline mỗi lớp".
//
#include "moe_device.h"

namespace moe {

namespace {

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
    const float inv = __builtin_amdgcn_rsqf(ss * pow2f(-__builtin_ctz((unsigned)H)) + a.s.eps);

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
            a.ws.z[(size_t)t * logit_stride(E) + r] = acc;
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
// k_router_split (H = 2048 or 4096): the router rows, shared gate, x, gamma,
// H and E come as leading scalar parameters, which the hardware preloads into
// SGPRs (the library is built with kernel-argument preloading), so the first
// loads wait for no read of the argument segment: 0.25 us less per layer.
// k_gateup and k_down take the pointers of their own first loads the same way.
// k_gateup also takes the shared expert's pointer and F, and derives the gate
// and up matrices' layout from H and F with a few shifts, so that the shared
// expert's weight loads wait for no argument read either (2-bit layer 13.35 ->
// 12.78 us, 4-bit 15.05 -> 14.86 us); the rest of the layout and the other
// pointers, needed once those loads are out, stay in FwdArgs (deriving all of
// them on the device costs more scalar instructions per wave than the
// argument read).  The 4 waves of a block split H into
// quarters of the block's RB router rows (one row per block measures fastest:
// 513 blocks spread the 4 MiB over the whole chip), so a wave reads 1/4 of x
// and gamma instead of all of it.  The dot products use x * gamma; the factor
// 1 / rms(x) is applied to the block's sum (the norm's two passes are the
// waves' sums of squares, then the scaling).  The first H / 256 blocks also
// write the limb form of h for k_gateup.
// ---------------------------------------------------------------------------
constexpr int kRouterSplitRows = 1;

template <int CPL_R>
__global__ __launch_bounds__(256) void k_router_split(const uint16_t *__restrict__ p_router,
                                                      const uint16_t *__restrict__ p_sgate,
                                                      const float *__restrict__ p_x,
                                                      const uint16_t *__restrict__ p_gamma, int H, int E, FwdArgs a) {
    constexpr int RB = kRouterSplitRows;
    const int t = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float *x = p_x + (size_t)t * H;
    const int r0 = blockIdx.x * RB;
    // lane's chunks of 8 entries: wave quarter + lane + 64 j
    const int kq = wave * (H / 4);
    uint4 wv[RB][CPL_R];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const int row = r0 + r <= E ? r0 + r : E;  // rows past the end re-read the gate row, unused
        const uint16_t *src = (row < E) ? p_router + (size_t)row * H : p_sgate;
#pragma unroll
        for (int j = 0; j < CPL_R; ++j) wv[r][j] = ld_stream16(src + kq + 8 * (lane + 64 * j));
    }
    float xv[CPL_R * 8];
    uint4 gv[CPL_R];
#pragma unroll
    for (int j = 0; j < CPL_R; ++j) {
        const int k0 = kq + 8 * (lane + 64 * j);
        const float4 x0 = *(const float4 *)(x + k0);
        const float4 x1 = *(const float4 *)(x + k0 + 4);
        xv[8 * j + 0] = x0.x; xv[8 * j + 1] = x0.y; xv[8 * j + 2] = x0.z; xv[8 * j + 3] = x0.w;
        xv[8 * j + 4] = x1.x; xv[8 * j + 5] = x1.y; xv[8 * j + 6] = x1.z; xv[8 * j + 7] = x1.w;
        gv[j] = *(const uint4 *)(p_gamma + k0);
    }
    // this block's share of the limb encoding: entry k of h (x and gamma fetched now)
    const int ke = blockIdx.x * 256 + threadIdx.x;
    const bool enc = blockIdx.x * 256 < H;
    const float xe = x[ke < H ? ke : 0];
    const float ge = __uint_as_float((uint32_t)p_gamma[ke < H ? ke : 0] << 16);

    float ss = 0.0f;
    float xg[CPL_R * 8];
#pragma unroll
    for (int j = 0; j < CPL_R; ++j) {
        const uint32_t g[4] = {gv[j].x, gv[j].y, gv[j].z, gv[j].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            xg[8 * j + 2 * q] = xv[8 * j + 2 * q] * bf16_lo(g[q]);
            xg[8 * j + 2 * q + 1] = xv[8 * j + 2 * q + 1] * bf16_hi(g[q]);
        }
    }
#pragma unroll
    for (int i = 0; i < CPL_R * 8; ++i) ss = fmaf(xv[i], xv[i], ss);
    float acc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        float v = 0.0f;
#pragma unroll
        for (int j = 0; j < CPL_R; ++j) {
            const uint32_t w[4] = {wv[r][j].x, wv[r][j].y, wv[r][j].z, wv[r][j].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v = fmaf(bf16_lo(w[q]), xg[8 * j + 2 * q], v);
                v = fmaf(bf16_hi(w[q]), xg[8 * j + 2 * q + 1], v);
            }
        }
        acc[r] = v;
    }
    const float red = multi_reduce<RB, 64>(acc);
    const int jr = multi_index<RB, 64>(lane);
    ss = lane_sum<64>(ss);
    __shared__ float s_part[4][RB];
    __shared__ float s_ss[4];
    if ((lane & (64 / RB - 1)) == 0) s_part[wave][jr] = red;
    if (lane == 0) s_ss[wave] = ss;
    __syncthreads();
    // 1 / rms by the hardware reciprocal square root (router stage 3.29 -> 3.24 us);
    // the mean by an exact power-of-two scale (H is a power of two)
    const float inv = __builtin_amdgcn_rsqf(((s_ss[0] + s_ss[1]) + (s_ss[2] + s_ss[3])) * pow2f(-__builtin_ctz((unsigned)H)) + a.s.eps);
    if (threadIdx.x < RB) {
        const int row = r0 + threadIdx.x;
        const float z = (((s_part[0][threadIdx.x] + s_part[1][threadIdx.x]) + s_part[2][threadIdx.x]) +
                         s_part[3][threadIdx.x]) * inv;
        if (row < E)
            a.ws.z[(size_t)t * logit_stride(E) + row] = z;
        else if (row == E)
            a.ws.gs[t] = z;
    }
    if (enc) {  // one wave = one group of 64
        const float h = (ke < H) ? xe * inv * ge : 0.0f;
        const float m = lane_max<64>(fabsf(h));
        int l[kLimbs];
        limb_split(limb_value(h, m), l);
        const float half = lane_sum<32>(h);
        uint32_t packed[kLimbs];
#pragma unroll
        for (int xl = 0; xl < kLimbs; ++xl) packed[xl] = lane_or8((uint32_t)(l[xl] & 15) << (4 * (lane & 7)));
        if (ke < H) {
            uint32_t *hl = (uint32_t *)a.ws.hl + (size_t)t * kLimbs * (H / 8);
            if ((lane & 7) == 0) {
#pragma unroll
                for (int xl = 0; xl < kLimbs; ++xl) hl[(size_t)xl * (H / 8) + ke / 8] = packed[xl];
            }
            if (lane == 0) a.ws.hs[(size_t)t * (H / 64) + ke / 64] = limb_scale(m);
            if ((lane & 31) == 0) a.ws.hx[(size_t)t * (H / 32) + ke / 32] = half;
        }
    }
}

// ---------------------------------------------------------------------------
// k_router_tokens (H = 2048 or 4096, batches of 4 tokens or more): as
// k_router_split, with TB tokens per block, so that a batch reads each router
// row once per TB tokens (8 tokens: 8.8 against 11.3 us).  The block's tokens
// are reduced together: entry tt of the list is token tt's dot product, entry
// TB + tt its sum of squares.
// ---------------------------------------------------------------------------
template <int CPL_R, int TB>
__global__ __launch_bounds__(256) void k_router_tokens(FwdArgs a) {
    const int t0 = blockIdx.y * TB;
    const int H = a.s.H, E = a.s.E, T = a.T;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r0 = blockIdx.x;  // the block's router row (E: the shared gate; past E: encoding only)
    // lane's chunks of 8 entries: wave quarter + lane + 64 j
    const int kq = wave * (H / 4);
    uint4 wv[CPL_R];
    {
        const int row = r0 <= E ? r0 : E;  // rows past the end re-read the gate row, unused
        // both bases and the batch size fetched at once, before the choice
        // (else their kernel-argument loads move behind a branch and a second
        // wait, and every weight load waits for them)
        const uint16_t *router = a.router, *sgate = a.sgate;
        asm volatile("" ::"s"(router), "s"(sgate), "s"(T));
        const uint16_t *src = (row < E) ? router + (size_t)row * H : sgate;
#pragma unroll
        for (int j = 0; j < CPL_R; ++j) wv[j] = ld_stream16(src + kq + 8 * (lane + 64 * j));
    }
    // the block's tokens (past the batch: the last token again, unused)
    const float *xt[TB];
#pragma unroll
    for (int tt = 0; tt < TB; ++tt) xt[tt] = a.x + (size_t)(t0 + tt < T ? t0 + tt : T - 1) * H;
    float xv[TB][CPL_R * 8];
    uint4 gv[CPL_R];
#pragma unroll
    for (int j = 0; j < CPL_R; ++j) {
        const int k0 = kq + 8 * (lane + 64 * j);
#pragma unroll
        for (int tt = 0; tt < TB; ++tt) {
            const float4 x0 = *(const float4 *)(xt[tt] + k0);
            const float4 x1 = *(const float4 *)(xt[tt] + k0 + 4);
            xv[tt][8 * j + 0] = x0.x; xv[tt][8 * j + 1] = x0.y; xv[tt][8 * j + 2] = x0.z; xv[tt][8 * j + 3] = x0.w;
            xv[tt][8 * j + 4] = x1.x; xv[tt][8 * j + 5] = x1.y; xv[tt][8 * j + 6] = x1.z; xv[tt][8 * j + 7] = x1.w;
        }
        gv[j] = *(const uint4 *)(a.gamma + k0);
    }
    // this block's share of the limb encoding: entry k of h (x and gamma fetched now)
    const int ke = blockIdx.x * 256 + threadIdx.x;
    const bool enc = blockIdx.x * 256 < H;
    float xe[TB];
#pragma unroll
    for (int tt = 0; tt < TB; ++tt) xe[tt] = xt[tt][ke < H ? ke : 0];
    const float ge = __uint_as_float((uint32_t)a.gamma[ke < H ? ke : 0] << 16);

    // per token: the router dot product (entry tt) and the sum of squares
    // (entry TB + tt), reduced over the wave together
    float v[2 * TB];
#pragma unroll
    for (int tt = 0; tt < TB; ++tt) {
        float dot = 0.0f, ss = 0.0f;
#pragma unroll
        for (int j = 0; j < CPL_R; ++j) {
            const uint32_t w[4] = {wv[j].x, wv[j].y, wv[j].z, wv[j].w};
            const uint32_t g[4] = {gv[j].x, gv[j].y, gv[j].z, gv[j].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float x0 = xv[tt][8 * j + 2 * q], x1 = xv[tt][8 * j + 2 * q + 1];
                dot = fmaf(bf16_lo(w[q]), x0 * bf16_lo(g[q]), dot);
                dot = fmaf(bf16_hi(w[q]), x1 * bf16_hi(g[q]), dot);
            }
        }
#pragma unroll
        for (int i = 0; i < CPL_R * 8; ++i) ss = fmaf(xv[tt][i], xv[tt][i], ss);
        v[tt] = dot;
        v[TB + tt] = ss;
    }
    static_assert(TB >= 2 && TB <= 32, "tokens per block");
    const float red = multi_reduce<2 * TB, 64>(v);
    const int jr = multi_index<2 * TB, 64>(lane);
    constexpr int DL = 32 / TB;  // lanes sharing one reduced entry
    __shared__ float s_part[4][2 * TB];
    if ((lane & (DL - 1)) == 0) s_part[wave][jr] = red;
    __syncthreads();
    auto inv_of = [&](int tt) {
        const float ss = (s_part[0][TB + tt] + s_part[1][TB + tt]) + (s_part[2][TB + tt] + s_part[3][TB + tt]);
        return __builtin_amdgcn_rsqf(ss * pow2f(-__builtin_ctz((unsigned)H)) + a.s.eps);
    };
    if (threadIdx.x < TB && t0 + (int)threadIdx.x < T) {
        const int tt = threadIdx.x, t = t0 + tt;
        const float z = (((s_part[0][tt] + s_part[1][tt]) + s_part[2][tt]) + s_part[3][tt]) * inv_of(tt);
        if (r0 < E)
            a.ws.z[(size_t)t * logit_stride(E) + r0] = z;
        else if (r0 == E)
            a.ws.gs[t] = z;
    }
    if (enc) {  // one wave = one group of 64
#pragma unroll
        for (int tt = 0; tt < TB; ++tt) {
            const int t = t0 + tt;
            if (t >= T) break;
            const float h = (ke < H) ? xe[tt] * inv_of(tt) * ge : 0.0f;
            const float m = lane_max<64>(fabsf(h));
            int l[kLimbs];
            limb_split(limb_value(h, m), l);
            const float half = lane_sum<32>(h);
            uint32_t packed[kLimbs];
#pragma unroll
            for (int xl = 0; xl < kLimbs; ++xl) packed[xl] = lane_or8((uint32_t)(l[xl] & 15) << (4 * (lane & 7)));
            if (ke < H) {
                uint32_t *hl = (uint32_t *)a.ws.hl + (size_t)t * kLimbs * (H / 8);
                if ((lane & 7) == 0) {
#pragma unroll
                    for (int xl = 0; xl < kLimbs; ++xl) hl[(size_t)xl * (H / 8) + ke / 8] = packed[xl];
                }
                if (lane == 0) a.ws.hs[(size_t)t * (H / 64) + ke / 64] = limb_scale(m);
                if ((lane & 31) == 0) a.ws.hx[(size_t)t * (H / 32) + ke / 32] = half;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// k_gateup: RPW row-steps per wave over the (K+1) x F gate/up row pairs.
// A wave's row-steps belong to one slot (F / rows-per-step is a multiple of
// RPW).  Every wave loads all E logits of the token (EPL per lane, two or four
// 16-byte loads); a routed slot s takes s + 1 routing rounds (route_slot) to
// find its expert; the shared expert needs none, and its blocks are
// dispatched first.  The limb form of h is staged in LDS once per block.
// BR false: every wave of a routed slot routes and issues its weight loads as
// soon as its expert is known; the block's one barrier comes after every wave
// has issued them, so it only orders the staging before the products.
// BR true (a block's waves share one slot): only wave 0 of a routed block
// routes and hands the expert to the other waves through LDS at the block's
// barrier, which then also orders the staging; the other waves' routing
// instructions are saved (the products are VALU-bound once the weights land).
// With BR every block holds one slot, so the shared expert's blocks find their
// rows from blockIdx and the preloaded F alone and issue their weight loads
// before the argument segment arrives.
// Block 0's wave 0 finally takes all K rounds and writes the selection, the
// renormalised weights and sigmoid(g_s).
// ---------------------------------------------------------------------------
// the gate (m = 0) or up (m = 1) matrix of make_layout(H, F, BITS), for H and
// F powers of two: shifts and adds only
template <int BITS>
__device__ __forceinline__ QMat gate_up_qmat(int H, int F, int m) {
    QMat q;
    q.rows = F;
    q.cols = H;
    q.bits = BITS;
    q.order = kOrderNibble;
    q.row_bytes = H * BITS / 8;
    q.ngroups = H / kGroup;
    q.nchunks = H / codes_per_chunk(BITS);
    q.lpr = q.nchunks < 64 ? q.nchunks : 64;
    q.cpl = q.nchunks >> __builtin_ctz((unsigned)q.lpr);
    const size_t mat = (size_t)F * q.row_bytes;  // one matrix's codes
    q.codes_off = (size_t)m * mat;
    q.sb_off = 3 * mat + (size_t)m * F * q.ngroups * 4;
    return q;
}

// LPR: lanes per row when the step's partial sums are reduced together (64);
// 0: one reduction per row
// TIER: the selected experts' routing is already done (k_route) and their
// weights sit in cache slots, sl.s[t * K + rank] (a.experts = the slots' base)
template <int BITS, int CPL, int RPW, int EPL, int LPR, bool TIER, bool BR>
__global__ __launch_bounds__(256) void k_gateup(const float *__restrict__ p_z, const float *__restrict__ p_gs,
                                                const uint32_t *__restrict__ p_hl, const float *__restrict__ p_hs,
                                                const float *__restrict__ p_hx, int H, uint32_t ef,
                                                const uint8_t *__restrict__ p_shared, FwdArgs a, SlotParam<TIER> sl) {
    using Q = QSlice<BITS, CPL>;
    const int t = blockIdx.y;
    const int E = (int)(ef & 0xFFFFu), F = (int)(ef >> 16);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

    // 1. loads that do not depend on the routing, from the preloaded
    //    parameters alone (issued before anything reads FwdArgs): the logits
    //    (resident path), the shared-gate logit and this thread's share of h's
    //    limb form
    float zv[EPL];
    if constexpr (!TIER) load_logits_lane<EPL>(p_z + (size_t)t * logit_stride(E), logit_stride(E), zv);
    const float gs = p_gs[t];
    // kStage 16-byte pieces per thread (a native vector type: an array of
    // int4 can keep dead copies in scratch memory)
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    constexpr int kStage = (kLimbs * kMaxDim / 32 + 255) / 256;
    const int n16 = kLimbs * H / 32;
    i32x4 st[kStage];
    {
        const i32x4 *src = (const i32x4 *)(p_hl + (size_t)t * kLimbs * (H / 8));
#pragma unroll
        for (int j = 0; j < kStage; ++j) {
            const int i = threadIdx.x + 256 * j;
            st[j] = src[i < n16 ? i : 0];
        }
    }
    const float hs = p_hs[(size_t)t * (H / 64) + (threadIdx.x < H / 64 ? threadIdx.x : 0)];
    const float hx = p_hx[(size_t)t * (H / 32) + (threadIdx.x < H / 32 ? threadIdx.x : 0)];

    const int K = a.s.K;
    // the gate and up matrices' layout from H and F (powers of two), not from
    // FwdArgs: the shared expert's loads then wait for no argument read
    const QMat G = gate_up_qmat<BITS>(H, F, 0);
    const QMat U = gate_up_qmat<BITS>(H, F, 1);
    const int lpr = G.lpr, lsh = __builtin_ctz((unsigned)lpr), rpi = 64 >> lsh;
    const int lr = lane & (lpr - 1), rsub = lane >> lsh;
    const int fsh = __builtin_ctz((unsigned)F) - (6 - lsh);  // log2(F / rpi): row-steps per slot
    // the blocks of the shared expert (the last slot) run first: their loads
    // need no routing and keep HBM busy while the routed waves route
    const int nbs = ((1 << fsh) + 4 * RPW - 1) / (4 * RPW);
    // BR (slots fill whole blocks, grid (K + 1) nbs): a block's slot and rows
    // from blockIdx alone
    constexpr bool kAligned = BR && !TIER;
    const int nrs = (K + 1) << fsh;
    const int lb = blockIdx.x < nbs ? blockIdx.x + (kAligned ? K * nbs : gridDim.x - nbs) : blockIdx.x - nbs;
    const int rs0 = (lb * 4 + wave) * RPW;
    const bool active = kAligned || rs0 < nrs;
    // slot of every row-step of the wave (waves past the end take the last one;
    // with BR the whole block's)
    const int slot = kAligned ? (blockIdx.x < nbs ? K : __builtin_amdgcn_readfirstlane((blockIdx.x - nbs) * 4 * RPW) >> fsh)
                              : __builtin_amdgcn_readfirstlane((active ? rs0 : nrs - 1) >> fsh);

    __shared__ __align__(16) uint32_t s_hl[kLimbs * kMaxDim / 8];  // limbs of h, [kLimbs][H/8]
    __shared__ float s_hs[kMaxDim / 64];
    __shared__ float s_hx[kMaxDim / 32];
    __shared__ int s_ex;  // BR: the block's expert

    // 2. the wave's expert (the shared expert's waves do not wait for the logits)
    const uint8_t *ex = p_shared;
    // BR, routed block: weight loads after the barrier (known without K)
    const bool late = kAligned && blockIdx.x >= nbs;
    if constexpr (TIER) {
        ex = (slot < K) ? a.experts + (size_t)sl.s[t * K + slot] * a.L.bytes : p_shared;
    } else if constexpr (BR) {
        if (late && __builtin_amdgcn_readfirstlane(wave) == 0) {
            // 2-bit codes: the routing wave takes issue priority over the
            // product waves sharing its SIMD until its weight loads are out
            // (2-bit layer 14.0 -> 13.6 us; the 4-bit layer measured slower)
            if constexpr (BITS == 2) __builtin_amdgcn_s_setprio(3);
            uint32_t key[EPL];
            logit_keys<EPL>(zv, E, key);
            const int e = route_slot<EPL>(key, E, slot);
            if (lane == 0) s_ex = e;
        }
    } else {
        if (slot < K) {
            uint32_t key[EPL];
            logit_keys<EPL>(zv, E, key);
            ex = a.experts + (size_t)route_slot<EPL>(key, E, slot) * a.L.bytes;
        }
    }

    // h's limbs into LDS (the staged loads were issued first, so this waits
    // for them only), then the block's barrier
    auto stage = [&]() {
        i32x4 *dst = (i32x4 *)s_hl;
#pragma unroll
        for (int j = 0; j < kStage; ++j) {
            const int i = threadIdx.x + 256 * j;
            if (i < n16) dst[i] = st[j];
        }
        if (threadIdx.x < H / 64) s_hs[threadIdx.x] = hs;
        if (threadIdx.x < H / 32) s_hx[threadIdx.x] = hx;
        __syncthreads();
    };
    if (late) {  // block-uniform
        stage();
        ex = a.experts + (size_t)__builtin_amdgcn_readfirstlane(s_ex) * a.L.bytes;
    }

    // 3. weight loads, all unconditional (row-steps past the end re-read the
    //    last one), addresses first, then every load back to back
    uint4 gc[RPW][CPL], uc[RPW][CPL];
    uint32_t gsb[RPW][Q::NGL], usb[RPW][Q::NGL];
    {
        int jr[RPW];
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            // row within the expert (aligned slots: from the block's position in its slot)
            const int rs = kAligned ? ((blockIdx.x < nbs ? blockIdx.x : blockIdx.x - nbs) * 4 + wave) * RPW + i
                                    : (rs0 + i < nrs ? rs0 + i : nrs - 1);
            jr[i] = ((rs * rpi) & (F - 1)) + rsub;
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            load_row<BITS, CPL>(ex, G, jr[i], lr, gc[i], gsb[i]);
            load_row<BITS, CPL>(ex, U, jr[i], lr, uc[i], usb[i]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // 4. the staging and barrier of the other blocks, behind their weight loads
    if (!late) stage();

    // 5. every row against the lane's limb slice of h in LDS, limb-major
    if constexpr (BITS == 2 && BR) __builtin_amdgcn_s_setprio(0);
    if (active) {
        constexpr int NV = 2 * RPW;  // entries 2i (gate) and 2i + 1 (up) of row-step i
        const int k0 = lr * Q::NV;
        uint4 cl[NV][CPL];
        float sc[NV][Q::NGL], of[NV][Q::NGL];
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                cl[2 * i][j] = gc[i][j];
                cl[2 * i + 1][j] = uc[i][j];
            }
#pragma unroll
            for (int g = 0; g < Q::NGL; ++g) {
                sc[2 * i][g] = bf16_lo(gsb[i][g]);
                of[2 * i][g] = fmaf(Q::kCodeOffset, sc[2 * i][g], bf16_hi(gsb[i][g]));
                sc[2 * i + 1][g] = bf16_lo(usb[i][g]);
                of[2 * i + 1][g] = fmaf(Q::kCodeOffset, sc[2 * i + 1][g], bf16_hi(usb[i][g]));
            }
        }
        float part[NV];
        rows_dot_lds<BITS, CPL, NV>(cl, sc, of, s_hl, s_hs, s_hx, H, k0, part);

        float *act = a.ws.act + (size_t)t * (K + 1) * F;
        if constexpr (LPR != 0) {
            // rows past the end are computed on re-read registers and not written
            const float r = multi_reduce<NV, LPR>(part);
            constexpr int DL = LPR / NV;  // lanes sharing one reduced entry
            const int rs = rs0 + multi_index<NV, LPR>(lane) / 2;
            const float up = xchg<DL>(r);  // the up sum sits across the last halving bit
            // SwiGLU with the hardware exp and reciprocal (as in the grouped
            // kernels): the IEEE division's ~15 instructions sat in the tail
            if ((lane & (2 * DL - 1)) == 0 && rs < nrs) act[rs * rpi + rsub] = r * up * __builtin_amdgcn_rcpf(1.0f + __expf(-r));
        } else {
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                const int rs = rs0 + i;
                const float g = lane_group_sum(part[2 * i], lpr);
                const float u = lane_group_sum(part[2 * i + 1], lpr);
                if (rs < nrs && lr == 0) act[rs * rpi + rsub] = g * u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
            }
        }
    }

    // 6. block 0, wave 0: the whole routing of the token (k_down reads it)
    if constexpr (!TIER) {
        if (blockIdx.x == 0 && wave == 0) {
            uint32_t key[EPL];
            logit_keys<EPL>(zv, E, key);
            const RouteK rt = route_all<EPL>(key, E, K);
            if (lane < K) {
                a.ws.sel[t * K + lane] = rt.sel;
                a.ws.coef[t * (K + 1) + lane] = rt.w;
                if (a.route_idx) a.route_idx[t * K + lane] = rt.sel;
                if (a.route_w) a.route_w[t * K + lane] = rt.w;
            }
            if (lane == 0) a.ws.coef[t * (K + 1) + K] = sigmoidf_(gs);
        }
    }
}

// ---------------------------------------------------------------------------
// k_down: RPW row-steps of the H output rows per wave, all K+1 experts in
// batches of SB slots whose loads are all in flight together.
// ---------------------------------------------------------------------------
// k_down processes the K+1 slots in batches of at most kDownBatch; a batch's
// activations are staged in LDS once per block, in fixed point: the NV
// consecutive activations that one lane multiplies with its codes (a lane
// slice) share one exponent e (max |a| < 2^e, from the slice's 2 to 8 staging
// threads), and a value is V = rint(a 2^(22-e)) in three byte limbs
// (byte_limbs), with the slice's scale 2^(e-22) (NaN when the slice holds a
// NaN or an inf) and the half-group sums of the activations beside them.  The
// products then take one v_dot4 per limb and four codes (qdot_limbs) instead
// of a conversion and an fma per code: they are what remains once the
// weights land, on one SIMD for two waves.  A pad of 4 words after every
// slice's limbs puts consecutive lanes on odd multiples of 16 bytes.
constexpr int kDownBatch = 5;
constexpr int kDownStageValues = 5120;  // activations staged per batch (batch * F <= this)

// LPR: lanes per row for one butterfly over the wave's RPW rows (16, 32, 64);
// 0: one reduction per row
// ONE: all K+1 slots in a single batch (straight-line code: no loop-header
// wait holds back the first loads)
// SPLIT: wave groups per block (1 or 2), so that a SIMD runs SPLIT waves (one
// alone exposes its LDS and VALU latencies: the products are VALU-bound once
// the weights land).
// ROWS: group g takes the g-th 4 RPW row-steps of the block and every wave
// every slot position; else group g takes the slot positions g, g + SPLIT, ...
// of every batch for all the block's rows, and the groups' row sums are added
// in group order through LDS before the one write per row.  With the K + 1 = 5
// slot positions of top-4, the slot split leaves 3 products per row on one
// group and 2 on the other, and the group with 3 sets the block's end; the row
// split gives every wave the same work and needs no exchange.
// TIER: the selected experts sit in cache slots, sl.s[t * K + rank] (a.experts
// = the slots' base)
template <int BITS, int CPL, int RPW, int LPR, bool ONE, bool TIER, int SPLIT, bool ROWS = false>
__global__ __launch_bounds__(256 * SPLIT) void k_down(const float *__restrict__ p_x, const int32_t *__restrict__ p_sel,
                                                     const float *__restrict__ p_coef, const float *__restrict__ p_act,
                                                     int H, int F, int K, int batch, uint32_t f4_recip, FwdArgs a,
                                                     SlotParam<TIER> sl) {
    using Q = QSlice<BITS, CPL>;
    constexpr int NT = 256 * SPLIT;                                  // threads per block
    constexpr int kPer = ROWS ? kDownBatch : (kDownBatch + SPLIT - 1) / SPLIT;  // slot positions per wave
    const int t = blockIdx.y;
    const int E = a.s.E;
    // wave and group are wave-uniform (so are the slots and experts they select:
    // the weight loads then take the scalar-base form)
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) & 3),
              grp = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);
    const QMat &Dm = a.L.m[2];
    const int lpr = LPR ? LPR : Dm.lpr, rpi = 64 / lpr;
    const int lr = lane % lpr, rsub = lane / lpr;
    const int nrs = H / rpi;
    const int rs0 = (ROWS ? blockIdx.x * 4 * SPLIT + grp * 4 + wave : blockIdx.x * 4 + wave) * RPW;
    const bool active = rs0 < nrs;
    const int k0 = lr * Q::NV;
    const uint32_t F4 = F / 4;

    // the residual of the rows this lane may write, fetched now
    float xres[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int rs = rs0 + i < nrs ? rs0 + i : nrs - 1;
        xres[i] = p_x[(size_t)t * H + rs * rpi + rsub];
    }

    constexpr int NP = Q::NV / 4;   // four-value pieces per lane slice
    constexpr int LS = 3 * NP + 4;  // words per staged slice: limbs L0, L1, L2, pad
    const int nsl = F / Q::NV;      // slices per slot
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t *s_lmb = (uint32_t *)smem;                          // [batch][nsl][LS]
    float *s_lsc = (float *)(s_lmb + (size_t)batch * nsl * LS);  // [batch][nsl]
    float *s_half = s_lsc + (size_t)batch * nsl;                 // [batch][F/32]

    // lane s (s <= K) holds slot s: expert index (s < K) and combine
    // coefficient; only those lanes are ever read (unconditional loads, lanes
    // past the end read a valid entry)
    int my_e;
    if constexpr (TIER) my_e = sl.s[t * K + (lane < K ? lane : K - 1)];
    else my_e = p_sel[t * K + (lane < K ? lane : K - 1)];
    const float my_c = p_coef[t * (K + 1) + (lane <= K ? lane : K)];

    float acc[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) acc[i] = 0.0f;

    // slot positions run shared, 0, 1, ..., K-1: the shared expert's loads need no routing
    constexpr int kStageMax = (kDownStageValues + 4 * NT - 1) / (4 * NT);  // float4 pieces per thread and batch
    auto run_batch = [&](int b0) {
        const int nb = (K + 1 - b0) < batch ? (K + 1 - b0) : batch;
        // this batch's activations first: the staging then waits on them only
        // (loads complete in order), while the weight loads stay in flight
        // every load below is unconditional (indices past the end are
        // clamped to valid ones and their results unused), so that all of
        // them are in flight before the first wait
        // float4 piece p = tid + NT r: slot p / (F/4) by a multiply-high
        // with f4_recip = ceil(2^32 / (F/4)) (exact: p (F/4) < 2^32)
        float4 stv[kStageMax];
        uint32_t sti[kStageMax], stj[kStageMax];
        const float *act_t = p_act + (size_t)t * (K + 1) * F;
#pragma unroll
        for (int r = 0; r < kStageMax; ++r) {
            const uint32_t p = threadIdx.x + NT * r;
            const uint32_t pc = p < (uint32_t)(nb * F4) ? p : 0u;
            const uint32_t si = __umulhi(pc, f4_recip), j = (pc - __umul24(si, F4)) * 4;
            const uint32_t s = (b0 + si == 0) ? K : b0 + si - 1;
            sti[r] = si;
            stj[r] = j;
            stv[r] = *(const float4 *)(act_t + (__umul24(s, (uint32_t)F) + j));
        }
        // weights of this group's slot positions grp, grp + SPLIT, ... of
        // the batch, all in flight together
        uint4 wc[kPer][RPW][CPL];
        uint32_t wsb[kPer][RPW][Q::NGL];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int si = ROWS ? u : grp + SPLIT * u;
            const int sc = si < nb ? si : nb - 1;
            const int s = (b0 + sc == 0) ? K : b0 + sc - 1;
            const uint8_t *ex;
            if constexpr (TIER) {
                ex = (s == K) ? a.shared : a.experts + (size_t)lane_bcast(my_e, s) * a.L.bytes;
            } else {
                const int e = (s == K) ? E : lane_bcast(my_e, s);
                ex = (e < E) ? a.experts + (size_t)e * a.L.bytes : a.shared;
            }
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                const int rs = rs0 + i < nrs ? rs0 + i : nrs - 1;
                load_row<BITS, CPL>(ex, Dm, rs * rpi + rsub, lr, wc[u][i], wsb[u][i]);
            }
        }
        // stage this batch's activations (limbs and slice scales) and
        // half-group sums; a slice's NP pieces are NP consecutive threads
        if (b0 > 0) __syncthreads();  // the previous batch is done with the LDS
#pragma unroll
        for (int r = 0; r < kStageMax; ++r) {
            const int v0 = threadIdx.x * 4 + 4 * NT * r;
            if (4 * NT * r < batch * F) {  // uniform: whole slices are live or not
                const bool live = v0 < nb * F;
                const uint32_t si = sti[r], j = stj[r];
                const float4 v = stv[r];
                // the slice maximum of |a| as bits (NaN and inf above every finite value)
                uint32_t mb = __float_as_uint(v.x) & 0x7FFFFFFFu;
                mb = max(mb, __float_as_uint(v.y) & 0x7FFFFFFFu);
                mb = max(mb, __float_as_uint(v.z) & 0x7FFFFFFFu);
                mb = max(mb, __float_as_uint(v.w) & 0x7FFFFFFFu);
                const float m = __uint_as_float(lane_max_u32<NP>(mb));
                const float up = pow2f(kFixBits - limb_exponent(m));
                uint32_t l0, l1, l2;
                byte_limbs((int)rintf(v.x * up), (int)rintf(v.y * up), (int)rintf(v.z * up), (int)rintf(v.w * up),
                           l0, l1, l2);
                const float half = lane_sum<8>((v.x + v.y) + (v.z + v.w));  // 8 threads = 32 values
                if (live) {
                    const uint32_t sl = si * nsl + j / Q::NV, pc = (j % Q::NV) / 4;
                    uint32_t *d = s_lmb + sl * LS + pc;
                    d[0] = l0;
                    d[NP] = l1;
                    d[2 * NP] = l2;
                    if (pc == 0) s_lsc[sl] = limb_scale(m);
                    if ((threadIdx.x & 7) == 0) s_half[v0 / 32] = half;
                }
            }
        }
        __syncthreads();
        if (active) {
#pragma unroll
            for (int u = 0; u < kPer; ++u) {
                const int si = ROWS ? u : grp + SPLIT * u;
                if (si < nb) {
                    const int s = (b0 + si == 0) ? K : b0 + si - 1;
                    const float c = lane_bcast(my_c, s);
                    uint32_t L[3][NP];
                    const uint32_t *src = s_lmb + (si * nsl + lr) * LS;
#pragma unroll
                    for (int x = 0; x < 3; ++x)
#pragma unroll
                        for (int i = 0; i < NP / 4; ++i) {
                            const uint4 w = *(const uint4 *)(src + x * NP + 4 * i);
                            L[x][4 * i] = w.x; L[x][4 * i + 1] = w.y; L[x][4 * i + 2] = w.z; L[x][4 * i + 3] = w.w;
                        }
                    const float lsc = s_lsc[si * nsl + lr];
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
                        if (rs0 + i < nrs) acc[i] = fmaf(c, qdot_limbs<BITS, CPL>(wc[u][i], wsb[u][i], L, lsc, X), acc[i]);
                }
            }
        }
    };
    if constexpr (ONE) {
        run_batch(0);
    } else {
        for (int b0 = 0; b0 <= K; b0 += batch) run_batch(b0);
    }
    // row sums; with SPLIT groups, group g > 0 hands its sums to group 0 through LDS
    if constexpr (LPR != 0 && RPW <= LPR) {
        float v = multi_reduce<RPW, LPR>(acc);
        const int i = multi_index<RPW, LPR>(lane);
        constexpr int DL = LPR / RPW;  // lanes sharing one reduced row
        if constexpr (SPLIT > 1 && !ROWS) {
            __shared__ float s_part[SPLIT - 1][4][64];
            if (grp > 0) s_part[grp - 1][wave][lane] = v;
            __syncthreads();
            if (grp > 0) return;
#pragma unroll
            for (int q = 0; q < SPLIT - 1; ++q) v += s_part[q][wave][lane];
        }
        if (!active) return;
        float xr = xres[0];
#pragma unroll
        for (int q = 1; q < RPW; ++q) xr = (i == q) ? xres[q] : xr;
        if ((lane & (DL - 1)) == 0 && rs0 + i < nrs) a.y[(size_t)t * H + (rs0 + i) * rpi + rsub] = xr + v;
    } else {
        static_assert(SPLIT == 1 || ROWS, "split slots need the one-butterfly reduction");
        if (!active) return;
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int rs = rs0 + i;
            const float v = lane_group_sum(acc[i], lpr);
            if (rs < nrs && lr == 0) a.y[(size_t)t * H + rs * rpi + rsub] = xres[i] + v;
        }
    }
}

// k_route: softmax -> top-K -> renormalise of one token per one-wave block,
// from the router's logits: the routing that k_gateup's waves do for
// themselves, as a kernel of its own for callers that need the selection
// before the experts run (tiered residency copies the missing experts in
// between).  Same functions, same results, same writes as k_gateup's block 0.
template <int EPL>
__global__ __launch_bounds__(64) void k_route(FwdArgs a) {
    const int t = blockIdx.x, K = a.s.K, E = a.s.E;
    const int lane = threadIdx.x & 63;
    float zv[EPL];
    load_logits_lane<EPL>(a.ws.z + (size_t)t * logit_stride(E), logit_stride(E), zv);
    const float gs = a.ws.gs[t];
    uint32_t key[EPL];
    logit_keys<EPL>(zv, E, key);
    const RouteK rt = route_all<EPL>(key, E, K);
    if (lane < K) {
        a.ws.sel[t * K + lane] = rt.sel;
        a.ws.coef[t * (K + 1) + lane] = rt.w;
        if (a.route_idx) a.route_idx[t * K + lane] = rt.sel;
        if (a.route_w) a.route_w[t * K + lane] = rt.w;
        if (a.sel_host) a.sel_host[t * K + lane] = ((uint64_t)a.sel_tag << 32) | (uint32_t)rt.sel;
    }
    if (lane == 0) a.ws.coef[t * (K + 1) + K] = sigmoidf_(gs);
    // push the tagged entries out to host memory now (each entry validates
    // itself, so no write has to land before another)
    if (a.sel_host) __threadfence_system();
}

// k_fetch: whole experts from host memory into cache slots over the host
// link; each block copies its share of every listed expert (a few dozen
// blocks keep the link busy; more only add contention)
__global__ __launch_bounds__(256) void k_fetch(FetchArgs f) {
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const uint64_t n16 = f.bytes / 16;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (int i = 0; i < f.n; ++i) {
        const v4u *src = (const v4u *)(f.src + (uint64_t)f.expert[i] * f.bytes);
        v4u *dst = (v4u *)(f.dst + (uint64_t)f.slot[i] * f.bytes);
        for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n16; j += stride)
            dst[j] = __builtin_nontemporal_load(src + j);
    }
}

// gate/up row-steps per wave: with 4-bit codes the routed blocks route once
// per block and take one row-step per wave (more waves share the products)
template <int BITS, bool TIER>
constexpr int kRpwGateUp = (BITS == 4 && !TIER) ? 1 : 2;
constexpr int kRouterTokens = 4;  // tokens per k_router_tokens block
constexpr int kRpwDown4 = 2;  // 4-bit codes
constexpr int kRpwDown2 = 1;  // 2-bit codes

template <int BITS, bool TIER>
hipError_t launch_stage(const FwdArgs &a, int stage, hipStream_t st, const SlotParam<TIER> &sl = {}) {
    const int H = a.s.H, F = a.s.F, E = a.s.E, K = a.s.K, T = a.T;
    constexpr int RD = BITS == 4 ? kRpwDown4 : kRpwDown2;  // down row-steps per wave group
    // two wave groups per block split its rows when the row-steps halve
    // (4-bit k_down 4.97 -> 4.58 us), else its slot positions
    constexpr bool DR = RD % 2 == 0;
    constexpr int RDS = DR ? RD / 2 : RD;  // row-steps per wave with two groups
    if (stage == 0 && (H == 2048 || H == 4096)) {  // RMSNorm + router + limbs of h, H split over 4 waves
        const int rows = (E + 1 + kRouterSplitRows - 1) / kRouterSplitRows;
        const int blocks = rows > H / 256 ? rows : H / 256;
        // one token per block for up to 3 tokens, else four (each router row
        // read once per four tokens)
        const bool one = T < kRouterTokens;
        const dim3 grid(blocks, one ? T : (T + kRouterTokens - 1) / kRouterTokens);
        if (H == 4096) {
            if (one) hipLaunchKernelGGL(k_router_split<2>, grid, dim3(256), 0, st, a.router, a.sgate, a.x, a.gamma, H, E, a);
            else hipLaunchKernelGGL((k_router_tokens<2, kRouterTokens>), grid, dim3(256), 0, st, a);
        } else {
            if (one) hipLaunchKernelGGL(k_router_split<1>, grid, dim3(256), 0, st, a.router, a.sgate, a.x, a.gamma, H, E, a);
            else hipLaunchKernelGGL((k_router_tokens<1, kRouterTokens>), grid, dim3(256), 0, st, a);
        }
    } else if (stage == 0) {  // RMSNorm + router + limbs of h
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
        constexpr int RG = kRpwGateUp<BITS, TIER>;
        if ((F / rpi) % RG != 0) return hipErrorInvalidValue;  // a wave's row-steps share one slot
        const int nrs = (K + 1) * F / rpi;
        const int blocks = (nrs + 4 * RG - 1) / (4 * RG);
        dim3 grid(blocks, T);
        const bool wide = E > 512;
        const bool full = G.lpr == 64;  // rows of 64 lanes: one butterfly for the whole step
        // routing once per block when a block's waves share one slot
        const bool br = !TIER && (F / rpi) % (4 * RG) == 0;
        const int sel = (br ? 16 : 0) + G.cpl * 4 + (wide ? 2 : 0) + (full ? 1 : 0);
#define MOE_GATEUP(CPL, EPL, LPR, BR)                                                                      \
    hipLaunchKernelGGL((k_gateup<BITS, CPL, RG, EPL, LPR, TIER, BR>), grid, dim3(256), 0, st, a.ws.z, a.ws.gs, \
                       (const uint32_t *)a.ws.hl, a.ws.hs, a.ws.hx, H, (uint32_t)E | (uint32_t)F << 16, a.shared, a, sl)
        switch (sel) {
            case 4: MOE_GATEUP(1, 8, 0, false); break;
            case 5: MOE_GATEUP(1, 8, 64, false); break;
            case 6: MOE_GATEUP(1, 16, 0, false); break;
            case 7: MOE_GATEUP(1, 16, 64, false); break;
            case 9: MOE_GATEUP(2, 8, 64, false); break;
            case 11: MOE_GATEUP(2, 16, 64, false); break;
            case 20: MOE_GATEUP(1, 8, 0, !TIER); break;
            case 21: MOE_GATEUP(1, 8, 64, !TIER); break;
            case 22: MOE_GATEUP(1, 16, 0, !TIER); break;
            case 23: MOE_GATEUP(1, 16, 64, !TIER); break;
            case 25: MOE_GATEUP(2, 8, 64, !TIER); break;
            case 27: MOE_GATEUP(2, 16, 64, !TIER); break;
            default: return hipErrorInvalidValue;
        }
#undef MOE_GATEUP
    } else if (stage == 2) {  // down + combine + residual
        const QMat &Dm = a.L.m[2];
        const int rpi = 64 / Dm.lpr;
        const int nrs = H / rpi;
        // rows of fewer than 16 lanes (small F, e.g. 128): one row-step per wave and
        // twice the blocks (hidden 256 / FFN 128 layer: k_down 3.55 -> 3.11 us)
        const int rdl = (Dm.cpl == 1 && Dm.lpr < 16) ? 1 : RD;
        const int blocks = (nrs + 4 * rdl - 1) / (4 * rdl);
        dim3 grid(blocks, T);
        // per slot: limb words (3 per 4 values, a 4-word pad per lane slice),
        // slice scales and half-group sums
        const size_t per_slot = (size_t)(3 * F / 4 + 5 * Dm.lpr + F / 32) * 4;
        int batch = kDownStageValues / F;
        if (batch > kDownBatch) batch = kDownBatch;
        if (batch > K + 1) batch = K + 1;
        if (batch < 1) batch = 1;
        const size_t lds = per_slot * batch;
        const bool one = K + 1 <= batch;
        const uint32_t f4r = (uint32_t)((0x100000000ull + F / 4 - 1) / (F / 4));
        // two wave groups per block (slots split between them) when all slots
        // fit one batch and there are at least two of them
        const bool split = one && K + 1 >= 2;
        const dim3 b1(256), b2(512);
        if (Dm.cpl == 2) {
            if (split) hipLaunchKernelGGL((k_down<BITS, 2, RDS, 64, true, TIER, 2, DR>), grid, b2, lds, st, a.x, a.ws.sel, a.ws.coef, a.ws.act, H, F, K, batch, f4r, a, sl);
            else if (one) hipLaunchKernelGGL((k_down<BITS, 2, RD, 64, true, TIER, 1>), grid, b1, lds, st, a.x, a.ws.sel, a.ws.coef, a.ws.act, H, F, K, batch, f4r, a, sl);
            else hipLaunchKernelGGL((k_down<BITS, 2, RD, 64, false, TIER, 1>), grid, b1, lds, st, a.x, a.ws.sel, a.ws.coef, a.ws.act, H, F, K, batch, f4r, a, sl);
        } else if (Dm.cpl == 1) {
            const int key = (Dm.lpr == 64 ? 0 : Dm.lpr == 32 ? 1 : Dm.lpr == 16 ? 2 : 3) * 3 + (split ? 2 : one ? 1 : 0);
            switch (key) {
                case 0: hipLaunchKernelGGL((k_down<BITS, 1, RD, 64, false, TIER, 1>), grid, b1, lds, st, a.x, a.ws.sel, a.ws.coef, a.ws.act, H, F, K, batch, f4r, a, sl); break;
                case 1: hipLaunchKernelGGL((k_down<BITS, 1, RD, 64, true, TIER, 1>), grid, b1, lds, st, a.x, a.ws.sel, a.ws.coef, a.ws.act, H, F, K, batch, f4r, a, sl); break;
                case 2: hipLaunchKernelGGL((k_down<BITS, 1, RDS, 64, true, TIER, 2, DR>), grid, b2, lds, st, a.x, a.ws.sel, a.ws.coef, a.ws.act, H, F, K, batch, f4r, a, sl); break;
                case 3: hipLaunchKernelGGL((k_down<BITS, 1, RD, 32, false, TIER, 1>), grid, b1, lds, st, a.x, a.ws.sel, a.ws.coef, a.ws.act, H, F, K, batch, f4r, a, sl); break;
                case 4: hipLaunchKernelGGL((k_down<BITS, 1, RD, 32, true, TIER, 1>), grid, b1, lds, st, a.x, a.ws.sel, a.ws.coef, a.ws.act, H, F, K, batch, f4r, a, sl); break;
                case 5: hipLaunchKernelGGL((k_down<BITS, 1, RDS, 32, true, TIER, 2, DR>), grid, b2, lds, st, a.x, a.ws.sel, a.ws.coef, a.ws.act, H, F, K, batch, f4r, a, sl); break;
                case 6: hipLaunchKernelGGL((k_down<BITS, 1, RD, 16, false, TIER, 1>), grid, b1, lds, st, a.x, a.ws.sel, a.ws.coef, a.ws.act, H, F, K, batch, f4r, a, sl); break;
                case 7: hipLaunchKernelGGL((k_down<BITS, 1, RD, 16, true, TIER, 1>), grid, b1, lds, st, a.x, a.ws.sel, a.ws.coef, a.ws.act, H, F, K, batch, f4r, a, sl); break;
                case 8: hipLaunchKernelGGL((k_down<BITS, 1, RDS, 16, true, TIER, 2, DR>), grid, b2, lds, st, a.x, a.ws.sel, a.ws.coef, a.ws.act, H, F, K, batch, f4r, a, sl); break;
                case 9: hipLaunchKernelGGL((k_down<BITS, 1, 1, 0, false, TIER, 1>), grid, b1, lds, st, a.x, a.ws.sel, a.ws.coef, a.ws.act, H, F, K, batch, f4r, a, sl); break;
                default: hipLaunchKernelGGL((k_down<BITS, 1, 1, 0, true, TIER, 1>), grid, b1, lds, st, a.x, a.ws.sel, a.ws.coef, a.ws.act, H, F, K, batch, f4r, a, sl); break;
            }
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_stage(const FwdArgs &a, int stage, hipStream_t stream) {
    (void)hipGetLastError();  // report only this call's launches
    if (a.s.bits == 4) return launch_stage<4, false>(a, stage, stream);
    if (a.s.bits == 2) return launch_stage<2, false>(a, stage, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_forward(const FwdArgs &a, hipStream_t stream) {
    for (int stage = 0; stage < kForwardStages; ++stage) {
        const hipError_t e = launch_forward_stage(a, stage, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_fetch(const FetchArgs &f, hipStream_t stream) {
    if (f.n < 1 || f.n > kSlotArgs || f.bytes % 16 != 0) return hipErrorInvalidValue;
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_fetch, dim3(64), dim3(256), 0, stream, f);
    return hipGetLastError();
}

hipError_t launch_forward_route(const FwdArgs &a, hipStream_t stream) {
    (void)hipGetLastError();
    hipError_t e = a.s.bits == 4 ? launch_stage<4, false>(a, 0, stream) : launch_stage<2, false>(a, 0, stream);
    if (e != hipSuccess) return e;
    // experts per lane as in k_gateup: 8 up to 512 experts, else 16
    if (a.s.E > 512) hipLaunchKernelGGL(k_route<16>, dim3(a.T), dim3(64), 0, stream, a);
    else hipLaunchKernelGGL(k_route<8>, dim3(a.T), dim3(64), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_forward_slots(const FwdArgs &a, const SlotArgs &slots, hipStream_t stream) {
    if (a.T * a.s.K > kSlotArgs) return hipErrorInvalidValue;
    (void)hipGetLastError();
    for (int stage = 1; stage < kForwardStages; ++stage) {
        const hipError_t e = a.s.bits == 4 ? launch_stage<4, true>(a, stage, stream, slots)
                                           : launch_stage<2, true>(a, stage, stream, slots);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace moe

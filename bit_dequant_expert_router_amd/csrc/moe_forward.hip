// moe_forward.hip -- the expert layer as three stream-ordered kernels.
//
//   k_router : two-pass RMSNorm + router GEMV (E rows) + shared-gate logit;
//              a few blocks also store h in the fixed-point limb form below
//              (k_router_split for H = 2048 / 4096, one token per block;
//              k_router_tokens from 4 tokens, four per block; k_router else)
//   k_gateup : per block, softmax/top-K/renormalise from the logits, then the
//              fused gate+up dequant GEMV of the selected experts and the
//              shared expert with SwiGLU in registers
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
// k_router_split (H = 2048 or 4096): the 4 waves of a block split H into
// quarters of the block's RB router rows (one row per block measures fastest:
// 513 blocks spread the 4 MiB over the whole chip), so a wave reads 1/4 of x
// and gamma instead of all of it.  The dot products use x * gamma; the factor
// 1 / rms(x) is applied to the block's sum (the norm's two passes are the
// waves' sums of squares, then the scaling).  The first H / 256 blocks also
// write the limb form of h for k_gateup.
// ---------------------------------------------------------------------------
constexpr int kRouterSplitRows = 1;

template <int CPL_R>
__global__ __launch_bounds__(256) void k_router_split(FwdArgs a) {
    constexpr int RB = kRouterSplitRows;
    const int t = blockIdx.y;
    const int H = a.s.H, E = a.s.E;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float *x = a.x + (size_t)t * H;
    const int r0 = blockIdx.x * RB;
    // lane's chunks of 8 entries: wave quarter + lane + 64 j
    const int kq = wave * (H / 4);
    uint4 wv[RB][CPL_R];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const int row = r0 + r <= E ? r0 + r : E;  // rows past the end re-read the gate row, unused
        const uint16_t *src = (row < E) ? a.router + (size_t)row * H : a.sgate;
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
        gv[j] = *(const uint4 *)(a.gamma + k0);
    }
    // this block's share of the limb encoding: entry k of h (x and gamma fetched now)
    const int ke = blockIdx.x * 256 + threadIdx.x;
    const bool enc = blockIdx.x * 256 < H;
    const float xe = x[ke < H ? ke : 0];
    const float ge = __uint_as_float((uint32_t)a.gamma[ke < H ? ke : 0] << 16);

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
    const float inv = 1.0f / sqrtf(((s_ss[0] + s_ss[1]) + (s_ss[2] + s_ss[3])) / (float)H + a.s.eps);
    if (threadIdx.x < RB) {
        const int row = r0 + threadIdx.x;
        const float z = (((s_part[0][threadIdx.x] + s_part[1][threadIdx.x]) + s_part[2][threadIdx.x]) +
                         s_part[3][threadIdx.x]) * inv;
        if (row < E)
            a.ws.z[(size_t)t * E + row] = z;
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
        return 1.0f / sqrtf(ss / (float)H + a.s.eps);
    };
    if (threadIdx.x < TB && t0 + (int)threadIdx.x < T) {
        const int tt = threadIdx.x, t = t0 + tt;
        const float z = (((s_part[0][tt] + s_part[1][tt]) + s_part[2][tt]) + s_part[3][tt]) * inv_of(tt);
        if (r0 < E)
            a.ws.z[(size_t)t * E + r0] = z;
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
// k_gateup: RPW row-steps per wave over the (K+1) x F gate/up row pairs
// ---------------------------------------------------------------------------
// LPR: lanes per row when the step's partial sums are reduced together (64);
// 0: one reduction per row
// TIER: the selected experts' routing is already done (k_route) and their
// weights sit in cache slots, sl.s[t * K + rank] (a.experts = the slots' base)
template <int BITS, int CPL, int RPW, int EPL, int LPR, bool TIER>
__global__ __launch_bounds__(256) void k_gateup(FwdArgs a, SlotParam<TIER> sl) {
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
    const bool block_routed = !TIER && (blockIdx.x * 4 * RPW * rpi) / F < K;
    const bool wave_shared_only = (rs0 * rpi) / F >= K;

    __shared__ __align__(16) uint32_t s_hl[kLimbs * kMaxDim / 8];  // limbs of h, [kLimbs][H/8]
    __shared__ float s_hs[kMaxDim / 64];
    __shared__ float s_hx[kMaxDim / 32];

    // the block's four waves route together, a quarter of the logits each
    // (route_candidates, then route_select after the block's barrier): the
    // logit loads go first (loads complete in order)
    constexpr int EPW = EPL / 4;
    __shared__ __align__(16) uint64_t s_cand[4 * kMaxTopK];
    float zq[EPW];
    if (block_routed) load_logits_quarter<EPW>(a.ws.z + (size_t)t * E, E, zq);
    const float gs = a.ws.gs[t];  // shared-gate logit (block 0 writes its coefficient)

    // stage the limb form of h in LDS, once per block
    {
        // kStage 16-byte pieces per thread (a native vector type: an array of
        // int4 can keep dead copies in scratch memory)
        typedef int i32x4 __attribute__((ext_vector_type(4)));
        const i32x4 *src = (const i32x4 *)((const uint32_t *)a.ws.hl + (size_t)t * kLimbs * (H / 8));
        const int n16 = kLimbs * H / 32;
        constexpr int kStage = (kLimbs * kMaxDim / 32 + 255) / 256;
        i32x4 st[kStage];
#pragma unroll
        for (int j = 0; j < kStage; ++j) {
            const int i = threadIdx.x + 256 * j;
            st[j] = src[i < n16 ? i : 0];
        }
        float hs = 0.0f, hx = 0.0f;
        if (threadIdx.x < H / 64) hs = a.ws.hs[(size_t)t * (H / 64) + threadIdx.x];
        if (threadIdx.x < H / 32) hx = a.ws.hx[(size_t)t * (H / 32) + threadIdx.x];
        if (block_routed) route_candidates<EPW>(zq, E, K, s_cand);
        {
            i32x4 *dst = (i32x4 *)s_hl;
#pragma unroll
            for (int j = 0; j < kStage; ++j) {
                const int i = threadIdx.x + 256 * j;
                if (i < n16) dst[i] = st[j];
            }
        }
        if (threadIdx.x < H / 64) s_hs[threadIdx.x] = hs;
        if (threadIdx.x < H / 32) s_hx[threadIdx.x] = hx;
    }

    // weight loads: shared-only waves issue theirs before the routing is known
    uint4 gc[RPW][CPL], uc[RPW][CPL];
    uint32_t gsb[RPW][Q::NGL], usb[RPW][Q::NGL];
    // every row's loads unconditional (rows past the end re-read the last
    // row), so that they are all in flight before the first wait
    // (addresses first, then every load back to back)
    // er[i]: the expert of row-step i when its slot is routed
    auto issue_loads = [&](const int (&er)[RPW]) {
        const uint8_t *exr[RPW];
        int jr[RPW];
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int rs = rs0 + i < nrs ? rs0 + i : nrs - 1;
            const int p = rs * rpi + rsub;
            const int s = p / F;
            jr[i] = p - s * F;
            exr[i] = (s < K) ? a.experts + (size_t)er[i] * a.L.bytes : a.shared;
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            load_row<BITS, CPL>(exr[i], G, jr[i], lr, gc[i], gsb[i]);
            load_row<BITS, CPL>(exr[i], U, jr[i], lr, uc[i], usb[i]);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (TIER) {  // the slots are known: every wave issues its loads now
        if (active) {
            int er[RPW];
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                const int rs = rs0 + i < nrs ? rs0 + i : nrs - 1;
                const int s = (rs * rpi) / F;
                er[i] = sl.s[t * K + (s < K ? s : K - 1)];
            }
            issue_loads(er);
        }
    } else if (active && wave_shared_only) {
        const int none[RPW] = {};
        issue_loads(none);
    }
    __syncthreads();
    if (!active) return;
    if (!TIER && !wave_shared_only) {
        // every routed wave ranks the block's candidates itself
        const RouteSel rt = route_select(K, s_cand);
        if (blockIdx.x == 0 && wave == 0) {
            if (rt.rank < K) {
                a.ws.sel[t * K + rt.rank] = rt.sel;
                a.ws.coef[t * (K + 1) + rt.rank] = rt.w;
                if (a.route_idx) a.route_idx[t * K + rt.rank] = rt.sel;
                if (a.route_w) a.route_w[t * K + rt.rank] = rt.w;
            }
            if (lane == 0) a.ws.coef[t * (K + 1) + K] = sigmoidf_(gs);
        }
        int er[RPW];
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int rs = rs0 + i < nrs ? rs0 + i : nrs - 1;
            const int s = (rs * rpi) / F;  // uniform: a row-step's rows share their slot
            er[i] = routed_expert(rt, s < K ? s : K - 1);
        }
        issue_loads(er);
    }

    // codes prepared once, then every row against the lane's limb slice of h
    // in LDS, limb-major
    constexpr int NV = 2 * RPW;  // entries 2i (gate) and 2i + 1 (up) of row-step i
    const int k0 = lr * Q::NV;
    uint4 cl[NV][CPL];
    float sc[NV][Q::NGL], of[NV][Q::NGL];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        prep_codes<BITS, CPL>(gc[i]);
        prep_codes<BITS, CPL>(uc[i]);
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
        // rows past the end are computed on unloaded registers and not written
        const float r = multi_reduce<NV, LPR>(part);
        constexpr int DL = LPR / NV;  // lanes sharing one reduced entry
        const int rs = rs0 + multi_index<NV, LPR>(lane) / 2;
        const float up = xchg<DL>(r);  // the up sum sits across the last halving bit
        if ((lane & (2 * DL - 1)) == 0 && rs < nrs) act[rs * rpi + rsub] = r * sigmoidf_(r) * up;
    } else {
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int rs = rs0 + i;
            if (rs < nrs) {
                const float g = lane_group_sum(part[2 * i], lpr);
                const float u = lane_group_sum(part[2 * i + 1], lpr);
                if (lr == 0) act[rs * rpi + rsub] = g * sigmoidf_(g) * u;
            }
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
// k_down processes the K+1 slots in batches of at most kDownBatch; a batch's
// activations and their half-group sums are staged in LDS once per block.
// Each lane reads the NV consecutive activations of its slice; a pad of 4
// floats after every slice puts consecutive lanes on consecutive 16-byte bank
// groups (unpadded, slices 128 or 256 bytes apart share their banks).
constexpr int kDownBatch = 5;
constexpr int kDownStageValues = 5120;  // activations staged per batch (batch * F <= this)

// LPR: lanes per row for one butterfly over the wave's RPW rows (16, 32, 64);
// 0: one reduction per row
// ONE: all K+1 slots in a single batch (straight-line code: no loop-header
// wait holds back the first loads)
// TIER: the selected experts sit in cache slots, sl.s[t * K + rank] (a.experts
// = the slots' base)
template <int BITS, int CPL, int RPW, int LPR, bool ONE, bool TIER>
__global__ __launch_bounds__(256) void k_down(FwdArgs a, int batch, uint32_t f4_recip, SlotParam<TIER> sl) {
    using Q = QSlice<BITS, CPL>;
    const int t = blockIdx.y;
    const int H = a.s.H, F = a.s.F, E = a.s.E, K = a.s.K;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const QMat &Dm = a.L.m[2];
    const int lpr = LPR ? LPR : Dm.lpr, rpi = 64 / lpr;
    const int lr = lane % lpr, rsub = lane / lpr;
    const int nrs = H / rpi;
    const int rs0 = (blockIdx.x * 4 + wave) * RPW;
    const bool active = rs0 < nrs;
    const int k0 = lr * Q::NV;
    const uint32_t F4 = F / 4;

    // the residual of the rows this lane may write, fetched now
    float xres[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int rs = rs0 + i < nrs ? rs0 + i : nrs - 1;
        xres[i] = a.x[(size_t)t * H + rs * rpi + rsub];
    }

    constexpr int NVP = Q::NV + 4;  // padded slice
    const int FP = F / Q::NV * NVP;  // padded activations of one slot
    extern __shared__ __align__(16) unsigned char smem[];
    float *s_act = (float *)smem;               // [batch][F / NV][NVP]
    float *s_half = s_act + (size_t)batch * FP;  // [batch][F/32]

    // lane s (s <= K) holds slot s: expert index (s < K) and combine
    // coefficient; only those lanes are ever read (unconditional loads, lanes
    // past the end read a valid entry)
    int my_e;
    if constexpr (TIER) my_e = sl.s[t * K + (lane < K ? lane : K - 1)];
    else my_e = a.ws.sel[t * K + (lane < K ? lane : K - 1)];
    const float my_c = a.ws.coef[t * (K + 1) + (lane <= K ? lane : K)];

    float acc[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) acc[i] = 0.0f;

    // slot positions run shared, 0, 1, ..., K-1: the shared expert's loads need no routing
    constexpr int kStageMax = kDownStageValues / 1024;  // float4 pieces per thread and batch
    auto run_batch = [&](int b0) {
        const int nb = (K + 1 - b0) < batch ? (K + 1 - b0) : batch;
        // this batch's activations first: the staging then waits on them only
        // (loads complete in order), while the weight loads stay in flight
        // every load below is unconditional (indices past the end are
        // clamped to valid ones and their results unused), so that all of
        // them are in flight before the first wait
        // float4 piece p = tid + 256 r: slot p / (F/4) by a multiply-high
        // with f4_recip = ceil(2^32 / (F/4)) (exact: p (F/4) < 2^32)
        float4 stv[kStageMax];
        uint32_t sti[kStageMax], stj[kStageMax];
        const float *act_t = a.ws.act + (size_t)t * (K + 1) * F;
#pragma unroll
        for (int r = 0; r < kStageMax; ++r) {
            const uint32_t p = threadIdx.x + 256 * r;
            const uint32_t pc = p < (uint32_t)(nb * F4) ? p : 0u;
            const uint32_t si = __umulhi(pc, f4_recip), j = (pc - __umul24(si, F4)) * 4;
            const uint32_t s = (b0 + si == 0) ? K : b0 + si - 1;
            sti[r] = si;
            stj[r] = j;
            stv[r] = *(const float4 *)(act_t + (__umul24(s, (uint32_t)F) + j));
        }
        // weights of up to kDownBatch slots of this batch, all in flight together
        uint4 wc[kDownBatch][RPW][CPL];
        uint32_t wsb[kDownBatch][RPW][Q::NGL];
#pragma unroll
        for (int si = 0; si < kDownBatch; ++si) {
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
                load_row<BITS, CPL>(ex, Dm, rs * rpi + rsub, lr, wc[si][i], wsb[si][i]);
            }
        }
        // stage this batch's activations and half-group sums
        if (b0 > 0) __syncthreads();  // the previous batch is done with the LDS
#pragma unroll
        for (int r = 0; r < kStageMax; ++r) {
            const int v0 = threadIdx.x * 4 + 1024 * r;
            if (1024 * r < batch * F) {  // uniform: whole 8-thread groups are live or not
                const bool live = v0 < nb * F;
                const uint32_t si = sti[r], j = stj[r];
                if (live) *(float4 *)(s_act + si * FP + j / Q::NV * NVP + j % Q::NV) = stv[r];
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
                        const float4 v = *(const float4 *)(s_act + si * FP + lr * NVP + 4 * i);
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
    };
    if constexpr (ONE) {
        run_batch(0);
    } else {
        for (int b0 = 0; b0 <= K; b0 += batch) run_batch(b0);
    }
    if (!active) return;
    if constexpr (LPR != 0 && RPW <= LPR) {
        const float v = multi_reduce<RPW, LPR>(acc);
        const int i = multi_index<RPW, LPR>(lane);
        constexpr int DL = LPR / RPW;  // lanes sharing one reduced row
        float xr = xres[0];
#pragma unroll
        for (int q = 1; q < RPW; ++q) xr = (i == q) ? xres[q] : xr;
        if ((lane & (DL - 1)) == 0 && rs0 + i < nrs) a.y[(size_t)t * H + (rs0 + i) * rpi + rsub] = xr + v;
    } else {
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int rs = rs0 + i;
            const float v = lane_group_sum(acc[i], lpr);
            if (rs < nrs && lr == 0) a.y[(size_t)t * H + rs * rpi + rsub] = xres[i] + v;
        }
    }
}

// k_route: softmax -> top-K -> renormalise of one token per block, from the
// router's logits: the routing that k_gateup's routed blocks do for
// themselves, as a kernel of its own for callers that need the selection
// before the experts run (tiered residency copies the missing experts in
// between).  Same functions, same results, same writes as k_gateup's block 0.
template <int EPW>
__global__ __launch_bounds__(256) void k_route(FwdArgs a) {
    const int t = blockIdx.x, K = a.s.K, E = a.s.E;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __shared__ __align__(16) uint64_t s_cand[4 * kMaxTopK];
    float zq[EPW];
    load_logits_quarter<EPW>(a.ws.z + (size_t)t * E, E, zq);
    const float gs = a.ws.gs[t];
    route_candidates<EPW>(zq, E, K, s_cand);
    __syncthreads();
    if (wave == 0) {
        const RouteSel rt = route_select(K, s_cand);
        if (rt.rank < K) {
            a.ws.sel[t * K + rt.rank] = rt.sel;
            a.ws.coef[t * (K + 1) + rt.rank] = rt.w;
            if (a.route_idx) a.route_idx[t * K + rt.rank] = rt.sel;
            if (a.route_w) a.route_w[t * K + rt.rank] = rt.w;
            if (a.sel_host) a.sel_host[t * K + rt.rank] = rt.sel;
        }
        if (lane == 0) a.ws.coef[t * (K + 1) + K] = sigmoidf_(gs);
        if (a.flag_host) {  // the selection first, then the flag, both pushed out to the host
            __threadfence_system();
            if (lane == 0) a.flag_host[t] = a.flag_value;
            __threadfence_system();
        }
    }
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

constexpr int kRpwGateUp = 2;
constexpr int kRouterTokens = 4;  // tokens per k_router_tokens block
constexpr int kRpwDown4 = 2;  // 4-bit codes
constexpr int kRpwDown2 = 1;  // 2-bit codes

template <int BITS, bool TIER>
hipError_t launch_stage(const FwdArgs &a, int stage, hipStream_t st, const SlotParam<TIER> &sl = {}) {
    const int H = a.s.H, F = a.s.F, E = a.s.E, K = a.s.K, T = a.T;
    constexpr int RD = BITS == 4 ? kRpwDown4 : kRpwDown2;  // down row-steps per wave
    if (stage == 0 && (H == 2048 || H == 4096)) {  // RMSNorm + router + limbs of h, H split over 4 waves
        const int rows = (E + 1 + kRouterSplitRows - 1) / kRouterSplitRows;
        const int blocks = rows > H / 256 ? rows : H / 256;
        // one token per block for up to 3 tokens, else four (each router row
        // read once per four tokens)
        const bool one = T < kRouterTokens;
        const dim3 grid(blocks, one ? T : (T + kRouterTokens - 1) / kRouterTokens);
        if (H == 4096) {
            if (one) hipLaunchKernelGGL(k_router_split<2>, grid, dim3(256), 0, st, a);
            else hipLaunchKernelGGL((k_router_tokens<2, kRouterTokens>), grid, dim3(256), 0, st, a);
        } else {
            if (one) hipLaunchKernelGGL(k_router_split<1>, grid, dim3(256), 0, st, a);
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
        const int nrs = (K + 1) * F / rpi;
        const int blocks = (nrs + 4 * kRpwGateUp - 1) / (4 * kRpwGateUp);
        dim3 grid(blocks, T);
        const bool wide = E > 512;
        const bool full = G.lpr == 64;  // rows of 64 lanes: one butterfly for the whole step
        switch (G.cpl * 4 + (wide ? 2 : 0) + (full ? 1 : 0)) {
            case 4: hipLaunchKernelGGL((k_gateup<BITS, 1, kRpwGateUp, 8, 0, TIER>), grid, dim3(256), 0, st, a, sl); break;
            case 5: hipLaunchKernelGGL((k_gateup<BITS, 1, kRpwGateUp, 8, 64, TIER>), grid, dim3(256), 0, st, a, sl); break;
            case 6: hipLaunchKernelGGL((k_gateup<BITS, 1, kRpwGateUp, 16, 0, TIER>), grid, dim3(256), 0, st, a, sl); break;
            case 7: hipLaunchKernelGGL((k_gateup<BITS, 1, kRpwGateUp, 16, 64, TIER>), grid, dim3(256), 0, st, a, sl); break;
            case 9: hipLaunchKernelGGL((k_gateup<BITS, 2, kRpwGateUp, 8, 64, TIER>), grid, dim3(256), 0, st, a, sl); break;
            case 11: hipLaunchKernelGGL((k_gateup<BITS, 2, kRpwGateUp, 16, 64, TIER>), grid, dim3(256), 0, st, a, sl); break;
            default: return hipErrorInvalidValue;
        }
    } else if (stage == 2) {  // down + combine + residual
        const QMat &Dm = a.L.m[2];
        const int rpi = 64 / Dm.lpr;
        const int nrs = H / rpi;
        const int blocks = (nrs + 4 * RD - 1) / (4 * RD);
        dim3 grid(blocks, T);
        // padded activations (4 floats per lane slice) and half-group sums
        const size_t per_slot = (size_t)(F + 4 * Dm.lpr) * 4 + (size_t)(F / 32) * 4;
        int batch = kDownStageValues / F;
        if (batch > kDownBatch) batch = kDownBatch;
        if (batch > K + 1) batch = K + 1;
        if (batch < 1) batch = 1;
        const size_t lds = per_slot * batch;
        const bool one = K + 1 <= batch;
        const uint32_t f4r = (uint32_t)((0x100000000ull + F / 4 - 1) / (F / 4));
        if (Dm.cpl == 2) {
            if (one) hipLaunchKernelGGL((k_down<BITS, 2, RD, 64, true, TIER>), grid, dim3(256), lds, st, a, batch, f4r, sl);
            else hipLaunchKernelGGL((k_down<BITS, 2, RD, 64, false, TIER>), grid, dim3(256), lds, st, a, batch, f4r, sl);
        } else if (Dm.cpl == 1) {
            const int key = (Dm.lpr == 64 ? 0 : Dm.lpr == 32 ? 1 : Dm.lpr == 16 ? 2 : 3) * 2 + (one ? 1 : 0);
            switch (key) {
                case 0: hipLaunchKernelGGL((k_down<BITS, 1, RD, 64, false, TIER>), grid, dim3(256), lds, st, a, batch, f4r, sl); break;
                case 1: hipLaunchKernelGGL((k_down<BITS, 1, RD, 64, true, TIER>), grid, dim3(256), lds, st, a, batch, f4r, sl); break;
                case 2: hipLaunchKernelGGL((k_down<BITS, 1, RD, 32, false, TIER>), grid, dim3(256), lds, st, a, batch, f4r, sl); break;
                case 3: hipLaunchKernelGGL((k_down<BITS, 1, RD, 32, true, TIER>), grid, dim3(256), lds, st, a, batch, f4r, sl); break;
                case 4: hipLaunchKernelGGL((k_down<BITS, 1, RD, 16, false, TIER>), grid, dim3(256), lds, st, a, batch, f4r, sl); break;
                case 5: hipLaunchKernelGGL((k_down<BITS, 1, RD, 16, true, TIER>), grid, dim3(256), lds, st, a, batch, f4r, sl); break;
                case 6: hipLaunchKernelGGL((k_down<BITS, 1, RD, 0, false, TIER>), grid, dim3(256), lds, st, a, batch, f4r, sl); break;
                default: hipLaunchKernelGGL((k_down<BITS, 1, RD, 0, true, TIER>), grid, dim3(256), lds, st, a, batch, f4r, sl); break;
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
    if (a.s.E > 512) hipLaunchKernelGGL(k_route<4>, dim3(a.T), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(k_route<2>, dim3(a.T), dim3(256), 0, stream, a);
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

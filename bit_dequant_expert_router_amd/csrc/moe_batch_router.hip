// moe_batch_router.hip -- RMSNorm and router logits for a batch of tokens.
//
// The per-token path recomputes the norm inside every router wave and reads
// the whole router matrix (E x H bf16, 4 MiB at E = 512, H = 4096) once per
// token.  For a batch the router is a dense [T x H] x [H x (E+1)] product (the
// extra column is the shared-expert gate), so it runs on the matrix cores:
//
//   k_norm_batch   one block per token: two-pass RMSNorm (sum of squares, then
//                  h = x * rsqrt(mean + eps) * gamma), written as
//                    - the fixed-point limb form the gate/up kernels read, and
//                    - h = hi + mid + lo, three bf16 values per entry (each the
//                      bf16 rounding of what the previous ones leave), so that
//                      a bf16 matrix product sees 24 significant bits of h.
//   k_router_mfma  v_mfma_f32_32x32x16_bf16 over 32 router rows x 32 tokens per
//                  wave tile; every 16-wide reduction step issues three
//                  products (lo, mid, hi) into one fp32 accumulator.  The
//                  router weights are bf16 already, so every product is exact
//                  and only the fp32 accumulation rounds, as in an fp32 GEMV.
//                  The waves of a block split the block's reduction range and
//                  are summed in LDS in a fixed order; KS = H / 512 blocks
//                  split H and leave KS partial logits, which the routing step
//                  adds in a fixed order (no atomics: deterministic).
//
// Steps computed: RMSNorm in two passes and the routing GEMV of the pages
// ("48GB内存运行397B模型：Flash-Moe的极端量化与SSD流式加载实践", section
// "Metal GPU管线：手写Kernel与FMA优化"; flash-moe README translation,
// "Pipeline mỗi lớp").
#include "moe_device.h"

namespace moe {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// k_norm_batch: a thread owns 16 consecutive entries, four threads a group of 64
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_norm_batch(FwdArgs a) {
    const int t = blockIdx.x, H = a.s.H;
    const int u = threadIdx.x;
    const bool live = u < H / 16;
    const int k0 = live ? 16 * u : 0;
    const float *x = a.x + (size_t)t * H + k0;
    float v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 q = *(const float4 *)(x + 4 * i);
        v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
    }
    const uint4 g0 = *(const uint4 *)(a.gamma + k0);
    const uint4 g1 = *(const uint4 *)(a.gamma + k0 + 8);
    // pass 1: sum of squares
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) ss = fmaf(v[i], v[i], ss);
    if (!live) ss = 0.0f;
    ss = lane_sum<64>(ss);
    __shared__ float s_ss[4];
    if ((threadIdx.x & 63) == 0) s_ss[threadIdx.x >> 6] = ss;
    __syncthreads();
    ss = (s_ss[0] + s_ss[1]) + (s_ss[2] + s_ss[3]);
    const float inv = 1.0f / sqrtf(ss / (float)H + a.s.eps);
    // pass 2: h
    const uint32_t gw[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    float h[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        h[2 * i] = v[2 * i] * inv * bf16_lo(gw[i]);
        h[2 * i + 1] = v[2 * i + 1] * inv * bf16_hi(gw[i]);
    }
    // three-way bf16 split in the matrix products' fragment order
    if (live) store_split_fragments(a.ws.hb, H, t, u, h);
    // limb form (entry k of a dword's 8 in nibble k): group max over 4 threads,
    // half-group sums over 2
    float m = 0.0f, sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        m = nan_max(m, fabsf(h[i]));
        sum += h[i];
    }
    sum += __shfl_xor(sum, 1, 64);
    m = nan_max(m, __shfl_xor(m, 1, 64));
    m = nan_max(m, __shfl_xor(m, 2, 64));
    uint32_t pk[kLimbs][2];
#pragma unroll
    for (int xl = 0; xl < kLimbs; ++xl) pk[xl][0] = pk[xl][1] = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        int l[kLimbs];
        limb_split(limb_value(h[i], m), l);
#pragma unroll
        for (int xl = 0; xl < kLimbs; ++xl) pk[xl][i / 8] |= (uint32_t)(l[xl] & 15) << (4 * (i % 8));
    }
    if (live) {
        uint32_t *hl = (uint32_t *)a.ws.hl + (size_t)t * kLimbs * (H / 8) + 2 * u;
#pragma unroll
        for (int xl = 0; xl < kLimbs; ++xl) *(uint2 *)(hl + (size_t)xl * (H / 8)) = make_uint2(pk[xl][0], pk[xl][1]);
        if ((u & 1) == 0) a.ws.hx[(size_t)t * (H / 32) + u / 2] = sum;
        if ((u & 3) == 0) a.ws.hs[(size_t)t * (H / 64) + u / 4] = limb_scale(m);
    }
}

// ---------------------------------------------------------------------------
// k_router_mfma: block (row tile of 32, k-split of 512 entries, token tile of
// 32) with W = min(8, H / 64) waves, each over 64 reduction entries (4 steps).
// Operand layouts of the 32x32x16 bf16 product: lane l holds row (or token)
// l % 32 and reduction entries 8 (l / 32) .. +7 of the step; result entry v of
// lane l is row 8 (v / 4) + 4 (l / 32) + v % 4, token l % 32.  A wave reads its
// 32 x 64 router tile as whole 128-byte row segments (8 lanes per row) and
// regroups it through LDS; the h fragments are stored in lane order already.
// ---------------------------------------------------------------------------
constexpr int kRouterSteps = 4;
constexpr int kRouterMaxWaves = 8;
constexpr int kTileStride = 9;  // 16-byte pieces per LDS tile row (8 + 1 of padding)

__global__ __launch_bounds__(64 * kRouterMaxWaves) void k_router_mfma(FwdArgs a) {
    const int H = a.s.H, E = a.s.E, T = a.T;
    const int W = (H / router_ksplit(H)) / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rt = blockIdx.x, ks = blockIdx.y, tt = blockIdx.z;
    const int kbase = (ks * W + wave) * 64;
    // router tile: load j covers rows 8j .. 8j+7 of the tile, 8 lanes per row
    uint4 ra[kRouterSteps];
#pragma unroll
    for (int j = 0; j < kRouterSteps; ++j) {
        const int r = rt * 32 + 8 * j + (lane >> 3);
        const uint16_t *row = (r < E) ? a.router + (size_t)r * H : a.sgate;  // row E: shared gate
        ra[j] = ld_stream16(row + kbase + 8 * (lane & 7));
        if (r > E) ra[j] = make_uint4(0u, 0u, 0u, 0u);
    }
    // h fragments of the 4 steps, 3 parts each
    const uint4 *hf = (const uint4 *)a.ws.hb + ((size_t)tt * (H / 16) + kbase / 16) * 3 * 64 + lane;
    uint4 hb[kRouterSteps][3];
#pragma unroll
    for (int i = 0; i < kRouterSteps; ++i)
#pragma unroll
        for (int p = 0; p < 3; ++p) hb[i][p] = hf[(i * 3 + p) * 64];
    const bool tlive = tt * 32 + (lane & 31) < T;
    if (!tlive) {
#pragma unroll
        for (int i = 0; i < kRouterSteps; ++i)
#pragma unroll
            for (int p = 0; p < 3; ++p) hb[i][p] = make_uint4(0u, 0u, 0u, 0u);
    }
    // regroup the router tile into fragments: step i of lane (r, kb) is piece
    // 2i + kb of row r
    __shared__ uint4 s_lds[kRouterMaxWaves * 32 * kTileStride];
    uint4 *tile = s_lds + wave * 32 * kTileStride;
#pragma unroll
    for (int j = 0; j < kRouterSteps; ++j) tile[(8 * j + (lane >> 3)) * kTileStride + (lane & 7)] = ra[j];
    __builtin_amdgcn_wave_barrier();
    uint4 af[kRouterSteps];
#pragma unroll
    for (int i = 0; i < kRouterSteps; ++i) af[i] = tile[(lane & 31) * kTileStride + 2 * i + (lane >> 5)];
    f32x16_t c = {};
#pragma unroll
    for (int i = 0; i < kRouterSteps; ++i) {
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, af[i]);
#pragma unroll
        for (int p = 2; p >= 0; --p)
            c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8_t, hb[i][p]), c, 0, 0, 0);
    }
    // sum of the block's waves in a fixed order (the tiles are dead: reuse LDS)
    __syncthreads();
    float *s_c = (float *)s_lds;  // [W][16][64]
#pragma unroll
    for (int v = 0; v < 16; ++v) s_c[(wave * 16 + v) * 64 + lane] = c[v];
    __syncthreads();
    for (int idx = threadIdx.x; idx < 1024; idx += 64 * W) {
        const int v = idx >> 6, l = idx & 63;
        float sum = s_c[v * 64 + l];
        for (int w = 1; w < W; ++w) sum += s_c[(w * 16 + v) * 64 + l];
        const int row = rt * 32 + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
        const int tok = tt * 32 + (l & 31);
        if (row <= E && tok < T) a.ws.zp[((size_t)ks * T + tok) * (E + 1) + row] = sum;
    }
}

}  // namespace

hipError_t launch_batch_router(const FwdArgs &a, int stage, hipStream_t st) {
    if (stage == 0) {
        hipLaunchKernelGGL(k_norm_batch, dim3((unsigned)a.T), dim3(256), 0, st, a);
    } else {
        const int H = a.s.H;
        const int W = (H / router_ksplit(H)) / 64;
        const dim3 grid((unsigned)((a.s.E + 1 + 31) / 32), (unsigned)router_ksplit(H), (unsigned)token_tiles(a.T));
        hipLaunchKernelGGL(k_router_mfma, grid, dim3((unsigned)(64 * W)), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace moe

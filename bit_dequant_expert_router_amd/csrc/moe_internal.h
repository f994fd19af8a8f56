// moe_internal.h -- library-internal declarations shared by the ABI and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "moe_layout.h"

namespace moe {

constexpr size_t kAlign = 256;
constexpr size_t kCtrlBytes = 8192;  // 2 launches x 2 counters x kClaimGroups x 256 bytes

MOE_HD size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

// Workspace of one forward call, carved from the caller's buffer.
struct Workspace {
    uint32_t *ctrl;  // control block, kCtrlBytes, zeroed by moe_workspace_init: the streaming
                     // launches' run and exit counters (each launch leaves them at zero)
    float *h;        // [T][H]   normalised tokens
    float *z;        // [T][logit_stride(E)] router logits
    float *gs;       // [T]      shared-gate logits
    int32_t *sel;    // [T][K]   selected experts
    float *coef;     // [T][K+1] combine coefficients (renormalised weights, sigmoid(gs))
    float *act;      // [T][K+1][F] SwiGLU activations of the selected experts and the shared one
    int8_t *hl;      // [T][kLimbs][H/8] dwords: base-16 limbs of the fixed-point normalised tokens
    float *hs;       // [T][H/64]  group scales (powers of two) of the limbs
    float *hx;       // [T][H/32]  sums of h over each half group
    // batched (grouped-by-expert) path
    int32_t *grp;    // [4 + 3 * (G + 1) + T*K]: n_touched, then expert, first slot and count of
                     // each touched expert, then the assignments t*K+k sorted by (expert, token)
    float *ys;       // [T][K+1][H] per-slot expert outputs
    int8_t *al;      // [T][K+1][kLimbs][F/8] dwords: limbs of the activations, in the down codes' order
    float *as;       // [T][K+1][F/64] group scales of those limbs
    float *ax;       // [T][K+1][F/32] sums of the activations over each half group
    uint16_t *hb;    // h = hi + mid + lo in bf16, the router GEMM's operand, in fragment order:
                     // [ceil(T/32)][H/16][3][64 lanes][8] (see k_norm_batch)
    float *zp;       // [KS][T][E+1] partial router logits (column E: shared gate), KS = router_ksplit(H)
    float *sp;       // [kMaxMfmaKsplit][2][T][F] partial gate and up sums of the shared expert's
                     // matrix-core units (one per reduction chunk)
    uint16_t *ab;    // the shared expert's activations a = hi + mid + lo in bf16, fragment order
                     // [ceil(T/32)][F/16][3][64 lanes][8] (the shared down product's operand)
    int32_t *sched;  // passes of the two streaming launches (gate/up, down), each
                     // sched_launch_ints(T, K) ints: head, then kPassRecord ints per pass
};

// row stride (floats) of the router logits in the workspace: a multiple of 16,
// so that a lane reads its 8 or 16 logits with 16-byte loads (the padding is
// never read as a logit)
MOE_HD int logit_stride(int E) { return (E + 15) & ~15; }

// k-splits of the batched router GEMM: 512 reduction entries per block when H >= 512
constexpr int kMaxKsplit = kMaxDim / 512;
MOE_HD int router_ksplit(int H) { return H >= 512 ? H / 512 : 1; }
MOE_HD int token_tiles(int T) { return (T + 31) / 32; }

struct Shape {
    int H, F, E, K, bits;
    float eps;
};

// Work of the grouped path's streaming kernels.  A "pass" applies one expert's
// rows to up to tp (<= kMaxPassVectors) of its vectors; every pass is cut into
// nbs block-steps (4 waves x RPW row slots) and those into runs of up to
// `run_items` block-steps.  A persistent grid of nb blocks (a multiple of
// kClaimGroups) takes the runs: block b runs b first, then claims runs
// nb + G c + b % G, c = 0, 1, ... from the counter of its group in the control
// block (claimed one run ahead, so the claim's latency is hidden).  The
// grouping kernel writes, per launch, a head ([0]
// passes, [1] runs) and one record per pass: expert (E: the shared one),
// vector count, then the vectors' output indices t * (K+1) + slot.
constexpr int kMaxPassVectors = 16;
constexpr int kPassRecord = 2 + kMaxPassVectors;
MOE_HD int sched_max_passes(int T, int K) { return T * (K + 1); }
MOE_HD int sched_launch_ints(int T, int K) { return 4 + kPassRecord * sched_max_passes(T, K); }
struct StreamPlan {
    int tp;         // vectors staged per pass
    int nbs;        // block-steps per pass
    int run_items;  // block-steps per run
    int rpp;        // runs per pass, ceil(nbs / run_items)
    int nb;         // blocks of the persistent grid
    int n_mfma;     // matrix-core units of the shared expert (runs 0 .. n_mfma-1; then it has no passes)
    int mfma_ks;    // reduction chunks per unit row block and token tile (> 1: partial sums in sp)
};
constexpr int kMaxMfmaKsplit = 8;
// Run claims go through kClaimGroups counters (block b uses counter b % G and
// claims the runs r = b mod G), so that no single address takes every claim;
// each counter sits in its own 256-byte line of the control block, after the
// claim counters of launch 0 and 1 come the exit counters.
constexpr int kClaimGroups = 8;
constexpr int kCtrlStride = 64;  // words between counters
MOE_HD int ctrl_run_counter(int launch, int g) { return ((launch * 2 + 0) * kClaimGroups + g) * kCtrlStride; }
MOE_HD int ctrl_exit_counter(int launch, int g) { return ((launch * 2 + 1) * kClaimGroups + g) * kCtrlStride; }

// touched-expert bound of a batch and the integers of the grouping table
inline int touched_bound(const Shape &s, int T) { return (T * s.K < s.E) ? T * s.K : s.E; }
inline size_t grouped_ints(const Shape &s, int T) {
    return 4 + 3 * ((size_t)touched_bound(s, T) + 1) + (size_t)T * s.K;
}

inline size_t workspace_bytes(const Shape &s, int T) {
    size_t b = kCtrlBytes;
    b += align_up((size_t)T * s.H * 4);
    b += align_up((size_t)T * logit_stride(s.E) * 4);
    b += align_up((size_t)T * 4);
    b += align_up((size_t)T * s.K * 4);
    b += align_up((size_t)T * (s.K + 1) * 4);
    b += align_up((size_t)T * (s.K + 1) * s.F * 4);
    b += align_up((size_t)T * 4 * s.H);  // kLimbs (<= 8) limbs x H/2 bytes fit in 4 H
    b += align_up((size_t)T * (s.H / 64) * 4);
    b += align_up((size_t)T * (s.H / 32) * 4);
    b += align_up(grouped_ints(s, T) * 4);
    b += align_up((size_t)T * (s.K + 1) * s.H * 4);
    b += align_up((size_t)T * (s.K + 1) * 4 * s.F);  // kLimbs (<= 8) limbs x F/2 bytes fit in 4 F
    b += align_up((size_t)T * (s.K + 1) * (s.F / 64) * 4);
    b += align_up((size_t)T * (s.K + 1) * (s.F / 32) * 4);
    b += align_up((size_t)token_tiles(T) * 32 * 3 * s.H * 2);
    b += align_up((size_t)router_ksplit(s.H) * T * (s.E + 1) * 4);
    b += align_up((size_t)kMaxMfmaKsplit * 2 * T * s.F * 4);
    b += align_up((size_t)token_tiles(T) * 32 * 3 * s.F * 2);
    b += align_up((size_t)2 * sched_launch_ints(T, s.K) * 4);
    return b;
}

inline Workspace carve_workspace(void *base, const Shape &s, int T) {
    char *p = (char *)base;
    Workspace w;
    w.ctrl = (uint32_t *)p;
    p += kCtrlBytes;
    w.h = (float *)p;
    p += align_up((size_t)T * s.H * 4);
    w.z = (float *)p;
    p += align_up((size_t)T * logit_stride(s.E) * 4);
    w.gs = (float *)p;
    p += align_up((size_t)T * 4);
    w.sel = (int32_t *)p;
    p += align_up((size_t)T * s.K * 4);
    w.coef = (float *)p;
    p += align_up((size_t)T * (s.K + 1) * 4);
    w.act = (float *)p;
    p += align_up((size_t)T * (s.K + 1) * s.F * 4);
    w.hl = (int8_t *)p;
    p += align_up((size_t)T * 4 * s.H);
    w.hs = (float *)p;
    p += align_up((size_t)T * (s.H / 64) * 4);
    w.hx = (float *)p;
    p += align_up((size_t)T * (s.H / 32) * 4);
    w.grp = (int32_t *)p;
    p += align_up(grouped_ints(s, T) * 4);
    w.ys = (float *)p;
    p += align_up((size_t)T * (s.K + 1) * s.H * 4);
    w.al = (int8_t *)p;
    p += align_up((size_t)T * (s.K + 1) * 4 * s.F);
    w.as = (float *)p;
    p += align_up((size_t)T * (s.K + 1) * (s.F / 64) * 4);
    w.ax = (float *)p;
    p += align_up((size_t)T * (s.K + 1) * (s.F / 32) * 4);
    w.hb = (uint16_t *)p;
    p += align_up((size_t)token_tiles(T) * 32 * 3 * s.H * 2);
    w.zp = (float *)p;
    p += align_up((size_t)router_ksplit(s.H) * T * (s.E + 1) * 4);
    w.sp = (float *)p;
    p += align_up((size_t)kMaxMfmaKsplit * 2 * T * s.F * 4);
    w.ab = (uint16_t *)p;
    p += align_up((size_t)token_tiles(T) * 32 * 3 * s.F * 2);
    w.sched = (int32_t *)p;
    return w;
}

// Everything a forward launch needs (passed by value as a kernel argument).
struct FwdArgs {
    Shape s;
    ExpertLayout L;
    const uint16_t *gamma;
    const uint16_t *router;
    const uint16_t *sgate;
    const uint8_t *experts;
    const uint8_t *shared;
    const float *x;
    float *y;
    int T;
    int32_t *route_idx;
    float *route_w;
    Workspace ws;
    // k_route only: where the selection also goes (host memory mapped into the
    // device's address space), or null.  Entry t * K + k is one 8-byte word,
    // sel_tag in the high half and the expert in the low half, so that the
    // host can tell a landed entry from a stale one without relying on the
    // order in which separate writes reach host memory.
    uint64_t *sel_host = nullptr;
    uint32_t sel_tag = 0;
};

// Slots of one call's selected experts, [T][K] with T*K <= kSlotArgs, passed
// by value to the expert kernels when the experts are read from cache slots
// (tiered residency); the kernels of the resident path take an empty one.
constexpr int kSlotArgs = 64;
struct SlotArgs {
    int32_t s[kSlotArgs];
};
struct NoSlotArgs {};
template <bool TIER>
using SlotParam = typename std::conditional<TIER, SlotArgs, NoSlotArgs>::type;

constexpr int kForwardStages = 3;
// Batches of at least kGroupMinAssign assignments (tokens x top-K) and at most
// kGroupMaxAssign take the grouped-by-expert path; smaller batches run the
// per-token kernels, one row of blocks per token.  On the 4096/1024/512-expert
// shape the per-token kernels are ahead up to 64 assignments with top-4 (by 1%
// there) and 70 with top-10 (the grouped path's seven launches and its grouping
// cost more than re-reading the few experts two tokens share), the grouped path
// from 80 with either (by 5% and 3%).
constexpr int kGroupMinAssign = 72;
constexpr int kGroupMaxAssign = 4096;
constexpr int kGroupedStages = 7;
inline bool uses_grouped(const Shape &s, int T) {
    const long a = (long)T * s.K;
    return a >= kGroupMinAssign && a <= kGroupMaxAssign;
}
hipError_t launch_grouped(const FwdArgs &a, hipStream_t stream);
hipError_t launch_grouped_stage(const FwdArgs &a, int stage, hipStream_t stream);
// batched RMSNorm (stage 0) and router GEMM (stage 1) of the grouped path
hipError_t launch_batch_router(const FwdArgs &a, int stage, hipStream_t stream);
hipError_t launch_forward(const FwdArgs &a, hipStream_t stream);
hipError_t launch_forward_stage(const FwdArgs &a, int stage, hipStream_t stream);
// the per-token path with the selected experts read from cache slots: stage 0
// as above, then the routing alone (launch_forward_route), then, once the slots
// are filled, stage 1 without routing and stage 2, both addressing the experts
// as a.experts + slot * bytes (launch_forward_slots, T*K <= kSlotArgs)
hipError_t launch_forward_route(const FwdArgs &a, hipStream_t stream);
// copies n whole packed experts, expert[i] of src (host memory mapped into the
// device's address space) into slot[i] of dst, with one launch
struct FetchArgs {
    const uint8_t *src;
    uint8_t *dst;
    uint64_t bytes;  // of one expert, a multiple of 16
    int32_t n;
    int32_t expert[kSlotArgs];
    int32_t slot[kSlotArgs];
};
hipError_t launch_fetch(const FetchArgs &f, hipStream_t stream);
hipError_t launch_forward_slots(const FwdArgs &a, const SlotArgs &slots, hipStream_t stream);

struct PackArgs {
    ExpertLayout L;
    const uint8_t *codes[3];
    const uint16_t *scale[3];
    const uint16_t *bias[3];
    uint8_t *dst;
};
hipError_t launch_pack(const PackArgs &a, hipStream_t stream);

struct GenArgs {
    ExpertLayout L;
    uint64_t seed;
    uint32_t layer;
    int first_expert;  // expert index of dst's first expert (E = the shared expert)
    int count;         // number of consecutive experts to write
    uint8_t *dst;
};
hipError_t launch_generate(const GenArgs &a, hipStream_t stream);

hipError_t launch_clear_ctrl(uint32_t *ctrl, hipStream_t stream);

}  // namespace moe

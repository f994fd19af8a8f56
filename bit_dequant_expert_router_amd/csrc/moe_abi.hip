// moe_abi.hip -- the extern "C" boundary declared in include/moe.h.
//
// Every argument is checked on the host before anything is enqueued; the
// checks make no HIP call, so they behave the same with or without a GPU.
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/moe.h"
#include "moe_internal.h"
#include "moe_tier.h"

namespace {

using namespace moe;

thread_local hipError_t g_last_hip = hipSuccess;

int hip_status(hipError_t e) {
    g_last_hip = e;
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }
bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_dims_impl(const moe_dims_t *d) {
    if (!d) return MOE_ERR_INVALID_ARG;
    if (d->hidden <= 0 || d->ffn <= 0 || d->n_experts <= 0 || d->top_k <= 0) return MOE_ERR_INVALID_ARG;
    if (d->bits <= 0 || d->bits > 8) return MOE_ERR_INVALID_ARG;
    if (d->group_size <= 0) return MOE_ERR_INVALID_ARG;
    if (!(d->rms_eps >= 0.0f) || !isfinite(d->rms_eps)) return MOE_ERR_INVALID_ARG;
    if (d->hidden % d->group_size != 0 || d->ffn % d->group_size != 0) return MOE_ERR_INVALID_ARG;
    if (d->top_k > d->n_experts) return MOE_ERR_INVALID_ARG;
    if (d->bits != 2 && d->bits != 4) return MOE_ERR_UNSUPPORTED;
    if (d->group_size != kGroup) return MOE_ERR_UNSUPPORTED;
    if (d->n_experts > kMaxExperts || d->top_k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
    if (!is_pow2(d->hidden) || d->hidden < kMinDim || d->hidden > kMaxDim) return MOE_ERR_UNSUPPORTED;
    if (!is_pow2(d->ffn) || d->ffn < kMinDim || d->ffn > kMaxDim) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

Shape shape_of(const moe_dims_t *d) {
    Shape s;
    s.H = d->hidden;
    s.F = d->ffn;
    s.E = d->n_experts;
    s.K = d->top_k;
    s.bits = d->bits;
    s.eps = d->rms_eps;
    return s;
}

int check_layer(const moe_layer_t *l) {
    if (!l || !l->norm_weight || !l->router_weight || !l->shared_gate || !l->experts || !l->shared_expert)
        return MOE_ERR_INVALID_ARG;
    if (!aligned(l->norm_weight, 16) || !aligned(l->router_weight, 16) || !aligned(l->shared_gate, 16) ||
        !aligned(l->experts, kAlign) || !aligned(l->shared_expert, kAlign))
        return MOE_ERR_ALIGNMENT;
    return MOE_OK;
}

size_t workspace_bytes_checked(const moe_dims_t *dims, int32_t n_tokens) {
    if (check_dims_impl(dims) != MOE_OK || n_tokens < 1) return 0;
    return workspace_bytes(shape_of(dims), n_tokens);
}

// batches of kGroupMinAssign to kGroupMaxAssign assignments are grouped by expert
hipError_t launch_layer(const FwdArgs &a, hipStream_t stream) {
    if (uses_grouped(a.s, a.T)) return launch_grouped(a, stream);
    return launch_forward(a, stream);
}

bool overlap_not_equal(const void *a, const void *b, size_t bytes) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    if (x == y) return false;
    return x < y + bytes && y < x + bytes;
}

// the checks of a forward call that do not concern its workspace
int check_forward_io(const moe_dims_t *dims, const float *x, float *y, int32_t n_tokens, int32_t *route_idx,
                     float *route_w) {
    int rc = check_dims_impl(dims);
    if (rc != MOE_OK) return rc;
    if (n_tokens < 1 || n_tokens > 65535) return MOE_ERR_INVALID_ARG;
    if (!x || !y) return MOE_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(y, 16)) return MOE_ERR_ALIGNMENT;
    if ((route_idx && !aligned(route_idx, 4)) || (route_w && !aligned(route_w, 4))) return MOE_ERR_ALIGNMENT;
    if (overlap_not_equal(x, y, (size_t)n_tokens * dims->hidden * sizeof(float))) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

int check_forward_common(const moe_dims_t *dims, const float *x, float *y, int32_t n_tokens,
                         int32_t *route_idx, float *route_w, void *workspace, size_t workspace_bytes) {
    const int rc = check_forward_io(dims, x, y, n_tokens, route_idx, route_w);
    if (rc != MOE_OK) return rc;
    if (!workspace) return MOE_ERR_INVALID_ARG;
    if (!aligned(workspace, kAlign)) return MOE_ERR_ALIGNMENT;
    if (workspace_bytes < workspace_bytes_checked(dims, n_tokens)) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

// ---------------------------------------------------------------------------
// the library's own workspace, for moe_layer_forward_noalloc: one fixed array
// per GPU (each device that loads the library holds its own copy until the
// process ends).  Its name is a host-side stand-in, not a device address: host
// code uses only the address that hipGetSymbolAddress returns on each device,
// looked up once per device and kept in g_scratch_ptr.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 256;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices];

// the array's address on the current device (first call per device: looked up)
hipError_t scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p || !aligned(p, kAlign)) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// tiered expert residency: the state the caller holds in pinned host memory,
// a header followed by int32 arrays (the LRU lists and key map), then the
// 8-byte landing area of one call's selection; pointers into it are derived
// from its base on every call
// ---------------------------------------------------------------------------
constexpr uint64_t kTierMagic = 0x7265695465754d31ull;

struct TierState {
    uint64_t magic;
    moe_dims_t dims;
    int32_t n_layers, n_slots, max_tokens, pad;
    uint64_t expert_bytes;
    uint8_t *slots;      // device: n_slots packed experts
    uint64_t *route_dev;  // the landing area as the device addresses it (set by the first call)
    moe_tier_stats_t stats;
    int32_t head, tail;  // of the LRU list
};

struct TierView {
    TierState *st;
    SlotLru lru;
    uint64_t *route;  // [max_tokens][K] host landing area of the selected experts (tag << 32 | expert)
};

constexpr size_t tier_header_bytes() { return (sizeof(TierState) + 255) / 256 * 256; }

size_t tier_ints(const moe_dims_t *d, int32_t n_layers, int32_t n_slots, int32_t max_tokens) {
    // the LRU (padded to 8 bytes), then the selection of one call in 8-byte entries
    return (SlotLru::ints(n_slots, n_layers * d->n_experts) + 1) / 2 * 2 + 2 * (size_t)max_tokens * d->top_k;
}

int check_tier_args(const moe_dims_t *dims, int32_t n_layers, int32_t n_slots, int32_t max_tokens) {
    const int rc = check_dims_impl(dims);
    if (rc != MOE_OK) return rc;
    if (n_layers < 1 || max_tokens < 1 || max_tokens > 65535) return MOE_ERR_INVALID_ARG;
    if ((int64_t)n_layers * dims->n_experts >= ((int64_t)1 << 31)) return MOE_ERR_INVALID_ARG;
    if ((int64_t)n_slots < (int64_t)max_tokens * dims->top_k) return MOE_ERR_INVALID_ARG;
    if (max_tokens * dims->top_k > kSlotArgs) return MOE_ERR_UNSUPPORTED;  // the slots travel as kernel arguments
    return MOE_OK;
}

// the view of a state (the list is read back from the header; store_lru writes it)
TierView tier_view(void *state) {
    TierView v;
    v.st = (TierState *)state;
    int32_t *ints = (int32_t *)((uint8_t *)state + tier_header_bytes());
    const int32_t ns = v.st->n_slots, nk = v.st->n_layers * v.st->dims.n_experts;
    v.lru.n_slots = ns;
    v.lru.n_keys = nk;
    v.lru.key = ints;
    v.lru.prev = ints + ns;
    v.lru.next = ints + 2 * (size_t)ns;
    v.lru.slot_of = ints + 3 * (size_t)ns;
    v.lru.head = v.st->head;
    v.lru.tail = v.st->tail;
    v.route = (uint64_t *)(ints + (SlotLru::ints(ns, nk) + 1) / 2 * 2);
    return v;
}

void store_lru(TierView &v) {
    v.st->head = v.lru.head;
    v.st->tail = v.lru.tail;
}

const TierState *tier_header(const void *state) {
    if (!state || !aligned(state, 8)) return nullptr;
    const TierState *st = (const TierState *)state;
    return st->magic == kTierMagic ? st : nullptr;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

int moe_check_dims(const moe_dims_t *dims) { return check_dims_impl(dims); }

size_t moe_expert_bytes(const moe_dims_t *dims) {
    if (check_dims_impl(dims) != MOE_OK) return 0;
    return make_layout(dims->hidden, dims->ffn, dims->bits).bytes;
}

size_t moe_workspace_bytes(const moe_dims_t *dims, int32_t n_tokens) {
    return workspace_bytes_checked(dims, n_tokens);
}

int moe_workspace_init(void *workspace, size_t workspace_bytes, void *stream) {
    if (!workspace) return MOE_ERR_INVALID_ARG;
    if (workspace_bytes < kCtrlBytes) return MOE_ERR_WORKSPACE;
    if (!aligned(workspace, kAlign)) return MOE_ERR_ALIGNMENT;
    return hip_status(launch_clear_ctrl((uint32_t *)workspace, (hipStream_t)stream));
}

int moe_pack_expert(const moe_dims_t *dims, const uint8_t *const codes[3], const uint16_t *const scale[3],
                    const uint16_t *const bias[3], void *dst, void *stream) {
    int rc = check_dims_impl(dims);
    if (rc != MOE_OK) return rc;
    if (!codes || !scale || !bias || !dst) return MOE_ERR_INVALID_ARG;
    PackArgs a;
    for (int m = 0; m < 3; ++m) {
        if (!codes[m] || !scale[m] || !bias[m]) return MOE_ERR_INVALID_ARG;
        if (!aligned(scale[m], 2) || !aligned(bias[m], 2)) return MOE_ERR_ALIGNMENT;
        a.codes[m] = codes[m];
        a.scale[m] = scale[m];
        a.bias[m] = bias[m];
    }
    if (!aligned(dst, kAlign)) return MOE_ERR_ALIGNMENT;
    a.L = make_layout(dims->hidden, dims->ffn, dims->bits);
    a.dst = (uint8_t *)dst;
    return hip_status(launch_pack(a, (hipStream_t)stream));
}

int moe_generate_layer(const moe_dims_t *dims, uint64_t seed, uint32_t layer, void *experts,
                       void *shared_expert, void *stream) {
    int rc = check_dims_impl(dims);
    if (rc != MOE_OK) return rc;
    if (!experts && !shared_expert) return MOE_ERR_INVALID_ARG;
    if ((experts && !aligned(experts, kAlign)) || (shared_expert && !aligned(shared_expert, kAlign)))
        return MOE_ERR_ALIGNMENT;
    GenArgs a;
    a.L = make_layout(dims->hidden, dims->ffn, dims->bits);
    a.seed = seed;
    a.layer = layer;
    if (experts) {
        a.first_expert = 0;
        a.count = dims->n_experts;
        a.dst = (uint8_t *)experts;
        if (hip_status(launch_generate(a, (hipStream_t)stream)) != MOE_OK) return MOE_ERR_HIP;
    }
    if (shared_expert) {
        a.first_expert = dims->n_experts;
        a.count = 1;
        a.dst = (uint8_t *)shared_expert;
        if (hip_status(launch_generate(a, (hipStream_t)stream)) != MOE_OK) return MOE_ERR_HIP;
    }
    return MOE_OK;
}

static FwdArgs make_fwd(const moe_dims_t *dims, const moe_layer_t *layer, const float *x, float *y, int T,
                        int32_t *route_idx, float *route_w, void *workspace) {
    FwdArgs a;
    a.s = shape_of(dims);
    a.L = make_layout(dims->hidden, dims->ffn, dims->bits);
    a.gamma = layer->norm_weight;
    a.router = layer->router_weight;
    a.sgate = layer->shared_gate;
    a.experts = (const uint8_t *)layer->experts;
    a.shared = (const uint8_t *)layer->shared_expert;
    a.x = x;
    a.y = y;
    a.T = T;
    a.route_idx = route_idx;
    a.route_w = route_w;
    a.ws = carve_workspace(workspace, a.s, T);
    return a;
}

int moe_layer_forward(const moe_dims_t *dims, const moe_layer_t *layer, const float *x, float *y,
                      int32_t n_tokens, int32_t *route_idx, float *route_w, void *workspace,
                      size_t workspace_bytes, void *stream) {
    int rc = check_forward_common(dims, x, y, n_tokens, route_idx, route_w, workspace, workspace_bytes);
    if (rc != MOE_OK) return rc;
    rc = check_layer(layer);
    if (rc != MOE_OK) return rc;
    const FwdArgs a = make_fwd(dims, layer, x, y, n_tokens, route_idx, route_w, workspace);
    return hip_status(launch_layer(a, (hipStream_t)stream));
}

int moe_layer_forward_noalloc(const moe_dims_t *dims, const moe_layer_t *layer, const float *x, float *y,
                              int32_t n_tokens, int32_t *route_idx, float *route_w, void *stream) {
    int rc = check_forward_io(dims, x, y, n_tokens, route_idx, route_w);
    if (rc != MOE_OK) return rc;
    rc = check_layer(layer);
    if (rc != MOE_OK) return rc;
    if (workspace_bytes_checked(dims, n_tokens) > kScratchBytes) return MOE_ERR_WORKSPACE;
    void *ws = nullptr;
    if (hip_status(scratch_address(&ws)) != MOE_OK) return MOE_ERR_HIP;
    const hipStream_t hs = (hipStream_t)stream;
    const FwdArgs a = make_fwd(dims, layer, x, y, n_tokens, route_idx, route_w, ws);
    // the grouped kernels claim work through counters in the control block,
    // which must start at zero: cleared by a kernel (no memset node under capture)
    if (uses_grouped(a.s, n_tokens) && hip_status(launch_clear_ctrl(a.ws.ctrl, hs)) != MOE_OK) return MOE_ERR_HIP;
    return hip_status(launch_layer(a, hs));
}

int moe_layer_forward_stage(const moe_dims_t *dims, const moe_layer_t *layer, const float *x, float *y,
                            int32_t n_tokens, int32_t *route_idx, float *route_w, void *workspace,
                            size_t workspace_bytes, int32_t stage, void *stream) {
    int rc = check_forward_common(dims, x, y, n_tokens, route_idx, route_w, workspace, workspace_bytes);
    if (rc != MOE_OK) return rc;
    rc = check_layer(layer);
    if (rc != MOE_OK) return rc;
    const bool grouped = uses_grouped(shape_of(dims), n_tokens);
    if (stage < 0 || stage >= (grouped ? kGroupedStages : kForwardStages)) return MOE_ERR_INVALID_ARG;
    const FwdArgs a = make_fwd(dims, layer, x, y, n_tokens, route_idx, route_w, workspace);
    if (grouped) return hip_status(launch_grouped_stage(a, stage, (hipStream_t)stream));
    return hip_status(launch_forward_stage(a, stage, (hipStream_t)stream));
}

int moe_forward_stage_count(const moe_dims_t *dims, int32_t n_tokens) {
    const int rc = check_dims_impl(dims);
    if (rc != MOE_OK) return rc;
    if (n_tokens < 1 || n_tokens > 65535) return MOE_ERR_INVALID_ARG;
    return uses_grouped(shape_of(dims), n_tokens) ? kGroupedStages : kForwardStages;
}

int moe_stack_forward(const moe_dims_t *dims, const moe_layer_t *layers, int32_t n_layers, const float *x,
                      float *y, int32_t n_tokens, int32_t *route_idx, float *route_w, void *workspace,
                      size_t workspace_bytes, void *stream) {
    int rc = check_forward_common(dims, x, y, n_tokens, route_idx, route_w, workspace, workspace_bytes);
    if (rc != MOE_OK) return rc;
    if (!layers || n_layers < 1) return MOE_ERR_INVALID_ARG;
    for (int l = 0; l < n_layers; ++l) {
        rc = check_layer(&layers[l]);
        if (rc != MOE_OK) return rc;
    }
    const size_t per_layer = (size_t)n_tokens * dims->top_k;
    for (int l = 0; l < n_layers; ++l) {
        const FwdArgs a = make_fwd(dims, &layers[l], l == 0 ? x : y, y, n_tokens,
                                   route_idx ? route_idx + l * per_layer : nullptr,
                                   route_w ? route_w + l * per_layer : nullptr, workspace);
        if (hip_status(launch_layer(a, (hipStream_t)stream)) != MOE_OK) return MOE_ERR_HIP;
    }
    return MOE_OK;
}

size_t moe_tier_state_bytes(const moe_dims_t *dims, int32_t n_layers, int32_t n_slots, int32_t max_tokens) {
    if (check_tier_args(dims, n_layers, n_slots, max_tokens) != MOE_OK) return 0;
    return tier_header_bytes() + tier_ints(dims, n_layers, n_slots, max_tokens) * sizeof(int32_t);
}

size_t moe_tier_device_bytes(const moe_dims_t *dims, int32_t n_slots, int32_t max_tokens) {
    if (check_tier_args(dims, 1, n_slots, max_tokens) != MOE_OK) return 0;
    const size_t eb = make_layout(dims->hidden, dims->ffn, dims->bits).bytes;
    return (size_t)n_slots * eb;
}

int moe_tier_init(const moe_dims_t *dims, int32_t n_layers, int32_t n_slots, int32_t max_tokens, void *state,
                  size_t state_bytes, void *device, size_t device_bytes) {
    const int rc = check_tier_args(dims, n_layers, n_slots, max_tokens);
    if (rc != MOE_OK) return rc;
    if (!state || !device) return MOE_ERR_INVALID_ARG;
    if (!aligned(state, 8) || !aligned(device, kAlign)) return MOE_ERR_ALIGNMENT;
    if (state_bytes < moe_tier_state_bytes(dims, n_layers, n_slots, max_tokens)) return MOE_ERR_WORKSPACE;
    if (device_bytes < moe_tier_device_bytes(dims, n_slots, max_tokens)) return MOE_ERR_WORKSPACE;
    TierState *st = (TierState *)state;
    memset(st, 0, sizeof(TierState));
    st->dims = *dims;
    st->n_layers = n_layers;
    st->n_slots = n_slots;
    st->max_tokens = max_tokens;
    st->expert_bytes = make_layout(dims->hidden, dims->ffn, dims->bits).bytes;
    st->slots = (uint8_t *)device;
    st->route_dev = nullptr;
    TierView v = tier_view(state);
    v.lru.init(n_slots, n_layers * dims->n_experts, v.lru.key);
    store_lru(v);
    st->magic = kTierMagic;
    return MOE_OK;
}

int moe_tier_layer_forward(void *state, int32_t layer_index, const moe_layer_t *layer, const float *x,
                           float *y, int32_t n_tokens, int32_t *route_idx, float *route_w, void *workspace,
                           size_t workspace_bytes, void *stream) {
    if (!tier_header(state)) return MOE_ERR_INVALID_ARG;
    TierView v = tier_view(state);
    TierState *st = v.st;
    const moe_dims_t *dims = &st->dims;
    int rc = check_forward_common(dims, x, y, n_tokens, route_idx, route_w, workspace, workspace_bytes);
    if (rc != MOE_OK) return rc;
    if (n_tokens > st->max_tokens || layer_index < 0 || layer_index >= st->n_layers) return MOE_ERR_INVALID_ARG;
    rc = check_layer(layer);
    if (rc != MOE_OK) return rc;
    const hipStream_t hs = (hipStream_t)stream;
    FwdArgs a = make_fwd(dims, layer, x, y, n_tokens, route_idx, route_w, workspace);
    const int K = dims->top_k, E = dims->n_experts, n = n_tokens * K;
    // 1. norm, router and routing; the routing kernel also writes the selection
    // into the state (pinned host memory, mapped into the device's address space)
    if (!st->route_dev) {
        void *p = nullptr;
        if (hipHostGetDevicePointer(&p, v.route, 0) != hipSuccess || !p) return MOE_ERR_INVALID_ARG;  // not pinned
        st->route_dev = (uint64_t *)p;
    }
    // every entry carries a tag, odd and different from call to call, in its
    // high half; the entries are cleared before the launch
    a.sel_host = st->route_dev;
    a.sel_tag = (uint32_t)(st->stats.calls + 1) * 2u + 1u;
    for (int i = 0; i < n; ++i) __atomic_store_n(&v.route[i], (uint64_t)0, __ATOMIC_RELAXED);
    if (hip_status(launch_forward_route(a, hs)) != MOE_OK) return MOE_ERR_HIP;
    // 2. wait for it by polling the entries: the thread sees the selection as
    // soon as it lands, where a stream synchronisation would add the runtime's
    // completion signal and the thread's wake-up to every layer.  An entry is
    // taken only once it holds this call's tag, whatever order the writes
    // reach host memory in.  An entry that never lands (a failed launch) ends
    // the spin after ~1e8 polls: the stream is then synchronised, which
    // reports the error.
    {
        long spins = 0;
        for (int i = 0; i < n; ++i) {
            while ((uint32_t)(__atomic_load_n(&v.route[i], __ATOMIC_ACQUIRE) >> 32) != a.sel_tag) {
                if (++spins > 100000000L) {
                    if (hip_status(hipStreamSynchronize(hs)) != MOE_OK) return MOE_ERR_HIP;
                    if ((uint32_t)(__atomic_load_n(&v.route[i], __ATOMIC_ACQUIRE) >> 32) != a.sel_tag)
                        return hip_status(hipErrorUnknown);
                }
            }
        }
    }
    // 3. lookups in token order, then rank order; a miss takes a slot and is
    // listed for copying
    const uint8_t *host = (const uint8_t *)layer->experts;
    const size_t eb = st->expert_bytes;
    SlotArgs sl;
    FetchArgs fa;
    fa.n = 0;
    fa.dst = st->slots;
    fa.bytes = eb;
    for (int i = 0; i < n; ++i) {
        const int32_t e = (int32_t)(uint32_t)__atomic_load_n(&v.route[i], __ATOMIC_RELAXED);
        if (e < 0 || e >= E) return hip_status(hipErrorUnknown);  // cannot happen: routing selects valid experts
        bool hit;
        const int32_t slot = v.lru.acquire(layer_index * E + e, &hit);
        store_lru(v);
        sl.s[i] = slot;
        st->stats.lookups += 1;
        if (hit) {
            st->stats.hits += 1;
            continue;
        }
        st->stats.misses += 1;
        fa.expert[fa.n] = e;
        fa.slot[fa.n] = slot;
        fa.n += 1;
        st->stats.bytes_copied += eb;
    }
    // the misses' copies: one kernel reading the host store over the link
    // (56.9 GB/s per miss, against 52.9 for one DMA copy per expert, whose
    // engine idles between copies); a store that is not mapped pinned memory
    // is copied by DMA instead
    if (fa.n > 0) {
        void *p = nullptr;
        if (hipHostGetDevicePointer(&p, (void *)host, 0) == hipSuccess && p) {
            fa.src = (const uint8_t *)p;
            if (hip_status(launch_fetch(fa, hs)) != MOE_OK) return MOE_ERR_HIP;
        } else {
            (void)hipGetLastError();
            for (int i = 0; i < fa.n; ++i)
                if (hip_status(hipMemcpyAsync(st->slots + (size_t)fa.slot[i] * eb, host + (size_t)fa.expert[i] * eb,
                                              eb, hipMemcpyHostToDevice, hs)) != MOE_OK)
                    return MOE_ERR_HIP;
        }
    }
    // 4. the expert kernels, reading the selected experts from their slots
    // (passed as kernel arguments)
    a.sel_host = nullptr;
    a.experts = st->slots;
    if (hip_status(launch_forward_slots(a, sl, hs)) != MOE_OK) return MOE_ERR_HIP;
    st->stats.calls += 1;
    return MOE_OK;
}

int moe_tier_stack_forward(void *state, const moe_layer_t *layers, int32_t n_layers, const float *x, float *y,
                           int32_t n_tokens, int32_t *route_idx, float *route_w, void *workspace,
                           size_t workspace_bytes, void *stream) {
    const TierState *st = tier_header(state);
    if (!st || !layers || n_layers < 1 || n_layers > st->n_layers || n_tokens < 1) return MOE_ERR_INVALID_ARG;
    const size_t per_layer = (size_t)n_tokens * st->dims.top_k;
    for (int l = 0; l < n_layers; ++l) {
        const int rc = moe_tier_layer_forward(state, l, &layers[l], l == 0 ? x : y, y, n_tokens,
                                              route_idx ? route_idx + l * per_layer : nullptr,
                                              route_w ? route_w + l * per_layer : nullptr, workspace,
                                              workspace_bytes, stream);
        if (rc != MOE_OK) return rc;
    }
    return MOE_OK;
}

int moe_tier_get_stats(const void *state, moe_tier_stats_t *out) {
    const TierState *st = tier_header(state);
    if (!st || !out) return MOE_ERR_INVALID_ARG;
    *out = st->stats;
    return MOE_OK;
}

int moe_tier_lookup(const void *state, int32_t layer_index, int32_t expert, int32_t *slot) {
    const TierState *st = tier_header(state);
    if (!st || !slot) return MOE_ERR_INVALID_ARG;
    if (layer_index < 0 || layer_index >= st->n_layers || expert < 0 || expert >= st->dims.n_experts)
        return MOE_ERR_INVALID_ARG;
    const TierView v = tier_view((void *)state);
    *slot = v.lru.slot_of[layer_index * st->dims.n_experts + expert];
    return MOE_OK;
}

const char *moe_last_error(void) {
    return g_last_hip == hipSuccess ? "no HIP error" : hipGetErrorString(g_last_hip);
}

const char *moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape or parameter";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_ALIGNMENT: return "misaligned pointer";
        case MOE_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

}  // extern "C"

// moe_pack.hip -- canonical -> packed experts, and the on-device synthetic
// expert generator.
//
// The generator draws every code, scale and bias from counter-based
// SplitMix64 streams (Steele, Lea & Flood, OOPSLA 2014), so any expert of any
// layer can be regenerated independently, on the device or on a host:
//   mix64(z)  = SplitMix64 finaliser (constants 0xBF58476D1CE4E5B9,
//               0x94D049BB133111EB; shifts 30, 27, 31)
//   tag       = layer << 32 | expert << 16 | matrix << 8 | kind
//               (matrix 0 gate, 1 up, 2 down; kind 0 codes, 1 scale, 2 bias;
//                expert E = the shared expert)
//   base      = mix64(mix64(seed + GAMMA) ^ tag),  GAMMA = 0x9E3779B97F4A7C15
//   word[i]   = mix64(base + (i+1) * GAMMA)
// code c (row-major over [rows][cols]) = bits [bits*(c % (64/bits)), +bits) of
// word[c / (64/bits)]; scale / bias of group g (row-major over [rows][cols/64]):
// u = (word[g] >> 40) * 2^-24, s = fl64(fl64(0.015*u) + 0.005),
// b = fl64(fl64(0.1*u) - 0.1), then fp64 -> fp32 -> bf16, round to nearest even.
// These are the uniform code, scale and bias distributions of the synthetic
// workloads (scale in [0.005, 0.02), bias in [-0.1, 0)).
#include "moe_internal.h"

namespace moe {

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t stream_base(uint64_t seed, uint32_t layer, uint32_t expert,
                                                uint32_t matrix, uint32_t kind) {
    const uint64_t tag = ((uint64_t)layer << 32) | ((uint64_t)expert << 16) | ((uint64_t)matrix << 8) | kind;
    return mix64(mix64(seed + kGamma) ^ tag);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// u = top 24 bits of a word as a fraction; value = fl64(fl64(mul*u) + add)
__device__ __forceinline__ uint16_t uniform_bf16(uint64_t word, double mul, double add) {
    const double u = (double)(word >> 40) * 0x1p-24;
    const double v = __dadd_rn(__dmul_rn(mul, u), add);
    return f32_to_bf16_rne(__double2float_rn(v));
}

// Place C codes (provided by `code_of(i)`) into a 16-byte chunk.
template <typename CodeFn>
__device__ __forceinline__ uint4 make_chunk(int bits, int order, CodeFn code_of) {
    uint32_t d[4] = {0u, 0u, 0u, 0u};
    const int C = 128 / bits;
    const uint32_t mask = (1u << bits) - 1u;
    // 4-bit nibble order stores q XOR 8: the signed code q - 8 as v_dot8_i32_i4 reads it
    const uint32_t flip = (bits == 4 && order == kOrderNibble) ? 8u : 0u;
    for (int i = 0; i < C; ++i) {
        int dw, shift;
        code_pos(bits, order, i, dw, shift);
        d[dw] |= (((uint32_t)code_of(i) & mask) ^ flip) << shift;
    }
    return make_uint4(d[0], d[1], d[2], d[3]);
}

// Work decomposition shared by the packer and the generator: one thread per
// 16-byte code chunk, then one thread per scale/bias dword, over the three
// matrices of an expert.
struct ExpertWork {
    size_t chunk_begin[4];  // prefix sums over matrices
    size_t sb_begin[4];
};

__host__ __device__ inline ExpertWork expert_work(const ExpertLayout &L) {
    ExpertWork w;
    w.chunk_begin[0] = 0;
    w.sb_begin[0] = 0;
    for (int m = 0; m < 3; ++m) {
        w.chunk_begin[m + 1] = w.chunk_begin[m] + (size_t)L.m[m].rows * L.m[m].nchunks;
        w.sb_begin[m + 1] = w.sb_begin[m] + (size_t)L.m[m].rows * L.m[m].ngroups;
    }
    return w;
}

__device__ __forceinline__ int which_matrix(const size_t *begin, size_t i) {
    return i < begin[1] ? 0 : (i < begin[2] ? 1 : 2);
}

__global__ __launch_bounds__(256) void k_pack(PackArgs a) {
    const ExpertWork w = expert_work(a.L);
    const size_t total = w.chunk_begin[3] + w.sb_begin[3];
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
        if (i < w.chunk_begin[3]) {
            const int m = which_matrix(w.chunk_begin, i);
            const QMat &q = a.L.m[m];
            const size_t local = i - w.chunk_begin[m];
            const int r = (int)(local / q.nchunks);
            const int p = (int)(local % q.nchunks);
            const int Lc = logical_chunk(q, p);
            const int C = 128 / q.bits;
            const uint8_t *src = a.codes[m] + (size_t)r * q.cols + (size_t)Lc * C;
            const uint4 v = make_chunk(q.bits, q.order, [&](int c) { return src[c]; });
            *(uint4 *)(a.dst + q.codes_off + (size_t)r * q.row_bytes + (size_t)p * 16) = v;
        } else {
            const size_t j = i - w.chunk_begin[3];
            const int m = which_matrix(w.sb_begin, j);
            const QMat &q = a.L.m[m];
            const size_t g = j - w.sb_begin[m];
            const uint32_t v = (uint32_t)a.scale[m][g] | ((uint32_t)a.bias[m][g] << 16);
            ((uint32_t *)(a.dst + q.sb_off))[g] = v;
        }
    }
}

__global__ __launch_bounds__(256) void k_generate(GenArgs a, size_t expert_bytes) {
    const ExpertWork w = expert_work(a.L);
    const size_t per_expert = w.chunk_begin[3] + w.sb_begin[3];
    const int e = a.first_expert + (int)blockIdx.y;
    uint8_t *dst = a.dst + (size_t)blockIdx.y * expert_bytes;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < per_expert; i += (size_t)gridDim.x * 256) {
        if (i < w.chunk_begin[3]) {
            const int m = which_matrix(w.chunk_begin, i);
            const QMat &q = a.L.m[m];
            const size_t local = i - w.chunk_begin[m];
            const int r = (int)(local / q.nchunks);
            const int p = (int)(local % q.nchunks);
            const int Lc = logical_chunk(q, p);
            const int C = 128 / q.bits;
            const int per_word = 64 / q.bits;
            const size_t first_code = (size_t)r * q.cols + (size_t)Lc * C;  // multiple of per_word
            const uint64_t base = stream_base(a.seed, a.layer, (uint32_t)e, (uint32_t)m, 0u);
            const size_t w0 = first_code / per_word;
            const uint64_t z0 = mix64(base + (uint64_t)(w0 + 1) * kGamma);
            const uint64_t z1 = mix64(base + (uint64_t)(w0 + 2) * kGamma);
            const int bits = q.bits;
            const uint4 v = make_chunk(bits, q.order, [&](int c) {
                const uint64_t zz = (c < per_word) ? z0 : z1;
                return (uint32_t)(zz >> (bits * (c % per_word)));
            });
            *(uint4 *)(dst + q.codes_off + (size_t)r * q.row_bytes + (size_t)p * 16) = v;
        } else {
            const size_t j = i - w.chunk_begin[3];
            const int m = which_matrix(w.sb_begin, j);
            const QMat &q = a.L.m[m];
            const size_t g = j - w.sb_begin[m];
            const uint64_t bs = stream_base(a.seed, a.layer, (uint32_t)e, (uint32_t)m, 1u);
            const uint64_t bb = stream_base(a.seed, a.layer, (uint32_t)e, (uint32_t)m, 2u);
            const uint16_t s = uniform_bf16(mix64(bs + (uint64_t)(g + 1) * kGamma), 0.015, 0.005);
            const uint16_t b = uniform_bf16(mix64(bb + (uint64_t)(g + 1) * kGamma), 0.1, -0.1);
            ((uint32_t *)(dst + q.sb_off))[g] = (uint32_t)s | ((uint32_t)b << 16);
        }
    }
}

__global__ void k_clear_ctrl(uint32_t *ctrl) {
    for (int i = threadIdx.x; i < (int)(kCtrlBytes / 4); i += blockDim.x) ctrl[i] = 0u;
}

}  // namespace

hipError_t launch_pack(const PackArgs &a, hipStream_t stream) {
    const ExpertWork w = expert_work(a.L);
    const size_t total = w.chunk_begin[3] + w.sb_begin[3];
    size_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    (void)hipGetLastError();  // report only this launch's status
    hipLaunchKernelGGL(k_pack, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_generate(const GenArgs &a, hipStream_t stream) {
    const ExpertWork w = expert_work(a.L);
    const size_t per_expert = w.chunk_begin[3] + w.sb_begin[3];
    size_t bx = (per_expert + 255) / 256;
    if (bx > 4096) bx = 4096;
    (void)hipGetLastError();
    for (int first = 0; first < a.count; first += 65535) {
        GenArgs part = a;
        part.first_expert = a.first_expert + first;
        part.count = (a.count - first) < 65535 ? (a.count - first) : 65535;
        part.dst = a.dst + (size_t)first * a.L.bytes;
        hipLaunchKernelGGL(k_generate, dim3((unsigned)bx, (unsigned)part.count), dim3(256), 0, stream,
                           part, a.L.bytes);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

hipError_t launch_clear_ctrl(uint32_t *ctrl, hipStream_t stream) {
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_clear_ctrl, dim3(1), dim3(64), 0, stream, ctrl);
    return hipGetLastError();
}

}  // namespace moe

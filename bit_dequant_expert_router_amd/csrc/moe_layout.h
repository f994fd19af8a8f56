// moe_layout.h -- packed expert layout and lane mapping (library-internal).
//
// A packed expert holds three quantised matrices, gate [F][H], up [F][H] and
// down [H][F] (row = output index, column = reduction index), each as
//   codes: rows x (cols*bits/8) bytes, then (after all three code blocks)
//   scale+bias: rows x (cols/64) dwords, dword = scale_bf16 | bias_bf16 << 16.
// Order in memory: gate codes, up codes, down codes, gate sb, up sb, down sb.
// Every block starts on a 256-byte boundary for the shapes the library builds.
//
// Codes of a row are stored in 16-byte chunks.  A chunk holds C = 128/bits
// consecutive codes of the row ("logical chunk" L covers columns
// [L*C, L*C + C)), D = 32/bits codes per dword; code i sits in dword i / D at a
// bit position t = i % D that depends on the matrix's order:
//   nibble order (gate, up): 4-bit code t at bits [4t, 4t+4), stored as
//     q XOR 8 (the signed value q - 8 in two's complement); 2-bit code t < 8
//     at bits [4t, 4t+2) and code t >= 8 at bits [4(t-8)+2, 4(t-8)+4).  The
//     dword itself (4-bit) or each of d & 0x33333333 and (d >> 2) & 0x33333333
//     (2-bit) is then eight 4-bit lanes holding consecutive codes, the operand
//     form of v_dot8.
//   byte order (down): code t in byte t % 4 at bits [bits*(t/4), +bits) of
//     that byte.  One mask per bit slot leaves four consecutive codes in bytes,
//     the operand form of v_dot4 against four values' byte limbs.
//
// Chunks are ordered for coalescing: a row of NC chunks is read by LPR =
// min(NC, 64) lanes, each lane owning CPL = NC/LPR logically consecutive
// chunks (a contiguous slice of the reduction axis).  Lane l's j-th chunk
// (logical chunk l*CPL + j) is stored at physical position l + LPR*j, so one
// 16-byte load per lane at position (l + LPR*j) covers LPR*16 contiguous bytes:
// whole 128-byte lines for a wave.
#pragma once
#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define MOE_HD __host__ __device__ __forceinline__
#else
#define MOE_HD inline
#endif

namespace moe {

constexpr int kGroup = 64;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;
constexpr int kMinDim = 128;
constexpr int kMaxDim = 4096;

enum CodeOrder { kOrderNibble = 0, kOrderByte = 1 };

struct QMat {
    int rows, cols, bits;
    int order;       // CodeOrder
    int row_bytes;   // cols * bits / 8
    int ngroups;     // cols / 64
    int nchunks;     // chunks per row
    int lpr;         // lanes per row
    int cpl;         // chunks per lane
    size_t codes_off;
    size_t sb_off;
};

struct ExpertLayout {
    QMat m[3];
    size_t bytes;
};

MOE_HD int codes_per_chunk(int bits) { return 128 / bits; }

MOE_HD QMat make_qmat(int rows, int cols, int bits, int order) {
    QMat q;
    q.rows = rows;
    q.cols = cols;
    q.bits = bits;
    q.order = order;
    q.row_bytes = cols * bits / 8;
    q.ngroups = cols / kGroup;
    q.nchunks = cols / codes_per_chunk(bits);
    q.lpr = q.nchunks < 64 ? q.nchunks : 64;
    q.cpl = q.nchunks / q.lpr;
    q.codes_off = 0;
    q.sb_off = 0;
    return q;
}

MOE_HD ExpertLayout make_layout(int H, int F, int bits) {
    ExpertLayout L;
    L.m[0] = make_qmat(F, H, bits, kOrderNibble);
    L.m[1] = make_qmat(F, H, bits, kOrderNibble);
    L.m[2] = make_qmat(H, F, bits, kOrderByte);
    size_t off = 0;
    for (int i = 0; i < 3; ++i) {
        L.m[i].codes_off = off;
        off += (size_t)L.m[i].rows * L.m[i].row_bytes;
    }
    for (int i = 0; i < 3; ++i) {
        L.m[i].sb_off = off;
        off += (size_t)L.m[i].rows * L.m[i].ngroups * 4;
    }
    L.bytes = off;
    return L;
}

// logical chunk (16 bytes of codes in reduction order) stored at physical
// chunk p of a row: lane l of a row's lpr lanes loads physical chunks l,
// l + lpr, ..., which hold its cpl consecutive logical chunks l cpl ..
MOE_HD int logical_chunk(const QMat &q, int p) { return (p % q.lpr) * q.cpl + p / q.lpr; }

// position of code i (0 <= i < C) inside a 16-byte chunk: dword index and
// bit shift within that dword
MOE_HD void code_pos(int bits, int order, int i, int &dword, int &shift) {
    const int D = 32 / bits;
    const int t = i % D;
    dword = i / D;
    if (order == kOrderByte)
        shift = 8 * (t % 4) + bits * (t / 4);
    else if (bits == 4)
        shift = 4 * t;
    else
        shift = (t < 8) ? 4 * t : 4 * (t - 8) + 2;
}

}  // namespace moe

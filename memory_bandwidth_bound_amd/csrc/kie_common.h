// kie_common.h - layout rules shared by the host repacker and the device kernels.
//
// Everything here is plain integer arithmetic on shapes, usable from host C++
// (g++) and from HIP device code. It fixes:
//  * the phase matrices of one decoder layer and their row order,
//  * how each phase's rows are split over the workgroups of the persistent
//    grid (the same split for the output projection and the FFN down
//    projection, so each residual element has exactly one owner),
//  * the streaming unit: 1 KiB = one wave-wide 16-byte-per-lane load (fp16
//    weights: 512 columns of one row; fp8 weights: 512 columns of a pair of
//    rows, lane l holding 8 bytes of each; fp4 weights: 512 columns of four
//    rows, lane l holding 4 bytes of each),
//  * the per-workgroup weight stream: for every layer, one contiguous piece
//    holding that workgroup's rows of every phase in phase order, then its
//    rows of the LM head.
#pragma once
#include <stdint.h>
#include <stddef.h>

#if defined(__HIPCC__)
#define KIE_HD __host__ __device__ inline
#else
#define KIE_HD inline
#endif

#ifndef KIE_HEAD_MODE_MAX
#define KIE_HEAD_MODE_MAX 1152
#endif
#ifndef KIE_HEAD_CHUNK
#define KIE_HEAD_CHUNK 384
#endif

namespace kie {

constexpr int kGrid = 256;                 // persistent workgroups: one per MI355X compute unit
constexpr int kXcds = 8;                   // XCDs of MI355X: workgroup w of the grid runs on XCD w % kXcds
constexpr int kXcdGrid = kGrid / kXcds;    // workgroups per XCD
constexpr int kUnitBytes = 1024;           // one 16-byte-per-lane load of a wave
constexpr int kUnitHalves = 512;           // fp16 elements per unit
constexpr int kMaxGroup = 8;               // query heads per KV head supported
constexpr int kAttnChunkMin = 32;          // fewest positions per attention work item
constexpr int kAttnHeadModeMax = KIE_HEAD_MODE_MAX;   // up to this many attended positions, work
                                           // items per (KV group, query head)
constexpr int kAttnHeadChunk = KIE_HEAD_CHUNK;   // most positions per head-mode work item
constexpr int kMaxSeq = 65536;
constexpr int kMaxRowsWg = 256;            // rows of one phase per workgroup
constexpr int kMaxOwnRows = 32;            // residual rows per workgroup
constexpr int kMaxInput = 8192;            // longest GEMV input (fp16 elements)
constexpr int kTracePhases = 2048;         // phases covered by the phase timeline

// Phase kinds of the per-layer pipeline.
enum Phase : int {
    PH_QKV = 0,    // fused [Wq;Wk;Wv], rotary pairs adjacent, gains folded
    PH_WO = 1,     // output projection, residual add
    PH_GU = 2,     // fused gate/up, rows interleaved (g_j, u_j), gains folded
    PH_DOWN = 3,   // down projection, residual add
    PH_ROUTER = 4, // MoE router rows, gains folded
    PH_LM = 5,     // LM head, gains folded
    PH_EGU = 6,    // selected experts' gate/up rows (virtual matrix top_k*2F x d)
    PH_EDOWN = 7,  // selected experts' down rows (virtual matrix d x top_k*F)
    PH_COUNT = 8
};

struct Dims {
    int L, d, H, Hkv, hd, F, V, E, topk, max_seq;
    int w8;   // 1: quantised weights (fp8 E4M3 or fp4 E2M1) with one fp32 scale per row; 0: fp16
    int w4;   // 1: the quantised weights are fp4 (E2M1), four rows per unit; 0: fp8, two rows per unit
};

struct RowSplit {
    int row0;
    int nrows;
};

// Even split of M rows in groups of `gran` over nwg workgroups; the first
// (M/gran) % nwg workgroups get one extra group.
KIE_HD RowSplit split_rows(int M, int gran, int nwg, int w) {
    int groups = M / gran;
    int base = groups / nwg, rem = groups % nwg;
    int g0 = w * base + (w < rem ? w : rem);
    int ng = base + (w < rem ? 1 : 0);
    RowSplit r;
    r.row0 = g0 * gran;
    r.nrows = ng * gran;
    return r;
}

KIE_HD int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Head mode of attention at c attended positions (2 to 8 query heads per KV
// head, at most kAttnHeadModeMax positions): one work item per (query head,
// chunk). Beyond it, the split over positions.
KIE_HD bool head_mode_at(const Dims& D, int c) {
    const int Gq = D.H / D.Hkv;
    return Gq >= 2 && Gq <= kMaxGroup && D.H <= kGrid && c <= kAttnHeadModeMax;
}

// Can every XCD compute all query heads' attention itself (XCD-local
// attention)? It needs head mode and at most one XCD's workgroups' worth of
// query heads; at a given context it runs while the heads' chunks fit too.
KIE_HD bool xcd_attention_ok(const Dims& D) {
    const int Gq = D.H / D.Hkv;
    return Gq >= 2 && Gq <= kMaxGroup && D.H <= kXcdGrid;
}

// Units of a slab of nrows rows of K fp16 each, padded to whole units.
KIE_HD int slab_units(int nrows, int K) { return ceil_div(nrows * K, kUnitHalves); }
// The same for the weight format of D (fp8 rows take one byte per weight and
// come in pairs, a unit holding 1024 weights; fp4 rows half a byte and come
// in fours, a unit holding 2048 weights).
KIE_HD int slab_units_of(const Dims& D, int nrows, int K) {
    if (D.w4) return ceil_div(nrows * K, 4 * kUnitHalves);
    return D.w8 ? ceil_div(nrows * K, 2 * kUnitHalves) : slab_units(nrows, K);
}

// Shape of a phase matrix: rows M, row length K (fp16), split granularity.
struct PhaseShape {
    int M, K, gran;
};

KIE_HD PhaseShape phase_shape(const Dims& D, int ph) {
    PhaseShape s;
    switch (ph) {
    // Granularities: QKV rows come in groups of 4 (two rotary pairs, so the
    // new key and value rows are written as whole 32-bit pairs), gate/up rows
    // in groups of 4 (two (gate, up) pairs -> one fp16 pair of h), residual
    // rows (Wo, down) in pairs (one fp16 pair of x per exchanged word).
    case PH_QKV: s.M = (D.H + 2 * D.Hkv) * D.hd; s.K = D.d; s.gran = 4; break;
    case PH_WO: s.M = D.d; s.K = D.H * D.hd; s.gran = D.w4 ? 4 : 2; break;   // fp4: rows in fours
    case PH_GU: s.M = 2 * D.F; s.K = D.d; s.gran = 4; break;
    case PH_DOWN: s.M = D.d; s.K = D.F; s.gran = D.w4 ? 4 : 2; break;
    case PH_ROUTER: s.M = D.E; s.K = D.d; s.gran = D.w4 ? 4 : D.w8 ? 2 : 1; break;   // fp8: pairs, fp4: fours
    case PH_LM: s.M = D.V; s.K = D.d; s.gran = D.w4 ? 4 : D.w8 ? 2 : 1; break;   // fp8: pairs, fp4: fours
    case PH_EGU: s.M = D.topk * 2 * D.F; s.K = D.d; s.gran = 4; break;
    case PH_EDOWN: s.M = D.d; s.K = D.F; s.gran = D.w4 ? 4 : 2; break;   // K per selected expert; = PH_WO
    default: s.M = 0; s.K = 0; s.gran = 1; break;
    }
    return s;
}

// Units of workgroup w in phase ph (for PH_EDOWN: all top_k segments).
KIE_HD int phase_units(const Dims& D, int ph, int nwg, int w) {
    PhaseShape s = phase_shape(D, ph);
    RowSplit r = split_rows(s.M, s.gran, nwg, w);
    if (ph == PH_EDOWN) return D.topk * slab_units_of(D, r.nrows, s.K);
    if (ph == PH_EGU) {
        // the workgroup's virtual rows may span several experts; each expert
        // segment is padded on its own
        int per = 2 * D.F;
        int u = 0;
        int a = r.row0, end = r.row0 + r.nrows;
        while (a < end) {
            int seg_end = (a / per + 1) * per;
            if (seg_end > end) seg_end = end;
            u += slab_units_of(D, seg_end - a, s.K);
            a = seg_end;
        }
        return u;
    }
    return slab_units_of(D, r.nrows, s.K);
}

// Phases whose weights sit in the per-layer streaming block, in stream order.
KIE_HD int layer_block_phase_count(const Dims& D) { return D.E ? 3 : 4; }
KIE_HD int layer_block_phase(const Dims& D, int i) {
    if (D.E) {
        const int p[3] = {PH_QKV, PH_WO, PH_ROUTER};
        return p[i];
    }
    const int p[4] = {PH_QKV, PH_WO, PH_GU, PH_DOWN};
    return p[i];
}

// Units of workgroup w's piece of one layer block.
KIE_HD int piece_units(const Dims& D, int nwg, int w) {
    int u = 0;
    for (int i = 0; i < layer_block_phase_count(D); ++i)
        u += phase_units(D, layer_block_phase(D, i), nwg, w);
    return u;
}

// Virtual QKV row -> original (matrix 0=q 1=k 2=v, row in that matrix).
// q and k heads store each rotary pair (i, i + hd/2) as adjacent rows
// (2i, 2i+1) of the head; v keeps its natural order.
KIE_HD void qkv_row_source(const Dims& D, int r, int* mat, int* row) {
    int qd = D.H * D.hd, kd = D.Hkv * D.hd;
    int m = 0;
    if (r >= qd + kd) { *mat = 2; *row = r - qd - kd; return; }
    if (r >= qd) { m = 1; r -= qd; }
    int head = r / D.hd, w = r % D.hd;
    int pair = w >> 1, which = w & 1;
    *mat = m;
    *row = head * D.hd + pair + which * (D.hd / 2);
}

}  // namespace kie

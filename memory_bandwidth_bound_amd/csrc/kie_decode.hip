// kie_decode.hip - the persistent batch-1 decode kernel for gfx950.
//
// One launch runs n whole forward passes: one resident grid for the whole
// decode loop, with weight prefetch, inter-CU synchronisation and on-device
// greedy sampling inside it (the monokernel design of the news.creeta.com
// article, "Inside the monokernel"). The grid is one 512-thread workgroup per
// compute unit (256 on MI355X); each workgroup owns a fixed share of every
// weight matrix (rows, laid out contiguously by the host) and of the residual.
//
// Waves of a workgroup:
//   wave 0 (communication): gathers each phase's input from the other
//     workgroups through flagged words, normalises it into LDS, runs the
//     phase epilogue (RoPE, KV-cache append, SwiGLU, residual add, argmax) and
//     publishes the outputs as flagged words;
//   waves 1..7 (compute): stream this workgroup's weights from HBM into a
//     per-wave LDS ring by LDS DMA (non-temporal 16-byte loads per lane), two
//     batches of 8 units of 1 KiB in flight per wave, and take the dot
//     products (v_dot2 on fp16, converted FP8 / FP4) against the LDS input;
//     they also run the attention of the workgroups that hold an attention
//     item.
//     A batch is refilled as soon as it is consumed, with the next units in
//     phase order, so weight streaming runs on across phase boundaries while
//     the communication wave waits for the next input.
//
// Phase sequence of one pass (each phase has a unique 32-bit id that tags
// every word it publishes):
//   per layer:  QKV | ATTN | COMB | WO | GU | DOWN               (dense FFN)
//               QKV | ATTN | COMB | WO | ROUTER | EGU | EDOWN     (top-k MoE)
//   then        LM | SAMPLE
// Up to kAttnHeadModeMax attended positions, ATTN runs per query head: its
// positions in chunks of at most kAttnHeadChunk, one workgroup each, and the
// first chunk's workgroup folds in the others' states and publishes o itself;
// COMB then has no work. Beyond that, every workgroup takes a chunk of a KV
// group's positions for all the group's query heads (on the matrix cores for
// head_dim 128) and COMB merges the chunk states.
// There is no grid-wide barrier: a phase waits only for the words it reads.
// A workgroup reads a phase's input only when it has work in that phase; then
// every overwrite of a buffer it reads depends, through the words the
// overwriting workgroup had to read first, on this workgroup having finished
// its read, so one buffer per exchanged vector suffices.
#include <hip/hip_runtime.h>

#include "kie_common.h"
#include "kie_device.h"
#include "kie_kernels.h"

namespace kie {

constexpr float kLog2e = 1.4426950408889634f;

enum Kind : int {
    K_QKV = 0, K_ATTN = 1, K_COMB = 2, K_WO = 3, K_GU = 4, K_DOWN = 5,
    K_ROUTER = 6, K_EGU = 7, K_EDOWN = 8, K_LM = 9, K_SAMPLE = 10, K_COUNT = 11
};

__device__ __forceinline__ int ppl_of(const Dims& D) { return D.E ? 7 : 6; }
__device__ __forceinline__ int pps_of(const Dims& D) { return D.L * ppl_of(D) + 2; }

__device__ __forceinline__ bool is_gemv(int kind) {
    return kind == K_QKV || kind == K_WO || kind == K_GU || kind == K_DOWN || kind == K_ROUTER ||
           kind == K_EGU || kind == K_EDOWN || kind == K_LM;
}

// Walks the phase sequence: q = global phase index within the launch; layer
// == D.L for the per-pass LM / SAMPLE phases (k = 0 / 1).
struct PIter {
    int q, step, layer, k;
};

__device__ __forceinline__ int kind_of(const Dims& D, const PIter& it) {
    if (it.layer == D.L) return it.k == 0 ? K_LM : K_SAMPLE;
    if (it.k < 4) return it.k;
    return D.E ? K_ROUTER + it.k - 4 : K_GU + it.k - 4;
}

__device__ __forceinline__ void advance(const Dims& D, PIter& it) {
    ++it.q;
    ++it.k;
    if (it.layer < D.L) {
        if (it.k == ppl_of(D)) {
            it.k = 0;
            ++it.layer;
        }
    } else if (it.k == 2) {
        it.k = 0;
        it.layer = 0;
        ++it.step;
    }
}

// Attention of c positions is cut into nper chunks of CH positions per KV head.
__device__ __forceinline__ int attn_split(int c, int items, int* CH) {
    int nper = ceil_div(c, kAttnChunkMin);
    if (nper > items) nper = items;
    *CH = ceil_div(c, nper);
    return ceil_div(c, *CH);
}

// Head mode (short context, groups of 2 to 8 query heads): the work items of
// query head h = (KV group h % Hkv, head h / Hkv of the group) split its c
// positions into nch chunks of at most kAttnHeadChunk; item i is chunk
// i / H of head i % H (so g = i % Hkv, as in the split over positions).
// Chunk 0 combines the other chunks' states of its head and publishes o
// itself: no combine phase over the grid. (Configurations hold at most 128
// query heads, since n_heads * head_dim is at most 8192 and head_dim at least
// 64, so the items fit the grid.)
__device__ __forceinline__ bool head_mode(const Dims& D, int c) { return head_mode_at(D, c); }

// Split attention on the matrix cores: head_dim 128 outside head mode (the
// group's at most kMaxGroup query heads fit the 16 columns of an MFMA tile),
// in the kernel variant built with it (MS; see launch_decode).
template <bool MS>
__device__ __forceinline__ bool mfma_attention(const Dims& D, int c) {
    return MS && D.hd == 128 && !head_mode(D, c);
}

// Chunks per head in head mode.
__device__ __forceinline__ int head_chunks(const DecodeArgs& a, int c) {
    int nch = ceil_div(c, kAttnHeadChunk);
    const int cap = kGrid / a.D.H;
    if (nch > cap) nch = cap;
    if (nch > a.items_per_head) nch = a.items_per_head;
    return nch;
}

// Attention work items (one workgroup each) for c attended positions.
__device__ __forceinline__ int attn_items(const DecodeArgs& a, int c) {
    if (head_mode(a.D, c)) return a.D.H * head_chunks(a, c);
    int CH;
    return a.D.Hkv * attn_split(c, a.items_per_head, &CH);
}

// XCD-local attention (F_XCD_ATTN; attention recomputed per die instead of
// exchanged between dies, its buffers replicated per die): while the
// head-mode items fit one XCD's workgroups, every XCD computes all of them
// for itself, workgroup w taking item w / kXcds, and writes its own copy
// (w % kXcds) of the chunk states and of o, which only the workgroups of the
// same XCD read. The words stay device-scope: an XCD's L2 is reached only by
// workgroup-scope accesses, and those may be served by a compute unit's own
// L1, which does not see the other units' stores. The kernel checks at its
// start that workgroup w runs on XCD w % kXcds.
template <bool XA>
__device__ __forceinline__ bool xcd_attention(const DecodeArgs& a, int c) {
    if constexpr (!XA) return false;   // kernels built without it (the host picks the variant)
    return (a.flags & F_XCD_ATTN) && head_mode(a.D, c) && a.D.H * head_chunks(a, c) <= kXcdGrid;
}
// This workgroup's attention work item at c positions, and the copy of the
// attention exchange buffers (part, o) it writes and reads.
template <bool XA>
__device__ __forceinline__ int attn_item(const DecodeArgs& a, int c, int wg) {
    return xcd_attention<XA>(a, c) ? wg / kXcds : wg;
}
template <bool XA>
__device__ __forceinline__ int attn_copy(const DecodeArgs& a, int c, int wg) {
    return xcd_attention<XA>(a, c) ? wg % kXcds : 0;
}

__device__ __forceinline__ bool lm_skipped(const DecodeArgs& a, int step) {
    return (a.flags & F_SKIP_LM) && step != a.n_steps - 1;
}

// Do this workgroup's waves meet at the two barriers of a phase? Every wave
// evaluates the same test, so the barrier sequences match.
template <bool XA>
__device__ __forceinline__ bool phase_bars(const DecodeArgs& a, int kind, int step, int wg) {
    if (kind == K_ATTN) return attn_item<XA>(a, a.pos0 + step + 1, wg) < attn_items(a, a.pos0 + step + 1);
    if (kind == K_LM) return !lm_skipped(a, step);
    return is_gemv(kind);
}

// This workgroup's share of each phase.
struct WgPlan {
    int q0, qn, wo0, won, gu0, gun, r0, rn, egu0, egun, lm0, lmn;
    int nq, nwo, ngu, nd, nr, negu, ned, nlm;
};

__device__ __forceinline__ void make_plan(const Dims& D, int wg, WgPlan& P) {
    const int G = kGrid;
    RowSplit r;
    PhaseShape s = phase_shape(D, PH_QKV);
    r = split_rows(s.M, s.gran, G, wg);
    P.q0 = r.row0; P.qn = r.nrows;
    s = phase_shape(D, PH_WO);
    r = split_rows(s.M, s.gran, G, wg);   // residual ownership (Wo, down)
    P.wo0 = r.row0; P.won = r.nrows;
    r = split_rows(D.V, phase_shape(D, PH_LM).gran, G, wg);
    P.lm0 = r.row0; P.lmn = r.nrows;
    P.nq = phase_units(D, PH_QKV, G, wg);
    P.nwo = phase_units(D, PH_WO, G, wg);
    P.nlm = phase_units(D, PH_LM, G, wg);
    P.gu0 = P.gun = P.r0 = P.rn = P.egu0 = P.egun = 0;
    P.ngu = P.nd = P.nr = P.negu = P.ned = 0;
    if (D.E) {
        r = split_rows(D.E, phase_shape(D, PH_ROUTER).gran, G, wg);
        P.r0 = r.row0; P.rn = r.nrows;
        s = phase_shape(D, PH_EGU);
        r = split_rows(s.M, s.gran, G, wg);
        P.egu0 = r.row0; P.egun = r.nrows;
        P.nr = phase_units(D, PH_ROUTER, G, wg);
        P.negu = phase_units(D, PH_EGU, G, wg);
        P.ned = phase_units(D, PH_EDOWN, G, wg);
    } else {
        s = phase_shape(D, PH_GU);
        r = split_rows(s.M, s.gran, G, wg);
        P.gu0 = r.row0; P.gun = r.nrows;
        P.ngu = phase_units(D, PH_GU, G, wg);
        P.nd = phase_units(D, PH_DOWN, G, wg);
    }
}

// Per-phase geometry of this workgroup, kept in LDS for the compute waves.
struct Geo {
    int n;      // units
    int nrows;  // rows
    int K;      // row length per segment (fp16)
    int nseg;   // segments per row (MoE down: top_k)
    int off;    // units from the start of the layer block (LM: of the LM block)
    int row0;   // first row (MoE gate/up: virtual row)
    int gin;    // words of the exchanged input vector this workgroup gathers (0: none)
};

// LDS shared by the waves of one workgroup.
struct Smem {
    // per compute wave: kNS batches of kNB weight units, written by LDS DMA
    alignas(16) uint8_t ring[kCompute * kNS * kBatchBytes];
    union {
        struct {                                // GEMV phases: the input as two fp16 terms,
            alignas(16) uint16_t xin[kMaxIn];   // hi = fp16(v)
            alignas(16) uint16_t xlo[kMaxIn];   // lo = fp16(v - hi)
            float part[kMaxRowsWg * kCompute];  // per (row, compute wave) partial dot products
        };
        struct {
            float att_o[kCompute * kMaxGroup * 128];   // attention: per compute wave, unnormalised o
            alignas(16) uint16_t att_qh[kMaxGroup * 128];   // matrix-core attention: the queries as
            alignas(16) uint16_t att_ql[kMaxGroup * 128];   // two fp16 terms (hi, lo = fp16(q - hi))
        };
    };
    float att_q[kMaxGroup * 128];               // queries of the attention group, pre-scaled (also scratch)
    static_assert(sizeof(uint16_t) * 2 * kMaxIn == sizeof(float) * kMaxIn, "fp32 staging reuses xin and xlo");
    alignas(16) uint16_t att_k[128];            // the new position's key and value
    alignas(16) uint16_t att_v[128];
    float att_ml[kCompute * kMaxGroup * 2];     // per compute wave: (max, sum)
    float own_x[kMaxOwnRows];                   // this workgroup's residual rows (fp32)
    uint32_t sel[16];                           // MoE: experts selected for the current layer
    float pi[16];                               //      and their router probabilities
    float esc[16 * kMaxOwnRows];                // quantised MoE: down-row scales [selected expert][own row]
    Geo geo[K_COUNT];
    float ssp[kWaves];                          // per wave: sum of squares of its share of the input
    uint32_t abort;                             // set when the communication wave gave up
};

__device__ __forceinline__ void set_geo(KIE_LDS Geo* g, int n, int nrows, int K, int nseg, int off, int row0,
                                        int gin = 0) {
    g->n = n;
    g->nrows = nrows;
    g->K = K;
    g->nseg = nseg;
    g->off = off;
    g->row0 = row0;
    g->gin = gin;
}

__device__ __forceinline__ void write_geo(const DecodeArgs& a, const WgPlan& W, int wg, KIE_LDS Geo* geo) {
    const Dims& D = a.D;
    for (int k = 0; k < K_COUNT; ++k) set_geo(geo + k, 0, 0, kUnitHalves, 1, 0, 0);
    const int piece = a.plan[wg];
    // the input vector is gathered only where it is used: by workgroups with
    // units in the phase (MoE: the router's input also feeds gate/up and down)
    set_geo(geo + K_QKV, W.nq, W.qn, D.d, 1, piece, W.q0, W.nq ? D.d : 0);
    set_geo(geo + K_WO, W.nwo, W.won, D.H * D.hd, 1, piece + W.nq, W.wo0, W.nwo ? D.H * D.hd : 0);
    if (D.E) {
        set_geo(geo + K_ROUTER, W.nr, W.rn, D.d, 1, piece + W.nq + W.nwo, W.r0, (W.nr || W.negu || W.ned) ? D.d : 0);
        set_geo(geo + K_EGU, W.negu, W.egun, D.d, 1, 0, W.egu0);
        set_geo(geo + K_EDOWN, W.ned, W.won, D.F, D.topk, 0, W.wo0, W.ned ? D.topk * D.F : 0);
    } else {
        set_geo(geo + K_GU, W.ngu, W.gun, D.d, 1, piece + W.nq + W.nwo, W.gu0, W.ngu ? D.d : 0);
        set_geo(geo + K_DOWN, W.nd, W.won, D.F, 1, piece + W.nq + W.nwo + W.ngu, W.wo0, W.nd ? D.F : 0);
    }
    set_geo(geo + K_LM, W.nlm, W.lmn, D.d, 1, a.plan[kGrid + 1 + wg], W.lm0, W.nlm ? D.d : 0);
}

// Stage input element i in LDS as two fp16 terms: xin = fp16(v), xlo =
// fp16(v - xin). A GEMV sums the products with both, so its input keeps about
// 22 significant bits while every product is a v_dot2 of fp16 pairs. With
// quantised weights (W8: fp8 or fp4) the input is staged as fp32 over the same
// bytes (xf) and the products are fp32 multiply-adds of converted weights.
__device__ __forceinline__ KIE_LDS float* xf_of(KIE_LDS Smem* S) { return (KIE_LDS float*)S->xin; }
template <bool W8>
__device__ __forceinline__ void stage1(KIE_LDS Smem* S, int i, float v) {
    if constexpr (W8) {
        xf_of(S)[i] = v;
    } else {
        const _Float16 hi = (_Float16)v;
        S->xin[i] = __builtin_bit_cast(uint16_t, hi);
        S->xlo[i] = __builtin_bit_cast(uint16_t, (_Float16)(v - (float)hi));
    }
}

// Every wave of the workgroup gathers its slice of the phase's input vector
// (x, o or h as flagged fp32 words; all of a wave's loads are in flight at
// once), stages it and leaves the slice's sum of squares in ssp[w]. The RMS
// norm scale is applied to the row sums afterwards, which is the same product
// since a GEMV is linear. c: positions the pass attends (with XCD-local
// attention, Wo reads its own XCD's copy of o). Returns 0, or 1 (this wave
// timed out) / 2 (another workgroup reported a failure).
template <bool W8, bool XA>
__device__ __forceinline__ int gather_input(const DecodeArgs& a, KIE_LDS Smem* S, int kind, int n, uint32_t id,
                                            int w, int c) {
    const uint64_t* src = kind == K_WO ? a.ex.o + (size_t)attn_copy<XA>(a, c, blockIdx.x) * a.ex.o_copy
                                       : ((kind == K_DOWN || kind == K_EDOWN) ? a.ex.h : a.ex.x);
    const int i0 = n * w / kWaves, i1 = n * (w + 1) / kWaves;
    float ss = 0.f;
    const int r = fw_gather(src + i0, i1 - i0, id, a.spin, a.status, [&](int i, uint32_t v) {
        const float x = __builtin_bit_cast(float, v);
        ss += x * x;
        stage1<W8>(S, i0 + i, x);
    });
    ss = wave_sum(ss);
    if (lane_id() == 0) S->ssp[w] = ss;
    return r;
}

// Does every wave gather a share of this phase's input? Then all waves first
// meet at a barrier, so that no share overwrites the staged input, the sums of
// squares or the attention scratch that shares their LDS while the
// communication wave still finishes the previous phases.
__device__ __forceinline__ bool shared_gather(KIE_LDS Smem* S, int kind, int layer) {
    return __builtin_amdgcn_readfirstlane(S->geo[kind].gin) > 0 && !(kind == K_QKV && layer == 0);
}

// Merge the compute waves' attention states of this chunk and publish o (the
// whole row is here) or the chunk's partial state. Wave w8 of 8 takes every
// 8th block of 64 (head, dim pair) slots.
template <int HD, bool XA>
__device__ __forceinline__ int attn_merge(const DecodeArgs& a, KIE_LDS Smem* S, int pos, uint32_t id, int w8) {
    const Dims& D = a.D;
    const int lane = lane_id(), wg = blockIdx.x;
    const int Gq = D.H / D.Hkv;
    int CH;
    const bool hm = head_mode(D, pos + 1);
    const int nch = hm ? head_chunks(a, pos + 1) : 1;
    // head mode: this workgroup holds chunk it / H of query head it % H; chunks
    // 1 .. nch-1 publish their states, chunk 0 combines them
    const int nper = hm ? nch : attn_split(pos + 1, a.items_per_head, &CH);
    const int it = attn_item<XA>(a, pos + 1, wg);
    uint64_t* const part = a.ex.part + (size_t)attn_copy<XA>(a, pos + 1, wg) * a.ex.part_copy;
    uint64_t* const ob = a.ex.o + (size_t)attn_copy<XA>(a, pos + 1, wg) * a.ex.o_copy;
    const int g = it % D.Hkv, chunk = hm ? it / D.H : it / D.Hkv;
    const int i0 = hm ? ((it % D.H) / D.Hkv) * HD : 0, i1 = hm ? i0 + HD : Gq * HD;
    for (int idx = i0 + 2 * (w8 * 64 + lane); idx < i1; idx += 2 * 64 * kWaves) {
        const int j = idx / HD, dd = idx % HD;
        float M = -3.0e38f;
#pragma unroll
        for (int w = 0; w < kCompute; ++w) M = fmaxf(M, S->att_ml[(w * kMaxGroup + j) * 2]);
        float L = 0.f, O0 = 0.f, O1 = 0.f;
#pragma unroll
        for (int w = 0; w < kCompute; ++w) {
            const float f = __builtin_amdgcn_exp2f(S->att_ml[(w * kMaxGroup + j) * 2] - M);
            L += f * S->att_ml[(w * kMaxGroup + j) * 2 + 1];
            O0 += f * S->att_o[(w * kMaxGroup + j) * HD + dd];
            O1 += f * S->att_o[(w * kMaxGroup + j) * HD + dd + 1];
        }
        const int head = g * Gq + j;
        if (hm && chunk == 0 && nch > 1) {
            // fold in the other chunks' states of this head, up to four chunks
            // per trip (all their words polled at once), then publish o
            for (int k0 = 1; k0 < nch; k0 += 4) {
                const int kn = nch - k0 < 4 ? nch - k0 : 4;
                uint64_t wv[4][4];
                uint32_t spins = 0;
                while (true) {
                    bool ok = true;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        if (u < kn) {
                            const uint64_t* pp = part + ((size_t)head * a.items_per_head + k0 + u) * (HD + 2);
                            wv[u][0] = fw_load(pp);
                            wv[u][1] = fw_load(pp + 1);
                            wv[u][2] = fw_load(pp + 2 + dd);
                            wv[u][3] = fw_load(pp + 3 + dd);
                        }
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (u < kn)
                            ok = ok && fw_ok(wv[u][0], id) && fw_ok(wv[u][1], id) && fw_ok(wv[u][2], id) &&
                                 fw_ok(wv[u][3], id);
                    if (__builtin_amdgcn_ballot_w64(!ok) == 0) break;
                    if (++spins > a.spin) return 1;
                    if ((spins & 63) == 0 && stop_requested(a.status)) return 2;
#if KIE_POLL_SLEEP > 0
                    __builtin_amdgcn_s_sleep(KIE_POLL_SLEEP);
#endif
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (u < kn) {
                        const float m2 = __builtin_bit_cast(float, fw_val(wv[u][0]));
                        const float l2 = __builtin_bit_cast(float, fw_val(wv[u][1]));
                        const float Mn = fmaxf(M, m2);
                        const float f1 = __builtin_amdgcn_exp2f(M - Mn), f2 = __builtin_amdgcn_exp2f(m2 - Mn);
                        L = L * f1 + l2 * f2;
                        O0 = O0 * f1 + __builtin_bit_cast(float, fw_val(wv[u][2])) * f2;
                        O1 = O1 * f1 + __builtin_bit_cast(float, fw_val(wv[u][3])) * f2;
                        M = Mn;
                    }
                }
            }
        }
        if (nper == 1 || (hm && chunk == 0)) {
            // the whole row is here: publish o under the combine phase's id
            fw_store(ob + head * HD + dd, __builtin_bit_cast(uint32_t, O0 / L), id + 1);
            fw_store(ob + head * HD + dd + 1, __builtin_bit_cast(uint32_t, O1 / L), id + 1);
        } else {
            uint64_t* pp = part + ((size_t)head * a.items_per_head + chunk) * (HD + 2);
            fw_store(pp + 2 + dd, __builtin_bit_cast(uint32_t, O0), id);
            fw_store(pp + 3 + dd, __builtin_bit_cast(uint32_t, O1), id);
            if (dd == 0) {
                fw_store(pp, __builtin_bit_cast(uint32_t, M), id);
                fw_store(pp + 1, __builtin_bit_cast(uint32_t, L), id);
            }
        }
    }
    return 0;
}

// ------------------------------------------------------------------------
// Communication wave.
// ------------------------------------------------------------------------
template <int HD, int WF, bool MS, bool XA>
struct Comm {
    static constexpr bool W8 = WF != 0;   // quantised weights (fp8 or fp4): fp32 inputs, row scales
    const DecodeArgs& a;
    KIE_LDS Smem* S;
    WgPlan W;
    int wg, lane, tok;
    int att_c;     // positions the current pass attends
    bool dead;
    float rq[4];   // QKV epilogue: (cos, sin) of this lane's two rotary pairs, loaded before the input gather
    float rs[4];   // quantised weights: scales of the rows this lane's epilogue handles, loaded before the gather
    float esr[8];  // quantised MoE: down-row scales of the selected experts (entry lane + 64 j), after routing

    __device__ __forceinline__ Comm(const DecodeArgs& args, KIE_LDS Smem* s, const WgPlan& plan)
        : a(args), S(s), W(plan) {
        wg = blockIdx.x;
        lane = lane_id();
        tok = a.pending;
        att_c = a.pos0 + 1;
        dead = false;
    }

    __device__ __forceinline__ uint32_t id_of(int q) { return a.id0 + (uint32_t)q; }

    // why: 1 = this wave's wait timed out, 2 = another workgroup reported one
    __device__ __forceinline__ void fail(int why) {
        if (!dead && lane == 0) {
            if (why == 1) sys_store32(a.status, (uint32_t)kStatusTimeout);
            S->abort = 1u;
        }
        dead = true;
    }

    template <class F>
    __device__ __forceinline__ bool gather(const uint64_t* src, int n, uint32_t id, F f) {
        if (dead) return false;
        const int r = fw_gather(src, n, id, a.spin, a.status, f);
        if (r) fail(r);
        return r == 0;
    }

    // this wave's slice of the phase input (the compute waves gather theirs)
    __device__ __forceinline__ void input_share(int kind, uint32_t id) {
        if (dead) return;
        const int n = S->geo[kind].gin;
        const int r = gather_input<W8, XA>(a, S, kind, n, id, 0, att_c);
        if (r) fail(r);
    }

    // quantised weights: the row scales this lane's epilogue multiplies by. Row
    // r of lane e-th slot: QKV and gate/up 4 lane + e, Wo and down 2 lane + e,
    // LM lane + 64 e (the epilogues' row loops below). Read before the input
    // gather, so the trip overlaps it; rows past the phase read scale 1.
    __device__ __forceinline__ void load_row_scales(int kind, int layer) {
        if constexpr (W8) {
            const Dims& D = a.D;
            const int mq = (D.H + 2 * D.Hkv) * HD, mo = D.d, mg = 2 * D.F;
            const KIE_GLOBAL float* b = gptr(a.scales) + (size_t)layer * a.layer_scales;
            int r0 = 0, n = 0, step = 1, mul = 1;
            switch (kind) {
            case K_QKV: b += 0; r0 = W.q0; n = W.qn; mul = 4; break;
            case K_WO: b += mq; r0 = W.wo0; n = W.won; mul = 2; break;
            case K_GU: b += mq + mo; r0 = W.gu0; n = W.gun; mul = 4; break;
            case K_DOWN: b += mq + mo + mg; r0 = W.wo0; n = W.won; mul = 2; break;
            case K_ROUTER: b += mq + mo; r0 = W.r0; n = W.rn; step = 64; break;
            case K_LM: b = gptr(a.scales) + (size_t)D.L * a.layer_scales; r0 = W.lm0; n = W.lmn; step = 64; mul = 1;
                break;
            default: break;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = step == 64 ? lane + 64 * e : mul * lane + e;
                rs[e] = (r < n && (step == 64 || e < mul)) ? b[r0 + r] : 1.0f;
            }
        }
    }
    // quantised MoE, right after routing: the gate/up row scales of this lane's
    // epilogue rows (4 lane + e of the workgroup's virtual rows) and the
    // down-row scales of every selected expert (staged in LDS before the down
    // phase, for the compute waves).
    __device__ __forceinline__ void load_expert_scales(int layer) {
        if constexpr (W8) {
            const Dims& D = a.D;
            const int per = 2 * D.F + D.d;
            const KIE_GLOBAL float* b = gptr(a.escales) + (size_t)layer * D.E * per;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * lane + e;
                rs[e] = 1.0f;
                if (r < W.egun) {
                    const int vr = W.egu0 + r, k = vr / (2 * D.F);
                    rs[e] = b[(size_t)S->sel[k] * per + (vr - k * 2 * D.F)];
                }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int i = lane + 64 * j, k = W.won ? i / W.won : 0;
                esr[j] = 1.0f;
                if (i < D.topk * W.won) esr[j] = b[(size_t)S->sel[k] * per + 2 * D.F + W.wo0 + (i - k * W.won)];
            }
        }
    }
    __device__ __forceinline__ void stage_expert_scales() {
        if constexpr (W8) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int i = lane + 64 * j;
                if (i < a.D.topk * W.won) S->esc[i] = esr[j];
            }
        }
    }

    __device__ __forceinline__ float rsc(int e) const {
        if constexpr (W8) return rs[e];
        return 1.0f;
    }

    // the first layer's input: the token's embedding row, staged whole here
    __device__ __forceinline__ void input_embedding(const uint16_t* e) {
        const int d = a.D.d;
        float ss = 0.f;
        for (int i = lane; i < d; i += 64) {
            const float x = h2f_bits(gptr(e)[i]);
            ss += x * x;
            stage1<W8>(S, i, x);
        }
        ss = wave_sum(ss);
        if (lane < kWaves) S->ssp[lane] = lane == 0 ? ss : 0.f;
    }

    // RMS norm scale of the staged input: rsqrt(mean(v^2) + eps)
    __device__ __forceinline__ float in_scale() {
        float ss = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) ss += S->ssp[w];
        return 1.0f / sqrtf(ss / (float)a.D.d + a.eps);
    }

    __device__ __forceinline__ void zero_part(int nrows) {
        for (int i = lane; i < nrows * kCompute; i += 64) S->part[i] = 0.f;
    }
    __device__ __forceinline__ float rowsum(int r) {
        const KIE_LDS float* p = S->part + r * kCompute;
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kCompute; ++w) s += p[w];
        return s;
    }

    // Add the projection to the owned residual rows and publish them.
    __device__ __forceinline__ void residual_add_publish(uint32_t id) {
        for (int j = 2 * lane; j < W.won; j += 128) {   // at most 32 rows: one trip
            const float x0 = S->own_x[j] + rowsum(j) * rsc(0);
            const float x1 = S->own_x[j + 1] + rowsum(j + 1) * rsc(1);
            S->own_x[j] = x0;
            S->own_x[j + 1] = x1;
            fw_store(a.ex.x + W.wo0 + j, __builtin_bit_cast(uint32_t, x0), id);
            fw_store(a.ex.x + W.wo0 + j + 1, __builtin_bit_cast(uint32_t, x1), id);
        }
    }

    // Softmax over the router logits, then the top k (ties to the lower
    // expert index) with their probabilities, into LDS.
    __device__ __forceinline__ void route(int q, const PIter& it) {
        const Dims& D = a.D;
        const int E = D.E;
        KIE_LDS float* lg = S->att_q;   // scratch (E <= 1024): no attention is running
        if (!gather(a.ex.r, E, id_of(q - 1), [&](int i, uint32_t v) { lg[i] = __builtin_bit_cast(float, v); }))
            return;
        if ((a.flags & F_DBG_EXPERTS) && wg == 0)
            for (int e = lane; e < E; e += 64)
                gptr(a.dbg_router)[((size_t)(it.step % 64) * D.L + it.layer) * E + e] = lg[e];
        float mx = -3.0e38f;
        for (int e = lane; e < E; e += 64) mx = fmaxf(mx, lg[e]);
        mx = wave_max(mx);
        float sum = 0.f;
        for (int e = lane; e < E; e += 64) sum += __expf(lg[e] - mx);
        sum = wave_sum(sum);
        // rank of each logit among all E (larger first, ties to the lower
        // index); the k of rank < top_k are the selection. The logits are
        // padded to a multiple of 8 so the reads below come in independent 8s.
        const int E8 = (E + 7) & ~7;
        for (int e = E + lane; e < E8; e += 64) lg[e] = -3.4e38f;
        if (lane < 16) S->sel[lane] = 0u;   // in range even if NaN logits leave ranks unfilled
        for (int e = lane; e < E; e += 64) {
            const float v = lg[e];
            int rank = 0;
            for (int j0 = 0; j0 < E8; j0 += 8) {
                float u[8];
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) u[jj] = lg[j0 + jj];
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) rank += (u[jj] > v || (u[jj] == v && j0 + jj < e)) ? 1 : 0;
            }
            if (rank < D.topk) {
                S->sel[rank] = (uint32_t)e;
                S->pi[rank] = __expf(v - mx) / sum;
                if ((a.flags & F_DBG_EXPERTS) && wg == 0)
                    gptr(a.dbg_experts)[((size_t)(it.step % 64) * D.L + it.layer) * D.topk + rank] = e;
            }
        }
    }

    // ---- before the compute waves run: gather and prepare the input -------
    __device__ __forceinline__ void pre(int kind, const PIter& it) {
        const Dims& D = a.D;
        if (dead) return;
        const int q = it.q;
        att_c = a.pos0 + it.step + 1;
        load_row_scales(kind, it.layer);
        switch (kind) {
        case K_QKV: {
            // the epilogue's RoPE table entries, read now so that their trip
            // overlaps the input gather instead of following the compute
            const int qk = D.H * HD + D.Hkv * HD, vr = W.q0 + 4 * lane;
            if (lane < W.qn / 4 && vr < qk) {
                const int i = (vr % HD) >> 1;
                const KIE_GLOBAL float* r = gptr(a.rope) + ((size_t)(a.pos0 + it.step) * HD + 2 * i);
#pragma unroll
                for (int e = 0; e < 4; ++e) rq[e] = r[e];
            }
            zero_part(W.qn);
            if (it.layer == 0) {
                const uint16_t* e = a.emb + (size_t)tok * D.d;
                for (int j = lane; j < W.won; j += 64) S->own_x[j] = h2f_bits(gptr(e)[W.wo0 + j]);
                if (W.nq) input_embedding(e);
            } else if (W.nq) {
                input_share(kind, id_of(q - 1));   // the previous layer's last phase
            }
            break;
        }
        case K_ATTN: {
            const int Gq = D.H / D.Hkv, GW = (Gq + 1) * HD, g = attn_item<XA>(a, att_c, wg) % D.Hkv;
            const float qs = kLog2e / sqrtf((float)HD);
            const bool q16 = mfma_attention<MS>(D, a.pos0 + it.step + 1);
            gather(a.ex.qkv + (size_t)g * GW, GW, id_of(q - 1), [&](int i, uint32_t v) {
                if (i < Gq * HD) {
                    const float x = __builtin_bit_cast(float, v) * qs;
                    if (q16) {
                        const _Float16 h = (_Float16)x;
                        S->att_qh[i] = __builtin_bit_cast(uint16_t, h);
                        S->att_ql[i] = __builtin_bit_cast(uint16_t, (_Float16)(x - (float)h));
                    } else {
                        S->att_q[i] = x;
                    }
                } else if (i < Gq * HD + HD / 2) {
                    const int k = i - Gq * HD;
                    S->att_k[k] = (uint16_t)v;
                    S->att_k[k + HD / 2] = (uint16_t)(v >> 16);
                } else {
                    const int k = i - Gq * HD - HD / 2;
                    S->att_v[2 * k] = (uint16_t)v;
                    S->att_v[2 * k + 1] = (uint16_t)(v >> 16);
                }
            });
            break;
        }
        case K_WO:
            zero_part(W.won);
            if (W.nwo) input_share(kind, id_of(q - 1));
            break;
        case K_GU:
            zero_part(W.gun);
            if (W.ngu) input_share(kind, id_of(q - 1));
            break;
        case K_DOWN:
            zero_part(W.won);
            if (W.nd) input_share(kind, id_of(q - 1));
            break;
        case K_ROUTER:
            zero_part(W.rn);
            if (W.nr || W.negu || W.ned) input_share(kind, id_of(q - 1));
            break;
        case K_EGU:
            zero_part(W.egun);
            if (W.negu || W.ned) {
                route(q, it);   // xin and ssp still hold the router's input
                if (!dead) load_expert_scales(it.layer);
            }
            break;
        case K_EDOWN:
            zero_part(W.won);
            stage_expert_scales();
            if (W.ned) input_share(kind, id_of(q - 1));
            break;
        case K_LM:
            zero_part(W.lmn);
            if (W.nlm) input_share(kind, id_of(q - 1));
            break;
        default: break;
        }
    }

    // ---- after the compute waves: epilogue and publication ----------------
    __device__ __forceinline__ void post(int kind, const PIter& it, int pos) {
        const Dims& D = a.D;
        if (dead) return;
        const uint32_t id = id_of(it.q);
        const int Gq = D.H / D.Hkv, GW = (Gq + 1) * HD;
        switch (kind) {
        case K_QKV: {
            const int qd = D.H * HD, kd = D.Hkv * HD;
            const float sc = in_scale();
            // one lane per group of 4 rows (at most 64 groups): two rotary pairs, or 4 values
            for (int j = lane; j < W.qn / 4; j += 64) {
                const int vr = W.q0 + 4 * j;
                float y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = rowsum(4 * j + e) * sc * rsc(e);   // one trip: qn / 4 <= 64
                if (vr < qd + kd) {
                    // rows (4j, 4j+1) = elements (i, i+hd/2), rows (4j+2, 4j+3) = (i+1, i+1+hd/2)
                    const int i = (vr % HD) >> 1;
                    float r[4];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const float c = rq[2 * e], s = rq[2 * e + 1];
                        const float x0 = y[2 * e], x1 = y[2 * e + 1];
                        r[2 * e] = x0 * c - x1 * s;
                        r[2 * e + 1] = x1 * c + x0 * s;
                    }
                    if (vr < qd) {
                        const int head = vr / HD;
                        uint64_t* b = a.ex.qkv + (size_t)(head / Gq) * GW + (head % Gq) * HD;
                        fw_store(b + i, __builtin_bit_cast(uint32_t, r[0]), id);
                        fw_store(b + i + HD / 2, __builtin_bit_cast(uint32_t, r[1]), id);
                        fw_store(b + i + 1, __builtin_bit_cast(uint32_t, r[2]), id);
                        fw_store(b + i + 1 + HD / 2, __builtin_bit_cast(uint32_t, r[3]), id);
                    } else {
                        const int g = (vr - qd) / HD;
                        uint64_t* b = a.ex.qkv + (size_t)g * GW + Gq * HD;
                        fw_store(b + i, pack_h2(r[0], r[1]), id);
                        fw_store(b + i + 1, pack_h2(r[2], r[3]), id);
                        uint16_t* kp = a.kc + (((size_t)it.layer * D.Hkv + g) * D.max_seq + pos) * HD;
                        dev_store32(kp + i, pack_h2(r[0], r[2]));
                        dev_store32(kp + i + HD / 2, pack_h2(r[1], r[3]));
                    }
                } else {
                    const int vi = vr - qd - kd, g = vi / HD, dd = vi % HD;
                    uint64_t* b = a.ex.qkv + (size_t)g * GW + Gq * HD + HD / 2;
                    fw_store(b + dd / 2, pack_h2(y[0], y[1]), id);
                    fw_store(b + dd / 2 + 1, pack_h2(y[2], y[3]), id);
                    uint16_t* vp = a.vc + (((size_t)it.layer * D.Hkv + g) * D.max_seq + pos) * HD;
                    dev_store64(vp + dd, (uint64_t)pack_h2(y[0], y[1]) | ((uint64_t)pack_h2(y[2], y[3]) << 32));
                }
            }
            break;
        }
        case K_ATTN: {
            const int r = attn_merge<HD, XA>(a, S, pos, id, 0);   // the compute waves merge the other slices
            if (r) fail(r);
            break;
        }
        case K_WO:
        case K_DOWN:
        case K_EDOWN:
            residual_add_publish(id);
            break;
        case K_GU: {
            // rows (4j .. 4j+3) = (g_m, u_m, g_m+1, u_m+1) with m = (gu0 + 4j) / 2
            const float sc = in_scale();
            for (int j = lane; j < W.gun / 4; j += 64) {   // one trip: gun / 4 <= 64
                float h[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const float gv = rowsum(4 * j + 2 * e) * sc * rsc(2 * e);
                    const float uv = rowsum(4 * j + 2 * e + 1) * sc * rsc(2 * e + 1);
                    h[e] = gv / (1.0f + __expf(-gv)) * uv;
                }
                const int m = W.gu0 / 2 + 2 * j;
                fw_store(a.ex.h + m, __builtin_bit_cast(uint32_t, h[0]), id);
                fw_store(a.ex.h + m + 1, __builtin_bit_cast(uint32_t, h[1]), id);
            }
            break;
        }
        case K_ROUTER: {
            const float sc = in_scale();
            for (int j = lane; j < W.rn; j += 64)   // one trip: rn <= 4
                fw_store(a.ex.r + W.r0 + j, __builtin_bit_cast(uint32_t, rowsum(j) * sc * rsc(0)), id);
            break;
        }
        case K_EGU: {
            const float sc = in_scale();
            for (int j = lane; j < W.egun / 4; j += 64) {
                const int vr = W.egu0 + 4 * j;
                const int k = vr / (2 * D.F), m = (vr % (2 * D.F)) >> 1;
                float h[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {   // one trip of j: egun / 4 <= 64
                    const float gv = rowsum(4 * j + 2 * e) * sc * rsc(2 * e);
                    const float uv = rowsum(4 * j + 2 * e + 1) * sc * rsc(2 * e + 1);
                    h[e] = S->pi[k] * (gv / (1.0f + __expf(-gv))) * uv;
                }
                fw_store(a.ex.h + k * D.F + m, __builtin_bit_cast(uint32_t, h[0]), id);
                fw_store(a.ex.h + k * D.F + m + 1, __builtin_bit_cast(uint32_t, h[1]), id);
            }
            break;
        }
        case K_LM: {
            float bv = -3.0e38f;
            int bi = 0x7fffffff;
            const bool dbg = (a.flags & F_DBG_LOGITS) != 0;
            const float sc = in_scale();
#pragma unroll
            for (int e = 0; e < kMaxRowsWg / 64; ++e) {   // lmn <= 256 rows
                const int j = lane + 64 * e;
                if (j < W.lmn) {
                    const float v = rowsum(j) * sc * rsc(e);
                    const int r = W.lm0 + j;
                    if (dbg) gptr(a.dbg_logits)[(size_t)(it.step % 64) * D.V + r] = v;
                    if (v > bv || (v == bv && r < bi)) { bv = v; bi = r; }
                }
            }
            wave_argmax(bv, bi);
            if (lane == 0) {
                fw_store(a.ex.am + 2 * wg, __builtin_bit_cast(uint32_t, bv), id);
                fw_store(a.ex.am + 2 * wg + 1, (uint32_t)bi, id);
            }
            break;
        }
        default: break;
        }
    }

    // ---- phases the compute waves take no part in --------------------------
    __device__ __forceinline__ void solo(int kind, const PIter& it, int pos) {
        if (dead) return;
        if (kind == K_COMB) {
            combine(it.q, pos);
        } else if (kind == K_SAMPLE) {
            if (lm_skipped(a, it.step)) {
                tok = gptr(a.force_ids)[it.step];
                return;
            }
            if (!(W.nq || W.won || wg == 0)) return;   // this workgroup never reads the token
            KIE_LDS uint32_t* t = (KIE_LDS uint32_t*)S->att_q;   // scratch: 2 x 256 words
            if (!gather(a.ex.am, 2 * kGrid, id_of(it.q - 1), [&](int i, uint32_t v) { t[i] = v; })) return;
            float bv = -3.0e38f;
            int bi = 0x7fffffff;
            for (int w = lane; w < kGrid; w += 64) {
                const float v = __builtin_bit_cast(float, t[2 * w]);
                const int i = (int)t[2 * w + 1];
                if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
            }
            wave_argmax(bv, bi);
            int next = (bi >= 0 && bi < a.D.V) ? bi : 0;   // out of range only with NaN logits
            if (wg == 0 && lane == 0) gptr(a.out_ids)[it.step] = next;
            if (a.flags & F_FORCE) {
                const int f = gptr(a.force_ids)[it.step];
                if (f >= 0) next = f;
            }
            tok = next;
        }
    }

    // One trip of the combine gather: states t0 .. t0 + 64R - 1 (clamped to
    // T - 1, so every poll issues the same 4R loads and the compiler waits for
    // them once), polled until all carry ida, then staged in LDS as
    // [t][m, l, o0, o1]. Returns false when the wave gave up.
    template <int R>
    __device__ __forceinline__ bool combine_trip(int t0, int T, int p0, int nper, int g, int Gq, uint32_t ida,
                                                 KIE_LDS float* st) {
        const uint64_t* ad[R][4];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            int t = t0 + r * 64 + lane;
            t = t < T ? t : T - 1;
            const int pr = p0 + t / nper, ch = t % nper;
            const int idx = 2 * pr, head = g * Gq + idx / HD, dd = idx % HD;
            const uint64_t* pp = a.ex.part + ((size_t)head * a.items_per_head + ch) * (HD + 2);
            ad[r][0] = pp;
            ad[r][1] = pp + 1;
            ad[r][2] = pp + 2 + dd;
            ad[r][3] = pp + 3 + dd;
        }
        uint64_t w[R][4];
        uint32_t spins = 0;
        while (true) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int e = 0; e < 4; ++e) w[r][e] = fw_load(ad[r][e]);
            bool ok = true;
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int e = 0; e < 4; ++e) ok = fw_ok(w[r][e], ida) && ok;
            if (__builtin_amdgcn_ballot_w64(!ok) == 0) break;
            if (++spins > a.spin) {
                fail(1);
                return false;
            }
            if ((spins & 63) == 0 && stop_requested(a.status)) {
                fail(2);
                return false;
            }
#if KIE_POLL_SLEEP > 0
            __builtin_amdgcn_s_sleep(KIE_POLL_SLEEP);
#endif
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int t = t0 + r * 64 + lane;
            if (t < T)
#pragma unroll
                for (int e = 0; e < 4; ++e) st[t * 4 + e] = __builtin_bit_cast(float, fw_val(w[r][e]));
        }
        return true;
    }

    // Split attention: the workgroup of chunk c of KV group g combines the
    // nper partial states of its slice of the group's output pairs. Every
    // (pair, chunk) state is read in one trip (lanes over pairs x chunks),
    // staged in LDS, then a group of lanes per pair merges its chunks.
    __device__ __forceinline__ void combine(int q, int pos) {
        const Dims& D = a.D;
        int CH;
        if (head_mode(D, pos + 1)) return;   // every workgroup published its heads' o
        const int nper = attn_split(pos + 1, a.items_per_head, &CH);
        if (nper == 1 || wg >= D.Hkv * nper) return;
        const int Gq = D.H / D.Hkv, g = wg % D.Hkv, chunk = wg / D.Hkv;
        const int P = Gq * HD / 2;
        const int p0 = chunk * P / nper, p1 = (chunk + 1) * P / nper, np = p1 - p0;
        const int T = np * nper;   // (pair, chunk) states, at most P + nper <= 768
        const uint32_t ida = id_of(q - 1);
        KIE_LDS float* st = S->att_o;   // scratch: [T][4] (m, l, o0, o1)
        for (int t0 = 0; t0 < T; t0 += 8 * 64) {   // one trip unless T > 512
            const int per = (T - t0 + 63) / 64;
            bool ok;
            if (per <= 2) ok = combine_trip<2>(t0, T, p0, nper, g, Gq, ida, st);
            else if (per <= 4) ok = combine_trip<4>(t0, T, p0, nper, g, Gq, ida, st);
            else ok = combine_trip<8>(t0, T, p0, nper, g, Gq, ida, st);
            if (!ok) return;
        }
        // LP lanes per pair (a power of two, LP * np <= 64 where np allows):
        // each merges every LP-th chunk, then the LP lanes merge pairwise
        int LP = 64;
        while (LP > 1 && LP * np > 64) LP >>= 1;
        const int sl = lane % LP, PPR = 64 / LP;
        for (int j0 = 0; j0 < np; j0 += PPR) {
            const int j = j0 + lane / LP;
            float m = -3.0e38f, l = 0.f, o0 = 0.f, o1 = 0.f;
            if (j < np)
                for (int ch = sl; ch < nper; ch += LP) {
                    const KIE_LDS float* e = st + (j * nper + ch) * 4;
                    const float M = fmaxf(m, e[0]);
                    const float fo = __builtin_amdgcn_exp2f(m - M), fn = __builtin_amdgcn_exp2f(e[0] - M);
                    l = l * fo + e[1] * fn;
                    o0 = o0 * fo + e[2] * fn;
                    o1 = o1 * fo + e[3] * fn;
                    m = M;
                }
            for (int off = 1; off < LP; off <<= 1) {
                const float m2 = shfl_xor_f(m, off), l2 = shfl_xor_f(l, off);
                const float a0 = shfl_xor_f(o0, off), a1 = shfl_xor_f(o1, off);
                const float M = fmaxf(m, m2);
                const float fo = __builtin_amdgcn_exp2f(m - M), fn = __builtin_amdgcn_exp2f(m2 - M);
                l = l * fo + l2 * fn;
                o0 = o0 * fo + a0 * fn;
                o1 = o1 * fo + a1 * fn;
                m = M;
            }
            if (j < np && sl == 0) {
                const int idx = 2 * (p0 + j), head = g * Gq + idx / HD, dd = idx % HD;
                fw_store(a.ex.o + head * HD + dd, __builtin_bit_cast(uint32_t, o0 / l), id_of(q));
                fw_store(a.ex.o + head * HD + dd + 1, __builtin_bit_cast(uint32_t, o1 / l), id_of(q));
            }
        }
    }

    // phase timeline: event e of phase q at the constant 100 MHz clock
    __device__ __forceinline__ void stamp(int q, int e) {
        if ((a.flags & F_TRACE) && q < kTracePhases && lane == 0)
            gptr(a.trace)[((size_t)q * kGrid + wg) * 4 + e] = (int64_t)__builtin_amdgcn_s_memrealtime();
    }

    __device__ __forceinline__ void run() {
        const Dims& D = a.D;
        const int Q = a.n_steps * pps_of(D);
        // The exchange (polls, publications) is the critical path: let this
        // wave's instructions issue ahead of the compute waves' (their weight
        // DMA keeps the memory pipeline busy). Measured on the ~2.1B decoder:
        // +1.0% tok/s fp16, +0.1% fp8; MoE +0.3%.
        __builtin_amdgcn_s_setprio(3);
        PIter it{0, 0, 0, 0};
        for (; it.q < Q; advance(D, it)) {
            const int kind = kind_of(D, it);
            const int pos = a.pos0 + it.step;
            stamp(it.q, 0);
            if (phase_bars<XA>(a, kind, it.step, wg)) {
                if (shared_gather(S, kind, it.layer)) wg_barrier();   // the previous phases are done
                pre(kind, it);
                wg_barrier();   // every wave's share of the input is staged
                if (S->abort) dead = true;
                stamp(it.q, 1);
                wg_barrier();
                stamp(it.q, 2);
                post(kind, it, pos);
                if (kind == K_ATTN) wg_barrier();   // every slice is merged: att_o is free again
            } else {
                solo(kind, it, pos);
            }
            stamp(it.q, 3);
        }
        wait_vm0();
    }
};

// ------------------------------------------------------------------------
// Compute waves.
// ------------------------------------------------------------------------
// Each compute wave owns an LDS ring of kNS batches of kNB weight units,
// filled by LDS DMA in phase order and consumed oldest first. Every fill
// issues exactly kNB loads (a short batch tops up from the idle region, an
// idle batch loads only from it), so when the oldest batch is consumed the
// kNS-1 younger batches' loads are the only ones issued after it and
// vmcnt((kNS-1)*kNB) is the exact wait. A batch is refilled right after it
// is consumed, so up to kNS*kNB units stay in flight across phase
// boundaries while the communication wave waits for the next input.
struct Slot {
    int q, kind, layer, step, u0, n;   // n == 0: idle batch; q: the phase to reach before consuming it
};

// Geometry of one GEMV phase as seen by one compute wave (uniform values).
struct WaveGeo {
    int q, kind, layer;
    int n, nrows, K, nseg, off, row0;
    int lo, hi;   // this wave's unit range
    int upr;      // units per row segment (0: 256-wide rows, two per unit)
};

typedef float v2f_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

// Buffer resource over one KV head's cache rows of one layer: loads past
// `bytes` return zeros instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t kv_rsrc(const uint16_t* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, (int)bytes, 0x00020000);
}
// 16 bytes at byte offset off, device scope (sc1: rows appended by other
// workgroups earlier in the launch are seen); the compiler tracks the load.
__device__ __forceinline__ uint4 kv_load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16));
}
// Half t (0..7) of four 16-byte value rows, packed as the eight fp16 k slots of
// an MFMA operand: rows 0..3, then the same four again.
__device__ __forceinline__ h8_t v_col(const uint4 (&v)[4], int t) {
    uint32_t d[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t x = (t >> 1) == 0 ? v[r].x : (t >> 1) == 1 ? v[r].y : (t >> 1) == 2 ? v[r].z : v[r].w;
        d[r] = (t & 1) ? (x >> 16) : (x & 0xffffu);
    }
    const uint32_t lo = d[0] | (d[1] << 16), hi = d[2] | (d[3] << 16);
    typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
    const u4_t u = {lo, hi, lo, hi};
    return __builtin_bit_cast(h8_t, u);
}

// One fp8 unit against 8 fp32 inputs: the lane's 16 bytes are 8 E4M3 weights
// of row a then 8 of row b (the same 8 columns); each is converted exactly to
// fp32 (v_cvt_pk_f32_fp8, two per instruction) and multiplied-added into its
// row's accumulator.
__device__ __forceinline__ void dot8_fp8(uint4 w, const float (&x)[8], float& aa, float& ab) {
    v2f_t p;
    p = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false);
    aa = fmaf(p.x, x[0], aa);
    aa = fmaf(p.y, x[1], aa);
    p = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
    aa = fmaf(p.x, x[2], aa);
    aa = fmaf(p.y, x[3], aa);
    p = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false);
    aa = fmaf(p.x, x[4], aa);
    aa = fmaf(p.y, x[5], aa);
    p = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
    aa = fmaf(p.x, x[6], aa);
    aa = fmaf(p.y, x[7], aa);
    p = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.z, false);
    ab = fmaf(p.x, x[0], ab);
    ab = fmaf(p.y, x[1], ab);
    p = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.z, true);
    ab = fmaf(p.x, x[2], ab);
    ab = fmaf(p.y, x[3], ab);
    p = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.w, false);
    ab = fmaf(p.x, x[4], ab);
    ab = fmaf(p.y, x[5], ab);
    p = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.w, true);
    ab = fmaf(p.x, x[6], ab);
    ab = fmaf(p.y, x[7], ab);
}

// One fp4 unit against 8 fp32 inputs: the lane's 16 bytes are 4 bytes of
// each of 4 rows (the same 8 columns; byte b holds columns 2b (low nibble)
// and 2b+1); each E2M1 code converts exactly to fp32
// (v_cvt_scalef32_pk_f32_fp4 with scale 1, two per instruction) and is
// multiplied-added into its row's accumulator.
__device__ __forceinline__ void dot8_fp4(uint4 w, const float (&x)[8], float& a0, float& a1, float& a2, float& a3) {
    v2f_t p;
#define KIE_FP4_ROW(word, acc)                                     \
    p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((word), 1.0f, 0); \
    acc = fmaf(p.x, x[0], acc);                                    \
    acc = fmaf(p.y, x[1], acc);                                    \
    p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((word), 1.0f, 1); \
    acc = fmaf(p.x, x[2], acc);                                    \
    acc = fmaf(p.y, x[3], acc);                                    \
    p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((word), 1.0f, 2); \
    acc = fmaf(p.x, x[4], acc);                                    \
    acc = fmaf(p.y, x[5], acc);                                    \
    p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((word), 1.0f, 3); \
    acc = fmaf(p.x, x[6], acc);                                    \
    acc = fmaf(p.y, x[7], acc);
    KIE_FP4_ROW(w.x, a0)
    KIE_FP4_ROW(w.y, a1)
    KIE_FP4_ROW(w.z, a2)
    KIE_FP4_ROW(w.w, a3)
#undef KIE_FP4_ROW
}

// The 8 fp32 inputs of this lane in input segment c (512 elements).
__device__ __forceinline__ void load_xf(KIE_LDS Smem* S, int off, float (&x)[8]) {
    const uint4 u0 = lds_ld16(xf_of(S) + off), u1 = lds_ld16(xf_of(S) + off + 4);
    x[0] = __builtin_bit_cast(float, u0.x);
    x[1] = __builtin_bit_cast(float, u0.y);
    x[2] = __builtin_bit_cast(float, u0.z);
    x[3] = __builtin_bit_cast(float, u0.w);
    x[4] = __builtin_bit_cast(float, u1.x);
    x[5] = __builtin_bit_cast(float, u1.y);
    x[6] = __builtin_bit_cast(float, u1.z);
    x[7] = __builtin_bit_cast(float, u1.w);
}

template <int HD, int WF, bool MS, bool XA>
struct Compute {
    static constexpr bool W8 = WF != 0;   // quantised weights (fp8 or fp4)
    static constexpr bool W4 = WF == 2;   // fp4: four rows per unit
    const DecodeArgs& a;
    KIE_LDS Smem* S;
    int w, lane, wg, Q;
    uint32_t ring0;    // LDS byte address of this wave's ring
    PIter ic;          // issue cursor phase
    WaveGeo ig;        // its geometry
    int iu;            // next unit to issue in it
    int routed;        // last MoE gate/up phase whose routing is in LDS
    bool stop;         // the communication wave gave up: stream nothing more
    PIter cc;          // next phase to enter (or the entered one when `entered`)
    bool entered;
    WaveGeo cg;        // geometry of the phase being consumed
    int crow, cseg, ck;   // row, unit in the row segment and segment (MoE down: expert) of the next unit
    float acc;         // running partial dot product of the current row
    float acc2;        // fp8 weights: the second row of the current pair (crow counts pairs)
    float acc3, acc4;  // fp4 weights: the third and fourth rows of the current four (crow counts fours)

    __device__ __forceinline__ Compute(const DecodeArgs& args, KIE_LDS Smem* s, int wi) : a(args), S(s), w(wi) {
        lane = lane_id();
        wg = blockIdx.x;
        Q = a.n_steps * pps_of(a.D);
        ring0 = lds_addr_of(S->ring) + (uint32_t)(w * kNS * kBatchBytes);
        routed = -1;
        stop = false;
        cc = PIter{0, 0, 0, 0};
        entered = false;
        cg.q = -1;
        crow = cseg = ck = 0;
        acc = acc2 = acc3 = acc4 = 0.f;
        ic = PIter{0, 0, 0, 0};
        seek(false);
    }

    __device__ __forceinline__ void load_geo(WaveGeo& g, int q, int kind, int layer, int step) const {
        const KIE_LDS int* p = (const KIE_LDS int*)&S->geo[kind];
        g.q = q;
        g.kind = kind;
        g.layer = layer;
        g.n = (kind == K_LM && lm_skipped(a, step)) ? 0 : __builtin_amdgcn_readfirstlane(p[0]);
        g.nrows = __builtin_amdgcn_readfirstlane(p[1]);
        g.K = __builtin_amdgcn_readfirstlane(p[2]);
        g.nseg = __builtin_amdgcn_readfirstlane(p[3]);
        g.off = __builtin_amdgcn_readfirstlane(p[4]);
        g.row0 = __builtin_amdgcn_readfirstlane(p[5]);
        g.lo = g.n * w / kCompute;
        g.hi = g.n * (w + 1) / kCompute;
        g.upr = g.K / kUnitHalves;
    }

    // move the issue cursor (from ic, or past it when `next`) to the first
    // GEMV phase that has units for this wave
    __device__ __forceinline__ void seek(bool next) {
        if (next) advance(a.D, ic);
        for (; ic.q < Q; advance(a.D, ic)) {
            const int kind = kind_of(a.D, ic);
            if (!is_gemv(kind)) continue;
            load_geo(ig, ic.q, kind, ic.layer, ic.step);
            if (ig.hi > ig.lo) {
                iu = ig.lo;
                return;
            }
        }
    }

    // kNB loads into the batch at LDS address dst: units iu .. iu+n-1 of the
    // cursor phase, then units of the idle region
    __device__ __forceinline__ void load_units(uint32_t dst, int n) {
        const Dims& D = a.D;
        const uint8_t* idle = a.idle + lane * 16;
        const int kind = ig.kind;
        if (kind == K_EGU || kind == K_EDOWN) {
            // expert units come in contiguous runs (one per selected expert):
            // the address is worked out at the start of each run only
            const uint8_t* lb = a.experts + (size_t)ig.layer * D.E * a.expert_bytes + lane * 16;
            const int upr = ig.upr;
            const uint8_t* p = lb;
            int run = 0;
#pragma unroll
            for (int s = 0; s < kNB; ++s) {
                const uint8_t* src = idle + (size_t)s * kUnitBytes;
                if (s < n) {
                    if (run == 0) {
                        const int u = iu + s;
                        size_t off;
                        int k;
                        // fp8: units hold pairs of rows (one byte per weight), fp4
                        // fours (half a byte): unit counts run over pairs or fours
                        // and byte offsets shrink with the weight
                        constexpr int rpu = W4 ? 4 : W8 ? 2 : 1;   // rows per unit column
                        constexpr int wb2 = W4 ? 1 : W8 ? 2 : 4;   // twice the bytes per weight
                        if (kind == K_EGU) {
                            // virtual rows k * 2F + r: row r of the gate/up block of expert k
                            const int vr = ig.row0 + rpu * (u / upr), c = u - (u / upr) * upr;
                            k = vr / (2 * D.F);
                            const int rr = vr - k * 2 * D.F;
                            int vend = (k + 1) * 2 * D.F;
                            if (vend > ig.row0 + ig.nrows) vend = ig.row0 + ig.nrows;
                            run = ((vend - vr) / rpu) * upr - c;
                            off = (size_t)rr * D.d * wb2 / 2 + (size_t)c * kUnitBytes;
                        } else {
                            // expert-major: the workgroup's down rows of expert 0, then 1, ...
                            const int per = (ig.nrows / rpu) * upr;
                            k = u / per;
                            const int rem = u - k * per;
                            run = per - rem;
                            off = ((size_t)2 * D.F * D.d + (size_t)ig.row0 * D.F) * wb2 / 2 + (size_t)rem * kUnitBytes;
                        }
                        const int e = __builtin_amdgcn_readfirstlane(S->sel[k]);
                        p = lb + (size_t)e * a.expert_bytes + off;
                    }
                    src = p;
                    p += kUnitBytes;
                    --run;
                }
                dma_unit(src, dst + s * kUnitBytes);
            }
        } else {
            // contiguous units: one m0 per four, the instruction offset steps both addresses
            static_assert(kNB % 4 == 0, "dense batches are issued in fours");
            const uint8_t* base = (kind == K_LM) ? a.lm : a.layers + (size_t)ig.layer * a.layer_bytes;
            const uint8_t* src = base + (size_t)(ig.off + iu) * kUnitBytes + lane * 16;
#pragma unroll
            for (int g = 0; g < kNB; g += 4) {
                const uint8_t* sg = src + (size_t)g * kUnitBytes;
                const uint8_t* ig4 = idle + (size_t)g * kUnitBytes;
                dma_unit4(g + 0 < n ? sg : ig4, g + 1 < n ? sg : ig4, g + 2 < n ? sg : ig4, g + 3 < n ? sg : ig4,
                          dst + g * kUnitBytes);
            }
        }
    }

    __device__ __forceinline__ void load_idle(uint32_t dst) {
        const uint8_t* idle = a.idle + lane * 16;
#pragma unroll
        for (int g = 0; g < kNB; g += 4) {
            const uint8_t* ig4 = idle + (size_t)g * kUnitBytes;
            dma_unit4(ig4, ig4, ig4, ig4, dst + g * kUnitBytes);
        }
    }

    // Refill the batch at dst: the next units in phase order, or an idle batch
    // tagged with the phase whose first barrier must pass before issue can go
    // on (the MoE gate/up phase of a blocked layer) or with Q (nothing left).
    __device__ __forceinline__ Slot fill(uint32_t dst) {
        if (!stop && ic.q < Q) {
            const int gate = ig.kind == K_EGU ? ic.q : (ig.kind == K_EDOWN ? ic.q - 1 : -1);
            if (gate <= routed) {
                const int n = (ig.hi - iu < kNB) ? ig.hi - iu : kNB;
                load_units(dst, n);
                const Slot sl{ic.q, ig.kind, ic.layer, ic.step, iu, n};
                iu += n;
                if (iu >= ig.hi) seek(true);
                return sl;
            }
            load_idle(dst);
            return Slot{gate, 0, 0, 0, 0, 0};
        }
        load_idle(dst);
        return Slot{Q, 0, 0, 0, 0, 0};
    }

    __device__ __forceinline__ void enter() {
        const int kind = kind_of(a.D, cc);
        if (!phase_bars<XA>(a, kind, cc.step, wg)) return;
        if (shared_gather(S, kind, cc.layer)) {
            wg_barrier();   // the communication wave is done with the previous phases
            if (!stop) {
                const int n = __builtin_amdgcn_readfirstlane(S->geo[kind].gin);
                const int r = gather_input<W8, XA>(a, S, kind, n, a.id0 + (uint32_t)(cc.q - 1), w + 1,
                                               a.pos0 + cc.step + 1);
                if (r && lane == 0) {
                    if (r == 1) sys_store32(a.status, (uint32_t)kStatusTimeout);
                    S->abort = 1u;
                }
            }
        }
        wg_barrier();   // the input (and the routing, for MoE gate/up) is in LDS
        stop = S->abort != 0u;
        if (kind == K_EGU) routed = cc.q;
    }

    __device__ __forceinline__ void finish() {
        const int kind = kind_of(a.D, cc);
        if (!phase_bars<XA>(a, kind, cc.step, wg)) return;
        if (kind == K_ATTN && !stop && head_mode(a.D, a.pos0 + cc.step + 1)) {
            const int it = attn_item<XA>(a, a.pos0 + cc.step + 1, wg);
            attention<1>(cc.layer, a.pos0 + cc.step, (it % a.D.H) / a.D.Hkv);   // one head, one chunk
        } else if (kind == K_ATTN && !stop) {
            const int G = a.D.H / a.D.Hkv, l = cc.layer, pos = a.pos0 + cc.step;
            // register arrays sized for the group (1, 2, 4 or 5 heads; 6 to 8
            // heads in two passes over the positions); head_dim 128 on the
            // matrix cores
            if constexpr (HD == 128 && MS) attention_mfma(l, pos);   // mfma_attention() holds here
            else if (G == 1) attention<1>(l, pos);
            else if (G == 2) attention<2>(l, pos);
            else if (G <= 4) attention<4>(l, pos);
            else if (G == 5) attention<5>(l, pos);
            else {
                attention<4>(l, pos, 0);
                attention<4>(l, pos, 4);
            }
        }
        wg_barrier();   // partial sums / attention states are in LDS
        if (kind == K_ATTN) {
            if (!stop) (void)attn_merge<HD, XA>(a, S, a.pos0 + cc.step, a.id0 + (uint32_t)cc.q, w + 1);   // no polls here
            wg_barrier();
        }
    }

    // When the batch just consumed was this wave's last of the entered phase
    // (the next batch belongs to a later phase), finish the phase before the
    // refill: issuing the refill may wait for the memory pipeline, and the
    // phase's epilogue should not.
    __device__ __forceinline__ void finish_if_done(const Slot (&sq)[kNS]) {
        static_assert(kNS >= 2, "the ring holds at least two batches");
        if (entered && sq[0].n > 0 && !stop && sq[0].q == cc.q && sq[1].q != cc.q) {
            // a GEMV phase (the batch had units): finishing it is its second barrier
            if (phase_bars<XA>(a, kind_of(a.D, cc), cc.step, wg)) wg_barrier();
            advance(a.D, cc);
            entered = false;
        }
    }

    // Afterwards phase qx is entered and not finished (qx == Q: all finished).
    __device__ __forceinline__ void goto_phase(int qx) {
        while (true) {
            if (entered) {
                if (cc.q == qx) return;
                finish();
                advance(a.D, cc);
                entered = false;
            }
            if (cc.q >= Q) return;
            enter();
            entered = true;
        }
    }

    // Consume one batch with the phase's input segments in registers: xh[j],
    // xq[j] hold the hi and lo terms of segment (cseg + j) % UPR, so unit s of
    // the batch uses xh[s % UPR]; a full batch rotates them by kNB % UPR.
    template <int UPR>
    __device__ __forceinline__ void consume_reg(uint32_t src, const Slot& sl, uint4 (&xh)[UPR], uint4 (&xq)[UPR]) {
        const KIE_LDS uint8_t* wb = (const KIE_LDS uint8_t*)(uintptr_t)src + lane * 16;
        uint4 wv[kNB];
#pragma unroll
        for (int s = 0; s < kNB; ++s)
            if (s < sl.n) wv[s] = lds_ld16(wb + s * kUnitBytes);
        const int last = cg.hi - 1 - sl.u0;   // batch index of the range's last unit
#pragma unroll
        for (int s = 0; s < kNB; ++s) {
            if (s < sl.n) {
                acc = dot8(wv[s], xq[s % UPR], dot8(wv[s], xh[s % UPR], acc));
                const bool seg_done = cseg + 1 == UPR;
                if (seg_done || s == last) {
                    const float r = wave_sum_to_lane63(acc);
                    if (lane == 63) S->part[crow * kCompute + w] += r;
                    acc = 0.f;
                }
                if (seg_done) {
                    cseg = 0;
                    ++crow;
                } else {
                    ++cseg;
                }
            }
        }
        constexpr int R = kNB % UPR;
        if (R && sl.n == kNB) {   // a short batch ends the wave's range: nothing follows in this phase
            uint4 th[UPR], tq[UPR];
#pragma unroll
            for (int j = 0; j < UPR; ++j) {
                th[j] = xh[(j + R) % UPR];
                tq[j] = xq[(j + R) % UPR];
            }
#pragma unroll
            for (int j = 0; j < UPR; ++j) {
                xh[j] = th[j];
                xq[j] = tq[j];
            }
        }
    }

    // fp8 weights: the same with pairs of rows per unit; xf[j] holds the fp32
    // input of segment (cseg + j) % UPR.
    template <int UPR>
    __device__ __forceinline__ void consume_reg_fp8(uint32_t src, const Slot& sl, float (&xf)[UPR][8]) {
        const KIE_LDS uint8_t* wb = (const KIE_LDS uint8_t*)(uintptr_t)src + lane * 16;
        uint4 wv[kNB];
#pragma unroll
        for (int s = 0; s < kNB; ++s)
            if (s < sl.n) wv[s] = lds_ld16(wb + s * kUnitBytes);
        const int last = cg.hi - 1 - sl.u0;
#pragma unroll
        for (int s = 0; s < kNB; ++s) {
            if (s < sl.n) {
                dot8_fp8(wv[s], xf[s % UPR], acc, acc2);
                const bool seg_done = cseg + 1 == UPR;
                if (seg_done || s == last) {
                    const float ra = wave_sum_to_lane63(acc), rb = wave_sum_to_lane63(acc2);
                    if (lane == 63) {
                        S->part[(2 * crow) * kCompute + w] += ra;
                        S->part[(2 * crow + 1) * kCompute + w] += rb;
                    }
                    acc = acc2 = 0.f;
                }
                if (seg_done) {
                    cseg = 0;
                    ++crow;
                } else {
                    ++cseg;
                }
            }
        }
        constexpr int R = kNB % UPR;
        if (R && sl.n == kNB) {
            float t[UPR][8];
#pragma unroll
            for (int j = 0; j < UPR; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) t[j][e] = xf[(j + R) % UPR][e];
#pragma unroll
            for (int j = 0; j < UPR; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) xf[j][e] = t[j][e];
        }
    }

    // fp4 weights: the same with fours of rows per unit (crow counts fours).
    template <int UPR>
    __device__ __forceinline__ void consume_reg_fp4(uint32_t src, const Slot& sl, float (&xf)[UPR][8]) {
        const KIE_LDS uint8_t* wb = (const KIE_LDS uint8_t*)(uintptr_t)src + lane * 16;
        uint4 wv[kNB];
#pragma unroll
        for (int s = 0; s < kNB; ++s)
            if (s < sl.n) wv[s] = lds_ld16(wb + s * kUnitBytes);
        const int last = cg.hi - 1 - sl.u0;
#pragma unroll
        for (int s = 0; s < kNB; ++s) {
            if (s < sl.n) {
                dot8_fp4(wv[s], xf[s % UPR], acc, acc2, acc3, acc4);
                const bool seg_done = cseg + 1 == UPR;
                if (seg_done || s == last) {
                    const float r0 = wave_sum_to_lane63(acc), r1 = wave_sum_to_lane63(acc2);
                    const float r2 = wave_sum_to_lane63(acc3), r3 = wave_sum_to_lane63(acc4);
                    if (lane == 63) {
                        S->part[(4 * crow) * kCompute + w] += r0;
                        S->part[(4 * crow + 1) * kCompute + w] += r1;
                        S->part[(4 * crow + 2) * kCompute + w] += r2;
                        S->part[(4 * crow + 3) * kCompute + w] += r3;
                    }
                    acc = acc2 = acc3 = acc4 = 0.f;
                }
                if (seg_done) {
                    cseg = 0;
                    ++crow;
                } else {
                    ++cseg;
                }
            }
        }
        constexpr int R = kNB % UPR;
        if (R && sl.n == kNB) {
            float t[UPR][8];
#pragma unroll
            for (int j = 0; j < UPR; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) t[j][e] = xf[(j + R) % UPR][e];
#pragma unroll
            for (int j = 0; j < UPR; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) xf[j][e] = t[j][e];
        }
    }

    // Consume every batch of the current phase at the head of the ring with
    // the input in registers (rows of UPR units, one input segment for all
    // rows), refilling each batch as it goes. On return sq[0] belongs to a
    // later phase (or is idle).
    template <int UPR>
    __device__ __forceinline__ void stream_phase(Slot (&sq)[kNS], int& head) {
        const int q = sq[0].q;
        if (cg.q != q) enter_geo(sq[0]);
        if constexpr (W8) {
            float xf[UPR][8];
#pragma unroll
            for (int j = 0; j < UPR; ++j) load_xf(S, ((cseg + j) % UPR) * kUnitHalves + lane * 8, xf[j]);
            while (sq[0].q == q && sq[0].n > 0) {
                const uint32_t at = ring0 + head * kBatchBytes;
                wait_vm<(kNS - 1) * kNB>();
                if constexpr (W4) consume_reg_fp4<UPR>(at, sq[0], xf);
                else consume_reg_fp8<UPR>(at, sq[0], xf);
                wait_lgkm0();
                finish_if_done(sq);
                const Slot t = fill(at);
#pragma unroll
                for (int i = 0; i + 1 < kNS; ++i) sq[i] = sq[i + 1];
                sq[kNS - 1] = t;
                head = (head + 1 == kNS) ? 0 : head + 1;
            }
            return;
        }
        uint4 xh[UPR], xq[UPR];
#pragma unroll
        for (int j = 0; j < UPR; ++j) {
            const int c = (cseg + j) % UPR;
            xh[j] = lds_ld16(S->xin + c * kUnitHalves + lane * 8);
            xq[j] = lds_ld16(S->xlo + c * kUnitHalves + lane * 8);
        }
        while (sq[0].q == q && sq[0].n > 0) {
            const uint32_t at = ring0 + head * kBatchBytes;
            wait_vm<(kNS - 1) * kNB>();
            consume_reg<UPR>(at, sq[0], xh, xq);
            wait_lgkm0();   // this batch's LDS reads are done before it is overwritten
            finish_if_done(sq);
            const Slot t = fill(at);
#pragma unroll
            for (int i = 0; i + 1 < kNS; ++i) sq[i] = sq[i + 1];
            sq[kNS - 1] = t;
            head = (head + 1 == kNS) ? 0 : head + 1;
        }
    }

    // consume the batch at LDS address src: all LDS reads of the batch are
    // issued before the first product. Units run through row segments of upr
    // units, rows 0 .. nrows-1, then (MoE down) the same rows for the next
    // selected expert, whose input follows in xin; a segment's partial dot
    // product is added to the (row, wave) partial sum.
    // geometry of the phase of batch sl, and the position of its first unit
    __device__ __forceinline__ void enter_geo(const Slot& sl) {
        load_geo(cg, sl.q, sl.kind, sl.layer, sl.step);
        if (cg.upr) {
            // crow counts rows (fp8: pairs of rows, two per unit; fp4: fours)
            const int per_seg = (W4 ? cg.nrows / 4 : W8 ? cg.nrows / 2 : cg.nrows) * cg.upr;
            ck = cg.lo / per_seg;
            const int rem = cg.lo - ck * per_seg;
            crow = rem / cg.upr;
            cseg = rem - crow * cg.upr;   // unit position within the row segment
        }
    }

    // fp8 weights, any row length: the inputs of each unit read from LDS.
    // MoE down (ck = selected expert, its input segment ck of xf): each
    // expert's row partial sum is scaled by that expert's row scale before
    // it joins the row's sum over experts.
    __device__ __forceinline__ void consume_fp8(uint32_t src, const Slot& sl) {
        const KIE_LDS uint8_t* wb = (const KIE_LDS uint8_t*)(uintptr_t)src + lane * 16;
        const int upr = cg.upr, npair = cg.nrows / 2;
        const bool edown = cg.kind == K_EDOWN;
        uint4 wv[kNB];
#pragma unroll
        for (int s = 0; s < kNB; ++s)
            if (s < sl.n) wv[s] = lds_ld16(wb + s * kUnitBytes);
        const int last = cg.hi - 1 - sl.u0;
#pragma unroll
        for (int s = 0; s < kNB; ++s) {
            if (s < sl.n) {
                float x[8];
                load_xf(S, ck * cg.K + cseg * kUnitHalves + lane * 8, x);
                dot8_fp8(wv[s], x, acc, acc2);
                const bool seg_done = cseg + 1 == upr;
                if (seg_done || s == last) {
                    float ra = wave_sum_to_lane63(acc), rb = wave_sum_to_lane63(acc2);
                    if (edown) {
                        ra *= S->esc[ck * cg.nrows + 2 * crow];
                        rb *= S->esc[ck * cg.nrows + 2 * crow + 1];
                    }
                    if (lane == 63) {
                        S->part[(2 * crow) * kCompute + w] += ra;
                        S->part[(2 * crow + 1) * kCompute + w] += rb;
                    }
                    acc = acc2 = 0.f;
                }
                if (seg_done) {
                    cseg = 0;
                    if (++crow == npair) {
                        crow = 0;
                        ++ck;
                    }
                } else {
                    ++cseg;
                }
            }
        }
    }

    // fp4 weights, any row length: the inputs of each unit read from LDS, fours
    // of rows per unit. ED (MoE down) as in consume_fp8: ck = selected expert,
    // its input segment and its row scales on the row partial sums.
    template <bool ED>
    __device__ __forceinline__ void consume_fp4(uint32_t src, const Slot& sl) {
        const KIE_LDS uint8_t* wb = (const KIE_LDS uint8_t*)(uintptr_t)src + lane * 16;
        const int upr = cg.upr, nquad = cg.nrows / 4;
        uint4 wv[kNB];
#pragma unroll
        for (int s = 0; s < kNB; ++s)
            if (s < sl.n) wv[s] = lds_ld16(wb + s * kUnitBytes);
        const int last = cg.hi - 1 - sl.u0;
#pragma unroll
        for (int s = 0; s < kNB; ++s) {
            if (s < sl.n) {
                float x[8];
                load_xf(S, (ED ? ck * cg.K : 0) + cseg * kUnitHalves + lane * 8, x);
                dot8_fp4(wv[s], x, acc, acc2, acc3, acc4);
                const bool seg_done = cseg + 1 == upr;
                if (seg_done || s == last) {
                    float r0 = wave_sum_to_lane63(acc), r1 = wave_sum_to_lane63(acc2);
                    float r2 = wave_sum_to_lane63(acc3), r3 = wave_sum_to_lane63(acc4);
                    if constexpr (ED) {
                        const KIE_LDS float* e = S->esc + ck * cg.nrows + 4 * crow;
                        r0 *= e[0];
                        r1 *= e[1];
                        r2 *= e[2];
                        r3 *= e[3];
                    }
                    if (lane == 63) {
                        S->part[(4 * crow) * kCompute + w] += r0;
                        S->part[(4 * crow + 1) * kCompute + w] += r1;
                        S->part[(4 * crow + 2) * kCompute + w] += r2;
                        S->part[(4 * crow + 3) * kCompute + w] += r3;
                    }
                    acc = acc2 = acc3 = acc4 = 0.f;
                }
                if (seg_done) {
                    cseg = 0;
                    ++crow;
                    if (ED && crow == nquad) {
                        crow = 0;
                        ++ck;
                    }
                } else {
                    ++cseg;
                }
            }
        }
    }

    __device__ __forceinline__ void consume(uint32_t src, const Slot& sl) {
        if (cg.q != sl.q) enter_geo(sl);
        if constexpr (W4) {
            if (cg.kind == K_EDOWN) consume_fp4<true>(src, sl);
            else consume_fp4<false>(src, sl);
            return;
        } else if constexpr (W8) {
            consume_fp8(src, sl);
            return;
        }
        const KIE_LDS uint8_t* wb = (const KIE_LDS uint8_t*)(uintptr_t)src + lane * 16;
        uint4 wv[kNB], xv[kNB], xl[kNB];
        if (cg.upr) {
            const int upr = cg.upr, nrows = cg.nrows;
            int rs = cseg, rr = crow, rk = ck;
#pragma unroll
            for (int s = 0; s < kNB; ++s) {
                if (s < sl.n) {
                    const int xo = rk * cg.K + rs * kUnitHalves + lane * 8;
                    wv[s] = lds_ld16(wb + s * kUnitBytes);
                    xv[s] = lds_ld16(S->xin + xo);
                    xl[s] = lds_ld16(S->xlo + xo);
                    if (++rs == upr) {
                        rs = 0;
                        if (++rr == nrows) {
                            rr = 0;
                            ++rk;
                        }
                    }
                }
            }
            const int last = cg.hi - 1 - sl.u0;   // batch index of the range's last unit
#pragma unroll
            for (int s = 0; s < kNB; ++s) {
                if (s < sl.n) {
                    acc = dot8(wv[s], xl[s], dot8(wv[s], xv[s], acc));
                    const bool seg_done = cseg + 1 == upr;
                    if (seg_done || s == last) {
                        const float r = wave_sum_to_lane63(acc);
                        if (lane == 63) S->part[crow * kCompute + w] += r;
                        acc = 0.f;
                    }
                    if (seg_done) {
                        cseg = 0;
                        if (++crow == nrows) {
                            crow = 0;
                            ++ck;
                        }
                    } else {
                        ++cseg;
                    }
                }
            }
        } else {
            // 256-wide rows: one unit holds two rows (lanes 0-31 and 32-63)
            const uint4 x = lds_ld16(S->xin + (lane & 31) * 8);
            const uint4 xlo = lds_ld16(S->xlo + (lane & 31) * 8);
#pragma unroll
            for (int s = 0; s < kNB; ++s)
                if (s < sl.n) wv[s] = lds_ld16(wb + s * kUnitBytes);
#pragma unroll
            for (int s = 0; s < kNB; ++s) {
                if (s < sl.n) {
                    const float r = half32_sum_from_rows(row16_sum(dot8(wv[s], xlo, dot8(wv[s], x, 0.f))));
                    const int row = 2 * (sl.u0 + s) + (lane >> 5);
                    if ((lane & 31) == 31 && row < cg.nrows) S->part[row * kCompute + w] = r;
                }
            }
        }
    }

    __device__ __forceinline__ void run() {
        Slot sq[kNS];   // batches in issue order; sq[i] sits at ring slot (head + i) % kNS
        int head = 0;
#pragma unroll
        for (int i = 0; i < kNS; ++i) sq[i] = fill(ring0 + i * kBatchBytes);
        while (cc.q < Q) {
            const uint32_t at = ring0 + head * kBatchBytes;
            goto_phase(sq[0].q);   // sq[0].q == Q once nothing is left: finishes every phase
            if (sq[0].n > 0 && !stop && sq[0].kind != K_EDOWN) {
                // rows of at most 5 units share one input segment set: keep it in registers
                const int upr = __builtin_amdgcn_readfirstlane(S->geo[sq[0].kind].K) / kUnitHalves;
                if (upr == 5) { stream_phase<5>(sq, head); continue; }
                if (upr == 4) { stream_phase<4>(sq, head); continue; }
            }
            wait_vm<(kNS - 1) * kNB>();
            if (sq[0].n > 0 && !stop) consume(at, sq[0]);
            wait_lgkm0();          // this batch's LDS reads are done before it is overwritten
            finish_if_done(sq);
            const Slot t = fill(at);
#pragma unroll
            for (int i = 0; i + 1 < kNS; ++i) sq[i] = sq[i + 1];
            sq[kNS - 1] = t;
            head = (head + 1 == kNS) ? 0 : head + 1;
        }
        wait_vm0();
    }

    // Split attention on the matrix cores (head_dim 128, at most 8 query heads
    // per KV head, so they fit the 16 columns): this workgroup's chunk of a KV
    // group's positions. Each compute wave takes every 7th round of 16
    // positions of the chunk. The scores come out transposed,
    // S^T = K Q^T on v_mfma_f32_16x16x32_f16: the keys are the A operand,
    // 16 contiguous bytes of a cache row per lane and step, the queries the B
    // operand as two fp16 terms (hi, lo) in two products, read from LDS. Lane l then holds
    // the scores of head l%16 at positions 4(l/16) .. 4(l/16)+3, which is the
    // B operand of O^T = V^T P^T with P as two fp16 terms (k slots: the four
    // positions' hi terms, then their lo terms, against the same four values
    // twice). Row i of output block t (t = 0..7) is dimension 8i + t, so the
    // A operand reads 16 contiguous bytes of each value row too. Each lane
    // keeps the online-softmax state of its head (the maximum, equal on the
    // four lanes of a head, and a partial sum) and O^T block t, whose rows
    // 4(l/16)+r are dimensions 8(4(l/16)+r) + t. The next round's keys and
    // values are loaded while a round is computed.
    __device__ __forceinline__ void attention_mfma(int layer, int pos) {
        static_assert(HD == 128, "the operand layouts are for head_dim 128");
        const Dims& D = a.D;
        int CH;
        const int c = pos + 1;
        attn_split(c, a.items_per_head, &CH);
        const int Gq = D.H / D.Hkv;
        const int g = wg % D.Hkv, chunk = wg / D.Hkv;
        const int p0 = chunk * CH, p1 = (p0 + CH < c) ? p0 + CH : c;
        const int li = lane & 15, lg = lane >> 4;
        // B operands of the scores: the queries' two fp16 terms, staged in LDS
        // by the communication wave (columns past the group read zeros)
        const int qrow = (li < Gq ? li : 0) * HD + 8 * lg;
        const bool qon = li < Gq;
        auto qop = [&](const KIE_LDS uint16_t* base, int s) {
            // read in every round, not held across rounds: the opaque copy of
            // the row offset keeps the compiler from hoisting the reads (32
            // registers) out of the loop
            int r = qrow;
            asm volatile("" : "+v"(r));
            const uint4 u = lds_ld16(base + r + 32 * s);
            return __builtin_bit_cast(h8_t, qon ? u : make_uint4(0u, 0u, 0u, 0u));
        };
        const size_t kvoff = ((size_t)layer * D.Hkv + g) * D.max_seq * HD;
        const uint32_t kvbytes = (uint32_t)D.max_seq * HD * 2u;
        const __amdgpu_buffer_rsrc_t kr = kv_rsrc(a.kc + kvoff, kvbytes), vr = kv_rsrc(a.vc + kvoff, kvbytes);
        float m = -3.0e38f, ls = 0.f;
        f4_t o[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) o[t] = f4_t{0.f, 0.f, 0.f, 0.f};
        constexpr int kStep = 16 * kCompute;
        // rows past the chunk (padding, and every row of a round past its end)
        // and at or past pos (the new position, whose row may not be visible
        // yet) are read from row 0 and replaced or masked below
        auto issue = [&](int bb, uint4 (&kx)[4], uint4 (&vx)[4]) {
            const int pk = bb + li, sk = (pk < pos && pk < p1) ? pk : 0;
#pragma unroll
            for (int s = 0; s < 4; ++s) kx[s] = kv_load(kr, (uint32_t)(sk * HD + 32 * s + 8 * lg) * 2u);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int pv = bb + 4 * lg + r, sv = (pv < pos && pv < p1) ? pv : 0;
                vx[r] = kv_load(vr, (uint32_t)(sv * HD + 8 * li) * 2u);
            }
        };
        auto round = [&](int b, uint4 (&kw)[4], uint4 (&vw)[4]) {
            if (b + 16 > pos) {
                // this round holds the new position: its key and value from LDS
                // (and every padding row too, so that all values are finite)
                if (b + li >= pos)
#pragma unroll
                    for (int s = 0; s < 4; ++s) kw[s] = lds_ld16(S->att_k + 32 * s + 8 * lg);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (b + 4 * lg + r >= pos) vw[r] = lds_ld16(S->att_v + 8 * li);
            }
            f4_t sc = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const h8_t kh = __builtin_bit_cast(h8_t, kw[s]);
                sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kh, qop(S->att_qh, s), sc, 0, 0, 0);
                sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kh, qop(S->att_ql, s), sc, 0, 0, 0);
            }
            float sr[4], mx = m;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sr[r] = (b + 4 * lg + r < p1) ? sc[r] : -3.0e38f;
                mx = fmaxf(mx, sr[r]);
            }
            mx = fmaxf(mx, shfl_xor_f(mx, 16));
            mx = fmaxf(mx, shfl_xor_f(mx, 32));
            const float cr = __builtin_amdgcn_exp2f(m - mx);
            float pr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) pr[r] = sr[r] > -1.0e38f ? __builtin_amdgcn_exp2f(sr[r] - mx) : 0.f;
            ls = ls * cr + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
            m = mx;
            if (__builtin_amdgcn_ballot_w64(cr != 1.f) != 0)
#pragma unroll
                for (int t = 0; t < 8; ++t) o[t] *= cr;
            h8_t pb;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const _Float16 h = (_Float16)pr[r];
                pb[r] = h;
                pb[4 + r] = (_Float16)(pr[r] - (float)h);
            }
#pragma unroll
            for (int t = 0; t < 8; ++t) o[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v_col(vw, t), pb, o[t], 0, 0, 0);
        };
        // two rounds of keys and values in flight per wave: the round being
        // computed and the next one (issued unconditionally, past the chunk
        // from row 0, so every wait the compiler places is vmcnt(8))
        uint4 ka[4], va[4], kb[4], vb[4];
        int b = p0 + 16 * w;
        issue(b, ka, va);
        while (b < p1) {
            issue(b + kStep, kb, vb);
            round(b, ka, va);
            b += kStep;
            if (b >= p1) break;
            issue(b + kStep, ka, va);
            round(b, kb, vb);
            b += kStep;
        }
        ls += shfl_xor_f(ls, 16);
        ls += shfl_xor_f(ls, 32);
        if (li < Gq) {
            KIE_LDS float* ob = S->att_o + (w * kMaxGroup + li) * HD;
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int t = 0; t < 8; ++t) ob[8 * (4 * lg + r) + t] = o[t][r];
            if (lg == 0) {
                S->att_ml[(w * kMaxGroup + li) * 2] = m;
                S->att_ml[(w * kMaxGroup + li) * 2 + 1] = ls;
            }
        }
    }

    // Attention of this workgroup's chunk: each compute wave takes every 7th
    // block of positions, keeps an online-softmax state per query head of the
    // group (GB >= heads per group), and leaves it in LDS for the
    // communication wave to merge. Lanes: HD/8 per position, 8 dims each; a
    // round reads the keys and values of 4 x 64/(HD/8) positions in one trip.
    template <int GB>
    __device__ __forceinline__ void attention(int layer, int pos, int h0 = 0) {
        const Dims& D = a.D;
        constexpr int LPP = HD / 8;       // lanes per position
        constexpr int PPI = 64 / LPP;     // positions per wave instruction
        constexpr int U = 4;              // instructions per round
        int CH;
        const int c = pos + 1;
        const bool hm = head_mode(D, c);
        if (hm) CH = ceil_div(c, head_chunks(a, c));
        else attn_split(c, a.items_per_head, &CH);
        const int Gq = (D.H / D.Hkv - h0 < GB) ? D.H / D.Hkv - h0 : GB;   // heads h0 .. h0 + Gq - 1
        const int it = attn_item<XA>(a, c, wg);
        const int g = it % D.Hkv, chunk = hm ? it / D.H : it / D.Hkv;
        const int p0 = chunk * CH, p1 = (p0 + CH < c) ? p0 + CH : c;
        const int gi = lane / LPP, dl = (lane % LPP) * 8;
        float qv[GB][8];
#pragma unroll
        for (int j = 0; j < GB; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) qv[j][e] = (j < Gq) ? S->att_q[(h0 + j) * HD + dl + e] : 0.f;
        float m[GB], ls[GB], o[GB][8];
#pragma unroll
        for (int j = 0; j < GB; ++j) {
            m[j] = -3.0e38f;
            ls[j] = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[j][e] = 0.f;
        }
        const uint16_t* Kb = a.kc + ((size_t)layer * D.Hkv + g) * D.max_seq * HD;
        const uint16_t* Vb = a.vc + ((size_t)layer * D.Hkv + g) * D.max_seq * HD;
        const uint4 knew = lds_ld16(S->att_k + dl);
        const uint4 vnew = lds_ld16(S->att_v + dl);
        static_assert(U == 4, "the cache loads below come in fours");
        for (int b = p0 + w * PPI * U; b < p1; b += kCompute * PPI * U) {
            uint4 kw[U], vw[U];
            const uint16_t* kp[U];
            const uint16_t* vp[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int pp = b + u * PPI + gi;
                const int src = (pp < pos && pp < p1) ? pp : 0;   // in-bounds address for every lane
                kp[u] = Kb + (size_t)src * HD + dl;
                vp[u] = Vb + (size_t)src * HD + dl;
            }
            dev_load128x8_sync(kp[0], kp[1], kp[2], kp[3], vp[0], vp[1], vp[2], vp[3], kw[0], kw[1], kw[2], kw[3],
                               vw[0], vw[1], vw[2], vw[3]);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int pp = b + u * PPI + gi;
                if (!(pp < pos && pp < p1)) {
                    kw[u] = knew;   // the new position (or padding, masked below)
                    vw[u] = vnew;
                }
            }
            // the round's scores first, then one online-softmax update per head
            float vf[U][8], sc[U][GB];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float kf[8];
                const uint32_t kk[4] = {kw[u].x, kw[u].y, kw[u].z, kw[u].w};
                const uint32_t vv[4] = {vw[u].x, vw[u].y, vw[u].z, vw[u].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kf[2 * e] = h2f_bits((uint16_t)kk[e]);
                    kf[2 * e + 1] = h2f_bits((uint16_t)(kk[e] >> 16));
                    vf[u][2 * e] = h2f_bits((uint16_t)vv[e]);
                    vf[u][2 * e + 1] = h2f_bits((uint16_t)(vv[e] >> 16));
                }
                const bool valid = b + u * PPI + gi < p1;
#pragma unroll
                for (int j = 0; j < GB; ++j) {
                    float d = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) d += qv[j][e] * kf[e];
                    d = LPP == 16 ? row16_sum(d) : row8_sum(d);
                    sc[u][j] = valid ? d : -3.0e38f;
                }
            }
#pragma unroll
            for (int j = 0; j < GB; ++j) {
                if (j < Gq) {
                    float mx = m[j];
#pragma unroll
                    for (int u = 0; u < U; ++u) mx = fmaxf(mx, sc[u][j]);
                    const float cr = __builtin_amdgcn_exp2f(m[j] - mx);
                    float pr[U];
#pragma unroll
                    for (int u = 0; u < U; ++u)   // padding positions weigh nothing
                        pr[u] = sc[u][j] > -1.0e38f ? __builtin_amdgcn_exp2f(sc[u][j] - mx) : 0.f;
                    ls[j] = ls[j] * cr + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        o[j][e] = o[j][e] * cr + ((pr[0] * vf[0][e] + pr[1] * vf[1][e]) +
                                                  (pr[2] * vf[2][e] + pr[3] * vf[3][e]));
                    m[j] = mx;
                }
            }
        }
        // merge the position groups of this wave
#pragma unroll
        for (int off = LPP; off < 64; off <<= 1) {
#pragma unroll
            for (int j = 0; j < GB; ++j) {
                if (j < Gq) {
                    const float m2 = shfl_xor_f(m[j], off), l2 = shfl_xor_f(ls[j], off);
                    const float mn = fmaxf(m[j], m2);
                    const float f1 = __builtin_amdgcn_exp2f(m[j] - mn), f2 = __builtin_amdgcn_exp2f(m2 - mn);
                    ls[j] = ls[j] * f1 + l2 * f2;
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[j][e] = o[j][e] * f1 + shfl_xor_f(o[j][e], off) * f2;
                    m[j] = mn;
                }
            }
        }
        if (lane < LPP) {
#pragma unroll
            for (int j = 0; j < GB; ++j) {
                if (j < Gq) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) S->att_o[(w * kMaxGroup + h0 + j) * HD + dl + e] = o[j][e];
                    if (lane == 0) {
                        S->att_ml[(w * kMaxGroup + h0 + j) * 2] = m[j];
                        S->att_ml[(w * kMaxGroup + h0 + j) * 2 + 1] = ls[j];
                    }
                }
            }
        }
    }
};

template <int HD, int WF, bool MS, bool XA>
__device__ __forceinline__ void kernel_body(const DecodeArgs& a, KIE_LDS Smem* S) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    WgPlan W;
    if (wave == 0) {
        make_plan(a.D, blockIdx.x, W);
        if (threadIdx.x == 0) {
            S->abort = 0u;
            write_geo(a, W, blockIdx.x, S->geo);
            if (XA && xcc_id() != (int)blockIdx.x % kXcds) {
                // XCD-local attention would exchange words between XCDs
                // through L2 caches that do not see each other: refuse
                sys_store32(a.status, kStatusWrongXcd);
                S->abort = 1u;
            }
        }
    }
    __syncthreads();
    if (wave == 0) {
        Comm<HD, WF, MS, XA> cm(a, S, W);
        cm.run();
    } else {
        Compute<HD, WF, MS, XA> cp(a, S, wave - 1);
        cp.run();
    }
}

// Two symbols for the same code, so that profiles keep the prompt's passes
// apart from the generation requests. XA: built with the attention recomputed
// per XCD (launched only in that mode; the other kernels carry none of it).
template <int HD, int WF, bool MS, bool XA>
__global__ void __launch_bounds__(kThreads, 1) decode_kernel(const DecodeArgs* __restrict__ ap) {
    __shared__ Smem smem_;
    kernel_body<HD, WF, MS, XA>(*ap, (KIE_LDS Smem*)&smem_);
}

template <int HD, int WF, bool MS>
__global__ void __launch_bounds__(kThreads, 1) prefill_kernel(const DecodeArgs* __restrict__ ap) {
    __shared__ Smem smem_;
    kernel_body<HD, WF, MS, false>(*ap, (KIE_LDS Smem*)&smem_);
}

// The quantised-weight kernels are built for head_dim 128 only (the decoders
// whose widths fp8 and fp4 need: every projection width a multiple of 512).
// With XCD-local attention (xa) the prompt's passes run the decode symbol.
hipError_t launch_decode(const DecodeArgs* dev_args, int hd, int wf, bool ms, bool xa, bool prefill, int grid,
                         hipStream_t s) {
    void* args[] = {&dev_args};
    if ((wf != 0 || ms) && hd != 128) return hipErrorInvalidValue;
    if (wf < 0 || wf > 2) return hipErrorInvalidValue;
    // hd 64: fp16 without the matrix-core split; hd 128: [weight format][ms]
    const void* fn;
    if (hd == 64) {
        fn = xa ? (const void*)decode_kernel<64, 0, false, true>
                : prefill ? (const void*)prefill_kernel<64, 0, false> : (const void*)decode_kernel<64, 0, false, false>;
    } else if (xa) {
        const void* t[3][2] = {{(const void*)decode_kernel<128, 0, false, true>, (const void*)decode_kernel<128, 0, true, true>},
                               {(const void*)decode_kernel<128, 1, false, true>, (const void*)decode_kernel<128, 1, true, true>},
                               {(const void*)decode_kernel<128, 2, false, true>, (const void*)decode_kernel<128, 2, true, true>}};
        fn = t[wf][ms ? 1 : 0];
    } else if (prefill) {
        const void* t[3][2] = {{(const void*)prefill_kernel<128, 0, false>, (const void*)prefill_kernel<128, 0, true>},
                               {(const void*)prefill_kernel<128, 1, false>, (const void*)prefill_kernel<128, 1, true>},
                               {(const void*)prefill_kernel<128, 2, false>, (const void*)prefill_kernel<128, 2, true>}};
        fn = t[wf][ms ? 1 : 0];
    } else {
        const void* t[3][2] = {{(const void*)decode_kernel<128, 0, false, false>, (const void*)decode_kernel<128, 0, true, false>},
                               {(const void*)decode_kernel<128, 1, false, false>, (const void*)decode_kernel<128, 1, true, false>},
                               {(const void*)decode_kernel<128, 2, false, false>, (const void*)decode_kernel<128, 2, true, false>}};
        fn = t[wf][ms ? 1 : 0];
    }
    return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kThreads), args, 0, s);
}

}  // namespace kie

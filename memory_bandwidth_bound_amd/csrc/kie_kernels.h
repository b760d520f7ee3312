// kie_kernels.h - kernel argument blocks and launchers shared by the kernels
// (kie_decode.hip, kie_probes.hip) and the C ABI (kie_api.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kie_common.h"

namespace kie {

// Waves of a persistent workgroup: wave 0 exchanges data with the other
// workgroups and runs the epilogues; waves 1..7 stream weights into LDS and
// compute the dot products.
constexpr int kWaves = 8;
constexpr int kCompute = kWaves - 1;
constexpr int kThreads = 64 * kWaves;
// Ring geometry (compile-time tuning knobs).
#ifndef KIE_NB
#define KIE_NB 8
#endif
#ifndef KIE_NS
#define KIE_NS 2
#endif
constexpr int kNB = KIE_NB;               // 1 KiB units per batch
constexpr int kNS = KIE_NS;               // batches in flight per compute wave (an LDS ring)
constexpr int kBatchBytes = kNB * kUnitBytes;
constexpr int kIdleBytes = kBatchBytes;   // zero region loaded by batches with nothing to stream
constexpr int kMaxIn = kMaxInput;

enum : int {
    F_FORCE = 1,        // force_ids drives the next input where >= 0
    F_DBG_LOGITS = 2,   // write every pass's logits to dbg_logits
    F_DBG_EXPERTS = 4,  // write every pass's expert ids and router logits to dbg_experts, dbg_router
    F_SKIP_LM = 8,      // skip the LM head on every pass but the last (prefill)
    F_TRACE = 16,       // record the phase timeline in trace
    F_XCD_ATTN = 32     // XCD-local attention where it fits (every XCD computes all heads for itself)
};

// Status word values (0: running or done).
constexpr uint32_t kStatusWrongXcd = 3;   // XCD-local attention: a workgroup found itself off XCD w % kXcds

// Flagged-word exchange buffers (64-bit words: phase id << 32 | payload).
struct Exchange {
    uint64_t* x;     // [d]      residual after Wo / down, fp32
    uint64_t* qkv;   // [Hkv][(G+1)*hd] per KV group (G query heads): the group's
                     //          rotated queries (fp32), then the new key as
                     //          rotary pairs (k[i], k[i+hd/2]) and the new value
                     //          as pairs (v[2i], v[2i+1]), fp16
    uint64_t* part;  // [H][items][hd+2] split attention partials (m, l, o), fp32
    uint64_t* o;     // [H*hd]   attention output, fp32
                     // part and o hold kXcds copies (XCD-local attention: copy x
                     // is written and read by the workgroups of XCD x only)
    int64_t part_copy;   // words from one copy of part to the next
    int64_t o_copy;      // words from one copy of o to the next
    uint64_t* h;     // [F or topk*F] SwiGLU output (MoE: times pi), fp32
    uint64_t* r;     // [E] router logits, fp32
    uint64_t* am;    // [grid][2] per-workgroup argmax value, index
};

struct DecodeArgs {
    Dims D;
    float eps;
    int items_per_head;
    uint32_t spin;           // polls before a device-side wait gives up
    const uint8_t* layers;   // L streaming blocks
    uint64_t layer_bytes;
    const uint8_t* lm;       // LM head block
    const uint16_t* emb;     // [V][d]
    const uint8_t* experts;  // MoE expert blocks
    uint64_t expert_bytes;
    const float* rope;       // [max_seq][hd/2][2]
    uint16_t* kc;            // [L][Hkv][max_seq][hd]
    uint16_t* vc;
    Exchange ex;
    uint32_t* status;        // pinned host memory: 0, kStatusTimeout from a workgroup, or set by the host's watchdog
    int32_t* out_ids;
    const int32_t* force_ids;
    float* dbg_logits;
    int32_t* dbg_experts;
    float* dbg_router;
    const int32_t* plan;     // piece_off[kGrid+1], lm_off[kGrid+1]
    const uint8_t* idle;     // kIdleBytes of zeros: target of loads that keep a batch slot busy
    int64_t* trace;          // [kTracePhases][kGrid][4] phase timeline (F_TRACE)
    const float* scales;     // fp8/fp4 weights: per layer [QKV][Wo][gate/up][down] row scales, then [V] LM
    int32_t layer_scales;    // floats per layer in scales
    const float* escales;    // fp8/fp4 MoE: per (layer, expert) [2F gate/up rows][d down rows] row scales
    int32_t pos0;
    int32_t pending;
    int32_t n_steps;
    int32_t flags;
    uint32_t id0;            // phase id of this launch's first phase (ids never repeat)
};

struct GemvArgs {
    const uint8_t* A;      // copies*M rows of K fp16, row stride lda elements
    const uint16_t* x;     // [K] fp16
    float* y;              // [copies*M]
    const uint8_t* idle;   // kIdleBytes of readable memory (streaming variant)
    int64_t lda;
    int32_t M, K, copies, accumulate;
};

// Weight rows of one GEMM: row m of M rows of K fp16 is at base +
// slab[w] KiB + (m - row0(w)) K 2 bytes, w its owner in the even split of M
// rows in groups of gran over the persistent grid (the decode layout), or at
// base + m K 2 bytes when dense.
struct GemmRows {
    const uint8_t* base;
    const int32_t* slab;   // [kGrid] units (device memory)
    int32_t M, K, gran, dense;
    int32_t wf;            // weight format: 0 fp16, 1 fp8 (rows in pairs), 2 fp4 (rows in fours)
    const float* scales;   // wf != 0: the phase's row scales [M] (device memory)
};

// Row-wise prefill kernels (kie_prefill.hip).
enum : int { PF_EMBED = 0, PF_RMSNORM, PF_RESIDUAL, PF_SWIGLU, PF_QKV, PF_ATTN, PF_ARGMAX };
struct PrefillRowArgs {
    Dims D;
    float eps;
    int32_t n;        // rows (tokens) of this chunk
    int32_t pos0;     // position of row 0
    int32_t layer;
    int32_t ldy;      // row stride of Y
    const uint16_t* emb;
    const int32_t* tok;
    float* X;         // [n][d] residual
    float* A;         // GEMM input rows ([n][d], attention output [n][H hd], SwiGLU output [n][F])
    const float* Y;   // GEMM output rows (PF_ARGMAX: the one row to reduce, V wide)
    float* Q;         // [n][H hd] rotated queries
    const float* rope;
    uint16_t* kc;
    uint16_t* vc;
    int32_t* out;     // PF_ARGMAX: the index
};

// Phases per decode step (used by the host to advance phase ids).
inline int phases_per_layer(const Dims& D) { return D.E ? 7 : 6; }
inline int phases_per_step(const Dims& D) { return D.L * phases_per_layer(D) + 2; }

// Launchers. dev_args: the argument block already copied to device memory.
// The persistent kernel comes in variants: hd 64 or 128, the weight format
// wf (0 fp16, 1 FP8, 2 FP4; quantised formats with hd 128 only), and, for hd
// 128, with the matrix-core split attention (ms) or without: the host takes
// ms only for launches with a pass beyond head mode (head_mode_at), since
// carrying that code costs the short-context passes about 1%. xa: the
// variant with attention recomputed per XCD (F_XCD_ATTN set), likewise kept
// out of the other kernels.
hipError_t launch_decode(const DecodeArgs* dev_args, int hd, int wf, bool ms, bool xa, bool prefill, int grid,
                         hipStream_t s);
// Persistent GEMV with the decode kernel's LDS-DMA weight streaming (8 waves
// per workgroup, a contiguous range of units per wave, row sums added into y,
// which the caller zeroes). Needs K <= kMaxInput.
hipError_t launch_gemv_stream(const GemvArgs& a, int grid, hipStream_t s);
// Plain GEMV: one wave per 4 rows, all loads of a row block in flight.
hipError_t launch_gemv_direct(const GemvArgs& a, hipStream_t s);
// Inter-workgroup exchange probe. variant 0: fenced grid barrier; variant 1:
// every workgroup publishes 5 flagged words per round and gathers all of them
// (the residual exchange of the decode kernel). words: >= 2 * grid * 8 words.
hipError_t launch_barrier_probe(int variant, uint64_t* words, uint32_t* status, int32_t* errors, int rounds,
                                int grid, hipStream_t s);
hipError_t launch_empty(hipStream_t s);
// Y[p][m] = sum_k A[p][k] W(m)[k] on the matrix cores, p < n, m < R.M; A fp32
// (row stride lda, a multiple of 4), taken as two fp16 terms; R.K a multiple
// of 64.
hipError_t launch_gemm_mfma(const float* A, int lda, int n, const GemmRows& R, float* Y, int ldy, hipStream_t s);
hipError_t launch_prefill_rows(int op, const PrefillRowArgs& r, hipStream_t s);
// out[c] = the device's fp8 (E4M3) conversion of code c, c < 256.
hipError_t launch_e4m3_table(float* out, hipStream_t s);
hipError_t launch_e2m1_table(float* out64, hipStream_t s);
// out[w] = the XCD workgroup w of a grid-sized cooperative launch ran on.
hipError_t launch_xcd_map(int32_t* out, int grid, hipStream_t s);
// Zero n 32-bit words with a kernel.
hipError_t launch_fill_zero(uint32_t* p, int n, hipStream_t s);
// Device address of the no-alloc probe's scratch array on the current device
// (looked up once per device), and its size.
hipError_t noalloc_scratch(void** out);
size_t noalloc_scratch_bytes();

}  // namespace kie

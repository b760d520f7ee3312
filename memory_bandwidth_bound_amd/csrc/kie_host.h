// kie_host.h - host-only preparation: validation, workspace layout, weight
// repacking and the rotary table. No HIP in here, so it builds with g++ too.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/kie.h"
#include "kie_common.h"

namespace kie {

constexpr int kDebugRows = 64;    // logits rows buffered on the device per launch
constexpr int kPrefillRows = 256; // prompt tokens per batched-prefill chunk

// Does the batched (matrix-core) prefill support this model? Dense fp16.
inline bool batched_prefill_ok(const Dims& D) { return D.E == 0; }

// Byte offsets of every region of the caller's device workspace.
struct Layout {
    Dims D;
    size_t layer_bytes;           // one layer's streaming block
    size_t off_layers;            // L blocks
    size_t off_lm;                // LM head block
    size_t lm_bytes;
    size_t off_emb;               // embedding table [V][d] fp16
    size_t off_experts;           // MoE: per layer, per expert [GU interleaved 2F x d][Wd d x F]
    size_t expert_bytes;          // one expert block
    size_t off_rope;              // float2 [max_seq][hd/2] (cos, sin)
    size_t off_k, off_v;          // fp16 [L][Hkv][max_seq][hd]
    size_t kv_bytes;              // one of K or V
    // flagged-word exchange buffers (64-bit words), zeroed at load
    size_t off_ex_x;              // [d/2]
    size_t off_ex_qkv;            // [Hkv][(H/Hkv + 1) * hd]
    size_t off_ex_part;           // kXcds copies of [H][items per kv head][hd + 2]
    size_t off_ex_o;              // kXcds copies of [H*hd]
    size_t ex_part_copy;          // words from one copy of part (or o) to the next
    size_t ex_o_copy;
    size_t off_ex_h;              // [max(F, topk*F)/2]
    size_t off_ex_r;              // [max(E, 1)]
    size_t off_ex_am;             // [kGrid][2]
    size_t ex_bytes;              // whole exchange region, from off_ex_x
    size_t off_status;            // u32 [64]
    size_t off_out;               // i32 [max_seq]
    size_t off_force;             // i32 [max_seq]
    size_t off_dbg_logits;        // f32 [kDebugRows][V]
    size_t off_dbg_experts;       // i32 [kDebugRows][L][topk]
    size_t off_dbg_router;        // f32 [kDebugRows][L][E] (MoE router logits)
    size_t off_plan;              // i32 piece_off[kGrid+1], lm_off[kGrid+1]
    size_t off_args;              // kernel argument block (4 KiB)
    size_t off_idle;              // 16 KiB read by weight batches that have nothing to stream
    size_t off_trace;             // i64 [kTracePhases][kGrid][4] phase timeline
    size_t off_scales;            // fp8/fp4: f32 per layer [QKV rows][Wo rows][gate/up rows][down rows], then [V] LM
    // batched prefill (dense fp16 models), chunks of kPrefillRows tokens
    size_t off_pf_x;              // f32 [R][d] residual
    size_t off_pf_a;              // f32 [R][max(d, H hd, F)] GEMM input
    size_t off_pf_y;              // f32 [R][max(QKV rows, 2F, V)] GEMM output
    size_t off_pf_q;              // f32 [R][H hd] queries
    size_t off_pf_tok;            // i32 [R] tokens, then i32 [4] argmax
    size_t off_pf_slab;           // i32 [5][kGrid] slab offsets: QKV, Wo, gate/up, down (layer block), LM
    size_t layer_scales;          // floats per layer
    size_t off_escales;           // fp8/fp4 MoE: f32 per (layer, expert) [2F gate/up rows][d down rows]
    size_t total;
    int piece_off[kGrid + 1];     // units: start of workgroup w's piece in a layer block
    int lm_off[kGrid + 1];        // units: start of workgroup w's LM slab
    int attn_items_per_head;
};

Dims dims_of(const kie_config& c);
// Returns KIE_OK or an error code with a message.
int validate_config(const kie_config& c, std::string* err);
int tensor_count(const kie_config& c);
void make_layout(const kie_config& c, Layout* lay);

// fp16 <-> fp32 (IEEE binary16, round to nearest even).
uint16_t f32_to_f16(float f);
float f16_to_f32(uint16_t h);

// Fill one layer's streaming block (layer_bytes bytes) from the canonical tensors.
void repack_layer(const kie_config& c, const Layout& lay, const uint16_t* const* t, int layer,
                  uint16_t* dst);
// Fill the LM head block (lm_bytes bytes).
void repack_lm(const kie_config& c, const Layout& lay, const uint16_t* const* t, uint16_t* dst);
// Fill one expert block (expert_bytes bytes).
void repack_expert(const kie_config& c, const Layout& lay, const uint16_t* const* t, int layer,
                   int expert, uint16_t* dst);
// cos/sin table, angles formed in double precision. dst: float [max_seq][hd/2][2].
void rope_table(const kie_config& c, float* dst);

// FP4 (E2M1) rows: the quantizer of kie_quantize_e2m1_rows (codes 0..15).
uint8_t e2m1_encode(float v);                 // nearest code, ties to even, saturating at 6
float e2m1_decode(uint8_t q);
void quantize_row_e2m1(const uint16_t* w, const uint16_t* gain, int K, uint8_t* q, float* scale);
// FP8 (E4M3) rows: the quantizer of kie_quantize_e4m3_rows.
uint8_t e4m3_encode(float v);                 // nearest code, ties to even, saturating
float e4m3_decode(uint8_t q);
void quantize_row_e4m3(const uint16_t* w, const uint16_t* gain, int K, uint8_t* q, float* scale);
// fp8 / fp4 weights (D.w4 picks fp4): one layer's streaming block (layer_bytes bytes) and its row
// scales (layer_scales floats), and the LM head block and its V scales.
void repack_layer_fp8(const kie_config& c, const Layout& lay, const uint16_t* const* t, int layer, uint8_t* dst,
                      float* scales);
void repack_lm_fp8(const kie_config& c, const Layout& lay, const uint16_t* const* t, uint8_t* dst, float* scales);
// Quantised MoE: one expert block and its 2F + d row scales. fp8: gate/up
// row pairs (g_p, u_p), then down row pairs; fp4: gate/up rows in fours
// (g_p, u_p, g_p+1, u_p+1), then down rows in fours (expert_bytes).
void repack_expert_quant(const kie_config& c, const Layout& lay, const uint16_t* const* t, int layer, int expert,
                       uint8_t* dst, float* scales);

// Canonical tensor index helpers (same order as kie.h documents).
int tidx_emb();
int tidx_layer(const kie_config& c, int layer, int which);   // which: 0 g_attn,1 Wq,2 Wk,3 Wv,4 Wo,5 g_ffn,6 Wg|Wr,7 Wu,8 Wd
int tidx_expert(const kie_config& c, int layer, int expert, int which);  // which: 0 Wg, 1 Wu, 2 Wd
int tidx_gfinal(const kie_config& c);
int tidx_lm(const kie_config& c);

}  // namespace kie

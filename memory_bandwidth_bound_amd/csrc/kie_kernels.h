// kie_kernels.h - kernel argument blocks and launch helpers shared by the
// kernels (kie_kernels.hip) and the C ABI (kie_api.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kie_common.h"

namespace kie {

// Waves of the persistent workgroup: 2 weight-streaming waves + 6 compute waves.
constexpr int kProducers = 2;
constexpr int kConsumers = 6;
constexpr int kThreads = 64 * (kProducers + kConsumers);
constexpr int kSlots = 128;                    // 1 KiB LDS ring slots
constexpr int kDepth = 40;                     // loads in flight per streaming wave
constexpr int kRegionA = 28 * 1024;            // input vector + partials | attention scratch
constexpr int kXinBytes = 16 * 1024;           // fp16 GEMV input, up to 8192 elements
constexpr int kPartFloats = 1024;              // per-phase partial sums
constexpr int kCtlBytes = 512;
constexpr int kLdsBytes = kSlots * 1024 + kRegionA + kCtlBytes;

enum : int {
    F_FORCE = 1,        // force_ids drives the next input where >= 0
    F_DBG_LOGITS = 2,   // write every pass's logits to dbg_logits
    F_DBG_EXPERTS = 4,  // write every pass's expert ids to dbg_experts
    F_SKIP_LM = 8       // skip the LM head on every pass but the last (prefill)
};

struct DecodeArgs {
    Dims D;
    float eps;
    int items_per_head;
    uint32_t spin_lds;       // spin limit of LDS waits
    uint32_t spin_grid;      // spin limit of grid-barrier polls
    const uint8_t* layers;   // L streaming blocks
    uint64_t layer_bytes;
    const uint8_t* lm;       // LM head block
    const uint16_t* emb;     // [V][d]
    const uint8_t* experts;  // MoE expert blocks
    uint64_t expert_bytes;
    const float* rope;       // [max_seq][hd/2][2]
    uint16_t* kc;            // [L][Hkv][max_seq][hd]
    uint16_t* vc;
    float* x;
    float* q;
    uint16_t* o16;
    uint16_t* h16;
    float* router;
    float* attn_part;
    uint32_t* attn_cnt;
    float* argmax;           // [grid][2] (value, index bits)
    uint32_t* bar;
    uint32_t* status;
    int32_t* out_ids;
    const int32_t* force_ids;
    float* dbg_logits;
    int32_t* dbg_experts;
    const int32_t* plan;     // piece_off[kGrid+1], lm_off[kGrid+1]
    int32_t pos0;
    int32_t pending;
    int32_t n_steps;
    int32_t flags;
    uint32_t epoch0;         // barrier epoch before the first barrier of this launch
};

struct GemvArgs {
    const uint8_t* A;
    const uint16_t* x;
    float* y;
    int32_t M, K, copies;
    uint32_t spin_lds;
};

// Launchers (defined in kie_kernels.hip). Return the hipError_t of the launch.
// dev_args: the argument block already copied to device memory.
hipError_t launch_decode(const DecodeArgs* dev_args, int hd, int grid, hipStream_t s);
hipError_t launch_gemv_ring(const GemvArgs& a, int grid, hipStream_t s);
hipError_t launch_gemv_direct(const GemvArgs& a, hipStream_t s);
hipError_t launch_barrier_probe(uint32_t* bar, uint32_t* status, float* vals, int32_t* errors, int rounds,
                                int grid, hipStream_t s);
hipError_t launch_empty(hipStream_t s);
hipError_t decode_kernel_setup();

}  // namespace kie

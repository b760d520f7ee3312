/*
 * kie.h - C ABI of the batch-1 decode library for MI355X (gfx950).
 *
 * The library runs single-request (batch 1) greedy decode of a pre-norm
 * transformer decoder as ONE persistent kernel launch per call, with sampling
 * on the device and no host in the token loop. This is the method of the
 * news.creeta.com monokernel article ("Inside the monokernel": one resident
 * grid for the whole decode loop, on-device sampling, no relaunch or CPU
 * wake-up between tokens) and of the agentlenshq.com article ("Core technical
 * innovations": a single persistent program for the whole decode path). The
 * metric is per-request decode speed at batch 1 (paper-digest.app digest,
 * "Core Mechanics"); prefill is not part of it.
 *
 * Conventions for every call:
 *  - Every int-returning call returns KIE_OK (0) or a negative KIE_ERR_* code.
 *    No exception crosses the ABI. kie_last_error() gives a message.
 *  - Host pointers are plain CPU memory owned by the caller. Device pointers
 *    are device memory owned by the caller (for example a torch tensor); the
 *    library never allocates or frees device memory (kie_load takes 64 bytes
 *    of pinned host memory for the kernel's status word, see kie_set_limits).
 *  - All device work is enqueued on the HIP stream given to kie_load (NULL =
 *    the default stream). Calls that return data to host buffers synchronise
 *    that stream before returning.
 *  - A model is used by one host thread at a time.
 *  - After KIE_ERR_TIMEOUT the device state is undefined: call kie_reset
 *    before further use, or kie_free.
 */
#ifndef KIE_H
#define KIE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    KIE_OK = 0,
    KIE_ERR_ARG = -1,        /* null pointer, negative count, token out of range */
    KIE_ERR_CONFIG = -2,     /* dimensions the kernels do not support */
    KIE_ERR_CAPACITY = -3,   /* position + tokens would exceed max_seq */
    KIE_ERR_WORKSPACE = -4,  /* workspace smaller than kie_workspace_bytes() */
    KIE_ERR_DEVICE = -5,     /* not gfx950, or the persistent grid cannot be co-resident */
    KIE_ERR_HIP = -6,        /* a HIP runtime call failed */
    KIE_ERR_TIMEOUT = -7,    /* a device-side wait hit its spin limit; the kernel exited */
    KIE_ERR_STATE = -8       /* call order violated (e.g. decode before prefill) */
};

/*
 * Decoder shape. The block is the plain pre-norm decoder the pages imply
 * (RMSNorm, Q/K/V projections with rotary embedding, grouped-query attention
 * over a KV cache, output projection, RMSNorm, SwiGLU FFN or top-k MoE;
 * final RMSNorm and an untied LM head; no biases).
 *  n_experts = 0 selects a dense SwiGLU FFN of width ffn_dim; otherwise each
 *  layer has n_experts SwiGLU experts of width ffn_dim, a softmax router, and
 *  the top_k experts by router probability are mixed with those
 *  probabilities (ties to the lower expert index, no renormalisation).
 * Supported (KIE_ERR_CONFIG otherwise): head_dim in {64, 128}; n_heads a
 * multiple of n_kv_heads with at most 8 query heads per KV head and at most
 * 256 KV heads; d_model, ffn_dim and n_heads*head_dim each 256 or a multiple
 * of 512 (MoE: d_model and ffn_dim multiples of 512, top_k <= 16, at most
 * 1024 experts); the longest matrix-vector input (d_model, n_heads*head_dim,
 * ffn_dim, or top_k*ffn_dim for MoE) at most 8192; 2 <= vocab <= 65536;
 * max_seq <= 65536.
 * weight_format selects how the streamed projection weights are held:
 *  KIE_WEIGHTS_FP16: the fp16 tensors as given (RMSNorm gains folded in).
 *  KIE_WEIGHTS_FP8:  OCP FP8 E4M3 with one fp32 scale per row, the route to
 *    fewer bytes per token that the agentlenshq.com article names ("Scaling to
 *    frontier MoE models": FP8/FP4 quantisation). kie_load quantizes each
 *    projection after folding in the RMSNorm gain that precedes it (Wq, Wk,
 *    Wv: g_attn; Wg, Wu: g_ffn; W_lm: g_final; Wo, Wd: none): for a row v of
 *    fp32 values (v_k = w_k * g_k), s = fp32(max_k |v_k| / 448) (1 for an
 *    all-zero row) and q_k = E4M3 nearest to fp32(v_k / s), ties to the even
 *    code (kie_quantize_e4m3_rows). The embedding stays fp16. MoE: the router
 *    (g_ffn folded) and every expert's Wg, Wu (g_ffn folded) and Wd the same
 *    way. head_dim 128 only; d_model, ffn_dim and n_heads*head_dim multiples
 *    of 512, vocab and n_experts even.
 *  KIE_WEIGHTS_FP4:  OCP FP4 E2M1 (the element type of the OCP microscaling
 *    formats: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) with one fp32 scale per
 *    row, the FP4 of the same passage, quantized like FP8 with 6 in place of
 *    448: s = fp32(max_k |v_k| / 6) (1 for an all-zero row), q_k = E2M1
 *    nearest to fp32(v_k / s), ties to the even code, saturating at 6
 *    (kie_quantize_e2m1_rows). MoE as for FP8. head_dim 128; d_model,
 *    ffn_dim and n_heads*head_dim multiples of 512; vocab and n_experts
 *    multiples of 4.
 */
typedef struct kie_config {
    int32_t n_layers;
    int32_t d_model;
    int32_t n_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t ffn_dim;
    int32_t vocab;
    int32_t n_experts;   /* 0 = dense */
    int32_t top_k;       /* experts per token (MoE only) */
    float rms_eps;       /* RMSNorm: x / sqrt(mean(x^2) + eps) * g */
    float rope_theta;    /* rotary base; pairs (i, i + head_dim/2) */
    int32_t max_seq;     /* KV-cache capacity in positions */
    int32_t weight_format;   /* KIE_WEIGHTS_FP16 (0), KIE_WEIGHTS_FP8 (1) or KIE_WEIGHTS_FP4 (2) */
} kie_config;

enum { KIE_WEIGHTS_FP16 = 0, KIE_WEIGHTS_FP8 = 1, KIE_WEIGHTS_FP4 = 2 };

/*
 * The library's FP8 quantizer, as kie_load applies it (host only, no device
 * call): rows x K fp16 weights w (row-major, host) and an optional fp16 gain
 * [K] (NULL = 1) -> q [rows][K] E4M3 codes and scales [rows] fp32, with
 * s = fp32(max_k |fp32(w_k) * fp32(g_k)| / 448) (1 for an all-zero row) and
 * q_k the E4M3 code nearest to fp32(fp32(w_k) * fp32(g_k) / s), ties to the
 * even code, saturating at 448. E4M3 is the OCP 8-bit float with 4 exponent
 * bits (bias 7), 3 mantissa bits, no infinities, code 0x7f/0xff = NaN.
 * Returns KIE_OK or KIE_ERR_ARG.
 */
int kie_quantize_e4m3_rows(const void* w_fp16, const void* gain_fp16, int32_t rows, int32_t K, uint8_t* q,
                           float* scales);

/*
 * The library's FP4 quantizer, as kie_load applies it (host only, no device
 * call): rows x K fp16 weights w and an optional fp16 gain [K] (NULL = 1) ->
 * q [rows][K] E2M1 codes (0..15, one per byte; bit 3 is the sign) and scales
 * [rows] fp32, with s = fp32(max_k |fp32(w_k) * fp32(g_k)| / 6) (1 for an
 * all-zero row) and q_k the E2M1 code nearest to fp32(fp32(w_k) * fp32(g_k) /
 * s), ties to the even code, saturating at 6; a negative value that rounds to
 * zero keeps its sign (code 8). Returns KIE_OK or KIE_ERR_ARG.
 */
int kie_quantize_e2m1_rows(const void* w_fp16, const void* gain_fp16, int32_t rows, int32_t K, uint8_t* q,
                           float* scales);

/*
 * Optional per-call debug outputs and teacher forcing (all host memory).
 *  force_ids: if non-NULL, [n] tokens; pass i is still sampled greedily
 *             (its argmax is returned in out_ids[i]) but the token fed to pass
 *             i+1 is force_ids[i].
 *  logits:    if non-NULL, [n][vocab] fp32 logits of every pass.
 *  experts:   if non-NULL (MoE only), [n][n_layers][top_k] selected expert
 *             ids of every pass, in descending router probability.
 *  router:    if non-NULL (MoE only), [n][n_layers][n_experts] fp32 router
 *             logits of every pass, the values the device ranked to choose
 *             `experts` (larger first, ties to the lower expert index).
 *  trace:     if non-NULL, [KIE_TRACE_PHASES][256][4] int64 phase timeline of
 *             the call's first launch: for each of its first
 *             KIE_TRACE_PHASES phases (see kie_phases_per_pass) and each
 *             workgroup, the device's constant 100 MHz clock when the
 *             workgroup's communication wave began the phase, had gathered
 *             its input, saw the compute waves finish, and had published its
 *             output (entries past the call's phases are left untouched).
 * Debug outputs add device-to-host copies; they are for tests and profiling,
 * not timing.
 */
#define KIE_TRACE_PHASES 2048
typedef struct kie_debug {
    const int32_t* force_ids;
    float* logits;
    int32_t* experts;
    int64_t* trace;
    float* router;
} kie_debug;

/* Phases of one forward pass: n_layers * (6 dense | 7 MoE) + 2, in the order
 * per layer QKV, ATTN, COMB, WO, then GU, DOWN (dense) or ROUTER, EGU,
 * EDOWN (MoE); then LM, SAMPLE. 0 if the configuration is invalid. */
int32_t kie_phases_per_pass(const kie_config* cfg);

typedef struct kie_model kie_model;   /* opaque, owned by the library */

/* Device bytes the caller must allocate for kie_load's workspace (weights in
 * the streaming layout, KV cache, the words workgroups exchange, status and
 * debug buffers). 0 if the configuration is invalid. Pure host computation. */
size_t kie_workspace_bytes(const kie_config* cfg);

/* Number of fp16 tensors kie_load expects for this configuration. */
int32_t kie_tensor_count(const kie_config* cfg);

/*
 * Load a model. host_tensors[i] points to the i-th fp16 tensor in the
 * canonical order, each row-major [out][in]:
 *   E[vocab][d];
 *   per layer: g_attn[d], Wq[H*hd][d], Wk[Hkv*hd][d], Wv[Hkv*hd][d],
 *              Wo[d][H*hd], g_ffn[d], then either Wg[F][d], Wu[F][d], Wd[d][F]
 *              or Wr[n_experts][d] followed by (Wg, Wu, Wd) per expert;
 *   g_final[d]; W_lm[vocab][d].
 * The host repacks them once (offline preparation in the sense of the
 * monokernel article's fused, precomputed steps: RMSNorm gains folded into
 * the following projection, Q/K/V fused into one streamable matrix, a rotary
 * cos/sin table built in double precision) and copies them into
 * dev_workspace, which must stay allocated until kie_free.
 * hip_stream is a hipStream_t (NULL = default stream). On success *out is a
 * new model at position 0 with no pending token.
 */
int kie_load(const kie_config* cfg, const void* const* host_tensors, int32_t n_tensors,
             void* dev_workspace, size_t ws_bytes, void* hip_stream, kie_model** out);

/*
 * Prefill: process the prompt's tokens at positions 0..n-1 (cache entries at
 * those positions are overwritten) and return the greedy first generated
 * token, which becomes the pending token. Not part of the decode metric
 * (paper-digest.app digest, "Core Mechanics"). Two ways, one result (up to
 * rounding order):
 *  - batched (dense fp16 models, the default): the prompt's projections as
 *    GEMMs on the matrix cores in chunks of 256 tokens, with causal attention
 *    over the cache, norms, RoPE, SwiGLU and residuals as row kernels;
 *  - passes (other models, kie_set_prefill_mode(m, KIE_PREFILL_PASSES), or
 *    when dbg->trace is set): one decode pass per token in one persistent
 *    launch (launches of at most 64 passes when debug logits are requested),
 *    the LM head on the last pass only.
 * dbg may be NULL; dbg->logits, if set, receives [n][vocab].
 */
int kie_prefill(kie_model* m, const int32_t* tokens, int32_t n, int32_t* first_token,
                const kie_debug* dbg);

enum { KIE_PREFILL_AUTO = 0, KIE_PREFILL_PASSES = 1 };
/* Choose how later kie_prefill calls run (see kie_prefill). KIE_ERR_ARG for
 * an unknown mode or a null model. */
int kie_set_prefill_mode(kie_model* m, int32_t mode);

enum { KIE_ATTN_GLOBAL = 0, KIE_ATTN_XCD_LOCAL = 1 };
/*
 * Choose how later persistent launches (kie_decode; kie_prefill in passes
 * mode) run attention at short context.
 *  - KIE_ATTN_GLOBAL (the default): one workgroup of the grid per (query
 *    head, chunk of positions); the attention output crosses the chip to the
 *    workgroups of the output projection.
 *  - KIE_ATTN_XCD_LOCAL: attention recomputed on every XCD instead of
 *    exchanged between dies, with its exchange buffers replicated per XCD
 *    (news.creeta.com monokernel article: "Inside the monokernel", attention
 *    recompute; "MI300X die topology and the 256-CU mapping", work grouped by
 *    die and buffers replicated per die). While a pass's head-mode work items
 *    (query heads x chunks of at most 384 positions) fit the 32 workgroups of
 *    one XCD, every XCD computes all of them and its output-projection
 *    workgroups read the result from their own XCD's copy (32 readers per
 *    copy instead of the whole grid on one buffer). Other passes run as in
 *    KIE_ATTN_GLOBAL. The arithmetic and its order
 *    are those of KIE_ATTN_GLOBAL, so the results are identical.
 * Errors: KIE_ERR_ARG (null model, unknown mode); KIE_ERR_CONFIG
 * (KIE_ATTN_XCD_LOCAL needs 2 to 8 query heads per KV head and at most 32
 * query heads). In KIE_ATTN_XCD_LOCAL every workgroup checks at the start of
 * a launch that it runs on XCD (its index mod 8); if one does not, the launch
 * exits early and returns KIE_ERR_DEVICE.
 */
int kie_set_attention_mode(kie_model* m, int32_t mode);

/*
 * Store already-rotated keys and values for positions 0..n_pos-1 directly in
 * the cache (host fp16 arrays [n_layers][n_pos][n_kv_heads][head_dim], each
 * n_layers*n_pos*n_kv_heads*head_dim elements; read, not kept), set the
 * position to n_pos and the pending token to pending_token. Every other
 * cache entry is zeroed. Used to start decoding at long context without a
 * prefill: the paper-digest.app digest ("Core Mechanics") counts the key and
 * value bytes of the context next to the weights in the bytes each decoded
 * token must read, so a long cache is a workload of its own. KIE_ERR_ARG for
 * null arrays, a negative n_pos or a token outside [0, vocab);
 * KIE_ERR_CAPACITY if n_pos > max_seq.
 */
int kie_set_kv(kie_model* m, const void* k_fp16, const void* v_fp16, int32_t n_pos,
               int32_t pending_token);

/*
 * Decode: exactly n_tokens forward passes in ONE kernel launch, starting at
 * the current position with the pending token. out_ids[i] (host, [n_tokens])
 * is the greedy token of pass i; the last one becomes the new pending token
 * (or the last forced one when teacher forcing). The position advances by
 * n_tokens. Returns KIE_ERR_CAPACITY if position + n_tokens > max_seq.
 */
int kie_decode(kie_model* m, int32_t n_tokens, int32_t* out_ids, const kie_debug* dbg);

/* Move back to an earlier position pos (0 <= pos <= current) with the given
 * pending token; cache entries at positions >= pos are overwritten by later
 * passes, and the attention of a pass never reads beyond its own position
 * (the causal decode of the news.creeta.com monokernel article, "Inside the
 * monokernel": each step attends over the cached keys and values so far).
 * Lets a benchmark repeat the same decode request. No device work.
 * KIE_ERR_ARG if pos is out of range or the token outside [0, vocab). */
int kie_rewind(kie_model* m, int32_t pos, int32_t pending_token);

/* Clear the KV cache and the exchange words on the model's stream (and wait
 * for it); position 0, no pending token. The state a request starts from in
 * the pages' batch-1 decode (paper-digest.app digest, "Core Mechanics": one
 * request, no batching). Also the way back after KIE_ERR_TIMEOUT. */
int kie_reset(kie_model* m);

/* Current position and pending token (-1 if none), both host-side values:
 * the decode loop's state between calls (news.creeta.com monokernel
 * article, "Inside the monokernel": the position advances on the device
 * inside a launch and is handed back at its end). KIE_ERR_ARG on a null
 * argument. */
int kie_state(const kie_model* m, int32_t* pos, int32_t* pending_token);

/* Device time in milliseconds of the last kernel launch made by
 * kie_decode/kie_prefill, measured with HIP events on the model's stream
 * around that one launch. */
float kie_last_kernel_ms(const kie_model* m);

/*
 * Failure detection (not from the pages: the persistent kernel's workgroups
 * wait on each other, so a broken dependency must end in an error, not a
 * hang). spin_limit: polls a device-side wait makes before it gives up
 * (0 = the default, 2^22); the workgroup then flags the failure, every other
 * workgroup's waits give up too and the kernel exits; the call returns
 * KIE_ERR_TIMEOUT. watchdog_ms: the host's wall-clock limit per launch
 * (0 = automatic: 10 s plus 20 ms per pass; < 0 = none). The host polls the
 * launch's completion; past the limit it sets the kernel's status word (in
 * pinned host memory allocated by kie_load, 64 bytes), which the kernel's
 * waits read once they have polled in vain, lets the launch end and returns
 * KIE_ERR_TIMEOUT. A
 * launch still making progress is not cut short; its overrun is reported the
 * same way. Applies to later kie_prefill / kie_decode calls. KIE_ERR_ARG for a
 * null model.
 */
int kie_set_limits(kie_model* m, uint32_t spin_limit, int32_t watchdog_ms);

/* Workgroups of the persistent grid (one per compute unit). */
int32_t kie_grid_size(const kie_model* m);

void kie_free(kie_model* m);
const char* kie_last_error(const kie_model* m);   /* m may be NULL: last global error */
const char* kie_status_str(int status);

/*
 * GEMV bandwidth probe: y[r][i] = sum_k A_r[i][k] x[k] for r < copies, where
 * A_r = A + r*M*K (fp16, row-major, device), x fp16 [K] (device), y fp32
 * [copies][M] (device), products accumulated in fp32 with v_dot2.
 * variant 0: the persistent 256-workgroup GEMV streaming weights the way
 *            the decode kernel does (LDS DMA into a per-wave ring of
 *            batches kept in flight, 8 waves per workgroup, a contiguous
 *            range of the matrices' 1 KiB units per wave, x staged in LDS,
 *            row partial sums added into y); K above 8192 runs as column
 *            blocks of 8192, one launch each, accumulated into y.
 * variant 1: a plain many-wave GEMV (4 rows per wave, all loads in flight).
 * K must be a multiple of 512, at most 65536, and copies*M*K*2 >= 4096.
 * *ms_out (host, may be NULL) receives the device time of the launches.
 * Used to measure achieved HBM bandwidth per shape (the pages' statement that
 * batch-1 decode is a bandwidth-bound matrix-vector product:
 * paper-digest.app digest, "Core Mechanics").
 */
int kie_gemv_probe(const void* A, const void* x, float* y, int32_t M, int32_t K, int32_t copies,
                   int32_t variant, void* hip_stream, float* ms_out);

/*
 * Inter-workgroup exchange probe: one persistent launch of 256 one-wave
 * workgroups running `rounds` exchange rounds.
 * variant 0: every workgroup stores one value, then a fenced grid barrier
 *            (agent-scope release, flag, poll, acquire), then reads all
 *            256 values.
 * variant 1: every workgroup publishes 5 flagged words (phase id + payload in
 *            one 64-bit store) and gathers all 1280 words, waiting only until
 *            every word carries the round's id - the residual exchange of the
 *            decode kernel.
 * variant 2: an XCD-aware barrier (the die-topology-aware barrier of the
 *            news.creeta.com monokernel article, "MI300X die topology and the
 *            256-CU mapping", re-made for MI355X's 8 XCDs): every workgroup
 *            stores one value and arrives at its own XCD's counter; the XCD's
 *            first workgroup waits for its peers there, exchanges one flag
 *            per XCD across the chip and releases its XCD through one word;
 *            then all 256 values are read. The XCD of every workgroup is
 *            read from the hardware.
 * scratch is device memory of at least kie_barrier_probe_bytes() bytes.
 * *us_per_round receives the mean time of one round; *errors the number of
 * values read wrong (must be 0), plus 1000000 per workgroup that gave up.
 */
size_t kie_barrier_probe_bytes(void);
int kie_barrier_probe(void* scratch, int32_t variant, int32_t rounds, void* hip_stream, float* us_per_round,
                      int32_t* errors);

/*
 * Allocation-free variant of kie_barrier_probe, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same probe kernel, with its words,
 * status and error count in a 64 KiB array that the library holds in device
 * memory, one per GPU, until the process ends (its address is looked up once
 * per device, at the first call on it). The caller passes no scratch. Each
 * call clears the array with a fill kernel (no hipMemsetAsync), then runs the
 * probe on hip_stream and waits for it. Calls that overlap on one GPU share
 * the array and race: issue them one at a time per device. *us_per_round is
 * host wall time of the launch (from launch to completion, no HIP events)
 * divided by rounds; *errors as for kie_barrier_probe. KIE_ERR_ARG for bad
 * arguments, KIE_ERR_WORKSPACE if the probe ever needs more than the 64 KiB.
 * Calls no hipMalloc or hipFree.
 */
int kie_barrier_probe_noalloc(int32_t variant, int32_t rounds, void* hip_stream, float* us_per_round,
                              int32_t* errors);

/*
 * Matrix-core GEMM probe (the kernel of the batched prefill): Y[p][m] =
 * sum_k A[p][k] W[m][k] for p < n, m < M, with A fp32 [n][K], W fp16 [M][K]
 * and Y fp32 [n][M], all row-major device memory owned by the caller; A is
 * taken as two fp16 terms (about 22 significant bits), products accumulated
 * in fp32 on v_mfma_f32_32x32x8_f16. K a multiple of 64. *ms_out (may be
 * NULL) receives the device time. Waits for the launch.
 */
int kie_gemm_probe(const float* A, const void* W, float* Y, int32_t n, int32_t M, int32_t K, void* hip_stream,
                   float* ms_out);

/* FP8 conversion probe: out256 (host) receives the fp32 value the device's
 * E4M3 conversion (the one the fp8 GEMVs use) gives each code 0..255. Uses the
 * library's own 64 KiB device array (no allocation); waits for the launch. */
int kie_e4m3_table_probe(float* out256, void* hip_stream);

/* FP4 conversion probe: out64 (host) receives what the device's E2M1
 * conversion (the one the fp4 GEMVs use, scale 1) gives for eight 32-bit
 * words: word l (l < 8) holds in byte b the codes (2l + b) % 16 (low nibble)
 * and (2l + b + 8) % 16 (high nibble); out64[8 l + 2 b] and [8 l + 2 b + 1]
 * are byte b's low- and high-nibble values. Uses the library's own 64 KiB
 * device array (no allocation); waits for the launch. */
int kie_e2m1_table_probe(float* out64, void* hip_stream);

/* XCD placement probe: out_xcd (host, [256]) receives the XCD (0..7 on
 * MI355X) that workgroup w of a 256-workgroup cooperative launch ran on, read
 * from the hardware register. Uses the library's own 64 KiB device array (no
 * allocation); waits for the launch. */
int kie_xcd_map(int32_t* out_xcd, void* hip_stream);

/* Launch-overhead probe: `launches` back-to-back launches of an empty kernel;
 * *us_per_launch receives host wall time per launch including completion. */
int kie_launch_probe(int32_t launches, void* hip_stream, float* us_per_launch);

#ifdef __cplusplus
}
#endif

#endif /* KIE_H */

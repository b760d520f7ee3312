// kie_api.hip - the C ABI of include/kie.h: argument checks, model state,
// uploads into the caller's workspace, and one cooperative launch per
// kie_decode / kie_prefill call.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <chrono>
#include <string>
#include <thread>
#include <vector>

#include "../../include/kie.h"
#include "kie_host.h"
#include "kie_kernels.h"

using namespace kie;

struct kie_model {
    kie_config cfg;
    Layout lay;
    uint8_t* ws;
    hipStream_t stream;
    int pos;
    int pending;   // -1: none
    uint32_t id_next;   // phase id of the next launch's first phase (ids never repeat)
    hipEvent_t ev0, ev1;
    float last_ms;
    uint32_t spin_limit;    // polls before a device-side wait gives up
    int32_t watchdog_ms;    // host limit per launch: 0 automatic, < 0 none
    uint32_t* hstatus;      // pinned host word: the kernel's status (the host's watchdog writes it too)
    int32_t prefill_mode;   // KIE_PREFILL_AUTO or KIE_PREFILL_PASSES
    int32_t attn_mode;      // KIE_ATTN_GLOBAL or KIE_ATTN_XCD_LOCAL
    std::string err;
};

constexpr uint32_t kDefaultSpin = 1u << 22;
constexpr uint32_t kStatusHostAbort = 2;   // written by the host's watchdog (kernel timeouts write 1)

// Wall-clock limit of one launch of n passes: the automatic limit allows
// 10 s plus 20 ms per pass (a pass takes about 1.3 ms on the ~2.1B decoder).
static double watchdog_limit_ms(const kie_model* m, int n) {
    if (m->watchdog_ms < 0) return -1.0;
    if (m->watchdog_ms > 0) return (double)m->watchdog_ms;
    return 10000.0 + 20.0 * n;
}

static thread_local std::string g_err;

static int fail(kie_model* m, int code, const std::string& msg) {
    if (m) m->err = msg;
    g_err = msg;
    return code;
}

static int hip_fail(kie_model* m, hipError_t e, const char* what) {
    std::string msg = std::string(what) + ": " + hipGetErrorString(e);
    int code = (e == hipErrorCooperativeLaunchTooLarge) ? KIE_ERR_DEVICE : KIE_ERR_HIP;
    return fail(m, code, msg);
}

#define HIP_TRY(m, call)                                  \
    do {                                                  \
        hipError_t e_ = (call);                           \
        if (e_ != hipSuccess) return hip_fail(m, e_, #call); \
    } while (0)

extern "C" {

const char* kie_status_str(int s) {
    switch (s) {
    case KIE_OK: return "ok";
    case KIE_ERR_ARG: return "invalid argument";
    case KIE_ERR_CONFIG: return "unsupported configuration";
    case KIE_ERR_CAPACITY: return "KV cache capacity exceeded";
    case KIE_ERR_WORKSPACE: return "workspace too small";
    case KIE_ERR_DEVICE: return "unsupported device or grid not co-resident";
    case KIE_ERR_HIP: return "HIP runtime error";
    case KIE_ERR_TIMEOUT: return "device wait timed out";
    case KIE_ERR_STATE: return "invalid call order";
    default: return "unknown status";
    }
}

const char* kie_last_error(const kie_model* m) { return m ? m->err.c_str() : g_err.c_str(); }

size_t kie_workspace_bytes(const kie_config* cfg) {
    if (!cfg) return 0;
    std::string err;
    if (validate_config(*cfg, &err) != KIE_OK) {
        g_err = err;
        return 0;
    }
    Layout* lay = new Layout;
    make_layout(*cfg, lay);
    size_t t = lay->total;
    delete lay;
    return t;
}

int32_t kie_phases_per_pass(const kie_config* cfg) {
    if (!cfg) return 0;
    std::string err;
    if (validate_config(*cfg, &err) != KIE_OK) return 0;
    return phases_per_step(dims_of(*cfg));
}

int32_t kie_tensor_count(const kie_config* cfg) {
    if (!cfg) return 0;
    return tensor_count(*cfg);
}

static int check_device(kie_model* m) {
    int dev = 0;
    HIP_TRY(m, hipGetDevice(&dev));
    hipDeviceProp_t p;
    HIP_TRY(m, hipGetDeviceProperties(&p, dev));
    if (strncmp(p.gcnArchName, "gfx950", 6) != 0)
        return fail(m, KIE_ERR_DEVICE, std::string("device is ") + p.gcnArchName + ", kernels are built for gfx950");
    if (p.multiProcessorCount < kGrid)
        return fail(m, KIE_ERR_DEVICE, "device has fewer compute units than the 256-workgroup persistent grid");
    if (!p.cooperativeLaunch) return fail(m, KIE_ERR_DEVICE, "cooperative launch not supported");
    return KIE_OK;
}

static int upload(kie_model* m, size_t off, const void* src, size_t bytes) {
    HIP_TRY(m, hipMemcpyAsync(m->ws + off, src, bytes, hipMemcpyHostToDevice, m->stream));
    HIP_TRY(m, hipStreamSynchronize(m->stream));
    return KIE_OK;
}

// Zero the KV cache (optional) and the exchange words; phase ids restart at 1.
static int clear_state(kie_model* m, bool kv) {
    const Layout& L = m->lay;
    if (kv) {
        HIP_TRY(m, hipMemsetAsync(m->ws + L.off_k, 0, L.kv_bytes, m->stream));
        HIP_TRY(m, hipMemsetAsync(m->ws + L.off_v, 0, L.kv_bytes, m->stream));
    }
    HIP_TRY(m, hipMemsetAsync(m->ws + L.off_ex_x, 0, L.ex_bytes, m->stream));
    HIP_TRY(m, hipStreamSynchronize(m->stream));
    m->id_next = 1;
    return KIE_OK;
}

int kie_load(const kie_config* cfg, const void* const* host_tensors, int32_t n_tensors, void* dev_workspace,
             size_t ws_bytes, void* hip_stream, kie_model** out) {
    if (!cfg || !host_tensors || !dev_workspace || !out) return fail(nullptr, KIE_ERR_ARG, "null argument");
    *out = nullptr;
    std::string err;
    int rc = validate_config(*cfg, &err);
    if (rc != KIE_OK) return fail(nullptr, rc, err);
    if (n_tensors != tensor_count(*cfg))
        return fail(nullptr, KIE_ERR_ARG, "tensor count does not match the configuration");
    for (int i = 0; i < n_tensors; ++i)
        if (!host_tensors[i]) return fail(nullptr, KIE_ERR_ARG, "null tensor pointer");
    kie_model* m = new kie_model;
    m->cfg = *cfg;
    make_layout(*cfg, &m->lay);
    m->ws = (uint8_t*)dev_workspace;
    m->stream = (hipStream_t)hip_stream;
    m->pos = 0;
    m->pending = -1;
    m->id_next = 1;
    m->last_ms = 0.f;
    m->ev0 = m->ev1 = nullptr;
    m->spin_limit = kDefaultSpin;
    m->watchdog_ms = 0;
    m->hstatus = nullptr;
    m->prefill_mode = KIE_PREFILL_AUTO;
    m->attn_mode = KIE_ATTN_GLOBAL;
    if (ws_bytes < m->lay.total) {
        rc = fail(nullptr, KIE_ERR_WORKSPACE, "workspace smaller than kie_workspace_bytes()");
        delete m;
        return rc;
    }
    if ((rc = check_device(m)) != KIE_OK) {
        g_err = m->err;
        delete m;
        return rc;
    }
    const Layout& L = m->lay;
    const Dims& D = L.D;
    const uint16_t* const* T = (const uint16_t* const*)host_tensors;
    size_t stage_bytes = L.layer_bytes;
    if (L.lm_bytes > stage_bytes) stage_bytes = L.lm_bytes;
    if (L.expert_bytes > stage_bytes) stage_bytes = L.expert_bytes;
    size_t rope_bytes = (size_t)D.max_seq * (D.hd / 2) * 8;
    if (rope_bytes > stage_bytes) stage_bytes = rope_bytes;
    std::vector<uint8_t> stage(stage_bytes);
    auto bail = [&](int code) {
        g_err = m->err;
        delete m;
        return code;
    };
    std::vector<float> scales(D.w8 ? (size_t)D.L * L.layer_scales + D.V : 0);
    for (int l = 0; l < D.L; ++l) {
        if (D.w8)
            repack_layer_fp8(*cfg, L, T, l, stage.data(), scales.data() + (size_t)l * L.layer_scales);
        else
            repack_layer(*cfg, L, T, l, (uint16_t*)stage.data());
        if ((rc = upload(m, L.off_layers + (size_t)l * L.layer_bytes, stage.data(), L.layer_bytes)) != KIE_OK)
            return bail(rc);
        if (D.E) {
            std::vector<float> esc(D.w8 ? (size_t)(2 * D.F + D.d) : 0);
            for (int e = 0; e < D.E; ++e) {
                if (D.w8) {
                    repack_expert_quant(*cfg, L, T, l, e, stage.data(), esc.data());
                    size_t so = L.off_escales + ((size_t)l * D.E + e) * esc.size() * 4;
                    if ((rc = upload(m, so, esc.data(), esc.size() * 4)) != KIE_OK) return bail(rc);
                } else {
                    repack_expert(*cfg, L, T, l, e, (uint16_t*)stage.data());
                }
                size_t off = L.off_experts + ((size_t)l * D.E + e) * L.expert_bytes;
                if ((rc = upload(m, off, stage.data(), L.expert_bytes)) != KIE_OK) return bail(rc);
            }
        }
    }
    if (D.w8) {
        repack_lm_fp8(*cfg, L, T, stage.data(), scales.data() + (size_t)D.L * L.layer_scales);
        if ((rc = upload(m, L.off_scales, scales.data(), scales.size() * 4)) != KIE_OK) return bail(rc);
    } else {
        repack_lm(*cfg, L, T, (uint16_t*)stage.data());
    }
    if ((rc = upload(m, L.off_lm, stage.data(), L.lm_bytes)) != KIE_OK) return bail(rc);
    if ((rc = upload(m, L.off_emb, T[tidx_emb()], (size_t)D.V * D.d * 2)) != KIE_OK) return bail(rc);
    rope_table(*cfg, (float*)stage.data());
    if ((rc = upload(m, L.off_rope, stage.data(), rope_bytes)) != KIE_OK) return bail(rc);
    std::vector<int32_t> plan(2 * (kGrid + 1));
    for (int w = 0; w <= kGrid; ++w) {
        plan[w] = L.piece_off[w];
        plan[kGrid + 1 + w] = L.lm_off[w];
    }
    if ((rc = upload(m, L.off_plan, plan.data(), plan.size() * 4)) != KIE_OK) return bail(rc);
    if (batched_prefill_ok(D)) {
        // where each workgroup's rows of QKV, Wo, gate/up and down start in a
        // layer block, and its LM rows in the LM block (units)
        std::vector<int32_t> slab(5 * kGrid);
        for (int w = 0; w < kGrid; ++w) {
            int off = L.piece_off[w];
            for (int i = 0; i < layer_block_phase_count(D); ++i) {
                slab[i * kGrid + w] = off;
                off += phase_units(D, layer_block_phase(D, i), kGrid, w);
            }
            slab[4 * kGrid + w] = L.lm_off[w];
        }
        if ((rc = upload(m, L.off_pf_slab, slab.data(), slab.size() * 4)) != KIE_OK) return bail(rc);
    }
    static_assert(kIdleBytes <= 16384, "idle region");
    if (hipMemsetAsync(m->ws + L.off_idle, 0, 16384, m->stream) != hipSuccess) return bail(KIE_ERR_HIP);
    if ((rc = clear_state(m, true)) != KIE_OK) return bail(rc);
    hipError_t e = hipEventCreate(&m->ev0);
    if (e == hipSuccess) e = hipEventCreate(&m->ev1);
    if (e == hipSuccess) e = hipHostMalloc((void**)&m->hstatus, 64, hipHostMallocDefault);
    if (e != hipSuccess) {
        hip_fail(m, e, "hipEventCreate / hipHostMalloc");
        if (m->ev0) (void)hipEventDestroy(m->ev0);
        if (m->ev1) (void)hipEventDestroy(m->ev1);
        return bail(KIE_ERR_HIP);
    }
    __atomic_store_n(m->hstatus, 0u, __ATOMIC_SEQ_CST);
    *out = m;
    return KIE_OK;
}

// n passes from the current position. force (host, may be null): next input
// of pass i where force[i] >= 0. One launch unless debug rows are requested,
// then launches of at most kDebugRows passes.
static int run_passes(kie_model* m, int n, const int32_t* force, int32_t* out_ids, float* dbg_logits,
                      int32_t* dbg_experts, float* dbg_router, int64_t* trace, bool skip_lm) {
    const Layout& L = m->lay;
    const Dims& D = L.D;
    const bool debug = dbg_logits || dbg_experts || dbg_router;
    const int chunk = debug ? kDebugRows : n;
    int tok = m->pending;
    for (int s0 = 0; s0 < n; s0 += chunk) {
        int nc = (n - s0 < chunk) ? n - s0 : chunk;
        const uint32_t nphase = (uint32_t)nc * (uint32_t)phases_per_step(D);
        if (m->id_next > 0xffffffffu - nphase) {
            // phase ids would wrap: forget every published word and restart
            int rc = clear_state(m, false);
            if (rc != KIE_OK) return rc;
        }
        if (force)
            HIP_TRY(m, hipMemcpyAsync(m->ws + L.off_force, force + s0, (size_t)nc * 4, hipMemcpyHostToDevice,
                                      m->stream));
        DecodeArgs a;
        memset(&a, 0, sizeof(a));
        a.D = D;
        a.eps = m->cfg.rms_eps;
        a.items_per_head = L.attn_items_per_head;
        a.spin = m->spin_limit;
        a.layers = m->ws + L.off_layers;
        a.layer_bytes = L.layer_bytes;
        a.lm = m->ws + L.off_lm;
        a.emb = (const uint16_t*)(m->ws + L.off_emb);
        a.experts = m->ws + L.off_experts;
        a.expert_bytes = L.expert_bytes;
        a.rope = (const float*)(m->ws + L.off_rope);
        a.kc = (uint16_t*)(m->ws + L.off_k);
        a.vc = (uint16_t*)(m->ws + L.off_v);
        a.ex.x = (uint64_t*)(m->ws + L.off_ex_x);
        a.ex.qkv = (uint64_t*)(m->ws + L.off_ex_qkv);
        a.ex.part = (uint64_t*)(m->ws + L.off_ex_part);
        a.ex.o = (uint64_t*)(m->ws + L.off_ex_o);
        a.ex.part_copy = (int64_t)L.ex_part_copy;
        a.ex.o_copy = (int64_t)L.ex_o_copy;
        a.ex.h = (uint64_t*)(m->ws + L.off_ex_h);
        a.ex.r = (uint64_t*)(m->ws + L.off_ex_r);
        a.ex.am = (uint64_t*)(m->ws + L.off_ex_am);
        a.status = m->hstatus;
        a.out_ids = (int32_t*)(m->ws + L.off_out);
        a.force_ids = (const int32_t*)(m->ws + L.off_force);
        a.dbg_logits = (float*)(m->ws + L.off_dbg_logits);
        a.dbg_experts = (int32_t*)(m->ws + L.off_dbg_experts);
        a.dbg_router = (float*)(m->ws + L.off_dbg_router);
        a.plan = (const int32_t*)(m->ws + L.off_plan);
        a.idle = m->ws + L.off_idle;
        a.trace = (int64_t*)(m->ws + L.off_trace);
        a.scales = D.w8 ? (const float*)(m->ws + L.off_scales) : nullptr;
        a.escales = (D.w8 && D.E) ? (const float*)(m->ws + L.off_escales) : nullptr;
        a.layer_scales = (int32_t)L.layer_scales;
        a.pos0 = m->pos + s0;
        a.pending = tok;
        a.n_steps = nc;
        a.flags = (force ? F_FORCE : 0) | (dbg_logits ? F_DBG_LOGITS : 0) | ((dbg_experts || dbg_router) ? F_DBG_EXPERTS : 0) |
                  ((skip_lm && !debug) ? F_SKIP_LM : 0) | ((trace && s0 == 0) ? F_TRACE : 0) |
                  (m->attn_mode == KIE_ATTN_XCD_LOCAL ? F_XCD_ATTN : 0);
        a.id0 = m->id_next;
        m->id_next += nphase;
        static_assert(sizeof(DecodeArgs) <= 4096, "argument block");
        static_assert(KIE_TRACE_PHASES == kTracePhases, "trace length");
        HIP_TRY(m, hipMemcpyAsync(m->ws + L.off_args, &a, sizeof(a), hipMemcpyHostToDevice, m->stream));
        __atomic_store_n(m->hstatus, 0u, __ATOMIC_SEQ_CST);   // the previous launch has ended
        HIP_TRY(m, hipEventRecord(m->ev0, m->stream));
        // the variant with the matrix-core split attention only where a pass
        // of this launch (the last attends pos0 + nc positions) leaves head mode
        const bool ms = D.hd == 128 && !head_mode_at(D, a.pos0 + nc);
        HIP_TRY(m, launch_decode((const DecodeArgs*)(m->ws + L.off_args), D.hd, D.w4 ? 2 : D.w8 ? 1 : 0, ms,
                                 (a.flags & F_XCD_ATTN) != 0, skip_lm, kGrid, m->stream));
        HIP_TRY(m, hipEventRecord(m->ev1, m->stream));
        // Host watchdog: poll the launch's end event against a wall-clock
        // limit. Past it, set the status word the kernel's long waits read
        // (workgroups that wait on each other then give up and exit), let the
        // launch end and report KIE_ERR_TIMEOUT. A kernel that still makes
        // progress runs to its end; the overrun is reported all the same.
        const double limit = watchdog_limit_ms(m, nc);
        const auto t0 = std::chrono::steady_clock::now();
        bool fired = false;
        while (true) {
            hipError_t q = hipEventQuery(m->ev1);
            if (q == hipSuccess) break;
            if (q != hipErrorNotReady) return hip_fail(m, q, "hipEventQuery");
            const double el = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
            if (!fired && limit >= 0.0 && el > limit) {
                __atomic_store_n(m->hstatus, kStatusHostAbort, __ATOMIC_SEQ_CST);
                fired = true;
            }
            if (el < 5.0) std::this_thread::yield();   // short launches: no sleep granularity
            else std::this_thread::sleep_for(std::chrono::microseconds(20));
        }
        HIP_TRY(m, hipEventElapsedTime(&m->last_ms, m->ev0, m->ev1));
        const uint32_t status = __atomic_load_n(m->hstatus, __ATOMIC_SEQ_CST);
        if (fired) {
            m->pending = -1;
            return fail(m, KIE_ERR_TIMEOUT, "the launch exceeded the host watchdog's wall-clock limit");
        }
        if (status == kStatusWrongXcd) {
            m->pending = -1;
            return fail(m, KIE_ERR_DEVICE,
                        "XCD-local attention: a workgroup did not run on XCD (its index mod 8); the launch exited");
        }
        if (status != 0) {
            m->pending = -1;
            return fail(m, KIE_ERR_TIMEOUT, "a device-side wait for another workgroup hit its spin limit");
        }
        HIP_TRY(m, hipMemcpy(out_ids + s0, m->ws + L.off_out, (size_t)nc * 4, hipMemcpyDeviceToHost));
        if (dbg_logits)
            HIP_TRY(m, hipMemcpy(dbg_logits + (size_t)s0 * D.V, m->ws + L.off_dbg_logits, (size_t)nc * D.V * 4,
                                 hipMemcpyDeviceToHost));
        if (dbg_experts)
            HIP_TRY(m, hipMemcpy(dbg_experts + (size_t)s0 * D.L * D.topk, m->ws + L.off_dbg_experts,
                                 (size_t)nc * D.L * D.topk * 4, hipMemcpyDeviceToHost));
        if (dbg_router)
            HIP_TRY(m, hipMemcpy(dbg_router + (size_t)s0 * D.L * D.E, m->ws + L.off_dbg_router,
                                 (size_t)nc * D.L * D.E * 4, hipMemcpyDeviceToHost));
        if (trace && s0 == 0) {
            size_t np = (size_t)nphase < (size_t)kTracePhases ? (size_t)nphase : (size_t)kTracePhases;
            HIP_TRY(m, hipMemcpy(trace, m->ws + L.off_trace, np * kGrid * 4 * 8, hipMemcpyDeviceToHost));
        }
        int last = nc - 1;
        tok = (force && force[s0 + last] >= 0) ? force[s0 + last] : out_ids[s0 + last];
    }
    m->pos += n;
    m->pending = tok;
    return KIE_OK;
}

// The prompt as batched GEMMs on the matrix cores (kie_prefill.hip), in chunks
// of kPrefillRows tokens: per layer RMSNorm, QKV GEMM, RoPE and KV append,
// causal attention over the cache, Wo GEMM + residual, RMSNorm, gate/up GEMM,
// SwiGLU, down GEMM + residual; then the final norm, the LM head GEMM (every
// row when logits are asked for, else the chunk that holds the last token)
// and the argmax of the last row. Many small launches on the model's stream:
// prefill is not the decode metric.
static int run_batched_prefill(kie_model* m, const int32_t* tokens, int n, int32_t* first, float* dbg_logits) {
    const Layout& L = m->lay;
    const Dims& D = L.D;
    hipStream_t s = m->stream;
    uint8_t* ws = m->ws;
    const int32_t* slab = (const int32_t*)(ws + L.off_pf_slab);
    const int qkvM = (D.H + 2 * D.Hkv) * D.hd, qd = D.H * D.hd;
    PrefillRowArgs r;
    memset(&r, 0, sizeof(r));
    r.D = D;
    r.eps = m->cfg.rms_eps;
    r.emb = (const uint16_t*)(ws + L.off_emb);
    r.tok = (const int32_t*)(ws + L.off_pf_tok);
    r.X = (float*)(ws + L.off_pf_x);
    r.A = (float*)(ws + L.off_pf_a);
    r.Y = (const float*)(ws + L.off_pf_y);
    r.Q = (float*)(ws + L.off_pf_q);
    r.rope = (const float*)(ws + L.off_rope);
    r.kc = (uint16_t*)(ws + L.off_k);
    r.vc = (uint16_t*)(ws + L.off_v);
    r.out = (int32_t*)(ws + L.off_pf_tok) + kPrefillRows;
    float* Y = (float*)(ws + L.off_pf_y);
    auto rows = [&](int op) -> hipError_t { return launch_prefill_rows(op, r, s); };
    // quantised weights: each phase's row scales (per layer: QKV, Wo, gate/up,
    // down rows; the LM head's after the last layer)
    const float* sc = D.w8 ? (const float*)(ws + L.off_scales) : nullptr;
    const int wf = D.w4 ? 2 : D.w8 ? 1 : 0;
    auto gemm = [&](const float* A, int lda, const uint8_t* base, const int32_t* sl, int ph, const float* scales) {
        const PhaseShape ps = phase_shape(D, ph);
        GemmRows R;
        R.base = base;
        R.slab = sl;
        R.M = ps.M;
        R.K = ps.K;
        R.gran = ps.gran;
        R.dense = 0;
        R.wf = wf;
        R.scales = scales;
        return launch_gemm_mfma(A, lda, r.n, R, Y, ps.M, s);
    };
#define PF_TRY(call)                                         \
    do {                                                     \
        hipError_t e_ = (call);                              \
        if (e_ != hipSuccess) return hip_fail(m, e_, #call); \
    } while (0)
    for (int c0 = 0; c0 < n; c0 += kPrefillRows) {
        const int nc = (n - c0 < kPrefillRows) ? n - c0 : kPrefillRows;
        const bool last = c0 + nc == n;
        r.n = nc;
        r.pos0 = c0;
        PF_TRY(hipMemcpyAsync(ws + L.off_pf_tok, tokens + c0, (size_t)nc * 4, hipMemcpyHostToDevice, s));
        PF_TRY(rows(PF_EMBED));
        for (int l = 0; l < D.L; ++l) {
            const uint8_t* blk = ws + L.off_layers + (size_t)l * L.layer_bytes;
            const float* ls = sc ? sc + (size_t)l * L.layer_scales : nullptr;
            const int mo = D.d, mg = 2 * D.F;
            r.layer = l;
            PF_TRY(rows(PF_RMSNORM));
            PF_TRY(gemm(r.A, D.d, blk, slab + 0 * kGrid, PH_QKV, ls));
            r.ldy = qkvM;
            PF_TRY(rows(PF_QKV));
            PF_TRY(rows(PF_ATTN));
            PF_TRY(gemm(r.A, qd, blk, slab + 1 * kGrid, PH_WO, ls ? ls + qkvM : nullptr));
            r.ldy = D.d;
            PF_TRY(rows(PF_RESIDUAL));
            PF_TRY(rows(PF_RMSNORM));
            PF_TRY(gemm(r.A, D.d, blk, slab + 2 * kGrid, PH_GU, ls ? ls + qkvM + mo : nullptr));
            r.ldy = 2 * D.F;
            PF_TRY(rows(PF_SWIGLU));
            PF_TRY(gemm(r.A, D.F, blk, slab + 3 * kGrid, PH_DOWN, ls ? ls + qkvM + mo + mg : nullptr));
            r.ldy = D.d;
            PF_TRY(rows(PF_RESIDUAL));
        }
        if (!last && !dbg_logits) continue;
        PF_TRY(rows(PF_RMSNORM));
        PF_TRY(gemm(r.A, D.d, ws + L.off_lm, slab + 4 * kGrid, PH_LM, sc ? sc + (size_t)D.L * L.layer_scales : nullptr));
        if (dbg_logits)
            PF_TRY(hipMemcpyAsync(dbg_logits + (size_t)c0 * D.V, Y, (size_t)nc * D.V * 4, hipMemcpyDeviceToHost, s));
        if (last) {
            PrefillRowArgs am = r;
            am.Y = Y + (size_t)(nc - 1) * D.V;
            PF_TRY(launch_prefill_rows(PF_ARGMAX, am, s));
            PF_TRY(hipMemcpyAsync(first, r.out, 4, hipMemcpyDeviceToHost, s));
        }
    }
#undef PF_TRY
    HIP_TRY(m, hipStreamSynchronize(s));
    m->last_ms = 0.f;
    return KIE_OK;
}

int kie_prefill(kie_model* m, const int32_t* tokens, int32_t n, int32_t* first_token, const kie_debug* dbg) {
    if (!m) return fail(nullptr, KIE_ERR_ARG, "null model");
    if (!tokens || !first_token || n < 1) return fail(m, KIE_ERR_ARG, "need at least one prompt token");
    if (n > m->cfg.max_seq) return fail(m, KIE_ERR_CAPACITY, "prompt longer than max_seq");
    for (int i = 0; i < n; ++i)
        if (tokens[i] < 0 || tokens[i] >= m->cfg.vocab) return fail(m, KIE_ERR_ARG, "prompt token out of range");
    if (dbg && (dbg->experts || dbg->router) && m->cfg.n_experts == 0)
        return fail(m, KIE_ERR_ARG, "experts or router logits requested for a dense model");
    if (m->prefill_mode == KIE_PREFILL_AUTO && batched_prefill_ok(m->lay.D) && !(dbg && dbg->trace)) {
        m->pos = 0;
        m->pending = -1;
        int32_t first = 0;
        int rc = run_batched_prefill(m, tokens, n, &first, dbg ? dbg->logits : nullptr);
        if (rc != KIE_OK) return rc;
        m->pos = n;
        m->pending = first;
        *first_token = first;
        return KIE_OK;
    }
    std::vector<int32_t> force(n);
    for (int i = 0; i + 1 < n; ++i) force[i] = tokens[i + 1];
    force[n - 1] = -1;
    std::vector<int32_t> ids(n);
    m->pos = 0;
    m->pending = tokens[0];
    int rc = run_passes(m, n, force.data(), ids.data(), dbg ? dbg->logits : nullptr, dbg ? dbg->experts : nullptr,
                        dbg ? dbg->router : nullptr, dbg ? dbg->trace : nullptr, true);
    if (rc != KIE_OK) return rc;
    *first_token = ids[n - 1];
    return KIE_OK;
}

int kie_decode(kie_model* m, int32_t n, int32_t* out_ids, const kie_debug* dbg) {
    if (!m) return fail(nullptr, KIE_ERR_ARG, "null model");
    if (!out_ids || n < 1) return fail(m, KIE_ERR_ARG, "need n_tokens >= 1 and an output buffer");
    if (m->pending < 0) return fail(m, KIE_ERR_STATE, "no pending token: call kie_prefill or kie_set_kv first");
    if ((long)m->pos + n > m->cfg.max_seq) return fail(m, KIE_ERR_CAPACITY, "position + n_tokens exceeds max_seq");
    if (dbg && (dbg->experts || dbg->router) && m->cfg.n_experts == 0)
        return fail(m, KIE_ERR_ARG, "experts or router logits requested for a dense model");
    const int32_t* force = dbg ? dbg->force_ids : nullptr;
    if (force)
        for (int i = 0; i < n; ++i)
            if (force[i] >= m->cfg.vocab) return fail(m, KIE_ERR_ARG, "forced token out of range");
    return run_passes(m, n, force, out_ids, dbg ? dbg->logits : nullptr, dbg ? dbg->experts : nullptr,
                      dbg ? dbg->router : nullptr, dbg ? dbg->trace : nullptr, false);
}

int kie_set_kv(kie_model* m, const void* k, const void* v, int32_t n_pos, int32_t pending) {
    if (!m) return fail(nullptr, KIE_ERR_ARG, "null model");
    if (!k || !v || n_pos < 0) return fail(m, KIE_ERR_ARG, "null cache or negative length");
    if (n_pos > m->cfg.max_seq) return fail(m, KIE_ERR_CAPACITY, "n_pos exceeds max_seq");
    if (pending < 0 || pending >= m->cfg.vocab) return fail(m, KIE_ERR_ARG, "pending token out of range");
    const Layout& L = m->lay;
    const Dims& D = L.D;
    int rc = clear_state(m, true);
    if (rc != KIE_OK) return rc;
    // host [L][n_pos][Hkv][hd] -> device [L][Hkv][max_seq][hd]
    size_t blk = (size_t)n_pos * D.hd;   // halves per (layer, head)
    std::vector<uint16_t> stage((size_t)D.Hkv * blk);
    for (int which = 0; which < 2; ++which) {
        const uint16_t* src = (const uint16_t*)(which ? v : k);
        size_t base = which ? L.off_v : L.off_k;
        for (int l = 0; l < D.L; ++l) {
            for (int p = 0; p < n_pos; ++p)
                for (int g = 0; g < D.Hkv; ++g)
                    memcpy(&stage[(size_t)g * blk + (size_t)p * D.hd],
                           src + (((size_t)l * n_pos + p) * D.Hkv + g) * D.hd, (size_t)D.hd * 2);
            for (int g = 0; g < D.Hkv; ++g) {
                size_t off = base + (((size_t)l * D.Hkv + g) * D.max_seq) * D.hd * 2;
                if ((rc = upload(m, off, &stage[(size_t)g * blk], blk * 2)) != KIE_OK) return rc;
            }
        }
    }
    m->pos = n_pos;
    m->pending = pending;
    return KIE_OK;
}

int kie_rewind(kie_model* m, int32_t pos, int32_t pending) {
    if (!m) return fail(nullptr, KIE_ERR_ARG, "null model");
    if (pos < 0 || pos > m->pos) return fail(m, KIE_ERR_ARG, "can only rewind to an earlier position");
    if (pending < 0 || pending >= m->cfg.vocab) return fail(m, KIE_ERR_ARG, "pending token out of range");
    m->pos = pos;
    m->pending = pending;
    return KIE_OK;
}

int kie_reset(kie_model* m) {
    if (!m) return fail(nullptr, KIE_ERR_ARG, "null model");
    int rc = clear_state(m, true);
    if (rc != KIE_OK) return rc;
    m->pos = 0;
    m->pending = -1;
    return KIE_OK;
}

int kie_state(const kie_model* m, int32_t* pos, int32_t* pending) {
    if (!m || !pos || !pending) return fail(nullptr, KIE_ERR_ARG, "null argument");
    *pos = m->pos;
    *pending = m->pending;
    return KIE_OK;
}

float kie_last_kernel_ms(const kie_model* m) { return m ? m->last_ms : 0.f; }
int32_t kie_grid_size(const kie_model* m) { return m ? kGrid : 0; }

int kie_quantize_e4m3_rows(const void* w_fp16, const void* gain_fp16, int32_t rows, int32_t K, uint8_t* q,
                           float* scales) {
    if (!w_fp16 || !q || !scales || rows < 0 || K < 1) return fail(nullptr, KIE_ERR_ARG, "bad argument");
    const uint16_t* w = (const uint16_t*)w_fp16;
    for (int r = 0; r < rows; ++r)
        quantize_row_e4m3(w + (size_t)r * K, (const uint16_t*)gain_fp16, K, q + (size_t)r * K, scales + r);
    return KIE_OK;
}

int kie_quantize_e2m1_rows(const void* w_fp16, const void* gain_fp16, int32_t rows, int32_t K, uint8_t* q,
                           float* scales) {
    if (!w_fp16 || !q || !scales || rows < 0 || K < 1) return fail(nullptr, KIE_ERR_ARG, "bad argument");
    const uint16_t* w = (const uint16_t*)w_fp16;
    for (int r = 0; r < rows; ++r)
        quantize_row_e2m1(w + (size_t)r * K, (const uint16_t*)gain_fp16, K, q + (size_t)r * K, scales + r);
    return KIE_OK;
}

int kie_set_prefill_mode(kie_model* m, int32_t mode) {
    if (!m) return fail(nullptr, KIE_ERR_ARG, "null model");
    if (mode != KIE_PREFILL_AUTO && mode != KIE_PREFILL_PASSES) return fail(m, KIE_ERR_ARG, "unknown prefill mode");
    m->prefill_mode = mode;
    return KIE_OK;
}

int kie_set_attention_mode(kie_model* m, int32_t mode) {
    if (!m) return fail(nullptr, KIE_ERR_ARG, "null model");
    if (mode != KIE_ATTN_GLOBAL && mode != KIE_ATTN_XCD_LOCAL) return fail(m, KIE_ERR_ARG, "unknown attention mode");
    if (mode == KIE_ATTN_XCD_LOCAL && !xcd_attention_ok(m->lay.D))
        return fail(m, KIE_ERR_CONFIG,
                    "XCD-local attention needs 2 to 8 query heads per KV head and at most 32 query heads");
    m->attn_mode = mode;
    return KIE_OK;
}

int kie_gemm_probe(const float* A, const void* W, float* Y, int32_t n, int32_t M, int32_t K, void* hip_stream,
                   float* ms_out) {
    if (!A || !W || !Y || n < 1 || M < 1 || K < 64 || K % 64) return fail(nullptr, KIE_ERR_ARG, "bad argument");
    hipStream_t s = (hipStream_t)hip_stream;
    GemmRows R;
    R.base = (const uint8_t*)W;
    R.slab = nullptr;
    R.M = M;
    R.K = K;
    R.gran = 1;
    R.dense = 1;
    R.wf = 0;
    R.scales = nullptr;
    hipEvent_t e0, e1;
    HIP_TRY(nullptr, hipEventCreate(&e0));
    HIP_TRY(nullptr, hipEventCreate(&e1));
    HIP_TRY(nullptr, hipEventRecord(e0, s));
    hipError_t le = launch_gemm_mfma(A, K, n, R, Y, M, s);
    if (le != hipSuccess) return hip_fail(nullptr, le, "gemm probe launch");
    HIP_TRY(nullptr, hipEventRecord(e1, s));
    HIP_TRY(nullptr, hipEventSynchronize(e1));
    float ms = 0.f;
    HIP_TRY(nullptr, hipEventElapsedTime(&ms, e0, e1));
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (ms_out) *ms_out = ms;
    return KIE_OK;
}

int kie_set_limits(kie_model* m, uint32_t spin_limit, int32_t watchdog_ms) {
    if (!m) return fail(nullptr, KIE_ERR_ARG, "null model");
    m->spin_limit = spin_limit ? spin_limit : kDefaultSpin;
    m->watchdog_ms = watchdog_ms;
    return KIE_OK;
}

void kie_free(kie_model* m) {
    if (!m) return;
    if (m->ev0) (void)hipEventDestroy(m->ev0);
    if (m->ev1) (void)hipEventDestroy(m->ev1);
    if (m->hstatus) (void)hipHostFree(m->hstatus);
    delete m;
}

// ---------------------------------------------------------------- probes --
int kie_gemv_probe(const void* A, const void* x, float* y, int32_t M, int32_t K, int32_t copies,
                   int32_t variant, void* hip_stream, float* ms_out) {
    if (!A || !x || !y) return fail(nullptr, KIE_ERR_ARG, "null pointer");
    if (M < 1 || copies < 1 || K < 512 || K % 512 || K > 65536)
        return fail(nullptr, KIE_ERR_ARG, "need M >= 1, copies >= 1, K a multiple of 512 up to 65536");
    if (variant != 0 && variant != 1) return fail(nullptr, KIE_ERR_ARG, "variant must be 0 (stream) or 1 (direct)");
    if ((long)M * copies * K < kIdleBytes / 2)
        return fail(nullptr, KIE_ERR_ARG, "the matrices must hold at least one batch (kNB KiB)");
    hipStream_t s = (hipStream_t)hip_stream;
    hipEvent_t e0, e1;
    HIP_TRY(nullptr, hipEventCreate(&e0));
    HIP_TRY(nullptr, hipEventCreate(&e1));
    GemvArgs a;
    a.A = (const uint8_t*)A;
    a.x = (const uint16_t*)x;
    a.y = y;
    a.idle = (const uint8_t*)A;   // any readable 4 KiB: the loads it serves are never used
    a.lda = K;
    a.M = M;
    a.K = K;
    a.copies = copies;
    a.accumulate = 0;
    // the streaming variant adds row partial sums into y
    if (variant == 0) HIP_TRY(nullptr, hipMemsetAsync(y, 0, (size_t)M * copies * sizeof(float), s));
    HIP_TRY(nullptr, hipEventRecord(e0, s));
    if (variant == 0) {
        // the streaming kernel keeps x in LDS: column blocks of at most kMaxInput
        for (int k0 = 0; k0 < K; k0 += kMaxInput) {
            GemvArgs b = a;
            b.A = a.A + (size_t)k0 * 2;
            b.x = a.x + k0;
            b.K = (K - k0 < kMaxInput) ? K - k0 : kMaxInput;
            b.accumulate = k0 > 0;
            hipError_t le = launch_gemv_stream(b, kGrid, s);
            if (le != hipSuccess) return hip_fail(nullptr, le, "gemv probe launch");
        }
    } else {
        hipError_t le = launch_gemv_direct(a, s);
        if (le != hipSuccess) return hip_fail(nullptr, le, "gemv probe launch");
    }
    HIP_TRY(nullptr, hipEventRecord(e1, s));
    HIP_TRY(nullptr, hipEventSynchronize(e1));
    float ms = 0.f;
    HIP_TRY(nullptr, hipEventElapsedTime(&ms, e0, e1));
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (ms_out) *ms_out = ms;
    return KIE_OK;
}

size_t kie_barrier_probe_bytes(void) { return 65536; }

int kie_barrier_probe(void* scratch, int32_t variant, int32_t rounds, void* hip_stream, float* us_per_round,
                      int32_t* errors) {
    if (!scratch || !us_per_round || !errors || rounds < 1) return fail(nullptr, KIE_ERR_ARG, "bad argument");
    if (variant < 0 || variant > 2)
        return fail(nullptr, KIE_ERR_ARG, "variant must be 0 (fenced), 1 (flagged) or 2 (XCD-aware)");
    hipStream_t s = (hipStream_t)hip_stream;
    uint8_t* b = (uint8_t*)scratch;
    uint64_t* words = (uint64_t*)b;               // 2 x 5 x 256 words = 20 KiB
    uint32_t* status = (uint32_t*)(b + 32768);
    int32_t* err = (int32_t*)(b + 32768 + 256);
    HIP_TRY(nullptr, hipMemsetAsync(scratch, 0, kie_barrier_probe_bytes(), s));
    hipEvent_t e0, e1;
    HIP_TRY(nullptr, hipEventCreate(&e0));
    HIP_TRY(nullptr, hipEventCreate(&e1));
    HIP_TRY(nullptr, hipEventRecord(e0, s));
    hipError_t le = launch_barrier_probe(variant, words, status, err, rounds, kGrid, s);
    if (le != hipSuccess) return hip_fail(nullptr, le, "barrier probe launch");
    HIP_TRY(nullptr, hipEventRecord(e1, s));
    HIP_TRY(nullptr, hipEventSynchronize(e1));
    float ms = 0.f;
    HIP_TRY(nullptr, hipEventElapsedTime(&ms, e0, e1));
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    HIP_TRY(nullptr, hipMemcpy(errors, err, 4, hipMemcpyDeviceToHost));
    *us_per_round = ms * 1000.f / (float)rounds;
    return KIE_OK;
}

int kie_barrier_probe_noalloc(int32_t variant, int32_t rounds, void* hip_stream, float* us_per_round,
                              int32_t* errors) {
    if (!us_per_round || !errors || rounds < 1) return fail(nullptr, KIE_ERR_ARG, "bad argument");
    if (variant < 0 || variant > 2)
        return fail(nullptr, KIE_ERR_ARG, "variant must be 0 (fenced), 1 (flagged) or 2 (XCD-aware)");
    if (kie_barrier_probe_bytes() > noalloc_scratch_bytes())
        return fail(nullptr, KIE_ERR_WORKSPACE, "the probe needs more scratch than the library's 64 KiB array");
    void* ptr = nullptr;
    HIP_TRY(nullptr, noalloc_scratch(&ptr));
    hipStream_t s = (hipStream_t)hip_stream;
    uint8_t* b = (uint8_t*)ptr;
    uint64_t* words = (uint64_t*)b;               // same layout as kie_barrier_probe's scratch
    uint32_t* status = (uint32_t*)(b + 32768);
    int32_t* err = (int32_t*)(b + 32768 + 256);
    // the previous call's words, status and count are still there: clear them
    HIP_TRY(nullptr, launch_fill_zero((uint32_t*)ptr, (int)(kie_barrier_probe_bytes() / 4), s));
    HIP_TRY(nullptr, hipStreamSynchronize(s));
    const auto t0 = std::chrono::steady_clock::now();
    hipError_t le = launch_barrier_probe(variant, words, status, err, rounds, kGrid, s);
    if (le != hipSuccess) return hip_fail(nullptr, le, "barrier probe launch");
    HIP_TRY(nullptr, hipStreamSynchronize(s));
    const auto t1 = std::chrono::steady_clock::now();
    HIP_TRY(nullptr, hipMemcpy(errors, err, 4, hipMemcpyDeviceToHost));
    *us_per_round = (float)(std::chrono::duration<double, std::micro>(t1 - t0).count() / rounds);
    return KIE_OK;
}

int kie_e4m3_table_probe(float* out256, void* hip_stream) {
    if (!out256) return fail(nullptr, KIE_ERR_ARG, "null output");
    hipStream_t s = (hipStream_t)hip_stream;
    void* ptr = nullptr;   // the no-alloc scratch: 256 floats of output
    HIP_TRY(nullptr, noalloc_scratch(&ptr));
    HIP_TRY(nullptr, launch_e4m3_table((float*)ptr, s));
    HIP_TRY(nullptr, hipStreamSynchronize(s));
    HIP_TRY(nullptr, hipMemcpy(out256, ptr, 256 * sizeof(float), hipMemcpyDeviceToHost));
    return KIE_OK;
}

int kie_e2m1_table_probe(float* out64, void* hip_stream) {
    if (!out64) return fail(nullptr, KIE_ERR_ARG, "null output");
    hipStream_t s = (hipStream_t)hip_stream;
    void* ptr = nullptr;   // the no-alloc scratch: 64 floats of output
    HIP_TRY(nullptr, noalloc_scratch(&ptr));
    HIP_TRY(nullptr, launch_e2m1_table((float*)ptr, s));
    HIP_TRY(nullptr, hipStreamSynchronize(s));
    HIP_TRY(nullptr, hipMemcpy(out64, ptr, 64 * sizeof(float), hipMemcpyDeviceToHost));
    return KIE_OK;
}

int kie_xcd_map(int32_t* out_xcd, void* hip_stream) {
    if (!out_xcd) return fail(nullptr, KIE_ERR_ARG, "null output");
    hipStream_t s = (hipStream_t)hip_stream;
    void* ptr = nullptr;   // the no-alloc scratch: kGrid words of output
    HIP_TRY(nullptr, noalloc_scratch(&ptr));
    hipError_t le = launch_xcd_map((int32_t*)ptr, kGrid, s);
    if (le != hipSuccess) return hip_fail(nullptr, le, "xcd map launch");
    HIP_TRY(nullptr, hipStreamSynchronize(s));
    HIP_TRY(nullptr, hipMemcpy(out_xcd, ptr, kGrid * sizeof(int32_t), hipMemcpyDeviceToHost));
    return KIE_OK;
}

int kie_launch_probe(int32_t launches, void* hip_stream, float* us_per_launch) {
    if (launches < 1 || !us_per_launch) return fail(nullptr, KIE_ERR_ARG, "bad argument");
    hipStream_t s = (hipStream_t)hip_stream;
    HIP_TRY(nullptr, launch_empty(s));
    HIP_TRY(nullptr, hipStreamSynchronize(s));
    auto t0 = std::chrono::steady_clock::now();
    for (int i = 0; i < launches; ++i) HIP_TRY(nullptr, launch_empty(s));
    HIP_TRY(nullptr, hipStreamSynchronize(s));
    auto t1 = std::chrono::steady_clock::now();
    *us_per_launch = (float)(std::chrono::duration<double, std::micro>(t1 - t0).count() / launches);
    return KIE_OK;
}

}  // extern "C"

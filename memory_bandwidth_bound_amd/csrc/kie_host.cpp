// kie_host.cpp - host-only preparation (no HIP): configuration checks, the
// workspace layout, the offline weight repack and the rotary table.
//
// The repack is the offline preparation the news.creeta.com monokernel
// article lists under "Inside the monokernel": RMSNorm is folded into the
// adjacent projection (gains multiply the columns of the next matrix), the
// Q/K/V projections are repacked into one streamable matrix, and the rotary
// embedding is precomputed as a table. On top of that every phase's rows are
// cut per workgroup and laid out so that one workgroup's weights for a whole
// layer are one contiguous run of memory in the order it consumes them.
#include "kie_host.h"

#include <cmath>
#include <cstring>

namespace kie {

Dims dims_of(const kie_config& c) {
    Dims D;
    D.L = c.n_layers;
    D.d = c.d_model;
    D.H = c.n_heads;
    D.Hkv = c.n_kv_heads;
    D.hd = c.head_dim;
    D.F = c.ffn_dim;
    D.V = c.vocab;
    D.E = c.n_experts;
    D.topk = c.n_experts ? c.top_k : 0;
    D.max_seq = c.max_seq;
    D.w8 = (c.weight_format == KIE_WEIGHTS_FP8 || c.weight_format == KIE_WEIGHTS_FP4) ? 1 : 0;
    D.w4 = c.weight_format == KIE_WEIGHTS_FP4 ? 1 : 0;
    return D;
}

static int per_layer_tensors(const kie_config& c) {
    return 6 + (c.n_experts ? 1 + 3 * c.n_experts : 3);
}
int tidx_emb() { return 0; }
int tidx_layer(const kie_config& c, int layer, int which) {
    return 1 + layer * per_layer_tensors(c) + which;
}
int tidx_expert(const kie_config& c, int layer, int expert, int which) {
    return 1 + layer * per_layer_tensors(c) + 7 + 3 * expert + which;
}
int tidx_gfinal(const kie_config& c) { return 1 + c.n_layers * per_layer_tensors(c); }
int tidx_lm(const kie_config& c) { return 2 + c.n_layers * per_layer_tensors(c); }
int tensor_count(const kie_config& c) { return 3 + c.n_layers * per_layer_tensors(c); }

static bool width_ok(int x) { return x == 256 || (x > 0 && x % 512 == 0); }

int validate_config(const kie_config& c, std::string* err) {
    auto fail = [&](const char* m) {
        if (err) *err = m;
        return (int)KIE_ERR_CONFIG;
    };
    if (c.n_layers < 1 || c.n_layers > 4096) return fail("n_layers must be in [1, 4096]");
    if (c.head_dim != 64 && c.head_dim != 128) return fail("head_dim must be 64 or 128");
    if (c.n_heads < 1 || c.n_kv_heads < 1 || c.n_heads % c.n_kv_heads)
        return fail("n_heads must be a positive multiple of n_kv_heads");
    if (c.n_heads / c.n_kv_heads > kMaxGroup) return fail("at most 8 query heads per KV head");
    if (c.n_kv_heads > kGrid) return fail("too many KV heads");
    if (!width_ok(c.d_model)) return fail("d_model must be 256 or a multiple of 512");
    if (!width_ok(c.ffn_dim)) return fail("ffn_dim must be 256 or a multiple of 512");
    if (!width_ok(c.n_heads * c.head_dim)) return fail("n_heads*head_dim must be 256 or a multiple of 512");
    if (c.vocab < 2 || c.vocab > (1 << 24)) return fail("vocab must be in [2, 2^24]");
    if (c.max_seq < 1 || c.max_seq > kMaxSeq) return fail("max_seq must be in [1, 65536]");
    if (!(c.rms_eps > 0.f) || !(c.rope_theta > 1.f)) return fail("rms_eps must be > 0 and rope_theta > 1");
    if (c.n_experts < 0) return fail("n_experts must be >= 0");
    if (c.n_experts) {
        if (c.top_k < 1 || c.top_k > c.n_experts || c.top_k > 16)
            return fail("top_k must be in [1, min(n_experts, 16)]");
        if (c.n_experts > 1024) return fail("at most 1024 experts");
        if (c.d_model % 512 || c.ffn_dim % 512) return fail("MoE needs d_model and ffn_dim multiples of 512");
    }
    if (c.vocab > kMaxRowsWg * kGrid) return fail("vocab must be at most 65536");
    if (c.weight_format != KIE_WEIGHTS_FP16 && c.weight_format != KIE_WEIGHTS_FP8 &&
        c.weight_format != KIE_WEIGHTS_FP4)
        return fail("weight_format must be KIE_WEIGHTS_FP16, KIE_WEIGHTS_FP8 or KIE_WEIGHTS_FP4");
    if (c.weight_format == KIE_WEIGHTS_FP4) {
        if (c.n_experts % 4) return fail("fp4 weights need a multiple of 4 experts (router rows come in fours)");
        if (c.head_dim != 128) return fail("fp4 weights are supported for head_dim 128 only");
        if (c.d_model % 512 || c.ffn_dim % 512 || (c.n_heads * c.head_dim) % 512)
            return fail("fp4 weights need d_model, ffn_dim and n_heads*head_dim multiples of 512");
        if (c.vocab % 4) return fail("fp4 weights need a vocab that is a multiple of 4 (LM rows come in fours)");
    }
    if (c.weight_format == KIE_WEIGHTS_FP8) {
        if (c.n_experts % 2) return fail("fp8 weights need an even number of experts (router rows come in pairs)");
        if (c.head_dim != 128) return fail("fp8 weights are supported for head_dim 128 only");
        if (c.d_model % 512 || c.ffn_dim % 512 || (c.n_heads * c.head_dim) % 512)
            return fail("fp8 weights need d_model, ffn_dim and n_heads*head_dim multiples of 512");
        if (c.vocab % 2) return fail("fp8 weights need an even vocab (LM rows come in pairs)");
    }
    Dims D = dims_of(c);
    // LDS budget: input vector, per-phase partial sums, owned residual rows
    int max_in = c.d_model;
    if (c.n_heads * c.head_dim > max_in) max_in = c.n_heads * c.head_dim;
    int kdown = c.n_experts ? c.top_k * c.ffn_dim : c.ffn_dim;
    if (kdown > max_in) max_in = kdown;
    if (max_in > kMaxInput) return fail("largest GEMV input must be at most 8192 elements");
    for (int ph = 0; ph < PH_COUNT; ++ph) {
        if (c.n_experts == 0 && (ph == PH_ROUTER || ph == PH_EGU || ph == PH_EDOWN)) continue;
        if (c.n_experts != 0 && (ph == PH_GU || ph == PH_DOWN)) continue;
        PhaseShape s = phase_shape(D, ph);
        if (s.M % s.gran) return fail("phase rows not a multiple of their split granularity");
        RowSplit r = split_rows(s.M, s.gran, kGrid, 0);   // workgroup 0 has the largest share
        if (r.nrows > kMaxRowsWg) return fail("a workgroup's share of a phase exceeds 256 rows");
        if ((ph == PH_WO || ph == PH_DOWN || ph == PH_EDOWN) && r.nrows > kMaxOwnRows)
            return fail("a workgroup's share of the residual exceeds 32 rows");
    }
    if (err) err->clear();
    return KIE_OK;
}

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

void make_layout(const kie_config& c, Layout* lay) {
    Dims D = dims_of(c);
    Layout& Y = *lay;
    std::memset(&Y, 0, sizeof(Y));
    Y.D = D;
    int acc = 0;
    for (int w = 0; w < kGrid; ++w) {
        Y.piece_off[w] = acc;
        acc += piece_units(D, kGrid, w);
    }
    Y.piece_off[kGrid] = acc;
    Y.layer_bytes = (size_t)acc * kUnitBytes;
    acc = 0;
    for (int w = 0; w < kGrid; ++w) {
        Y.lm_off[w] = acc;
        acc += phase_units(D, PH_LM, kGrid, w);
    }
    Y.lm_off[kGrid] = acc;
    Y.lm_bytes = (size_t)acc * kUnitBytes;
    Y.attn_items_per_head = kGrid / D.Hkv;

    const size_t A = 4096;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align_up(off + bytes, A);
        return o;
    };
    Y.off_layers = take(Y.layer_bytes * D.L);
    Y.off_lm = take(Y.lm_bytes);
    Y.off_emb = take((size_t)D.V * D.d * 2);
    // fp16: 2 bytes per weight, fp8: 1, fp4: 1/2
    Y.expert_bytes = D.E ? (size_t)(2 * D.F * D.d + D.d * D.F) * (D.w4 ? 1 : D.w8 ? 2 : 4) / 2 : 0;
    Y.off_experts = take(Y.expert_bytes * D.E * D.L);
    Y.off_rope = take((size_t)D.max_seq * (D.hd / 2) * 8);
    Y.kv_bytes = (size_t)D.L * D.Hkv * D.max_seq * D.hd * 2;
    Y.off_k = take(Y.kv_bytes);
    Y.off_v = take(Y.kv_bytes);
    Y.off_ex_x = take((size_t)D.d * 8);
    Y.off_ex_qkv = take((size_t)(D.H + D.Hkv) * D.hd * 8);
    // one copy per XCD (XCD-local attention), each on its own 4 KiB
    Y.ex_part_copy = align_up((size_t)D.H * Y.attn_items_per_head * (D.hd + 2), A / 8);
    Y.ex_o_copy = align_up((size_t)D.H * D.hd, A / 8);
    Y.off_ex_part = take(Y.ex_part_copy * 8 * kXcds);
    Y.off_ex_o = take(Y.ex_o_copy * 8 * kXcds);
    size_t hlen = D.E ? (size_t)D.topk * D.F : (size_t)D.F;
    Y.off_ex_h = take(hlen * 8);
    Y.off_ex_r = take((size_t)(D.E ? D.E : 1) * 8);
    Y.off_ex_am = take((size_t)kGrid * 2 * 8);
    Y.ex_bytes = off - Y.off_ex_x;
    Y.off_status = take(64 * 4);
    Y.off_out = take((size_t)D.max_seq * 4);
    Y.off_force = take((size_t)D.max_seq * 4);
    Y.off_dbg_logits = take((size_t)kDebugRows * D.V * 4);
    Y.off_dbg_experts = take((size_t)kDebugRows * D.L * (D.topk ? D.topk : 1) * 4);
    Y.off_dbg_router = take((size_t)kDebugRows * D.L * (D.E ? D.E : 1) * 4);
    Y.off_plan = take((size_t)2 * (kGrid + 1) * 4);
    Y.off_args = take(4096);
    Y.off_idle = take(16384);
    Y.off_trace = take((size_t)kTracePhases * kGrid * 4 * 8);
    if (batched_prefill_ok(D)) {
        const size_t R = kPrefillRows;
        size_t kmax = D.d, ymax = (size_t)(D.H + 2 * D.Hkv) * D.hd;
        if ((size_t)D.H * D.hd > kmax) kmax = (size_t)D.H * D.hd;
        if ((size_t)D.F > kmax) kmax = D.F;
        if ((size_t)2 * D.F > ymax) ymax = (size_t)2 * D.F;
        if ((size_t)D.V > ymax) ymax = D.V;
        if ((size_t)D.d > ymax) ymax = D.d;
        Y.off_pf_x = take(R * D.d * 4);
        Y.off_pf_a = take(R * kmax * 4);
        Y.off_pf_y = take(R * ymax * 4);
        Y.off_pf_q = take(R * D.H * D.hd * 4);
        Y.off_pf_tok = take((R + 4) * 4);
        Y.off_pf_slab = take((size_t)5 * kGrid * 4);
    }
    Y.layer_scales = 0;
    if (D.w8) {
        for (int i = 0; i < layer_block_phase_count(D); ++i) Y.layer_scales += phase_shape(D, layer_block_phase(D, i)).M;
        Y.off_scales = take(((size_t)D.L * Y.layer_scales + D.V) * 4);
        if (D.E) Y.off_escales = take((size_t)D.L * D.E * (2 * D.F + D.d) * 4);
    }
    Y.total = off;
}

uint16_t f32_to_f16(float f) {
    uint32_t x;
    std::memcpy(&x, &f, 4);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t exp = (x >> 23) & 0xffu;
    uint32_t man = x & 0x7fffffu;
    if (exp == 0xff) return (uint16_t)(sign | 0x7c00u | (man ? 0x200u : 0u));   // inf / nan
    int e = (int)exp - 127 + 15;
    if (e >= 31) return (uint16_t)(sign | 0x7c00u);                           // overflow -> inf
    if (e <= 0) {                                                              // subnormal or zero
        if (e < -10) return (uint16_t)sign;
        man |= 0x800000u;
        int shift = 14 - e;
        uint32_t h = man >> shift;
        uint32_t rem = man & ((1u << shift) - 1u);
        uint32_t half = 1u << (shift - 1);
        if (rem > half || (rem == half && (h & 1u))) h++;
        return (uint16_t)(sign | h);
    }
    uint32_t h = ((uint32_t)e << 10) | (man >> 13);
    uint32_t rem = man & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h++;   // may carry into the exponent: correct
    return (uint16_t)(sign | h);
}

float f16_to_f32(uint16_t h) {
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t exp = (h >> 10) & 0x1fu;
    uint32_t man = h & 0x3ffu;
    uint32_t x;
    if (exp == 0) {
        if (man == 0) {
            x = sign;
        } else {
            int e = -1;
            do { man <<= 1; ++e; } while (!(man & 0x400u));
            x = sign | ((uint32_t)(127 - 15 - e) << 23) | ((man & 0x3ffu) << 13);
        }
    } else if (exp == 31) {
        x = sign | 0x7f800000u | (man << 13);
    } else {
        x = sign | ((exp - 15 + 127) << 23) | (man << 13);
    }
    float f;
    std::memcpy(&f, &x, 4);
    return f;
}

// Copy one row of K fp16 values, multiplying column k by gain[k] in fp32 and
// rounding back to fp16 (exact copy when every gain is 1).
static void put_row(uint16_t* dst, const uint16_t* src, int K, const uint16_t* gain, bool unit_gain) {
    if (!gain || unit_gain) {
        std::memcpy(dst, src, (size_t)K * 2);
        return;
    }
    for (int k = 0; k < K; ++k) dst[k] = f32_to_f16(f16_to_f32(src[k]) * f16_to_f32(gain[k]));
}

static bool all_one(const uint16_t* g, int n) {
    for (int i = 0; i < n; ++i)
        if (g[i] != 0x3c00u) return false;
    return true;
}

void repack_layer(const kie_config& c, const Layout& lay, const uint16_t* const* t, int l,
                  uint16_t* dst) {
    const Dims& D = lay.D;
    const uint16_t* g_attn = t[tidx_layer(c, l, 0)];
    const uint16_t* g_ffn = t[tidx_layer(c, l, 5)];
    bool ga1 = all_one(g_attn, D.d), gf1 = all_one(g_ffn, D.d);
    const uint16_t* Wq = t[tidx_layer(c, l, 1)];
    const uint16_t* Wk = t[tidx_layer(c, l, 2)];
    const uint16_t* Wv = t[tidx_layer(c, l, 3)];
    const uint16_t* Wo = t[tidx_layer(c, l, 4)];
    std::memset(dst, 0, lay.layer_bytes);
    for (int w = 0; w < kGrid; ++w) {
        uint16_t* p = dst + (size_t)lay.piece_off[w] * kUnitHalves;
        for (int i = 0; i < layer_block_phase_count(D); ++i) {
            int ph = layer_block_phase(D, i);
            PhaseShape s = phase_shape(D, ph);
            RowSplit r = split_rows(s.M, s.gran, kGrid, w);
            for (int j = 0; j < r.nrows; ++j) {
                int row = r.row0 + j;
                uint16_t* out = p + (size_t)j * s.K;
                switch (ph) {
                case PH_QKV: {
                    int mat, src;
                    qkv_row_source(D, row, &mat, &src);
                    const uint16_t* W = mat == 0 ? Wq : (mat == 1 ? Wk : Wv);
                    put_row(out, W + (size_t)src * D.d, D.d, g_attn, ga1);
                    break;
                }
                case PH_WO:
                    put_row(out, Wo + (size_t)row * s.K, s.K, nullptr, true);
                    break;
                case PH_GU: {
                    const uint16_t* W = t[tidx_layer(c, l, (row & 1) ? 7 : 6)];
                    put_row(out, W + (size_t)(row >> 1) * D.d, D.d, g_ffn, gf1);
                    break;
                }
                case PH_DOWN:
                    put_row(out, t[tidx_layer(c, l, 8)] + (size_t)row * s.K, s.K, nullptr, true);
                    break;
                case PH_ROUTER:
                    put_row(out, t[tidx_layer(c, l, 6)] + (size_t)row * D.d, D.d, g_ffn, gf1);
                    break;
                }
            }
            p += (size_t)slab_units(r.nrows, s.K) * kUnitHalves;
        }
    }
}

void repack_lm(const kie_config& c, const Layout& lay, const uint16_t* const* t, uint16_t* dst) {
    const Dims& D = lay.D;
    const uint16_t* g = t[tidx_gfinal(c)];
    bool g1 = all_one(g, D.d);
    const uint16_t* W = t[tidx_lm(c)];
    std::memset(dst, 0, lay.lm_bytes);
    for (int w = 0; w < kGrid; ++w) {
        RowSplit r = split_rows(D.V, 1, kGrid, w);
        uint16_t* p = dst + (size_t)lay.lm_off[w] * kUnitHalves;
        for (int j = 0; j < r.nrows; ++j)
            put_row(p + (size_t)j * D.d, W + (size_t)(r.row0 + j) * D.d, D.d, g, g1);
    }
}

void repack_expert(const kie_config& c, const Layout& lay, const uint16_t* const* t, int l, int e,
                   uint16_t* dst) {
    const Dims& D = lay.D;
    const uint16_t* g = t[tidx_layer(c, l, 5)];
    bool g1 = all_one(g, D.d);
    const uint16_t* Wg = t[tidx_expert(c, l, e, 0)];
    const uint16_t* Wu = t[tidx_expert(c, l, e, 1)];
    const uint16_t* Wd = t[tidx_expert(c, l, e, 2)];
    for (int r = 0; r < 2 * D.F; ++r)
        put_row(dst + (size_t)r * D.d, ((r & 1) ? Wu : Wg) + (size_t)(r >> 1) * D.d, D.d, g, g1);
    std::memcpy(dst + (size_t)2 * D.F * D.d, Wd, (size_t)D.d * D.F * 2);
}

// ---------------------------------------------------------------- fp8 ------
// E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is
// subnormal (m/8 * 2^-6), exponent 15 with mantissa 7 is NaN, so the largest
// finite value is 1.75 * 2^8 = 448.
float e4m3_decode(uint8_t q) {
    const int e = (q >> 3) & 15, m = q & 7;
    const float s = (q & 0x80) ? -1.f : 1.f;
    if (e == 15 && m == 7) return std::nanf("");
    if (e == 0) return s * std::ldexp((float)m, -9);
    return s * std::ldexp(8.f + m, e - 10);
}

uint8_t e4m3_encode(float v) {
    if (std::isnan(v)) return 0x7f;
    uint8_t sign = std::signbit(v) ? 0x80 : 0;
    float a = std::fabs(v);
    if (a >= 448.f) return sign | 0x7e;                       // saturate (no infinity)
    if (a == 0.f) return sign;                                 // (+-)0: frexp gives no binade
    // spacing of E4M3 values around a: 2^-9 below 2^-6, else 2^(E-3) for a in [2^E, 2^(E+1))
    int E;
    std::frexp(a, &E);                                         // a = f * 2^E, f in [0.5, 1)
    --E;
    if (E < -6) E = -6;
    const float step = std::ldexp(1.f, E - 3);
    const float n = std::nearbyint(a / step);                  // exact division by a power of two; ties to even
    // n counts steps: 0..8 below 2^-6 (8 = 2^-6, the smallest normal), else 8..16
    int e = E + 7, m;
    if (E == -6 && n < 8.f) {
        e = 0;
        m = (int)n;
    } else if (n >= 16.f) {                                     // rounded up to the next binade
        ++e;
        m = 0;
    } else {
        m = (int)n - 8;
    }
    if (e > 15 || (e == 15 && m == 7)) return sign | 0x7e;    // beyond 448 rounds down to it
    return sign | (uint8_t)(e << 3) | (uint8_t)m;
}

void quantize_row_e4m3(const uint16_t* w, const uint16_t* gain, int K, uint8_t* q, float* scale) {
    float amax = 0.f;
    for (int k = 0; k < K; ++k) {
        const float v = f16_to_f32(w[k]) * (gain ? f16_to_f32(gain[k]) : 1.f);
        amax = std::fmax(amax, std::fabs(v));
    }
    const float s = amax > 0.f ? amax / 448.f : 1.f;
    for (int k = 0; k < K; ++k) {
        const float v = f16_to_f32(w[k]) * (gain ? f16_to_f32(gain[k]) : 1.f);
        q[k] = e4m3_encode(v / s);
    }
    *scale = s;
}

// ---------------------------------------------------------------- fp4 ------
// E2M1: sign bit 3, 2 exponent bits e (bias 1), 1 mantissa bit m; e = 0 is
// subnormal (m/2), otherwise (1 + m/2) * 2^(e-1): magnitudes 0, 0.5, 1, 1.5,
// 2, 3, 4, 6, no infinity or NaN.
float e2m1_decode(uint8_t q) {
    const int e = (q >> 1) & 3, m = q & 1;
    const float mag = e == 0 ? 0.5f * m : std::ldexp(1.f + 0.5f * m, e - 1);
    return (q & 8) ? -mag : mag;
}

uint8_t e2m1_encode(float v) {
    const uint8_t sign = std::signbit(v) ? 8 : 0;
    const float a = std::isnan(v) ? 0.f : std::fabs(v);
    if (a >= 6.f) return sign | 7;                               // saturate
    // spacing 0.5 below 2, 1 in [2, 4), 2 in [4, 6); codes step with the
    // values, so rounding the count of steps to even rounds the code to even
    if (a < 2.f) return sign | (uint8_t)std::nearbyint(a * 2.f);          // codes 0..4
    if (a < 4.f) return sign | (uint8_t)(std::nearbyint(a) + 2.f);        // codes 4..6
    return sign | (uint8_t)(std::nearbyint(a * 0.5f) + 4.f);              // codes 6..7
}

void quantize_row_e2m1(const uint16_t* w, const uint16_t* gain, int K, uint8_t* q, float* scale) {
    float amax = 0.f;
    for (int k = 0; k < K; ++k) {
        const float v = f16_to_f32(w[k]) * (gain ? f16_to_f32(gain[k]) : 1.f);
        amax = std::fmax(amax, std::fabs(v));
    }
    const float s = amax > 0.f ? amax / 6.f : 1.f;
    for (int k = 0; k < K; ++k) {
        const float v = f16_to_f32(w[k]) * (gain ? f16_to_f32(gain[k]) : 1.f);
        q[k] = e2m1_encode(v / s);
    }
    *scale = s;
}

// Four quantized rows q[0..3] of K columns as K/512 units: unit s, lane l
// holds 4 bytes per row r (rows in order), byte b of row r holding the codes
// of columns 512 s + 8 l + 2 b (low nibble) and + 1 (high nibble).
static void put_quad_fp4(uint8_t* dst, const uint8_t* const* q, int K) {
    for (int s = 0; s < K / 512; ++s)
        for (int l = 0; l < 64; ++l)
            for (int r = 0; r < 4; ++r)
                for (int b = 0; b < 4; ++b) {
                    const int c = s * 512 + 8 * l + 2 * b;
                    dst[((size_t)s * 64 + l) * 16 + 4 * r + b] = (uint8_t)(q[r][c] | (q[r][c + 1] << 4));
                }
}

// One pair of quantized rows (qa, qb) of K columns as K/512 units: unit s,
// lane l holds qa[512 s + 8 l .. + 8] then qb[512 s + 8 l .. + 8].
static void put_pair_fp8(uint8_t* dst, const uint8_t* qa, const uint8_t* qb, int K) {
    for (int s = 0; s < K / 512; ++s)
        for (int l = 0; l < 64; ++l) {
            std::memcpy(dst + ((size_t)s * 64 + l) * 16, qa + s * 512 + 8 * l, 8);
            std::memcpy(dst + ((size_t)s * 64 + l) * 16 + 8, qb + s * 512 + 8 * l, 8);
        }
}

void repack_layer_fp8(const kie_config& c, const Layout& lay, const uint16_t* const* t, int l, uint8_t* dst,
                      float* scales) {
    const Dims& D = lay.D;
    const uint16_t* g_attn = t[tidx_layer(c, l, 0)];
    const uint16_t* g_ffn = t[tidx_layer(c, l, 5)];
    std::memset(dst, 0, lay.layer_bytes);
    std::vector<uint8_t> qa(kMaxInput), qb(kMaxInput);
    std::vector<uint8_t> q4[4] = {std::vector<uint8_t>(kMaxInput), std::vector<uint8_t>(kMaxInput),
                                  std::vector<uint8_t>(kMaxInput), std::vector<uint8_t>(kMaxInput)};
    // source row (pointer, gain) of a phase row
    auto source = [&](int ph, int row, const uint16_t** src, const uint16_t** g) {
        *g = nullptr;
        switch (ph) {
        case PH_QKV: {
            int mat, r;
            qkv_row_source(D, row, &mat, &r);
            *src = t[tidx_layer(c, l, 1 + mat)] + (size_t)r * D.d;
            *g = g_attn;
            break;
        }
        case PH_WO: *src = t[tidx_layer(c, l, 4)] + (size_t)row * D.H * D.hd; break;
        case PH_GU:
            *src = t[tidx_layer(c, l, (row & 1) ? 7 : 6)] + (size_t)(row >> 1) * D.d;
            *g = g_ffn;
            break;
        case PH_ROUTER:
            *src = t[tidx_layer(c, l, 6)] + (size_t)row * D.d;
            *g = g_ffn;
            break;
        default: *src = t[tidx_layer(c, l, 8)] + (size_t)row * D.F; break;   // PH_DOWN
        }
    };
    size_t sbase = 0;   // this phase's first scale in the layer's scale block
    for (int i = 0; i < layer_block_phase_count(D); ++i) {
        const int ph = layer_block_phase(D, i);
        const PhaseShape s = phase_shape(D, ph);
        for (int w = 0; w < kGrid; ++w) {
            size_t off = (size_t)lay.piece_off[w] * kUnitBytes;
            for (int j = 0; j < i; ++j)
                off += (size_t)phase_units(D, layer_block_phase(D, j), kGrid, w) * kUnitBytes;
            const RowSplit r = split_rows(s.M, s.gran, kGrid, w);
            if (D.w4) {
                // fp4: rows in fours, one unit column per 512 columns of the four
                for (int j = 0; j < r.nrows; j += 4) {
                    const uint8_t* qr[4] = {q4[0].data(), q4[1].data(), q4[2].data(), q4[3].data()};
                    for (int i2 = 0; i2 < 4; ++i2) {
                        const uint16_t *sr, *gr;
                        source(ph, r.row0 + j + i2, &sr, &gr);
                        quantize_row_e2m1(sr, gr, s.K, q4[i2].data(), &scales[sbase + r.row0 + j + i2]);
                    }
                    put_quad_fp4(dst + off + (size_t)(j / 4) * s.K * 2, qr, s.K);
                }
                continue;
            }
            for (int j = 0; j < r.nrows; j += 2) {
                const uint16_t *sa, *sb, *ga, *gb;
                source(ph, r.row0 + j, &sa, &ga);
                source(ph, r.row0 + j + 1, &sb, &gb);
                quantize_row_e4m3(sa, ga, s.K, qa.data(), &scales[sbase + r.row0 + j]);
                quantize_row_e4m3(sb, gb, s.K, qb.data(), &scales[sbase + r.row0 + j + 1]);
                put_pair_fp8(dst + off + (size_t)(j / 2) * s.K * 2, qa.data(), qb.data(), s.K);
            }
        }
        sbase += s.M;
    }
}

void repack_expert_quant(const kie_config& c, const Layout& lay, const uint16_t* const* t, int l, int e, uint8_t* dst,
                       float* scales) {
    const Dims& D = lay.D;
    const uint16_t* g = t[tidx_layer(c, l, 5)];
    const uint16_t* Wg = t[tidx_expert(c, l, e, 0)];
    const uint16_t* Wu = t[tidx_expert(c, l, e, 1)];
    const uint16_t* Wd = t[tidx_expert(c, l, e, 2)];
    std::vector<uint8_t> qa(kMaxInput), qb(kMaxInput);
    if (D.w4) {
        // fp4: rows in fours. Gate/up four p = rows (g_2p, u_2p, g_2p+1, u_2p+1)
        // at 2 d bytes per four; down rows r .. r+3 at 2 F bytes per four.
        std::vector<uint8_t> q4[4] = {std::vector<uint8_t>(kMaxInput), std::vector<uint8_t>(kMaxInput),
                                      std::vector<uint8_t>(kMaxInput), std::vector<uint8_t>(kMaxInput)};
        const uint8_t* qr[4] = {q4[0].data(), q4[1].data(), q4[2].data(), q4[3].data()};
        for (int p = 0; p < D.F; p += 2) {
            for (int i = 0; i < 4; ++i) {
                const uint16_t* W = (i & 1) ? Wu : Wg;
                quantize_row_e2m1(W + (size_t)(p + i / 2) * D.d, g, D.d, q4[i].data(), &scales[2 * p + i]);
            }
            put_quad_fp4(dst + (size_t)(p / 2) * D.d * 2, qr, D.d);
        }
        uint8_t* down = dst + (size_t)D.F * D.d;
        for (int r = 0; r < D.d; r += 4) {
            for (int i = 0; i < 4; ++i)
                quantize_row_e2m1(Wd + (size_t)(r + i) * D.F, nullptr, D.F, q4[i].data(), &scales[2 * D.F + r + i]);
            put_quad_fp4(down + (size_t)(r / 4) * D.F * 2, qr, D.F);
        }
        return;
    }
    // gate/up rows interleaved (g_p, u_p): pair p is units p * d / 512 ..
    for (int p = 0; p < D.F; ++p) {
        quantize_row_e4m3(Wg + (size_t)p * D.d, g, D.d, qa.data(), &scales[2 * p]);
        quantize_row_e4m3(Wu + (size_t)p * D.d, g, D.d, qb.data(), &scales[2 * p + 1]);
        put_pair_fp8(dst + (size_t)p * D.d * 2, qa.data(), qb.data(), D.d);
    }
    uint8_t* down = dst + (size_t)2 * D.F * D.d;
    for (int r = 0; r < D.d; r += 2) {
        quantize_row_e4m3(Wd + (size_t)r * D.F, nullptr, D.F, qa.data(), &scales[2 * D.F + r]);
        quantize_row_e4m3(Wd + (size_t)(r + 1) * D.F, nullptr, D.F, qb.data(), &scales[2 * D.F + r + 1]);
        put_pair_fp8(down + (size_t)(r / 2) * D.F * 2, qa.data(), qb.data(), D.F);
    }
}

void repack_lm_fp8(const kie_config& c, const Layout& lay, const uint16_t* const* t, uint8_t* dst, float* scales) {
    const Dims& D = lay.D;
    const uint16_t* g = t[tidx_gfinal(c)];
    const uint16_t* W = t[tidx_lm(c)];
    std::memset(dst, 0, lay.lm_bytes);
    std::vector<uint8_t> qa(D.d), qb(D.d);
    for (int w = 0; w < kGrid; ++w) {
        const RowSplit r = split_rows(D.V, D.w4 ? 4 : 2, kGrid, w);
        uint8_t* p = dst + (size_t)lay.lm_off[w] * kUnitBytes;
        if (D.w4) {
            std::vector<uint8_t> q4[4] = {std::vector<uint8_t>(D.d), std::vector<uint8_t>(D.d),
                                          std::vector<uint8_t>(D.d), std::vector<uint8_t>(D.d)};
            const uint8_t* qr[4] = {q4[0].data(), q4[1].data(), q4[2].data(), q4[3].data()};
            for (int j = 0; j < r.nrows; j += 4) {
                for (int i2 = 0; i2 < 4; ++i2)
                    quantize_row_e2m1(W + (size_t)(r.row0 + j + i2) * D.d, g, D.d, q4[i2].data(),
                                      &scales[r.row0 + j + i2]);
                put_quad_fp4(p + (size_t)(j / 4) * D.d * 2, qr, D.d);
            }
            continue;
        }
        for (int j = 0; j < r.nrows; j += 2) {
            const int row = r.row0 + j;
            quantize_row_e4m3(W + (size_t)row * D.d, g, D.d, qa.data(), &scales[row]);
            quantize_row_e4m3(W + (size_t)(row + 1) * D.d, g, D.d, qb.data(), &scales[row + 1]);
            put_pair_fp8(p + (size_t)(j / 2) * D.d * 2, qa.data(), qb.data(), D.d);
        }
    }
}

void rope_table(const kie_config& c, float* dst) {
    int half = c.head_dim / 2;
    for (int p = 0; p < c.max_seq; ++p) {
        for (int i = 0; i < half; ++i) {
            double inv = std::pow((double)c.rope_theta, -2.0 * i / c.head_dim);
            double a = (double)p * inv;
            dst[((size_t)p * half + i) * 2 + 0] = (float)std::cos(a);
            dst[((size_t)p * half + i) * 2 + 1] = (float)std::sin(a);
        }
    }
}

}  // namespace kie

// repack_check.cpp - host check of the offline weight repack (kie_host.cpp),
// built with g++ and AddressSanitizer by tests/test_host_repack.py; no HIP.
//
// For a dense and a top-k MoE configuration, with random fp16 weights and
// non-unit RMSNorm gains, it unpacks every streaming block the repacker wrote
// and checks, element by element (quantised MoE experts: check_expert_quant):
//  * every weight row lands exactly once, at the place this file works out on
//    its own from the layout rules (rows split over 256 workgroups, each
//    workgroup's rows of a layer contiguous in phase order; QKV rows with each
//    rotary pair (i, i + hd/2) of a q or k head adjacent; gate/up rows
//    interleaved g_0, u_0, g_1, u_1, ...);
//  * the gain fold W' = W diag(g): each element equals fp16(w * g) computed
//    here in double precision and rounded to nearest even (exact copy when
//    every gain is 1);
//  * unused padding is zero and no byte outside the blocks is written;
//  * the rotary table holds (cos, sin) of p * theta^(-2i/hd) rounded to fp32;
//  * fp16 <-> fp32 conversion: every fp16 value round-trips, and fp32 -> fp16
//    rounds to nearest even (checked against a double-precision reference).
// Prints "OK" and exits 0, or prints the first mismatch and exits 1.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "kie_host.h"

using namespace kie;

static int g_fail = 0;
#define CHECK(c, ...)                                   \
    do {                                                \
        if (!(c)) {                                     \
            if (g_fail++ < 10) {                        \
                std::printf("FAIL %s:%d: ", __FILE__, __LINE__); \
                std::printf(__VA_ARGS__);               \
                std::printf("\n");                      \
            }                                           \
        }                                               \
    } while (0)

static uint64_t g_rng = 88172645463325252ull;
static uint32_t rnd() {   // xorshift64
    g_rng ^= g_rng << 13;
    g_rng ^= g_rng >> 7;
    g_rng ^= g_rng << 17;
    return (uint32_t)(g_rng >> 11);
}
static double urand() { return (rnd() & 0xffffff) / 16777216.0; }

// fp32 -> fp16 by round to nearest even, from double arithmetic.
static uint16_t ref_half(double v) {
    if (std::isnan(v)) return 0x7e00;
    uint16_t sign = std::signbit(v) ? 0x8000 : 0;
    double a = std::fabs(v);
    if (a >= 65520.0) return sign | 0x7c00;   // rounds to infinity
    int e;
    std::frexp(a, &e);                        // a = f * 2^e, f in [0.5, 1)
    int ex = e - 1;                           // a in [2^ex, 2^(ex+1))
    if (ex < -14) ex = -14;                   // subnormal spacing 2^-24
    double q = std::ldexp(1.0, ex - 10);      // spacing of fp16 values there
    double m = a / q;
    double r = std::nearbyint(m);             // current rounding mode: to nearest even
    double h = r * q;
    // encode h
    if (h == 0) return sign;
    int eh;
    std::frexp(h, &eh);
    int exh = eh - 1;
    if (exh < -14) return sign | (uint16_t)(h / std::ldexp(1.0, -24));
    uint16_t mant = (uint16_t)(h / std::ldexp(1.0, exh - 10) - 1024.0);
    return sign | (uint16_t)((exh + 15) << 10) | mant;
}
static double half_val(uint16_t h) {
    int e = (h >> 10) & 31, m = h & 1023;
    double s = (h & 0x8000) ? -1.0 : 1.0;
    if (e == 0) return s * m * std::ldexp(1.0, -24);
    if (e == 31) return m ? NAN : s * INFINITY;
    return s * (1024 + m) * std::ldexp(1.0, e - 25);
}

static std::vector<uint16_t> random_tensor(size_t n, double sigma) {
    std::vector<uint16_t> t(n);
    for (auto& x : t) {
        // roughly normal: sum of 4 uniforms, centred
        double v = (urand() + urand() + urand() + urand() - 2.0) * sigma * 1.7;
        x = ref_half(v);
    }
    return t;
}

struct Model {
    kie_config c;
    std::vector<std::vector<uint16_t>> t;
    std::vector<const uint16_t*> p;
};

static Model make_model(const kie_config& c, bool unit_gains) {
    Model M;
    M.c = c;
    const int d = c.d_model, q = c.n_heads * c.head_dim, kv = c.n_kv_heads * c.head_dim, f = c.ffn_dim;
    auto gain = [&]() {
        std::vector<uint16_t> g(d);
        for (auto& x : g) x = unit_gains ? 0x3c00 : ref_half(1.0 + (urand() - 0.5) * 0.8);
        return g;
    };
    M.t.push_back(random_tensor((size_t)c.vocab * d, 0.02));
    for (int l = 0; l < c.n_layers; ++l) {
        M.t.push_back(gain());
        M.t.push_back(random_tensor((size_t)q * d, 0.02));
        M.t.push_back(random_tensor((size_t)kv * d, 0.02));
        M.t.push_back(random_tensor((size_t)kv * d, 0.02));
        M.t.push_back(random_tensor((size_t)d * q, 0.02));
        M.t.push_back(gain());
        if (c.n_experts) {
            M.t.push_back(random_tensor((size_t)c.n_experts * d, 0.1));
            for (int e = 0; e < c.n_experts; ++e) {
                M.t.push_back(random_tensor((size_t)f * d, 0.02));
                M.t.push_back(random_tensor((size_t)f * d, 0.02));
                M.t.push_back(random_tensor((size_t)d * f, 0.02));
            }
        } else {
            M.t.push_back(random_tensor((size_t)f * d, 0.02));
            M.t.push_back(random_tensor((size_t)f * d, 0.02));
            M.t.push_back(random_tensor((size_t)d * f, 0.02));
        }
    }
    M.t.push_back(gain());
    M.t.push_back(random_tensor((size_t)c.vocab * d, 0.02));
    for (auto& v : M.t) M.p.push_back(v.data());
    return M;
}

// Expected fp16 of w * g (g absent: w itself).
static uint16_t folded(uint16_t w, const uint16_t* g, int k) {
    if (!g) return w;
    return ref_half(half_val(w) * half_val(g[k]));
}

// Rows [r0, r0 + n) of an even split of M rows in groups of gran over 256
// workgroups, for workgroup w: this file's own statement of the split.
static void my_split(int M, int gran, int w, int* r0, int* n) {
    int groups = M / gran, base = groups / 256, extra = groups % 256;
    int before = w * base + (w < extra ? w : extra);
    *r0 = before * gran;
    *n = (base + (w < extra ? 1 : 0)) * gran;
}

// Source of virtual QKV row r: matrix (0 q, 1 k, 2 v) and row.
static void my_qkv_source(int H, int Hkv, int hd, int r, int* mat, int* row) {
    int qd = H * hd, kd = Hkv * hd;
    if (r >= qd + kd) { *mat = 2; *row = r - qd - kd; return; }
    *mat = r >= qd ? 1 : 0;
    int rr = r >= qd ? r - qd : r;
    int head = rr / hd, w = rr % hd;
    // adjacent rows 2i, 2i+1 hold elements i and i + hd/2
    *row = head * hd + (w % 2 == 0 ? w / 2 : w / 2 + hd / 2);
}

static int check_model(const kie_config& c, bool unit_gains) {
    Model M = make_model(c, unit_gains);
    std::string err;
    CHECK(validate_config(c, &err) == KIE_OK, "config rejected: %s", err.c_str());
    CHECK((int)M.t.size() == tensor_count(c), "tensor count %d vs %d", (int)M.t.size(), tensor_count(c));
    Layout* L = new Layout;
    make_layout(c, L);
    const int d = c.d_model, H = c.n_heads, Hkv = c.n_kv_heads, hd = c.head_dim, F = c.ffn_dim;
    const int per_layer = 6 + (c.n_experts ? 1 + 3 * c.n_experts : 3);
    auto T = [&](int l, int which) { return M.t[1 + l * per_layer + which].data(); };
    // phase order of a layer block and each phase's (rows, row length, granularity)
    struct Ph { int M, K, gran, kind; };
    std::vector<Ph> phases;
    phases.push_back({(H + 2 * Hkv) * hd, d, 4, 0});
    phases.push_back({d, H * hd, 2, 1});
    if (c.n_experts) phases.push_back({c.n_experts, d, 1, 4});
    else {
        phases.push_back({2 * F, d, 4, 2});
        phases.push_back({d, F, 2, 3});
    }
    // one guard unit past the block: must stay untouched
    const size_t guard = 512;
    std::vector<uint16_t> blk(L->layer_bytes / 2 + guard, 0xA5A5);
    for (int l = 0; l < c.n_layers; ++l) {
        std::fill(blk.begin(), blk.end(), 0xA5A5);
        repack_layer(c, *L, M.p.data(), l, blk.data());
        std::vector<int> seen_rows;
        size_t pos = 0;   // halves, walking the pieces in workgroup order
        for (int w = 0; w < 256; ++w) {
            CHECK(pos == (size_t)L->piece_off[w] * 512, "piece %d starts at %zu, layout says %zu", w, pos,
                  (size_t)L->piece_off[w] * 512);
            for (const Ph& ph : phases) {
                int r0, n;
                my_split(ph.M, ph.gran, w, &r0, &n);
                for (int j = 0; j < n; ++j) {
                    int r = r0 + j;
                    const uint16_t* src;
                    const uint16_t* g = nullptr;
                    if (ph.kind == 0) {
                        int mat, row;
                        my_qkv_source(H, Hkv, hd, r, &mat, &row);
                        src = T(l, 1 + mat) + (size_t)row * d;
                        g = T(l, 0);
                    } else if (ph.kind == 1) {
                        src = T(l, 4) + (size_t)r * ph.K;
                    } else if (ph.kind == 2) {
                        src = T(l, (r % 2) ? 7 : 6) + (size_t)(r / 2) * d;
                        g = T(l, 5);
                    } else if (ph.kind == 3) {
                        src = T(l, 8) + (size_t)r * ph.K;
                    } else {
                        src = T(l, 6) + (size_t)r * d;
                        g = T(l, 5);
                    }
                    for (int k = 0; k < ph.K; ++k) {
                        uint16_t want = folded(src[k], unit_gains ? nullptr : g, k);
                        uint16_t got = blk[pos + (size_t)j * ph.K + k];
                        CHECK(got == want, "layer %d wg %d phase %d row %d col %d: %04x vs %04x", l, w, ph.kind, r,
                              k, got, want);
                    }
                }
                size_t used = (size_t)n * ph.K, padded = (used + 511) / 512 * 512;
                for (size_t k = used; k < padded; ++k) CHECK(blk[pos + k] == 0, "padding not zero");
                pos += padded;
            }
        }
        CHECK(pos * 2 == L->layer_bytes, "layer block is %zu bytes, layout says %zu", pos * 2, L->layer_bytes);
        for (size_t k = 0; k < guard; ++k) CHECK(blk[L->layer_bytes / 2 + k] == 0xA5A5, "write past the block");
        if (c.n_experts) {
            std::vector<uint16_t> ex(L->expert_bytes / 2 + guard, 0xA5A5);
            for (int e = 0; e < c.n_experts; ++e) {
                std::fill(ex.begin(), ex.end(), 0xA5A5);
                repack_expert(c, *L, M.p.data(), l, e, ex.data());
                const uint16_t* Wg = T(l, 7 + 3 * e);
                const uint16_t* Wu = T(l, 8 + 3 * e);
                const uint16_t* Wd = T(l, 9 + 3 * e);
                for (int r = 0; r < 2 * F; ++r)
                    for (int k = 0; k < d; ++k) {
                        const uint16_t* s = (r % 2 ? Wu : Wg) + (size_t)(r / 2) * d;
                        uint16_t want = folded(s[k], unit_gains ? nullptr : T(l, 5), k);
                        CHECK(ex[(size_t)r * d + k] == want, "expert %d gate/up row %d col %d", e, r, k);
                    }
                for (size_t k = 0; k < (size_t)d * F; ++k)
                    CHECK(ex[(size_t)2 * F * d + k] == Wd[k], "expert %d down element %zu", e, k);
                for (size_t k = 0; k < guard; ++k)
                    CHECK(ex[L->expert_bytes / 2 + k] == 0xA5A5, "write past the expert block");
            }
        }
    }
    // LM head: rows split one by one, gains of the final norm folded
    std::vector<uint16_t> lm(L->lm_bytes / 2 + guard, 0xA5A5);
    repack_lm(c, *L, M.p.data(), lm.data());
    const uint16_t* Wlm = M.t.back().data();
    const uint16_t* gf = M.t[M.t.size() - 2].data();
    for (int w = 0; w < 256; ++w) {
        int r0, n;
        my_split(c.vocab, 1, w, &r0, &n);
        const uint16_t* piece = lm.data() + (size_t)L->lm_off[w] * 512;
        for (int j = 0; j < n; ++j)
            for (int k = 0; k < d; ++k) {
                uint16_t want = folded(Wlm[(size_t)(r0 + j) * d + k], unit_gains ? nullptr : gf, k);
                CHECK(piece[(size_t)j * d + k] == want, "LM wg %d row %d col %d", w, r0 + j, k);
            }
    }
    for (size_t k = 0; k < guard; ++k) CHECK(lm[L->lm_bytes / 2 + k] == 0xA5A5, "write past the LM block");
    // rotary table
    std::vector<float> rope((size_t)c.max_seq * (hd / 2) * 2 + 64, -7.f);
    rope_table(c, rope.data());
    for (int p = 0; p < c.max_seq; p += 7)
        for (int i = 0; i < hd / 2; ++i) {
            double ang = p * std::pow((double)c.rope_theta, -2.0 * i / hd);
            CHECK(rope[((size_t)p * (hd / 2) + i) * 2] == (float)std::cos(ang), "rope cos p %d i %d", p, i);
            CHECK(rope[((size_t)p * (hd / 2) + i) * 2 + 1] == (float)std::sin(ang), "rope sin p %d i %d", p, i);
        }
    CHECK(rope[(size_t)c.max_seq * (hd / 2) * 2] == -7.f, "write past the rope table");
    delete L;
    return g_fail;
}

// Quantised MoE experts (repack_expert_quant): for every expert, each row's
// codes and scale equal the row quantizer's output on that row (gate/up rows
// with the folded gain, down rows without), at the place this file works out
// from the unit rules: fp8 rows in pairs (unit column s of a pair: lane l
// holds 8 codes of row a, then 8 of row b, columns 512 s + 8 l ..), fp4 rows in
// fours (lane l holds 4 bytes per row, byte b = columns 512 s + 8 l + 2 b
// (low nibble) and + 1 (high nibble)); gate/up rows interleaved g_p, u_p; the
// down rows after the 2F gate/up rows; nothing written past expert_bytes.
static int check_expert_quant(const kie_config& c) {
    Model M = make_model(c, false);
    std::string err;
    CHECK(validate_config(c, &err) == KIE_OK, "quantised MoE config rejected: %s", err.c_str());
    Layout* L = new Layout;
    make_layout(c, L);
    const int d = c.d_model, F = c.ffn_dim;
    const bool fp4 = c.weight_format == KIE_WEIGHTS_FP4;
    const int rpu = fp4 ? 4 : 2;                       // rows per unit column
    const size_t want_bytes = (size_t)3 * F * d / (fp4 ? 2 : 1);
    CHECK(L->expert_bytes == want_bytes, "expert_bytes %zu, want %zu", L->expert_bytes, want_bytes);
    const int per_layer = 6 + 1 + 3 * c.n_experts;
    std::vector<uint8_t> blk(L->expert_bytes + 4096);
    std::vector<float> sc(2 * F + d + 16);
    std::vector<uint8_t> q(8192);
    for (int l = 0; l < c.n_layers; ++l)
        for (int e = 0; e < c.n_experts; ++e) {
            std::fill(blk.begin(), blk.end(), 0xA5);
            std::fill(sc.begin(), sc.end(), -7.f);
            repack_expert_quant(c, *L, M.p.data(), l, e, blk.data(), sc.data());
            const uint16_t* g = M.t[1 + l * per_layer + 5].data();
            const uint16_t* W[3];
            for (int i = 0; i < 3; ++i) W[i] = M.t[1 + l * per_layer + 7 + 3 * e + i].data();
            // virtual row v: gate/up v < 2F (g_{v/2} or u_{v/2}), down 2F + r
            for (int v = 0; v < 2 * F + d; ++v) {
                const bool gu = v < 2 * F;
                const int K = gu ? d : F;
                const uint16_t* src = gu ? W[v % 2] + (size_t)(v / 2) * d : W[2] + (size_t)(v - 2 * F) * F;
                float s;
                if (fp4) quantize_row_e2m1(src, gu ? g : nullptr, K, q.data(), &s);
                else quantize_row_e4m3(src, gu ? g : nullptr, K, q.data(), &s);
                CHECK(sc[v] == s, "layer %d expert %d row %d scale %g, want %g", l, e, v, sc[v], s);
                const int local = gu ? v : v - 2 * F;            // row within its matrix block
                const size_t base = gu ? 0 : (size_t)2 * F * d / (fp4 ? 2 : 1);
                const size_t group = (size_t)(local / rpu) * K * rpu / (fp4 ? 2 : 1);   // bytes before its group
                const int r = local % rpu;
                for (int k = 0; k < K; ++k) {
                    const int su = k / 512, ln = (k % 512) / 8, c8 = k % 8;
                    uint8_t got;
                    if (fp4) {
                        const uint8_t byte = blk[base + group + ((size_t)su * 64 + ln) * 16 + 4 * r + c8 / 2];
                        got = (c8 % 2) ? (byte >> 4) : (byte & 15);
                    } else {
                        got = blk[base + group + ((size_t)su * 64 + ln) * 16 + 8 * r + c8];
                    }
                    if (got != q[k]) {
                        CHECK(false, "layer %d expert %d row %d col %d code %d, want %d", l, e, v, k, got, q[k]);
                        break;
                    }
                }
            }
            CHECK(sc[2 * F + d] == -7.f, "scale written past the expert's rows");
            for (size_t i = L->expert_bytes; i < blk.size(); ++i)
                if (blk[i] != 0xA5) {
                    CHECK(false, "byte %zu written past the expert block", i);
                    break;
                }
        }
    delete L;
    return g_fail;
}

// The codes of virtual row r (within its group of rpu rows, r % rpu) at
// column k of a group that starts at byte base of blk, for a row length K:
// the unit rules stated once more, as in check_expert_quant.
static uint8_t code_at(const std::vector<uint8_t>& blk, size_t base, bool fp4, int r, int k) {
    const int su = k / 512, ln = (k % 512) / 8, c8 = k % 8;
    if (fp4) {
        const uint8_t byte = blk[base + ((size_t)su * 64 + ln) * 16 + 4 * r + c8 / 2];
        return (c8 % 2) ? (byte >> 4) : (byte & 15);
    }
    return blk[base + ((size_t)su * 64 + ln) * 16 + 8 * r + c8];
}

// Quantised layer blocks and LM head (repack_layer_fp8, repack_lm_fp8, both
// formats): each workgroup's rows of each phase, in phase order and whole
// groups (fp8 pairs, fp4 fours: QKV and gate/up in fours of rows, Wo, down and
// the router and LM head in the format's group), carry the row quantizer's
// codes of the row the layout rules name (gains folded as for fp16) and its
// scale at the phase's offset in the layer's scale block; padding is zero and
// nothing is written past a block.
static int check_layer_quant(const kie_config& c) {
    Model M = make_model(c, false);
    std::string err;
    CHECK(validate_config(c, &err) == KIE_OK, "quantised config rejected: %s", err.c_str());
    Layout* L = new Layout;
    make_layout(c, L);
    const bool fp4 = c.weight_format == KIE_WEIGHTS_FP4;
    const int rpu = fp4 ? 4 : 2, d = c.d_model, H = c.n_heads, Hkv = c.n_kv_heads, hd = c.head_dim, F = c.ffn_dim;
    const int per_layer = 6 + (c.n_experts ? 1 + 3 * c.n_experts : 3);
    auto T = [&](int l, int which) { return M.t[1 + l * per_layer + which].data(); };
    struct Ph { int M, K, gran, kind; };
    std::vector<Ph> phases;
    phases.push_back({(H + 2 * Hkv) * hd, d, 4, 0});
    phases.push_back({d, H * hd, rpu, 1});
    if (c.n_experts) phases.push_back({c.n_experts, d, rpu, 4});
    else {
        phases.push_back({2 * F, d, 4, 2});
        phases.push_back({d, F, rpu, 3});
    }
    std::vector<uint8_t> q(8192);
    const size_t guard = 1024;
    std::vector<uint8_t> blk(L->layer_bytes + guard);
    std::vector<float> sc(L->layer_scales + 16);
    for (int l = 0; l < c.n_layers; ++l) {
        std::fill(blk.begin(), blk.end(), 0xA5);
        std::fill(sc.begin(), sc.end(), -7.f);
        repack_layer_fp8(c, *L, M.p.data(), l, blk.data(), sc.data());
        size_t pos = 0;   // bytes, walking the pieces in workgroup order
        for (int w = 0; w < 256; ++w) {
            CHECK(pos == (size_t)L->piece_off[w] * 1024, "piece %d starts at %zu", w, pos);
            size_t sbase = 0;
            for (const Ph& ph : phases) {
                int r0, n;
                my_split(ph.M, ph.gran, w, &r0, &n);
                for (int j = 0; j < n; ++j) {
                    const int r = r0 + j;
                    const uint16_t* src;
                    const uint16_t* g = nullptr;
                    if (ph.kind == 0) {
                        int mat, row;
                        my_qkv_source(H, Hkv, hd, r, &mat, &row);
                        src = T(l, 1 + mat) + (size_t)row * d;
                        g = T(l, 0);
                    } else if (ph.kind == 1) {
                        src = T(l, 4) + (size_t)r * ph.K;
                    } else if (ph.kind == 2) {
                        src = T(l, (r % 2) ? 7 : 6) + (size_t)(r / 2) * d;
                        g = T(l, 5);
                    } else if (ph.kind == 3) {
                        src = T(l, 8) + (size_t)r * ph.K;
                    } else {
                        src = T(l, 6) + (size_t)r * d;
                        g = T(l, 5);
                    }
                    float s;
                    if (fp4) quantize_row_e2m1(src, g, ph.K, q.data(), &s);
                    else quantize_row_e4m3(src, g, ph.K, q.data(), &s);
                    CHECK(sc[sbase + r] == s, "layer %d phase %d row %d scale %g, want %g", l, ph.kind, r,
                          sc[sbase + r], s);
                    const size_t gbase = pos + (size_t)(j / rpu) * ph.K * rpu / (fp4 ? 2 : 1);
                    for (int k = 0; k < ph.K; ++k)
                        if (code_at(blk, gbase, fp4, j % rpu, k) != q[k]) {
                            CHECK(false, "layer %d wg %d phase %d row %d col %d", l, w, ph.kind, r, k);
                            break;
                        }
                }
                const size_t used = (size_t)n * ph.K / (fp4 ? 2 : 1), padded = (used + 1023) / 1024 * 1024;
                for (size_t k = used; k < padded; ++k) CHECK(blk[pos + k] == 0, "padding not zero");
                pos += padded;
                sbase += ph.M;
            }
        }
        CHECK(pos == L->layer_bytes, "layer block is %zu bytes, layout says %zu", pos, L->layer_bytes);
        for (size_t k = 0; k < guard; ++k) CHECK(blk[L->layer_bytes + k] == 0xA5, "write past the layer block");
        CHECK(sc[L->layer_scales] == -7.f, "scale written past the layer's scale block");
    }
    // LM head: rows in the format's groups, the final norm's gain folded
    std::vector<uint8_t> lm(L->lm_bytes + guard, 0xA5);
    std::vector<float> lsc(c.vocab + 16, -7.f);
    repack_lm_fp8(c, *L, M.p.data(), lm.data(), lsc.data());
    const uint16_t* Wlm = M.t.back().data();
    const uint16_t* gf = M.t[M.t.size() - 2].data();
    for (int w = 0; w < 256; ++w) {
        int r0, n;
        my_split(c.vocab, rpu, w, &r0, &n);
        const size_t piece = (size_t)L->lm_off[w] * 1024;
        for (int j = 0; j < n; ++j) {
            float s;
            if (fp4) quantize_row_e2m1(Wlm + (size_t)(r0 + j) * d, gf, d, q.data(), &s);
            else quantize_row_e4m3(Wlm + (size_t)(r0 + j) * d, gf, d, q.data(), &s);
            CHECK(lsc[r0 + j] == s, "LM row %d scale", r0 + j);
            const size_t gbase = piece + (size_t)(j / rpu) * d * rpu / (fp4 ? 2 : 1);
            for (int k = 0; k < d; ++k)
                if (code_at(lm, gbase, fp4, j % rpu, k) != q[k]) {
                    CHECK(false, "LM wg %d row %d col %d", w, r0 + j, k);
                    break;
                }
        }
    }
    for (size_t k = 0; k < guard; ++k) CHECK(lm[L->lm_bytes + k] == 0xA5, "write past the LM block");
    CHECK(lsc[c.vocab] == -7.f, "scale written past the LM rows");
    delete L;
    return g_fail;
}

int main() {
    // fp16 <-> fp32
    for (uint32_t h = 0; h < 65536; ++h) {
        if (((h >> 10) & 31) == 31 && (h & 1023)) continue;   // NaN payloads
        float f = f16_to_f32((uint16_t)h);
        CHECK((double)f == half_val((uint16_t)h), "f16_to_f32(%04x)", h);
        CHECK(f32_to_f16(f) == h, "round trip %04x", h);
    }
    for (int i = 0; i < 200000; ++i) {
        uint32_t bits = rnd() ^ (rnd() << 21);
        float f;
        std::memcpy(&f, &bits, 4);
        if (std::isnan(f)) continue;
        CHECK(f32_to_f16(f) == ref_half((double)f), "f32_to_f16(%a) = %04x, want %04x", (double)f, f32_to_f16(f),
              ref_half((double)f));
    }
    kie_config dense = {2, 512, 8, 2, 128, 1024, 1000, 0, 0, 1e-5f, 1e4f, 300};
    kie_config moe = {2, 512, 4, 2, 64, 512, 700, 6, 2, 1e-5f, 1e4f, 200};
    kie_config tiny = {1, 256, 4, 4, 64, 256, 300, 0, 0, 1e-5f, 1e4f, 50};
    for (bool unit : {false, true}) {
        check_model(dense, unit);
        check_model(moe, unit);
        check_model(tiny, unit);
    }
    // quantised experts: fp8 (even expert count) and fp4 (experts in fours)
    kie_config moe8 = {1, 512, 4, 2, 128, 1024, 700, 6, 2, 1e-5f, 1e4f, 64};
    moe8.weight_format = KIE_WEIGHTS_FP8;
    kie_config moe4 = {1, 1024, 8, 2, 128, 512, 704, 8, 2, 1e-5f, 1e4f, 64};
    moe4.weight_format = KIE_WEIGHTS_FP4;
    check_expert_quant(moe8);
    check_expert_quant(moe4);
    // quantised layer blocks and LM head: dense and MoE, both formats
    kie_config dense8 = {2, 1024, 8, 2, 128, 1536, 1002, 0, 0, 1e-5f, 1e4f, 64};
    dense8.weight_format = KIE_WEIGHTS_FP8;
    kie_config dense4 = dense8;
    dense4.vocab = 1004;
    dense4.weight_format = KIE_WEIGHTS_FP4;
    check_layer_quant(dense8);
    check_layer_quant(dense4);
    check_layer_quant(moe8);
    check_layer_quant(moe4);
    if (g_fail) {
        std::printf("%d mismatches\n", g_fail);
        return 1;
    }
    std::printf("OK\n");
    return 0;
}

// kie_kernels.hip - the persistent batch-1 decode kernel and the probes, gfx950.
//
// One launch runs n whole forward passes. Each of the 256 workgroups (one per
// compute unit) has 8 waves:
//   waves 0-1  stream the workgroup's weights from HBM into a 128 KiB LDS ring
//              with non-temporal global_load_lds_dwordx4, in exactly the order
//              the compute waves use them, never waiting on the grid;
//   waves 2-7  compute: per layer the phases
//                QKV GEMV (+RoPE, +KV append) | attention | Wo GEMV (+residual)
//                | gate/up GEMV (+SwiGLU)      | down GEMV (+residual)
//              (MoE: Wo | router | top-k | expert gate/up | expert down), then
//              LM head + argmax; a grid barrier separates dependent phases.
// Because the weights do not depend on activations, the streaming waves run
// ahead across barriers and attention: the next phase's weights are already
// in LDS when its inputs become ready. This is the monokernel of the
// news.creeta.com article ("Inside the monokernel": one resident grid for the
// whole decode loop, weight prefetch inside it, inter-CU barriers, on-device
// sampling, batch-1 GEMV on dot-product instructions rather than matrix
// cores) built for CDNA4: the grid is one workgroup per CU rather than the
// pages' 256-of-304-CU MI300X mapping, and no die-local buffer replication is
// used.
#include <hip/hip_runtime.h>

#include "kie_common.h"
#include "kie_device.h"
#include "kie_kernels.h"

namespace kie {

typedef RingCfg<kProducers, kConsumers, kSlots> RC;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxNormPerThread = (8192 + 64 * kConsumers - 1) / (64 * kConsumers);

// One workgroup's share of every phase: first row, row count and units.
struct WgPlan {
    int q0, qn, wo0, won, gu0, gun, r0, rn, egu0, egun, lm0, lmn;
    int nq, nwo, ngu, nd, nr, negu, ned, nlm;
    int piece, piece_off, lm_off;
};

__device__ __forceinline__ void make_plan(const DecodeArgs& a, int wg, WgPlan& P) {
    const Dims& D = a.D;
    const int G = kGrid;
    RowSplit r;
    r = split_rows(phase_shape(D, PH_QKV).M, 2, G, wg);
    P.q0 = r.row0; P.qn = r.nrows;
    r = split_rows(D.d, 1, G, wg);        // output projection, FFN down and residual ownership
    P.wo0 = r.row0; P.won = r.nrows;
    r = split_rows(D.V, 1, G, wg);
    P.lm0 = r.row0; P.lmn = r.nrows;
    P.nq = phase_units(D, PH_QKV, G, wg);
    P.nwo = phase_units(D, PH_WO, G, wg);
    P.nlm = phase_units(D, PH_LM, G, wg);
    if (D.E) {
        r = split_rows(D.E, 1, G, wg);
        P.r0 = r.row0; P.rn = r.nrows;
        r = split_rows(phase_shape(D, PH_EGU).M, 2, G, wg);
        P.egu0 = r.row0; P.egun = r.nrows;
        P.gu0 = P.gun = 0;
        P.nr = phase_units(D, PH_ROUTER, G, wg);
        P.negu = phase_units(D, PH_EGU, G, wg);
        P.ned = phase_units(D, PH_EDOWN, G, wg);
        P.ngu = P.nd = 0;
    } else {
        r = split_rows(2 * D.F, 2, G, wg);
        P.gu0 = r.row0; P.gun = r.nrows;
        P.r0 = P.rn = P.egu0 = P.egun = 0;
        P.ngu = phase_units(D, PH_GU, G, wg);
        P.nd = phase_units(D, PH_DOWN, G, wg);
        P.nr = P.negu = P.ned = 0;
    }
    P.piece_off = a.plan[wg];
    P.piece = a.plan[wg + 1] - a.plan[wg];
    P.lm_off = a.plan[G + 1 + wg];
}

__device__ __forceinline__ bool do_lm(const DecodeArgs& a, int step) {
    return !(a.flags & F_SKIP_LM) || step == a.n_steps - 1;
}

// ------------------------------------------------------------ producer ----
__device__ __forceinline__ void run_producer(const DecodeArgs& a, KIE_LDS RingCtl* ctl, KIE_LDS uint8_t* ring, int p) {
    Producer<RC, kDepth> P;
    P.init(ctl, ring, (uint32_t)p, a.spin_lds);
    const int wg = blockIdx.x;
    const Dims& D = a.D;
    WgPlan W;
    make_plan(a, wg, W);
    for (int step = 0; step < a.n_steps; ++step) {
        for (int l = 0; l < D.L; ++l) {
            if (!P.stream(a.layers + (size_t)l * a.layer_bytes + (size_t)W.piece_off * kUnitBytes, W.piece))
                return;
            if (D.E) {
                // expert weights depend on this layer's routing decision
                P.publish_all();
                uint32_t need = (uint32_t)(step * D.L + l + 1);
                uint32_t spins = 0;
                while ((int)(lds_ld_u32(&ctl->route) - need) < 0) {
                    if (lds_ld_u32(&ctl->abort)) return;
                    if (++spins > a.spin_lds) {
                        lds_st_u32(&ctl->abort, 1);
                        return;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                const uint8_t* lb = a.experts + (size_t)l * D.E * a.expert_bytes;
                // gate/up: virtual rows [row0, row0+nrows) of top_k stacked 2F x d blocks
                const int per = 2 * D.F;
                int r0 = W.egu0, r1 = W.egu0 + W.egun;
                while (r0 < r1) {
                    int k = r0 / per;
                    int seg_end = (k + 1) * per < r1 ? (k + 1) * per : r1;
                    uint32_t e = lds_ld_u32(&ctl->sel[k]);
                    const uint8_t* src = lb + (size_t)e * a.expert_bytes + (size_t)(r0 - k * per) * D.d * 2;
                    if (!P.stream(src, (uint32_t)slab_units(seg_end - r0, D.d))) return;
                    r0 = seg_end;
                }
                // down: rows [row0, row0+nrows) of every selected expert's d x F block
                for (int k = 0; k < D.topk; ++k) {
                    uint32_t e = lds_ld_u32(&ctl->sel[k]);
                    const uint8_t* src = lb + (size_t)e * a.expert_bytes + (size_t)per * D.d * 2 +
                                         (size_t)W.wo0 * D.F * 2;
                    if (!P.stream(src, (uint32_t)slab_units(W.won, D.F))) return;
                }
            }
        }
        if (do_lm(a, step))
            if (!P.stream(a.lm + (size_t)W.lm_off * kUnitBytes, W.nlm)) return;
    }
    P.publish_all();
}

// ------------------------------------------------------------ consumer ----
template <int HD>
struct Consumer {
    const DecodeArgs& a;
    KIE_LDS RingCtl* ctl;
    KIE_LDS uint8_t* ring;
    KIE_LDS uint16_t* xin;     // fp16 GEMV input
    KIE_LDS float* part;       // partial sums
    KIE_LDS float* attn_lds;   // attention scratch (aliases xin/part)
    int cw, lane, t, wg;
    uint32_t avail;    // stream units below this are in LDS
    uint32_t sgen;
    uint32_t epoch;
    uint32_t U;        // next stream unit
    WgPlan W;
    const Dims& D;

    __device__ __forceinline__ Consumer(const DecodeArgs& args, KIE_LDS RingCtl* c, KIE_LDS uint8_t* r,
                                        KIE_LDS uint8_t* regA, int cwi)
        : a(args), ctl(c), ring(r), cw(cwi), D(args.D) {
        xin = (KIE_LDS uint16_t*)regA;
        part = (KIE_LDS float*)(regA + kXinBytes);
        attn_lds = (KIE_LDS float*)regA;
        lane = lane_id();
        t = cw * 64 + lane;
        wg = blockIdx.x;
        avail = 0;
        sgen = 0;
        epoch = a.epoch0;
        U = 0;
        make_plan(a, wg, W);
    }

    __device__ __forceinline__ bool sync() {
        sgen += kConsumers;
        return consumer_sync(ctl, sgen, a.spin_lds);
    }

    // All consumer waves: finish global stores, meet, leader crosses the grid.
    __device__ __forceinline__ bool grid_sync() {
        wait_vm0();
        if (!sync()) return false;
        ++epoch;
        if (cw == 0) {
            bool ok = grid_barrier_leader(a.bar, a.status, kGrid, wg, epoch, a.spin_grid);
            if (!ok && lane == 0) lds_st_u32(&ctl->abort, 1);
        }
        return sync();
    }

    // --- GEMV input preparation -----------------------------------------
    // xin = fp16(x * rsqrt(mean(x^2) + eps)); source is the fp32 residual, or
    // the fp16 embedding row for the first layer.
    __device__ __forceinline__ bool prep_norm(const float* xs, const uint16_t* es) {
        float v[kMaxNormPerThread];
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < kMaxNormPerThread; ++j) {
            int k = t + j * 64 * kConsumers;
            float val = 0.f;
            if (k < D.d) val = xs ? xs[k] : h2f_bits(es[k]);
            v[j] = val;
            ss += val * val;
        }
        ss = wave_sum_to_lane63(ss);
        if (lane == 63) ctl->scratch[cw] = ss;
        if (!sync()) return false;
        float tot = 0.f;
#pragma unroll
        for (int c = 0; c < kConsumers; ++c) tot += ctl->scratch[c];
        float s = 1.0f / sqrtf(tot / (float)D.d + a.eps);
#pragma unroll
        for (int j = 0; j < kMaxNormPerThread; ++j) {
            int k = t + j * 64 * kConsumers;
            if (k < D.d) xin[k] = f2h_bits(v[j] * s);
        }
        return sync();
    }

    // xin[0..n) = src[0..n) (fp16, n a multiple of 8)
    __device__ __forceinline__ bool prep_copy(const uint16_t* src, int n) {
        const uint4* s4 = (const uint4*)src;
        for (int i = t; i < n / 8; i += 64 * kConsumers) lds_st16(xin + i * 8, s4[i]);
        return sync();
    }

    // The next stream unit this wave will consume after phase-local unit i of
    // a phase of n units starting at U0: the next unit of its residue class in
    // this phase, else its first unit of the following phase. Publishing
    // anything larger would let the streamer overwrite a slot not yet read.
    __device__ __forceinline__ uint32_t next_unit(uint32_t U0, int i, int n) {
        return (i + kConsumers < n) ? U0 + (uint32_t)(i + kConsumers) : U0 + (uint32_t)(n + cw);
    }

    // --- the streamed GEMV ------------------------------------------------
    // Units U..U+n-1 of the stream hold this workgroup's rows. Segment-major:
    // nseg segments of nrows rows of K fp16 each (nseg > 1 only for the MoE
    // down projection, whose input is the concatenation of the experts' h).
    // part[row * nseg*upr + seg*upr + cc] receives each 512-wide slice's dot.
    __device__ __forceinline__ bool gemv(int n, int nrows, int K, int nseg) {
        const uint32_t U0 = U;
        if (K >= 512) {
            const int upr = K / 512;
            const int per_seg = nrows * upr;
            for (int i = cw; i < n; i += kConsumers) {
                uint32_t u = U0 + (uint32_t)i;
                if (!ring_wait_ready(ctl, u, avail, a.spin_lds)) return false;
                uint4 w = lds_ld16(ring + (u & RC::kMask) * kUnitBytes + lane * 16);
                int seg = i / per_seg;
                int rem = i - seg * per_seg;
                int row = rem / upr;
                int cc = rem - row * upr;
                uint4 xv = lds_ld16(xin + seg * K + cc * 512 + lane * 8);
                float acc = dot8(w, xv, 0.f);
                lds_st_u32(&ctl->cons[cw], next_unit(U0, i, n));
                acc = wave_sum_to_lane63(acc);
                if (lane == 63) part[row * (nseg * upr) + seg * upr + cc] = acc;
            }
        } else {
            // K = 256: one unit covers two rows (lanes 0-31 and 32-63)
            for (int i = cw; i < n; i += kConsumers) {
                uint32_t u = U0 + (uint32_t)i;
                if (!ring_wait_ready(ctl, u, avail, a.spin_lds)) return false;
                uint4 w = lds_ld16(ring + (u & RC::kMask) * kUnitBytes + lane * 16);
                uint4 xv = lds_ld16(xin + (lane & 31) * 8);
                float acc = dot8(w, xv, 0.f);
                lds_st_u32(&ctl->cons[cw], next_unit(U0, i, n));
                acc = half32_sum_from_rows(row16_sum(acc));
                int row = 2 * i + (lane >> 5);
                if ((lane & 31) == 31 && row < nrows) part[row] = acc;
            }
        }
        U = U0 + (uint32_t)n;
        lds_st_u32(&ctl->cons[cw], U + (uint32_t)cw);
        return sync();
    }

    __device__ __forceinline__ float rowsum(int r, int cols) {
        float s = 0.f;
        const KIE_LDS float* p = part + r * cols;
        for (int j = 0; j < cols; ++j) s += p[j];
        return s;
    }
    __device__ __forceinline__ int cols_of(int K, int nseg) { return K >= 512 ? nseg * (K / 512) : 1; }

    // --- phases -------------------------------------------------------------
    __device__ __forceinline__ bool phase_qkv(int l, int pos, int tok) {
        const bool first = (l == 0);
        if (first) {
            // owners of the residual rows start it from the embedding row
            const uint16_t* e = a.emb + (size_t)tok * D.d;
            for (int j = t; j < W.won; j += 64 * kConsumers)
                a.x[W.wo0 + j] = h2f_bits(e[W.wo0 + j]);
            if (!prep_norm(nullptr, e)) return false;
        } else {
            if (!prep_norm(a.x, nullptr)) return false;
        }
        if (!gemv(W.nq, W.qn, D.d, 1)) return false;
        const int cols = cols_of(D.d, 1);
        const int qd = D.H * HD, kd = D.Hkv * HD;
        const float* rope = a.rope + (size_t)pos * HD;   // [hd/2][2]
        for (int j = t; j < W.qn / 2; j += 64 * kConsumers) {
            float y0 = rowsum(2 * j, cols), y1 = rowsum(2 * j + 1, cols);
            int vr = W.q0 + 2 * j;
            if (vr < qd + kd) {
                int i = (vr % HD) >> 1;
                float c = rope[2 * i], s = rope[2 * i + 1];
                float r0 = y0 * c - y1 * s, r1 = y1 * c + y0 * s;
                if (vr < qd) {
                    int head = vr / HD;
                    a.q[head * HD + i] = r0;
                    a.q[head * HD + i + HD / 2] = r1;
                } else {
                    int g = (vr - qd) / HD;
                    uint16_t* kp = a.kc + (((size_t)l * D.Hkv + g) * D.max_seq + pos) * HD;
                    kp[i] = f2h_bits(r0);
                    kp[i + HD / 2] = f2h_bits(r1);
                }
            } else {
                int vi = vr - qd - kd;
                int g = vi / HD, dd = vi % HD;
                uint16_t* vp = a.vc + (((size_t)l * D.Hkv + g) * D.max_seq + pos) * HD;
                vp[dd] = f2h_bits(y0);
                vp[dd + 1] = f2h_bits(y1);
            }
        }
        return grid_sync();
    }

    // attention of one query position over positions 0..pos of layer l
    __device__ __forceinline__ bool phase_attn(int l, int pos) {
        constexpr int LPP = HD / 8;          // lanes per position
        constexpr int PPI = 64 / LPP;        // positions per wave instruction
        const int c = pos + 1;
        const int Gq = D.H / D.Hkv;
        int nper = ceil_div(c, kAttnChunkMin);
        if (nper > a.items_per_head) nper = a.items_per_head;
        const int CH = ceil_div(c, nper);
        nper = ceil_div(c, CH);
        const int items = D.Hkv * nper;
        const int g = wg % D.Hkv, chunk = wg / D.Hkv;
        const bool mine = wg < items;
        KIE_LDS float* wst = attn_lds;                                   // [NC][8][HD] o
        KIE_LDS float* wml = attn_lds + kConsumers * kMaxGroup * HD;     // [NC][8][2] m, l
        if (mine) {
            const int p0 = chunk * CH;
            const int p1 = (p0 + CH < c) ? p0 + CH : c;
            const int gi = lane / LPP, dl = (lane % LPP) * 8;
            const float qs = kLog2e / sqrtf((float)HD);
            float qv[kMaxGroup][8];
#pragma unroll
            for (int j = 0; j < kMaxGroup; ++j) {
                if (j < Gq) {
                    const float4* qp = (const float4*)(a.q + (g * Gq + j) * HD + dl);
                    float4 q0 = qp[0], q1 = qp[1];
                    qv[j][0] = q0.x * qs; qv[j][1] = q0.y * qs; qv[j][2] = q0.z * qs; qv[j][3] = q0.w * qs;
                    qv[j][4] = q1.x * qs; qv[j][5] = q1.y * qs; qv[j][6] = q1.z * qs; qv[j][7] = q1.w * qs;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) qv[j][e] = 0.f;
                }
            }
            float m[kMaxGroup], ls[kMaxGroup], o[kMaxGroup][8];
#pragma unroll
            for (int j = 0; j < kMaxGroup; ++j) {
                m[j] = -1e30f;
                ls[j] = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[j][e] = 0.f;
            }
            const uint16_t* Kb = a.kc + ((size_t)l * D.Hkv + g) * D.max_seq * HD;
            const uint16_t* Vb = a.vc + ((size_t)l * D.Hkv + g) * D.max_seq * HD;
            for (int b = p0 + cw * PPI; b < p1; b += kConsumers * PPI) {
                const int pp = b + gi;
                const bool valid = pp < p1;
                uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
                if (valid) {
                    kv = *(const uint4*)(Kb + (size_t)pp * HD + dl);
                    vv = *(const uint4*)(Vb + (size_t)pp * HD + dl);
                }
                float kf[8], vf[8];
                {
                    const uint16_t* kh = (const uint16_t*)&kv;
                    const uint16_t* vh = (const uint16_t*)&vv;
#pragma unroll
                    for (int e = 0; e < 8; ++e) { kf[e] = h2f_bits(kh[e]); vf[e] = h2f_bits(vh[e]); }
                }
#pragma unroll
                for (int j = 0; j < kMaxGroup; ++j) {
                    if (j < Gq) {
                        float s = 0.f;
#pragma unroll
                        for (int e = 0; e < 8; ++e) s += qv[j][e] * kf[e];
                        s = (LPP == 16) ? row16_sum(s) : row8_sum(s);
                        if (valid) {
                            float mn = fmaxf(m[j], s);
                            float cr = __builtin_amdgcn_exp2f(m[j] - mn);
                            float p = __builtin_amdgcn_exp2f(s - mn);
                            ls[j] = ls[j] * cr + p;
#pragma unroll
                            for (int e = 0; e < 8; ++e) o[j][e] = o[j][e] * cr + p * vf[e];
                            m[j] = mn;
                        }
                    }
                }
            }
            // merge the position groups of this wave
#pragma unroll
            for (int off = LPP; off < 64; off <<= 1) {
#pragma unroll
                for (int j = 0; j < kMaxGroup; ++j) {
                    if (j < Gq) {
                        float m2 = shfl_xor_f(m[j], off), l2 = shfl_xor_f(ls[j], off);
                        float mn = fmaxf(m[j], m2);
                        float f1 = __builtin_amdgcn_exp2f(m[j] - mn), f2 = __builtin_amdgcn_exp2f(m2 - mn);
                        ls[j] = ls[j] * f1 + l2 * f2;
#pragma unroll
                        for (int e = 0; e < 8; ++e) o[j][e] = o[j][e] * f1 + shfl_xor_f(o[j][e], off) * f2;
                        m[j] = mn;
                    }
                }
            }
            if (lane < LPP) {
#pragma unroll
                for (int j = 0; j < kMaxGroup; ++j) {
                    if (j < Gq) {
                        KIE_LDS float* dst = wst + (cw * kMaxGroup + j) * HD + dl;
#pragma unroll
                        for (int e = 0; e < 8; ++e) dst[e] = o[j][e];
                        if (lane == 0) {
                            wml[(cw * kMaxGroup + j) * 2 + 0] = m[j];
                            wml[(cw * kMaxGroup + j) * 2 + 1] = ls[j];
                        }
                    }
                }
            }
        }
        if (!sync()) return false;
        if (mine) {
            // merge the waves; write the result or this chunk's partial state
            for (int idx = t; idx < Gq * HD; idx += 64 * kConsumers) {
                int j = idx / HD, dd = idx % HD;
                float M = -1e30f;
                for (int w = 0; w < kConsumers; ++w) M = fmaxf(M, wml[(w * kMaxGroup + j) * 2]);
                float L = 0.f, O = 0.f;
                for (int w = 0; w < kConsumers; ++w) {
                    float f = __builtin_amdgcn_exp2f(wml[(w * kMaxGroup + j) * 2] - M);
                    L += f * wml[(w * kMaxGroup + j) * 2 + 1];
                    O += f * wst[(w * kMaxGroup + j) * HD + dd];
                }
                int head = g * Gq + j;
                if (nper == 1) {
                    a.o16[head * HD + dd] = f2h_bits(O / L);
                } else {
                    float* pp = a.attn_part + ((size_t)head * a.items_per_head + chunk) * (HD + 2);
                    pp[2 + dd] = O;
                    if (dd == 0) { pp[0] = M; pp[1] = L; }
                }
            }
        }
        if (nper > 1) {
            // the last chunk of each KV head to finish combines all chunks
            bool last = false;
            if (mine) {
                wait_vm0();
                if (!sync()) return false;
                if (cw == 0) {
                    uint32_t old = 0;
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                    if (lane == 0)
                        old = __hip_atomic_fetch_add(&a.attn_cnt[g * 16], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
                    old = __builtin_amdgcn_readfirstlane(old);
                    uint32_t is_last = (old == (uint32_t)(nper - 1)) ? 1u : 0u;
                    if (is_last) {
                        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                        if (lane == 0)
                            __hip_atomic_store(&a.attn_cnt[g * 16], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                    if (lane == 0) lds_st_u32(&ctl->flag, is_last);
                }
                if (!sync()) return false;
                last = lds_ld_u32(&ctl->flag) != 0;
            }
            if (last) {
                for (int idx = t; idx < Gq * HD; idx += 64 * kConsumers) {
                    int j = idx / HD, dd = idx % HD;
                    int head = g * Gq + j;
                    const float* base = a.attn_part + (size_t)head * a.items_per_head * (HD + 2);
                    float M = -1e30f;
                    for (int ch = 0; ch < nper; ++ch) M = fmaxf(M, base[ch * (HD + 2)]);
                    float L = 0.f, O = 0.f;
                    for (int ch = 0; ch < nper; ++ch) {
                        float f = __builtin_amdgcn_exp2f(base[ch * (HD + 2)] - M);
                        L += f * base[ch * (HD + 2) + 1];
                        O += f * base[ch * (HD + 2) + 2 + dd];
                    }
                    a.o16[head * HD + dd] = f2h_bits(O / L);
                }
            }
        }
        return grid_sync();
    }

    __device__ __forceinline__ bool phase_wo(int l) {
        if (!prep_copy(a.o16, D.H * HD)) return false;
        if (!gemv(W.nwo, W.won, D.H * HD, 1)) return false;
        const int cols = cols_of(D.H * HD, 1);
        for (int j = t; j < W.won; j += 64 * kConsumers) a.x[W.wo0 + j] += rowsum(j, cols);
        return grid_sync();
    }

    __device__ __forceinline__ bool phase_gu() {
        if (!prep_norm(a.x, nullptr)) return false;
        if (!gemv(W.ngu, W.gun, D.d, 1)) return false;
        const int cols = cols_of(D.d, 1);
        for (int j = t; j < W.gun / 2; j += 64 * kConsumers) {
            float gv = rowsum(2 * j, cols), uv = rowsum(2 * j + 1, cols);
            float sg = gv / (1.0f + __expf(-gv));
            a.h16[W.gu0 / 2 + j] = f2h_bits(sg * uv);
        }
        return grid_sync();
    }

    __device__ __forceinline__ bool phase_down() {
        if (!prep_copy(a.h16, D.F)) return false;
        if (!gemv(W.nd, W.won, D.F, 1)) return false;
        const int cols = cols_of(D.F, 1);
        for (int j = t; j < W.won; j += 64 * kConsumers) a.x[W.wo0 + j] += rowsum(j, cols);
        return grid_sync();
    }

    __device__ __forceinline__ bool phase_router() {
        if (!prep_norm(a.x, nullptr)) return false;
        if (!gemv(W.nr, W.rn, D.d, 1)) return false;
        const int cols = cols_of(D.d, 1);
        for (int j = t; j < W.rn; j += 64 * kConsumers) a.router[W.r0 + j] = rowsum(j, cols);
        return grid_sync();
    }

    // softmax over the router logits, top-k (ties to the lower expert index),
    // computed redundantly by every workgroup; published to the producers.
    __device__ __forceinline__ bool route(int step, int l) {
        if (cw == 0) {
            float mx = -3.0e38f;
            for (int e = lane; e < D.E; e += 64) mx = fmaxf(mx, a.router[e]);
            for (int off = 32; off; off >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, off));
            float sum = 0.f;
            for (int e = lane; e < D.E; e += 64) sum += __expf(a.router[e] - mx);
            for (int off = 32; off; off >>= 1) sum += shfl_xor_f(sum, off);
            // k-th pick: the largest (logit, -index) strictly below the previous pick
            float pv = 3.0e38f;
            int pix = -1;
            for (int k = 0; k < D.topk; ++k) {
                float bv = -3.0e38f;
                int bi = 0x7fffffff;
                for (int e = lane; e < D.E; e += 64) {
                    float v = a.router[e];
                    bool below = (v < pv) || (v == pv && e > pix);
                    if (below && (v > bv || (v == bv && e < bi))) { bv = v; bi = e; }
                }
                for (int off = 32; off; off >>= 1) {
                    float ov = shfl_xor_f(bv, off);
                    int oi = shfl_xor_i(bi, off);
                    if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
                }
                pv = bv;
                pix = bi;
                if (lane == 0) {
                    ctl->sel[k] = (uint32_t)bi;
                    ctl->pi[k] = __expf(bv - mx) / sum;
                }
            }
            if (lane == 0) {
                if ((a.flags & F_DBG_EXPERTS) && wg == 0) {
                    int row = step % 64;
                    for (int k = 0; k < D.topk; ++k)
                        a.dbg_experts[((size_t)row * D.L + l) * D.topk + k] = (int32_t)ctl->sel[k];
                }
                wait_lgkm0();
                lds_st_u32(&ctl->route, (uint32_t)(step * D.L + l + 1));
            }
        }
        return sync();
    }

    __device__ __forceinline__ bool phase_egu() {
        if (!prep_norm(a.x, nullptr)) return false;
        if (!gemv(W.negu, W.egun, D.d, 1)) return false;
        const int cols = cols_of(D.d, 1);
        for (int j = t; j < W.egun / 2; j += 64 * kConsumers) {
            float gv = rowsum(2 * j, cols), uv = rowsum(2 * j + 1, cols);
            int vr = W.egu0 + 2 * j;
            int k = vr / (2 * D.F), jj = (vr % (2 * D.F)) >> 1;
            float sg = gv / (1.0f + __expf(-gv));
            a.h16[k * D.F + jj] = f2h_bits(ctl->pi[k] * sg * uv);
        }
        return grid_sync();
    }

    __device__ __forceinline__ bool phase_edown() {
        if (!prep_copy(a.h16, D.topk * D.F)) return false;
        if (!gemv(W.ned, W.won, D.F, D.topk)) return false;
        const int cols = cols_of(D.F, D.topk);
        for (int j = t; j < W.won; j += 64 * kConsumers) a.x[W.wo0 + j] += rowsum(j, cols);
        return grid_sync();
    }

    // LM head, local argmax, grid-wide argmax. Returns the token (or -1 on abort).
    __device__ __forceinline__ int phase_lm(int step) {
        if (!prep_norm(a.x, nullptr)) return -1;
        if (!gemv(W.nlm, W.lmn, D.d, 1)) return -1;
        const int cols = cols_of(D.d, 1);
        float bv = -3.0e38f;
        int bi = 0x7fffffff;
        const bool dbg = (a.flags & F_DBG_LOGITS) != 0;
        for (int j = t; j < W.lmn; j += 64 * kConsumers) {
            float v = rowsum(j, cols);
            int r = W.lm0 + j;
            if (dbg) a.dbg_logits[(size_t)(step % 64) * D.V + r] = v;
            if (v > bv || (v == bv && r < bi)) { bv = v; bi = r; }
        }
        for (int off = 32; off; off >>= 1) {
            float ov = shfl_xor_f(bv, off);
            int oi = shfl_xor_i(bi, off);
            if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
        }
        if (lane == 0) {
            ctl->scratch[2 * cw] = bv;
            ctl->scratch[2 * cw + 1] = __builtin_bit_cast(float, bi);
        }
        if (!sync()) return -1;
        if (t == 0) {
            float b = ctl->scratch[0];
            int ix = __builtin_bit_cast(int, ctl->scratch[1]);
            for (int c = 1; c < kConsumers; ++c) {
                float v = ctl->scratch[2 * c];
                int i = __builtin_bit_cast(int, ctl->scratch[2 * c + 1]);
                if (v > b || (v == b && i < ix)) { b = v; ix = i; }
            }
            a.argmax[2 * wg] = b;
            a.argmax[2 * wg + 1] = __builtin_bit_cast(float, ix);
        }
        if (!grid_sync()) return -1;
        if (cw == 0) {
            float b = -3.0e38f;
            int ix = 0x7fffffff;
            for (int w = lane; w < kGrid; w += 64) {
                float v = a.argmax[2 * w];
                int i = __builtin_bit_cast(int, a.argmax[2 * w + 1]);
                if (v > b || (v == b && i < ix)) { b = v; ix = i; }
            }
            for (int off = 32; off; off >>= 1) {
                float ov = shfl_xor_f(b, off);
                int oi = shfl_xor_i(ix, off);
                if (ov > b || (ov == b && oi < ix)) { b = ov; ix = oi; }
            }
            if (lane == 0) lds_st_u32(&ctl->token, (uint32_t)ix);
        }
        if (!sync()) return -1;
        return (int)lds_ld_u32(&ctl->token);
    }

    __device__ __forceinline__ void run() {
        int tok = a.pending;
        for (int step = 0; step < a.n_steps; ++step) {
            const int pos = a.pos0 + step;
            for (int l = 0; l < D.L; ++l) {
                if (!phase_qkv(l, pos, tok)) return;
                if (!phase_attn(l, pos)) return;
                if (!phase_wo(l)) return;
                if (D.E) {
                    if (!phase_router()) return;
                    if (!route(step, l)) return;
                    if (!phase_egu()) return;
                    if (!phase_edown()) return;
                } else {
                    if (!phase_gu()) return;
                    if (!phase_down()) return;
                }
            }
            int next = -1;
            if (do_lm(a, step)) {
                next = phase_lm(step);
                if (next < 0) return;
            }
            if (wg == 0 && t == 0) a.out_ids[step] = next;
            if ((a.flags & F_FORCE) && a.force_ids[step] >= 0) next = a.force_ids[step];
            tok = next;
        }
    }
};

template <int HD>
__global__ void __launch_bounds__(kThreads, 1) decode_kernel(const DecodeArgs* __restrict__ ap) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const DecodeArgs& a = *ap;
    KIE_LDS uint8_t* ring = (KIE_LDS uint8_t*)lds;
    KIE_LDS uint8_t* regA = ring + kSlots * kUnitBytes;
    KIE_LDS RingCtl* ctl = (KIE_LDS RingCtl*)(regA + kRegionA);
    if (threadIdx.x < kCtlBytes / 4) ((KIE_LDS uint32_t*)ctl)[threadIdx.x] = 0u;
    __syncthreads();
    if (threadIdx.x < kConsumers) ctl->cons[threadIdx.x] = threadIdx.x;
    __syncthreads();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (wave < kProducers) {
        run_producer(a, ctl, ring, wave);
    } else {
        Consumer<HD> c(a, ctl, ring, regA, wave - kProducers);
        c.run();
    }
}

// ------------------------------------------------------------ GEMV probe --
// The same streamer + consumer GEMV over `copies` rotating matrices: each
// workgroup streams its rows of every copy in turn.
__global__ void __launch_bounds__(kThreads, 1) gemv_ring_kernel(GemvArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    KIE_LDS uint8_t* ring = (KIE_LDS uint8_t*)lds;
    KIE_LDS uint8_t* regA = ring + kSlots * kUnitBytes;
    KIE_LDS RingCtl* ctl = (KIE_LDS RingCtl*)(regA + kRegionA);
    KIE_LDS float* part = (KIE_LDS float*)regA;
    if (threadIdx.x < kCtlBytes / 4) ((KIE_LDS uint32_t*)ctl)[threadIdx.x] = 0u;
    __syncthreads();
    if (threadIdx.x < kConsumers) ctl->cons[threadIdx.x] = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const RowSplit r = split_rows(a.M, 1, gridDim.x, blockIdx.x);
    const int n = slab_units(r.nrows, a.K);
    const size_t mat = (size_t)a.M * a.K * 2;
    __syncthreads();
    if (wave < kProducers) {
        Producer<RC, kDepth> P;
        P.init(ctl, ring, (uint32_t)wave, a.spin_lds);
        for (int c = 0; c < a.copies; ++c)
            if (!P.stream(a.A + c * mat + (size_t)r.row0 * a.K * 2, (uint32_t)n)) return;
        P.publish_all();
        return;
    }
    const int cw = wave - kProducers, lane = lane_id(), t = cw * 64 + lane;
    const int upr = a.K / 512;
    uint32_t avail = 0, sgen = 0, U = 0;
    for (int c = 0; c < a.copies; ++c) {
        for (int i = cw; i < n; i += kConsumers) {
            uint32_t u = U + (uint32_t)i;
            if (!ring_wait_ready(ctl, u, avail, a.spin_lds)) return;
            uint4 w = lds_ld16(ring + (u & RC::kMask) * kUnitBytes + lane * 16);
            int row = i / upr, cc = i - row * upr;
            uint4 xv = *(const uint4*)(a.x + cc * 512 + lane * 8);   // x stays in L1/L2
            float acc = dot8(w, xv, 0.f);
            // the next unit this wave consumes (see Consumer::next_unit)
            lds_st_u32(&ctl->cons[cw], (i + kConsumers < n) ? u + kConsumers : U + (uint32_t)(n + cw));
            acc = wave_sum_to_lane63(acc);
            if (lane == 63) part[row * upr + cc] = acc;
        }
        U += (uint32_t)n;
        lds_st_u32(&ctl->cons[cw], U + (uint32_t)cw);
        sgen += kConsumers;
        if (!consumer_sync(ctl, sgen, a.spin_lds)) return;
        for (int j = t; j < r.nrows; j += 64 * kConsumers) {
            float s = 0.f;
            for (int q = 0; q < upr; ++q) s += part[j * upr + q];
            a.y[(size_t)c * a.M + r.row0 + j] = s;
        }
        sgen += kConsumers;
        if (!consumer_sync(ctl, sgen, a.spin_lds)) return;
    }
}

// A plain many-wave GEMV for comparison: each wave owns 4 rows of one copy and
// keeps all their loads in flight at once.
__global__ void __launch_bounds__(256) gemv_direct_kernel(GemvArgs a) {
    const int lane = lane_id();
    const long wave = ((long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const long rows_total = (long)a.M * a.copies;
    const long r0 = wave * 4;
    if (r0 >= rows_total) return;
    const int upr = a.K / 512;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int cc0 = 0; cc0 < upr; cc0 += 4) {
        uint4 w[4][4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                long row = r0 + r;
                int cc = cc0 + q;
                if (row < rows_total && cc < upr)
                    w[r][q] = ld_nt16(a.A + ((size_t)row * a.K + (size_t)cc * 512 + lane * 8) * 2);
                else
                    w[r][q] = make_uint4(0, 0, 0, 0);
            }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            int cc = cc0 + q;
            if (cc < upr) {
                uint4 xv = *(const uint4*)(a.x + cc * 512 + lane * 8);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = dot8(w[r][q], xv, acc[r]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float s = wave_sum_to_lane63(acc[r]);
        long row = r0 + r;
        if (lane == 63 && row < rows_total) {
            long c = row / a.M, i = row % a.M;
            a.y[(size_t)c * a.M + i] = s;
        }
    }
}

// ---------------------------------------------------------- barrier probe --
// rounds x (publish my value, grid barrier, read every workgroup's value).
__global__ void __launch_bounds__(64, 1) barrier_probe_kernel(uint32_t* bar, uint32_t* status, float* vals,
                                                              int32_t* errors, int rounds) {
    const int wg = blockIdx.x, nwg = gridDim.x, lane = lane_id();
    int err = 0;
    for (int r = 1; r <= rounds; ++r) {
        float* slot = vals + (size_t)(r & 1) * nwg * 2;
        if (lane == 0) {
            slot[2 * wg] = (float)wg;
            slot[2 * wg + 1] = (float)r;
        }
        if (!grid_barrier_leader(bar, status, nwg, wg, (uint32_t)r, 1u << 22)) {
            if (lane == 0) atomicAdd(errors, 1000000);
            return;
        }
        for (int w = lane; w < nwg; w += 64)
            if (slot[2 * w] != (float)w || slot[2 * w + 1] != (float)r) ++err;
    }
    for (int off = 32; off; off >>= 1) err += shfl_xor_i(err, off);
    if (lane == 0 && err) atomicAdd(errors, err);
}

__global__ void empty_kernel() {}

// --------------------------------------------------------------- launch ---
hipError_t decode_kernel_setup() {
    hipError_t e = hipFuncSetAttribute((const void*)decode_kernel<64>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)decode_kernel<128>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            kLdsBytes);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute((const void*)gemv_ring_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                               kLdsBytes);
}

hipError_t launch_decode(const DecodeArgs* dev_args, int hd, int grid, hipStream_t s) {
    void* args[] = {&dev_args};
    const void* fn = hd == 64 ? (const void*)decode_kernel<64> : (const void*)decode_kernel<128>;
    return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kThreads), args, kLdsBytes, s);
}

hipError_t launch_gemv_ring(const GemvArgs& a, int grid, hipStream_t s) {
    GemvArgs copy = a;
    void* args[] = {&copy};
    return hipLaunchCooperativeKernel((const void*)gemv_ring_kernel, dim3(grid), dim3(kThreads), args,
                                      kLdsBytes, s);
}

hipError_t launch_gemv_direct(const GemvArgs& a, hipStream_t s) {
    long waves = ((long)a.M * a.copies + 3) / 4;
    long blocks = (waves + 3) / 4;
    hipLaunchKernelGGL(gemv_direct_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_barrier_probe(uint32_t* bar, uint32_t* status, float* vals, int32_t* errors, int rounds,
                                int grid, hipStream_t s) {
    void* args[] = {&bar, &status, &vals, &errors, &rounds};
    return hipLaunchCooperativeKernel((const void*)barrier_probe_kernel, dim3(grid), dim3(64), args, 0, s);
}

hipError_t launch_empty(hipStream_t s) {
    hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, s);
    return hipGetLastError();
}

}  // namespace kie

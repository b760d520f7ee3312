// kie_prefill.hip - batched prefill on the matrix cores (gfx950 MFMA).
//
// Decode at batch 1 is a matrix-vector product; a prompt of P tokens is not:
// its projections multiply P activation rows by every weight row, a dense
// contraction, so they run here as tiled GEMMs on v_mfma_f32_32x32x16_f16
// (fp16 x fp16 -> fp32). The pages measure decode, not prefill (paper-digest.app
// digest, "Core Mechanics": time-to-first-token is outside the metric); this
// path exists so that a prompt is not P sequential decode passes.
//
// The GEMMs read the decode kernel's repacked weights in place (each
// workgroup's rows of a phase are one contiguous slab; a row map finds row r),
// so RMSNorm gains are already folded in and QKV / gate-up rows come in the
// decode kernel's virtual order (rotary pairs adjacent, gate/up interleaved).
// Activations enter the GEMM as two fp16 terms (hi = fp16(a), lo =
// fp16(a - hi)), two MFMAs per step, so inputs keep about 22 significant bits
// as in decode. Everything else (norms, RoPE, the KV append, causal attention,
// SwiGLU, residual adds, the argmax) is plain VALU work on [rows][width]
// buffers, one small kernel each.
#include <hip/hip_runtime.h>

#include "kie_common.h"
#include "kie_device.h"
#include "kie_kernels.h"

namespace kie {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f16x_t __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------------ GEMM --
// Y[p][m] = sum_k A[p][k] * W(m)[k] for p < n rows of A (fp32, row stride
// lda) and m < M weight rows (fp16, K each) found by the row map.
constexpr int kTile = 64;          // rows of A and of W per workgroup
constexpr int kTk = 64;            // K per step
constexpr int kLdsStride = kTk + 8;   // halves per LDS row (16-byte rows; padding spreads the banks)

__device__ __forceinline__ const uint16_t* row_addr(const GemmRows& R, int m) {
    if (R.dense) return (const uint16_t*)(R.base + (size_t)m * R.K * 2);
    // owner workgroup of row m in the even split of M rows in groups of gran
    const int groups = R.M / R.gran, base = groups / kGrid, rem = groups % kGrid;
    const int g = m / R.gran;
    int w;
    if (g < rem * (base + 1)) w = g / (base + 1);
    else w = rem + (g - rem * (base + 1)) / base;
    const int row0 = (w * base + (w < rem ? w : rem)) * R.gran;
    return (const uint16_t*)(R.base + (size_t)R.slab[w] * kUnitBytes + (size_t)(m - row0) * R.K * 2);
}

// Quantised weights (fp8: rows in pairs, fp4: rows in fours): the byte
// address of row m's columns 0..7 in its group's first unit. Columns c of the
// row sit in unit c / 512 of the group, lane (c % 512) / 8, at byte 8 (fp8:
// second row of the pair) or 4 r (fp4: row r of the four) of the lane's 16.
__device__ __forceinline__ const uint8_t* row_qbase(const GemmRows& R, int m) {
    const int groups = R.M / R.gran, base = groups / kGrid, rem = groups % kGrid;
    const int g = m / R.gran;
    int w;
    if (g < rem * (base + 1)) w = g / (base + 1);
    else w = rem + (g - rem * (base + 1)) / base;
    const int row0 = (w * base + (w < rem ? w : rem)) * R.gran;
    const int rpu = R.wf == 2 ? 4 : 2, lr = m - row0;
    const size_t unit = (size_t)(lr / rpu) * (R.K / 512);
    return R.base + (size_t)R.slab[w] * kUnitBytes + unit * kUnitBytes + (lr % rpu) * (R.wf == 2 ? 4 : 8);
}

// 16 consecutive columns k0 .. k0 + 15 (k0 a multiple of 16) of a quantised
// row, converted exactly to fp16 (E4M3 and E2M1 values all are fp16 values).
template <int WF>
__device__ __forceinline__ void load_w_quant(const uint8_t* qb, int k0, uint4 (&b)[2]) {
    typedef float v2f __attribute__((ext_vector_type(2)));
    const uint8_t* p = qb + (size_t)(k0 / 512) * kUnitBytes + ((k0 % 512) / 8) * 16;
    float f[16];
    if constexpr (WF == 1) {
        const uint2 u0 = *(const uint2*)p, u1 = *(const uint2*)(p + 16);
        const uint32_t d[4] = {u0.x, u0.y, u1.x, u1.y};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)d[i], false);
            const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)d[i], true);
            f[4 * i] = lo.x;
            f[4 * i + 1] = lo.y;
            f[4 * i + 2] = hi.x;
            f[4 * i + 3] = hi.y;
        }
    } else {
        const uint32_t d[2] = {*(const uint32_t*)p, *(const uint32_t*)(p + 16)};
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const v2f b0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[i], 1.0f, 0);
            const v2f b1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[i], 1.0f, 1);
            const v2f b2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[i], 1.0f, 2);
            const v2f b3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[i], 1.0f, 3);
            f[8 * i] = b0.x;
            f[8 * i + 1] = b0.y;
            f[8 * i + 2] = b1.x;
            f[8 * i + 3] = b1.y;
            f[8 * i + 4] = b2.x;
            f[8 * i + 5] = b2.y;
            f[8 * i + 6] = b3.x;
            f[8 * i + 7] = b3.y;
        }
    }
    h8_t h0, h1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        h0[e] = (_Float16)f[e];
        h1[e] = (_Float16)f[8 + e];
    }
    b[0] = __builtin_bit_cast(uint4, h0);
    b[1] = __builtin_bit_cast(uint4, h1);
}

// One step's share of a thread: 16 consecutive k of one row of A (fp32) and
// of one row of W (fp16). Thread t loads row t / 4 at k offset 16 (t % 4).
// Rows past n (A) or M (W) load the last valid row instead: they only feed
// outputs that are not stored, and the loads need no branch, which keeps the
// compiler's waits exact across the pipelined steps.
struct GemmStage {
    float a[16];
    uint4 b[2];
};

template <int WF>
__device__ __forceinline__ void gemm_load(GemmStage& st, const float* ap, const void* bp, int k0, int kq0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 u = *(const float4*)(ap + k0 + 4 * q);
        st.a[4 * q] = u.x;
        st.a[4 * q + 1] = u.y;
        st.a[4 * q + 2] = u.z;
        st.a[4 * q + 3] = u.w;
    }
    if constexpr (WF == 0) {
#pragma unroll
        for (int q = 0; q < 2; ++q) st.b[q] = *(const uint4*)((const uint16_t*)bp + k0 + 8 * q);
    } else {
        load_w_quant<WF>((const uint8_t*)bp, k0 + kq0, st.b);
    }
}

// Three K steps are in flight per thread (registers) while a fourth is
// multiplied from LDS: a step's 24 KiB per workgroup take about one memory
// latency to arrive, so one step in flight left the matrix cores idle most
// of the time. Loads past the last step re-read the last step (in bounds,
// unused), so every wait the compiler places covers exactly the step needed.
template <int WF>
__global__ void __launch_bounds__(256) gemm_mfma_kernel(const float* __restrict__ A, int lda, int n, GemmRows R,
                                                        float* __restrict__ Y, int ldy) {
    __shared__ __attribute__((aligned(16))) _Float16 ahi[kTile * kLdsStride];
    __shared__ __attribute__((aligned(16))) _Float16 alo[kTile * kLdsStride];
    __shared__ __attribute__((aligned(16))) _Float16 bt[kTile * kLdsStride];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m0 = blockIdx.x * kTile, p0 = blockIdx.y * kTile;
    const int wr = (wave >> 1) * 32, wc = (wave & 1) * 32;   // this wave's 32 x 32 sub-tile
    const int lr = tid >> 2, lk = (tid & 3) * 16;
    const int pa = p0 + lr < n ? p0 + lr : n - 1, mb = m0 + lr < R.M ? m0 + lr : R.M - 1;
    const float* ap = A + (size_t)pa * lda + lk;
    // fp16: this thread's 16 columns start at bp; quantised: the row's group
    // base (the column offset lk is added per step)
    const void* bp;
    if constexpr (WF == 0) bp = row_addr(R, mb) + lk;
    else bp = row_qbase(R, mb);
    const int kq0 = WF == 0 ? 0 : lk;
    const int klast = R.K - kTk;
    f16x_t acc = {};
    auto stage_in = [&](const GemmStage& st) {
        __syncthreads();   // the previous step's LDS reads are done
        h8_t h[2], l[2];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const _Float16 x = (_Float16)st.a[e];
            h[e >> 3][e & 7] = x;
            l[e >> 3][e & 7] = (_Float16)(st.a[e] - (float)x);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            *(h8_t*)&ahi[lr * kLdsStride + lk + 8 * q] = h[q];
            *(h8_t*)&alo[lr * kLdsStride + lk + 8 * q] = l[q];
            *(uint4*)&bt[lr * kLdsStride + lk + 8 * q] = st.b[q];
        }
        __syncthreads();
    };
    auto multiply = [&]() {
#pragma unroll
        for (int kk = 0; kk < kTk; kk += 16) {
            // v_mfma_f32_32x32x16_f16: A[i][k] lane i + 32 (k / 8) holds k % 8;
            // B[k][j] lane j + 32 (k / 8)
            const int kq = kk + 8 * (lane >> 5);
            const h8_t a_h = *(const h8_t*)&ahi[(wr + (lane & 31)) * kLdsStride + kq];
            const h8_t a_l = *(const h8_t*)&alo[(wr + (lane & 31)) * kLdsStride + kq];
            const h8_t b = *(const h8_t*)&bt[(wc + (lane & 31)) * kLdsStride + kq];
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_h, b, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_l, b, acc, 0, 0, 0);
        }
    };
    auto kat = [&](int k) { return k < klast ? k : klast; };
    GemmStage s0, s1, s2;
    gemm_load<WF>(s0, ap, bp, 0, kq0);
    gemm_load<WF>(s1, ap, bp, kat(kTk), kq0);
    gemm_load<WF>(s2, ap, bp, kat(2 * kTk), kq0);
    for (int k0 = 0; k0 < R.K; k0 += 3 * kTk) {
        stage_in(s0);
        gemm_load<WF>(s0, ap, bp, kat(k0 + 3 * kTk), kq0);
        multiply();
        if (k0 + kTk >= R.K) break;
        stage_in(s1);
        gemm_load<WF>(s1, ap, bp, kat(k0 + 4 * kTk), kq0);
        multiply();
        if (k0 + 2 * kTk >= R.K) break;
        stage_in(s2);
        gemm_load<WF>(s2, ap, bp, kat(k0 + 5 * kTk), kq0);
        multiply();
    }
    // D[i][j]: lane j + 32 ((i / 4) % 2), register (i % 4) + 4 (i / 8)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int i = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3), j = lane & 31;
        const int p = p0 + wr + i, m = m0 + wc + j;
        if (p < n && m < R.M) Y[(size_t)p * ldy + m] = WF == 0 ? acc[v] : acc[v] * R.scales[m];
    }
}

hipError_t launch_gemm_mfma(const float* A, int lda, int n, const GemmRows& R, float* Y, int ldy, hipStream_t s) {
    if (R.K % kTk || lda % 4 || n < 1 || R.M < 1) return hipErrorInvalidValue;
    dim3 grid((unsigned)ceil_div(R.M, kTile), (unsigned)ceil_div(n, kTile));
    if (R.wf != 0 && (R.dense || !R.scales || R.K % 512 || R.gran % (R.wf == 2 ? 4 : 2)))
        return hipErrorInvalidValue;
    if (R.wf == 1) hipLaunchKernelGGL(gemm_mfma_kernel<1>, grid, dim3(256), 0, s, A, lda, n, R, Y, ldy);
    else if (R.wf == 2) hipLaunchKernelGGL(gemm_mfma_kernel<2>, grid, dim3(256), 0, s, A, lda, n, R, Y, ldy);
    else hipLaunchKernelGGL(gemm_mfma_kernel<0>, grid, dim3(256), 0, s, A, lda, n, R, Y, ldy);
    return hipGetLastError();
}

// ----------------------------------------------------------- row kernels --
// X[t][:] = E[tok[t]] (fp16 -> fp32)
__global__ void pf_embed_kernel(const uint16_t* __restrict__ E, const int32_t* __restrict__ tok, int d,
                                float* __restrict__ X) {
    const int t = blockIdx.x;
    const uint16_t* e = E + (size_t)tok[t] * d;
    for (int i = threadIdx.x; i < d; i += blockDim.x) X[(size_t)t * d + i] = h2f_bits(e[i]);
}

// A[t][:] = X[t][:] / sqrt(mean(X[t]^2) + eps) (the gains are in the weights)
__global__ void __launch_bounds__(256) pf_rmsnorm_kernel(const float* __restrict__ X, int d, float eps,
                                                         float* __restrict__ Aout) {
    __shared__ float part[4];
    const int t = blockIdx.x;
    const float* x = X + (size_t)t * d;
    float ss = 0.f;
    for (int i = threadIdx.x; i < d; i += blockDim.x) ss += x[i] * x[i];
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float s = 1.0f / sqrtf((part[0] + part[1] + part[2] + part[3]) / (float)d + eps);
    for (int i = threadIdx.x; i < d; i += blockDim.x) Aout[(size_t)t * d + i] = x[i] * s;
}

// X += Y (rows of d)
__global__ void pf_residual_kernel(float* __restrict__ X, const float* __restrict__ Y, int d, int ldy) {
    const int t = blockIdx.x;
    for (int i = threadIdx.x; i < d; i += blockDim.x) X[(size_t)t * d + i] += Y[(size_t)t * ldy + i];
}

// A[t][m] = silu(Y[t][2m]) * Y[t][2m+1]: gate/up rows come interleaved
__global__ void pf_swiglu_kernel(const float* __restrict__ Y, int F, int ldy, float* __restrict__ Aout) {
    const int t = blockIdx.x;
    for (int m = threadIdx.x; m < F; m += blockDim.x) {
        const float g = Y[(size_t)t * ldy + 2 * m], u = Y[(size_t)t * ldy + 2 * m + 1];
        Aout[(size_t)t * F + m] = g / (1.0f + __expf(-g)) * u;
    }
}

// QKV rows of token t at position pos0 + t: rotate the rotary pairs of q and k
// (virtual rows 2i, 2i+1 of a head are elements i, i + hd/2) with the table
// row of that position; q to Q[t][H*hd] (natural order), k and v (fp16) to
// the cache. One thread per pair of virtual rows.
__global__ void pf_qkv_kernel(const float* __restrict__ Y, int ldy, int pos0, int layer, Dims D,
                              const float* __restrict__ rope, float* __restrict__ Q, uint16_t* __restrict__ kc,
                              uint16_t* __restrict__ vc) {
    const int t = blockIdx.x, hd = D.hd, qd = D.H * hd, kd = D.Hkv * hd;
    const int pos = pos0 + t;
    const float* y = Y + (size_t)t * ldy;
    for (int pr = threadIdx.x; pr < (qd + 2 * kd) / 2; pr += blockDim.x) {
        const int r = 2 * pr;
        const float y0 = y[r], y1 = y[r + 1];
        if (r < qd + kd) {
            const bool isq = r < qd;
            const int rr = isq ? r : r - qd, head = rr / hd, i = (rr % hd) >> 1;
            const float c = rope[((size_t)pos * (hd / 2) + i) * 2], s = rope[((size_t)pos * (hd / 2) + i) * 2 + 1];
            const float a = y0 * c - y1 * s, b = y1 * c + y0 * s;
            if (isq) {
                Q[(size_t)t * qd + head * hd + i] = a;
                Q[(size_t)t * qd + head * hd + i + hd / 2] = b;
            } else {
                uint16_t* kp = kc + (((size_t)layer * D.Hkv + head) * D.max_seq + pos) * hd;
                kp[i] = f2h_bits(a);
                kp[i + hd / 2] = f2h_bits(b);
            }
        } else {
            const int vi = r - qd - kd, g = vi / hd, dd = vi % hd;
            uint16_t* vp = vc + (((size_t)layer * D.Hkv + g) * D.max_seq + pos) * hd;
            vp[dd] = f2h_bits(y0);
            vp[dd + 1] = f2h_bits(y1);
        }
    }
}

// Causal attention of token t (position pos0 + t) for query head j (one wave):
// softmax over positions u <= pos of q . K[u] / sqrt(hd), times V[u], with
// the keys and values read back from the cache (fp16, as decode reads them).
// Lanes take 64 positions at a time for the scores (online softmax across
// blocks), then the head dimensions for the weighted sum.
template <int HD>
__global__ void __launch_bounds__(64) pf_attention_kernel(const float* __restrict__ Q, int pos0, int layer, Dims D,
                                                          const uint16_t* __restrict__ kc,
                                                          const uint16_t* __restrict__ vc, float* __restrict__ O) {
    __shared__ float q[HD];
    __shared__ float pr[64];
    const int t = blockIdx.x, j = blockIdx.y, lane = threadIdx.x;
    const int g = j / (D.H / D.Hkv), c = pos0 + t + 1;
    const float scale = 1.0f / sqrtf((float)HD);
    for (int i = lane; i < HD; i += 64) q[i] = Q[(size_t)t * D.H * HD + j * HD + i] * scale;
    __syncthreads();
    const uint16_t* Kb = kc + ((size_t)layer * D.Hkv + g) * D.max_seq * HD;
    const uint16_t* Vb = vc + ((size_t)layer * D.Hkv + g) * D.max_seq * HD;
    constexpr int DPL = HD / 64;   // head dimensions per lane in the weighted sum
    float m = -3.0e38f, l = 0.f, o[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] = 0.f;
    for (int u0 = 0; u0 < c; u0 += 64) {
        const int u = u0 + lane;
        float sc = -3.0e38f;
        if (u < c) {
            const uint16_t* kr = Kb + (size_t)u * HD;
            float acc = 0.f;
            for (int i = 0; i < HD; i += 8) {
                const uint4 w = *(const uint4*)(kr + i);
                const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc += h2f_bits((uint16_t)ww[e]) * q[i + 2 * e];
                    acc += h2f_bits((uint16_t)(ww[e] >> 16)) * q[i + 2 * e + 1];
                }
            }
            sc = acc;
        }
        const float mx = fmaxf(m, wave_max(sc));
        const float p = u < c ? __expf(sc - mx) : 0.f;
        const float cr = __expf(m - mx);
        l = l * cr + wave_sum(p);
        __syncthreads();
        pr[lane] = p;
        __syncthreads();
        const int nb = (c - u0 < 64) ? c - u0 : 64;
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[e] *= cr;
        for (int k = 0; k < nb; ++k) {
            const float pk = pr[k];
            const uint16_t* vr = Vb + (size_t)(u0 + k) * HD;
#pragma unroll
            for (int e = 0; e < DPL; ++e) o[e] += pk * h2f_bits(vr[lane + 64 * e]);
        }
        m = mx;
    }
#pragma unroll
    for (int e = 0; e < DPL; ++e) O[(size_t)t * D.H * HD + j * HD + lane + 64 * e] = o[e] / l;
}

// Index of the largest of n values (ties to the lowest index); one workgroup.
__global__ void __launch_bounds__(256) pf_argmax_kernel(const float* __restrict__ y, int n, int32_t* out) {
    __shared__ float bv[4];
    __shared__ int bi[4];
    float v = -3.4e38f;
    int idx = 0x7fffffff;
    for (int i = threadIdx.x; i < n; i += blockDim.x)
        if (y[i] > v || (y[i] == v && i < idx)) { v = y[i]; idx = i; }
    wave_argmax(v, idx);
    if ((threadIdx.x & 63) == 0) { bv[threadIdx.x >> 6] = v; bi[threadIdx.x >> 6] = idx; }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < 4; ++w)
            if (bv[w] > v || (bv[w] == v && bi[w] < idx)) { v = bv[w]; idx = bi[w]; }
        out[0] = (idx >= 0 && idx < n) ? idx : 0;   // out of range only with NaN logits
    }
}

hipError_t launch_prefill_rows(int op, const PrefillRowArgs& r, hipStream_t s) {
    const dim3 rows((unsigned)r.n);
    switch (op) {
    case PF_EMBED: hipLaunchKernelGGL(pf_embed_kernel, rows, dim3(256), 0, s, r.emb, r.tok, r.D.d, r.X); break;
    case PF_RMSNORM: hipLaunchKernelGGL(pf_rmsnorm_kernel, rows, dim3(256), 0, s, r.X, r.D.d, r.eps, r.A); break;
    case PF_RESIDUAL: hipLaunchKernelGGL(pf_residual_kernel, rows, dim3(256), 0, s, r.X, r.Y, r.D.d, r.ldy); break;
    case PF_SWIGLU: hipLaunchKernelGGL(pf_swiglu_kernel, rows, dim3(256), 0, s, r.Y, r.D.F, r.ldy, r.A); break;
    case PF_QKV:
        hipLaunchKernelGGL(pf_qkv_kernel, rows, dim3(256), 0, s, r.Y, r.ldy, r.pos0, r.layer, r.D, r.rope, r.Q,
                           r.kc, r.vc);
        break;
    case PF_ATTN:
        if (r.D.hd == 64)
            hipLaunchKernelGGL(pf_attention_kernel<64>, dim3((unsigned)r.n, (unsigned)r.D.H), dim3(64), 0, s, r.Q,
                               r.pos0, r.layer, r.D, r.kc, r.vc, r.A);
        else
            hipLaunchKernelGGL(pf_attention_kernel<128>, dim3((unsigned)r.n, (unsigned)r.D.H), dim3(64), 0, s, r.Q,
                               r.pos0, r.layer, r.D, r.kc, r.vc, r.A);
        break;
    case PF_ARGMAX: hipLaunchKernelGGL(pf_argmax_kernel, dim3(1), dim3(256), 0, s, r.Y, r.D.V, r.out); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kie

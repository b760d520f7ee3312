// kie_probes.hip - measurement kernels behind the kie_*_probe entry points:
// the weight-streaming GEMV on its own, a plain GEMV for comparison, the
// inter-workgroup exchange (fenced grid barrier vs. flagged words), and an
// empty kernel for the launch cost. None of them is on the decode path.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kie_common.h"
#include "kie_device.h"
#include "kie_kernels.h"

namespace kie {

// Persistent GEMV with the decode kernel's weight streaming: wave gw of the
// grid streams the contiguous unit range [U gw / W, U (gw + 1) / W) of the
// row-major matrices (U units of 512 fp16 in all, W waves), through its own
// LDS ring of kNS batches of kNB units filled by LDS DMA; it consumes the
// oldest batch after vmcnt((kNS-1)*kNB) and refills it at once. Unit
// positions (row, segment) advance by counting, without divisions per unit.
// A row's partial sum is added to y[row] with a no-return atomic when the
// row or the wave's range ends (y is zeroed by the caller); a row is split
// over at most a few waves. x (K <= 8192) is staged in LDS; A has row stride
// lda elements.
__global__ void __launch_bounds__(512, 1) gemv_stream_kernel(GemvArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t ring[8 * kNS * kBatchBytes];
    __shared__ __attribute__((aligned(16))) uint16_t xs[kMaxInput];
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = lane_id();
    const long nwaves = (long)gridDim.x * 8;
    const long gw = (long)blockIdx.x * 8 + w;
    for (int i = threadIdx.x; i < a.K / 8; i += blockDim.x)
        lds_st16((KIE_LDS void*)(xs + 8 * i), *(const uint4*)(a.x + 8 * i));
    __syncthreads();
    const int upr = a.K / kUnitHalves;
    const long U = (long)a.M * a.copies * upr;
    const long u0 = U * gw / nwaves;
    const int n = (int)(U * (gw + 1) / nwaves - u0);   // units of this wave
    const uint32_t ring0 = lds_addr_of((KIE_LDS void*)ring) + (uint32_t)(w * kNS * kBatchBytes);
    const uint8_t* idle = a.idle + lane * 16;
    // fill cursor: next unit to load, as (row, segment) and its row's address
    long frow = u0 / upr;
    int fseg = (int)(u0 - frow * upr);
    const uint8_t* fbase = a.A + (size_t)frow * a.lda * 2 + lane * 16;
    int iu = 0;
    auto fill = [&](uint32_t dst) {
        const int c = (n - iu < kNB) ? n - iu : kNB;
#pragma unroll
        for (int s = 0; s < kNB; ++s) {
            if (s < c) {
                dma_unit(fbase + (size_t)fseg * kUnitBytes, dst + s * kUnitBytes);
                if (++fseg == upr) {
                    fseg = 0;
                    fbase += (size_t)a.lda * 2;
                }
            } else {
                dma_unit(idle + (size_t)s * kUnitBytes, dst + s * kUnitBytes);
            }
        }
        iu += c;
        return c;
    };
    int sn[kNS];
#pragma unroll
    for (int i = 0; i < kNS; ++i) sn[i] = fill(ring0 + i * kBatchBytes);
    // consume cursor
    long crow = u0 / upr;
    int cseg = (int)(u0 - crow * upr);
    int left = n;
    int head = 0;
    float acc = 0.f;
    while (sn[0] > 0) {
        const uint32_t at = ring0 + head * kBatchBytes;
        wait_vm<(kNS - 1) * kNB>();
        const KIE_LDS uint8_t* wb = (const KIE_LDS uint8_t*)(uintptr_t)at + lane * 16;
        // every LDS read of the batch first, then the products
        uint4 wv[kNB], xv[kNB];
        {
            int sg = cseg;
#pragma unroll
            for (int s = 0; s < kNB; ++s) {
                if (s < sn[0]) {
                    wv[s] = lds_ld16(wb + s * kUnitBytes);
                    xv[s] = lds_ld16((const KIE_LDS void*)(xs + sg * kUnitHalves + lane * 8));
                    if (++sg == upr) sg = 0;
                }
            }
        }
#pragma unroll
        for (int s = 0; s < kNB; ++s) {
            if (s < sn[0]) {
                acc = dot8(wv[s], xv[s], acc);
                --left;
                if (cseg == upr - 1 || left == 0) {
                    const float r = wave_sum_to_lane63(acc);
                    // a no-return atomic: a load here would make the compiler wait for
                    // every LDS DMA in flight
                    if (lane == 63)
                        __hip_atomic_fetch_add(gptr(a.y + crow), r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    acc = 0.f;
                }
                if (++cseg == upr) {
                    cseg = 0;
                    ++crow;
                }
            }
        }
        wait_lgkm0();
        const int c = fill(at);
#pragma unroll
        for (int i = 0; i + 1 < kNS; ++i) sn[i] = sn[i + 1];
        sn[kNS - 1] = c;
        head = (head + 1 == kNS) ? 0 : head + 1;
    }
    wait_vm0();
}

// A plain many-wave GEMV for comparison: each wave owns 4 rows and keeps all
// loads of a 4-row x 4-unit block in flight at once.
__global__ void __launch_bounds__(256) gemv_direct_kernel(GemvArgs a) {
    const int lane = lane_id();
    const long wave = ((long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const long rows_total = (long)a.M * a.copies;
    const long r0 = wave * 4;
    if (r0 >= rows_total) return;
    const int upr = a.K / kUnitHalves;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int cc0 = 0; cc0 < upr; cc0 += 4) {
        uint4 wv[4][4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const long row = r0 + r;
                const int cc = cc0 + q;
                if (row < rows_total && cc < upr)
                    wv[r][q] = ld_nt16(a.A + ((size_t)row * a.lda + (size_t)cc * kUnitHalves + lane * 8) * 2);
                else
                    wv[r][q] = make_uint4(0, 0, 0, 0);
            }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int cc = cc0 + q;
            if (cc < upr) {
                const uint4 xv = *(const uint4*)(a.x + cc * kUnitHalves + lane * 8);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = dot8(wv[r][q], xv, acc[r]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float s = wave_sum_to_lane63(acc[r]);
        const long row = r0 + r;
        if (lane == 63 && row < rows_total) a.y[row] = a.accumulate ? a.y[row] + s : s;
    }
}

// ------------------------------------------------------------ exchange probe


// XCD-aware barrier state in the probe's scratch (bytes from the scratch base).
constexpr int kXcdMax = 16;
constexpr size_t kHierCnt = 36864;              // u32 per XCD, each on its own 256 bytes
constexpr size_t kHierGen = kHierCnt + 4096;    // u32 per XCD, own 256 bytes
constexpr size_t kHierFlag = kHierGen + 4096;   // u32 per XCD, own 64-byte line (read across XCDs)
constexpr size_t kHierMap = kHierFlag + 1024;   // u64 [grid]: flagged XCD id of every workgroup
constexpr size_t kHierEnd = kHierMap + 8 * 1024;
static_assert(kHierEnd <= 65536, "the XCD-aware barrier's state fits the probe's 64 KiB scratch");

// variant 0: per round, publish one value with a plain store, fenced grid
// barrier, read every workgroup's value.
// variant 1: per round, publish 5 flagged words and gather all 5 x grid words
// (buffers alternate by round parity, so a workgroup that runs a round ahead
// cannot overwrite words another one is still reading).
// variant 2: the XCD-aware barrier. Per round every workgroup stores its
// value (device scope, so it reaches memory), waits for the store, and
// arrives at its own XCD's counter (an atomic add); the XCD's
// lowest-numbered workgroup waits on that counter for all of its XCD's
// workgroups, publishes one flag per XCD, waits for the other XCDs' flags,
// and releases its XCD through one word; then every workgroup reads all
// values. Each workgroup polls one word (its XCD's release) instead of one
// per workgroup, and only the 8 XCD leaders poll across XCDs. Every poll is a
// device-scope load: a workgroup-scope load may be served from the compute
// unit's own L1 and never see another unit's update. The placement of
// workgroups on XCDs is read from the hardware (XCC_ID) and exchanged once
// before the first round.
__global__ void __launch_bounds__(64, 1) barrier_probe_kernel(int variant, uint64_t* words, uint32_t* status,
                                                              int32_t* errors, int rounds) {
    const int wg = blockIdx.x, nwg = gridDim.x, lane = lane_id();
    int err = 0;
    // XCD-aware barrier: who shares this workgroup's XCD, and who leads it
    uint8_t* base = (uint8_t*)words;
    uint32_t* hcnt = nullptr;
    uint32_t* hgen = nullptr;
    uint32_t* hflag = (uint32_t*)(base + kHierFlag);
    int members = 0, leader = 0, xcd = 0;
    uint32_t xcd_mask = 0;
    if (variant == 2) {
        xcd = xcc_id();
        uint64_t* map = (uint64_t*)(base + kHierMap);
        if (lane == 0) fw_store(map + wg, (uint32_t)xcd, 1u);
        int mem = 0, lead = nwg;
        uint32_t mask = 0;
        const int e = fw_gather(map, nwg, 1u, 1u << 22, status, [&](int i, uint32_t v) {
            mask |= 1u << (v & 15);
            if ((int)v == xcd) {
                ++mem;
                lead = i < lead ? i : lead;
            }
        });
        for (int off = 32; off; off >>= 1) {
            mem += shfl_xor_i(mem, off);
            const int o = shfl_xor_i(lead, off);
            lead = o < lead ? o : lead;
            mask |= (uint32_t)shfl_xor_i((int)mask, off);
        }
        if (e) {
            if (lane == 0) atomicAdd(errors, 1000000);
            return;
        }
        members = mem;
        leader = lead;
        xcd_mask = mask;
        hcnt = (uint32_t*)(base + kHierCnt + 256 * xcd);
        hgen = (uint32_t*)(base + kHierGen + 256 * xcd);
    }
    for (int r = 1; r <= rounds; ++r) {
        if (variant == 2) {
            uint32_t* vals = (uint32_t*)words + (size_t)(r & 1) * nwg;
            bool ok = true;
            uint32_t spins = 0;
            if (lane == 0) {
                dev_store32(vals + wg, (uint32_t)(wg * 4096 + r));
                wait_vm0();   // the value is in memory before this workgroup arrives
                __hip_atomic_fetch_add(gptr(hcnt), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            if (wg == leader) {
                // one lane waits for the XCD's arrivals, then lane x watches XCD x's flag
                if (lane == 0) {
                    while (dev_load32(hcnt) < (uint32_t)(members * r)) {
                        if (++spins > (1u << 22)) { ok = false; break; }
                    }
                    if (ok) dev_store32(hflag + 16 * xcd, (uint32_t)r);
                }
                ok = __builtin_amdgcn_readfirstlane(ok ? 1 : 0) != 0;
                const bool mine = lane < kXcdMax && (xcd_mask & (1u << lane));
                while (ok) {
                    const bool here = !mine || (int)(dev_load32(hflag + 16 * (lane & (kXcdMax - 1))) - (uint32_t)r) >= 0;
                    if (__builtin_amdgcn_ballot_w64(!here) == 0) break;
                    if (++spins > (1u << 22)) ok = false;
                }
                if (ok && lane == 0) dev_store32(hgen, (uint32_t)r);
            } else if (lane == 0) {
                while ((int)(dev_load32(hgen) - (uint32_t)r) < 0) {
                    if (++spins > (1u << 22)) { ok = false; break; }
                }
            }
            if (!ok && lane == 0) dev_store32(status, (uint32_t)kStatusTimeout);
            if (__builtin_amdgcn_readfirstlane(ok ? 1 : 0) == 0) {
                if (lane == 0) atomicAdd(errors, 1000000);
                return;
            }
            for (int i = lane; i < nwg; i += 64)
                if (dev_load32(vals + i) != (uint32_t)(i * 4096 + r)) ++err;
        } else if (variant == 0) {
            uint32_t* bar = (uint32_t*)words;
            uint32_t* vals = (uint32_t*)(words + nwg) + (size_t)(r & 1) * nwg;
            if (lane == 0) vals[wg] = (uint32_t)(wg * 4096 + r);
            if (!grid_barrier_fenced(bar, status, nwg, wg, (uint32_t)r, 1u << 22)) {
                if (lane == 0) atomicAdd(errors, 1000000);
                return;
            }
            for (int i = lane; i < nwg; i += 64)
                if (vals[i] != (uint32_t)(i * 4096 + r)) ++err;
        } else {
            uint64_t* buf = words + (size_t)(r & 1) * 5 * nwg;
            if (lane < 5) fw_store(buf + 5 * wg + lane, (uint32_t)((wg * 8 + lane) ^ r), (uint32_t)r);
            const int e = fw_gather(buf, 5 * nwg, (uint32_t)r, 1u << 22, status, [&](int i, uint32_t v) {
                if (v != (uint32_t)(((i / 5) * 8 + i % 5) ^ r)) ++err;
            });
            if (e) {
                if (lane == 0) {
                    if (e == 1)
                        __hip_atomic_store(status, (uint32_t)kStatusTimeout, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    atomicAdd(errors, 1000000);
                }
                return;
            }
        }
    }
    for (int off = 32; off; off >>= 1) err += shfl_xor_i(err, off);
    if (lane == 0 && err) atomicAdd(errors, err);
}

__global__ void empty_kernel() {}

// Every E4M3 code converted by the device's fp8 conversion (the one the fp8
// GEMVs use): out[c] = value of code c, one workgroup of 64 lanes, 4 codes
// per lane.
__global__ void __launch_bounds__(64, 1) e4m3_table_kernel(float* out) {
    typedef float v2f __attribute__((ext_vector_type(2)));
    const int l = threadIdx.x;
    const uint32_t w = (uint32_t)(4 * l) | ((uint32_t)(4 * l + 1) << 8) | ((uint32_t)(4 * l + 2) << 16) |
                       ((uint32_t)(4 * l + 3) << 24);
    const v2f a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false), b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    out[4 * l] = a.x;
    out[4 * l + 1] = a.y;
    out[4 * l + 2] = b.x;
    out[4 * l + 3] = b.y;
}

hipError_t launch_e4m3_table(float* out, hipStream_t s) {
    hipLaunchKernelGGL(e4m3_table_kernel, dim3(1), dim3(64), 0, s, out);
    return hipGetLastError();
}

// The device's E2M1 conversion (v_cvt_scalef32_pk_f32_fp4, scale 1) of
// eight words; word l holds in byte b the codes (2l + b) % 16 (low nibble)
// and (2l + b + 8) % 16 (high nibble).
__global__ void __launch_bounds__(64, 1) e2m1_table_kernel(float* out) {
    typedef float v2f __attribute__((ext_vector_type(2)));
    const int l = threadIdx.x;
    if (l >= 8) return;
    uint32_t w = 0;
    for (int b = 0; b < 4; ++b) w |= (uint32_t)(((2 * l + b) % 16) | (((2 * l + b + 8) % 16) << 4)) << (8 * b);
    const v2f p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const v2f p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const v2f p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const v2f p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    float* o = out + 8 * l;
    o[0] = p0.x;
    o[1] = p0.y;
    o[2] = p1.x;
    o[3] = p1.y;
    o[4] = p2.x;
    o[5] = p2.y;
    o[6] = p3.x;
    o[7] = p3.y;
}

hipError_t launch_e2m1_table(float* out, hipStream_t s) {
    hipLaunchKernelGGL(e2m1_table_kernel, dim3(1), dim3(64), 0, s, out);
    return hipGetLastError();
}

// The XCD every workgroup of a grid-sized launch runs on.
__global__ void __launch_bounds__(64, 1) xcd_map_kernel(int32_t* out) {
    if (threadIdx.x == 0) out[blockIdx.x] = xcc_id();
}

hipError_t launch_xcd_map(int32_t* out, int grid, hipStream_t s) {
    void* args[] = {&out};
    return hipLaunchCooperativeKernel((const void*)xcd_map_kernel, dim3(grid), dim3(64), args, 0, s);
}

// Zero n 32-bit words (a kernel, so that a caller may capture it in a graph;
// no hipMemsetAsync).
__global__ void fill_zero_kernel(uint32_t* p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// ------------------------------------------- scratch for the no-alloc probe
// The exchange probe's words, status and error count for callers that cannot
// allocate device memory: one array per GPU, held until the process ends. In
// host code `scratch` names a host-side stand-in, not the device array: its
// device address comes from hipGetSymbolAddress, once per device, and only
// that address is ever handed to a kernel.
constexpr size_t kNoAllocScratchBytes = 65536;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
static void* g_scratch_dev[kMaxDevices];
static std::mutex g_scratch_mu;

size_t noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

hipError_t noalloc_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with `dev` current
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return hipSuccess;
}

hipError_t launch_fill_zero(uint32_t* p, int n, hipStream_t s) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3(64), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_gemv_stream(const GemvArgs& a, int grid, hipStream_t s) {
    GemvArgs copy = a;
    void* args[] = {&copy};
    return hipLaunchCooperativeKernel((const void*)gemv_stream_kernel, dim3(grid), dim3(512), args, 0, s);
}

hipError_t launch_gemv_direct(const GemvArgs& a, hipStream_t s) {
    const long waves = ((long)a.M * a.copies + 3) / 4;
    const long blocks = (waves + 3) / 4;
    hipLaunchKernelGGL(gemv_direct_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_barrier_probe(int variant, uint64_t* words, uint32_t* status, int32_t* errors, int rounds,
                                int grid, hipStream_t s) {
    void* args[] = {&variant, &words, &status, &errors, &rounds};
    return hipLaunchCooperativeKernel((const void*)barrier_probe_kernel, dim3(grid), dim3(64), args, 0, s);
}

hipError_t launch_empty(hipStream_t s) {
    hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, s);
    return hipGetLastError();
}

}  // namespace kie

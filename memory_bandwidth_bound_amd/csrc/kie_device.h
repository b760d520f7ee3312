// kie_device.h - gfx950 device primitives of the persistent decode kernel.
//
//  * v_dot2 fp16 x fp16 -> fp32 inner products and wave-wide DPP reductions:
//    batch-1 projections are matrix-vector products done on the vector ALU,
//    not on matrix cores (news.creeta.com monokernel article, "Inside the
//    monokernel": VDOT/SDOT instead of matrix cores at batch 1).
//  * Non-temporal 16-byte weight loads into registers (same section: weights
//    are streamed non-temporally rather than through the caches).
//  * Flagged words for data exchange between workgroups: a 64-bit word holds
//    a 32-bit payload and the 32-bit id of the phase that wrote it; it is
//    stored and loaded as one device-scope (sc1) access, so a reader that sees
//    the expected id also sees the payload, with no cache flush or grid
//    barrier. This plays the part of the pages' publish buffer ("Inside the
//    monokernel": a 2,048-byte publish buffer across 256 CUs).
//  * The classic fenced grid barrier, kept for the barrier probe.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kie_common.h"

namespace kie {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Pointers into LDS carry address space 3 explicitly so that every access
// through them is a ds_* instruction (a generic pointer would become flat_*).
#define KIE_LDS __attribute__((address_space(3)))
// Pointers read from the argument block are generic; casting them to the
// global address space makes every access a global_* instruction (a flat_*
// access would also count against lgkmcnt, which the LDS waits rely on).
#define KIE_GLOBAL __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ KIE_GLOBAL T* gptr(T* p) {
    return (KIE_GLOBAL T*)p;
}

constexpr int kStatusTimeout = 1;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ------------------------------------------------------------- loads -------
// 16-byte non-temporal global load.
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
    u32x4_t v = __builtin_nontemporal_load((const KIE_GLOBAL u32x4_t*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// One streaming unit (1 KiB: 16 bytes per lane, lane l's bytes at
// gsrc_lane = base + 16 l) straight from global memory into LDS at byte
// address lds_addr + 16 l, non-temporally and without passing through
// registers. The load is written in assembly, so the compiler neither tracks
// it nor inserts waits for it: the caller waits with wait_vm<N>() (vmcnt
// counts these loads in issue order) before reading the LDS bytes, and
// makes sure its own earlier LDS reads of the target have returned before
// issuing the next load into it.
__device__ __forceinline__ void dma_unit(const void* gsrc_lane, uint32_t lds_addr) {
    uint32_t saved;   // m0 is reserved by the compiler: put its value back
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off nt\n\t"
        "s_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(gsrc_lane), "s"(lds_addr)
        : "memory");
}
// Four units with one m0: unit s goes from p_s + 1024 s (+ 16 lane) to LDS
// lds_addr + 1024 s (+ 16 lane) - the instruction offset applies to both
// addresses. Same rules as dma_unit.
__device__ __forceinline__ void dma_unit4(const void* p0, const void* p1, const void* p2, const void* p3,
                                          uint32_t lds_addr) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %5\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off nt\n\t"
        "global_load_lds_dwordx4 %2, off offset:1024 nt\n\t"
        "global_load_lds_dwordx4 %3, off offset:2048 nt\n\t"
        "global_load_lds_dwordx4 %4, off offset:3072 nt\n\t"
        "s_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(p0), "v"(p1), "v"(p2), "v"(p3), "s"(lds_addr)
        : "memory");
}
__device__ __forceinline__ uint32_t lds_addr_of(const KIE_LDS void* p) { return (uint32_t)(uintptr_t)p; }

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
// Also a compiler barrier for memory accesses, so LDS reads of DMA'd data
// are not moved above it.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Workgroup barrier that waits for this wave's LDS traffic only: weight loads
// still in flight stay in flight across it.
__device__ __forceinline__ void wg_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ----------------------------------------------------------------- LDS ------
__device__ __forceinline__ uint4 lds_ld16(const KIE_LDS void* p) {
    u32x4_t v = *(const KIE_LDS u32x4_t*)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void lds_st16(KIE_LDS void* p, uint4 v) {
    u32x4_t w = {v.x, v.y, v.z, v.w};
    *(KIE_LDS u32x4_t*)p = w;
}

// ------------------------------------------------------------------ DPP -----
template <int CTRL, int RM = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, RM, 0xF, false));
}
// Sum over each row of 16 lanes, result in every lane of the row.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_f<0x124>(v);   // row_ror:4
    v += dpp_f<0x128>(v);   // row_ror:8
    return v;
}
// Sum over each group of 8 lanes, result in every lane of the group.
__device__ __forceinline__ float row8_sum(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);   // row_half_mirror
    return v;
}
// After row16_sum: lanes 16..31 hold the sum of lanes 0..31, lanes 48..63 the
// sum of lanes 32..63.
__device__ __forceinline__ float half32_sum_from_rows(float v) { return v + dpp_f<0x142, 0xA>(v); }
// After half32_sum_from_rows: lanes 48..63 hold the sum of all 64 lanes.
__device__ __forceinline__ float full_sum_from_halves(float v) { return v + dpp_f<0x143, 0xC>(v); }
__device__ __forceinline__ float wave_sum_to_lane63(float v) {
    return full_sum_from_halves(half32_sum_from_rows(row16_sum(v)));
}
__device__ __forceinline__ float shfl_xor_f(float v, int m) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane_id() ^ m) << 2, __builtin_bit_cast(int, v)));
}
__device__ __forceinline__ int shfl_xor_i(int v, int m) {
    return __builtin_amdgcn_ds_bpermute((lane_id() ^ m) << 2, v);
}
__device__ __forceinline__ float wave_max(float v) {
    for (int off = 32; off; off >>= 1) v = fmaxf(v, shfl_xor_f(v, off));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    for (int off = 32; off; off >>= 1) v += shfl_xor_f(v, off);
    return v;
}
// (value, index) maximum over the wave, ties to the lower index.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
    for (int off = 32; off; off >>= 1) {
        float ov = shfl_xor_f(v, off);
        int oi = shfl_xor_i(i, off);
        if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
    }
}

// ---------------------------------------------------------------- dot2 ------
__device__ __forceinline__ float dot8(uint4 w, uint4 x, float acc) {
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, w.x), __builtin_bit_cast(h2_t, x.x), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, w.y), __builtin_bit_cast(h2_t, x.y), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, w.z), __builtin_bit_cast(h2_t, x.z), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, w.w), __builtin_bit_cast(h2_t, x.w), acc, false);
    return acc;
}

__device__ __forceinline__ uint16_t f2h_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
__device__ __forceinline__ float h2f_bits(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    return (uint32_t)f2h_bits(a) | ((uint32_t)f2h_bits(b) << 16);
}

// ------------------------------------------------------- flagged words -----
// Word = (phase id << 32) | payload; one device-scope 64-bit store / load.
__device__ __forceinline__ void fw_store(uint64_t* p, uint32_t payload, uint32_t id) {
    __hip_atomic_store(gptr(p), ((uint64_t)id << 32) | payload, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t fw_load(const uint64_t* p) {
    return __hip_atomic_load(gptr(const_cast<uint64_t*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool fw_ok(uint64_t w, uint32_t id) { return (uint32_t)(w >> 32) == id; }

// The XCD (accelerator complex die) this wave runs on, from the hardware.
__device__ __forceinline__ int xcc_id() {
    uint32_t v;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(v));
    return (int)v;
}
__device__ __forceinline__ uint32_t fw_val(uint64_t w) { return (uint32_t)w; }

// Device-scope plain data (the KV cache): 8-byte loads and stores that are
// coherent across the XCDs' L2 caches without a flush.
__device__ __forceinline__ void dev_store64(void* p, uint64_t v) {
    __hip_atomic_store(gptr((uint64_t*)p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void dev_store32(void* p, uint32_t v) {
    __hip_atomic_store(gptr((uint32_t*)p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// System-scope store (the decode kernel's status word in pinned host memory).
__device__ __forceinline__ void sys_store32(void* p, uint32_t v) {
    __hip_atomic_store(gptr((uint32_t*)p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ uint64_t dev_load64(const void* p) {
    return __hip_atomic_load(gptr((uint64_t*)const_cast<void*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t dev_load32(const void* p) {
    return __hip_atomic_load(gptr((uint32_t*)const_cast<void*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Four device-scope 8-byte loads per lane whose data has arrived when the
// statement returns (the wait is part of it). Code that also keeps LDS DMA in
// flight uses this so that the compiler never sees a load of its own in
// flight there (it would otherwise insert waits that also drain the DMA).
__device__ __forceinline__ void dev_load64x4_sync(const void* p0, const void* p1, const void* p2, const void* p3,
                                                  uint64_t& v0, uint64_t& v1, uint64_t& v2, uint64_t& v3) {
    asm volatile(
        "global_load_dwordx2 %0, %4, off sc1\n\t"
        "global_load_dwordx2 %1, %5, off sc1\n\t"
        "global_load_dwordx2 %2, %6, off sc1\n\t"
        "global_load_dwordx2 %3, %7, off sc1\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)
        : "v"(p0), "v"(p1), "v"(p2), "v"(p3)
        : "memory");
}

// Eight 16-byte device-scope loads (four keys, four values) and the wait for
// them in one statement, so the compiler neither sees a pending load nor
// waits for loads it cannot see (the LDS DMA ring) at other places.
__device__ __forceinline__ void dev_load128x8_sync(const void* k0, const void* k1, const void* k2, const void* k3,
                                                   const void* v0, const void* v1, const void* v2, const void* v3,
                                                   uint4& a0, uint4& a1, uint4& a2, uint4& a3, uint4& b0, uint4& b1,
                                                   uint4& b2, uint4& b3) {
    asm volatile(
        "global_load_dwordx4 %0, %8, off sc1\n\t"
        "global_load_dwordx4 %1, %9, off sc1\n\t"
        "global_load_dwordx4 %2, %10, off sc1\n\t"
        "global_load_dwordx4 %3, %11, off sc1\n\t"
        "global_load_dwordx4 %4, %12, off sc1\n\t"
        "global_load_dwordx4 %5, %13, off sc1\n\t"
        "global_load_dwordx4 %6, %14, off sc1\n\t"
        "global_load_dwordx4 %7, %15, off sc1\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&v"(b0), "=&v"(b1), "=&v"(b2), "=&v"(b3)
        : "v"(k0), "v"(k1), "v"(k2), "v"(k3), "v"(v0), "v"(v1), "v"(v2), "v"(v3)
        : "memory");
}

// Should a waiting wave give up? *status is set non-zero by a workgroup that
// timed out or by the host's watchdog (the decode kernel's status word lives
// in pinned host memory). Read only by waits that have already polled in vain
// many times, so its trip is off every normal path.
__device__ __forceinline__ bool stop_requested(const uint32_t* status) {
    return __hip_atomic_load(gptr(const_cast<uint32_t*>(status)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != 0;
}

// Wait until words [0, n) of src all carry `id`, then call f(i, payload) for
// every word (lane l handles i = l, l + 64, ...). One wave calls this.
//
// A block of 64R words is polled as a whole: every poll issues the same R
// loads per lane (lanes past the end re-read word 0; a word that carries `id`
// keeps it until this wave has published something its producer waits for,
// so re-reading it is harmless) and waits for them once. Loads that depend on
// what the previous poll returned would sit in divergent branches, where the
// compiler's wait counting gives up and waits after each load, one trip
// through the memory pipeline per load instead of one per poll.
// Returns 0, or 1 when spin_limit polls went by, or 2 when stop_requested()
// (another workgroup gave up, or the host's watchdog fired).
constexpr int kGatherRegs = 16;     // words per lane per block (at most)
// Back-off after a poll that found words still unpublished, in units of 64
// clocks: a waiting workgroup re-reads its whole slice every trip, and with
// most of the grid waiting on the last producers that traffic slows the ones
// still streaming. 4 (256 clocks, a fraction of a poll trip) measured best.
#ifndef KIE_POLL_SLEEP
#define KIE_POLL_SLEEP 4
#endif

template <int R, class F>
__device__ __forceinline__ int fw_gather_block(const uint64_t* src, int n, uint32_t id, uint32_t spin_limit,
                                               const uint32_t* status, uint32_t& spins, F& f) {
    const int lane = lane_id();
    const uint64_t* p[R];
#pragma unroll
    for (int c = 0; c < R; ++c) {
        const int i = c * 64 + lane;
        p[c] = src + (i < n ? i : 0);
    }
    uint64_t x[R];
    while (true) {
#pragma unroll
        for (int c = 0; c < R; ++c) x[c] = fw_load(p[c]);
        bool ok = true;
#pragma unroll
        for (int c = 0; c < R; ++c) ok = fw_ok(x[c], id) && ok;
        if (__builtin_amdgcn_ballot_w64(!ok) == 0) break;
        if (++spins > spin_limit) return 1;
        if ((spins & 63) == 0 && stop_requested(status)) return 2;
#if KIE_POLL_SLEEP > 0
        __builtin_amdgcn_s_sleep(KIE_POLL_SLEEP);
#endif
    }
#pragma unroll
    for (int c = 0; c < R; ++c) {
        const int i = c * 64 + lane;
        if (i < n) f(i, fw_val(x[c]));
    }
    return 0;
}

template <class F>
__device__ __forceinline__ int fw_gather(const uint64_t* src, int n, uint32_t id, uint32_t spin_limit,
                                         const uint32_t* status, F f) {
    uint32_t spins = 0;
    for (int base = 0; base < n; base += 64 * kGatherRegs) {
        const int m = (n - base < 64 * kGatherRegs) ? n - base : 64 * kGatherRegs;
        const int per = (m + 63) / 64;
        auto g = [&](int i, uint32_t v) { f(base + i, v); };
        int r;
        if (per <= 2) r = fw_gather_block<2>(src + base, m, id, spin_limit, status, spins, g);
        else if (per <= 4) r = fw_gather_block<4>(src + base, m, id, spin_limit, status, spins, g);
        else if (per <= 8) r = fw_gather_block<8>(src + base, m, id, spin_limit, status, spins, g);
        else r = fw_gather_block<16>(src + base, m, id, spin_limit, status, spins, g);
        if (r) return r;
    }
    return 0;
}

// ------------------------------------------------------- fenced barrier -----
// Grid barrier executed by ONE wave per workgroup: agent-scope release, publish
// `epoch` in bar[wg], poll every workgroup's word, agent-scope acquire.
// Returns false on timeout or when *status reports a failure.
__device__ __forceinline__ bool grid_barrier_fenced(uint32_t* bar, uint32_t* status, int nwg, int wg,
                                                    uint32_t epoch, uint32_t limit) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (lane_id() == 0) dev_store32(&bar[wg], epoch);
    uint32_t spins = 0;
    while (true) {
        bool ok = true;
        for (int i = lane_id(); i < nwg; i += 64) {
            uint32_t v = dev_load32(&bar[i]);
            ok = ok && ((int)(v - epoch) >= 0);
        }
        if (__builtin_amdgcn_ballot_w64(!ok) == 0) break;
        if (dev_load32(status) != 0) return false;
        if (++spins > limit) {
            if (lane_id() == 0) dev_store32(status, (uint32_t)kStatusTimeout);
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return true;
}

}  // namespace kie

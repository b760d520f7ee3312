// kie_device.h - gfx950 device primitives of the persistent decode kernel.
//
//  * LDS helpers that bypass the compiler's LDS-DMA tracking (inline asm), so a
//    wave that issues global_load_lds can poll LDS without draining vmcnt.
//  * The weight streamer ("producer" waves): non-temporal 16-byte-per-lane
//    global_load_lds_dwordx4 into a ring of 1 KiB LDS slots, a fixed number of
//    loads kept in flight, readiness published per slot in issue order.
//    This is the monokernel article's non-temporal streaming of weights into
//    LDS and registers ("Inside the monokernel"), done with CDNA4's direct
//    global->LDS loads.
//  * Wave-wide DPP reductions (row_ror / row_bcast, gfx9 family).
//  * v_dot2 fp16 x fp16 -> fp32 inner products (the pages' VDOT path for
//    batch-1 GEMV, same section).
//  * The grid barrier: each workgroup's leader publishes an epoch in its own
//    word of a flat array and polls the whole array (an all-gather barrier,
//    the shape of the 256-CU / 2,048-byte publish test in "Inside the
//    monokernel"), with agent-scope release/acquire and a bounded spin.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kie_common.h"

namespace kie {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte non-temporal global load.
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
    u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
// Pointers into LDS carry address space 3 explicitly so that every access
// through them is a ds_* instruction (a generic pointer would become flat_*).
#define KIE_LDS __attribute__((address_space(3)))

constexpr int kStatusTimeout = 1;

__device__ __forceinline__ uint32_t lds_off(const KIE_LDS void* p) { return (uint32_t)(uintptr_t)p; }

// LDS load/store the compiler does not see as LDS accesses (so it inserts no
// vmcnt wait for in-flight LDS-DMA). The load waits for its own result and
// returns it as a wave-uniform value (every lane reads the same word).
__device__ __forceinline__ uint32_t lds_ld_u32(const KIE_LDS uint32_t* p) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_off(p)) : "memory");
    return __builtin_amdgcn_readfirstlane(v);
}
// 16-byte LDS load/store (ds_read_b128 / ds_write_b128).
__device__ __forceinline__ uint4 lds_ld16(const KIE_LDS void* p) {
    u32x4_t v = *(const KIE_LDS u32x4_t*)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void lds_st16(KIE_LDS void* p, uint4 v) {
    u32x4_t w = {v.x, v.y, v.z, v.w};
    *(KIE_LDS u32x4_t*)p = w;
}
__device__ __forceinline__ void lds_st_u32(KIE_LDS uint32_t* p, uint32_t v) {
    asm volatile("ds_write_b32 %0, %1" ::"v"(lds_off(p)), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_add_u32(KIE_LDS uint32_t* p, uint32_t v) {
    asm volatile("ds_add_u32 %0, %1" ::"v"(lds_off(p)), "v"(v) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ------------------------------------------------------------------ DPP ---
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
__device__ __forceinline__ float readlane_f(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) {
    int src = (lane_id() ^ m) << 2;
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, v)));
}
__device__ __forceinline__ int shfl_xor_i(int v, int m) {
    return __builtin_amdgcn_ds_bpermute((lane_id() ^ m) << 2, v);
}

// ---------------------------------------------------------------- dot2 ----
__device__ __forceinline__ float dot8(uint4 w, uint4 x, float acc) {
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, w.x), __builtin_bit_cast(h2_t, x.x), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, w.y), __builtin_bit_cast(h2_t, x.y), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, w.z), __builtin_bit_cast(h2_t, x.z), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, w.w), __builtin_bit_cast(h2_t, x.w), acc, false);
    return acc;
}

__device__ __forceinline__ uint16_t f2h_bits(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ float h2f_bits(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// ------------------------------------------------------------ LDS ring ----
// Control block shared by the waves of one workgroup (lives in LDS).
struct RingCtl {
    uint32_t ready[2];        // per producer wave: its units landed in LDS
    uint32_t cons[8];         // per consumer wave: lower bound of its next unit
    uint32_t sync;            // consumer-wave LDS barrier counter
    uint32_t abort;           // nonzero: every wave leaves its loops
    uint32_t flag;            // leader -> other consumer waves broadcast
    uint32_t route;           // MoE: number of routing decisions published
    uint32_t token;           // broadcast of the sampled token
    uint32_t sel[16];         // MoE: selected experts of the current layer
    float pi[16];             // MoE: their router probabilities
    float scratch[64];        // small cross-wave reductions
};

template <int NP, int NC, int NSLOT>
struct RingCfg {
    static constexpr int kNP = NP;
    static constexpr int kNC = NC;
    static constexpr int kSlots = NSLOT;
    static constexpr uint32_t kMask = NSLOT - 1;
    static_assert((NSLOT & (NSLOT - 1)) == 0, "slot count must be a power of two");
    static_assert(NP == 2, "readiness is tracked per unit parity");
};

// Consumer side: wait until stream unit u is in LDS. Producer 0 has landed
// units 0, 2, .., 2*ready[0]-2 and producer 1 units 1, 3, .., 2*ready[1]-1, so
// every unit below min(2*ready[0], 2*ready[1]+1) is in LDS; `avail` caches
// that bound. Returns false on abort.
__device__ __forceinline__ bool ring_wait_ready(KIE_LDS RingCtl* ctl, uint32_t u, uint32_t& avail, uint32_t limit) {
    if ((int)(u - avail) < 0) return true;
    uint32_t spins = 0;
    while (true) {
        uint32_t r0 = 2u * lds_ld_u32(&ctl->ready[0]);
        uint32_t r1 = 2u * lds_ld_u32(&ctl->ready[1]) + 1u;
        avail = ((int)(r0 - r1) < 0) ? r0 : r1;
        if ((int)(u - avail) < 0) return true;
        if (lds_ld_u32(&ctl->abort)) return false;
        if (++spins > limit) {
            lds_st_u32(&ctl->abort, 1);
            return false;
        }
        __builtin_amdgcn_s_sleep(0);
    }
}

// Consumer-wave LDS barrier (producers do not take part). Returns false on abort.
// `gen` is the value the counter must reach (caller adds NC per sync).
__device__ __forceinline__ bool consumer_sync(KIE_LDS RingCtl* ctl, uint32_t gen, uint32_t limit) {
    wait_lgkm0();
    if (lane_id() == 0) lds_add_u32(&ctl->sync, 1u);   // one arrival per wave
    uint32_t spins = 0;
    while (true) {
        uint32_t v = lds_ld_u32(&ctl->sync);
        if ((int)(v - gen) >= 0) return true;
        if (lds_ld_u32(&ctl->abort)) return false;
        if (++spins > limit) {
            lds_st_u32(&ctl->abort, 1);
            return false;
        }
        __builtin_amdgcn_s_sleep(0);
    }
}

// Grid barrier executed by ONE wave per workgroup (the leader wave).
// Publishes `epoch` in bar[wg] after an agent-scope release, then polls every
// workgroup's word until all reached `epoch`, then acquires. Returns false on
// timeout or when another workgroup reported a failure in *status.
__device__ __forceinline__ bool grid_barrier_leader(uint32_t* bar, uint32_t* status, int nwg, int wg,
                                                    uint32_t epoch, uint32_t limit) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (lane_id() == 0) __hip_atomic_store(&bar[wg], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t spins = 0;
    while (true) {
        bool ok = true;
        for (int i = lane_id(); i < nwg; i += 64) {
            uint32_t v = __hip_atomic_load(&bar[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ok = ok && ((int)(v - epoch) >= 0);
        }
        if (__builtin_amdgcn_ballot_w64(!ok) == 0) break;
        if (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return false;
        if (++spins > limit) {
            if (lane_id() == 0)
                __hip_atomic_store(status, (uint32_t)kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return true;
}

// ----------------------------------------------------------- producer -----
// The producer waves walk the workgroup's weight stream unit by unit; wave p
// issues the units of parity p. A unit may be loaded into slot u % NSLOT only
// when every consumer wave has moved past unit u - NSLOT.
template <class RC, int DEPTH>
struct Producer {
    KIE_LDS RingCtl* ctl;
    KIE_LDS uint8_t* ring;   // LDS ring base
    uint32_t p;              // producer index (unit parity)
    uint32_t u;              // next stream unit index (both parities)
    uint32_t issued;         // units issued by this wave
    uint32_t published;      // ready value last published
    uint32_t free_lim;       // units below this may be issued
    uint32_t limit;
    uint32_t aux;            // cache-policy bits of the load (non-temporal)

    __device__ __forceinline__ void init(KIE_LDS RingCtl* c, KIE_LDS uint8_t* r, uint32_t pi, uint32_t spin_limit) {
        ctl = c;
        ring = r;
        p = pi;
        u = 0;
        issued = 0;
        published = 0;
        free_lim = RC::kSlots;
        limit = spin_limit;
    }

    __device__ __forceinline__ uint32_t min_cons() {
        uint32_t m = lds_ld_u32(&ctl->cons[0]);
#pragma unroll
        for (int c = 1; c < RC::kNC; ++c) {
            uint32_t v = lds_ld_u32(&ctl->cons[c]);
            if ((int)(v - m) < 0) m = v;
        }
        return m;
    }

    __device__ __forceinline__ void publish_all() {
        wait_vm0();
        if (issued != published) {
            published = issued;
            lds_st_u32(p ? &ctl->ready[1] : &ctl->ready[0], issued);
        }
    }

    // Wait until unit u may be loaded. Returns false on abort.
    __device__ __forceinline__ bool wait_slot() {
        if ((int)(u - free_lim) < 0) return true;
        free_lim = min_cons() + RC::kSlots;
        if ((int)(u - free_lim) < 0) return true;
        publish_all();   // consumers may be waiting for units already in flight
        uint32_t spins = 0;
        while (true) {
            __builtin_amdgcn_s_sleep(1);
            free_lim = min_cons() + RC::kSlots;
            if ((int)(u - free_lim) < 0) return true;
            if (lds_ld_u32(&ctl->abort)) return false;
            if (++spins > limit) {
                lds_st_u32(&ctl->abort, 1);
                return false;
            }
        }
    }

    // Stream n units starting at global address src (1 KiB each). Returns false on abort.
    __device__ __forceinline__ bool stream(const uint8_t* src, uint32_t n) {
        uint32_t end = u + n;
        // first unit of my parity
        uint32_t j = (u & 1u) == p ? 0u : 1u;
        u += j;
        for (; (int)(u - end) < 0; u += 2, j += 2) {
            if (!wait_slot()) return false;
            const uint8_t* g = src + (size_t)j * kUnitBytes + lane_id() * 16;
            KIE_LDS uint8_t* dst = ring + (u & RC::kMask) * kUnitBytes;
            __builtin_amdgcn_global_load_lds((const void*)g, (KIE_LDS void*)dst, 16, 0, 2 /* nt */);
            ++issued;
            if (issued - published > (uint32_t)DEPTH) {
                wait_vm<DEPTH>();
                published = issued - DEPTH;
                lds_st_u32(p ? &ctl->ready[1] : &ctl->ready[0], published);
            }
        }
        u = end;
        return true;
    }
};

}  // namespace kie

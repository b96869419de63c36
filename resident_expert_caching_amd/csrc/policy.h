// The placement policy of one access, run by a single wave ("Luce Spark runs
// 35B MoE models on 16GB GPU without speed loss", paragraph "The key
// components": a pinned most-used set and a fixed ring of spare slots; a cold
// expert is copied from pinned host memory into a spare slot, evicting the
// least recently used entry).  Shared by the decode gate/up kernel and the
// prefill policy kernel so that both follow one implementation:
//  - a pinned expert is served from its slot;
//  - any other access is a cold hit: a ring entry owned by the expert is a
//    ring hit (its stamp becomes ++clock); otherwise the expert is filled
//    into the lowest-index empty ring slot, else into the entry with the
//    smallest stamp (stamps are unique, so this is the LRU entry), the fill
//    is logged and requested from the host fill agent through the FIFO.
#pragma once
#include "device_common.h"
#include "internal.h"

namespace moe {

struct RingState {
    uint64_t clock, fseq, qseq;
    int64_t nev;
    int64_t n_pin, n_cold, n_ring, n_fill, n_evict, n_pref;
};

// Copy the ring tables into LDS (whole wave).
__device__ inline void ring_load(const PolicyTables& pt, int32_t* r_owner, uint64_t* r_stamp, uint64_t* r_seq,
                                 RingState& s) {
    const int lane = threadIdx.x & 63;
    for (int r = lane; r < pt.R; r += 64) {
        r_owner[r] = pt.ring_owner[r];
        r_stamp[r] = pt.ring_stamp[r];
        r_seq[r] = pt.ring_seq[r];
    }
    s.clock = *pt.clock;
    s.fseq = *pt.fill_seq;
    s.qseq = *pt.req_seq;
    s.nev = *pt.n_events;
    __builtin_amdgcn_wave_barrier();
}

// Write the LDS copies back (whole wave).
__device__ inline void ring_store(const PolicyTables& pt, const int32_t* r_owner, const uint64_t* r_stamp,
                                  const uint64_t* r_seq, const RingState& s) {
    const int lane = threadIdx.x & 63;
    __builtin_amdgcn_wave_barrier();
    for (int r = lane; r < pt.R; r += 64) {
        pt.ring_owner[r] = r_owner[r];
        pt.ring_stamp[r] = r_stamp[r];
        pt.ring_seq[r] = r_seq[r];
    }
    if (lane == 0) {
        *pt.clock = s.clock;
        *pt.fill_seq = s.fseq;
        *pt.req_seq = s.qseq;
        *pt.n_events = s.nev;
    }
}

// Copy (layer, expert) into a ring slot: the lowest-index empty slot, else
// the entry with the smallest stamp (the least recently used), whose owner is
// evicted; the entry takes a fresh stamp.  The copy is logged with `kind`
// (MOE_SPARK_EV_FILL or MOE_SPARK_EV_PREFETCH) and, unless the kernels pull
// fills themselves, requested from the host fill agent.  Wave-uniform
// arguments and results: slot (global id) and wseq (the fill number).
__device__ inline void ring_fill(const PolicyTables& pt, int layer, int expert, int32_t* r_owner,
                                 uint64_t* r_stamp, uint64_t* r_seq, RingState& s, int kind, int& slot,
                                 uint64_t& wseq) {
    const int lane = threadIdx.x & 63;
    const int R = pt.R;
    const int32_t key = layer * pt.E + expert;
    int v = -1;
    for (int base = 0; base < R && v < 0; base += 64) {
        const int r = base + lane;
        const uint64_t m = __ballot(r < R && r_owner[r] < 0);
        if (m) v = base + __builtin_ctzll(m);
    }
    if (v < 0) {  // least recently used: smallest stamp (stamps are unique)
        uint64_t bs = ~0ull;
        int bi = 0x7fffffff;
        for (int r = lane; r < R; r += 64)
            if (r_stamp[r] < bs) {
                bs = r_stamp[r];
                bi = r;
            }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            const uint64_t os = __shfl_xor(bs, m, 64);
            const int oi = __shfl_xor(bi, m, 64);
            if (os < bs || (os == bs && oi < bi)) {
                bs = os;
                bi = oi;
            }
        }
        v = bi;
    }
    const int32_t victim = r_owner[v];
    if (victim >= 0) ++s.n_evict;
    ++s.clock;
    ++s.fseq;
    if (kind == MOE_SPARK_EV_PREFETCH)
        ++s.n_pref;
    else
        ++s.n_fill;
    if (lane == 0) {
        r_owner[v] = key;
        r_stamp[v] = s.clock;
        r_seq[v] = s.fseq;
        if (s.nev < pt.event_cap) {
            moe_spark_event ev;
            ev.seq = (int64_t)s.fseq;
            ev.layer = layer;
            ev.expert = expert;
            ev.slot = (int32_t)(pt.P + v);
            ev.kind = kind;
            ev.victim = victim;
            ev.pad = 0;
            pt.events[s.nev] = ev;
        }
        if (!pt.pull) {  // a copy for the host agent (pulled fills are copied by the kernels)
            FifoEntry* fe = pt.fifo + (s.qseq % kFifoCap);
            fe->key = key;
            fe->ring = v;
            fe->fill = s.fseq;
            __threadfence_system();
            __hip_atomic_store(&fe->seq, s.qseq + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
        }
    }
    if (!pt.pull) ++s.qseq;
    __builtin_amdgcn_wave_barrier();
    ++s.nev;
    wseq = s.fseq;
    slot = (int)(pt.P + v);
}

// Index of the ring entry owned by key, or -1 (wave-uniform).
__device__ inline int ring_find(const PolicyTables& pt, int32_t key, const int32_t* r_owner) {
    const int lane = threadIdx.x & 63;
    int hit = -1;
    for (int base = 0; base < pt.R && hit < 0; base += 64) {
        const int r = base + lane;
        const uint64_t m = __ballot(r < pt.R && r_owner[r] == key);
        if (m) hit = base + __builtin_ctzll(m);
    }
    return hit;
}

// One access of (layer, expert) whose pinned slot is `pin` (-1: not pinned).
// Wave-uniform arguments and results.  wseq: fill number to wait for, 0 when
// the data is already resident.
__device__ inline void ring_access(const PolicyTables& pt, int layer, int expert, int pin, int32_t* r_owner,
                                   uint64_t* r_stamp, uint64_t* r_seq, RingState& s, int& slot, uint64_t& wseq) {
    const int lane = threadIdx.x & 63;
    wseq = 0;
    if (pin >= 0) {
        slot = pin;
        ++s.n_pin;
        return;
    }
    ++s.n_cold;
    const int hit = ring_find(pt, layer * pt.E + expert, r_owner);
    if (hit >= 0) {
        // filled by an earlier access (or prefetch) whose copy has landed
        ++s.n_ring;
        ++s.clock;
        if (lane == 0) r_stamp[hit] = s.clock;
        __builtin_amdgcn_wave_barrier();
        slot = (int)(pt.P + hit);
        return;
    }
    ring_fill(pt, layer, expert, r_owner, r_stamp, r_seq, s, MOE_SPARK_EV_FILL, slot, wseq);
}

// Speculative prefetch of (layer, expert): nothing when it is pinned or
// already in the ring (no stamp change: a prefetch is not an access);
// otherwise a copy into a ring slot by the fill rule.  Returns whether a
// copy was made (slot, wseq as ring_fill).  Wave-uniform.
__device__ inline bool ring_prefetch(const PolicyTables& pt, int layer, int expert, int pin, int32_t* r_owner,
                                     uint64_t* r_stamp, uint64_t* r_seq, RingState& s, int& slot,
                                     uint64_t& wseq) {
    if (pin >= 0 || ring_find(pt, layer * pt.E + expert, r_owner) >= 0) return false;
    ring_fill(pt, layer, expert, r_owner, r_stamp, r_seq, s, MOE_SPARK_EV_PREFETCH, slot, wseq);
    return true;
}

// Add this policy run's counters to the device statistics (lane 0).
__device__ inline void stats_flush(const PolicyTables& pt, int64_t accesses, const RingState& s) {
    if ((threadIdx.x & 63) != 0) return;
    unsigned long long* st = reinterpret_cast<unsigned long long*>(pt.stats);
    atomicAdd(st + DS_ACC, (unsigned long long)accesses);
    if (s.n_pin) atomicAdd(st + DS_PIN, (unsigned long long)s.n_pin);
    if (s.n_cold) atomicAdd(st + DS_COLD, (unsigned long long)s.n_cold);
    if (s.n_ring) atomicAdd(st + DS_RING, (unsigned long long)s.n_ring);
    if (s.n_fill) atomicAdd(st + DS_FILL, (unsigned long long)s.n_fill);
    if (s.n_pref) atomicAdd(st + DS_PREF, (unsigned long long)s.n_pref);
    if (s.n_fill + s.n_pref)
        atomicAdd(st + DS_H2D, (unsigned long long)((s.n_fill + s.n_pref) * pt.slot_bytes));
    if (s.n_evict) atomicAdd(st + DS_EVICT, (unsigned long long)s.n_evict);
}

}  // namespace moe

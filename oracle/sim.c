/*
 * CPU simulator of expert placement and the spare-slot LRU ring — TEST
 * INFRASTRUCTURE (shares no code with the GPU library).
 *
 * Source: "Luce Spark runs 35B MoE models on 16GB GPU without speed loss"
 * (theneuralfeed.com), paragraph "The key components":
 *  (1) calibrated placement accumulates per-expert routing counts and pins
 *      the most-used set;
 *  (2) a bounded cache — a fixed ring of spare GPU slots; a cold expert is
 *      copied from pinned host memory into a spare slot, evicting the least
 *      recently used entry.
 *
 * Readings taken where the page is silent (each is a plain reading of it):
 *  - The pinned budget P is global and split into per-layer quotas
 *    q_l = floor(P/L) + [l < P mod L]; the R ring slots are in addition to P
 *    and shared by all layers (one ring).
 *  - Uniform placement pins experts 0..q_l-1 of every layer; pinned slot ids
 *    0..P-1 follow (layer, expert) ascending; ring slots are P..P+R-1.
 *  - Calibration pins the top q_l experts of each layer by (count desc,
 *    expert asc).  Experts that stay pinned keep their slot; freed slots, in
 *    ascending order, go to newly pinned experts in (layer, expert) order; a
 *    newly pinned expert's ring entry, if any, is emptied.
 *  - A cold hit is an access to an expert that is not pinned.  A cold hit
 *    already in the ring refreshes its stamp; otherwise it is a fill into the
 *    lowest-index empty ring slot, else into the slot with the smallest stamp
 *    (the least recently used), whose owner is evicted.  Stamps come from one
 *    clock that ticks once per ring access, so they are unique.
 *  - Decode accesses run in (token, layer, rank) order.  A prefill batch
 *    accesses each layer's distinct experts once, in ascending id.
 *  - counts[l][e] grows by one per (token, rank) that selects e.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

struct oracle_sim {
    int L, E, R;
    int64_t P, slot_bytes;
    int32_t* slot_of;     /* [L*E], -1 if not pinned */
    int64_t* counts;      /* [L*E] */
    int32_t* ring_owner;  /* [R], l*E+e or -1 */
    int64_t* ring_stamp;  /* [R] */
    int64_t clock;
    int64_t fill_seq;
    int64_t st[ORACLE_N_STATS];
    int pf_last_cold;     /* cold experts in the last chunk of the last prefill layer */
    oracle_event* ev;
    int64_t n_ev, cap_ev;
};

enum { S_ACC = 0, S_PIN, S_COLD, S_RING, S_FILL, S_EVICT, S_H2D, S_PREF };

int64_t oracle_sim_quota(int L, int64_t P, int layer) {
    return P / L + ((int64_t)layer < P % L ? 1 : 0);
}

oracle_sim* oracle_sim_create(int L, int E, int64_t P, int R, int64_t slot_bytes) {
    if (L <= 0 || E <= 0 || R < 0 || P < 0 || P > (int64_t)L * E) return NULL;
    oracle_sim* s = (oracle_sim*)calloc(1, sizeof(oracle_sim));
    s->L = L; s->E = E; s->P = P; s->R = R; s->slot_bytes = slot_bytes;
    s->slot_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)L * E);
    s->counts = (int64_t*)calloc((size_t)L * E, sizeof(int64_t));
    s->ring_owner = (int32_t*)malloc(sizeof(int32_t) * (size_t)(R > 0 ? R : 1));
    s->ring_stamp = (int64_t*)calloc((size_t)(R > 0 ? R : 1), sizeof(int64_t));
    for (int64_t i = 0; i < (int64_t)L * E; ++i) s->slot_of[i] = -1;
    for (int r = 0; r < R; ++r) s->ring_owner[r] = -1;
    return s;
}

void oracle_sim_destroy(oracle_sim* s) {
    if (!s) return;
    free(s->slot_of); free(s->counts); free(s->ring_owner); free(s->ring_stamp); free(s->ev);
    free(s);
}

static void empty_ring(oracle_sim* s) {
    for (int r = 0; r < s->R; ++r) { s->ring_owner[r] = -1; s->ring_stamp[r] = 0; }
}

void oracle_sim_place_uniform(oracle_sim* s) {
    int32_t next = 0;
    for (int l = 0; l < s->L; ++l) {
        int64_t q = oracle_sim_quota(s->L, s->P, l);
        for (int e = 0; e < s->E; ++e)
            s->slot_of[(int64_t)l * s->E + e] = (e < q) ? next++ : -1;
    }
    empty_ring(s);
}

/* rank experts of one layer by (count desc, expert asc) */
static const int64_t* g_cnt;
static int cmp_count_desc(const void* a, const void* b) {
    int ea = *(const int*)a, eb = *(const int*)b;
    if (g_cnt[ea] != g_cnt[eb]) return g_cnt[ea] > g_cnt[eb] ? -1 : 1;
    return ea - eb;
}

void oracle_sim_calibrate(oracle_sim* s, int reset_counts) {
    const int L = s->L, E = s->E;
    char* want = (char*)calloc((size_t)L * E, 1);
    int* order = (int*)malloc(sizeof(int) * (size_t)E);
    for (int l = 0; l < L; ++l) {
        for (int e = 0; e < E; ++e) order[e] = e;
        g_cnt = s->counts + (int64_t)l * E;
        qsort(order, (size_t)E, sizeof(int), cmp_count_desc);
        int64_t q = oracle_sim_quota(L, s->P, l);
        for (int64_t i = 0; i < q; ++i) want[(int64_t)l * E + order[i]] = 1;
    }
    /* slots freed by experts leaving the pinned set, ascending */
    int64_t n_free = 0;
    int32_t* freed = (int32_t*)malloc(sizeof(int32_t) * (size_t)(s->P > 0 ? s->P : 1));
    char* used = (char*)calloc((size_t)(s->P > 0 ? s->P : 1), 1);
    for (int64_t i = 0; i < (int64_t)L * E; ++i)
        if (s->slot_of[i] >= 0 && !want[i]) used[s->slot_of[i]] = 1;
    for (int64_t p = 0; p < s->P; ++p)
        if (used[p]) freed[n_free++] = (int32_t)p;
    for (int64_t i = 0; i < (int64_t)L * E; ++i)
        if (s->slot_of[i] >= 0 && !want[i]) s->slot_of[i] = -1;
    /* newly pinned experts, (layer, expert) ascending, take freed slots */
    int64_t next = 0;
    for (int64_t i = 0; i < (int64_t)L * E; ++i) {
        if (!want[i] || s->slot_of[i] >= 0) continue;
        s->slot_of[i] = freed[next++];
        for (int r = 0; r < s->R; ++r)
            if (s->ring_owner[r] == (int32_t)i) { s->ring_owner[r] = -1; s->ring_stamp[r] = 0; }
    }
    if (reset_counts) memset(s->counts, 0, sizeof(int64_t) * (size_t)L * E);
    free(want); free(order); free(freed); free(used);
}

/* Online self-tuning step (reading of the same paragraph: the engine keeps
 * profiling traffic and re-deciding what stays resident).  Per layer, with
 * experts ranked by (count desc, expert asc): walk the unpinned experts from
 * the strongest and the pinned ones from the weakest in step; the pair
 * (x, y) swaps while 100*count[x] > (100 + hyst_pct)*count[y], and the first
 * pair that fails ends the layer.  Freed slots then go, ascending, to the
 * entering experts in (layer, expert) order, whose ring entries are emptied
 * (as in calibration); finally every count is shifted right by decay_shift.
 * Returns the number of swaps. */
int64_t oracle_sim_retune(oracle_sim* s, int hyst_pct, int decay_shift) {
    const int L = s->L, E = s->E;
    int* order = (int*)malloc(sizeof(int) * (size_t)E);
    int* outs = (int*)malloc(sizeof(int) * (size_t)E);
    int* ins = (int*)malloc(sizeof(int) * (size_t)E);
    char* enter = (char*)calloc((size_t)L * E, 1);
    int32_t* freed = (int32_t*)malloc(sizeof(int32_t) * (size_t)(s->P > 0 ? s->P : 1));
    int64_t swaps = 0, n_free = 0;
    for (int l = 0; l < L; ++l) {
        const int64_t base = (int64_t)l * E;
        for (int e = 0; e < E; ++e) order[e] = e;
        g_cnt = s->counts + base;
        qsort(order, (size_t)E, sizeof(int), cmp_count_desc);
        int n_out = 0, n_in = 0;
        for (int i = 0; i < E; ++i)
            if (s->slot_of[base + order[i]] < 0) outs[n_out++] = order[i];
        for (int i = E - 1; i >= 0; --i)
            if (s->slot_of[base + order[i]] >= 0) ins[n_in++] = order[i];
        for (int i = 0; i < n_out && i < n_in; ++i) {
            const int64_t cx = g_cnt[outs[i]], cy = g_cnt[ins[i]];
            if (!(100 * cx > (int64_t)(100 + hyst_pct) * cy)) break;
            enter[base + outs[i]] = 1;
            freed[n_free++] = s->slot_of[base + ins[i]];
            s->slot_of[base + ins[i]] = -1;
            ++swaps;
        }
    }
    /* freed slots ascending (insertion sort: a handful per step) */
    for (int64_t i = 1; i < n_free; ++i) {
        const int32_t v = freed[i];
        int64_t j = i - 1;
        while (j >= 0 && freed[j] > v) { freed[j + 1] = freed[j]; --j; }
        freed[j + 1] = v;
    }
    int64_t next = 0;
    for (int64_t i = 0; i < (int64_t)L * E; ++i) {
        if (!enter[i]) continue;
        s->slot_of[i] = freed[next++];
        for (int r = 0; r < s->R; ++r)
            if (s->ring_owner[r] == (int32_t)i) { s->ring_owner[r] = -1; s->ring_stamp[r] = 0; }
    }
    if (decay_shift > 0)
        for (int64_t i = 0; i < (int64_t)L * E; ++i) s->counts[i] >>= decay_shift;
    free(order); free(outs); free(ins); free(enter); free(freed);
    return swaps;
}

static void log_fill(oracle_sim* s, int l, int e, int slot, int victim, int kind) {
    if (s->n_ev == s->cap_ev) {
        s->cap_ev = s->cap_ev ? 2 * s->cap_ev : 1024;
        s->ev = (oracle_event*)realloc(s->ev, sizeof(oracle_event) * (size_t)s->cap_ev);
    }
    oracle_event* v = &s->ev[s->n_ev++];
    v->seq = s->fill_seq; v->layer = l; v->expert = e; v->slot = slot;
    v->kind = kind; v->victim = victim; v->pad = 0;
}

/* Copy (l, e) into a ring slot: the lowest-index empty slot, else the one
 * with the smallest stamp (least recently used), whose owner is evicted; the
 * entry takes a fresh stamp.  kind: ORACLE_EV_FILL or ORACLE_EV_PREFETCH. */
static void sim_fill(oracle_sim* s, int l, int e, int kind) {
    int32_t key = l * s->E + e;
    int victim_slot = -1;
    for (int r = 0; r < s->R; ++r)
        if (s->ring_owner[r] < 0) { victim_slot = r; break; }
    if (victim_slot < 0) {
        victim_slot = 0;
        for (int r = 1; r < s->R; ++r)
            if (s->ring_stamp[r] < s->ring_stamp[victim_slot]) victim_slot = r;
    }
    int victim = s->ring_owner[victim_slot];
    if (victim >= 0) s->st[S_EVICT]++;
    s->ring_owner[victim_slot] = key;
    s->ring_stamp[victim_slot] = ++s->clock;
    s->st[kind == ORACLE_EV_PREFETCH ? S_PREF : S_FILL]++;
    s->st[S_H2D] += s->slot_bytes;
    s->fill_seq++;
    log_fill(s, l, e, (int)(s->P + victim_slot), victim, kind);
}

static void sim_access(oracle_sim* s, int l, int e) {
    int32_t key = l * s->E + e;
    s->st[S_ACC]++;
    if (s->slot_of[key] >= 0) { s->st[S_PIN]++; return; }
    s->st[S_COLD]++;
    for (int r = 0; r < s->R; ++r) {
        if (s->ring_owner[r] == key) {
            s->st[S_RING]++;
            s->ring_stamp[r] = ++s->clock;
            return;
        }
    }
    if (s->R == 0) return; /* unreachable for valid shapes: R >= K whenever P < L*E */
    sim_fill(s, l, e, ORACLE_EV_FILL);
}

void oracle_sim_decode_layer(oracle_sim* s, int l, int K, const int32_t* idx) {
    for (int k = 0; k < K; ++k) s->counts[(int64_t)l * s->E + idx[k]]++;
    for (int k = 0; k < K; ++k) sim_access(s, l, idx[k]);
}

void oracle_sim_decode_token(oracle_sim* s, int K, const int32_t* idx) {
    for (int l = 0; l < s->L; ++l) oracle_sim_decode_layer(s, l, K, idx + (int64_t)l * K);
}

/* Batched decode (reading: B tokens advance through the stack together, so a
 * layer's accesses come from all B tokens, in batch order, before the next
 * layer's): accesses in (layer, token, rank) order.  idx is [B][L][K]. */
void oracle_sim_decode_batch(oracle_sim* s, int B, int K, const int32_t* idx) {
    for (int l = 0; l < s->L; ++l)
        for (int b = 0; b < B; ++b) oracle_sim_decode_layer(s, l, K, idx + ((int64_t)b * s->L + l) * K);
}

void oracle_sim_prefill_layer(oracle_sim* s, int l, int T, int K, const int32_t* idx) {
    char* hit = (char*)calloc((size_t)s->E, 1);
    for (int64_t i = 0; i < (int64_t)T * K; ++i) {
        s->counts[(int64_t)l * s->E + idx[i]]++;
        hit[idx[i]] = 1;
    }
    int n_cold = 0;
    for (int e = 0; e < s->E; ++e)
        if (hit[e]) {
            n_cold += s->slot_of[(int64_t)l * s->E + e] < 0;
            sim_access(s, l, e);
        }
    /* the layer's cold experts stream through the ring in chunks of R; the
     * last chunk holds the remainder (R when it divides evenly) */
    s->pf_last_cold = (n_cold == 0 || s->R == 0) ? 0 : (n_cold - 1) % s->R + 1;
    free(hit);
}

/* Speculative prefetch after a prefill layer (a reading of the pages' bounded
 * async cache, for the next layer's experts before its routing is known):
 * the candidates are the experts of `layer` whose predicted assignment count
 * hist[e] is positive, in ascending id.  A candidate that is pinned or
 * already in the ring is skipped (no access, no stamp change); any other is
 * filled by the rule of a cold miss, until `budget` prefetches have been
 * made, budget = R minus the cold experts of the last chunk of the preceding
 * prefill layer (those ring entries are still being read, and they carry the
 * newest stamps, so no prefetch evicts them).  Prefetches are not accesses:
 * they count as prefetches, their evictions as evictions and their bytes as
 * host-to-device bytes, and the log lists them with kind PREFETCH.  Returns
 * the number of prefetches. */
int64_t oracle_sim_prefetch(oracle_sim* s, int layer, const int32_t* hist) {
    const int budget = s->R - s->pf_last_cold;
    int64_t n = 0;
    for (int e = 0; e < s->E && n < budget; ++e) {
        if (hist[e] <= 0) continue;
        const int32_t key = layer * s->E + e;
        if (s->slot_of[key] >= 0) continue;
        int in_ring = 0;
        for (int r = 0; r < s->R; ++r) in_ring |= s->ring_owner[r] == key;
        if (in_ring) continue;
        sim_fill(s, layer, e, ORACLE_EV_PREFETCH);
        ++n;
    }
    return n;
}

void oracle_sim_stats(const oracle_sim* s, int64_t* out) {
    memcpy(out, s->st, sizeof(s->st));
}

void oracle_sim_reset_stats(oracle_sim* s) { memset(s->st, 0, sizeof(s->st)); }

void oracle_sim_placement(const oracle_sim* s, int32_t* slot_of, int32_t* ring_owner,
                          int64_t* ring_stamp, int64_t* counts) {
    size_t n = (size_t)s->L * s->E;
    if (slot_of) memcpy(slot_of, s->slot_of, sizeof(int32_t) * n);
    if (ring_owner) memcpy(ring_owner, s->ring_owner, sizeof(int32_t) * (size_t)s->R);
    if (ring_stamp) memcpy(ring_stamp, s->ring_stamp, sizeof(int64_t) * (size_t)s->R);
    if (counts) memcpy(counts, s->counts, sizeof(int64_t) * n);
}

int64_t oracle_sim_events(const oracle_sim* s, oracle_event* out, int64_t cap) {
    int64_t n = s->n_ev < cap ? s->n_ev : cap;
    if (out && n > 0) memcpy(out, s->ev, sizeof(oracle_event) * (size_t)n);
    return s->n_ev;
}

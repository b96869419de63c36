"""Shared helpers of the GPU tests: build a context from a seeded workload
through the C ABI, and the comparison rules against the oracle.

Comparison rules (the method's parity bar):
 * top-k indices bit-exact, except a token-layer whose oracle K-th and
   (K+1)-th logits differ by less than 1e-5 (a router near-tie): there the
   oracle adopts the GPU's selection for the output check;
 * placement bookkeeping (pinned set, ring owners and stamps, fill/eviction
   log, counters) bit-exact against the simulator replaying the GPU's own
   top-k trace;
 * layer outputs within max|err| <= 2e-3 * max|ref| of the fp64 oracle;
 * outputs bit-identical across residencies.
"""
import numpy as np

import oracle
import resident_expert_caching_amd as ms
import workload as wl

TIE_GAP = 1e-5
REL_TOL = 2e-3


def config_for(w, P, R, max_tokens=0, event_cap=0):
    return ms.Config(n_layers=w.L, d_model=w.d, n_experts=w.E, top_k=w.K, d_ff=w.f, wfmt=w.wfmt,
                     rms_eps=1e-6, n_bias_rows=len(w.bias_seeds), resident_cap=P, ring_slots=R,
                     max_tokens=max_tokens, event_cap=event_cap)


class Model:
    """Host copy of a workload's weights (drawn once by the seeded generator)."""

    def __init__(self, w):
        self.w = w
        self.routers = [np.ascontiguousarray(w.router(l)) for l in range(w.L)]
        self.biases = [w.bias_rows(l) for l in range(w.L)]
        self.blob = w.experts_blob()

    def experts(self, layer):
        w = self.w
        return [wl.split_expert(self.blob[layer * w.E + e], w.d, w.f, w.wfmt) for e in range(w.E)]

    def make_ctx(self, P, R, max_tokens=0, compute_stream=None):
        w = self.w
        ctx = ms.moe_spark_create(config_for(w, P, R, max_tokens), compute_stream, None)
        for l in range(w.L):
            b = self.biases[l]
            ms.moe_spark_set_router(ctx, l, self.routers[l].ctypes.data,
                                    None if b is None else np.ascontiguousarray(b).ctypes.data)
        ms.moe_spark_set_experts(ctx, 0, w.L * w.E, self.blob.ctypes.data)
        ms.moe_spark_place_uniform(ctx)
        return ctx


def oracle_topk_and_gap(logits, K):
    E = logits.size
    order = np.lexsort((np.arange(E), -logits))
    gap = np.inf if K == E else logits[order[K - 1]] - logits[order[K]]
    return order[:K].astype(np.int32), gap


def placement(ctx, w, R):
    slot_of = np.empty((w.L, w.E), np.int32)
    owner = np.empty(max(R, 1), np.int32)
    stamp = np.empty(max(R, 1), np.int64)
    counts = np.empty((w.L, w.E), np.int64)
    ms.moe_spark_get_placement(ctx, slot_of.ctypes.data, owner.ctypes.data, stamp.ctypes.data,
                               counts.ctypes.data)
    return slot_of, owner[:R], stamp[:R], counts


def events(ctx):
    n = ms.moe_spark_get_events(ctx, None, 0)
    arr = (ms.Event * max(n, 1))()
    ms.moe_spark_get_events(ctx, arr, n)
    return [(e.seq, e.layer, e.expert, e.slot, e.kind, e.victim) for e in arr[:n]]


def sim_events(sim):
    return [(int(e["seq"]), int(e["layer"]), int(e["expert"]), int(e["slot"]), int(e["kind"]),
             int(e["victim"])) for e in sim.events()]


STAT_KEYS = ("accesses", "pinned_hits", "cold_hits", "ring_hits", "fills", "evictions", "h2d_bytes",
             "prefetches")


def assert_outputs_close(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref).max()
    scale = np.abs(ref).max()
    assert err <= REL_TOL * scale, f"{what}: max|err| {err:.3e} > {REL_TOL} * max|ref| {scale:.3e}"
    return err / scale

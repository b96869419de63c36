"""Benchmark of resident expert caching on one MI355X.

Headline (the JSON line's `value`): decode tok/s of a 40-layer stack of MoE
layers at 60% expert residency.
 - Layer shape: d=2048, 256 experts, top-8, SwiGLU f=512.
 - Weights: Q4_0 experts drawn from N(0, 0.02); fp32 router N(0, 0.02).
 - Stack: residual x += MoE(RMSNorm(x)); attention omitted.
 - Routing: Zipf-skewed (logit bias 2 ln p_r, p_r ~ r^-1.1 over a per-layer
   seeded permutation).
 - Residency: P = 6144 of 10,240 experts pinned, plus a 32-slot LRU spare
   ring.
 - Placement: calibrated from a 256-token warm-up trace decoded under uniform
   placement (always 256 tokens, whatever --warmup says).
Protocol of a decode setting: the 256 calibration tokens (t = 0..255) under
uniform placement, calibration, then --warmup untimed decode tokens (drawn
after the measured stream), a statistics reset, and --steps timed tokens
(t = 256..): a step is one decode token through all 40 layers (one graph
launch).  The same protocol at full residency gives the ratio and the
bit-identity check.

Nested in the same line, each on the fixed 512-token measured stream
(t = 256..767), independent of --steps:
 - `sweep`: residency 100/60/30% x {uniform static, calibrated + ring}, with
   tok/s, cold-hit %, fill %, PCIe bytes and bit-identity of the outputs.
 - `batched`: the same decode in steps of B tokens (moe_spark_decode_batched),
   the ring widened to B*top_k slots where it is smaller; tok/s, distinct
   experts per layer-step, algorithmic weight GB/s, the largest difference
   from batch-1 outputs, counter-measured bytes per launch at B = 16.
 - `self_tuning`: calibrated under router bias row A, the stream decoded
   under row B with the placement fixed and with online self-tuning.
 - `fill_path`: host-to-device rates of cold fills: the pulled fills'
   effective rate in the fill-bound 60%-uniform arm, and the host agent's
   copies (MOE_SPARK_PULL_FILLS=0) in the same arm; `agent_headline` runs
   the headline's own protocol and tokens with the agent's copies.
Also:
 - `prefill`: 2048 tokens through the stack in one batch, 60% residency.
   1. Placement is calibrated from the decode warm-up under permutation A.
   2. The Zipf permutation switches to B at token 1024.
   3. Then a 256-token decode probe under B runs before and after
      recalibration.
 - `prefill_prefetch`: the same prefill from the same state with speculative
   prefetch of each next layer's predicted experts (moe_spark_set_prefetch).
 - `roofline`: the dominant decode kernel, timed by HIP events over isolated
   replays.
 - `h2d_link`: a pinned host-to-device copy probe of the PCIe link.
 - `cpu_baseline`: the fp64 oracle on a bounded sample of the decode stream,
   on all host threads and on one, and on 48 tokens of the prefill batch.

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tok/s @60% expert residency; expert GEMV HBM GB/s; cold-hit %"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
EXPERT_BYTES = 1_769_472          # one Q4_0 expert: gate | up | down
GATEUP_BYTES = 8 * 2 * 589_824    # algorithmic bytes of one gate/up launch (8 experts)
DOWN_BYTES = 8 * 589_824 + 256 * 2048 * 4  # down weights of 8 experts + the next layer's router
TOKEN_BYTES_PER_LAYER = 8 * EXPERT_BYTES + 256 * 2048 * 4
CALIB_TOKENS = 256   # the warm-up trace placement is calibrated from
STREAM_TOKENS = 512  # the measured stream of the sweep, batched and self-tuning legs


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class Model:
    """Host copy of the stack's weights and a loader into a context."""

    def __init__(self, w):
        import workload as wl
        self.w, self.wl = w, wl
        self.routers = [np.ascontiguousarray(w.router(l)) for l in range(w.L)]
        self.biases = [w.bias_rows(l) for l in range(w.L)]
        self.blob = w.experts_blob()

    def experts(self, layer):
        w = self.w
        return [self.wl.split_expert(self.blob[layer * w.E + e], w.d, w.f, w.wfmt)
                for e in range(w.E)]

    def make_ctx(self, P, R, biases=None, max_tokens=0):
        import resident_expert_caching_amd as ms
        w = self.w
        biases = self.biases if biases is None else biases
        cfg = ms.Config(n_layers=w.L, d_model=w.d, n_experts=w.E, top_k=w.K, d_ff=w.f,
                        wfmt=w.wfmt, rms_eps=1e-6, n_bias_rows=biases[0].shape[0],
                        resident_cap=P, ring_slots=R, max_tokens=max_tokens, event_cap=0)
        ctx = ms.moe_spark_create(cfg)
        for l in range(w.L):
            ms.moe_spark_set_router(ctx, l, self.routers[l].ctypes.data,
                                    np.ascontiguousarray(biases[l]).ctypes.data)
        ms.moe_spark_set_experts(ctx, 0, w.L * w.E, self.blob.ctypes.data)
        ms.moe_spark_place_uniform(ctx)
        return ctx


def rates(st):
    acc = max(st["accesses"], 1)
    return dict(cold_hit_pct=round(100.0 * st["cold_hits"] / acc, 4),
                fill_pct=round(100.0 * st["fills"] / acc, 4))


def run_decode(ms, torch, model, P, R, calib, untimed, meas, row, calibrate, kernel_iters=0):
    """One residency setting: the calibration trace under uniform placement,
    optional calibration, untimed warm-up tokens, then the timed decode of
    `meas` (statistics cover exactly the timed tokens)."""
    t0 = time.time()
    ctx = model.make_ctx(P=P, R=R)
    log(f"P={P} R={R} calibrated={calibrate}: context ready in {time.time() - t0:.1f}s")
    try:
        xc = torch.from_numpy(calib).cuda()
        xm = torch.from_numpy(meas).cuda()
        ms.moe_spark_decode(ctx, xc.data_ptr(), xc.shape[0], row.data_ptr())
        ms.moe_spark_synchronize(ctx)
        if calibrate:
            ms.moe_spark_calibrate(ctx, True)
        if untimed is not None and untimed.shape[0]:
            xu = torch.from_numpy(untimed).cuda()
            ms.moe_spark_decode(ctx, xu.data_ptr(), xu.shape[0], row.data_ptr())
            ms.moe_spark_synchronize(ctx)
        ms.moe_spark_reset_stats(ctx)
        ms.moe_spark_decode(ctx, xm.data_ptr(), 0, row.data_ptr())  # build the graph
        ms.moe_spark_synchronize(ctx)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms.moe_spark_decode(ctx, xm.data_ptr(), xm.shape[0], row.data_ptr())
        ms.moe_spark_synchronize(ctx)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t1
        st = ms.moe_spark_get_stats(ctx)
        out = dict(tok_s=xm.shape[0] / dt, ms_per_tok=dt * 1e3 / xm.shape[0], stats=st,
                   elapsed_s=dt, x_out=xm.cpu().numpy())
        if kernel_iters:
            out["us_gateup"], out["us_down"], out["us_route"] = \
                ms.moe_spark_time_expert_kernels(ctx, kernel_iters)
            out["us_stream_probe"] = ms.moe_spark_time_stream_probe(ctx, kernel_iters * model.w.L)
        r = rates(st)
        log(f"P={P} calibrated={calibrate}: {out['tok_s']:.1f} tok/s, cold {r['cold_hit_pct']}%, "
            f"fills {st['fills']}")
        return out
    finally:
        ms.moe_spark_destroy(ctx)


def batched_traffic(path, B):
    """Counter-measured HBM bytes per launch of the batched kernels at B = 16,
    only while their sources hash to the measured ones."""
    if B != 16 or not os.path.exists(path):
        return None
    try:
        tj = json.load(open(path)).get("batched_b16")
        h = hashlib.sha256()
        for f in tj["kernel_sources"]:
            h.update(open(os.path.join(ROOT, "resident_expert_caching_amd", "csrc", f), "rb").read())
        if tj.get("kernel_source_sha256") != h.hexdigest():
            return None
        return dict(gateup_hbm_bytes_per_launch=tj["qb_gateup_hbm_bytes_per_launch"],
                    down_hbm_bytes_per_launch=tj["qb_down_hbm_bytes_per_launch"],
                    distinct_experts_per_layer_step=tj["distinct_experts_per_layer_step"])
    except (OSError, ValueError, KeyError):
        return None


def run_batched(ms, torch, model, P, R, B, warm, meas, row, ref_x, traffic_json):
    """Batched decode: warm-up batch-1 under uniform placement, calibration,
    then `meas` in steps of B tokens.  Each layer-step reads each of its
    distinct experts once; the traced top-k gives their number.  The expert
    products run on the matrix cores, so outputs differ from batch 1 by fp32
    rounding (reported as max|x_B - x_1| / max|x_1|)."""
    w = model.w
    t0 = time.time()
    ctx = model.make_ctx(P=P, R=R)
    log(f"batched B={B}: P={P} R={R}: context ready in {time.time() - t0:.1f}s")
    try:
        T = meas.shape[0]
        tr_k = torch.zeros((T, w.L, w.K), dtype=torch.int32, device="cuda")
        tr_g = torch.zeros((T, w.L, w.K), dtype=torch.float32, device="cuda")
        xw = torch.from_numpy(warm).cuda()
        xm = torch.from_numpy(meas).cuda()
        ms.moe_spark_decode(ctx, xw.data_ptr(), xw.shape[0], row.data_ptr())
        ms.moe_spark_synchronize(ctx)
        ms.moe_spark_calibrate(ctx, True)
        ms.moe_spark_reset_stats(ctx)
        ms.moe_spark_set_trace(ctx, None, tr_k.data_ptr(), tr_g.data_ptr(), T)
        ms.moe_spark_decode_batched(ctx, xm.data_ptr(), 0, B, row.data_ptr())  # build the step graph
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms.moe_spark_decode_batched(ctx, xm.data_ptr(), T, B, row.data_ptr())
        ms.moe_spark_synchronize(ctx)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t1
        st = ms.moe_spark_get_stats(ctx)
        k = tr_k.cpu().numpy()
        distinct = sum(len(np.unique(k[t0:t0 + B, l])) for t0 in range(0, T, B) for l in range(w.L))
        steps = (T + B - 1) // B
        weight_bytes = distinct * EXPERT_BYTES + steps * w.L * w.E * w.d * 4
        gbps = weight_bytes / dt / 1e9
        xo = xm.cpu().numpy()
        out = dict(batch=B, ring_slots=R, tok_s=round(T / dt, 1), ms_per_step=round(dt * 1e3 / steps, 4),
                   **rates(st), fills=st["fills"],
                   distinct_experts_per_layer_step=round(distinct / (steps * w.L), 2),
                   algorithmic_bytes=weight_bytes, hbm_gbps=round(gbps, 1),
                   hbm_frac=round(gbps / HBM_PEAK_GBPS, 4),
                   max_rel_diff_to_batch1=None if ref_x is None else
                   float(f"{np.abs(xo - ref_x).max() / np.abs(ref_x).max():.3e}"),
                   traffic=batched_traffic(traffic_json, B),
                   arithmetic="Q4_0 codes as exact fp16 (q-8) x fp16 activations on the matrix cores, "
                              "fp32 accumulation, fp16 block scales applied in fp32")
        log(f"batched B={B}: {out['tok_s']} tok/s, {out['distinct_experts_per_layer_step']} distinct experts "
            f"per layer-step, {out['hbm_gbps']} GB/s algorithmic, cold {out['cold_hit_pct']}%, "
            f"max|x_B - x_1| / max|x_1| {out['max_rel_diff_to_batch1']}")
        return out
    finally:
        ms.moe_spark_destroy(ctx)


def run_prefill(ms, torch, model, P, R, warm, probe, layers, prefetch=False):
    """Batched prefill with a popularity shift, then recalibration; with
    prefetch, the next layer's predicted experts are copied during each
    layer's last chunk of cold experts."""
    import workload as wl
    wp = wl.prefill(layers)
    biases = [wp.bias_rows(l) for l in range(model.w.L)]  # rows: permutation A, permutation B
    X = wp.tokens()
    T = X.shape[0]
    rows = torch.from_numpy((np.arange(T) >= T // 2).astype(np.int32)).cuda()
    row_a = torch.zeros(max(warm.shape[0], probe.shape[0]), dtype=torch.int32, device="cuda")
    row_b = torch.ones_like(row_a)
    ctx = model.make_ctx(P=P, R=R, biases=biases, max_tokens=T)
    try:
        ms.moe_spark_set_prefetch(ctx, prefetch)
        xw = torch.from_numpy(warm).cuda()
        ms.moe_spark_decode(ctx, xw.data_ptr(), xw.shape[0], row_a.data_ptr())
        ms.moe_spark_calibrate(ctx, True)
        ms.moe_spark_reset_stats(ctx)
        xd = torch.from_numpy(X).cuda()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms.moe_spark_prefill(ctx, xd.data_ptr(), T, rows.data_ptr())
        ms.moe_spark_synchronize(ctx)
        dt = time.perf_counter() - t1
        st = ms.moe_spark_get_stats(ctx)

        def probe_decode():
            ms.moe_spark_reset_stats(ctx)
            xp = torch.from_numpy(probe).cuda()
            ms.moe_spark_decode(ctx, xp.data_ptr(), xp.shape[0], row_b.data_ptr())
            ms.moe_spark_synchronize(ctx)
            return rates(ms.moe_spark_get_stats(ctx))["cold_hit_pct"]

        before = probe_decode()
        ms.moe_spark_calibrate(ctx, True)
        after = probe_decode()
        gflop = 2.0 * T * model.w.K * (3 * model.w.d * model.w.f) * model.w.L / 1e9
        out = dict(tokens=T, layers=model.w.L, tok_s=round(T / dt, 1), ms=round(dt * 1e3, 3),
                   expert_gflop=round(gflop, 1), expert_tflops_end_to_end=round(gflop / dt / 1e3, 2),
                   accesses=st["accesses"], fills=st["fills"], evictions=st["evictions"],
                   prefetches=st["prefetches"], ring_hits=st["ring_hits"],
                   h2d_bytes=st["h2d_bytes"], cold_hit_pct=rates(st)["cold_hit_pct"],
                   probe_cold_hit_pct_before_recalibration=before,
                   probe_cold_hit_pct_after_recalibration=after,
                   arithmetic="Q4_0 codes as exact fp16 (q - 8), activations rounded once to fp16, "
                              "fp32 accumulation, fp16 block scales applied in fp32")
        log(f"prefill (prefetch {'on' if prefetch else 'off'}): {out['tok_s']} tok/s, fills {st['fills']}, "
            f"prefetches {st['prefetches']}, cold probe {before}% -> {after}%")
        return out
    finally:
        ms.moe_spark_destroy(ctx)


def run_autotune(ms, torch, model, P, R, warm, meas, layers, every=64, hyst=25, shift=1):
    """Decode through a popularity shift: calibrated on router bias row A,
    then `meas` tokens under row B, with the placement fixed and with online
    self-tuning (a step every `every` tokens)."""
    import workload as wl
    wp = wl.prefill(layers)
    biases = [wp.bias_rows(l) for l in range(model.w.L)]  # rows: permutation A, permutation B
    n_tail = meas.shape[0] // 4
    row_a = torch.zeros(warm.shape[0], dtype=torch.int32, device="cuda")
    row_b = torch.ones(meas.shape[0], dtype=torch.int32, device="cuda")
    out = {}
    for name, on in (("fixed", False), ("self_tuned", True)):
        ctx = model.make_ctx(P=P, R=R, biases=biases)
        try:
            xw = torch.from_numpy(warm).cuda()
            ms.moe_spark_decode(ctx, xw.data_ptr(), xw.shape[0], row_a.data_ptr())
            ms.moe_spark_calibrate(ctx, True)
            ms.moe_spark_reset_stats(ctx)
            if on:
                ms.moe_spark_set_autotune(ctx, every, hyst, shift)
            xm = torch.from_numpy(meas).cuda()
            head = meas.shape[0] - n_tail
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            ms.moe_spark_decode(ctx, xm.data_ptr(), head, row_b.data_ptr())
            ms.moe_spark_synchronize(ctx)
            s_head = ms.moe_spark_get_stats(ctx)
            ms.moe_spark_decode(ctx, xm[head:].data_ptr(), n_tail, row_b.data_ptr())
            ms.moe_spark_synchronize(ctx)
            dt = time.perf_counter() - t1
            st = ms.moe_spark_get_stats(ctx)
            tail = {k: st[k] - s_head[k] for k in ("accesses", "cold_hits")}
            out[name] = dict(tok_s=round(meas.shape[0] / dt, 1), **rates(st),
                             tail_tokens=n_tail,
                             tail_cold_hit_pct=round(100.0 * tail["cold_hits"] / max(tail["accesses"], 1), 4),
                             fills=st["fills"], retunes=st["retunes"], retune_swaps=st["retune_swaps"],
                             pinned_uploads=st["calib_uploads"])
            log(f"popularity shift, {name}: {out[name]['tok_s']} tok/s, cold {out[name]['cold_hit_pct']}% "
                f"(last {n_tail} tokens {out[name]['tail_cold_hit_pct']}%), {st['retunes']} steps, "
                f"{st['retune_swaps']} swaps")
        finally:
            ms.moe_spark_destroy(ctx)
    out["setting"] = dict(every_tokens=every, hysteresis_pct=hyst, decay_shift=shift,
                          calibrated_on="router bias row A", measured_on="row B")
    return out


def h2d_probe(torch, mib=256, reps=5):
    """Pinned host -> device copy rate (the cold-fill link)."""
    src = torch.empty(mib << 20, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    best = 1e9
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src, non_blocking=True)
        e1.record()
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1) / 1e3)
    return dict(bytes=mib << 20, gbps=round((mib << 20) / best / 1e9, 2))


def cpu_baseline(model, tokens, budget_s, single_tokens=1, prefill=None):
    """The fp64 oracle on a bounded sample of the same decode stream: on all
    host threads (OpenMP) and on one; with prefill = (X, bias rows per layer,
    token rows, n), also n tokens of the prefill batch through the stack
    (the oracle's prefill is the same per-token definition)."""
    import oracle
    w = model.w
    experts = [model.experts(l) for l in range(w.L)]

    def run(n_max, budget):
        n, t0 = 0, time.perf_counter()
        while n < n_max and (n < 1 or time.perf_counter() - t0 < budget):
            oracle.stack(tokens[n:n + 1].astype(np.float64), model.routers, model.biases, experts, K=w.K,
                         wfmt=w.wfmt, bias_row=np.zeros(1, np.int32))
            n += 1
        return n, time.perf_counter() - t0

    threads = oracle.num_threads()
    n, dt = run(tokens.shape[0], budget_s)
    oracle.set_num_threads(1)
    n1, dt1 = run(single_tokens, 0.0)
    oracle.set_num_threads(threads)
    model_name = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model_name = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    out = dict(value=round(n / dt, 3), unit="tok/s", cores=threads, kind="oracle",
               sample=f"{n} decode tokens of the {w.L}-layer stack (fp64, all layers) on {threads} threads, "
                      f"{dt:.1f} s of CPU work; {n1} token(s) on 1 thread, {dt1:.1f} s",
               single_thread_tok_s=round(n1 / dt1, 4), cpu_model=model_name,
               host_cpus=os.cpu_count())
    if prefill is not None:
        X, biases, rows, n_pf = prefill
        # tokens around the switch of router bias rows, so both rows are used
        t0 = max(0, X.shape[0] // 2 - n_pf // 2)
        sl = slice(t0, t0 + n_pf)
        tp = time.perf_counter()
        oracle.stack(X[sl].astype(np.float64), model.routers, biases, experts, K=w.K, wfmt=w.wfmt,
                     bias_row=rows[sl])
        dtp = time.perf_counter() - tp
        out["prefill_tok_s"] = round(n_pf / dtp, 3)
        out["prefill_sample"] = (f"tokens {t0}..{t0 + n_pf - 1} of the {X.shape[0]}-token prefill batch through "
                                 f"the {w.L}-layer stack on {threads} threads, {dtp:.1f} s")
    return out


def with_agent_fills(fn):
    """Run fn with contexts created under MOE_SPARK_PULL_FILLS=0: cold fills
    copied by the host fill agent (hipMemcpyAsync on the copy streams)."""
    old = os.environ.get("MOE_SPARK_PULL_FILLS")
    os.environ["MOE_SPARK_PULL_FILLS"] = "0"
    try:
        return fn()
    finally:
        if old is None:
            os.environ.pop("MOE_SPARK_PULL_FILLS", None)
        else:
            os.environ["MOE_SPARK_PULL_FILLS"] = old


def fill_path(ms, torch, model, P, R, calib, meas, row, full_tok_s, pulled_row):
    """Host-to-device rates of cold fills in the fill-bound 60%-uniform arm.
    Pulled fills (the default) have no copy of their own to time: their
    effective rate is the arm's fill bytes over the time the arm spends
    beyond full-residency decode of the same tokens.  Host-agent copies
    (MOE_SPARK_PULL_FILLS=0, read at context creation) report the agent's
    request-to-ready latency per fill."""
    out = {}
    if pulled_row is not None and full_tok_s:
        n = pulled_row["x_out"].shape[0]
        extra = pulled_row["elapsed_s"] - n / full_tok_s
        st = pulled_row["stats"]
        out["pulled"] = dict(fills=st["fills"], h2d_bytes=st["h2d_bytes"],
                             fills_per_token=round(st["fills"] / n, 2),
                             effective_gbps=round(st["h2d_bytes"] / extra / 1e9, 2) if extra > 0 else None,
                             us_per_fill=round(extra * 1e6 / max(st["fills"], 1), 2))
    r = with_agent_fills(lambda: run_decode(ms, torch, model, P, R, calib, None, meas, row, calibrate=False))
    st = r["stats"]
    out["agent"] = dict(tokens=meas.shape[0], tok_s=round(r["tok_s"], 2), fills=st["fills"],
                        h2d_bytes=st["h2d_bytes"],
                        gbps_per_fill=round(st["h2d_bytes"] / st["fill_ns_sum"], 2) if st["fill_ns_sum"] else None,
                        mean_fill_us=round(st["fill_ns_sum"] / max(st["fills"], 1) / 1e3, 2),
                        max_fill_us=round(st["fill_ns_max"] / 1e3, 2),
                        note="per fill: slot bytes over the agent's request-seen -> copy-landed time")
    log(f"fill path: pulled {out.get('pulled')}, agent {out['agent']}")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=STREAM_TOKENS, help="timed decode tokens of the headline")
    ap.add_argument("--warmup", type=int, default=16,
                    help="untimed decode tokens after calibration, before the timed ones")
    ap.add_argument("--calib-tokens", type=int, default=CALIB_TOKENS,
                    help="length of the warm-up trace the placement is calibrated from")
    ap.add_argument("--layers", type=int, default=40)
    ap.add_argument("--residency", type=float, default=0.6)
    ap.add_argument("--ring", type=int, default=32)
    ap.add_argument("--placement", choices=("calibrated", "uniform"), default="calibrated",
                    help="placement of the headline setting (uniform: the static-placement arm)")
    ap.add_argument("--no-full", action="store_true", help="skip the full-residency run")
    ap.add_argument("--no-sweep", action="store_true", help="skip the residency sweep")
    ap.add_argument("--no-prefill", action="store_true", help="skip the batched prefill")
    ap.add_argument("--no-autotune", action="store_true", help="skip the popularity-shift self-tuning runs")
    ap.add_argument("--no-fill-path", action="store_true", help="skip the fill-path leg")
    ap.add_argument("--batches", default="4,16",
                    help="batched decode step sizes to run beside batch 1 (empty: none)")
    ap.add_argument("--kernel-iters", type=int, default=10)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "gemv_traffic.json"))
    ap.add_argument("--copy-probe", action="store_true",
                    help="end with a 256 MiB device-to-device copy (a known-size kernel for "
                         "calibrating the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(each GPU would run its own decode stream with its own cache).", file=sys.stderr)
        sys.exit(2)

    import torch
    import workload as wl
    import resident_expert_caching_amd as ms

    w = wl.stack(args.layers)
    t0 = time.time()
    log(f"drawing {w.L * w.E} experts ({w.L * w.E * w.expert_bytes / 1e9:.1f} GB Q4_0)")
    model = Model(w)
    log(f"weights ready in {time.time() - t0:.1f}s")
    C = args.calib_tokens
    n_stream = max(args.steps, STREAM_TOKENS)
    toks = w.tokens(0, C + n_stream + args.warmup)
    calib = toks[:C]                               # t = 0..C-1: the calibration trace
    meas = toks[C:C + args.steps]                  # the headline's timed tokens
    stream = toks[C:C + STREAM_TOKENS]             # the fixed measured stream of the other legs
    untimed = toks[C + n_stream:C + n_stream + args.warmup]  # untimed warm-up tokens
    row = torch.zeros(max(C, n_stream, args.warmup, 1), dtype=torch.int32, device="cuda")
    LE = w.L * w.E
    P = int(round(args.residency * LE))
    R = args.ring if P < LE else 0

    full = None
    if not args.no_full and P < LE:
        full = run_decode(ms, torch, model, LE, 0, calib, untimed, meas, row, calibrate=False)
    part = run_decode(ms, torch, model, P, R, calib, untimed, meas, row,
                      calibrate=args.placement == "calibrated", kernel_iters=args.kernel_iters)

    st = part["stats"]
    us = part["us_gateup"]
    achieved = GATEUP_BYTES / (us * 1e-6) / 1e9
    traffic = None  # counter-measured HBM bytes, only while the kernel source is the one measured
    if os.path.exists(args.traffic_json):
        try:
            tj = json.load(open(args.traffic_json))
            h = hashlib.sha256()
            for f in tj.get("kernel_sources", []):
                h.update(open(os.path.join(ROOT, "resident_expert_caching_amd", "csrc", f), "rb").read())
            if tj.get("kernel_source_sha256") == h.hexdigest():
                traffic = tj.get("gateup_hbm_bytes_per_launch")
        except (OSError, ValueError):
            traffic = None
    token_gbps = TOKEN_BYTES_PER_LAYER * w.L * part["tok_s"] / 1e9
    res = {
        "metric": METRIC,
        "value": round(part["tok_s"], 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(part["ms_per_tok"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4_0*f16->f32",  # Q4_0 codes times fp16 activations, fp32 accumulation; router and norms fp32
        "data": "synthetic",
        "config": {
            "workload": f"{w.L}-layer Q4_0 MoE stack decode, batch 1: d=2048, 256 experts, top-8, "
                        f"SwiGLU f=512, Zipf-routed; {args.residency:.0%} residency "
                        f"(P={P} pinned slots) + {args.ring}-slot LRU ring, "
                        + (f"placement calibrated from a {C}-token warm-up trace" if args.placement == "calibrated"
                           else f"uniform static placement ({C}-token warm-up trace, no calibration)")
                        + f"; {args.warmup} untimed then {args.steps} timed decode tokens",
            "layers": w.L, "d_model": w.d, "experts": w.E, "top_k": w.K, "d_ff": w.f,
            "weights": "Q4_0", "resident_cap": P, "ring_slots": args.ring, "calibration_tokens": C,
            "placement": args.placement,
            "parallelism": "none (one GPU)",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "q4_gateup_kernel (router-partial reduce, top-8, gate+up GEMV of 8 Q4_0 "
                      "experts + SwiGLU)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "traffic_source": ("FETCH_SIZE + WRITE_SIZE counters per launch, scaled by a known-size copy, "
                               "from profiles/gemv_traffic.json (valid while the kernel sources hash to "
                               "the measured ones)") if traffic is not None else None,
            "algorithmic_bytes_per_launch": GATEUP_BYTES,
            "avg_launch_us": round(us, 3),
            "timing": f"HIP events on the compute stream around {args.kernel_iters} x {w.L} isolated "
                      f"replays of the kernel with each layer's last selection",
            "ceiling": {
                "kernel": "q4_stream_probe_kernel (the gate/up launch's grid and weight loads alone: "
                          "no routing, no arithmetic)",
                "bytes_per_launch": GATEUP_BYTES,
                "avg_launch_us": round(part["us_stream_probe"], 3),
                "gbps": round(GATEUP_BYTES / (part["us_stream_probe"] * 1e-6) / 1e9, 1),
                "frac": round(GATEUP_BYTES / (part["us_stream_probe"] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                "timing": "HIP events on the compute stream, back-to-back launches",
            },
            "down_kernel_us": round(part["us_down"], 3),
            "down_kernel_gbps": round(DOWN_BYTES / (part["us_down"] * 1e-6) / 1e9, 1),
            "token_algorithmic_bytes": TOKEN_BYTES_PER_LAYER * w.L,
            "token_gbps": round(token_gbps, 1),
            "token_frac": round(token_gbps / HBM_PEAK_GBPS, 4),
        },
        "fills": st["fills"],
        "h2d_bytes": st["h2d_bytes"],
    }
    res.update(rates(st))
    if full is not None:
        res["full_residency_tok_s"] = round(full["tok_s"], 2)
        res["ratio_to_full"] = round(part["tok_s"] / full["tok_s"], 4)
        res["bit_identical_to_full"] = bool(np.array_equal(full["x_out"], part["x_out"]))
        log(f"outputs bit-identical to full residency: {res['bit_identical_to_full']}")
    same_stream = args.steps == STREAM_TOKENS
    sweep_rows = {}
    if not args.no_sweep:
        rows = []
        for frac in (1.0, 0.6, 0.3):
            Pf = int(round(frac * LE))
            for calibrated in (False, True):
                if frac == 1.0 and calibrated:
                    continue
                if frac == 1.0 and full is not None and same_stream:
                    r = full
                elif frac == args.residency and calibrated == (args.placement == "calibrated") and same_stream:
                    r = part
                else:
                    r = run_decode(ms, torch, model, Pf, args.ring if Pf < LE else 0, calib, untimed, stream,
                                   row, calibrate=calibrated)
                sweep_rows[(frac, calibrated)] = r
                s = r["stats"]
                rows.append(dict(residency=frac, placement="calibrated" if calibrated else "uniform",
                                 resident_cap=Pf, tokens=STREAM_TOKENS, tok_s=round(r["tok_s"], 2), **rates(s),
                                 fills=s["fills"], h2d_bytes=s["h2d_bytes"],
                                 h2d_gbps=round(s["h2d_bytes"] / r["elapsed_s"] / 1e9, 3)))
        ref = sweep_rows[(1.0, False)]["x_out"]
        for r, key in zip(rows, [k for k in sweep_rows]):
            r["bit_identical"] = bool(np.array_equal(sweep_rows[key]["x_out"], ref))
        full_s = sweep_rows[(1.0, False)]["tok_s"]
        for r in rows:
            r["ratio_to_full"] = round(r["tok_s"] / full_s, 4)
        res["sweep"] = rows
    batches = [int(b) for b in args.batches.split(",") if b.strip()]
    if batches:
        ref = sweep_rows[(1.0, False)]["x_out"] if (1.0, False) in sweep_rows else None
        res["batched"] = [run_batched(ms, torch, model, P, max(R, b * w.K) if P < LE else 0, b, calib, stream, row,
                                      ref, args.traffic_json) for b in batches]
    if not args.no_fill_path and P < LE:
        full_s = sweep_rows[(1.0, False)]["tok_s"] if (1.0, False) in sweep_rows else None
        res["fill_path"] = fill_path(ms, torch, model, P, args.ring, calib, stream[:64], row,
                                     full_s, sweep_rows.get((args.residency, False)) if full_s else None)
        if "pulled" in res["fill_path"]:
            res["fill_path"]["pulled"]["tokens"] = sweep_rows[(args.residency, False)]["x_out"].shape[0]
        res["h2d_gbps_per_fill"] = {
            "pulled_effective": res["fill_path"].get("pulled", {}).get("effective_gbps"),
            "agent_copy": res["fill_path"]["agent"]["gbps_per_fill"],
        }
        # the headline protocol again, with the host agent's copies instead of pulled fills
        ag = with_agent_fills(lambda: run_decode(ms, torch, model, P, R, calib, untimed, meas, row,
                                                 calibrate=args.placement == "calibrated"))
        ra = rates(ag["stats"])
        res["fill_path"]["agent_headline"] = dict(
            tok_s=round(ag["tok_s"], 2), ratio_to_pulled=round(ag["tok_s"] / part["tok_s"], 4),
            fills=ag["stats"]["fills"], cold_hit_pct=ra["cold_hit_pct"],
            bit_identical_to_pulled=bool(np.array_equal(ag["x_out"], part["x_out"])),
            note="the headline's protocol and tokens, cold fills copied by the host agent")
    if not args.no_prefill:
        probe = wl.stack(args.layers).tokens(C + n_stream + args.warmup, 256)
        res["prefill"] = run_prefill(ms, torch, model, P, args.ring, calib, probe, args.layers)
        if P < LE:
            res["prefill_prefetch"] = run_prefill(ms, torch, model, P, args.ring, calib, probe, args.layers,
                                                  prefetch=True)
    if not args.no_autotune and P < LE:
        res["self_tuning"] = run_autotune(ms, torch, model, P, args.ring, calib, stream, args.layers)
    res["h2d_link"] = h2d_probe(torch)
    if "h2d_gbps_per_fill" in res:
        res["h2d_gbps_per_fill"]["link_probe"] = res["h2d_link"]["gbps"]
    if args.copy_probe:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_probe_bytes"] = src.numel() * 4
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample of the same stream")
        wp = wl.prefill(args.layers)
        Xp = wp.tokens()
        res["cpu_baseline"] = cpu_baseline(
            model, stream, args.cpu_budget,
            prefill=(Xp, [wp.bias_rows(l) for l in range(w.L)],
                     (np.arange(Xp.shape[0]) >= Xp.shape[0] // 2).astype(np.int32), 48))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

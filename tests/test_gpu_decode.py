"""GPU parity of the decode path through the C ABI against the CPU oracle.

Workloads (seeded, synthetic; see ``workload``): the tiny fp32 layer, the
target-shape Q4_0 layer (d=2048, 256 experts, top-8, f=512), and residual
stacks of target-shape layers with Zipf routing at several residencies.
"""
import numpy as np
import pytest
import torch

import oracle
import workload as wl
from spark_harness import (STAT_KEYS, TIE_GAP, Model, assert_outputs_close, events,
                           oracle_topk_and_gap, placement, sim_events)

pytestmark = pytest.mark.gpu

import resident_expert_caching_amd as ms  # noqa: E402  (a missing library fails collection: no silent skip)


def _dev(a, dtype=torch.float32):
    return torch.as_tensor(np.ascontiguousarray(a)).to(device="cuda", dtype=dtype)


def _layer_parity(model, ctx, x, flags, sample, norm, bias=None, bias_row=None, layer=0):
    """Run moe_spark_layer_forward over all tokens of x; check top-k on every
    token and outputs on `sample` tokens."""
    w = model.w
    T = x.shape[0]
    xd = _dev(x)
    yd = torch.empty_like(xd)
    topk = torch.empty((T, w.K), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, w.K), dtype=torch.float32, device="cuda")
    br = None if bias_row is None else _dev(bias_row, torch.int32)
    ms.moe_spark_layer_forward(ctx, layer, xd.data_ptr(), yd.data_ptr(), T,
                               None if br is None else br.data_ptr(), flags, topk.data_ptr(),
                               gates.data_ptr())
    ms.moe_spark_synchronize(ctx)
    y = yd.cpu().numpy()
    idx = topk.cpu().numpy()
    g = gates.cpu().numpy()
    wr = model.routers[layer]
    ties = 0
    forced = np.full((T, w.K), -1, np.int32)
    for t in range(T):
        u = oracle.rmsnorm(x[t]) if norm else x[t].astype(np.float64)
        b = None if bias is None else bias[0 if bias_row is None else bias_row[t]]
        lg = oracle.router(wr, u, b)
        ref_idx, gap = oracle_topk_and_gap(lg, w.K)
        if gap < TIE_GAP:
            ties += 1
            forced[t] = idx[t]
        else:
            assert np.array_equal(idx[t], ref_idx), (t, idx[t], ref_idx)
    assert ties <= max(1, T // 50)
    experts = model.experts(layer)
    xs = x[sample].astype(np.float64)
    yref, iref, gref, _ = oracle.layer(xs, wr, experts, K=w.K, wfmt=w.wfmt, norm=norm,
                                       bias=bias, bias_row=None if bias_row is None else bias_row[sample],
                                       forced=forced[sample])
    if flags & ms.RESIDUAL:
        yref = yref + xs
        rel = assert_outputs_close(y[sample] - xs, yref - xs, "layer output")
    else:
        rel = assert_outputs_close(y[sample], yref, "layer output")
    np.testing.assert_allclose(g[sample], gref, rtol=2e-5, atol=1e-6)
    assert np.abs(g.sum(axis=1) - 1).max() <= 1e-6
    return y, idx, rel


def test_tiny_fp32_layer():
    w = wl.tiny()
    model = Model(w)
    ctx = model.make_ctx(P=w.E, R=0)
    try:
        x = w.tokens()
        print("tiny layer: 64 tokens, d=256, 16 experts, top-2", flush=True)
        y, idx, rel = _layer_parity(model, ctx, x, 0, np.arange(64), norm=False)
        st = ms.moe_spark_get_stats(ctx)
        assert st["accesses"] == 64 * 2 and st["pinned_hits"] == 128 and st["cold_hits"] == 0
        print(f"tiny layer rel err {rel:.2e}")
    finally:
        ms.moe_spark_destroy(ctx)


def test_tiny_fp32_layer_partial_residency():
    """The fp32 layer at 50% and 0% residency with a ring of 2 (every cold
    expert goes through host-agent fills): outputs bit-identical to full
    residency, bookkeeping equal to the simulator."""
    w = wl.tiny()
    model = Model(w)
    x = w.tokens()
    T = x.shape[0]
    outs = {}
    for P, R in [(w.E, 0), (w.E // 2, 2), (0, 2)]:
        ctx = model.make_ctx(P=P, R=R)
        try:
            print(f"tiny layer at P={P}, R={R}", flush=True)
            xd = _dev(x)
            yd = torch.empty_like(xd)
            topk = torch.empty((T, w.K), dtype=torch.int32, device="cuda")
            gates = torch.empty((T, w.K), dtype=torch.float32, device="cuda")
            ms.moe_spark_layer_forward(ctx, 0, xd.data_ptr(), yd.data_ptr(), T, None, 0, topk.data_ptr(),
                                       gates.data_ptr())
            ms.moe_spark_synchronize(ctx)
            outs[P] = yd.cpu().numpy()
            idx = topk.cpu().numpy()
            sim = oracle.Sim(1, w.E, P, R, ms.moe_spark_slot_bytes(ctx))
            sim.place_uniform()
            for t in range(T):
                sim.decode_layer(0, idx[t])
            st = ms.moe_spark_get_stats(ctx)
            assert {k: st[k] for k in STAT_KEYS} == sim.stats()
            assert events(ctx) == sim_events(sim)
            for got, ref in zip(placement(ctx, w, R), sim.placement()):
                assert np.array_equal(got, ref)
            if P < w.E:
                assert st["fills"] > 0 and st["evictions"] > 0
        finally:
            ms.moe_spark_destroy(ctx)
    assert np.array_equal(outs[w.E], outs[w.E // 2]) and np.array_equal(outs[w.E], outs[0])


def test_target_layer_q4_0_full_residency():
    w = wl.layer()
    model = Model(w)
    ctx = model.make_ctx(P=w.E, R=0)
    try:
        x = w.tokens()
        sample = np.array([0, 1, 2, 3, 50, 77, 128, 200, 254, 255])
        print("target layer: 256 tokens, d=2048, 256 experts, top-8, Q4_0", flush=True)
        y, idx, rel = _layer_parity(model, ctx, x, ms.PRE_RMSNORM, sample, norm=True)
        counts = placement(ctx, w, 0)[3]
        assert counts.sum() == 256 * 8
        assert np.array_equal(np.bincount(idx.ravel(), minlength=w.E), counts[0])
        print(f"target layer rel err {rel:.2e}")
    finally:
        ms.moe_spark_destroy(ctx)


def test_target_layer_partial_residency_is_bit_identical():
    """The same 64 tokens at 100% and at 60% residency (uniform placement, a
    ring of 8 slots, so most cold experts are filled and evicted): outputs
    bit-identical, bookkeeping equal to the simulator."""
    w = wl.layer()
    model = Model(w)
    x = w.tokens(0, 64)
    outs = {}
    for P, R in [(256, 0), (154, 8), (0, 8)]:
        ctx = model.make_ctx(P=P, R=R)
        try:
            print(f"target layer at P={P}, R={R}", flush=True)
            xd = _dev(x)
            yd = torch.empty_like(xd)
            topk = torch.empty((64, w.K), dtype=torch.int32, device="cuda")
            gates = torch.empty((64, w.K), dtype=torch.float32, device="cuda")
            ms.moe_spark_layer_forward(ctx, 0, xd.data_ptr(), yd.data_ptr(), 64, None,
                                       ms.PRE_RMSNORM | ms.RESIDUAL, topk.data_ptr(),
                                       gates.data_ptr())
            ms.moe_spark_synchronize(ctx)
            outs[P] = yd.cpu().numpy()
            idx = topk.cpu().numpy()
            sim = oracle.Sim(1, w.E, P, R, ms.moe_spark_slot_bytes(ctx))
            sim.place_uniform()
            for t in range(64):
                sim.decode_layer(0, idx[t])
            st = ms.moe_spark_get_stats(ctx)
            ss = sim.stats()
            assert {k: st[k] for k in STAT_KEYS} == ss
            assert events(ctx) == sim_events(sim)
            so, ow, stp, cnt = placement(ctx, w, R)
            sso, sow, sstp, scnt = sim.placement()
            assert np.array_equal(so, sso) and np.array_equal(ow, sow)
            assert np.array_equal(stp, sstp) and np.array_equal(cnt, scnt)
            if P < 256:
                assert ss["fills"] > 0 and ss["evictions"] > 0
        finally:
            ms.moe_spark_destroy(ctx)
    assert np.array_equal(outs[256], outs[154]) and np.array_equal(outs[256], outs[0])


def _small_stack(L=4, E=32):
    return wl.Workload("small-stack", d=2048, E=E, K=8, f=512, L=L, wfmt=wl.FMT_Q4_0, norm=True,
                       seed=2, n_tokens=80, token_stream=2, bias_seeds=(2,), warmup=32)


def _run_stack(model, P, R, calibrated, x_warm, x_meas):
    """Warm-up under uniform placement, optional calibration, then the
    measured tokens; both phases traced.  Returns outputs, traces, stats."""
    w = model.w
    Tw, Tm = x_warm.shape[0], x_meas.shape[0]
    ctx = model.make_ctx(P=P, R=R)
    try:
        cap = Tw + Tm
        tr_x = torch.zeros((cap, w.L, w.d), dtype=torch.float32, device="cuda")
        tr_k = torch.zeros((cap, w.L, w.K), dtype=torch.int32, device="cuda")
        tr_g = torch.zeros((cap, w.L, w.K), dtype=torch.float32, device="cuda")
        ms.moe_spark_set_trace(ctx, tr_x.data_ptr(), tr_k.data_ptr(), tr_g.data_ptr(), cap)
        xw = _dev(x_warm)
        xm = _dev(x_meas)
        row = torch.zeros(max(Tw, Tm), dtype=torch.int32, device="cuda")
        ms.moe_spark_decode(ctx, xw.data_ptr(), Tw, row.data_ptr())
        ms.moe_spark_synchronize(ctx)
        if calibrated:
            ms.moe_spark_calibrate(ctx, True)
        ms.moe_spark_reset_stats(ctx)
        ms.moe_spark_decode(ctx, xm.data_ptr(), Tm, row.data_ptr())
        ms.moe_spark_synchronize(ctx)
        out = dict(x_warm=xw.cpu().numpy(), x_meas=xm.cpu().numpy(), tr_x=tr_x.cpu().numpy(),
                   tr_k=tr_k.cpu().numpy(), tr_g=tr_g.cpu().numpy(),
                   stats=ms.moe_spark_get_stats(ctx), events=events(ctx),
                   placement=placement(ctx, w, R), slot_bytes=ms.moe_spark_slot_bytes(ctx))
        return out
    finally:
        ms.moe_spark_destroy(ctx)


def test_stack_residency_sweep_bit_identical_and_bookkeeping_exact():
    w = _small_stack()
    model = Model(w)
    x_all = w.tokens(0, 80)
    x_warm, x_meas = x_all[:32], x_all[32:]
    LE = w.L * w.E
    R = 8
    runs = {}
    for frac in (1.0, 0.6, 0.3):
        P = int(round(frac * LE))
        for calibrated in (False, True):
            if frac == 1.0 and calibrated:
                continue
            print(f"stack L={w.L} E={w.E}: P={P} R={R} calibrated={calibrated}", flush=True)
            r = _run_stack(model, P, R if P < LE else 0, calibrated, x_warm, x_meas)
            runs[(P, calibrated)] = r
            # bookkeeping: replay the GPU's own top-k trace through the simulator
            sim = oracle.Sim(w.L, w.E, P, R if P < LE else 0, r["slot_bytes"])
            sim.place_uniform()
            for t in range(32):
                sim.decode_token(r["tr_k"][t])
            if calibrated:
                sim.calibrate(True)
            sim.reset_stats()
            for t in range(32, 80):
                sim.decode_token(r["tr_k"][t])
            st = r["stats"]
            assert {k: st[k] for k in STAT_KEYS} == sim.stats(), (st, sim.stats())
            assert st["tokens"] == 48
            assert r["events"] == sim_events(sim)
            so, ow, stp, cnt = r["placement"]
            sso, sow, sstp, scnt = sim.placement()
            assert np.array_equal(so, sso) and np.array_equal(ow, sow)
            assert np.array_equal(stp, sstp) and np.array_equal(cnt, scnt)
    base = runs[(LE, False)]
    for key, r in runs.items():
        assert np.array_equal(r["x_meas"], base["x_meas"]), key
        assert np.array_equal(r["x_warm"], base["x_warm"]), key
        assert np.array_equal(r["tr_k"], base["tr_k"]), key
    cold = {k: v["stats"]["cold_hits"] / v["stats"]["accesses"] for k, v in runs.items()}
    print("cold-hit rates", cold)
    P60 = int(round(0.6 * LE))
    assert cold[(P60, True)] < cold[(P60, False)]  # calibration lowers the cold-hit rate
    # teacher-forced per-layer output parity on sampled tokens
    r = base
    tr_x, tr_k = r["tr_x"], r["tr_k"]
    x_final = np.concatenate([r["x_warm"], r["x_meas"]])
    for t in (0, 31, 32, 79):
        for l in range(w.L):
            xl = tr_x[t, l].astype(np.float64)
            xn = (tr_x[t, l + 1] if l + 1 < w.L else x_final[t]).astype(np.float64)
            lg = oracle.router(model.routers[l], oracle.rmsnorm(xl), model.biases[l][0])
            ref_idx, gap = oracle_topk_and_gap(lg, w.K)
            forced = tr_k[t, l][None] if gap < TIE_GAP else None
            if forced is None:
                assert np.array_equal(tr_k[t, l], ref_idx), (t, l)
            yref, _, _, _ = oracle.layer(xl[None], model.routers[l], model.experts(l), K=w.K,
                                         wfmt=w.wfmt, norm=True, bias=model.biases[l],
                                         bias_row=np.zeros(1, np.int32), forced=forced)
            assert_outputs_close(xn - xl, yref[0], f"token {t} layer {l}")

"""GPU edge cases of the Q4_0 path through the C ABI, checked against the
oracle and the placement simulator.

 * top-k extremes and expert counts that are not a multiple of the 64-expert
   ranking chunk: (E, K) = (16, 1), (100, 2), (100, 8), and E = 1024, the
   largest supported;
 * no pinned slot at all (every access goes through a ring of exactly K
   slots) next to full residency: bit-identical outputs;
 * prefill of a single token, and prefills whose layers need many ring
   chunks (far more cold experts than ring slots);
 * error paths: prefill beyond max_tokens, prefill without prefill buffers,
   forward before placement;
 * decode fills pulled by the kernels against fills copied by the host agent;
 * an expert updated after placement while it sits in a ring slot;
 * the measurement calls leave decode's results alone;
 * zero-token calls change nothing.
"""
import numpy as np
import pytest
import torch

import oracle
import workload as wl
from spark_harness import (STAT_KEYS, TIE_GAP, Model, events, oracle_topk_and_gap, placement,
                           sim_events)

pytestmark = pytest.mark.gpu

import resident_expert_caching_amd as ms  # noqa: E402  (a missing library fails collection: no silent skip)


def _wl(E, K, L=1, n_tokens=24, bias=True):
    return wl.Workload(f"edge-E{E}-K{K}", d=2048, E=E, K=K, f=512, L=L, wfmt=wl.FMT_Q4_0, norm=True,
                       seed=5 + E + K, n_tokens=n_tokens, token_stream=9,
                       bias_seeds=(3, 1003) if bias else ())


def _layer_run(model, P, R, x):
    w = model.w
    T = x.shape[0]
    ctx = model.make_ctx(P=P, R=R)
    try:
        xd = torch.from_numpy(x.copy()).cuda()
        yd = torch.empty_like(xd)
        topk = torch.empty((T, w.K), dtype=torch.int32, device="cuda")
        gates = torch.empty((T, w.K), dtype=torch.float32, device="cuda")
        rows = torch.from_numpy((np.arange(T) % 2).astype(np.int32)).cuda()
        ms.moe_spark_layer_forward(ctx, 0, xd.data_ptr(), yd.data_ptr(), T, rows.data_ptr(),
                                   ms.PRE_RMSNORM | ms.RESIDUAL, topk.data_ptr(), gates.data_ptr())
        ms.moe_spark_synchronize(ctx)
        return dict(y=yd.cpu().numpy(), topk=topk.cpu().numpy(), gates=gates.cpu().numpy(),
                    stats=ms.moe_spark_get_stats(ctx), events=events(ctx),
                    placement=placement(ctx, w, R), slot_bytes=ms.moe_spark_slot_bytes(ctx))
    finally:
        ms.moe_spark_destroy(ctx)


@pytest.mark.parametrize("E,K", [(16, 1), (100, 2), (100, 8), (1024, 8)])
def test_layer_extremes_against_oracle_and_simulator(E, K):
    w = _wl(E, K)
    model = Model(w)
    x = w.tokens()
    T = x.shape[0]
    rows = (np.arange(T) % 2).astype(np.int32)
    print(f"layer E={E} K={K}: full residency and no pinned slot (ring of {K})", flush=True)
    full = _layer_run(model, E, 0, x)
    none = _layer_run(model, 0, K, x)
    assert np.array_equal(full["y"], none["y"]) and np.array_equal(full["topk"], none["topk"])
    assert none["stats"]["pinned_hits"] == 0 and none["stats"]["cold_hits"] == T * K
    # bookkeeping of the ring-only run
    sim = oracle.Sim(1, E, 0, K, none["slot_bytes"])
    sim.place_uniform()
    for t in range(T):
        sim.decode_layer(0, none["topk"][t])
    assert {k: none["stats"][k] for k in STAT_KEYS} == sim.stats()
    assert none["events"] == sim_events(sim)
    for got, ref in zip(none["placement"], sim.placement()):
        assert np.array_equal(got, ref)
    # routing and outputs against the oracle
    wr, bias = model.routers[0], model.biases[0]
    forced = np.full((T, K), -1, np.int32)
    for t in range(T):
        lg = oracle.router(wr, oracle.rmsnorm(x[t]), bias[rows[t]])
        ref_idx, gap = oracle_topk_and_gap(lg, K)
        if gap < TIE_GAP:
            forced[t] = full["topk"][t]
        else:
            assert np.array_equal(full["topk"][t], ref_idx), (t, full["topk"][t], ref_idx)
    if K == 1:
        assert np.all(full["gates"] == 1.0)
    assert np.abs(full["gates"].sum(axis=1) - 1).max() <= 1e-6
    sample = np.arange(0, T, 3)
    yref, _, gref, _ = oracle.layer(x[sample].astype(np.float64), wr, model.experts(0), K=K,
                                    wfmt=w.wfmt, norm=True, bias=bias, bias_row=rows[sample],
                                    forced=forced[sample])
    np.testing.assert_allclose(full["gates"][sample], gref, rtol=2e-5, atol=1e-6)
    got = full["y"][sample].astype(np.float64) - x[sample]
    err = np.abs(got - yref).max()
    assert err <= 2e-3 * np.abs(yref).max(), err


def _prefill_run(model, P, R, x, rows, max_tokens):
    w = model.w
    T = x.shape[0]
    ctx = model.make_ctx(P=P, R=R, max_tokens=max_tokens)
    try:
        tr_x = torch.zeros((T, w.L, w.d), dtype=torch.float32, device="cuda")
        tr_k = torch.zeros((T, w.L, w.K), dtype=torch.int32, device="cuda")
        tr_g = torch.zeros((T, w.L, w.K), dtype=torch.float32, device="cuda")
        ms.moe_spark_set_trace(ctx, tr_x.data_ptr(), tr_k.data_ptr(), tr_g.data_ptr(), T)
        xd = torch.from_numpy(x.copy()).cuda()
        rd = torch.from_numpy(rows).cuda()
        ms.moe_spark_prefill(ctx, xd.data_ptr(), T, rd.data_ptr())
        ms.moe_spark_synchronize(ctx)
        return dict(x=xd.cpu().numpy(), tr_x=tr_x.cpu().numpy(), tr_k=tr_k.cpu().numpy(),
                    stats=ms.moe_spark_get_stats(ctx), events=events(ctx),
                    placement=placement(ctx, w, R), slot_bytes=ms.moe_spark_slot_bytes(ctx))
    finally:
        ms.moe_spark_destroy(ctx)


@pytest.mark.parametrize("T", [1, 130])
def test_prefill_ring_only_many_chunks(T):
    """E = 100 experts per layer, nothing pinned, a ring of K = 8 slots: a
    layer's distinct experts stream through the ring in many chunks."""
    w = _wl(100, 8, L=2, n_tokens=T)
    model = Model(w)
    x = w.tokens()
    rows = (np.arange(T) >= T // 2).astype(np.int32)
    print(f"prefill T={T}: full residency vs ring only", flush=True)
    full = _prefill_run(model, w.L * w.E, 0, x, rows, max_tokens=max(T, 4))
    ring = _prefill_run(model, 0, 8, x, rows, max_tokens=T)
    assert np.array_equal(full["x"], ring["x"]) and np.array_equal(full["tr_k"], ring["tr_k"])
    sim = oracle.Sim(w.L, w.E, 0, 8, ring["slot_bytes"])
    sim.place_uniform()
    for l in range(w.L):
        sim.prefill_layer(l, ring["tr_k"][:, l, :])
    assert {k: ring["stats"][k] for k in STAT_KEYS} == sim.stats()
    assert ring["events"] == sim_events(sim)
    for got, ref in zip(ring["placement"], sim.placement()):
        assert np.array_equal(got, ref)
    distinct = sum(len(np.unique(ring["tr_k"][:, l, :])) for l in range(w.L))
    assert ring["stats"]["accesses"] == distinct and ring["stats"]["pinned_hits"] == 0
    # teacher-forced output of the last layer on a few tokens
    l = w.L - 1
    for t in sorted({0, T // 2, T - 1}):
        xl = full["tr_x"][t, l].astype(np.float64)
        lg = oracle.router(model.routers[l], oracle.rmsnorm(xl), model.biases[l][rows[t]])
        ref_idx, gap = oracle_topk_and_gap(lg, w.K)
        forced = full["tr_k"][t, l][None] if gap < TIE_GAP else None
        if forced is None:
            assert np.array_equal(full["tr_k"][t, l], ref_idx)
        yref, _, _, _ = oracle.layer(xl[None], model.routers[l], model.experts(l), K=w.K, wfmt=w.wfmt,
                                     norm=True, bias=model.biases[l], bias_row=rows[t:t + 1], forced=forced)
        err = np.abs((full["x"][t].astype(np.float64) - xl) - yref[0]).max()
        assert err <= 2e-3 * np.abs(yref[0]).max(), (t, err)


def test_error_paths():
    w = _wl(16, 2, n_tokens=8)
    model = Model(w)
    x = torch.zeros((8, w.d), dtype=torch.float32, device="cuda")
    ctx = model.make_ctx(P=16, R=0, max_tokens=4)
    try:
        with pytest.raises(ms.MoeSparkError) as ei:
            ms.moe_spark_prefill(ctx, x.data_ptr(), 5, None)
        assert ei.value.status == ms.E_INVALID
        with pytest.raises(ms.MoeSparkError) as ei:
            ms.moe_spark_prefill(ctx, x.data_ptr(), 0, None)
        assert ei.value.status == ms.E_INVALID
    finally:
        ms.moe_spark_destroy(ctx)
    ctx = model.make_ctx(P=16, R=0, max_tokens=0)
    try:
        with pytest.raises(ms.MoeSparkError) as ei:
            ms.moe_spark_prefill(ctx, x.data_ptr(), 1, None)
        assert ei.value.status == ms.E_STATE
    finally:
        ms.moe_spark_destroy(ctx)
    # forward before any placement
    ctx = ms.moe_spark_create(ms.Config(n_layers=1, d_model=2048, n_experts=16, top_k=2, d_ff=512,
                                        wfmt=ms.W_Q4_0, rms_eps=1e-6, n_bias_rows=0, resident_cap=16,
                                        ring_slots=0, max_tokens=0, event_cap=0))
    try:
        with pytest.raises(ms.MoeSparkError) as ei:
            ms.moe_spark_layer_forward(ctx, 0, x.data_ptr(), x.data_ptr(), 1, None, 0, None, None)
        assert ei.value.status == ms.E_STATE
        with pytest.raises(ms.MoeSparkError) as ei:
            ms.moe_spark_decode(ctx, x.data_ptr(), 1, None)
        assert ei.value.status == ms.E_STATE
    finally:
        ms.moe_spark_destroy(ctx)


def test_pulled_and_agent_fills_agree(monkeypatch):
    """Decode fills pulled by the kernels (the default) and fills copied by the
    host agent (MOE_SPARK_PULL_FILLS=0, read at context creation) give the
    same outputs, counters, fill log and placement: every access goes
    through a ring of K = 8 slots."""
    w = _wl(100, 8)
    model = Model(w)
    x = w.tokens()
    print("ring-only layer: pulled fills, then agent fills", flush=True)
    pulled = _layer_run(model, 0, 8, x)
    monkeypatch.setenv("MOE_SPARK_PULL_FILLS", "0")
    agent = _layer_run(model, 0, 8, x)
    assert np.array_equal(pulled["y"], agent["y"]) and np.array_equal(pulled["topk"], agent["topk"])
    assert {k: pulled["stats"][k] for k in STAT_KEYS} == {k: agent["stats"][k] for k in STAT_KEYS}
    assert pulled["stats"]["fills"] > 0
    assert pulled["events"] == agent["events"]
    for a, b in zip(pulled["placement"], agent["placement"]):
        assert np.array_equal(a, b)


def test_expert_update_reaches_ring_copies():
    """moe_spark_set_expert after placement: an expert that sits in a ring
    slot is refreshed there too, so decode after the update gives the same
    bits at 60% residency (the expert ring-resident) as at full residency,
    and differs from decode without the update."""
    w = _wl(32, 8, L=2, n_tokens=32)
    model = Model(w)
    x = w.tokens()
    LE = w.L * w.E
    P60, R = int(round(0.6 * LE)), 8
    row = torch.zeros(32, dtype=torch.int32, device="cuda")

    def run(P, Rr, key=None, new=None):
        ctx = model.make_ctx(P=P, R=Rr)
        try:
            xa = torch.from_numpy(x[:16].copy()).cuda()
            xb = torch.from_numpy(x[16:].copy()).cuda()
            print(f"update test: P={P} R={Rr} key={key}", flush=True)
            ms.moe_spark_decode(ctx, xa.data_ptr(), 16, row.data_ptr())
            ms.moe_spark_synchronize(ctx)
            pl = placement(ctx, w, Rr)
            if key is not None:
                l, e = divmod(key, w.E)
                g, u, d = new
                ms.moe_spark_set_expert(ctx, l, e, g.ctypes.data, u.ctypes.data, d.ctypes.data)
            ms.moe_spark_decode(ctx, xb.data_ptr(), 16, row.data_ptr())
            ms.moe_spark_synchronize(ctx)
            return xb.cpu().numpy(), pl, ms.moe_spark_get_stats(ctx)
        finally:
            ms.moe_spark_destroy(ctx)

    _, (slot_of, owner, _, counts), _ = run(P60, R)
    ring = [int(k) for k in owner if k >= 0]
    assert ring, "no expert reached the ring"
    key = max(ring, key=lambda k: counts.reshape(-1)[k])  # the most-used ring resident
    assert slot_of.reshape(-1)[key] < 0
    # new weights: another expert's (a different layer's) bytes
    src = (key + w.E // 2) % LE
    new = tuple(np.ascontiguousarray(a) for a in wl.split_expert(model.blob[src], w.d, w.f, w.wfmt))
    y60, (_, owner2, _, _), st = run(P60, R, key, new)
    assert key in [int(k) for k in owner2] or st["fills"] > 0
    y100, _, _ = run(LE, 0, key, new)
    y_old, _, _ = run(LE, 0)
    assert np.array_equal(y60, y100)
    assert not np.array_equal(y100, y_old), "the updated expert was not used after the update"


def test_timing_calls_leave_outputs_alone():
    """The measurement calls (isolated kernel replays, the streaming probe)
    return finite positive times and do not change what decode computes; the
    streaming probe reads Q4_0 slots only."""
    w = _wl(16, 2, L=2, n_tokens=8)
    model = Model(w)
    x = w.tokens(0, 8)
    row = torch.zeros(8, dtype=torch.int32, device="cuda")
    outs = []
    for timed in (False, True):
        ctx = model.make_ctx(P=16 * 2, R=0)
        try:
            xa = torch.from_numpy(x[:4].copy()).cuda()
            ms.moe_spark_decode(ctx, xa.data_ptr(), 4, row.data_ptr())
            ms.moe_spark_synchronize(ctx)
            if timed:
                times = ms.moe_spark_time_expert_kernels(ctx, 2) + (ms.moe_spark_time_stream_probe(ctx, 4),)
                assert all(np.isfinite(t) and t > 0 for t in times), times
                with pytest.raises(ms.MoeSparkError) as ei:
                    ms.moe_spark_time_stream_probe(ctx, 0)
                assert ei.value.status == ms.E_INVALID
            xb = torch.from_numpy(x[4:].copy()).cuda()
            ms.moe_spark_decode(ctx, xb.data_ptr(), 4, row.data_ptr())
            ms.moe_spark_synchronize(ctx)
            outs.append((xa.cpu().numpy(), xb.cpu().numpy()))
        finally:
            ms.moe_spark_destroy(ctx)
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    wf = wl.tiny()
    ctx = Model(wf).make_ctx(P=wf.E, R=0)
    try:
        with pytest.raises(ms.MoeSparkError) as ei:
            ms.moe_spark_time_stream_probe(ctx, 1)
        assert ei.value.status == ms.E_INVALID
    finally:
        ms.moe_spark_destroy(ctx)


def test_zero_token_calls_change_nothing():
    """Empty inputs: decode, layer forward and the no-alloc layer forward
    with zero tokens leave the buffers, the counters and the placement as
    they were, and the next real token decodes as in a fresh context."""
    w = _wl(16, 2, L=2, n_tokens=4)
    model = Model(w)
    x = w.tokens(0, 1)
    outs = []
    for empty_first in (False, True):
        ctx = model.make_ctx(P=8, R=4)
        try:
            xd = torch.from_numpy(x.copy()).cuda()
            if empty_first:
                y = torch.full_like(xd, 7.0)
                ms.moe_spark_decode(ctx, xd.data_ptr(), 0, None)
                ms.moe_spark_layer_forward(ctx, 0, xd.data_ptr(), y.data_ptr(), 0, None,
                                           ms.PRE_RMSNORM | ms.RESIDUAL, None, None)
                ms.moe_spark_layer_forward_noalloc(ctx, 1, xd.data_ptr(), y.data_ptr(), 0, None,
                                                   ms.PRE_RMSNORM | ms.RESIDUAL, None, None)
                ms.moe_spark_synchronize(ctx)
                assert np.array_equal(xd.cpu().numpy(), x) and bool((y == 7.0).all())
                st = ms.moe_spark_get_stats(ctx)
                assert all(st[k] == 0 for k in STAT_KEYS if k in st), st
            ms.moe_spark_decode(ctx, xd.data_ptr(), 1, None)
            ms.moe_spark_synchronize(ctx)
            st = ms.moe_spark_get_stats(ctx)
            outs.append((xd.cpu().numpy(), {k: st[k] for k in STAT_KEYS}, placement(ctx, w, 4)))
        finally:
            ms.moe_spark_destroy(ctx)
    assert np.array_equal(outs[0][0], outs[1][0])
    assert outs[0][1] == outs[1][1]
    for a, b in zip(outs[0][2], outs[1][2]):
        assert np.array_equal(a, b)

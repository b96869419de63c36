"""Batched decode (moe_spark_decode_batched) through the C ABI.

A 4-layer stack of the target layer shape (d=2048, 64 experts, top-8, f=512,
Q4_0, Zipf-biased router) decodes 32 warm-up tokens batch-1 under uniform
placement, is calibrated, and then decodes 45 tokens in steps of B tokens
(45 is a whole number of steps for B = 1, 3 and ragged for B = 8, 16):

 * top-k is identical to batch-1 decode of the same tokens at full residency
   and outputs agree with it to fp32 rounding (the matrix cores sum in
   another order than the batch-1 dot products);
 * outputs are bit-identical for every batch size (a token's result does not
   depend on the tokens that share its step);
 * bookkeeping — counters, fill/eviction log, pinned set, ring, counts —
   equals the simulator replaying the GPU's own top-k trace with each step's
   accesses in (layer, token, rank) order;
 * sampled (token, layer) outputs match the fp64 oracle, teacher-forced;
 * at 100/60/30% residency with uniform placement and the smallest ring a
   step allows (R = B*K, so one step can turn the whole ring over), with
   pulled and with host-agent fills, outputs stay bit-identical to the other
   batched runs and bookkeeping exact.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import workload as wl
from spark_harness import (STAT_KEYS, TIE_GAP, Model, assert_outputs_close, events,
                           oracle_topk_and_gap, placement, sim_events)

pytestmark = pytest.mark.gpu

import resident_expert_caching_amd as ms  # noqa: E402  (a missing library fails collection: no silent skip)

WARM, MEAS = 32, 45
BATCH1_TOL = 2e-3  # max|batched - batch-1| / max|batch-1|: the parity bar; both paths also meet it against the oracle
_BATCHED = {}      # the first batched run's outputs: every other batched run must match them bitwise


@pytest.fixture(scope="module")
def model():
    w = wl.Workload("batched-L4-E64", d=2048, E=64, K=8, f=512, L=4, wfmt=wl.FMT_Q4_0, norm=True,
                    seed=51, n_tokens=WARM + MEAS, token_stream=53, bias_seeds=(5,))
    return Model(w)


def _run(model, P, R, B, calibrate=True, pull=True):
    """Warm-up batch-1, optional calibration, measured tokens in steps of B
    (B = 0: batch-1 decode).  Traced."""
    w = model.w
    x = w.tokens(0, WARM + MEAS)
    old = os.environ.get("MOE_SPARK_PULL_FILLS")
    os.environ["MOE_SPARK_PULL_FILLS"] = "1" if pull else "0"
    try:
        ctx = model.make_ctx(P=P, R=R)
    finally:
        if old is None:
            del os.environ["MOE_SPARK_PULL_FILLS"]
        else:
            os.environ["MOE_SPARK_PULL_FILLS"] = old
    try:
        cap = WARM + MEAS
        tr_x = torch.zeros((cap, w.L, w.d), dtype=torch.float32, device="cuda")
        tr_k = torch.zeros((cap, w.L, w.K), dtype=torch.int32, device="cuda")
        tr_g = torch.zeros((cap, w.L, w.K), dtype=torch.float32, device="cuda")
        ms.moe_spark_set_trace(ctx, tr_x.data_ptr(), tr_k.data_ptr(), tr_g.data_ptr(), cap)
        xw = torch.from_numpy(x[:WARM].copy()).cuda()
        xm = torch.from_numpy(x[WARM:].copy()).cuda()
        row = torch.zeros(cap, dtype=torch.int32, device="cuda")
        ms.moe_spark_decode(ctx, xw.data_ptr(), WARM, row.data_ptr())
        ms.moe_spark_synchronize(ctx)
        if calibrate:
            ms.moe_spark_calibrate(ctx, True)
        ms.moe_spark_reset_stats(ctx)
        if B:
            ms.moe_spark_decode_batched(ctx, xm.data_ptr(), MEAS, B, row.data_ptr())
        else:
            ms.moe_spark_decode(ctx, xm.data_ptr(), MEAS, row.data_ptr())
        ms.moe_spark_synchronize(ctx)
        return dict(x=np.concatenate([xw.cpu().numpy(), xm.cpu().numpy()]), tr_x=tr_x.cpu().numpy(),
                    tr_k=tr_k.cpu().numpy(), tr_g=tr_g.cpu().numpy(), stats=ms.moe_spark_get_stats(ctx),
                    events=events(ctx), placement=placement(ctx, w, R),
                    slot_bytes=ms.moe_spark_slot_bytes(ctx))
    finally:
        ms.moe_spark_destroy(ctx)


def _check_bookkeeping(model, r, P, R, B, calibrate):
    w = model.w
    sim = oracle.Sim(w.L, w.E, P, R, r["slot_bytes"])
    sim.place_uniform()
    for t in range(WARM):
        sim.decode_token(r["tr_k"][t])
    if calibrate:
        sim.calibrate(True)
    sim.reset_stats()
    for t0 in range(WARM, WARM + MEAS, B):
        sim.decode_batch(r["tr_k"][t0:min(t0 + B, WARM + MEAS)])
    st = r["stats"]
    assert {k: st[k] for k in STAT_KEYS} == sim.stats(), (st, sim.stats())
    assert st["tokens"] == MEAS
    assert r["events"] == sim_events(sim)
    for got, ref in zip(r["placement"], sim.placement()):
        assert np.array_equal(got, ref)
    return sim.stats()


@pytest.fixture(scope="module")
def batch1(model):
    w = model.w
    print("batch-1 reference decode at full residency", flush=True)
    return _run(model, w.L * w.E, 0, 0, calibrate=False)


@pytest.mark.parametrize("B", [1, 3, 8, 16])
def test_batched_matches_batch1_and_simulator(model, batch1, B):
    w = model.w
    LE = w.L * w.E
    P, R = int(round(0.6 * LE)), max(8, B * w.K)
    print(f"batched decode B={B}: P={P} R={R}, calibrated", flush=True)
    r = _run(model, P, R, B)
    assert np.array_equal(r["tr_k"], batch1["tr_k"])
    rel = np.abs(r["x"] - batch1["x"]).max() / np.abs(batch1["x"]).max()
    print(f"B={B}: max|batched - batch-1| / max|x| = {rel:.2e}", flush=True)
    assert rel <= BATCH1_TOL
    np.testing.assert_allclose(r["tr_g"], batch1["tr_g"], rtol=BATCH1_TOL, atol=1e-5)
    if _BATCHED:
        assert np.array_equal(r["x"], _BATCHED["x"]) and np.array_equal(r["tr_x"], _BATCHED["tr_x"])
        assert np.array_equal(r["tr_g"], _BATCHED["tr_g"])
    else:
        _BATCHED.update(x=r["x"], tr_x=r["tr_x"], tr_g=r["tr_g"])
    ss = _check_bookkeeping(model, r, P, R, B, True)
    print(f"B={B}: {ss}", flush=True)
    # teacher-forced oracle parity of sampled (token, layer) pairs of the batched run
    tr_x, tr_k = r["tr_x"], r["tr_k"]
    for t in (WARM, WARM + B // 2, WARM + MEAS - 1):
        for l in range(w.L):
            xl = tr_x[t, l].astype(np.float64)
            xn = (tr_x[t, l + 1] if l + 1 < w.L else r["x"][t]).astype(np.float64)
            lg = oracle.router(model.routers[l], oracle.rmsnorm(xl), model.biases[l][0])
            ref_idx, gap = oracle_topk_and_gap(lg, w.K)
            forced = tr_k[t, l][None] if gap < TIE_GAP else None
            if forced is None:
                assert np.array_equal(tr_k[t, l], ref_idx), (t, l)
            yref, _, gref, _ = oracle.layer(xl[None], model.routers[l], model.experts(l), K=w.K,
                                            wfmt=w.wfmt, norm=True, bias=model.biases[l],
                                            bias_row=np.zeros(1, np.int32), forced=forced)
            assert_outputs_close(xn - xl, yref[0], f"B={B} token {t} layer {l}")
            np.testing.assert_allclose(r["tr_g"][t, l], gref[0], rtol=2e-5, atol=1e-6)


@pytest.mark.parametrize("pull", [True, False], ids=["pulled-fills", "agent-fills"])
def test_batched_residency_sweep_uniform(model, batch1, pull):
    w = model.w
    LE = w.L * w.E
    B = 2
    R = B * w.K  # the smallest ring a step allows: a step can turn it over completely
    fills = {}
    for frac in (1.0, 0.6, 0.3):
        P = int(round(frac * LE))
        RR = R if P < LE else 0
        print(f"batched decode B={B}: P={P} R={RR}, uniform placement, pull={pull}", flush=True)
        r = _run(model, P, RR, B, calibrate=False, pull=pull)
        assert np.array_equal(r["tr_k"], batch1["tr_k"]), frac
        if not _BATCHED:
            _BATCHED.update(x=r["x"], tr_x=r["tr_x"], tr_g=r["tr_g"])
        assert np.array_equal(r["x"], _BATCHED["x"]), frac
        ss = _check_bookkeeping(model, r, P, RR, B, False)
        fills[frac] = ss["fills"]
        if P < LE:
            assert ss["fills"] > 0 and ss["evictions"] > 0
    print(f"fills by residency: {fills}", flush=True)


def test_batched_rejects_bad_arguments(model):
    w = model.w
    LE = w.L * w.E
    P = int(round(0.6 * LE))
    ctx = model.make_ctx(P=P, R=16)
    try:
        x = torch.zeros((4, w.d), dtype=torch.float32, device="cuda")
        for B, needle in ((0, "batch"), (17, "batch"), (3, "ring")):
            with pytest.raises(ms.MoeSparkError) as ei:
                ms.moe_spark_decode_batched(ctx, x.data_ptr(), 4, B, None)
            assert ei.value.status == ms.E_INVALID and needle in str(ei.value), (B, str(ei.value))
        with pytest.raises(ms.MoeSparkError) as ei:
            ms.moe_spark_decode_batched(ctx, x.data_ptr(), -1, 2, None)
        assert ei.value.status == ms.E_INVALID
        # a ring of 16 holds a step of 2 tokens x 8 experts
        ms.moe_spark_decode_batched(ctx, x.data_ptr(), 4, 2, None)
        ms.moe_spark_synchronize(ctx)
        assert ms.moe_spark_get_stats(ctx)["tokens"] == 4
    finally:
        ms.moe_spark_destroy(ctx)
    tiny = wl.tiny()
    tm = Model(tiny)
    ctx = tm.make_ctx(P=tiny.E, R=0)
    try:
        x = torch.zeros((2, tiny.d), dtype=torch.float32, device="cuda")
        with pytest.raises(ms.MoeSparkError) as ei:
            ms.moe_spark_decode_batched(ctx, x.data_ptr(), 2, 2, None)
        assert ei.value.status == ms.E_INVALID and "Q4_0" in str(ei.value)
    finally:
        ms.moe_spark_destroy(ctx)


def _stats_placement(ctx, w, R):
    return dict(stats=ms.moe_spark_get_stats(ctx), events=events(ctx), placement=placement(ctx, w, R),
                slot_bytes=ms.moe_spark_slot_bytes(ctx))


def _assert_matches_sim(got, sim):
    st = got["stats"]
    assert {k: st[k] for k in STAT_KEYS} == sim.stats(), (st, sim.stats())
    assert got["events"] == sim_events(sim)
    for g, r in zip(got["placement"], sim.placement()):
        assert np.array_equal(g, r)


def test_batched_short_calls_and_graph_reuse(model):
    """A call with no tokens (graph only), a call shorter than one step
    (3 tokens, B = 16), and a second call through the same cached graph
    (5 tokens): outputs equal one 8-token step's bit for bit, bookkeeping is
    the simulator's with steps [3] and [5], and the token counter is 8."""
    w = model.w
    LE = w.L * w.E
    P, B = int(round(0.6 * LE)), 16
    R = B * w.K
    x = w.tokens(0, WARM + 8)[WARM:]
    ref = {}
    for calls in ((8,), (0, 3, 5)):
        ctx = model.make_ctx(P=P, R=R)
        try:
            tr_k = torch.zeros((8, w.L, w.K), dtype=torch.int32, device="cuda")
            tr_g = torch.zeros((8, w.L, w.K), dtype=torch.float32, device="cuda")
            ms.moe_spark_set_trace(ctx, None, tr_k.data_ptr(), tr_g.data_ptr(), 8)
            xd = torch.from_numpy(x.copy()).cuda()
            done = 0
            for n in calls:
                print(f"batched call of {n} tokens (B={B})", flush=True)
                ms.moe_spark_decode_batched(ctx, xd[done:].data_ptr() if done else xd.data_ptr(), n, B, None)
                done += n
            ms.moe_spark_synchronize(ctx)
            got = _stats_placement(ctx, w, R)
            got.update(x=xd.cpu().numpy(), trk=tr_k.cpu().numpy())
        finally:
            ms.moe_spark_destroy(ctx)
        assert got["stats"]["tokens"] == 8
        sim = oracle.Sim(w.L, w.E, P, R, got["slot_bytes"])
        sim.place_uniform()
        t0 = 0
        for n in calls:
            if n:
                sim.decode_batch(got["trk"][t0:t0 + n])
                t0 += n
        _assert_matches_sim(got, sim)
        if not ref:
            ref = got
        else:
            assert np.array_equal(got["x"], ref["x"]) and np.array_equal(got["trk"], ref["trk"])


def test_batched_with_online_self_tuning(model):
    """Self-tuning steps fall between batched steps: warm-up and calibration,
    then 45 tokens in steps of 4 over two calls with a step every 8 tokens.
    Bookkeeping (counters, fill log, pinned set, ring, counts, steps and
    swaps) equals the simulator's with a self-tuning step before each batched
    step that finds 8 or more tokens since the last change; outputs equal the
    batched runs without self-tuning bit for bit."""
    w = model.w
    LE = w.L * w.E
    P, B, EVERY, HYST, SHIFT = int(round(0.6 * LE)), 4, 8, 25, 1
    R = B * w.K
    x = w.tokens(0, WARM + MEAS)
    ctx = model.make_ctx(P=P, R=R)
    try:
        tr_k = torch.zeros((WARM + MEAS, w.L, w.K), dtype=torch.int32, device="cuda")
        tr_g = torch.zeros((WARM + MEAS, w.L, w.K), dtype=torch.float32, device="cuda")
        ms.moe_spark_set_trace(ctx, None, tr_k.data_ptr(), tr_g.data_ptr(), WARM + MEAS)
        xw = torch.from_numpy(x[:WARM].copy()).cuda()
        xm = torch.from_numpy(x[WARM:].copy()).cuda()
        ms.moe_spark_decode(ctx, xw.data_ptr(), WARM, None)
        ms.moe_spark_synchronize(ctx)
        ms.moe_spark_calibrate(ctx, True)
        ms.moe_spark_reset_stats(ctx)
        ms.moe_spark_set_autotune(ctx, EVERY, HYST, SHIFT)
        print(f"batched decode B={B} with a self-tuning step every {EVERY} tokens", flush=True)
        ms.moe_spark_decode_batched(ctx, xm.data_ptr(), 20, B, None)
        ms.moe_spark_decode_batched(ctx, xm[20:].data_ptr(), MEAS - 20, B, None)
        ms.moe_spark_synchronize(ctx)
        got = _stats_placement(ctx, w, R)
        trk = tr_k.cpu().numpy()
        x_out = np.concatenate([xw.cpu().numpy(), xm.cpu().numpy()])
    finally:
        ms.moe_spark_destroy(ctx)
    sim = oracle.Sim(w.L, w.E, P, R, got["slot_bytes"])
    sim.place_uniform()
    for t in range(WARM):
        sim.decode_token(trk[t])
    sim.calibrate(True)
    sim.reset_stats()
    since = steps = swaps = 0
    for lo, hi in ((WARM, WARM + 20), (WARM + 20, WARM + MEAS)):
        for t0 in range(lo, hi, B):
            if since >= EVERY:
                swaps += sim.retune(HYST, SHIFT)
                steps += 1
                since = 0
            nb = min(B, hi - t0)
            sim.decode_batch(trk[t0:t0 + nb])
            since += nb
    _assert_matches_sim(got, sim)
    st = got["stats"]
    assert st["retunes"] == steps > 0 and st["retune_swaps"] == swaps
    print(f"self-tuning: {steps} steps, {swaps} swaps", flush=True)
    if _BATCHED:
        assert np.array_equal(x_out, _BATCHED["x"])

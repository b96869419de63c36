"""Online self-tuning of the placement during decode, through the C ABI.

A 4-layer stack of the target layer shape (d=2048, 64 experts, top-8, f=512,
Q4_0) at 60% residency with a 16-slot ring decodes 64 tokens under router
bias row A, is calibrated, and then decodes 192 tokens under row B (the
Zipf permutation switches, so the calibrated pinned set goes stale) with
self-tuning every 16 tokens (25% hysteresis, counts halved after each step).

 * bookkeeping — counters, fill/eviction log, pinned set, ring, counts, and
   the number of steps and swaps — equals the simulator replaying the GPU's
   own top-k trace with a step before every 16th token;
 * the steps act: after them the cold-hit rate under row B is lower than
   without self-tuning on the same stream;
 * outputs are bit-identical to full residency.
"""
import numpy as np
import pytest
import torch

import oracle
import workload as wl
from spark_harness import STAT_KEYS, Model, events, placement, sim_events

pytestmark = pytest.mark.gpu

import resident_expert_caching_amd as ms  # noqa: E402  (a missing library fails collection: no silent skip)

WARM, MEAS, EVERY, HYST, SHIFT = 64, 192, 16, 25, 1


@pytest.fixture(scope="module")
def model():
    w = wl.Workload("autotune-L4-E64", d=2048, E=64, K=8, f=512, L=4, wfmt=wl.FMT_Q4_0, norm=True,
                    seed=41, n_tokens=WARM + MEAS, token_stream=43, bias_seeds=(3, 1003))
    return Model(w)


def _decode(model, P, R, autotune):
    w = model.w
    x = w.tokens()
    T = WARM + MEAS
    ctx = model.make_ctx(P=P, R=R)
    try:
        tr_x = torch.zeros((T, w.L, w.d), dtype=torch.float32, device="cuda")
        tr_k = torch.zeros((T, w.L, w.K), dtype=torch.int32, device="cuda")
        tr_g = torch.zeros((T, w.L, w.K), dtype=torch.float32, device="cuda")
        ms.moe_spark_set_trace(ctx, tr_x.data_ptr(), tr_k.data_ptr(), tr_g.data_ptr(), T)
        xw = torch.from_numpy(x[:WARM].copy()).cuda()
        xm = torch.from_numpy(x[WARM:].copy()).cuda()
        ra = torch.zeros(WARM, dtype=torch.int32, device="cuda")
        rb = torch.ones(MEAS, dtype=torch.int32, device="cuda")
        ms.moe_spark_decode(ctx, xw.data_ptr(), WARM, ra.data_ptr())
        ms.moe_spark_synchronize(ctx)
        ms.moe_spark_calibrate(ctx, True)
        ms.moe_spark_reset_stats(ctx)
        if autotune:
            ms.moe_spark_set_autotune(ctx, EVERY, HYST, SHIFT)
        # two calls, so a step also falls on a call boundary (token 96 = 6 * 16)
        half = 96
        ms.moe_spark_decode(ctx, xm[:half].data_ptr(), half, rb.data_ptr())
        ms.moe_spark_decode(ctx, xm[half:].data_ptr(), MEAS - half, rb.data_ptr())
        ms.moe_spark_synchronize(ctx)
        return dict(stats=ms.moe_spark_get_stats(ctx), events=events(ctx), placement=placement(ctx, w, R),
                    slot_bytes=ms.moe_spark_slot_bytes(ctx), tr_k=tr_k.cpu().numpy(),
                    x=np.concatenate([xw.cpu().numpy(), xm.cpu().numpy()]))
    finally:
        ms.moe_spark_destroy(ctx)


def test_autotune_matches_simulator_and_tracks_the_shift(model):
    w = model.w
    LE = w.L * w.E
    P, R = int(round(0.6 * LE)), 16
    print("decode: full residency, fixed calibrated placement, self-tuned placement", flush=True)
    full = _decode(model, LE, 0, autotune=False)
    fixed = _decode(model, P, R, autotune=False)
    tuned = _decode(model, P, R, autotune=True)
    assert np.array_equal(full["x"], tuned["x"]) and np.array_equal(full["x"], fixed["x"])
    assert np.array_equal(full["tr_k"], tuned["tr_k"])

    sim = oracle.Sim(w.L, w.E, P, R, tuned["slot_bytes"])
    sim.place_uniform()
    trk = tuned["tr_k"]
    for t in range(WARM):
        sim.decode_token(trk[t])
    sim.calibrate(True)
    sim.reset_stats()
    steps = swaps = since = 0
    for t in range(WARM, WARM + MEAS):
        if since == EVERY:
            swaps += sim.retune(HYST, SHIFT)
            steps += 1
            since = 0
        sim.decode_token(trk[t])
        since += 1
    st = tuned["stats"]
    assert {k: st[k] for k in STAT_KEYS} == sim.stats()
    assert tuned["events"] == sim_events(sim)
    for got, ref in zip(tuned["placement"], sim.placement()):
        assert np.array_equal(got, ref)
    assert st["retunes"] == steps == MEAS // EVERY - 1
    assert st["retune_swaps"] == swaps > 0
    cold_fixed = fixed["stats"]["cold_hits"] / fixed["stats"]["accesses"]
    cold_tuned = st["cold_hits"] / st["accesses"]
    print(f"cold-hit under row B: fixed {cold_fixed:.3f}, self-tuned {cold_tuned:.3f}; "
          f"{steps} steps, {swaps} swaps", flush=True)
    assert cold_tuned < cold_fixed


def test_autotune_rejects_bad_arguments(model):
    ctx = model.make_ctx(P=model.w.L * model.w.E, R=0)
    try:
        for args in ((-1, 25, 1), (16, -1, 1), (16, 25, 63), (16, 100001, 0)):
            with pytest.raises(ms.MoeSparkError) as ei:
                ms.moe_spark_set_autotune(ctx, *args)
            assert ei.value.status == ms.E_INVALID
        ms.moe_spark_set_autotune(ctx, 0, 0, 0)
    finally:
        ms.moe_spark_destroy(ctx)

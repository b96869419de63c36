"""The allocation-free layer forward (moe_spark_layer_forward_noalloc),
through the C ABI, against moe_spark_layer_forward: two calls in a row, the
second with fewer tokens, each compared bit for bit (outputs, top-k, gates,
counters, fill log, placement) with the allocating entry point on a twin
context; at 60% residency with a small ring, so cold experts are filled and
their work-groups wait for the published selection.  The second call also
checks that the scratch the first call left behind does not leak into it."""
import numpy as np
import pytest
import torch

import workload as wl
from spark_harness import STAT_KEYS, Model, events, placement

pytestmark = pytest.mark.gpu

import resident_expert_caching_amd as ms  # noqa: E402  (a missing library fails collection: no silent skip)


def _run(fn, model, P, R, calls):
    w = model.w
    ctx = model.make_ctx(P=P, R=R)
    outs = []
    try:
        for x, rows in calls:
            T = x.shape[0]
            xd = torch.from_numpy(x.copy()).cuda()
            yd = torch.full_like(xd, float("nan"))
            rd = torch.from_numpy(rows).cuda()
            topk = torch.full((T, w.K), -1, dtype=torch.int32, device="cuda")
            gates = torch.zeros((T, w.K), dtype=torch.float32, device="cuda")
            print(f"{fn.__name__}: T={T} P={P} R={R}", flush=True)
            fn(ctx, 1, xd.data_ptr(), yd.data_ptr(), T, rd.data_ptr(), ms.PRE_RMSNORM | ms.RESIDUAL,
               topk.data_ptr(), gates.data_ptr())
            ms.moe_spark_synchronize(ctx)
            outs.append(dict(y=yd.cpu().numpy(), topk=topk.cpu().numpy(), gates=gates.cpu().numpy(),
                             stats=ms.moe_spark_get_stats(ctx), events=events(ctx),
                             placement=placement(ctx, w, R)))
        return outs
    finally:
        ms.moe_spark_destroy(ctx)


def test_noalloc_layer_forward_matches_layer_forward():
    w = wl.Workload("noalloc", d=2048, E=64, K=8, f=512, L=2, wfmt=wl.FMT_Q4_0, norm=True, seed=17,
                    n_tokens=40, token_stream=3, bias_seeds=(4, 1004))
    model = Model(w)
    x = w.tokens()
    calls = [(x[:24], (np.arange(24) % 2).astype(np.int32)),
             (x[24:34], np.ones(10, np.int32))]
    P, R = int(round(0.6 * w.L * w.E)), 8
    ref = _run(ms.moe_spark_layer_forward, model, P, R, calls)
    got = _run(ms.moe_spark_layer_forward_noalloc, model, P, R, calls)
    for i, (a, b) in enumerate(zip(ref, got)):
        assert np.isfinite(b["y"]).all(), i
        assert np.array_equal(a["y"], b["y"]), i
        assert np.array_equal(a["topk"], b["topk"]) and np.array_equal(a["gates"], b["gates"]), i
        assert {k: a["stats"][k] for k in STAT_KEYS} == {k: b["stats"][k] for k in STAT_KEYS}, i
        assert a["events"] == b["events"], i
        for u, v in zip(a["placement"], b["placement"]):
            assert np.array_equal(u, v), i
    assert ref[-1]["stats"]["fills"] > 0  # cold experts were filled and waited for


def test_noalloc_rejects_fp32_contexts():
    w = wl.tiny()
    model = Model(w)
    ctx = model.make_ctx(P=w.E, R=0)
    try:
        x = torch.zeros((2, w.d), dtype=torch.float32, device="cuda")
        with pytest.raises(ms.MoeSparkError) as e:
            ms.moe_spark_layer_forward_noalloc(ctx, 0, x.data_ptr(), x.data_ptr(), 2, None, 0, None, None)
        assert "Q4_0" in str(e.value)
    finally:
        ms.moe_spark_destroy(ctx)

"""The seeded input generator: Philox4x64-10 known answers (numpy's Philox
bit generator implements the same published block function), normal draws,
fp16 rounding against numpy, Q4_0 encoding properties, Zipf bias, and
regeneration of single experts."""
import numpy as np
import pytest
from scipy import stats

import workload as wl


@pytest.mark.parametrize("key", [(0, 0), (0x1234, 0x5678), (2**64 - 1, 7)])
def test_philox_matches_numpy(key):
    g = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=[0, 0, 0, 0])
    ref = g.random_raw(12)
    mine = np.concatenate([wl.philox4x64_10([c, 0, 0, 0], key) for c in (1, 2, 3)])
    assert np.array_equal(ref, mine)


def test_normals_are_standard_normal():
    z = wl.normal_f32(3, 11, 0, 0, 1_000_000, 1.0).astype(np.float64)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    assert stats.kstest(z[:200_000], "norm").pvalue > 1e-3
    assert np.abs(z).max() < 6.5


def test_f16_rounding_matches_numpy():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 5, 20000),
                        [0.0, -0.0, 65504.0, 65519.9, 65520.0, 1e-8, 2.0 ** -25, 3 * 2.0 ** -26]])
    x = x.astype(np.float32)
    mine = np.array([wl.lib().wl_f32_to_f16(float(v)) for v in x], dtype=np.uint16)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(mine, ref)


def test_q4_0_encoding_properties():
    w = wl.normal_f32(5, 1, 0, 0, 64 * 256, 0.02).reshape(64, 256)
    q = wl.q4_0_encode(w)
    scale = q[:, :, 0].astype(np.uint16) | (q[:, :, 1].astype(np.uint16) << 8)
    s = scale.view(np.float16).astype(np.float64)
    codes = np.concatenate([q[:, :, 2:] & 15, q[:, :, 2:] >> 4], axis=2).astype(np.int64)
    deq = (codes - 8) * s[:, :, None]
    err = np.abs(deq.reshape(64, 256) - w)
    # round-to-nearest against the fp16 scale: half a step; the largest
    # magnitude has the opposite sign of the scale and codes to 0, so the far
    # end of the range (w/s near +8) clamps from 16 to 15: up to one step there
    step = np.repeat(np.abs(s), 32, axis=1)
    c = codes.reshape(64, 256)
    assert np.all(err[c != 15] <= step[c != 15] * 0.5 * (1 + 1e-3) + 1e-7)
    assert np.all(err <= step * (1 + 1e-3) + 1e-7)
    assert codes.min() == 0 and codes.max() == 15
    z = wl.q4_0_encode(np.zeros((1, 32), np.float32))
    assert z[0, 0, 0] == 0 and z[0, 0, 1] == 0 and np.all(z[0, 0, 2:] == 0x88)


def test_zipf_bias_closed_form():
    E = 256
    b, r = wl.zipf_bias(2, 5, E)
    assert sorted(r.tolist()) == list(range(1, E + 1))
    p = np.arange(1, E + 1, dtype=np.float64) ** -1.1
    p /= p.sum()
    np.testing.assert_allclose(b, (2 * np.log(p[r - 1])).astype(np.float32), rtol=1e-6)
    b2, r2 = wl.zipf_bias(1002, 5, E)
    assert not np.array_equal(r, r2)  # the second permutation differs


def test_single_expert_regeneration_matches_blob():
    d, f = 256, 64
    blob = wl.experts_blob(9, 2, 2, 4, d, f, wl.FMT_Q4_0)
    for i, (l, e) in enumerate([(2, 0), (2, 3), (3, 1)]):
        row = blob[(l - 2) * 4 + e]
        g, u, dn = wl.expert(9, l, e, d, f, wl.FMT_Q4_0)
        assert np.array_equal(row, np.concatenate([g.ravel(), u.ravel(), dn.ravel()]))
    assert wl.expert_bytes(2048, 512, wl.FMT_Q4_0) == 1_769_472

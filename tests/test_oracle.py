"""Pins of the CPU oracle against facts that do not come from the oracle itself:
hand-worked golden blocks, closed forms, brute force on tiny inputs, library
routines (numpy float16, scipy softmax / expit, numpy matmul) on special cases,
and invariants of the method (gates sum to one, identical experts, dense
all-experts evaluation)."""
import os

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
import workload as wl

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def silu(z):
    return z * expit(z)


# ---------------------------------------------------------------- fp16 / Q4_0

def test_f16_decode_matches_numpy_for_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def _read_golden_blocks(path):
    blocks, values = [], []
    for line in open(path):
        line = line.strip()
        if line.startswith("block"):
            blocks.append(np.array([int(t, 16) for t in line.split()[1:]], dtype=np.uint8))
        elif line.startswith("values"):
            values.append(np.array([float(t) for t in line.split()[1:]]))
    return blocks, values


def test_q4_0_golden_blocks(golden_dir):
    blocks, values = _read_golden_blocks(os.path.join(golden_dir, "q4_0_blocks.txt"))
    assert len(blocks) == len(values) == 4
    for b, v in zip(blocks, values):
        assert b.size == 18 and v.size == 32
        assert np.array_equal(oracle.q4_0_block(b), v)


def _q4_matrix(codes, scales_f16):
    """Pack integer codes [rows][cols] and fp16 scales [rows][cols/32] into
    GGUF Q4_0 bytes (the block layout pinned by the golden blocks)."""
    rows, cols = codes.shape
    nb = cols // 32
    out = np.zeros((rows, nb, 18), dtype=np.uint8)
    sb = scales_f16.astype(np.float16).view(np.uint16)
    out[:, :, 0] = (sb & 0xff).astype(np.uint8)
    out[:, :, 1] = (sb >> 8).astype(np.uint8)
    c = codes.reshape(rows, nb, 32)
    out[:, :, 2:] = (c[:, :, :16] | (c[:, :, 16:] << 4)).astype(np.uint8)
    return out


def test_q4_0_matvec_against_numpy_matmul_on_exact_weights():
    rng = np.random.default_rng(5)
    rows, cols = 24, 96
    codes = rng.integers(0, 16, size=(rows, cols))
    scales = 2.0 ** rng.integers(-12, 2, size=(rows, cols // 32))  # exact in fp16
    w = (codes - 8) * np.repeat(scales, 32, axis=1)
    v = rng.standard_normal(cols)
    got = oracle.matvec(_q4_matrix(codes, scales), v, oracle.W_Q4_0, rows, cols)
    np.testing.assert_allclose(got, w @ v, rtol=1e-13, atol=1e-15)


def test_f32_matvec_against_numpy_matmul():
    rng = np.random.default_rng(6)
    w = rng.standard_normal((33, 70)).astype(np.float32)
    v = rng.standard_normal(70)
    got = oracle.matvec(w, v, oracle.W_F32, 33, 70)
    np.testing.assert_allclose(got, w.astype(np.float64) @ v, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- RMSNorm / router

def test_rmsnorm_closed_forms():
    c, d, eps = 3.0, 64, 1e-6
    u = oracle.rmsnorm(np.full(d, c), eps)
    assert np.allclose(u, c / np.sqrt(c * c + eps), rtol=1e-15)
    x = np.array([3.0, 4.0, 0.0, 0.0])
    assert np.allclose(oracle.rmsnorm(x, 0.0), x / 2.5, rtol=1e-15)
    assert np.array_equal(oracle.rmsnorm(np.zeros(8), eps), np.zeros(8))


def test_router_zero_input_gives_bias_and_one_hot_gives_column():
    rng = np.random.default_rng(7)
    E, d = 16, 256
    wr = rng.standard_normal((E, d)).astype(np.float32)
    bias = rng.standard_normal(E).astype(np.float32)
    assert np.array_equal(oracle.router(wr, np.zeros(d), bias), bias.astype(np.float64))
    j = 37
    u = np.zeros(d)
    u[j] = 1.0
    assert np.array_equal(oracle.router(wr, u, None), wr[:, j].astype(np.float64))


def test_batched_router_logits_equal_per_token_router():
    """The vectorised router (numpy matrix product) against the per-token C
    router with RMSNorm, bias rows chosen per token, on a ragged token count."""
    rng = np.random.default_rng(31)
    T, d, E = 37, 96, 20
    x = rng.standard_normal((T, d)) * 3.0
    wr = rng.standard_normal((E, d)).astype(np.float32)
    bias = rng.standard_normal((3, E)).astype(np.float32)
    rows = rng.integers(0, 3, T).astype(np.int32)
    got = oracle.router_logits(x, wr, bias, rows)
    for t in range(T):
        ref = oracle.router(wr, oracle.rmsnorm(x[t]), bias[rows[t]])
        np.testing.assert_allclose(got[t], ref, rtol=0, atol=1e-12 * np.abs(ref).max())
    raw = oracle.router_logits(x, wr, None, None, norm=False)
    np.testing.assert_allclose(raw[5], oracle.router(wr, x[5]), rtol=0, atol=1e-12 * np.abs(raw[5]).max())


# ---------------------------------------------------------------- top-k / gates

def _brute_topk(logits, K):
    order = np.lexsort((np.arange(logits.size), -logits))  # logit desc, index asc
    return order[:K]


@pytest.mark.parametrize("E,K", [(16, 2), (16, 16), (9, 1), (256, 8), (5, 5)])
def test_topk_matches_full_sort_with_planted_ties(E, K):
    rng = np.random.default_rng(E * 100 + K)
    for trial in range(50):
        lg = np.round(rng.standard_normal(E) * 2, 1)  # coarse values -> many exact ties
        if trial % 5 == 0:
            lg[:] = 0.5  # all tied: index order
        assert np.array_equal(oracle.topk(lg, K), _brute_topk(lg, K))


def test_gates_sum_to_one_and_match_scipy_softmax():
    rng = np.random.default_rng(8)
    for E, K in [(16, 2), (256, 8), (7, 7)]:
        lg = rng.standard_normal(E) * 3
        idx = _brute_topk(lg, K)
        g = oracle.gates(lg, idx)
        assert abs(g.sum() - 1.0) <= 1e-15
        full = softmax(lg)
        ref = full[idx] / full[idx].sum()
        np.testing.assert_allclose(g, ref, rtol=1e-13)
        assert np.all(np.diff(g) <= 0)  # rank order = descending gates
    assert np.array_equal(oracle.gates(np.array([0.3, -2.0]), np.array([1])), [1.0])


# ---------------------------------------------------------------- expert FFN

def _one_hot_rows(rows, cols, pos):
    w = np.zeros((rows, cols), dtype=np.float32)
    w[np.arange(rows), pos] = 1.0
    return w


@pytest.mark.parametrize("wfmt", [oracle.W_F32, oracle.W_Q4_0])
def test_expert_one_hot_closed_form(wfmt):
    """Gate row j picks u[a_j], up row j picks u[b_j], down row r picks h[c_r]:
    y_r = silu(u[a_{c_r}]) * u[b_{c_r}] — distinguishes gate from up and every
    transposition (d != f)."""
    rng = np.random.default_rng(9)
    d, f = 64, 32
    a, b = rng.integers(0, d, f), rng.integers(0, d, f)
    c = rng.integers(0, f, d)
    Wg, Wu, Wd = _one_hot_rows(f, d, a), _one_hot_rows(d, f, c), None
    Wu = _one_hot_rows(f, d, b)
    Wd = _one_hot_rows(d, f, c)
    u = rng.standard_normal(d) * 2
    if wfmt == oracle.W_Q4_0:  # one-hot as code 9 (value +1 at scale 1), others 8
        enc = lambda w: _q4_matrix((w * 1 + 8).astype(np.int64), np.ones((w.shape[0], w.shape[1] // 32)))
        Wg, Wu, Wd = enc(Wg), enc(Wu), enc(Wd)
    h, y = oracle.expert(Wg, Wu, Wd, u, wfmt, d, f)
    np.testing.assert_allclose(h, silu(u[a]) * u[b], rtol=1e-15, atol=0)
    np.testing.assert_allclose(y, silu(u[a[c]]) * u[b[c]], rtol=1e-15, atol=0)


# ---------------------------------------------------------------- layer

def _tiny_experts(E, d, f, seed, wfmt=oracle.W_F32):
    return [wl.expert(seed, 0, e, d, f, wfmt) for e in range(E)]


def test_layer_identical_experts_ignore_routing():
    rng = np.random.default_rng(10)
    d, f, E, K = 64, 32, 8, 3
    one = wl.expert(3, 0, 0, d, f, wl.FMT_F32)
    experts = [one] * E
    wr = rng.standard_normal((E, d)).astype(np.float32)
    x = rng.standard_normal((5, d))
    y, idx, g, _ = oracle.layer(x, wr, experts, K=K, wfmt=oracle.W_F32, norm=True)
    for t in range(5):
        _, ye = oracle.expert(*one, oracle.rmsnorm(x[t]), oracle.W_F32, d, f)
        np.testing.assert_allclose(y[t], ye, rtol=1e-13, atol=1e-16)


@pytest.mark.parametrize("K", [1, 2, 16])
def test_layer_equals_dense_all_experts_evaluation(K):
    """Sparse layer == all E experts evaluated densely and combined with a
    length-E gate vector that is the scipy softmax renormalised over the
    brute-force top-K set (zero elsewhere).  K = E is the ordinary softmax MoE."""
    w = wl.tiny()
    E, d, f = w.E, w.d, w.f
    experts = [w.expert(0, e) for e in range(E)]
    wr = w.router(0)
    x = w.tokens(0, 6).astype(np.float64)
    y, idx, g, lg = oracle.layer(x, wr, experts, K=K, wfmt=oracle.W_F32, norm=False,
                                 want_logits=True)
    for t in range(x.shape[0]):
        logits = wr.astype(np.float64) @ x[t]
        np.testing.assert_allclose(lg[t], logits, rtol=1e-12, atol=1e-14)
        S = _brute_topk(logits, K)
        assert np.array_equal(idx[t], S)
        p = softmax(logits)
        gate_vec = np.zeros(E)
        gate_vec[S] = p[S] / p[S].sum()
        dense = np.zeros(d)
        for e in range(E):
            _, ye = oracle.expert(*experts[e], x[t], oracle.W_F32, d, f)
            dense += gate_vec[e] * ye
        np.testing.assert_allclose(y[t], dense, rtol=1e-12, atol=1e-15)


def test_layer_zero_input_routes_by_bias_and_outputs_zero():
    """x = 0: RMSNorm gives u = 0, logits equal the Zipf bias, so the chosen
    experts are the K most popular (ranks 1..K, in rank order) and y = 0."""
    w = wl.layer()
    E, d, f, K = w.E, w.d, 64, w.K
    bias, rank = wl.zipf_bias(2, 0, E)
    experts = [wl.expert(1, 0, e, d, f, wl.FMT_Q4_0) for e in range(E)]
    y, idx, g, _ = oracle.layer(np.zeros((1, d)), w.router(0), experts, K=K, wfmt=oracle.W_Q4_0,
                                norm=True, bias=bias)
    assert np.array_equal(rank[idx[0]], np.arange(1, K + 1))
    assert np.array_equal(y, np.zeros((1, d)))
    # gates from logits = 2 ln p_r: g_k proportional to p_r^2 = r^-2.2
    r = np.arange(1, K + 1, dtype=np.float64)
    ref = r ** -2.2 / np.sum(r ** -2.2)
    np.testing.assert_allclose(g[0], ref, rtol=1e-6)  # bias was rounded to fp32


def test_layer_linear_in_down_weights_and_forced_selection():
    w = wl.tiny()
    experts = [w.expert(0, e) for e in range(w.E)]
    doubled = [(g, u, dn * np.float32(2.0)) for g, u, dn in experts]
    x = w.tokens(0, 4).astype(np.float64)
    y1, idx, g1, _ = oracle.layer(x, w.router(0), experts, K=2, wfmt=oracle.W_F32, norm=False)
    y2, _, _, _ = oracle.layer(x, w.router(0), doubled, K=2, wfmt=oracle.W_F32, norm=False)
    assert np.array_equal(y2, 2.0 * y1)
    y3, idx3, g3, _ = oracle.layer(x, w.router(0), experts, K=2, wfmt=oracle.W_F32, norm=False,
                                   forced=idx)
    assert np.array_equal(y3, y1) and np.array_equal(idx3, idx) and np.array_equal(g3, g1)
    rev = idx[:, ::-1].copy()  # forced order is honoured; gates follow it
    _, idx4, g4, _ = oracle.layer(x, w.router(0), experts, K=2, wfmt=oracle.W_F32, norm=False,
                                  forced=rev)
    assert np.array_equal(idx4, rev)
    np.testing.assert_allclose(g4, g1[:, ::-1], rtol=1e-14)


# ---------------------------------------------------------------- stack

def test_stack_zero_experts_keep_x_and_one_layer_is_residual():
    rng = np.random.default_rng(11)
    E, d, f, K, L = 8, 64, 32, 2, 3
    zero = (np.zeros((f, d), np.float32), np.zeros((f, d), np.float32), np.zeros((d, f), np.float32))
    wrs = [rng.standard_normal((E, d)).astype(np.float32) for _ in range(L)]
    x = rng.standard_normal((4, d))
    xo, idx, _ = oracle.stack(x, wrs, None, [[zero] * E] * L, K=K, wfmt=oracle.W_F32)
    assert np.array_equal(xo, x)
    experts = [wl.expert(4, 0, e, d, f, wl.FMT_F32) for e in range(E)]
    xo, idx, xt = oracle.stack(x, wrs[:1], None, [experts], K=K, wfmt=oracle.W_F32,
                               want_trace=True)
    y, idx1, _, _ = oracle.layer(x, wrs[0], experts, K=K, wfmt=oracle.W_F32, norm=True)
    assert np.array_equal(xo, x + y) and np.array_equal(idx[:, 0], idx1)
    assert np.array_equal(xt[:, 0], x)


def _numpy_stack(x, wrs, biases, rows, experts, K, eps=1e-6):
    """An independent fp64 numpy statement of the residual stack on fp32
    weights: RMSNorm, router + bias row, top-K by (logit desc, index asc),
    the softmax over the chosen logits, SwiGLU experts, rank-order combine,
    x += y, layer after layer."""
    x = x.astype(np.float64).copy()
    for l, wr in enumerate(wrs):
        u = x / np.sqrt((x * x).mean(axis=1, keepdims=True) + eps)
        lg = u @ wr.astype(np.float64).T + biases[l].astype(np.float64)[rows]
        y = np.zeros_like(x)
        for t in range(x.shape[0]):
            sel = np.lexsort((np.arange(lg.shape[1]), -lg[t]))[:K]
            g = np.exp(lg[t, sel] - lg[t, sel].max())
            g /= g.sum()
            for k, e in enumerate(sel):
                gw, uw, dw = (m.astype(np.float64) for m in experts[l][e])
                h = silu(gw @ u[t]) * (uw @ u[t])
                y[t] += g[k] * (dw @ h)
        x = x + y
    return x


def test_stack_distinct_layers_equal_chained_layers_and_numpy():
    """Three layers with distinct routers, bias tables (two rows, chosen per
    token) and experts: the stack equals the single-layer oracle chained with
    the residual, bit for bit, and an independent numpy statement to 1e-12.
    A wrong per-layer offset (layer 0's router, bias or experts reused, or the
    expert table indexed off by a layer) fails both."""
    rng = np.random.default_rng(23)
    E, d, f, K, L, T = 12, 64, 32, 3, 3, 6
    wrs = [(0.3 * rng.standard_normal((E, d))).astype(np.float32) for _ in range(L)]
    biases = [(0.5 * rng.standard_normal((2, E))).astype(np.float32) for _ in range(L)]
    experts = [[tuple((0.2 * rng.standard_normal(s)).astype(np.float32) for s in ((f, d), (f, d), (d, f)))
                for _ in range(E)] for _ in range(L)]
    rows = np.array([0, 1, 1, 0, 1, 0], np.int32)
    x = rng.standard_normal((T, d))
    xo, idx, xt = oracle.stack(x, wrs, biases, experts, K=K, wfmt=oracle.W_F32, bias_row=rows,
                               want_trace=True)
    xc = x.copy()
    for l in range(L):
        assert np.array_equal(xt[:, l], xc)
        y, il, _, _ = oracle.layer(xc, wrs[l], experts[l], K=K, wfmt=oracle.W_F32, norm=True,
                                   bias=biases[l], bias_row=rows)
        assert np.array_equal(idx[:, l], il)
        xc = xc + y
    assert np.array_equal(xo, xc)
    ref = _numpy_stack(x, wrs, biases, rows, experts, K)
    np.testing.assert_allclose(xo, ref, rtol=0, atol=1e-12 * np.abs(ref).max())
    # the layers really differ: each layer's routing is not layer 0's
    assert any(not np.array_equal(idx[:, l], idx[:, 0]) for l in range(1, L))


def test_thread_count_does_not_change_results():
    import subprocess
    import sys
    code = ("import numpy as np, oracle, workload as wl\n"
            "w = wl.tiny(); ex = [w.expert(0, e) for e in range(w.E)]\n"
            "y, *_ = oracle.layer(w.tokens(0, 8).astype(np.float64), w.router(0), ex, K=2,"
            " wfmt=0, norm=False)\n"
            "print(y.tobytes().hex()[:4096], float(y.sum()).hex())\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    outs = []
    for n in ("1", "3", "8"):
        env = dict(os.environ, OMP_NUM_THREADS=n)
        outs.append(subprocess.run([sys.executable, "-c", code], env=env, cwd=root, check=True,
                                   capture_output=True, text=True).stdout)
    assert outs[0] == outs[1] == outs[2]

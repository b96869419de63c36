"""ctypes view of the CPU oracle (``liboracle.so``) — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never uses it.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

W_F32 = 0
W_Q4_0 = 1
EV_FILL = 2
EV_PREFETCH = 3
STAT_NAMES = ("accesses", "pinned_hits", "cold_hits", "ring_hits", "fills", "evictions",
              "h2d_bytes", "prefetches")


class Shape(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("E", ctypes.c_int32), ("K", ctypes.c_int32),
                ("f", ctypes.c_int32), ("wfmt", ctypes.c_int32), ("norm", ctypes.c_int32),
                ("eps", ctypes.c_double)]


EVENT_DTYPE = np.dtype([("seq", np.int64), ("layer", np.int32), ("expert", np.int32),
                        ("slot", np.int32), ("kind", np.int32), ("victim", np.int32),
                        ("pad", np.int32)])


def build():
    """Compile ``liboracle.so`` (plain C, fp64, OpenMP)."""
    srcs = [os.path.join(_HERE, s) for s in ("oracle.c", "sim.c")]
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-o", _LIB_PATH + ".tmp"] + srcs + ["-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.oracle_num_threads.restype = i32
        L.oracle_set_num_threads.argtypes = [i32]
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f64.restype = dbl
        L.oracle_q4_0_block.argtypes = [vp, vp]
        L.oracle_rmsnorm.argtypes = [i32, vp, dbl, vp]
        L.oracle_router.argtypes = [i32, i32, vp, vp, vp, vp]
        L.oracle_topk.argtypes = [i32, i32, vp, vp]
        L.oracle_gates.argtypes = [i32, vp, vp, vp]
        L.oracle_matvec.argtypes = [i32, i32, i32, vp, vp, vp]
        L.oracle_expert.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp]
        L.oracle_layer.argtypes = [ctypes.POINTER(Shape), i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                   vp, vp, vp, vp]
        L.oracle_layer.restype = i32
        L.oracle_stack.argtypes = [ctypes.POINTER(Shape), i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                   vp, vp]
        L.oracle_stack.restype = i32
        L.oracle_sim_create.argtypes = [i32, i32, i64, i32, i64]
        L.oracle_sim_create.restype = vp
        L.oracle_sim_destroy.argtypes = [vp]
        L.oracle_sim_place_uniform.argtypes = [vp]
        L.oracle_sim_calibrate.argtypes = [vp, i32]
        L.oracle_sim_retune.argtypes = [vp, i32, i32]
        L.oracle_sim_retune.restype = ctypes.c_int64
        L.oracle_sim_decode_token.argtypes = [vp, i32, vp]
        L.oracle_sim_decode_layer.argtypes = [vp, i32, i32, vp]
        L.oracle_sim_decode_batch.argtypes = [vp, i32, i32, vp]
        L.oracle_sim_prefill_layer.argtypes = [vp, i32, i32, i32, vp]
        L.oracle_sim_prefetch.argtypes = [vp, i32, vp]
        L.oracle_sim_prefetch.restype = ctypes.c_int64
        L.oracle_sim_stats.argtypes = [vp, vp]
        L.oracle_sim_reset_stats.argtypes = [vp]
        L.oracle_sim_placement.argtypes = [vp, vp, vp, vp, vp]
        L.oracle_sim_events.argtypes = [vp, vp, i64]
        L.oracle_sim_events.restype = i64
        L.oracle_sim_quota.argtypes = [i32, i64, i32]
        L.oracle_sim_quota.restype = i64
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def _ptrs(arrs):
    return (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])


def num_threads():
    return int(lib().oracle_num_threads())


def set_num_threads(n):
    """OpenMP threads of the following calls (timing only; results do not depend on it)."""
    lib().oracle_set_num_threads(int(n))


def f16_to_f64(h):
    return lib().oracle_f16_to_f64(int(h))


def q4_0_block(blk):
    blk = np.ascontiguousarray(blk, dtype=np.uint8)
    assert blk.size == 18
    out = np.empty(32, dtype=np.float64)
    lib().oracle_q4_0_block(_p(blk), _p(out))
    return out


def rmsnorm(x, eps=1e-6):
    x = _f64(x)
    u = np.empty_like(x)
    lib().oracle_rmsnorm(x.size, _p(x), eps, _p(u))
    return u


def router(wr, u, bias=None):
    wr = _f32(wr)
    u = _f64(u)
    E, d = wr.shape
    out = np.empty(E, dtype=np.float64)
    lib().oracle_router(E, d, _p(wr), _p(u), _p(_f32(bias)), _p(out))
    return out


def router_logits(x, wr, bias=None, bias_row=None, norm=True, eps=1e-6):
    """Router logits of many tokens at once, in fp64: RMSNorm of each row of x
    (when norm), then u @ wr^T plus the token's bias row.  The same definition
    as ``router`` (a numpy matrix product in place of the per-token loop), for
    checking every token-layer of a large run."""
    x = np.atleast_2d(np.asarray(x, np.float64))
    u = x / np.sqrt((x * x).mean(axis=1, keepdims=True) + eps) if norm else x
    lg = u @ np.asarray(wr, np.float64).T
    if bias is not None:
        b = np.atleast_2d(np.asarray(bias, np.float64))
        rows = np.zeros(x.shape[0], np.int64) if bias_row is None else np.asarray(bias_row, np.int64)
        lg = lg + b[rows]
    return lg


def topk(logits, K):
    lg = _f64(logits)
    idx = np.empty(K, dtype=np.int32)
    lib().oracle_topk(lg.size, K, _p(lg), _p(idx))
    return idx


def gates(logits, idx):
    lg = _f64(logits)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    g = np.empty(idx.size, dtype=np.float64)
    lib().oracle_gates(idx.size, _p(lg), _p(idx), _p(g))
    return g


def matvec(w, v, wfmt, rows, cols):
    w = np.ascontiguousarray(w)
    v = _f64(v)
    out = np.empty(rows, dtype=np.float64)
    lib().oracle_matvec(rows, cols, wfmt, _p(w), _p(v), _p(out))
    return out


def expert(gate, up, down, u, wfmt, d, f):
    u = _f64(u)
    gate, up, down = (np.ascontiguousarray(a) for a in (gate, up, down))
    h = np.empty(f, dtype=np.float64)
    y = np.empty(d, dtype=np.float64)
    lib().oracle_expert(d, f, wfmt, _p(gate), _p(up), _p(down), _p(u), _p(h), _p(y))
    return h, y


def layer(x, wr, experts, *, K, wfmt, norm, eps=1e-6, bias=None, bias_row=None, forced=None,
          want_logits=False):
    """One MoE layer over T tokens.  ``experts`` is a list of (gate, up, down) per expert.
    Returns (y [T][d], idx [T][K], gates [T][K], logits [T][E] or None)."""
    x = np.atleast_2d(_f64(x))
    T, d = x.shape
    wr = _f32(wr)
    E = wr.shape[0]
    f = (experts[0][0].shape[0])
    keep = [tuple(np.ascontiguousarray(a) for a in ex) for ex in experts]
    gp = _ptrs([k[0] for k in keep])
    up = _ptrs([k[1] for k in keep])
    dp = _ptrs([k[2] for k in keep])
    s = Shape(d, E, K, f, wfmt, int(norm), eps)
    y = np.empty((T, d), dtype=np.float64)
    idx = np.empty((T, K), dtype=np.int32)
    g = np.empty((T, K), dtype=np.float64)
    lg = np.empty((T, E), dtype=np.float64) if want_logits else None
    b = _f32(None if bias is None else np.atleast_2d(bias))
    br = None if bias_row is None else np.ascontiguousarray(bias_row, dtype=np.int32)
    fc = None if forced is None else np.ascontiguousarray(forced, dtype=np.int32)
    rc = lib().oracle_layer(ctypes.byref(s), T, _p(x), _p(wr), _p(b), _p(br), gp, up, dp, _p(fc),
                            _p(y), _p(idx), _p(g), _p(lg))
    assert rc == 0
    return y, idx, g, lg


def stack(x, wrs, biases, experts, *, K, wfmt, eps=1e-6, bias_row=None, want_trace=False):
    """Residual stack over L layers.  ``experts[l]`` is the per-layer expert list.
    Returns (x_out [T][d], idx_trace [T][L][K], x_trace [T][L][d] or None)."""
    x = np.atleast_2d(_f64(x)).copy()
    T, d = x.shape
    L = len(wrs)
    E = wrs[0].shape[0]
    f = experts[0][0][0].shape[0]
    wrs = [_f32(w) for w in wrs]
    bs = None if biases is None else [_f32(np.atleast_2d(b)) for b in biases]
    keep = [tuple(np.ascontiguousarray(a) for a in ex) for lay in experts for ex in lay]
    gp = _ptrs([k[0] for k in keep])
    up = _ptrs([k[1] for k in keep])
    dp = _ptrs([k[2] for k in keep])
    wp = _ptrs(wrs)
    bp = None if bs is None else _ptrs(bs)
    br = None if bias_row is None else np.ascontiguousarray(bias_row, dtype=np.int32)
    s = Shape(d, E, K, f, wfmt, 1, eps)
    idx = np.empty((T, L, K), dtype=np.int32)
    xt = np.empty((T, L, d), dtype=np.float64) if want_trace else None
    rc = lib().oracle_stack(ctypes.byref(s), L, T, _p(x), wp, bp, _p(br), gp, up, dp, _p(idx),
                            _p(xt))
    assert rc == 0
    return x, idx, xt


class Sim:
    """The placement / LRU-ring simulator."""

    def __init__(self, L, E, P, R, slot_bytes):
        self.L, self.E, self.P, self.R = L, E, P, R
        self._h = lib().oracle_sim_create(L, E, P, R, slot_bytes)
        assert self._h, "invalid simulator shape"

    def __del__(self):
        if getattr(self, "_h", None):
            lib().oracle_sim_destroy(self._h)
            self._h = None

    def place_uniform(self):
        lib().oracle_sim_place_uniform(self._h)

    def calibrate(self, reset_counts=True):
        lib().oracle_sim_calibrate(self._h, int(reset_counts))

    def retune(self, hysteresis_pct, decay_shift):
        return int(lib().oracle_sim_retune(self._h, int(hysteresis_pct), int(decay_shift)))

    def decode_token(self, idx):
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        assert idx.shape[0] == self.L
        lib().oracle_sim_decode_token(self._h, idx.shape[1], _p(idx))

    def decode_batch(self, idx):
        """idx [B][L][K]: B tokens through the stack together."""
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        assert idx.ndim == 3 and idx.shape[1] == self.L
        lib().oracle_sim_decode_batch(self._h, idx.shape[0], idx.shape[2], _p(idx))

    def decode_layer(self, layer, idx):
        idx = np.ascontiguousarray(idx, dtype=np.int32).ravel()
        lib().oracle_sim_decode_layer(self._h, layer, idx.size, _p(idx))

    def prefill_layer(self, layer, idx):
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        T, K = idx.shape
        lib().oracle_sim_prefill_layer(self._h, layer, T, K, _p(idx))

    def prefetch(self, layer, hist):
        """After a prefill layer: prefetch layer `layer`'s experts with hist[e] > 0."""
        hist = np.ascontiguousarray(hist, dtype=np.int32)
        assert hist.size == self.E
        return int(lib().oracle_sim_prefetch(self._h, layer, _p(hist)))

    def stats(self):
        out = np.zeros(len(STAT_NAMES), dtype=np.int64)
        lib().oracle_sim_stats(self._h, _p(out))
        return dict(zip(STAT_NAMES, (int(v) for v in out)))

    def reset_stats(self):
        lib().oracle_sim_reset_stats(self._h)

    def placement(self):
        slot_of = np.empty((self.L, self.E), dtype=np.int32)
        owner = np.empty(max(self.R, 1), dtype=np.int32)
        stamp = np.empty(max(self.R, 1), dtype=np.int64)
        counts = np.empty((self.L, self.E), dtype=np.int64)
        lib().oracle_sim_placement(self._h, _p(slot_of), _p(owner), _p(stamp), _p(counts))
        return slot_of, owner[:self.R], stamp[:self.R], counts

    def events(self):
        n = lib().oracle_sim_events(self._h, None, 0)
        out = np.zeros(n, dtype=EVENT_DTYPE)
        if n:
            lib().oracle_sim_events(self._h, _p(out), n)
        return out


def quota(L, P, layer):
    return int(lib().oracle_sim_quota(L, P, layer))

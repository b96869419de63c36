"""Seeded synthetic inputs for the resident-expert-caching workloads.

Shared by the CPU oracle and the GPU path; holds no method arithmetic (see
``gen.c``).  Every draw is a pure function of (seed, tensor id, counter), so
one expert, one layer or one token range can be regenerated on its own.

Workload recipes (the five workloads of the method's evaluation):

* ``tiny``    d=256, 16 experts, top-2, f=128, fp32 weights N(0, 0.02), 64
              tokens x ~ N(0, 1), no RMSNorm, no bias; seed 0.
* ``layer``   d=2048, 256 experts, top-8, f=512, Q4_0 weights (from
              N(0, 0.02)), fp32 router N(0, 0.02), 256 tokens, RMSNorm in the
              layer, no bias; seed 1.
* ``stack``   40 of the ``layer`` shape, residual x += MoE(RMSNorm(x)), Zipf
              router bias 2 ln p_r, p_r ~ r^-1.1 over a per-layer permutation;
              weights seed 2; 256 warm-up + 512 measured tokens.
* ``prefill`` the ``stack`` weights; 2048 tokens in one batch; the first 1024
              use permutation A (seed 2), the rest permutation B (seed 1002).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libworkload.so")
_lib = None

FMT_F32 = 0
FMT_Q4_0 = 1
ZIPF_ALPHA = 1.1
ZIPF_SCALE = 2.0
WEIGHT_SIGMA = 0.02


def build():
    """Compile ``libworkload.so`` (plain C, OpenMP)."""
    cmd = ["gcc", "-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fno-math-errno", "-fopenmp", "-fPIC",
           "-shared", "-Wall", "-o", _LIB_PATH + ".tmp", os.path.join(_HERE, "gen.c"), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        u64, i64, i32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.wl_philox4x64_10.argtypes = [vp, vp, vp]
        L.wl_normal_f32.argtypes = [u64, u64, u64, u64, i64, ctypes.c_float, vp]
        L.wl_uniform.argtypes = [u64, u64, u64, u64, u64]
        L.wl_uniform.restype = ctypes.c_double
        L.wl_f32_to_f16.argtypes = [ctypes.c_float]
        L.wl_f32_to_f16.restype = ctypes.c_uint16
        L.wl_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.wl_f16_to_f32.restype = ctypes.c_float
        L.wl_q4_0_encode.argtypes = [i64, i64, vp, vp]
        L.wl_router.argtypes = [u64, i32, i32, i32, ctypes.c_float, vp]
        L.wl_matrix_bytes.argtypes = [i32, i32, i32]
        L.wl_matrix_bytes.restype = i64
        L.wl_expert.argtypes = [u64, i32, i32, i32, i32, i32, ctypes.c_float, vp, vp, vp, vp]
        L.wl_experts.argtypes = [u64, i32, i32, i32, i32, i32, i32, ctypes.c_float, vp]
        L.wl_tokens.argtypes = [u64, u64, i64, i64, i32, vp]
        L.wl_zipf_bias.argtypes = [u64, i32, i32, ctypes.c_double, ctypes.c_double, vp, vp]
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def philox4x64_10(ctr, key):
    c = np.ascontiguousarray(ctr, dtype=np.uint64)
    k = np.ascontiguousarray(key, dtype=np.uint64)
    out = np.zeros(4, dtype=np.uint64)
    lib().wl_philox4x64_10(_p(c), _p(k), _p(out))
    return out


def normal_f32(seed, tensor, a, b, n, sigma):
    out = np.empty(n, dtype=np.float32)
    lib().wl_normal_f32(seed, tensor, a, b, n, sigma, _p(out))
    return out


def q4_0_encode(w):
    """fp32 [rows][cols] -> GGUF Q4_0 bytes [rows][cols/32][18]."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    assert cols % 32 == 0
    out = np.empty((rows, cols // 32, 18), dtype=np.uint8)
    lib().wl_q4_0_encode(rows, cols, _p(w), _p(out))
    return out


def matrix_bytes(rows, cols, wfmt):
    return int(lib().wl_matrix_bytes(rows, cols, wfmt))


def expert_bytes(d, f, wfmt):
    return 2 * matrix_bytes(f, d, wfmt) + matrix_bytes(d, f, wfmt)


def router(seed, layer, E, d, sigma=WEIGHT_SIGMA):
    out = np.empty((E, d), dtype=np.float32)
    lib().wl_router(seed, layer, E, d, sigma, _p(out))
    return out


def _shape_w(rows, cols, wfmt):
    return (rows, cols) if wfmt == FMT_F32 else (rows, cols // 32, 18)


def expert(seed, layer, e, d, f, wfmt, sigma=WEIGHT_SIGMA):
    """(gate [f][d], up [f][d], down [d][f]) in fp32 or GGUF Q4_0 blocks."""
    dt = np.float32 if wfmt == FMT_F32 else np.uint8
    g = np.empty(_shape_w(f, d, wfmt), dtype=dt)
    u = np.empty(_shape_w(f, d, wfmt), dtype=dt)
    dn = np.empty(_shape_w(d, f, wfmt), dtype=dt)
    scratch = np.empty(d * f, dtype=np.float32)
    rc = lib().wl_expert(seed, layer, e, d, f, wfmt, sigma, _p(g), _p(u), _p(dn), _p(scratch))
    assert rc == 0
    return g, u, dn


def experts_blob(seed, layer0, n_layers, E, d, f, wfmt, sigma=WEIGHT_SIGMA, out=None):
    """All experts of ``n_layers`` layers as one uint8 array [n_layers*E][expert_bytes],
    each expert gate | up | down (the layout of one expert in ``expert``)."""
    per = expert_bytes(d, f, wfmt)
    if out is None:
        out = np.empty((n_layers * E, per), dtype=np.uint8)
    assert out.shape == (n_layers * E, per) and out.dtype == np.uint8 and out.flags.c_contiguous
    rc = lib().wl_experts(seed, layer0, n_layers, E, d, f, wfmt, sigma, _p(out))
    assert rc == 0
    return out


def split_expert(blob_row, d, f, wfmt):
    """View one expert row of ``experts_blob`` as (gate, up, down)."""
    mb = matrix_bytes(f, d, wfmt)
    g = blob_row[:mb]
    u = blob_row[mb:2 * mb]
    dn = blob_row[2 * mb:]
    if wfmt == FMT_F32:
        return g.view(np.float32).reshape(f, d), u.view(np.float32).reshape(f, d), \
            dn.view(np.float32).reshape(d, f)
    return g.reshape(f, d // 32, 18), u.reshape(f, d // 32, 18), dn.reshape(d, f // 32, 18)


def tokens(seed, stream, t0, T, d):
    out = np.empty((T, d), dtype=np.float32)
    lib().wl_tokens(seed, stream, t0, T, d, _p(out))
    return out


def zipf_bias(seed, layer, E, alpha=ZIPF_ALPHA, scale=ZIPF_SCALE):
    """(bias fp32 [E], rank int32 [E], 1-based)."""
    b = np.empty(E, dtype=np.float32)
    r = np.empty(E, dtype=np.int32)
    lib().wl_zipf_bias(seed, layer, E, alpha, scale, _p(b), _p(r))
    return b, r


# ---- workload definitions -------------------------------------------------

class Workload:
    """Shapes and seeds of one workload; arrays are drawn on demand."""

    def __init__(self, name, d, E, K, f, L, wfmt, norm, seed, n_tokens, token_stream,
                 bias_seeds=(), warmup=0):
        self.name, self.d, self.E, self.K, self.f, self.L = name, d, E, K, f, L
        self.wfmt, self.norm, self.seed = wfmt, norm, seed
        self.n_tokens, self.token_stream = n_tokens, token_stream
        self.bias_seeds = tuple(bias_seeds)
        self.warmup = warmup

    @property
    def expert_bytes(self):
        return expert_bytes(self.d, self.f, self.wfmt)

    def router(self, layer):
        return router(self.seed, layer, self.E, self.d)

    def bias_rows(self, layer):
        """fp32 [n_rows][E] (one row per permutation seed) or None."""
        if not self.bias_seeds:
            return None
        return np.stack([zipf_bias(s, layer, self.E)[0] for s in self.bias_seeds])

    def expert(self, layer, e):
        return expert(self.seed, layer, e, self.d, self.f, self.wfmt)

    def experts_blob(self, layer0=0, n_layers=None, out=None):
        n_layers = self.L if n_layers is None else n_layers
        return experts_blob(self.seed, layer0, n_layers, self.E, self.d, self.f, self.wfmt, out=out)

    def tokens(self, t0=0, T=None):
        T = self.n_tokens if T is None else T
        return tokens(self.seed, self.token_stream, t0, T, self.d)


def tiny():
    return Workload("tiny", d=256, E=16, K=2, f=128, L=1, wfmt=FMT_F32, norm=False, seed=0,
                    n_tokens=64, token_stream=0)


def layer():
    return Workload("layer", d=2048, E=256, K=8, f=512, L=1, wfmt=FMT_Q4_0, norm=True, seed=1,
                    n_tokens=256, token_stream=1)


def stack(n_layers=40):
    return Workload("stack", d=2048, E=256, K=8, f=512, L=n_layers, wfmt=FMT_Q4_0, norm=True,
                    seed=2, n_tokens=768, token_stream=2, bias_seeds=(2,), warmup=256)


def prefill(n_layers=40):
    return Workload("prefill", d=2048, E=256, K=8, f=512, L=n_layers, wfmt=FMT_Q4_0, norm=True,
                    seed=2, n_tokens=2048, token_stream=4, bias_seeds=(2, 1002))

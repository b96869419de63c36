"""Python binding of ``libmoe_spark.so`` (resident expert caching for MoE decode
on one MI355X).

Argument marshalling only: every step of the hot path runs in the HIP kernels
of the library.  The functions keep the C names (``moe_spark_*``); device
buffers are passed as integer addresses (e.g. ``tensor.data_ptr()``) and
streams as ``hipStream_t`` integers (e.g. ``torch.cuda.current_stream().cuda_stream``).

If the library has not been built, importing this package raises: there is no
fallback path.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_spark.so")

OK, E_INVALID, E_NOMEM, E_HIP, E_STATE = 0, 1, 2, 3, 4
W_F32, W_Q4_0 = 0, 1
PRE_RMSNORM, RESIDUAL = 1, 2
EV_FILL = 2
_STATUS = {0: "OK", 1: "E_INVALID", 2: "E_NOMEM", 3: "E_HIP", 4: "E_STATE"}


class Config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("wfmt", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("n_bias_rows", ctypes.c_int32),
                ("resident_cap", ctypes.c_int64), ("ring_slots", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("event_cap", ctypes.c_int64)]


class Stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "accesses", "pinned_hits", "cold_hits", "ring_hits", "fills", "evictions", "h2d_bytes",
        "fill_ns_sum", "fill_ns_max", "calib_uploads", "tokens", "retunes", "retune_swaps",
        "prefetches")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


class Event(ctypes.Structure):
    _fields_ = [("seq", ctypes.c_int64), ("layer", ctypes.c_int32), ("expert", ctypes.c_int32),
                ("slot", ctypes.c_int32), ("kind", ctypes.c_int32), ("victim", ctypes.c_int32),
                ("pad", ctypes.c_int32)]


class MoeSparkError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run resident_expert_caching_amd.build.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
    st = ctypes.c_int
    sig = {
        "moe_spark_create": (st, [ctypes.POINTER(Config), vp, vp, ctypes.POINTER(vp)]),
        "moe_spark_destroy": (None, [vp]),
        "moe_spark_last_error": (ctypes.c_char_p, [vp]),
        "moe_spark_slot_bytes": (i64, [vp]),
        "moe_spark_set_router": (st, [vp, i32, vp, vp]),
        "moe_spark_set_expert": (st, [vp, i32, i32, vp, vp, vp]),
        "moe_spark_set_experts": (st, [vp, i64, i64, vp]),
        "moe_spark_place_uniform": (st, [vp]),
        "moe_spark_calibrate": (st, [vp, i32]),
        "moe_spark_set_autotune": (st, [vp, i32, i32, i32]),
        "moe_spark_layer_forward": (st, [vp, i32, vp, vp, i32, vp, u32, vp, vp]),
        "moe_spark_layer_forward_noalloc": (st, [vp, i32, vp, vp, i32, vp, u32, vp, vp]),
        "moe_spark_decode": (st, [vp, vp, i32, vp]),
        "moe_spark_decode_batched": (st, [vp, vp, i32, i32, vp]),
        "moe_spark_token_forward": (st, [vp, vp, vp]),
        "moe_spark_prefill": (st, [vp, vp, i32, vp]),
        "moe_spark_set_trace": (st, [vp, vp, vp, vp, i64]),
        "moe_spark_set_prefetch": (st, [vp, i32]),
        "moe_spark_get_prefetch_hist": (st, [vp, vp]),
        "moe_spark_get_stats": (st, [vp, ctypes.POINTER(Stats)]),
        "moe_spark_reset_stats": (st, [vp]),
        "moe_spark_get_placement": (st, [vp, vp, vp, vp, vp]),
        "moe_spark_get_events": (st, [vp, vp, i64, ctypes.POINTER(i64)]),
        "moe_spark_synchronize": (st, [vp]),
        "moe_spark_time_expert_kernels": (st, [vp, i32, ctypes.POINTER(ctypes.c_float),
                                               ctypes.POINTER(ctypes.c_float),
                                               ctypes.POINTER(ctypes.c_float)]),
        "moe_spark_time_stream_probe": (st, [vp, i32, ctypes.POINTER(ctypes.c_float)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


_lib = _load()
EXPORTED = tuple(n for n in dir(_lib) if n.startswith("moe_spark_"))


def _check(ctx, status):
    if status != OK:
        raise MoeSparkError(status, _lib.moe_spark_last_error(ctx).decode())


def moe_spark_create(cfg, compute_stream=None, copy_stream=None):
    h = ctypes.c_void_p()
    _check(None, _lib.moe_spark_create(ctypes.byref(cfg), compute_stream, copy_stream, ctypes.byref(h)))
    return h.value


def moe_spark_destroy(ctx):
    _lib.moe_spark_destroy(ctx)


def moe_spark_last_error(ctx):
    return _lib.moe_spark_last_error(ctx).decode()


def moe_spark_slot_bytes(ctx):
    return int(_lib.moe_spark_slot_bytes(ctx))


def moe_spark_set_router(ctx, layer, w_host, bias_host=None):
    _check(ctx, _lib.moe_spark_set_router(ctx, layer, w_host, bias_host))


def moe_spark_set_expert(ctx, layer, expert, gate, up, down):
    _check(ctx, _lib.moe_spark_set_expert(ctx, layer, expert, gate, up, down))


def moe_spark_set_experts(ctx, first, n, blob):
    _check(ctx, _lib.moe_spark_set_experts(ctx, first, n, blob))


def moe_spark_place_uniform(ctx):
    _check(ctx, _lib.moe_spark_place_uniform(ctx))


def moe_spark_calibrate(ctx, reset_counts=True):
    _check(ctx, _lib.moe_spark_calibrate(ctx, int(reset_counts)))


def moe_spark_set_autotune(ctx, interval_tokens, hysteresis_pct=25, decay_shift=1):
    _check(ctx, _lib.moe_spark_set_autotune(ctx, int(interval_tokens), int(hysteresis_pct), int(decay_shift)))


def moe_spark_layer_forward(ctx, layer, x, y, n_tokens, bias_row=None, flags=0, topk_out=None,
                            gates_out=None):
    _check(ctx, _lib.moe_spark_layer_forward(ctx, layer, x, y, n_tokens, bias_row, flags, topk_out,
                                             gates_out))


def moe_spark_layer_forward_noalloc(ctx, layer, x, y, n_tokens, bias_row=None, flags=0, topk_out=None,
                                    gates_out=None):
    _check(ctx, _lib.moe_spark_layer_forward_noalloc(ctx, layer, x, y, n_tokens, bias_row, flags, topk_out,
                                                     gates_out))


def moe_spark_decode(ctx, x, n_tokens, bias_row=None):
    _check(ctx, _lib.moe_spark_decode(ctx, x, n_tokens, bias_row))


def moe_spark_decode_batched(ctx, x, n_tokens, batch, bias_row=None):
    _check(ctx, _lib.moe_spark_decode_batched(ctx, x, n_tokens, batch, bias_row))


def moe_spark_token_forward(ctx, x, bias_row=None):
    _check(ctx, _lib.moe_spark_token_forward(ctx, x, bias_row))


def moe_spark_prefill(ctx, x, n_tokens, bias_row=None):
    _check(ctx, _lib.moe_spark_prefill(ctx, x, n_tokens, bias_row))


def moe_spark_set_trace(ctx, x_layers, topk, gates, cap_tokens):
    _check(ctx, _lib.moe_spark_set_trace(ctx, x_layers, topk, gates, cap_tokens))


def moe_spark_set_prefetch(ctx, enable):
    _check(ctx, _lib.moe_spark_set_prefetch(ctx, 1 if enable else 0))


def moe_spark_get_prefetch_hist(ctx, out):
    """out: host address of an int32 [L][E] buffer (e.g. numpy ``arr.ctypes.data``)."""
    _check(ctx, _lib.moe_spark_get_prefetch_hist(ctx, out))


def moe_spark_get_stats(ctx):
    s = Stats()
    _check(ctx, _lib.moe_spark_get_stats(ctx, ctypes.byref(s)))
    return s.as_dict()


def moe_spark_reset_stats(ctx):
    _check(ctx, _lib.moe_spark_reset_stats(ctx))


def moe_spark_get_placement(ctx, slot_of=None, ring_owner=None, ring_stamp=None, counts=None):
    """Host buffers are integer addresses (e.g. numpy ``arr.ctypes.data``) or None."""
    _check(ctx, _lib.moe_spark_get_placement(ctx, slot_of, ring_owner, ring_stamp, counts))


def moe_spark_get_events(ctx, out, cap):
    n = ctypes.c_int64()
    _check(ctx, _lib.moe_spark_get_events(ctx, out, cap, ctypes.byref(n)))
    return int(n.value)


def moe_spark_synchronize(ctx):
    _check(ctx, _lib.moe_spark_synchronize(ctx))


def moe_spark_time_expert_kernels(ctx, iters):
    a, b, c = ctypes.c_float(), ctypes.c_float(), ctypes.c_float()
    _check(ctx, _lib.moe_spark_time_expert_kernels(ctx, iters, ctypes.byref(a), ctypes.byref(b),
                                                   ctypes.byref(c)))
    return float(a.value), float(b.value), float(c.value)


def moe_spark_time_stream_probe(ctx, iters):
    us = ctypes.c_float()
    _check(ctx, _lib.moe_spark_time_stream_probe(ctx, iters, ctypes.byref(us)))
    return float(us.value)

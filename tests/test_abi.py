"""The C-ABI library loads, exports every function the public header declares,
and rejects bad configurations before touching a GPU.  No compute calls."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_spark.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(moe_spark_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    import resident_expert_caching_amd as m
    lib = ctypes.CDLL(m.LIB_PATH)
    names = declared_functions()
    assert len(names) >= 20
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    nm = subprocess.run(["nm", "-D", "--defined-only", m.LIB_PATH], capture_output=True, text=True,
                        check=True).stdout
    for n in names:
        assert re.search(r"\bT " + n + r"\b", nm), n
    for n in names:  # the binding keeps the C names
        assert callable(getattr(m, n)), n


def test_struct_layouts_match_the_header(tmp_path):
    import resident_expert_caching_amd as m
    src = tmp_path / "sz.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "moe_spark.h"\n'
                   'int main(void){printf("%zu %zu %zu %zu %zu %zu\\n", sizeof(moe_spark_config),'
                   ' sizeof(moe_spark_stats), sizeof(moe_spark_event),'
                   ' offsetof(moe_spark_config, resident_cap), offsetof(moe_spark_config, event_cap),'
                   ' offsetof(moe_spark_event, victim));return 0;}\n')
    exe = tmp_path / "sz"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    want = [ctypes.sizeof(m.Config), ctypes.sizeof(m.Stats), ctypes.sizeof(m.Event),
            m.Config.resident_cap.offset, m.Config.event_cap.offset, m.Event.victim.offset]
    assert got == want


def _cfg(**kw):
    import resident_expert_caching_amd as m
    base = dict(n_layers=2, d_model=2048, n_experts=16, top_k=8, d_ff=512, wfmt=m.W_Q4_0,
                rms_eps=1e-6, n_bias_rows=0, resident_cap=16, ring_slots=8, max_tokens=0,
                event_cap=0)
    base.update(kw)
    return m.Config(**base)


@pytest.mark.parametrize("kw,needle", [
    (dict(top_k=0), "top_k"),
    (dict(top_k=17, n_experts=32), "top_k"),
    (dict(n_experts=18), "n_experts"),
    (dict(resident_cap=33), "resident_cap"),
    (dict(resident_cap=-1), "resident_cap"),
    (dict(ring_slots=4), "ring_slots"),           # R < K while not all pinned
    (dict(d_model=1000), "d_model"),
    (dict(d_model=4096), "Q4_0"),                 # Q4_0 kernels are built for the target shape
    (dict(wfmt=7), "format"),
    (dict(n_layers=0), "n_layers"),
])
def test_bad_configs_are_rejected_without_a_gpu(kw, needle):
    import resident_expert_caching_amd as m
    with pytest.raises(m.MoeSparkError) as ei:
        m.moe_spark_create(_cfg(**kw))
    assert ei.value.status == m.E_INVALID
    assert needle in str(ei.value)

"""Host-side helpers of bench.py (CPU only): the kernel-code hash that keys
the committed HBM-counter summaries, their lookup, and the seeded length
recipe of the continuous-batching mix."""
import numpy as np

import bench


def test_code_hash_ignores_comments_and_whitespace():
    a = "int f(int x) {\n  return x + 1;  // one\n}\n/* block\n comment */\n"
    b = "// header\nint f(int x)\n{ return x + 1; }\n"
    c = "int f(int x) { return x + 2; }\n"
    assert bench.code_hash(a) == bench.code_hash(b)
    assert bench.code_hash(a) != bench.code_hash(c)


def test_kernels_code_hash_covers_every_kernel_source():
    """The hash keys on every device source the library builds."""
    import importlib
    import os
    build = importlib.import_module("paged_kv_cache_62_amd.build")  # the module, not the function
    built = {os.path.basename(s) for s in build.SOURCES if s.endswith(".hip")}
    assert built <= set(bench.KERNEL_SOURCES)
    assert len(bench.kernels_code_hash()) == 64
    # decode workloads key on the append and decode units, prefill on its own
    assert set(bench.workload_sources("qwen")) == {"device.h", "append.hip", "decode.hip"}
    assert set(bench.workload_sources("prefill512")) == {"device.h", "prefill.hip"}
    assert bench.kernels_code_hash(bench.DECODE_SOURCES) != bench.kernels_code_hash(bench.PREFILL_SOURCES)


def test_committed_summaries_parse():
    """Every summary bench.py reads exists and holds the two fields it parses;
    a workload without one reports no traffic."""
    import os
    import re
    for cfg, path in bench.TRAFFIC_PROFILES.items():
        text = open(os.path.join(bench.ROOT, path), encoding="utf-8").read()
        assert re.search(r"traffic_bytes_per_launch: \d+", text), cfg
        assert re.search(r"kernels_code_sha256: [0-9a-f]{64}", text), cfg
    assert bench.measured_traffic("no-such-workload") is None


def test_mix_suffix_lengths_recipe():
    """round(X), X ~ lognormal with mean 300, clamped to [1, 1024]; seeded."""
    x = bench.mix_suffix_lengths(62004, 20000)
    assert x.min() >= 1 and x.max() <= 1024
    assert abs(float(np.mean(x)) - 300.0) < 15.0
    np.testing.assert_array_equal(x, bench.mix_suffix_lengths(62004, 20000))
    assert not np.array_equal(x[:100], bench.mix_suffix_lengths(62005, 100))


def test_cpu_model_is_a_string():
    assert isinstance(bench.cpu_model(), str)

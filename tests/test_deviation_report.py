"""The stored FP8-vs-BF16 deviation table (tests/golden/fp8_vs_bf16_deviation.txt, information only) is what
its committed script computes: the tiny workload's line is recomputed here from the oracle."""
import importlib.util
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def test_stored_tiny_line_matches_the_script():
    spec = importlib.util.spec_from_file_location("dev_report", os.path.join(HERE, "golden", "fp8_vs_bf16_deviation.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    line = mod.run("tiny (1 x 256)", mod.wl.WORKLOADS["tiny"], [0])
    stored = open(os.path.join(HERE, "golden", "fp8_vs_bf16_deviation.txt")).read().splitlines()
    assert line in stored

"""The line bench.py prints, built from stand-in numbers on the CPU: one JSON
object of a few KB carrying the fields the benchmark contract names, however
large the extras (sweeps, ceilings, oracle timings) grow."""
import json

import bench


def _extras():
    sweep = {"M%d_N%d" % (m, n): {"ms": 0.1, "TFLOP/s": 1.0, "graph_ms": 0.1}
             for m in range(64) for n in (4096, 14336)}
    return {
        "invariance_bitwise": {"matmul": True, "rmsnorm": True, "attn_decode": True},
        "cost_of_invariance": dict(
            {"matmul_%s_M%d" % (p, m): {"invariant_ms": 0.1, "splitk_ms": 0.12,
                                        "invariant_over_splitk": 0.8333333,
                                        "invariant_over_vendor": 1.02}
             for m in (1, 16, 64) for p in ("qkv", "o", "gate_up", "down", "lm_head")},
            matmul_step_2048x4096x14336={"invariant_ms": 0.23, "invariant_over_splitk": 0.8333333,
                                         "invariant_over_vendor": 1.02},
            stack_token_ms={m: {"invariant": 3.0, "splitk": 2.5, "vendor": 2.8,
                                "invariant_over_splitk": 1.2, "invariant_over_vendor": 1.07}
                            for m in (1, 16, 64)},
            decode_B64_L4096={"invariant_over_splitkv": 0.87}),
        "sweeps": {"matmul": sweep, "rmsnorm": sweep, "decode": sweep},
        "ceilings": {"read_4GiB": {"GB/s": 6280.123456}},
        "e2e_llama8b": {"config": {"layers": 32},
                        "invariant": {"alone_s": 0.84, "batched64_s": 1.33,
                                      "batched64_tokens_per_s": 6142.9, "tokens_equal": True,
                                      "logits_bitwise_equal": True,
                                      "unique_outputs_over_30_calls": 1},
                        "comparator": {"alone_s": 0.74, "tokens_equal": False,
                                       "logits_bitwise_equal": False,
                                       "unique_outputs_over_30_calls": 4}},
        "cpu_oracle": {"error": "RuntimeError('x')"},
    }


def _line():
    comp = {s: {"ms": 0.2345678, "graph_ms": 0.2, "GB/s": 5000.123, "hbm_frac": 0.625,
                "extra_field": list(range(100))}
            for s in ("rmsnorm", "matmul", "attn_prefill", "attn_decode")}
    cpu = {"value": 0.0707, "unit": "TFLOP/s", "cores": 16, "kind": "oracle",
           "sample": "1505 of 2048 rows"}
    return bench.headline(20, 5, 0.4961234, 1006.123456, comp, cpu, 563.9e6, _extras(),
                          "gpurun_out/bench_extras.json")


def test_line_is_short_and_one_json_object():
    s = json.dumps(_line())
    assert "\n" not in s and len(s) < 4096, len(s)
    assert json.loads(s)["value"] == 1006.123456


def test_line_carries_the_contract_fields():
    line = _line()
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in line, k
    assert line["metric"] == json.load(open(bench.os.path.join(bench.ROOT, "BASELINE.json")))[
        "metric"]
    r = line["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert abs(r["frac"] - 1006.123456 / 2500.0) < 1e-3
    assert r["traffic"] == 563.9e6
    assert line["cpu_baseline"]["kind"] == "oracle" and line["cpu_baseline"]["cores"] == 16
    assert "workload" in line["config"]
    assert "sweeps" not in line and "ceilings" not in line
    assert "extra_field" not in line["components"]["matmul"]
    assert line["failed_extras"] == ["cpu_oracle"]
    assert line["e2e_llama8b"]["invariant"]["unique_outputs_over_30_calls"] == 1
    coi = line["cost_of_invariance"]
    assert coi["matmul_step_2048x4096x14336"] == {"invariant_over_splitk": 0.8333,
                                                  "invariant_over_vendor": 1.02}
    assert coi["stack_token_matmuls"]["M1"] == {"invariant_over_splitk": 1.2,
                                                "invariant_over_vendor": 1.07}
    assert "matmul_qkv_M1" not in coi and coi["decode_B64_L4096"]["invariant_over_splitkv"] == 0.87

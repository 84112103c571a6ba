"""bench.py's host logic (no GPU): the step's calls, the one-GPU guard and the
counter-summary lookup."""
import os

import bench


def test_step_calls_are_the_measured_workloads():
    names = [c.name for c in bench.step_calls()]
    assert names == ["down_i8x2", "batch8", "batch8_down_res", "prefill64", "lm_head"]
    rows = sorted({c.rows for c in bench.step_calls()})
    assert rows == [1, 8, 64]


def test_other_calls_cover_every_mode_and_the_small_configs():
    calls = bench.other_calls()
    names = [c.name for c in calls]
    assert "tiny" in names and "attn" in names
    for shape in ("up", "down"):
        assert sorted(c.mode for c in calls if c.name.startswith(shape + "_")) == ["f32", "i8", "i8x2"]
    assert not set(names) & {c.name for c in bench.step_calls()} - {"down_i8x2"}


def test_more_than_one_gpu_is_refused():
    assert bench.main(["--gpus", "2"]) == 2


def test_counter_summary_is_keyed_on_its_sources(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel v1")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    h = bench.kernel_hash(["k.hip"])
    (tmp_path / "demo_counters.txt").write_text(
        f"# comment = ignored\ncall = demo\nkernel_sources = k.hip\nkernel_sources_sha256_16 = {h}\nhbm_bytes_per_launch = 1234\n")
    assert bench.stored_traffic("demo") == 1234.0
    assert bench.stored_traffic("other") is None
    assert bench.stored_traffic("dem") is None
    src.write_text("kernel v2")
    assert bench.stored_traffic("demo") is None
    assert os.path.exists(tmp_path / "demo_counters.txt")


def test_decode_layer_is_one_layers_projections():
    calls = bench.decode_layer_calls()
    assert [(c.n, c.k) for c in calls] == [(6144, 4096), (4096, 4096), (14336, 4096), (14336, 4096), (4096, 14336)]
    assert all(c.rows == 1 and c.mode == "i8x2" for c in calls)
    gate, up = calls[2], calls[3]
    assert gate.x_seed == up.x_seed and gate.w_seed != up.w_seed
    assert [c.residual_seed is not None for c in calls] == [False, True, False, False, True]


def test_rows_summary_keys_on_the_metric_shapes():
    """rows=1 is the 4096x14336 down projection alone (not mixed with the LM
    head), rows=8 the two batched calls, rows=64 the prefill, and the LM head
    is reported apart."""
    wb = 62390272
    per_call = {"down_i8x2": {"weight_bytes": wb, "project_us": 12.0},
                "batch8": {"weight_bytes": wb, "project_us": 14.0},
                "batch8_down_res": {"weight_bytes": wb, "project_us": 16.0},
                "prefill64": {"weight_bytes": wb, "project_us": 34.0},
                "lm_head": {"weight_bytes": 330612736, "project_us": 50.0}}
    ceiling = {str(wb): {"us": 10.0}, "330612736": {"us": 48.0}}
    s = bench.rows_summary(per_call, ceiling)
    assert s["1"]["calls"] == ["down_i8x2"] and s["lm_head"]["calls"] == ["lm_head"]
    assert abs(s["1"]["GBps"] - wb / 12.0 / 1e3) < 0.1
    assert abs(s["8"]["GBps"] - 2 * wb / 30.0 / 1e3) < 0.1
    assert s["64"]["pct_of_stream_ceiling"] == round(10.0 / 34.0 * 100, 1)
    assert s["1"]["pct_hbm_peak"] == round(wb / 12.0 / 1e3 / 8000 * 100, 1)

"""bench.py's host logic: the kernel-name map the counter summary relies on,
and the algorithmic bytes per element against the closed forms."""
import bench
from synth import WORKLOADS


def _name(inst):
    return f"void ob::(anonymous namespace)::{inst}(ob::Geometry, ob::WorkerArgs)"


def test_kind_of_maps_every_library_kernel():
    cases = {
        "worker_kernel<float, 0>": "worker_pass1",
        "worker_kernel<float, 1>": "worker_pass2",
        "worker_kernel<unsigned short, 1>": "worker_pass2",
        "worker_chunk_kernel<float, 2>": "worker_residual_first",
        "worker_chunk_kernel<float, 3>": "worker_residual",
        "worker_chunk_kernel<unsigned short, 3>": "worker_residual",
        "worker_chunk_kernel<float, 4>": "worker_pass2",
        "server_kernel<0, true>": "server_pass1",
        "server_kernel<2, false>": "server_pass2_update",
        "server_kernel<4, true>": "server_residual",
        "update_kernel<false, false>": "update_residual",
        "update_kernel<true, false>": "apply_update",
        "warmup_kernel<float, true>": "warmup",
        "topk_gather<float>": "cltk_gather",
        "topk_gather_chunk<unsigned short>": "cltk_gather",
        "topk_average<true>": "cltk_average",
        "topk_ties": "cltk_select",
        "topk_pass1<float>": "cltk_select",
        "topk_hist_shared<9, 11>": "cltk_select",
        "topk_reset": "cltk_select",
    }
    for inst, kind in cases.items():
        assert bench.kind_of(_name(inst)) == kind, inst
    assert bench.kind_of("__amd_rocclr_copyBuffer") == "copy"
    assert bench.kind_of("some_torch_kernel") is None


def test_algorithmic_bytes_closed_forms():
    bl, gpt = WORKLOADS["bert_large"], WORKLOADS["gpt_1p3b_bf16"]
    # 28 + (8 + g) W + W/4: 126 at W = 8 with fp32 gradients, 110 with bf16
    assert bench.step_bytes_per_element(bl) == 126.0
    assert bench.step_bytes_per_element(gpt) == 110.0
    kb = bench.kernel_bytes_per_element(bl)
    assert kb["worker_residual"] == 12 * 8 + 1 + 0.125
    assert kb["server_residual"] + kb["update_residual"] + kb["worker_residual"] == 118.375
    cl = bench.cltk_bytes_per_element(bl, 0.01)
    assert cl["cltk_select"] == 8.0 and abs(cl["cltk_gather"] - 96.36) < 1e-9


def test_more_than_one_gpu_is_refused():
    """One GPU holds every simulated worker: --gpus N > 1 exits with a message
    before touching a device."""
    import subprocess
    import sys
    root = bench.ROOT
    r = subprocess.run([sys.executable, f"{root}/bench.py", "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr + r.stdout


def test_summarize_reports_the_median_run_and_three_fractions():
    wl = WORKLOADS["bert_large"]
    n = sum(wl.numel)
    steps = 20
    runs = [0.140, 0.134, 0.150, 0.136, 0.138]          # seconds per run of 20 steps
    per = {"worker_residual": 5.3, "server_residual": 0.59, "update_residual": 0.69, "scale_finalize": 0.02}
    launches = {"worker_residual": 100, "server_residual": 100, "update_residual": 100, "scale_finalize": 200}
    kernels = {k: (per[k] * launches[k], launches[k]) for k in per}
    kernels.update({k: (0.0, 0) for k in bench.kernel_bytes_per_element(wl) if k not in kernels})
    r = bench.summarize(wl, n, steps, runs, kernels, "no_counters_for_this_name")
    assert r["repeats"] == 5
    assert abs(r["ms_per_step"] - 138 / 20) < 1e-9                   # the median run
    assert r["ms_per_step_min"] == round(134 / 20, 4) and r["ms_per_step_max"] == round(150 / 20, 4)
    f = r["step_fraction"]
    assert f["method_bytes_per_element"] == 126.0
    assert abs(f["moved_bytes_per_element"] - (97.125 + 9.125 + 12.125)) < 1e-9   # the residual kernels' bytes
    assert abs(f["by_bytes_moved"] / f["by_method_bytes"] - 118.375 / 126.0) < 1e-3
    assert f["by_counters"] is None and r["roofline"]["kernel"] == "worker_residual"


def test_cpu_baseline_runs_the_whole_list():
    import torch
    from synth import grads_for_step, init_state
    from synth.workloads import Workload
    wl = Workload(name="tiny", tensors=(("a", (1000,)), ("b", (8193,)), ("c", (64,))), workers=3,
                  grad_dtype="f32", steps=1, g_sigma=1e-3, v_kind="sq_normal", v_a=1e-3, v_b=1e-12)
    st = init_state(wl, "cpu")
    g = grads_for_step(wl, 0, "cpu")
    r = bench.cpu_baseline(wl, st, g, repeats=2)
    assert r["kind"] == "oracle" and r["cores"] == 1 and r["value"] > 0
    assert str(sum(wl.numel)) in r["sample"] and r["all_cores"]["repeats"] == 2
    assert r["host_nproc"] >= 1 and r["cpu_model"]
    assert torch.equal(st["p"], init_state(wl, "cpu")["p"])   # host copies: the caller's state is untouched


def test_server_pieces_matches_the_partition():
    for n in (1, 8192, 8193, 70001, 31254528):
        for c in (1, 2, 3, 8, 1000):
            blocks = -(-n // 8192)
            size = 8192 * -(-blocks // c)
            assert bench.server_pieces(n, c) == len(range(0, n, size))


def test_counter_traffic_is_dropped_when_its_sources_change(tmp_path, monkeypatch):
    """Stored HBM counters count only for the sources they measured: a kernel's
    own file plus the shared constants and the launch code."""
    import json
    shas = {s: bench.sha256_of(s) for s in bench.SOURCES}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "tiny_hbm_counters.json").write_text(json.dumps({
        "sources_sha256": shas,
        "per_launch_bytes": {"worker_residual": 1.0e9, "cltk_gather": 2.0e9}}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.counter_traffic("tiny", "worker_residual") == 1.0e9
    assert bench.counter_traffic("tiny", "cltk_gather") == 2.0e9
    assert bench.counter_traffic("tiny", "server_residual") is None       # not measured
    assert bench.counter_traffic("absent", "worker_residual") is None    # no file

    def changed(name):
        return lambda s: "0" * 64 if s == name else shas[s]
    for name, stale in [("api.cpp", {"worker_residual", "cltk_gather"}),
                        ("internal.h", {"worker_residual", "cltk_gather"}),
                        ("kernels.hip", {"worker_residual"}),
                        ("topk.hip", {"cltk_gather"})]:
        monkeypatch.setattr(bench, "sha256_of", changed(name))
        for kernel in ("worker_residual", "cltk_gather"):
            got = bench.counter_traffic("tiny", kernel)
            assert (got is None) == (kernel in stale), (name, kernel, got)

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
        "server_kernel<0, true>": "server_pass1",
        "server_kernel<2, false>": "server_pass2_update",
        "server_kernel<4, true>": "server_residual",
        "update_kernel<false, false>": "update_residual",
        "update_kernel<true, false>": "apply_update",
        "warmup_kernel<float, true>": "warmup",
        "topk_gather<float>": "cltk_gather",
        "topk_average<true>": "cltk_average",
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

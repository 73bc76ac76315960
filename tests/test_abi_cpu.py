"""The C-ABI library on the CPU: it loads, exports every symbol include/ob.h
declares, and its host-only entry points (layout, status strings, argument
checks that fail before any device work) behave as documented."""
import ctypes
import os
import re
import subprocess

import pytest

from synth.workloads import WORKLOADS, padded_layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ob.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ob_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from error_compensated_bit_02_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libob.so is not built: run python -m error_compensated_bit_02_amd.build")
    return binding.load_library()


def test_header_declares_the_boundary():
    names = _declared()
    for required in ("ob_init", "ob_compress_worker", "ob_server_reduce", "ob_apply_update",
                     "ob_step", "ob_destroy", "ob_layout", "ob_status_string"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    from error_compensated_bit_02_amd import binding
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (ob_[a-z_]+)\b", out))
    for name in _declared():
        assert name in exported, name
        assert hasattr(lib, name)
    assert set(binding.SIGNATURES) == set(_declared())


def test_layout_matches_padded_layout(lib):
    from error_compensated_bit_02_amd import binding
    for wl in WORKLOADS.values():
        off, _ = padded_layout(wl.numel)
        assert binding.layout(wl.numel) == off, wl.name
    assert binding.layout([1, 63, 64, 65, 1000]) == [0, 64, 128, 192, 320, 1344]


def test_layout_rejects_bad_input(lib):
    T = 3
    out = (ctypes.c_int64 * (T + 1))()
    assert lib.ob_layout(T, (ctypes.c_int64 * T)(5, 0, 7), out) == 1
    assert lib.ob_layout(T, (ctypes.c_int64 * T)(5, -1, 7), out) == 1
    assert lib.ob_layout(0, (ctypes.c_int64 * 1)(5), out) == 1
    assert lib.ob_layout(T, None, out) == 1


def test_status_strings(lib):
    for code, text in [(0, "ok"), (1, "invalid argument"), (3, "out of memory")]:
        assert lib.ob_status_string(code).decode() == text
    assert lib.ob_status_string(99).decode() == "unknown status"


def test_init_argument_checks_fail_before_device_work(lib):
    ctx = ctypes.c_void_p()
    n = (ctypes.c_int64 * 2)(100, 200)
    assert lib.ob_init(ctypes.byref(ctx), 2, n, 0, 0, 0.9, 1e-8) == 1       # W = 0
    assert lib.ob_init(ctypes.byref(ctx), 2, n, 4, 7, 0.9, 1e-8) == 1       # bad dtype
    assert lib.ob_init(ctypes.byref(ctx), 2, n, 4, 0, 1.0, 1e-8) == 1       # beta1 = 1
    assert lib.ob_init(ctypes.byref(ctx), 2, n, 4, 0, float("nan"), 1e-8) == 1
    assert lib.ob_init(ctypes.byref(ctx), 2, n, 4, 0, 0.9, 0.0) == 1        # eps = 0
    assert lib.ob_init(ctypes.byref(ctx), 2, (ctypes.c_int64 * 2)(100, 0), 4, 0, 0.9, 1e-8) == 1
    assert lib.ob_init(None, 2, n, 4, 0, 0.9, 1e-8) == 1
    assert lib.ob_init(ctypes.byref(ctx), 2, n, 4097, 0, 0.9, 1e-8) == 1    # W > 4096
    assert lib.ob_init(ctypes.byref(ctx), 2, n, 4, 0, 0.9, 1e-50) == 1     # eps rounds to 0 in fp32
    assert ctx.value is None


def test_init_rejects_lists_beyond_the_grid_limit(lib):
    """Checked on the host before any device call: 2^40 elements is 2^27 tiles
    of 8192, beyond 16,777,215 workgroups; 2^34 elements is 2^21 tiles, whose
    2^24 chunks of 1024 (the residual worker pass) exceed it by one; 4096
    workers x 20,000 tensors needs up to 81.92 M scale workgroups (one per
    worker and tensor)."""
    ctx = ctypes.c_void_p()
    big = (ctypes.c_int64 * 1)(1 << 40)
    assert lib.ob_init(ctypes.byref(ctx), 1, big, 1, 0, 0.9, 1e-8) == 1
    chunks = (ctypes.c_int64 * 1)(1 << 34)
    assert lib.ob_init(ctypes.byref(ctx), 1, chunks, 1, 0, 0.9, 1e-8) == 1
    many = (ctypes.c_int64 * 20000)(*([1] * 20000))
    assert lib.ob_init(ctypes.byref(ctx), 20000, many, 4096, 0, 0.9, 1e-8) == 1
    assert ctx.value is None
    # calls on a NULL context are rejected, nothing is launched
    assert lib.ob_step(None, *([None] * 10), 1e-4, None) == 1
    assert lib.ob_compress_worker(None, 0, 1, *([None] * 6)) == 1
    lib.ob_destroy(None)


def test_profile_kind_names(lib):
    k = lib.ob_profile_kinds()
    names = [lib.ob_profile_kind_name(i).decode() for i in range(k)]
    assert names[0] == "worker_pass1" and "server_pass2_update" in names
    assert lib.ob_profile_kind_name(k) is None


def test_every_method_declaration_cites_its_source():
    """Each entry point that computes a step of the method carries, in the
    comment above its declaration, the page and the section that define it."""
    import re
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "ob.h")
    with open(path) as f:
        text = f.read()
    sections = ("Abstract", "Proposed method", "One-line summary", "Main results")
    for name in ("ob_init", "ob_compress_worker", "ob_server_reduce", "ob_apply_update", "ob_step",
                 "ob_step_residual", "ob_materialize", "ob_warmup_step", "ob_begin_compression",
                 "ob_set_server_chunks", "ob_set_trust_ratio", "ob_cltk_configure"):
        m = re.search(r"\n(?:int|int32_t|void) " + name + r"\(", text)
        assert m, f"{name} is not declared"
        end = text.rfind("*/", 0, m.start())
        comment = text[text.rfind("/*", 0, end): end]
        assert "Source:" in comment, f"{name}: no Source line in the comment above its declaration"
        src = comment[comment.index("Source:"):]
        assert ("review" in src or "page" in src) and any(s in src for s in sections), \
            f"{name}: the Source line names no page and section"

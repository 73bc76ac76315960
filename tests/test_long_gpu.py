"""Long trajectories against the oracle: errors, momentum and parameters
compound over many steps, so a one-ulp difference anywhere would grow and
show; every compared float must stay bit-identical after every step."""
import pytest
import torch

from harness import log, parity_run
from test_cltk_gpu import _run as cltk_run
from test_parity_gpu import RAGGED, _report, _wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from error_compensated_bit_02_amd import load_library
    load_library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("residual", [False, True], ids=["strict", "residual"])
def test_hundred_steps(residual):
    wl = _wl("long_w4", RAGGED, 4, steps=100)
    rep = parity_run(wl, wl.steps, residual=residual)
    _report(wl.name + (" residual" if residual else " strict"), rep)
    assert rep.exact_floats == rep.total_floats


def test_sixty_steps_bf16_w8():
    wl = _wl("long_bf16_w8", RAGGED, 8, dtype="bf16", steps=60, g_sigma=5e-4)
    rep = parity_run(wl, wl.steps, residual=True)
    _report(wl.name, rep)
    assert rep.exact_floats == rep.total_floats


def test_cltk_sixty_exchanges():
    """The leader cycles through the 4 workers 15 times; memories accumulate."""
    wl = _wl("long_cltk_w4", RAGGED, 4, steps=60)
    exact, total = cltk_run(wl, 0.02, wl.steps)
    log(f"cltk 60 exchanges: {exact}/{total}")

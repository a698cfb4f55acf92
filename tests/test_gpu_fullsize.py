"""Parity at the workloads' full sizes, in the benchmark's launch
configuration, on sampled states (see tests/fullsize.py)."""
import pytest
import torch

from tests import fullsize
from workloads.configs import WORKLOADS

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free_memory():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_fullsize_b256_4layers():
    """Batch 256 x 32 heads x 4 layers (32,768 states), 1,024 tokens: the
    benchmarked workload, in the benchmark's default schedule (last token of
    each window fused with the close)."""
    s = fullsize.run(WORKLOADS["gdn_b256_h32_4layers"], n_forced=12, n_free=8, fused=True)
    assert s["flips"] <= 1e-3 * s["codes"]


def test_fullsize_b256_4layers_separate_close():
    """The benchmarked workload with p decode steps and one window close
    over all layers per window (bench.py --close separate)."""
    s = fullsize.run(WORKLOADS["gdn_b256_h32_4layers"], n_forced=12, n_free=8)
    assert s["flips"] <= 1e-3 * s["codes"]


def test_fullsize_gdn_layer_b64():
    s = fullsize.run(WORKLOADS["gdn_layer_h32_b64"], n_forced=8, n_free=8)
    assert s["flips"] <= 1e-3 * s["codes"]


def test_fullsize_kda_b128():
    s = fullsize.run(WORKLOADS["kda_h32_b128"], n_forced=8, n_free=8, fused=True)
    assert s["flips"] <= 1e-3 * s["codes"]


def test_fullsize_long_decode_64k():
    """65,536 tokens for 128 states: snapshots every 1,024 tokens, state MSE
    against the exact recurrence, resume from a mid-run snapshot."""
    s = fullsize.run(WORKLOADS["gdn_long64k_h16_b8"], n_forced=3, n_free=3, checkpoint_every=1024)
    assert s["flips"] <= 1e-3 * s["codes"]
    assert "resume" in s

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library, loaded once; fails (not skips) if it is missing on a GPU run."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from quantized_weight_verification_amd import _binding

    return _binding.lib()


def pytest_terminal_summary(terminalreporter):
    """The fp16 parity bars of the session: per test file, the largest max-abs-rel error and
    the largest element-wise relative error over the outputs with |r| > 0.1 max|r|."""
    try:
        from _util import FP_ERRORS
    except ImportError:
        return
    if not FP_ERRORS:
        return
    worst = {}
    for tid, e, el in FP_ERRORS:
        f = tid.split("::")[0]
        w = worst.setdefault(f, [0, 0.0, 0.0])
        w[0] += 1
        w[1] = max(w[1], e)
        w[2] = max(w[2], el)
    terminalreporter.write_sep("-", "fp16 parity (worst per file)")
    for f, (n, e, el) in sorted(worst.items()):
        terminalreporter.write_line(f"{f}: {n} checks, max-abs-rel {e:.3e}, "
                                    f"element-wise rel (|r| > 0.1 max) {el:.3e}")

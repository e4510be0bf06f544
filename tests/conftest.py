import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (full-size workloads)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP binding, with the built library loaded; skips cleanly only when no GPU exists."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_causal_gqa_cpattn_amd as cp
    cp.load()  # raises if the library is missing: no fallback path exists
    return cp


def pytest_terminal_summary(terminalreporter):
    """Parity margins of the run: every comparison of a named workload (labels starting
    with "cfg"), and the worst case of each bar over the rest, so that the tail of a
    quiet run still shows how close the HIP path came to each tolerance."""
    h = sys.modules.get("harness")
    if h is None or not h.MARGINS:
        return
    tr = terminalreporter
    tr.section("parity margins")
    for name, bar, _, _, line in h.MARGINS:
        if name.startswith("cfg"):
            tr.write_line(line)
    for bar in ("configs", "pages", "lse"):
        rest = [m for m in h.MARGINS if m[1] == bar and not m[0].startswith("cfg")]
        if rest:
            worst = max(rest, key=lambda m: m[2])
            worst_rl2 = max(rest, key=lambda m: m[3])
            tr.write_line(f"other bar={bar} comparisons={len(rest)} worst_max_abs: {worst[4]}")
            if bar != "lse":
                tr.write_line(f"other bar={bar} worst_rel_l2: {worst_rl2[4]}")

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests are collected everywhere but skipped cleanly where no GPU exists,
    # so that `-m "not gpu"` and a bare run both work on CPU-only hosts.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU on this host")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    """The floating-point comparisons of this run, largest fraction of the bar
    first (fp32: row-relative / 1e-5; bf16: the larger of absolute and
    row-relative / 2e-2)."""
    gu = sys.modules.get("gpu_util")
    recs = getattr(gu, "RECORDS", None)
    if not recs:
        return
    tr = terminalreporter
    tr.write_sep("-", f"parity margins: {len(recs)} comparisons against the oracle")
    worst = sorted(recs, key=lambda r: -r["frac_of_bar"])
    for r in worst[:12]:
        tr.write_line(f"{r['frac_of_bar']:7.3f} of bar  abs {r['max_abs']:.2e}  row_rel {r['max_row_rel']:.2e}  "
                      f"{r['dtype']}  {r['what']}")
    by = {}
    for r in recs:
        by.setdefault(r["dtype"], []).append(r["frac_of_bar"])
    tr.write_line("  ".join(f"{d}: {len(v)} checks, max {max(v):.3f} / median {sorted(v)[len(v) // 2]:.3f} of bar"
                            for d, v in sorted(by.items())))

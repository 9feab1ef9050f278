"""Helpers for GPU parity tests: host<->device transfer and the error metrics.

Metrics (floating point):
* fp32: the per-row relative error ``max_d |gpu - ref| / max_d |ref|`` (row = one
  (sequence, q head) output vector), maximised over rows, must be <= 1e-5;
* bf16: the max absolute error must be <= 2e-2 AND the per-row relative error
  must be <= 2e-2.
Element-wise relative error is not used: it is unbounded near zero.
"""

import json
import os
import sys
import tempfile

import numpy as np
import torch

FP32_ROW_REL = 1e-5
BF16_ABS = 2e-2
BF16_ROW_REL = 2e-2

# Every comparison's errors, kept for the run's summary and written one JSON
# line each to $PKV_PARITY_LOG (default: pkv_parity_margins.jsonl in the system
# temporary directory), so a run's margins against the bars can be read back.
RECORDS = []


def _record(what, dtype, max_abs, max_row_rel):
    bar = FP32_ROW_REL if dtype == "f32" else BF16_ROW_REL
    rec = {"test": os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], "what": what, "dtype": dtype,
           "max_abs": max_abs, "max_row_rel": max_row_rel,
           "frac_of_bar": max(max_row_rel / bar, 0.0 if dtype == "f32" else max_abs / BF16_ABS)}
    RECORDS.append(rec)
    path = os.environ.get("PKV_PARITY_LOG") or os.path.join(tempfile.gettempdir(), "pkv_parity_margins.jsonl")
    try:
        os.makedirs(os.path.dirname(path), exist_ok=True)
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")
    except OSError:
        pass


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    """numpy -> device tensor; uint16 arrays become bfloat16 (bit patterns preserved)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def host(t):
    """device tensor -> numpy in storage form (bfloat16 -> uint16 bits)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def host_f64(t):
    """device output -> exact float64 values."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got, ref):
    """(max abs error, max per-row relative error) over rows of the last axis."""
    got = np.asarray(got, np.float64).reshape(-1, got.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    diff = np.abs(got - ref)
    scale = np.max(np.abs(ref), axis=1)
    row = np.max(diff, axis=1) / np.where(scale > 0, scale, 1.0)
    return float(diff.max(initial=0.0)), float(row.max(initial=0.0))


def assert_close(got, ref, dtype, what=""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    a, r = errors(got, ref)
    say(f"  {what}: max_abs={a:.3e} max_row_rel={r:.3e} ({dtype})")
    _record(what, dtype, a, r)
    if dtype == "f32":
        assert r <= FP32_ROW_REL, f"{what}: fp32 row-relative error {r:.3e} > {FP32_ROW_REL}"
    else:
        assert a <= BF16_ABS, f"{what}: bf16 abs error {a:.3e} > {BF16_ABS}"
        assert r <= BF16_ROW_REL, f"{what}: bf16 row-relative error {r:.3e} > {BF16_ROW_REL}"

"""Shared helpers of the GPU parity tests: host<->device transfer of bf16 bit
patterns and the floating-point gates."""
from __future__ import annotations

import json
import os
import sys

import numpy as np

# Gates for bf16 inputs against the fp64 oracle: relative L2 and max abs error.
REL_L2 = 5e-3
MAX_ABS = 2e-2
LSE_ABS = 1e-3


_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MARGIN_LOG = os.path.join(_ROOT, "gpurun_out", "parity_margins.jsonl")


def say(*a):
    """Name the case on stdout (flushed) before a GPU step, and keep the line in
    the parity log (pulled back with the run's outputs)."""
    msg = " ".join(str(x) for x in a)
    print(msg, flush=True)
    sys.stdout.flush()
    _log({"msg": msg})


def _log(rec):
    rec = {"test": os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], **rec}
    try:
        os.makedirs(os.path.dirname(MARGIN_LOG), exist_ok=True)
        with open(MARGIN_LOG, "a") as f:
            f.write(json.dumps(rec) + "\n")
    except OSError:
        pass


def to_dev_bf16(bits: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def to_dev(x: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def bits_of(t) -> np.ndarray:
    """bf16 device tensor -> uint16 host array (bit patterns)."""
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64_of(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        from oracle.ref import bf16_to_f64
        return bf16_to_f64(bits_of(t))
    return t.detach().cpu().numpy().astype(np.float64)


def errors(got: np.ndarray, ref: np.ndarray):
    """(relative L2, max abs) of got against ref; relative L2 is 0 when both are
    exactly zero and undefined (None) when only the reference is."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = got - ref
    nd, nr = float(np.linalg.norm(diff)), float(np.linalg.norm(ref))
    rel = nd / nr if nr > 0 else (0.0 if nd == 0 else None)
    mx = float(np.abs(diff).max()) if diff.size else 0.0
    return rel, mx


def gate(name: str, got, ref, rel_tol=REL_L2, abs_tol=MAX_ABS):
    rel, mx = errors(got, ref)
    print(f"  {name}: relL2={'n/a (zero reference)' if rel is None else f'{rel:.3e}'} "
          f"maxabs={mx:.3e}", flush=True)
    _log({"gate": name, "relL2": rel, "maxabs": mx, "n": int(np.size(ref)),
          "rel_tol": rel_tol, "abs_tol": abs_tol})
    assert np.isfinite(ref).all(), f"{name}: non-finite reference"
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    if rel is not None:      # an exactly-zero reference is gated on max abs alone
        assert rel <= rel_tol, f"{name}: relL2 {rel:.3e} > {rel_tol}"
    assert mx <= abs_tol, f"{name}: maxabs {mx:.3e} > {abs_tol}"
    return rel, mx

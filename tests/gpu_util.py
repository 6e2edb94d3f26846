"""Helpers for the GPU parity tests: upload seeded inputs, compare with the oracle."""
from __future__ import annotations

import json
import os
import sys

import numpy as np
import torch

import workloads as W

ATOL = 2e-2     # max-abs bound on attention outputs
REL_L2 = 5e-3   # relative L2 bound on attention outputs


# When CPTHD_MARGINS names a file, every attention comparison appends one JSON line there: the case being
# checked (set_case), the tensor, its max-abs and relative-L2 error against the oracle and the entries compared.
_MARGINS = os.environ.get("CPTHD_MARGINS")
_CASE = {"case": ""}


def set_case(label):
    _CASE["case"] = label


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _record(name, mx, rel, n):
    if _MARGINS:
        with open(_MARGINS, "a") as f:
            f.write(json.dumps({"case": _CASE["case"], "tensor": name, "max_abs": mx, "rel_l2": rel, "n": int(n)})
                    + "\n")


def bf16_dev(x):
    """float32 values -> a bf16 device tensor (round to nearest even; values the seeded generators already rounded
    to bf16 keep their bits)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bits = (u >> np.uint32(16)).astype(np.uint16) if not (u & np.uint32(0xFFFF)).any() else W.to_bf16_bits(x)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda")


def i32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")


def status_dev():
    return torch.zeros(1, dtype=torch.int32, device="cuda")


def to_np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_attn_close(name, got, ref, valid=None):
    """Max-abs and relative-L2 on `valid` entries; everything else must match exactly.

    ``ref`` may hold NaN where the oracle did not compute (sampled checks): those
    entries are skipped.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    known = ~np.isnan(ref)
    if valid is None:
        valid = np.isfinite(ref)
    valid = np.broadcast_to(valid, ref.shape) & known
    exact = known & ~valid
    if exact.any():
        g, r = got[exact], ref[exact]
        same = (g == r) | (np.isinf(g) & np.isinf(r) & (np.sign(g) == np.sign(r)))
        assert same.all(), f"{name}: {np.count_nonzero(~same)} entries differ where exact values are required"
    if valid.any():
        g, r = got[valid], ref[valid]
        assert np.isfinite(g).all(), f"{name}: non-finite values"
        err = np.abs(g - r)
        mx = float(err.max())
        nrm = float(np.linalg.norm(r))
        rel = float(np.linalg.norm(g - r) / nrm) if nrm > 0 else float(np.linalg.norm(g - r))
        log(f"    {name}: max_abs={mx:.3e} rel_l2={rel:.3e} n={g.size}")
        _record(name, mx, rel, g.size)
        assert mx <= ATOL, f"{name}: max abs error {mx:.4e} > {ATOL}"
        assert rel <= REL_L2, f"{name}: relative L2 error {rel:.4e} > {REL_L2}"

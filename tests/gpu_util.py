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


def assert_attn_close(name, got, ref, valid=None, atol_rel_to_max=False):
    """Max-abs and relative-L2 on `valid` entries; everything else must match exactly.

    ``ref`` may hold NaN where the oracle did not compute (sampled checks): those
    entries are skipped.  With ``atol_rel_to_max`` the max-abs bound is ATOL times
    the larger of 1 and the reference's largest magnitude (for inputs far outside
    the measured workloads' value range, where the gradients grow with them).
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
        atol = ATOL * max(1.0, float(np.abs(r).max())) if atol_rel_to_max else ATOL
        log(f"    {name}: max_abs={mx:.3e} rel_l2={rel:.3e} n={g.size} (max |ref| {float(np.abs(r).max()):.3g})")
        _record(name, mx, rel, g.size)
        assert mx <= atol, f"{name}: max abs error {mx:.4e} > {atol}"
        assert rel <= REL_L2, f"{name}: relative L2 error {rel:.4e} > {REL_L2}"


def oracle_sampled(q_s, k_s, v_s, do_s, idx_s, cu_padded, cu_actual, scale, G, docs=None, rows=None, keys=None):
    """The oracle's forward (and backward when do_s is given) on pre-selected inputs: q_s / do_s hold the query
    rows idx_s (local order) of the sampled documents with the q heads of the sampled kv heads (G per kv head,
    kv head j's at columns j*G .. j*G+G-1), k_s / v_s all T rows of those kv heads.  The work is split into one
    oracle call per (document, kv head) and the calls run on a thread pool with a small BLAS thread count each:
    numpy's element-wise passes are single-threaded, and the units are independent (every output entry is
    computed by exactly one call, with the oracle's own arithmetic).  Returns o, lse, dq over the q_s rows and
    heads, and dk, dv over all T rows of the sampled kv heads (NaN where nothing was computed)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from threadpoolctl import threadpool_limits

    n, nh = q_s.shape[0], k_s.shape[1]
    T, D = k_s.shape[0], k_s.shape[2]
    doc_of = oracle.token_map(cu_padded, cu_actual)[0][np.asarray(idx_s, dtype=np.int64)]
    units = [(d, j) for d in (docs if docs is not None else [None]) for j in range(nh)]
    o = np.full((n, nh * G, D), np.nan)
    lse = np.full((n, nh * G), np.nan)
    dq = np.full((n, nh * G, D), np.nan)
    dk = np.full((T, nh, D), np.nan)
    dv = np.full((T, nh, D), np.nan)
    cu_p = np.asarray(cu_padded, dtype=np.int64)

    def run(unit):
        d, j = unit
        ru = np.arange(n) if d is None else np.nonzero(doc_of == d)[0]
        rr = None if rows is None else np.nonzero(np.isin(ru, rows))[0]
        hs = slice(j * G, (j + 1) * G)
        qu, iu = q_s[ru][:, hs], np.asarray(idx_s)[ru]
        ku, vu = k_s[:, j:j + 1], v_s[:, j:j + 1]
        dd = None if d is None else [d]
        ou, lu, _ = oracle.attn_fwd(qu, ku, vu, iu, cu_padded, cu_actual, scale, docs=dd, rows=rr)
        out = [ou, lu]
        if do_s is not None:
            out += list(oracle.attn_bwd(qu, ku, vu, do_s[ru][:, hs], iu, cu_padded, cu_actual, scale, docs=dd,
                                        rows=rr, keys=keys))
        return unit, ru, out

    with threadpool_limits(limits=2):
        with ThreadPoolExecutor(max_workers=min(len(units), os.cpu_count() or 1, 16)) as ex:
            results = list(ex.map(run, units))
    for (d, j), ru, out in results:
        hs = slice(j * G, (j + 1) * G)
        o[ru, hs], lse[ru, hs] = out[0], out[1]
        if do_s is not None:
            dq[ru, hs] = out[2]
            slot = slice(None) if d is None else slice(int(cu_p[d]), int(cu_p[d + 1]))
            dk[slot, j] = out[3][slot, 0]
            dv[slot, j] = out[4][slot, 0]
    return o, lse, dq, dk, dv

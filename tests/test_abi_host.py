"""The C-ABI library loads, exports every declared symbol, and rejects bad arguments
on the host before launching anything (no GPU needed: no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

from context_causal_thd_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cpthd.h")
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]


def _declared():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(cpthd_\w+)\s*\(", text))
    return sorted(names)


def _defines():
    out = {}
    for name, val in re.findall(r"#define\s+(CPTHD_\w+)\s+\(?(-?\d+)\)?", open(HEADER).read()):
        out[name] = int(val)
    return out


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert set(names) == set(_lib.SIGNATURES), "binding signatures must cover the header exactly"
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    d = _defines()
    for name, code in d.items():
        if name.startswith("CPTHD_ERR_") or name == "CPTHD_OK":
            s = lib.cpthd_status_string(code).decode()
            assert s and s != "unknown status", name
    assert lib.cpthd_status_string(12345) == b"unknown status"


FAKE = 0x10000   # never dereferenced: every call below fails validation first


def test_partition_host_errors(lib):
    d = _defines()
    f = lib.cpthd_partition_indices
    assert f(None, 3, 28, 2, 0, 0, FAKE, None, None) == d["CPTHD_ERR_NULL"]
    assert f(FAKE, 3, 28, 2, 0, 0, None, None, None) == d["CPTHD_ERR_NULL"]
    assert f(FAKE, 3, 28, 0, 0, 0, FAKE, None, None) == d["CPTHD_ERR_RANK"]
    assert f(FAKE, 3, 28, 2, 2, 0, FAKE, None, None) == d["CPTHD_ERR_RANK"]
    assert f(FAKE, 3, 28, 2, -1, 0, FAKE, None, None) == d["CPTHD_ERR_RANK"]
    assert f(FAKE, 3, 28, 2, 0, 7, FAKE, None, None) == d["CPTHD_ERR_STRATEGY"]
    assert f(FAKE, 3, 27, 2, 0, 1, FAKE, None, None) == d["CPTHD_ERR_TOKENS"]
    assert f(FAKE, 3, 0, 2, 0, 1, FAKE, None, None) == d["CPTHD_ERR_TOKENS"]
    assert f(FAKE, 0, 28, 2, 0, 1, FAKE, None, None) == d["CPTHD_ERR_TOKENS"]
    assert f(FAKE, 3, 1 << 33, 2, 0, 1, FAKE, None, None) == d["CPTHD_ERR_TOKENS"]
    assert f(FAKE, 3, 30, 2, 0, 2, FAKE, None, None) == d["CPTHD_ERR_TOKENS"]      # packed: 30 % 4 != 0
    assert f(FAKE, 3, 28, 2, 0, 3, FAKE, None, None) == d["CPTHD_ERR_STRATEGY"]


def test_reorder_host_errors(lib):
    d = _defines()
    f = lib.cpthd_reorder_kv
    A, B, C, E = 0x100000, 0x200000, 0x300000, 0x400000
    assert f(None, B, C, E, 64, FAKE, 3, 28, 28, 2, 0, None, None) == d["CPTHD_ERR_NULL"]
    assert f(A, B, C, E, 64, FAKE, 3, 28, 28, 0, 0, None, None) == d["CPTHD_ERR_RANK"]
    assert f(A, B, C, E, 64, FAKE, 3, 28, 28, 2, 3, None, None) == d["CPTHD_ERR_STRATEGY"]
    assert f(A, B, C, E, 64, FAKE, 3, 28, 20, 2, 0, None, None) == d["CPTHD_ERR_TOKENS"]
    assert f(A, B, C, E, 60, FAKE, 3, 28, 28, 2, 0, None, None) == d["CPTHD_ERR_ALIGN"]
    assert f(A + 8, B, C, E, 64, FAKE, 3, 28, 28, 2, 0, None, None) == d["CPTHD_ERR_ALIGN"]
    assert f(A, B, A + 64, E, 64, FAKE, 3, 28, 28, 2, 0, None, None) == d["CPTHD_ERR_ALIAS"]   # DCS out overlaps in
    assert f(A, B, A, B, 64, FAKE, 3, 28, 28, 2, 0, None, None) == d["CPTHD_ERR_ALIAS"]
    assert f(A, B, A, B, 64, FAKE, 3, 28, 28, 2, 1, None, None) == 0    # contiguous in place: nothing to do


def test_workspace_bytes(lib):
    f = lib.cpthd_attn_workspace_bytes
    n = f(65536, 4, 32, 8, 128, 200)
    assert n > 16384 * 32 * 4            # holds at least delta [S, Hq] fp32
    assert f(65536, 4, 32, 8, 128, 400) > n
    assert f(65536, 4, 32, 7, 128, 200) == 0    # Hq % Hkv
    assert f(65536, 4, 32, 8, 96, 200) == 0     # head_dim
    assert f(65536, 4, 128, 1, 128, 200) == 0   # G > 64
    assert f(65535, 4, 32, 8, 128, 200) == 0    # capacity % cp
    assert f(65536, 0, 32, 8, 128, 200) == 0
    assert f(65536, 4, 32, 8, 128, 0) == 0


def test_workspace_min_bytes(lib):
    """The smallest accepted workspace (no partial slots) is below the default one wherever the default has slots,
    equal to it where the capacity is too small for any, and 0 for the same rejected arguments."""
    fmin, fdef = lib.cpthd_attn_workspace_min_bytes, lib.cpthd_attn_workspace_bytes
    for args in ((65536, 4, 32, 8, 128, 200), (8192, 2, 16, 16, 128, 40), (4096, 2, 8, 2, 64, 9)):
        assert 0 < fmin(*args) < fdef(*args)
    assert fmin(64, 2, 4, 2, 16, 4) == fdef(64, 2, 4, 2, 16, 4)   # under 128 tokens: no slots
    assert fmin(65536, 4, 32, 7, 128, 200) == 0
    assert fmin(65535, 4, 32, 8, 128, 200) == 0
    assert fmin(65536, 4, 32, 8, 128, 0) == 0


def test_attention_host_errors(lib):
    d = _defines()
    ws_bytes = lib.cpthd_attn_workspace_bytes(64, 2, 4, 2, 16, 4)
    plan, fwd, bwd = lib.cpthd_attn_plan, lib.cpthd_attn_fwd, lib.cpthd_attn_bwd
    P = 0x100000  # 256-aligned fake pointer
    ok = dict(T=64, cap=64, B=4, cp=2, r=0, s=0, hq=4, hkv=2, D=16)

    def call_plan(**kw):
        a = dict(ok, **kw)
        return plan(P, P, a["B"], a["T"], a["cap"], a["cp"], a["r"], a["s"], a["hq"], a["hkv"], a["D"],
                    kw.get("ws", P), kw.get("wsb", ws_bytes), None, None)

    assert plan(None, P, 4, 64, 64, 2, 0, 0, 4, 2, 16, P, ws_bytes, None, None) == d["CPTHD_ERR_NULL"]
    assert call_plan(r=2) == d["CPTHD_ERR_RANK"]
    assert call_plan(s=3) == d["CPTHD_ERR_STRATEGY"]
    assert call_plan(s=2, T=62, cap=64) == d["CPTHD_ERR_TOKENS"]   # packed: T % (2*cp) != 0
    assert call_plan(T=66) == d["CPTHD_ERR_TOKENS"]
    assert call_plan(T=128) == d["CPTHD_ERR_TOKENS"]        # above capacity
    assert call_plan(hkv=3) == d["CPTHD_ERR_HEADS"]
    assert call_plan(D=48) == d["CPTHD_ERR_HEADS"]
    assert call_plan(ws=None) == d["CPTHD_ERR_WORKSPACE"]
    assert call_plan(wsb=lib.cpthd_attn_workspace_min_bytes(64, 2, 4, 2, 16, 4) - 1) == d["CPTHD_ERR_WORKSPACE"]
    assert call_plan(ws=P + 16) == d["CPTHD_ERR_WORKSPACE"]

    def call_fwd(**kw):
        a = dict(ok, **kw)
        return fwd(P, P, P, kw.get("cua", P), P, a["B"], a["T"], a["cap"], a["cp"], a["r"], a["s"], a["hq"], a["hkv"],
                   a["D"], 0.25, kw.get("causal", 1), kw.get("wl", -1), kw.get("wr", 0), P, P, P, ws_bytes, None, None)

    assert call_fwd(causal=0) == d["CPTHD_ERR_MASK"]
    assert call_fwd(wl=128) == d["CPTHD_ERR_MASK"]
    assert call_fwd(wr=1) == d["CPTHD_ERR_MASK"]
    assert call_fwd(cp=0) == d["CPTHD_ERR_RANK"]
    assert call_fwd(B=0) == d["CPTHD_ERR_TOKENS"]
    assert call_fwd(cua=None) == d["CPTHD_ERR_NULL"]          # the cu arrays are required
    assert fwd(P, None, P, P, P, 4, 64, 64, 2, 0, 0, 4, 2, 16, 0.25, 1, -1, 0, P, P, P, ws_bytes, None, None) \
        == d["CPTHD_ERR_NULL"]

    def call_bwd(**kw):
        a = dict(ok, **kw)
        return bwd(P, P, P, P, P, P, P, kw.get("cup", P), a["B"], a["T"], a["cap"], a["cp"], a["r"], a["s"], a["hq"],
                   a["hkv"], a["D"], 0.25, 1, -1, kw.get("wr", 0), P, P, kw.get("dv", P), P, kw.get("wsb", ws_bytes),
                   None, None)

    assert call_bwd(dv=None) == d["CPTHD_ERR_NULL"]
    assert call_bwd(cup=None) == d["CPTHD_ERR_NULL"]
    assert call_bwd(wr=1) == d["CPTHD_ERR_MASK"]
    assert call_bwd(wsb=16) == d["CPTHD_ERR_WORKSPACE"]


def test_product_path_has_no_oracle_or_cpu_fallback():
    pkg = os.path.join(ROOT, "context_causal_thd_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", text, flags=re.M), f
                assert "numpy" not in text, f


def test_gather_host_errors(lib):
    d = _defines()
    f = lib.cpthd_gather_rows
    A, B, I = 0x100000, 0x200000, 0x300000
    assert f(A, 10, 8, I, 0, B, None, None) == 0                         # nothing to gather
    assert f(None, 10, 8, I, 4, B, None, None) == d["CPTHD_ERR_NULL"]
    assert f(A, 10, 8, None, 4, B, None, None) == d["CPTHD_ERR_NULL"]
    assert f(A, 10, 6, I, 4, B, None, None) == d["CPTHD_ERR_ALIGN"]
    assert f(A + 2, 10, 8, I, 4, B, None, None) == d["CPTHD_ERR_ALIGN"]
    assert f(A, 10, 8, I, 4, A + 16, None, None) == d["CPTHD_ERR_ALIAS"]
    assert f(A, 10, 8, I, -1, B, None, None) == d["CPTHD_ERR_TOKENS"]


def test_allgathered_attention_host_errors(lib):
    """The rank-major K/V entry points validate like the physical-order ones, plus the 2 GiB K/V bound."""
    d = _defines()
    P = 0x100000
    fwd, bwd = lib.cpthd_attn_fwd_allgathered, lib.cpthd_attn_bwd_allgathered
    ws_small = lib.cpthd_attn_workspace_bytes(64, 2, 4, 2, 16, 4)
    assert fwd(P, None, P, P, P, 4, 64, 64, 2, 0, 0, 4, 2, 16, 0.25, 1, -1, 0, P, P, P, ws_small, None, None) \
        == d["CPTHD_ERR_NULL"]
    assert fwd(P, P, P, P, P, 4, 64, 64, 2, 0, 0, 4, 2, 16, 0.25, 0, -1, 0, P, P, P, ws_small, None, None) \
        == d["CPTHD_ERR_MASK"]
    assert bwd(P, P, P, P, P, P, P, P, 4, 64, 64, 2, 0, 0, 4, 2, 16, 0.25, 1, -1, 0, P, P, P, P, 16, None, None) \
        == d["CPTHD_ERR_WORKSPACE"]
    # T * Hkv * D * 2 = 2^31 bytes: the gathered K/V would not fit one 32-bit buffer range
    T, cp, hq, hkv, D = 1 << 20, 4, 32, 8, 128
    wsb = lib.cpthd_attn_workspace_bytes(T, cp, hq, hkv, D, 16)
    assert wsb > 0
    for s in (0, 2):
        assert fwd(P, P, P, P, P, 16, T, T, cp, 0, s, hq, hkv, D, 0.1, 1, -1, 0, P, P, P, wsb, None, None) \
            == d["CPTHD_ERR_TOKENS"]
        assert bwd(P, P, P, P, P, P, P, P, 16, T, T, cp, 0, s, hq, hkv, D, 0.1, 1, -1, 0, P, P, P, P, wsb, None,
                   None) == d["CPTHD_ERR_TOKENS"]


def test_timed_variants_validate_like_the_product_calls(lib):
    """The instrumentation entry points run the same host checks (and take no events when none are given)."""
    d = _defines()
    P = 0x100000
    wsb = lib.cpthd_attn_workspace_bytes(64, 2, 4, 2, 16, 4)
    fwd, bwd = lib.cpthd_attn_fwd_timed, lib.cpthd_attn_bwd_timed
    for ag in (0, 1):
        assert fwd(P, P, P, None, P, 4, 64, 64, 2, 0, 0, 4, 2, 16, 0.25, 1, -1, 0, P, P, P, wsb, None, None, ag, None,
                   0) == d["CPTHD_ERR_NULL"]
        assert fwd(P, P, P, P, P, 4, 64, 64, 2, 5, 0, 4, 2, 16, 0.25, 1, -1, 0, P, P, P, wsb, None, None, ag, None,
                   0) == d["CPTHD_ERR_RANK"]
        assert bwd(P, P, P, P, P, P, P, P, 4, 64, 64, 2, 0, 0, 4, 2, 16, 0.25, 1, -1, 0, P, P, P, P, 8, None, None,
                   ag, None, 0) == d["CPTHD_ERR_WORKSPACE"]


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU's rank share: asked for more GPUs it exits with status 2 and says why, before
    touching the GPU."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "--gpus 1" in r.stderr


def test_noalloc_backward_host_checks(lib):
    """The allocation-free backward refuses NULL pointers and calls whose plan and rows exceed its static array,
    on the host, before it touches a device."""
    d = _defines()
    P = 0x100000
    f = lib.cpthd_attn_bwd_noalloc
    assert f(P, P, P, P, P, P, None, P, 4, 64, 64, 2, 0, 0, 4, 2, 16, 0.25, 1, -1, 0, P, P, P, None, None) \
        == d["CPTHD_ERR_NULL"]
    assert f(P, P, P, P, P, P, P, P, 4, 64, 64, 2, 0, 0, 4, 2, 16, 0.25, 0, -1, 0, P, P, P, None, None) \
        == d["CPTHD_ERR_MASK"]
    import context_causal_thd_amd as cpthd
    assert cpthd.STATIC_SCRATCH_BYTES == d["CPTHD_STATIC_SCRATCH_BYTES"]
    T = 1 << 20   # -delta and LSE rows alone: 2 * 2^20 * 64 * 4 bytes, beyond the array
    assert lib.cpthd_attn_workspace_bytes(T, 1, 64, 8, 128, 1) > d["CPTHD_STATIC_SCRATCH_BYTES"]
    assert f(P, P, P, P, P, P, P, P, 1, T, T, 1, 0, 1, 64, 8, 128, 0.1, 1, -1, 0, P, P, P, None, None) \
        == d["CPTHD_ERR_SCRATCH"]

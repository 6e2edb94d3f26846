"""The C ABI from plain C, with no Python or torch between the program and the library.

- tests/c_abi/consumer.c, compiled here with gcc against include/cpthd.h and include/cpthd_timing.h and linked to
  the in-tree libcpthd.so, runs host-side calls (workspace sizes, status strings, argument refusals): no GPU.
- tests/c_abi/consumer_gpu.c (built by build() into tests/c_abi/bin/) allocates its own device buffers and runs
  one rank's share, partition indices, forward and backward, through the C ABI; its outputs are compared here
  with the fp64 oracle: indices bit-exact, attention at the parity tests' bounds.
"""
import importlib.util
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "context_causal_thd_amd")
_spec = importlib.util.spec_from_file_location("c_abi_build", os.path.join(ROOT, "tests", "c_abi", "build.py"))
c_abi = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(c_abi)


def test_c_program_links_and_calls_the_library(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    if not os.path.exists(os.path.join(LIBDIR, "libcpthd.so")):
        pytest.skip("libcpthd.so not built")
    exe = str(tmp_path / "consumer")
    r = subprocess.run(c_abi.command("consumer", exe), stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout


def _write_inputs(path, wl, strategy, rank):
    import oracle
    import workloads as W
    S = wl.T // wl.cp
    idx = oracle.partition_indices(wl.cu_padded, wl.cp, rank, strategy)
    hdr = np.array([wl.T, wl.cp, rank, strategy, wl.num_docs, wl.Hq, wl.Hkv, wl.D], dtype=np.int32)
    with open(path, "wb") as f:
        f.write(hdr.tobytes())
        f.write(np.array([wl.softmax_scale], dtype=np.float32).tobytes())
        f.write(np.asarray(wl.cu_actual, dtype=np.int32).tobytes())
        f.write(np.asarray(wl.cu_padded, dtype=np.int32).tobytes())
        for x in (wl.q(idx), wl.k(), wl.v(), wl.do(idx)):
            f.write(W.to_bf16_bits(np.ascontiguousarray(x, dtype=np.float32)).tobytes())
    assert S * wl.cp == wl.T
    return idx


def _read_outputs(path, wl):
    S, T, Hq, Hkv, D = wl.T // wl.cp, wl.T, wl.Hq, wl.Hkv, wl.D
    raw = open(path, "rb").read()
    off = 0

    def take(dtype, n):
        nonlocal off
        a = np.frombuffer(raw, dtype=dtype, count=n, offset=off)
        off += a.nbytes
        return a

    idx = take(np.int32, S)
    o = (take(np.uint16, S * Hq * D).astype(np.uint32) << 16).view(np.float32).reshape(S, Hq, D)
    lse = take(np.float32, S * Hq).reshape(S, Hq)
    dq = take(np.float32, S * Hq * D).reshape(S, Hq, D)
    dk = take(np.float32, T * Hkv * D).reshape(T, Hkv, D)
    dv = take(np.float32, T * Hkv * D).reshape(T, Hkv, D)
    assert off == len(raw)
    return idx, o, lse, dq, dk, dv


def _cases():
    import workloads as W
    return [(W.tiny_t28(bf16=True), 0, 1), (W.tiny_t28(bf16=True), 1, 0),
            (W.small_random(760, 2, 1, max_docs=4, max_len=600, Hq=8, Hkv=2, D=128, bf16=True, qkv_scale=0.5,
                            do_scale=1.0), 1, 1)]


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(3))
def test_c_program_runs_a_share_on_the_gpu(tmp_path, case):
    import oracle
    from tests.gpu_util import assert_attn_close, log, oracle_sampled, set_case
    exe = os.path.join(c_abi.BIN, "consumer_gpu")
    assert os.path.exists(exe), f"{exe} is missing: build() (or python tests/c_abi/build.py) builds it"
    wl, s, r = _cases()[case]
    set_case(f"{wl.name} c-consumer s{s} r{r}")
    log(f"C consumer: {wl.name} T={wl.T} D={wl.D} heads {wl.Hq}/{wl.Hkv} cp={wl.cp} strategy={s} rank={r}")
    idx = _write_inputs(tmp_path / "in.bin", wl, s, r)
    res = subprocess.run([exe, str(tmp_path / "in.bin"), str(tmp_path / "out.bin")], stdout=subprocess.PIPE,
                         stderr=subprocess.STDOUT, text=True, timeout=120)
    assert res.returncode == 0 and res.stdout.strip().endswith("ok"), res.stdout
    g_idx, o, lse, dq, dk, dv = _read_outputs(tmp_path / "out.bin", wl)
    assert np.array_equal(g_idx, idx)
    G = wl.Hq // wl.Hkv
    o_r, lse_r, dq_r, dk_r, dv_r = oracle_sampled(wl.q(idx), wl.k(), wl.v(), wl.do(idx), idx, wl.cu_padded,
                                                  wl.cu_actual, wl.softmax_scale, G)
    _, _, valid = oracle.token_map(wl.cu_padded, wl.cu_actual)
    vq = valid[idx]
    assert_attn_close("O", o.astype(np.float64), o_r, vq[:, None, None])
    assert_attn_close("LSE", lse.astype(np.float64), lse_r, vq[:, None])
    assert_attn_close("dQ", dq.astype(np.float64), dq_r, vq[:, None, None])
    assert_attn_close("dK", dk.astype(np.float64), dk_r, valid[:, None, None])
    assert_attn_close("dV", dv.astype(np.float64), dv_r, valid[:, None, None])

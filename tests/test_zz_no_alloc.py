"""The allocation-free backward (cpthd_attn_bwd_noalloc) against cpthd_attn_bwd, through the C ABI: two calls in a
row on one GPU, the second with a smaller input, each bit-identical to the workspace entry point's results."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import bf16_dev, i32_dev, log, status_dev

pytestmark = pytest.mark.gpu

cpthd = pytest.importorskip("context_causal_thd_amd")


def _inputs(wl, s, r):
    idx = oracle.partition_indices(wl.cu_padded, wl.cp, r, s)
    q, k, v, do = (bf16_dev(x) for x in (wl.q(idx), wl.k(), wl.v(), wl.do(idx)))
    return q, k, v, do


def _bwd_both(wl, s, r):
    q, k, v, do = _inputs(wl, s, r)
    T, S = wl.T, wl.T // wl.cp
    cu_a, cu_p = i32_dev(wl.cu_actual), i32_dev(wl.cu_padded)
    # a workspace of the static array's size: the same partial slots, so the same plan (and split tiles)
    plan = cpthd.AttnPlan(T, wl.cp, wl.Hq, wl.Hkv, wl.D, max_docs=wl.num_docs,
                          workspace_bytes=cpthd.STATIC_SCRATCH_BYTES)
    st = status_dev()
    plan.build(cu_a, cu_p, T, r, s, st)
    o, lse = cpthd.attn_fwd(q, k, v, plan, wl.softmax_scale, dev_status=st)
    ref = cpthd.attn_bwd(q, k, v, o, do, lse, plan, wl.softmax_scale, dev_status=st)
    got = [torch.full_like(x, float("nan")) for x in ref]
    st2 = status_dev()
    cpthd.cpthd_attn_bwd_noalloc(q, k, v, o, do, lse, cu_a, cu_p, wl.num_docs, T, T, wl.cp, r, s, wl.Hq, wl.Hkv,
                                 wl.D, wl.softmax_scale, 1, -1, 0, got[0], got[1], got[2], st2)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and int(st2.item()) == 0
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), name


def test_noalloc_backward_matches_workspace_entry_point_twice():
    big = W.small_random(61, 2, 0, max_docs=5, max_len=600, Hq=8, Hkv=2, D=128, bf16=True, qkv_scale=0.5,
                         do_scale=1.0)
    small = W.small_random(62, 2, 1, max_docs=3, max_len=120, Hq=4, Hkv=2, D=64, bf16=True, qkv_scale=0.5,
                           do_scale=1.0)
    assert small.T < big.T
    for wl, s in ((big, 0), (small, 1)):
        for r in range(wl.cp):
            log(f"noalloc {wl.name} T={wl.T} s={s} r={r}")
            _bwd_both(wl, s, r)


def test_noalloc_refuses_a_call_the_array_cannot_hold():
    """Sizes beyond the static array are refused on the host with CPTHD_ERR_SCRATCH, before any launch."""
    T, cp, hq, hkv, D = 1 << 20, 1, 64, 8, 128     # -delta and LSE rows alone: 2 * 2^20 * 64 * 4 bytes
    P = 0x100000
    rc = cpthd._lib.load().cpthd_attn_bwd_noalloc(P, P, P, P, P, P, P, P, 1, T, T, cp, 0, 1, hq, hkv, D, 0.1, 1, -1,
                                                   0, P, P, P, None, None)
    assert rc == -11

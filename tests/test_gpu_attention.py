"""GPU parity: attention forward (O, LSE) and backward (dQ, dK, dV) against the fp64 oracle.

Inputs are the seeded bf16 values (the oracle runs on exactly those values,
upcast to float64).  Small layouts are compared in full; the full-size
configurations are compared on sampled documents and kv heads, which the
oracle computes exactly, plus properties that hold everywhere (finite values,
exact zeros on pads and untouched rows, nothing written past the active rows).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import assert_attn_close, bf16_dev, i32_dev, log, status_dev, to_np64

pytestmark = pytest.mark.gpu

cpthd = pytest.importorskip("context_causal_thd_amd")


class Share:
    """One rank's share on the GPU: plan, forward and (optionally) backward."""

    def __init__(self, wl, strategy, rank, capacity=None, backward=True, poison=False, allgathered=False,
                 kv=None):
        self.wl, self.s, self.r = wl, strategy, rank
        T, cp = wl.T, wl.cp
        S = T // cp
        cap = capacity or T
        capS = cap // cp
        self.idx = oracle.partition_indices(wl.cu_padded, cp, rank, strategy)
        q = wl.q(self.idx)
        k, v = kv if kv is not None else (wl.k(), wl.v())   # kv: the workload's K, V, generated once by the caller
        self.q_np, self.k_np, self.v_np = q, k, v
        # rank-major all-gathered K/V (the simulated all-gather of every rank's local rows)
        self.allgathered = allgathered
        self.parts = [oracle.partition_indices(wl.cu_padded, cp, rr, strategy) for rr in range(cp)]
        if allgathered:
            k, v = oracle.all_gather(k, self.parts), oracle.all_gather(v, self.parts)
        fill = float("nan") if poison else 0.0

        def buf(shape_tail, src, dtype=torch.bfloat16, rows=cap):
            t = torch.full((rows,) + shape_tail, fill, dtype=dtype, device="cuda")
            if src is not None:
                t[:src.shape[0]] = bf16_dev(src) if dtype == torch.bfloat16 else src
            return t

        self.q = buf((wl.Hq, wl.D), q, rows=capS)
        self.k = buf((wl.Hkv, wl.D), k)
        self.v = buf((wl.Hkv, wl.D), v)
        self.cu_a, self.cu_p = i32_dev(wl.cu_actual), i32_dev(wl.cu_padded)
        self.plan = cpthd.AttnPlan(cap, cp, wl.Hq, wl.Hkv, wl.D, max_docs=max(wl.num_docs, 1))
        self.st = status_dev()
        self.plan.build(self.cu_a, self.cu_p, T, rank, strategy, self.st)
        canary = 7.0
        self.o = torch.full((capS, wl.Hq, wl.D), canary, dtype=torch.bfloat16, device="cuda")
        self.lse = torch.full((capS, wl.Hq), canary, dtype=torch.float32, device="cuda")
        cpthd.attn_fwd(self.q, self.k, self.v, self.plan, wl.softmax_scale, self.o, self.lse, self.st,
                       kv_allgathered=allgathered)
        self.S, self.capS, self.cap = S, capS, cap
        if backward:
            do = wl.do(self.idx)
            self.do_np = do
            self.do = buf((wl.Hq, wl.D), do, rows=capS)
            self.dq = torch.full((capS, wl.Hq, wl.D), canary, dtype=torch.float32, device="cuda")
            self.dk = torch.full((cap, wl.Hkv, wl.D), canary, dtype=torch.float32, device="cuda")
            self.dv = torch.full((cap, wl.Hkv, wl.D), canary, dtype=torch.float32, device="cuda")
            cpthd.attn_bwd(self.q, self.k, self.v, self.o, self.do, self.lse, self.plan, wl.softmax_scale,
                           self.dq, self.dk, self.dv, self.st, kv_allgathered=allgathered)
        torch.cuda.synchronize()
        assert int(self.st.item()) == 0, cpthd.api.describe_dev_status(int(self.st.item()))

    def check_tails(self):
        """Rows past the active prefix keep their canaries."""
        S, T = self.S, self.wl.T
        assert (self.o[S:].float() == 7.0).all() and (self.lse[S:] == 7.0).all()
        if hasattr(self, "dq"):
            assert (self.dq[S:] == 7.0).all() and (self.dk[T:] == 7.0).all() and (self.dv[T:] == 7.0).all()

    def compare(self, docs=None, kv_heads=None, backward=True):
        wl = self.wl
        S, T = self.S, wl.T
        o_ref, lse_ref, _ = oracle.attn_fwd(self.q_np, self.k_np, self.v_np, self.idx, wl.cu_padded, wl.cu_actual,
                                            wl.softmax_scale, docs=docs, kv_heads=kv_heads)
        o = to_np64(self.o[:S])
        lse = to_np64(self.lse[:S])
        assert np.isfinite(o).all(), "O must be finite everywhere"
        _, _, valid_tok = oracle.token_map(wl.cu_padded, wl.cu_actual)
        vq = valid_tok[self.idx]
        assert np.isneginf(lse[~vq]).all() and (o[~vq] == 0).all(), "pad rows: O = 0, LSE = -inf"
        assert np.isfinite(lse[vq]).all()
        assert_attn_close("O", o, o_ref, vq[:, None, None])
        assert_attn_close("LSE", lse, lse_ref, vq[:, None])
        if not backward:
            return
        dq_ref, dk_ref, dv_ref = oracle.attn_bwd(self.q_np, self.k_np, self.v_np, self.do_np, self.idx,
                                                 wl.cu_padded, wl.cu_actual, wl.softmax_scale, docs=docs,
                                                 kv_heads=kv_heads)
        dq = to_np64(self.dq[:S])
        dk = to_np64(self.dk[:T])
        dv = to_np64(self.dv[:T])
        if self.allgathered:   # back to physical order
            dk, dv = oracle.restore(dk, self.parts), oracle.restore(dv, self.parts)
        for name, x in (("dQ", dq), ("dK", dk), ("dV", dv)):
            assert np.isfinite(x).all(), f"{name} must be finite everywhere"
        assert (dq[~vq] == 0).all() and (dk[~valid_tok] == 0).all() and (dv[~valid_tok] == 0).all()
        assert_attn_close("dQ", dq, dq_ref, vq[:, None, None])
        assert_attn_close("dK", dk, dk_ref, valid_tok[:, None, None])
        assert_attn_close("dV", dv, dv_ref, valid_tok[:, None, None])


def _small_cases():
    cases = []
    seed = 0
    for D in (16, 32, 64, 128):
        for Hq, Hkv in ((2, 2), (4, 1), (8, 2), (6, 2), (16, 2)):
            for cp, s in ((1, 0), (2, 0), (3, 1), (4, 1), (2, 1), (4, 0), (2, 2), (3, 2)):
                seed += 1
                if (seed % 3) and D != 128:
                    continue
                # value scales of the measured workloads: Q/K/V ~ 0.5 N(0,1), dO ~ N(0,1)
                wl = W.small_random(seed, cp, s, max_docs=5, max_len=360, Hq=Hq, Hkv=Hkv, D=D, bf16=True,
                                    qkv_scale=0.5, do_scale=1.0)
                cases.append(wl)
    return cases


SMALL = _small_cases()


def test_tiny_t28_all_shares():
    wl = W.tiny_t28(bf16=True)
    for s in wl.strategies:
        for r in wl.ranks:
            log(f"tiny_t28 s={s} r={r}")
            sh = Share(wl, s, r)
            sh.compare()


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: f"{w.name}-D{w.D}-h{w.Hq}x{w.Hkv}-cp{w.cp}-s{w.strategies[0]}")
def test_small_full_parity(wl):
    s = wl.strategies[0]
    for r in range(wl.cp):
        log(f"{wl.name} T={wl.T} docs={wl.num_docs} s={s} r={r}")
        sh = Share(wl, s, r)
        sh.compare()


def test_t8192_mha16_forward_both_strategies():
    wl = W.t8192_mha16()
    for s in wl.strategies:
        for r in wl.ranks:
            log(f"t8192_mha16 s={s} r={r}")
            sh = Share(wl, s, r, backward=False)
            sh.compare(backward=False)


def _sample_docs(wl, idx, n=3):
    """Largest document the rank touches, smallest, and the one holding the rank's first row."""
    doc, _, _ = oracle.token_map(wl.cu_padded, wl.cu_actual)
    touched = np.unique(doc[idx])
    L = np.diff(wl.cu_padded.astype(np.int64))[touched]
    pick = {int(touched[np.argmax(L)]), int(touched[np.argmin(L)]), int(doc[idx[0]])}
    return sorted(pick)[:n]


@pytest.mark.parametrize("s", [0, 1, 2])
@pytest.mark.parametrize("r", [0, 3])
def test_t32768_gqa32x8_sampled(s, r):
    wl = W.t32768_gqa32x8()
    log(f"t32768_gqa32x8 s={s} r={r}")
    sh = Share(wl, s, r)
    docs = _sample_docs(wl, sh.idx)
    log(f"  docs {docs}")
    sh.compare(docs=docs, kv_heads=[0, 7])


@pytest.mark.parametrize("s", [1, 2])
@pytest.mark.parametrize("r", [0, 7])
def test_t131072_gqa64x8_sampled(s, r):
    wl = W.t131072_gqa64x8()
    log(f"t131072_gqa64x8 s={s} r={r}")
    sh = Share(wl, s, r)
    doc, _, _ = oracle.token_map(wl.cu_padded, wl.cu_actual)
    touched = np.unique(doc[sh.idx])
    L = np.diff(wl.cu_padded.astype(np.int64))[touched]
    docs = sorted({int(touched[np.argmin(L)]), int(doc[sh.idx[0]])})
    log(f"  docs {docs}")
    sh.compare(docs=docs, kv_heads=[5])


def test_dynamic_t_capacity_microbatches():
    """Fixed-capacity buffers, NaN-poisoned beyond the active T, canaries on output tails."""
    for m in (0, 5, 11):
        wl = W.dynamic_t(m)
        for s in wl.strategies + (2,):
            for r in (0, 3):
                log(f"dynamic_t mb={m} T={wl.T} s={s} r={r}")
                sh = Share(wl, s, r, capacity=W.DYNAMIC_T_CAPACITY, poison=True)
                sh.check_tails()
                docs = _sample_docs(wl, sh.idx, n=2)
                sh.compare(docs=docs, kv_heads=[3])


# ---------------------------------------------------------------------------
# K/V read straight from the rank-major all-gathered buffer (no restoration pass)
# ---------------------------------------------------------------------------
def test_tiny_t28_allgathered_all_shares():
    wl = W.tiny_t28(bf16=True)
    for s in wl.strategies + (2,):
        for r in wl.ranks:
            log(f"tiny_t28 allgathered s={s} r={r}")
            Share(wl, s, r, allgathered=True).compare()


SMALL_AG = [w for w in SMALL if w.strategies[0] != 1][::2] + [w for w in SMALL if w.strategies[0] == 1][:2]


@pytest.mark.parametrize("wl", SMALL_AG, ids=lambda w: f"{w.name}-D{w.D}-h{w.Hq}x{w.Hkv}-cp{w.cp}-s{w.strategies[0]}")
def test_small_allgathered_parity(wl):
    s = wl.strategies[0]
    for r in range(wl.cp):
        log(f"{wl.name} allgathered T={wl.T} s={s} r={r}")
        Share(wl, s, r, allgathered=True).compare()


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("case", ["t32768_gqa32x8-s0-r0", "t32768_gqa32x8-s0-r3", "t32768_gqa32x8-s2-r1", "dynamic_t.mb5-s0-r2"])
def test_allgathered_bitwise_equals_physical(case):
    """Same arithmetic, other addresses: O, LSE, dQ bit-identical; dK/dV are the physical ones permuted
    into rank-major order."""
    name, s, r = case.split("-")
    s, r = int(s[1:]), int(r[1:])
    if name == "t32768_gqa32x8":
        wl, kw = W.t32768_gqa32x8(), {}
    else:
        wl, kw = W.dynamic_t(int(name.split("mb")[1])), dict(capacity=W.DYNAMIC_T_CAPACITY, poison=True)
    log(f"{case} physical")
    a = Share(wl, s, r, **kw)
    log(f"{case} allgathered")
    b = Share(wl, s, r, allgathered=True, **kw)
    b.check_tails()
    S, T = wl.T // wl.cp, wl.T
    for x, y in ((a.o, b.o), (a.lse, b.lse), (a.dq, b.dq)):
        assert torch.equal(_bits(x[:S]), _bits(y[:S]))
    order = torch.from_numpy(oracle.all_gather(np.arange(T), a.parts)).to("cuda")
    assert torch.equal(_bits(a.dk[:T][order]), _bits(b.dk[:T]))
    assert torch.equal(_bits(a.dv[:T][order]), _bits(b.dv[:T]))


def _degenerate_cases():
    """Hand-made layouts: empty documents (first, in the middle, last), documents with no actual token, a
    document with one actual token, DualChunkSwap documents of exactly 2*cp tokens (one token per chunk)."""
    out = []
    for cp in (1, 2, 3):
        u = 2 * cp
        docs = [(0, 0), (u, 1), (0, 0), (2 * u, 0), (u, u), (3 * u + 2 * u * 40, 3 * u + 2 * u * 40 - 1), (0, 0)]
        padded = [p for p, _ in docs]
        actual = [a for _, a in docs]
        for s in (0, 1, 2):
            wl = W.Workload(f"degenerate-cp{cp}-s{s}", [77, cp, s], sum(padded), 8, 2, 64, W._cu(padded),
                            W._cu(actual), cp, (s,), tuple(range(cp)), True, qkv_scale=0.5, do_scale=1.0, bf16=True)
            oracle.check_layout(wl.cu_padded, wl.cu_actual, cp, s)
            out.append(wl)
    return out


DEGENERATE = _degenerate_cases()


@pytest.mark.parametrize("wl", DEGENERATE, ids=lambda w: w.name)
@pytest.mark.parametrize("allgathered", [False, True])
def test_degenerate_layouts(wl, allgathered):
    s = wl.strategies[0]
    for r in range(wl.cp):
        log(f"{wl.name} allgathered={allgathered} r={r}")
        Share(wl, s, r, allgathered=allgathered).compare()


def test_plan_mismatch_sets_status_and_writes_nothing():
    wl = W.tiny_t28(bf16=True)
    sh = Share(wl, 0, 0)
    st = status_dev()
    o = torch.full_like(sh.o, 3.0)
    lse = torch.full_like(sh.lse, 3.0)
    # rank 1 against a plan built for rank 0
    cpthd.cpthd_attn_fwd(sh.q, sh.k, sh.v, wl.T, wl.T, wl.num_docs, wl.cp, 1, 0, wl.Hq, wl.Hkv, wl.D,
                         wl.softmax_scale, 1, -1, 0, o, lse, sh.plan.workspace, st)
    torch.cuda.synchronize()
    assert int(st.item()) & 16
    assert (o.float() == 3.0).all() and (lse == 3.0).all()


def test_plan_rejects_bad_layouts():
    wl = W.tiny_t28(bf16=True)
    plan = cpthd.AttnPlan(64, 2, 2, 2, 16, max_docs=4)
    st = status_dev()
    cu_bad = i32_dev([0, 6, 20, 28])                          # 6 % 4 != 0 under DCS
    plan.build(i32_dev(wl.cu_actual), cu_bad, 28, 0, 0, st)
    torch.cuda.synchronize()
    assert int(st.item()) & 4
    st = status_dev()
    plan.build(i32_dev([0, 9, 17, 24]), i32_dev(wl.cu_padded), 28, 0, 0, st)   # actual 9 > padded 8
    torch.cuda.synchronize()
    assert int(st.item()) & 8


def test_plan_rejects_documents_of_2gib_kv():
    """A document whose K/V rows reach 2 GiB (2^20 tokens x 8 kv heads x 128 x 2 bytes) is refused with a
    device status bit; one just below the limit plans cleanly."""
    T = 1 << 20
    plan = cpthd.AttnPlan(T, 1, 8, 8, 128, max_docs=2)
    for lengths, bit in (([T], 64), ([T - 64, 64], 0)):
        cu = i32_dev(np.concatenate([[0], np.cumsum(lengths)]))
        st = status_dev()
        plan.build(cu, cu, T, 0, 1, st)
        torch.cuda.synchronize()
        assert int(st.item()) == bit, lengths


@pytest.mark.parametrize("allgathered", [False, True])
def test_autograd_wrapper_matches_entry_points(allgathered):
    """cpthd.attention (autograd) gives the entry points' O bit for bit, and gradients equal to the fp32
    dQ/dK/dV cast to the inputs' dtype; a plan rebuilt in any way before backward is refused."""
    wl = W.small_random(5, 2, 0, max_docs=4, max_len=300, Hq=8, Hkv=2, D=64, bf16=True, qkv_scale=0.5,
                        do_scale=1.0)
    S, T = wl.T // wl.cp, wl.T
    sh = Share(wl, 0, 1, allgathered=allgathered)
    q = sh.q[:S].clone().requires_grad_()
    k = sh.k[:T].clone().requires_grad_()
    v = sh.v[:T].clone().requires_grad_()
    o = cpthd.attention(q, k, v, sh.plan, wl.softmax_scale, kv_allgathered=allgathered)
    assert torch.equal(o.detach(), sh.o[:S])
    o.backward(sh.do[:S])
    torch.cuda.synchronize()
    assert torch.equal(q.grad, sh.dq[:S].to(torch.bfloat16))
    assert torch.equal(k.grad, sh.dk[:T].to(torch.bfloat16))
    assert torch.equal(v.grad, sh.dv[:T].to(torch.bfloat16))
    o2 = cpthd.attention(q, k, v, sh.plan, wl.softmax_scale, kv_allgathered=allgathered)
    sh.plan.build(sh.cu_a, sh.cu_p, T, 0, 0, sh.st)          # another rank's layout
    with pytest.raises(RuntimeError, match="rebuilt"):
        o2.backward(sh.do[:S])
    # a rebuild with the same sizes, rank and strategy (as for the next micro-batch of equal length) is
    # refused as well: other document boundaries would give other tiles
    sh.plan.build(sh.cu_a, sh.cu_p, T, 1, 0, sh.st)
    o3 = cpthd.attention(q, k, v, sh.plan, wl.softmax_scale, kv_allgathered=allgathered)
    sh.plan.build(sh.cu_a, sh.cu_p, T, 1, 0, sh.st)
    with pytest.raises(RuntimeError, match="rebuilt"):
        o3.backward(sh.do[:S])


# dK/dV sum G heads of P * dO, so their magnitude (and the absolute rounding of the bf16 P operand) grows
# like sqrt(G); dO is scaled by sqrt(4 / G) to keep dK/dV in the range of the measured workloads (G = 4),
# where the absolute bound applies.  Unscaled, G = 64 stays at relative L2 ~1e-3.
WIDE_GQA = [W.small_random(900 + i, cp, s, max_docs=4, max_len=200, Hq=hq, Hkv=hkv, D=d, bf16=True, qkv_scale=0.5,
                           do_scale=(4.0 / (hq // hkv)) ** 0.5)
            for i, (cp, s, hq, hkv, d) in enumerate([(2, 0, 64, 1, 64), (3, 1, 64, 1, 128), (2, 2, 32, 1, 32),
                                                    (4, 0, 64, 2, 16), (1, 0, 32, 1, 128)])]


@pytest.mark.parametrize("wl", WIDE_GQA, ids=lambda w: f"{w.name}-D{w.D}-h{w.Hq}x{w.Hkv}-cp{w.cp}-s{w.strategies[0]}")
@pytest.mark.parametrize("allgathered", [False, True])
def test_wide_gqa_groups(wl, allgathered):
    """32 and 64 q heads per kv head: 8 or 4 tokens per query tile, one or two tokens per key-tile chunk."""
    s = wl.strategies[0]
    for r in range(wl.cp):
        log(f"{wl.name} G={wl.Hq // wl.Hkv} allgathered={allgathered} r={r}")
        Share(wl, s, r, allgathered=allgathered).compare()


@pytest.mark.parametrize("name", ["t32768_gqa32x8", "t131072_gqa64x8"])
def test_strategies_agree_on_every_row(name):
    """Full-size property, every row: the strategies compute the same function of the same tokens, so all
    ranks' O, LSE, dQ scattered to physical rows, and dK, dV summed over ranks, agree between strategies (to
    rounding: the tiles, and so the accumulation order, differ).  Config 4's documents rule out DualChunkSwap."""
    wl = W.t32768_gqa32x8() if name == "t32768_gqa32x8" else W.t131072_gqa64x8()
    strategies = (0, 1, 2) if name == "t32768_gqa32x8" else (1, 2)
    T, cp = wl.T, wl.cp
    kv = (wl.k(), wl.v())
    res = {}
    for s in strategies:
        o = torch.zeros((T, wl.Hq, wl.D), dtype=torch.float32, device="cuda")
        lse = torch.zeros((T, wl.Hq), dtype=torch.float32, device="cuda")
        dq = torch.zeros((T, wl.Hq, wl.D), dtype=torch.float32, device="cuda")
        dk = torch.zeros((T, wl.Hkv, wl.D), dtype=torch.float32, device="cuda")
        dv = torch.zeros((T, wl.Hkv, wl.D), dtype=torch.float32, device="cuda")
        for r in range(cp):
            log(f"{name} s={s} r={r}")
            sh = Share(wl, s, r, kv=kv)
            idx = torch.from_numpy(sh.idx.astype(np.int64)).to("cuda")
            S = T // cp
            o[idx] = sh.o[:S].float()
            lse[idx] = sh.lse[:S]
            dq[idx] = sh.dq[:S]
            dk += sh.dk[:T]
            dv += sh.dv[:T]
            del sh
        res[s] = (o, lse, dq, dk, dv)
    _, _, valid_tok = oracle.token_map(wl.cu_padded, wl.cu_actual)
    vt = torch.from_numpy(valid_tok).to("cuda")
    s0 = strategies[0]
    for s in strategies[1:]:
        for t, a, b, tol in zip(("O", "LSE", "dQ", "dK", "dV"), res[s0], res[s], (2e-2, 1e-4, 2e-2, 2e-2, 2e-2)):
            same_pads = torch.equal(a[~vt], b[~vt])
            err = float((a[vt] - b[vt]).abs().max())
            rel = float((a[vt] - b[vt]).norm() / a[vt].norm())
            log(f"    strategy {s0} vs {s} {t}: max_abs={err:.3e} rel_l2={rel:.3e}")
            assert same_pads, f"{t}: pad rows differ between strategies"
            assert err <= tol and rel <= 5e-3, (t, s, err, rel)


def test_graph_replays_match_eager():
    """The plan, forward and backward launches captured in a HIP graph (torch.cuda.CUDAGraph) replay to the
    eager results bit for bit, several times, with eager work between the replays."""
    wl = W.small_random(77, 2, 0, max_docs=5, max_len=400, Hq=8, Hkv=2, D=128, bf16=True, qkv_scale=0.5,
                        do_scale=1.0)
    sh = Share(wl, 0, 1)                          # eager run: plan, forward, backward
    S, T = wl.T // wl.cp, wl.T
    outs = dict(o=torch.empty_like(sh.o), lse=torch.empty_like(sh.lse), dq=torch.empty_like(sh.dq),
                dk=torch.empty_like(sh.dk), dv=torch.empty_like(sh.dv))
    plan = cpthd.AttnPlan(T, wl.cp, wl.Hq, wl.Hkv, wl.D, max_docs=wl.num_docs)
    st = status_dev()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                 # warm-up launch outside the capture
        plan.build(sh.cu_a, sh.cu_p, T, 1, 0, st)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.build(sh.cu_a, sh.cu_p, T, 1, 0, st)
        cpthd.attn_fwd(sh.q, sh.k, sh.v, plan, wl.softmax_scale, outs["o"], outs["lse"], st)
        cpthd.attn_bwd(sh.q, sh.k, sh.v, outs["o"], sh.do, outs["lse"], plan, wl.softmax_scale, outs["dq"],
                       outs["dk"], outs["dv"], st)
    for rep in range(3):
        for t in outs.values():
            t.fill_(float("nan"))                 # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        assert torch.equal(outs["o"][:S], sh.o[:S]) and torch.equal(outs["lse"][:S], sh.lse[:S]), rep
        assert torch.equal(outs["dq"][:S], sh.dq[:S]), rep
        assert torch.equal(outs["dk"][:T], sh.dk[:T]) and torch.equal(outs["dv"][:T], sh.dv[:T]), rep

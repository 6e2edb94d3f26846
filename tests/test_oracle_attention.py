"""Pins of the oracle's attention forward/backward.

The method computes exactly the rank's rows of per-document causal softmax
attention (TransformerEngine PR #3221, "Scope and constraints": causal with
window (-1, 0), THD layout, documents isolated by the sequence metadata).  The
oracle is checked here against things other than itself: scalar brute-force
loops, closed forms at each document's first token, torch's SDPA and autograd in
float64 on the CPU (library special cases), and central finite differences.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _brute_fwd(q_local, k, v, idx, cu_p, cu_a, scale):
    """Scalar loops over (row, head, key) with a textbook softmax."""
    S, Hq, D = q_local.shape
    G = Hq // k.shape[1]
    o = np.zeros((S, Hq, D))
    lse = np.full((S, Hq), -np.inf)
    for i, p in enumerate(idx):
        d = max(j for j in range(len(cu_p) - 1) if cu_p[j] <= p)
        while cu_p[d + 1] <= p:
            d += 1
        pos = p - cu_p[d]
        if pos >= cu_a[d + 1] - cu_a[d]:
            continue
        keys = [cu_p[d] + j for j in range(pos + 1)]
        for h in range(Hq):
            g = h // G
            sc = [scale * sum(float(q_local[i, h, x]) * float(k[kk, g, x]) for x in range(D)) for kk in keys]
            mx = max(sc)
            z = sum(math.exp(s - mx) for s in sc)
            lse[i, h] = mx + math.log(z)
            for kk, s in zip(keys, sc):
                w = math.exp(s - lse[i, h])
                for x in range(D):
                    o[i, h, x] += w * float(v[kk, g, x])
    return o, lse


def _inputs(wl, rank, strategy):
    idx = oracle.partition_indices(wl.cu_padded, wl.cp, rank, strategy)
    return idx, wl.q(idx), wl.k(), wl.v(), wl.do(idx)


SMALL = [W.small_random(s, cp, st, max_docs=4, max_len=16, Hq=2, Hkv=1, D=4)
         for s, cp, st in [(1, 2, 0), (2, 2, 1), (3, 3, 0), (4, 3, 1), (5, 1, 0), (6, 4, 1), (7, 2, 0),
                           (8, 2, 2), (9, 3, 2)]]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: f"{w.name}-cp{w.cp}")
def test_fwd_matches_brute_force(wl):
    s = wl.strategies[0]
    for r in range(wl.cp):
        idx, q, k, v, _ = _inputs(wl, r, s)
        o, lse, comp = oracle.attn_fwd(q, k, v, idx, wl.cu_padded, wl.cu_actual, wl.softmax_scale)
        bo, blse = _brute_fwd(q, k, v, idx, wl.cu_padded.tolist(), wl.cu_actual.tolist(), wl.softmax_scale)
        assert comp.all()
        np.testing.assert_allclose(o, bo, rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(np.isinf(lse), np.isinf(blse))
        fin = np.isfinite(blse)
        np.testing.assert_allclose(lse[fin], blse[fin], rtol=1e-12, atol=1e-12)


def test_tiny_t28_fwd_brute_force_both_strategies():
    wl = W.tiny_t28()
    for s in wl.strategies:
        for r in wl.ranks:
            idx, q, k, v, _ = _inputs(wl, r, s)
            o, lse, _ = oracle.attn_fwd(q, k, v, idx, wl.cu_padded, wl.cu_actual, wl.softmax_scale)
            bo, blse = _brute_fwd(q, k, v, idx, wl.cu_padded.tolist(), wl.cu_actual.tolist(), wl.softmax_scale)
            np.testing.assert_allclose(o, bo, rtol=1e-12, atol=1e-12)
            fin = np.isfinite(blse)
            np.testing.assert_allclose(lse[fin], blse[fin], rtol=1e-12, atol=1e-12)


def test_first_token_closed_form_and_pads():
    # At a document's first actual token the softmax has one key: O = V[start], LSE = scale*q.k;
    # pads give O = 0 and LSE = -inf exactly.
    wl = W.tiny_t28()
    for s in wl.strategies:
        for r in wl.ranks:
            idx, q, k, v, _ = _inputs(wl, r, s)
            o, lse, _ = oracle.attn_fwd(q, k, v, idx, wl.cu_padded, wl.cu_actual, wl.softmax_scale)
            _, pos, valid = oracle.token_map(wl.cu_padded, wl.cu_actual)
            for i, p in enumerate(idx):
                if not valid[p]:
                    assert np.all(o[i] == 0) and np.all(lse[i] == -np.inf)
                elif pos[p] == 0:
                    for h in range(wl.Hq):
                        g = h // (wl.Hq // wl.Hkv)
                        np.testing.assert_allclose(o[i, h], v[p, g], rtol=0, atol=1e-14)
                        np.testing.assert_allclose(lse[i, h], wl.softmax_scale * float(np.dot(q[i, h].astype(np.float64), k[p, g])), rtol=1e-13)


def _sdpa_doc(q, k, v, scale):
    """torch SDPA (causal, float64, CPU) on one unpadded document, GQA by head repetition."""
    G = q.shape[1] // k.shape[1]
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)
    kt = torch.from_numpy(k.astype(np.float64)).repeat_interleave(G, dim=1).permute(1, 0, 2).contiguous()
    vt = torch.from_numpy(v.astype(np.float64)).repeat_interleave(G, dim=1).permute(1, 0, 2).contiguous()
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    return out.permute(1, 0, 2).numpy()


def test_fwd_single_unpadded_document_matches_sdpa():
    rng = np.random.default_rng(11)
    T, Hq, Hkv, D = 96, 4, 2, 8
    q = rng.standard_normal((T, Hq, D))
    k = rng.standard_normal((T, Hkv, D))
    v = rng.standard_normal((T, Hkv, D))
    cu = np.array([0, T], dtype=np.int32)
    scale = 0.3
    ref = _sdpa_doc(q, k, v, scale)
    for cp, s in [(1, 0), (4, 0), (3, 1), (2, 1)]:
        for r in range(cp):
            idx = oracle.partition_indices(cu, cp, r, s)
            o, _, _ = oracle.attn_fwd(q[idx], k, v, idx, cu, cu, scale)
            np.testing.assert_allclose(o, ref[idx], rtol=1e-11, atol=1e-11)


def _packed_autograd(q, k, v, do, cu_p, cu_a, scale):
    """Dense packed attention through torch SDPA with a boolean block-causal mask, float64 autograd."""
    doc, pos, valid = oracle.token_map(cu_p, cu_a)
    T, Hq, D = q.shape
    G = Hq // k.shape[1]
    allowed = (doc[:, None] == doc[None, :]) & (pos[None, :] <= pos[:, None]) & valid[:, None] & valid[None, :]
    rows = valid & allowed.any(axis=1)
    mask = torch.from_numpy(allowed[rows][:, :])
    qt = torch.tensor(q[rows], dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    vt = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    out = torch.nn.functional.scaled_dot_product_attention(
        qt.permute(1, 0, 2), kt.repeat_interleave(G, dim=1).permute(1, 0, 2),
        vt.repeat_interleave(G, dim=1).permute(1, 0, 2), attn_mask=mask, scale=scale)
    out = out.permute(1, 0, 2)
    (out * torch.from_numpy(do[rows])).sum().backward()
    o = np.zeros((T, Hq, D)); o[rows] = out.detach().numpy()
    dq = np.zeros((T, Hq, D)); dq[rows] = qt.grad.numpy()
    return o, dq, kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("wl", [W.tiny_t28()] + SMALL[:4] + SMALL[-2:], ids=lambda w: w.name)
def test_union_of_ranks_equals_unpartitioned_and_autograd(wl):
    T = wl.T
    q, k, v, do = wl.q(), wl.k(), wl.v(), wl.do()
    ref_o, ref_dq, ref_dk, ref_dv = _packed_autograd(q, k, v, do, wl.cu_padded, wl.cu_actual, wl.softmax_scale)
    for s in wl.strategies:
        o_all = np.full((T, wl.Hq, wl.D), np.nan)
        dq_all = np.full((T, wl.Hq, wl.D), np.nan)
        dk_sum = np.zeros((T, wl.Hkv, wl.D))
        dv_sum = np.zeros((T, wl.Hkv, wl.D))
        for r in range(wl.cp):
            idx = oracle.partition_indices(wl.cu_padded, wl.cp, r, s)
            o, _, _ = oracle.attn_fwd(q[idx], k, v, idx, wl.cu_padded, wl.cu_actual, wl.softmax_scale)
            dq, dk, dv = oracle.attn_bwd(q[idx], k, v, do[idx], idx, wl.cu_padded, wl.cu_actual, wl.softmax_scale)
            o_all[idx] = o
            dq_all[idx] = dq
            dk_sum += dk
            dv_sum += dv
        np.testing.assert_allclose(o_all, ref_o, rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(dq_all, ref_dq, rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(dk_sum, ref_dk, rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(dv_sum, ref_dv, rtol=1e-10, atol=1e-10)


def test_bwd_central_finite_differences_tiny_t28():
    wl = W.tiny_t28()
    q, k, v, do = wl.q(), wl.k(), wl.v(), wl.do()
    rng = np.random.default_rng(5)
    h = 1e-6
    for s in wl.strategies:
        for r in wl.ranks:
            idx = oracle.partition_indices(wl.cu_padded, 2, r, s)
            ql = q[idx].astype(np.float64)
            kk, vv, dl = k.astype(np.float64), v.astype(np.float64), do[idx].astype(np.float64)
            dq, dk, dv = oracle.attn_bwd(ql, kk, vv, dl, idx, wl.cu_padded, wl.cu_actual, wl.softmax_scale)

            def loss(qx, kx, vx):
                o, _, _ = oracle.attn_fwd(qx, kx, vx, idx, wl.cu_padded, wl.cu_actual, wl.softmax_scale)
                return float(np.sum(o * dl))

            for arr, grad, which in ((ql, dq, 0), (kk, dk, 1), (vv, dv, 2)):
                for flat in rng.choice(arr.size, size=40, replace=False):
                    pert = [ql.copy(), kk.copy(), vv.copy()]
                    pert[which].flat[flat] += h
                    up = loss(*pert)
                    pert[which].flat[flat] -= 2 * h
                    dn = loss(*pert)
                    assert abs((up - dn) / (2 * h) - grad.flat[flat]) < 1e-6


def test_bwd_pads_and_first_token_exact():
    wl = W.tiny_t28()
    q, k, v, do = wl.q(), wl.k(), wl.v(), wl.do()
    _, pos, valid = oracle.token_map(wl.cu_padded, wl.cu_actual)
    for s in wl.strategies:
        for r in wl.ranks:
            idx = oracle.partition_indices(wl.cu_padded, 2, r, s)
            dq, dk, dv = oracle.attn_bwd(q[idx], k, v, do[idx], idx, wl.cu_padded, wl.cu_actual, wl.softmax_scale)
            for i, p in enumerate(idx):
                if not valid[p]:
                    assert np.all(dq[i] == 0)            # pad row: exactly zero
                elif pos[p] == 0:
                    assert np.all(np.abs(dq[i]) < 1e-14)  # a softmax over one key has zero score gradient
            assert np.all(dk[~valid] == 0) and np.all(dv[~valid] == 0)


def test_docs_subset_matches_full():
    wl = W.small_random(3, 2, 0, max_docs=5, max_len=24, Hq=2, Hkv=1, D=4)
    idx, q, k, v, do = _inputs(wl, 1, 0)
    o, lse, _ = oracle.attn_fwd(q, k, v, idx, wl.cu_padded, wl.cu_actual, wl.softmax_scale)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, idx, wl.cu_padded, wl.cu_actual, wl.softmax_scale)
    for d in range(wl.num_docs):
        so, slse, comp = oracle.attn_fwd(q, k, v, idx, wl.cu_padded, wl.cu_actual, wl.softmax_scale, docs=[d])
        np.testing.assert_array_equal(so[comp], o[comp])
        np.testing.assert_array_equal(slse[comp], lse[comp])
        sdq, sdk, sdv = oracle.attn_bwd(q, k, v, do, idx, wl.cu_padded, wl.cu_actual, wl.softmax_scale, docs=[d])
        lo, hi = wl.cu_padded[d], wl.cu_padded[d + 1]
        np.testing.assert_array_equal(sdq[comp], dq[comp])
        np.testing.assert_array_equal(sdk[lo:hi], dk[lo:hi])
        np.testing.assert_array_equal(sdv[lo:hi], dv[lo:hi])


def test_kv_head_subset_matches_full():
    wl = W.small_random(9, 2, 1, max_docs=4, max_len=24, Hq=4, Hkv=2, D=4)
    idx, q, k, v, do = _inputs(wl, 0, 1)
    o, lse, _ = oracle.attn_fwd(q, k, v, idx, wl.cu_padded, wl.cu_actual, wl.softmax_scale)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, idx, wl.cu_padded, wl.cu_actual, wl.softmax_scale)
    for g in range(2):
        so, slse, _ = oracle.attn_fwd(q, k, v, idx, wl.cu_padded, wl.cu_actual, wl.softmax_scale, kv_heads=[g])
        sdq, sdk, sdv = oracle.attn_bwd(q, k, v, do, idx, wl.cu_padded, wl.cu_actual, wl.softmax_scale, kv_heads=[g])
        hs = slice(2 * g, 2 * g + 2)
        np.testing.assert_array_equal(so[:, hs], o[:, hs])
        np.testing.assert_array_equal(slse[:, hs], lse[:, hs])
        np.testing.assert_array_equal(sdq[:, hs], dq[:, hs])
        np.testing.assert_array_equal(sdk[:, g], dk[:, g])
        np.testing.assert_array_equal(sdv[:, g], dv[:, g])
        assert np.isnan(so[:, 2 * (1 - g)]).all() and np.isnan(sdk[:, 1 - g]).all()


def test_row_and_key_sampling_matches_full():
    """Restricting the oracle to sampled query rows (O, LSE, dQ) and sampled keys (dK, dV) gives exactly the full
    computation's values on those entries and NaN elsewhere."""
    for seed, cp, strat in ((31, 2, 0), (32, 3, 1), (33, 2, 2)):
        wl = W.small_random(seed, cp, strat, max_docs=5, max_len=120, Hq=4, Hkv=2, D=16)
        for r in range(cp):
            idx = oracle.partition_indices(wl.cu_padded, cp, r, strat)
            q, k, v, do = wl.q(idx), wl.k(), wl.v(), wl.do(idx)
            rng = np.random.default_rng(seed + r)
            rows = np.unique(rng.integers(0, max(idx.size, 1), size=max(idx.size // 3, 1)))
            keys = np.unique(rng.integers(0, wl.T, size=max(wl.T // 3, 1)))
            o, lse, _ = oracle.attn_fwd(q, k, v, idx, wl.cu_padded, wl.cu_actual, wl.softmax_scale)
            dq, dk, dv = oracle.attn_bwd(q, k, v, do, idx, wl.cu_padded, wl.cu_actual, wl.softmax_scale)
            o_s, lse_s, comp = oracle.attn_fwd(q, k, v, idx, wl.cu_padded, wl.cu_actual, wl.softmax_scale, rows=rows)
            dq_s, dk_s, dv_s = oracle.attn_bwd(q, k, v, do, idx, wl.cu_padded, wl.cu_actual, wl.softmax_scale,
                                               rows=rows, keys=keys)
            rmask = np.zeros(idx.size, dtype=bool)
            rmask[rows[rows < idx.size]] = True
            kmask = np.zeros(wl.T, dtype=bool)
            kmask[keys] = True
            assert np.array_equal(comp, rmask)
            for full, samp, m in ((o, o_s, rmask), (lse, lse_s, rmask), (dq, dq_s, rmask), (dk, dk_s, kmask),
                                  (dv, dv_s, kmask)):
                assert np.isnan(samp[~m]).all()
                np.testing.assert_allclose(samp[m], full[m], rtol=1e-12, atol=1e-12)

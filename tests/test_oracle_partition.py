"""Pins of the oracle's partition / all-gather / restoration against the pages' definitions.

The partition rule (TransformerEngine PR #3221, "Why" and "What changed"):
DualChunkSwap cuts every document into 2*cp_size chunks and gives each rank two of
them (two attention steps per rank); NO_LOAD_BALANCE gives each rank one contiguous
physical chunk of T/cp_size tokens (one step).  The checks here are invariants,
closed forms and hand-derived values, not a second copy of the rule.
"""
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_t28.txt")
STRAT = {"dcs": oracle.DUAL_CHUNK_SWAP, "contiguous": oracle.NO_LOAD_BALANCE}
PACKED = oracle.PACKED_SUPER_SEQUENCE


def _golden():
    out = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        key, vals = line.split(":")
        out[key.strip()] = [int(x) for x in vals.split()]
    return out


def test_tiny_t28_golden_indices_and_pairs():
    g = _golden()
    wl = W.tiny_t28()
    for name, s in STRAT.items():
        for r in (0, 1):
            idx = oracle.partition_indices(wl.cu_padded, 2, r, s)
            assert idx.tolist() == g[f"indices {name} {r}"]
            assert oracle.useful_pairs(idx, wl.cu_padded, wl.cu_actual) == g[f"pairs {name} {r}"][0]


def test_tiny_t28_golden_gather_restore_maps():
    g = _golden()
    wl = W.tiny_t28()
    parts = [oracle.partition_indices(wl.cu_padded, 2, r, oracle.DUAL_CHUNK_SWAP) for r in (0, 1)]
    phys = np.arange(wl.T)
    assert oracle.all_gather(phys, parts).tolist() == g["gathered_source dcs"]
    rows = np.arange(wl.T)
    # restore() applied to "gathered row numbers" tells which gathered row lands at each token
    assert oracle.restore(rows, parts).tolist() == g["restore_source dcs"]


def _random_layouts():
    cases = []
    for seed in range(40):
        for cp in (1, 2, 3, 4):
            for s in (oracle.DUAL_CHUNK_SWAP, oracle.NO_LOAD_BALANCE, PACKED):
                cases.append(W.small_random(seed, cp, s, max_docs=6, max_len=40))
    return cases


@pytest.mark.parametrize("wl", _random_layouts()[::3], ids=lambda w: f"{w.name}-cp{w.cp}-s{w.strategies[0]}")
def test_partition_invariants(wl):
    cp, s = wl.cp, wl.strategies[0]
    T = wl.T
    parts = [oracle.partition_indices(wl.cu_padded, cp, r, s) for r in range(cp)]
    # every rank holds T/cp tokens and the union is a permutation of the padded buffer
    for p in parts:
        assert p.size * cp == T
        assert np.all(np.diff(p) > 0), "local order follows physical order"
    assert np.array_equal(np.sort(np.concatenate(parts)), np.arange(T))
    doc, pos, _ = oracle.token_map(wl.cu_padded, wl.cu_actual)
    if s == oracle.NO_LOAD_BALANCE:
        S = T // cp
        for r, p in enumerate(parts):
            assert np.array_equal(p, r * S + np.arange(S))       # closed form: one contiguous chunk
    elif s == PACKED:
        c = T // (2 * cp)
        for r, p in enumerate(parts):
            # exactly the tokens of whole-buffer chunks r and 2cp-1-r, whatever the documents
            want = [x for x in range(T) if c and x // c in (r, 2 * cp - 1 - r)]
            assert p.tolist() == want
    else:
        L = np.diff(wl.cu_padded.astype(np.int64))
        for r, p in enumerate(parts):
            for d in range(wl.num_docs):
                c = L[d] // (2 * cp)
                mine = p[doc[p] == d]
                assert mine.size == 2 * c
                if c == 0:
                    continue
                chunk_ids = pos[mine] // c
                # exactly two whole chunks, the mirrored pair r and 2cp-1-r
                assert sorted(set(chunk_ids.tolist())) == sorted({r, 2 * cp - 1 - r})
                for ch in {r, 2 * cp - 1 - r}:
                    assert np.sum(chunk_ids == ch) == (c if r != 2 * cp - 1 - r else 2 * c)


@pytest.mark.parametrize("cp", [1, 2, 3, 4, 8])
def test_dcs_balances_causal_work_on_unpadded_documents(cp):
    # Closed form: a document of length 2*cp*c gives every rank c*(2*cp*c + 1) causal pairs,
    # which is why the mirrored pairing is the load-balanced default.
    rng = np.random.default_rng(cp)
    lens = [2 * cp * int(c) for c in rng.integers(1, 9, size=5)]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    expect = sum((L // (2 * cp)) * (L + 1) for L in lens)
    for r in range(cp):
        idx = oracle.partition_indices(cu, cp, r, oracle.DUAL_CHUNK_SWAP)
        assert oracle.useful_pairs(idx, cu, cu) == expect


def test_single_document_is_head_tail_split():
    # With one sequence, rank r holds a head piece [r*c, (r+1)*c) and the mirrored tail
    # piece [(2cp-1-r)*c, (2cp-r)*c) -- the head/tail balancing used for plain sequences.
    cp, c = 4, 5
    cu = np.array([0, 2 * cp * c], dtype=np.int32)
    for r in range(cp):
        idx = oracle.partition_indices(cu, cp, r, oracle.DUAL_CHUNK_SWAP)
        head, tail = idx[:c], idx[c:]
        assert head[0] == r * c and head[-1] == (r + 1) * c - 1
        assert tail[-1] == 2 * cp * c - 1 - r * c


@pytest.mark.parametrize("s", [oracle.DUAL_CHUNK_SWAP, oracle.NO_LOAD_BALANCE])
def test_cp1_is_identity(s):
    wl = W.small_random(7, 1, s)
    assert np.array_equal(oracle.partition_indices(wl.cu_padded, 1, 0, s), np.arange(wl.T))


@pytest.mark.parametrize("wl", _random_layouts()[1::5], ids=lambda w: f"{w.name}-cp{w.cp}-s{w.strategies[0]}")
def test_restore_inverts_all_gather(wl):
    cp, s = wl.cp, wl.strategies[0]
    x = np.random.default_rng(1).standard_normal((wl.T, 3, 4)).astype(np.float32)
    parts = [oracle.partition_indices(wl.cu_padded, cp, r, s) for r in range(cp)]
    ag = oracle.all_gather(x, parts)
    assert np.array_equal(oracle.restore(ag, parts), x)
    if s == oracle.NO_LOAD_BALANCE:
        assert np.array_equal(ag, x), "rank-major contiguous ownership needs no reorder"


def test_check_layout_rejections():
    cu = np.array([0, 6, 16], dtype=np.int32)
    with pytest.raises(ValueError):
        oracle.check_layout(cu, cu, 2, oracle.DUAL_CHUNK_SWAP)   # 6 % 4 != 0
    oracle.check_layout(cu, cu, 2, oracle.NO_LOAD_BALANCE)        # any document length is fine
    with pytest.raises(ValueError):
        oracle.check_layout(cu, cu, 3, oracle.NO_LOAD_BALANCE)    # 16 % 3 != 0
    with pytest.raises(ValueError):
        oracle.check_layout(cu, np.array([0, 7, 8], dtype=np.int32), 2, oracle.NO_LOAD_BALANCE)
    with pytest.raises(ValueError):
        oracle.check_layout(np.array([0, 8, 4], dtype=np.int32), None, 2, oracle.NO_LOAD_BALANCE)
    with pytest.raises(ValueError):
        oracle.partition_indices(cu, 2, 2, oracle.NO_LOAD_BALANCE)


def test_workload_layouts_are_valid():
    for wl in (W.tiny_t28(), W.t8192_mha16(), W.t32768_gqa32x8(), W.t131072_gqa64x8()):
        for s in wl.strategies:
            oracle.check_layout(wl.cu_padded, wl.cu_actual, wl.cp, s)
        assert int(wl.cu_padded[-1]) == wl.T
    for m in range(W.DYNAMIC_T_MICROBATCHES):
        wl = W.dynamic_t(m)
        assert 4096 <= wl.T <= W.DYNAMIC_T_CAPACITY and wl.T % 64 == 0
        for s in wl.strategies:
            oracle.check_layout(wl.cu_padded, wl.cu_actual, wl.cp, s)
    cu_p, cu_a = W.t1m_10k_docs()
    assert cu_p[-1] == 1 << 20 and cu_p.size == 10001
    oracle.check_layout(cu_p, cu_a, 4, oracle.DUAL_CHUNK_SWAP)


@pytest.mark.parametrize("cp", [1, 2, 3, 4])
def test_packed_super_sequence_on_one_document_is_dual_chunk_swap(cp):
    # with a single document filling the buffer the two mirrored policies coincide
    T = 2 * cp * 7
    cu = np.array([0, T], dtype=np.int32)
    for r in range(cp):
        assert np.array_equal(oracle.partition_indices(cu, cp, r, PACKED),
                              oracle.partition_indices(cu, cp, r, oracle.DUAL_CHUNK_SWAP))


def test_packed_super_sequence_accepts_indivisible_documents():
    cu = np.array([0, 5, 11, 16], dtype=np.int32)          # no length divisible by 2*cp = 4, T = 16 is
    oracle.check_layout(cu, cu, 2, PACKED)
    with pytest.raises(ValueError):
        oracle.check_layout(cu, cu, 2, oracle.DUAL_CHUNK_SWAP)
    with pytest.raises(ValueError):
        oracle.check_layout(np.array([0, 5, 14], dtype=np.int32), None, 2, PACKED)   # 14 % 4 != 0
    idx0 = oracle.partition_indices(cu, 2, 0, PACKED)
    assert idx0.tolist() == [0, 1, 2, 3, 12, 13, 14, 15]


@pytest.mark.parametrize("wl", _random_layouts()[2::7], ids=lambda w: f"{w.name}-cp{w.cp}-s{w.strategies[0]}")
def test_batch_on_rank_keeps_global_positions(wl):
    # Slicing (ids, labels, positions) per rank: concatenating the ranks' slices and putting
    # every row back at its physical index recovers the batch, and each rank's position ids
    # are the within-document positions of its physical tokens (positions stay global).
    cp, s = wl.cp, wl.strategies[0]
    rng = np.random.default_rng(3)
    ids = rng.integers(0, 50000, size=wl.T)
    labels = rng.integers(0, 50000, size=wl.T)
    _, pos, _ = oracle.token_map(wl.cu_padded, wl.cu_actual)
    slices = [oracle.batch_on_rank(wl.cu_padded, cp, r, s, ids, labels, pos) for r in range(cp)]
    parts = [oracle.partition_indices(wl.cu_padded, cp, r, s) for r in range(cp)]
    for j, full in enumerate((ids, labels, pos)):
        assert np.array_equal(oracle.restore(np.concatenate([sl[j] for sl in slices]), parts), full)
    for r in range(cp):
        cu = wl.cu_padded.astype(np.int64)
        doc = np.searchsorted(cu, parts[r], side="right") - 1
        assert np.array_equal(slices[r][2], parts[r] - cu[doc])


@pytest.mark.parametrize("strategy", [oracle.NO_LOAD_BALANCE, oracle.PACKED_SUPER_SEQUENCE])
def test_t131072_gqa64x8_pairs_sum_to_every_documents_causal_pairs(strategy):
    # CP is exact: the ranks' useful pairs add up to every document's causal pairs over its actual tokens,
    # sum of a(a+1)/2.  The per-rank split is what the config's "least and most work" ranks are checked on.
    wl = W.t131072_gqa64x8()
    a = np.diff(wl.cu_actual.astype(np.int64))
    per_rank = [oracle.useful_pairs(oracle.partition_indices(wl.cu_padded, wl.cp, r, strategy), wl.cu_padded,
                                    wl.cu_actual) for r in range(wl.cp)]
    assert sum(per_rank) == int(np.sum(a * (a + 1) // 2))
    if strategy == oracle.NO_LOAD_BALANCE:
        # with packed documents rank 7 holds the least causal work and rank 4 the most (not ranks 0 and 7)
        assert int(np.argmin(per_rank)) == 7 and int(np.argmax(per_rank)) == 4

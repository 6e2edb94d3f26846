"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that the pins catch each.

Every mutant is a one-token edit of the oracle source: a wrong chunk index, an
off-by-one mask, a dropped scale, a wrong sign, a transposed operand.  Each one
must make at least one pin in test_oracle_partition / test_oracle_attention fail.
"""
import importlib.util
import os
import types

import pytest

import oracle
import oracle.cpthd_oracle as base
import tests.test_oracle_attention as TA
import tests.test_oracle_partition as TP

SRC = open(base.__file__).read()

MUTANTS = [
    ("chunk_pair", "for chunk in (rank, 2 * cp_size - 1 - rank)", "for chunk in (rank, cp_size - 1 - rank)"),
    ("chunk_order", "for chunk in (rank, 2 * cp_size - 1 - rank)", "for chunk in (2 * cp_size - 1 - rank, rank)"),
    ("contig_offset", "np.arange(rank * S, (rank + 1) * S", "np.arange(rank * S + 1, (rank + 1) * S + 1"),
    ("restore_reversed", "out[p] = gathered[off:off + p.size]", "out[p] = gathered[off:off + p.size][::-1]"),
    ("mask_future", "allowed = kpos[None, :] <= qpos[b0:b0 + _ROW_BLOCK, None]",
     "allowed = kpos[None, :] <= qpos[b0:b0 + _ROW_BLOCK, None] + 1"),
    ("mask_strict", "allowed = kpos[None, :] <= qpos[b0:b0 + _ROW_BLOCK, None]",
     "allowed = kpos[None, :] < qpos[b0:b0 + _ROW_BLOCK, None]"),
    ("pad_rows_attend", "rows = np.nonzero((ldoc == d) & lval)[0]", "rows = np.nonzero(ldoc == d)[0]"),
    ("gqa_map", "kd = k[start:start + a, h // G]", "kd = k[start:start + a, h % k.shape[1]]"),
    ("no_scale_fwd", "s = scale * (q_local[r, h] @ kd.T)", "s = (q_local[r, h] @ kd.T)"),
    ("lse_no_max", "lse[r, h] = m + np.log(den)", "lse[r, h] = np.log(den)"),
    ("dk_no_scale", "dk[start + kk, g] += scale * (ds_k.T @ q_local[r, h])", "dk[start + kk, g] += (ds_k.T @ q_local[r, h])"),
    ("dq_wrong_operand", "dq[r[rq], h] = scale * (ds_r @ kd)", "dq[r[rq], h] = scale * (ds_r @ vd)"),
    ("ds_sign", "ds = p * (dout @ vd.T - delta[:, None])", "ds = p * (delta[:, None] - dout @ vd.T)"),
    ("ds_sign_sampled_rows", "ds_r = p[rq] * (dout[rq] @ vd.T - delta[rq, None])",
     "ds_r = p[rq] * (delta[rq, None] - dout[rq] @ vd.T)"),
    ("ds_sign_sampled_keys", "ds_k, p_k = p[:, kk] * (dout @ vd[kk].T - delta[:, None]), p[:, kk]",
     "ds_k, p_k = p[:, kk] * (delta[:, None] - dout @ vd[kk].T), p[:, kk]"),
    ("dv_wrong_operand", "dv[start + kk, g] += p_k.T @ dout", "dv[start + kk, g] += ds_k.T @ dout"),
    ("key_subset_drops_a_key", "kk = np.nonzero(ksel[start:start + a])[0]", "kk = np.nonzero(ksel[start:start + a])[0][1:]"),
    ("row_subset_drops_rows", "rq = rsel[r]", "rq = rsel[r] & (qpos[b0:b0 + _ROW_BLOCK] != 1)"),
    ("fwd_row_subset_drops_rows", "keep = rsel[drows]", "keep = rsel[drows] & (qpos != 1)"),
    ("bwd_needed_rows_too_few", "need = rsel[drows] | (qpos >= (kk[0] if kk.size else a))",
     "need = rsel[drows] | (qpos > (kk[0] if kk.size else a))"),
    ("delta_dropped", "delta = np.sum(dout * o, axis=1)", "delta = np.sum(dout * o, axis=1) * 0"),
    ("packed_per_half", "return partition_indices([0, cu_p[-1]], cp_size, rank, DUAL_CHUNK_SWAP)",
     "return partition_indices([0, cu_p[-1] // 2, cu_p[-1]], cp_size, rank, DUAL_CHUNK_SWAP)"),
]


def _load_mutant(src):
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, base.__file__, "exec"), mod.__dict__)
    return mod


PINS = [
    TP.test_tiny_t28_golden_indices_and_pairs,
    TP.test_tiny_t28_golden_gather_restore_maps,
    lambda: [TP.test_partition_invariants(w) for w in TP._random_layouts()[::7]],
    lambda: [TP.test_packed_super_sequence_on_one_document_is_dual_chunk_swap(cp) for cp in (2, 3)],
    lambda: [TP.test_restore_inverts_all_gather(w) for w in TP._random_layouts()[1::9]],
    lambda: [TP.test_dcs_balances_causal_work_on_unpadded_documents(cp) for cp in (2, 3)],
    lambda: [TA.test_fwd_matches_brute_force(w) for w in TA.SMALL[:3]],
    TA.test_tiny_t28_fwd_brute_force_both_strategies,
    TA.test_first_token_closed_form_and_pads,
    TA.test_fwd_single_unpadded_document_matches_sdpa,
    lambda: [TA.test_union_of_ranks_equals_unpartitioned_and_autograd(w) for w in [TA.W.tiny_t28()]],
    TA.test_bwd_pads_and_first_token_exact,
    TA.test_row_and_key_sampling_matches_full,
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, monkeypatch):
    assert old in SRC, f"mutation site for {name} not found in the oracle source"
    mut = _load_mutant(SRC.replace(old, new, 1))
    for attr in ("partition_indices", "all_gather", "restore", "useful_pairs", "attn_fwd", "attn_bwd",
                 "token_map", "check_layout"):
        monkeypatch.setattr(oracle, attr, getattr(mut, attr))
    caught = False
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught = True
            break
    assert caught, f"no pin failed for mutant {name}"

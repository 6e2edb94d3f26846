"""The binding refuses wrong dtypes and shapes before anything reaches the library (no GPU needed: meta
tensors carry shape and dtype only)."""
import types

import pytest
import torch

from context_causal_thd_amd import api


def _plan(T=64, cp=2, Hq=4, Hkv=2, D=16):
    lay = api.Layout(_t((2,), torch.int32), _t((2,), torch.int32), T, 0, 0)
    return types.SimpleNamespace(layout=lay, cp_size=cp, Hq=Hq, Hkv=Hkv, D=D, workspace=None, status=None,
                                 _args=lambda lay=None: ())


def test_layout_refuses_bad_cu_arrays():
    with pytest.raises(ValueError, match="cu_seqlens_padded: expected torch.int32"):
        api.Layout(_t((3,), torch.int32), _t((3,), torch.int64), 64, 0, 0)
    with pytest.raises(ValueError, match="same length"):
        api.Layout(_t((4,), torch.int32), _t((3,), torch.int32), 64, 0, 0)


def _t(shape, dtype=torch.bfloat16):
    return torch.empty(shape, dtype=dtype, device="meta")


def test_attn_fwd_refuses_bad_inputs():
    plan = _plan()
    good = dict(q_local=_t((32, 4, 16)), k=_t((64, 2, 16)), v=_t((64, 2, 16)))
    for key, bad, msg in (("q_local", _t((32, 4, 16), torch.float32), "q_local: expected torch.bfloat16"),
                          ("q_local", _t((31, 4, 16)), "q_local: expected shape"),
                          ("k", _t((63, 2, 16)), "k: expected shape"),
                          ("v", _t((64, 4, 16)), "v: expected shape"),
                          ("k", _t((64, 32)), "k: expected shape")):
        args = dict(good, **{key: bad})
        with pytest.raises(ValueError, match=msg):
            api.attn_fwd(args["q_local"], args["k"], args["v"], plan)
    with pytest.raises(ValueError, match="lse_local"):
        api.attn_fwd(good["q_local"], good["k"], good["v"], plan, lse_local=_t((32, 4), torch.float16))


def test_attn_bwd_refuses_bad_inputs():
    plan = _plan()
    q, o, do = _t((32, 4, 16)), _t((32, 4, 16)), _t((32, 4, 16))
    k, v, lse = _t((64, 2, 16)), _t((64, 2, 16)), _t((32, 4), torch.float32)
    with pytest.raises(ValueError, match="do_local"):
        api.attn_bwd(q, k, v, o, _t((32, 4, 8)), lse, plan)
    with pytest.raises(ValueError, match="dk: expected torch.float32"):
        api.attn_bwd(q, k, v, o, do, lse, plan, dk=_t((64, 2, 16)))
    with pytest.raises(ValueError, match="dv: expected shape"):
        api.attn_bwd(q, k, v, o, do, lse, plan, dv=_t((60, 2, 16), torch.float32))


def test_reorder_and_partition_refuse_bad_inputs():
    cu = _t((3,), torch.int32)
    with pytest.raises(ValueError, match="v_gathered: expected shape"):
        api.reorder_kv(_t((64, 2, 16)), _t((32, 2, 16)), cu, 64, 2, 0)
    with pytest.raises(ValueError, match="k_out"):
        api.reorder_kv(_t((64, 2, 16)), _t((64, 2, 16)), cu, 64, 2, 0, k_out=_t((64, 2, 16), torch.float32))
    with pytest.raises(ValueError, match="cu_seqlens_padded: expected torch.int32"):
        api.partition_indices(_t((3,), torch.int64), 64, 2, 0, 0)
    with pytest.raises(ValueError, match="out: expected shape"):
        api.partition_indices(cu, 64, 2, 0, 0, out=_t((16,), torch.int32))
    with pytest.raises(ValueError, match="index: expected torch.int32"):
        api.gather_rows(_t((10, 4), torch.int64), _t((5,), torch.int64))

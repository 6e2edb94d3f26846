"""GPU parity: partition indices and K/V restoration are bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import i32_dev, log, status_dev

pytestmark = pytest.mark.gpu

cpthd = pytest.importorskip("context_causal_thd_amd")


def _layouts():
    out = [("tiny_t28", W.tiny_t28()), ("t8192_mha16", W.t8192_mha16()), ("t32768_gqa32x8", W.t32768_gqa32x8()), ("t131072_gqa64x8", W.t131072_gqa64x8())]
    out += [(f"dynamic_t.mb{m}", W.dynamic_t(m)) for m in range(W.DYNAMIC_T_MICROBATCHES)]
    for seed in range(12):
        for cp in (1, 2, 3, 4, 8, 16):
            for s in (0, 1, 2):
                out.append((f"small{seed}.cp{cp}.s{s}", W.small_random(seed, cp, s, max_docs=7, max_len=200)))
    return out


LAYOUTS = _layouts()


def _gpu_indices(cu_p, T, cp, r, s):
    cu = i32_dev(cu_p)
    out = torch.full((T // cp + 8,), -7, dtype=torch.int32, device="cuda")   # canary tail
    st = status_dev()
    cpthd.cpthd_partition_indices(cu, cu.numel() - 1, T, cp, r, s, out, st)
    res = out.cpu().numpy()
    assert (res[T // cp:] == -7).all(), "wrote past T/cp"
    assert int(st.item()) == 0
    return res[:T // cp]


@pytest.mark.parametrize("name,wl", LAYOUTS, ids=[n for n, _ in LAYOUTS])
def test_partition_bit_exact(name, wl):
    log(f"partition {name}")
    for s in (0, 1, 2):
        try:
            oracle.check_layout(wl.cu_padded, wl.cu_actual, wl.cp, s)
        except ValueError:
            continue
        for r in range(wl.cp):
            ref = oracle.partition_indices(wl.cu_padded, wl.cp, r, s)
            got = _gpu_indices(wl.cu_padded, wl.T, wl.cp, r, s)
            np.testing.assert_array_equal(got, ref)


def _short_document_layouts():
    """3000 documents: 1000 of 2*cp or 4*cp tokens, a run of 100 long ones, then 1900 of 2*cp to 8*cp tokens.
    A wave's 256 outputs then span more than 63 documents (the kernel's per-lane search) or fewer (its register
    lookup), and some waves straddle the two."""
    out = []
    for seed, cp in enumerate((1, 2, 4, 8)):
        rng = np.random.default_rng([77, seed])
        units = rng.integers(1, 5, size=3000)
        units[:1000] = rng.integers(1, 3, size=1000)
        units[1000:1100] = rng.integers(50, 400, size=100)
        out.append((f"short_docs.cp{cp}", np.concatenate([[0], np.cumsum(2 * cp * units)]).astype(np.int32), cp))
    return out


SHORT_DOCS = _short_document_layouts()


@pytest.mark.parametrize("name,cu_p,cp", SHORT_DOCS, ids=[n for n, _, _ in SHORT_DOCS])
def test_partition_many_short_documents(name, cu_p, cp):
    T = int(cu_p[-1])
    for s in (0, 1, 2):
        for r in range(cp):
            log(f"partition {name} s={s} r={r}")
            np.testing.assert_array_equal(_gpu_indices(cu_p, T, cp, r, s), oracle.partition_indices(cu_p, cp, r, s))


def test_partition_million_tokens_ten_thousand_docs():
    cu_p, _ = W.t1m_10k_docs()
    T = int(cu_p[-1])
    for s in (0, 1, 2):
        for r in range(4):
            log(f"partition 5b s={s} r={r}")
            np.testing.assert_array_equal(_gpu_indices(cu_p, T, 4, r, s), oracle.partition_indices(cu_p, 4, r, s))


def test_partition_device_status_bits():
    cu = i32_dev([0, 6, 16])                     # 6 not divisible by 2*cp = 4
    out = torch.empty(8, dtype=torch.int32, device="cuda")
    st = status_dev()
    cpthd.cpthd_partition_indices(cu, 2, 16, 2, 0, 0, out, st)
    assert int(st.item()) & 4
    st = status_dev()
    cpthd.cpthd_partition_indices(cu, 2, 16, 2, 0, 1, out, st)   # contiguous accepts it
    assert int(st.item()) == 0
    st = status_dev()
    cpthd.cpthd_partition_indices(i32_dev([0, 8, 4, 16]), 3, 16, 2, 0, 1, out, st)
    assert int(st.item()) & 1
    st = status_dev()
    cpthd.cpthd_partition_indices(i32_dev([0, 8, 12]), 2, 16, 2, 0, 1, out, st)
    assert int(st.item()) & 2
    st = status_dev()
    cpthd.cpthd_partition_indices(i32_dev([0, 5, 11, 16]), 3, 16, 2, 1, 2, out, st)   # packed: any lengths
    assert int(st.item()) == 0
    assert out[:8].cpu().tolist() == [4, 5, 6, 7, 8, 9, 10, 11]
    torch.cuda.synchronize()


def _rand_rows(T, row_elems, seed):
    """Rows of arbitrary 16-bit patterns (NaNs included), drawn on the GPU by a seeded generator: the restoration
    copies bits, so any pattern is a valid input and the expected output is the input itself."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randint(-(1 << 15), 1 << 15, (T, row_elems), dtype=torch.int16, device="cuda", generator=g)


# every named workload (config 4 has no DualChunkSwap layout, but its contiguous copy is checked), every
# dynamic-T micro-batch, and every other small random layout
REORDER = [(n, wl) for n, wl in LAYOUTS if not n.startswith("small")] + \
    [(n, wl) for n, wl in LAYOUTS if n.startswith("small")][::2]


@pytest.mark.parametrize("name,wl", REORDER, ids=[n for n, _ in REORDER])
def test_reorder_bit_exact(name, wl):
    log(f"reorder {name}")
    row_elems = 1024 if wl.T >= 4096 else 8 * (1 + wl.T % 3)
    cap = max(wl.T, wl.capacity) + 16
    k_phys = _rand_rows(wl.T, row_elems, 1)
    v_phys = _rand_rows(wl.T, row_elems, 2)
    for s in (0, 1, 2):
        try:
            oracle.check_layout(wl.cu_padded, wl.cu_actual, wl.cp, s)
        except ValueError:
            continue
        parts = [oracle.partition_indices(wl.cu_padded, wl.cp, r, s) for r in range(wl.cp)]
        order = torch.from_numpy(oracle.all_gather(np.arange(wl.T), parts)).to("cuda")
        kg = torch.full((cap, row_elems), 0x7FC0, dtype=torch.int16, device="cuda")
        vg = torch.full((cap, row_elems), 0x7FC0, dtype=torch.int16, device="cuda")
        kg[:wl.T] = k_phys[order]          # simulated all-gather (rank-major), oracle partition
        vg[:wl.T] = v_phys[order]
        ko = torch.full((cap, row_elems), 123, dtype=torch.int16, device="cuda")
        vo = torch.full((cap, row_elems), 123, dtype=torch.int16, device="cuda")
        st = status_dev()
        cpthd.cpthd_reorder_kv(kg, vg, ko, vo, row_elems * 2, i32_dev(wl.cu_padded), wl.num_docs, wl.T, cap,
                               wl.cp, s, st)
        assert int(st.item()) == 0
        assert torch.equal(ko[:wl.T], k_phys) and torch.equal(vo[:wl.T], v_phys)
        assert (ko[wl.T:] == 123).all() and (vo[wl.T:] == 123).all(), "wrote past T"
        if s == 1:   # in place: nothing to do and nothing changes
            before = kg.clone()
            cpthd.cpthd_reorder_kv(kg, vg, kg, vg, row_elems * 2, i32_dev(wl.cu_padded), wl.num_docs, wl.T, cap,
                                   wl.cp, s, st)
            assert torch.equal(kg, before)
    torch.cuda.synchronize()


SLICE = [(n, wl) for n, wl in LAYOUTS if n.startswith(("tiny_t28", "t32768_gqa32x8", "dynamic_t.mb3")) or n.endswith(".cp3.s2")]


@pytest.mark.parametrize("name,wl", SLICE, ids=[n for n, _ in SLICE])
def test_batch_slicing_bit_exact(name, wl):
    """input_ids / labels / position_ids of a rank, sliced with the rank's partition indices."""
    log(f"slice {name}")
    rng = np.random.default_rng(7)
    ids = rng.integers(0, 1 << 40, size=wl.T, dtype=np.int64)
    labels = rng.integers(-100, 50000, size=wl.T, dtype=np.int64)
    _, pos, _ = oracle.token_map(wl.cu_padded, wl.cu_actual)
    dev = [torch.from_numpy(x).to("cuda") for x in (ids, labels, pos.astype(np.int64))]
    for s in (0, 1, 2):
        try:
            oracle.check_layout(wl.cu_padded, wl.cu_actual, wl.cp, s)
        except ValueError:
            continue
        for r in range(wl.cp):
            st = status_dev()
            got = cpthd.get_batch_on_this_cp_rank(i32_dev(wl.cu_padded), wl.T, wl.cp, r, s, *dev, dev_status=st)
            ref = oracle.batch_on_rank(wl.cu_padded, wl.cp, r, s, ids, labels, pos.astype(np.int64))
            assert int(st.item()) == 0
            for g, x in zip(got, ref):
                np.testing.assert_array_equal(g.cpu().numpy(), x)


def test_gather_rows_widths_and_bad_index():
    rng = np.random.default_rng(1)
    for shape in [(300, 4, 16), (300, 3), (300, 5, 2)]:     # 128-byte bf16 rows, 12-byte and 40-byte rows
        x = rng.integers(-(1 << 30), 1 << 30, size=shape, dtype=np.int32)
        if shape == (300, 4, 16):
            src = torch.from_numpy(x.astype(np.int16)).to("cuda")
            ref_src = x.astype(np.int16)
        else:
            src = torch.from_numpy(x).to("cuda")
            ref_src = x
        idx = rng.integers(0, 300, size=517).astype(np.int32)
        st = status_dev()
        out = cpthd.gather_rows(src, i32_dev(idx), dev_status=st)
        assert int(st.item()) == 0
        np.testing.assert_array_equal(out.cpu().numpy(), ref_src[idx])
    bad = np.array([0, 5, 300, -1, 7], dtype=np.int32)
    st = status_dev()
    out = cpthd.gather_rows(src, i32_dev(bad), dev_status=st)
    assert int(st.item()) & 32
    o = out.cpu().numpy()
    np.testing.assert_array_equal(o[[0, 1, 4]], ref_src[[0, 5, 7]])
    assert (o[2] == 0).all() and (o[3] == 0).all()

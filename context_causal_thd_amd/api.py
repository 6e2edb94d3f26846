"""Python binding of libcpthd.so: argument marshalling only.

The functions named ``cpthd_*`` map one to one onto the C entry points of
include/cpthd.h and take torch tensors (device memory) in place of pointers;
every step of the computation runs in the library's HIP kernels.  torch is
used for device memory and the current stream only.

Above them sit small conveniences (``partition_indices``, ``reorder_kv``,
``AttnPlan``, ``attention``) and ``CPAttention``, an autograd function that
captures the load-balancing strategy and the plan in forward so that backward
sees the same token layout (TransformerEngine PR #3221, "What changed":
backward reuses the strategy captured in forward).
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _lib

DUAL_CHUNK_SWAP = 0
NO_LOAD_BALANCE = 1
PACKED_SUPER_SEQUENCE = 2

_DEV_BITS = {1: "cu_seqlens_padded not non-decreasing or not starting at 0",
             2: "cu_seqlens_padded[B] != T",
             4: "DualChunkSwap: a padded document length is not divisible by 2*cp_size",
             8: "cu_seqlens not non-decreasing, or an actual length exceeds its padded length",
             16: "workspace does not hold a plan for these arguments",
             32: "a gather index lies outside the source rows",
             64: "a document's K/V rows reach 2 GiB (one 32-bit buffer range per document)"}


def _p(t):
    """Device pointer of a tensor (None -> NULL).  Rejects CPU / non-contiguous tensors."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _need(t, name, dtype, rows, tail):
    """t must be a `dtype` tensor of shape [>= rows, *tail]: the kernels touch rows [0, rows) and trust the row
    layout, so a wrong dtype or shape is refused here instead of being read out of bounds."""
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.dim() != 1 + len(tail) or tuple(t.shape[1:]) != tuple(tail) or t.shape[0] < rows:
        want = ", ".join([f">= {rows}"] + [str(x) for x in tail])
        raise ValueError(f"{name}: expected shape [{want}], got {tuple(t.shape)}")


def _s(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ev(events):
    if events is None:
        return None, 0
    return events.array_ptr(), events.n


def describe_dev_status(bits: int) -> str:
    return "; ".join(msg for b, msg in _DEV_BITS.items() if bits & b) or "ok"


# ----------------------------------------------------------------------------
# one-to-one wrappers of the C ABI
# ----------------------------------------------------------------------------
def cpthd_partition_indices(cu_seqlens_padded, num_docs, total_tokens, cp_size, rank, strategy, out_indices,
                            dev_status=None, stream=None):
    return _lib.call("cpthd_partition_indices", _p(cu_seqlens_padded), num_docs, total_tokens, cp_size, rank,
                     strategy, _p(out_indices), _p(dev_status), _s(stream))


def cpthd_reorder_kv(k_gathered, v_gathered, k_out, v_out, row_bytes, cu_seqlens_padded, num_docs, total_tokens,
                     capacity_tokens, cp_size, strategy, dev_status=None, stream=None):
    return _lib.call("cpthd_reorder_kv", _p(k_gathered), _p(v_gathered), _p(k_out), _p(v_out), row_bytes,
                     _p(cu_seqlens_padded), num_docs, total_tokens, capacity_tokens, cp_size, strategy,
                     _p(dev_status), _s(stream))


def cpthd_gather_rows(src, src_rows, row_bytes, index, n, dst, dev_status=None, stream=None):
    return _lib.call("cpthd_gather_rows", _p(src), src_rows, row_bytes, _p(index), n, _p(dst), _p(dev_status),
                     _s(stream))


def cpthd_attn_workspace_bytes(capacity_tokens, cp_size, num_q_heads, num_kv_heads, head_dim, max_docs):
    return int(_lib.load().cpthd_attn_workspace_bytes(capacity_tokens, cp_size, num_q_heads, num_kv_heads,
                                                      head_dim, max_docs))


def cpthd_attn_workspace_min_bytes(capacity_tokens, cp_size, num_q_heads, num_kv_heads, head_dim, max_docs):
    return int(_lib.load().cpthd_attn_workspace_min_bytes(capacity_tokens, cp_size, num_q_heads, num_kv_heads,
                                                          head_dim, max_docs))


def cpthd_attn_plan(cu_seqlens, cu_seqlens_padded, num_docs, total_tokens, capacity_tokens, cp_size, rank,
                    strategy, num_q_heads, num_kv_heads, head_dim, workspace, dev_status=None, stream=None):
    return _lib.call("cpthd_attn_plan", _p(cu_seqlens), _p(cu_seqlens_padded), num_docs, total_tokens,
                     capacity_tokens, cp_size, rank, strategy, num_q_heads, num_kv_heads, head_dim, _p(workspace),
                     workspace.numel() * workspace.element_size(), _p(dev_status), _s(stream))


_FWD_NAMES = {False: "cpthd_attn_fwd", True: "cpthd_attn_fwd_allgathered"}
_BWD_NAMES = {False: "cpthd_attn_bwd", True: "cpthd_attn_bwd_allgathered"}


def _fwd_args(q_local, k, v, cu_seqlens, cu_seqlens_padded, num_docs, total_tokens, capacity_tokens, cp_size, rank,
              strategy, num_q_heads, num_kv_heads, head_dim, softmax_scale, causal, window_left, window_right, o_local,
              lse_local, workspace, dev_status, stream):
    return (_p(q_local), _p(k), _p(v), _p(cu_seqlens), _p(cu_seqlens_padded), num_docs, total_tokens,
            capacity_tokens, cp_size, rank, strategy, num_q_heads, num_kv_heads, head_dim, softmax_scale, causal,
            window_left, window_right, _p(o_local), _p(lse_local), _p(workspace),
            workspace.numel() * workspace.element_size(), _p(dev_status), _s(stream))


def _bwd_args(q_local, k, v, o_local, do_local, lse_local, cu_seqlens, cu_seqlens_padded, num_docs, total_tokens,
              capacity_tokens, cp_size, rank, strategy, num_q_heads, num_kv_heads, head_dim, softmax_scale, causal,
              window_left, window_right, dq_local, dk, dv, workspace, dev_status, stream):
    return (_p(q_local), _p(k), _p(v), _p(o_local), _p(do_local), _p(lse_local), _p(cu_seqlens),
            _p(cu_seqlens_padded), num_docs, total_tokens, capacity_tokens, cp_size, rank, strategy, num_q_heads,
            num_kv_heads, head_dim, softmax_scale, causal, window_left, window_right, _p(dq_local), _p(dk), _p(dv),
            _p(workspace), workspace.numel() * workspace.element_size(), _p(dev_status), _s(stream))


def cpthd_attn_fwd(q_local, k, v, cu_seqlens, cu_seqlens_padded, num_docs, total_tokens, capacity_tokens, cp_size,
                   rank, strategy, num_q_heads, num_kv_heads, head_dim, softmax_scale, causal, window_left,
                   window_right, o_local, lse_local, workspace, dev_status=None, stream=None):
    return _lib.call("cpthd_attn_fwd", *_fwd_args(
        q_local, k, v, cu_seqlens, cu_seqlens_padded, num_docs, total_tokens, capacity_tokens, cp_size, rank,
        strategy, num_q_heads, num_kv_heads, head_dim, softmax_scale, causal, window_left, window_right, o_local,
        lse_local, workspace, dev_status, stream))


def cpthd_attn_fwd_allgathered(q_local, k_gathered, v_gathered, cu_seqlens, cu_seqlens_padded, num_docs,
                               total_tokens, capacity_tokens, cp_size, rank, strategy, num_q_heads, num_kv_heads,
                               head_dim, softmax_scale, causal, window_left, window_right, o_local, lse_local,
                               workspace, dev_status=None, stream=None):
    return _lib.call("cpthd_attn_fwd_allgathered", *_fwd_args(
        q_local, k_gathered, v_gathered, cu_seqlens, cu_seqlens_padded, num_docs, total_tokens, capacity_tokens,
        cp_size, rank, strategy, num_q_heads, num_kv_heads, head_dim, softmax_scale, causal, window_left,
        window_right, o_local, lse_local, workspace, dev_status, stream))


def cpthd_attn_fwd_timed(q_local, k, v, cu_seqlens, cu_seqlens_padded, num_docs, total_tokens, capacity_tokens,
                         cp_size, rank, strategy, num_q_heads, num_kv_heads, head_dim, softmax_scale, causal,
                         window_left, window_right, o_local, lse_local, workspace, dev_status, stream, kv_allgathered,
                         events):
    ev, nev = _ev(events)
    return _lib.call("cpthd_attn_fwd_timed", *_fwd_args(
        q_local, k, v, cu_seqlens, cu_seqlens_padded, num_docs, total_tokens, capacity_tokens, cp_size, rank,
        strategy, num_q_heads, num_kv_heads, head_dim, softmax_scale, causal, window_left, window_right, o_local,
        lse_local, workspace, dev_status, stream), int(bool(kv_allgathered)), ev, nev)


def cpthd_attn_bwd(q_local, k, v, o_local, do_local, lse_local, cu_seqlens, cu_seqlens_padded, num_docs, total_tokens,
                   capacity_tokens, cp_size, rank, strategy, num_q_heads, num_kv_heads, head_dim, softmax_scale,
                   causal, window_left, window_right, dq_local, dk, dv, workspace, dev_status=None, stream=None):
    return _lib.call("cpthd_attn_bwd", *_bwd_args(
        q_local, k, v, o_local, do_local, lse_local, cu_seqlens, cu_seqlens_padded, num_docs, total_tokens,
        capacity_tokens, cp_size, rank, strategy, num_q_heads, num_kv_heads, head_dim, softmax_scale, causal,
        window_left, window_right, dq_local, dk, dv, workspace, dev_status, stream))


def cpthd_attn_bwd_allgathered(q_local, k_gathered, v_gathered, o_local, do_local, lse_local, cu_seqlens,
                               cu_seqlens_padded, num_docs, total_tokens, capacity_tokens, cp_size, rank, strategy,
                               num_q_heads, num_kv_heads, head_dim, softmax_scale, causal, window_left, window_right,
                               dq_local, dk_gathered, dv_gathered, workspace, dev_status=None, stream=None):
    return _lib.call("cpthd_attn_bwd_allgathered", *_bwd_args(
        q_local, k_gathered, v_gathered, o_local, do_local, lse_local, cu_seqlens, cu_seqlens_padded, num_docs,
        total_tokens, capacity_tokens, cp_size, rank, strategy, num_q_heads, num_kv_heads, head_dim, softmax_scale,
        causal, window_left, window_right, dq_local, dk_gathered, dv_gathered, workspace, dev_status, stream))


# Bytes of the static scratch array cpthd_attn_bwd_noalloc uses as its workspace (CPTHD_STATIC_SCRATCH_BYTES).
# An AttnPlan with workspace_bytes=STATIC_SCRATCH_BYTES gets the plan that entry point builds.
STATIC_SCRATCH_BYTES = 16 << 20


def cpthd_attn_bwd_noalloc(q_local, k, v, o_local, do_local, lse_local, cu_seqlens, cu_seqlens_padded, num_docs,
                           total_tokens, capacity_tokens, cp_size, rank, strategy, num_q_heads, num_kv_heads,
                           head_dim, softmax_scale, causal, window_left, window_right, dq_local, dk, dv,
                           dev_status=None, stream=None):
    """cpthd_attn_bwd with the library's static scratch array in place of a workspace (no device allocation)."""
    return _lib.call("cpthd_attn_bwd_noalloc", _p(q_local), _p(k), _p(v), _p(o_local), _p(do_local), _p(lse_local),
                     _p(cu_seqlens), _p(cu_seqlens_padded), num_docs, total_tokens, capacity_tokens, cp_size, rank,
                     strategy, num_q_heads, num_kv_heads, head_dim, softmax_scale, causal, window_left,
                     window_right, _p(dq_local), _p(dk), _p(dv), _p(dev_status), _s(stream))


def cpthd_attn_bwd_timed(q_local, k, v, o_local, do_local, lse_local, cu_seqlens, cu_seqlens_padded, num_docs,
                         total_tokens, capacity_tokens, cp_size, rank, strategy, num_q_heads, num_kv_heads, head_dim,
                         softmax_scale, causal, window_left, window_right, dq_local, dk, dv, workspace, dev_status,
                         stream, kv_allgathered, events):
    ev, nev = _ev(events)
    return _lib.call("cpthd_attn_bwd_timed", *_bwd_args(
        q_local, k, v, o_local, do_local, lse_local, cu_seqlens, cu_seqlens_padded, num_docs, total_tokens,
        capacity_tokens, cp_size, rank, strategy, num_q_heads, num_kv_heads, head_dim, softmax_scale, causal,
        window_left, window_right, dq_local, dk, dv, workspace, dev_status, stream), int(bool(kv_allgathered)),
        ev, nev)


# ----------------------------------------------------------------------------
# HIP events for the optional per-kernel timing argument
# ----------------------------------------------------------------------------
class HipEvents:
    """n raw hipEvent_t handles, created through the HIP runtime torch already loaded."""

    def __init__(self, n: int):
        torch.cuda.init()
        self._hip = ctypes.CDLL("libamdhip64.so.7")
        self.n = n
        self._arr = (ctypes.c_void_p * n)()
        for i in range(n):
            rc = self._hip.hipEventCreate(ctypes.byref(self._arr, i * ctypes.sizeof(ctypes.c_void_p)))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")

    def array_ptr(self):
        return ctypes.cast(self._arr, ctypes.c_void_p)

    def elapsed_ms(self, i: int, j: int) -> float:
        """ms between events i and j (both must have been recorded)."""
        ms = ctypes.c_float()
        rc = self._hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self._arr[i]),
                                           ctypes.c_void_p(self._arr[j]))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def close(self):
        for i in range(self.n):
            if self._arr[i]:
                self._hip.hipEventDestroy(ctypes.c_void_p(self._arr[i]))
                self._arr[i] = None


# ----------------------------------------------------------------------------
# conveniences
# ----------------------------------------------------------------------------
def check_dev_status(dev_status) -> None:
    bits = int(dev_status.item())
    if bits:
        raise ValueError(f"device-detected metadata error (bits {bits}): {describe_dev_status(bits)}")


def partition_indices(cu_seqlens_padded, total_tokens, cp_size, rank, strategy, out=None, dev_status=None):
    """int32 [T/cp_size] physical token indices of ``rank`` (device tensor)."""
    _need(cu_seqlens_padded, "cu_seqlens_padded", torch.int32, 2, ())
    num_docs = cu_seqlens_padded.numel() - 1
    if out is None:
        out = torch.empty(total_tokens // cp_size, dtype=torch.int32, device=cu_seqlens_padded.device)
    _need(out, "out", torch.int32, total_tokens // cp_size, ())
    cpthd_partition_indices(cu_seqlens_padded, num_docs, total_tokens, cp_size, rank, strategy, out, dev_status)
    return out


def gather_rows(src, index, out=None, dev_status=None):
    """out[j] = src[index[j]] along the first dimension (any dtype)."""
    _need(index, "index", torch.int32, 0, ())
    n = index.numel()
    if out is None:
        out = torch.empty((n,) + tuple(src.shape[1:]), dtype=src.dtype, device=src.device)
    _need(out, "out", src.dtype, n, tuple(src.shape[1:]))
    row_bytes = (src[0].numel() if src.dim() > 1 else 1) * src.element_size()
    cpthd_gather_rows(src, src.shape[0], row_bytes, index, n, out, dev_status)
    return out


def get_batch_on_this_cp_rank(cu_seqlens_padded, total_tokens, cp_size, rank, strategy, *tensors, dev_status=None):
    """The rank's slice of per-token tensors (e.g. input_ids, labels, position_ids), partitioned with the
    same strategy as attention: rows at the rank's partition indices, in local order."""
    idx = partition_indices(cu_seqlens_padded, total_tokens, cp_size, rank, strategy, dev_status=dev_status)
    return tuple(gather_rows(t, idx, dev_status=dev_status) for t in tensors)


def reorder_kv(k_gathered, v_gathered, cu_seqlens_padded, total_tokens, cp_size, strategy, k_out=None, v_out=None,
               dev_status=None):
    """Physical-order K and V from the rank-major all-gathered buffers."""
    tail = tuple(k_gathered.shape[1:])
    _need(k_gathered, "k_gathered", k_gathered.dtype, total_tokens, tail)
    _need(v_gathered, "v_gathered", k_gathered.dtype, total_tokens, tail)
    _need(cu_seqlens_padded, "cu_seqlens_padded", torch.int32, 2, ())
    if k_out is None:
        k_out = torch.empty_like(k_gathered)
    if v_out is None:
        v_out = torch.empty_like(v_gathered)
    _need(k_out, "k_out", k_gathered.dtype, total_tokens, tail)
    _need(v_out, "v_out", k_gathered.dtype, total_tokens, tail)
    row_bytes = k_gathered[0].numel() * k_gathered.element_size()
    cpthd_reorder_kv(k_gathered, v_gathered, k_out, v_out, row_bytes, cu_seqlens_padded,
                     cu_seqlens_padded.numel() - 1, total_tokens, k_gathered.shape[0], cp_size, strategy, dev_status)
    return k_out, v_out


class Layout:
    """The document layout of one micro-batch as one rank sees it: the device cu arrays, T, rank and strategy."""

    def __init__(self, cu_seqlens, cu_seqlens_padded, total_tokens, rank, strategy):
        _need(cu_seqlens_padded, "cu_seqlens_padded", torch.int32, 2, ())
        _need(cu_seqlens, "cu_seqlens", torch.int32, cu_seqlens_padded.numel(), ())
        if cu_seqlens.numel() != cu_seqlens_padded.numel():
            raise ValueError("cu_seqlens and cu_seqlens_padded must have the same length")
        self.cu_seqlens, self.cu_seqlens_padded = cu_seqlens, cu_seqlens_padded
        self.num_docs = cu_seqlens_padded.numel() - 1
        self.total_tokens, self.rank, self.strategy = int(total_tokens), int(rank), int(strategy)

    def frozen(self):
        """A copy whose cu arrays later writes to the caller's tensors cannot change."""
        return Layout(self.cu_seqlens.clone(), self.cu_seqlens_padded.clone(), self.total_tokens, self.rank,
                      self.strategy)


class AttnPlan:
    """Workspace of one rank's attention calls, sized once for a token capacity and a document count, plus the
    layout of the current micro-batch (set by ``build``) and a device status word.

    The C entry points check the plan held in the workspace against the cu arrays of every call and rebuild it
    when it was built from others, so a call always computes with its own layout.

    ``workspace_bytes`` (default: ``cpthd_attn_workspace_bytes``) sizes the workspace otherwise: a larger one
    changes nothing, a smaller one (down to ``cpthd_attn_workspace_min_bytes``) holds fewer partial slots for split
    tiles, so the plan splits fewer of them.  Two workspaces of the same size get the same plan, and the same results."""

    def __init__(self, capacity_tokens, cp_size, num_q_heads, num_kv_heads, head_dim, max_docs, device="cuda",
                 workspace_bytes=None):
        self.capacity = capacity_tokens
        self.cp_size = cp_size
        self.Hq, self.Hkv, self.D = num_q_heads, num_kv_heads, head_dim
        self.max_docs = max_docs
        nbytes = cpthd_attn_workspace_bytes(capacity_tokens, cp_size, num_q_heads, num_kv_heads, head_dim, max_docs)
        if nbytes == 0:
            raise ValueError("unsupported attention configuration")
        if workspace_bytes is not None:
            nbytes = int(workspace_bytes)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)
        self.layout = None

    def build(self, cu_seqlens, cu_seqlens_padded, total_tokens, rank, strategy, dev_status=None):
        """Set the micro-batch's layout and build its plan now (a fresh status word unless ``dev_status``)."""
        lay = Layout(cu_seqlens, cu_seqlens_padded, total_tokens, rank, strategy)
        if lay.num_docs > self.max_docs:
            raise ValueError("more documents than the workspace was sized for")
        if dev_status is None:
            self.status.zero_()
            dev_status = self.status
        cpthd_attn_plan(cu_seqlens, cu_seqlens_padded, lay.num_docs, lay.total_tokens, self.capacity, self.cp_size,
                        lay.rank, lay.strategy, self.Hq, self.Hkv, self.D, self.workspace, dev_status)
        self.layout = lay
        return self

    def check(self):
        """Raise if a call using this plan's status word reported a device-side error (synchronises)."""
        check_dev_status(self.status)

    def _args(self, lay=None):
        lay = lay or self.layout
        if lay is None:
            raise RuntimeError("plan not built: no layout set")
        if lay.num_docs > self.max_docs:
            raise ValueError("more documents than the workspace was sized for")
        return (lay.cu_seqlens, lay.cu_seqlens_padded, lay.num_docs, lay.total_tokens, self.capacity, self.cp_size,
                lay.rank, lay.strategy, self.Hq, self.Hkv, self.D)


def attn_fwd(q_local, k, v, plan: AttnPlan, softmax_scale=None, o_local=None, lse_local=None, dev_status=None,
             events=None, kv_allgathered=False, layout=None):
    """O and LSE of the rank's query rows for ``layout`` (default: the plan's current one).  ``kv_allgathered``:
    k and v are in rank-major all-gathered order (as an all-gather of the ranks' local K/V leaves them) instead
    of physical order.  ``events`` (HipEvents of 8) times the call's kernels: plan check, attention, the merge of
    split tiles and the V^T pass (pairs the call leaves out are recorded back to back)."""
    lay = layout or plan.layout
    args = plan._args(lay)
    T = lay.total_tokens
    S = T // plan.cp_size
    bf = torch.bfloat16
    _need(q_local, "q_local", bf, S, (plan.Hq, plan.D))
    _need(k, "k", bf, T, (plan.Hkv, plan.D))
    _need(v, "v", bf, T, (plan.Hkv, plan.D))
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(plan.D)
    if o_local is None:
        o_local = torch.empty((S, plan.Hq, plan.D), dtype=torch.bfloat16, device=q_local.device)
    if lse_local is None:
        lse_local = torch.empty((S, plan.Hq), dtype=torch.float32, device=q_local.device)
    _need(o_local, "o_local", bf, S, (plan.Hq, plan.D))
    _need(lse_local, "lse_local", torch.float32, S, (plan.Hq,))
    if dev_status is None:
        dev_status = plan.status
    tail = (softmax_scale, 1, -1, 0, o_local, lse_local, plan.workspace, dev_status)
    if events is not None:
        cpthd_attn_fwd_timed(q_local, k, v, *args, *tail, None, kv_allgathered, events)
    else:
        (cpthd_attn_fwd_allgathered if kv_allgathered else cpthd_attn_fwd)(q_local, k, v, *args, *tail)
    return o_local, lse_local


def attn_bwd(q_local, k, v, o_local, do_local, lse_local, plan: AttnPlan, softmax_scale=None, dq_local=None,
             dk=None, dv=None, dev_status=None, events=None, kv_allgathered=False, layout=None):
    """dQ of the rank's rows and its partial dK, dV (fp32) for ``layout`` (default: the plan's current one).
    With ``kv_allgathered`` k, v and the returned dk, dv are in rank-major all-gathered order.  Gradients this
    function allocates have the inputs' row counts; rows past the active S (dq) or T (dk, dv) are zero.
    ``events`` (HipEvents of 8) times the call's kernels: plan check, query-tile pass, key-tile pass, and the merge
    of split tiles (when the workspace has partial slots)."""
    lay = layout or plan.layout
    args = plan._args(lay)
    T = lay.total_tokens
    S = T // plan.cp_size
    bf, f32 = torch.bfloat16, torch.float32
    for t, name in ((q_local, "q_local"), (o_local, "o_local"), (do_local, "do_local")):
        _need(t, name, bf, S, (plan.Hq, plan.D))
    _need(k, "k", bf, T, (plan.Hkv, plan.D))
    _need(v, "v", bf, T, (plan.Hkv, plan.D))
    _need(lse_local, "lse_local", f32, S, (plan.Hq,))
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(plan.D)

    def grad_buf(x, rows):
        g = torch.empty(x.shape, dtype=f32, device=x.device)
        if x.shape[0] > rows:   # capacity-sized input: the inactive tail gets a zero gradient
            g[rows:].zero_()
        return g

    if dq_local is None:
        dq_local = grad_buf(q_local, S)
    if dk is None:
        dk = grad_buf(k, T)
    if dv is None:
        dv = grad_buf(v, T)
    _need(dq_local, "dq_local", f32, S, (plan.Hq, plan.D))
    _need(dk, "dk", f32, T, (plan.Hkv, plan.D))
    _need(dv, "dv", f32, T, (plan.Hkv, plan.D))
    if dev_status is None:
        dev_status = plan.status
    tail = (softmax_scale, 1, -1, 0, dq_local, dk, dv, plan.workspace, dev_status)
    if events is not None:
        cpthd_attn_bwd_timed(q_local, k, v, o_local, do_local, lse_local, *args, *tail, None, kv_allgathered, events)
    else:
        (cpthd_attn_bwd_allgathered if kv_allgathered else cpthd_attn_bwd)(q_local, k, v, o_local, do_local,
                                                                           lse_local, *args, *tail)
    return dq_local, dk, dv


class CPAttention(torch.autograd.Function):
    """Causal THD attention of one CP rank; backward runs with the layout (cu arrays, rank, strategy) captured in
    forward, whatever the plan was rebuilt for in between (PR #3221 "What changed": the strategy captured in
    forward drives backward)."""

    @staticmethod
    def forward(ctx, q_local, k, v, plan: AttnPlan, softmax_scale, kv_allgathered=False, check=True):
        lay = plan.layout.frozen()
        o, lse = attn_fwd(q_local, k, v, plan, softmax_scale, kv_allgathered=kv_allgathered, layout=lay)
        if check:
            plan.check()
        ctx.plan, ctx.layout, ctx.scale, ctx.kv_allgathered, ctx.check = plan, lay, softmax_scale, kv_allgathered, check
        ctx.save_for_backward(q_local, k, v, o, lse)
        return o

    @staticmethod
    def backward(ctx, do):
        q_local, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = attn_bwd(q_local, k, v, o, do.contiguous(), lse, ctx.plan, ctx.scale,
                              kv_allgathered=ctx.kv_allgathered, layout=ctx.layout)
        if ctx.check:
            ctx.plan.check()
        return dq.to(q_local.dtype), dk.to(k.dtype), dv.to(v.dtype), None, None, None, None


def attention(q_local, k, v, plan: AttnPlan, softmax_scale=None, kv_allgathered=False, check=True):
    """Autograd attention of one CP rank for the plan's current layout; k and v in physical order, or in
    rank-major all-gathered order with ``kv_allgathered`` (their gradients then come back in the same order).
    ``check`` reads the plan's status word after forward and after backward (a synchronisation) and raises on a
    device-side error; with ``check=False`` call ``plan.check()`` when convenient."""
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(plan.D)
    return CPAttention.apply(q_local, k, v, plan, softmax_scale, kv_allgathered, check)

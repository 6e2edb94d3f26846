"""CPU oracle for one context-parallel rank's share of causal THD attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or calls
this module; only the tests, the smoke check and the benchmark's CPU-baseline
leg do.  It shares no code with the HIP path.

Everything is plain numpy in float64, written from the definitions on the
pages (TransformerEngine PR #3221 "[PyTorch] Add no-load-balance THD
all-gather CP", sections "How to use", "What changed", "Why", "Scope and
constraints", and its commit messages and review thread):

* ``partition_indices``  the tokens a rank owns.  DualChunkSwap ("Why"): every
  document is cut into 2*cp_size equal chunks and rank r owns the mirrored pair
  r and 2*cp_size-1-r.  NO_LOAD_BALANCE ("What changed", "Why"): the whole
  physical buffer is cut into cp_size contiguous chunks and rank r owns chunk r;
  documents stay separated only through the sequence metadata.
  PACKED_SUPER_SEQUENCE (the commit messages' earlier packed policy): the whole
  physical buffer is treated as one partitioning sequence, cut into 2*cp_size
  chunks with the same mirrored pairing, documents again separated only by the
  sequence metadata.
* ``all_gather`` / ``restore``  the rank-major concatenation that an all-gather
  of per-rank K/V produces, and its inverse ("K/V restoration" in the review
  thread; rank-major ownership "needs no KV reorder" in the commit messages).
* ``attn_fwd`` / ``attn_bwd``  causal softmax attention with window (-1, 0)
  ("Scope and constraints"), separately within each document, for the rank's
  query rows against all keys of the document (CP is exact: the rank's rows of
  the unpartitioned result).  Scores ``scale * q.k`` over keys of the same
  document at within-document position <= the query's, both tokens actual
  (not padding).  ``LSE`` is the natural-log log-sum-exp of those scores,
  ``O = softmax @ V``.  The backward pass is the exact gradient of that
  function for an upstream gradient dO.

Readings where the pages are silent (each also listed with the design notes):
pads occupy the tail of each padded slot and neither attend nor are attended;
a pad query row has O = 0, LSE = -inf and dQ = 0; q head h uses kv head
h // (Hq/Hkv); the rank's local rows are in document order, chunk r before
chunk 2*cp_size-1-r; dK/dV of one rank are its *partial* gradients over all T
physical rows (summing them over ranks gives the unpartitioned gradient).

Pins (tests/test_oracle_*.py): brute-force scalar loops, closed forms at each
document's first token, torch SDPA / autograd in float64 on the CPU as library
special cases, central finite differences, partition invariants and the
hand-derived config-1 values under tests/golden/.
"""
from __future__ import annotations

import numpy as np

DUAL_CHUNK_SWAP = 0
NO_LOAD_BALANCE = 1
PACKED_SUPER_SEQUENCE = 2
STRATEGIES = (DUAL_CHUNK_SWAP, NO_LOAD_BALANCE, PACKED_SUPER_SEQUENCE)

_ROW_BLOCK = 1024


# ----------------------------------------------------------------------------
# metadata
# ----------------------------------------------------------------------------
def check_layout(cu_padded, cu_actual, cp_size: int, strategy: int) -> None:
    """Raise ValueError unless the layout is one the strategy accepts.

    DualChunkSwap needs every padded document length divisible by 2*cp_size
    (the strategy cuts each document into 2*cp_size equal chunks; the
    contiguous strategy exists precisely because documents need not be, PR
    "Why").  The contiguous strategy needs T divisible by cp_size (equal local
    Q/K/V physical lengths, "Scope and constraints").
    """
    cu_p = [int(x) for x in cu_padded]
    cu_a = [int(x) for x in cu_actual] if cu_actual is not None else cu_p
    if cp_size < 1:
        raise ValueError("cp_size must be >= 1")
    if len(cu_p) < 2 or cu_p[0] != 0:
        raise ValueError("cu_seqlens_padded must start at 0 and hold B+1 entries")
    if len(cu_a) != len(cu_p) or cu_a[0] != 0:
        raise ValueError("cu_seqlens must start at 0 and match cu_seqlens_padded in length")
    for i in range(len(cu_p) - 1):
        L = cu_p[i + 1] - cu_p[i]
        a = cu_a[i + 1] - cu_a[i]
        if L < 0 or a < 0:
            raise ValueError(f"document {i}: negative length")
        if a > L:
            raise ValueError(f"document {i}: actual length {a} exceeds padded length {L}")
        if strategy == DUAL_CHUNK_SWAP and L % (2 * cp_size):
            raise ValueError(f"document {i}: padded length {L} not divisible by 2*cp_size")
    if strategy == NO_LOAD_BALANCE and cu_p[-1] % cp_size:
        raise ValueError("T not divisible by cp_size")
    if strategy == PACKED_SUPER_SEQUENCE and cu_p[-1] % (2 * cp_size):
        raise ValueError("T not divisible by 2*cp_size")
    if strategy not in STRATEGIES:
        raise ValueError("unknown strategy")


def token_map(cu_padded, cu_actual):
    """Per physical token: document id, within-document position, is-actual flag."""
    cu_p = [int(x) for x in cu_padded]
    cu_a = [int(x) for x in cu_actual]
    T = cu_p[-1]
    doc = np.empty(T, dtype=np.int64)
    pos = np.empty(T, dtype=np.int64)
    valid = np.empty(T, dtype=bool)
    for i in range(len(cu_p) - 1):
        lo, hi = cu_p[i], cu_p[i + 1]
        a = cu_a[i + 1] - cu_a[i]
        doc[lo:hi] = i
        pos[lo:hi] = np.arange(hi - lo)
        valid[lo:hi] = np.arange(hi - lo) < a
    return doc, pos, valid


# ----------------------------------------------------------------------------
# partition, all-gather, restoration
# ----------------------------------------------------------------------------
def partition_indices(cu_padded, cp_size: int, rank: int, strategy: int) -> np.ndarray:
    """Physical token indices owned by ``rank``, in the rank's local order."""
    cu_p = [int(x) for x in cu_padded]
    if not 0 <= rank < cp_size:
        raise ValueError("rank out of range")
    if strategy == DUAL_CHUNK_SWAP:
        out = []
        for i in range(len(cu_p) - 1):
            start, L = cu_p[i], cu_p[i + 1] - cu_p[i]
            if L % (2 * cp_size):
                raise ValueError(f"document {i} not divisible by 2*cp_size")
            c = L // (2 * cp_size)
            for chunk in (rank, 2 * cp_size - 1 - rank):
                out.extend(range(start + chunk * c, start + (chunk + 1) * c))
        return np.asarray(out, dtype=np.int64)
    if strategy == NO_LOAD_BALANCE:
        T = cu_p[-1]
        if T % cp_size:
            raise ValueError("T not divisible by cp_size")
        S = T // cp_size
        return np.arange(rank * S, (rank + 1) * S, dtype=np.int64)
    if strategy == PACKED_SUPER_SEQUENCE:
        # the physical buffer as a single partitioning sequence
        return partition_indices([0, cu_p[-1]], cp_size, rank, DUAL_CHUNK_SWAP)
    raise ValueError("unknown strategy")


def all_gather(x: np.ndarray, parts) -> np.ndarray:
    """Rank-major concatenation of every rank's rows ``x[parts[s]]``."""
    return np.concatenate([x[np.asarray(p)] for p in parts], axis=0)


def restore(gathered: np.ndarray, parts) -> np.ndarray:
    """Inverse of ``all_gather``: put every gathered row back at its physical index."""
    out = np.empty_like(gathered)
    off = 0
    for p in parts:
        p = np.asarray(p)
        out[p] = gathered[off:off + p.size]
        off += p.size
    if off != gathered.shape[0]:
        raise ValueError("parts do not cover the gathered buffer")
    return out


def batch_on_rank(cu_padded, cp_size: int, rank: int, strategy: int, *tensors):
    """The rank's slice of per-token tensors (input ids, labels, position ids, ...): rows
    ``x[idx_r]`` in local order ("How to use": input partitioning uses the same strategy as
    attention)."""
    idx = partition_indices(cu_padded, cp_size, rank, strategy)
    return tuple(np.asarray(x)[idx] for x in tensors)


def useful_pairs(idx, cu_padded, cu_actual) -> int:
    """Number of (query, key) pairs the causal mask allows for these query rows."""
    _, pos, valid = token_map(cu_padded, cu_actual)
    idx = np.asarray(idx)
    v = valid[idx]
    return int(np.sum(pos[idx][v] + 1))


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------
def _doc_rows(idx, cu_padded, cu_actual, docs):
    """For each document: (local rows of actual query tokens, their positions, doc start, actual length)."""
    cu_p = [int(x) for x in cu_padded]
    cu_a = [int(x) for x in cu_actual]
    doc, pos, valid = token_map(cu_p, cu_a)
    idx = np.asarray(idx, dtype=np.int64)
    ldoc, lpos, lval = doc[idx], pos[idx], valid[idx]
    for d in docs:
        rows = np.nonzero((ldoc == d) & lval)[0]
        yield d, rows, lpos[rows], cu_p[d], cu_a[d + 1] - cu_a[d]


def attn_fwd(q_local, k, v, idx, cu_padded, cu_actual, scale, docs=None, kv_heads=None, rows=None):
    """Forward for one rank: returns (O [S,Hq,D], LSE [S,Hq], computed [S]) in float64.

    ``docs`` restricts the work to those documents (rows of other documents are
    NaN and ``computed`` is False there); None means every document.
    ``kv_heads`` restricts it to the q heads of those kv heads (others NaN).
    ``rows`` (local row indices) restricts it to those query rows (others NaN):
    each row's result depends on that row's query and the keys alone.
    """
    q_local = np.asarray(q_local, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    S, Hq, D = q_local.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    B = len(cu_padded) - 1
    docs = range(B) if docs is None else docs
    o = np.full((S, Hq, D), np.nan)
    lse = np.full((S, Hq), np.nan)
    computed = np.zeros(S, dtype=bool)
    doc_of = token_map(cu_padded, cu_actual)[0][np.asarray(idx, dtype=np.int64)]
    hsel = np.array([kv_heads is None or h // G in kv_heads for h in range(Hq)])
    rsel = np.ones(S, dtype=bool)
    if rows is not None:
        rsel = np.zeros(S, dtype=bool)
        rsel[np.asarray(rows, dtype=np.int64)] = True
    for d in docs:
        sel = (doc_of == d) & rsel
        computed |= sel
        o[np.ix_(sel, hsel)] = 0.0      # pads: O = 0, LSE = -inf (overwritten for actual rows below)
        lse[np.ix_(sel, hsel)] = -np.inf
    for d, drows, qpos, start, a in _doc_rows(idx, cu_padded, cu_actual, docs):
        keep = rsel[drows]
        drows, qpos = drows[keep], qpos[keep]
        if drows.size == 0:
            continue
        kpos = np.arange(a)
        for h in range(Hq):
            if kv_heads is not None and h // G not in kv_heads:
                continue
            kd = k[start:start + a, h // G]
            vd = v[start:start + a, h // G]
            for b0 in range(0, drows.size, _ROW_BLOCK):
                r = drows[b0:b0 + _ROW_BLOCK]
                allowed = kpos[None, :] <= qpos[b0:b0 + _ROW_BLOCK, None]
                s = scale * (q_local[r, h] @ kd.T)
                s = np.where(allowed, s, -np.inf)
                m = s.max(axis=1)
                e = np.exp(s - m[:, None])
                den = e.sum(axis=1)
                lse[r, h] = m + np.log(den)
                o[r, h] = (e / den[:, None]) @ vd
    return o, lse, computed


def attn_bwd(q_local, k, v, do_local, idx, cu_padded, cu_actual, scale, docs=None, kv_heads=None, rows=None,
             keys=None):
    """Backward for one rank: returns (dQ [S,Hq,D], dK [T,Hkv,D], dV [T,Hkv,D]) in float64.

    dK/dV are the gradients contributed by this rank's query rows only (rows of
    keys no query of the rank sees are 0).  With ``docs`` given, dQ rows and
    dK/dV rows outside those documents are NaN; ``kv_heads`` restricts the
    work to those kv heads and their q heads in the same way.  ``rows`` (local
    row indices) restricts dQ to those rows and ``keys`` (physical token
    indices) restricts dK/dV to those keys (others NaN); a key's gradient still
    sums over every query row of the rank that sees it.
    """
    q_local = np.asarray(q_local, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do_local = np.asarray(do_local, dtype=np.float64)
    S, Hq, D = q_local.shape
    T, Hkv, _ = k.shape
    G = Hq // Hkv
    cu_p = [int(x) for x in cu_padded]
    B = len(cu_p) - 1
    docs = range(B) if docs is None else docs
    dq = np.full((S, Hq, D), np.nan)
    dk = np.full((T, Hkv, D), np.nan)
    dv = np.full((T, Hkv, D), np.nan)
    doc_of = token_map(cu_padded, cu_actual)[0][np.asarray(idx, dtype=np.int64)]
    hsel = np.array([kv_heads is None or h // G in kv_heads for h in range(Hq)])
    gsel = np.array([kv_heads is None or g in kv_heads for g in range(Hkv)])
    rsel = np.ones(S, dtype=bool)
    if rows is not None:
        rsel = np.zeros(S, dtype=bool)
        rsel[np.asarray(rows, dtype=np.int64)] = True
    ksel = np.ones(T, dtype=bool)
    if keys is not None:
        ksel = np.zeros(T, dtype=bool)
        ksel[np.asarray(keys, dtype=np.int64)] = True
    for d in docs:
        dq[np.ix_((doc_of == d) & rsel, hsel)] = 0.0
        slot = np.zeros(T, dtype=bool)
        slot[cu_p[d]:cu_p[d + 1]] = True
        dk[np.ix_(slot & ksel, gsel)] = 0.0
        dv[np.ix_(slot & ksel, gsel)] = 0.0
    for d, drows, qpos, start, a in _doc_rows(idx, cu_padded, cu_actual, docs):
        kpos = np.arange(a)
        kk = np.nonzero(ksel[start:start + a])[0]      # the requested keys among the document's actual keys
        # the rows whose results are requested (dQ) or that see a requested key (dK, dV); no other row
        # contributes to a requested output
        need = rsel[drows] | (qpos >= (kk[0] if kk.size else a))
        drows, qpos = drows[need], qpos[need]
        if drows.size == 0:
            continue
        for h in range(Hq):
            g = h // G
            if kv_heads is not None and g not in kv_heads:
                continue
            kd = k[start:start + a, g]
            vd = v[start:start + a, g]
            for b0 in range(0, drows.size, _ROW_BLOCK):
                r = drows[b0:b0 + _ROW_BLOCK]
                allowed = kpos[None, :] <= qpos[b0:b0 + _ROW_BLOCK, None]
                s = scale * (q_local[r, h] @ kd.T)
                s = np.where(allowed, s, -np.inf)
                m = s.max(axis=1)
                e = np.exp(s - m[:, None])
                p = e / e.sum(axis=1)[:, None]              # softmax over allowed keys
                o = p @ vd
                dout = do_local[r, h]
                delta = np.sum(dout * o, axis=1)             # rowsum(dO * O) = rowsum(P * dP)
                rq = rsel[r]
                if rq.all() or kk.size == a:                 # dL/dS of the whole block serves both
                    ds = p * (dout @ vd.T - delta[:, None])
                    ds_r, ds_k, p_k = ds[rq], ds[:, kk], p[:, kk]
                else:                                        # the requested rows over all keys, every row at
                    ds_r = p[rq] * (dout[rq] @ vd.T - delta[rq, None])       # the requested keys
                    ds_k, p_k = p[:, kk] * (dout @ vd[kk].T - delta[:, None]), p[:, kk]
                if rq.any():
                    dq[r[rq], h] = scale * (ds_r @ kd)
                if kk.size:
                    dk[start + kk, g] += scale * (ds_k.T @ q_local[r, h])
                    dv[start + kk, g] += p_k.T @ dout
    return dq, dk, dv

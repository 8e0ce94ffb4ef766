"""ctypes front end of the fp64 attention oracle (``fa_oracle.c``): the three-pass forward and the
chain-rule gradients.

Test infrastructure only. See ``fa_oracle.c`` for the definition it computes
and the passages it follows ("FlashAttention tiles exact softmax without
materializing the score matrix", opening definition; "transformer math: flash
attention math", sections "What we must compute..." and "Safe softmax").
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        lib.fa_oracle_fwd.restype = ctypes.c_int
        lib.fa_oracle_fwd.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
        ]
        lib.fa_oracle_fwd_masked.restype = ctypes.c_int
        lib.fa_oracle_fwd_masked.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
        ]
        lib.fa_oracle_fwd_blocksparse.restype = ctypes.c_int
        lib.fa_oracle_fwd_blocksparse.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_int64,
        ]
        lib.fa_oracle_bwd.restype = ctypes.c_int
        lib.fa_oracle_bwd.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
        ]
        lib.fa_oracle_bwd_masked.restype = ctypes.c_int
        lib.fa_oracle_bwd_masked.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
        ]
        lib.fa_oracle_bwd_blocksparse.restype = ctypes.c_int
        lib.fa_oracle_bwd_blocksparse.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
        ]
        lib.fa_oracle_threads.restype = ctypes.c_int
        lib.fa_oracle_threads.argtypes = []
        _lib = lib
    return _lib


def threads() -> int:
    """OpenMP threads the oracle runs on."""
    return int(_load().fa_oracle_threads())


def attention(q, k, v, scale, causal=False, rows=None):
    """Exact attention in fp64.

    q, k, v : array-likes of shape [B, H, N, d] (converted to contiguous fp64;
              fp16/bf16 inputs convert exactly).
    scale   : the logit multiplier, as a Python float (pass the exact value the
              GPU receives, e.g. ``float(np.float32(1/sqrt(d)))``).
    causal  : key j is excluded for j > i.
    rows    : None for every query row, else an int array [B*H, R] of row
              indices per (batch, head).
    Returns (o, lse): o [B,H,N,d] and lse [B,H,N] (rows=None), or
    o [B*H,R,d] and lse [B*H,R].
    """
    q = np.ascontiguousarray(np.asarray(q, dtype=np.float64))
    k = np.ascontiguousarray(np.asarray(k, dtype=np.float64))
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError(f"q, k, v must share one [B,H,N,d] shape, got {q.shape} {k.shape} {v.shape}")
    B, H, N, d = q.shape
    if rows is None:
        o = np.empty((B, H, N, d), dtype=np.float64)
        lse = np.empty((B, H, N), dtype=np.float64)
        rows_p, n_rows = None, 0
    else:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        if rows.ndim != 2 or rows.shape[0] != B * H:
            raise ValueError(f"rows must be [B*H, R], got {rows.shape}")
        n_rows = rows.shape[1]
        o = np.empty((B * H, n_rows, d), dtype=np.float64)
        lse = np.empty((B * H, n_rows), dtype=np.float64)
        rows_p = rows.ctypes.data
    rc = _load().fa_oracle_fwd(q.ctypes.data, k.ctypes.data, v.ctypes.data, o.ctypes.data, lse.ctypes.data,
                               B, H, N, d, float(scale), int(bool(causal)), rows_p, n_rows)
    if rc != 0:
        raise RuntimeError(f"fa_oracle_fwd failed with code {rc}")
    return o, lse


def _index_list(idx, G, name):
    if idx is None:
        return None, 0, None
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int64))
    if idx.ndim != 2 or idx.shape[0] != G:
        raise ValueError(f"{name} must be [G, R] with G = {G} heads, got {idx.shape}")
    return idx, idx.shape[1], idx.ctypes.data


def attention_backward(q, k, v, dout, scale, causal=False, rows=None, keys=None):
    """Gradients of L = sum(dout * o) with respect to q, k, v, in fp64 (``fa_oracle_bwd``).

    q, k, v, dout : array-likes of one shape [..., N, d]; the leading axes are flattened into G
                    heads (fp16/bf16 inputs convert exactly).
    rows          : None for dq of every row, else int [G, R] row indices per head.
    keys          : None for dk, dv of every key, else int [G, C] key indices per head.
    Returns (dq, dk, dv, lse, delta): dq [G, R or N, d], dk and dv [G, C or N, d], lse and delta
    [G, N] (the log-sum-exp of each row's logits and D_i = sum_j a_ij (dout_i . v_j)).
    """
    arrs = [np.ascontiguousarray(np.asarray(t, dtype=np.float64)) for t in (q, k, v, dout)]
    shape = arrs[0].shape
    if len(shape) < 2 or any(a.shape != shape for a in arrs):
        raise ValueError(f"q, k, v, dout must share one [..., N, d] shape, got {[a.shape for a in arrs]}")
    N, d = shape[-2], shape[-1]
    G = int(np.prod(shape[:-2])) if len(shape) > 2 else 1
    q, k, v, dout = (a.reshape(G, N, d) for a in arrs)
    rows, n_rows, rows_p = _index_list(rows, G, "rows")
    keys, n_keys, keys_p = _index_list(keys, G, "keys")
    dq = np.empty((G, n_rows if rows is not None else N, d), dtype=np.float64)
    dk = np.empty((G, n_keys if keys is not None else N, d), dtype=np.float64)
    dv = np.empty_like(dk)
    lse = np.empty((G, N), dtype=np.float64)
    delta = np.empty((G, N), dtype=np.float64)
    rc = _load().fa_oracle_bwd(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
                               dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, lse.ctypes.data, delta.ctypes.data,
                               G, N, d, float(scale), int(bool(causal)), rows_p, n_rows, keys_p, n_keys)
    if rc != 0:
        raise RuntimeError(f"fa_oracle_bwd failed with code {rc}")
    return dq, dk, dv, lse, delta


def attention_backward_masked(q, k, v, dout, scale, window_left=-1, window_right=-1, seqlens_k=None, rows=None,
                              keys=None):
    """Gradients of L = sum(dout * o) under the mask of ``attention_masked``, in fp64
    (``fa_oracle_bwd_masked``). q, k, v, dout : [B, H, N, d]; rows / keys : None or int [B*H, R].
    Returns (dq, dk, dv, lse, delta) shaped as ``attention_backward``'s with G = B*H. A row with no
    allowed key has lse = -inf, delta = 0 and dq = 0; a key no row allows has dk = dv = 0."""
    arrs = [np.ascontiguousarray(np.asarray(t, dtype=np.float64)) for t in (q, k, v, dout)]
    shape = arrs[0].shape
    if len(shape) != 4 or any(a.shape != shape for a in arrs):
        raise ValueError(f"q, k, v, dout must share one [B,H,N,d] shape, got {[a.shape for a in arrs]}")
    B, H, N, d = shape
    G = B * H
    q, k, v, dout = (a.reshape(G, N, d) for a in arrs)
    sl = None
    if seqlens_k is not None:
        sl = np.ascontiguousarray(np.asarray(seqlens_k, dtype=np.int64))
        if sl.shape != (B,):
            raise ValueError(f"seqlens_k must be [B], got {sl.shape}")
    rows, n_rows, rows_p = _index_list(rows, G, "rows")
    keys, n_keys, keys_p = _index_list(keys, G, "keys")
    dq = np.empty((G, n_rows if rows is not None else N, d), dtype=np.float64)
    dk = np.empty((G, n_keys if keys is not None else N, d), dtype=np.float64)
    dv = np.empty_like(dk)
    lse = np.empty((G, N), dtype=np.float64)
    delta = np.empty((G, N), dtype=np.float64)
    rc = _load().fa_oracle_bwd_masked(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
                                      dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, lse.ctypes.data,
                                      delta.ctypes.data, B, H, N, d, float(scale), int(window_left),
                                      int(window_right), sl.ctypes.data if sl is not None else None,
                                      rows_p, n_rows, keys_p, n_keys)
    if rc != 0:
        raise RuntimeError(f"fa_oracle_bwd_masked failed with code {rc}")
    return dq, dk, dv, lse, delta


def attention_backward_blocksparse(q, k, v, dout, scale, block_mask, block_q, block_k, window_left=-1,
                                   window_right=-1, seqlens_k=None, rows=None, keys=None):
    """Gradients of L = sum(dout * o) under the block mask of ``attention_blocksparse`` (on top of
    the window / key-length mask), in fp64 (``fa_oracle_bwd_blocksparse``). Shapes and results as
    ``attention_backward_masked``; ``block_mask`` as in ``block_mask_strides``."""
    arrs = [np.ascontiguousarray(np.asarray(t, dtype=np.float64)) for t in (q, k, v, dout)]
    shape = arrs[0].shape
    if len(shape) != 4 or any(a.shape != shape for a in arrs):
        raise ValueError(f"q, k, v, dout must share one [B,H,N,d] shape, got {[a.shape for a in arrs]}")
    B, H, N, d = shape
    if block_q < 1 or block_k < 1:
        raise ValueError("block sizes must be >= 1")
    bm, sb, sh = block_mask_strides(block_mask, B, H, N, block_q, block_k)
    G = B * H
    q, k, v, dout = (a.reshape(G, N, d) for a in arrs)
    sl = None
    if seqlens_k is not None:
        sl = np.ascontiguousarray(np.asarray(seqlens_k, dtype=np.int64))
        if sl.shape != (B,):
            raise ValueError(f"seqlens_k must be [B], got {sl.shape}")
    rows, n_rows, rows_p = _index_list(rows, G, "rows")
    keys, n_keys, keys_p = _index_list(keys, G, "keys")
    dq = np.empty((G, n_rows if rows is not None else N, d), dtype=np.float64)
    dk = np.empty((G, n_keys if keys is not None else N, d), dtype=np.float64)
    dv = np.empty_like(dk)
    lse = np.empty((G, N), dtype=np.float64)
    delta = np.empty((G, N), dtype=np.float64)
    rc = _load().fa_oracle_bwd_blocksparse(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
                                           dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, lse.ctypes.data,
                                           delta.ctypes.data, B, H, N, d, float(scale), int(window_left),
                                           int(window_right), sl.ctypes.data if sl is not None else None,
                                           bm.ctypes.data, int(block_q), int(block_k), sb, sh,
                                           rows_p, n_rows, keys_p, n_keys)
    if rc != 0:
        raise RuntimeError(f"fa_oracle_bwd_blocksparse failed with code {rc}")
    return dq, dk, dv, lse, delta


def attention_masked(q, k, v, scale, window_left=-1, window_right=-1, seqlens_k=None, rows=None):
    """Exact attention in fp64 under a general mask (``fa_oracle_fwd_masked``): key j is allowed
    for query i when j >= i - window_left (window_left >= 0), j <= i + window_right
    (window_right >= 0) and j < seqlens_k[b] (seqlens_k given). A row with no allowed key gets
    o = 0 and lse = -inf. Shapes and ``rows`` as for ``attention``."""
    q = np.ascontiguousarray(np.asarray(q, dtype=np.float64))
    k = np.ascontiguousarray(np.asarray(k, dtype=np.float64))
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError(f"q, k, v must share one [B,H,N,d] shape, got {q.shape} {k.shape} {v.shape}")
    B, H, N, d = q.shape
    sl = None
    if seqlens_k is not None:
        sl = np.ascontiguousarray(np.asarray(seqlens_k, dtype=np.int64))
        if sl.shape != (B,):
            raise ValueError(f"seqlens_k must be [B], got {sl.shape}")
    if rows is None:
        o = np.empty((B, H, N, d))
        lse = np.empty((B, H, N))
        rows_p, n_rows = None, 0
    else:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        if rows.ndim != 2 or rows.shape[0] != B * H:
            raise ValueError(f"rows must be [B*H, R], got {rows.shape}")
        n_rows = rows.shape[1]
        o = np.empty((B * H, n_rows, d))
        lse = np.empty((B * H, n_rows))
        rows_p = rows.ctypes.data
    rc = _load().fa_oracle_fwd_masked(q.ctypes.data, k.ctypes.data, v.ctypes.data, o.ctypes.data, lse.ctypes.data,
                                      B, H, N, d, float(scale), int(window_left), int(window_right),
                                      sl.ctypes.data if sl is not None else None, rows_p, n_rows)
    if rc != 0:
        raise RuntimeError(f"fa_oracle_fwd_masked failed with code {rc}")
    return o, lse


def block_mask_strides(mask, B, H, N, block_q, block_k):
    """(contiguous uint8 mask, stride_b, stride_h) for a block mask of shape [n_qb, n_kb] (one
    for every head), [H, n_qb, n_kb] (one per head, shared over the batch) or
    [B, H, n_qb, n_kb], with n_qb = ceil(N / block_q) and n_kb = ceil(N / block_k)."""
    mask = np.ascontiguousarray(np.asarray(mask) != 0, dtype=np.uint8)
    n_qb, n_kb = -(-N // block_q), -(-N // block_k)
    per = n_qb * n_kb
    if mask.shape == (n_qb, n_kb):
        return mask, 0, 0
    if mask.shape == (H, n_qb, n_kb):
        return mask, 0, per
    if mask.shape == (B, H, n_qb, n_kb):
        return mask, H * per, per
    raise ValueError(f"block mask must be [{n_qb},{n_kb}], [H,{n_qb},{n_kb}] or [B,H,{n_qb},{n_kb}], "
                     f"got {mask.shape}")


def attention_blocksparse(q, k, v, scale, block_mask, block_q, block_k, window_left=-1, window_right=-1,
                          seqlens_k=None, rows=None):
    """Exact attention in fp64 under a mask over blocks of the score matrix
    (``fa_oracle_fwd_blocksparse``): the pair (i, j) is allowed when the mask byte of query block
    i // block_q and key block j // block_k is non-zero and the general mask of
    ``attention_masked`` allows it. ``block_mask`` as in ``block_mask_strides``. A row with no
    allowed key gets o = 0 and lse = -inf. Shapes and ``rows`` as for ``attention``."""
    q = np.ascontiguousarray(np.asarray(q, dtype=np.float64))
    k = np.ascontiguousarray(np.asarray(k, dtype=np.float64))
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError(f"q, k, v must share one [B,H,N,d] shape, got {q.shape} {k.shape} {v.shape}")
    B, H, N, d = q.shape
    if block_q < 1 or block_k < 1:
        raise ValueError("block sizes must be >= 1")
    bm, sb, sh = block_mask_strides(block_mask, B, H, N, block_q, block_k)
    sl = None
    if seqlens_k is not None:
        sl = np.ascontiguousarray(np.asarray(seqlens_k, dtype=np.int64))
        if sl.shape != (B,):
            raise ValueError(f"seqlens_k must be [B], got {sl.shape}")
    if rows is None:
        o = np.empty((B, H, N, d))
        lse = np.empty((B, H, N))
        rows_p, n_rows = None, 0
    else:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        if rows.ndim != 2 or rows.shape[0] != B * H:
            raise ValueError(f"rows must be [B*H, R], got {rows.shape}")
        n_rows = rows.shape[1]
        o = np.empty((B * H, n_rows, d))
        lse = np.empty((B * H, n_rows))
        rows_p = rows.ctypes.data
    rc = _load().fa_oracle_fwd_blocksparse(q.ctypes.data, k.ctypes.data, v.ctypes.data, o.ctypes.data,
                                           lse.ctypes.data, B, H, N, d, float(scale), int(window_left),
                                           int(window_right), sl.ctypes.data if sl is not None else None,
                                           bm.ctypes.data, int(block_q), int(block_k), sb, sh, rows_p, n_rows)
    if rc != 0:
        raise RuntimeError(f"fa_oracle_fwd_blocksparse failed with code {rc}")
    return o, lse

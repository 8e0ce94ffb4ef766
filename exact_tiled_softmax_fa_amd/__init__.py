"""Exact tiled-softmax attention on MI355X (gfx950): Python binding.

A thin ctypes layer over the C ABI declared in ``include/fa_fwd.h`` and
``include/fa_bwd.h`` (``libfa_fwd.so``, built from ``csrc/fa_fwd.hip`` and
``csrc/fa_bwd.hip``). It only marshals arguments: shapes, dtypes, device
pointers and torch's current HIP stream. Every step of the computation runs in
the HIP kernels. PyTorch supplies device memory and streams.

    o, lse = forward(q, k, v, causal=False, scale=None)
    dq, dk, dv = backward(q, k, v, o, lse, dout, causal=False, scale=None)
    o, lse = forward_cpu(q_cpu, k_cpu, v_cpu, causal=False)   # the host-CPU variant (fa_cpu.h)

q, k, v: contiguous CUDA (HIP) tensors [B, H, N, d], float16 or bfloat16,
d in {64, 128}. forward returns o (same shape and dtype) and lse ([B, H, N]
float32, natural log of each row's softmax denominator); backward returns the
gradients of a loss L with respect to q, k, v given dout = dL/do. There is no
CPU fallback: if the library is missing or the tensors are not on the GPU, the
call raises.
"""
import ctypes
import math
import os

import torch

from . import build as _build

FA_F16 = 0
FA_BF16 = 1
_DTYPES = {torch.float16: FA_F16, torch.bfloat16: FA_BF16}

_lib = None


class FaOptions(ctypes.Structure):
    """Mirror of fa_fwd_options in include/fa_fwd.h."""
    _fields_ = [("rescale_threshold_log2", ctypes.c_float), ("variant", ctypes.c_int)]


class FaMask(ctypes.Structure):
    """Mirror of fa_mask in include/fa_fwd.h."""
    _fields_ = [("window_left", ctypes.c_int64), ("window_right", ctypes.c_int64), ("seqlens_k", ctypes.c_void_p)]


class FaBlockMask(ctypes.Structure):
    """Mirror of fa_block_mask in include/fa_fwd.h."""
    _fields_ = [("mask", ctypes.c_void_p), ("block_q", ctypes.c_int64), ("block_k", ctypes.c_int64),
                ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64)]


class FaError(RuntimeError):
    """A non-zero status returned by the C library."""

    def __init__(self, status: int, message: str):
        super().__init__(f"fa call failed with status {status}: {message}")
        self.status = status


def library_path() -> str:
    return _build.LIB


def lib():
    """The loaded C library. Loaded after torch so that it binds to the HIP runtime
    torch already has in the process (both carry the soname libamdhip64.so.7)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            raise ImportError(
                f"{_build.LIB} is not built; run `python -m exact_tiled_softmax_fa_amd.build` "
                "(or __graft_entry__.build()) first. There is no fallback path.")
        L = ctypes.CDLL(_build.LIB)
        L.fa_fwd.restype = ctypes.c_int
        L.fa_fwd.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
        ]
        L.fa_fwd_ex.restype = ctypes.c_int
        L.fa_fwd_ex.argtypes = L.fa_fwd.argtypes + [ctypes.POINTER(FaOptions)]
        L.fa_fwd_masked.restype = ctypes.c_int
        L.fa_fwd_masked.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 4 + [
            ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(FaMask)]
        L.fa_fwd_blocksparse.restype = ctypes.c_int
        L.fa_fwd_blocksparse.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 4 + [
            ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(FaMask), ctypes.POINTER(FaBlockMask)]
        L.fa_fwd_splitkv.restype = ctypes.c_int
        L.fa_fwd_splitkv.argtypes = L.fa_fwd.argtypes + [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t]
        L.fa_fwd_splitkv_noalloc.restype = ctypes.c_int
        L.fa_fwd_splitkv_noalloc.argtypes = L.fa_fwd.argtypes + [ctypes.c_int]
        L.fa_fwd_splitkv_masked.restype = ctypes.c_int
        L.fa_fwd_splitkv_masked.argtypes = L.fa_fwd_masked.argtypes + [ctypes.c_int, ctypes.c_void_p,
                                                                        ctypes.c_size_t]
        L.fa_fwd_splitkv_blocksparse.restype = ctypes.c_int
        L.fa_fwd_splitkv_blocksparse.argtypes = L.fa_fwd_blocksparse.argtypes + [ctypes.c_int, ctypes.c_void_p,
                                                                                  ctypes.c_size_t]
        L.fa_fwd_splitkv_workspace_size.restype = ctypes.c_size_t
        L.fa_fwd_splitkv_workspace_size.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int]
        L.fa_fwd_splitkv_heuristic.restype = ctypes.c_int
        L.fa_fwd_splitkv_heuristic.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int]
        L.fa_fwd_cpu.restype = ctypes.c_int
        L.fa_fwd_cpu.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 4 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.fa_bwd_masked.restype = ctypes.c_int
        L.fa_bwd_masked.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int64] * 4 + [
            ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(FaMask)]
        L.fa_bwd_blocksparse.restype = ctypes.c_int
        L.fa_bwd_blocksparse.argtypes = L.fa_bwd_masked.argtypes + [ctypes.POINTER(FaBlockMask)]
        L.fa_bwd.restype = ctypes.c_int
        L.fa_bwd.argtypes = [ctypes.c_void_p] * 10 + [
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
        ]
        L.fa_status_string.restype = ctypes.c_char_p
        L.fa_status_string.argtypes = [ctypes.c_int]
        L.fa_version.restype = ctypes.c_int
        L.fa_version.argtypes = []
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().fa_status_string(int(status)).decode()


def default_scale(d: int) -> float:
    """fp32 value of 1/sqrt(d)."""
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32).item())


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream, dtype, options=None) -> int:
    """Raw call of the C entry point with integer pointers; returns the status code.
    options: None (fa_fwd) or an FaOptions (fa_fwd_ex)."""
    if options is None:
        return int(lib().fa_fwd(q, k, v, o, lse, B, H, N, d, float(scale), int(causal), stream, int(dtype)))
    return int(lib().fa_fwd_ex(q, k, v, o, lse, B, H, N, d, float(scale), int(causal), stream, int(dtype),
                               ctypes.byref(options)))


def fa_fwd_splitkv(q, k, v, o, lse, B, H, N, d, scale, causal, stream, dtype, num_splits, workspace,
                   workspace_bytes) -> int:
    """Raw call of the C entry point fa_fwd_splitkv; returns the status code."""
    return int(lib().fa_fwd_splitkv(q, k, v, o, lse, B, H, N, d, float(scale), int(causal), stream, int(dtype),
                                    int(num_splits), workspace, int(workspace_bytes)))


def fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, N, d, scale, causal, stream, dtype, num_splits) -> int:
    """Raw call of the C entry point fa_fwd_splitkv_noalloc (no workspace: the library's fixed
    scratch); returns the status code."""
    return int(lib().fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, N, d, float(scale), int(causal), stream,
                                            int(dtype), int(num_splits)))


def splitkv_workspace_size(B, H, N, d, num_splits) -> int:
    return int(lib().fa_fwd_splitkv_workspace_size(B, H, N, d, int(num_splits)))


def splitkv_heuristic(B, H, N, d, causal) -> int:
    return int(lib().fa_fwd_splitkv_heuristic(B, H, N, d, int(bool(causal))))


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False, scale=None,
            out: torch.Tensor = None, lse: torch.Tensor = None, return_lse: bool = True,
            rescale_threshold_log2=None, variant: int = 0, num_splits=None, workspace: torch.Tensor = None):
    """Attention forward on the current stream of q's device. See the module docstring.

    rescale_threshold_log2 / variant: the fa_fwd_options of include/fa_fwd.h (None and 0 keep the
    library defaults, i.e. plain fa_fwd).
    num_splits: None for fa_fwd / fa_fwd_ex; an int runs fa_fwd_splitkv with that many key splits
    (0: the library's heuristic). workspace: a device tensor of at least
    splitkv_workspace_size(...) bytes; allocated here when not given."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, d], got shape {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.shape != k.shape or q.shape != v.shape:
        raise ValueError(f"q, k, v shapes differ: {tuple(q.shape)} {tuple(k.shape)} {tuple(v.shape)}")
    if q.dtype != k.dtype or q.dtype != v.dtype or q.dtype not in _DTYPES:
        raise ValueError(f"q, k, v must all be float16 or all bfloat16, got {q.dtype} {k.dtype} {v.dtype}")
    if q.device != k.device or q.device != v.device:
        raise ValueError("q, k, v must be on one device")
    B, H, N, d = q.shape
    if scale is None:
        scale = default_scale(d)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    if return_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous()
                            or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 tensor [B, H, N] on q's device")
    if num_splits is not None:
        if rescale_threshold_log2 is not None or variant != 0:
            raise ValueError("num_splits cannot be combined with rescale_threshold_log2 or variant")
        if num_splits == 0:
            num_splits = splitkv_heuristic(B, H, N, d, causal)
        need = splitkv_workspace_size(B, H, N, d, num_splits)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        elif not workspace.is_cuda or workspace.device != q.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on q's device")
        with torch.cuda.device(q.device):
            stream = torch.cuda.current_stream(q.device).cuda_stream
            st = fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                lse.data_ptr() if lse is not None else None, B, H, N, d, scale, causal, stream,
                                _DTYPES[q.dtype], num_splits, workspace.data_ptr(),
                                workspace.numel() * workspace.element_size())
        if st != 0:
            raise FaError(st, status_string(st))
        return (out, lse) if return_lse else out
    options = None
    if rescale_threshold_log2 is not None or variant != 0:
        options = FaOptions(8.0 if rescale_threshold_log2 is None else float(rescale_threshold_log2), int(variant))
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                    lse.data_ptr() if lse is not None else None,
                    B, H, N, d, scale, causal, stream, _DTYPES[q.dtype], options)
    if st != 0:
        raise FaError(st, status_string(st))
    return (out, lse) if return_lse else out


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, scale, causal, stream, dtype) -> int:
    """Raw call of the C entry point fa_bwd with integer pointers; returns the status code."""
    return int(lib().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, float(scale), int(causal),
                            stream, int(dtype)))


def _check_like(name, t, ref, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.shape != (ref.shape if shape is None else shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(ref.shape if shape is None else shape)}")
    if t.dtype != (ref.dtype if dtype is None else dtype):
        raise ValueError(f"{name} has dtype {t.dtype}")
    if not t.is_contiguous() or t.device != ref.device:
        raise ValueError(f"{name} must be contiguous and on {ref.device}")


def _backward_args(q, k, v, o, lse, dout, dq, dk, dv, delta):
    """Checks shared by backward and backward_masked; allocates the outputs not given."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, d], got shape {tuple(t.shape)}")
    if q.dtype not in _DTYPES:
        raise ValueError(f"q must be float16 or bfloat16, got {q.dtype}")
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_like(name, t, q)
    _check_like("q", q, q)
    _check_like("lse", lse, q, torch.float32, (B, H, N))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if delta is None else delta
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_like(name, t, q)
    _check_like("delta", delta, q, torch.float32, (B, H, N))
    return B, H, N, d, dq, dk, dv, delta


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
             dout: torch.Tensor, causal: bool = False, scale=None, dq=None, dk=None, dv=None, delta=None,
             return_delta: bool = False):
    """Gradients (dq, dk, dv) of a loss L with respect to q, k, v, given dout = dL/do and the
    forward's o and lse (same q, k, v, causal and scale). Runs on the current stream of q's device.
    delta ([B, H, N] float32, receives dout_i . o_i) is allocated if not given; with
    return_delta=True it is returned as a fourth value."""
    B, H, N, d, dq, dk, dv, delta = _backward_args(q, k, v, o, lse, dout, dq, dk, dv, delta)
    if scale is None:
        scale = default_scale(d)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                    dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), B, H, N, d, scale, causal,
                    stream, _DTYPES[q.dtype])
    if st != 0:
        raise FaError(st, status_string(st))
    return (dq, dk, dv, delta) if return_delta else (dq, dk, dv)


def fa_bwd_masked(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, scale, stream, dtype, mask) -> int:
    """Raw call of the C entry point fa_bwd_masked (mask: an FaMask or None); returns the status."""
    return int(lib().fa_bwd_masked(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, float(scale), stream,
                                   int(dtype), ctypes.byref(mask) if mask is not None else None))


def backward_masked(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                    dout: torch.Tensor, window_left: int = -1, window_right: int = -1,
                    seqlens_k: torch.Tensor = None, scale=None, dq=None, dk=None, dv=None, delta=None,
                    return_delta: bool = False):
    """Gradients under the mask of forward_masked (window_left / window_right / seqlens_k as there),
    given the o and lse forward_masked returned with that mask. Rows with no allowed key get
    dq = 0; keys no row allows get dk = dv = 0. Otherwise as backward."""
    B, H, N, d, dq, dk, dv, delta = _backward_args(q, k, v, o, lse, dout, dq, dk, dv, delta)
    _check_seqlens(seqlens_k, q)
    if scale is None:
        scale = default_scale(d)
    mask = FaMask(int(window_left), int(window_right), seqlens_k.data_ptr() if seqlens_k is not None else None)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = fa_bwd_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                           dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), B, H, N, d, scale, stream,
                           _DTYPES[q.dtype], mask)
    if st != 0:
        raise FaError(st, status_string(st))
    return (dq, dk, dv, delta) if return_delta else (dq, dk, dv)


def _check_seqlens(seqlens_k, q):
    if seqlens_k is not None and (not seqlens_k.is_cuda or seqlens_k.dtype != torch.int32
                                  or seqlens_k.shape != (q.shape[0],) or not seqlens_k.is_contiguous()
                                  or seqlens_k.device != q.device):
        raise ValueError("seqlens_k must be a contiguous int32 GPU tensor [B] on q's device")


def _block_mask_arg(block_mask, block_q, block_k, q) -> "FaBlockMask":
    """The FaBlockMask of a [n_qb, n_kb], [H, n_qb, n_kb] or [B, H, n_qb, n_kb] byte mask."""
    B, H, N, _ = q.shape
    if block_q < 1 or block_k < 1:
        raise ValueError("block sizes must be positive")
    n_qb, n_kb = -(-N // block_q), -(-N // block_k)
    if (not isinstance(block_mask, torch.Tensor) or not block_mask.is_cuda or block_mask.device != q.device
            or block_mask.dtype not in (torch.uint8, torch.bool) or not block_mask.is_contiguous()):
        raise ValueError("block_mask must be a contiguous uint8 or bool GPU tensor on q's device")
    per = n_qb * n_kb
    shapes = {(n_qb, n_kb): (0, 0), (H, n_qb, n_kb): (0, per), (B, H, n_qb, n_kb): (H * per, per)}
    if tuple(block_mask.shape) not in shapes:
        raise ValueError(f"block_mask must be [{n_qb},{n_kb}], [H,{n_qb},{n_kb}] or [B,H,{n_qb},{n_kb}], "
                         f"got {tuple(block_mask.shape)}")
    stride_b, stride_h = shapes[tuple(block_mask.shape)]
    return FaBlockMask(block_mask.data_ptr(), int(block_q), int(block_k), stride_b, stride_h)


def fa_bwd_blocksparse(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, scale, stream, dtype, mask,
                       blocks) -> int:
    """Raw call of the C entry point fa_bwd_blocksparse (mask: an FaMask or None; blocks: an
    FaBlockMask or None); returns the status code."""
    return int(lib().fa_bwd_blocksparse(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, float(scale), stream,
                                        int(dtype), ctypes.byref(mask) if mask is not None else None,
                                        ctypes.byref(blocks) if blocks is not None else None))


def backward_blocksparse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                         dout: torch.Tensor, block_mask: torch.Tensor, block_q: int, block_k: int,
                         window_left: int = -1, window_right: int = -1, seqlens_k: torch.Tensor = None, scale=None,
                         dq=None, dk=None, dv=None, delta=None, return_delta: bool = False):
    """Gradients under the masks of forward_blocksparse (block_mask, block_q, block_k, window_left,
    window_right, seqlens_k as there), given the o and lse forward_blocksparse returned with those
    masks. Rows with no allowed key get dq = 0; keys no row allows get dk = dv = 0. Otherwise as
    backward."""
    B, H, N, d, dq, dk, dv, delta = _backward_args(q, k, v, o, lse, dout, dq, dk, dv, delta)
    blocks = _block_mask_arg(block_mask, block_q, block_k, q)
    _check_seqlens(seqlens_k, q)
    if scale is None:
        scale = default_scale(d)
    mask = FaMask(int(window_left), int(window_right), seqlens_k.data_ptr() if seqlens_k is not None else None)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = fa_bwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                                lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), B, H, N,
                                d, scale, stream, _DTYPES[q.dtype], mask, blocks)
    if st != 0:
        raise FaError(st, status_string(st))
    return (dq, dk, dv, delta) if return_delta else (dq, dk, dv)


def fa_fwd_masked(q, k, v, o, lse, B, H, N, d, scale, stream, dtype, mask) -> int:
    """Raw call of the C entry point fa_fwd_masked (mask: an FaMask or None); returns the status."""
    return int(lib().fa_fwd_masked(q, k, v, o, lse, B, H, N, d, float(scale), stream, int(dtype),
                                   ctypes.byref(mask) if mask is not None else None))


def fa_fwd_splitkv_masked(q, k, v, o, lse, B, H, N, d, scale, stream, dtype, mask, num_splits, workspace,
                          workspace_bytes) -> int:
    """Raw call of the C entry point fa_fwd_splitkv_masked (mask: an FaMask or None); returns the
    status code."""
    return int(lib().fa_fwd_splitkv_masked(q, k, v, o, lse, B, H, N, d, float(scale), stream, int(dtype),
                                           ctypes.byref(mask) if mask is not None else None, int(num_splits),
                                           workspace, workspace_bytes))


def forward_masked(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, window_left: int = -1, window_right: int = -1,
                   seqlens_k: torch.Tensor = None, scale=None, out: torch.Tensor = None, lse: torch.Tensor = None,
                   num_splits=None, workspace: torch.Tensor = None):
    """Attention under a general mask (include/fa_fwd.h, fa_mask): key j is allowed for query i when
    j >= i - window_left (window_left >= 0), j <= i + window_right (window_right >= 0) and
    j < seqlens_k[b] (seqlens_k: int32 GPU tensor [B], or None). Returns (o, lse); rows with no
    allowed key get o = 0 and lse = -inf. num_splits (an int) runs fa_fwd_splitkv_masked with that
    many key splits of each query tile's window; workspace as for forward (allocated when not
    given)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor [B, H, N, d]")
    if q.shape != k.shape or q.shape != v.shape or q.dtype != k.dtype or q.dtype != v.dtype or q.dtype not in _DTYPES:
        raise ValueError("q, k, v must share one shape and one of float16 / bfloat16")
    B, H, N, d = q.shape
    _check_seqlens(seqlens_k, q)
    if scale is None:
        scale = default_scale(d)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_like("out", out, q)
    _check_like("lse", lse, q, torch.float32, (B, H, N))
    mask = FaMask(int(window_left), int(window_right), seqlens_k.data_ptr() if seqlens_k is not None else None)
    if num_splits is not None:
        if num_splits < 1:
            raise ValueError("num_splits must be at least 1")
        need = splitkv_workspace_size(B, H, N, d, num_splits)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        elif not workspace.is_cuda or workspace.device != q.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on q's device")
        with torch.cuda.device(q.device):
            stream = torch.cuda.current_stream(q.device).cuda_stream
            st = fa_fwd_splitkv_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H,
                                       N, d, scale, stream, _DTYPES[q.dtype], mask, num_splits, workspace.data_ptr(),
                                       workspace.numel() * workspace.element_size())
        if st != 0:
            raise FaError(st, status_string(st))
        return out, lse
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = fa_fwd_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
                           scale, stream, _DTYPES[q.dtype], mask)
    if st != 0:
        raise FaError(st, status_string(st))
    return out, lse


def fa_fwd_blocksparse(q, k, v, o, lse, B, H, N, d, scale, stream, dtype, mask, blocks) -> int:
    """Raw call of the C entry point fa_fwd_blocksparse (mask: an FaMask or None; blocks: an
    FaBlockMask or None); returns the status code."""
    return int(lib().fa_fwd_blocksparse(q, k, v, o, lse, B, H, N, d, float(scale), stream, int(dtype),
                                        ctypes.byref(mask) if mask is not None else None,
                                        ctypes.byref(blocks) if blocks is not None else None))


def fa_fwd_splitkv_blocksparse(q, k, v, o, lse, B, H, N, d, scale, stream, dtype, mask, blocks, num_splits,
                               workspace, workspace_bytes) -> int:
    """Raw call of the C entry point fa_fwd_splitkv_blocksparse (mask: an FaMask or None; blocks:
    an FaBlockMask or None); returns the status code."""
    return int(lib().fa_fwd_splitkv_blocksparse(q, k, v, o, lse, B, H, N, d, float(scale), stream, int(dtype),
                                                ctypes.byref(mask) if mask is not None else None,
                                                ctypes.byref(blocks) if blocks is not None else None,
                                                int(num_splits), workspace, int(workspace_bytes)))


def forward_blocksparse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_mask: torch.Tensor,
                        block_q: int, block_k: int, window_left: int = -1, window_right: int = -1,
                        seqlens_k: torch.Tensor = None, scale=None, out: torch.Tensor = None,
                        lse: torch.Tensor = None, num_splits=None, workspace: torch.Tensor = None):
    """Block-sparse attention (include/fa_fwd.h, fa_block_mask): the pair (i, j) is allowed when
    block_mask[.., i // block_q, j // block_k] != 0 and the window / key-length mask of
    forward_masked allows it. block_mask: a contiguous uint8 (or bool) GPU tensor of shape
    [n_qb, n_kb] (all heads), [H, n_qb, n_kb] (per head) or [B, H, n_qb, n_kb], with
    n_qb = ceil(N / block_q), n_kb = ceil(N / block_k); block sizes are multiples of 64.
    Returns (o, lse); rows with no allowed key get o = 0 and lse = -inf. num_splits (an int) runs
    fa_fwd_splitkv_blocksparse with that many key splits of each query tile's window; workspace
    as for forward (allocated when not given)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor [B, H, N, d]")
    if q.shape != k.shape or q.shape != v.shape or q.dtype != k.dtype or q.dtype != v.dtype or q.dtype not in _DTYPES:
        raise ValueError("q, k, v must share one shape and one of float16 / bfloat16")
    B, H, N, d = q.shape
    blocks = _block_mask_arg(block_mask, block_q, block_k, q)
    _check_seqlens(seqlens_k, q)
    if scale is None:
        scale = default_scale(d)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_like("out", out, q)
    _check_like("lse", lse, q, torch.float32, (B, H, N))
    mask = FaMask(int(window_left), int(window_right), seqlens_k.data_ptr() if seqlens_k is not None else None)
    if num_splits is not None:
        if num_splits < 1:
            raise ValueError("num_splits must be at least 1")
        need = splitkv_workspace_size(B, H, N, d, num_splits)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        elif not workspace.is_cuda or workspace.device != q.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on q's device")
        with torch.cuda.device(q.device):
            stream = torch.cuda.current_stream(q.device).cuda_stream
            st = fa_fwd_splitkv_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                            B, H, N, d, scale, stream, _DTYPES[q.dtype], mask, blocks, num_splits,
                                            workspace.data_ptr(), workspace.numel() * workspace.element_size())
        if st != 0:
            raise FaError(st, status_string(st))
        return out, lse
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = fa_fwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
                                scale, stream, _DTYPES[q.dtype], mask, blocks)
    if st != 0:
        raise FaError(st, status_string(st))
    return out, lse


def fa_fwd_cpu(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, num_threads) -> int:
    """Raw call of the C entry point fa_fwd_cpu (host pointers); returns the status code."""
    return int(lib().fa_fwd_cpu(q, k, v, o, lse, B, H, N, d, float(scale), int(causal), int(dtype),
                                int(num_threads)))


def forward_cpu(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False, scale=None,
                num_threads: int = 0, out: torch.Tensor = None, lse: torch.Tensor = None):
    """The same attention on the host CPU (include/fa_cpu.h): contiguous CPU tensors [B, H, N, d] of
    float16 or bfloat16. Returns (o, lse). Explicitly a host entry point: the GPU functions above
    never call it."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.is_cuda or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous CPU tensor [B, H, N, d]")
    if q.shape != k.shape or q.shape != v.shape or q.dtype != k.dtype or q.dtype != v.dtype or q.dtype not in _DTYPES:
        raise ValueError("q, k, v must share one shape and one of float16 / bfloat16")
    B, H, N, d = q.shape
    if scale is None:
        scale = default_scale(d)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32) if lse is None else lse
    if out.shape != q.shape or out.dtype != q.dtype or out.is_cuda or not out.is_contiguous():
        raise ValueError("out must be a contiguous CPU tensor like q")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or lse.is_cuda or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 CPU tensor [B, H, N]")
    st = fa_fwd_cpu(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d, scale,
                    causal, _DTYPES[q.dtype], num_threads)
    if st != 0:
        raise FaError(st, status_string(st))
    return out, lse

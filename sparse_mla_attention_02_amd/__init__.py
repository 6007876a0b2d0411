"""Sparse Flash-MLA Softmax-L1Norm on MI355X (gfx950).

Thin Python binding over the C ABI in ``include/smla.h`` (``libsmla.so``,
built in-tree by ``__graft_entry__.build()``). Arguments are only marshalled
here: every step of the operation runs in the library's HIP kernels. PyTorch
supplies device memory and the current stream. There is no CPU fallback: if
the library is missing, importing this package raises.

Names and defaults follow the page's PyTorch API (the
"SparseFlashMlaSoftmaxL1Norm" article, section 调用方式二 PyTorch API):

* :func:`sparse_flash_mla_softmax_l1_norm_metadata` (alias
  :func:`smla_l1norm_metadata`) returns the int32 (64,) metadata on the CPU;
* :func:`sparse_flash_mla_softmax_l1_norm` (alias :func:`smla_softmax_l1norm`)
  returns the fp32 output, (B,S1,N2,S2) or (T1,N2,T2);
* :func:`sparse_flash_mla_softmax_lse` (alias :func:`smla_softmax_lse`) returns
  the forward softmax_lse that the main call consumes, computed on the GPU
  over the same used entries.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # loads the HIP runtime the library binds to

__all__ = [
    "SmlaError", "library_path", "smla_l1norm_metadata", "smla_softmax_l1norm",
    "smla_softmax_lse", "sparse_flash_mla_softmax_l1_norm_metadata",
    "sparse_flash_mla_softmax_l1_norm", "sparse_flash_mla_softmax_lse",
    "output_shape", "smla_check_indices", "SMLA_METADATA_SIZE",
]

SMLA_METADATA_SIZE = 64
SMLA_SUCCESS = 0
SMLA_ERR_PARAM_NULLPTR = 161001
SMLA_ERR_PARAM_INVALID = 161002
SMLA_ERR_UNSUPPORTED = 161101
SMLA_ERR_RUNTIME = 561001

_LAYOUTS = {"BSND": 0, "TND": 1}
_DTYPES = {torch.float16: 0, torch.bfloat16: 1}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIBPATH = os.path.join(_HERE, "libsmla.so")


class SmlaError(RuntimeError):
    """A non-success status from the library (``.status`` holds the code)."""

    def __init__(self, status: int, msg: str):
        super().__init__(f"[{status}] {msg}")
        self.status = status


def library_path() -> str:
    return _LIBPATH


def _load():
    if not os.path.exists(_LIBPATH):
        raise ImportError(f"{_LIBPATH} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(_LIBPATH)
    i64, i32, p, dbl = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_double
    lib.smla_l1norm_metadata.argtypes = [i64, i64, i64, p, p, p, p, p, p, i64, i64, i64, i64,
                                         i32, i32, i64, i64, i32, i32, p]
    lib.smla_l1norm_metadata.restype = i32
    lib.smla_softmax_l1norm.argtypes = [p, p, p, p, p, p, p, p, p, p, p, i32, i64, i64, i64,
                                        i64, i64, i64, i64, dbl, i64, i64, i64, i32, i32, p,
                                        p]
    lib.smla_softmax_l1norm.restype = i32
    lib.smla_softmax_l1norm_kwide.argtypes = lib.smla_softmax_l1norm.argtypes
    lib.smla_softmax_l1norm_kwide.restype = i32
    lib.smla_softmax_lse.argtypes = [p, p, p, p, p, p, p, p, p, p, i32, i64, i64, i64, i64, i64,
                                     i64, i64, dbl, i64, i64, i64, i32, i32, p, p]
    lib.smla_softmax_lse.restype = i32
    lib.smla_output_numel.argtypes = [i32, i64, i64, i64, i64]
    lib.smla_output_numel.restype = i64
    lib.smla_last_error.argtypes = []
    lib.smla_last_error.restype = ctypes.c_char_p
    lib.smla_version.argtypes = []
    lib.smla_version.restype = i32
    lib.smla_check_indices.argtypes = [p, p, i64, i64, ctypes.POINTER(i64)]
    lib.smla_check_indices.restype = i32
    return lib


_lib = _load()


def _check(status: int):
    if status != SMLA_SUCCESS:
        raise SmlaError(status, _lib.smla_last_error().decode(errors="replace"))


def _layout(name: Optional[str]) -> int:
    name = "BSND" if name is None else name
    if name not in _LAYOUTS:
        raise SmlaError(SMLA_ERR_PARAM_INVALID, f"layout must be BSND or TND, got {name!r}")
    return _LAYOUTS[name]


def _host_i32(t) -> Optional[torch.Tensor]:
    if t is None:
        return None
    t = torch.as_tensor(t)
    if t.dtype != torch.int32:
        raise SmlaError(SMLA_ERR_PARAM_INVALID, "index tensors must be int32")
    return t.detach().to("cpu").contiguous()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def smla_check_indices(sparse_indices, topk_length=None) -> None:
    """Check the distinct-entries precondition of the main calls on host
    copies (``smla_check_indices`` of the C ABI): raises ``SmlaError`` naming
    the first row whose used entries (t < topk_length, index >= 0) repeat a
    key. ``sparse_indices`` is int32 with the rows first and K last."""
    idx = _host_i32(sparse_indices)
    K = int(idx.shape[-1]) if idx.dim() else 0
    rows = idx.numel() // K if K else 0
    tl = _host_i32(topk_length)
    if tl is not None and tl.numel() != rows:
        raise SmlaError(SMLA_ERR_PARAM_INVALID, "topk_length must hold one count per row")
    bad = ctypes.c_int64(-1)
    _check(_lib.smla_check_indices(_ptr(idx), _ptr(tl), rows, K, ctypes.byref(bad)))


def sparse_flash_mla_softmax_l1_norm_metadata(
        num_heads_q, num_heads_k, head_dim, *, cu_seqlens_q=None, cu_seqlens_k=None,
        seqused_q=None, seqused_k=None, cmp_residual_k=None, topk_length=None,
        batch_size=None, max_seqlen_q=None, max_seqlen_k=None, topk=None, layout_q=None,
        layout_k=None, mask_mode=None, cmp_ratio=None, device=None,
        core_budget: int = 0) -> torch.Tensor:
    """Plan the work split; returns the int32 (64,) metadata on the CPU.

    ``None`` attributes take the page's defaults (BSND, mask 0, cmp_ratio 1).
    For TND, ``batch_size`` defaults to ``len(cu_seqlens_q) - 1``. Sequence
    tensors may live on the GPU; they are copied to the host.
    ``core_budget`` (not on the page) overrides the number of workgroups to
    split over; 0 takes the device's co-resident capacity.
    """
    lq, lk = _layout(layout_q), _layout(layout_k)
    cq, ck = _host_i32(cu_seqlens_q), _host_i32(cu_seqlens_k)
    sq, sk = _host_i32(seqused_q), _host_i32(seqused_k)
    cr, tl = _host_i32(cmp_residual_k), _host_i32(topk_length)
    if batch_size is None:
        batch_size = (cq.numel() - 1) if cq is not None else 0
    if device is None:
        device = torch.cuda.current_device() if torch.cuda.is_available() else 0
    elif isinstance(device, torch.device):
        device = device.index or 0
    meta = torch.zeros(SMLA_METADATA_SIZE, dtype=torch.int32)
    _check(_lib.smla_l1norm_metadata(
        int(num_heads_q), int(num_heads_k), int(head_dim), _ptr(cq), _ptr(ck), _ptr(sq),
        _ptr(sk), _ptr(cr), _ptr(tl), int(batch_size),
        int(max_seqlen_q or 0), int(max_seqlen_k or 0), int(topk or 0), lq, lk,
        int(mask_mode or 0), int(1 if cmp_ratio is None else cmp_ratio), int(device),
        int(core_budget), _ptr(meta)))
    return meta


def output_shape(q: torch.Tensor, k: torch.Tensor, layout_q: str = "BSND"):
    """(B,S1,N2,S2) for BSND, (T1,N2,T2) for TND (the page's parameter table)."""
    if layout_q == "BSND":
        return (q.shape[0], q.shape[1], k.shape[2], k.shape[1])
    return (q.shape[0], k.shape[1], k.shape[0])


def _dev_i32(t, device, name) -> Optional[torch.Tensor]:
    if t is None:
        return None
    if t.dtype != torch.int32:
        raise SmlaError(SMLA_ERR_PARAM_INVALID, f"{name} must be int32")
    if t.device != device:
        raise SmlaError(SMLA_ERR_PARAM_INVALID, f"{name} must be on {device}")
    return t.contiguous()


class _Call:
    """Checked, contiguous device arguments of one main or lse call."""


def _marshal(q, k, sparse_indices, cu_seqlens_q, cu_seqlens_k, seqused_q, seqused_k,
             cmp_residual_k, topk_length, layout_q, layout_k) -> _Call:
    if q is None or k is None:
        raise SmlaError(SMLA_ERR_PARAM_INVALID, "q and k are required")
    if q.dtype not in _DTYPES or k.dtype != q.dtype:
        raise SmlaError(SMLA_ERR_PARAM_INVALID, "q and k must share dtype fp16 or bf16")
    dev = q.device
    if dev.type != "cuda" or k.device != dev:
        raise SmlaError(SMLA_ERR_PARAM_INVALID, "q and k must be on one GPU")
    c = _Call()
    c.dev = dev
    c.lq, c.lk = _layout(layout_q), _layout(layout_k)
    c.q, c.k = q.contiguous(), k.contiguous()
    c.idx = _dev_i32(sparse_indices, dev, "sparse_indices")
    c.cq = _dev_i32(cu_seqlens_q, dev, "cu_seqlens_q")
    c.ck = _dev_i32(cu_seqlens_k, dev, "cu_seqlens_k")
    c.sq = _dev_i32(seqused_q, dev, "seqused_q")
    c.sk = _dev_i32(seqused_k, dev, "seqused_k")
    c.cr = _dev_i32(cmp_residual_k, dev, "cmp_residual_k")
    c.tl = _dev_i32(topk_length, dev, "topk_length")

    if c.lq == 0:
        if q.dim() != 4 or k.dim() != 4:
            raise SmlaError(SMLA_ERR_PARAM_INVALID, "BSND q and k must be 4-D")
        B, S1, N1, D = q.shape
        _, S2, N2, _ = k.shape
        if k.shape[0] != B or k.shape[3] != D:
            raise SmlaError(SMLA_ERR_PARAM_INVALID, "k's B and D must match q's")
        c.sq_len, c.sk_len = S1, S2
    else:
        if q.dim() != 3 or k.dim() != 3:
            raise SmlaError(SMLA_ERR_PARAM_INVALID, "TND q and k must be 3-D")
        T1, N1, D = q.shape
        T2, N2, _ = k.shape
        if k.shape[2] != D:
            raise SmlaError(SMLA_ERR_PARAM_INVALID, "k's D must match q's")
        B = (c.cq.numel() - 1) if c.cq is not None else 0
        c.sq_len, c.sk_len = T1, T2
    c.B, c.N1, c.N2, c.D = B, N1, N2, D
    c.K = c.idx.shape[-1] if c.idx is not None else 0
    c.out_shape = output_shape(q, k, "BSND" if c.lq == 0 else "TND")
    G = N1 // N2 if N2 else 0
    c.lse_shape = (B, N2, c.sq_len, G) if c.lq == 0 else (N2, c.sq_len, G)
    if c.idx is not None:
        want = (B, c.sq_len, N2, c.K) if c.lq == 0 else (c.sq_len, N2, c.K)
        if tuple(c.idx.shape) != want:
            raise SmlaError(SMLA_ERR_PARAM_INVALID, f"sparse_indices shape != {want}")
    if c.tl is not None:
        want = (B, c.sq_len, N2) if c.lq == 0 else (c.sq_len, N2)
        if tuple(c.tl.shape) != want:
            raise SmlaError(SMLA_ERR_PARAM_INVALID, f"topk_length shape != {want}")
    if c.cr is not None and c.cr.numel() != B:
        raise SmlaError(SMLA_ERR_PARAM_INVALID, "cmp_residual_k must have B elements")
    for t, name in ((c.sq, "seqused_q"), (c.sk, "seqused_k")):
        if t is not None and t.numel() != B:
            raise SmlaError(SMLA_ERR_PARAM_INVALID, f"{name} must have B elements")
    if (c.cq is None) != (c.ck is None) or (c.cq is not None and c.ck.numel() != c.cq.numel()):
        raise SmlaError(SMLA_ERR_PARAM_INVALID, "cu_seqlens_q/k must come as a pair of B+1")
    return c


def _out_tensor(out, shape, dev, what):
    if out is None:
        return torch.empty(shape, dtype=torch.float32, device=dev)
    if (out.dtype != torch.float32 or tuple(out.shape) != tuple(shape)
            or out.device != dev or not out.is_contiguous()):
        raise SmlaError(SMLA_ERR_PARAM_INVALID, f"{what} must be contiguous fp32 of shape {shape}")
    return out


def _metadata(metadata):
    if metadata is None:
        raise SmlaError(SMLA_ERR_PARAM_NULLPTR, "metadata is required")
    metadata = _host_i32(metadata)
    if metadata.numel() != SMLA_METADATA_SIZE:
        raise SmlaError(SMLA_ERR_PARAM_INVALID, "metadata must have 64 elements")
    return metadata


def _tail(c, softmax_scale, max_seqlen_k, cmp_ratio, mask_mode, out):
    stream = torch.cuda.current_stream(c.dev).cuda_stream
    return (_DTYPES[c.q.dtype], int(c.B), int(c.sq_len), int(c.sk_len), int(c.N1), int(c.N2),
            int(c.D), int(c.K), float(softmax_scale), int(max_seqlen_k or 0), int(cmp_ratio),
            int(mask_mode), c.lq, c.lk, _ptr(out), ctypes.c_void_p(stream))


def sparse_flash_mla_softmax_l1_norm(
        q, k, softmax_lse, *, sparse_indices=None, cu_seqlens_q=None, cu_seqlens_k=None,
        seqused_q=None, seqused_k=None, cmp_residual_k=None, topk_length=None,
        metadata=None, softmax_scale=1.0, max_seqlen_k=0, cmp_ratio=1, mask_mode=0,
        layout_q="BSND", layout_k="BSND", out: Optional[torch.Tensor] = None,
        kwide: bool = False) -> torch.Tensor:
    """Softmax-L1Norm: head mean of exp(mask(q.k_sel^T*scale) - lse).

    All tensors must be on the same GPU; they are made contiguous (the page's
    op definition declares AutoContiguous inputs). ``metadata`` (int32 (64,),
    from the metadata call) is required and must be on the CPU. ``out``
    (optional, fp32, contiguous, output shape) receives the result.
    ``kwide`` (not a page argument) selects the K-wide output of the page's
    shape inference: entry t's value at column t of a row of K columns
    (without sparse_indices: S2, or max_seqlen_k for TND).
    Enqueued on the current stream.
    """
    if softmax_lse is None:
        raise SmlaError(SMLA_ERR_PARAM_INVALID, "q, k and softmax_lse are required")
    c = _marshal(q, k, sparse_indices, cu_seqlens_q, cu_seqlens_k, seqused_q, seqused_k,
                 cmp_residual_k, topk_length, layout_q, layout_k)
    if softmax_lse.dtype != torch.float32:
        raise SmlaError(SMLA_ERR_PARAM_INVALID, "softmax_lse must be float32")
    if softmax_lse.device != c.dev:
        raise SmlaError(SMLA_ERR_PARAM_INVALID, "q, k and softmax_lse must be on one GPU")
    softmax_lse = softmax_lse.contiguous()
    if tuple(softmax_lse.shape) != tuple(c.lse_shape):
        raise SmlaError(SMLA_ERR_PARAM_INVALID,
                        f"softmax_lse shape {tuple(softmax_lse.shape)} != {c.lse_shape}")
    shape = c.out_shape
    if kwide:
        w = c.K if c.idx is not None else (c.sk_len if c.lq == 0 else int(max_seqlen_k or 0))
        shape = tuple(shape[:-1]) + (w,)
    out = _out_tensor(out, shape, c.dev, "out")
    if out.numel() == 0:
        return out  # empty q or empty output: nothing to compute
    metadata = _metadata(metadata)
    fn = _lib.smla_softmax_l1norm_kwide if kwide else _lib.smla_softmax_l1norm
    with torch.cuda.device(c.dev):
        _check(fn(
            _ptr(c.q), _ptr(c.k), _ptr(softmax_lse), _ptr(c.idx), _ptr(c.cq), _ptr(c.ck),
            _ptr(c.sq), _ptr(c.sk), _ptr(c.cr), _ptr(c.tl), _ptr(metadata),
            *_tail(c, softmax_scale, max_seqlen_k, cmp_ratio, mask_mode, out)))
    return out


def sparse_flash_mla_softmax_lse(
        q, k, *, sparse_indices=None, cu_seqlens_q=None, cu_seqlens_k=None,
        seqused_q=None, seqused_k=None, cmp_residual_k=None, topk_length=None,
        metadata=None, softmax_scale=1.0, max_seqlen_k=0, cmp_ratio=1, mask_mode=0,
        layout_q="BSND", layout_k="BSND", out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The forward softmax_lse over the same used entries, on the GPU.

    ``lse[row, g] = log sum_{t used} exp(softmax_scale * q[row,g,:].k[key(t),:])``,
    -inf for a row with no used entry; fp32 of shape (B,N2,S1,G) or
    (N2,T1,G), the ``softmax_lse`` input of
    :func:`sparse_flash_mla_softmax_l1_norm`. Takes that call's keyword
    arguments (same metadata). Enqueued on the current stream.
    """
    c = _marshal(q, k, sparse_indices, cu_seqlens_q, cu_seqlens_k, seqused_q, seqused_k,
                 cmp_residual_k, topk_length, layout_q, layout_k)
    out = _out_tensor(out, c.lse_shape, c.dev, "out")
    if out.numel() == 0:
        return out  # empty q: nothing to compute
    metadata = _metadata(metadata)
    with torch.cuda.device(c.dev):
        _check(_lib.smla_softmax_lse(
            _ptr(c.q), _ptr(c.k), _ptr(c.idx), _ptr(c.cq), _ptr(c.ck), _ptr(c.sq), _ptr(c.sk),
            _ptr(c.cr), _ptr(c.tl), _ptr(metadata),
            *_tail(c, softmax_scale, max_seqlen_k, cmp_ratio, mask_mode, out)))
    return out


# Names of the C entry points.
smla_l1norm_metadata = sparse_flash_mla_softmax_l1_norm_metadata
smla_softmax_l1norm = sparse_flash_mla_softmax_l1_norm
smla_softmax_lse = sparse_flash_mla_softmax_lse

"""ctypes binding of libmosaic_bsa (include/mosaic_bsa.h): argument marshalling only.

Every step of the BSA forward pass runs in the library's HIP kernels; this
module checks that the torch tensors have the layout the C ABI documents,
passes their device pointers and torch's current HIP stream, and turns a
non-OK status into MosaicError.  There is no fallback: without the built
library every call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmosaic_bsa.so")

MOSAIC_OK = 0
STATUS_NAMES = {
    0: "MOSAIC_OK", 1: "MOSAIC_ERR_NULL_POINTER", 2: "MOSAIC_ERR_BAD_SHAPE",
    3: "MOSAIC_ERR_UNSUPPORTED", 4: "MOSAIC_ERR_MISALIGNED", 5: "MOSAIC_ERR_WORKSPACE",
    6: "MOSAIC_ERR_HIP",
}

EXPORTED = (
    "mosaic_bsa_abi_version", "mosaic_status_string", "mosaic_last_error",
    "mosaic_bsa_workspace_bytes", "mosaic_bsa_forward", "mosaic_bsa_forward_noalloc", "mosaic_bsa_pool",
    "mosaic_bsa_compress_select", "mosaic_bsa_fine", "mosaic_bsa_select_bound",
    "mosaic_bsa_saved_bytes", "mosaic_bsa_forward_train",
    "mosaic_bsa_layer_workspace_bytes", "mosaic_bsa_layer_forward", "mosaic_bsa_layer_in", "mosaic_bsa_layer_out",
    "mosaic_bsa_layer_out_merged",
    "mosaic_healpix_coarsen", "mosaic_interp_workspace_bytes", "mosaic_interp_attention",
    "mosaic_bsa_backward_workspace_bytes", "mosaic_bsa_backward",
)


class MosaicError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmosaic_bsa.so from the package directory (no search path, no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m spherical_block_sparse_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.mosaic_bsa_abi_version.restype = I
        L.mosaic_bsa_abi_version.argtypes = []
        L.mosaic_status_string.restype = ctypes.c_char_p
        L.mosaic_status_string.argtypes = [I]
        L.mosaic_last_error.restype = ctypes.c_char_p
        L.mosaic_last_error.argtypes = []
        L.mosaic_bsa_workspace_bytes.restype = S
        L.mosaic_bsa_workspace_bytes.argtypes = [I, I, I, I, I, I]
        L.mosaic_bsa_forward.restype = I
        L.mosaic_bsa_forward.argtypes = [P, P, P, P, I, I, I, I, I, I, I, P, P, P, S, P]
        L.mosaic_bsa_forward_noalloc.restype = I
        L.mosaic_bsa_forward_noalloc.argtypes = [P, P, P, P, I, I, I, I, I, I, I, P, P, P]
        L.mosaic_bsa_pool.restype = I
        L.mosaic_bsa_pool.argtypes = [P, P, P, I, I, I, I, I, P, P, P, P, P, P, P]
        L.mosaic_bsa_compress_select.restype = I
        L.mosaic_bsa_compress_select.argtypes = [P, P, P, I, I, I, I, I, I, P, P, P, P, P]
        L.mosaic_bsa_fine.restype = I
        L.mosaic_bsa_fine.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, P, P]
        L.mosaic_bsa_select_bound.restype = I
        L.mosaic_bsa_select_bound.argtypes = [P, P, I, I, I, I, I, I, P, P]
        L.mosaic_bsa_backward_workspace_bytes.restype = S
        L.mosaic_bsa_backward_workspace_bytes.argtypes = [I, I, I, I, I, I]
        L.mosaic_interp_workspace_bytes.restype = S
        L.mosaic_interp_workspace_bytes.argtypes = [I, I]
        L.mosaic_interp_attention.restype = I
        L.mosaic_interp_attention.argtypes = [P, P, P, P, P, I, I, I, I, I, I, P, P, S, P]
        L.mosaic_healpix_coarsen.restype = I
        L.mosaic_healpix_coarsen.argtypes = [P, I, I, I, I, P, P]
        L.mosaic_bsa_layer_workspace_bytes.restype = S
        L.mosaic_bsa_layer_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
        L.mosaic_bsa_layer_forward.restype = I
        L.mosaic_bsa_layer_forward.argtypes = [P, P, P, I, I, I, I, I, I, I, I, P, P, P, S, P]
        L.mosaic_bsa_layer_in.restype = I
        L.mosaic_bsa_layer_in.argtypes = [P, P, I, I, I, I, I, P, P, P, P, P]
        L.mosaic_bsa_layer_out.restype = I
        L.mosaic_bsa_layer_out.argtypes = [P, P, P, I, I, I, I, I, P, P]
        L.mosaic_bsa_layer_out_merged.restype = I
        L.mosaic_bsa_layer_out_merged.argtypes = [P, P, P, I, I, I, I, I, P, P]
        L.mosaic_bsa_saved_bytes.restype = S
        L.mosaic_bsa_saved_bytes.argtypes = [I, I, I, I, I]
        L.mosaic_bsa_forward_train.restype = I
        L.mosaic_bsa_forward_train.argtypes = [P, P, P, P, I, I, I, I, I, I, I, P, P, P, S, P]
        L.mosaic_bsa_backward.restype = I
        L.mosaic_bsa_backward.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, P, S, P, P, P, P, P, S, P]
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != MOSAIC_OK:
        raise MosaicError(status, lib().mosaic_last_error().decode())


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else int(stream)


def _ptr(t: torch.Tensor, dtype: torch.dtype, shape: tuple, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    return t.data_ptr()


def _saved_ptr(saved):
    if saved is None:
        return None
    if not isinstance(saved, torch.Tensor) or saved.dtype != torch.uint8 or saved.dim() != 1 \
            or saved.device.type != "cuda":
        raise ValueError("saved must be the 1-D uint8 device tensor of mosaic_bsa_forward_train")
    return saved.data_ptr()


def _dims(q: torch.Tensor, nside: int):
    if q.dim() != 4:
        raise ValueError("q must be [batch, heads, N, head_dim]")
    b, h, n, d = q.shape
    if n != 12 * nside * nside:
        raise ValueError(f"N = {n} but 12*nside^2 = {12 * nside * nside}")
    return b, h, n, d


def mosaic_bsa_abi_version() -> int:
    return lib().mosaic_bsa_abi_version()


def mosaic_bsa_workspace_bytes(batch, heads, head_dim, nside, block, topn) -> int:
    return lib().mosaic_bsa_workspace_bytes(batch, heads, head_dim, nside, block, topn)


def mosaic_bsa_forward(q, k, v, gates, nside, block, topn, window, out=None, sel_idx=None,
                       workspace=None, stream=None):
    """out [b,H,N,d] fp32 and sel_idx [b,H,m,topn] int32 from bf16 q, k, v and fp32 gates."""
    b, h, n, d = _dims(q, nside)
    m = n // block
    if out is None:
        out = torch.empty((b, h, n, d), dtype=torch.float32, device=q.device)
    if sel_idx is None:
        sel_idx = torch.empty((b, h, m, topn), dtype=torch.int32, device=q.device)
    need = mosaic_bsa_workspace_bytes(b, h, d, nside, block, topn)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if workspace.dtype != torch.uint8 or workspace.dim() != 1 or workspace.device.type != "cuda":
        raise ValueError("workspace must be a 1-D uint8 device tensor")
    _check(lib().mosaic_bsa_forward(
        _ptr(q, torch.bfloat16, (b, h, n, d), "q"), _ptr(k, torch.bfloat16, (b, h, n, d), "k"),
        _ptr(v, torch.bfloat16, (b, h, n, d), "v"), _ptr(gates, torch.float32, (b, h, n, 3), "gates"),
        b, h, d, nside, block, topn, window,
        _ptr(out, torch.float32, (b, h, n, d), "out"),
        _ptr(sel_idx, torch.int32, (b, h, m, topn), "sel_idx"),
        workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return out, sel_idx


def mosaic_bsa_forward_noalloc(q, k, v, gates, nside, block, topn, window, out=None, sel_idx=None, stream=None):
    """mosaic_bsa_forward with the library's static device scratch as the workspace (the C entry point
    allocates nothing; out and sel_idx are allocated here only when not given)."""
    b, h, n, d = _dims(q, nside)
    m = n // block
    if out is None:
        out = torch.empty((b, h, n, d), dtype=torch.float32, device=q.device)
    if sel_idx is None:
        sel_idx = torch.empty((b, h, m, topn), dtype=torch.int32, device=q.device)
    _check(lib().mosaic_bsa_forward_noalloc(
        _ptr(q, torch.bfloat16, (b, h, n, d), "q"), _ptr(k, torch.bfloat16, (b, h, n, d), "k"),
        _ptr(v, torch.bfloat16, (b, h, n, d), "v"), _ptr(gates, torch.float32, (b, h, n, 3), "gates"),
        b, h, d, nside, block, topn, window,
        _ptr(out, torch.float32, (b, h, n, d), "out"),
        _ptr(sel_idx, torch.int32, (b, h, m, topn), "sel_idx"), _stream(stream)))
    return out, sel_idx


def mosaic_bsa_pool(q, k, v, nside, block, qbar=None, kbar=None, vbar=None, knorm=None, kpieces=None,
                    kbn2=None, stream=None):
    """q̄, k̄ (float64) and v̄ (float32), [b,H,m,d]: block means.  knorm, if given (float32
    [b,H,m]), receives each block's largest key norm; kpieces (bf16 [b,H,m,2,d]) and kbn2
    (float32 [b,H,m]), given together, receive k̄'s two bf16 pieces and |k̄_j|^2."""
    b, h, n, d = _dims(q, nside)
    m = n // block
    qbar = torch.empty((b, h, m, d), dtype=torch.float64, device=q.device) if qbar is None else qbar
    kbar = torch.empty((b, h, m, d), dtype=torch.float64, device=q.device) if kbar is None else kbar
    vbar = torch.empty((b, h, m, d), dtype=torch.float32, device=q.device) if vbar is None else vbar
    _check(lib().mosaic_bsa_pool(
        _ptr(q, torch.bfloat16, (b, h, n, d), "q"), _ptr(k, torch.bfloat16, (b, h, n, d), "k"),
        _ptr(v, torch.bfloat16, (b, h, n, d), "v"), b, h, d, nside, block,
        _ptr(qbar, torch.float64, (b, h, m, d), "qbar"), _ptr(kbar, torch.float64, (b, h, m, d), "kbar"),
        _ptr(vbar, torch.float32, (b, h, m, d), "vbar"),
        None if knorm is None else _ptr(knorm, torch.float32, (b, h, m), "knorm"),
        None if kpieces is None else _ptr(kpieces, torch.bfloat16, (b, h, m, 2, d), "kpieces"),
        None if kbn2 is None else _ptr(kbn2, torch.float32, (b, h, m), "kbn2"), _stream(stream)))
    return qbar, kbar, vbar


def mosaic_bsa_compress_select(qbar, kbar, vbar, nside, block, topn, o_cg=None, sel_idx=None, kpieces=None,
                               kbn2=None, stream=None):
    """o_cg [b,H,m,d] fp32 and sel_idx [b,H,m,topn] int32 from the pooled tensors.  kpieces and
    kbn2: the pool's bf16 pieces of k̄ and |k̄_j|^2 (together), which topn <= 16 ranks on."""
    b, h, m, d = qbar.shape
    if m * block != 12 * nside * nside:
        raise ValueError("m * block must equal 12*nside^2")
    o_cg = torch.empty((b, h, m, d), dtype=torch.float32, device=qbar.device) if o_cg is None else o_cg
    sel_idx = torch.empty((b, h, m, topn), dtype=torch.int32, device=qbar.device) if sel_idx is None else sel_idx
    _check(lib().mosaic_bsa_compress_select(
        _ptr(qbar, torch.float64, (b, h, m, d), "qbar"), _ptr(kbar, torch.float64, (b, h, m, d), "kbar"),
        _ptr(vbar, torch.float32, (b, h, m, d), "vbar"), b, h, d, nside, block, topn,
        None if kpieces is None else _ptr(kpieces, torch.bfloat16, (b, h, m, 2, d), "kpieces"),
        None if kbn2 is None else _ptr(kbn2, torch.float32, (b, h, m), "kbn2"),
        _ptr(o_cg, torch.float32, (b, h, m, d), "o_cg"),
        _ptr(sel_idx, torch.int32, (b, h, m, topn), "sel_idx"), _stream(stream)))
    return o_cg, sel_idx


def mosaic_bsa_fine(q, k, v, gates, o_cg, sel_idx, nside, block, topn, window, out=None, knorm=None,
                    sel_bound=None, stream=None):
    """out [b,H,N,d] fp32: gated sum of o_cg with the selected and local fine branches.  knorm: the
    pool's largest key norm per block (float32 [b,H,m]), or None for the running-maximum softmax.
    sel_bound: mosaic_bsa_select_bound's output for the same sel_idx and knorm, or None."""
    b, h, n, d = _dims(q, nside)
    m = n // block
    out = torch.empty((b, h, n, d), dtype=torch.float32, device=q.device) if out is None else out
    _check(lib().mosaic_bsa_fine(
        _ptr(q, torch.bfloat16, (b, h, n, d), "q"), _ptr(k, torch.bfloat16, (b, h, n, d), "k"),
        _ptr(v, torch.bfloat16, (b, h, n, d), "v"), _ptr(gates, torch.float32, (b, h, n, 3), "gates"),
        _ptr(o_cg, torch.float32, (b, h, m, d), "o_cg"), _ptr(sel_idx, torch.int32, (b, h, m, topn), "sel_idx"),
        None if knorm is None else _ptr(knorm, torch.float32, (b, h, m), "knorm"),
        None if sel_bound is None else _ptr(sel_bound, torch.float32, (b, h, m), "sel_bound"),
        b, h, d, nside, block, topn, window, _ptr(out, torch.float32, (b, h, n, d), "out"), _stream(stream)))
    return out


def mosaic_bsa_select_bound(sel_idx, knorm, nside, block, topn, head_dim, sel_bound=None, stream=None):
    """sel_bound [b,H,m] fp32: the largest knorm over each query block's topn selected blocks
    (m = 12*nside^2 / block; sel_idx and knorm are checked against it)."""
    if not isinstance(sel_idx, torch.Tensor) or sel_idx.dim() != 4:
        raise ValueError("sel_idx must be [batch, heads, m, topn]")
    if block < 1 or (12 * nside * nside) % block:
        raise ValueError(f"block {block} does not divide N = 12*{nside}^2")
    b, h = sel_idx.shape[:2]
    m = 12 * nside * nside // block
    sel_bound = torch.empty((b, h, m), dtype=torch.float32, device=sel_idx.device) if sel_bound is None \
        else sel_bound
    _check(lib().mosaic_bsa_select_bound(
        _ptr(sel_idx, torch.int32, (b, h, m, topn), "sel_idx"), _ptr(knorm, torch.float32, (b, h, m), "knorm"),
        b, h, head_dim, nside, block, topn, _ptr(sel_bound, torch.float32, (b, h, m), "sel_bound"),
        _stream(stream)))
    return sel_bound


def mosaic_bsa_saved_bytes(batch, heads, head_dim, nside, block) -> int:
    return lib().mosaic_bsa_saved_bytes(batch, heads, head_dim, nside, block)


def mosaic_bsa_forward_train(q, k, v, gates, nside, block, topn, window, out=None, sel_idx=None, saved=None,
                             stream=None):
    """mosaic_bsa_forward plus the state the backward reads: returns (out, sel_idx, saved), saved a
    1-D uint8 device tensor of mosaic_bsa_saved_bytes(...) bytes."""
    b, h, n, d = _dims(q, nside)
    m = n // block
    if out is None:
        out = torch.empty((b, h, n, d), dtype=torch.float32, device=q.device)
    if sel_idx is None:
        sel_idx = torch.empty((b, h, m, topn), dtype=torch.int32, device=q.device)
    need = mosaic_bsa_saved_bytes(b, h, d, nside, block)
    if saved is None:
        saved = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if saved.dtype != torch.uint8 or saved.dim() != 1 or saved.device.type != "cuda":
        raise ValueError("saved must be a 1-D uint8 device tensor")
    _check(lib().mosaic_bsa_forward_train(
        _ptr(q, torch.bfloat16, (b, h, n, d), "q"), _ptr(k, torch.bfloat16, (b, h, n, d), "k"),
        _ptr(v, torch.bfloat16, (b, h, n, d), "v"), _ptr(gates, torch.float32, (b, h, n, 3), "gates"),
        b, h, d, nside, block, topn, window,
        _ptr(out, torch.float32, (b, h, n, d), "out"),
        _ptr(sel_idx, torch.int32, (b, h, m, topn), "sel_idx"),
        saved.data_ptr(), saved.numel(), _stream(stream)))
    return out, sel_idx, saved


def mosaic_bsa_backward_workspace_bytes(batch, heads, head_dim, nside, block, topn) -> int:
    return lib().mosaic_bsa_backward_workspace_bytes(batch, heads, head_dim, nside, block, topn)


def mosaic_bsa_backward(q, k, v, gates, sel_idx, dout, nside, block, topn, window, dq=None, dk=None, dv=None,
                        dgates=None, workspace=None, stream=None, saved=None):
    """dq, dk, dv [b,H,N,d] and dgates [b,H,N,3] (fp32): gradient of the forward's out given dout,
    with the selection sel_idx held fixed.  `saved`: the state of mosaic_bsa_forward_train for
    these inputs (None: recomputed)."""
    b, h, n, d = _dims(q, nside)
    m = n // block
    dq = torch.empty((b, h, n, d), dtype=torch.float32, device=q.device) if dq is None else dq
    dk = torch.empty((b, h, n, d), dtype=torch.float32, device=q.device) if dk is None else dk
    dv = torch.empty((b, h, n, d), dtype=torch.float32, device=q.device) if dv is None else dv
    dgates = torch.empty((b, h, n, 3), dtype=torch.float32, device=q.device) if dgates is None else dgates
    need = mosaic_bsa_backward_workspace_bytes(b, h, d, nside, block, topn)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if workspace.dtype != torch.uint8 or workspace.dim() != 1 or workspace.device.type != "cuda":
        raise ValueError("workspace must be a 1-D uint8 device tensor")
    _check(lib().mosaic_bsa_backward(
        _ptr(q, torch.bfloat16, (b, h, n, d), "q"), _ptr(k, torch.bfloat16, (b, h, n, d), "k"),
        _ptr(v, torch.bfloat16, (b, h, n, d), "v"), _ptr(gates, torch.float32, (b, h, n, 3), "gates"),
        _ptr(sel_idx, torch.int32, (b, h, m, topn), "sel_idx"), _ptr(dout, torch.float32, (b, h, n, d), "dout"),
        b, h, d, nside, block, topn, window,
        _saved_ptr(saved), 0 if saved is None else saved.numel(),
        _ptr(dq, torch.float32, (b, h, n, d), "dq"), _ptr(dk, torch.float32, (b, h, n, d), "dk"),
        _ptr(dv, torch.float32, (b, h, n, d), "dv"), _ptr(dgates, torch.float32, (b, h, n, 3), "dgates"),
        workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return dq, dk, dv, dgates


def _layer_dims(x: torch.Tensor, nside: int):
    if x.dim() != 3:
        raise ValueError("x must be [batch, N, channels]")
    b, n, c = x.shape
    if n != 12 * nside * nside:
        raise ValueError(f"N = {n} but 12*nside^2 = {12 * nside * nside}")
    return b, n, c


def mosaic_bsa_layer_workspace_bytes(batch, heads, head_dim, channels, nside, block, topn) -> int:
    return lib().mosaic_bsa_layer_workspace_bytes(batch, heads, head_dim, channels, nside, block, topn)


def mosaic_bsa_layer_forward(x, w_in, w_out, heads, head_dim, nside, block, topn, window, y=None, sel_idx=None,
                             workspace=None, stream=None):
    """One encoder layer: y [b,N,C] bf16 and sel_idx [b,H,m,topn] from x [b,N,C] bf16,
    w_in [3*H*d + 3*H, C] and w_out [C, H*d] (bf16)."""
    b, n, c = _layer_dims(x, nside)
    m = n // block
    e = 3 * heads * head_dim + 3 * heads
    y = torch.empty((b, n, c), dtype=torch.bfloat16, device=x.device) if y is None else y
    sel_idx = torch.empty((b, heads, m, topn), dtype=torch.int32, device=x.device) if sel_idx is None else sel_idx
    need = mosaic_bsa_layer_workspace_bytes(b, heads, head_dim, c, nside, block, topn)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    if workspace.dtype != torch.uint8 or workspace.dim() != 1 or workspace.device.type != "cuda":
        raise ValueError("workspace must be a 1-D uint8 device tensor")
    _check(lib().mosaic_bsa_layer_forward(
        _ptr(x, torch.bfloat16, (b, n, c), "x"), _ptr(w_in, torch.bfloat16, (e, c), "w_in"),
        _ptr(w_out, torch.bfloat16, (c, heads * head_dim), "w_out"),
        b, heads, head_dim, c, nside, block, topn, window,
        _ptr(y, torch.bfloat16, (b, n, c), "y"), _ptr(sel_idx, torch.int32, (b, heads, m, topn), "sel_idx"),
        workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return y, sel_idx


def mosaic_bsa_layer_in(x, w_in, heads, head_dim, nside, q=None, k=None, v=None, gates=None, stream=None):
    """q, k, v [b,H,N,d] bf16 and gates [b,H,N,3] fp32 from x [b,N,C] and w_in."""
    b, n, c = _layer_dims(x, nside)
    e = 3 * heads * head_dim + 3 * heads
    shp = (b, heads, n, head_dim)
    q = torch.empty(shp, dtype=torch.bfloat16, device=x.device) if q is None else q
    k = torch.empty(shp, dtype=torch.bfloat16, device=x.device) if k is None else k
    v = torch.empty(shp, dtype=torch.bfloat16, device=x.device) if v is None else v
    gates = torch.empty((b, heads, n, 3), dtype=torch.float32, device=x.device) if gates is None else gates
    _check(lib().mosaic_bsa_layer_in(
        _ptr(x, torch.bfloat16, (b, n, c), "x"), _ptr(w_in, torch.bfloat16, (e, c), "w_in"),
        b, heads, head_dim, c, nside,
        _ptr(q, torch.bfloat16, shp, "q"), _ptr(k, torch.bfloat16, shp, "k"), _ptr(v, torch.bfloat16, shp, "v"),
        _ptr(gates, torch.float32, (b, heads, n, 3), "gates"), _stream(stream)))
    return q, k, v, gates


def mosaic_bsa_layer_out(attn, w_out, x, nside, y=None, stream=None):
    """y [b,N,C] bf16 = x + merge_heads(attn) w_outᵀ, attn [b,H,N,d] fp32."""
    b, n, c = _layer_dims(x, nside)
    _, heads, _, head_dim = attn.shape
    y = torch.empty((b, n, c), dtype=torch.bfloat16, device=x.device) if y is None else y
    _check(lib().mosaic_bsa_layer_out(
        _ptr(attn, torch.float32, (b, heads, n, head_dim), "attn"),
        _ptr(w_out, torch.bfloat16, (c, heads * head_dim), "w_out"), _ptr(x, torch.bfloat16, (b, n, c), "x"),
        b, heads, head_dim, c, nside, _ptr(y, torch.bfloat16, (b, n, c), "y"), _stream(stream)))
    return y


def mosaic_bsa_layer_out_merged(attn, w_out, x, nside, heads, y=None, stream=None):
    """y [b,N,C] bf16 = x + attn w_outᵀ, attn [b,N,H*d] bf16 (the heads side by side)."""
    b, n, c = _layer_dims(x, nside)
    hd = attn.shape[-1]
    if hd % heads:
        raise ValueError(f"attn's last dimension {hd} is not a multiple of heads={heads}")
    head_dim = hd // heads
    y = torch.empty((b, n, c), dtype=torch.bfloat16, device=x.device) if y is None else y
    _check(lib().mosaic_bsa_layer_out_merged(
        _ptr(attn, torch.bfloat16, (b, n, hd), "attn"),
        _ptr(w_out, torch.bfloat16, (c, hd), "w_out"), _ptr(x, torch.bfloat16, (b, n, c), "x"),
        b, heads, head_dim, c, nside, _ptr(y, torch.bfloat16, (b, n, c), "y"), _stream(stream)))
    return y


def mosaic_healpix_coarsen(x, nside, levels, y=None, stream=None):
    """y [b, 12*(nside>>levels)^2, C] fp32: mean of each coarse pixel's descendants, x [b, N, C] bf16."""
    b, n, c = _layer_dims(x, nside)
    nc = 12 * (nside >> levels) ** 2
    y = torch.empty((b, nc, c), dtype=torch.float32, device=x.device) if y is None else y
    _check(lib().mosaic_healpix_coarsen(_ptr(x, torch.bfloat16, (b, n, c), "x"), b, c, nside, levels,
                                        _ptr(y, torch.float32, (b, nc, c), "y"), _stream(stream)))
    return y


def mosaic_interp_workspace_bytes(slices, n_src) -> int:
    return lib().mosaic_interp_workspace_bytes(slices, n_src)


def mosaic_interp_attention(k, v, w_q, nbr, rel, out=None, workspace=None, stream=None):
    """out [S, n_dst, 64] fp32: cross-attention of each target over its neighbours (k, v bf16
    [S, n_src, d] / [S, n_src, 64], w_q [d, 3] fp32, nbr [n_dst, K] int32, rel [n_dst, K, 3] fp32)."""
    s, n_src, d = k.shape
    dv = v.shape[-1]
    n_dst, n_nbr = nbr.shape
    out = torch.empty((s, n_dst, dv), dtype=torch.float32, device=k.device) if out is None else out
    need = mosaic_interp_workspace_bytes(s, n_src)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=k.device)
    _check(lib().mosaic_interp_attention(
        _ptr(k, torch.bfloat16, (s, n_src, d), "k"), _ptr(v, torch.bfloat16, (s, n_src, dv), "v"),
        _ptr(w_q, torch.float32, (d, 3), "w_q"), _ptr(nbr, torch.int32, (n_dst, n_nbr), "nbr"),
        _ptr(rel, torch.float32, (n_dst, n_nbr, 3), "rel"), s, n_src, n_dst, n_nbr, d, dv,
        _ptr(out, torch.float32, (s, n_dst, dv), "out"), workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return out

"""Python binding of libbsa.so (block-sparse spatiotemporal attention, gfx950).

Argument marshalling only: every computation runs in the HIP kernels behind
the C ABI declared in ``include/bsa.h``.  PyTorch supplies device memory and
the current stream.  There is no fallback: if the library is not built, or a
call fails, an exception is raised.
"""

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsa.so")

MASK_ALL, MASK_WINDOW_ANCHOR, MASK_RADIAL = 0, 1, 2
DT_BF16, DT_F32 = 0, 1

_lib = None


class BsaError(RuntimeError):
    pass


class MaskDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("kind", "frames", "frame_tokens", "block", "window", "anchor_period",
                 "anchor_step", "anchor_rows", "radial_w")]


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("D", ctypes.c_int32), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64)]


_P = ctypes.c_void_p
_SIGNATURES = {
    "bsa_mask_num_blocks": (ctypes.c_int32, [ctypes.POINTER(MaskDesc)]),
    "bsa_build_block_mask": (ctypes.c_int, [ctypes.POINTER(MaskDesc), _P, _P, ctypes.c_int64, _P, _P]),
    "bsa_block_sparse_attn_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_int,
                                                 ctypes.POINTER(Shape), _P, _P, _P, ctypes.c_int32,
                                                 ctypes.c_float, _P]),
    "bsa_transpose_block_mask": (ctypes.c_int, [_P, _P, ctypes.c_int32, _P, _P, ctypes.c_int64, _P]),
    "bsa_block_sparse_attn_bwd_workspace": (ctypes.c_size_t, [ctypes.POINTER(Shape)]),
    "bsa_block_sparse_attn_bwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_int, ctypes.POINTER(Shape), _P,
                                                 _P, _P, _P, ctypes.c_int32, ctypes.c_float, _P, _P, _P, _P,
                                                 ctypes.c_size_t, _P]),
    "bsa_linear_attn_workspace": (ctypes.c_size_t, [ctypes.POINTER(Shape)]),
    "bsa_linear_attn_fwd": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int, ctypes.POINTER(Shape), _P, _P,
                                           _P, ctypes.c_size_t, _P]),
    "bsa_linear_attn_fwd_noalloc": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int, ctypes.POINTER(Shape), _P, _P,
                                                   _P]),
    "bsa_linear_attn_noalloc_max_scratch": (ctypes.c_size_t, []),
    "bsa_causal_linear_attn_workspace": (ctypes.c_size_t, [ctypes.POINTER(Shape)]),
    "bsa_causal_linear_attn_fwd": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int, ctypes.POINTER(Shape), _P, _P,
                                                  _P, _P, _P, ctypes.c_size_t, _P]),
    "bsa_kmeans_workspace": (ctypes.c_size_t, [ctypes.POINTER(Shape), ctypes.c_int32]),
    "bsa_kmeans": (ctypes.c_int, [_P, ctypes.c_int, ctypes.POINTER(Shape), ctypes.c_int32, ctypes.c_int32, _P, _P,
                                  _P, _P, _P, ctypes.c_size_t, _P]),
    "bsa_gather_rows": (ctypes.c_int, [_P, ctypes.c_int, ctypes.POINTER(Shape), _P, _P, _P]),
    "bsa_scatter_rows": (ctypes.c_int, [_P, ctypes.c_int, ctypes.POINTER(Shape), _P, _P, _P]),
    "bsa_cluster_centroids": (ctypes.c_int, [_P, _P, _P, ctypes.c_int, ctypes.POINTER(Shape), _P,
                                             ctypes.c_int32, _P, ctypes.c_int32, _P, _P, _P, _P]),
    "bsa_route_scores_workspace": (ctypes.c_size_t, [ctypes.POINTER(Shape), ctypes.c_int32, ctypes.c_int32]),
    "bsa_route_scores": (ctypes.c_int, [_P, _P, ctypes.c_int, ctypes.POINTER(Shape), _P, ctypes.c_int32, _P,
                                        ctypes.c_int32, _P, _P, _P, ctypes.c_float, _P, _P, ctypes.c_size_t,
                                        _P]),
    "bsa_route_select_workspace": (ctypes.c_size_t, [ctypes.POINTER(Shape), ctypes.c_int32, ctypes.c_int32]),
    "bsa_route_select": (ctypes.c_int, [_P, ctypes.POINTER(Shape), _P, ctypes.c_int32, _P, ctypes.c_int32,
                                        ctypes.c_int32, _P, _P, _P, ctypes.c_size_t, _P]),
    "bsa_route_budget": (ctypes.c_int64, [ctypes.c_int32, ctypes.c_int32]),
    "bsa_check_csr": (ctypes.c_int, [_P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64]),
    "bsa_hbm_read_probe": (ctypes.c_int, [_P, ctypes.c_size_t, _P, _P]),
    "bsa_compensated_attn_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_int, ctypes.POINTER(Shape), _P,
                                                ctypes.c_int32, _P, ctypes.c_int32, _P, _P, _P, _P,
                                                ctypes.c_float, _P, ctypes.c_size_t, _P]),
    "bsa_compensated_attn_workspace": (ctypes.c_size_t, [ctypes.POINTER(Shape), ctypes.c_int32, ctypes.c_int32]),
    "bsa_centroid_compensate_workspace": (ctypes.c_size_t, [ctypes.POINTER(Shape), ctypes.c_int32,
                                                            ctypes.c_int32]),
    "bsa_centroid_compensate": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_int, ctypes.POINTER(Shape), _P,
                                               ctypes.c_int32, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_float, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "bsa_mixed_attn_fwd": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int, ctypes.POINTER(Shape), _P, _P, _P,
                                          ctypes.c_int32, ctypes.c_float, ctypes.c_float, _P, ctypes.c_size_t,
                                          _P]),
    "bsa_lipar_prune": (ctypes.c_int, [_P, ctypes.c_int, ctypes.POINTER(Shape), ctypes.c_int32, ctypes.c_float,
                                       _P, _P, _P, _P, _P, _P]),
    "bsa_lipar_restore": (ctypes.c_int, [_P, ctypes.c_int, ctypes.POINTER(Shape), ctypes.c_int32, _P, _P, _P,
                                         _P]),
    "bsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "bsa_last_error": (ctypes.c_char_p, []),
}


def load(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise BsaError(f"{path} not found: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def exported_names():
    return list(_SIGNATURES)


def _check(status: int, fn: str):
    if status != 0:
        lib = load()
        raise BsaError(f"{fn}: {lib.bsa_status_string(status).decode()}: {lib.bsa_last_error().decode()}")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def mask_desc(params: dict) -> MaskDesc:
    return MaskDesc(**{k: int(params[k]) for k, _ in MaskDesc._fields_})


def num_blocks(params: dict) -> int:
    nb = load().bsa_mask_num_blocks(ctypes.byref(mask_desc(params)))
    if nb < 0:
        raise BsaError(f"invalid mask description: {load().bsa_last_error().decode()}")
    return nb


def build_block_mask(params: dict, device="cuda", row_ptr=None, col_idx=None, row_order=None,
                     with_order: bool = False):
    """CSR (row_ptr int32[nb+1], col_idx int32[nb*nb]) of the block mask, on the device.

    Only the first row_ptr[nb] entries of col_idx are meaningful.  With
    ``with_order`` (or a given ``row_order`` buffer) also returns the rows sorted
    schedule ``block_sparse_attn_fwd`` accepts: int32[nb + 1], rows with at least
    1.5x the mean length first (longest first), then the others in index order,
    and the number of those long rows last.
    """
    lib = load()
    desc = mask_desc(params)
    nb = num_blocks(params)
    if row_ptr is None:
        row_ptr = torch.empty(nb + 1, dtype=torch.int32, device=device)
    if col_idx is None:
        col_idx = torch.empty(nb * nb, dtype=torch.int32, device=device)
    if row_order is None and with_order:
        row_order = torch.empty(nb + 1, dtype=torch.int32, device=device)
    if row_ptr.dtype != torch.int32 or row_ptr.numel() < nb + 1 or not row_ptr.is_cuda:
        raise BsaError("row_ptr must be an int32 device tensor of nb + 1 entries")
    if col_idx.dtype != torch.int32 or not col_idx.is_cuda:
        raise BsaError("col_idx must be an int32 device tensor")
    if row_order is not None and (row_order.dtype != torch.int32 or row_order.numel() < nb + 1
                                  or not row_order.is_cuda):
        raise BsaError("row_order must be an int32 device tensor of nb + 1 entries")
    _check(lib.bsa_build_block_mask(ctypes.byref(desc), _ptr(row_ptr), _ptr(col_idx),
                                    col_idx.numel(), _ptr(row_order), _stream(row_ptr.device)),
           "bsa_build_block_mask")
    if row_order is not None:
        return row_ptr, col_idx, row_order
    return row_ptr, col_idx


def _shape_of(q: torch.Tensor) -> Shape:
    if q.dim() != 4:
        raise BsaError("tensors must be [B, H, N, D]")
    B, H, N, D = q.shape
    if q.stride(3) != 1:
        raise BsaError("the D axis must be contiguous")
    return Shape(B, H, N, D, q.stride(0), q.stride(1), q.stride(2))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DT_BF16
    if t.dtype == torch.float32:
        return DT_F32
    raise BsaError(f"unsupported dtype {t.dtype}")


def block_sparse_attn_fwd(q, k, v, row_ptr, col_idx, block: int, scale=None, out=None,
                          return_lse: bool = True, lse=None, row_order=None):
    """O (and LSE, fp32 [B, H, N]) of block-sparse softmax attention on the device."""
    lib = load()
    for t in (q, k, v):
        if not t.is_cuda:
            raise BsaError("q, k, v must be device tensors")
    if k.shape != q.shape or v.shape != q.shape or k.stride() != q.stride() or v.stride() != q.stride():
        raise BsaError("q, k, v must share one shape and one stride layout")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise BsaError("q, k, v must share one dtype")
    shape = _shape_of(q)
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    if out.stride() != q.stride() or out.dtype != q.dtype:
        raise BsaError("out must have the layout and dtype of q")
    if lse is None and return_lse:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != tuple(q.shape[:3])):
        raise BsaError("lse must be a contiguous float32 [B, H, N] tensor")
    if row_order is not None:
        nb = -(-q.shape[2] // int(block)) if int(block) > 0 else 0
        if row_order.dtype != torch.int32 or not row_order.is_cuda or row_order.numel() < nb + 1:
            raise BsaError("row_order must be an int32 device tensor of nb + 1 entries")
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    _check(lib.bsa_block_sparse_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                         _dtype_code(q), ctypes.byref(shape), _ptr(row_ptr),
                                         _ptr(col_idx), _ptr(row_order), int(block), float(scale),
                                         _stream(q.device)),
           "bsa_block_sparse_attn_fwd")
    return out, lse


def _check_qkv(q, k, v):
    for t in (q, k, v):
        if not t.is_cuda:
            raise BsaError("q, k, v must be device tensors")
    if k.shape != q.shape or v.shape != q.shape or k.stride() != q.stride() or v.stride() != q.stride():
        raise BsaError("q, k, v must share one shape and one stride layout")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise BsaError("q, k, v must share one dtype")


def transpose_block_mask(row_ptr, col_idx, col_ptr=None, row_idx=None):
    """(col_ptr, row_idx): the transposed block CSR (query blocks per key block)."""
    lib = load()
    nb = row_ptr.numel() - 1
    if col_ptr is None:
        col_ptr = torch.empty(nb + 1, dtype=torch.int32, device=row_ptr.device)
    if row_idx is None:
        row_idx = torch.empty(nb * nb, dtype=torch.int32, device=row_ptr.device)
    _check(lib.bsa_transpose_block_mask(_ptr(row_ptr), _ptr(col_idx), nb, _ptr(col_ptr), _ptr(row_idx),
                                        row_idx.numel(), _stream(row_ptr.device)), "bsa_transpose_block_mask")
    return col_ptr, row_idx


def block_sparse_attn_bwd_workspace(shape_like) -> int:
    return int(load().bsa_block_sparse_attn_bwd_workspace(ctypes.byref(_shape_of(shape_like))))


def block_sparse_attn_bwd(q, k, v, o, do, lse, row_ptr, col_idx, block: int = 128, scale=None,
                          col_ptr=None, row_idx=None, dq=None, dk=None, dv=None, workspace=None):
    """(dq, dk, dv) of block-sparse attention (bf16, D = 128, block 128)."""
    lib = load()
    _check_qkv(q, k, v)
    for t in (o, do):
        if t.dtype != q.dtype or t.stride() != q.stride() or t.shape != q.shape:
            raise BsaError("o and do must have the layout and dtype of q")
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise BsaError("lse must be a contiguous fp32 tensor [B, H, N]")
    shape = _shape_of(q)
    scale = 1.0 / math.sqrt(q.shape[3]) if scale is None else scale
    if col_ptr is None:
        col_ptr, row_idx = transpose_block_mask(row_ptr, col_idx)
    outs = []
    for t in (dq, dk, dv):
        outs.append(torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device) if t is None else t)
    if workspace is None:
        need = int(lib.bsa_block_sparse_attn_bwd_workspace(ctypes.byref(shape)))
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib.bsa_block_sparse_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _dtype_code(q),
                                         ctypes.byref(shape), _ptr(row_ptr), _ptr(col_idx), _ptr(col_ptr),
                                         _ptr(row_idx), int(block), float(scale), _ptr(outs[0]), _ptr(outs[1]),
                                         _ptr(outs[2]), _ptr(workspace), workspace.numel(), _stream(q.device)),
           "bsa_block_sparse_attn_bwd")
    return tuple(outs)


def linear_attn_workspace(shape_like) -> int:
    return int(load().bsa_linear_attn_workspace(ctypes.byref(_shape_of(shape_like))))


def linear_attn_fwd(q, k, v, out=None, return_state: bool = False, workspace=None):
    """elu+1 linear attention; returns out (bf16), plus S [B,H,D,D] and z [B,H,D] (fp32) if asked."""
    lib = load()
    _check_qkv(q, k, v)
    shape = _shape_of(q)
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    if out.stride() != q.stride() or out.dtype != q.dtype:
        raise BsaError("out must have the layout and dtype of q")
    B, H, N, D = q.shape
    S = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device) if return_state else None
    z = torch.empty((B, H, D), dtype=torch.float32, device=q.device) if return_state else None
    need = int(lib.bsa_linear_attn_workspace(ctypes.byref(shape)))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(lib.bsa_linear_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _dtype_code(q),
                                   ctypes.byref(shape), _ptr(S), _ptr(z), _ptr(workspace),
                                   workspace.numel(), _stream(q.device)),
           "bsa_linear_attn_fwd")
    return (out, S, z) if return_state else out


def linear_attn_fwd_noalloc(q, k, v, out=None, return_state: bool = False):
    """linear_attn_fwd through the no-allocation entry point (the library's own
    per-GPU scratch instead of a workspace); the caller still supplies out and,
    with return_state, S and z are allocated here as ordinary outputs."""
    lib = load()
    _check_qkv(q, k, v)
    shape = _shape_of(q)
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    if out.stride() != q.stride() or out.dtype != q.dtype:
        raise BsaError("out must have the layout and dtype of q")
    B, H, N, D = q.shape
    S = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device) if return_state else None
    z = torch.empty((B, H, D), dtype=torch.float32, device=q.device) if return_state else None
    _check(lib.bsa_linear_attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _dtype_code(q),
                                           ctypes.byref(shape), _ptr(S), _ptr(z), _stream(q.device)),
           "bsa_linear_attn_fwd_noalloc")
    return (out, S, z) if return_state else out


def causal_linear_attn_workspace(shape_like) -> int:
    return int(load().bsa_causal_linear_attn_workspace(ctypes.byref(_shape_of(shape_like))))


def _state_tensor(t, shape, name):
    if t is None:
        return None
    if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != shape:
        raise BsaError(f"{name} must be a contiguous fp32 device tensor of shape {shape}")
    return t


def causal_linear_attn_fwd(q, k, v, out=None, state=None, return_state: bool = False, state_out=None,
                           workspace=None):
    """Causal elu+1 linear attention (bf16, D = 128).

    ``state`` = (S, z) carried in from earlier tokens (fp32 [B,H,D,D], [B,H,D]);
    with ``return_state`` (or a given ``state_out`` pair, which may be ``state``
    itself) the state after the last token is returned as well."""
    lib = load()
    _check_qkv(q, k, v)
    shape = _shape_of(q)
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    if out.stride() != q.stride() or out.dtype != q.dtype:
        raise BsaError("out must have the layout and dtype of q")
    B, H, N, D = q.shape
    S_in = z_in = None
    if state is not None:
        S_in = _state_tensor(state[0], (B, H, D, D), "S")
        z_in = _state_tensor(state[1], (B, H, D), "z")
    S_out = z_out = None
    if state_out is not None:
        S_out = _state_tensor(state_out[0], (B, H, D, D), "S_out")
        z_out = _state_tensor(state_out[1], (B, H, D), "z_out")
    elif return_state:
        S_out = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
        z_out = torch.empty((B, H, D), dtype=torch.float32, device=q.device)
    if workspace is None:
        need = int(lib.bsa_causal_linear_attn_workspace(ctypes.byref(shape)))
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib.bsa_causal_linear_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _dtype_code(q),
                                          ctypes.byref(shape), _ptr(S_in), _ptr(z_in), _ptr(S_out), _ptr(z_out),
                                          _ptr(workspace), workspace.numel(), _stream(q.device)),
           "bsa_causal_linear_attn_fwd")
    return (out, S_out, z_out) if (return_state or state_out is not None) else out


# ---- token clustering -----------------------------------------------------------

def kmeans_workspace(shape_like, C: int) -> int:
    return int(load().bsa_kmeans_workspace(ctypes.byref(_shape_of(shape_like)), int(C)))


def kmeans(x, C: int, iters: int, init, workspace=None):
    """k-means of the token rows of every (batch, head) of x (bf16 [B, H, N, 128]).

    ``init``: fp32 [B*H, C, D] initial centres (copied).  Returns (labels int32
    [B*H, N], centres fp32 [B*H, C, D], perm int32 [B*H, N], offsets int32
    [B*H, C + 1]); perm / offsets are the stable cluster order of the labels."""
    lib = load()
    if x.dtype != torch.bfloat16 or not x.is_cuda or x.dim() != 4:
        raise BsaError("x must be a bf16 device tensor [B, H, N, D]")
    B, H, N, D = x.shape
    shape = _shape_of(x)
    cent = init.to(device=x.device, dtype=torch.float32).contiguous().clone()
    if tuple(cent.shape) != (B * H, C, D):
        raise BsaError(f"init must have shape {(B * H, C, D)}")
    labels = torch.empty((B * H, N), dtype=torch.int32, device=x.device)
    perm = torch.empty((B * H, N), dtype=torch.int32, device=x.device)
    off = torch.empty((B * H, C + 1), dtype=torch.int32, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(kmeans_workspace(x, C), 1), dtype=torch.uint8, device=x.device)
    _check(lib.bsa_kmeans(_ptr(x), _dtype_code(x), ctypes.byref(shape), int(C), int(iters), _ptr(cent),
                          _ptr(labels), _ptr(perm), _ptr(off), _ptr(workspace), workspace.numel(),
                          _stream(x.device)), "bsa_kmeans")
    return labels, cent, perm, off


def _rows_permute(fn, x, perm, out):
    lib = load()
    if not x.is_cuda or x.dim() != 4:
        raise BsaError("x must be a device tensor [B, H, N, D]")
    if perm.dtype != torch.int32 or not perm.is_cuda or not perm.is_contiguous() or \
            tuple(perm.shape) != (x.shape[0] * x.shape[1], x.shape[2]):
        raise BsaError("perm must be a contiguous int32 device tensor [B*H, N]")
    if out is None:
        out = torch.empty_strided(x.shape, x.stride(), dtype=x.dtype, device=x.device)
    if out.stride() != x.stride() or out.dtype != x.dtype:
        raise BsaError("out must have the layout and dtype of x")
    _check(getattr(lib, fn)(_ptr(x), _dtype_code(x), ctypes.byref(_shape_of(x)), _ptr(perm), _ptr(out),
                            _stream(x.device)), fn)
    return out


def gather_rows(x, perm, out=None):
    """out[b, h, i] = x[b, h, perm[b*H + h, i]] (rows into cluster order)."""
    return _rows_permute("bsa_gather_rows", x, perm, out)


def scatter_rows(y, perm, out=None):
    """out[b, h, perm[b*H + h, i]] = y[b, h, i] (rows back to token order)."""
    return _rows_permute("bsa_scatter_rows", y, perm, out)


# ---- clustered compensation ---------------------------------------------------

def _check_offsets(q, q_off, k_off):
    B, H = q.shape[0], q.shape[1]
    for t in (q_off, k_off):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous() or t.dim() != 2 or t.shape[0] != B * H:
            raise BsaError("offsets must be contiguous int32 device tensors [B*H, C+1]")
    return q_off.shape[1] - 1, k_off.shape[1] - 1


def cluster_centroids(q, k, v, q_off, k_off, which: str = "all"):
    """fp32 centroids (q_cent [B*H, Cq, D], k_cent, v_cent [B*H, Ck, D]); with
    which="query" or "key" only that set is computed (the others are None)."""
    lib = load()
    _check_qkv(q, k, v)
    Cq, Ck = _check_offsets(q, q_off, k_off)
    B, H, N, D = q.shape
    if which not in ("all", "query", "key"):
        raise BsaError("which must be 'all', 'query' or 'key'")
    qc = torch.empty((B * H, Cq, D), dtype=torch.float32, device=q.device) if which != "key" else None
    kc = torch.empty((B * H, Ck, D), dtype=torch.float32, device=q.device) if which != "query" else None
    vc = torch.empty((B * H, Ck, D), dtype=torch.float32, device=q.device) if which != "query" else None
    _check(lib.bsa_cluster_centroids(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), ctypes.byref(_shape_of(q)),
                                     _ptr(q_off), Cq, _ptr(k_off), Ck, _ptr(qc), _ptr(kc), _ptr(vc),
                                     _stream(q.device)), "bsa_cluster_centroids")
    return qc, kc, vc


def route_scores(k, v, q_off, k_off, q_cent, scale=None, k_cent=None, v_cent=None):
    """fp32 routing scores [B*H, Cq, Ck] from the query centroids; returns
    (score, k_cent, v_cent), the key / value centroids coming from the same pass."""
    lib = load()
    _check_qkv(k, k, v)
    Cq, Ck = _check_offsets(k, q_off, k_off)
    B, H, N, D = k.shape
    shape = _shape_of(k)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    score = torch.empty((B * H, Cq, Ck), dtype=torch.float32, device=k.device)
    if k_cent is None:
        k_cent = torch.empty((B * H, Ck, D), dtype=torch.float32, device=k.device)
    if v_cent is None:
        v_cent = torch.empty((B * H, Ck, D), dtype=torch.float32, device=k.device)
    for t, name in ((k_cent, "k_cent"), (v_cent, "v_cent")):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != B * H * Ck * D:
            raise BsaError(f"{name} must be a contiguous float32 [B*H, Ck, D] tensor")
    ws = torch.empty(int(lib.bsa_route_scores_workspace(ctypes.byref(shape), Cq, Ck)), dtype=torch.uint8,
                     device=k.device)
    _check(lib.bsa_route_scores(_ptr(k), _ptr(v), _dtype_code(k), ctypes.byref(shape), _ptr(q_off), Cq,
                                _ptr(k_off), Ck, _ptr(q_cent.contiguous()), _ptr(k_cent), _ptr(v_cent),
                                float(scale), _ptr(score), _ptr(ws), ws.numel(), _stream(k.device)),
           "bsa_route_scores")
    return score, k_cent, v_cent


def route_select(score, shape_like, q_off, k_off, density_ppm: int):
    """Route CSR (row_ptr int32 [B*H, Cq+1], col int32 [B*H, Cq*Ck]) from a score array."""
    lib = load()
    Cq, Ck = _check_offsets(shape_like, q_off, k_off)
    B, H = shape_like.shape[0], shape_like.shape[1]
    shape = _shape_of(shape_like)
    if score.dtype != torch.float32 or not score.is_contiguous() or score.numel() != B * H * Cq * Ck:
        raise BsaError("score must be a contiguous float32 [B*H, Cq, Ck] tensor")
    rrow = torch.empty((B * H, Cq + 1), dtype=torch.int32, device=score.device)
    rcol = torch.empty((B * H, Cq * Ck), dtype=torch.int32, device=score.device)
    ws = torch.empty(int(lib.bsa_route_select_workspace(ctypes.byref(shape), Cq, Ck)), dtype=torch.uint8,
                     device=score.device)
    _check(lib.bsa_route_select(_ptr(score), ctypes.byref(shape), _ptr(q_off), Cq, _ptr(k_off), Ck,
                                int(density_ppm), _ptr(rrow), _ptr(rcol), _ptr(ws), ws.numel(),
                                _stream(score.device)), "bsa_route_select")
    return rrow, rcol


def compensated_attn_fwd(q, k, v, q_off, k_off, rrow, rcol, k_cent, v_cent, scale=None, out=None,
                         return_lse: bool = True):
    """Compensated attention in cluster order; returns (out bf16, lse fp32 or None)."""
    lib = load()
    _check_qkv(q, k, v)
    Cq, Ck = _check_offsets(q, q_off, k_off)
    shape = _shape_of(q)
    scale = 1.0 / math.sqrt(q.shape[-1]) if scale is None else scale
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    need = int(lib.bsa_compensated_attn_workspace(ctypes.byref(shape), Cq, Ck))
    ws = torch.empty(need, dtype=torch.uint8, device=q.device) if need > 0 else None
    _check(lib.bsa_compensated_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _dtype_code(q),
                                        ctypes.byref(shape), _ptr(q_off), Cq, _ptr(k_off), Ck, _ptr(rrow),
                                        _ptr(rcol), _ptr(k_cent.contiguous()), _ptr(v_cent.contiguous()),
                                        float(scale), _ptr(ws), need, _stream(q.device)),
           "bsa_compensated_attn_fwd")
    return out, lse


def centroid_compensate(q, k, v, q_off, k_off, density_ppm: int, scale=None, out=None, lse=None,
                        return_score: bool = False, workspace=None, rrow=None, rcol=None, score=None,
                        use_given_route: bool = False):
    """All four steps; returns (out, lse, route_row_ptr, route_col[, score]).
    With use_given_route, rrow / rcol are the route to use (inputs)."""
    lib = load()
    _check_qkv(q, k, v)
    Cq, Ck = _check_offsets(q, q_off, k_off)
    B, H, N, D = q.shape
    shape = _shape_of(q)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if use_given_route and (rrow is None or rcol is None):
        raise BsaError("use_given_route needs rrow and rcol")
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if rrow is None:
        rrow = torch.empty((B * H, Cq + 1), dtype=torch.int32, device=q.device)
    if rcol is None:
        rcol = torch.empty((B * H, Cq * Ck), dtype=torch.int32, device=q.device)
    if score is None and return_score:
        score = torch.empty((B * H, Cq, Ck), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(int(lib.bsa_centroid_compensate_workspace(ctypes.byref(shape), Cq, Ck)),
                                dtype=torch.uint8, device=q.device)
    _check(lib.bsa_centroid_compensate(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _dtype_code(q),
                                       ctypes.byref(shape), _ptr(q_off), Cq, _ptr(k_off), Ck, int(density_ppm),
                                       int(bool(use_given_route)), float(scale), _ptr(rrow), _ptr(rcol),
                                       _ptr(score), _ptr(workspace), workspace.numel(), _stream(q.device)),
           "bsa_centroid_compensate")
    return (out, lse, rrow, rcol, score) if return_score else (out, lse, rrow, rcol)


def lipar_prune(x, frames: int, tau: float, outputs=None):
    """Latent inter-frame pruning of x [B, H, N, D] (bf16); returns
    (keep uint8 [B*H, N], cpos int32 [B*H, N], kept_idx int32 [B*H, N],
    n_kept int32 [B*H], x_pruned bf16 [B*H, N, D] with rows < n_kept valid).
    ``outputs``: optionally that tuple, preallocated, to be written in place."""
    lib = load()
    shape = _shape_of(x)
    B, H, N, D = x.shape
    dev = x.device
    want = (((B * H, N), torch.uint8), ((B * H, N), torch.int32), ((B * H, N), torch.int32),
            ((B * H,), torch.int32), ((B * H, N, D), x.dtype))
    if outputs is None:
        keep, cpos, kidx, nk, xp = (torch.empty(sh, dtype=dt, device=dev) for sh, dt in want)
    else:
        if len(outputs) != 5 or any(
                tuple(t.shape) != sh or t.dtype != dt or t.device != dev or not t.is_contiguous()
                for t, (sh, dt) in zip(outputs, want)):
            raise BsaError("outputs must be contiguous (keep, cpos, kept_idx, n_kept, x_pruned) device tensors "
                           "of the shapes and dtypes lipar_prune returns")
        keep, cpos, kidx, nk, xp = outputs
    _check(lib.bsa_lipar_prune(_ptr(x), _dtype_code(x), ctypes.byref(shape), int(frames), float(tau), _ptr(keep),
                               _ptr(cpos), _ptr(kidx), _ptr(nk), _ptr(xp), _stream(dev)), "bsa_lipar_prune")
    return keep, cpos, kidx, nk, xp


def lipar_restore(y_pruned, keep, cpos, frames: int, out):
    """Restoration into out [B, H, N, D] (bf16) from dense pruned rows y_pruned [B*H, N, D]."""
    lib = load()
    shape = _shape_of(out)
    if y_pruned.shape != (shape.B * shape.H, shape.N, shape.D) or not y_pruned.is_contiguous():
        raise BsaError("y_pruned must be a contiguous [B*H, N, D] tensor")
    _check(lib.bsa_lipar_restore(_ptr(y_pruned), _dtype_code(out), ctypes.byref(shape), int(frames), _ptr(keep),
                                 _ptr(cpos), _ptr(out), _stream(out.device)), "bsa_lipar_restore")
    return out


def mixed_attn_fwd(q, k, v, r: float, row_ptr=None, col_idx=None, block: int = 128, scale=None, out=None,
                   row_order=None, workspace=None):
    """r * block-sparse softmax attention + (1 - r) * elu+1 linear attention (bf16, D = 128)."""
    lib = load()
    _check_qkv(q, k, v)
    shape = _shape_of(q)
    D = q.shape[3]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    if workspace is None and r < 1.0:
        workspace = torch.empty(linear_attn_workspace(q), dtype=torch.uint8, device=q.device)
    _check(lib.bsa_mixed_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _dtype_code(q), ctypes.byref(shape),
                                  _ptr(row_ptr), _ptr(col_idx), _ptr(row_order), int(block), float(scale),
                                  float(r), _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                  _stream(q.device)), "bsa_mixed_attn_fwd")
    return out


def check_csr(row_ptr, col_idx, nrows: int, ncols: int, capacity=None):
    """Host-side check of a block CSR (numpy int32 arrays): bsa_check_csr.
    Raises BsaError naming the first violated invariant."""
    import numpy as np
    lib = load()
    rp = np.ascontiguousarray(row_ptr, dtype=np.int32)
    ci = np.ascontiguousarray(col_idx, dtype=np.int32)
    if rp.size != nrows + 1:
        raise BsaError(f"check_csr: row_ptr has {rp.size} entries, expected {nrows + 1}")
    cap = int(ci.size) if capacity is None else int(capacity)
    if cap > ci.size:
        raise BsaError("check_csr: capacity exceeds the column array")
    ci_p = ci.ctypes.data if ci.size else rp.ctypes.data
    _check(lib.bsa_check_csr(rp.ctypes.data, ci_p, nrows, ncols, cap), "bsa_check_csr")


def hbm_read_probe(buf, sink):
    """Read every byte of the device tensor `buf` once (bsa_hbm_read_probe);
    `sink` is a device int32 tensor of at least one element."""
    import torch
    lib = load()
    nbytes = buf.numel() * buf.element_size()
    _check(lib.bsa_hbm_read_probe(buf.data_ptr(), nbytes, sink.data_ptr(),
                                  torch.cuda.current_stream(buf.device).cuda_stream), "bsa_hbm_read_probe")


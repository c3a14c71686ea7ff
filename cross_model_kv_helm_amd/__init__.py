"""Python binding of libhelmkv.so, the gfx950 cross-model KV-cache transfer.

Argument marshalling only: every step of the transfer runs in the HIP
kernels behind include/helm_kv.h.  The names mirror the C ABI
(``helm_kv_transfer``, ``helm_kv_transfer_paged``, ...).  torch supplies
device memory and the current stream; tensors are passed by ``data_ptr()``.

The library is loaded from this directory; if it is missing the import of
any entry point raises — there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhelmkv.so")

HELM_BF16 = 0
HELM_F32 = 1

STATUS = {0: "HELM_OK", 1: "HELM_E_INVALID_ARG", 2: "HELM_E_PAIR_SHAPE", 3: "HELM_E_LAYER_SEL",
          4: "HELM_E_NO_DEVICE", 5: "HELM_E_DTYPE", 6: "HELM_E_ARCH", 7: "HELM_E_WORKSPACE",
          8: "HELM_E_ALIAS", 9: "HELM_E_PAGED_TABLE", 10: "HELM_E_LAUNCH"}

HELM_STAGE_TABLES, HELM_STAGE_MAP, HELM_STAGE_ALL = 1, 2, 3
HELM_PATH_MATRIX, HELM_PATH_PORTABLE = 1, 2

EXPORTED = ("helm_kv_transfer", "helm_kv_transfer_stage", "helm_kv_transfer_path", "helm_kv_transfer_paged",
            "helm_kv_cosine", "helm_kv_transfer_wide", "helm_kv_transfer_wide_stage", "helm_kv_wide_workspace_bytes",
            "helm_ridge_fit", "helm_ridge_fit_stage", "helm_ridge_workspace_bytes", "helm_kv_workspace_bytes",
            "helm_kv_paged_workspace_bytes", "helm_mapper_check", "helm_paged_check",
            "helm_device_check", "helm_arch_supported", "helm_last_error", "helm_status_string",
            "helm_abi_version", "helm_kv_transfer_noalloc", "helm_kv_noalloc_max_bytes")


class HelmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class HelmShape(ctypes.Structure):
    _fields_ = [
        ("n_src_layers", ctypes.c_int32), ("n_tgt_layers", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("k", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("n_tokens", ctypes.c_int64),
        ("rope_theta_src", ctypes.c_double), ("rope_theta_tgt", ctypes.c_double),
        ("stream", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class HelmRidgeShape(ctypes.Structure):
    _fields_ = [
        ("n_groups", ctypes.c_int64), ("n_obs", ctypes.c_int64),
        ("in_features", ctypes.c_int32), ("out_features", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("lambda_", ctypes.c_double),
        ("stream", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class HelmPagedShape(ctypes.Structure):
    _fields_ = [
        ("n_src_layers", ctypes.c_int32), ("n_tgt_layers", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("k", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("n_requests", ctypes.c_int32),
        ("max_blocks_src", ctypes.c_int32), ("max_blocks_tgt", ctypes.c_int32),
        ("n_src_blocks", ctypes.c_int32), ("n_tgt_blocks", ctypes.c_int32),
        ("n_tokens_total", ctypes.c_int64),
        ("rope_theta_src", ctypes.c_double), ("rope_theta_tgt", ctypes.c_double),
        ("stream", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Loads libhelmkv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(the transfer has no other implementation)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32p = ctypes.c_void_p, ctypes.c_void_p
        L.helm_kv_transfer.restype = ctypes.c_int
        L.helm_kv_transfer.argtypes = [vp] * 11 + [ctypes.POINTER(HelmShape)]
        L.helm_kv_transfer_stage.argtypes = [ctypes.c_int] + [vp] * 11 + [ctypes.POINTER(HelmShape)]
        L.helm_kv_transfer_stage.restype = ctypes.c_int
        L.helm_kv_transfer_path.argtypes = [vp] * 11 + [ctypes.POINTER(HelmShape), ctypes.POINTER(ctypes.c_int)]
        L.helm_kv_transfer_path.restype = ctypes.c_int
        L.helm_kv_transfer_noalloc.argtypes = [vp] * 11 + [ctypes.POINTER(HelmShape)]
        L.helm_kv_transfer_noalloc.restype = ctypes.c_int
        L.helm_kv_noalloc_max_bytes.argtypes = []
        L.helm_kv_noalloc_max_bytes.restype = ctypes.c_size_t
        L.helm_kv_transfer_wide.restype = ctypes.c_int
        L.helm_kv_transfer_wide.argtypes = [vp] * 11 + [ctypes.POINTER(HelmShape)]
        L.helm_ridge_workspace_bytes.restype = ctypes.c_size_t
        L.helm_ridge_workspace_bytes.argtypes = [ctypes.POINTER(HelmRidgeShape)]
        L.helm_ridge_fit.restype = ctypes.c_int
        L.helm_ridge_fit.argtypes = [vp] * 4 + [ctypes.POINTER(HelmRidgeShape)]
        L.helm_ridge_fit_stage.restype = ctypes.c_int
        L.helm_ridge_fit_stage.argtypes = [ctypes.c_int] + [vp] * 4 + [ctypes.POINTER(HelmRidgeShape)]
        L.helm_kv_transfer_wide_stage.restype = ctypes.c_int
        L.helm_kv_transfer_wide_stage.argtypes = [ctypes.c_int] + [vp] * 11 + [ctypes.POINTER(HelmShape)]
        L.helm_kv_wide_workspace_bytes.restype = ctypes.c_size_t
        L.helm_kv_wide_workspace_bytes.argtypes = [ctypes.POINTER(HelmShape)]
        L.helm_kv_cosine.restype = ctypes.c_int
        L.helm_kv_cosine.argtypes = [vp] * 5 + [ctypes.POINTER(HelmShape)]
        L.helm_kv_transfer_paged.restype = ctypes.c_int
        L.helm_kv_transfer_paged.argtypes = [vp] * 14 + [ctypes.POINTER(HelmPagedShape)]
        L.helm_kv_workspace_bytes.restype = ctypes.c_size_t
        L.helm_kv_workspace_bytes.argtypes = [ctypes.POINTER(HelmShape)]
        L.helm_kv_paged_workspace_bytes.restype = ctypes.c_size_t
        L.helm_kv_paged_workspace_bytes.argtypes = [ctypes.POINTER(HelmPagedShape)]
        L.helm_mapper_check.restype = ctypes.c_int
        L.helm_mapper_check.argtypes = [ctypes.POINTER(HelmShape), i32p]
        L.helm_paged_check.restype = ctypes.c_int
        L.helm_paged_check.argtypes = [ctypes.POINTER(HelmPagedShape), i32p, i32p, i32p]
        L.helm_device_check.restype = ctypes.c_int
        L.helm_device_check.argtypes = [ctypes.c_int]
        L.helm_arch_supported.restype = ctypes.c_int
        L.helm_arch_supported.argtypes = [ctypes.c_char_p]
        L.helm_last_error.restype = ctypes.c_char_p
        L.helm_last_error.argtypes = []
        L.helm_status_string.restype = ctypes.c_char_p
        L.helm_status_string.argtypes = [ctypes.c_int]
        L.helm_abi_version.restype = ctypes.c_int
        L.helm_abi_version.argtypes = []
        _lib = L
    return _lib


def helm_last_error() -> str:
    return lib().helm_last_error().decode()


def helm_status_string(status: int) -> str:
    return lib().helm_status_string(status).decode()


def helm_abi_version() -> int:
    return int(lib().helm_abi_version())


def helm_arch_supported(name: str) -> bool:
    return bool(lib().helm_arch_supported(name.encode()))


def helm_device_check(device: int = -1) -> int:
    return int(lib().helm_device_check(device))


def _raise(status: int):
    if status != 0:
        raise HelmError(status, helm_last_error())


def helm_kv_workspace_bytes(shape: HelmShape) -> int:
    n = int(lib().helm_kv_workspace_bytes(ctypes.byref(shape)))
    if n == 0:
        raise HelmError(1, helm_last_error())
    return n


def helm_kv_paged_workspace_bytes(shape: HelmPagedShape) -> int:
    n = int(lib().helm_kv_paged_workspace_bytes(ctypes.byref(shape)))
    if n == 0:
        raise HelmError(1, helm_last_error())
    return n


def _host_i32(a):
    """(pointer, keepalive) of a host int32 buffer from a torch tensor or numpy array."""
    import numpy as np
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(a, dtype=np.int32)
    return ctypes.c_void_p(a.ctypes.data), a


def helm_mapper_check(shape: HelmShape, layer_sel_host) -> int:
    p, keep = _host_i32(layer_sel_host)
    return int(lib().helm_mapper_check(ctypes.byref(shape), p))


def helm_paged_check(shape: HelmPagedShape, src_block_table_host, tgt_block_table_host,
                     cu_seqlens_host) -> int:
    (a, ka), (b, kb), (c, kc) = (_host_i32(x) for x in
                                 (src_block_table_host, tgt_block_table_host, cu_seqlens_host))
    return int(lib().helm_paged_check(ctypes.byref(shape), a, b, c))


# ---------------------------------------------------------------- torch glue
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return HELM_BF16
    if t.dtype == torch.float32:
        return HELM_F32
    raise TypeError(f"unsupported storage dtype {t.dtype} (bfloat16 or float32)")


def _dev_ptr(t, name, dtype=None, shape=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _workspace_ptr(ws, device):
    """(address, bytes) of a caller's workspace: a contiguous tensor on the
    same GPU as the data (any dtype; its size in bytes counts)."""
    import torch
    if not isinstance(ws, torch.Tensor):
        raise TypeError("workspace must be a torch tensor")
    if ws.device.type != "cuda" or ws.device != torch.device(device):
        raise ValueError(f"workspace must live on {device} (got {ws.device})")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def current_stream_ptr(device=None) -> int:
    import torch
    return int(torch.cuda.current_stream(device).cuda_stream)


def _call_shape(shape, device):
    """A copy of the caller's shape for one call, with the launch stream
    resolved (the caller's stream, else torch's current stream on `device`
    at this call); the caller's structure is left as it was."""
    s = type(shape).from_buffer_copy(shape)
    if not s.stream:
        s.stream = current_stream_ptr(device) or None
    return s


def _own_workspace(nbytes, device, stream_ptr):
    """A workspace allocated for one call.  It is freed when the call returns
    while the kernels may still read it on the launch stream, so the caching
    allocator is told that stream uses it (record_stream): the memory is not
    handed to another allocation before that stream's work is done."""
    import torch
    dev = torch.device(device)
    if dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    ptr = int(stream_ptr or 0)
    if ptr != current_stream_ptr(dev):   # allocated on torch's current stream: nothing to record
        launch = torch.cuda.default_stream(dev) if ptr == 0 else torch.cuda.ExternalStream(ptr, device=dev)
        ws.record_stream(launch)
    return ws


def make_shape(src_k, W_k, layer_sel, theta_src: float, theta_tgt: float) -> HelmShape:
    """helm_shape_t from tensor shapes: src_k [L_s,H,T,D], W_k [L_t,H,k*D,D], layer_sel [L_t,k]."""
    L_s, H, T, D = src_k.shape
    L_t, k = layer_sel.shape
    s = HelmShape()
    s.n_src_layers, s.n_tgt_layers, s.n_kv_heads, s.head_dim, s.k = L_s, L_t, H, D, k
    s.dtype = _dtype_code(src_k)
    s.n_tokens = T
    s.rope_theta_src, s.rope_theta_tgt = theta_src, theta_tgt
    return s


def helm_kv_transfer(src_k, src_v, src_pos, tgt_pos, layer_sel, W_k, b_k, W_v, b_v, out_k, out_v,
                     shape: HelmShape, workspace=None) -> None:
    """Enqueues the contiguous transfer on ``shape.stream`` (torch's current
    stream when unset).  ``workspace``: a uint8 device tensor of at least
    helm_kv_workspace_bytes(shape) bytes; allocated here when omitted.
    Raises HelmError on a refused call (nothing is written then)."""
    helm_kv_transfer_stage(HELM_STAGE_ALL, src_k, src_v, src_pos, tgt_pos, layer_sel, W_k, b_k, W_v, b_v,
                           out_k, out_v, shape, workspace)


def _transfer_ptrs(shape, src_k, src_v, src_pos, tgt_pos, layer_sel, W_k, b_k, W_v, b_v, out_k, out_v):
    import torch
    L_s, L_t, H, D, k, T = (shape.n_src_layers, shape.n_tgt_layers, shape.n_kv_heads,
                            shape.head_dim, shape.k, shape.n_tokens)
    dt = torch.bfloat16 if shape.dtype == HELM_BF16 else torch.float32
    return [
        _dev_ptr(src_k, "src_k", dt, (L_s, H, T, D)), _dev_ptr(src_v, "src_v", dt, (L_s, H, T, D)),
        _dev_ptr(src_pos, "src_pos", torch.int32, (T,)), _dev_ptr(tgt_pos, "tgt_pos", torch.int32, (T,)),
        _dev_ptr(layer_sel, "layer_sel", torch.int32, (L_t, k)),
        _dev_ptr(W_k, "W_k", dt, (L_t, H, k * D, D)), _dev_ptr(b_k, "b_k", torch.float32, (L_t, H, D)),
        _dev_ptr(W_v, "W_v", dt, (L_t, H, k * D, D)), _dev_ptr(b_v, "b_v", torch.float32, (L_t, H, D)),
        _dev_ptr(out_k, "out_k", dt, (L_t, H, T, D)), _dev_ptr(out_v, "out_v", dt, (L_t, H, T, D)),
    ]


def helm_kv_transfer_stage(stages: int, src_k, src_v, src_pos, tgt_pos, layer_sel, W_k, b_k, W_v, b_v,
                           out_k, out_v, shape: HelmShape, workspace=None) -> None:
    """One or both stages of the transfer (HELM_STAGE_TABLES, HELM_STAGE_MAP,
    HELM_STAGE_ALL); the map stage reads the tables an earlier tables stage
    left in the same ``workspace``."""
    ptrs = _transfer_ptrs(shape, src_k, src_v, src_pos, tgt_pos, layer_sel, W_k, b_k, W_v, b_v, out_k, out_v)
    s = _call_shape(shape, src_k.device)
    if stages != HELM_STAGE_ALL and workspace is None:
        raise ValueError("a single stage needs the caller's workspace (the tables live there)")
    if workspace is None:
        workspace = _own_workspace(helm_kv_workspace_bytes(s), src_k.device, s.stream)
    s.workspace, s.workspace_bytes = _workspace_ptr(workspace, src_k.device)
    _raise(lib().helm_kv_transfer_stage(int(stages), *ptrs, ctypes.byref(s)))


def helm_kv_transfer_noalloc(src_k, src_v, src_pos, tgt_pos, layer_sel, W_k, b_k, W_v, b_v, out_k, out_v,
                             shape: HelmShape) -> None:
    """helm_kv_transfer without a workspace: the tables go to the library's
    static per-GPU scratch (helm_kv_noalloc_max_bytes(); up to 65,536 tokens
    at head_dim 128).  Nothing is allocated, here or in the library.  Calls
    that overlap on one GPU share that scratch and race."""
    ptrs = _transfer_ptrs(shape, src_k, src_v, src_pos, tgt_pos, layer_sel, W_k, b_k, W_v, b_v, out_k, out_v)
    s = _call_shape(shape, src_k.device)
    _raise(lib().helm_kv_transfer_noalloc(*ptrs, ctypes.byref(s)))


def helm_kv_noalloc_max_bytes() -> int:
    return int(lib().helm_kv_noalloc_max_bytes())


def helm_kv_transfer_path(src_k, src_v, src_pos, tgt_pos, layer_sel, W_k, b_k, W_v, b_v, out_k, out_v,
                          shape: HelmShape) -> int:
    """HELM_PATH_MATRIX or HELM_PATH_PORTABLE: the kernel helm_kv_transfer
    would run with these arguments (nothing is enqueued)."""
    ptrs = _transfer_ptrs(shape, src_k, src_v, src_pos, tgt_pos, layer_sel, W_k, b_k, W_v, b_v, out_k, out_v)
    s = _call_shape(shape, src_k.device)
    path = ctypes.c_int(0)
    _raise(lib().helm_kv_transfer_path(*ptrs, ctypes.byref(s), ctypes.byref(path)))
    return int(path.value)


def helm_kv_wide_workspace_bytes(shape: HelmShape) -> int:
    n = int(lib().helm_kv_wide_workspace_bytes(ctypes.byref(shape)))
    if n == 0:
        raise HelmError(1, helm_last_error())
    return n


def wide_in(k: int, H: int, D: int) -> int:
    """Input width of the wide-input map: k layers x {K, V} x H heads x D."""
    return k * 2 * H * D


def helm_kv_transfer_wide(src_k, src_v, src_pos, tgt_pos, layer_sel, W_k, b_k, W_v, b_v, out_k, out_v,
                          shape: HelmShape, workspace=None) -> None:
    """The wide-input map (see include/helm_kv.h): W_k, W_v [L_t, H, k*2*H*D, D] bf16."""
    helm_kv_transfer_wide_stage(HELM_STAGE_ALL, src_k, src_v, src_pos, tgt_pos, layer_sel, W_k, b_k, W_v, b_v,
                                out_k, out_v, shape, workspace)


def helm_kv_transfer_wide_stage(stages: int, src_k, src_v, src_pos, tgt_pos, layer_sel, W_k, b_k, W_v, b_v,
                                out_k, out_v, shape: HelmShape, workspace=None) -> None:
    """helm_kv_transfer_wide in stages (HELM_STAGE_TABLES: tables, un-rotated
    keys and transposed maps into the workspace; HELM_STAGE_MAP: the product
    reading them)."""
    import torch
    L_s, L_t, H, D, k, T = (shape.n_src_layers, shape.n_tgt_layers, shape.n_kv_heads,
                            shape.head_dim, shape.k, shape.n_tokens)
    IN = wide_in(k, H, D)
    dt = torch.bfloat16
    ptrs = [
        _dev_ptr(src_k, "src_k", dt, (L_s, H, T, D)), _dev_ptr(src_v, "src_v", dt, (L_s, H, T, D)),
        _dev_ptr(src_pos, "src_pos", torch.int32, (T,)), _dev_ptr(tgt_pos, "tgt_pos", torch.int32, (T,)),
        _dev_ptr(layer_sel, "layer_sel", torch.int32, (L_t, k)),
        _dev_ptr(W_k, "W_k", dt, (L_t, H, IN, D)), _dev_ptr(b_k, "b_k", torch.float32, (L_t, H, D)),
        _dev_ptr(W_v, "W_v", dt, (L_t, H, IN, D)), _dev_ptr(b_v, "b_v", torch.float32, (L_t, H, D)),
        _dev_ptr(out_k, "out_k", dt, (L_t, H, T, D)), _dev_ptr(out_v, "out_v", dt, (L_t, H, T, D)),
    ]
    s = _call_shape(shape, src_k.device)
    if workspace is None:
        workspace = _own_workspace(helm_kv_wide_workspace_bytes(s), src_k.device, s.stream)
    s.workspace, s.workspace_bytes = _workspace_ptr(workspace, src_k.device)
    _raise(lib().helm_kv_transfer_wide_stage(int(stages), *ptrs, ctypes.byref(s)))


def helm_kv_cosine(k_mapped, v_mapped, k_ref, v_ref, shape: HelmShape, out=None):
    """KV-cosine diagnostic: [2, L_t, H] float32 on the caches' device, the
    cosine of every (K|V, layer, head) slab of the mapped cache against the
    reference cache (see include/helm_kv.h)."""
    import torch
    L_t, H, D, T = shape.n_tgt_layers, shape.n_kv_heads, shape.head_dim, shape.n_tokens
    dt = torch.bfloat16 if shape.dtype == HELM_BF16 else torch.float32
    ptrs = [_dev_ptr(k_mapped, "k_mapped", dt, (L_t, H, T, D)), _dev_ptr(v_mapped, "v_mapped", dt, (L_t, H, T, D)),
            _dev_ptr(k_ref, "k_ref", dt, (L_t, H, T, D)), _dev_ptr(v_ref, "v_ref", dt, (L_t, H, T, D))]
    if out is None:
        out = torch.empty((2, L_t, H), dtype=torch.float32, device=k_mapped.device)
    optr = _dev_ptr(out, "out", torch.float32, (2, L_t, H))
    s = _call_shape(shape, k_mapped.device)
    _raise(lib().helm_kv_cosine(*ptrs, optr, ctypes.byref(s)))
    return out


def make_paged_shape(src_k_pool, tgt_k_pool, W_k, layer_sel, src_block_table, tgt_block_table,
                     n_tokens_total: int, theta_src: float, theta_tgt: float) -> HelmPagedShape:
    """helm_paged_shape_t from tensor shapes (pools [L, n_blocks, B, H, D])."""
    L_s, nsb, B, H, D = src_k_pool.shape
    L_t, ntb = tgt_k_pool.shape[:2]
    k = layer_sel.shape[1]
    s = HelmPagedShape()
    s.n_src_layers, s.n_tgt_layers, s.n_kv_heads, s.head_dim, s.k = L_s, L_t, H, D, k
    s.dtype = _dtype_code(src_k_pool)
    s.block_size, s.n_requests = B, src_block_table.shape[0]
    s.max_blocks_src, s.max_blocks_tgt = src_block_table.shape[1], tgt_block_table.shape[1]
    s.n_src_blocks, s.n_tgt_blocks = nsb, ntb
    s.n_tokens_total = n_tokens_total
    s.rope_theta_src, s.rope_theta_tgt = theta_src, theta_tgt
    return s


def helm_kv_transfer_paged(src_k_pool, src_v_pool, src_block_table, tgt_block_table, cu_seqlens,
                           src_pos, tgt_pos, layer_sel, W_k, b_k, W_v, b_v, tgt_k_pool, tgt_v_pool,
                           shape: HelmPagedShape, workspace=None) -> None:
    """Enqueues the paged transfer; same conventions as helm_kv_transfer."""
    import torch
    s = shape
    dt = torch.bfloat16 if s.dtype == HELM_BF16 else torch.float32
    L_s, L_t, H, D, k, B = s.n_src_layers, s.n_tgt_layers, s.n_kv_heads, s.head_dim, s.k, s.block_size
    N, R = s.n_tokens_total, s.n_requests
    ptrs = [
        _dev_ptr(src_k_pool, "src_k_pool", dt, (L_s, s.n_src_blocks, B, H, D)),
        _dev_ptr(src_v_pool, "src_v_pool", dt, (L_s, s.n_src_blocks, B, H, D)),
        _dev_ptr(src_block_table, "src_block_table", torch.int32, (R, s.max_blocks_src)),
        _dev_ptr(tgt_block_table, "tgt_block_table", torch.int32, (R, s.max_blocks_tgt)),
        _dev_ptr(cu_seqlens, "cu_seqlens", torch.int32, (R + 1,)),
        _dev_ptr(src_pos, "src_pos", torch.int32, (N,)), _dev_ptr(tgt_pos, "tgt_pos", torch.int32, (N,)),
        _dev_ptr(layer_sel, "layer_sel", torch.int32, (L_t, k)),
        _dev_ptr(W_k, "W_k", dt, (L_t, H, k * D, D)), _dev_ptr(b_k, "b_k", torch.float32, (L_t, H, D)),
        _dev_ptr(W_v, "W_v", dt, (L_t, H, k * D, D)), _dev_ptr(b_v, "b_v", torch.float32, (L_t, H, D)),
        _dev_ptr(tgt_k_pool, "tgt_k_pool", dt, (L_t, s.n_tgt_blocks, B, H, D)),
        _dev_ptr(tgt_v_pool, "tgt_v_pool", dt, (L_t, s.n_tgt_blocks, B, H, D)),
    ]
    s = _call_shape(s, src_k_pool.device)
    if workspace is None:
        workspace = _own_workspace(helm_kv_paged_workspace_bytes(s), src_k_pool.device, s.stream)
    s.workspace, s.workspace_bytes = _workspace_ptr(workspace, src_k_pool.device)
    _raise(lib().helm_kv_transfer_paged(*ptrs, ctypes.byref(s)))


def ridge_shape(n_groups: int, n_obs: int, in_features: int, out_features: int = 128, lam: float = 0.01,
                dtype: int = HELM_BF16) -> HelmRidgeShape:
    s = HelmRidgeShape()
    s.n_groups, s.n_obs, s.in_features, s.out_features = n_groups, n_obs, in_features, out_features
    s.dtype, s.lambda_ = dtype, lam
    return s


def helm_ridge_workspace_bytes(shape: HelmRidgeShape) -> int:
    n = int(lib().helm_ridge_workspace_bytes(ctypes.byref(shape)))
    if n == 0:
        raise HelmError(1, helm_last_error())
    return n


def helm_ridge_fit(X, Y, lam: float = 0.01, W=None, b=None, workspace=None, stages: int = HELM_STAGE_ALL):
    """Ridge fit of G maps (see include/helm_kv.h): X [G, N, IN] and Y
    [G, N, 128] bf16 on the GPU.  Returns (W [G, IN, 128], b [G, 128]) fp32,
    enqueued on torch's current stream."""
    import torch
    G, N, IN = X.shape
    D = Y.shape[2]
    shape = ridge_shape(G, N, IN, D, lam)
    if W is None:
        W = torch.empty((G, IN, D), dtype=torch.float32, device=X.device)
    if b is None:
        b = torch.empty((G, D), dtype=torch.float32, device=X.device)
    ptrs = [_dev_ptr(X, "X", torch.bfloat16, (G, N, IN)), _dev_ptr(Y, "Y", torch.bfloat16, (G, N, D)),
            _dev_ptr(W, "W", torch.float32, (G, IN, D)), _dev_ptr(b, "b", torch.float32, (G, D))]
    shape.stream = current_stream_ptr(X.device)
    if workspace is None:
        workspace = _own_workspace(helm_ridge_workspace_bytes(shape), X.device, shape.stream)
    shape.workspace, shape.workspace_bytes = _workspace_ptr(workspace, X.device)
    _raise(lib().helm_ridge_fit_stage(int(stages), *ptrs, ctypes.byref(shape)))
    return W, b

"""fp64 CPU oracle of the cross-model KV-cache transfer — TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it and
shares no code with it.  The arithmetic lives in ``helm_oracle.c`` (plain C,
fp64); this module only marshals numpy arrays into it.

What it computes, per target layer l, KV head h and token t (pages: "Helm
Intelligent Routing", section "Why carrying the cache across is the hard
part"; the Qwen3 cache-mapping write-up, section "A linear bridge, strangely
enough, suffices", its fit/map listing and its strip/map/apply diagram):

    x_k = concat_j R(-src_pos[t]) src_k[layer_sel[l, j], h, t, :]
    x_v = concat_j src_v[layer_sel[l, j], h, t, :]
    out_k[l, h, t, :] = R(+tgt_pos[t]) (x_k @ W_k[l, h] + b_k[l, h])
    out_v[l, h, t, :] = x_v @ W_v[l, h] + b_v[l, h]

with R the rotate-half RoPE rotation.  In ``quantize_content`` mode x_k is
rounded once to the storage dtype before the product.

``transfer_wide_rows`` is the wide-input map (the Qwen3 write-up's full
mapper): x concatenates the K (un-rotated) and V features of all heads of the
k selected source layers, IN = k*2*H*D, one (IN, D) map per target head and
K|V.

``kv_cosine`` is the KV-cosine diagnostic ("Helm Intelligent Routing", the
retention / KL / KV-cosine table): per (layer, head) slab, the cosine of a
mapped cache and a reference cache taken as flat vectors, in fp64.

``ridge_fit`` is the calibration's ridge fit of the maps (the Qwen3
write-up's closed-form fit: centred data, lambda = 0.01, the bias from the
means), in numpy fp64 with LAPACK's solve as one step.

Pins: every function here is checked in tests/test_oracle_pins.py against
closed forms, invariants, special cases that reduce to library routines,
an independent complex-number / matrix-exponential formulation and a
pure-Python brute force.  No function is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import numpy as np
import scipy.linalg

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhelm_oracle.so")

BF16 = 0
F32 = 1


class _Problem(ctypes.Structure):
    _fields_ = [
        ("n_src_layers", ctypes.c_int32),
        ("n_tgt_layers", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("k", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("quantize_content", ctypes.c_int32),
        ("n_threads", ctypes.c_int32),
        ("n_tokens", ctypes.c_int64),
        ("theta_src", ctypes.c_double),
        ("theta_tgt", ctypes.c_double),
    ]


class _Paged(ctypes.Structure):
    _fields_ = [
        ("block_size", ctypes.c_int32),
        ("n_requests", ctypes.c_int32),
        ("max_blocks_src", ctypes.c_int32),
        ("max_blocks_tgt", ctypes.c_int32),
        ("n_src_blocks", ctypes.c_int32),
        ("n_tgt_blocks", ctypes.c_int32),
    ]


@dataclass
class Problem:
    n_src_layers: int
    n_tgt_layers: int
    n_kv_heads: int
    head_dim: int
    k: int
    n_tokens: int = 0
    theta_src: float = 1e6
    theta_tgt: float = 1e6
    dtype: int = BF16
    quantize_content: bool = True
    n_threads: int = 0

    def _c(self) -> _Problem:
        return _Problem(self.n_src_layers, self.n_tgt_layers, self.n_kv_heads,
                        self.head_dim, self.k, self.dtype,
                        1 if self.quantize_content else 0, self.n_threads,
                        self.n_tokens, self.theta_src, self.theta_tgt)


@dataclass
class Paged:
    block_size: int
    n_requests: int
    max_blocks_src: int
    max_blocks_tgt: int
    n_src_blocks: int
    n_tgt_blocks: int

    def _c(self) -> _Paged:
        return _Paged(self.block_size, self.n_requests, self.max_blocks_src,
                      self.max_blocks_tgt, self.n_src_blocks, self.n_tgt_blocks)


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build()
        L = ctypes.CDLL(LIB_PATH)
        vp, i64p, dp = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)
        L.oracle_round_bf16.restype = ctypes.c_double
        L.oracle_round_bf16.argtypes = [ctypes.c_double]
        L.oracle_round_f32.restype = ctypes.c_double
        L.oracle_round_f32.argtypes = [ctypes.c_double]
        L.oracle_rope_freq.restype = ctypes.c_double
        L.oracle_rope_freq.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_double]
        L.oracle_rope.restype = None
        L.oracle_rope.argtypes = [dp, dp, ctypes.c_int32, ctypes.c_double, ctypes.c_double]
        L.oracle_transfer_rows.restype = ctypes.c_int
        L.oracle_transfer_rows.argtypes = [ctypes.POINTER(_Problem)] + [vp] * 9 + [ctypes.c_int64, i64p, dp, dp]
        L.oracle_transfer_paged_rows.restype = ctypes.c_int
        L.oracle_transfer_paged_rows.argtypes = ([ctypes.POINTER(_Problem), ctypes.POINTER(_Paged)]
                                                + [vp] * 12 + [ctypes.c_int64, i64p, dp, dp, i64p])
        L.oracle_max_threads.restype = ctypes.c_int
        L.oracle_max_threads.argtypes = []
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _check_data(a: np.ndarray, dtype: int, name: str) -> None:
    want = np.uint16 if dtype == BF16 else np.float32
    if a.dtype != want:
        raise TypeError(f"{name}: expected {np.dtype(want).name} storage, got {a.dtype}")


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def round_bf16(x) -> np.ndarray:
    """Rounds fp64 values once to bf16 (nearest, ties to even); returns fp64."""
    f = lib().oracle_round_bf16
    x = np.asarray(x, dtype=np.float64)
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.float64).reshape(x.shape)


def rope_freq(i: int, D: int, theta: float) -> float:
    return float(lib().oracle_rope_freq(i, D, theta))


def rope(vec, p: float, theta: float) -> np.ndarray:
    """Applies R(p; theta) (rotate-half) to one D-vector, in fp64."""
    v = np.ascontiguousarray(np.asarray(vec, dtype=np.float64))
    out = np.empty_like(v)
    dp = ctypes.POINTER(ctypes.c_double)
    lib().oracle_rope(v.ctypes.data_as(dp), out.ctypes.data_as(dp), v.shape[-1], float(p), float(theta))
    return out


def rope_rows(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """R(pos[t]) applied to every row x[..., t, :] (fp64 in, fp64 out)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    flat_in = x.reshape(-1, x.shape[-2], x.shape[-1])
    flat_out = out.reshape(flat_in.shape)
    for b in range(flat_in.shape[0]):
        for t in range(flat_in.shape[1]):
            flat_out[b, t] = rope(flat_in[b, t], float(pos[t]), theta)
    return out


def transfer_rows(pb: Problem, src_k, src_v, src_pos, tgt_pos, layer_sel,
                  W_k, b_k, W_v, b_v, rows=None):
    """Contiguous transfer for the given flat rows ((l*H + h)*T + t), or all.

    Caches / W are numpy uint16 (bf16 bits) or float32 per ``pb.dtype``;
    biases float32; positions and layer_sel int32.  Returns fp64
    (out_k, out_v), each [n_rows, D] (or [L_t, H, T, D] when rows is None).
    """
    for a, n in ((src_k, "src_k"), (src_v, "src_v"), (W_k, "W_k"), (W_v, "W_v")):
        _check_data(a, pb.dtype, n)
    src_pos = np.ascontiguousarray(src_pos, dtype=np.int32)
    tgt_pos = np.ascontiguousarray(tgt_pos, dtype=np.int32)
    layer_sel = np.ascontiguousarray(layer_sel, dtype=np.int32)
    b_k = np.ascontiguousarray(b_k, dtype=np.float32)
    b_v = np.ascontiguousarray(b_v, dtype=np.float32)
    D = pb.head_dim
    if rows is None:
        n = pb.n_tgt_layers * pb.n_kv_heads * pb.n_tokens
        rows_p = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows.size
        rows_p = rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    out_k = np.empty((n, D), dtype=np.float64)
    out_v = np.empty((n, D), dtype=np.float64)
    dp = ctypes.POINTER(ctypes.c_double)
    c = pb._c()
    rc = lib().oracle_transfer_rows(
        ctypes.byref(c), _ptr(src_k), _ptr(src_v), _ptr(src_pos), _ptr(tgt_pos),
        _ptr(layer_sel), _ptr(W_k), _ptr(b_k), _ptr(W_v), _ptr(b_v),
        n, rows_p, out_k.ctypes.data_as(dp), out_v.ctypes.data_as(dp))
    if rc != 0:
        raise ValueError("oracle_transfer_rows: invalid arguments")
    if rows is None:
        shape = (pb.n_tgt_layers, pb.n_kv_heads, pb.n_tokens, D)
        return out_k.reshape(shape), out_v.reshape(shape)
    return out_k, out_v


def transfer_paged_rows(pb: Problem, pg: Paged, src_k_pool, src_v_pool, src_bt, tgt_bt,
                        cu_seqlens, src_pos, tgt_pos, layer_sel, W_k, b_k, W_v, b_v,
                        rows=None):
    """Paged transfer for flat rows ((l*H + h)*N + n) over packed tokens n.

    Returns (out_k, out_v, dst_off): fp64 [n_rows, D] each, and the element
    offset of every row's destination inside the target pool.
    """
    for a, n in ((src_k_pool, "src_k_pool"), (src_v_pool, "src_v_pool"), (W_k, "W_k"), (W_v, "W_v")):
        _check_data(a, pb.dtype, n)
    arrs = [np.ascontiguousarray(a, dtype=np.int32) for a in (src_bt, tgt_bt, cu_seqlens, src_pos, tgt_pos, layer_sel)]
    src_bt, tgt_bt, cu_seqlens, src_pos, tgt_pos, layer_sel = arrs
    b_k = np.ascontiguousarray(b_k, dtype=np.float32)
    b_v = np.ascontiguousarray(b_v, dtype=np.float32)
    D = pb.head_dim
    N = int(cu_seqlens[-1])
    if rows is None:
        n = pb.n_tgt_layers * pb.n_kv_heads * N
        rows_p = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows.size
        rows_p = rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    out_k = np.empty((n, D), dtype=np.float64)
    out_v = np.empty((n, D), dtype=np.float64)
    dst = np.empty((n,), dtype=np.int64)
    dp = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    c, g = pb._c(), pg._c()
    rc = lib().oracle_transfer_paged_rows(
        ctypes.byref(c), ctypes.byref(g), _ptr(src_k_pool), _ptr(src_v_pool),
        _ptr(src_bt), _ptr(tgt_bt), _ptr(cu_seqlens), _ptr(src_pos), _ptr(tgt_pos),
        _ptr(layer_sel), _ptr(W_k), _ptr(b_k), _ptr(W_v), _ptr(b_v),
        n, rows_p, out_k.ctypes.data_as(dp), out_v.ctypes.data_as(dp), dst.ctypes.data_as(i64p))
    if rc != 0:
        raise ValueError("oracle_transfer_paged_rows: invalid arguments")
    return out_k, out_v, dst


def encode_keys(content, pos, theta: float, dtype: int, n_threads: int = 0) -> np.ndarray:
    """Position-encodes content keys the way a model stores them in its cache.

    ``content`` is [n_layers, H, T, D] in storage dtype (uint16 bf16 bits or
    float32); returns the same shape and storage holding
    round_dtype(R(pos[t]; theta) content[l, h, t, :]).
    """
    _check_data(content, dtype, "content")
    content = np.ascontiguousarray(content)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    L_, H, T, D = content.shape
    if pos.shape != (T,):
        raise ValueError("pos must have one entry per token")
    L = lib()
    if not hasattr(L, "_enc_set"):
        L.oracle_encode_keys.restype = ctypes.c_int
        L.oracle_encode_keys.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                         ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int32, ctypes.c_void_p, ctypes.c_double,
                                         ctypes.c_int32]
        L._enc_set = True
    out = np.empty_like(content)
    rc = L.oracle_encode_keys(_ptr(content), _ptr(out), dtype, L_, H, T, D, _ptr(pos),
                              float(theta), n_threads)
    if rc != 0:
        raise ValueError("oracle_encode_keys: invalid arguments")
    return out


def kv_cosine(a, b, dtype: int, n_threads: int = 0) -> np.ndarray:
    """Per-slab cosine of two caches [..., T, D] (storage dtype: uint16 bf16
    bits or float32): for every index of the leading dimensions, the cosine
    between the two [T, D] slabs taken as flat vectors, in fp64 (NaN for a
    slab of zeros).  Returns the leading shape, fp64.  "Helm Intelligent
    Routing", the retention / KL / KV-cosine table (KV cosine)."""
    _check_data(a, dtype, "a")
    _check_data(b, dtype, "b")
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    if a.shape != b.shape or a.ndim < 2:
        raise ValueError("a and b must be caches of one shape [..., T, D]")
    lead = a.shape[:-2]
    n_slabs = int(np.prod(lead)) if lead else 1
    n_elems = a.shape[-2] * a.shape[-1]
    L = lib()
    if not hasattr(L, "_cos_set"):
        L.oracle_kv_cosine.restype = ctypes.c_int
        L.oracle_kv_cosine.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.POINTER(ctypes.c_double), ctypes.c_int32]
        L._cos_set = True
    out = np.empty(n_slabs, dtype=np.float64)
    rc = L.oracle_kv_cosine(_ptr(a), _ptr(b), dtype, n_slabs, n_elems,
                            out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), n_threads)
    if rc != 0:
        raise ValueError("oracle_kv_cosine: invalid arguments")
    return out.reshape(lead)


def wide_in(k: int, H: int, D: int) -> int:
    """Input width of the wide-input map: k layers x {K, V} x H heads x D."""
    return k * 2 * H * D


def transfer_wide_rows(pb: Problem, src_k, src_v, src_pos, tgt_pos, layer_sel,
                       W_k, b_k, W_v, b_v, rows=None):
    """Wide-input transfer (the Qwen3 write-up's full mapper: x concatenates
    the K and V features of all heads of the k selected source layers) for
    the given flat rows ((l*H + h)*T + t), or all.  W_k / W_v are
    [L_t, H, k*2*H*D, D]; feature order (j, K|V, source head, d), keys
    un-rotated.  Returns fp64 (out_k, out_v) like ``transfer_rows``."""
    for a, n in ((src_k, "src_k"), (src_v, "src_v"), (W_k, "W_k"), (W_v, "W_v")):
        _check_data(a, pb.dtype, n)
    src_pos = np.ascontiguousarray(src_pos, dtype=np.int32)
    tgt_pos = np.ascontiguousarray(tgt_pos, dtype=np.int32)
    layer_sel = np.ascontiguousarray(layer_sel, dtype=np.int32)
    b_k = np.ascontiguousarray(b_k, dtype=np.float32)
    b_v = np.ascontiguousarray(b_v, dtype=np.float32)
    D = pb.head_dim
    IN = wide_in(pb.k, pb.n_kv_heads, D)
    for a, n in ((W_k, "W_k"), (W_v, "W_v")):
        if a.shape != (pb.n_tgt_layers, pb.n_kv_heads, IN, D):
            raise ValueError(f"{n} must be [L_t, H, {IN}, D], got {a.shape}")
    L = lib()
    if not hasattr(L, "_wide_set"):
        vp, i64p, dp = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)
        L.oracle_transfer_wide_rows.restype = ctypes.c_int
        L.oracle_transfer_wide_rows.argtypes = [ctypes.POINTER(_Problem)] + [vp] * 9 + [ctypes.c_int64, i64p, dp, dp]
        L._wide_set = True
    if rows is None:
        n = pb.n_tgt_layers * pb.n_kv_heads * pb.n_tokens
        rows_p = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows.size
        rows_p = rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    out_k = np.empty((n, D), dtype=np.float64)
    out_v = np.empty((n, D), dtype=np.float64)
    dp = ctypes.POINTER(ctypes.c_double)
    c = pb._c()
    rc = L.oracle_transfer_wide_rows(
        ctypes.byref(c), _ptr(src_k), _ptr(src_v), _ptr(src_pos), _ptr(tgt_pos),
        _ptr(layer_sel), _ptr(np.ascontiguousarray(W_k)), _ptr(b_k), _ptr(np.ascontiguousarray(W_v)), _ptr(b_v),
        n, rows_p, out_k.ctypes.data_as(dp), out_v.ctypes.data_as(dp))
    if rc != 0:
        raise ValueError("oracle_transfer_wide_rows: invalid arguments")
    if rows is None:
        shape = (pb.n_tgt_layers, pb.n_kv_heads, pb.n_tokens, D)
        return out_k.reshape(shape), out_v.reshape(shape)
    return out_k, out_v


def _decode(a, dtype):
    """Storage -> fp64: bf16 bits (uint16) are the upper half of an fp32;
    float arrays are taken as they are."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        if dtype != BF16:
            raise TypeError("uint16 storage is bf16")
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def ridge_fit(x, y, lam: float = 0.01, dtype: int = BF16):
    """The ridge fit of the per-(target layer, head, K|V) maps, fp64 (the
    Qwen3 cache-mapping write-up, section "A linear bridge, strangely enough,
    suffices": each target head's key map and value map are fitted
    separately by ridge regression, lambda = 0.01, with an unpenalised bias).

    x: [G, N, IN] observations of the map's input per group (bf16 storage as
    uint16, or float); y: [G, N, D] the targets.  For every group g the fit
    is the minimiser of the ridge objective
        |x[g] W + 1 b - y[g]|^2 + lam |W|^2        (b not penalised),
    written as one ordinary least-squares problem on the augmented system
        [ x[g]          1 ] [W]   [ y[g] ]
        [ sqrt(lam) I   0 ] [b] = [  0   ]
    and solved by LAPACK's SVD-based least squares (gelsd, through
    scipy.linalg.lstsq) in fp64.  (The write-up's listing reaches the same minimiser by centring x
    and y and solving the normal equations; the pins check the two agree.)
    Returns (W [G, IN, D], b [G, D]) in fp64."""
    X = _decode(x, dtype)
    Y = _decode(y, dtype)
    if X.ndim != 3 or Y.ndim != 3 or X.shape[:2] != Y.shape[:2]:
        raise ValueError("x [G, N, IN] and y [G, N, D] must share G and N")
    if lam < 0:
        raise ValueError("lambda must be >= 0")
    G, N, IN = X.shape
    D = Y.shape[2]
    if N < 1:
        raise ValueError("the fit needs at least one observation")
    W = np.empty((G, IN, D))
    b = np.empty((G, D))
    for g in range(G):
        A = np.zeros((N + IN, IN + 1), order="F")
        A[:N, :IN] = X[g]
        A[:N, IN] = 1.0
        A[N:, :IN] = math.sqrt(lam) * np.eye(IN)
        rhs = np.zeros((N + IN, D), order="F")
        rhs[:N] = Y[g]
        sol = scipy.linalg.lstsq(A, rhs, lapack_driver="gelsd", overwrite_a=True, overwrite_b=True,
                                 check_finite=False)[0]
        W[g] = sol[:IN]
        b[g] = sol[IN]
    return W, b

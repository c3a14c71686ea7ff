"""The C ABI without a GPU: the library loads, exports every declared entry
point, and refuses bad calls with the specific status before any device work.

None of these tests launches a kernel.  Calls that pass fake device pointers
always carry a defect that host validation rejects first.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import cross_model_kv_helm_amd as hk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "helm_kv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(helm_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_abi():
    names = declared_functions()
    assert "helm_kv_transfer" in names and "helm_kv_transfer_paged" in names
    assert set(names) == set(hk.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = hk.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_abi_version_and_status_strings():
    assert hk.helm_abi_version() == 1
    for code, name in hk.STATUS.items():
        assert hk.helm_status_string(code) == name
    assert hk.helm_status_string(99) == "unknown"


@pytest.mark.parametrize("name,ok", [("gfx950", True), ("gfx950:sramecc+:xnack-", True),
                                     ("gfx942", False), ("gfx9500", False), ("gfx90a", False),
                                     ("gfx1100", False), ("", False)])
def test_arch_gate_pure_function(name, ok):
    assert hk.helm_arch_supported(name) is ok


def shape(**kw):
    s = hk.HelmShape()
    s.n_src_layers, s.n_tgt_layers, s.n_kv_heads, s.head_dim, s.k = 40, 64, 8, 128, 4
    s.dtype, s.n_tokens = hk.HELM_BF16, 32768
    s.rope_theta_src = s.rope_theta_tgt = 1e6
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def test_workspace_bytes():
    s = shape()
    n = hk.helm_kv_workspace_bytes(s)
    assert n == 2 * 32768 * 64 * 8                      # two fp32 (cos, sin) tables
    assert n % 256 == 0
    s.n_tokens = 0
    assert hk.helm_kv_workspace_bytes(s) == 256


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 127, 2), ("head_dim", 96, 2), ("head_dim", 0, 2), ("k", 0, 1), ("k", 41, 1),
    ("dtype", 7, 5), ("n_src_layers", 0, 1), ("n_kv_heads", 0, 1), ("rope_theta_src", 0.0, 1),
    ("rope_theta_tgt", float("inf"), 1), ("n_tokens", -1, 1)])
def test_invalid_shapes_refused(field, value, status):
    s = shape(**{field: value})
    fake = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(11)]
    rc = hk.lib().helm_kv_transfer(*fake, ctypes.byref(s))
    assert rc == status, hk.helm_last_error()
    assert hk.helm_last_error()


@pytest.mark.parametrize("stages", [0, 4, -1])
def test_invalid_stage_refused(stages):
    s = shape()
    fake = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(11)]
    assert hk.lib().helm_kv_transfer_stage(stages, *fake, ctypes.byref(s)) == 1
    assert "stages" in hk.helm_last_error()


def test_null_pointer_refused():
    s = shape()
    ptrs = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(11)]
    ptrs[5] = ctypes.c_void_p(0)
    assert hk.lib().helm_kv_transfer(*ptrs, ctypes.byref(s)) == 1
    assert hk.lib().helm_kv_transfer(*ptrs, None) == 1


def test_alias_refused():
    s = shape(n_tokens=16, n_src_layers=2, n_tgt_layers=2, k=1, n_kv_heads=1)
    base = 0x10000000
    ptrs = [ctypes.c_void_p(base + 0x1000000 * i) for i in range(11)]
    ptrs[9] = ptrs[0]          # out_k on top of src_k
    assert hk.lib().helm_kv_transfer(*ptrs, ctypes.byref(s)) == 8
    assert "out_k overlaps src_k" in hk.helm_last_error()


def test_workspace_checks():
    s = shape(n_tokens=16, n_src_layers=2, n_tgt_layers=2, k=1, n_kv_heads=1)
    ptrs = [ctypes.c_void_p(0x10000000 + 0x1000000 * i) for i in range(11)]
    assert hk.lib().helm_kv_transfer(*ptrs, ctypes.byref(s)) == 7       # no workspace
    s.workspace, s.workspace_bytes = 0x40000000, 16
    assert hk.lib().helm_kv_transfer(*ptrs, ctypes.byref(s)) == 7       # too small
    s.workspace, s.workspace_bytes = 0x40000004, 1 << 20
    assert hk.lib().helm_kv_transfer(*ptrs, ctypes.byref(s)) == 7       # misaligned
    assert "aligned" in hk.helm_last_error()


def test_path_query_checks_like_the_transfer():
    """helm_kv_transfer_path runs the transfer's checks (same statuses) and
    needs no workspace; with every argument valid it stops only at the
    device gate (no GPU here) or reports a path."""
    s = shape(n_tokens=16, n_src_layers=2, n_tgt_layers=2, k=1, n_kv_heads=1)
    ptrs = [ctypes.c_void_p(0x10000000 + 0x1000000 * i) for i in range(11)]
    path = ctypes.c_int(0)
    assert hk.lib().helm_kv_transfer_path(*ptrs, ctypes.byref(s), None) == 1
    assert "path_out" in hk.helm_last_error()
    bad = list(ptrs)
    bad[9] = bad[0]
    assert hk.lib().helm_kv_transfer_path(*bad, ctypes.byref(s), ctypes.byref(path)) == 8
    assert hk.lib().helm_kv_transfer_path(*ptrs, ctypes.byref(shape(head_dim=96)), ctypes.byref(path)) == 2
    rc = hk.lib().helm_kv_transfer_path(*ptrs, ctypes.byref(s), ctypes.byref(path))
    if _gpu_present():
        assert rc == 0 and path.value in (hk.HELM_PATH_MATRIX, hk.HELM_PATH_PORTABLE)
    else:
        assert rc == 4 and path.value == 0


def test_mapper_check():
    s = shape(n_src_layers=5, n_tgt_layers=3, k=2)
    good = np.array([[0, 4], [3, 3], [1, 2]], np.int32)
    assert hk.helm_mapper_check(s, good) == 0
    bad = good.copy()
    bad[2, 1] = 5
    assert hk.helm_mapper_check(s, bad) == 3
    assert "layer_sel[2][1] = 5" in hk.helm_last_error()
    bad[2, 1] = -1
    assert hk.helm_mapper_check(s, bad) == 3


def paged_shape(**kw):
    s = hk.HelmPagedShape()
    s.n_src_layers, s.n_tgt_layers, s.n_kv_heads, s.head_dim, s.k = 4, 4, 2, 128, 2
    s.dtype, s.block_size, s.n_requests = hk.HELM_BF16, 16, 2
    s.max_blocks_src = s.max_blocks_tgt = 3
    s.n_src_blocks, s.n_tgt_blocks = 8, 6
    s.n_tokens_total = 40
    s.rope_theta_src = s.rope_theta_tgt = 1e6
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def test_paged_check():
    s = paged_shape()
    cu = np.array([0, 17, 40], np.int32)       # 2 pages + 2 pages
    sbt = np.array([[5, 1, -1], [7, 0, -1]], np.int32)
    tbt = np.array([[2, 3, -1], [0, 5, -1]], np.int32)
    assert hk.helm_paged_check(s, sbt, tbt, cu) == 0, hk.helm_last_error()
    t2 = tbt.copy(); t2[1, 1] = 2
    assert hk.helm_paged_check(s, sbt, t2, cu) == 9 and "used twice" in hk.helm_last_error()
    s2 = sbt.copy(); s2[0, 1] = 8
    assert hk.helm_paged_check(s, s2, tbt, cu) == 9
    assert hk.helm_paged_check(s, sbt, tbt, np.array([0, 17, 12], np.int32)) == 9
    assert hk.helm_paged_check(s, sbt, tbt, np.array([1, 17, 40], np.int32)) == 9
    assert hk.helm_paged_check(s, sbt, tbt, np.array([0, 17, 70], np.int32)) == 9   # needs 4 pages
    assert hk.helm_paged_check(paged_shape(n_tokens_total=41), sbt, tbt, cu) == 9


def test_paged_workspace_bytes():
    s = paged_shape()
    n = hk.helm_kv_paged_workspace_bytes(s)
    assert n == 2 * (48 * 64 * 8) + 2 * 256          # 40 tokens: tables padded to whole 16-token blocks


def test_paged_invalid_refused():
    s = paged_shape(block_size=0)
    fake = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(14)]
    assert hk.lib().helm_kv_transfer_paged(*fake, ctypes.byref(s)) == 1
    s = paged_shape(head_dim=80)
    assert hk.lib().helm_kv_transfer_paged(*fake, ctypes.byref(s)) == 2


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_gpu_present(), reason="checks the no-device path")
def test_no_device():
    assert hk.helm_device_check(-1) == 4
    assert hk.helm_device_check(0) == 4


def test_kv_cosine_refusals_before_any_device_access():
    """helm_kv_cosine: argument errors are reported without touching a
    device: no shape, no output, a NULL cache with tokens, an output that
    overlaps a cache, an invalid shape field."""
    L = hk.lib()
    s = shape(n_tokens=64)
    caches = [ctypes.c_void_p(0x10000000 * (i + 1)) for i in range(4)]
    out = ctypes.c_void_p(0x70000000)
    assert L.helm_kv_cosine(*caches, out, None) == 1
    assert L.helm_kv_cosine(*caches, None, ctypes.byref(s)) == 1
    assert "cos_out" in hk.helm_last_error()
    assert L.helm_kv_cosine(caches[0], None, caches[2], caches[3], out, ctypes.byref(s)) == 1
    # cache bytes: 64 layers * 8 heads * 64 tokens * 128 * 2 = 8 MiB; an output inside k_ref overlaps it
    inside = ctypes.c_void_p(0x30000000 + 4096)
    assert L.helm_kv_cosine(*caches, inside, ctypes.byref(s)) == 8
    assert "overlaps k_ref" in hk.helm_last_error()
    assert L.helm_kv_cosine(*caches, out, ctypes.byref(shape(n_tokens=64, head_dim=96))) == 2
    assert L.helm_kv_cosine(*caches, out, ctypes.byref(shape(n_tokens=-1))) == 1


def test_wide_map_workspace_and_refusals():
    """helm_kv_transfer_wide / helm_kv_wide_workspace_bytes: bf16 and
    head_dim 128 only; the workspace holds the two RoPE tables, the
    un-rotated source keys and both transposed maps."""
    s = shape(n_tokens=32768)
    IN = hk.wide_in(4, 8, 128)
    assert IN == 8192
    n = hk.helm_kv_wide_workspace_bytes(s)
    assert n == 2 * 32768 * 64 * 8 + 40 * 8 * 32768 * 128 * 2 + 2 * 64 * 8 * 128 * IN * 2
    L = hk.lib()
    fake = [ctypes.c_void_p((1 << 34) * (i + 1)) for i in range(11)]      # far apart: no overlaps
    assert L.helm_kv_transfer_wide(*fake, ctypes.byref(shape(dtype=hk.HELM_F32))) == 5
    assert "bf16" in hk.helm_last_error()
    assert L.helm_kv_transfer_wide(*fake, ctypes.byref(shape(head_dim=64))) == 2
    assert L.helm_kv_wide_workspace_bytes(ctypes.byref(shape(head_dim=64))) == 0
    assert L.helm_kv_transfer_wide(*fake, ctypes.byref(shape(n_tokens=0))) == 0      # nothing to do
    s = shape(n_tokens=64)
    assert L.helm_kv_transfer_wide(*fake, ctypes.byref(s)) == 7                       # no workspace
    for stages in (1, 2, 3):
        assert L.helm_kv_transfer_wide_stage(stages, *fake, ctypes.byref(s)) == 7
    for stages in (0, 4, -1):
        assert L.helm_kv_transfer_wide_stage(stages, *fake, ctypes.byref(s)) == 1
    # outputs not 16-byte aligned: refused (the epilogue stores 16-byte pieces), before any device access
    ws_s = shape(n_tokens=64)
    ws_s.workspace = ctypes.c_void_p(1 << 40)
    ws_s.workspace_bytes = hk.helm_kv_wide_workspace_bytes(ws_s)
    for bad in (9, 10):                                                       # out_k, out_v
        args = list(fake)
        args[bad] = ctypes.c_void_p(args[bad].value + 2)
        assert L.helm_kv_transfer_wide(*args, ctypes.byref(ws_s)) == 1
        assert "16-byte aligned" in hk.helm_last_error()


def test_ridge_workspace_and_refusals():
    """helm_ridge_fit / helm_ridge_workspace_bytes: bf16, out_features 128,
    in_features a multiple of 128 up to 1024; the workspace holds the fp32
    products and sums and the fp64 solve matrix; every refusal comes before
    any device access."""
    L = hk.lib()
    s = hk.ridge_shape(1024, 131072, 512)
    n = hk.helm_ridge_workspace_bytes(s)
    assert n == 1024 * (512 * 512 * 4 + 512 * 128 * 4 + 640 * 8 + 512 * 640 * 8)   # sums and shifts: 640 * 4 each
    fake = [ctypes.c_void_p((1 << 40) * (i + 1)) for i in range(4)]     # far apart: no overlaps
    assert L.helm_ridge_fit(*fake, ctypes.byref(hk.ridge_shape(2, 100, 256, dtype=hk.HELM_F32))) == 5
    assert "bf16" in hk.helm_last_error()
    assert L.helm_ridge_fit(*fake, ctypes.byref(hk.ridge_shape(2, 100, 256, out_features=64))) == 2
    for IN in (64, 200, 1152):
        assert L.helm_ridge_fit(*fake, ctypes.byref(hk.ridge_shape(2, 100, IN))) == 2
        assert L.helm_ridge_workspace_bytes(ctypes.byref(hk.ridge_shape(2, 100, IN))) == 0
    assert L.helm_ridge_fit(*fake, ctypes.byref(hk.ridge_shape(2, 0, 256))) == 1
    assert L.helm_ridge_fit(*fake, ctypes.byref(hk.ridge_shape(0, 10, 256))) == 1
    assert L.helm_ridge_fit(*fake, ctypes.byref(hk.ridge_shape(2, 10, 256, lam=-1.0))) == 1
    assert L.helm_ridge_fit(*fake, ctypes.byref(hk.ridge_shape(2, 10, 256, lam=float("nan")))) == 1
    assert L.helm_ridge_fit(*fake, ctypes.byref(hk.ridge_shape(1, 1 << 22, 1024))) == 1   # one group over 4 GB
    s = hk.ridge_shape(2, 100, 256)
    assert L.helm_ridge_fit(*fake, ctypes.byref(s)) == 7                                   # no workspace
    s.workspace, s.workspace_bytes = (1 << 40) * 8, hk.helm_ridge_workspace_bytes(s)
    assert L.helm_ridge_fit(fake[0], fake[1], fake[0], fake[3], ctypes.byref(s)) == 8      # W overlaps X
    assert L.helm_ridge_fit(fake[0], fake[1], fake[2], fake[2], ctypes.byref(s)) == 8      # b overlaps W
    s.workspace = fake[1].value
    assert L.helm_ridge_fit(*fake, ctypes.byref(s)) == 8                                   # workspace overlaps Y
    s.workspace = (1 << 40) * 8 + 16
    assert L.helm_ridge_fit(*fake, ctypes.byref(s)) == 7                                   # misaligned
    for stages in (0, 4):
        assert L.helm_ridge_fit_stage(stages, *fake, ctypes.byref(s)) == 1
    assert L.helm_ridge_fit(None, *fake[1:], ctypes.byref(s)) == 1


def test_binding_refuses_a_workspace_off_the_gpu():
    """The binding hands the library only device memory: a caller's
    workspace on the host, or not contiguous, is refused before any call."""
    import torch
    with pytest.raises(ValueError, match="workspace must live on"):
        hk._workspace_ptr(torch.empty(64, dtype=torch.uint8), torch.device("cuda:0"))
    with pytest.raises(TypeError):
        hk._workspace_ptr(bytearray(64), torch.device("cuda:0"))

"""GPU parity over seeded random shapes: the contiguous and the paged
transfer and the wide-input map through the C ABI against the fp64 oracle,
every output element compared (tolerances: tests/parity.py).

The fixed cases elsewhere pin chosen corners; these draw the shape itself —
source and target layer counts, heads, head_dim 64 or 128, k (up to 5, past
the matrix-core kernel's limit), ragged token counts, bf16 or fp32 storage,
the position pattern and the RoPE base — and, for paged caches, the block
size (1 to 32 slots), the number of requests and their lengths (zero-length
requests included).  Each case also asserts which kernel the library says it
runs (helm_kv_transfer_path): the matrix-core kernel exactly for bf16,
head_dim 128 and k <= 4 on aligned tensors, the portable kernel otherwise,
so a shape that silently fell off the fast path would fail here.
"""
import numpy as np
import pytest
import torch

import synth
from tests.parity import Case, PagedCase, WideCase, check_case, log

pytestmark = pytest.mark.gpu

N_CONTIGUOUS = 14
N_PAGED = 8


@pytest.fixture(scope="module", autouse=True)
def _library():
    import cross_model_kv_helm_amd as hk
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert hk.helm_device_check(-1) == 0, hk.helm_last_error()
    yield


def _contiguous_workload(i: int) -> synth.Workload:
    rng = np.random.default_rng(7000 + i)
    L_s = int(rng.integers(1, 10))
    L_t = int(rng.integers(1, 9))
    H = int(rng.choice([1, 2, 3, 5, 8]))
    D = 64 if i % 4 == 3 else 128
    dtype = "f32" if i % 5 == 4 else "bf16"
    k = int(rng.integers(1, min(5, L_s) + 1))
    T = int(rng.integers(1, 520))
    positions = str(rng.choice(["same", "shift4096", "gap1000"]))
    theta = float(rng.choice([1e4, 1e6]))
    return synth.Workload(f"sweep{i}", L_s, L_t, H, D, T, k, dtype, theta, positions, 7000 + i)


def _expected_path(w: synth.Workload) -> int:
    import cross_model_kv_helm_amd as hk
    fast = w.dtype == "bf16" and w.head_dim == 128 and w.k <= 4
    return hk.HELM_PATH_MATRIX if fast else hk.HELM_PATH_PORTABLE


@pytest.mark.parametrize("i", range(N_CONTIGUOUS))
def test_random_shape_contiguous_full(i):
    import cross_model_kv_helm_amd as hk
    w = _contiguous_workload(i)
    log(f"sweep {i}: L_s={w.n_src_layers} L_t={w.n_tgt_layers} H={w.n_kv_heads} D={w.head_dim} "
        f"k={w.k} T={w.n_tokens} {w.dtype} {w.positions} theta={w.theta:g}")
    case = Case(w)
    d = case.dev
    shape = (w.n_tgt_layers, w.n_kv_heads, case.T, w.head_dim)
    out = (torch.empty(shape, dtype=d["src_k"].dtype, device="cuda"),
           torch.empty(shape, dtype=d["src_k"].dtype, device="cuda"))
    s = hk.make_shape(d["src_k"], d["W_k"], d["layer_sel"], w.theta, w.theta)
    path = hk.helm_kv_transfer_path(d["src_k"], d["src_v"], d["src_pos"], d["tgt_pos"], d["layer_sel"],
                                    d["W_k"], d["b_k"], d["W_v"], d["b_v"], out[0], out[1], s)
    assert path == _expected_path(w), (path, w)
    case.run_gpu(out)
    torch.cuda.synchronize()
    check_case(case, *out)


def _paged_case(i: int):
    rng = np.random.default_rng(8000 + i)
    L_s = int(rng.integers(1, 8))
    L_t = int(rng.integers(1, 7))
    H = int(rng.choice([1, 2, 8]))
    D = 64 if i == 5 else 128
    dtype = "f32" if i == 6 else "bf16"
    k = int(rng.integers(1, min(4, L_s) + 1))
    B = (1, 5, 16, 32)[i % 4]
    R = int(rng.integers(1, 7))
    lens = rng.integers(0, 200, R)
    if i % 3 == 0:
        lens[rng.integers(0, R)] = 0          # a request with no tokens
    if lens.sum() == 0:
        lens[-1] = 1
    w = synth.Workload(f"psweep{i}", L_s, L_t, H, D, 0, k, dtype, 1e6, "same", 8000 + i, paged=True,
                       n_requests=R, block_size=B, max_offset=int(rng.integers(0, 5000)))
    return w, [int(x) for x in lens]


@pytest.mark.parametrize("i", range(N_PAGED))
def test_random_shape_paged_full(i):
    w, lens = _paged_case(i)
    log(f"paged sweep {i}: L_s={w.n_src_layers} L_t={w.n_tgt_layers} H={w.n_kv_heads} D={w.head_dim} "
        f"k={w.k} {w.dtype} block={w.block_size} lens={lens}")
    pc = PagedCase(w, lens=lens)
    tk, tv = pc.run_gpu()
    torch.cuda.synchronize()
    pc.check(tk, tv)


N_WIDE = 8


def _wide_workload(i: int) -> synth.Workload:
    rng = np.random.default_rng(9000 + i)
    L_s = int(rng.integers(1, 10))
    L_t = int(rng.integers(1, 5))
    H = int(rng.integers(1, 5))
    k = int(rng.integers(1, min(4, L_s) + 1))
    T = int(rng.integers(1, 600))
    positions = str(rng.choice(["same", "shift4096", "gap1000"]))
    theta = float(rng.choice([1e4, 1e6]))
    return synth.Workload(f"wsweep{i}", L_s, L_t, H, 128, T, k, "bf16", theta, positions, 9000 + i)


@pytest.mark.parametrize("i", range(N_WIDE))
def test_random_shape_wide_full(i):
    """The wide-input map (helm_kv_transfer_wide) over seeded random shapes:
    input widths IN = k*2*H*128 from 256 to 4,096 and token counts that end
    anywhere inside a 256-token tile."""
    w = _wide_workload(i)
    log(f"wide sweep {i}: L_s={w.n_src_layers} L_t={w.n_tgt_layers} H={w.n_kv_heads} k={w.k} "
        f"T={w.n_tokens} {w.positions} theta={w.theta:g}")
    case = WideCase(w)
    out = case.run_gpu()
    torch.cuda.synchronize()
    case.check(*out)

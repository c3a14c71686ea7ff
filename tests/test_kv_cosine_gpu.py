"""GPU parity of the KV-cosine diagnostic (helm_kv_cosine) against the fp64
oracle (oracle.kv_cosine), through the C ABI.

"Helm Intelligent Routing", the retention / KL / KV-cosine table: the KV
cosine says how close a mapped cache is to the target's own.  Here the
"target's own" cache is the oracle's fp64 mapping rounded to the storage
dtype, so a correct transfer scores within ~1e-5 of 1, and the diagnostic
must resolve differences of that size: the library's value is within 2e-7
of the oracle's (its sums are fp64 over fp32 16-byte pieces; the result is
rounded once to fp32, 6e-8 near 1).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import parity
from tests.parity import Case, log

pytestmark = pytest.mark.gpu

BF16, F32 = 0, 1
ATOL = 2e-7


@pytest.fixture(scope="module", autouse=True)
def _library():
    import cross_model_kv_helm_amd as hk
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert hk.helm_device_check(-1) == 0, hk.helm_last_error()
    yield


def cos_shape(L_t, H, T, D, dtype):
    import cross_model_kv_helm_amd as hk
    s = hk.HelmShape()
    s.n_src_layers, s.n_tgt_layers, s.n_kv_heads, s.head_dim, s.k = L_t, L_t, H, D, 1
    s.dtype, s.n_tokens = dtype, T
    s.rope_theta_src = s.rope_theta_tgt = 1e6
    return s


def storage(t):
    return parity.to_np_storage(t)


def compare(got, want, label):
    got = got.double().cpu().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), f"{label}: NaN pattern differs"
    err = np.abs(got[~nan] - want[~nan])
    log(f"{label}: {want.size} cosines, min {np.nanmin(want) if (~nan).any() else float('nan'):.8f}, "
        f"max |gpu - oracle| {err.max() if err.size else 0.0:.2e}")
    assert err.size == 0 or err.max() <= ATOL, f"{label}: max error {err.max():.3e}"


def to_bf16_storage(x64):
    return storage(torch.from_numpy(np.ascontiguousarray(x64)).to(torch.bfloat16))


def test_mapped_cache_vs_oracle_mapping_bf16():
    """The transfer's own output against the oracle's fp64 mapping rounded
    to bf16: cosines just below 1, resolved to 2e-7."""
    import cross_model_kv_helm_amd as hk
    w = synth.Workload("cos_small", 6, 5, 2, 128, 300, 3, "bf16", 1e6, "shift4096", 31)
    case = Case(w)
    out_k, out_v = case.run_gpu()
    ref_k, ref_v = case.oracle_rows()
    L_t, H, T, D = out_k.shape
    rk = to_bf16_storage(ref_k.reshape(L_t, H, T, D))
    rv = to_bf16_storage(ref_v.reshape(L_t, H, T, D))
    got = hk.helm_kv_cosine(out_k, out_v, parity.from_np_storage(rk, "cuda"), parity.from_np_storage(rv, "cuda"),
                            cos_shape(L_t, H, T, D, BF16))
    torch.cuda.synchronize()
    want = np.stack([oracle.kv_cosine(storage(out_k), rk, BF16), oracle.kv_cosine(storage(out_v), rv, BF16)])
    assert np.all(want > 0.9999)
    compare(got, want, "mapped vs oracle mapping")


def test_fp32_random_negated_and_zero_slabs():
    """fp32 caches: random pairs, one slab against its negation (-1), one
    slab of zeros (NaN)."""
    import cross_model_kv_helm_amd as hk
    g = torch.Generator(device="cuda").manual_seed(5)
    L_t, H, T, D = 4, 2, 128, 64
    a = [torch.randn((L_t, H, T, D), generator=g, device="cuda") for _ in range(2)]
    b = [0.5 * x + torch.randn(x.shape, generator=g, device="cuda") for x in a]
    b[0][1, 0] = -a[0][1, 0]
    a[1][2, 1] = 0.0
    got = hk.helm_kv_cosine(a[0], a[1], b[0], b[1], cos_shape(L_t, H, T, D, F32))
    torch.cuda.synchronize()
    want = np.stack([oracle.kv_cosine(storage(a[i]), storage(b[i]), F32) for i in range(2)])
    assert want[0, 1, 0] == pytest.approx(-1.0, abs=1e-12) and np.isnan(want[1, 2, 1])
    compare(got, want, "fp32 random")


def test_misaligned_caches_take_the_element_path():
    """Caches starting 2 bytes past a 16-byte boundary (the element-wise
    path), ragged token count."""
    import cross_model_kv_helm_amd as hk
    g = torch.Generator(device="cuda").manual_seed(6)
    L_t, H, T, D = 3, 2, 77, 64
    n = L_t * H * T * D
    bufs = [torch.randn(n + 8, generator=g, device="cuda").to(torch.bfloat16) for _ in range(4)]
    t = [x[1:1 + n].view(L_t, H, T, D) for x in bufs]
    assert all(x.data_ptr() % 16 == 2 for x in t)
    got = hk.helm_kv_cosine(t[0], t[1], t[2], t[3], cos_shape(L_t, H, T, D, BF16))
    torch.cuda.synchronize()
    want = np.stack([oracle.kv_cosine(storage(t[0]), storage(t[2]), BF16),
                     oracle.kv_cosine(storage(t[1]), storage(t[3]), BF16)])
    compare(got, want, "misaligned bf16")


def test_zero_tokens_gives_nan():
    import cross_model_kv_helm_amd as hk
    z = torch.empty((2, 2, 0, 128), dtype=torch.bfloat16, device="cuda")
    got = hk.helm_kv_cosine(z, z, z.clone(), z.clone(), cos_shape(2, 2, 0, 128, BF16))
    torch.cuda.synchronize()
    assert torch.isnan(got).all()


def test_qwen3_14b_32b_t32k_sampled_slabs():
    """The benchmark's full cache shape (64 layers x 8 heads x 32,768 tokens x
    128, bf16): a random cache against a copy perturbed by ~1e-3 relative
    noise (so the cosines sit ~1e-6 below 1), checked on 24 slabs of each
    kind."""
    import cross_model_kv_helm_amd as hk
    w = synth.CONFIGS["qwen3_14b_32b_t32k"]
    L_t, H, T, D = w.n_tgt_layers, w.n_kv_heads, w.n_tokens, w.head_dim
    g = torch.Generator(device="cuda").manual_seed(7)
    caches = []
    for _ in range(2):
        a = torch.empty((L_t, H, T, D), dtype=torch.bfloat16, device="cuda")
        b = torch.empty_like(a)
        for l in range(L_t):
            x = torch.randn((H, T, D), generator=g, device="cuda")
            a[l] = x.to(torch.bfloat16)
            b[l] = (x * (1.0 + 1e-3 * torch.randn((H, T, D), generator=g, device="cuda"))).to(torch.bfloat16)
        caches.append((a, b))
    got = hk.helm_kv_cosine(caches[0][0], caches[1][0], caches[0][1], caches[1][1], cos_shape(L_t, H, T, D, BF16))
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    picks = [(0, 0), (L_t - 1, H - 1)] + [tuple(p) for p in zip(rng.integers(0, L_t, 22), rng.integers(0, H, 22))]
    got_h = got.double().cpu().numpy()
    worst = 0.0
    for kv in range(2):
        a, b = caches[kv]
        for l, h in picks:
            want = oracle.kv_cosine(storage(a[l, h:h + 1]), storage(b[l, h:h + 1]), BF16)[0]
            assert 0.999 < want < 1.0
            worst = max(worst, abs(got_h[kv, l, h] - want))
    log(f"t32k sampled: max |gpu - oracle| {worst:.2e} over {2 * len(picks)} slabs")
    assert worst <= ATOL


@pytest.mark.parametrize("i", range(6))
def test_random_shapes(i):
    """Seeded random shapes: 1-9 layers, 1-8 heads, 1-2,999 tokens, head_dim
    64 or 128, bf16 or fp32, pairs of any correlation (from unrelated to
    nearly equal), every cosine against the oracle."""
    import cross_model_kv_helm_amd as hk
    rng = np.random.default_rng(9700 + i)
    L_t, H = int(rng.integers(1, 10)), int(rng.integers(1, 9))
    T, D = int(rng.integers(1, 3000)), int(rng.choice([64, 128]))
    dt = BF16 if i % 2 == 0 else F32
    rho = float(rng.choice([0.0, 0.5, 0.99, 0.999999]))
    label = f"cosine sweep {i}: L_t={L_t} H={H} T={T} D={D} {'bf16' if dt == BF16 else 'fp32'} rho={rho}"
    log(label)
    g = torch.Generator(device="cuda").manual_seed(9700 + i)
    tdt = torch.bfloat16 if dt == BF16 else torch.float32
    a = [torch.randn((L_t, H, T, D), generator=g, device="cuda") for _ in range(2)]
    b = [rho * x + (1 - rho * rho) ** 0.5 * torch.randn(x.shape, generator=g, device="cuda") for x in a]
    a = [x.to(tdt) for x in a]
    b = [x.to(tdt) for x in b]
    got = hk.helm_kv_cosine(a[0], a[1], b[0], b[1], cos_shape(L_t, H, T, D, dt))
    torch.cuda.synchronize()
    want = np.stack([oracle.kv_cosine(storage(a[j]), storage(b[j]), dt) for j in range(2)])
    compare(got, want, label)

"""GPU parity of the wide-input map (helm_kv_transfer_wide) against the fp64
oracle (oracle.transfer_wide_rows), through the C ABI.

The Qwen3 cache-mapping write-up, section "A linear bridge, strangely enough,
suffices": the full mapper's x concatenates the KV features of all selected
source layers, with one fit per target head for keys and one for values.
Tolerance: the bf16 rule of tests/parity.py (per slab, the excess over half
an output ulp at most 1e-2 rms, cosine at least 0.9999), the oracle in DTYPE
mode (the un-rotated key rounded once to bf16, the map's operand type).
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from tests.parity import WideCase, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _library():
    import cross_model_kv_helm_amd as hk
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert hk.helm_device_check(-1) == 0, hk.helm_last_error()
    yield


def W(name, *args, **kw):
    return synth.Workload(name, *args, **kw)


def test_wide_small_ragged_full():
    """Two token tiles (the second ragged), two heads, k = 2 (IN = 1024)."""
    case = WideCase(W("wide_small", 5, 3, 2, 128, 300, 2, "bf16", 1e6, "shift4096", 61))
    out = case.run_gpu()
    torch.cuda.synchronize()
    case.check(*out)


@pytest.mark.parametrize("k", [3, 6])
def test_wide_k3_k6_full(k):
    """k = 3 (IN = 1,536 with two heads) and k = 6 (more selected layers
    than the per-head kernel takes; IN = 1,536 with one head), 100 tokens."""
    H = 2 if k == 3 else 1
    case = WideCase(W(f"wide_k{k}", 8, 3, H, 128, 100, k, "bf16", 1e6, "shift4096", 70 + k))
    out = case.run_gpu()
    torch.cuda.synchronize()
    case.check(*out)


def test_wide_one_head_k1_short_full():
    """H = 1 (one column tile: the key map and the value map of head 0),
    k = 1 (IN = 256, four pipeline steps), 33 tokens."""
    case = WideCase(W("wide_h1", 3, 2, 1, 128, 33, 1, "bf16", 1e4, "gap1000", 62))
    out = case.run_gpu()
    torch.cuda.synchronize()
    case.check(*out)


def test_wide_three_heads_mixed_tile_full():
    """H = 3: column tile 1 holds the key map of head 2 and the value map of
    head 0, so the two waves of a row-half take different kinds."""
    case = WideCase(W("wide_h3", 4, 2, 3, 128, 257, 2, "bf16", 1e6, "same", 63))
    out = case.run_gpu()
    torch.cuda.synchronize()
    case.check(*out)


def test_wide_xcd_order_full():
    """2,048 tokens = 8 token tiles: the XCD-aware tile order (the column
    tiles of a token tile consecutive on one XCD)."""
    case = WideCase(W("wide_xcd", 4, 2, 2, 128, 2048, 2, "bf16", 1e6, "shift4096", 64))
    out = case.run_gpu()
    torch.cuda.synchronize()
    case.check(*out)


def test_wide_qwen3_14b_32b_t32k_sampled():
    """The benchmark's wide workload (40 -> 64 layers, 8 heads, k = 4, IN =
    8192, 32,768 tokens) on sampled rows of every slab: fixed tokens, a few
    random ones and one random token in every 256-token tile, so every
    (token tile, column tile) of the product's XCD-ordered schedule is
    compared."""
    w = synth.CONFIGS["qwen3_14b_32b_t32k_wide"]
    case = WideCase(w)
    out = case.run_gpu()
    torch.cuda.synchronize()
    rows = sample_rows(w.n_tgt_layers, w.n_kv_heads, case.T, 2, 2, tile=256)
    case.check(*out, rows=rows)


def test_wide_stages_equal_one_call():
    """The preparation and the product enqueued separately
    (helm_kv_transfer_wide_stage) write exactly what one call writes, and a
    second product from the same workspace does too."""
    import cross_model_kv_helm_amd as hk
    case = WideCase(W("wide_stages", 5, 3, 2, 128, 300, 2, "bf16", 1e6, "shift4096", 65))
    d, w = case.dev, case.w
    whole = case.run_gpu()
    s = hk.make_shape(d["src_k"], d["W_k"], d["layer_sel"], w.theta, w.theta)
    ws = torch.empty(hk.helm_kv_wide_workspace_bytes(s), dtype=torch.uint8, device="cuda")
    for rep in range(2):
        out = (torch.full_like(whole[0], float("nan")), torch.full_like(whole[1], float("nan")))
        stages = (hk.HELM_STAGE_TABLES, hk.HELM_STAGE_MAP) if rep == 0 else (hk.HELM_STAGE_MAP,)
        for st in stages:
            hk.helm_kv_transfer_wide_stage(st, d["src_k"], d["src_v"], d["src_pos"], d["tgt_pos"], d["layer_sel"],
                                           d["W_k"], d["b_k"], d["W_v"], d["b_v"], out[0], out[1], s, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out[0], whole[0]) and torch.equal(out[1], whole[1]), f"pass {rep}"
    case.check(*whole)


@pytest.mark.parametrize("bad,value", [(1, 99), (3, -1)])
def test_wide_invalid_device_layer_sel_leaves_target_layer_unwritten(bad, value):
    """A layer_sel row with an index outside [0, L_s) that reaches the device
    is not read: that target layer keeps its previous contents (every
    column tile of every token tile of it), the other layers are mapped."""
    import cross_model_kv_helm_amd as hk
    case = WideCase(W(f"wide_bad_{bad}", 5, 4, 2, 128, 600, 2, "bf16", 1e6, "shift4096", 66 + bad))
    d, w = case.dev, case.w
    sel = case.host["layer_sel"].copy()
    sel[bad, 1] = value
    d["layer_sel"] = torch.from_numpy(sel).cuda()
    shape = (w.n_tgt_layers, w.n_kv_heads, case.T, w.head_dim)
    sentinel = torch.full(shape, 3.0, dtype=torch.bfloat16, device="cuda")
    out = (sentinel.clone(), sentinel.clone())
    s = hk.make_shape(d["src_k"], d["W_k"], d["layer_sel"], w.theta, w.theta)
    hk.helm_kv_transfer_wide(d["src_k"], d["src_v"], d["src_pos"], d["tgt_pos"], d["layer_sel"], d["W_k"],
                             d["b_k"], d["W_v"], d["b_v"], out[0], out[1], s)
    torch.cuda.synchronize()
    assert torch.equal(out[0][bad], sentinel[bad]) and torch.equal(out[1][bad], sentinel[bad])
    good = [l for l in range(w.n_tgt_layers) if l != bad]
    rows = np.concatenate([(l * w.n_kv_heads + h) * case.T + np.arange(case.T)
                           for l in good for h in range(w.n_kv_heads)])
    case.host["layer_sel"] = np.where((sel < 0) | (sel >= w.n_src_layers), 0, sel).astype(np.int32)
    case.check(*out, rows=rows, label="valid rows of ")


def test_wide_maps_not_16_byte_aligned_full():
    """W_k and W_v in buffers offset by one element (not 16-byte aligned):
    the preparation transposes them with 2-byte accesses instead of 16-byte
    ones; the outputs are the same as from aligned maps, bit for bit, and
    within the tolerance of the oracle."""
    import cross_model_kv_helm_amd as hk
    case = WideCase(W("wide_misaligned_w", 5, 3, 2, 128, 300, 2, "bf16", 1e6, "shift4096", 67))
    d, w = case.dev, case.w
    aligned = case.run_gpu()

    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        return v
    Wk, Wv = shifted(d["W_k"]), shifted(d["W_v"])
    assert Wk.data_ptr() % 16 != 0 and Wv.data_ptr() % 16 != 0
    out = (torch.full_like(aligned[0], float("nan")), torch.full_like(aligned[1], float("nan")))
    s = hk.make_shape(d["src_k"], Wk, d["layer_sel"], w.theta, w.theta)
    hk.helm_kv_transfer_wide(d["src_k"], d["src_v"], d["src_pos"], d["tgt_pos"], d["layer_sel"], Wk, d["b_k"],
                             Wv, d["b_v"], out[0], out[1], s)
    torch.cuda.synchronize()
    assert torch.equal(out[0], aligned[0]) and torch.equal(out[1], aligned[1])
    case.check(*out)


def test_wide_131k_tokens_shifted_sampled():
    """The 14B -> 32B wide shape at 131,072 tokens with target positions
    shifted by 4,096 (positions up to 135,167; 512 token tiles a layer on the
    persistent grid, the epilogue's table slice at token offsets up to
    130,816): 24 slabs (the first and last target layer's 8 heads and 8 more
    spread over the rest), one random token in every 256-token tile of each
    plus fixed tokens, against the oracle."""
    w = dataclasses.replace(synth.CONFIGS["qwen3_14b_32b_t32k_wide"], name="wide_t128k_shift", n_tokens=131072,
                            positions="shift4096", seed=312)
    case = WideCase(w)
    out = case.run_gpu()
    torch.cuda.synchronize()
    H, T = w.n_kv_heads, case.T
    rng = np.random.default_rng(5)
    slabs = sorted(set(list(range(H)) + list(range((w.n_tgt_layers - 1) * H, w.n_tgt_layers * H)) +
                       rng.choice(np.arange(H, (w.n_tgt_layers - 1) * H), 8, replace=False).tolist()))
    starts = np.arange(0, T, 256)
    toks = np.unique(np.concatenate([starts + rng.integers(0, 256, starts.size), [0, 1, 65535, 65536, T - 1]]))
    rows = np.concatenate([g * T + toks for g in slabs]).astype(np.int64)
    case.check(*out, rows=rows)

"""The seeded input generator: determinism and the structure of its draws."""
import numpy as np
import pytest
import torch

import synth


def test_same_seed_same_bytes():
    w = synth.CONFIGS["tiny_fp32"]
    a = synth.contiguous_inputs(w)
    b = synth.contiguous_inputs(w)
    for key in a:
        assert torch.equal(a[key], b[key]), key


def test_shapes_and_dtypes():
    w = synth.CONFIGS["qwen3_0.6b_1.7b_t512"]
    c = synth.contiguous_inputs(w, n_tokens=32)
    assert c["k_content"].shape == (28, 8, 32, 128) and c["k_content"].dtype == torch.bfloat16
    assert c["W_k"].shape == (28, 8, 512, 128) and c["W_k"].dtype == torch.bfloat16
    assert c["b_k"].shape == (28, 8, 128) and c["b_k"].dtype == torch.float32
    assert c["layer_sel"].shape == (28, 4) and c["layer_sel"].dtype == torch.int32


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_layer_selection_distinct_in_range(name):
    w = synth.CONFIGS[name]
    sel = synth.layer_selection(w)
    assert sel.shape == (w.n_tgt_layers, w.k)
    assert sel.min() >= 0 and sel.max() < w.n_src_layers
    for row in sel:
        assert len(set(row.tolist())) == w.k
    # draw order is kept: most rows are not sorted
    if w.k > 1:
        assert sum(list(r) != sorted(r) for r in sel) > 0


def test_positions_rules():
    s, t = synth.positions(synth.CONFIGS["qwen3_14b_32b_t128k_gap"], 131072)
    assert s[65535] == 65535 and s[65536] == 66536 and t[0] == 4096 and t[-1] == 4096 + 131071
    s, t = synth.positions(synth.CONFIGS["qwen3_14b_32b_t128k_shift"], 10)
    assert list(t - s) == [4096] * 10


def test_value_distribution_moments():
    """rms of content keys ~ sqrt(E[exp(z)]) = exp(1/4) (lognormal(0, 0.5) scales)."""
    w = synth.CONFIGS["qwen3_0.6b_1.7b_t512"]
    c = synth.contiguous_inputs(w, n_tokens=256)
    rms = c["k_content"].float().pow(2).mean().sqrt().item()
    assert abs(rms - np.exp(0.25)) < 0.1
    assert abs(c["W_k"].float().std().item() - 1 / np.sqrt(512)) < 2e-3
    assert abs(c["b_k"].std().item() - 0.1) < 5e-3


def test_paged_layout_invariants():
    w = synth.CONFIGS["paged_32req"]
    lay = synth.paged_layout(w)
    assert len(lay.lens) == 32 and lay.lens.min() >= 256 and lay.lens.max() <= 16384
    for bt, nb in ((lay.src_bt, lay.n_src_blocks), (lay.tgt_bt, lay.n_tgt_blocks)):
        used = bt[bt >= 0]
        assert used.max() < nb
        assert len(np.unique(used)) == used.size          # injective
        pages = (lay.lens + 15) // 16
        assert (bt >= 0).sum(axis=1).tolist() == pages.tolist()
    assert (lay.tgt_pos - lay.src_pos).min() >= 0 and (lay.tgt_pos - lay.src_pos).max() <= 2048


def test_scatter_to_pool_places_rows():
    w = synth.Workload("t", 2, 2, 2, 8, 0, 1, "bf16", 1e6, "same", 7, paged=True, n_requests=3)
    lay = synth.paged_layout(w, lens=[5, 16, 17])
    x = torch.randn(2, 2, lay.n_tokens, 8).to(torch.bfloat16)
    pool = synth.scatter_to_pool(x, lay, lay.src_bt, lay.n_src_blocks, fill_bits=synth.CANARY_BITS)
    slots = synth.slot_index(lay, lay.src_bt)
    flat = pool.view(2, -1, 2, 8)
    for n in range(lay.n_tokens):
        assert torch.equal(flat[:, slots[n]], x[:, :, n])
    unused = np.setdiff1d(np.arange(lay.n_src_blocks * 16), slots)
    assert (flat[:, unused].view(torch.int16) == np.int16(np.uint16(synth.CANARY_BITS).view(np.int16))).all()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_pool_canary_per_storage_dtype(dtype):
    """Unused slots hold the canary in either storage type: a NaN that no
    transfer output equals, compared on the element's whole bit pattern
    (for fp32 the 16-bit pattern fills both halves)."""
    w = synth.Workload("t", 2, 2, 2, 8, 0, 1, "bf16" if dtype == torch.bfloat16 else "f32", 1e6, "same", 9,
                       paged=True, n_requests=2, block_size=5)
    lay = synth.paged_layout(w, lens=[7, 0])
    x = torch.randn(2, 2, lay.n_tokens, 8).to(dtype)
    pool = synth.scatter_to_pool(x, lay, lay.src_bt, lay.n_src_blocks, fill_bits=synth.CANARY_BITS)
    slots = synth.slot_index(lay, lay.src_bt)
    flat = pool.view(2, -1, 2, 8)
    for n in range(lay.n_tokens):
        assert torch.equal(flat[:, slots[n]], x[:, :, n])
    unused = np.setdiff1d(np.arange(lay.n_src_blocks * 5), slots)
    bits, canary = synth.canary_view(flat)
    assert (bits[:, unused] == canary).all()
    assert torch.isnan(flat[:, unused]).all()
    tgt = synth.empty_target_pool(w, lay)
    assert tgt.dtype == dtype
    tbits, tcanary = synth.canary_view(tgt)
    assert (tbits == tcanary).all() and torch.isnan(tgt).all()
    if dtype == torch.float32:
        assert tcanary == 0x7FA57FA5

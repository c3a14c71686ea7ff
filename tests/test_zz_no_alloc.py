"""The allocation-free transfer (helm_kv_transfer_noalloc) through the C ABI:
its outputs equal helm_kv_transfer's bit for bit on two calls in a row, the
second with a smaller input (the static scratch keeps the first call's
tables, which the second must not read), and both match the oracle.  A call
beyond the scratch's limit is refused before anything is enqueued, and the
call captured in a HIP graph replays bit for bit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from tests.parity import Case, check_case, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _library():
    import cross_model_kv_helm_amd as hk
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert hk.helm_device_check(-1) == 0, hk.helm_last_error()
    yield


def run_both(case):
    import cross_model_kv_helm_amd as hk
    d, w = case.dev, case.w
    shape = (w.n_tgt_layers, w.n_kv_heads, case.T, w.head_dim)
    ref = case.run_gpu()
    out = (torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda"),
           torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda"))
    s = hk.make_shape(d["src_k"], d["W_k"], d["layer_sel"], w.theta, w.theta)
    hk.helm_kv_transfer_noalloc(d["src_k"], d["src_v"], d["src_pos"], d["tgt_pos"], d["layer_sel"], d["W_k"],
                                d["b_k"], d["W_v"], d["b_v"], out[0], out[1], s)
    torch.cuda.synchronize()
    return ref, out


def test_noalloc_equals_transfer_on_two_calls_second_smaller():
    big = dataclasses.replace(synth.CONFIGS["qwen3_0.6b_1.7b_t2048"], name="noalloc_big", n_src_layers=6,
                              n_tgt_layers=5, positions="shift4096", seed=91)
    small = dataclasses.replace(big, name="noalloc_small", n_tokens=300, positions="gap1000", seed=92)
    for w in (big, small):
        case = Case(w)
        ref, out = run_both(case)
        for r, o, nm in ((ref[0], out[0], "K"), (ref[1], out[1], "V")):
            assert torch.equal(r.view(torch.int16), o.view(torch.int16)), f"{w.name} {nm}: not bit-identical"
        log(f"{w.name}: {case.T} tokens bit-identical to helm_kv_transfer")
        check_case(case, *out, label="noalloc ")


def test_noalloc_limit_refused_before_any_work():
    import cross_model_kv_helm_amd as hk
    limit = hk.helm_kv_noalloc_max_bytes()
    assert limit == 64 << 20
    w = dataclasses.replace(synth.CONFIGS["tiny_fp32"], head_dim=128)
    s = hk.HelmShape()
    s.n_src_layers, s.n_tgt_layers, s.n_kv_heads, s.head_dim, s.k = 2, 2, 1, 128, 1
    s.dtype, s.rope_theta_src, s.rope_theta_tgt = hk.HELM_BF16, 1e6, 1e6
    s.n_tokens = limit // 1024 + 32          # one tile past what the scratch holds at head_dim 128
    T = s.n_tokens
    src = torch.zeros((2, 1, T, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full((2, 1, T, 128), 5.0, dtype=torch.bfloat16, device="cuda")
    out2 = out.clone()
    pos = torch.zeros(T, dtype=torch.int32, device="cuda")
    sel = torch.zeros((2, 1), dtype=torch.int32, device="cuda")
    W = torch.zeros((2, 1, 128, 128), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((2, 1, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(hk.HelmError) as e:
        hk.helm_kv_transfer_noalloc(src, src, pos, pos, sel, W, b, W, b, out, out2, s)
    assert e.value.status == 7 and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 5.0).all()) and bool((out2 == 5.0).all())
    del w


def test_noalloc_captured_in_a_graph_replays_bit_for_bit():
    """The call captured in a HIP graph (torch.cuda.CUDAGraph) on torch's
    capture stream, for callers that record their work as graphs: three
    replays, with the outputs overwritten in between, reproduce the eager
    call bit for bit (nothing in the call allocates or clears memory)."""
    import cross_model_kv_helm_amd as hk
    w = dataclasses.replace(synth.CONFIGS["qwen3_0.6b_1.7b_t512"], name="graph", n_src_layers=6, n_tgt_layers=5,
                            positions="shift4096", seed=93)
    case = Case(w)
    d = case.dev
    shape = (w.n_tgt_layers, w.n_kv_heads, case.T, w.head_dim)
    out = (torch.empty(shape, dtype=torch.bfloat16, device="cuda"),
           torch.empty(shape, dtype=torch.bfloat16, device="cuda"))

    def call():
        s = hk.make_shape(d["src_k"], d["W_k"], d["layer_sel"], w.theta, w.theta)   # stream: the current one
        hk.helm_kv_transfer_noalloc(d["src_k"], d["src_v"], d["src_pos"], d["tgt_pos"], d["layer_sel"], d["W_k"],
                                    d["b_k"], d["W_v"], d["b_v"], out[0], out[1], s)

    call()                       # eager: the first call looks up the static scratch's device address
    torch.cuda.synchronize()
    ref = (out[0].clone(), out[1].clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        out[0].fill_(float("nan"))
        out[1].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out[0].view(torch.int16), ref[0].view(torch.int16)), f"replay {rep}: K"
        assert torch.equal(out[1].view(torch.int16), ref[1].view(torch.int16)), f"replay {rep}: V"
    log(f"{w.name}: 3 graph replays bit-identical to the eager call")

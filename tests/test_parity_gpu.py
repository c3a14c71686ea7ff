"""GPU parity: the HIP library against the fp64 oracle on identical seeded inputs.

Every call goes through the C ABI (via the ctypes binding).  Small cases are
compared element by element in full; full-size workloads are compared on
sampled rows (every (layer, head) slab, with first/last tokens and tile edges
always included) in exactly the launch configuration the benchmark times.
Tolerances: see tests/parity.py.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import parity
from tests.parity import Case, PagedCase, check_case, log, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _library():
    import cross_model_kv_helm_amd as hk
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert hk.helm_device_check(-1) == 0, hk.helm_last_error()
    yield


def W(name, **kw):
    return dataclasses.replace(synth.CONFIGS[name], **kw)


SMALL_BF16 = synth.Workload("small_bf16", 6, 5, 2, 128, 300, 3, "bf16", 1e6, "same", 11)

# Token-window width of the full-size samples: one random token inside every
# TILE-token window of every slab, so each token tile of the matrix-core
# kernel's schedule (16 or 32 tokens; both are covered by 16) is compared.
TILE = 16


# ---------------------------------------------------------------- small, full compare
def test_tiny_fp32_full():
    case = Case(synth.CONFIGS["tiny_fp32"])
    out = case.run_gpu()
    torch.cuda.synchronize()
    check_case(case, *out)


def test_small_bf16_ragged_full():
    case = Case(SMALL_BF16)
    out = case.run_gpu()
    torch.cuda.synchronize()
    check_case(case, *out)


def test_small_bf16_d64_full():
    case = Case(dataclasses.replace(SMALL_BF16, name="small_bf16_d64", head_dim=64, n_tokens=77, seed=12))
    out = case.run_gpu()
    torch.cuda.synchronize()
    check_case(case, *out)


def test_fp32_d128_shift_full():
    w = dataclasses.replace(SMALL_BF16, name="small_f32_shift", dtype="f32", positions="shift4096",
                            n_tokens=70, seed=13)
    case = Case(w)
    out = case.run_gpu()
    torch.cuda.synchronize()
    check_case(case, *out)


def test_qwen3_06b_17b_t512_full():
    case = Case(synth.CONFIGS["qwen3_0.6b_1.7b_t512"])
    out = case.run_gpu()
    torch.cuda.synchronize()
    check_case(case, *out)


def test_qwen3_06b_17b_t2048_sampled():
    w = synth.CONFIGS["qwen3_0.6b_1.7b_t2048"]
    case = Case(w)
    out = case.run_gpu()
    torch.cuda.synchronize()
    check_case(case, *out, rows=sample_rows(w.n_tgt_layers, w.n_kv_heads, case.T, 8, 1, tile=TILE))


# ---------------------------------------------------------------- edge cases
def test_single_token_and_duplicate_selection():
    w = dataclasses.replace(SMALL_BF16, name="one_token_dup", n_tokens=1, k=3, seed=14)
    sel = np.array([[2, 2, 0], [5, 1, 5], [0, 0, 0], [3, 4, 1], [1, 1, 2]], np.int32)
    case = Case(w, layer_sel=sel, src_pos=[77], tgt_pos=[123456])
    out = case.run_gpu()
    torch.cuda.synchronize()
    check_case(case, *out)


def test_k1_negative_and_large_positions_distinct_thetas():
    w = dataclasses.replace(SMALL_BF16, name="k1_positions", k=1, n_tokens=200, seed=15)
    rng = np.random.default_rng(3)
    src = rng.integers(-100000, 2 ** 31 - 1, 200).astype(np.int32)
    tgt = rng.integers(-(2 ** 31), 2 ** 31 - 1, 200).astype(np.int32)
    case = Case(w, src_pos=src, tgt_pos=tgt)
    # a target whose RoPE base differs from the pilot's
    case.w = dataclasses.replace(w, theta=1e6)
    d = case.dev
    import cross_model_kv_helm_amd as hk
    shape = (w.n_tgt_layers, w.n_kv_heads, case.T, w.head_dim)
    ok_, ov_ = torch.empty(shape, dtype=torch.bfloat16, device="cuda"), torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    s = hk.make_shape(d["src_k"], d["W_k"], d["layer_sel"], 1e6, 5e5)
    hk.helm_kv_transfer(d["src_k"], d["src_v"], d["src_pos"], d["tgt_pos"], d["layer_sel"], d["W_k"],
                        d["b_k"], d["W_v"], d["b_v"], ok_, ov_, s)
    torch.cuda.synchronize()
    pb = case.problem()
    pb.theta_tgt = 5e5
    h = case.host
    ref_k, ref_v = oracle.transfer_rows(pb, h["src_k"], h["src_v"], h["src_pos"], h["tgt_pos"], h["layer_sel"],
                                        h["W_k"], h["b_k"], h["W_v"], h["b_v"])
    D = w.head_dim
    slab = np.arange(ref_k.size // D) // case.T
    parity.compare(parity.storage_to_f64(parity.to_np_storage(ok_)).reshape(-1, D), ref_k.reshape(-1, D),
                   slab, "bf16", "k1_positions K")
    parity.compare(parity.storage_to_f64(parity.to_np_storage(ov_)).reshape(-1, D), ref_v.reshape(-1, D),
                   slab, "bf16", "k1_positions V")


def test_positions_inside_and_outside_tile_windows():
    """Position patterns within and across 32-token tiles: tiles 0-3
    ascending, 4 holding a jump of 100,000, 5 constant, 6-7 scattered, 8-9
    (the last one ragged) ascending again; target positions descending, with
    one scattered tile."""
    T = 300
    t = np.arange(T)
    src = np.where(t < 150, t + 7, t + 100000)
    src[160:192] = 42
    rng = np.random.default_rng(21)
    src[192:256] = rng.integers(0, 200000, 64)
    tgt = 5000 - t                              # descending: every tile is a window
    tgt[200:232] = rng.integers(-70000, 70000, 32)
    w = dataclasses.replace(SMALL_BF16, name="tile_windows", n_tokens=T, k=2, seed=22)
    case = Case(w, src_pos=src.astype(np.int32), tgt_pos=tgt.astype(np.int32))
    out = case.run_gpu()
    torch.cuda.synchronize()
    check_case(case, *out)


def test_zero_tokens_writes_nothing():
    import cross_model_kv_helm_amd as hk
    w = dataclasses.replace(SMALL_BF16, n_tokens=0)
    c = synth.contiguous_inputs(w, device="cuda", n_tokens=0)
    out = torch.full((5, 2, 0, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    s = hk.make_shape(c["k_content"], c["W_k"], c["layer_sel"], 1e6, 1e6)
    hk.helm_kv_transfer(c["k_content"], c["src_v"], c["src_pos"], c["tgt_pos"], c["layer_sel"], c["W_k"],
                        c["b_k"], c["W_v"], c["b_v"], out, out.clone(), s)
    torch.cuda.synchronize()


@pytest.mark.parametrize("bad,T", [(2, 40), (2, 3000), (3, 3000)])
def test_invalid_device_layer_sel_leaves_target_layer_unwritten(bad, T):
    """A layer_sel row with an index outside [0, L_s) that reaches the device
    is not read: that target layer is left as it was; the others are mapped.
    With 3000 tokens every work item spans several token tiles, and the
    matrix-core kernel pairs target layers (2l, 2l+1): an invalid even layer
    must not starve its odd partner of anything (its tables included)."""
    w = dataclasses.replace(SMALL_BF16, name=f"bad_sel_{bad}_{T}", n_tokens=T, seed=16)
    case = Case(w)
    sel = case.host["layer_sel"].copy()
    sel[bad, 1] = 99
    case.dev["layer_sel"] = torch.from_numpy(sel).cuda()
    shape = (w.n_tgt_layers, w.n_kv_heads, case.T, w.head_dim)
    sentinel = torch.full(shape, 3.0, dtype=torch.bfloat16, device="cuda")
    out = (sentinel.clone(), sentinel.clone())
    case.run_gpu(out)
    torch.cuda.synchronize()
    assert torch.equal(out[0][bad], sentinel[bad]) and torch.equal(out[1][bad], sentinel[bad])
    good = np.array([l for l in range(5) if l != bad])
    rows = np.concatenate([(l * w.n_kv_heads + h) * case.T + np.arange(case.T)
                           for l in good for h in range(w.n_kv_heads)])
    case.host["layer_sel"] = np.where(sel == 99, 0, sel).astype(np.int32)
    check_case(case, *out, rows=rows, label="valid rows of ")


def test_staged_call_equals_full_call():
    """Tables stage, then map stage (reading the tables from the same
    workspace) gives bit-identical results to the one-call transfer."""
    import cross_model_kv_helm_amd as hk
    case = Case(dataclasses.replace(SMALL_BF16, name="staged", n_tokens=700, seed=19))
    full = case.run_gpu()
    d = case.dev
    shape_ = (case.w.n_tgt_layers, case.w.n_kv_heads, case.T, case.w.head_dim)
    out = (torch.empty(shape_, dtype=torch.bfloat16, device="cuda"),
           torch.empty(shape_, dtype=torch.bfloat16, device="cuda"))
    s = hk.make_shape(d["src_k"], d["W_k"], d["layer_sel"], case.w.theta, case.w.theta)
    ws = torch.empty(hk.helm_kv_workspace_bytes(s), dtype=torch.uint8, device="cuda")
    args = (d["src_k"], d["src_v"], d["src_pos"], d["tgt_pos"], d["layer_sel"], d["W_k"], d["b_k"], d["W_v"],
            d["b_v"], out[0], out[1], s)
    hk.helm_kv_transfer_stage(hk.HELM_STAGE_TABLES, *args, workspace=ws)
    hk.helm_kv_transfer_stage(hk.HELM_STAGE_MAP, *args, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out[0].view(torch.int16), full[0].view(torch.int16))
    assert torch.equal(out[1].view(torch.int16), full[1].view(torch.int16))


def test_side_stream_with_the_bindings_own_workspace():
    """The call runs on a side stream with the workspace the binding
    allocates itself, while torch's current stream immediately allocates and
    overwrites memory of the same size: the binding marks its workspace as
    used by the launch stream, so the caching allocator cannot hand it to
    those allocations while the transfer still reads its tables.  The
    result matches the oracle, and the caller's shape keeps its stream field
    (an unset stream is resolved per call, never written back)."""
    import cross_model_kv_helm_amd as hk
    case = Case(dataclasses.replace(SMALL_BF16, name="side_stream", n_tokens=3000, seed=23))
    d, w = case.dev, case.w
    shape_ = (w.n_tgt_layers, w.n_kv_heads, case.T, w.head_dim)
    out = (torch.empty(shape_, dtype=torch.bfloat16, device="cuda"),
           torch.empty(shape_, dtype=torch.bfloat16, device="cuda"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    s = hk.make_shape(d["src_k"], d["W_k"], d["layer_sel"], w.theta, w.theta)
    s.stream = side.cuda_stream
    nbytes = hk.helm_kv_workspace_bytes(s)
    hk.helm_kv_transfer(d["src_k"], d["src_v"], d["src_pos"], d["tgt_pos"], d["layer_sel"], d["W_k"], d["b_k"],
                        d["W_v"], d["b_v"], out[0], out[1], s)
    junk = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(0xFF) for _ in range(8)]
    torch.cuda.synchronize()
    assert s.stream == side.cuda_stream
    unset = hk.make_shape(d["src_k"], d["W_k"], d["layer_sel"], w.theta, w.theta)
    case.run_gpu()
    hk.helm_kv_transfer(d["src_k"], d["src_v"], d["src_pos"], d["tgt_pos"], d["layer_sel"], d["W_k"], d["b_k"],
                        d["W_v"], d["b_v"], torch.empty_like(out[0]), torch.empty_like(out[1]), unset)
    torch.cuda.synchronize()
    assert not unset.stream, "the binding wrote the resolved stream into the caller's shape"
    del junk
    check_case(case, *out, label="side stream ")


def test_bitwise_deterministic():
    case = Case(dataclasses.replace(SMALL_BF16, name="det", n_tokens=513, seed=17))
    a = case.run_gpu()
    b = case.run_gpu()
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1].view(torch.int16), b[1].view(torch.int16))


# ---------------------------------------------------------------- paged
def test_paged_small_full():
    w = synth.Workload("paged_small", 5, 4, 2, 128, 0, 2, "bf16", 1e6, "same", 31, paged=True,
                       n_requests=5, max_offset=300)
    pc = PagedCase(w, lens=[1, 16, 17, 40, 3])
    tk, tv = pc.run_gpu()
    torch.cuda.synchronize()
    pc.check(tk, tv)


@pytest.mark.parametrize("k", [1, 3, 4])
def test_paged_small_k1_k3_k4_full(k):
    """The paged instantiations for k = 1, 3 and 4 on a shape small enough
    that keys and values go into one launch (the 32-request test takes k = 4
    through the two launches): four requests whose lengths cross 16-token
    tiles and pages unevenly, with per-request target offsets."""
    w = synth.Workload(f"paged_k{k}", 6, 5, 2, 128, 0, k, "bf16", 1e6, "same", 40 + k, paged=True,
                       n_requests=4, max_offset=500)
    pc = PagedCase(w, lens=[33, 70, 5, 129])
    tk, tv = pc.run_gpu()
    torch.cuda.synchronize()
    pc.check(tk, tv)


def test_paged_32_requests_sampled():
    w = synth.CONFIGS["paged_32req"]
    pc = PagedCase(w)
    log(f"paged: N={pc.lay.n_tokens} tokens, {pc.lay.n_src_blocks} src blocks")
    tk, tv = pc.run_gpu()
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    N = pc.lay.n_tokens
    # every slab, each request's first and last token, plus random tokens
    edges = np.concatenate([pc.lay.cu_seqlens[:-1], pc.lay.cu_seqlens[1:] - 1])
    toks = np.unique(np.concatenate([edges, rng.integers(0, N, 32)]))
    rows = np.concatenate([g * N + toks for g in range(w.n_tgt_layers * w.n_kv_heads)])
    pc.check(tk, tv, rows=rows)


# ---------------------------------------------------------------- full-size workloads
def test_qwen3_14b_32b_t32k_sampled():
    """The benchmark's workload in its launch configuration: every slab, one
    random token in every 16-token window, compared with the oracle (DTYPE
    mode, gated); the same rows against the un-rounded oracle (EXACT mode)
    are reported, not gated."""
    w = synth.CONFIGS["qwen3_14b_32b_t32k"]
    case = Case(w)
    out = case.run_gpu()
    torch.cuda.synchronize()
    check_case(case, *out, rows=sample_rows(w.n_tgt_layers, w.n_kv_heads, case.T, 8, 2, tile=TILE), exact=True)


@pytest.mark.parametrize("name", ["qwen3_14b_32b_t128k_shift", "qwen3_14b_32b_t128k_gap"])
def test_qwen3_14b_32b_t128k_sampled(name):
    """131,072 tokens, transferred prefix placed at target offset 4096, and a
    1,000-position gap in the source positions at token 65,536: every sampled
    row must be re-rotated at its own target position."""
    w = synth.CONFIGS[name]
    case = Case(w)
    out = case.run_gpu()
    torch.cuda.synchronize()
    rows = sample_rows(w.n_tgt_layers, w.n_kv_heads, case.T, 8, 3, tile=TILE)
    # the rows either side of the gap, in every slab
    edge = np.array([65535, 65536], dtype=np.int64)
    rows = np.unique(np.concatenate([rows] + [g * case.T + edge for g in range(w.n_tgt_layers * w.n_kv_heads)]))
    check_case(case, *out, rows=rows)
    del out, case


# ---------------------------------------------------------------- portable-kernel paths
def test_k5_bf16_portable_kernel_full():
    """k = 5 is outside the matrix-core kernel's range: the portable kernel maps it."""
    w = synth.Workload("k5_bf16", 8, 3, 2, 128, 70, 5, "bf16", 1e6, "shift4096", 18)
    case = Case(w)
    out = case.run_gpu()
    torch.cuda.synchronize()
    check_case(case, *out)


def test_misaligned_pointers_portable_kernel_full():
    """Tensors offset by one element (not 16-byte aligned) go to the portable kernel."""
    import cross_model_kv_helm_amd as hk
    w = dataclasses.replace(SMALL_BF16, name="misaligned", n_tokens=33, seed=19)
    case = Case(w)
    d = case.dev
    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        return v
    sk, sv = shifted(d["src_k"]), shifted(d["src_v"])
    shape = (w.n_tgt_layers, w.n_kv_heads, case.T, w.head_dim)
    ok_ = shifted(torch.empty(shape, dtype=torch.bfloat16, device="cuda"))
    ov_ = shifted(torch.empty(shape, dtype=torch.bfloat16, device="cuda"))
    s = hk.make_shape(sk, d["W_k"], d["layer_sel"], w.theta, w.theta)
    hk.helm_kv_transfer(sk, sv, d["src_pos"], d["tgt_pos"], d["layer_sel"], d["W_k"], d["b_k"], d["W_v"],
                        d["b_v"], ok_, ov_, s)
    torch.cuda.synchronize()
    check_case(case, ok_, ov_)


def test_matrix_core_and_portable_kernels_agree():
    """The same bf16 case through both kernels: aligned buffers take the
    matrix-core kernel, the same data in one-element-offset buffers the
    portable one (helm_kv_transfer_path reports which).  Both outputs are
    within the bf16 tolerance of the oracle and of each other."""
    import cross_model_kv_helm_amd as hk
    w = dataclasses.replace(SMALL_BF16, name="two_kernels", n_tokens=100, seed=20)
    case = Case(w)
    d = case.dev
    a = case.run_gpu()

    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        return v
    sk, sv = shifted(d["src_k"]), shifted(d["src_v"])
    shape = (w.n_tgt_layers, w.n_kv_heads, case.T, w.head_dim)
    pk = shifted(torch.empty(shape, dtype=torch.bfloat16, device="cuda"))
    pv = shifted(torch.empty(shape, dtype=torch.bfloat16, device="cuda"))
    s = hk.make_shape(sk, d["W_k"], d["layer_sel"], w.theta, w.theta)
    assert hk.helm_kv_transfer_path(sk, sv, d["src_pos"], d["tgt_pos"], d["layer_sel"], d["W_k"], d["b_k"],
                                    d["W_v"], d["b_v"], pk, pv, s) == hk.HELM_PATH_PORTABLE
    s_al = hk.make_shape(d["src_k"], d["W_k"], d["layer_sel"], w.theta, w.theta)
    assert hk.helm_kv_transfer_path(d["src_k"], d["src_v"], d["src_pos"], d["tgt_pos"], d["layer_sel"], d["W_k"],
                                    d["b_k"], d["W_v"], d["b_v"], a[0], a[1], s_al) == hk.HELM_PATH_MATRIX
    hk.helm_kv_transfer(sk, sv, d["src_pos"], d["tgt_pos"], d["layer_sel"], d["W_k"], d["b_k"], d["W_v"],
                        d["b_v"], pk, pv, s)
    torch.cuda.synchronize()
    check_case(case, *a, label="matrix-core ")
    check_case(case, pk, pv, label="portable ")
    D = w.head_dim
    slab = np.arange(w.n_tgt_layers * w.n_kv_heads * case.T) // case.T
    for x, y, nm in ((a[0], pk, "K"), (a[1], pv, "V")):
        parity.compare(parity.storage_to_f64(parity.to_np_storage(x)).reshape(-1, D),
                       parity.storage_to_f64(parity.to_np_storage(y)).reshape(-1, D), slab, "bf16",
                       f"matrix-core vs portable {nm}")

"""Benchmark of the cross-model KV-cache transfer on one MI355X.

One step = one full transfer (RoPE table kernel + the transfer kernel) of the
Qwen3-14B -> 32B-shaped workload: 40 source -> 64 target layers, 8 KV heads,
head_dim 128, k = 4 selected source layers per target layer, 32,768 tokens,
bf16 caches and maps, fp32 bias — the configuration the headline mapper time
is quoted on (Qwen3 cache-mapping write-up, section "What the headline number
actually covers").  Inputs are seeded synthetic draws (synth/) resident in
HBM before the timed region.

Prints ONE JSON line: mapped KV tokens/s (tokens whose K and V are written
for every target layer and head), ms per 32K-token transfer, the roofline of
the transfer kernel, and the CPU oracle's throughput on a bounded sample.

The roofline's `achieved` divides the algorithmic work of one launch by the
transfer kernel's own average duration, timed live with HIP events around
the map stage alone (helm_kv_transfer_stage with HELM_STAGE_MAP, on the
stream it is launched on).  `traffic` is the HBM byte count per launch that
rocprofv3's FETCH_SIZE / WRITE_SIZE counters gave for this kernel source
(profiles/transfer_mfma_qwen3_14b_32b_t32k_counters.md, scaled by a plain
copy of known size); it is null when the kernel source has changed since.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # B/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15    # flop/s, dense bf16 matrix cores


COUNTERS_MD = os.path.join(ROOT, "profiles", "transfer_mfma_qwen3_14b_32b_t32k_counters.md")
PAGED_MD = os.path.join(ROOT, "profiles", "transfer_mfma_paged_32req_counters.md")
KERNEL_SRC = os.path.join(ROOT, "cross_model_kv_helm_amd", "csrc", "transfer_mfma.hip")
COSINE_MD = os.path.join(ROOT, "profiles", "kv_cosine_qwen3_14b_32b_t32k.md")
COSINE_SRC = os.path.join(ROOT, "cross_model_kv_helm_amd", "csrc", "cosine.hip")
WIDE_MD = os.path.join(ROOT, "profiles", "wide_gemm_qwen3_14b_32b_t32k_wide.md")
WIDE_SRC = os.path.join(ROOT, "cross_model_kv_helm_amd", "csrc", "wide.hip")
RIDGE_MD = os.path.join(ROOT, "profiles", "ridge_gram_qwen3_14b_32b_calibration.md")
RIDGE_SRC = os.path.join(ROOT, "cross_model_kv_helm_amd", "csrc", "ridge.hip")


def kernel_source_digest(path: str = KERNEL_SRC) -> str:
    """sha256 of the kernel source's code: comments (from // to the end of a
    line) and blank lines removed, trailing spaces stripped, lines joined by
    newlines, followed by the code of the local headers it includes that
    hold device code (every one but internal.hpp, the library's host-side
    declarations).  Edits to comments keep recorded counters valid; edits to
    code do not."""
    def code_lines(p):
        out = []
        with open(p) as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    out.append(code)
        return out
    lines = code_lines(path)
    for line in list(lines):
        if line.startswith('#include "') and line != '#include "internal.hpp"':
            lines += code_lines(os.path.join(os.path.dirname(path), line.split('"')[1]))
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def recorded_traffic(md: str = COUNTERS_MD, src: str = KERNEL_SRC, units: float | None = None):
    """(bytes per launch, note) from a committed counter summary, or
    (None, reason) when it is missing or was taken on another kernel source.
    A summary may record bytes per independent unit of work
    (hbm_bytes_per_group) instead of per launch; then `units` (the launch's
    count) scales it."""
    try:
        text = open(md).read()
    except OSError:
        return None, "no counter summary"
    keys = ("sha256:", "hbm_bytes_per_launch:", "hbm_bytes_per_group:")
    fields = dict(line.split(":", 1) for line in text.splitlines() if line.startswith(keys))
    if fields.get("sha256", "").strip() != kernel_source_digest(src):
        return None, "counters were taken on another kernel source"
    note = "rocprofv3 FETCH_SIZE x2 + WRITE_SIZE (copy-calibrated)"
    if "hbm_bytes_per_launch" in fields:
        return float(fields["hbm_bytes_per_launch"]), note
    if "hbm_bytes_per_group" in fields and units is not None:
        return float(fields["hbm_bytes_per_group"]) * units, note + ", per group x groups"
    return None, "no per-launch figure for this launch"


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def algorithmic_work(w, layer_sel, T):
    """(bytes, flops) one transfer must move / compute at minimum.

    bytes = every selected source layer read once (K and V) + the target
    cache written once (K and V) + W and bias read once + positions.
    flops = 2 * (K and V) * L_t * H * T * (k*D) * D (the two maps)."""
    import numpy as np
    L_t, H, D, k = w.n_tgt_layers, w.n_kv_heads, w.head_dim, w.k
    used = len(np.unique(np.asarray(layer_sel)))
    es = 2 if w.dtype == "bf16" else 4
    src = 2 * used * H * T * D * es
    tgt = 2 * L_t * H * T * D * es
    wts = 2 * L_t * H * k * D * D * es + 2 * L_t * H * D * 4
    pos = 2 * T * 4
    flops = 2 * 2 * L_t * H * T * (k * D) * D
    return src + tgt + wts + pos, flops, dict(src=src, tgt=tgt, weights=wts, positions=pos, used_src_layers=used)


def encode_keys_on_gpu(hk, k_content, src_pos, theta):
    """Position-encodes the synthetic content keys with the library itself
    (k = 1, identity map, zero bias, un-rotation at position 0): the source
    cache then holds R(src_pos) * key rounded to bf16, as a model leaves it."""
    import torch
    L, H, T, D = k_content.shape
    dev = k_content.device
    eye = torch.eye(D, dtype=k_content.dtype, device=dev).expand(L, H, D, D).contiguous()
    zero_b = torch.zeros((L, H, D), dtype=torch.float32, device=dev)
    sel = torch.arange(L, dtype=torch.int32, device=dev).reshape(L, 1)
    zeros = torch.zeros_like(src_pos)
    out_k = torch.empty_like(k_content)
    out_v = torch.empty_like(k_content)
    s = hk.make_shape(k_content, eye, sel, theta, theta)
    hk.helm_kv_transfer(k_content, k_content, zeros, src_pos, sel, eye, zero_b, eye, zero_b, out_k, out_v, s)
    torch.cuda.synchronize()
    del out_v, eye
    return out_k


def cpu_baseline(w, budget_s: float):
    """The fp64 oracle (as is) on a bounded sample of the same workload: all
    target layers and heads, K and V, for the first T_s tokens; T_s grows
    until one run takes at least budget_s/2, and that run is the measurement
    (aimed at about budget_s of CPU work)."""
    import numpy as np
    import oracle
    import synth
    from tests.parity import oracle_dtype, to_np_storage

    threads = oracle.max_threads()
    T_s, elapsed = 8, 0.0
    while True:
        c = synth.contiguous_inputs(w, device="cpu", n_tokens=T_s)
        host = {k: to_np_storage(v) for k, v in c.items() if k != "k_content"}
        host["src_k"] = oracle.encode_keys(to_np_storage(c["k_content"]), host["src_pos"], w.theta, oracle_dtype(w))
        pb = oracle.Problem(w.n_src_layers, w.n_tgt_layers, w.n_kv_heads, w.head_dim, w.k, n_tokens=T_s,
                            theta_src=w.theta, theta_tgt=w.theta, dtype=oracle_dtype(w), quantize_content=True)
        t0 = time.perf_counter()
        oracle.transfer_rows(pb, host["src_k"], host["src_v"], host["src_pos"], host["tgt_pos"],
                             host["layer_sel"], host["W_k"], host["b_k"], host["W_v"], host["b_v"])
        elapsed = time.perf_counter() - t0
        log(f"cpu oracle: {T_s} tokens in {elapsed:.2f} s on {threads} threads")
        if elapsed >= budget_s / 2 or T_s >= w.n_tokens:
            break
        T_s = min(w.n_tokens, int(T_s * max(2.0, min(8.0, budget_s / max(elapsed, 1e-3)))))
    return {"value": T_s / elapsed, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{w.name} shapes (all {w.n_tgt_layers} target layers x {w.n_kv_heads} heads, K and V), "
                      f"first {T_s} tokens, fp64 C oracle with OpenMP, {elapsed:.2f} s"}


def wide_leg(hk, synth, w, src_k, c, out_k, out_v, steps, stream):
    """The wide-input map on the same caches, positions and selection: every
    target head's key and value maps read the K and V features of all heads
    of the k selected layers (IN = k*2*H*D), with maps drawn as
    synth.wide_maps.  Times whole calls and the product kernel alone (the
    HELM_STAGE_MAP stage, after one preparation), with HIP events on the
    launch stream; the product's roofline is the matrix cores' bf16 peak."""
    import numpy as np
    import torch
    log("wide-input map: drawing maps")
    W_k, b_k, W_v, b_v = synth.wide_maps(w, src_k.device)
    T = src_k.shape[2]
    shape = hk.make_shape(src_k, W_k, c["layer_sel"], w.theta, w.theta)
    shape.stream = hk.current_stream_ptr(src_k.device)
    ws = torch.empty(hk.helm_kv_wide_workspace_bytes(shape), dtype=torch.uint8, device=src_k.device)

    def call(stages):
        hk.helm_kv_transfer_wide_stage(stages, src_k, c["src_v"], c["src_pos"], c["tgt_pos"], c["layer_sel"], W_k,
                                       b_k, W_v, b_v, out_k, out_v, shape, workspace=ws)

    n = max(2, steps // 4)          # ~72 ms per call at the 14B -> 32B shape
    for _ in range(2):
        call(hk.HELM_STAGE_ALL)
    torch.cuda.synchronize()
    res = {}
    for name, stages in (("call", hk.HELM_STAGE_ALL), ("product", hk.HELM_STAGE_MAP)):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        torch.cuda.synchronize()
        for e0, e1 in ev:
            e0.record(stream)
            call(stages)
            e1.record(stream)
        torch.cuda.synchronize()
        res[name] = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    IN = hk.wide_in(w.k, w.n_kv_heads, w.head_dim)
    flops = 2.0 * w.n_tgt_layers * T * IN * 2 * w.n_kv_heads * w.head_dim
    gms = res["product"]
    log(f"wide-input map: call {res['call']:.3f} ms, product {gms:.3f} ms, "
        f"{flops / (gms * 1e-3) / 1e12:.1f} TFLOP/s over {n} launches")
    traffic, note = recorded_traffic(WIDE_MD, WIDE_SRC)
    del ws, W_k, W_v
    torch.cuda.empty_cache()
    return {"ms_per_transfer": res["call"], "tokens_per_s": T / (res["call"] * 1e-3), "in_features": IN,
            "launches": n, "kernel": "wide_gemm_kernel",
            "roofline": {"bound": "mfma", "achieved": flops / (gms * 1e-3) / 1e12,
                         "peak": MFMA_BF16_PEAK / 1e12, "unit": "TFLOP/s",
                         "frac": flops / (gms * 1e-3) / MFMA_BF16_PEAK, "traffic": traffic,
                         "kernel_ms": gms, "algorithmic_flops": flops, "traffic_source": note}}


def paged_leg(hk, synth, steps, stream):
    """The paged transfer (block tables, 16-token pages) on its workload:
    28 -> 28 layers, 8 heads, k = 4, 32 requests of 256 .. 16,384 tokens with
    per-request target offsets, pools with 12.5% spare blocks in seeded
    permutation order (synth.paged_layout).  Times whole calls (tables,
    slot maps, the keys and values launches) with HIP events; the roofline
    divides the transfer's algorithmic bytes by that time."""
    import numpy as np
    import torch
    dev = torch.device("cuda:0")
    w = synth.CONFIGS["paged_32req"]
    lay = synth.paged_layout(w)
    N = lay.n_tokens
    log(f"paged transfer: {len(lay.lens)} requests, {N} tokens; building pools")
    c = synth.paged_content(w, lay, device=dev)
    k_enc = encode_keys_on_gpu(hk, c.pop("k_content"), c["src_pos"], w.theta)
    src_k_pool = synth.scatter_to_pool(k_enc, lay, lay.src_bt, lay.n_src_blocks)
    del k_enc
    src_v_pool = synth.scatter_to_pool(c.pop("src_v"), lay, lay.src_bt, lay.n_src_blocks)
    torch.cuda.empty_cache()
    tk = synth.empty_target_pool(w, lay, dev)
    tv = synth.empty_target_pool(w, lay, dev)
    sbt, tbt, cu = (torch.from_numpy(x).to(dev) for x in (lay.src_bt, lay.tgt_bt, lay.cu_seqlens))
    shape = hk.make_paged_shape(src_k_pool, tk, c["W_k"], c["layer_sel"], sbt, tbt, N, w.theta, w.theta)
    if hk.helm_paged_check(shape, lay.src_bt, lay.tgt_bt, lay.cu_seqlens) != 0:
        raise SystemExit(f"paged check failed: {hk.helm_last_error()}")
    shape.stream = hk.current_stream_ptr(dev)
    ws = torch.empty(hk.helm_kv_paged_workspace_bytes(shape), dtype=torch.uint8, device=dev)

    def call():
        hk.helm_kv_transfer_paged(src_k_pool, src_v_pool, sbt, tbt, cu, c["src_pos"], c["tgt_pos"],
                                  c["layer_sel"], c["W_k"], c["b_k"], c["W_v"], c["b_v"], tk, tv, shape,
                                  workspace=ws)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in ev:
        e0.record(stream)
        call()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    B, F, parts = algorithmic_work(w, c["layer_sel"].cpu().numpy(), N)
    B += 2 * lay.src_bt.size * 4 + (len(lay.lens) + 1) * 4   # the block tables and cu_seqlens
    traffic, note = recorded_traffic(PAGED_MD, KERNEL_SRC)
    log(f"paged transfer: {ms:.3f} ms for {N} tokens, {N / ms * 1e3 / 1e6:.2f} M tok/s, "
        f"{B / (ms * 1e-3) / 1e12:.2f} TB/s algorithmic")
    del src_k_pool, src_v_pool, tk, tv, ws, c
    torch.cuda.empty_cache()
    return {"ms_per_transfer": ms, "tokens": N, "requests": int(len(lay.lens)), "tokens_per_s": N / (ms * 1e-3),
            "launches": steps, "kernel": "transfer_mfma_kernel (paged instantiations), whole call",
            "config": {"src_layers": w.n_src_layers, "tgt_layers": w.n_tgt_layers, "kv_heads": w.n_kv_heads,
                       "head_dim": w.head_dim, "k": w.k, "block_size": lay.block_size},
            "roofline": {"bound": "hbm", "achieved": B / (ms * 1e-3) / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                         "frac": B / (ms * 1e-3) / HBM_PEAK, "traffic": traffic, "algorithmic_bytes": B,
                         "mfma_frac": F / (ms * 1e-3) / MFMA_BF16_PEAK, "traffic_source": note}}


def config_leg(hk, synth, name, steps, stream):
    """One more contiguous configuration, timed like the main workload: whole
    transfers (tables + map) with HIP events on the launch stream, inputs
    resident in HBM; workloads that fit the 256 MB last-level cache get a
    512 MB buffer rewritten between steps, so they are timed from HBM.  The
    roofline divides the configuration's algorithmic bytes and flops by the
    map stage's time in the same steps."""
    import numpy as np
    import torch
    dev = torch.device("cuda:0")
    w = synth.CONFIGS[name]
    c = synth.contiguous_inputs(w, device=dev)
    src_k = encode_keys_on_gpu(hk, c.pop("k_content"), c["src_pos"], w.theta)
    T = src_k.shape[2]
    out_k = torch.empty((w.n_tgt_layers, w.n_kv_heads, T, w.head_dim), dtype=src_k.dtype, device=dev)
    out_v = torch.empty_like(out_k)
    shape = hk.make_shape(src_k, c["W_k"], c["layer_sel"], w.theta, w.theta)
    shape.stream = hk.current_stream_ptr(dev)
    ws = torch.empty(hk.helm_kv_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if out_k.numel() * 8 < (1 << 30) else None

    def st(stages):
        hk.helm_kv_transfer_stage(stages, src_k, c["src_v"], c["src_pos"], c["tgt_pos"], c["layer_sel"], c["W_k"],
                                  c["b_k"], c["W_v"], c["b_v"], out_k, out_v, shape, workspace=ws)

    for _ in range(3):
        st(hk.HELM_STAGE_ALL)
    n = steps if flush is None else max(steps, 50)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        if flush is not None:
            flush.fill_(i & 0xFF)
        ev[i][0].record(stream)
        st(hk.HELM_STAGE_TABLES)
        ev[i][1].record(stream)
        st(hk.HELM_STAGE_MAP)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    ms = float(np.median([e[0].elapsed_time(e[2]) for e in ev]))
    kms = float(np.median([e[1].elapsed_time(e[2]) for e in ev]))
    B, F, parts = algorithmic_work(w, c["layer_sel"].cpu().numpy(), T)
    t_hbm, t_mfma = B / HBM_PEAK, F / MFMA_BF16_PEAK
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    hbm_frac, mfma_frac = B / (kms * 1e-3) / HBM_PEAK, F / (kms * 1e-3) / MFMA_BF16_PEAK
    log(f"{name}: transfer {ms:.4f} ms (median of {n}), map stage {kms:.4f} ms, HBM {hbm_frac:.3f}, "
        f"MFMA {mfma_frac:.3f} of peak")
    del src_k, out_k, out_v, ws, c, flush
    torch.cuda.empty_cache()
    roof = ({"bound": "hbm", "achieved": B / (kms * 1e-3) / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
             "frac": hbm_frac} if bound == "hbm" else
            {"bound": "mfma", "achieved": F / (kms * 1e-3) / 1e12, "peak": MFMA_BF16_PEAK / 1e12,
             "unit": "TFLOP/s", "frac": mfma_frac})
    roof.update({"kernel_ms": kms, "hbm_frac": hbm_frac, "mfma_frac": mfma_frac, "algorithmic_bytes": B,
                 "algorithmic_flops": F, "traffic": None, "binding_time_ms": max(t_hbm, t_mfma) * 1e3,
                 "roofline_frac_of_binding": max(t_hbm, t_mfma) / (kms * 1e-3)})
    return {"workload": name, "tokens": T, "ms_per_transfer": ms, "tokens_per_s": T / (ms * 1e-3),
            "steps": n, "statistic": "median", "positions": w.positions,
            "config": {"src_layers": w.n_src_layers, "tgt_layers": w.n_tgt_layers, "kv_heads": w.n_kv_heads,
                       "head_dim": w.head_dim, "k": w.k},
            "roofline": roof}


def ridge_leg(hk, synth, w, groups, steps, stream):
    """The ridge fit of the maps at the calibration's shape: one group per
    (target layer, head, K|V) map of the 40 -> 64-layer pair (64 x 8 x 2 =
    1,024 groups), ~128K observations each (131,072), IN = k*D = 512 inputs
    and D = 128 targets per observation; synthetic observations
    (synth.ridge_inputs).  Fewer groups (a multiple of 8) when device memory
    is short; the line says how many.  Times whole fits and the two stages
    alone with HIP events on the launch stream; the roofline of the Gram
    kernel counts the symmetric half of X^T X, X^T Y and the sums."""
    import numpy as np
    import torch
    dev = torch.device("cuda:0")
    N, IN, D = 131072, w.k * w.head_dim, w.head_dim
    per_group = N * (IN + D) * 2 + IN * IN * 4 + IN * D * 4 + (IN + D) * 8 + IN * (IN + D) * 8 + IN * D * 4 + D * 4
    free, total = torch.cuda.mem_get_info(dev)
    # headroom beyond the leg's own tensors: the input draws' 6 GiB of
    # temporaries, and device memory that tools attached to the process
    # (profilers collecting counters per dispatch) allocate as it runs
    headroom = (6 << 30) + max(16 << 30, total // 20)
    fit_groups = min(groups, int((free - headroom) // per_group) // 8 * 8)
    if fit_groups < 8:
        log(f"ridge fit: skipped ({free / 2**30:.1f} GiB free)")
        return {"skipped": f"{free / 2**30:.1f} GiB of device memory free"}
    log(f"ridge fit: drawing {fit_groups} groups of {N} x {IN} observations")
    X, Y = synth.ridge_inputs(fit_groups, N, IN, D, 511, dev)
    shape = hk.ridge_shape(fit_groups, N, IN, D, 0.01)
    ws = torch.empty(hk.helm_ridge_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    W = torch.empty((fit_groups, IN, D), dtype=torch.float32, device=dev)
    b = torch.empty((fit_groups, D), dtype=torch.float32, device=dev)

    def call(stages):
        hk.helm_ridge_fit(X, Y, lam=0.01, W=W, b=b, workspace=ws, stages=stages)

    call(hk.HELM_STAGE_ALL)
    torch.cuda.synchronize()
    n = max(2, steps // 4)
    res = {}
    for name, stages in (("fit", hk.HELM_STAGE_ALL), ("gram", hk.HELM_STAGE_TABLES), ("solve", hk.HELM_STAGE_MAP)):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        torch.cuda.synchronize()
        for e0, e1 in ev:
            e0.record(stream)
            call(stages)
            e1.record(stream)
        torch.cuda.synchronize()
        res[name] = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    flops = float(fit_groups) * (N * IN * (IN + 1) + 2.0 * N * IN * D)
    gms = res["gram"]
    log(f"ridge fit: {fit_groups} groups, fit {res['fit']:.3f} ms (gram {gms:.3f}, solve {res['solve']:.3f}), "
        f"{flops / (gms * 1e-3) / 1e12:.1f} TFLOP/s in the Gram kernel")
    traffic, note = recorded_traffic(RIDGE_MD, RIDGE_SRC, units=fit_groups)
    finite = bool(torch.isfinite(W).all().item() and torch.isfinite(b).all().item())
    del X, Y, ws, W, b
    torch.cuda.empty_cache()
    return {"groups": fit_groups, "observations": N, "in_features": IN, "out_features": D, "lambda": 0.01,
            "ms_per_fit": res["fit"], "gram_ms": gms, "solve_ms": res["solve"], "launches": n,
            "groups_per_s": fit_groups / (res["fit"] * 1e-3), "finite": finite, "kernel": "ridge_gram_kernel",
            "roofline": {"bound": "mfma", "achieved": flops / (gms * 1e-3) / 1e12, "peak": MFMA_BF16_PEAK / 1e12,
                         "unit": "TFLOP/s", "frac": flops / (gms * 1e-3) / MFMA_BF16_PEAK, "traffic": traffic,
                         "kernel_ms": gms, "algorithmic_flops": flops, "traffic_source": note}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_14b_32b_t32k")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work (0 = skip)")
    ap.add_argument("--wide", type=int, default=1, help="also time the wide-input map (0 = skip)")
    ap.add_argument("--paged", type=int, default=1, help="also time the paged transfer (0 = skip)")
    ap.add_argument("--configs", default="qwen3_0.6b_1.7b_t512,qwen3_0.6b_1.7b_t2048,qwen3_14b_32b_t128k_shift",
                    help="other contiguous configurations timed after the main one (comma list; '' = none)")
    ap.add_argument("--ridge-groups", type=int, default=1024,
                    help="groups of the ridge-fit leg (0 = skip); fewer when device memory is short")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB three times (the reference "
                         "kernel that scales HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the transfer shards by KV head with no exchange, "
              f"so one MI355X's throughput is the figure (got --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import cross_model_kv_helm_amd as hk
    import synth

    if not os.path.exists(hk.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if hk.helm_device_check(0) != 0:
        raise SystemExit(f"device check failed: {hk.helm_last_error()}")

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copied {args.copy_calibration_mib} MiB three times (reads {n} B, writes {n} B per copy)")
        return

    w = synth.CONFIGS[args.workload]
    assert not w.paged, "bench.py times the contiguous workloads"
    log(f"workload {w.name}: drawing inputs on the GPU")
    c = synth.contiguous_inputs(w, device=dev)
    src_k = encode_keys_on_gpu(hk, c.pop("k_content"), c["src_pos"], w.theta)
    T = src_k.shape[2]
    out_shape = (w.n_tgt_layers, w.n_kv_heads, T, w.head_dim)
    out_k = torch.empty(out_shape, dtype=src_k.dtype, device=dev)
    out_v = torch.empty(out_shape, dtype=src_k.dtype, device=dev)
    shape = hk.make_shape(src_k, c["W_k"], c["layer_sel"], w.theta, w.theta)
    shape.stream = hk.current_stream_ptr(dev)
    ws = torch.empty(hk.helm_kv_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    # a buffer larger than the 256 MB last-level cache, rewritten between steps
    # so small workloads are timed from HBM, not from cache
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if out_k.numel() * 4 < (1 << 30) else None

    def step(stages=hk.HELM_STAGE_ALL):
        hk.helm_kv_transfer_stage(stages, src_k, c["src_v"], c["src_pos"], c["tgt_pos"], c["layer_sel"], c["W_k"],
                                  c["b_k"], c["W_v"], c["b_v"], out_k, out_v, shape, workspace=ws)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # each timed step is the two stages of one transfer, with an event
    # between them: the step time (tables + map) and the transfer kernel's
    # time (the map stage: its keys and values launches) come from the same
    # launches, so the kernel time never exceeds the step time
    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        if flush is not None:
            flush.fill_(i & 0xFF)
        ev[i][0].record(stream)
        step(hk.HELM_STAGE_TABLES)
        ev[i][1].record(stream)
        step(hk.HELM_STAGE_MAP)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per = np.array([e[0].elapsed_time(e[2]) for e in ev])   # ms
    kper = np.array([e[1].elapsed_time(e[2]) for e in ev])
    ms = float(per.mean())
    kms = float(kper.mean())
    log(f"per step: mean {ms:.4f} ms, median {np.median(per):.4f}, p10 {np.percentile(per, 10):.4f}, "
        f"p90 {np.percentile(per, 90):.4f}; wall {wall:.3f} s")
    log(f"transfer kernel (map stage) in the same steps: mean {kms:.4f} ms, median {np.median(kper):.4f}")

    # the KV-cosine diagnostic on the mapped cache against a reference cache
    # of the same shape (here a copy: the timing does not depend on values)
    log(f"timing {args.steps} launches of the KV-cosine diagnostic")
    ref_k, ref_v = out_k.clone(), out_v.clone()
    cos_out = torch.empty((2, w.n_tgt_layers, w.n_kv_heads), dtype=torch.float32, device=dev)
    hk.helm_kv_cosine(out_k, out_v, ref_k, ref_v, shape, out=cos_out)
    cstarts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    cends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        cstarts[i].record(stream)
        hk.helm_kv_cosine(out_k, out_v, ref_k, ref_v, shape, out=cos_out)
        cends[i].record(stream)
    torch.cuda.synchronize()
    cms = float(np.mean([s_.elapsed_time(e_) for s_, e_ in zip(cstarts, cends)]))
    cos_bytes = 4 * out_k.numel() * out_k.element_size()   # both caches, K and V, read once
    log(f"KV cosine: mean {cms:.4f} ms, {cos_bytes / cms / 1e6:.1f} GB/s (reference = a copy: timing only)")
    del ref_k, ref_v
    cos_traffic, cos_note = recorded_traffic(COSINE_MD, COSINE_SRC)
    kv_cos = {"ms": cms, "kernel": "kv_cosine_kernel",
              "reference": "a copy of the mapped cache: the time does not depend on the values, so the "
                           "cosines themselves carry no information here (parity tests check them)",
              "roofline": {"bound": "hbm", "achieved": cos_bytes / (cms * 1e-3) / 1e9, "peak": HBM_PEAK / 1e9,
                           "unit": "GB/s", "frac": cos_bytes / (cms * 1e-3) / HBM_PEAK, "traffic": cos_traffic,
                           "algorithmic_bytes": cos_bytes, "traffic_source": cos_note}}

    wide = wide_leg(hk, synth, w, src_k, c, out_k, out_v, args.steps, stream) if args.wide else None
    others = [config_leg(hk, synth, nm, args.steps, stream) for nm in args.configs.split(",") if nm]
    paged = paged_leg(hk, synth, args.steps, stream) if args.paged else None
    ridge = ridge_leg(hk, synth, w, args.ridge_groups, args.steps, stream) if args.ridge_groups > 0 else None

    B, F, parts = algorithmic_work(w, c["layer_sel"].cpu().numpy(), T)
    t_s = ms * 1e-3
    t_k = kms * 1e-3
    hbm_frac = B / t_k / HBM_PEAK
    mfma_frac = F / t_k / MFMA_BF16_PEAK
    t_hbm, t_mfma = B / HBM_PEAK, F / MFMA_BF16_PEAK
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    traffic, traffic_note = recorded_traffic()
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": B / t_k / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                "frac": hbm_frac, "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": F / t_k / 1e12, "peak": MFMA_BF16_PEAK / 1e12, "unit": "TFLOP/s",
                "frac": mfma_frac, "traffic": traffic}
    roof["kernel"] = "transfer_mfma_kernel"
    roof["kernel_ms"] = kms
    roof["mfma_frac"] = mfma_frac
    roof["hbm_frac"] = hbm_frac
    roof["algorithmic_bytes"] = B
    roof["algorithmic_flops"] = F
    roof["traffic_source"] = traffic_note

    cpu = None
    if args.cpu_budget > 0:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(w, args.cpu_budget)

    line = {
        "metric": "mapped KV tokens/s (and ms per 32K-token transfer)",
        "value": T / t_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_transfer": ms,
        "higher_is_better": True,
        "scaling": None,
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "src_layers": w.n_src_layers, "tgt_layers": w.n_tgt_layers,
                   "kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "k": w.k, "tokens": T,
                   "rope_theta": w.theta, "positions": w.positions, "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "bytes_breakdown": parts,
        "other_configs": others,
        "kv_cosine": kv_cos,
        "wide_map": wide,
        "paged": paged,
        "ridge_fit": ridge,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Parity helpers: build seeded cases, run the HIP library, compare with the oracle.

Tolerance rule (bf16 storage), per slab (K|V, target layer, head) over the
compared rows: with ref the fp64 oracle in quantize-content mode (the content
key rounded once to bf16 — the map is a bf16 contraction) and gpu the
library's bf16 output,
    excess_e = max(0, |gpu_e - ref_e| - ulp_bf16(max(|ref_e|, |gpu_e|)) / 2)
    pass  iff  max excess <= 1e-2 * rms(ref)  and  cosine(gpu, ref) >= 0.9999.
The half-ulp exemption is the output's own rounding: no bf16 writer can do
better, and above |x| = 4 half an ulp alone exceeds 1e-2 * rms.
fp32 storage: max |gpu - ref| <= 1e-5 * rms(ref) per slab.
"""
from __future__ import annotations

import math
import time

import numpy as np
import torch

import oracle
import synth

BF16_TOL = 1e-2
COS_TOL = 0.9999
F32_TOL = 1e-5


def log(msg: str) -> None:
    print(f"[parity {time.strftime('%H:%M:%S')}] {msg}", flush=True)


def to_np_storage(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def from_np_storage(a: np.ndarray, device) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def storage_to_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def oracle_dtype(w: synth.Workload) -> int:
    return oracle.BF16 if w.dtype == "bf16" else oracle.F32


class Case:
    """One contiguous case: device tensors for the library, host copies for the oracle."""

    def __init__(self, w: synth.Workload, device="cuda", n_tokens=None, layer_sel=None,
                 src_pos=None, tgt_pos=None):
        self.w = w
        c = synth.contiguous_inputs(w, device=device, n_tokens=n_tokens)
        if layer_sel is not None:
            c["layer_sel"] = torch.as_tensor(np.asarray(layer_sel, np.int32)).to(device)
        if src_pos is not None:
            c["src_pos"] = torch.as_tensor(np.asarray(src_pos, np.int32)).to(device)
        if tgt_pos is not None:
            c["tgt_pos"] = torch.as_tensor(np.asarray(tgt_pos, np.int32)).to(device)
        self.T = c["k_content"].shape[2]
        self.host = {k: to_np_storage(v) for k, v in c.items() if k != "k_content"}
        # the source key cache holds the content keys position-encoded at src_pos
        self.host["src_k"] = oracle.encode_keys(to_np_storage(c.pop("k_content")), self.host["src_pos"],
                                                w.theta, oracle_dtype(w))
        c["src_k"] = from_np_storage(self.host["src_k"], device)
        self.dev = c

    def problem(self) -> oracle.Problem:
        w = self.w
        return oracle.Problem(w.n_src_layers, w.n_tgt_layers, w.n_kv_heads, w.head_dim, w.k,
                              n_tokens=self.T, theta_src=w.theta, theta_tgt=w.theta,
                              dtype=oracle_dtype(w), quantize_content=True)

    def run_gpu(self, out=None):
        import cross_model_kv_helm_amd as hk
        d, w = self.dev, self.w
        if out is None:
            shape = (w.n_tgt_layers, w.n_kv_heads, self.T, w.head_dim)
            out = (torch.empty(shape, dtype=d["src_k"].dtype, device=d["src_k"].device),
                   torch.empty(shape, dtype=d["src_k"].dtype, device=d["src_k"].device))
        s = hk.make_shape(d["src_k"], d["W_k"], d["layer_sel"], w.theta, w.theta)
        hk.helm_kv_transfer(d["src_k"], d["src_v"], d["src_pos"], d["tgt_pos"], d["layer_sel"], d["W_k"],
                            d["b_k"], d["W_v"], d["b_v"], out[0], out[1], s)
        return out

    def oracle_rows(self, rows=None, quantize_content=True):
        h = self.host
        pb = self.problem()
        pb.quantize_content = quantize_content
        return oracle.transfer_rows(pb, h["src_k"], h["src_v"], h["src_pos"], h["tgt_pos"],
                                    h["layer_sel"], h["W_k"], h["b_k"], h["W_v"], h["b_v"], rows=rows)


def sample_rows(L_t: int, H: int, T: int, per_slab: int, seed: int, tile: int = 0) -> np.ndarray:
    """Flat rows (l*H + h)*T + t: per (l, h) slab the first and last token,
    tile edges, `per_slab` random tokens on top of those, and, when `tile` is
    set, one random token inside every `tile`-token window [i*tile, (i+1)*tile)
    so that every tile of a launch's schedule is compared in every slab."""
    rng = np.random.default_rng(seed)
    fixed = np.array(sorted({0, T - 1, min(T - 1, 15), min(T - 1, 16), min(T - 1, 63), min(T - 1, 64), T // 2}))
    n_tiles = (T + tile - 1) // tile if tile else 0
    starts = np.arange(n_tiles, dtype=np.int64) * tile if tile else None
    out = []
    for g in range(L_t * H):
        parts = [fixed, rng.integers(0, T, per_slab)]
        if tile:
            span = np.minimum(starts + tile, T) - starts
            parts.append(starts + (rng.random(n_tiles) * span).astype(np.int64))
        out.append(g * T + np.unique(np.concatenate(parts)))
    return np.concatenate(out).astype(np.int64)


def gather_rows(out: torch.Tensor, rows: np.ndarray) -> np.ndarray:
    D = out.shape[-1]
    idx = torch.from_numpy(rows).to(out.device)
    return storage_to_f64(to_np_storage(out.reshape(-1, D).index_select(0, idx)))


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def slab_stats(gpu: np.ndarray, ref: np.ndarray, dtype: str) -> dict:
    diff = np.abs(gpu - ref)
    rms = math.sqrt(float(np.mean(ref * ref)))
    cos = float(np.sum(gpu * ref) / max(np.linalg.norm(gpu) * np.linalg.norm(ref), 1e-300))
    if dtype == "bf16":
        excess = np.maximum(0.0, diff - bf16_half_ulp(np.maximum(np.abs(ref), np.abs(gpu))))
        ok = excess.max() <= BF16_TOL * rms and cos >= COS_TOL
        return dict(ok=bool(ok), max_excess_rel=float(excess.max() / rms), max_err_rel=float(diff.max() / rms),
                    cos=cos, rms=rms)
    ok = diff.max() <= F32_TOL * rms
    return dict(ok=bool(ok), max_err_rel=float(diff.max() / rms), cos=cos, rms=rms)


def compare(gpu: np.ndarray, ref: np.ndarray, slab_of_row: np.ndarray, dtype: str, name: str) -> dict:
    """Per-slab comparison; raises AssertionError naming the worst slab."""
    assert gpu.shape == ref.shape
    assert np.isfinite(gpu).all(), f"{name}: non-finite GPU output"
    stats = [(int(s), slab_stats(gpu[slab_of_row == s].ravel(), ref[slab_of_row == s].ravel(), dtype))
             for s in np.unique(slab_of_row)]
    metric = (lambda st: st["max_excess_rel"]) if dtype == "bf16" else (lambda st: st["max_err_rel"])
    n_bad = sum(not st["ok"] for _, st in stats)
    worst_slab, worst = max(stats, key=lambda x: (not x[1]["ok"], metric(x[1])))
    summary = dict(name=name, slabs=len(stats), bad=n_bad, worst_slab=worst_slab, **worst,
                   min_cos=min(st["cos"] for _, st in stats))
    log(f"{name}: {summary}")
    assert n_bad == 0, f"{name}: {n_bad} slab(s) out of tolerance; worst {summary}"
    return summary


def check_case(case: Case, out_k: torch.Tensor, out_v: torch.Tensor, rows=None, label="", exact=False):
    """Compares the library's outputs with the oracle on `rows` (all when None).
    With `exact`, also reports (never gates) the same outputs against the
    oracle without the bf16 operand rounding (EXACT mode): what the mandated
    bf16 contraction costs against the unrounded definition."""
    w = case.w
    D = w.head_dim
    if rows is None:
        ref_k, ref_v = case.oracle_rows(None)
        ref_k, ref_v = ref_k.reshape(-1, D), ref_v.reshape(-1, D)
        g_k = storage_to_f64(to_np_storage(out_k)).reshape(-1, D)
        g_v = storage_to_f64(to_np_storage(out_v)).reshape(-1, D)
        slab = np.arange(ref_k.shape[0]) // case.T
    else:
        ref_k, ref_v = case.oracle_rows(rows)
        g_k, g_v = gather_rows(out_k, rows), gather_rows(out_v, rows)
        slab = rows // case.T
    sk = compare(g_k, ref_k, slab, w.dtype, f"{label}{w.name} K")
    sv = compare(g_v, ref_v, slab, w.dtype, f"{label}{w.name} V")
    if exact:
        ex_k, ex_v = case.oracle_rows(rows, quantize_content=False)
        sk["exact"] = exact_report(g_k, ex_k.reshape(-1, D), slab, f"{label}{w.name} K")
        sv["exact"] = exact_report(g_v, ex_v.reshape(-1, D), slab, f"{label}{w.name} V")
    return sk, sv


def exact_report(gpu: np.ndarray, ref: np.ndarray, slab_of_row: np.ndarray, name: str) -> dict:
    """EXACT-mode statistics (reported, not gated): per slab max |gpu - ref| /
    rms(ref), the excess over half an output ulp / rms, and the cosine; the
    worst over slabs, plus the overall rms error / rms."""
    worst_err = worst_excess = 0.0
    min_cos = 1.0
    sq_err = sq_ref = 0.0
    for s in np.unique(slab_of_row):
        g, r = gpu[slab_of_row == s].ravel(), ref[slab_of_row == s].ravel()
        st = slab_stats(g, r, "bf16")
        worst_err = max(worst_err, st["max_err_rel"])
        worst_excess = max(worst_excess, st["max_excess_rel"])
        min_cos = min(min_cos, st["cos"])
        sq_err += float(np.sum((g - r) ** 2))
        sq_ref += float(np.sum(r * r))
    rep = dict(max_err_rel=worst_err, max_excess_rel=worst_excess, min_cos=min_cos,
               rms_err_rel=math.sqrt(sq_err / max(sq_ref, 1e-300)))
    log(f"{name} EXACT mode (reported, not gated): {rep}")
    return rep


class PagedCase:
    def __init__(self, w: synth.Workload, lens=None):
        self.w = w
        self.lay = lay = synth.paged_layout(w, lens=lens)
        c = synth.paged_content(w, lay, device="cuda")
        dt = oracle_dtype(w)
        k_enc = oracle.encode_keys(to_np_storage(c.pop("k_content")), lay.src_pos, w.theta, dt)
        k_dev = from_np_storage(k_enc, "cuda")
        del k_enc
        self.dev = dict(c)
        self.dev["src_k_pool"] = synth.scatter_to_pool(k_dev, lay, lay.src_bt, lay.n_src_blocks, synth.CANARY_BITS)
        self.dev["src_v_pool"] = synth.scatter_to_pool(c["src_v"], lay, lay.src_bt, lay.n_src_blocks, synth.CANARY_BITS)
        del k_dev, self.dev["src_v"]
        for name, arr in (("src_bt", lay.src_bt), ("tgt_bt", lay.tgt_bt), ("cu", lay.cu_seqlens)):
            self.dev[name] = torch.from_numpy(arr).cuda()
        self.host = {k: to_np_storage(v) for k, v in self.dev.items()}

    def run_gpu(self):
        import cross_model_kv_helm_amd as hk
        d, w, lay = self.dev, self.w, self.lay
        tk = synth.empty_target_pool(w, lay, "cuda")
        tv = synth.empty_target_pool(w, lay, "cuda")
        s = hk.make_paged_shape(d["src_k_pool"], tk, d["W_k"], d["layer_sel"], d["src_bt"], d["tgt_bt"],
                                lay.n_tokens, w.theta, w.theta)
        assert hk.helm_paged_check(s, lay.src_bt, lay.tgt_bt, lay.cu_seqlens) == 0, hk.helm_last_error()
        hk.helm_kv_transfer_paged(d["src_k_pool"], d["src_v_pool"], d["src_bt"], d["tgt_bt"], d["cu"],
                                  d["src_pos"], d["tgt_pos"], d["layer_sel"], d["W_k"], d["b_k"], d["W_v"],
                                  d["b_v"], tk, tv, s)
        return tk, tv

    def check(self, tk, tv, rows=None):
        w, lay, h = self.w, self.lay, self.host
        pb = oracle.Problem(w.n_src_layers, w.n_tgt_layers, w.n_kv_heads, w.head_dim, w.k,
                            n_tokens=lay.n_tokens, theta_src=w.theta, theta_tgt=w.theta,
                            dtype=oracle_dtype(w))
        pg = oracle.Paged(lay.block_size, len(lay.lens), lay.max_blocks, lay.max_blocks,
                          lay.n_src_blocks, lay.n_tgt_blocks)
        ref_k, ref_v, dst = oracle.transfer_paged_rows(
            pb, pg, h["src_k_pool"], h["src_v_pool"], h["src_bt"], h["tgt_bt"], h["cu"], h["src_pos"],
            h["tgt_pos"], h["layer_sel"], h["W_k"], h["b_k"], h["W_v"], h["b_v"], rows=rows)
        D = w.head_dim
        idx = torch.from_numpy(dst[:, None] + np.arange(D)[None, :]).cuda()
        g_k = storage_to_f64(to_np_storage(tk.reshape(-1)[idx]))
        g_v = storage_to_f64(to_np_storage(tv.reshape(-1)[idx]))
        n_rows = np.arange(ref_k.shape[0]) if rows is None else rows
        slab = n_rows // lay.n_tokens
        compare(g_k, ref_k, slab, w.dtype, f"{w.name} K")
        compare(g_v, ref_v, slab, w.dtype, f"{w.name} V")
        # every slot no token owns still holds the canary
        owned = torch.from_numpy(synth.slot_index(lay, lay.tgt_bt)).cuda()
        for pool in (tk, tv):
            bits, canary = synth.canary_view(pool)
            flat = bits.view(w.n_tgt_layers, -1, w.n_kv_heads, D)
            mask = torch.ones(flat.shape[1], dtype=torch.bool, device="cuda")
            mask[owned] = False
            assert bool((flat[:, mask] == canary).all()), "a slot outside every request was written"
            assert not bool((flat[:, owned] == canary).any()), "an owned slot was not written"


class WideCase:
    """Device tensors for the library, host copies for the oracle."""

    def __init__(self, w: synth.Workload):
        self.w = w
        c = synth.contiguous_inputs(w, device="cuda")
        c["W_k"], c["b_k"], c["W_v"], c["b_v"] = synth.wide_maps(w, "cuda")
        self.T = c["k_content"].shape[2]
        self.host = {k: to_np_storage(v) for k, v in c.items() if k != "k_content"}
        self.host["src_k"] = oracle.encode_keys(to_np_storage(c.pop("k_content")), self.host["src_pos"],
                                                w.theta, oracle.BF16)
        c["src_k"] = from_np_storage(self.host["src_k"], "cuda")
        self.dev = c

    def run_gpu(self):
        import cross_model_kv_helm_amd as hk
        d, w = self.dev, self.w
        shape = (w.n_tgt_layers, w.n_kv_heads, self.T, w.head_dim)
        out = (torch.empty(shape, dtype=torch.bfloat16, device="cuda"),
               torch.empty(shape, dtype=torch.bfloat16, device="cuda"))
        s = hk.make_shape(d["src_k"], d["W_k"], d["layer_sel"], w.theta, w.theta)
        hk.helm_kv_transfer_wide(d["src_k"], d["src_v"], d["src_pos"], d["tgt_pos"], d["layer_sel"], d["W_k"],
                                 d["b_k"], d["W_v"], d["b_v"], out[0], out[1], s)
        return out

    def check(self, out_k, out_v, rows=None, label=""):
        w, h, D = self.w, self.host, self.w.head_dim
        pb = oracle.Problem(w.n_src_layers, w.n_tgt_layers, w.n_kv_heads, D, w.k, n_tokens=self.T,
                            theta_src=w.theta, theta_tgt=w.theta, dtype=oracle.BF16, quantize_content=True)
        ref_k, ref_v = oracle.transfer_wide_rows(pb, h["src_k"], h["src_v"], h["src_pos"], h["tgt_pos"],
                                                 h["layer_sel"], h["W_k"], h["b_k"], h["W_v"], h["b_v"], rows=rows)
        gk = storage_to_f64(to_np_storage(out_k)).reshape(-1, D)
        gv = storage_to_f64(to_np_storage(out_v)).reshape(-1, D)
        if rows is None:
            rows = np.arange(gk.shape[0])
        else:
            gk, gv = gk[rows], gv[rows]
        slab = rows // self.T
        sk = compare(gk, ref_k.reshape(-1, D), slab, "bf16", f"{label}{w.name} K")
        sv = compare(gv, ref_v.reshape(-1, D), slab, "bf16", f"{label}{w.name} V")
        log(f"{label}{w.name}: {len(rows)} rows; K {sk}; V {sv}")

"""Seeded synthetic inputs for the cross-model KV-cache transfer.

This module only draws numbers and lays them out.  It holds none of the
transfer's arithmetic (no rotation, no map), so the oracle and the HIP path
can both take their inputs from it without sharing any of the method.

Workloads stand in for real Qwen3 caches and fitted maps, which are not
available: the shapes are those of the pairs the pages discuss (Qwen3-0.6B ->
1.7B in "Helm Intelligent Routing", section "What the transfer costs";
Qwen3-14B -> 32B in the Qwen3 cache-mapping write-up, section "What the
headline number actually covers"), with prompts of 512 to 131,072 tokens.

Recipe (all draws seeded; big tensors are drawn on the device they are
used on, per source layer, with torch's counter-based Philox generator):

* content keys  k[l, h, t, d] = z * s_K[l, h, d],  z ~ N(0, 1),
  s_K = exp(0.5 * N(0, 1)) one scale per (layer, head, channel);
  the cache holds these keys position-encoded at src_pos — that encoding is
  the method's own rotation, so the caller applies it (the tests with the
  oracle, the benchmark with the library), never this module;
* values        v[l, h, t, d] = z' * s_V[l, h, d], drawn like the keys;
* maps          W ~ N(0, 1/(k*D)) (the second parameter is a variance),
  biases b ~ N(0, 0.01) (variance; std 0.1), kept in fp32;
* wide maps     (the wide-input map, IN = k*2*H*D input features)
  W ~ N(0, 1/IN), biases as above;
* ridge data    (calibration observations of the ridge fit) X[g, n, i] =
  (z + m[g, i]) * s[g, i] and Y[g, n, d] drawn the same way, independently
  of X: z ~ N(0, 1), per-feature means m ~ N(0, 1) and scales
  s = exp(0.5 * N(0, 1)), rounded to bf16;
* layer_sel[l]  k distinct source layers by a partial Fisher-Yates shuffle,
  kept in draw order (not sorted);
* positions     per workload (see CONFIGS);
* paged         request lengths ~ U{256..16384}, per-request target offsets
  ~ U{0..2048}, 16-token pages, physical block ids a seeded permutation of a
  pool with 12.5% spare blocks (independent for source and target), unused
  table entries -1, every target slot pre-filled with a canary pattern.
Storage dtype is bf16 (fp32 for the tiny workload); rounding to storage is
torch's round-to-nearest-even.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

CANARY_BITS = 0x7FA5  # a bf16 NaN payload no transfer can produce


@dataclass(frozen=True)
class Workload:
    name: str
    n_src_layers: int
    n_tgt_layers: int
    n_kv_heads: int
    head_dim: int
    n_tokens: int
    k: int
    dtype: str            # "bf16" | "f32"
    theta: float
    positions: str        # "same" | "shift4096" | "gap1000"
    seed: int
    paged: bool = False
    n_requests: int = 0
    block_size: int = 16
    min_len: int = 256
    max_len: int = 16384
    max_offset: int = 2048


CONFIGS = {
    "tiny_fp32": Workload("tiny_fp32", 4, 4, 2, 64, 128, 2, "f32", 1e4, "same", 101),
    "qwen3_0.6b_1.7b_t512": Workload("qwen3_0.6b_1.7b_t512", 28, 28, 8, 128, 512, 4, "bf16", 1e6, "same", 201),
    "qwen3_0.6b_1.7b_t2048": Workload("qwen3_0.6b_1.7b_t2048", 28, 28, 8, 128, 2048, 4, "bf16", 1e6, "same", 202),
    "qwen3_14b_32b_t32k": Workload("qwen3_14b_32b_t32k", 40, 64, 8, 128, 32768, 4, "bf16", 1e6, "same", 301),
    "qwen3_14b_32b_t128k_shift": Workload("qwen3_14b_32b_t128k_shift", 40, 64, 8, 128, 131072, 4, "bf16", 1e6,
                                          "shift4096", 401),
    "qwen3_14b_32b_t128k_gap": Workload("qwen3_14b_32b_t128k_gap", 40, 64, 8, 128, 131072, 4, "bf16", 1e6,
                                        "gap1000", 402),
    # the wide-input map at the 14B -> 32B shape (IN = 4 x 2 x 8 x 128 = 8192)
    "qwen3_14b_32b_t32k_wide": Workload("qwen3_14b_32b_t32k_wide", 40, 64, 8, 128, 32768, 4, "bf16", 1e6,
                                        "same", 311),
    "paged_32req": Workload("paged_32req", 28, 28, 8, 128, 0, 4, "bf16", 1e6, "same", 501, paged=True,
                            n_requests=32),
}


def torch_dtype(w: Workload) -> torch.dtype:
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def _gen(device, seed: int, tensor_id: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + tensor_id)
    return g


def positions(w: Workload, T: int):
    """(src_pos, tgt_pos) int32 numpy arrays for the contiguous workloads."""
    t = np.arange(T, dtype=np.int64)
    if w.positions == "same":
        src, tgt = t, t
    elif w.positions == "shift4096":
        src, tgt = t, t + 4096
    elif w.positions == "gap1000":
        # the source prompt skips 1,000 positions at token 65,536; the target
        # places the whole prefix contiguously from 4,096
        src, tgt = t + 1000 * (t >= 65536), 4096 + t
    else:
        raise ValueError(w.positions)
    return src.astype(np.int32), tgt.astype(np.int32)


def layer_selection(w: Workload) -> np.ndarray:
    """[L_t, k] int32: k distinct source layers per target layer, draw order."""
    rng = np.random.Generator(np.random.Philox(w.seed * 1000 + 7))
    out = np.empty((w.n_tgt_layers, w.k), dtype=np.int32)
    for l in range(w.n_tgt_layers):
        idx = np.arange(w.n_src_layers)
        for j in range(w.k):
            r = j + int(rng.integers(0, w.n_src_layers - j))
            idx[j], idx[r] = idx[r], idx[j]
        out[l] = idx[:w.k]
    return out


def _scaled_normal(shape_per_layer, n_layers, scales, dtype, device, seed, tid):
    """[n_layers, *shape] = z * scales[l] (broadcast), drawn layer by layer."""
    g = _gen(device, seed, tid)
    out = torch.empty((n_layers, *shape_per_layer), dtype=dtype, device=device)
    for l in range(n_layers):
        z = torch.randn(shape_per_layer, generator=g, device=device, dtype=torch.float32)
        out[l] = (z * scales[l]).to(dtype)
    return out


def channel_scales(n_layers, H, D, device, seed, tid):
    g = _gen(device, seed, tid)
    z = torch.randn((n_layers, H, 1, D), generator=g, device=device, dtype=torch.float32)
    return torch.exp(0.5 * z)


def maps(w: Workload, device):
    """W_k, W_v [L_t, H, k*D, D] (storage dtype), b_k, b_v [L_t, H, D] fp32."""
    L, H, D, k = w.n_tgt_layers, w.n_kv_heads, w.head_dim, w.k
    dt = torch_dtype(w)
    std = 1.0 / math.sqrt(k * D)
    W = []
    for tid in (20, 21):
        g = _gen(device, w.seed, tid)
        Wt = torch.empty((L, H, k * D, D), dtype=dt, device=device)
        for l in range(L):
            Wt[l] = (torch.randn((H, k * D, D), generator=g, device=device) * std).to(dt)
        W.append(Wt)
    b = [torch.randn((L, H, D), generator=_gen(device, w.seed, tid), device=device) * 0.1
         for tid in (22, 23)]
    return W[0], b[0], W[1], b[1]


def wide_maps(w: Workload, device):
    """Wide-input maps: W_k, W_v [L_t, H, k*2*H*D, D] (storage dtype) with
    W ~ N(0, 1/IN), b_k, b_v [L_t, H, D] fp32 ~ N(0, 0.01)."""
    L, H, D, k = w.n_tgt_layers, w.n_kv_heads, w.head_dim, w.k
    IN = k * 2 * H * D
    dt = torch_dtype(w)
    std = 1.0 / math.sqrt(IN)
    W = []
    for tid in (30, 31):
        g = _gen(device, w.seed, tid)
        Wt = torch.empty((L, H, IN, D), dtype=dt, device=device)
        for l in range(L):
            for h in range(H):
                Wt[l, h] = (torch.randn((IN, D), generator=g, device=device) * std).to(dt)
        W.append(Wt)
    b = [torch.randn((L, H, D), generator=_gen(device, w.seed, tid), device=device) * 0.1
         for tid in (32, 33)]
    return W[0], b[0], W[1], b[1]


def contiguous_inputs(w: Workload, device="cpu", n_tokens: int | None = None):
    """Draws one contiguous case.  Returns a dict of tensors on ``device``:
    k_content, src_v [L_s, H, T, D]; W_k, W_v; b_k, b_v; layer_sel [L_t, k];
    src_pos, tgt_pos [T] (int32).  ``k_content`` still has to be
    position-encoded at src_pos to become the source key cache."""
    T = n_tokens if n_tokens is not None else w.n_tokens
    L, H, D = w.n_src_layers, w.n_kv_heads, w.head_dim
    dt = torch_dtype(w)
    sk = channel_scales(L, H, D, device, w.seed, 1)
    sv = channel_scales(L, H, D, device, w.seed, 2)
    k_content = _scaled_normal((H, T, D), L, sk, dt, device, w.seed, 10)
    src_v = _scaled_normal((H, T, D), L, sv, dt, device, w.seed, 11)
    W_k, b_k, W_v, b_v = maps(w, device)
    src_pos, tgt_pos = positions(w, T)
    return dict(
        k_content=k_content, src_v=src_v, W_k=W_k, b_k=b_k, W_v=W_v, b_v=b_v,
        layer_sel=torch.from_numpy(layer_selection(w)).to(device),
        src_pos=torch.from_numpy(src_pos).to(device),
        tgt_pos=torch.from_numpy(tgt_pos).to(device))


@dataclass
class PagedLayout:
    lens: np.ndarray          # [R] tokens per request
    cu_seqlens: np.ndarray    # [R+1] int32
    src_bt: np.ndarray        # [R, max_blocks] int32, -1 where unused
    tgt_bt: np.ndarray
    n_src_blocks: int
    n_tgt_blocks: int
    src_pos: np.ndarray       # [N] int32 over packed tokens
    tgt_pos: np.ndarray
    block_size: int = 16

    @property
    def n_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def max_blocks(self) -> int:
        return int(self.src_bt.shape[1])


def paged_layout(w: Workload, lens=None) -> PagedLayout:
    rng = np.random.Generator(np.random.Philox(w.seed * 1000 + 9))
    R, B = w.n_requests, w.block_size
    if lens is None:
        lens = rng.integers(w.min_len, w.max_len + 1, R)
    lens = np.asarray(lens, dtype=np.int64)
    R = len(lens)
    offs = rng.integers(0, w.max_offset + 1, R)
    pages = (lens + B - 1) // B
    total = int(pages.sum())
    maxb = max(int(pages.max()), 1)
    n_src = total + (total + 7) // 8
    n_tgt = total + (total + 7) // 8
    src_ids = rng.permutation(n_src)[:total]
    tgt_ids = rng.permutation(n_tgt)[:total]
    sbt = np.full((R, maxb), -1, np.int32)
    tbt = np.full((R, maxb), -1, np.int32)
    c = 0
    for r in range(R):
        sbt[r, :pages[r]] = src_ids[c:c + pages[r]]
        tbt[r, :pages[r]] = tgt_ids[c:c + pages[r]]
        c += int(pages[r])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    src_pos = np.concatenate([np.arange(n) for n in lens]).astype(np.int32)
    tgt_pos = np.concatenate([o + np.arange(n) for o, n in zip(offs, lens)]).astype(np.int32)
    return PagedLayout(lens, cu, sbt, tbt, n_src, n_tgt, src_pos, tgt_pos, B)


def paged_content(w: Workload, lay: PagedLayout, device="cpu"):
    """Packed token content [L_s, H, N, D] for keys (pre-encoding) and values,
    plus the maps.  Place rows into pools with :func:`scatter_to_pool`."""
    c = contiguous_inputs(replace(w, positions="same"), device=device, n_tokens=lay.n_tokens)
    c["src_pos"] = torch.from_numpy(lay.src_pos).to(device)
    c["tgt_pos"] = torch.from_numpy(lay.tgt_pos).to(device)
    return c


def slot_index(lay: PagedLayout, table: np.ndarray) -> np.ndarray:
    """Physical slot (block * block_size + offset) of every packed token."""
    out = np.empty(lay.n_tokens, dtype=np.int64)
    B = lay.block_size
    for r, n in enumerate(lay.lens):
        t = np.arange(n)
        out[lay.cu_seqlens[r]:lay.cu_seqlens[r + 1]] = table[r, t // B].astype(np.int64) * B + t % B
    return out


def scatter_to_pool(x: torch.Tensor, lay: PagedLayout, table: np.ndarray, n_blocks: int,
                    fill_bits: int | None = None) -> torch.Tensor:
    """Lays packed rows x [L, H, N, D] into a pool [L, n_blocks, B, H, D].
    Slots no token uses hold the canary ``fill_bits`` (see fill_canary) or zeros."""
    L, H, N, D = x.shape
    B = lay.block_size
    pool = torch.zeros((L, n_blocks * B, H, D), dtype=x.dtype, device=x.device)
    if fill_bits is not None:
        fill_canary(pool, fill_bits)
    idx = torch.from_numpy(slot_index(lay, table)).to(x.device)
    for l in range(L):
        pool[l, idx] = x[l].permute(1, 0, 2)
    return pool.view(L, n_blocks, B, H, D)


def empty_target_pool(w: Workload, lay: PagedLayout, device="cpu") -> torch.Tensor:
    """Target pool [L_t, n_tgt_blocks, B, H, D] with every slot holding the canary."""
    pool = torch.empty((w.n_tgt_layers, lay.n_tgt_blocks, lay.block_size, w.n_kv_heads, w.head_dim),
                       dtype=torch_dtype(w), device=device)
    fill_canary(pool)
    return pool


def canary_view(pool: torch.Tensor, bits: int = CANARY_BITS):
    """(integer view of pool, the canary as an element of that view): bf16
    elements are 16-bit patterns, fp32 elements hold the pattern in both
    halves (a NaN as well)."""
    if pool.dtype == torch.bfloat16:
        return pool.view(torch.int16), int(np.uint16(bits).view(np.int16))
    if pool.dtype == torch.float32:
        return pool.view(torch.int32), int(np.uint32(bits * 0x10001).view(np.int32))
    raise ValueError(f"no canary for {pool.dtype}")


def fill_canary(pool: torch.Tensor, bits: int = CANARY_BITS) -> None:
    view, value = canary_view(pool, bits)
    view.fill_(value)


def ridge_inputs(n_groups: int, n_obs: int, in_features: int, out_features: int, seed: int, device):
    """Observations X [G, N, IN] and targets Y [G, N, D] (bf16) for the ridge
    fit, drawn per group on ``device``: every feature has its own mean and
    scale (see the module docstring); Y is independent of X."""
    out = []
    for tid, F in ((40, in_features), (41, out_features)):
        g = _gen(device, seed, tid)
        m = torch.randn((n_groups, 1, F), generator=g, device=device)
        sc = torch.exp(0.5 * torch.randn((n_groups, 1, F), generator=g, device=device))
        t = torch.empty((n_groups, n_obs, F), dtype=torch.bfloat16, device=device)
        # about 4 GiB of fp32 per draw, transformed in place and rounded once
        # on the copy into t: four kernel launches per draw
        step = max(1, (4 << 30) // max(1, n_obs * F * 4))
        for i in range(0, n_groups, step):
            j = min(n_groups, i + step)
            z = torch.randn((j - i, n_obs, F), generator=g, device=device)
            z.add_(m[i:j]).mul_(sc[i:j])
            t[i:j].copy_(z)
            del z
        out.append(t)
    return out[0], out[1]

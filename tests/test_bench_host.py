"""Host-side logic of bench.py, on the CPU: the one-GPU refusal, the kernel
source digest that keys the committed counter summaries, the lookup of
recorded HBM bytes, and the algorithmic bytes and flops the roofline divides
by (checked against the transfer's sizes written out by hand)."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def _write(path, text):
    with open(path, "w") as f:
        f.write(text)


def test_digest_ignores_comments_and_follows_device_headers(tmp_path):
    hdr = tmp_path / "dev.hpp"
    src = tmp_path / "k.hip"
    _write(hdr, "__device__ int f() { return 1; }\n")
    _write(src, '#include "internal.hpp"\n#include "dev.hpp"\n__global__ void k() {}\n')
    d0 = bench.kernel_source_digest(str(src))
    # comment-only and blank-line edits keep the digest
    _write(src, '// a note\n#include "internal.hpp"\n\n#include "dev.hpp"   // header\n__global__ void k() {}\n')
    assert bench.kernel_source_digest(str(src)) == d0
    # a code edit in the included device header changes it
    _write(hdr, "__device__ int f() { return 2; }\n")
    assert bench.kernel_source_digest(str(src)) != d0


def test_recorded_traffic_only_for_the_source_it_was_taken_on(tmp_path):
    src = tmp_path / "k.hip"
    _write(src, "__global__ void k() {}\n")
    md = tmp_path / "c.md"
    _write(md, f"sha256: {bench.kernel_source_digest(str(src))}\nhbm_bytes_per_launch: 12345\n")
    assert bench.recorded_traffic(str(md), str(src))[0] == 12345.0
    _write(md, f"sha256: {bench.kernel_source_digest(str(src))}\nhbm_bytes_per_group: 10\n")
    assert bench.recorded_traffic(str(md), str(src), units=7)[0] == 70.0
    _write(src, "__global__ void k() { int x = 0; }\n")
    val, why = bench.recorded_traffic(str(md), str(src), units=7)
    assert val is None and "another kernel source" in why
    assert bench.recorded_traffic(str(tmp_path / "missing.md"), str(src))[0] is None


def test_committed_summaries_name_a_figure_and_a_digest():
    for md in (bench.COUNTERS_MD, bench.PAGED_MD, bench.WIDE_MD, bench.COSINE_MD, bench.RIDGE_MD):
        text = open(md).read()
        keys = [line.split(":", 1)[0] for line in text.splitlines()]
        assert "sha256" in keys, md
        assert "hbm_bytes_per_launch" in keys or "hbm_bytes_per_group" in keys, md


def test_algorithmic_work_of_the_headline_transfer():
    # 40 -> 64 layers, 8 heads, head_dim 128, k = 4, 32,768 tokens, bf16
    w = synth.CONFIGS["qwen3_14b_32b_t32k"]
    sel = synth.layer_selection(w)
    used = len(set(sel.ravel().tolist()))
    T = 32768
    src = 2 * used * 8 * T * 128 * 2          # K and V of every selected source layer, once
    tgt = 2 * 64 * 8 * T * 128 * 2           # K and V of every target layer
    wts = 2 * 64 * 8 * 512 * 128 * 2 + 2 * 64 * 8 * 128 * 4   # W_k, W_v (bf16) and b_k, b_v (fp32)
    pos = 2 * T * 4
    flops = 2 * 64 * 8 * 2 * T * 512 * 128   # K and V maps: 2 flop per multiply-add
    nbytes, nflops, parts = bench.algorithmic_work(w, sel, T)
    assert used == 40
    assert nbytes == src + tgt + wts + pos == 14_093_647_872
    assert nflops == flops == 4_398_046_511_104
    assert parts["used_src_layers"] == used


def test_algorithmic_bytes_count_each_selected_layer_once():
    w = synth.CONFIGS["qwen3_14b_32b_t32k"]
    sel = np.array([[0, 1, 2, 3]] * w.n_tgt_layers, dtype=np.int32)   # every target layer selects the same 4
    nbytes, _, parts = bench.algorithmic_work(w, sel, 16)
    assert parts["used_src_layers"] == 4
    assert parts["src"] == 2 * 4 * 8 * 16 * 128 * 2

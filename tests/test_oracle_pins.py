"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test names what pins it: a closed form, an invariant of rotations, a
special case that reduces to a textbook operation or a library routine, an
independent formulation (RoPE as complex multiplication, or as the matrix
exponential of its skew-symmetric generator), or a pure-Python brute force.
The plausible mistakes each catches are noted: a sign flip in the rotation,
interleaved instead of rotate-half pairing, a wrong frequency exponent, a
transposed W, a dropped bias or bias added after the rotation, a wrong
concatenation order, re-rotation at source positions, a skipped re-rotation.

Passages followed: "Helm Intelligent Routing", section "Why carrying the
cache across is the hard part" (un-rotate, map, re-rotate; step 3 never
skipped); the Qwen3 cache-mapping write-up, section "A linear bridge,
strangely enough, suffices" (select and concatenate source layers; separate
K and V fits per target head; x @ w + b; strip source RoPE -> map -> apply
target RoPE).
"""
import math

import numpy as np
import pytest
import scipy.linalg
import torch

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")

BF16, F32 = 0, 1


# ---------------------------------------------------------------- helpers
def freqs_np(D, theta):
    """Independent statement of the rotate-half frequencies theta^(-2i/D)."""
    return np.array([theta ** (-2.0 * i / D) for i in range(D // 2)])


def rope_complex(v, p, theta):
    """RoPE as complex multiplication: z_i = v_i + j v_{i+D/2}, z_i *= e^{j p w_i}."""
    v = np.asarray(v, dtype=np.float64)
    D = v.shape[-1]
    h = D // 2
    z = v[..., :h] + 1j * v[..., h:]
    z = z * np.exp(1j * p * freqs_np(D, theta))
    return np.concatenate([z.real, z.imag], axis=-1)


def generator_matrix(D, theta):
    """Skew-symmetric generator G with R(p) = expm(p G) (rotate-half planes)."""
    h = D // 2
    G = np.zeros((D, D))
    for i, w in enumerate(freqs_np(D, theta)):
        G[i + h, i] = w
        G[i, i + h] = -w
    return G


def to_bf16_bits(x64: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 storage bits through torch (fp64 values already bf16-exact)."""
    t = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def random_case(rng, L_s, L_t, H, D, T, k, dtype=F32):
    """Small random case in storage dtype (test-local; the oracle gets the bytes)."""
    sel = np.stack([rng.permutation(L_s)[:k] for _ in range(L_t)]).astype(np.int32)

    def store(x):
        if dtype == F32:
            return x.astype(np.float32)
        return to_bf16_bits(x)

    src_k = store(rng.standard_normal((L_s, H, T, D)))
    src_v = store(rng.standard_normal((L_s, H, T, D)))
    W_k = store(rng.standard_normal((L_t, H, k * D, D)) / math.sqrt(k * D))
    W_v = store(rng.standard_normal((L_t, H, k * D, D)) / math.sqrt(k * D))
    b_k = (0.1 * rng.standard_normal((L_t, H, D))).astype(np.float32)
    b_v = (0.1 * rng.standard_normal((L_t, H, D))).astype(np.float32)
    return dict(src_k=src_k, src_v=src_v, layer_sel=sel, W_k=W_k, b_k=b_k, W_v=W_v, b_v=b_v)


def as_f64(a, dtype):
    return a.astype(np.float64) if dtype == F32 else bf16_bits_to_f64(a)


def run(oracle_mod, L_s, L_t, H, D, T, k, case, src_pos, tgt_pos, theta_s=1e4, theta_t=1e4,
        dtype=F32, quantize=False):
    pb = oracle_mod.Problem(L_s, L_t, H, D, k, n_tokens=T, theta_src=theta_s, theta_tgt=theta_t,
                            dtype=dtype, quantize_content=quantize)
    return oracle_mod.transfer_rows(pb, case["src_k"], case["src_v"], src_pos, tgt_pos,
                                    case["layer_sel"], case["W_k"], case["b_k"], case["W_v"], case["b_v"])


# ---------------------------------------------------------------- rounding
def test_round_bf16_matches_torch_rne(oracle_mod):
    """Pin: bf16 rounding equals torch's binary32 -> bf16 conversion (RNE)
    on binary32 inputs, including exact ties and subnormals."""
    rng = np.random.default_rng(1)
    vals = [rng.standard_normal(4000).astype(np.float32),
            (rng.standard_normal(500) * 1e-38).astype(np.float32),
            (rng.standard_normal(500) * 1e30).astype(np.float32)]
    # exact ties: 1 + (2m+1) * 2^-8 lies halfway between two bf16 values
    ties = np.array([1 + (2 * m + 1) * 2.0 ** -8 for m in range(16)], dtype=np.float32)
    vals.append(np.concatenate([ties, -ties, ties * 2.0 ** -100]))
    x = np.concatenate(vals)
    ours = oracle_mod.round_bf16(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_round_bf16_ties_to_even_closed_form(oracle_mod):
    """Pin: 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1);
    1 + 3*2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6 -> even (1 + 2^-6)."""
    r = oracle_mod.round_bf16([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)])
    assert list(r) == [1.0, 1 + 2 ** -6, -1.0]


# ---------------------------------------------------------------- rotation
def test_freq_closed_form(oracle_mod):
    """Pin: w_0 = 1; for D = 4, w_1 = theta^(-1/2); w_i = theta^(-2i/D)."""
    assert oracle_mod.rope_freq(0, 128, 1e6) == 1.0
    assert oracle_mod.rope_freq(1, 4, 1e4) == pytest.approx(0.01, rel=1e-15)
    assert oracle_mod.rope_freq(32, 128, 1e6) == pytest.approx(1e-3, rel=1e-14)


def test_rotation_d2_is_plain_angle(oracle_mod):
    """P11 closed form: with D = 2 (w_0 = 1), R(p) turns by exactly p radians,
    counter-clockwise: e0 -> (cos p, sin p), e1 -> (-sin p, cos p)."""
    for p in [0, 1, -1, 3, 7, 100, 4096, 131071, -65536]:
        a = oracle_mod.rope([1.0, 0.0], p, 1e6)
        b = oracle_mod.rope([0.0, 1.0], p, 1e6)
        assert a == pytest.approx([math.cos(p), math.sin(p)], abs=1e-15)
        assert b == pytest.approx([-math.sin(p), math.cos(p)], abs=1e-15)


def test_rotation_d4_rotate_half_pairing(oracle_mod):
    """Closed form pinning rotate-half (not interleaved) pairing, D = 4,
    theta = 1e4: pair (0, 2) turns by p, pair (1, 3) by p / 100."""
    v = [1.0, 2.0, 3.0, 4.0]
    p = 1.0
    c0, s0 = math.cos(p), math.sin(p)
    c1, s1 = math.cos(p / 100), math.sin(p / 100)
    expect = [1 * c0 - 3 * s0, 2 * c1 - 4 * s1, 3 * c0 + 1 * s0, 4 * c1 + 2 * s1]
    assert oracle_mod.rope(v, p, 1e4) == pytest.approx(expect, abs=1e-15)


@pytest.mark.parametrize("D,theta", [(8, 1e4), (64, 1e4), (128, 1e6)])
def test_rotation_matches_complex_form(oracle_mod, D, theta):
    """Independent formulation: RoPE as complex multiplication."""
    rng = np.random.default_rng(D)
    for p in [0, 1, 17, 127, 4096, 32767, 136000, -500]:
        v = rng.standard_normal(D)
        np.testing.assert_allclose(oracle_mod.rope(v, p, theta), rope_complex(v, p, theta),
                                   rtol=0, atol=1e-12 * np.abs(v).max())


def test_rotation_matches_matrix_exponential(oracle_mod):
    """Independent formulation: R(p) = expm(p G), G the skew generator."""
    D, theta = 16, 1e4
    G = generator_matrix(D, theta)
    rng = np.random.default_rng(5)
    for p in [1, 2, 5, -3]:
        R = scipy.linalg.expm(p * G)
        v = rng.standard_normal(D)
        np.testing.assert_allclose(oracle_mod.rope(v, p, theta), R @ v, atol=1e-12)


def test_inverse_rotation_is_identity(oracle_mod):
    """P1: R(-p) R(p) = I (fp64, <= 1e-14 relative)."""
    rng = np.random.default_rng(2)
    for p in [1, 511, 32767, 131071]:
        v = rng.standard_normal(128)
        back = oracle_mod.rope(oracle_mod.rope(v, p, 1e6), -p, 1e6)
        assert np.linalg.norm(back - v) <= 1e-14 * np.linalg.norm(v) * 10


def test_rotation_preserves_pair_norms(oracle_mod):
    """P2: each (i, i + D/2) pair keeps its Euclidean norm."""
    rng = np.random.default_rng(3)
    v = rng.standard_normal(128)
    r = oracle_mod.rope(v, 12345, 1e6)
    np.testing.assert_allclose(np.hypot(r[:64], r[64:]), np.hypot(v[:64], v[64:]), rtol=1e-14)


def test_relative_position_property(oracle_mod):
    """P3: <R(p+d) q, R(p'+d) k> = <R(p) q, R(p') k>."""
    rng = np.random.default_rng(4)
    q, kk = rng.standard_normal(128), rng.standard_normal(128)
    base = oracle_mod.rope(q, 100, 1e6) @ oracle_mod.rope(kk, 37, 1e6)
    for d in [1, 4096, 65536]:
        shifted = oracle_mod.rope(q, 100 + d, 1e6) @ oracle_mod.rope(kk, 37 + d, 1e6)
        assert shifted == pytest.approx(base, rel=1e-12, abs=1e-12)


# ---------------------------------------------------------------- transfer
def test_identity_map_returns_input(oracle_mod):
    """P4: k = 1, W = I, b = 0, tgt_pos = src_pos, same theta -> out = src."""
    L, H, D, T = 3, 2, 16, 9
    rng = np.random.default_rng(6)
    case = random_case(rng, L, L, H, D, T, 1)
    case["layer_sel"] = np.arange(L, dtype=np.int32).reshape(L, 1)
    case["W_k"] = np.broadcast_to(np.eye(D, dtype=np.float32), (L, H, D, D)).copy()
    case["W_v"] = case["W_k"].copy()
    case["b_k"][:] = 0
    case["b_v"][:] = 0
    pos = rng.integers(0, 5000, T).astype(np.int32)
    ok, ov = run(oracle_mod, L, L, H, D, T, 1, case, pos, pos)
    np.testing.assert_allclose(ok, case["src_k"].astype(np.float64), rtol=0, atol=1e-13)
    np.testing.assert_allclose(ov, case["src_v"].astype(np.float64), rtol=0, atol=0)


def test_shift_is_textbook_rope_shift(oracle_mod):
    """P5: k = 1, W = I, b = 0, tgt = src + d -> out_k = R(d) src_k (complex
    form), out_v = src_v.  Also catches re-rotation at source positions."""
    L, H, D, T = 2, 2, 32, 7
    rng = np.random.default_rng(7)
    case = random_case(rng, L, L, H, D, T, 1)
    case["layer_sel"] = np.array([[1], [0]], dtype=np.int32)
    case["W_k"] = np.broadcast_to(np.eye(D, dtype=np.float32), (L, H, D, D)).copy()
    case["W_v"] = case["W_k"].copy()
    case["b_k"][:] = 0
    case["b_v"][:] = 0
    src = rng.integers(0, 1000, T).astype(np.int32)
    for d in [0, 1, 4096, -300]:
        ok, ov = run(oracle_mod, L, L, H, D, T, 1, case, src, src + d)
        for l in range(L):
            s = case["layer_sel"][l, 0]
            want = rope_complex(case["src_k"][s].astype(np.float64), d, 1e4)
            np.testing.assert_allclose(ok[l], want, atol=1e-12)
            np.testing.assert_array_equal(ov[l], case["src_v"][s].astype(np.float64))


@pytest.mark.parametrize("quantize,dtype", [(False, F32), (True, BF16)])
def test_transfer_relative_position_shift(oracle_mod, quantize, dtype):
    """P3 applied to the transfer itself, with a random map and bias: moving
    every target position by d rotates each key output by R(d) (complex
    form) and leaves the values unchanged, so q.k between the transferred
    keys and any query moved by the same d is unchanged.  Links the 32K-token
    workload at tgt_pos = src_pos with the long-context one at src_pos + 4096.
    Catches re-rotation at source positions, a bias added after the rotation,
    a map applied after the re-rotation."""
    L_s, L_t, H, D, T, k = 5, 3, 2, 16, 11, 3
    rng = np.random.default_rng(31)
    case = random_case(rng, L_s, L_t, H, D, T, k, dtype=dtype)
    src = rng.integers(-5000, 5000, T).astype(np.int32)
    tgt = rng.integers(0, 100000, T).astype(np.int32)
    k0, v0 = run(oracle_mod, L_s, L_t, H, D, T, k, case, src, tgt, 1e6, 1e6, dtype=dtype, quantize=quantize)
    for d in [1, 4096, -777]:
        k1, v1 = run(oracle_mod, L_s, L_t, H, D, T, k, case, src, tgt + d, 1e6, 1e6, dtype=dtype, quantize=quantize)
        np.testing.assert_allclose(k1, rope_complex(k0, d, 1e6), rtol=0, atol=1e-11)
        np.testing.assert_array_equal(v1, v0)
        q = rng.standard_normal(D)
        for t in range(T):
            a = rope_complex(q, int(tgt[t]) + 50, 1e6) @ k0[0, 0, t]
            b = rope_complex(q, int(tgt[t]) + 50 + d, 1e6) @ k1[0, 0, t]
            assert b == pytest.approx(a, rel=1e-9, abs=1e-9)


def test_selector_pins_concatenation_order(oracle_mod):
    """P6: W = selector of row block j -> output is layer layer_sel[l, j]
    (in the order of the layer_sel row as given), re-rotated by the offset."""
    L_s, L_t, H, D, T, k = 5, 3, 2, 8, 6, 3
    rng = np.random.default_rng(8)
    case = random_case(rng, L_s, L_t, H, D, T, k)
    case["layer_sel"] = np.array([[4, 0, 2], [1, 3, 0], [2, 4, 1]], dtype=np.int32)
    case["b_k"][:] = 0
    case["b_v"][:] = 0
    src = rng.integers(0, 300, T).astype(np.int32)
    tgt = src + 11
    for j in range(k):
        Wsel = np.zeros((k * D, D), dtype=np.float32)
        Wsel[j * D:(j + 1) * D] = np.eye(D, dtype=np.float32)
        case["W_k"] = np.broadcast_to(Wsel, (L_t, H, k * D, D)).copy()
        case["W_v"] = case["W_k"].copy()
        ok, ov = run(oracle_mod, L_s, L_t, H, D, T, k, case, src, tgt)
        for l in range(L_t):
            s = case["layer_sel"][l, j]
            want_k = rope_complex(case["src_k"][s].astype(np.float64), 11, 1e4)
            np.testing.assert_allclose(ok[l], want_k, atol=1e-12)
            np.testing.assert_array_equal(ov[l], case["src_v"][s].astype(np.float64))


def test_zero_map_gives_rotated_bias(oracle_mod):
    """P7: W = 0 -> out_k = R(tgt_pos) b_k, out_v = b_v: the bias is added in
    content space, before the forward rotation."""
    L_s, L_t, H, D, T, k = 2, 2, 2, 16, 5, 2
    rng = np.random.default_rng(9)
    case = random_case(rng, L_s, L_t, H, D, T, k)
    case["W_k"][:] = 0
    case["W_v"][:] = 0
    src = rng.integers(0, 100, T).astype(np.int32)
    tgt = rng.integers(0, 100000, T).astype(np.int32)
    ok, ov = run(oracle_mod, L_s, L_t, H, D, T, k, case, src, tgt)
    for l in range(L_t):
        for h in range(H):
            for t in range(T):
                want = rope_complex(case["b_k"][l, h].astype(np.float64), tgt[t], 1e4)
                np.testing.assert_allclose(ok[l, h, t], want, atol=1e-12)
                np.testing.assert_array_equal(ov[l, h, t], case["b_v"][l, h].astype(np.float64))


def test_zero_positions_reduce_to_batched_matmul(oracle_mod):
    """P8: all positions 0 -> a batched GEMM plus bias (numpy einsum, fp64).
    Catches a transposed W or a dropped bias."""
    L_s, L_t, H, D, T, k = 4, 3, 2, 16, 10, 3
    rng = np.random.default_rng(10)
    case = random_case(rng, L_s, L_t, H, D, T, k)
    z = np.zeros(T, dtype=np.int32)
    ok, ov = run(oracle_mod, L_s, L_t, H, D, T, k, case, z, z)
    for name, out, src, W, b in (("k", ok, case["src_k"], case["W_k"], case["b_k"]),
                                 ("v", ov, case["src_v"], case["W_v"], case["b_v"])):
        X = src.astype(np.float64)[case["layer_sel"]]          # [L_t, k, H, T, D]
        X = np.transpose(X, (0, 2, 3, 1, 4)).reshape(L_t, H, T, k * D)
        want = np.einsum("lhtm,lhmn->lhtn", X, W.astype(np.float64)) + b[:, :, None, :]
        np.testing.assert_allclose(out, want, rtol=1e-13, atol=1e-13, err_msg=name)


def test_skipping_rerotation_is_detectably_wrong(oracle_mod):
    """P9: an output that skips step 3 has per-head cosine far below 0.99
    against the true output (so the GPU test's 0.9999 gate rejects it)."""
    L_s, L_t, H, D, T, k = 4, 2, 2, 64, 256, 2
    rng = np.random.default_rng(11)
    case = random_case(rng, L_s, L_t, H, D, T, k)
    pos = np.arange(T, dtype=np.int32)
    ok, _ = run(oracle_mod, L_s, L_t, H, D, T, k, case, pos, pos)
    no_rerot = np.stack([[[rope_complex(ok[l, h, t], -pos[t], 1e4) for t in range(T)]
                          for h in range(H)] for l in range(L_t)])
    for l in range(L_t):
        for h in range(H):
            a, b = ok[l, h].ravel(), no_rerot[l, h].ravel()
            cos = a @ b / np.linalg.norm(a) / np.linalg.norm(b)
            assert cos < 0.9


def test_brute_force_triple_loop(oracle_mod):
    """P10: a pure-Python loop (dense rotation matrices built from the complex
    form, explicit sums) agrees with the oracle to 1e-12 on tiny shapes."""
    L_s, L_t, H, D, T, k = 3, 2, 2, 8, 4, 2
    rng = np.random.default_rng(12)
    case = random_case(rng, L_s, L_t, H, D, T, k)
    src = rng.integers(0, 50, T).astype(np.int32)
    tgt = rng.integers(0, 50, T).astype(np.int32)
    ok, ov = run(oracle_mod, L_s, L_t, H, D, T, k, case, src, tgt, theta_s=1e4, theta_t=500.0)

    def rot_matrix(p, theta):
        cols = [rope_complex(np.eye(D)[c], p, theta) for c in range(D)]
        return [[float(cols[c][r]) for c in range(D)] for r in range(D)]

    for l in range(L_t):
        for h in range(H):
            for t in range(T):
                Rin = rot_matrix(-int(src[t]), 1e4)
                Rout = rot_matrix(int(tgt[t]), 500.0)
                xk, xv = [], []
                for j in range(k):
                    s = int(case["layer_sel"][l, j])
                    u = [float(case["src_k"][s, h, t, d]) for d in range(D)]
                    xk += [sum(Rin[r][c] * u[c] for c in range(D)) for r in range(D)]
                    xv += [float(case["src_v"][s, h, t, d]) for d in range(D)]
                yk = [float(case["b_k"][l, h, n]) + sum(xk[m] * float(case["W_k"][l, h, m, n])
                                                       for m in range(k * D)) for n in range(D)]
                yv = [float(case["b_v"][l, h, n]) + sum(xv[m] * float(case["W_v"][l, h, m, n])
                                                       for m in range(k * D)) for n in range(D)]
                outk = [sum(Rout[r][c] * yk[c] for c in range(D)) for r in range(D)]
                np.testing.assert_allclose(ok[l, h, t], outk, rtol=0, atol=1e-12)
                np.testing.assert_allclose(ov[l, h, t], yv, rtol=0, atol=1e-12)


def test_linearity_in_map_and_input(oracle_mod):
    """P12: fixed positions -> the output is linear in (W, b) and in x."""
    L_s, L_t, H, D, T, k = 3, 2, 1, 8, 5, 2
    rng = np.random.default_rng(13)
    A = random_case(rng, L_s, L_t, H, D, T, k)
    B = random_case(rng, L_s, L_t, H, D, T, k)
    B["layer_sel"] = A["layer_sel"]
    for case in (A, B):   # coarse dyadic values: the mixes below stay exact in fp32
        for key in ("src_k", "src_v", "W_k", "W_v", "b_k", "b_v"):
            case[key] = (np.round(case[key] * 256) / 256).astype(np.float32)
    src = rng.integers(0, 99, T).astype(np.int32)
    tgt = rng.integers(0, 99, T).astype(np.int32)
    a, c = 0.75, -1.5   # exact binary fractions keep fp32 storage exact
    mix_map = dict(A, W_k=(a * A["W_k"] + c * B["W_k"]).astype(np.float32),
                   b_k=(a * A["b_k"] + c * B["b_k"]).astype(np.float32))
    ka, _ = run(oracle_mod, L_s, L_t, H, D, T, k, A, src, tgt)
    kb, _ = run(oracle_mod, L_s, L_t, H, D, T, k, dict(A, W_k=B["W_k"], b_k=B["b_k"]), src, tgt)
    km, _ = run(oracle_mod, L_s, L_t, H, D, T, k, mix_map, src, tgt)
    np.testing.assert_allclose(km, a * ka + c * kb, atol=1e-12)
    zero_b = dict(A, b_k=np.zeros_like(A["b_k"]), b_v=np.zeros_like(A["b_v"]))
    x1, v1 = run(oracle_mod, L_s, L_t, H, D, T, k, zero_b, src, tgt)
    x2, v2 = run(oracle_mod, L_s, L_t, H, D, T, k, dict(zero_b, src_k=B["src_k"], src_v=B["src_v"]), src, tgt)
    xm, vm = run(oracle_mod, L_s, L_t, H, D, T, k,
                 dict(zero_b, src_k=(a * A["src_k"] + c * B["src_k"]).astype(np.float32),
                      src_v=(a * A["src_v"] + c * B["src_v"]).astype(np.float32)), src, tgt)
    np.testing.assert_allclose(xm, a * x1 + c * x2, atol=1e-12)
    np.testing.assert_allclose(vm, a * v1 + c * v2, atol=1e-12)


def test_quantize_content_mode(oracle_mod):
    """The bf16 mode rounds the un-rotated key once to bf16 before the map.
    Pinned by a brute force that rounds with torch (RNE) and maps with numpy;
    at src_pos = 0 the un-rotation is exact so both modes agree exactly."""
    L_s, L_t, H, D, T, k = 3, 2, 2, 16, 6, 2
    rng = np.random.default_rng(14)
    case = random_case(rng, L_s, L_t, H, D, T, k, dtype=BF16)
    src = rng.integers(1, 3000, T).astype(np.int32)
    tgt = src + 5
    qk, qv = run(oracle_mod, L_s, L_t, H, D, T, k, case, src, tgt, 1e6, 1e6, BF16, True)
    ek, ev = run(oracle_mod, L_s, L_t, H, D, T, k, case, src, tgt, 1e6, 1e6, BF16, False)
    np.testing.assert_array_equal(qv, ev)                   # values are never rounded again
    assert np.abs(qk - ek).max() > 0                        # rounding is really applied
    sk = bf16_bits_to_f64(case["src_k"])
    W = bf16_bits_to_f64(case["W_k"])
    for l in range(L_t):
        for h in range(H):
            for t in range(T):
                x = np.concatenate([rope_complex(sk[s, h, t], -src[t], 1e6) for s in case["layer_sel"][l]])
                xq = torch.tensor(x).to(torch.bfloat16).to(torch.float64).numpy()
                # torch rounds fp64 -> bf16 through binary32 (two roundings); accept
                # a one-ulp difference only where that double rounding can differ.
                xo = oracle_mod.round_bf16(x)
                assert np.all(np.abs(xq - xo) <= np.abs(xo) * 2.0 ** -7)
                want = rope_complex(xo @ W[l, h] + case["b_k"][l, h], tgt[t], 1e6)
                np.testing.assert_allclose(qk[l, h, t], want, atol=1e-12)
    z = np.zeros(T, dtype=np.int32)
    qk0, _ = run(oracle_mod, L_s, L_t, H, D, T, k, case, z, tgt, 1e6, 1e6, BF16, True)
    ek0, _ = run(oracle_mod, L_s, L_t, H, D, T, k, case, z, tgt, 1e6, 1e6, BF16, False)
    np.testing.assert_array_equal(qk0, ek0)


def test_row_subset_matches_full(oracle_mod):
    """Sampled rows equal the same rows of the full computation."""
    L_s, L_t, H, D, T, k = 3, 3, 2, 16, 11, 2
    rng = np.random.default_rng(15)
    case = random_case(rng, L_s, L_t, H, D, T, k, dtype=BF16)
    src = np.arange(T, dtype=np.int32)
    tgt = src + 4096
    fk, fv = run(oracle_mod, L_s, L_t, H, D, T, k, case, src, tgt, 1e6, 1e6, BF16, True)
    rows = rng.choice(L_t * H * T, 20, replace=False)
    pb = oracle_mod.Problem(L_s, L_t, H, D, k, n_tokens=T, dtype=BF16)
    sk, sv = oracle_mod.transfer_rows(pb, case["src_k"], case["src_v"], src, tgt, case["layer_sel"],
                                      case["W_k"], case["b_k"], case["W_v"], case["b_v"], rows=rows)
    np.testing.assert_array_equal(sk, fk.reshape(-1, D)[rows])
    np.testing.assert_array_equal(sv, fv.reshape(-1, D)[rows])


def test_bad_layer_sel_rejected(oracle_mod):
    L_s, L_t, H, D, T, k = 3, 2, 1, 8, 4, 2
    case = random_case(np.random.default_rng(16), L_s, L_t, H, D, T, k)
    case["layer_sel"][1, 1] = 3
    with pytest.raises(ValueError):
        run(oracle_mod, L_s, L_t, H, D, T, k, case, np.zeros(T, np.int32), np.zeros(T, np.int32))


# ---------------------------------------------------------------- paged
def test_paged_equals_contiguous_through_block_tables(oracle_mod):
    """The paged oracle equals the contiguous oracle run per request, with
    rows fetched and placed through the block tables (knlp routing page,
    request-flow figure: block tables map a request's pages to blocks)."""
    L_s, L_t, H, D, k, Bs = 3, 2, 2, 16, 2, 4
    rng = np.random.default_rng(17)
    lens = [5, 8, 1, 11]
    R = len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N = int(cu[-1])
    pages = [(n + Bs - 1) // Bs for n in lens]
    maxb = max(pages)
    n_src_blocks, n_tgt_blocks = sum(pages) + 3, sum(pages) + 2
    src_ids = rng.permutation(n_src_blocks)[:sum(pages)]
    tgt_ids = rng.permutation(n_tgt_blocks)[:sum(pages)]
    sbt = np.full((R, maxb), -1, np.int32)
    tbt = np.full((R, maxb), -1, np.int32)
    c = 0
    for r in range(R):
        for p in range(pages[r]):
            sbt[r, p], tbt[r, p] = src_ids[c], tgt_ids[c]
            c += 1
    case = random_case(rng, L_s, L_t, H, D, N, k, dtype=BF16)
    src_pos = np.concatenate([np.arange(n) for n in lens]).astype(np.int32)
    tgt_pos = np.concatenate([np.arange(n) + rng.integers(0, 50) for n in lens]).astype(np.int32)
    # Build pools [L, n_blocks, Bs, H, D] from the contiguous [L, H, N, D] cache.
    def to_pool(x, nb, bt):
        pool = np.zeros((x.shape[0], nb, Bs, H, D), np.uint16)
        for r in range(R):
            for t in range(lens[r]):
                pool[:, bt[r, t // Bs], t % Bs] = x[:, :, cu[r] + t]
        return pool
    sk_pool, sv_pool = to_pool(case["src_k"], n_src_blocks, sbt), to_pool(case["src_v"], n_src_blocks, sbt)
    pb = oracle_mod.Problem(L_s, L_t, H, D, k, n_tokens=N, dtype=BF16)
    pg = oracle_mod.Paged(Bs, R, maxb, maxb, n_src_blocks, n_tgt_blocks)
    pk, pv, dst = oracle_mod.transfer_paged_rows(pb, pg, sk_pool, sv_pool, sbt, tbt, cu, src_pos, tgt_pos,
                                                 case["layer_sel"], case["W_k"], case["b_k"],
                                                 case["W_v"], case["b_v"])
    ck, cv = oracle_mod.transfer_rows(pb, case["src_k"], case["src_v"], src_pos, tgt_pos, case["layer_sel"],
                                      case["W_k"], case["b_k"], case["W_v"], case["b_v"])
    np.testing.assert_array_equal(pk, ck.reshape(-1, D))
    np.testing.assert_array_equal(pv, cv.reshape(-1, D))
    # destinations: element offsets into the target pool [L_t, n_tgt_blocks, Bs, H, D]
    index = np.arange(L_t * n_tgt_blocks * Bs * H * D).reshape(L_t, n_tgt_blocks, Bs, H, D)
    want = []
    for l in range(L_t):
        for h in range(H):
            for r in range(R):
                for t in range(lens[r]):
                    want.append(index[l, tbt[r, t // Bs], t % Bs, h, 0])
    np.testing.assert_array_equal(dst, np.array(want))


def test_encode_keys_is_rounded_rotation(oracle_mod):
    """encode_keys = RNE_bf16(R(pos) x) per row (complex form + torch RNE,
    accepting a one-ulp difference only from torch's double rounding)."""
    rng = np.random.default_rng(18)
    x = to_bf16_bits(rng.standard_normal((2, 2, 5, 16)))
    pos = rng.integers(0, 100000, 5).astype(np.int32)
    enc = bf16_bits_to_f64(oracle_mod.encode_keys(x, pos, 1e6, BF16))
    xf = bf16_bits_to_f64(x)
    for l in range(2):
        for h in range(2):
            for t in range(5):
                exact = rope_complex(xf[l, h, t], pos[t], 1e6)
                assert np.all(np.abs(enc[l, h, t] - exact) <= np.abs(exact) * 2.0 ** -8 * (1 + 1e-9))


# ---------------------------------------------------------------- KV-cosine diagnostic
# "Helm Intelligent Routing", the retention / KL / KV-cosine table: the KV
# cosine says how close a mapped cache is to the target's own.  Reading: per
# (layer, head) slab, the cosine of the two [T, D] slabs as flat vectors.
def _bf16_bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_kv_cosine_closed_forms(oracle_mod):
    """Hand-computed values: (3,4).(4,3) = 24 over 5*5; a slab against
    itself, its negation and a positive multiple; disjoint supports give 0.
    Catches a missing square root, a norm of only one side, a dropped sign."""
    a = np.array([[[[3.0, 4.0]]]], np.float32)
    b = np.array([[[[4.0, 3.0]]]], np.float32)
    assert oracle_mod.kv_cosine(a, b, F32)[0, 0] == pytest.approx(24.0 / 25.0, abs=1e-15)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 3, 17, 8)).astype(np.float32)
    np.testing.assert_allclose(oracle_mod.kv_cosine(x, x, F32), 1.0, atol=1e-14)
    np.testing.assert_allclose(oracle_mod.kv_cosine(x, -x, F32), -1.0, atol=1e-14)
    np.testing.assert_allclose(oracle_mod.kv_cosine(x, 4.0 * x, F32), 1.0, atol=1e-14)
    even, odd = x.copy(), x.copy()
    even[..., 1::2] = 0
    odd[..., 0::2] = 0
    assert np.all(oracle_mod.kv_cosine(even, odd, F32) == 0.0)


def test_kv_cosine_brute_force_and_slab_independence(oracle_mod):
    """Pure-Python fsum brute force on a tiny case (each slab its own flat
    vectors), and changing one slab changes that entry only.  Catches slabs
    mixed up (a wrong stride or a reduction over the wrong axes)."""
    rng = np.random.default_rng(2)
    a = rng.standard_normal((3, 2, 5, 4)).astype(np.float32)
    b = (a + 0.3 * rng.standard_normal(a.shape)).astype(np.float32)
    got = oracle_mod.kv_cosine(a, b, F32)
    assert got.shape == (3, 2)
    for l in range(3):
        for h in range(2):
            x = [float(v) for v in a[l, h].ravel()]
            y = [float(v) for v in b[l, h].ravel()]
            dot = math.fsum(p * q for p, q in zip(x, y))
            want = dot / (math.sqrt(math.fsum(p * p for p in x)) * math.sqrt(math.fsum(q * q for q in y)))
            assert got[l, h] == pytest.approx(want, abs=1e-14)
    b2 = b.copy()
    b2[1, 0] = rng.standard_normal((5, 4))
    got2 = oracle_mod.kv_cosine(a, b2, F32)
    changed = np.abs(got2 - got) > 0
    assert changed[1, 0] and changed.sum() == 1


def test_kv_cosine_bf16_storage_and_zero_slab(oracle_mod):
    """bf16 storage decodes to the same values as their fp32 spelling (so
    the two dtypes agree exactly on bf16-representable data), and a slab of
    zeros gives NaN (0/0), not a number that looks like a verdict."""
    rng = np.random.default_rng(3)
    x = oracle_mod.round_bf16(rng.standard_normal((2, 2, 6, 4))).astype(np.float32)
    y = oracle_mod.round_bf16(rng.standard_normal((2, 2, 6, 4))).astype(np.float32)
    np.testing.assert_array_equal(oracle_mod.kv_cosine(_bf16_bits(x), _bf16_bits(y), BF16),
                                  oracle_mod.kv_cosine(x, y, F32))
    z = np.zeros_like(x)
    assert np.all(np.isnan(oracle_mod.kv_cosine(z, y, F32)))


# ---------------------------------------------------------------- wide-input map
# The Qwen3 write-up's full mapper: x concatenates the K and V features of all
# heads of the selected source layers; one fit per target head for keys and
# one for values.  Reading of the feature order: (layer j in layer_sel row
# order, keys then values, source head g, dimension d).
def run_wide(oracle_mod, L_s, L_t, H, D, T, k, case, src_pos, tgt_pos, theta_s=1e4, theta_t=1e4,
             dtype=F32, quantize=False):
    pb = oracle_mod.Problem(L_s, L_t, H, D, k, n_tokens=T, theta_src=theta_s, theta_tgt=theta_t,
                            dtype=dtype, quantize_content=quantize)
    return oracle_mod.transfer_wide_rows(pb, case["src_k"], case["src_v"], src_pos, tgt_pos,
                                         case["layer_sel"], case["W_k"], case["b_k"], case["W_v"], case["b_v"])


@pytest.mark.parametrize("dtype,quantize", [(F32, False), (BF16, True)])
def test_wide_map_reduces_to_per_head_map(oracle_mod, dtype, quantize):
    """A wide W that is zero outside the target head's own keys (for W_k) and
    own values (for W_v) gives exactly the per-head transfer: pins the key and
    value blocks of the feature order, the per-head un-rotation (and its
    rounding in quantize_content mode) and the re-rotation against the
    (already pinned) per-head oracle."""
    L_s, L_t, H, D, T, k = 5, 3, 3, 8, 7, 2
    rng = np.random.default_rng(41)
    case = random_case(rng, L_s, L_t, H, D, T, k, dtype=dtype)
    IN = oracle_mod.wide_in(k, H, D)
    Wk = np.zeros((L_t, H, IN, D), case["W_k"].dtype)
    Wv = np.zeros((L_t, H, IN, D), case["W_v"].dtype)
    for l in range(L_t):
        for h in range(H):
            for j in range(k):
                Wk[l, h, ((j * 2 + 0) * H + h) * D:((j * 2 + 0) * H + h + 1) * D] = case["W_k"][l, h, j * D:(j + 1) * D]
                Wv[l, h, ((j * 2 + 1) * H + h) * D:((j * 2 + 1) * H + h + 1) * D] = case["W_v"][l, h, j * D:(j + 1) * D]
    wide = dict(case, W_k=Wk, W_v=Wv)
    src = rng.integers(-500, 5000, T).astype(np.int32)
    tgt = rng.integers(0, 90000, T).astype(np.int32)
    nk, nv = run(oracle_mod, L_s, L_t, H, D, T, k, case, src, tgt, theta_s=1e4, theta_t=5e5, dtype=dtype,
                 quantize=quantize)
    wk, wv = run_wide(oracle_mod, L_s, L_t, H, D, T, k, wide, src, tgt, theta_s=1e4, theta_t=5e5, dtype=dtype,
                      quantize=quantize)
    np.testing.assert_allclose(wk, nk, atol=1e-12)
    np.testing.assert_allclose(wv, nv, atol=1e-12)


def test_wide_map_one_hot_features(oracle_mod):
    """One-hot W columns pick single features: for target (l, h), output
    column n of the value map equals feature m of x, which must be the key of
    source head g of layer layer_sel[l, j] un-rotated at src_pos (kv = 0) or
    that head's value as stored (kv = 1); the key map's output is the same
    feature re-rotated at tgt_pos.  Catches a transposed (g, kv) order, a
    rotated value, a missing un-rotation, features taken from the target head
    instead of the source head."""
    L_s, L_t, H, D, T, k = 4, 2, 2, 4, 5, 2
    rng = np.random.default_rng(42)
    case = random_case(rng, L_s, L_t, H, D, T, k)
    case["layer_sel"] = np.array([[3, 1], [0, 2]], np.int32)
    case["b_k"][:] = 0
    case["b_v"][:] = 0
    IN = oracle_mod.wide_in(k, H, D)
    src = rng.integers(0, 300, T).astype(np.int32)
    tgt = rng.integers(0, 300, T).astype(np.int32)
    for (j, kv, g, d, n) in [(0, 0, 1, 2, 1), (1, 1, 0, 3, 0), (1, 0, 0, 0, 3), (0, 1, 1, 1, 2)]:
        m = ((j * 2 + kv) * H + g) * D + d
        W = np.zeros((L_t, H, IN, D), np.float32)
        W[:, :, m, n] = 1.0
        ok, ov = run_wide(oracle_mod, L_s, L_t, H, D, T, k, dict(case, W_k=W, W_v=W), src, tgt)
        for l in range(L_t):
            s = case["layer_sel"][l, j]
            for t in range(T):
                if kv == 0:
                    feat = rope_complex(case["src_k"][s, g, t].astype(np.float64), -src[t], 1e4)[d]
                else:
                    feat = float(case["src_v"][s, g, t, d])
                y = np.zeros(D)
                y[n] = feat
                for h in range(H):
                    np.testing.assert_allclose(ov[l, h, t], y, atol=1e-12)
                    np.testing.assert_allclose(ok[l, h, t], rope_complex(y, tgt[t], 1e4), atol=1e-12)


def test_wide_map_brute_force(oracle_mod):
    """Pure-Python loops (math.fsum dot products, complex-number RoPE) on a
    tiny wide case with random W and bias."""
    L_s, L_t, H, D, T, k = 3, 2, 2, 4, 3, 2
    rng = np.random.default_rng(43)
    case = random_case(rng, L_s, L_t, H, D, T, k)
    IN = oracle_mod.wide_in(k, H, D)
    case["W_k"] = (rng.standard_normal((L_t, H, IN, D)) / math.sqrt(IN)).astype(np.float32)
    case["W_v"] = (rng.standard_normal((L_t, H, IN, D)) / math.sqrt(IN)).astype(np.float32)
    src = rng.integers(0, 1000, T).astype(np.int32)
    tgt = rng.integers(0, 1000, T).astype(np.int32)
    ok, ov = run_wide(oracle_mod, L_s, L_t, H, D, T, k, case, src, tgt)
    for l in range(L_t):
        for t in range(T):
            x = []
            for j in range(k):
                s = int(case["layer_sel"][l, j])
                for kv in range(2):
                    for g in range(H):
                        if kv == 0:
                            x += list(rope_complex(case["src_k"][s, g, t].astype(np.float64), -int(src[t]), 1e4))
                        else:
                            x += [float(v) for v in case["src_v"][s, g, t]]
            for h in range(H):
                yk = [math.fsum(x[m] * float(case["W_k"][l, h, m, n]) for m in range(IN)) + float(case["b_k"][l, h, n])
                      for n in range(D)]
                yv = [math.fsum(x[m] * float(case["W_v"][l, h, m, n]) for m in range(IN)) + float(case["b_v"][l, h, n])
                      for n in range(D)]
                np.testing.assert_allclose(ov[l, h, t], yv, atol=1e-12)
                np.testing.assert_allclose(ok[l, h, t], rope_complex(np.array(yk), int(tgt[t]), 1e4), atol=1e-12)


# ------------------------------------------------------------- ridge fit
# The Qwen3 write-up, section "A linear bridge, strangely enough, suffices":
# every target head's K and V maps are fitted separately by ridge regression
# on centred data with lambda = 0.01; the bias comes from the means.

def _planted(rng, G, N, IN, D, x_shift=3.0):
    X = rng.standard_normal((G, N, IN)) + x_shift * rng.standard_normal((G, 1, IN))
    Wt = rng.standard_normal((G, IN, D))
    bt = rng.standard_normal((G, D))
    Y = X @ Wt + bt[:, None, :]
    return X, Y, Wt, bt


def test_ridge_recovers_planted_map_and_bias(oracle_mod):
    """Noiseless data y = x W* + b* (x with non-zero means, IN != D): a
    vanishing lambda recovers W* and b*.  Catches a dropped centring, a
    wrong bias sign or formula, and a transposed W."""
    rng = np.random.default_rng(11)
    X, Y, Wt, bt = _planted(rng, 3, 400, 7, 5)
    W, b = oracle_mod.ridge_fit(X, Y, lam=1e-12, dtype=F32)
    assert W.shape == (3, 7, 5) and b.shape == (3, 5)
    np.testing.assert_allclose(W, Wt, rtol=0, atol=1e-9)
    np.testing.assert_allclose(b, bt, rtol=0, atol=1e-9)


@pytest.mark.parametrize("lam", [0.01, 3.0])
def test_ridge_equals_the_centred_closed_form(oracle_mod, lam):
    """The write-up's own route to the fit (centre x and y, add lambda on the
    diagonal of xc^T xc, solve for W, b = mean(y) - mean(x) W), written out
    here with numpy's solve, gives the oracle's minimiser of the augmented
    least-squares problem."""
    rng = np.random.default_rng(21)
    X = rng.standard_normal((2, 250, 9)) * np.linspace(0.3, 3, 9) + 4.0
    Y = rng.standard_normal((2, 250, 5)) + X[:, :, :5] * 0.2
    W, b = oracle_mod.ridge_fit(X, Y, lam=lam, dtype=F32)
    for g in range(2):
        mx, my = X[g].mean(axis=0), Y[g].mean(axis=0)
        xc, yc = X[g] - mx, Y[g] - my
        Wc = np.linalg.solve(xc.T @ xc + lam * np.eye(9), xc.T @ yc)
        np.testing.assert_allclose(W[g], Wc, rtol=0, atol=1e-11)
        np.testing.assert_allclose(b[g], my - mx @ Wc, rtol=0, atol=1e-10)


def test_ridge_rank_deficient_with_penalty(oracle_mod):
    """N <= IN (fewer observations than inputs, as in the short GPU cases):
    lambda > 0 makes the minimiser unique; it matches the closed form
    W = xc^T (xc xc^T + lambda I)^-1 yc (the push-through identity, an N x N
    solve) and b = mean(y) - mean(x) W."""
    rng = np.random.default_rng(22)
    X = rng.standard_normal((1, 6, 10)) + 1.0
    Y = rng.standard_normal((1, 6, 3))
    lam = 0.01
    W, b = oracle_mod.ridge_fit(X, Y, lam=lam, dtype=F32)
    mx, my = X[0].mean(axis=0), Y[0].mean(axis=0)
    xc, yc = X[0] - mx, Y[0] - my
    Wp = xc.T @ np.linalg.solve(xc @ xc.T + lam * np.eye(6), yc)
    np.testing.assert_allclose(W[0], Wp, rtol=0, atol=1e-9)
    np.testing.assert_allclose(b[0], my - mx @ Wp, rtol=0, atol=1e-9)


def test_ridge_zero_lambda_is_least_squares_with_intercept(oracle_mod):
    """lambda = 0 is ordinary least squares with an intercept column:
    numpy's lstsq (an SVD route) on [x, 1] gives the same map and bias."""
    rng = np.random.default_rng(12)
    X = rng.standard_normal((2, 300, 6)) + 2.0
    Y = rng.standard_normal((2, 300, 4))
    W, b = oracle_mod.ridge_fit(X, Y, lam=0.0, dtype=F32)
    for g in range(2):
        A = np.hstack([X[g], np.ones((300, 1))])
        sol = np.linalg.lstsq(A, Y[g], rcond=None)[0]
        np.testing.assert_allclose(W[g], sol[:6], rtol=0, atol=1e-11)
        np.testing.assert_allclose(b[g], sol[6], rtol=0, atol=1e-11)


def test_ridge_large_lambda_asymptote(oracle_mod):
    """lambda -> infinity: lambda * W -> xc^T yc (the penalty dominates the
    normal matrix), the closed-form limit; pins lambda on the diagonal,
    unscaled."""
    rng = np.random.default_rng(13)
    X = rng.standard_normal((1, 200, 5)) + 1.0
    Y = rng.standard_normal((1, 200, 3))
    lam = 1e10
    W, _ = oracle_mod.ridge_fit(X, Y, lam=lam, dtype=F32)
    xc = X[0] - X[0].mean(axis=0)
    yc = Y[0] - Y[0].mean(axis=0)
    np.testing.assert_allclose(lam * W[0], xc.T @ yc, rtol=1e-6, atol=0)


def test_ridge_scalar_closed_form_brute_force(oracle_mod):
    """IN = D = 1 in pure Python: w = Sxy / (Sxx + lambda), b = ybar - xbar w,
    with lambda = 0.01 on a small sample (where lambda is not negligible)."""
    xs = [0.3, -1.2, 2.5, 0.7, 1.1]
    ys = [1.0, -0.4, 3.3, 0.2, 2.0]
    n = len(xs)
    xb, yb = math.fsum(xs) / n, math.fsum(ys) / n
    sxy = math.fsum((a - xb) * (c - yb) for a, c in zip(xs, ys))
    sxx = math.fsum((a - xb) ** 2 for a in xs)
    w = sxy / (sxx + 0.01)
    bb = yb - xb * w
    W, b = oracle_mod.ridge_fit(np.array(xs).reshape(1, n, 1), np.array(ys).reshape(1, n, 1), lam=0.01, dtype=F32)
    assert W[0, 0, 0] == pytest.approx(w, rel=1e-13)
    assert b[0, 0] == pytest.approx(bb, rel=1e-13)


def test_ridge_optimality_conditions(oracle_mod):
    """The fitted (W, b) is the minimiser of |y - x W - b|^2 + lambda |W|^2:
    the gradient in W, xc^T (xc W - yc) + lambda W, vanishes and the mean
    residual is zero."""
    rng = np.random.default_rng(14)
    X = rng.standard_normal((2, 150, 8)) * np.linspace(0.5, 4, 8) + 1.5
    Y = rng.standard_normal((2, 150, 3)) + X[:, :, :3] * 0.7
    lam = 0.5
    W, b = oracle_mod.ridge_fit(X, Y, lam=lam, dtype=F32)
    for g in range(2):
        xc = X[g] - X[g].mean(axis=0)
        yc = Y[g] - Y[g].mean(axis=0)
        grad = xc.T @ (xc @ W[g] - yc) + lam * W[g]
        assert np.abs(grad).max() < 1e-10
        assert np.abs((Y[g] - X[g] @ W[g] - b[g]).mean(axis=0)).max() < 1e-12


def test_ridge_shift_invariances(oracle_mod):
    """Shifting x by a constant vector c leaves W and moves b by -c W;
    shifting y by d moves only b, by d (centring at work)."""
    rng = np.random.default_rng(15)
    X = rng.standard_normal((1, 120, 4))
    Y = rng.standard_normal((1, 120, 2))
    c = np.array([5.0, -3.0, 0.5, 10.0])
    d = np.array([-7.0, 2.0])
    W0, b0 = oracle_mod.ridge_fit(X, Y, dtype=F32)
    W1, b1 = oracle_mod.ridge_fit(X + c, Y, dtype=F32)
    W2, b2 = oracle_mod.ridge_fit(X, Y + d, dtype=F32)
    np.testing.assert_allclose(W1, W0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(b1[0], b0[0] - c @ W0[0], rtol=0, atol=1e-11)
    np.testing.assert_allclose(W2, W0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(b2[0], b0[0] + d, rtol=0, atol=1e-12)


def test_ridge_bf16_storage_and_group_independence(oracle_mod):
    """bf16 storage (uint16 bits) fits the same as its fp32 spelling, and
    each group's fit depends on that group's data only."""
    rng = np.random.default_rng(16)
    X = torch.from_numpy(rng.standard_normal((3, 90, 6)).astype(np.float32)).to(torch.bfloat16)
    Y = torch.from_numpy(rng.standard_normal((3, 90, 4)).astype(np.float32)).to(torch.bfloat16)
    xb = X.view(torch.int16).numpy().view(np.uint16)
    yb = Y.view(torch.int16).numpy().view(np.uint16)
    Wb, bb = oracle_mod.ridge_fit(xb, yb, dtype=BF16)
    Wf, bf = oracle_mod.ridge_fit(X.float().numpy(), Y.float().numpy(), dtype=F32)
    np.testing.assert_array_equal(Wb, Wf)
    np.testing.assert_array_equal(bb, bf)
    W1, b1 = oracle_mod.ridge_fit(X[1:2].float().numpy(), Y[1:2].float().numpy(), dtype=F32)
    np.testing.assert_array_equal(W1[0], Wf[1])
    np.testing.assert_array_equal(b1[0], bf[1])

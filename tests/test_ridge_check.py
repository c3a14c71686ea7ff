"""The ridge acceptance check (tests/ridge_check.py) has the power the GPU
parity tests claim: on the CPU, with candidates made by the oracle, it
accepts the true fit rounded to fp32 and rejects fits that dropped the last
64-observation step or a single row, that skipped the centring, or whose
bias ignores the means — in exactly the shapes the GPU tests run, including
N <= IN where the centred Gram is rank-deficient and the old cond(A)-scaled
bound allowed a 10-30x relative error in W.

The planted mistakes live in the candidates (what a faulty kernel would
return), computed here on the CPU from the oracle; nothing runs on a GPU.
The bounds are those of the library's stated arithmetic (`ARITH`: fp32 sums
of exact products of the observations as stored); the large-mean cases use
the arithmetic of products of shifted observations (the observations minus
the group's first observation), the form that keeps fp32 sums near the
centred values.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import ridge_check


def bf16_data(rng, G, N, IN, mean):
    mu = rng.standard_normal((G, 1, IN)) * mean
    X = torch.from_numpy((rng.standard_normal((G, N, IN)) + mu).astype(np.float32)).to(torch.bfloat16)
    Wt = rng.standard_normal((G, IN, 128)) / IN ** 0.5
    Y = X.double().numpy() @ Wt + rng.standard_normal((G, 1, 128)) + 0.05 * rng.standard_normal((G, N, 128))
    Y = torch.from_numpy(Y.astype(np.float32)).to(torch.bfloat16)
    return X.double().numpy(), Y.double().numpy()


def first_row_shift(x, y):
    return dict(shift_x=x[0], shift_y=y[0])


def ARITH(x, y):
    """The shifts of the library's stated arithmetic: none."""
    return dict(shift_x=None, shift_y=None)


CASES = [(1000, 256, 0.01, 2.0), (64, 128, 0.01, 2.0), (65, 256, 0.01, 2.0), (3000, 512, 0.0, 2.0)]


@pytest.mark.parametrize("N,IN,lam,mean", CASES)
def test_check_accepts_the_true_fit_in_fp32(N, IN, lam, mean):
    rng = np.random.default_rng(N + IN)
    X, Y = bf16_data(rng, 1, N, IN, mean)
    W, b = oracle.ridge_fit(X, Y, lam=lam, dtype=oracle.F32)
    W32, b32 = W[0].astype(np.float32).astype(np.float64), b[0].astype(np.float32).astype(np.float64)
    st = ridge_check.check_fit(X[0], Y[0], W32, b32, lam, **ARITH(X[0], Y[0]), W_ref=W[0])
    assert st["res_ratio"] <= 1.0 and st["b_ratio"] <= 1.0 and st["fwd_ratio"] <= 1.0, st


@pytest.mark.parametrize("N,IN,lam,mean", CASES)
def test_check_rejects_a_dropped_step_or_row(N, IN, lam, mean):
    """Dropping the last 64-observation step (or the last row, when N = 65 or
    N = 64 holds a single step) moves the normal equations by far more than
    fp32 accumulation can."""
    rng = np.random.default_rng(N + IN)
    X, Y = bf16_data(rng, 1, N, IN, mean)
    keep = N - 64 if N > 128 else N - 1
    W, b = oracle.ridge_fit(X[:, :keep], Y[:, :keep], lam=lam, dtype=oracle.F32)
    st = ridge_check.check_fit(X[0], Y[0], W[0], b[0], lam, **ARITH(X[0], Y[0]))
    assert st["res_ratio"] > 1.0 or st["b_ratio"] > 1.0, st
    assert st["res_ratio"] > 10.0, st


@pytest.mark.parametrize("N,IN,lam,mean", [CASES[0], CASES[3]])
def test_check_rejects_uncentred_normal_equations(N, IN, lam, mean):
    """A fit that skipped the centring (X^T X + lambda I) W = X^T Y, b = 0.
    (With N <= IN such a fit differs from the minimiser mostly in the
    directions that only lambda constrains, where a backward error is small
    by construction; the wrong-penalty case below covers those shapes.)"""
    rng = np.random.default_rng(N + IN + 1)
    X, Y = bf16_data(rng, 1, N, IN, mean)
    x, y = X[0], Y[0]
    A = x.T @ x + lam * np.eye(IN)
    W = np.linalg.solve(A, x.T @ y)
    st = ridge_check.check_fit(x, y, W, np.zeros(128), lam, **ARITH(x, y))
    assert st["res_ratio"] > 10.0, st


@pytest.mark.parametrize("mean", [30.0, 100.0])
def test_check_power_with_large_means(mean):
    """Means of 30 and 100 standard deviations (where fp32 sums of the raw
    data would lose the centred Gram to cancellation): the check still
    accepts the true fit and rejects one that dropped a 64-observation step."""
    rng = np.random.default_rng(int(mean))
    X, Y = bf16_data(rng, 1, 2000, 256, mean)
    W, b = oracle.ridge_fit(X, Y, lam=0.01, dtype=oracle.F32)
    st = ridge_check.check_fit(X[0], Y[0], W[0].astype(np.float32).astype(np.float64),
                               b[0].astype(np.float32).astype(np.float64), 0.01, **first_row_shift(X[0], Y[0]),
                               W_ref=W[0])
    assert st["res_ratio"] <= 1.0 and st["b_ratio"] <= 1.0, st
    Wd, bd = oracle.ridge_fit(X[:, :-64], Y[:, :-64], lam=0.01, dtype=oracle.F32)
    st = ridge_check.check_fit(X[0], Y[0], Wd[0], bd[0], 0.01, **first_row_shift(X[0], Y[0]))
    assert st["res_ratio"] > 10.0, st


@pytest.mark.parametrize("N,IN,lam,mean", CASES[:3])
def test_check_rejects_a_wrong_penalty(N, IN, lam, mean):
    """lambda scaled by N (a plausible misreading of the penalty) in the
    shapes where N <= IN leaves lambda as the only constraint on part of W."""
    rng = np.random.default_rng(N + IN + 2)
    X, Y = bf16_data(rng, 1, N, IN, mean)
    W, b = oracle.ridge_fit(X, Y, lam=lam * N, dtype=oracle.F32)
    st = ridge_check.check_fit(X[0], Y[0], W[0], b[0], lam, **ARITH(X[0], Y[0]))
    assert st["res_ratio"] > 10.0, st


def test_check_rejects_a_bias_without_the_means():
    """The true W with b = mean(Y) (the mean(X) W term dropped)."""
    rng = np.random.default_rng(7)
    X, Y = bf16_data(rng, 1, 1000, 256, 2.0)
    W, _ = oracle.ridge_fit(X, Y, lam=0.01, dtype=oracle.F32)
    st = ridge_check.check_fit(X[0], Y[0], W[0], Y[0].mean(axis=0), 0.01, **ARITH(X[0], Y[0]))
    assert st["res_ratio"] <= 1.0 and st["b_ratio"] > 10.0, st

"""The acceptance check of a ridge fit against the definition, shared by the
GPU parity tests and the CPU tests that show the check can fail.

What is checked (the Qwen3 cache-mapping write-up, section "A linear bridge,
strangely enough, suffices": ridge regression with lambda = 0.01 and an
unpenalised bias).  The minimiser satisfies the normal equations of the
centred data,
    A W = B   with   A = Xc^T Xc + lambda I,   B = Xc^T Yc,
and b = mean(Y) - mean(X) W.  A candidate (W, b) is accepted when

  1. the residual  R = A W - B  (formed in fp64 from the data, the candidate
     W as given) satisfies  |R|_F <= K sigma_R, and
  2. every entry of  b - (mean(Y) - mean(X) W)  is within K sigma_b (+ the
     fp32 rounding of b).

Neither test involves cond(A): the residual is a backward error, so the check
keeps its power when N <= IN (a rank-deficient Xc, where A is held away from
singular only by lambda).  The forward error against the oracle,
W - W_ref = A^-1 R, is reported with |A^-1|_2 |R|_F.

sigma_R and sigma_b are the standard deviations of what fp32 accumulation
leaves in R and b under the standard model of rounding (Higham and Mary, "A
new approach to probabilistic rounding error analysis", 2019): every
addition into an fp32 accumulator commits an independent, unbiased relative
error of variance u^2/3 (u = 2^-24; round to nearest even), so a sum
accumulated through partial sums s_k has error variance (u^2/3) sum_k s_k^2.
The arithmetic is the one the library states (include/helm_kv.h): the
products X^T X and X^T Y are accumulated in fp32 in observation order, one
rounding per 16 observations (one 16-deep product), from exact products of
the data the library feeds them (`fed`: the observations, or the
observations minus a per-feature shift); the column sums likewise, one
rounding per 64 observations; the centring (A = G - s s^T / N) and the
solve are fp64; W and b are stored as fp32.  With V_A[i,j] = (u^2/3)
sum_k s_k[i,j]^2 and the sums' variances v_x, v_y,
    sigma_R^2 = sum_ij (V_A[i,j] + (v_x[i] s_x[j]^2 + s_x[i]^2 v_x[j]) / N^2) |W_j.|^2
              + sum_id (V_B[i,d] + (v_x[i] s_y[d]^2 + s_x[i]^2 v_y[d]) / N^2)
              + (|A|_2 u / sqrt(3))^2 |W|_F^2              (W rounded to fp32)
    sigma_b[d]^2 = (v_y[d] + sum_i v_x[i] W_id^2) / N^2 + (u/sqrt(3))^2 (sum_i |mean(x)_i W_id| + |b_d|)^2.
|R|_F^2 is a sum of IN * D such terms, so it concentrates tightly around its
mean; K = 6 leaves a wide margin for a model that is only approximately
right (hardware that rounds more often inside a product, say) while staying
within about 10x of the errors actually achieved.
"""
from __future__ import annotations

import math

import numpy as np

U32 = 2.0 ** -24
K_SIGMA = 6.0


def centred_system(x: np.ndarray, y: np.ndarray, lam: float):
    """(A, B, mean x, mean y) of one group in fp64 from its data [N, IN], [N, D]."""
    mx = x.mean(axis=0)
    my = y.mean(axis=0)
    xc = x - mx
    A = xc.T @ xc
    A[np.diag_indices_from(A)] += lam
    B = xc.T @ (y - my)
    return A, B, mx, my


def partial_sum_energy(f: np.ndarray, g: np.ndarray, step: int):
    """(E, e_f, e_g, s_f, s_g): E[i, j] = sum over k of (sum_{n < k step} f_ni g_nj)^2
    (the partial sums an in-order accumulator holds after every `step`
    observations), e_f / e_g the same for the column sums (every 64
    observations), s_f / s_g the column sums.  fp64."""
    N = f.shape[0]
    run = np.zeros((f.shape[1], g.shape[1]))
    energy = np.zeros_like(run)
    rf, rg = np.zeros(f.shape[1]), np.zeros(g.shape[1])
    ef, eg = np.zeros_like(rf), np.zeros_like(rg)
    for n0 in range(0, N, step):
        fc, gc = f[n0:n0 + step], g[n0:n0 + step]
        run += fc.T @ gc
        energy += run * run
        rf += fc.sum(axis=0)
        rg += gc.sum(axis=0)
        if (n0 // step + 1) % (64 // step) == 0 or n0 + step >= N:
            ef += rf * rf
            eg += rg * rg
    return energy, ef, eg, rf, rg


def check_fit(x: np.ndarray, y: np.ndarray, W: np.ndarray, b: np.ndarray, lam: float,
              shift_x: np.ndarray | None = None, shift_y: np.ndarray | None = None,
              W_ref: np.ndarray | None = None) -> dict:
    """Check of one group's candidate (W [IN, D], b [D]) against data x [N, IN],
    y [N, D] (fp64).  shift_x / shift_y: the per-feature values the library
    subtracts before its fp32 products (None = nothing).  Returns the ratios
    (<= 1 passes) and the reported forward error; does not assert."""
    N, IN = x.shape
    fx = x - shift_x if shift_x is not None else x
    fy = y - shift_y if shift_y is not None else y
    A, B, mx, my = centred_system(x, y, lam)
    R = A @ W - B
    # partial sums every 16 observations (every 64, scaled by 4, for long inputs)
    step, scale = (16, 1.0) if N <= 16384 else (64, 4.0)
    EA, ex, _, sx, _ = partial_sum_energy(fx, fx, step)
    EB, _, ey, _, sy = partial_sum_energy(fx, fy, step)
    q = U32 * U32 / 3.0
    VA = q * scale * EA + q * (np.outer(ex, sx * sx) + np.outer(sx * sx, ex)) / (N * N)
    VB = q * scale * EB + q * (np.outer(ex, sy * sy) + np.outer(sx * sx, ey)) / (N * N)
    w2 = (W * W).sum(axis=1)                      # |W_j.|^2
    normA = np.linalg.norm(A, 2)
    var_R = float(VA.sum(axis=0) @ w2 + VB.sum() + (normA * U32) ** 2 / 3.0 * (W * W).sum())
    sigma_R = math.sqrt(var_R)
    b_def = my - mx @ W
    var_b = q * (ey + ex @ (W * W)) / (N * N) + q * (np.abs(mx) @ np.abs(W) + np.abs(b)) ** 2
    tol_b = K_SIGMA * np.sqrt(var_b) + U32 * np.abs(b) + 1e-300
    out = dict(res_ratio=float(np.linalg.norm(R) / (K_SIGMA * sigma_R)),
               b_ratio=float((np.abs(b - b_def) / tol_b).max()),
               res_rel=float(np.linalg.norm(R) / max(np.linalg.norm(B), 1e-300)),
               tol_rel=float(K_SIGMA * sigma_R / max(np.linalg.norm(B), 1e-300)))
    if W_ref is not None:
        inv_norm = 1.0 / max(np.linalg.eigvalsh(A).min(), 1e-300)
        out["fwd_err_rel"] = float(np.abs(W - W_ref).max() / max(np.abs(W_ref).max(), 1e-300))
        out["fwd_ratio"] = float(np.linalg.norm(W - W_ref) / (inv_norm * K_SIGMA * sigma_R))
    return out

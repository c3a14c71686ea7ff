"""GPU parity of the ridge fit (helm_ridge_fit) against the fp64 oracle
(oracle.ridge_fit) and the definition, through the C ABI.

The Qwen3 cache-mapping write-up, section "A linear bridge, strangely enough,
suffices": each map is fitted by ridge regression with lambda = 0.01 and the
bias from the means.

Acceptance (tests/ridge_check.py): the candidate W must satisfy the centred
normal equations A W = B to within a backward-error bound derived from the
library's stated arithmetic (fp32 sums of exact products, probabilistic
rounding bound with c = 8), and b must equal mean(Y) - mean(X) W to within
the fp32 sums' bound.  The bounds do not grow with cond(A), so the cases with
N <= IN (a rank-deficient centred Gram) are checked as strictly as the rest.
The forward error against the oracle's W is logged with its implied bound
|A^-1| |R|; tests/test_ridge_check.py shows on the CPU that a fit that
dropped the last 64-observation step, or one row, is rejected.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import parity, ridge_check
from tests.parity import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _library():
    import cross_model_kv_helm_amd as hk
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert hk.helm_device_check(-1) == 0, hk.helm_last_error()
    yield


def draw(G, N, IN, seed, mean=2.0, noise=0.05):
    """X with per-feature means ~ N(0, mean^2) and unit-variance noise;
    Y = X W* + b* + noise (a planted map), both rounded to bf16."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    mu = torch.randn((G, 1, IN), generator=g, device="cuda") * mean
    X = (torch.randn((G, N, IN), generator=g, device="cuda") + mu).to(torch.bfloat16)
    Wt = torch.randn((G, IN, 128), generator=g, device="cuda") / IN ** 0.5
    bt = torch.randn((G, 1, 128), generator=g, device="cuda")
    Y = (torch.bmm(X.float(), Wt) + bt + noise * torch.randn((G, N, 128), generator=g, device="cuda"))
    return X, Y.to(torch.bfloat16)


def check(X, Y, W, b, lam, label, groups=None, oracle_groups=None):
    """Checks every group in `groups` against the definition; the groups in
    `oracle_groups` (default: all of them) also against the oracle's W."""
    G, N, IN = X.shape
    groups = range(G) if groups is None else groups
    oracle_groups = set(groups if oracle_groups is None else oracle_groups)
    xs = parity.to_np_storage(X)
    ys = parity.to_np_storage(Y)
    Wg = W.double().cpu().numpy()
    bg = b.double().cpu().numpy()
    worst = {}
    for gi in groups:
        assert np.isfinite(Wg[gi]).all() and np.isfinite(bg[gi]).all(), f"{label} group {gi}: non-finite"
        W_ref = None
        if gi in oracle_groups:
            W_ref = oracle.ridge_fit(xs[gi:gi + 1], ys[gi:gi + 1], lam=lam, dtype=oracle.BF16)[0][0]
        x = parity.storage_to_f64(xs[gi])
        y = parity.storage_to_f64(ys[gi])
        st = ridge_check.check_fit(x, y, Wg[gi], bg[gi], lam, **hk_shift(x, y), W_ref=W_ref)
        for key, v in st.items():
            worst[key] = max(worst.get(key, 0.0), v)
        assert st["res_ratio"] <= 1.0, f"{label} group {gi}: normal-equation residual over its bound {st}"
        assert st["b_ratio"] <= 1.0, f"{label} group {gi}: bias off mean(Y) - mean(X) W beyond its bound {st}"
        if W_ref is not None:
            assert st["fwd_ratio"] <= 1.0, f"{label} group {gi}: W off the oracle's beyond |A^-1| bound_R {st}"
    log(f"{label}: {len(groups)} groups; worst {worst}")


def hk_shift(x, y):
    """The per-feature shifts the library subtracts before its fp32 products
    (include/helm_kv.h, helm_ridge_fit): a feature's first value when its
    first min(N, 64) values share one sign and lie within a factor 1.5 of
    each other, else 0 (the comparisons in fp32, as the library makes them;
    every value here is a bf16 number, so they are exact)."""
    def rule(a):
        head = a[:64].astype(np.float32)
        lo, hi, first = head.min(axis=0), head.max(axis=0), head[0]
        k = np.float32(1.5)
        tight = ((lo > 0) & (hi <= k * lo)) | ((hi < 0) & (lo >= k * hi))
        return np.where(tight, first, np.float32(0)).astype(np.float64)
    return dict(shift_x=rule(x), shift_y=rule(y))


def fit(X, Y, lam):
    import cross_model_kv_helm_amd as hk
    W, b = hk.helm_ridge_fit(X, Y, lam=lam)
    torch.cuda.synchronize()
    return W, b


def test_ridge_small_ragged_three_groups():
    """3 groups (not a multiple of 8: plain tile order), N = 1000 (the last
    64-observation step ragged), IN = 256 (one X tile)."""
    X, Y = draw(3, 1000, 256, 1)
    check(X, Y, *fit(X, Y, 0.01), 0.01, "ridge G3 N1000 IN256")


def test_ridge_in128_single_step():
    """IN = 128 (half of the one X tile idle), N = 64 (one step)."""
    X, Y = draw(2, 64 * 9, 128, 2)
    X, Y = X[:, :64].contiguous(), Y[:, :64].contiguous()
    check(X, Y, *fit(X, Y, 0.01), 0.01, "ridge G2 N64 IN128")


def test_ridge_in384_xcd_order_strong_penalty():
    """IN = 384 (two X tiles, the second half idle; three upper tiles), 8
    groups (the XCD tile order), N = 4097, lambda = 50."""
    X, Y = draw(8, 4097, 384, 3)
    check(X, Y, *fit(X, Y, 50.0), 50.0, "ridge G8 N4097 IN384 lam50")


def test_ridge_zero_penalty():
    """lambda = 0: plain least squares with an intercept."""
    X, Y = draw(2, 3000, 512, 4)
    check(X, Y, *fit(X, Y, 0.0), 0.0, "ridge G2 N3000 IN512 lam0")


def test_ridge_in1024():
    """IN = 1024 (the largest width: four X tiles, ten upper tiles), N = 2500."""
    X, Y = draw(1, 2500, 1024, 5, mean=0.5)
    check(X, Y, *fit(X, Y, 0.01), 0.01, "ridge G1 N2500 IN1024")


@pytest.mark.parametrize("IN", [640, 768, 896])
def test_ridge_five_to_seven_feature_groups(IN):
    """IN = 640 / 768 / 896: 5, 6 and 7 groups of 128 features, the widths
    whose last diagonal tile holds a single group (5, 7) and whose X^T Y
    blocks of the odd groups leave a half-empty pairing tile (6, 7)."""
    X, Y = draw(2, 1500, IN, 20 + IN // 128, mean=0.5)
    check(X, Y, *fit(X, Y, 0.01), 0.01, f"ridge G2 N1500 IN{IN}")


def test_ridge_stages_equal_one_call():
    """The products stage and the solve stage enqueued separately write
    exactly what one call writes."""
    import cross_model_kv_helm_amd as hk
    X, Y = draw(3, 777, 256, 6)
    W1, b1 = fit(X, Y, 0.01)
    ws = torch.empty(hk.helm_ridge_workspace_bytes(hk.ridge_shape(3, 777, 256)), dtype=torch.uint8, device="cuda")
    W2 = torch.full_like(W1, float("nan"))
    b2 = torch.full_like(b1, float("nan"))
    hk.helm_ridge_fit(X, Y, W=W2, b=b2, workspace=ws, stages=hk.HELM_STAGE_TABLES)
    hk.helm_ridge_fit(X, Y, W=W2, b=b2, workspace=ws, stages=hk.HELM_STAGE_MAP)
    torch.cuda.synchronize()
    assert torch.equal(W1, W2) and torch.equal(b1, b2)


def test_ridge_calibration_shape_sampled():
    """The calibration's shape per group (about 128K observations, IN = k*D =
    512 at k = 4): 16 groups (two rounds of the XCD order), 3 checked
    against the oracle."""
    X, Y = draw(16, 131072, 512, 7, mean=1.0, noise=0.1)
    W, b = fit(X, Y, 0.01)
    check(X, Y, W, b, 0.01, "ridge G16 N131072 IN512", groups=[0, 7, 11, 15], oracle_groups=[0, 15])


def test_ridge_one_observation():
    """N = 1: the centred data are zero, so W = 0 and b = that observation's
    targets (exactly, after the fp32 store)."""
    X, Y = draw(2, 1, 256, 8)
    W, b = fit(X, Y, 0.01)
    assert torch.equal(W, torch.zeros_like(W))
    assert torch.equal(b, Y[:, 0].float())


def test_ridge_one_row_in_the_last_step():
    """N = 65: the second 64-observation step holds one row (the other 63
    read zeros)."""
    X, Y = draw(3, 65, 256, 9)
    check(X, Y, *fit(X, Y, 0.01), 0.01, "ridge G3 N65 IN256")


def test_ridge_large_means():
    """Features and targets whose means are 30 to 100 times their spread.
    Sums of raw products lose about (mean / std)^2 * 2^-24 of relative
    accuracy to cancellation in the centring (up to 6e-4 here); the library
    shifts such features by their first observation before the products, so
    the fit must meet the bound of the shifted data.  The bound a library
    without the shift would need is logged beside it."""
    G, N, IN = 2, 20000, 256
    g = torch.Generator(device="cuda").manual_seed(11)
    sd = 0.5
    ratio = 30.0 + 70.0 * torch.rand((G, 1, IN), generator=g, device="cuda")
    sign = torch.where(torch.rand((G, 1, IN), generator=g, device="cuda") < 0.5, -1.0, 1.0)
    X = (sd * torch.randn((G, N, IN), generator=g, device="cuda") + sign * ratio * sd).to(torch.bfloat16)
    Wt = torch.randn((G, IN, 128), generator=g, device="cuda") / IN ** 0.5
    bt = 40.0 + torch.randn((G, 1, 128), generator=g, device="cuda")
    Y = (torch.bmm(X.float(), Wt) + bt + 0.05 * torch.randn((G, N, 128), generator=g, device="cuda"))
    Y = Y.to(torch.bfloat16)
    W, b = fit(X, Y, 0.01)
    xs, ys = parity.to_np_storage(X), parity.to_np_storage(Y)
    shifted = 0
    for gi in range(G):
        x, y = parity.storage_to_f64(xs[gi]), parity.storage_to_f64(ys[gi])
        sh = hk_shift(x, y)
        shifted += int((sh["shift_x"] != 0).sum())
        plain = ridge_check.check_fit(x, y, W[gi].double().cpu().numpy(), b[gi].double().cpu().numpy(), 0.01)
        log(f"ridge large means group {gi}: bound without shifts tol_rel {plain['tol_rel']:.3g}")
    assert shifted >= G * IN * 0.95, f"only {shifted} of {G * IN} features shifted"
    check(X, Y, W, b, 0.01, "ridge G2 N20000 IN256 mean/std 30-100")


@pytest.mark.parametrize("i", range(6))
def test_ridge_random_shapes(i):
    """Seeded random fits: 1-3 groups, 1-2,499 observations (so the last
    64-observation step ends anywhere, and N <= IN happens), IN any multiple
    of 128 up to 1,024, lambda 0.01 or 1, feature means 0, 2 or 30 sigma (the
    last ones shifted before the products); every group checked against the
    definition and the oracle."""
    rng = np.random.default_rng(9500 + i)
    IN = 128 * int(rng.integers(1, 9))
    G = int(rng.integers(1, 4))
    N = int(rng.integers(1, 2500))
    lam = float(rng.choice([0.01, 1.0]))
    mean = float(rng.choice([0.0, 2.0, 30.0]))
    label = f"ridge sweep {i}: G={G} N={N} IN={IN} lambda={lam} mean={mean}"
    log(label)
    X, Y = draw(G, N, IN, 9500 + i, mean=mean)
    W, b = fit(X, Y, lam)
    check(X, Y, W, b, lam, label)

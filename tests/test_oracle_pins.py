"""Pins of the float64 oracle against what the method pages and the mathematics fix (CPU only).

Each test names the fact it checks.  None of them re-types an oracle formula: the references are printed
values of the GPTQ tutorial page's worked examples (tests/golden/), textbook procedures with explicit
inverses or least squares, brute force, closed-form identities, and library routines.
"""
import json
import os

import numpy as np
from fractions import Fraction
import pytest
import torch

import oracle as O
import workloads


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _sse(X, cand, w):
    return float(np.sum((np.asarray(X) @ (np.asarray(cand) - np.asarray(w))) ** 2))


# ------------------------------------------------------------------ worked examples of the GPTQ tutorial page
def test_two_weight_example(golden_dir):
    g = _load(golden_dir, "two_weight_example.json")
    X = np.array(g["X"])
    H = O.gram([X])
    np.testing.assert_allclose(H, g["H"], atol=1e-12)
    prep = O.prepare(H, 0.0)
    np.testing.assert_allclose(prep["P"], g["P"], atol=1e-12)
    U = prep["U"]
    assert abs(U[1, 1] ** 2 - g["U11_squared"]) < 1e-12
    assert abs(U[1, 1] ** 2 - prep["P"][1, 1]) > 0.1          # the factor is not the inverse's entry
    w = np.array(g["w"])[:, None]
    r = O.quantize_layer(w, U, bits=g["bits"], scales=np.array([g["scale"]], np.float32), record_trace=True)
    q = (r["codes"][:, 0] - g["zero_point"]).astype(float)
    np.testing.assert_allclose(q, g["quantized"], atol=0)
    np.testing.assert_allclose(r["trace"][0][:, 0], g["weights_after_first_step"], atol=1e-12)
    assert abs(_sse(X, r["trace"][0][:, 0], g["w"]) - g["output_error_after_first_step"]) < 1e-12
    assert abs(_sse(X, q, g["w"]) - g["final_output_error"]) < 1e-12
    assert abs(O.layer_objective(H, w, q[:, None]) - g["final_output_error"]) < 1e-12
    rtn = O.fixed_grid_quantize(np.array(g["w"]))
    assert abs(_sse(X, rtn, g["w"]) - g["rtn_output_error"]) < 1e-12
    assert abs(np.mean((rtn - g["w"]) ** 2) - g["weight_mse_rtn"]) < 1e-12
    assert abs(np.mean((q - g["w"]) ** 2) - g["weight_mse_final"]) < 1e-12
    # first step written with the inverse directly: delta = -r P[:,0] / P[0,0]
    P = np.array(g["P"])
    delta = -(g["w"][0] - 0.0) * P[:, 0] / P[0, 0]
    np.testing.assert_allclose(delta, g["first_step_update"], atol=1e-12)
    seq = O.obq_sequential(H, g["w"], O.fixed_grid_quantize)
    np.testing.assert_allclose(seq["trace"][0], g["weights_after_first_step"], atol=1e-12)


def test_three_weight_counterexample(golden_dir):
    g = _load(golden_dir, "three_weight_counterexample.json")
    X = np.array(g["X"])
    H = O.gram([X])
    np.testing.assert_allclose(H, g["H"], atol=1e-12)
    prep = O.prepare(H, 0.0)
    np.testing.assert_allclose(prep["P"], g["P"], atol=1e-12)
    np.testing.assert_allclose(prep["U"], g["U"], atol=1e-12)
    np.testing.assert_allclose(np.array(g["H"]) @ np.array(g["P"]), np.eye(3), atol=1e-12)
    w = np.array(g["w"])[:, None]
    r = O.quantize_layer(w, prep["U"], bits=4, scales=np.array([1.0], np.float32), record_trace=True)
    q = (r["codes"][:, 0] - 8).astype(float)
    np.testing.assert_allclose(q, g["quantized"], atol=0)
    assert abs(r["trace"][1][2, 0] - g["trace_step2_coord3"]) < 1e-12
    assert abs(_sse(X, q, g["w"]) - g["sequential_output_error"]) < 1e-12
    rtn = O.fixed_grid_quantize(np.array(g["w"]))
    assert abs(_sse(X, rtn, g["w"]) - g["rtn_output_error"]) < 1e-12
    grid = range(-8, 8)
    assert len(grid) ** 3 == g["grid_points"]
    best, arg = O.exhaustive_best(lambda c: _sse(X, c, g["w"]), 3, grid)
    assert abs(best - g["best_output_error"]) < 1e-12
    assert [list(map(float, a)) for a in arg] == [g["best"]]
    assert _sse(X, q, g["w"]) > best                          # sequential is not the discrete optimum


# ------------------------------------------------------------------ textbook and brute-force references
@pytest.mark.parametrize("K,seed", [(2, 0), (3, 1), (5, 2), (8, 3), (8, 4)])
def test_loop_equals_explicit_inverse_obq(K, seed):
    """U-row algorithm == sequential compensation that re-inverts H[F,F] at every step (K <= 8)."""
    rng = np.random.default_rng(seed)
    Hd = workloads.random_spd(K, seed)
    w = rng.normal(0, 2.0, size=K)
    prep = O.prepare(Hd, 0.0)
    r = O.quantize_layer(w[:, None], prep["U"], bits=4, scales=np.array([1.0], np.float32))
    seq = O.obq_sequential(Hd, w, O.fixed_grid_quantize)
    np.testing.assert_allclose(r["Q"][:, 0], seq["w"], atol=1e-12)
    # per-step added objective r^2 / (2 P_F[q,q]) == 1/2 E_q^2
    np.testing.assert_allclose(0.5 * r["E"][:, 0] ** 2, seq["added"], rtol=1e-9, atol=1e-14)


def test_exhaustive_lower_bound():
    """The sequential result can never beat the exhaustive optimum of the same grid (K = 3, 4)."""
    for K, seed in [(3, 5), (4, 6)]:
        Hd = workloads.random_spd(K, seed)
        w = np.random.default_rng(seed).normal(0, 1.5, size=K)
        prep = O.prepare(Hd, 0.0)
        r = O.quantize_layer(w[:, None], prep["U"], bits=3, scales=np.array([1.0], np.float32))
        obj = lambda c: 0.5 * (c - w) @ Hd @ (c - w)
        best, _ = O.exhaustive_best(obj, K, range(-4, 4))
        assert obj(r["Q"][:, 0]) >= best - 1e-12


def test_factor_schur_property():
    """[T4]: U[q:,q:]^T U[q:,q:] is the inverse of the remaining Hessian for every q."""
    K = 12
    Hd = workloads.random_spd(K, 7)
    U = O.prepare(Hd, 0.0)["U"]
    assert np.allclose(np.tril(U, -1), 0)
    for q in range(K):
        np.testing.assert_allclose(U[q:, q:].T @ U[q:, q:], np.linalg.inv(Hd[q:, q:]), rtol=1e-9, atol=1e-12)
        assert abs(U[q, q] ** 2 - np.linalg.inv(Hd[q:, q:])[0, 0]) < 1e-10
    # scipy's Cholesky of the inverse, read as upper factor, agrees
    import scipy.linalg
    np.testing.assert_allclose(U, scipy.linalg.cholesky(np.linalg.inv(Hd), lower=False), rtol=1e-8, atol=1e-12)


@pytest.mark.parametrize("B", [7, 64, 128])
def test_lazy_blocks_equal_eager(B):
    """[T5]: lazy block updates are the same computation as updating every free weight at once."""
    K, N = 300, 17
    rng = np.random.default_rng(11)
    H = O.gram([rng.normal(size=(600, K)) * np.exp(rng.normal(0, 1, K))])
    prep = O.prepare(H, 0.01)
    W = rng.normal(0, 0.02, size=(K, N))
    a = O.quantize_layer(W, prep["U"], bits=3)
    b = O.quantize_layer(W, prep["U"], bits=3, blocksize=B)
    assert np.array_equal(a["codes"], b["codes"])
    np.testing.assert_allclose(a["E"], b["E"], rtol=0, atol=1e-9 * np.abs(a["E"]).max())


def test_loss_identity():
    """Sum of 1/2 E^2 over a channel equals 1/2 d0^T H_d d0 with d0 = W_hat - W (dead rows zeroed)."""
    K, N = 96, 9
    rng = np.random.default_rng(12)
    H = O.gram([rng.normal(size=(256, K))])
    prep = O.prepare(H, 0.01)
    W = rng.normal(0, 0.02, size=(K, N))
    r = O.quantize_layer(W, prep["U"], bits=4, blocksize=32)
    d0 = r["Q"] - r["W0"]
    np.testing.assert_allclose(r["losses"], 0.5 * np.sum((prep["Hd"] @ d0) * d0, axis=0), rtol=1e-9)


def test_codes_invariant_under_hessian_scaling():
    """[T1], [T6]: normalising H by a constant rescales damping too, so codes do not change."""
    K, N = 64, 16
    rng = np.random.default_rng(13)
    H = O.gram([rng.normal(size=(128, K)) * np.exp(rng.normal(0, 1, K))])
    W = rng.normal(0, 0.02, size=(K, N))
    a = O.quantize_layer(W, O.prepare(H, 0.01)["U"], bits=4)
    b = O.quantize_layer(W, O.prepare(H * 0.25, 0.01)["U"], bits=4)      # power of two: exact
    c = O.quantize_layer(W, O.prepare(H * 3.7, 0.01)["U"], bits=4)
    assert np.array_equal(a["codes"], b["codes"])
    assert np.array_equal(a["codes"], c["codes"])


def test_dead_coordinates():
    """[T6]: a zero-energy input coordinate gets diagonal 1, decouples, and its weight row goes to zero."""
    K, N = 20, 6
    rng = np.random.default_rng(14)
    X = rng.normal(size=(64, K))
    X[:, [3, 11]] = 0.0
    H = O.gram([X])
    prep = O.prepare(H, 0.01)
    assert list(np.flatnonzero(prep["dead"])) == [3, 11]
    np.testing.assert_allclose(prep["damp"], 0.01 * (np.trace(H) + 2) / K)
    U = prep["U"]
    for k in (3, 11):
        off = np.concatenate([U[k, :k], U[k, k + 1:], U[:k, k], U[k + 1:, k]])
        assert np.abs(off).max() < 1e-12
        assert abs(U[k, k] - 1.0 / np.sqrt(1.0 + prep["damp"])) < 1e-12
    W = rng.normal(0, 0.02, size=(K, N))
    r = O.quantize_layer(W, U, bits=4, dead=prep["dead"])
    assert np.all(r["codes"][[3, 11]] == 8)
    np.testing.assert_allclose(r["scales"], O.channel_scales(W, 4))   # scales from W before zeroing


def test_not_positive_definite():
    with pytest.raises(O.NotPositiveDefinite):
        O.prepare(np.array([[1.0, 2.0], [2.0, 1.0]]), 0.01)


def test_channel_scale_rule_properties():
    W = np.random.default_rng(15).normal(0, 0.02, size=(50, 7)).astype(np.float32)
    W[:, 3] = 0.0
    for b in (2, 3, 4, 8):
        s = O.channel_scales(W, b)
        assert s.dtype == np.float32
        assert s[3] == 1.0
        np.testing.assert_array_equal(s, O.channel_scales(-W, b))        # symmetric
        amax = np.abs(W).max(0)
        live = amax > 0
        np.testing.assert_allclose(s[live] * (2 ** b - 1) / 2, amax[live], rtol=2e-7)
    # 4-bit: codes 0..15 with zero point 8, as in the tutorial's fixed grid
    r = O.quantize_layer(np.array([[-1.0], [0.51], [7.4]]), np.eye(3), bits=4,
                         scales=np.array([1.0], np.float32))
    assert list(r["codes"][:, 0]) == [7, 9, 15]


def test_channel_scale_is_the_symmetric_min_max_grid():
    """[T] T2 contrasts its fixed teaching grid with the grid a quantiser normally gets from the weights by min-max;
    [G] makes that grid symmetric per channel.  A min-max grid of 2^b codes spans [lo, hi] in 2^b - 1 equal steps with
    the zero point rint(-lo / step); for the symmetric range lo = -max|w|, hi = max|w|.  Built here from that
    definition (float64 range and step, codes by nearest rounding) and compared with the oracle's scales and its
    fixed zero point 2^(b-1) and codes."""
    rng = np.random.default_rng(21)
    W = rng.normal(0, 0.02, size=(64, 9)) * np.exp(rng.normal(0, 1, size=9))
    W = W.astype(np.float32)
    for b in (2, 3, 4, 5, 6):
        s = O.channel_scales(W, b)
        for n in range(W.shape[1]):
            w = W[:, n].astype(np.float64)
            m = np.abs(w).max()
            lo, hi = -m, m                                    # symmetric range of the channel
            step = (hi - lo) / (2 ** b - 1)                   # 2^b levels from lo to hi
            zero = round(Fraction(2 ** b - 1, 2))             # rint(-lo / step) = rint((2^b - 1) / 2), exactly
            assert zero == 2 ** (b - 1)                       # the oracle's fixed zero point, 8 at 4 bits as in T2
            assert abs(s[n] - step) <= 2 ** -23 * step        # the oracle's scale is that step (fp32-rounded)
            # the grid covers the whole range: every weight of the channel, its extremes included, is
            # reconstructed within half a step (no clipping), rounding each weight on its own (U = I)
            r = O.quantize_layer(w[:, None], np.eye(len(w)), bits=b, scales=s[n:n + 1])
            rec = s[n] * (r["codes"][:, 0].astype(np.float64) - zero)
            assert np.all(np.abs(rec - w) <= 0.5 * step * (1 + 1e-6))


def test_tie_codes_adopted_only_in_band():
    U = np.eye(2)
    W = np.array([[0.5, 0.5], [1.25, 0.3]])
    base = O.quantize_layer(W, U, bits=4, scales=np.array([1.0, 1.0], np.float32))
    assert base["codes"][0, 0] == 8                                   # 0.5 -> 0 (half to even)
    forced = np.array([[9, 9], [0, 0]])
    r = O.quantize_layer(W, U, bits=4, scales=np.array([1.0, 1.0], np.float32), tie_codes=forced)
    assert r["codes"][0, 0] == 9 and r["codes"][0, 1] == 9 and r["n_adopted"] == 2
    assert r["codes"][1, 0] == base["codes"][1, 0]                     # not in band: ignored


# ------------------------------------------------------------------ Gram and asymmetric-calibration pieces
def test_gram_identities(golden_dir):
    rng = np.random.default_rng(16)
    X = rng.normal(size=(200, 9))
    H = O.gram([X[:70], X[70:150], X[150:]])
    for _ in range(5):
        v = rng.normal(size=9)
        assert abs(np.sum((X @ v) ** 2) - 0.5 * v @ H @ v) < 1e-9 * np.sum((X @ v) ** 2)
    np.testing.assert_allclose(H, H.T, atol=0)
    brute = np.zeros((9, 9))
    for t in range(200):
        for i in range(9):
            for j in range(9):
                brute[i, j] += 2.0 * X[t, i] * X[t, j]
    np.testing.assert_allclose(H, brute, rtol=1e-12)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(17)
    x = np.concatenate([rng.normal(size=4000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 4000),
                        np.array([0.0, -0.0, 1.00390625, 1.01171875, 3.0e38, -3.0e38, 1e-40, np.inf],
                                 np.float32)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(O.bf16_round(x), ref)


def test_row_scaled_gram():
    rng = np.random.default_rng(18)
    X = O.bf16_round(rng.normal(size=(100, 12)).astype(np.float32))
    H = O.gram([X])
    np.testing.assert_array_equal(O.gram_row_scaled(X, np.ones(100)), H)
    np.testing.assert_array_equal(O.gram_row_scaled(X, np.full(100, 0.5)), H * 0.25)
    rho = rng.uniform(0.5, 1.5, size=100)
    Hg = O.gram_row_scaled(X, rho)
    ref = torch.from_numpy((rho.astype(np.float32)[:, None] * X)).to(torch.bfloat16).double().numpy()
    np.testing.assert_allclose(Hg, 2.0 * ref.T @ ref, rtol=1e-12)


def test_cross_gram_and_asym_objective():
    rng = np.random.default_rng(19)
    M, K, N = 80, 7, 3
    Xf = rng.normal(size=(M, K))
    X = Xf + 0.05 * np.abs(Xf) * rng.normal(size=(M, K))
    H, A, G = O.gram([X]), O.cross_gram(Xf, X), O.gram([Xf])
    np.testing.assert_allclose(H + A, 2.0 * Xf.T @ X, rtol=1e-12, atol=1e-12)  # X~^T X = X^T X + dX^T X
    W = rng.normal(size=(K, N))
    Wh = np.round(W * 4) / 4
    direct = float(np.sum((X @ Wh - Xf @ W) ** 2))
    assert abs(O.asym_objective(H, A, G, W, Wh) - direct) < 1e-9 * direct
    np.testing.assert_allclose(O.cross_gram(X, X), 0.0)


def test_asym_correction_forms_agree():
    """[R] item 3's triangular form equals the per-step ridge least-squares definition and lstsq."""
    rng = np.random.default_rng(20)
    M, K = 200, 24
    Xf = rng.normal(size=(M, K)) * np.exp(rng.normal(0, 0.7, K))
    X = Xf + 0.05 * np.abs(Xf) * rng.normal(size=(M, K))
    prep = O.prepare(O.gram([X]), 0.01)
    A = O.cross_gram(Xf, X)
    P_tri = O.asym_correction(prep["U"], A)
    P_def = O.asym_correction_by_definition(prep["Hd"], A)
    np.testing.assert_allclose(P_tri, P_def, rtol=1e-8, atol=1e-10 * np.abs(P_def).max())
    assert np.allclose(np.tril(P_tri), 0)
    lam = np.sqrt(prep["damp"] / 2.0)
    dX = Xf - X
    for q in (0, 5, K - 2):
        rest = list(range(q + 1, K))
        lhs = np.vstack([X[:, rest], lam * np.eye(len(rest))])
        rhs = np.concatenate([dX[:, q], np.zeros(len(rest))])
        np.testing.assert_allclose(P_tri[q, rest], np.linalg.lstsq(lhs, rhs, rcond=None)[0], rtol=1e-7,
                                   atol=1e-10)
    np.testing.assert_allclose(O.asym_correction(prep["U"], np.zeros((K, K))), 0.0)


def test_asym_loop_equals_explicit_solves():
    """GPTAQ loop with P1 == sequential compensation with explicit inverses plus a per-step lstsq."""
    rng = np.random.default_rng(21)
    M, K = 60, 6
    Xf = rng.normal(size=(M, K))
    X = Xf + 0.1 * np.abs(Xf) * rng.normal(size=(M, K))
    prep = O.prepare(O.gram([X]), 0.01)
    A = O.cross_gram(Xf, X)
    P1 = O.asym_correction(prep["U"], A)
    w = rng.normal(0, 1.5, size=K)
    r = O.quantize_layer(w[:, None], prep["U"], bits=4, scales=np.array([1.0], np.float32), P1=P1)
    seq = O.obq_sequential(prep["Hd"], w, O.fixed_grid_quantize, damp=prep["damp"], X_free_basis=(X, Xf - X))
    np.testing.assert_allclose(r["Q"][:, 0], seq["w"], atol=1e-10)
    rb = O.quantize_layer(w[:, None], prep["U"], bits=4, scales=np.array([1.0], np.float32), P1=P1,
                          blocksize=4)
    np.testing.assert_array_equal(rb["codes"], r["codes"])
    # no input mismatch -> no correction -> plain GPTQ
    r0 = O.quantize_layer(w[:, None], prep["U"], bits=4, scales=np.array([1.0], np.float32),
                          P1=O.asym_correction(prep["U"], O.cross_gram(X, X)))
    rg = O.quantize_layer(w[:, None], prep["U"], bits=4, scales=np.array([1.0], np.float32))
    np.testing.assert_array_equal(r0["codes"], rg["codes"])


def test_generator_asym_mismatch_is_bf16_exact():
    cfg = workloads.CONFIGS["c4_up_proj_8b_gptaq"].scaled(K=64, N=8, M=512)
    L = workloads.make_layer(cfg)
    d = L["X_float"].float() - L["X"].float()
    assert torch.equal(d.to(torch.bfloat16).float(), d)


# ------------------------------------------------------------------------------------------------ CAE term
def _cae_problem(seed, K=6, M=60, dead=()):
    rng = np.random.default_rng(seed)
    Xf = rng.normal(size=(M, K))
    X = Xf + 0.1 * np.abs(Xf) * rng.normal(size=(M, K))
    for k in dead:
        X[:, k] = 0.0
        Xf[:, k] = 0.0
    H = O.gram([X])
    prep = O.prepare(H, 0.01)
    A = O.cross_gram(Xf, X)
    return rng, X, Xf, H, prep, A


def test_cae_correction_forms_agree():
    """P2 from the masked-U form equals the per-row ridge solve of [R] item 3's decomposition."""
    _, X, Xf, H, prep, A = _cae_problem(31, K=9)
    P2 = O.cae_correction(prep["U"], H, A)
    P2d = O.cae_correction_by_definition(prep["Hd"], 2.0 * (Xf.T @ X))
    np.testing.assert_allclose(P2, P2d, rtol=1e-9, atol=1e-12)
    assert np.count_nonzero(np.tril(P2)) == 0


@pytest.mark.parametrize("dead", [(), (2,)])
def test_cae_correction_closed_form(dead):
    """H_d U^T = R is upper triangular with R_jj = 1/U_jj, and damping and the dead fix are diagonal, so
    P2 = P1 + I - diag(U)^-1 U exactly (the identity the library uses instead of a third K x K product)."""
    _, X, Xf, H, prep, A = _cae_problem(32, K=8, dead=dead)
    U = prep["U"]
    P1 = O.asym_correction(U, A)
    P2 = O.cae_correction(U, H, A)
    closed = P1 + np.eye(len(U)) - U / np.diag(U)[:, None]
    np.testing.assert_allclose(P2, closed, atol=1e-12 * np.abs(P2).max())
    # with no input mismatch P2 is I - diag(U)^-1 U
    np.testing.assert_allclose(O.cae_correction(U, H), np.eye(len(U)) - U / np.diag(U)[:, None],
                               atol=1e-12 * np.abs(P2).max())


@pytest.mark.parametrize("asym", [False, True])
def test_cae_loop_equals_explicit_solves(asym):
    """Loop with P2 (and P1) == sequential compensation with explicit inverses plus a per-step lstsq of the
    r1 + r2 residual; with the closed form the same update reads w_k -= (U_jk/U_jj)(w0_j - q_j) + P1_jk w0_j."""
    rng, X, Xf, H, prep, A = _cae_problem(33 + asym, K=7)
    if not asym:
        Xf = X.copy()
        A = np.zeros_like(H)
    U = prep["U"]
    P1 = O.asym_correction(U, A) if asym else None
    P2 = O.cae_correction(U, H, A)
    w = rng.normal(0, 1.5, size=len(U))
    one = np.array([1.0], np.float32)
    r = O.quantize_layer(w[:, None], U, bits=4, scales=one, P1=P1, P2=P2)
    seq = O.obq_sequential(prep["Hd"], w, O.fixed_grid_quantize, damp=prep["damp"], X_free_basis=(X, Xf - X),
                           cae=True)
    np.testing.assert_allclose(r["Q"][:, 0], seq["w"], atol=1e-10)
    rb = O.quantize_layer(w[:, None], U, bits=4, scales=one, P1=P1, P2=P2, blocksize=3)
    np.testing.assert_array_equal(rb["codes"], r["codes"])
    # the CAE term changes the result on this input (so the test would see it dropped)
    plain = O.quantize_layer(w[:, None], U, bits=4, scales=one, P1=P1)
    assert not np.allclose(plain["W_pre"], r["W_pre"])
    # closed form of the combined step, coordinate by coordinate
    z = 8
    Wk = w.copy()
    for j in range(len(U)):
        q = float(np.clip(np.rint(Wk[j]) + z, 0, 15) - z)
        Wk[j + 1:] += -(U[j, j + 1:] / U[j, j]) * (w[j] - q) + (P1[j, j + 1:] * w[j] if asym else 0.0)
        Wk[j] = q
    np.testing.assert_allclose(Wk, r["Q"][:, 0], atol=1e-10)


# ------------------------------------------------------------------------------------------------ packing
def test_pack_codes_worked_examples():
    """Hand-worked words of the bitstream layout (code k at stream bits [b k, b k + b))."""
    c = np.zeros((32, 1), np.int64)
    c[0, 0] = 1                  # bit 0
    c[10, 0] = 7                 # bits 30, 31, 32 -> word 0 bits 30-31, word 1 bit 0
    c[31, 0] = 5                 # bits 93..95 = 1, 0, 1 -> word 2 bits 29 and 31
    w = O.pack_codes(c, 3)
    assert w.shape == (3, 1)
    assert int(w[0, 0]) == (1 | (1 << 30) | (1 << 31))
    assert int(w[1, 0]) == 1
    assert int(w[2, 0]) == ((1 << 29) | (1 << 31))
    assert int(O.pack_codes(np.full((32, 1), 7), 3)[1, 0]) == 0xFFFFFFFF
    # 4-bit: codes 0..15 in order -> nibbles 0x76543210, 0xFEDCBA98
    w4 = O.pack_codes(np.arange(16)[:, None], 4)
    assert [int(v) for v in w4[:, 0]] == [0x76543210, 0xFEDCBA98]
    # 2-bit: 3, 0, 1, 2 -> 0b10_01_00_11 = 0x93; K = 5 leaves the rest of the word zero
    w2 = O.pack_codes(np.array([[3], [0], [1], [2], [3]]), 2)
    assert w2.shape == (1, 1) and int(w2[0, 0]) == 0x93 | (3 << 8)
    # 8-bit: bytes in order
    assert int(O.pack_codes(np.array([[0x11], [0x22], [0x33], [0x44]]), 8)[0, 0]) == 0x44332211


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 8])
def test_pack_round_trip(bits):
    rng = np.random.default_rng(bits)
    for K in (1, 31, 32, 33, 100):
        c = rng.integers(0, 1 << bits, size=(K, 7))
        w = O.pack_codes(c, bits)
        assert w.shape == ((K * bits + 31) // 32, 7)
        np.testing.assert_array_equal(O.unpack_codes(w, K, bits), c)


# ------------------------------------------------------------------------------------------------ Hadamard rotation
def test_sylvester_against_scipy_and_orthogonality():
    import scipy.linalg
    for K in (1, 2, 4, 64, 512):
        H = O.sylvester(K)
        np.testing.assert_array_equal(H, scipy.linalg.hadamard(K))
        np.testing.assert_array_equal(H @ H.T, K * np.eye(K))
    np.testing.assert_array_equal(O.sylvester(2), [[1, 1], [1, -1]])


def test_hadamard_rotation_properties():
    rng = np.random.default_rng(3)
    K = 256
    x = rng.normal(size=(5, K))
    d = rng.choice([-1.0, 1.0], size=K)
    y = O.hadamard_rotate_rows(x, d)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    # unit vector e_k -> d_k * row k of H / sqrt(K)
    e = np.zeros((1, K)); e[0, 7] = 1.0
    np.testing.assert_allclose(O.hadamard_rotate_rows(e, d)[0], d[7] * O.sylvester(K)[7] / 16.0, atol=1e-15)
    # rotating activations and nn.Linear-layout weight rows the same way keeps x W^T
    W = rng.normal(size=(9, K))
    np.testing.assert_allclose(y @ O.hadamard_rotate_rows(W, d).T, x @ W.T, rtol=1e-10, atol=1e-10)
    # without signs the rotation is its own inverse
    np.testing.assert_allclose(O.hadamard_rotate_rows(O.hadamard_rotate_rows(x)), x, atol=1e-12)


# ------------------------------------------------------------------------------------------------ groups, act-order, MSE clipping
def _sym_quant(s, bits):
    z, qmax = 2 ** (bits - 1), 2 ** bits - 1
    return lambda v: s * (np.clip(np.rint(v / s) + z, 0, qmax) - z)


def test_act_order_perm_worked_example():
    H = np.diag([3.0, 0.0, 5.0, 3.0])          # dead coordinate 1 counts as 1; equal diagonals keep their order
    assert list(O.act_order_perm(H)) == [2, 0, 3, 1]


def test_act_order_loop_equals_explicit_order():
    """Loop over the permuted problem == sequential compensation with explicit inverses in that order."""
    rng = np.random.default_rng(41)
    K = 9
    X = rng.normal(size=(40, K)) * np.exp(rng.normal(size=K))
    prep = O.prepare(O.gram([X]), 0.01)
    perm = O.act_order_perm(prep["Hd"])
    assert not np.array_equal(perm, np.arange(K))
    Up = O.prepare(O.gram([X[:, perm]]), 0.01)["U"]
    w = rng.normal(0, 1.5, size=K)
    one = np.array([1.0], np.float32)
    r = O.quantize_layer(w[:, None], Up, bits=4, scales=one, perm=perm)
    seq = O.obq_sequential(prep["Hd"], w, O.fixed_grid_quantize, order=perm)
    np.testing.assert_allclose(r["Q"][:, 0], seq["w"], atol=1e-10)
    rb = O.quantize_layer(w[:, None], Up, bits=4, scales=one, perm=perm, blocksize=4)
    np.testing.assert_array_equal(rb["codes"], r["codes"])


@pytest.mark.parametrize("G,act", [(4, False), (4, True), (8, False)])
def test_dynamic_groups_equal_explicit_regrid(G, act):
    """Re-estimated group scales == sequential compensation that recomputes the grid from the current weights
    at every group start (explicit inverses, any order)."""
    rng = np.random.default_rng(43 + G)
    K, bits = 12, 3
    X = rng.normal(size=(60, K)) * np.exp(rng.normal(size=K))
    prep = O.prepare(O.gram([X]), 0.01)
    perm = O.act_order_perm(prep["Hd"]) if act else np.arange(K)
    Up = O.prepare(O.gram([X[:, perm]]), 0.01)["U"]
    w = rng.normal(0, 0.05, size=K)
    r = O.quantize_layer(w[:, None], Up, bits, groupsize=G, perm=perm)

    state = {}

    def quant_at(i, wc):
        if i % G == 0:
            grp = perm[i:i + G]
            state["s"] = float(O.grid_scales(wc[grp][:, None], bits)[0])
        return _sym_quant(state["s"], bits)

    seq = O.obq_sequential(prep["Hd"], w, None, order=perm, quant_at=quant_at)
    np.testing.assert_allclose(r["Q"][:, 0], seq["w"], atol=1e-10)
    # group index of each original coordinate, and W_hat through it
    np.testing.assert_array_equal(r["g_idx"][perm], np.arange(K) // G)
    np.testing.assert_array_equal(r["W_hat_fp32"], (r["scales"][r["g_idx"]] * (r["codes"] - 4)).astype(np.float32))
    rb = O.quantize_layer(w[:, None], Up, bits, groupsize=G, perm=perm, blocksize=G)
    np.testing.assert_array_equal(rb["codes"], r["codes"])


def test_group_scales_reduce_to_per_channel():
    rng = np.random.default_rng(44)
    K, N = 16, 5
    W = rng.normal(size=(K, N))
    W[3] = 0.0
    U = O.prepare(O.gram([rng.normal(size=(50, K))]), 0.01)["U"]
    ref = O.quantize_layer(W, U, 3)
    np.testing.assert_array_equal(O.grid_scales(W, 3), O.channel_scales(W, 3))
    for static in (False, True):
        r = O.quantize_layer(W, U, 3, groupsize=K, static_groups=static)
        np.testing.assert_array_equal(r["scales"][0], ref["scales"])
        np.testing.assert_array_equal(r["codes"], ref["codes"])
    # static groups take their scales from the original rows of their group
    r = O.quantize_layer(W, U, 3, groupsize=4, static_groups=True)
    for g in range(4):
        np.testing.assert_array_equal(r["scales"][g], O.channel_scales(W[4 * g:4 * g + 4], 3))


def test_mse_clipping():
    bits = 3
    # all |w| equal: the unclipped grid reproduces them exactly (zero error), so alpha = 1 is kept
    W = np.array([[0.5, -1.0], [-0.5, 1.0], [0.5, 1.0]], np.float32)
    np.testing.assert_array_equal(O.grid_scales(W, bits, mse=True), O.grid_scales(W, bits))
    # one outlier among many small values: clipping lowers the squared error, never raises it
    rng = np.random.default_rng(45)
    W = rng.normal(0, 0.1, size=(128, 6)).astype(np.float32)
    W[7] = 1.0
    s1 = O.grid_scales(W, bits)
    sm = O.grid_scales(W, bits, mse=True)
    assert (sm <= s1).all() and (sm < s1).any()

    def err(s):
        q = s * (np.clip(np.rint(W / s) + 4, 0, 7) - 4)
        return ((W.astype(np.float64) - q) ** 2).sum(axis=0)

    assert (err(sm.astype(np.float64)) <= err(s1.astype(np.float64))).all()
    # the chosen scale is one of the fp32 candidates, and no candidate has a smaller error
    cands = (np.float32(2) * np.abs(W).max(axis=0))[None, :] * O.MSE_SHRINK[:, None] / np.float32(7)
    for n in range(W.shape[1]):
        assert sm[n] in cands[:, n]
        assert err(sm.astype(np.float64))[n] <= min(err(np.full(6, c, np.float64))[n] for c in cands[:, n])
